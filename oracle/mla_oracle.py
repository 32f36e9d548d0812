"""Plain, slow fp64 CPU oracle for one Multi-head Latent Attention (MLA) decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The GPU
library never routes through it, and it shares no code, constant or helper with
the HIP path; it imports numpy and nothing else.

Sources (web pages, cited by title and section):
  [Report]  "《DeepSeek-V2》深度解读报告" (zako-mio.github.io knowledge base):
            §2.1 KV cache, §2.2 low-rank key-value joint compression,
            §2.3 absorption, §2.4 decoupled RoPE, §3.1 full MLA data flow.
  [Wiki]    "DeepSeek-V2" paper notes (wiki.hugogu.cn): the MLA inference flow
            (latent cached, all history decompressed to per-head K/V, then
            attention) and the decode timeline (Q is never cached).
  [Digest]  "DeepSeek-V2论文解读 ... KV缓存压93.3%" (xdnf.cn), §2.1: cache size
            2*n_h*d_h*l for MHA versus one latent per token for MLA.

What is computed here is the NON-ABSORBED definition: per-head keys and values
are decompressed explicitly from the cached latent and attention runs per head
in fp64 ([Wiki] inference flow; [Report] §2.2).  A separately written absorbed
companion ([Report] §2.3) is provided for cheap coverage of large inputs; the
two must agree to rounding (associativity), which is one of the pins.

Readings taken where the pages are silent (all inline formulas were lost):
  * softmax scale tau = 1/sqrt(d_h + d_R) unless the caller passes one;
  * RoPE rotates adjacent pairs (x[2k], x[2k+1]) by angle pos*theta_k with
    theta_k = base**(-2k/d_R); angles in fp64; YaRN ([Report] §3.3 gives only
    its parameters) follows the published method (:class:`Yarn`);
  * decode position t = L-1: the new token is appended first and attends to
    positions 0..L-1 inclusive;
  * q^C = W_Q h, or with the query's low-rank compression c^Q = W_DQ h and
    q^C = W_UQ c^Q ([Report] §3.1 flow; no norm on c^Q, none is drawn); q^R is
    taken from h either way; no norm on the latent;
  * head i owns rows i*d_h:(i+1)*d_h of W_Q, W_UK, W_UV (and i*d_R:(i+1)*d_R
    of W_QR) and columns i*d_h:(i+1)*d_h of W_O;
  * cache row = [c^KV (d_c) | k^R (d_R)]; paged in pages of ``page_size`` rows:
    logical position j of sequence b lives in physical row
    block_table[b][j // page_size] * page_size + j % page_size;
  * split s of a sequence of length L under S splits covers logical positions
    [s*chunk, min(L, (s+1)*chunk)) with chunk = page_size*ceil(ceil(L/S)/page_size);
    an empty split has lse = -inf and a zero output.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "Yarn", "yarn_logit_factor", "rope_theta", "rope", "latent_rows", "page_slot", "query_heads", "compressed_query",
    "query_heads_cq",
    "mla_decode_step", "mla_decode_step_absorbed", "split_bounds",
    "attention_partials", "merge_lse", "absorb_q", "absorb_out",
    "mla_cache_elems_per_token", "mha_cache_elems_per_token", "E4M3_MAX", "e4m3_values",
    "e4m3_encode", "fp8_row_scale_exponent", "bf16_bits", "fp8_quantize_row",
    "fp8_dequantize_row", "fp8_page_bytes", "fp8_page_image",
    "prefill_attention_partials", "mla_prefill_step",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- positions --
class Yarn:
    """RoPE stretched by YaRN, the long-context extension [Report] §3.3 (its
    long-context paragraph) names for DeepSeek-V2: the window is taken from 4K to
    128K with scale 40, alpha = 1, beta = 32.  The pages give only those
    numbers; the method followed is the published one (Peng, Quesnelle, Fan and
    Shippole, "YaRN: Efficient Context Window Extension of Large Language Models",
    2023), with ``orig_len`` the context the frequencies were trained for:

      * pair k rotates r_k = orig_len / lambda_k times over the original window,
        lambda_k = 2 pi / theta_k its wavelength;
      * ramp gamma_k = 0 for r_k < alpha, 1 for r_k > beta, linear in between;
      * theta'_k = (1 - gamma_k) theta_k / scale + gamma_k theta_k: pairs that turn
        fewer than alpha times are interpolated by the scale, pairs that turn
        more than beta times keep their frequency;
      * the logits are multiplied by 1/t with sqrt(1/t) = 0.1 ln(scale) + 1
        (the method's temperature; here on the whole score, content plus RoPE
        channel, since [Report] §2.4 puts both under one softmax).

    A scale <= 1 is plain RoPE.  Passed wherever a RoPE ``base`` is taken."""

    def __init__(self, base: float, scale: float, orig_len: int, alpha: float, beta: float):
        self.base, self.scale, self.orig_len = float(base), float(scale), int(orig_len)
        self.alpha, self.beta = float(alpha), float(beta)


def _base_of(base):
    return base.base if isinstance(base, Yarn) else float(base)


def yarn_logit_factor(base) -> float:
    """1/t of YaRN's temperature, (0.1 ln s + 1)^2, for a :class:`Yarn` base with
    s > 1; 1 for plain RoPE."""
    if isinstance(base, Yarn) and base.scale > 1.0:
        return (0.1 * math.log(base.scale) + 1.0) ** 2
    return 1.0


def rope_theta(d_rope: int, base) -> np.ndarray:
    """theta_k = base**(-2k/d_R), k = 0..d_R/2-1 ([Report] §2.4: RoPE acts only on
    the decoupled d_R-wide branch; base 10000 per the workload definitions), or
    the YaRN-stretched frequencies for a :class:`Yarn` base."""
    k = np.arange(d_rope // 2, dtype=np.float64)
    theta = np.power(_base_of(base), -2.0 * k / d_rope)
    if not isinstance(base, Yarn) or base.scale <= 1.0:
        return theta
    wavelength = 2.0 * math.pi / theta
    rotations = base.orig_len / wavelength
    gamma = np.clip((rotations - base.alpha) / (base.beta - base.alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / base.scale + gamma * theta


def rope(x, pos, base: float) -> np.ndarray:
    """Rotate adjacent pairs of the last axis of ``x`` by pos*theta_k.

    ``pos`` broadcasts against ``x.shape[:-1]``.  [Report] §2.4: the decoupled
    query q^R and the shared key k^R carry the position; nothing else does.
    """
    x = _f64(x)
    d = x.shape[-1]
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_theta(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


# -------------------------------------------------------------- cache rows --
def latent_rows(h, w_dkv, w_kr, pos, base: float) -> np.ndarray:
    """Cache rows [c^KV | k^R] for hidden states ``h`` [N, H] at positions ``pos``.

    c^KV = W_DKV h ([Report] §2.2: the joint down-projection; the latent is the
    only K/V object that is cached) and k^R = RoPE(W_KR h, pos) ([Report] §2.4:
    one RoPE key shared by every head, also cached).  Row width d_c + d_R.
    """
    h = _f64(h)
    c = h @ _f64(w_dkv).T
    kr = rope(h @ _f64(w_kr).T, pos, base)
    return np.concatenate([c, kr], axis=-1)


def page_slot(block_table, seq: int, pos, page_size: int = 64):
    """Physical row of logical position(s) ``pos`` of sequence ``seq`` in a paged
    pool (paged cache management is named in [Digest] §3.1; the page size and
    the permuted page table are workload parameters)."""
    pos = np.asarray(pos, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    return bt[seq, pos // page_size] * page_size + pos % page_size


def gather_rows(pool, block_table, seq: int, length: int, page_size: int = 64):
    """Logical rows 0..length-1 of sequence ``seq`` read out of a paged pool
    [num_pages, page_size, row] (any float dtype), upcast to fp64."""
    flat = np.asarray(pool).reshape(-1, np.asarray(pool).shape[-1])
    return _f64(flat[page_slot(block_table, seq, np.arange(length), page_size)])


# ------------------------------------------------------------------- query --
def query_heads(h_t, w_q, w_qr, pos: int, n_heads: int, d_head: int, d_rope: int,
                base: float):
    """q^C_i = W_Q,i h_t (d_h) and q^R_i = RoPE(W_QR,i h_t, t) (d_R) per head
    ([Report] §3.1 data flow: per-head RoPE query from h_t; query is not cached,
    [Wiki] decode timeline).  Returns ([n_h, d_h], [n_h, d_R])."""
    h_t = _f64(h_t)
    qc = (_f64(w_q) @ h_t).reshape(n_heads, d_head)
    qr = rope((_f64(w_qr) @ h_t).reshape(n_heads, d_rope), pos, base)
    return qc, qr


def compressed_query(h_t, w_dq, w_uq):
    """Query through its low-rank compression, the MLA information flow of
    [Report] §3.1: c^Q = W_D^Q h_t (d_c', 1536 there), then q^C = W_U^Q c^Q
    (n_h d_h; the up-projection's name follows W_U^K / W_U^V).  Returns q^C."""
    c_q = _f64(w_dq) @ _f64(h_t)
    return _f64(w_uq) @ c_q


def query_heads_cq(h_t, w_dq, w_uq, w_qr, pos: int, n_heads: int, d_head: int, d_rope: int,
                   base: float):
    """q^C_i from the compressed query and q^R_i = RoPE(W_QR,i h_t, t): per the
    same flow, the RoPE query is still taken from h_t.  Returns ([n_h, d_h], [n_h, d_R])."""
    qc = compressed_query(h_t, w_dq, w_uq).reshape(n_heads, d_head)
    qr = rope((_f64(w_qr) @ _f64(h_t)).reshape(n_heads, d_rope), pos, base)
    return qc, qr


def _default_scale(d_head: int, d_rope: int, scale, base=None):
    """tau: ``scale`` if given, else 1/sqrt(d_h + d_R); times YaRN's logit factor
    when ``base`` is a stretched RoPE (:class:`Yarn`)."""
    tau = 1.0 / math.sqrt(d_head + d_rope) if (scale is None or scale <= 0) else float(scale)
    return tau * yarn_logit_factor(base)


# -------------------------------------------------- the definition (oracle) --
def mla_decode_step(h_t, rows, w_q, w_qr, w_uk, w_uv, w_o, pos: int, n_heads: int,
                    d_head: int, d_latent: int, d_rope: int, base: float, scale=None,
                    w_dq=None, w_uq=None):
    """Non-absorbed MLA decode for one sequence, fp64.

    ``rows`` [L, d_c + d_R] are the cached rows of logical positions 0..L-1 (the
    decode token's own row included, at L-1 = ``pos``).  For each head i:
      k^C_{j,i} = W_UK,i c_j, v^C_{j,i} = W_UV,i c_j      ([Report] §2.2)
      k_{j,i} = [k^C_{j,i}; k^R_j],  q_i = [q^C_i; q^R_i]   ([Report] §2.4, the
                content-channel and RoPE-channel scores add up)
      p_i = softmax_j(tau * q_i . k_{j,i}),  o_i = sum_j p_ij v^C_{j,i}
    then u = W_O [o_1; ...; o_n_h].  Returns dict(u [H], o [n_h, d_h],
    lse [n_h]) where lse_i = log sum_j exp(s_ij).  With ``w_dq``/``w_uq`` the
    query goes through its compression (:func:`query_heads_cq`; ``w_q`` unused).
    """
    rows = _f64(rows)
    c, kr = rows[:, :d_latent], rows[:, d_latent:d_latent + d_rope]
    tau = _default_scale(d_head, d_rope, scale, base)
    if w_dq is None:
        qc, qr = query_heads(h_t, w_q, w_qr, pos, n_heads, d_head, d_rope, base)
    else:
        qc, qr = query_heads_cq(h_t, w_dq, w_uq, w_qr, pos, n_heads, d_head, d_rope, base)
    w_uk, w_uv = _f64(w_uk), _f64(w_uv)
    o = np.zeros((n_heads, d_head))
    lse = np.zeros(n_heads)
    for i in range(n_heads):
        blk = slice(i * d_head, (i + 1) * d_head)
        k_c = c @ w_uk[blk].T                      # [L, d_h] decompressed keys
        v_c = c @ w_uv[blk].T                      # [L, d_h] decompressed values
        k = np.concatenate([k_c, kr], axis=1)      # per-head key with shared RoPE key
        q = np.concatenate([qc[i], qr[i]])
        s = tau * (k @ q)
        m = s.max()
        e = np.exp(s - m)
        z = e.sum()
        o[i] = (e / z) @ v_c
        lse[i] = m + math.log(z)
    u = _f64(w_o) @ o.reshape(-1)
    return {"u": u, "o": o, "lse": lse, "q_c": qc, "q_r": qr}


# ------------------------------------------------ absorbed fp64 companion --
def absorb_q(h_t, w_q, w_qr, w_uk, pos: int, n_heads: int, d_head: int, d_latent: int,
             d_rope: int, base: float, w_dq=None, w_uq=None):
    """Absorbed query: q_lat,i = W_UK,i^T q^C_i ([Report] §2.3: q.(W_UK c) is
    regrouped as (W_UK^T q).c) and q_pe,i = q^R_i; q^C from W_Q, or from the
    compression when ``w_dq``/``w_uq`` are given.  Returns ([n_h, d_c], [n_h, d_R])."""
    if w_dq is None:
        qc, qr = query_heads(h_t, w_q, w_qr, pos, n_heads, d_head, d_rope, base)
    else:
        qc, qr = query_heads_cq(h_t, w_dq, w_uq, w_qr, pos, n_heads, d_head, d_rope, base)
    w_uk = _f64(w_uk).reshape(n_heads, d_head, d_latent)
    q_lat = np.einsum("ihc,ih->ic", w_uk, qc)
    return q_lat, qr


def absorb_out(o_lat, w_uv, w_o, n_heads: int, d_head: int, d_latent: int):
    """Absorbed output for one token: o_i = W_UV,i o_lat,i, u = W_O [o_1..o_n_h]
    ([Report] §2.3: W_UV is folded into the output projection)."""
    w_uv = _f64(w_uv).reshape(n_heads, d_head, d_latent)
    o = np.einsum("ihc,ic->ih", w_uv, _f64(o_lat))
    return _f64(w_o) @ o.reshape(-1)


def _latent_attention(q_lat, q_pe, rows, d_latent: int, d_rope: int, tau: float):
    """Attention of every head over latent rows: s_ij = tau (q_lat,i.c_j + q_pe,i.k^R_j).
    Returns (o_lat [n_h, d_c], lse [n_h]); an empty row set gives (0, -inf)."""
    rows = _f64(rows)
    n_h = np.asarray(q_lat).shape[0]
    if rows.shape[0] == 0:
        return np.zeros((n_h, d_latent)), np.full(n_h, -np.inf)
    c, kr = rows[:, :d_latent], rows[:, d_latent:d_latent + d_rope]
    s = tau * (_f64(q_lat) @ c.T + _f64(q_pe) @ kr.T)        # [n_h, L]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ c, (m + np.log(z))[:, 0]


def mla_decode_step_absorbed(h_t, rows, w_q, w_qr, w_uk, w_uv, w_o, pos: int,
                             n_heads: int, d_head: int, d_latent: int, d_rope: int,
                             base: float, scale=None, w_dq=None, w_uq=None):
    """Absorbed fp64 form of :func:`mla_decode_step` (same inputs): attention runs
    in the d_c-wide latent space and per-head K/V are never formed ([Report]
    §2.3).  Returns dict(u, q_lat, q_pe, o_lat, lse)."""
    tau = _default_scale(d_head, d_rope, scale, base)
    q_lat, q_pe = absorb_q(h_t, w_q, w_qr, w_uk, pos, n_heads, d_head, d_latent, d_rope, base,
                           w_dq, w_uq)
    o_lat, lse = _latent_attention(q_lat, q_pe, rows, d_latent, d_rope, tau)
    u = absorb_out(o_lat, w_uv, w_o, n_heads, d_head, d_latent)
    return {"u": u, "q_lat": q_lat, "q_pe": q_pe, "o_lat": o_lat, "lse": lse}


# ------------------------------------------------------- split and merge --
def split_bounds(length: int, num_splits: int, page_size: int = 64):
    """[(start, end)] of each split: page-aligned equal chunks, trailing splits empty."""
    per = -(-length // num_splits)
    chunk = page_size * (-(-per // page_size))
    return [(min(length, s * chunk), min(length, (s + 1) * chunk)) for s in range(num_splits)]


def attention_partials(q_lat, q_pe, rows, num_splits: int, d_latent: int, d_rope: int,
                       scale: float, page_size: int = 64):
    """Per-split partial attention of one sequence: for each split s,
    (o_s [n_h, d_c] normalised within the split, lse_s [n_h])."""
    out_o, out_l = [], []
    for (a, b) in split_bounds(_f64(rows).shape[0], num_splits, page_size):
        o, l = _latent_attention(q_lat, q_pe, _f64(rows)[a:b], d_latent, d_rope, scale)
        out_o.append(o)
        out_l.append(l)
    return np.stack(out_o), np.stack(out_l)


def prefill_attention_partials(q_lat, q_pe, rows, positions, num_splits: int, d_latent: int,
                               d_rope: int, scale: float, page_size: int = 64):
    """Chunked-prefill attention of one sequence: query t is the prompt token at
    position ``positions[t]`` and attends causally to cached rows 0..positions[t]
    (its own row included) -- every prompt token takes the per-token MLA flow of
    [Report] §3.1 over the cache as it stands at its position.  Returns, per query,
    the split partials of :func:`attention_partials` over those rows."""
    rows = _f64(rows)
    return [attention_partials(q_lat[t], q_pe[t], rows[:int(p) + 1], num_splits, d_latent,
                               d_rope, scale, page_size) for t, p in enumerate(positions)]


def mla_prefill_step(h_chunk, rows_before, w_q, w_qr, w_dkv, w_kr, w_uk, w_uv, w_o, n_heads: int,
                     d_head: int, d_latent: int, d_rope: int, base: float, scale=None):
    """Non-absorbed prefill of a chunk of T prompt tokens of one sequence whose
    first P = len(rows_before) rows are cached: the chunk's tokens sit at
    positions P..P+T-1, their latent rows are appended ([Report] §2.2, §2.4), and
    token t's output is the decode step (:func:`mla_decode_step`) of the context
    of rows 0..P+t.  Returns dict(u [T, H], o [T, n_h, d_h], lse [T, n_h])."""
    h_chunk = _f64(h_chunk)
    P, T = len(rows_before), len(h_chunk)
    pos = np.arange(P, P + T)
    rows = np.concatenate([_f64(rows_before).reshape(P, d_latent + d_rope),
                           latent_rows(h_chunk, w_dkv, w_kr, pos, base)])
    out = [mla_decode_step(h_chunk[t], rows[:P + t + 1], w_q, w_qr, w_uk, w_uv, w_o, P + t,
                           n_heads, d_head, d_latent, d_rope, base, scale) for t in range(T)]
    return {k: np.stack([o[k] for o in out]) for k in ("u", "o", "lse")}


def merge_lse(o_parts, lse_parts):
    """Combine split partials: lse* = max_s lse_s, w_s = exp(lse_s - lse*),
    o = sum_s w_s o_s / sum_s w_s, lse = lse* + log sum_s w_s.  Splits with
    lse = -inf carry zero weight.  o_parts [S, ..., d], lse_parts [S, ...]."""
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    top = lse_parts.max(axis=0)
    safe = np.where(np.isfinite(top), top, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - safe), 0.0)
    z = w.sum(axis=0)
    o = (w[..., None] * o_parts).sum(axis=0) / np.where(z > 0, z, 1.0)[..., None]
    lse = np.where(z > 0, safe + np.log(np.where(z > 0, z, 1.0)), -np.inf)
    return o, lse


# ------------------------------------------------------------- FP8 cache --
# [Report] §4.2: inference quantizes the (already 576-wide) latent cache to about
# 6 bits per element; the scheme is not on the pages.  The reading used here:
# c^KV in e4m3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, largest
# finite 448, no infinities) with one power-of-two scale per row; k^R in bf16.
E4M3_MAX = 448.0


def e4m3_values() -> np.ndarray:
    """Value of every e4m3 byte 0..255 from the format's definition (NaN for the
    two NaN codes 0x7f, 0xff): exponent field 0 is subnormal, m * 2^-9."""
    out = np.empty(256)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e, m = (code >> 3) & 0xF, code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * m * 2.0 ** -9
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def e4m3_encode(x) -> np.ndarray:
    """Round-to-nearest-even of each value (|x| <= 448) to its e4m3 byte: the
    nearest of the finite codes, ties to the code with an even mantissa."""
    x = np.asarray(x, dtype=np.float64)
    vals = e4m3_values()
    pos = np.array([c for c in range(128) if np.isfinite(vals[c])])   # 0x00..0x7e, increasing
    pv = vals[pos]
    a = np.abs(x)
    if np.any(a > E4M3_MAX):
        raise ValueError("value beyond the e4m3 range")
    hi = np.searchsorted(pv, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, len(pv) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - pv[lo], pv[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (pos[hi] % 2 == 0))
    pick_hi |= pv[hi] == a
    code = np.where(pick_hi, pos[hi], pos[lo])
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def fp8_row_scale_exponent(amax: float) -> int:
    """Exponent e of the row scale 2^e: the smallest e with amax / 2^e <= 448
    (448 = 0.875 * 2^9).  With amax = m 2^x, m in [0.5, 1): e = x - 9, plus one
    when m > 0.875; amax = 0 gives e = 0.  Clamped to [-126, 127]."""
    if amax == 0.0:
        return 0
    m, x = math.frexp(amax)
    e = x - 9 + (1 if m > 0.875 else 0)
    return int(min(max(e, -126), 127))


def bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns (round to nearest even) of fp32 values."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def fp8_quantize_row(row_f32, d_latent: int):
    """One cache row [c (d_c) | k^R (d_R)] given in fp32 -> (e4m3 codes of c,
    bf16 bits of k^R, scale exponent e): codes = RNE_e4m3(c / 2^e)."""
    row = np.asarray(row_f32, dtype=np.float32)
    c = row[:d_latent].astype(np.float64)
    e = fp8_row_scale_exponent(float(np.abs(c).max()) if c.size else 0.0)
    codes = e4m3_encode(np.ldexp(c, -e))             # exact: a power-of-two scale
    return codes, bf16_bits(row[d_latent:]), e


def fp8_dequantize_row(codes, kr_bits, e: int) -> np.ndarray:
    """fp64 row [c^ | k^R] of a quantized row: c^ = code value * 2^e."""
    c = np.ldexp(e4m3_values()[np.asarray(codes)], e)
    kr = (np.asarray(kr_bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.concatenate([c, kr])


def fp8_page_bytes(page_size: int, d_latent: int, d_rope: int) -> int:
    """Bytes of one FP8 page: page_size rows of [d_c e4m3 bytes | d_R bf16], then
    page_size fp32 row scales."""
    return page_size * (d_latent + 2 * d_rope) + 4 * page_size


def fp8_page_image(rows_f32, d_latent: int, d_rope: int) -> np.ndarray:
    """Byte image of one FP8 page holding ``rows_f32`` [n <= page_size, d_c + d_R]
    in slots 0..n-1 (other slots zero; page_size = n)."""
    n = len(rows_f32)
    rb = d_latent + 2 * d_rope
    img = np.zeros(fp8_page_bytes(n, d_latent, d_rope), dtype=np.uint8)
    for r, row in enumerate(rows_f32):
        codes, kr, e = fp8_quantize_row(row, d_latent)
        img[r * rb:r * rb + d_latent] = codes
        img[r * rb + d_latent:(r + 1) * rb] = kr.view(np.uint8)
        img[n * rb + 4 * r:n * rb + 4 * r + 4] = np.array([2.0 ** e], dtype=np.float32).view(np.uint8)
    return img


# ------------------------------------------------------------ cache sizes --
def mla_cache_elems_per_token(d_latent: int, d_rope: int, layers: int = 1) -> int:
    """Elements cached per token: (d_c + d_R) per layer ([Report] §2.4, §3.1)."""
    return (d_latent + d_rope) * layers


def mha_cache_elems_per_token(n_heads: int, d_head: int, layers: int = 1) -> int:
    """MHA caches K and V per head: 2 n_h d_h per layer ([Digest] §2.1; [Report] §2.1)."""
    return 2 * n_heads * d_head * layers
