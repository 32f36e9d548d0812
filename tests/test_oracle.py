"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: numbers printed on the pages
(tests/golden/), closed forms, textbook special cases written independently
here (multi-head attention, a multi-query RoPE channel, RoPE as a complex
multiplication), library routines (torch scaled_dot_product_attention,
scipy logsumexp) and brute force on tiny inputs.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _weights(rng, H, nh, dh, dc, dr):
    return dict(
        w_q=rng.normal(size=(nh * dh, H)) / math.sqrt(H),
        w_qr=rng.normal(size=(nh * dr, H)) / math.sqrt(H),
        w_dkv=rng.normal(size=(dc, H)) / math.sqrt(H),
        w_kr=rng.normal(size=(dr, H)) / math.sqrt(H),
        w_uk=rng.normal(size=(nh * dh, dc)) / math.sqrt(dc),
        w_uv=rng.normal(size=(nh * dh, dc)) / math.sqrt(dc),
        w_o=rng.normal(size=(H, nh * dh)) / math.sqrt(nh * dh),
    )


def _complex_rope(x, pos, base):
    """RoPE written independently: pair (x[2k], x[2k+1]) as the complex number
    x[2k] + i x[2k+1], multiplied by exp(i * pos * base**(-2k/d))."""
    d = len(x)
    out = []
    for k in range(d // 2):
        z = complex(x[2 * k], x[2 * k + 1]) * cmath.exp(1j * pos * base ** (-2.0 * k / d))
        out += [z.real, z.imag]
    return np.array(out)


# ------------------------------------------------------------------- RoPE --
def test_rope_closed_form_values():
    # d=2: theta_0 = 1, so [1, 0] at position 1 becomes [cos 1, sin 1]
    np.testing.assert_allclose(O.rope(np.array([1.0, 0.0]), 1, 10000.0),
                               [math.cos(1.0), math.sin(1.0)], rtol=0, atol=1e-15)
    # d=4, base 10000: theta_1 = 10000**(-1/2) = 0.01; position 100 turns pair 1 by 1 rad
    np.testing.assert_allclose(O.rope(np.array([0.0, 0.0, 1.0, 0.0]), 100, 10000.0),
                               [0.0, 0.0, math.cos(1.0), math.sin(1.0)], atol=1e-14)
    # pair 0 at position 100 turns by 100 rad; [0, 1] -> [-sin, cos]
    np.testing.assert_allclose(O.rope(np.array([0.0, 1.0, 0.0, 0.0]), 100, 10000.0),
                               [-math.sin(100.0), math.cos(100.0), 0.0, 0.0], atol=1e-13)


def test_rope_matches_complex_multiplication():
    rng = _rng(1)
    for d, pos, base in [(8, 0, 10000.0), (8, 63, 10000.0), (64, 4095, 10000.0),
                         (64, 131071, 10000.0), (6, 17, 500.0)]:
        x = rng.normal(size=d)
        # fp64 angle pos*theta carries ~pos * 1e-16 rad of rounding in either form
        np.testing.assert_allclose(O.rope(x, pos, base), _complex_rope(x, pos, base),
                                   rtol=0, atol=1e-12 + 4e-15 * pos)


def test_rope_invariants():
    rng = _rng(2)
    q, k = rng.normal(size=64), rng.normal(size=64)
    np.testing.assert_array_equal(O.rope(q, 0, 10000.0), q)
    for m in (1, 77, 131071):
        assert abs(np.linalg.norm(O.rope(q, m, 10000.0)) - np.linalg.norm(q)) < 1e-12
    # the score of a rotated pair depends only on the offset m - n
    ref = O.rope(q, 40, 10000.0) @ O.rope(k, 15, 10000.0)
    for shift in (1, 1000, 90000):
        got = O.rope(q, 40 + shift, 10000.0) @ O.rope(k, 15 + shift, 10000.0)
        assert abs(got - ref) < 1e-9 * max(1.0, abs(ref))


# ---------------------------------------------------------- cache sizes --
def test_cache_sizes_match_printed_numbers():
    g = json.load(open(os.path.join(GOLDEN, "cache_sizes.json")))
    d = g["full_model_dims"]
    nh, dh, dc, dr, layers = d["n_heads"], d["d_head"], d["d_latent"], d["d_rope"], d["layers"]
    assert O.mla_cache_elems_per_token(dc, dr) == g["mla_elems_per_token_per_layer"]["value"]
    assert O.mla_cache_elems_per_token(dc, dr, layers) == g["mla_elems_per_token_60_layers"]["value"]
    lat = g["latent_vs_per_head_kv_width"]
    assert nh * dh == lat["per_head_kv"] and lat["per_head_kv"] // dc == lat["ratio"]
    # GQA with g groups caches 2*g*d_h per token per layer
    assert O.mla_cache_elems_per_token(dc, dr) / (2 * dh) == g["gqa_equivalent_groups"]["value"]
    assert dr * 2 == dh
    mha = g["mha_elems_per_token_60_layers_printed"]
    assert O.mha_cache_elems_per_token(nh, dh, layers) == mha["formula_value"]
    assert abs(O.mha_cache_elems_per_token(nh, dh, layers) / O.mla_cache_elems_per_token(dc, dr, layers)
               - 56.888) < 1e-2


def test_cache_row_width_is_latent_plus_rope():
    rng = _rng(3)
    H, dc, dr = 24, 12, 6
    rows = O.latent_rows(rng.normal(size=(5, H)), rng.normal(size=(dc, H)),
                         rng.normal(size=(dr, H)), np.arange(5), 10000.0)
    assert rows.shape == (5, O.mla_cache_elems_per_token(dc, dr))


def test_latent_rows_brute_force():
    rng = _rng(4)
    H, dc, dr = 10, 6, 4
    h = rng.normal(size=(3, H))
    wd, wk = rng.normal(size=(dc, H)), rng.normal(size=(dr, H))
    rows = O.latent_rows(h, wd, wk, np.array([0, 5, 9]), 10000.0)
    for r, p in enumerate([0, 5, 9]):
        c = [sum(wd[a, b] * h[r, b] for b in range(H)) for a in range(dc)]
        k = [sum(wk[a, b] * h[r, b] for b in range(H)) for a in range(dr)]
        np.testing.assert_allclose(rows[r], np.concatenate([c, _complex_rope(k, p, 10000.0)]),
                                   rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- paging --
def test_page_slot_brute_force():
    page = 4
    bt = np.array([[5, 2, 0], [1, 4, 3]])
    expect = {}
    for b in range(2):
        for j in range(12):
            expect[(b, j)] = bt[b][j // page] * page + (j % page)
    for (b, j), slot in expect.items():
        assert O.page_slot(bt, b, j, page) == slot
    slots = sorted(expect.values())
    assert slots == list(range(24))          # the table covers every physical row once
    pool = np.full((6, page, 3), np.nan)
    for (b, j), slot in expect.items():
        pool.reshape(-1, 3)[slot] = [b, j, -j]
    for b in range(2):
        got = O.gather_rows(pool, bt, b, 11, page)
        np.testing.assert_array_equal(got[:, 0], b)
        np.testing.assert_array_equal(got[:, 1], np.arange(11))


# --------------------------------------------- MLA reduces to plain MHA --
def _mha_triple_loop(h_ctx, h_t, wq, wk, wv, wo, nh, dh, tau):
    L, H = h_ctx.shape
    q = [sum(wq[r, c] * h_t[c] for c in range(H)) for r in range(nh * dh)]
    k = [[sum(wk[r, c] * h_ctx[j, c] for c in range(H)) for r in range(nh * dh)] for j in range(L)]
    v = [[sum(wv[r, c] * h_ctx[j, c] for c in range(H)) for r in range(nh * dh)] for j in range(L)]
    o = []
    for i in range(nh):
        s = [tau * sum(q[i * dh + a] * k[j][i * dh + a] for a in range(dh)) for j in range(L)]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        z = sum(e)
        o += [sum(e[j] / z * v[j][i * dh + a] for j in range(L)) for a in range(dh)]
    return np.array([sum(wo[r, c] * o[c] for c in range(nh * dh)) for r in range(wo.shape[0])])


def _mha_as_mla(rng, H, nh, dh, dr):
    """MLA weights that make MLA equal MHA: d_c = 2 n_h d_h, W_DKV = [W_K; W_V],
    W_UK / W_UV select head i's K / V block, W_QR = 0 (RoPE channel adds 0)."""
    dc = 2 * nh * dh
    wq, wk, wv = (rng.normal(size=(nh * dh, H)) for _ in range(3))
    wo = rng.normal(size=(H, nh * dh))
    w_uk = np.zeros((nh * dh, dc))
    w_uv = np.zeros((nh * dh, dc))
    for r in range(nh * dh):
        w_uk[r, r] = 1.0
        w_uv[r, nh * dh + r] = 1.0
    mla = dict(w_q=wq, w_qr=np.zeros((nh * dr, H)), w_dkv=np.concatenate([wk, wv]),
               w_kr=rng.normal(size=(dr, H)), w_uk=w_uk, w_uv=w_uv, w_o=wo)
    return mla, (wq, wk, wv, wo), dc


@pytest.mark.parametrize("H,nh,dh,dr,L", [(6, 2, 3, 2, 5), (8, 3, 2, 4, 7), (5, 1, 4, 2, 1)])
def test_mla_reduces_to_mha(H, nh, dh, dr, L):
    rng = _rng(10 + L)
    mla, (wq, wk, wv, wo), dc = _mha_as_mla(rng, H, nh, dh, dr)
    h_ctx = rng.normal(size=(L, H))
    rows = O.latent_rows(h_ctx, mla["w_dkv"], mla["w_kr"], np.arange(L), 10000.0)
    tau = 1.0 / math.sqrt(dh + dr)
    for fn in (O.mla_decode_step, O.mla_decode_step_absorbed):
        out = fn(h_ctx[-1], rows, mla["w_q"], mla["w_qr"], mla["w_uk"], mla["w_uv"], mla["w_o"],
                 L - 1, nh, dh, dc, dr, 10000.0)
        ref = _mha_triple_loop(h_ctx, h_ctx[-1], wq, wk, wv, wo, nh, dh, tau)
        np.testing.assert_allclose(out["u"], ref, rtol=1e-10, atol=1e-10)


def test_mla_as_mha_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    rng = _rng(20)
    H, nh, dh, dr, L = 16, 4, 8, 4, 33
    mla, (wq, wk, wv, wo), dc = _mha_as_mla(rng, H, nh, dh, dr)
    h_ctx = rng.normal(size=(L, H))
    rows = O.latent_rows(h_ctx, mla["w_dkv"], mla["w_kr"], np.arange(L), 10000.0)
    out = O.mla_decode_step(h_ctx[-1], rows, mla["w_q"], mla["w_qr"], mla["w_uk"], mla["w_uv"],
                            mla["w_o"], L - 1, nh, dh, dc, dr, 10000.0)
    tau = 1.0 / math.sqrt(dh + dr)
    q = torch.tensor(wq @ h_ctx[-1]).view(1, nh, 1, dh)
    k = torch.tensor(h_ctx @ wk.T).view(1, L, nh, dh).transpose(1, 2).contiguous()
    v = torch.tensor(h_ctx @ wv.T).view(1, L, nh, dh).transpose(1, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=tau)
    ref = wo @ o.reshape(-1).numpy()
    np.testing.assert_allclose(out["u"], ref, rtol=1e-10, atol=1e-10)


def test_rope_channel_alone_is_mqa_with_shared_rotated_key():
    """W_UK = 0: the score is the RoPE channel only, one rotated key shared by all heads."""
    rng = _rng(30)
    H, nh, dh, dc, dr, L = 7, 3, 2, 5, 4, 6
    w = _weights(rng, H, nh, dh, dc, dr)
    w["w_uk"] = np.zeros_like(w["w_uk"])
    h_ctx = rng.normal(size=(L, H)) * 3.0
    rows = O.latent_rows(h_ctx, w["w_dkv"], w["w_kr"], np.arange(L), 10000.0)
    out = O.mla_decode_step(h_ctx[-1], rows, w["w_q"], w["w_qr"], w["w_uk"], w["w_uv"], w["w_o"],
                            L - 1, nh, dh, dc, dr, 10000.0)
    tau = 1.0 / math.sqrt(dh + dr)
    kr = [_complex_rope(w["w_kr"] @ h_ctx[j], j, 10000.0) for j in range(L)]
    c = [w["w_dkv"] @ h_ctx[j] for j in range(L)]
    o = []
    for i in range(nh):
        qr = _complex_rope(w["w_qr"][i * dr:(i + 1) * dr] @ h_ctx[-1], L - 1, 10000.0)
        s = [tau * float(qr @ kr[j]) for j in range(L)]
        e = [math.exp(x - max(s)) for x in s]
        v = [w["w_uv"][i * dh:(i + 1) * dh] @ c[j] for j in range(L)]
        o.append(sum(e[j] * v[j] for j in range(L)) / sum(e))
    np.testing.assert_allclose(out["u"], w["w_o"] @ np.concatenate(o), rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------ associativity --
@pytest.mark.parametrize("H,nh,dh,dc,dr,L", [(64, 4, 16, 32, 8, 64), (40, 3, 8, 24, 6, 19),
                                            (96, 2, 32, 128, 16, 130)])
def test_absorbed_equals_non_absorbed(H, nh, dh, dc, dr, L):
    rng = _rng(40 + L)
    w = _weights(rng, H, nh, dh, dc, dr)
    h_ctx = rng.normal(size=(L, H))
    rows = O.latent_rows(h_ctx, w["w_dkv"], w["w_kr"], np.arange(L), 10000.0)
    args = (h_ctx[-1], rows, w["w_q"], w["w_qr"], w["w_uk"], w["w_uv"], w["w_o"], L - 1,
            nh, dh, dc, dr, 10000.0)
    a, b = O.mla_decode_step(*args), O.mla_decode_step_absorbed(*args)
    np.testing.assert_allclose(b["u"], a["u"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(b["lse"], a["lse"], rtol=1e-12, atol=1e-12)
    # o_lat is the softmax-weighted latent; W_UV,i o_lat,i must be the per-head output
    per_head = np.stack([w["w_uv"][i * dh:(i + 1) * dh] @ b["o_lat"][i] for i in range(nh)])
    np.testing.assert_allclose(per_head, a["o"], rtol=1e-10, atol=1e-12)


def test_absorb_q_brute_force():
    rng = _rng(50)
    H, nh, dh, dc, dr = 6, 2, 3, 4, 2
    w = _weights(rng, H, nh, dh, dc, dr)
    h = rng.normal(size=H)
    q_lat, q_pe = O.absorb_q(h, w["w_q"], w["w_qr"], w["w_uk"], 9, nh, dh, dc, dr, 10000.0)
    for i in range(nh):
        qc = [sum(w["w_q"][i * dh + a, b] * h[b] for b in range(H)) for a in range(dh)]
        for cc in range(dc):
            ref = sum(w["w_uk"][i * dh + a, cc] * qc[a] for a in range(dh))
            assert abs(q_lat[i, cc] - ref) < 1e-12
        qr = [sum(w["w_qr"][i * dr + a, b] * h[b] for b in range(H)) for a in range(dr)]
        np.testing.assert_allclose(q_pe[i], _complex_rope(qr, 9, 10000.0), atol=1e-12)


# -------------------------------------------------- query compression --
@pytest.mark.parametrize("H,nh,dh,dc,dr,dcq,L", [(64, 4, 16, 32, 8, 24, 40), (48, 3, 8, 16, 4, 6, 9)])
def test_compressed_query_equals_the_composed_projection(H, nh, dh, dc, dr, dcq, L):
    """W_UQ (W_DQ h) = (W_UQ W_DQ) h: the compressed query path must reproduce the
    uncompressed one whose W_Q is the product of the two factors, through the
    absorbed query and the whole non-absorbed step (a transposed factor, a wrong
    head split of W_UQ or a RoPE query taken from c^Q instead of h all fail)."""
    rng = _rng(70 + L)
    w = _weights(rng, H, nh, dh, dc, dr)
    w_dq = rng.normal(size=(dcq, H)) / math.sqrt(H)
    w_uq = rng.normal(size=(nh * dh, dcq)) / math.sqrt(dcq)
    h_ctx = rng.normal(size=(L, H))
    rows = O.latent_rows(h_ctx, w["w_dkv"], w["w_kr"], np.arange(L), 10000.0)
    ql_c, qp_c = O.absorb_q(h_ctx[-1], None, w["w_qr"], w["w_uk"], L - 1, nh, dh, dc, dr, 10000.0,
                            w_dq=w_dq, w_uq=w_uq)
    ql, qp = O.absorb_q(h_ctx[-1], w_uq @ w_dq, w["w_qr"], w["w_uk"], L - 1, nh, dh, dc, dr,
                        10000.0)
    np.testing.assert_allclose(ql_c, ql, rtol=1e-11, atol=1e-12)
    np.testing.assert_array_equal(qp_c, qp)
    args = (h_ctx[-1], rows, None, w["w_qr"], w["w_uk"], w["w_uv"], w["w_o"], L - 1, nh, dh, dc,
            dr, 10000.0)
    a = O.mla_decode_step(*args, w_dq=w_dq, w_uq=w_uq)
    b = O.mla_decode_step(h_ctx[-1], rows, w_uq @ w_dq, *args[3:])
    np.testing.assert_allclose(a["u"], b["u"], rtol=1e-10, atol=1e-12)
    c = O.mla_decode_step_absorbed(*args, w_dq=w_dq, w_uq=w_uq)
    np.testing.assert_allclose(c["u"], a["u"], rtol=1e-10, atol=1e-12)


def test_compressed_query_rank_one_closed_form():
    """d_c' = 1: c^Q is the scalar w.h and q^C = (w.h) u, so q^C is a multiple of u."""
    rng = _rng(77)
    H, nh, dh = 10, 2, 3
    wd, u, h = rng.normal(size=(1, H)), rng.normal(size=(nh * dh, 1)), rng.normal(size=H)
    np.testing.assert_allclose(O.compressed_query(h, wd, u), float(wd[0] @ h) * u[:, 0],
                               rtol=1e-13, atol=1e-14)


def test_absorb_out_brute_force():
    rng = _rng(51)
    H, nh, dh, dc = 5, 3, 2, 4
    w_uv = rng.normal(size=(nh * dh, dc))
    w_o = rng.normal(size=(H, nh * dh))
    o_lat = rng.normal(size=(nh, dc))
    u = O.absorb_out(o_lat, w_uv, w_o, nh, dh, dc)
    o = [sum(w_uv[i * dh + a, c] * o_lat[i, c] for c in range(dc)) for i in range(nh) for a in range(dh)]
    ref = [sum(w_o[r, k] * o[k] for k in range(nh * dh)) for r in range(H)]
    np.testing.assert_allclose(u, ref, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ closed forms --
def test_single_token_context():
    """L = 1: the one weight is 1, o_lat = c_t, u = W_O blockdiag(W_UV) c_t."""
    rng = _rng(60)
    H, nh, dh, dc, dr = 12, 3, 4, 8, 4
    w = _weights(rng, H, nh, dh, dc, dr)
    h = rng.normal(size=(1, H))
    rows = O.latent_rows(h, w["w_dkv"], w["w_kr"], [0], 10000.0)
    out = O.mla_decode_step(h[0], rows, w["w_q"], w["w_qr"], w["w_uk"], w["w_uv"], w["w_o"], 0,
                            nh, dh, dc, dr, 10000.0)
    c = w["w_dkv"] @ h[0]
    np.testing.assert_allclose(out["u"], w["w_o"] @ (w["w_uv"] @ c), rtol=1e-12, atol=1e-12)


def test_zero_query_gives_uniform_average_and_identical_rows_give_the_row():
    rng = _rng(61)
    nh, dc, dr, L = 3, 8, 4, 9
    rows = rng.normal(size=(L, dc + dr))
    o, lse = O.attention_partials(np.zeros((nh, dc)), np.zeros((nh, dr)), rows, 1, dc, dr, 0.3, 4)
    np.testing.assert_allclose(o[0], np.tile(rows[:, :dc].mean(0), (nh, 1)), rtol=1e-12)
    np.testing.assert_allclose(lse[0], np.full(nh, math.log(L)), rtol=1e-12)
    same = np.tile(rows[:1], (L, 1))
    o, _ = O.attention_partials(rng.normal(size=(nh, dc)), rng.normal(size=(nh, dr)), same, 1,
                                dc, dr, 0.3, 4)
    np.testing.assert_allclose(o[0], np.tile(rows[0, :dc], (nh, 1)), rtol=1e-12)


# ------------------------------------------------------------ split / merge --
def test_split_bounds_partition():
    for L in (1, 63, 64, 65, 4096, 4097, 131072, 777):
        for S in (1, 2, 3, 8, 64):
            b = O.split_bounds(L, S, 64)
            assert len(b) == S and b[0][0] == 0 and b[-1][1] == L
            for (a0, a1), (b0, _) in zip(b, b[1:]):
                assert a1 == b0 and a0 <= a1
            for a0, a1 in b:
                assert a0 % 64 == 0 or a0 == L
    assert O.split_bounds(131072, 64, 64)[1] == (2048, 4096)


def test_split_merge_equals_whole_and_lse_is_logsumexp():
    sp = pytest.importorskip("scipy.special")
    rng = _rng(70)
    nh, dc, dr, L, tau = 4, 16, 8, 300, 0.2
    q_lat, q_pe = rng.normal(size=(nh, dc)) * 2, rng.normal(size=(nh, dr)) * 2
    rows = rng.normal(size=(L, dc + dr))
    scores = np.array([[tau * (q_lat[i] @ rows[j, :dc] + q_pe[i] @ rows[j, dc:]) for j in range(L)]
                       for i in range(nh)])
    ref_lse = sp.logsumexp(scores, axis=1)
    p = sp.softmax(scores, axis=1)
    ref_o = p @ rows[:, :dc]
    for S in (1, 2, 5, 16):
        o_s, l_s = O.attention_partials(q_lat, q_pe, rows, S, dc, dr, tau, 16)
        o, lse = O.merge_lse(o_s, l_s)
        np.testing.assert_allclose(o, ref_o, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-12)
        if S == 16:
            assert np.isneginf(l_s[-1]).all() and not o_s[-1].any()   # 300 rows fill 10 of 16 splits


def test_merge_lse_brute_force():
    rng = _rng(71)
    o_s = rng.normal(size=(3, 2, 5))
    l_s = np.array([[0.5, -np.inf], [2.0, 1.0], [-np.inf, 3.0]])
    o, lse = O.merge_lse(o_s, l_s)
    for i in range(2):
        ws = [math.exp(l_s[s, i]) if np.isfinite(l_s[s, i]) else 0.0 for s in range(3)]
        ref = sum(ws[s] * o_s[s, i] for s in range(3)) / sum(ws)
        np.testing.assert_allclose(o[i], ref, rtol=1e-12)
        assert abs(lse[i] - math.log(sum(ws))) < 1e-12


# ------------------------------------------------------------- FP8 cache --
def test_e4m3_table_matches_torch_float8():
    torch = pytest.importorskip("torch")
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_values()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert np.nanmax(got) == O.E4M3_MAX == 448.0


def test_e4m3_encode_matches_torch_cast_including_ties():
    torch = pytest.importorskip("torch")
    rng = _rng(80)
    x = np.concatenate([rng.normal(size=20000) * s for s in (1e-3, 0.05, 1.0, 30.0, 120.0)])
    x = x[np.abs(x) <= 448.0]
    fin = np.unique(O.e4m3_values()[np.isfinite(O.e4m3_values())])
    mids = (fin[1:] + fin[:-1]) / 2                          # exact ties
    x = np.concatenate([x, mids, -mids, [0.0, -0.0, 448.0, 2.0 ** -9, 2.0 ** -10]]).astype(np.float32)
    want = torch.tensor(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(x), want)


def test_fp8_scale_is_the_smallest_power_of_two_that_fits():
    rng = _rng(81)
    for amax in np.concatenate([np.exp(rng.uniform(-20, 20, 2000)), [448.0, 224.0, 448.0001, 1.0]]):
        e = O.fp8_row_scale_exponent(float(amax))
        assert amax / 2.0 ** e <= 448.0
        assert amax / 2.0 ** (e - 1) > 448.0                  # e - 1 would overflow the format
    assert O.fp8_row_scale_exponent(0.0) == 0


def test_bf16_bits_match_torch():
    torch = pytest.importorskip("torch")
    x = _rng(82).normal(size=5000).astype(np.float32) * 7.0
    want = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.bf16_bits(x), want)


def test_fp8_row_roundtrip_and_page_layout():
    rng = _rng(83)
    dc, dr = 32, 8
    rows = (rng.normal(size=(5, dc + dr)) * np.array([[1e-3], [1.0], [50.0], [0.0], [3.0]])).astype(np.float32)
    img = O.fp8_page_image(rows, dc, dr)
    assert img.size == O.fp8_page_bytes(5, dc, dr) == 5 * (dc + 2 * dr) + 20
    for r, row in enumerate(rows):
        codes, kr, e = O.fp8_quantize_row(row, dc)
        back = O.fp8_dequantize_row(codes, kr, e)
        # every latent value lands on the nearest multiple of its e4m3 spacing
        spacing = np.ldexp(2.0 ** (np.maximum(np.floor(np.log2(np.maximum(np.abs(row[:dc]) / 2.0 ** e, 2.0 ** -6))), -6) - 3), e)
        assert np.all(np.abs(back[:dc] - row[:dc]) <= spacing / 2 + 1e-30)
        np.testing.assert_allclose(back[dc:], row[dc:], rtol=2.0 ** -8)
        assert img[5 * (dc + 2 * dr) + 4 * r:5 * (dc + 2 * dr) + 4 * r + 4].view(np.float32)[0] == 2.0 ** e
    assert O.fp8_page_bytes(64, 512, 64) == 41216


# ---------------------------------------------------------------- prefill --
def test_prefill_of_mha_as_mla_is_causally_masked_sdpa():
    """A prompt chunk through the prefill definition equals causally masked
    attention computed by torch's scaled_dot_product_attention on the plain MHA
    the weights encode (token t of the chunk sees cache rows 0..P+t)."""
    torch = pytest.importorskip("torch")
    rng = _rng(60)
    H, nh, dh, dr, P, T = 12, 3, 4, 2, 5, 7
    mla, (wq, wk, wv, wo), dc = _mha_as_mla(rng, H, nh, dh, dr)
    h_all = rng.normal(size=(P + T, H))
    rows_before = O.latent_rows(h_all[:P], mla["w_dkv"], mla["w_kr"], np.arange(P), 10000.0)
    out = O.mla_prefill_step(h_all[P:], rows_before, mla["w_q"], mla["w_qr"], mla["w_dkv"],
                             mla["w_kr"], mla["w_uk"], mla["w_uv"], mla["w_o"], nh, dh, dc, dr,
                             10000.0)
    tau = 1.0 / math.sqrt(dh + dr)
    q = torch.tensor(h_all[P:] @ wq.T).view(1, T, nh, dh).transpose(1, 2).contiguous()
    k = torch.tensor(h_all @ wk.T).view(1, P + T, nh, dh).transpose(1, 2).contiguous()
    v = torch.tensor(h_all @ wv.T).view(1, P + T, nh, dh).transpose(1, 2).contiguous()
    allowed = torch.arange(P + T)[None, :] <= (P + torch.arange(T))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=allowed, scale=tau)
    ref = o.transpose(1, 2).reshape(T, nh * dh).numpy() @ wo.T
    np.testing.assert_allclose(out["u"], ref, rtol=1e-10, atol=1e-10)


def test_prefill_chunks_compose_and_match_the_partials():
    """Two chunks in turn give the same outputs as one chunk of both; each token's
    split partials, merged, give its absorbed output (the attention call's
    contract, checked against the step)."""
    rng = _rng(61)
    H, nh, dh, dc, dr, P, T = 20, 2, 8, 12, 4, 70, 9
    w = _weights(rng, H, nh, dh, dc, dr)
    h_all = rng.normal(size=(P + T, H))
    rows_before = O.latent_rows(h_all[:P], w["w_dkv"], w["w_kr"], np.arange(P), 10000.0)
    args = (w["w_q"], w["w_qr"], w["w_dkv"], w["w_kr"], w["w_uk"], w["w_uv"], w["w_o"], nh, dh, dc,
            dr, 10000.0)
    whole = O.mla_prefill_step(h_all[P:], rows_before, *args)
    first = O.mla_prefill_step(h_all[P:P + 4], rows_before, *args)
    rows_mid = O.latent_rows(h_all[:P + 4], w["w_dkv"], w["w_kr"], np.arange(P + 4), 10000.0)
    second = O.mla_prefill_step(h_all[P + 4:], rows_mid, *args)
    np.testing.assert_allclose(np.concatenate([first["u"], second["u"]]), whole["u"], rtol=1e-12,
                               atol=1e-13)
    rows = O.latent_rows(h_all, w["w_dkv"], w["w_kr"], np.arange(P + T), 10000.0)
    tau = 1.0 / math.sqrt(dh + dr)
    q = [O.absorb_q(h_all[P + t], w["w_q"], w["w_qr"], w["w_uk"], P + t, nh, dh, dc, dr, 10000.0)
         for t in range(T)]
    parts = O.prefill_attention_partials(np.stack([x[0] for x in q]), np.stack([x[1] for x in q]),
                                         rows, np.arange(P, P + T), 3, dc, dr, tau, 16)
    for t, (o_s, l_s) in enumerate(parts):
        o_lat, lse = O.merge_lse(o_s, l_s)
        np.testing.assert_allclose(lse, whole["lse"][t], rtol=1e-12, atol=1e-12)
        per_head = np.stack([w["w_uv"][i * dh:(i + 1) * dh] @ o_lat[i] for i in range(nh)])
        np.testing.assert_allclose(per_head, whole["o"][t], rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------- YaRN --
# [Report] §3.3 (the long-context paragraph) gives YaRN's parameters for the
# 4K -> 128K extension: scale 40, alpha 1, beta 32; the method is the published
# one (oracle.Yarn).  These pins fix it by its limit case, by where the published
# ramp must put the 64-wide RoPE branch's pairs, by position interpolation on the
# stretched pairs and by its temperature's closed form.
YARN_4K = dict(base=10000.0, scale=40.0, orig_len=4096, alpha=1.0, beta=32.0)


def test_yarn_with_scale_one_is_plain_rope():
    y = O.Yarn(10000.0, 1.0, 4096, 1.0, 32.0)
    np.testing.assert_array_equal(O.rope_theta(64, y), O.rope_theta(64, 10000.0))
    x = _rng(40).standard_normal((5, 64))
    np.testing.assert_array_equal(O.rope(x, np.arange(5) * 977, y), O.rope(x, np.arange(5) * 977, 10000.0))
    assert O.yarn_logit_factor(y) == 1.0 and O.yarn_logit_factor(10000.0) == 1.0


def test_yarn_frequency_split_of_the_4k_to_128k_extension():
    """d_R = 64, base 10000: theta_k = 10^(-k/8).  Pair k turns
    r_k = 4096 theta_k / (2 pi) times over the 4K window: r_10 = 36.6 > beta = 32
    and r_11 = 27.5 < 32, r_22 = 1.16 > alpha = 1 and r_23 = 0.87 < 1.  So pairs
    0..10 keep their frequency, pairs 23..31 are divided by the scale 40 (their
    wavelength stretched 40x, as position interpolation does), and 11..22 lie
    strictly between, the stretch growing with k."""
    plain = O.rope_theta(64, 10000.0)
    yarn = O.rope_theta(64, O.Yarn(**YARN_4K))
    np.testing.assert_array_equal(yarn[:11], plain[:11])
    np.testing.assert_allclose(yarn[23:], plain[23:] / 40.0, rtol=1e-15)
    ratio = yarn[11:23] / plain[11:23]
    assert np.all(ratio < 1.0) and np.all(ratio > 1.0 / 40.0)
    assert np.all(np.diff(ratio) < 0)


def test_yarn_stretched_pairs_are_position_interpolation():
    """On the pairs the ramp leaves fully interpolated (k >= 23 above), rotating at
    position s*m with YaRN equals plain RoPE at position m."""
    x = np.zeros((3, 64))
    x[:, 46:] = _rng(41).standard_normal((3, 18))            # pairs 23..31 only
    m = np.array([1, 777, 3000])
    got = O.rope(x, 40 * m, O.Yarn(**YARN_4K))
    np.testing.assert_allclose(got, O.rope(x, m, 10000.0), atol=1e-12)


def test_yarn_keeps_rope_a_relative_rotation():
    y = O.Yarn(**YARN_4K)
    rng = _rng(42)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for m, n in ((5, 2), (130000, 4096), (70000, 69999)):
        a = O.rope(q, m, y) @ O.rope(k, n, y)
        b = O.rope(q, m + 12345, y) @ O.rope(k, n + 12345, y)
        assert abs(a - b) < 1e-9
    np.testing.assert_allclose(np.linalg.norm(O.rope(q, 99999, y)), np.linalg.norm(q), rtol=1e-13)


def test_yarn_temperature_closed_form():
    """sqrt(1/t) = 0.1 ln s + 1: at s = e^10 the logits double twice (1/t = 4);
    at s = 40, 1/t = (1 + 0.1 ln 40)^2 = 1.3688879^2 = 1.8738542..."""
    assert abs(O.yarn_logit_factor(O.Yarn(10000.0, math.exp(10.0), 4096, 1, 32)) - 4.0) < 1e-12
    assert abs(O.yarn_logit_factor(O.Yarn(**YARN_4K)) - 1.8738542071) < 1e-9


def test_yarn_step_absorbed_equals_non_absorbed_and_scales_the_logits():
    """Associativity still holds with the stretched RoPE; and with W_UK = 0 the
    scores are tau/t q^R . k^R, so the lse of a one-token context is that score."""
    H, nh, dh, dc, dr, L = 16, 2, 4, 8, 8, 9
    rng = _rng(43)
    w = _weights(rng, H, nh, dh, dc, dr)
    y = O.Yarn(10000.0, 8.0, 4, 1.0, 4.0)
    h_ctx = rng.standard_normal((L, H))
    rows = O.latent_rows(h_ctx, w["w_dkv"], w["w_kr"], np.arange(L), y)
    args = (h_ctx[-1], rows, w["w_q"], w["w_qr"], w["w_uk"], w["w_uv"], w["w_o"], L - 1, nh, dh,
            dc, dr, y)
    a = O.mla_decode_step_absorbed(*args)
    d = O.mla_decode_step(*args)
    np.testing.assert_allclose(a["u"], d["u"], rtol=1e-10, atol=1e-12)
    one = O.mla_decode_step(h_ctx[0], rows[:1], w["w_q"], w["w_qr"], 0 * w["w_uk"], w["w_uv"],
                            w["w_o"], 0, nh, dh, dc, dr, y)
    qr = (w["w_qr"] @ h_ctx[0]).reshape(nh, dr)              # position 0: no rotation
    want = O.yarn_logit_factor(y) / math.sqrt(dh + dr) * (qr @ rows[0, dc:])
    np.testing.assert_allclose(one["lse"], want, rtol=1e-12)
