"""FP8 latent pool: row quantization, append, attention and the decode step
against the fp64 oracle.

The quantizer is checked byte for byte against the oracle's page format on
seeded rows and on rows built to reach the format's corner cases (zero rows,
exact powers of two, round-to-nearest-even ties, very small and very large
rows).  Attention and the step compare with the oracle run on the oracle's own
dequantization of the same seeded fp32 rows.
"""
import functools

import numpy as np
import pytest

import mla_latent_kv_dkv_amd as M
import oracle as O
from mla_latent_kv_dkv_amd import inputs as I
from mla_latent_kv_dkv_amd.harness import DeviceWorkload, fill_fp8_pool
from tests.gpu_util import assert_parity, host_tensor, device_tensor, note, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PATHS = [0, 1]
SENTINEL = 0xA5


@pytest.fixture(autouse=True)
def _path_reset():
    M.load()
    yield
    M.mla_set_kernel_path(0)


def _wl(name, **kw):
    fields = dict(I.WORKLOADS[name].__dict__)
    fields.update(kw)
    return I.Workload(**fields)


def _dims(w):
    return M.make_dims(w.hidden, w.n_heads, w.d_head, w.d_latent, w.d_rope, w.dtype, w.page_size,
                       w.rope_base)


def _row_image(row_f32, d_c):
    """Oracle bytes of one row slot and of its scale."""
    codes, kr, e = O.fp8_quantize_row(row_f32, d_c)
    return np.concatenate([codes, kr.view(np.uint8)]), np.array([2.0 ** e], np.float32).view(np.uint8)


def _special_rows(d_c, d_R):
    """Rows at the corners of the format (d_c >= 32, d_R >= 8)."""
    out = []
    z = np.zeros(d_c + d_R, np.float32)
    out.append(z.copy())                                     # all zero: scale 1, codes 0
    r = z.copy()                                             # amax 448 exactly: scale 1
    vals = [448.0, 1.0625, 1.1875, -2.125, 2.0 ** -10, 3 * 2.0 ** -10, -5 * 2.0 ** -10,
            0.5 + 2.0 ** -5, 240.0, -416.0, 2.0 ** -9, 13 * 2.0 ** -11, 7 * 2.0 ** -11]
    r[:len(vals)] = vals                                     # e4m3 ties (to even) and subnormals
    r[d_c:d_c + 4] = [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3.0]   # bf16 ties
    out.append(r)
    r = z.copy()
    r[0] = np.float32(448.0 * 8) * np.float32(1 + 2.0 ** -20)  # just over 448*2^3: scale 2^4
    r[1] = -3.0
    out.append(r)
    r = z.copy()
    r[3] = -448.0 * 2.0 ** -5                                # amax exactly 448*2^-5: scale 2^-5
    r[4] = 0.1
    out.append(r)
    for mag in (1e-30, 3e37):                                # far from 1 both ways
        out.append((np.linspace(-1, 1, d_c + d_R) * mag).astype(np.float32))
    return np.stack(out)


def _seeded_rows(n, d_c, d_R, seed):
    """n seeded rows, row r scaled by 2^(r % 41 - 20) (many scale exponents)."""
    v = I.normal_f32(I.stream_key(seed, "fp8_rows"), 0, n * (d_c + d_R)).reshape(n, d_c + d_R)
    return (v * np.ldexp(1.0, (np.arange(n) % 41 - 20))[:, None]).astype(np.float32)


def _fp8_rows(rows, d_c):
    """The oracle's dequantization of rows (each first rounded to fp32, the format's input)."""
    return np.stack([O.fp8_dequantize_row(*O.fp8_quantize_row(r, d_c)) for r in rows])


# ------------------------------------------------------------- quantize --
QUANT_CASES = [("full-fp8", 64), ("tiny-fp8", 16), ("tiny-fp8", 1)]


@pytest.mark.parametrize("name,page", QUANT_CASES)
def test_quantize_rows_bytes_match_the_format(name, page):
    w = _wl(name, page_size=page)
    d = _dims(w)
    dc, dr = w.d_latent, w.d_rope
    pb = M.mla_fp8_page_bytes(d)
    rb = dc + 2 * dr
    assert pb == O.fp8_page_bytes(page, dc, dr)
    pages = 3 if page > 1 else 40
    n_slots = pages * page
    special = _special_rows(dc, dr)
    rows = np.concatenate([special, _seeded_rows(n_slots, dc, dr, w.seed)])[:n_slots - min(5, page - 1)]
    n = len(rows)
    rng = np.random.default_rng(11)
    order = rng.permutation(n)                          # rows enqueued in scrambled order
    bt = rng.permutation(pages).astype(np.int32)[None]  # one sequence over permuted pages
    note(f"quantize {name} page={page} rows={n}")
    pool = torch.full((pages, pb), SENTINEL, dtype=torch.uint8, device="cuda")
    dev_rows = torch.tensor(rows[order], device="cuda")
    M.mla_quantize_rows_fp8(d, dev_rows, torch.zeros(n, dtype=torch.int32, device="cuda"),
                            torch.tensor(order.astype(np.int32), device="cuda"),
                            torch.tensor(bt, device="cuda"), pool)
    got = pool.cpu().numpy()
    want = np.full((pages, pb), SENTINEL, np.uint8)
    for j in range(n):
        pg, slot = bt[0, j // page], j % page
        img, sc = _row_image(rows[j], dc)
        want[pg, slot * rb:(slot + 1) * rb] = img
        want[pg, page * rb + 4 * slot:page * rb + 4 * slot + 4] = sc
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at (page, byte) {bad[0].tolist()}"
    # the oracle's whole-page image agrees for the (full) first page
    np.testing.assert_array_equal(got[bt[0, 0]], O.fp8_page_image(rows[:page], dc, dr))
    assert M.mla_device_error() == 0


def test_quantize_rows_out_of_range_rows_write_nothing():
    w = _wl("tiny-fp8", page_size=16)
    d = _dims(w)
    pb = M.mla_fp8_page_bytes(d)
    pool = torch.full((2, pb), SENTINEL, dtype=torch.uint8, device="cuda")
    rows = torch.ones((3, w.row), dtype=torch.float32, device="cuda")
    bt = torch.tensor([[0, 9]], dtype=torch.int32, device="cuda")      # page 9 does not exist
    note("quantize bad rows")
    M.mla_device_error(clear=True)
    M.mla_quantize_rows_fp8(d, rows, torch.tensor([0, 0, 3], dtype=torch.int32, device="cuda"),
                            torch.tensor([20, 40, 0], dtype=torch.int32, device="cuda"), bt, pool)
    err = M.mla_device_error(clear=True)
    assert err & 1 and err & 2 and err & 4      # bad page (20), position (40), sequence (3)
    assert (pool.cpu().numpy() == SENTINEL).all()


# --------------------------------------------------------------- append --
def _assert_codes_near(got_img, ref_row, dc, dr, what):
    """Bytes of an appended row vs the oracle's fp64 row.  The row's scale must be
    the oracle's; a code may differ from the oracle's only by one step, where the
    oracle's scaled value lies within the GPU projection's fp32 rounding of the
    midpoint between the two codes; k^R within bf16 rounding."""
    vals = O.e4m3_values()
    codes, kr_bits, e = O.fp8_quantize_row(ref_row, dc)
    rb = dc + 2 * dr
    g_codes = got_img[:rb][:dc]
    g_scale = got_img[rb:rb + 4].view(np.float32)[0]
    assert g_scale == np.float32(2.0 ** e), f"{what}: scale {g_scale} != 2^{e}"
    diff = np.flatnonzero(g_codes != codes)
    if diff.size:
        x = np.ldexp(np.asarray(ref_row[:dc], np.float64), -e)[diff]
        g, r = g_codes[diff].astype(int), codes[diff].astype(int)
        gv, rv = vals[g], vals[r]
        amax = np.abs(np.ldexp(np.asarray(ref_row[:dc], np.float64), -e)).max()
        gi, ri = g & 0x7F, r & 0x7F          # neighbours: same sign one code apart, or around 0
        adjacent = (np.abs(gi - ri) == 1) & (((g >> 7) == (r >> 7)) | (gi == 0) | (ri == 0))
        assert adjacent.all(), f"{what}: a code moved more than one step"
        mid = 0.5 * (gv + rv)
        assert np.all(np.abs(x - mid) <= 1e-5 * amax), f"{what}: code differs away from a tie"
        assert diff.size <= max(2, dc // 50), f"{what}: {diff.size} codes differ"
    g_kr = (got_img[dc:rb].view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    ref_kr = np.asarray(ref_row[dc:], np.float64)
    assert np.all(np.abs(g_kr - ref_kr) <= 2.0 ** -8 * np.abs(ref_kr) + 1e-6 * np.abs(ref_kr).max()
                  ), f"{what}: k^R beyond bf16 rounding"
    return diff.size


@pytest.mark.parametrize("name", ["tiny-fp8", "full-fp8"])
@pytest.mark.parametrize("path", PATHS)
def test_append_latent_fp8(name, path):
    w = _wl(name, batch=3)
    M.mla_set_kernel_path(path)
    d = _dims(w)
    lens = np.array([5, 130, 64], dtype=np.int32) if name == "tiny-fp8" else np.array(
        [70, 200, 64], dtype=np.int32)
    bt, total = I.page_table(w, lens)
    rng = np.random.default_rng(5)
    seqs = np.concatenate([np.full(l, b) for b, l in enumerate(lens)]).astype(np.int32)
    poss = np.concatenate([np.arange(l) for l in lens]).astype(np.int32)
    sel = rng.permutation(len(seqs))[:97]
    seqs, poss = seqs[sel], poss[sel]
    n = len(sel)
    note(f"append fp8 {name} path={path} rows={n}")
    std = 1 / np.sqrt(w.hidden)
    h = device_tensor(torch, w, "h_rows", (n, w.hidden))
    wd = device_tensor(torch, w, "w_dkv", (w.d_latent, w.hidden), std)
    wk = device_tensor(torch, w, "w_kr", (w.d_rope, w.hidden), std)
    pb = M.mla_fp8_page_bytes(d)
    pool = torch.full((total, pb), SENTINEL, dtype=torch.uint8, device="cuda")
    M.mla_append_latent_fp8(d, h, wd, wk, torch.tensor(seqs, device="cuda"),
                            torch.tensor(poss, device="cuda"), torch.tensor(bt, device="cuda"), pool)
    got = pool.cpu().numpy()
    ref = O.latent_rows(host_tensor(w, "h_rows", (n, w.hidden)),
                        host_tensor(w, "w_dkv", (w.d_latent, w.hidden), std),
                        host_tensor(w, "w_kr", (w.d_rope, w.hidden), std), poss, w.rope_base)
    P, rb = w.page_size, w.d_latent + 2 * w.d_rope
    written = np.zeros((total, pb), bool)
    flips = 0
    for r in range(n):
        pg, slot = bt[seqs[r], poss[r] // P], poss[r] % P
        img = np.concatenate([got[pg, slot * rb:(slot + 1) * rb], got[pg, P * rb + 4 * slot:P * rb + 4 * slot + 4]])
        flips += _assert_codes_near(img, ref[r], w.d_latent, w.d_rope, f"row {r}")
        written[pg, slot * rb:(slot + 1) * rb] = True
        written[pg, P * rb + 4 * slot:P * rb + 4 * slot + 4] = True
    note(f"  codes at a tie resolved the other way: {flips} of {n * w.d_latent}")
    assert (got[~written] == SENTINEL).all(), "bytes outside the written slots changed"
    assert M.mla_device_error() == 0


# ------------------------------------------------ fused query + FP8 append --
def _fused_fp8_case(w, B, lens, seqs, poss, bt, total):
    """Run mla_absorb_q_append_fp8 on seeded weights; return the pool bytes, the
    queries, mla_absorb_q's queries and the host operands."""
    sh = {n: w.weight_shape(n) for n in ("w_q", "w_qr", "w_uk", "w_dkv", "w_kr")}
    std = {n: 1 / np.sqrt(w.fan_in(n)) for n in sh}
    dev = {n: device_tensor(torch, w, n, sh[n], std[n]) for n in sh}
    h = device_tensor(torch, w, "h_q", (B, w.hidden))
    d = _dims(w)
    ws = torch.empty(M.mla_absorb_q_append_fp8_workspace_bytes(d, B), dtype=torch.uint8,
                     device="cuda")
    q_lat = torch.empty((B, w.n_heads, w.d_latent), dtype=torch.float32, device="cuda")
    q_pe = torch.empty((B, w.n_heads, w.d_rope), dtype=torch.float32, device="cuda")
    pool = torch.full((total, M.mla_fp8_page_bytes(d)), SENTINEL, dtype=torch.uint8, device="cuda")
    pos_t = torch.tensor(poss, device="cuda")
    M.mla_absorb_q_append_fp8(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], dev["w_dkv"],
                              dev["w_kr"], pos_t, torch.tensor(seqs, device="cuda"),
                              torch.tensor(bt, device="cuda"), pool, q_lat, q_pe, ws)
    q_lat2, q_pe2 = torch.empty_like(q_lat), torch.empty_like(q_pe)
    ws2 = torch.empty(M.mla_workspace_bytes(d, B), dtype=torch.uint8, device="cuda")
    M.mla_absorb_q(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], pos_t, q_lat2, q_pe2, ws2)
    hh = host_tensor(w, "h_q", (B, w.hidden))
    hw = {n: host_tensor(w, n, sh[n], std[n]) for n in sh}
    return pool.cpu().numpy(), (q_lat, q_pe), (q_lat2, q_pe2), hh, hw


def _check_appended(w, got, bt, total, seqs, poss, ref_rows, rows):
    """Each row in `rows` at its slot near the oracle's row; every other byte untouched."""
    P, rb, pb = w.page_size, w.d_latent + 2 * w.d_rope, got.shape[1]
    written = np.zeros((total, pb), bool)
    flips = 0
    for r in rows:
        pg, slot = bt[seqs[r], poss[r] // P], poss[r] % P
        img = np.concatenate([got[pg, slot * rb:(slot + 1) * rb],
                              got[pg, P * rb + 4 * slot:P * rb + 4 * slot + 4]])
        flips += _assert_codes_near(img, ref_rows[r], w.d_latent, w.d_rope, f"row {r}")
        written[pg, slot * rb:(slot + 1) * rb] = True
        written[pg, P * rb + 4 * slot:P * rb + 4 * slot + 4] = True
    assert (got[~written] == SENTINEL).all(), "bytes outside the appended slots changed"
    return flips


# full-fp8 B = 5: the K-split product and its finish pass; B = 64: the largest batch of
# the fused weight stream; B = 65 and tiny-fp8 (fp32): the two separate calls;
# B = 256: the fused tiled product; lite-fp8 B = 32: 4 K slices; lite-fp8 with a
# 512-wide hidden state: one K slice (rows straight from the product's epilogue)
@pytest.mark.parametrize("name,B,hidden", [("full-fp8", 5, 0), ("full-fp8", 64, 0),
                                           ("full-fp8", 65, 0), ("full-fp8", 256, 0),
                                           ("lite-fp8", 32, 0), ("lite-fp8", 32, 512),
                                           ("tiny-fp8", 5, 0)])
def test_absorb_q_append_fp8(name, B, hidden):
    """The fused query + FP8 append: queries equal to mla_absorb_q's bit for bit and
    at the oracle's bar; each appended row quantized as the oracle quantizes its
    fp64 row (scale equal, codes equal up to a tie within fp32 rounding, k^R
    within bf16 rounding); the rest of the pool untouched."""
    w = _wl(name, batch=B, **({"hidden": hidden} if hidden else {}))
    note(f"absorb_q_append_fp8 {name} B={B} hidden={w.hidden}")
    # token b at lens[b] - 1; the 256-row batch stays under 300 tokens (a small pool)
    lens = np.array([3 + 37 * b if B <= 64 else 1 + (37 * b) % 300 for b in range(B)],
                    dtype=np.int32)
    bt, total = I.page_table(w, lens)
    seqs = np.arange(B, dtype=np.int32)
    poss = (lens - 1).astype(np.int32)
    M.mla_device_error(clear=True)
    got, q, q2, hh, hw = _fused_fp8_case(w, B, lens, seqs, poss, bt, total)
    assert torch.equal(q[0], q2[0]) and torch.equal(q[1], q2[1]), "queries differ from mla_absorb_q"
    # every row bit for bit against mla_absorb_q; every 8th (and the last) of a
    # 256-row batch against the fp64 oracle
    rows = list(range(B)) if B <= 64 else sorted(set(range(0, B, 8)) | {B - 1})
    rl, rp = zip(*[O.absorb_q(hh[b], hw["w_q"], hw["w_qr"], hw["w_uk"], int(poss[b]), w.n_heads,
                              w.d_head, w.d_latent, w.d_rope, w.rope_base) for b in rows])
    assert_parity(to_np(q[0])[rows], np.stack(rl), w.dtype, "q_lat")
    assert_parity(to_np(q[1])[rows], np.stack(rp), w.dtype, "q_pe")
    ref_rows = O.latent_rows(hh, hw["w_dkv"], hw["w_kr"], poss, w.rope_base)
    flips = _check_appended(w, got, bt, total, seqs, poss, ref_rows, range(B))
    note(f"  codes at a tie resolved the other way: {flips} of {B * w.d_latent}")
    assert M.mla_device_error() == 0


@pytest.mark.parametrize("B", [5, 64, 256])
def test_absorb_q_append_fp8_out_of_range_rows(B):
    """A row whose table entry is outside the pool and one whose sequence is
    outside the table: neither is written, the error word names both, and the
    queries are still mla_absorb_q's (B = 256: the fused tiled product)."""
    w = _wl("full-fp8", batch=B)
    note(f"absorb_q_append_fp8 out-of-range rows B={B}")
    lens = np.array([3 + 37 * b if B <= 64 else 1 + (37 * b) % 300 for b in range(B)],
                    dtype=np.int32)
    bt, total = I.page_table(w, lens)
    seqs = np.arange(B, dtype=np.int32)
    poss = (lens - 1).astype(np.int32)
    bt[1, poss[1] // w.page_size] = total + 3
    seqs[3] = B + 9
    M.mla_device_error(clear=True)
    got, q, q2, hh, hw = _fused_fp8_case(w, B, lens, seqs, poss, bt, total)
    err = M.mla_device_error(clear=True)
    assert err & 1 and err & 4, err
    assert torch.equal(q[0], q2[0]) and torch.equal(q[1], q2[1])
    ref_rows = O.latent_rows(hh, hw["w_dkv"], hw["w_kr"], poss, w.rope_base)
    _check_appended(w, got, bt, total, seqs, poss, ref_rows,
                    [b for b in range(B) if b not in (1, 3)])


def test_absorb_q_append_fp8_misaligned_input_falls_back():
    """h starting 2 bytes past a 16-byte boundary: the fused product cannot take
    it, so the call makes mla_absorb_q and mla_append_latent_fp8 in turn and gives
    their results byte for byte."""
    w = _wl("full-fp8", batch=8)
    B = 8
    lens = np.array([100 + 9 * b for b in range(B)], dtype=np.int32)
    bt, total = I.page_table(w, lens)
    poss = (lens - 1).astype(np.int32)
    note("absorb_q_append_fp8 misaligned h")
    sh = {n: w.weight_shape(n) for n in ("w_q", "w_qr", "w_uk", "w_dkv", "w_kr")}
    std = {n: 1 / np.sqrt(w.fan_in(n)) for n in sh}
    dev = {n: device_tensor(torch, w, n, sh[n], std[n]) for n in sh}
    h_al = device_tensor(torch, w, "h_q", (B, w.hidden))
    flat = torch.empty(B * w.hidden + 1, dtype=h_al.dtype, device="cuda")
    h = flat[1:].view(B, w.hidden)
    h.copy_(h_al)
    assert h.data_ptr() % 16 == 2 and h.is_contiguous()
    d = _dims(w)
    ws = torch.empty(M.mla_absorb_q_append_fp8_workspace_bytes(d, B), dtype=torch.uint8,
                     device="cuda")
    pos_t = torch.tensor(poss, device="cuda")
    seq_t = torch.arange(B, dtype=torch.int32, device="cuda")
    bt_t = torch.tensor(bt, device="cuda")
    outs = []
    for fused in (True, False):
        q_lat = torch.empty((B, w.n_heads, w.d_latent), dtype=torch.float32, device="cuda")
        q_pe = torch.empty((B, w.n_heads, w.d_rope), dtype=torch.float32, device="cuda")
        pool = torch.full((total, M.mla_fp8_page_bytes(d)), SENTINEL, dtype=torch.uint8,
                          device="cuda")
        if fused:
            M.mla_absorb_q_append_fp8(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], dev["w_dkv"],
                                      dev["w_kr"], pos_t, seq_t, bt_t, pool, q_lat, q_pe, ws)
        else:
            M.mla_absorb_q(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], pos_t, q_lat, q_pe, ws)
            M.mla_append_latent_fp8(d, h, dev["w_dkv"], dev["w_kr"], seq_t, pos_t, bt_t, pool)
        outs.append((q_lat, q_pe, pool))
    for x, y in zip(outs[0], outs[1]):
        assert torch.equal(x, y)
    assert M.mla_device_error() == 0


# ------------------------------------------------------------ attention --
@functools.lru_cache(maxsize=None)
def _deq_rows(name, page, lens, b):
    """Oracle dequantization of the seeded fp32 rows of sequence b."""
    w = _wl(name, batch=len(lens), page_size=page)
    bt, _ = I.page_table(w, np.array(lens, dtype=np.int32))
    return _fp8_rows(I.pool_rows(w, bt, b, lens[b], f32=True), w.d_latent)


ATTN_CASES = [
    ("tiny-fp8", (1, 64, 100, 129), 3, 16),
    ("lite-fp8", (64, 777, 4096), 2, 64),
    ("full-fp8", (1, 65, 1000, 4096), 4, 64),
    ("full-fp8", (100, 37, 4097), 3, 64),      # partial tiles in the middle of splits
    ("full-fp8", (3000, 130), 8, 64),
    ("full-fp8", (2,), 5, 64),                 # most splits empty
    ("full-fp8", (33000,), 1, 64),             # one split over 516 pages: page-id window reloads
]


def _attn_inputs(w, lens, page):
    bt, total = I.page_table(w, np.array(lens, dtype=np.int32))
    B, nh = len(lens), w.n_heads
    q_lat = device_tensor(torch, w, "q_lat_in", (B, nh, w.d_latent), 0.5).float().contiguous()
    q_pe = device_tensor(torch, w, "q_pe_in", (B, nh, w.d_rope), 1.0).float().contiguous()
    d = _dims(w)
    pool = torch.empty((total, M.mla_fp8_page_bytes(d)), dtype=torch.uint8, device="cuda")
    fill_fp8_pool(d, pool, I.stream_key(w.seed, "pool"))
    hq = host_tensor(w, "q_lat_in", (B, nh, w.d_latent), 0.5)
    hp = host_tensor(w, "q_pe_in", (B, nh, w.d_rope), 1.0)
    return d, bt, q_lat, q_pe, pool, hq, hp


@pytest.mark.parametrize("name,lens,S,page", ATTN_CASES)
@pytest.mark.parametrize("path", PATHS)
def test_decode_attention_fp8(name, lens, S, page, path):
    w = _wl(name, batch=len(lens), page_size=page)
    M.mla_set_kernel_path(path)
    note(f"attention fp8 {name} lens={list(lens)} S={S} page={page} path={path}")
    d, bt, q_lat, q_pe, pool, hq, hp = _attn_inputs(w, lens, page)
    B, nh = len(lens), w.n_heads
    o_part = torch.full((B, S, nh, w.d_latent), 123.0, device="cuda")
    lse_part = torch.full((B, S, nh), 123.0, device="cuda")
    M.mla_decode_attention_fp8(d, q_lat, q_pe, pool, torch.tensor(bt, device="cuda"),
                               torch.tensor(np.array(lens, dtype=np.int32), device="cuda"), o_part,
                               lse_part)
    got_o, got_l = to_np(o_part), to_np(lse_part)
    tau = M.default_scale(d)
    for b in range(B):
        rows = _deq_rows(name, page, lens, b)
        ro, rl = O.attention_partials(hq[b], hp[b], rows, S, w.d_latent, w.d_rope, tau, page)
        assert_parity(got_o[b], ro, w.dtype, f"o_part b={b}")
        assert_parity(got_l[b], rl, w.dtype, f"lse_part b={b}")
    assert M.mla_device_error() == 0


def _row_factor(phys):
    """Per-row magnitude 2^((p % 7) - 3) of physical row p: neighbouring rows of a
    tile get different scales."""
    return np.ldexp(1.0, (np.asarray(phys) % 7) - 3)


@pytest.mark.parametrize("name", ["full-fp8", "lite-fp8"])
@pytest.mark.parametrize("path", PATHS)
def test_attention_fp8_rows_with_different_scales(name, path):
    """Each row's own scale must weigh its codes: rows of one tile alternate over
    seven magnitudes (2^-3 .. 2^3), so a scale taken from the wrong row shows."""
    w = _wl(name, batch=3)
    lens = (1000, 4096, 77)
    S = 4
    M.mla_set_kernel_path(path)
    note(f"attention fp8 varied row scales {name} path={path}")
    d = _dims(w)
    bt, total = I.page_table(w, np.array(lens, dtype=np.int32))
    nh = w.n_heads
    rows = torch.empty((total * 64, w.row), dtype=torch.float32, device="cuda")
    I.fill_device(rows, I.stream_key(w.seed, "pool"))
    fac = torch.tensor(_row_factor(np.arange(total * 64)), dtype=torch.float32, device="cuda")
    rows *= fac[:, None]
    pool = torch.empty((total, M.mla_fp8_page_bytes(d)), dtype=torch.uint8, device="cuda")
    phys = torch.arange(total * 64, dtype=torch.int32, device="cuda")
    M.mla_quantize_rows_fp8(d, rows, (phys // 64).contiguous(), (phys % 64).contiguous(),
                            torch.arange(total, dtype=torch.int32, device="cuda").reshape(-1, 1), pool)
    q_lat = device_tensor(torch, w, "q_lat_in", (3, nh, w.d_latent), 0.5).float().contiguous()
    q_pe = device_tensor(torch, w, "q_pe_in", (3, nh, w.d_rope), 1.0).float().contiguous()
    o_part = torch.full((3, S, nh, w.d_latent), 123.0, device="cuda")
    lse_part = torch.full((3, S, nh), 123.0, device="cuda")
    M.mla_decode_attention_fp8(d, q_lat, q_pe, pool, torch.tensor(bt, device="cuda"),
                               torch.tensor(np.array(lens, dtype=np.int32), device="cuda"), o_part,
                               lse_part)
    hq = host_tensor(w, "q_lat_in", (3, nh, w.d_latent), 0.5)
    hp = host_tensor(w, "q_pe_in", (3, nh, w.d_rope), 1.0)
    for b, L in enumerate(lens):
        pos = np.arange(L)
        ph = bt[b, pos // 64].astype(np.int64) * 64 + pos % 64
        src = I.pool_rows(w, bt, b, L, f32=True).astype(np.float64) * _row_factor(ph)[:, None]
        ro, rl = O.attention_partials(hq[b], hp[b], _fp8_rows(src.astype(np.float32), w.d_latent), S,
                                      w.d_latent, w.d_rope, M.default_scale(d), 64)
        assert_parity(to_np(o_part)[b], ro, w.dtype, f"o_part b={b}")
        assert_parity(to_np(lse_part)[b], rl, w.dtype, f"lse_part b={b}")
    assert M.mla_device_error() == 0


@pytest.mark.parametrize("name", ["full-fp8", "lite-fp8"])
@pytest.mark.parametrize("path", PATHS)
def test_attention_fp8_skips_bad_page(name, path):
    """An out-of-pool table entry on the split's first page takes no weight and is
    flagged.  Physical page 0, which no sequence owns here, holds NaN codes: the
    kernels must not let those bytes reach the output either."""
    w = _wl(name, batch=1)
    M.mla_set_kernel_path(path)
    L = 200
    note(f"attention fp8 bad first page {name} path={path}")
    bt, total = I.page_table(w, np.array([L], dtype=np.int32))
    bt = bt + 1                                            # pages 1..total; page 0 unowned
    d = _dims(w)
    nh = w.n_heads
    pool = torch.empty((total + 1, M.mla_fp8_page_bytes(d)), dtype=torch.uint8, device="cuda")
    fill_fp8_pool(d, pool, I.stream_key(w.seed, "pool"))
    pool[0] = 0x7F
    q_lat = device_tensor(torch, w, "q_lat_in", (1, nh, w.d_latent), 0.5).float().contiguous()
    q_pe = device_tensor(torch, w, "q_pe_in", (1, nh, w.d_rope), 1.0).float().contiguous()
    bad = bt.copy()
    bad[0, 0] = total + 8
    o_part = torch.full((1, 1, nh, w.d_latent), 123.0, device="cuda")
    lse_part = torch.full((1, 1, nh), 123.0, device="cuda")
    M.mla_device_error(clear=True)
    M.mla_decode_attention_fp8(d, q_lat, q_pe, pool, torch.tensor(bad, device="cuda"),
                               torch.tensor([L], dtype=torch.int32, device="cuda"), o_part, lse_part)
    assert M.mla_device_error(clear=True) & 1
    rows = _fp8_rows(I.pool_rows(w, bt, 0, L, f32=True)[64:], w.d_latent)
    ro, rl = O.attention_partials(host_tensor(w, "q_lat_in", (1, nh, w.d_latent), 0.5)[0],
                                  host_tensor(w, "q_pe_in", (1, nh, w.d_rope), 1.0)[0], rows, 1,
                                  w.d_latent, w.d_rope, M.default_scale(d), 64)
    assert_parity(to_np(o_part)[0], ro, w.dtype, "o_part without the bad page")
    assert_parity(to_np(lse_part)[0], rl, w.dtype, "lse_part without the bad page")


# ----------------------------------------------------------------- step --
@pytest.mark.parametrize("name", ["tiny-fp8", "lite-fp8", "full-fp8"])
def test_step_fp8(name):
    """The decode step on the FP8 pool: the oracle quantizes the same context rows
    (and the appended decode row) and runs the absorbed fp64 step on them."""
    w = I.WORKLOADS[name]
    note(f"step {name}")
    dw = DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    assert M.mla_device_error() == 0
    hw = dw.host_weights()
    seqs = list(range(w.batch)) if w.batch <= 4 else [0, w.batch // 2, w.batch - 1]
    dw.merge_o_lat()     # the step's fused merge does not store o_lat
    got = {k: to_np(getattr(dw, k)) for k in ("u", "q_lat", "o_lat", "lse")}
    ref = {k: [] for k in got}
    for b in seqs:
        L = int(dw.lens[b])
        if w.cache_from_h:
            rows = O.latent_rows(dw.host_h_ctx(b), hw["w_dkv"], hw["w_kr"], np.arange(L), w.rope_base)
        else:
            rows = dw.host_pool_rows(b, L)
            rows[L - 1] = O.latent_rows(dw.host_h(b)[None], hw["w_dkv"], hw["w_kr"], [L - 1],
                                        w.rope_base)[0]
        a = O.mla_decode_step_absorbed(dw.host_h(b), _fp8_rows(rows, w.d_latent), hw["w_q"],
                                       hw["w_qr"], hw["w_uk"], hw["w_uv"], hw["w_o"], L - 1,
                                       w.n_heads, w.d_head, w.d_latent, w.d_rope, w.rope_base)
        for k in ref:
            ref[k].append(a[k])
    for k in ref:
        assert_parity(got[k][seqs], np.stack(ref[k]), w.dtype, f"{k} seqs={seqs}")
