"""Per-call parity of the five C-ABI entry points against the fp64 oracle.

Inputs of every call come from the seeded generator (never from another GPU
call); both kernel paths (automatic = MFMA where the shape allows, and the
plain vector kernels) are checked.
"""
import math

import numpy as np
import pytest

import mla_latent_kv_dkv_amd as M
import oracle as O
from mla_latent_kv_dkv_amd import inputs as I
from tests.gpu_util import assert_parity, device_tensor, host_tensor, note, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

DIMS = {n: I.WORKLOADS[n] for n in ("tiny", "lite", "full", "tiny-cq", "lite-cq", "full-cq")}
PATHS = [0, 1]


@pytest.fixture(autouse=True)
def _path_reset():
    M.load()
    yield
    M.mla_set_kernel_path(0)


def _wl(name, **kw):
    w = DIMS[name]
    fields = dict(w.__dict__)
    fields.update(kw)
    return I.Workload(**fields)


def _dims(w):
    return M.make_dims(w.hidden, w.n_heads, w.d_head, w.d_latent, w.d_rope, w.dtype, w.page_size,
                       w.rope_base)


# ------------------------------------------------------------ generator --
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_device_fill_is_bit_identical_to_host(dtype):
    w = _wl("tiny", dtype=dtype)
    note(f"fill {dtype}")
    t = device_tensor(torch, w, "probe", (3, 1000), std=0.7)
    torch.cuda.synchronize()
    host = I.tensor_values(w, "probe", (3, 1000), 0.7)
    if dtype == "f32":
        np.testing.assert_array_equal(t.cpu().numpy().view(np.uint32), host.view(np.uint32))
    else:
        np.testing.assert_array_equal(t.view(torch.int16).cpu().numpy().view(np.uint16), host)
    # sub-range start offset
    u = torch.empty(500, dtype=t.dtype, device="cuda")
    I.fill_device(u, I.stream_key(w.seed, "probe"), 0.7, start=1234)
    np.testing.assert_array_equal(to_np(u), to_np(t).reshape(-1)[1234:1734])


# --------------------------------------------------------------- append --
def _sentinel_pool(w, pages):
    pool = torch.full((pages, w.page_size, w.row), -3.5,
                      dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16, device="cuda")
    return pool


@pytest.mark.parametrize("name", ["tiny", "full"])
@pytest.mark.parametrize("path", PATHS)
def test_append_latent_placement_and_values(name, path):
    w = _wl(name, batch=3)
    M.mla_set_kernel_path(path)
    lens = np.array([5, 130, 64], dtype=np.int32) if name == "tiny" else np.array([70, 200, 64],
                                                                                    dtype=np.int32)
    bt, total = I.page_table(w, lens)
    rng = np.random.default_rng(5)
    seqs = np.concatenate([np.full(l, b) for b, l in enumerate(lens)]).astype(np.int32)
    poss = np.concatenate([np.arange(l) for l in lens]).astype(np.int32)
    sel = rng.permutation(len(seqs))[:97]                  # 97 rows in scrambled order
    seqs, poss = seqs[sel], poss[sel]
    n = len(sel)
    note(f"append {name} path={path} rows={n}")
    h = device_tensor(torch, w, "h_rows", (n, w.hidden))
    wd = device_tensor(torch, w, "w_dkv", (w.d_latent, w.hidden), 1 / math.sqrt(w.hidden))
    wk = device_tensor(torch, w, "w_kr", (w.d_rope, w.hidden), 1 / math.sqrt(w.hidden))
    pool = _sentinel_pool(w, total)
    d = _dims(w)
    M.mla_append_latent(d, h, wd, wk, torch.tensor(seqs, device="cuda"),
                        torch.tensor(poss, device="cuda"),
                        torch.tensor(bt, device="cuda"), pool)
    got = to_np(pool).reshape(-1, w.row)
    ref_rows = O.latent_rows(host_tensor(w, "h_rows", (n, w.hidden)),
                             host_tensor(w, "w_dkv", (w.d_latent, w.hidden), 1 / math.sqrt(w.hidden)),
                             host_tensor(w, "w_kr", (w.d_rope, w.hidden), 1 / math.sqrt(w.hidden)),
                             poss, w.rope_base)
    slots = np.array([O.page_slot(bt, s, p, w.page_size) for s, p in zip(seqs, poss)])
    assert len(set(slots.tolist())) == n
    untouched = np.ones(got.shape[0], bool)
    untouched[slots] = False
    assert (got[untouched] == -3.5).all(), "rows outside the written slots changed"
    assert_parity(got[slots], ref_rows, w.dtype, "appended rows")
    assert M.mla_device_error() == 0


@pytest.mark.parametrize("path", PATHS)
def test_append_is_page_table_invariant_bit_exact(path):
    """The same rows appended under two page tables land as a bit-exact permutation."""
    w = _wl("full", batch=2)
    M.mla_set_kernel_path(path)
    lens = np.array([256, 192], dtype=np.int32)
    bt_perm, total = I.page_table(w, lens)
    bt_id, _ = I.page_table(_wl("full", batch=2, permute_pages=False), lens)
    seqs = np.concatenate([np.full(l, b) for b, l in enumerate(lens)]).astype(np.int32)
    poss = np.concatenate([np.arange(l) for l in lens]).astype(np.int32)
    note(f"append invariance path={path}")
    h = device_tensor(torch, w, "h_rows", (len(seqs), w.hidden))
    wd = device_tensor(torch, w, "w_dkv", (w.d_latent, w.hidden), 1 / math.sqrt(w.hidden))
    wk = device_tensor(torch, w, "w_kr", (w.d_rope, w.hidden), 1 / math.sqrt(w.hidden))
    out = []
    for bt in (bt_perm, bt_id):
        pool = _sentinel_pool(w, total)
        M.mla_append_latent(_dims(w), h, wd, wk, torch.tensor(seqs, device="cuda"),
                            torch.tensor(poss, device="cuda"), torch.tensor(bt, device="cuda"), pool)
        bits = pool.view(torch.int16).cpu().numpy().reshape(-1, w.row)
        out.append(np.stack([bits[O.page_slot(bt, s, p, 64)] for s, p in zip(seqs, poss)]))
    np.testing.assert_array_equal(out[0], out[1])


def test_append_bad_page_sets_error_and_writes_nothing():
    w = _wl("tiny", batch=1)
    pool = _sentinel_pool(w, 2)
    h = device_tensor(torch, w, "h_rows", (2, w.hidden))
    wd = device_tensor(torch, w, "w_dkv", (w.d_latent, w.hidden))
    wk = device_tensor(torch, w, "w_kr", (w.d_rope, w.hidden))
    bt = torch.tensor([[0, 9]], dtype=torch.int32, device="cuda")     # page 9 does not exist
    note("append bad page")
    M.mla_device_error(clear=True)
    M.mla_append_latent(_dims(w), h, wd, wk, torch.zeros(2, dtype=torch.int32, device="cuda"),
                        torch.tensor([70, 200], dtype=torch.int32, device="cuda"), bt, pool)
    err = M.mla_device_error(clear=True)
    assert err & 1 and err & 2          # bad table entry (pos 70) and position beyond the table (200)
    assert (to_np(pool) == -3.5).all()


# ------------------------------------------------------------- absorb_q --
@pytest.mark.parametrize("name", ["tiny", "lite", "full"])
@pytest.mark.parametrize("path", PATHS)
def test_absorb_q(name, path):
    w = _wl(name)
    B = 5
    M.mla_set_kernel_path(path)
    note(f"absorb_q {name} path={path}")
    sh = {n: w.weight_shape(n) for n in ("w_q", "w_qr", "w_uk")}
    std = {n: 1 / math.sqrt(w.fan_in(n)) for n in sh}
    dev = {n: device_tensor(torch, w, n, sh[n], std[n]) for n in sh}
    h = device_tensor(torch, w, "h_q", (B, w.hidden))
    pos_np = np.array([0, 1, 63, 4095, 131071][:B], dtype=np.int32)
    q_lat = torch.empty((B, w.n_heads, w.d_latent), dtype=torch.float32, device="cuda")
    q_pe = torch.empty((B, w.n_heads, w.d_rope), dtype=torch.float32, device="cuda")
    d = _dims(w)
    ws = torch.empty(M.mla_workspace_bytes(d, B), dtype=torch.uint8, device="cuda")
    M.mla_absorb_q(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], torch.tensor(pos_np, device="cuda"),
                   q_lat, q_pe, ws)
    hh = host_tensor(w, "h_q", (B, w.hidden))
    hw = {n: host_tensor(w, n, sh[n], std[n]) for n in sh}
    ref_lat, ref_pe = [], []
    for b in range(B):
        ql, qp = O.absorb_q(hh[b], hw["w_q"], hw["w_qr"], hw["w_uk"], int(pos_np[b]), w.n_heads,
                            w.d_head, w.d_latent, w.d_rope, w.rope_base)
        ref_lat.append(ql)
        ref_pe.append(qp)
    assert_parity(to_np(q_lat), np.stack(ref_lat), w.dtype, "q_lat")
    assert_parity(to_np(q_pe), np.stack(ref_pe), w.dtype, "q_pe")


@pytest.mark.parametrize("name", ["tiny-cq", "lite-cq", "full-cq"])
@pytest.mark.parametrize("path", PATHS)
def test_absorb_q_cq(name, path):
    """Query through its low-rank compression (c^Q = W_DQ h, q^C = W_UQ c^Q)."""
    w = _wl(name)
    B = 5
    M.mla_set_kernel_path(path)
    note(f"absorb_q_cq {name} path={path}")
    sh = {n: w.weight_shape(n) for n in ("w_dq", "w_uq", "w_qr", "w_uk")}
    std = {n: 1 / math.sqrt(w.fan_in(n)) for n in sh}
    dev = {n: device_tensor(torch, w, n, sh[n], std[n]) for n in sh}
    h = device_tensor(torch, w, "h_q", (B, w.hidden))
    pos_np = np.array([0, 1, 63, 4095, 131071][:B], dtype=np.int32)
    q_lat = torch.empty((B, w.n_heads, w.d_latent), dtype=torch.float32, device="cuda")
    q_pe = torch.empty((B, w.n_heads, w.d_rope), dtype=torch.float32, device="cuda")
    d = _dims(w)
    ws = torch.empty(M.mla_workspace_bytes_cq(d, w.d_cq, B), dtype=torch.uint8, device="cuda")
    M.mla_absorb_q_cq(d, h, dev["w_dq"], dev["w_uq"], dev["w_qr"], dev["w_uk"],
                      torch.tensor(pos_np, device="cuda"), q_lat, q_pe, ws)
    hh = host_tensor(w, "h_q", (B, w.hidden))
    hw = {n: host_tensor(w, n, sh[n], std[n]) for n in sh}
    ref_lat, ref_pe = [], []
    for b in range(B):
        ql, qp = O.absorb_q(hh[b], None, hw["w_qr"], hw["w_uk"], int(pos_np[b]), w.n_heads,
                            w.d_head, w.d_latent, w.d_rope, w.rope_base, w_dq=hw["w_dq"],
                            w_uq=hw["w_uq"])
        ref_lat.append(ql)
        ref_pe.append(qp)
    assert_parity(to_np(q_lat), np.stack(ref_lat), w.dtype, "q_lat")
    assert_parity(to_np(q_pe), np.stack(ref_pe), w.dtype, "q_pe")


# ------------------------------------------------------------ attention --
ATTN_CASES = [
    ("tiny", [1, 64, 100, 129], 3, 16),
    ("tiny", [64], 1, 64),
    ("lite", [64, 777, 4096], 2, 64),
    ("full", [1, 65, 1000, 4096], 4, 64),
    ("full", [3000, 130], 8, 64),
    ("full", [2], 5, 64),          # most splits empty
    ("full", [33000], 1, 64),      # one split over 516 pages: the kernel's page-id window reloads
    # 16 heads: the Lite kernel (each wave its own 16-token tiles)
    ("lite", [1, 65, 1000, 4096], 8, 64),
    ("lite", [17, 33, 130], 5, 64),   # partial tiles, waves without tiles, empty splits
    ("lite", [33000], 1, 64),         # one split: every wave streams 516 tiles
]


@pytest.mark.parametrize("name,lens,S,page", ATTN_CASES)
@pytest.mark.parametrize("path", PATHS)
def test_decode_attention_partials(name, lens, S, page, path):
    w = _wl(name, batch=len(lens), page_size=page)
    M.mla_set_kernel_path(path)
    lens = np.array(lens, dtype=np.int32)
    bt, total = I.page_table(w, lens)
    B, nh = w.batch, w.n_heads
    note(f"attention {name} lens={lens.tolist()} S={S} page={page} path={path}")
    # q holds values exactly representable in the pool's storage type (the MFMA
    # path rounds q to bf16 once per work unit; the rounding of computed
    # queries is covered by the end-to-end step tests)
    q_lat = device_tensor(torch, w, "q_lat_in", (B, nh, w.d_latent), 0.5).float().contiguous()
    q_pe = device_tensor(torch, w, "q_pe_in", (B, nh, w.d_rope), 1.0).float().contiguous()
    pool = device_tensor(torch, w, "pool", (total, page, w.row))
    o_part = torch.full((B, S, nh, w.d_latent), 123.0, device="cuda")
    lse_part = torch.full((B, S, nh), 123.0, device="cuda")
    d = _dims(w)
    M.mla_decode_attention(d, q_lat, q_pe, pool, torch.tensor(bt, device="cuda"),
                           torch.tensor(lens, device="cuda"), o_part, lse_part)
    got_o, got_l = to_np(o_part), to_np(lse_part)
    hq = host_tensor(w, "q_lat_in", (B, nh, w.d_latent), 0.5)
    hp = host_tensor(w, "q_pe_in", (B, nh, w.d_rope), 1.0)
    tau = M.default_scale(d)
    for b in range(B):
        rows = I.to_f64(w, I.pool_rows(w, bt, b, int(lens[b])))
        ro, rl = O.attention_partials(hq[b], hp[b], rows, S, w.d_latent, w.d_rope, tau, page)
        assert_parity(got_o[b], ro, w.dtype, f"o_part b={b}")
        assert_parity(got_l[b], rl, w.dtype, f"lse_part b={b}")
    assert M.mla_device_error() == 0


@pytest.mark.parametrize("name", ["full", "lite"])
@pytest.mark.parametrize("path", PATHS)
def test_attention_skips_bad_page(path, name):
    """A table entry outside the pool is skipped (its tokens take no weight) and
    flagged in the error word.  The bad page is the first one of the split, so
    the MFMA kernel's first tile has no valid score."""
    w = _wl(name, batch=1)
    M.mla_set_kernel_path(path)
    L = 200
    lens = np.array([L], dtype=np.int32)
    bt, total = I.page_table(w, lens)
    bad = bt.copy()
    bad[0, 0] = total + 7                                  # page 0 (tokens 0..63) is out of range
    note(f"attention bad first page {name} path={path}")
    nh = w.n_heads
    q_lat = device_tensor(torch, w, "q_lat_in", (1, nh, w.d_latent), 0.5).float().contiguous()
    q_pe = device_tensor(torch, w, "q_pe_in", (1, nh, w.d_rope), 1.0).float().contiguous()
    pool = device_tensor(torch, w, "pool", (total, 64, w.row))
    o_part = torch.full((1, 1, nh, w.d_latent), 123.0, device="cuda")
    lse_part = torch.full((1, 1, nh), 123.0, device="cuda")
    M.mla_device_error(clear=True)
    M.mla_decode_attention(_dims(w), q_lat, q_pe, pool, torch.tensor(bad, device="cuda"),
                           torch.tensor(lens, device="cuda"), o_part, lse_part)
    assert M.mla_device_error(clear=True) & 1
    rows = I.to_f64(w, I.pool_rows(w, bt, 0, L))[64:]      # the tokens that remain
    ro, rl = O.attention_partials(host_tensor(w, "q_lat_in", (1, nh, w.d_latent), 0.5)[0],
                                  host_tensor(w, "q_pe_in", (1, nh, w.d_rope), 1.0)[0], rows, 1,
                                  w.d_latent, w.d_rope, M.default_scale(_dims(w)), 64)
    assert_parity(to_np(o_part)[0], ro, w.dtype, "o_part without the bad page")
    assert_parity(to_np(lse_part)[0], rl, w.dtype, "lse_part without the bad page")


def test_attention_is_page_table_invariant():
    """Output is bit-identical under a different physical placement of the same rows."""
    w = _wl("full", batch=2)
    lens = np.array([1000, 333], dtype=np.int32)
    bt_p, total = I.page_table(w, lens)
    bt_i, _ = I.page_table(_wl("full", batch=2, permute_pages=False), lens)
    note("attention page-table invariance")
    pool_p = device_tensor(torch, w, "pool", (total, 64, w.row))
    # same logical rows, identity placement: move page bt_p[b][k] to page bt_i[b][k]
    pool_i = torch.empty_like(pool_p)
    src = torch.tensor(np.concatenate([bt_p[b, :(l + 63) // 64] for b, l in enumerate(lens)]),
                       device="cuda").long()
    dst = torch.tensor(np.concatenate([bt_i[b, :(l + 63) // 64] for b, l in enumerate(lens)]),
                       device="cuda").long()
    pool_i[dst] = pool_p[src]
    q_lat = device_tensor(torch, w, "q_lat_in", (2, w.n_heads, w.d_latent), 0.5).float().contiguous()
    q_pe = device_tensor(torch, w, "q_pe_in", (2, w.n_heads, w.d_rope), 1.0).float().contiguous()
    res = []
    for pool, bt in ((pool_p, bt_p), (pool_i, bt_i)):
        o = torch.empty((2, 4, w.n_heads, w.d_latent), device="cuda")
        l = torch.empty((2, 4, w.n_heads), device="cuda")
        M.mla_decode_attention(_dims(w), q_lat, q_pe, pool, torch.tensor(bt, device="cuda"),
                               torch.tensor(lens, device="cuda"), o, l)
        res.append((o.cpu().numpy(), l.cpu().numpy()))
    np.testing.assert_array_equal(res[0][0], res[1][0])
    np.testing.assert_array_equal(res[0][1], res[1][1])


# ---------------------------------------------------------------- merge --
@pytest.mark.parametrize("name,S", [("tiny", 3), ("full", 8), ("full", 64)])
@pytest.mark.parametrize("path", PATHS)
def test_merge_lse(name, S, path):
    w = _wl(name)
    B, nh = 3, w.n_heads
    M.mla_set_kernel_path(path)
    note(f"merge {name} S={S} path={path}")
    o_part = device_tensor(torch, w, "o_part_in", (B, S, nh, w.d_latent), 1.0, dtype=torch.float32)
    lse_part = device_tensor(torch, w, "lse_part_in", (B, S, nh), 3.0, dtype=torch.float32)
    lse_host = I.normal_f32(I.stream_key(w.seed, "lse_part_in"), 0, B * S * nh, 3.0).astype(
        np.float64).reshape(B, S, nh)
    # empty splits: every other split of sequence 1, and all splits of head 0 of sequence 2
    lse_part[1, ::2] = -math.inf
    lse_part[2, :, 0] = -math.inf
    lse_host[1, ::2] = -np.inf
    lse_host[2, :, 0] = -np.inf
    o_host = I.normal_f32(I.stream_key(w.seed, "o_part_in"), 0, B * S * nh * w.d_latent).astype(
        np.float64).reshape(B, S, nh, w.d_latent)
    o_lat = torch.empty((B, nh, w.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, nh), device="cuda")
    M.mla_merge_lse(_dims(w), o_part, lse_part, o_lat, lse)
    ro, rl = zip(*[O.merge_lse(o_host[b], lse_host[b]) for b in range(B)])
    assert_parity(to_np(o_lat), np.stack(ro), w.dtype, "o_lat")
    assert_parity(to_np(lse), np.stack(rl), w.dtype, "lse")
    assert (to_np(o_lat)[2, 0] == 0).all() and np.isneginf(to_np(lse)[2, 0])


# ----------------------------------------------------------- absorb_out --
@pytest.mark.parametrize("name", ["tiny", "lite", "full"])
@pytest.mark.parametrize("path", PATHS)
def test_absorb_out(name, path):
    w = _wl(name)
    B = 6
    M.mla_set_kernel_path(path)
    note(f"absorb_out {name} path={path}")
    std = {n: 1 / math.sqrt(w.fan_in(n)) for n in ("w_uv", "w_o")}
    wuv = device_tensor(torch, w, "w_uv", w.weight_shape("w_uv"), std["w_uv"])
    wo = device_tensor(torch, w, "w_o", w.weight_shape("w_o"), std["w_o"])
    o_lat = device_tensor(torch, w, "o_lat_in", (B, w.n_heads, w.d_latent), dtype=torch.float32)
    u = torch.empty((B, w.hidden), dtype=torch.float32, device="cuda")
    d = _dims(w)
    ws = torch.empty(M.mla_workspace_bytes(d, B), dtype=torch.uint8, device="cuda")
    M.mla_absorb_out(d, o_lat, wuv, wo, u, ws)
    hu = host_tensor(w, "w_uv", w.weight_shape("w_uv"), std["w_uv"])
    ho = host_tensor(w, "w_o", w.weight_shape("w_o"), std["w_o"])
    hl = I.normal_f32(I.stream_key(w.seed, "o_lat_in"), 0, B * w.n_heads * w.d_latent).astype(
        np.float64).reshape(B, w.n_heads, w.d_latent)
    ref = np.stack([O.absorb_out(hl[b], hu, ho, w.n_heads, w.d_head, w.d_latent) for b in range(B)])
    assert_parity(to_np(u), ref, w.dtype, "u")


# ------------------------------------------- prefill-sized activation batches --
# M = 300 rows takes the tiled large-M product (128-row tiles: two full ones and a
# ragged tail of 44); the oracle is evaluated on sampled rows, tile edges included.
ROWS = [0, 1, 127, 128, 200, 255, 256, 299]


@pytest.mark.parametrize("name", ["lite", "full"])
def test_absorb_q_large_batch(name):
    w = _wl(name)
    B = 300
    note(f"absorb_q {name} B={B}")
    sh = {n: w.weight_shape(n) for n in ("w_q", "w_qr", "w_uk")}
    std = {n: 1 / math.sqrt(w.fan_in(n)) for n in sh}
    dev = {n: device_tensor(torch, w, n, sh[n], std[n]) for n in sh}
    h = device_tensor(torch, w, "h_q", (B, w.hidden))
    pos_np = ((np.arange(B, dtype=np.int64) * 4099) % 131072).astype(np.int32)
    q_lat = torch.empty((B, w.n_heads, w.d_latent), dtype=torch.float32, device="cuda")
    q_pe = torch.empty((B, w.n_heads, w.d_rope), dtype=torch.float32, device="cuda")
    d = _dims(w)
    ws = torch.empty(max(1, M.mla_workspace_bytes(d, B)), dtype=torch.uint8, device="cuda")
    M.mla_absorb_q(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], torch.tensor(pos_np, device="cuda"),
                   q_lat, q_pe, ws)
    hh = host_tensor(w, "h_q", (B, w.hidden))
    hw = {n: host_tensor(w, n, sh[n], std[n]) for n in sh}
    ref_lat, ref_pe = [], []
    for b in ROWS:
        ql, qp = O.absorb_q(hh[b], hw["w_q"], hw["w_qr"], hw["w_uk"], int(pos_np[b]), w.n_heads,
                            w.d_head, w.d_latent, w.d_rope, w.rope_base)
        ref_lat.append(ql)
        ref_pe.append(qp)
    assert_parity(to_np(q_lat)[ROWS], np.stack(ref_lat), w.dtype, "q_lat")
    assert_parity(to_np(q_pe)[ROWS], np.stack(ref_pe), w.dtype, "q_pe")


@pytest.mark.parametrize("name", ["lite", "full"])
def test_absorb_out_large_batch(name):
    w = _wl(name)
    B = 300
    note(f"absorb_out {name} B={B}")
    std = {n: 1 / math.sqrt(w.fan_in(n)) for n in ("w_uv", "w_o")}
    wuv = device_tensor(torch, w, "w_uv", w.weight_shape("w_uv"), std["w_uv"])
    wo = device_tensor(torch, w, "w_o", w.weight_shape("w_o"), std["w_o"])
    o_lat = device_tensor(torch, w, "o_lat_in", (B, w.n_heads, w.d_latent), dtype=torch.float32)
    u = torch.empty((B, w.hidden), dtype=torch.float32, device="cuda")
    d = _dims(w)
    ws = torch.empty(max(1, M.mla_workspace_bytes(d, B)), dtype=torch.uint8, device="cuda")
    M.mla_absorb_out(d, o_lat, wuv, wo, u, ws)
    hu = host_tensor(w, "w_uv", w.weight_shape("w_uv"), std["w_uv"])
    ho = host_tensor(w, "w_o", w.weight_shape("w_o"), std["w_o"])
    hl = I.normal_f32(I.stream_key(w.seed, "o_lat_in"), 0, B * w.n_heads * w.d_latent).astype(
        np.float64).reshape(B, w.n_heads, w.d_latent)
    ref = np.stack([O.absorb_out(hl[b], hu, ho, w.n_heads, w.d_head, w.d_latent) for b in ROWS])
    assert_parity(to_np(u)[ROWS], ref, w.dtype, "u")


# ------------------------------------------------- fused absorb_q + append --
def _append_lens(B):
    """Context lengths of the fused-append tests: token b at lens[b] - 1 (across
    page boundaries); the 256-row batches stay under 300 tokens to keep the pool small."""
    if B <= 64:
        return np.array([3 + 37 * b for b in range(B)], dtype=np.int32)
    return np.array([1 + (37 * b) % 300 for b in range(B)], dtype=np.int32)


def _oracle_rows(B):
    """Rows checked against the fp64 oracle: all of them, or every 8th and the last
    for 256-row batches (all rows are still compared bit for bit with mla_absorb_q)."""
    return list(range(B)) if B <= 64 else sorted(set(range(0, B, 8)) | {B - 1})


# K slices of the fused product: lite 4 (B = 32 and B = 5), full 5 (B = 64, and
# B = 5 with one-block partial tiles), lite with a 512-wide hidden state 1 (the
# output stage straight from the product); full B = 256: the tiled product, its
# last 4.5 weight tiles the appended rows; tiny (fp32) takes the two calls
@pytest.mark.parametrize("name,B,hidden", [("tiny", 5, 0), ("lite", 5, 0), ("lite", 32, 0),
                                           ("lite", 32, 512), ("full", 5, 0), ("full", 64, 0),
                                           ("full", 256, 0)])
def test_absorb_q_append(name, B, hidden):
    """The fused call against the oracle (queries and appended rows), its queries
    equal to mla_absorb_q's, the pool untouched outside the appended slots (the
    f32 shape exercises the fallback to the two calls)."""
    w = _wl(name, batch=B, **({"hidden": hidden} if hidden else {}))
    note(f"absorb_q_append {name} B={B} hidden={w.hidden}")
    lens = _append_lens(B)   # token b at lens[b] - 1
    bt, total = I.page_table(w, lens)
    seqs = np.arange(B, dtype=np.int32)
    poss = (lens - 1).astype(np.int32)
    sh = {n: w.weight_shape(n) for n in ("w_q", "w_qr", "w_uk", "w_dkv", "w_kr")}
    std = {n: 1 / math.sqrt(w.fan_in(n)) for n in sh}
    dev = {n: device_tensor(torch, w, n, sh[n], std[n]) for n in sh}
    h = device_tensor(torch, w, "h_q", (B, w.hidden))
    d = _dims(w)
    ws = torch.empty(M.mla_workspace_bytes(d, B), dtype=torch.uint8, device="cuda")
    q_lat = torch.empty((B, w.n_heads, w.d_latent), dtype=torch.float32, device="cuda")
    q_pe = torch.empty((B, w.n_heads, w.d_rope), dtype=torch.float32, device="cuda")
    pool = _sentinel_pool(w, total)
    pos_t, seq_t = torch.tensor(poss, device="cuda"), torch.tensor(seqs, device="cuda")
    M.mla_device_error(clear=True)
    M.mla_absorb_q_append(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], dev["w_dkv"], dev["w_kr"],
                          pos_t, seq_t, torch.tensor(bt, device="cuda"), pool, q_lat, q_pe, ws)
    q_lat2, q_pe2 = torch.empty_like(q_lat), torch.empty_like(q_pe)
    M.mla_absorb_q(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], pos_t, q_lat2, q_pe2, ws)
    assert torch.equal(q_lat, q_lat2) and torch.equal(q_pe, q_pe2), "queries differ from mla_absorb_q"
    hh = host_tensor(w, "h_q", (B, w.hidden))
    hw = {n: host_tensor(w, n, sh[n], std[n]) for n in sh}
    rows = _oracle_rows(B)
    rl, rp = zip(*[O.absorb_q(hh[b], hw["w_q"], hw["w_qr"], hw["w_uk"], int(poss[b]), w.n_heads,
                              w.d_head, w.d_latent, w.d_rope, w.rope_base) for b in rows])
    assert_parity(to_np(q_lat)[rows], np.stack(rl), w.dtype, "q_lat")
    assert_parity(to_np(q_pe)[rows], np.stack(rp), w.dtype, "q_pe")
    got = to_np(pool).reshape(-1, w.row)
    ref_rows = O.latent_rows(hh, hw["w_dkv"], hw["w_kr"], poss, w.rope_base)
    slots = np.array([O.page_slot(bt, s, p, w.page_size) for s, p in zip(seqs, poss)])
    untouched = np.ones(got.shape[0], bool)
    untouched[slots] = False
    assert (got[untouched] == -3.5).all(), "rows outside the appended slots changed"
    assert_parity(got[slots], ref_rows, w.dtype, "appended rows")
    assert M.mla_device_error() == 0


@pytest.mark.parametrize("B", [5, 64, 256])
def test_absorb_q_append_out_of_range_rows(B):
    """Rows whose table entry or sequence is out of range: nothing is written to
    the pool, the error word says which, and their queries are still computed
    (equal to mla_absorb_q's).  B = 5 goes through the K-split finish pass of the
    fused product, B = 64 straight through its epilogue, B = 256 through the
    tiled product's."""
    w = _wl("full", batch=B)
    lens = _append_lens(B)
    bt, total = I.page_table(w, lens)
    seqs = np.arange(B, dtype=np.int32)
    poss = (lens - 1).astype(np.int32)
    bad_bt = bt.copy()
    bad_bt[1, poss[1] // 64] = total + 3          # row 1: table entry outside the pool
    seqs[3] = B + 9                               # row 3: sequence outside the table
    note(f"absorb_q_append out-of-range rows B={B}")
    sh = {n: w.weight_shape(n) for n in ("w_q", "w_qr", "w_uk", "w_dkv", "w_kr")}
    std = {n: 1 / math.sqrt(w.fan_in(n)) for n in sh}
    dev = {n: device_tensor(torch, w, n, sh[n], std[n]) for n in sh}
    h = device_tensor(torch, w, "h_q", (B, w.hidden))
    d = _dims(w)
    ws = torch.empty(M.mla_workspace_bytes(d, B), dtype=torch.uint8, device="cuda")
    q_lat = torch.empty((B, w.n_heads, w.d_latent), dtype=torch.float32, device="cuda")
    q_pe = torch.empty((B, w.n_heads, w.d_rope), dtype=torch.float32, device="cuda")
    pool = _sentinel_pool(w, total)
    pos_t = torch.tensor(poss, device="cuda")
    M.mla_device_error(clear=True)
    M.mla_absorb_q_append(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], dev["w_dkv"], dev["w_kr"],
                          pos_t, torch.tensor(seqs, device="cuda"),
                          torch.tensor(bad_bt, device="cuda"), pool, q_lat, q_pe, ws)
    err = M.mla_device_error(clear=True)
    assert err & 1 and err & 4, err
    q_lat2, q_pe2 = torch.empty_like(q_lat), torch.empty_like(q_pe)
    M.mla_absorb_q(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], pos_t, q_lat2, q_pe2, ws)
    assert torch.equal(q_lat, q_lat2) and torch.equal(q_pe, q_pe2)
    got = to_np(pool).reshape(-1, w.row)
    good = [b for b in range(B) if b not in (1, 3)]
    slots = np.array([O.page_slot(bad_bt, seqs[b], poss[b], 64) for b in good])
    untouched = np.ones(got.shape[0], bool)
    untouched[slots] = False
    assert (got[untouched] == -3.5).all(), "an out-of-range row was written"
    hh = host_tensor(w, "h_q", (B, w.hidden))
    hw = {n: host_tensor(w, n, sh[n], std[n]) for n in ("w_dkv", "w_kr")}
    ref_rows = O.latent_rows(hh[good], hw["w_dkv"], hw["w_kr"], poss[good], w.rope_base)
    assert_parity(got[slots], ref_rows, w.dtype, "appended rows")


def test_absorb_q_append_misaligned_input_falls_back():
    """h starting 2 bytes past a 16-byte boundary: the fused product cannot take it,
    so the call makes the two calls in turn and gives their results."""
    w = _wl("full", batch=8)
    B = 8
    lens = np.array([100 + 9 * b for b in range(B)], dtype=np.int32)
    bt, total = I.page_table(w, lens)
    poss = (lens - 1).astype(np.int32)
    note("absorb_q_append misaligned h")
    sh = {n: w.weight_shape(n) for n in ("w_q", "w_qr", "w_uk", "w_dkv", "w_kr")}
    std = {n: 1 / math.sqrt(w.fan_in(n)) for n in sh}
    dev = {n: device_tensor(torch, w, n, sh[n], std[n]) for n in sh}
    h_al = device_tensor(torch, w, "h_q", (B, w.hidden))
    flat = torch.empty(B * w.hidden + 1, dtype=h_al.dtype, device="cuda")
    h = flat[1:].view(B, w.hidden)
    h.copy_(h_al)
    assert h.data_ptr() % 16 == 2 and h.is_contiguous()
    d = _dims(w)
    ws = torch.empty(M.mla_workspace_bytes(d, B), dtype=torch.uint8, device="cuda")
    pos_t = torch.tensor(poss, device="cuda")
    seq_t = torch.arange(B, dtype=torch.int32, device="cuda")
    bt_t = torch.tensor(bt, device="cuda")
    outs = []
    for fused in (True, False):
        q_lat = torch.empty((B, w.n_heads, w.d_latent), dtype=torch.float32, device="cuda")
        q_pe = torch.empty((B, w.n_heads, w.d_rope), dtype=torch.float32, device="cuda")
        pool = _sentinel_pool(w, total)
        if fused:
            M.mla_absorb_q_append(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], dev["w_dkv"],
                                  dev["w_kr"], pos_t, seq_t, bt_t, pool, q_lat, q_pe, ws)
        else:
            M.mla_absorb_q(d, h, dev["w_q"], dev["w_qr"], dev["w_uk"], pos_t, q_lat, q_pe, ws)
            M.mla_append_latent(d, h, dev["w_dkv"], dev["w_kr"], seq_t, pos_t, bt_t, pool)
        outs.append((q_lat, q_pe, pool))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    assert M.mla_device_error() == 0
