"""Chunked prefill: many prompt tokens per sequence attending causally to the
latent cache (mla_prefill_attention), and the whole prefill step built from the
decode calls with batch = prompt tokens, against the fp64 oracle."""
import numpy as np
import pytest

import mla_latent_kv_dkv_amd as M
import oracle as O
from mla_latent_kv_dkv_amd import inputs as I
from mla_latent_kv_dkv_amd.harness import DeviceWorkload, fill_fp8_pool
from tests.gpu_util import (assert_parity, assert_partials_within_weight_rounding, device_tensor,
                            host_tensor, note, to_np)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PATHS = [0, 1]


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


def _fp8_rows(rows, d_c):
    return np.stack([O.fp8_dequantize_row(*O.fp8_quantize_row(r, d_c)) for r in rows])


# queries (sequence, position): first and last positions, page and tile edges
CASES = [
    ("tiny", (40, 17), 16, 2, [(0, 0), (0, 15), (0, 16), (0, 39), (1, 0), (1, 16), (1, 5)]),
    ("full", (300, 77), 64, 2, [(0, 0), (0, 31), (0, 32), (0, 63), (0, 64), (0, 150), (0, 299),
                                (1, 0), (1, 5), (1, 76)]),
    ("full", (2100,), 64, 3, [(0, 2099), (0, 1024), (0, 64), (0, 700)]),
    ("lite", (300, 77), 64, 2, [(0, 0), (0, 15), (0, 16), (0, 63), (0, 64), (0, 299), (1, 5),
                                (1, 76)]),
]


@pytest.mark.parametrize("name,lens,page,S,queries", CASES)
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("fp8", [False, True])
def test_prefill_attention(name, lens, page, S, queries, path, fp8):
    w = _wl(name + ("-fp8" if fp8 else ""), batch=len(lens), page_size=page)
    M.mla_set_kernel_path(path)
    lens = np.array(lens, dtype=np.int32)
    bt, total = I.page_table(w, lens)
    nq, nh = len(queries), w.n_heads
    qs = np.array([q[0] for q in queries], dtype=np.int32)
    qp = np.array([q[1] for q in queries], dtype=np.int32)
    note(f"prefill attention {w.name} lens={lens.tolist()} S={S} path={path} queries={queries}")
    d = _dims(w)
    q_lat = device_tensor(torch, w, "q_lat_in", (nq, nh, w.d_latent), 0.5).float().contiguous()
    q_pe = device_tensor(torch, w, "q_pe_in", (nq, nh, w.d_rope), 1.0).float().contiguous()
    if fp8:
        pool = torch.empty((total, M.mla_fp8_page_bytes(d)), dtype=torch.uint8, device="cuda")
        fill_fp8_pool(d, pool, I.stream_key(w.seed, "pool"))
    else:
        pool = device_tensor(torch, w, "pool", (total, page, w.row))
    o_part = torch.full((nq, S, nh, w.d_latent), 123.0, device="cuda")
    lse_part = torch.full((nq, S, nh), 123.0, device="cuda")
    M.mla_prefill_attention(d, q_lat, q_pe, pool, torch.tensor(bt, device="cuda"),
                            torch.tensor(qs, device="cuda"), torch.tensor(qp, device="cuda"),
                            o_part, lse_part, fp8=fp8)
    o_lat = torch.empty((nq, nh, w.d_latent), device="cuda")
    lse = torch.empty((nq, nh), device="cuda")
    M.mla_merge_lse(d, o_part, lse_part, o_lat, lse)
    got_o, got_l, got_m, got_ml = to_np(o_part), to_np(lse_part), to_np(o_lat), to_np(lse)
    hq = host_tensor(w, "q_lat_in", (nq, nh, w.d_latent), 0.5)
    hp = host_tensor(w, "q_pe_in", (nq, nh, w.d_rope), 1.0)
    tau = M.default_scale(d)
    dt = w.dtype
    for b in range(len(lens)):
        sel = np.flatnonzero(qs == b)
        if fp8:
            rows = _fp8_rows(I.pool_rows(w, bt, b, int(lens[b]), f32=True), w.d_latent)
        else:
            rows = I.to_f64(w, I.pool_rows(w, bt, b, int(lens[b])))
        ref = O.prefill_attention_partials(hq[sel], hp[sel], rows, qp[sel], S, w.d_latent, w.d_rope,
                                           tau, page)
        for k, i in enumerate(sel):
            what = f"q=({b},{qp[i]})"
            # the attention output (splits merged by the library's merge) at the stated bar
            ref_m, ref_ml = O.merge_lse(*ref[k])
            assert_parity(got_m[i], ref_m, dt, f"o_lat {what}")
            assert_parity(got_ml[i], ref_ml, dt, f"lse {what}")
            assert_parity(got_l[i], ref[k][1], dt, f"lse_part {what}")
            # each split's output at the stated bar, and for bf16 also within the bound
            # its bf16 weights allow element by element
            assert_parity(got_o[i], ref[k][0], dt, f"o_part {what}")
            if dt != "f32":
                assert_partials_within_weight_rounding(got_o[i], ref[k][0], hq[i], hp[i], rows,
                                                       int(qp[i]) + 1, S, page, tau, w.d_latent,
                                                       what, exact_normaliser=fp8)
    assert M.mla_device_error() == 0


@pytest.mark.parametrize("path", PATHS)
def test_prefill_attention_bad_queries(path):
    """A query naming a sequence outside the table, or a position past it, gets an
    empty result and flags the error word; the others are unaffected."""
    w = _wl("full", batch=1)
    M.mla_set_kernel_path(path)
    lens = np.array([200], dtype=np.int32)
    bt, total = I.page_table(w, lens)
    qs = np.array([0, 3, 0, -1], dtype=np.int32)
    qp = np.array([199, 10, 4096, 5], dtype=np.int32)       # seq 3, pos 4096 = max_pages*64, seq -1
    nh = w.n_heads
    note(f"prefill bad queries path={path}")
    d = _dims(w)
    q_lat = device_tensor(torch, w, "q_lat_in", (4, nh, w.d_latent), 0.5).float().contiguous()
    q_pe = device_tensor(torch, w, "q_pe_in", (4, nh, w.d_rope), 1.0).float().contiguous()
    pool = device_tensor(torch, w, "pool", (total, 64, w.row))
    o_part = torch.full((4, 1, nh, w.d_latent), 123.0, device="cuda")
    lse_part = torch.full((4, 1, nh), 123.0, device="cuda")
    M.mla_device_error(clear=True)
    M.mla_prefill_attention(d, q_lat, q_pe, pool, torch.tensor(bt, device="cuda"),
                            torch.tensor(qs, device="cuda"), torch.tensor(qp, device="cuda"),
                            o_part, lse_part)
    err = M.mla_device_error(clear=True)
    assert err & 2 and err & 4
    lse = to_np(lse_part)
    assert np.isneginf(lse[1:]).all() and (to_np(o_part)[1:] == 0).all()
    rows = I.to_f64(w, I.pool_rows(w, bt, 0, 200))
    ro, rl = O.attention_partials(host_tensor(w, "q_lat_in", (4, nh, w.d_latent), 0.5)[0],
                                  host_tensor(w, "q_pe_in", (4, nh, w.d_rope), 1.0)[0], rows, 1,
                                  w.d_latent, w.d_rope, M.default_scale(d), 64)
    assert_parity(to_np(o_part)[0], ro, w.dtype, "o_part of the good query")
    assert_parity(lse[0], rl, w.dtype, "lse of the good query")


# ----------------------------------------------------------------- step --
def _step_ref(dw, hw, idx, absorbed):
    """Oracle outputs of step tokens idx (cache rows as the oracle sees them)."""
    w = dw.w
    out = {k: [] for k in ("u", "lse", "o_lat")}
    rows_of = {}
    for i in idx:
        b, p = int(dw.q_seq_host[i]), int(dw.q_pos_host[i])
        if b not in rows_of:
            L = int(dw.lens[b])
            first = L - w.chunk
            if w.cache_from_h:
                rows = O.latent_rows(dw.host_h_ctx(b), hw["w_dkv"], hw["w_kr"], np.arange(L),
                                     w.rope_base)
            else:
                rows = dw.host_pool_rows(b, L)
                hs = np.stack([dw.host_h(j) for j in np.flatnonzero(dw.q_seq_host == b)])
                rows[first:] = O.latent_rows(hs, hw["w_dkv"], hw["w_kr"], np.arange(first, L),
                                             w.rope_base)
            rows_of[b] = rows
        rows = rows_of[b][:p + 1]
        fn = O.mla_decode_step_absorbed if absorbed else O.mla_decode_step
        a = fn(dw.host_h(i), rows, hw["w_q"], hw["w_qr"], hw["w_uk"], hw["w_uv"], hw["w_o"], p,
               w.n_heads, w.d_head, w.d_latent, w.d_rope, w.rope_base)
        out["u"].append(a["u"])
        out["lse"].append(a["lse"])
        if absorbed:
            out["o_lat"].append(a["o_lat"])
    return {k: np.stack(v) for k, v in out.items() if v}


@pytest.mark.parametrize("name", ["tiny-pre", "lite-pre", "full-pre"])
def test_prefill_step(name):
    """absorb_q -> append (the chunk) -> prefill attention -> merge -> absorb_out
    with batch = the chunk's tokens; tiny checks every token against the
    non-absorbed definition, the others a seeded sample against the absorbed one."""
    w = I.WORKLOADS[name]
    note(f"prefill step {name}")
    dw = DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    assert M.mla_device_error() == 0
    hw = dw.host_weights()
    if name == "tiny-pre":
        idx = list(range(dw.nq))
    else:
        rng = np.random.default_rng(7)
        idx = sorted({0, dw.nq - 1, w.chunk - 1, w.chunk} | set(rng.choice(dw.nq, 4, replace=False).tolist()))
    ref = _step_ref(dw, hw, idx, absorbed=name != "tiny-pre")
    dw.merge_o_lat()     # the step's fused merge does not store o_lat
    got = {k: to_np(getattr(dw, k))[idx] for k in ref}
    for k in ref:
        assert_parity(got[k], ref[k], w.dtype, f"{k} tokens={idx}")
