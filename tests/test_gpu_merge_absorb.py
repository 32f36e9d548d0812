"""mla_merge_absorb_out: the split merge folded into the W_UV product.

Against the two calls it replaces (mla_merge_lse or mla_merge_lse_planned, then
mla_absorb_out) bit for bit on every path, and against the oracle's merge
followed by its absorbed output at the bf16 bar.  Cases: uniform splits with
empty splits and an all-empty (row, head), batches that leave a ragged 64-row
block, length-proportional plans (an empty sequence among them), lse omitted,
and a plan range outside the unit list (flagged, the row merges nothing).
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

PATHS = [0, 1]


@pytest.fixture(autouse=True)
def _path_reset():
    M.load()
    yield
    M.mla_set_kernel_path(0)


def _dims(w):
    return M.make_dims(w.hidden, w.n_heads, w.d_head, w.d_latent, w.d_rope, w.dtype, w.page_size,
                       w.rope_base)


def _weights(w):
    std = {n: 1 / math.sqrt(w.fan_in(n)) for n in ("w_uv", "w_o")}
    dev = {n: device_tensor(torch, w, n, w.weight_shape(n), std[n]) for n in std}
    host = {n: host_tensor(w, n, w.weight_shape(n), std[n]) for n in std}
    return dev, host


def _partials(w, n_rows, nh, empty):
    """Seeded partials [n_rows, nh, d_c] and lse [n_rows, nh] (device and fp64 host),
    with lse = -inf (and o = 0, as the attention writes them) at the `empty` mask."""
    o = device_tensor(torch, w, "o_part_in", (n_rows, nh, w.d_latent), 1.0, dtype=torch.float32)
    lse = device_tensor(torch, w, "lse_part_in", (n_rows, nh), 3.0, dtype=torch.float32)
    o_h = I.normal_f32(I.stream_key(w.seed, "o_part_in"), 0, n_rows * nh * w.d_latent).astype(
        np.float64).reshape(n_rows, nh, w.d_latent)
    l_h = I.normal_f32(I.stream_key(w.seed, "lse_part_in"), 0, n_rows * nh, 3.0).astype(
        np.float64).reshape(n_rows, nh)
    m = torch.tensor(empty, device="cuda")
    lse[m] = -math.inf
    o[m] = 0.0
    l_h[empty] = -np.inf
    o_h[empty] = 0.0
    return o, lse, o_h, l_h


def _two_calls(d, o_part, lse_part, wdev, B, plan=None, n_units=0):
    nh = d.n_heads
    o_lat = torch.empty((B, nh, d.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, nh), dtype=torch.float32, device="cuda")
    if plan is None:
        M.mla_merge_lse(d, o_part, lse_part, o_lat, lse)
    else:
        M.mla_merge_lse_planned(d, o_part, lse_part, plan, n_units, o_lat, lse)
    u = torch.empty((B, d.hidden), dtype=torch.float32, device="cuda")
    ws = torch.empty(M.mla_workspace_bytes(d, B), dtype=torch.uint8, device="cuda")
    M.mla_absorb_out(d, o_lat, wdev["w_uv"], wdev["w_o"], u, ws)
    return u, lse


def _fused(d, o_part, lse_part, wdev, B, plan=None, n_units=0, with_lse=True):
    u = torch.full((B, d.hidden), 123.0, dtype=torch.float32, device="cuda")
    lse = torch.full((B, d.n_heads), 123.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(M.mla_merge_absorb_out_workspace_bytes(d, B), dtype=torch.uint8,
                     device="cuda")
    M.mla_merge_absorb_out(d, o_part, lse_part, wdev["w_uv"], wdev["w_o"], u, ws,
                           lse=lse if with_lse else None, plan=plan, n_units=n_units)
    return u, lse


def _oracle_rows(w, host, o_h, l_h, groups):
    """u and lse of the oracle's merge of each row's partial indices, then its
    absorbed output."""
    us, ls = [], []
    for idx in groups:
        if len(idx):
            o, l = O.merge_lse(o_h[idx], l_h[idx])
        else:
            o, l = np.zeros((w.n_heads, w.d_latent)), np.full(w.n_heads, -np.inf)
        us.append(O.absorb_out(o, host["w_uv"], host["w_o"], w.n_heads, w.d_head, w.d_latent))
        ls.append(l)
    return np.stack(us), np.stack(ls)


# full B = 6, S = 4: the fused product; S = 1: no merge at all; B = 70 (past one 64-row
# block), S = 64 (long rows), lite (a small grid) and tiny (fp32): the two calls inside
@pytest.mark.parametrize("name,B,S", [("full", 6, 4), ("full", 6, 1), ("full", 70, 3),
                                      ("full", 3, 64), ("lite", 9, 8), ("tiny", 5, 3)])
@pytest.mark.parametrize("path", PATHS)
def test_merge_absorb_out_uniform(name, B, S, path):
    w = I.WORKLOADS[name]
    nh = w.n_heads
    M.mla_set_kernel_path(path)
    note(f"merge_absorb_out {name} B={B} S={S} path={path}")
    d = _dims(w)
    wdev, host = _weights(w)
    empty = np.zeros((B * S, nh), dtype=bool)
    empty.reshape(B, S, nh)[1, ::2] = True       # every other split of row 1
    empty.reshape(B, S, nh)[2, :, 0] = True      # every split of (row 2, head 0)
    if S > 1:
        empty.reshape(B, S, nh)[0, 1:] = True    # row 0: one live split
    o, lse, o_h, l_h = _partials(w, B * S, nh, empty)
    o4, lse3 = o.view(B, S, nh, w.d_latent), lse.view(B, S, nh)
    M.mla_device_error(clear=True)
    u_f, lse_f = _fused(d, o4, lse3, wdev, B)
    u_t, lse_t = _two_calls(d, o4, lse3, wdev, B)
    np.testing.assert_array_equal(to_np(u_f), to_np(u_t))
    np.testing.assert_array_equal(to_np(lse_f), to_np(lse_t))
    # the oracle on sampled rows: the empty cases, both sides of the 64-row block edge, the last
    rows = sorted({0, 1, 2, B // 2, B - 1} | ({63, 64} if B > 64 else set()))
    ru, rl = _oracle_rows(w, host, o_h, l_h, [list(range(b * S, (b + 1) * S)) for b in rows])
    assert_parity(to_np(u_f)[rows], ru, w.dtype, "u")
    assert_parity(to_np(lse_f)[rows], rl, w.dtype, "lse")
    assert np.isneginf(to_np(lse_f)[2, 0])
    # lse omitted: the same u
    u_n, _ = _fused(d, o4, lse3, wdev, B, with_lse=False)
    np.testing.assert_array_equal(to_np(u_n), to_np(u_f))
    assert M.mla_device_error() == 0


@pytest.mark.parametrize("name,lens,target", [("full", [1, 65, 1000, 4096, 0, 3000, 33000, 7], 24),
                                              ("lite", [17, 4096, 130, 2], 12)])
@pytest.mark.parametrize("path", PATHS)
def test_merge_absorb_out_planned(name, lens, target, path):
    w = I.WORKLOADS[name]
    nh, B = w.n_heads, len(lens)
    M.mla_set_kernel_path(path)
    n, plan = M.mla_decode_plan(lens, w.page_size, target)
    note(f"merge_absorb_out planned {name} lens={lens} units={n} path={path}")
    d = _dims(w)
    wdev, host = _weights(w)
    starts = plan[3 * n:]
    empty = np.zeros((n, nh), dtype=bool)
    empty[starts[1]] = True                      # all heads of row 1's first unit
    units = plan[:3 * n].reshape(n, 3)
    empty[(units[:, 1] == units[:, 2])] = True   # empty units (the empty sequence, padding)
    o, lse, o_h, l_h = _partials(w, n, nh, empty)
    plan_d = torch.tensor(plan, device="cuda")
    M.mla_device_error(clear=True)
    u_f, lse_f = _fused(d, o, lse, wdev, B, plan=plan_d, n_units=n)
    u_t, lse_t = _two_calls(d, o, lse, wdev, B, plan=plan_d, n_units=n)
    np.testing.assert_array_equal(to_np(u_f), to_np(u_t))
    np.testing.assert_array_equal(to_np(lse_f), to_np(lse_t))
    groups = [list(range(starts[b], starts[b + 1])) for b in range(B)]
    ru, rl = _oracle_rows(w, host, o_h, l_h, groups)
    assert_parity(to_np(u_f), ru, w.dtype, "u")
    assert_parity(to_np(lse_f), rl, w.dtype, "lse")
    assert M.mla_device_error() == 0


@pytest.mark.parametrize("path", PATHS)
def test_merge_absorb_out_bad_plan_range(path):
    """Row 1's unit range pointing past n_units is flagged (bit 1 of the error
    word) and merges nothing: lse -inf and u = W_O W_UV 0 = 0 for that row."""
    w = I.WORKLOADS["full"]
    nh, lens = w.n_heads, [1000, 300, 64]
    M.mla_set_kernel_path(path)
    note(f"merge_absorb_out bad plan range path={path}")
    n, plan = M.mla_decode_plan(lens, w.page_size, 4)
    d = _dims(w)
    wdev, host = _weights(w)
    o, lse, o_h, l_h = _partials(w, n, nh, np.zeros((n, nh), dtype=bool))
    bad = plan.copy()
    bad[3 * n + 2] = n + 5
    M.mla_device_error(clear=True)
    u_f, lse_f = _fused(d, o, lse, wdev, 3, plan=torch.tensor(bad, device="cuda"), n_units=n)
    assert M.mla_device_error(clear=True) == 2
    assert np.isneginf(to_np(lse_f)[1]).all() and (to_np(u_f)[1] == 0).all()
    starts = plan[3 * n:]
    ru, rl = _oracle_rows(w, host, o_h, l_h, [list(range(starts[0], starts[1]))])
    assert_parity(to_np(u_f)[:1], ru, w.dtype, "u row 0 beside the bad one")


def test_merge_absorb_out_256_rows_bf16_merge():
    """256 rows (the ragged batch): W_UV runs on the tiled product, so the merge
    writes its rows in bf16, the precision that product reads them in.  u and lse
    equal the two calls' bit for bit (mla_merge_lse writes fp32 o_lat, which
    mla_absorb_out's product rounds the same way), and the oracle's on sampled rows."""
    w = I.WORKLOADS["full"]
    B, S, nh = 256, 3, w.n_heads
    note(f"merge_absorb_out full B={B} S={S} (bf16 merge rows)")
    d = _dims(w)
    wdev, host = _weights(w)
    empty = np.zeros((B * S, nh), dtype=bool)
    empty.reshape(B, S, nh)[1, ::2] = True
    empty.reshape(B, S, nh)[2, :, 0] = True
    empty.reshape(B, S, nh)[0, 1:] = True
    o, lse, o_h, l_h = _partials(w, B * S, nh, empty)
    o4, lse3 = o.view(B, S, nh, w.d_latent), lse.view(B, S, nh)
    M.mla_device_error(clear=True)
    u_f, lse_f = _fused(d, o4, lse3, wdev, B)
    u_t, lse_t = _two_calls(d, o4, lse3, wdev, B)
    np.testing.assert_array_equal(to_np(u_f), to_np(u_t))
    np.testing.assert_array_equal(to_np(lse_f), to_np(lse_t))
    rows = [0, 1, 2, 127, 128, B - 1]
    ru, rl = _oracle_rows(w, host, o_h, l_h, [list(range(b * S, (b + 1) * S)) for b in rows])
    assert_parity(to_np(u_f)[rows], ru, w.dtype, "u")
    assert_parity(to_np(lse_f)[rows], rl, w.dtype, "lse")
    assert M.mla_device_error() == 0
