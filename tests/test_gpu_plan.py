"""Decode attention and merge over a length-proportional plan (mla_decode_plan,
mla_decode_attention_planned / _fp8_planned, mla_merge_lse_planned) against the
oracle: every unit's partial is the oracle's attention over exactly that unit's
rows, and the merged result the oracle's attention over the whole sequence.
Also: bad plan entries and unit ranges are flagged and taken as empty."""
import numpy as np
import pytest

import mla_latent_kv_dkv_amd as M
import oracle as O
from mla_latent_kv_dkv_amd import inputs as I
from mla_latent_kv_dkv_amd.harness import fill_fp8_pool
from tests.gpu_util import assert_parity, device_tensor, host_tensor, note, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PATHS = [0, 1]

CASES = [
    ("full", [1, 65, 1000, 4096, 0, 3000], 16),   # 128 heads, an empty sequence
    ("full", [33000, 100], 8),                     # long units: the page-id window reloads
    ("lite", [17, 4096, 130, 2], 12),              # 16 heads
    ("tiny", [1, 64, 100, 129], 5),                # fp32: the vector kernel
    ("full-fp8", [1, 65, 1000, 4096, 0], 10),      # FP8 pool
    ("lite-fp8", [17, 4096, 130, 2], 12),          # FP8 pool, 16 heads
]


@pytest.fixture(autouse=True)
def _path_reset():
    yield
    M.mla_set_kernel_path(0)


def _wl(name, **kw):
    fields = dict(I.WORKLOADS[name].__dict__)
    fields.update(kw)
    return I.Workload(**fields)


def _dims(w):
    return M.make_dims(w.hidden, w.n_heads, w.d_head, w.d_latent, w.d_rope, w.dtype, w.page_size,
                       w.rope_base)


def _setup(name, lens):
    w = _wl(name, batch=len(lens))
    lens = np.array(lens, dtype=np.int32)
    bt, total = I.page_table(w, lens)
    B, nh = len(lens), w.n_heads
    d = _dims(w)
    q_lat = device_tensor(torch, w, "q_lat_in", (B, nh, w.d_latent), 0.5).float().contiguous()
    q_pe = device_tensor(torch, w, "q_pe_in", (B, nh, w.d_rope), 1.0).float().contiguous()
    fp8 = w.cache == "fp8"
    if fp8:
        pool = torch.empty((total, M.mla_fp8_page_bytes(d)), dtype=torch.uint8, device="cuda")
        fill_fp8_pool(d, pool, I.stream_key(w.seed, "pool"))
    else:
        pool = device_tensor(torch, w, "pool", (total, w.page_size, w.row))
    hq = host_tensor(w, "q_lat_in", (B, nh, w.d_latent), 0.5)
    hp = host_tensor(w, "q_pe_in", (B, nh, w.d_rope), 1.0)
    return w, d, lens, bt, q_lat, q_pe, pool, hq, hp, fp8


def _rows(w, bt, b, L, fp8):
    if fp8:   # the oracle's dequantization of the seeded fp32 rows
        return np.stack([O.fp8_dequantize_row(*O.fp8_quantize_row(r, w.d_latent))
                         for r in I.pool_rows(w, bt, b, L, f32=True)]) if L else \
            np.zeros((0, w.row))
    return I.to_f64(w, I.pool_rows(w, bt, b, L))


@pytest.mark.parametrize("name,lens,target", CASES)
@pytest.mark.parametrize("path", PATHS)
def test_planned_attention_and_merge(name, lens, target, path):
    M.mla_set_kernel_path(path)
    w, d, lens, bt, q_lat, q_pe, pool, hq, hp, fp8 = _setup(name, lens)
    B, nh = len(lens), w.n_heads
    n, plan = M.mla_decode_plan(lens, w.page_size, target)
    units = plan[:3 * n].reshape(n, 3)
    note(f"planned attention {name} lens={lens.tolist()} target={target} units={n} path={path}")
    plan_d = torch.tensor(plan, device="cuda")
    o_part = torch.full((n, nh, w.d_latent), 123.0, device="cuda")
    lse_part = torch.full((n, nh), 123.0, device="cuda")
    attend = M.mla_decode_attention_fp8_planned if fp8 else M.mla_decode_attention_planned
    M.mla_device_error(clear=True)
    attend(d, q_lat, q_pe, pool, torch.tensor(bt, device="cuda"), plan_d, n, o_part, lse_part)
    o_lat = torch.full((B, nh, w.d_latent), 123.0, device="cuda")
    lse = torch.full((B, nh), 123.0, device="cuda")
    M.mla_merge_lse_planned(d, o_part, lse_part, plan_d, n, o_lat, lse)
    got_o, got_l = to_np(o_part), to_np(lse_part)
    got_m, got_ml = to_np(o_lat), to_np(lse)
    tau = M.default_scale(d)
    rows = {b: _rows(w, bt, b, int(lens[b]), fp8) for b in range(B)}
    for u, (b, t0, t1) in enumerate(units):
        ro, rl = O.attention_partials(hq[b], hp[b], rows[b][t0:t1], 1, w.d_latent, w.d_rope, tau,
                                      w.page_size)
        assert_parity(got_o[u], ro[0], w.dtype, f"o_part unit {u} ({b}, {t0}, {t1})")
        assert_parity(got_l[u], rl[0], w.dtype, f"lse_part unit {u}")
    for b in range(B):
        ro, rl = O.merge_lse(*O.attention_partials(hq[b], hp[b], rows[b], 1, w.d_latent, w.d_rope,
                                                   tau, w.page_size))
        assert_parity(got_m[b], ro, w.dtype, f"o_lat b={b}")
        assert_parity(got_ml[b], rl, w.dtype, f"lse b={b}")
    assert M.mla_device_error() == 0


@pytest.mark.parametrize("path", PATHS)
def test_plan_bad_entries_are_flagged(path):
    """A unit naming a sequence outside the batch, or a range past the table, is
    empty and sets bit 1 of the error word; so does a merge row whose unit range
    leaves [0, n_units].  The other units and rows are unaffected."""
    M.mla_set_kernel_path(path)
    w, d, lens, bt, q_lat, q_pe, pool, hq, hp, fp8 = _setup("full", [1000, 300])
    B, nh = 2, w.n_heads
    n, plan = M.mla_decode_plan(lens, w.page_size, 4)
    units = plan[:3 * n].reshape(n, 3).copy()
    bad = plan.copy()
    pad = int(plan[3 * n + B])        # first padding unit: no row merges it
    bad[3 * pad] = B                  # sequence outside the batch
    bad[3 * (pad + 1) + 2] = bt.shape[1] * w.page_size + 64   # range past the table
    plan_d = torch.tensor(bad, device="cuda")
    o_part = torch.full((n, nh, w.d_latent), 123.0, device="cuda")
    lse_part = torch.full((n, nh), 123.0, device="cuda")
    M.mla_device_error(clear=True)
    M.mla_decode_attention_planned(d, q_lat, q_pe, pool, torch.tensor(bt, device="cuda"), plan_d,
                                   n, o_part, lse_part)
    assert M.mla_device_error(clear=True) == 2
    got_l = to_np(lse_part)
    assert np.isneginf(got_l[pad]).all() and np.isneginf(got_l[pad + 1]).all()
    assert (to_np(o_part)[pad:pad + 2] == 0).all()
    tau = M.default_scale(d)
    rows0 = I.to_f64(w, I.pool_rows(w, bt, 0, 1000))
    b, t0, t1 = units[0]
    ro, rl = O.attention_partials(hq[b], hp[b], rows0[t0:t1], 1, w.d_latent, w.d_rope, tau, 64)
    assert_parity(to_np(o_part)[0], ro[0], w.dtype, "unit 0 beside the bad ones")
    # merge: row 1's range pointing past n_units
    merge_plan = plan.copy()
    merge_plan[3 * n + 2] = n + 5
    o_lat = torch.full((B, nh, w.d_latent), 123.0, device="cuda")
    lse = torch.full((B, nh), 123.0, device="cuda")
    M.mla_merge_lse_planned(d, o_part, lse_part, torch.tensor(merge_plan, device="cuda"), n,
                            o_lat, lse)
    assert M.mla_device_error(clear=True) == 2
    assert np.isneginf(to_np(lse)[1]).all() and (to_np(o_lat)[1] == 0).all()
