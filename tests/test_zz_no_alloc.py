"""mla_absorb_out_noalloc (the absorbed output with the library's static scratch
instead of a caller workspace) against mla_absorb_out on the same inputs: two
calls in a row, the second with a smaller batch, each bit-identical to the
workspace call (same kernels, same summation order)."""
import math

import numpy as np
import pytest

import mla_latent_kv_dkv_amd as M
import oracle as O
from mla_latent_kv_dkv_amd import inputs as I
from tests.gpu_util import assert_parity, device_tensor, note, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dims(w):
    return M.make_dims(w.hidden, w.n_heads, w.d_head, w.d_latent, w.d_rope, w.dtype, w.page_size,
                       w.rope_base)


@pytest.mark.parametrize("name,batches", [("full", (64, 9)), ("lite", (32, 3)), ("tiny", (5, 2))])
def test_absorb_out_noalloc_matches_the_workspace_call(name, batches):
    M.load()
    w = I.WORKLOADS[name]
    d = _dims(w)
    std = {n: 1 / math.sqrt(w.fan_in(n)) for n in ("w_uv", "w_o")}
    wuv = device_tensor(torch, w, "w_uv", w.weight_shape("w_uv"), std["w_uv"])
    wo = device_tensor(torch, w, "w_o", w.weight_shape("w_o"), std["w_o"])
    assert M.mla_absorb_out_noalloc_max_bytes() == 32 << 20
    for B in batches:
        note(f"absorb_out_noalloc {name} B={B}")
        o_lat = device_tensor(torch, w, f"o_lat_noalloc_{B}", (B, w.n_heads, w.d_latent),
                              dtype=torch.float32)
        u_ref = torch.full((B, w.hidden), 5.0, device="cuda")
        ws = torch.empty(M.mla_workspace_bytes(d, B), dtype=torch.uint8, device="cuda")
        M.mla_absorb_out(d, o_lat, wuv, wo, u_ref, ws)
        u = torch.full((B, w.hidden), -5.0, device="cuda")
        M.mla_absorb_out_noalloc(d, o_lat, wuv, wo, u)
        torch.cuda.synchronize()
        assert torch.equal(u, u_ref), f"B={B}: the static-scratch call differs"
        # and both against the oracle, on the first and last rows
        hu = I.to_f64(w, I.weight_values(w, "w_uv"))
        ho = I.to_f64(w, I.weight_values(w, "w_o"))
        hl = I.normal_f32(I.stream_key(w.seed, f"o_lat_noalloc_{B}"), 0,
                          B * w.n_heads * w.d_latent).astype(np.float64).reshape(B, w.n_heads, -1)
        rows = [0, B - 1]
        ref = np.stack([O.absorb_out(hl[b], hu, ho, w.n_heads, w.d_head, w.d_latent) for b in rows])
        assert_parity(to_np(u)[rows], ref, w.dtype, f"u B={B}")
    assert M.mla_device_error() == 0


def test_absorb_out_noalloc_rejects_a_batch_beyond_its_scratch():
    """Full shape at batch 4096: o alone is 128 MiB, past the 32 MiB array; the
    call returns MLA_ERR_WORKSPACE and enqueues nothing."""
    import ctypes
    lib = M.load()
    d = M.make_dims(5120, 128, 128, 512, 64, "bf16")
    p = ctypes.c_void_p(0x1000)
    assert lib.mla_absorb_out_noalloc(ctypes.byref(d), p, p, p, 4096, p, None) == -4
