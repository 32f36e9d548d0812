"""End-to-end parity of one decode step (absorb_q -> append -> attention ->
merge -> absorb_out) on the five workloads, against the fp64 oracle.

Small workloads are checked on every sequence; the large ones at their full
sizes on seeded samples of sequences (and layers), the shortest and longest
included.  The oracle's inputs are regenerated on the host from the seed.
"""
import numpy as np
import pytest

import mla_latent_kv_dkv_amd as M
import oracle as O
from mla_latent_kv_dkv_amd import inputs as I
from mla_latent_kv_dkv_amd.harness import DeviceWorkload
from tests.gpu_util import assert_parity, note, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _context_rows(dw: DeviceWorkload, b: int, hw) -> np.ndarray:
    """fp64 rows 0..L-1 of sequence b as the oracle sees them: the decode token's
    row (and, for cache-from-h workloads, every row) from h through the oracle."""
    w, L = dw.w, int(dw.lens[b])
    if w.cache_from_h:
        h = dw.host_h_ctx(b)
        return O.latent_rows(h, hw["w_dkv"], hw["w_kr"], np.arange(L), w.rope_base)
    rows = dw.host_pool_rows(b, L)
    rows[L - 1] = O.latent_rows(dw.host_h(b)[None], hw["w_dkv"], hw["w_kr"], [L - 1],
                                w.rope_base)[0]
    return rows


def _check(dw: DeviceWorkload, seqs, full_def=(), hw=None):
    """Compare u, q_lat, o_lat and lse of sequences ``seqs`` with the absorbed fp64
    companion and, for ``full_def``, u with the non-absorbed definition."""
    w = dw.w
    hw = hw or dw.host_weights()
    got = {k: to_np(getattr(dw, k)) for k in ("u", "q_lat", "o_lat", "lse")}
    ref = {k: [] for k in got}
    for b in seqs:
        L = int(dw.lens[b])
        rows = _context_rows(dw, b, hw)
        cq = dict(w_dq=hw["w_dq"], w_uq=hw["w_uq"]) if w.d_cq else {}
        a = O.mla_decode_step_absorbed(dw.host_h(b), rows, hw.get("w_q"), hw["w_qr"], hw["w_uk"],
                                       hw["w_uv"], hw["w_o"], L - 1, w.n_heads, w.d_head,
                                       w.d_latent, w.d_rope, w.rope_base, **cq)
        for k in ref:
            ref[k].append(a[k])
        if b in full_def:
            nd = O.mla_decode_step(dw.host_h(b), rows, hw.get("w_q"), hw["w_qr"], hw["w_uk"],
                                   hw["w_uv"], hw["w_o"], L - 1, w.n_heads, w.d_head, w.d_latent,
                                   w.d_rope, w.rope_base, **cq)
            assert_parity(got["u"][b], nd["u"], w.dtype, f"u (definition) b={b}")
    for k in ref:
        assert_parity(got[k][list(seqs)], np.stack(ref[k]), w.dtype, f"{k} seqs={list(seqs)}")


@pytest.mark.parametrize("path", [0, 1])
def test_step_tiny_fp32(path):
    M.load()
    M.mla_set_kernel_path(path)
    try:
        note(f"step tiny path={path}")
        dw = DeviceWorkload(I.WORKLOADS["tiny"])
        dw.step()
        torch.cuda.synchronize()
        _check(dw, [0], full_def=[0])
        assert M.mla_device_error() == 0
    finally:
        M.mla_set_kernel_path(0)


def test_step_lite_cache_built_by_append():
    note("step lite (cache from h)")
    dw = DeviceWorkload(I.WORKLOADS["lite"])
    dw.step()
    torch.cuda.synchronize()
    _check(dw, [0, 17, 31], full_def=[17])
    assert M.mla_device_error() == 0


def test_step_full_shape():
    note("step full shape B=64 L=4096")
    dw = DeviceWorkload(I.WORKLOADS["full"])
    dw.step()
    torch.cuda.synchronize()
    _check(dw, [0, 31, 63], full_def=[31])
    assert M.mla_device_error() == 0


@pytest.mark.parametrize("name", ["tiny-cq", "lite-cq", "full-cq"])
def test_step_compressed_query(name):
    """The step with the query's low-rank compression (c^Q = W_DQ h, q^C = W_UQ c^Q)."""
    w = I.WORKLOADS[name]
    note(f"step {name}")
    dw = DeviceWorkload(w)
    dw.step()
    torch.cuda.synchronize()
    seqs = list(range(w.batch)) if w.batch <= 4 else [0, w.batch // 2, w.batch - 1]
    _check(dw, seqs, full_def=seqs[:1])
    assert M.mla_device_error() == 0


def test_step_long_context_64_splits():
    note("step long context B=4 L=131072 S=64")
    dw = DeviceWorkload(I.WORKLOADS["long"])
    dw.step()
    torch.cuda.synchronize()
    _check(dw, [2], full_def=[2])      # the non-absorbed definition over all 131072 tokens
    assert M.mla_device_error() == 0


def test_step_ragged_60_layers():
    """256 sequences, lengths log-uniform in [512, 32768], permuted 64-token pages,
    60 layers with independent weights run back to back; layers 0 and 59 are
    checked on the shortest, the longest and a seeded third sequence."""
    w = I.WORKLOADS["ragged"]
    lens = I.seq_lengths(w)
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 100})
    note(f"step ragged 60 layers, checked seqs {seqs} lens {[int(lens[s]) for s in seqs]}")
    layers = [DeviceWorkload(w, layer=0)]
    layers += [DeviceWorkload(w, layer=l, outputs_from=layers[0]) for l in range(1, w.layers)]
    saved = {}
    for l, dw in enumerate(layers):
        dw.step()
        if l in (0, w.layers - 1):
            saved[l] = {k: getattr(dw, k).clone() for k in ("u", "q_lat", "o_lat", "lse")}
    torch.cuda.synchronize()
    assert M.mla_device_error() == 0
    # the non-absorbed definition on two (layer, sequence) pairs: the longest
    # sequence of layer 0 and the shortest of layer 59
    full_def = {0: [int(np.argmax(lens))], w.layers - 1: [int(np.argmin(lens))]}
    for l, outs in saved.items():
        dw = layers[l]
        for k, v in outs.items():
            setattr(dw, k, v)
        note(f"oracle layer {l}")
        _check(dw, seqs, full_def=full_def[l])
