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
from tests.gpu_util import (assert_parity, attention_rounds_queries, bf16_round, note, rope_base,
                            to_np)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _context_rows(dw: DeviceWorkload, b: int, hw) -> np.ndarray:
    """fp64 rows 0..L-1 of sequence b as the oracle sees them: the decode token's
    row (and, for cache-from-h workloads, every row) from h through the oracle."""
    w, L = dw.w, int(dw.lens[b])
    if w.cache_from_h:
        h = dw.host_h_ctx(b)
        return O.latent_rows(h, hw["w_dkv"], hw["w_kr"], np.arange(L), rope_base(w))
    rows = dw.host_pool_rows(b, L)
    rows[L - 1] = O.latent_rows(dw.host_h(b)[None], hw["w_dkv"], hw["w_kr"], [L - 1],
                                rope_base(w))[0]
    return rows


def _check(dw: DeviceWorkload, seqs, full_def=(), hw=None, path=0, merge=True):
    """Compare u, q_lat, o_lat and lse of sequences ``seqs`` with the absorbed fp64
    companion and, for ``full_def``, u with the non-absorbed definition (o_lat, which
    the step's fused merge does not store, merged from the step's partials first
    unless ``merge`` is False: already done by the caller).  Where the
    attention runs on a matrix-core kernel, which rounds the queries it is handed
    to bf16 (its stated input precision), o_lat is compared with the oracle's
    attention over the oracle's own queries rounded the same way; u, q_lat and lse
    are always held against the exact oracle."""
    w = dw.w
    hw = hw or dw.host_weights()
    if merge:
        dw.merge_o_lat()
    got = {k: to_np(getattr(dw, k)) for k in ("u", "q_lat", "o_lat", "lse")}
    ref = {k: [] for k in got}
    rounded = attention_rounds_queries(w, path)
    tau = O.yarn_logit_factor(rope_base(w)) / np.sqrt(w.d_head + w.d_rope)
    for b in seqs:
        L = int(dw.lens[b])
        rows = _context_rows(dw, b, hw)
        cq = dict(w_dq=hw["w_dq"], w_uq=hw["w_uq"]) if w.d_cq else {}
        a = O.mla_decode_step_absorbed(dw.host_h(b), rows, hw.get("w_q"), hw["w_qr"], hw["w_uk"],
                                       hw["w_uv"], hw["w_o"], L - 1, w.n_heads, w.d_head,
                                       w.d_latent, w.d_rope, rope_base(w), **cq)
        if rounded:
            q_lat = a["q_lat"]
            if w.d_cq:     # the compressed query holds c^Q in the storage type (mla.h)
                c_q = bf16_round(hw["w_dq"] @ dw.host_h(b))
                q_lat = O.absorb_q(c_q, hw["w_uq"], np.zeros((w.n_heads * w.d_rope, w.d_cq)),
                                   hw["w_uk"], L - 1, w.n_heads, w.d_head, w.d_latent, w.d_rope,
                                   rope_base(w))[0]
            a["o_lat"] = O.merge_lse(*O.attention_partials(
                bf16_round(q_lat), bf16_round(a["q_pe"]), rows, 1, w.d_latent, w.d_rope,
                tau, w.page_size))[0]
        for k in ref:
            ref[k].append(a[k])
        if b in full_def:
            nd = O.mla_decode_step(dw.host_h(b), rows, hw.get("w_q"), hw["w_qr"], hw["w_uk"],
                                   hw["w_uv"], hw["w_o"], L - 1, w.n_heads, w.d_head, w.d_latent,
                                   w.d_rope, rope_base(w), **cq)
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
        _check(dw, [0], full_def=[0], path=path)
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
            dw.merge_o_lat()     # the layers share their partials: merge this layer's now
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
        _check(dw, seqs, full_def=full_def[l], merge=False)


@pytest.mark.parametrize("path", [0, 1])
def test_step_tiny_yarn(path):
    """YaRN-stretched RoPE (scale 4 over a 16-token window, so the 64 positions
    cross its ramp) and its temperature, cache built from h through the append."""
    M.load()
    M.mla_set_kernel_path(path)
    try:
        note(f"step tiny-yarn path={path}")
        dw = DeviceWorkload(I.WORKLOADS["tiny-yarn"])
        dw.step()
        torch.cuda.synchronize()
        _check(dw, [0], full_def=[0], path=path)
        assert M.mla_device_error() == 0
    finally:
        M.mla_set_kernel_path(0)


@pytest.mark.parametrize("name,seqs", [("full-yarn", [0, 40, 63]), ("long-yarn", [1])])
def test_step_yarn_full_shape(name, seqs):
    """The 4K -> 128K YaRN setting (scale 40, alpha 1, beta 32) at the full shape
    and at context 131072 with 64 splits."""
    note(f"step {name}")
    dw = DeviceWorkload(I.WORKLOADS[name])
    dw.step()
    torch.cuda.synchronize()
    _check(dw, seqs, full_def=seqs[:1])
    assert M.mla_device_error() == 0
