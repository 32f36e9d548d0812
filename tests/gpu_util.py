"""Helpers shared by the GPU parity tests (tolerances, host copies, set-up)."""
import sys

import numpy as np

from mla_latent_kv_dkv_amd import inputs as I

# Tolerances of the decode outputs against the fp64 oracle: max |err| <= 1e-4 for
# fp32 storage, <= 2e-2 * RMS(oracle tensor) for bf16 storage.
F32_ABS = 1e-4
BF16_REL_RMS = 2e-2


def note(msg):
    """Name the case on stdout before a GPU step (flushed)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def assert_parity(got, ref, dtype, what=""):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: non-finite pattern differs"
    assert np.array_equal(got[~fin], ref[~fin]), f"{what}: infinities differ"
    if not fin.any():
        return
    err = np.abs(got[fin] - ref[fin]).max()
    if dtype == "f32":
        note(f"  {what}: max|err| {err:.3e} (bound {F32_ABS})")
        assert err <= F32_ABS, f"{what}: max|err| {err:.3e} > {F32_ABS}"
    else:
        rms = np.sqrt(np.mean(ref[fin] ** 2))
        note(f"  {what}: max|err|/rms {err / rms if rms > 0 else err:.4f} (bound {BF16_REL_RMS})")
        assert err <= BF16_REL_RMS * rms, f"{what}: max|err| {err:.3e} > {BF16_REL_RMS} * rms {rms:.3e}"
    return err


def assert_partials_within_weight_rounding(got, ref, q_lat, q_pe, rows, length, num_splits,
                                           page, tau, d_latent, what="", exact_normaliser=False):
    """Split partials of an MFMA path, element by element.  The bf16-pool kernel
    rounds each softmax weight p_j to bf16 (round to nearest even: relative error
    at most 2^-8) before the product with the latent rows and normalises by the
    sum of the rounded weights, so its output is sum_j p_j (1 + e_j) c_j /
    sum_j p_j (1 + e_j) with |e_j| <= 2^-8; element (i, k) of split s is then off
    from the exact average o_ik by at most
    2^-8 * sum_j p_j |c_jk - o_ik| / ((1 - 2^-8) sum_j p_j).
    With ``exact_normaliser`` (the FP8-pool kernel: weights carried as two e4m3
    terms, relative error at most 2^-8, normalised by the sum of the exact
    weights) the output is sum_j p_j (1 + e_j) c_j / sum_j p_j, off by at most
    2^-8 * sum_j p_j |c_jk| / sum_j p_j.
    The bound taken is that, with p_j and o_ik from fp64 scores computed here,
    widened by 1% (and 1e-6 absolute) for the fp32 rounding of scores and sums.
    Queries must be exactly representable in bf16.  A wrong row, scale or index
    lands far outside."""
    import oracle as O
    rows = np.asarray(rows, np.float64)[:length]
    for s, (a, b) in enumerate(O.split_bounds(length, num_splits, page)):
        if a >= b:
            continue
        c = rows[a:b, :d_latent]
        sc = tau * (c @ q_lat.T + rows[a:b, d_latent:] @ q_pe.T)        # [tokens, heads]
        p = np.exp(sc - sc.max(axis=0))
        o = (p.T @ c) / p.sum(axis=0)[:, None]                           # [heads, d_c]
        if exact_normaliser:
            bound = 1.01 * 2.0 ** -8 * (p.T @ np.abs(c)) / p.sum(axis=0)[:, None] + 1e-6
        else:
            dev = np.stack([p[:, i] @ np.abs(c - o[i]) for i in range(p.shape[1])])
            bound = 1.01 * 2.0 ** -8 * dev / ((1 - 2.0 ** -8) * p.sum(axis=0)[:, None]) + 1e-6
        err = np.abs(np.asarray(got[s], np.float64) - ref[s])
        worst = (err / bound).max()
        note(f"  o_part {what} split {s}: max err / bound {worst:.3f}")
        assert worst <= 1.0, f"o_part {what} split {s}: error {worst:.2f}x the weight-rounding bound"


def attention_rounds_queries(w, path: int = 0) -> bool:
    """True when the decode attention of workload ``w`` runs on a matrix-core
    kernel (kernel path 0, bf16 storage, n_h 128 or 16 -- 128 only for the FP8
    pool --, d_c 512, d_R 64, 64-token pages), which rounds q_lat and q_pe to
    bf16 once per work unit as include/mla.h states; the vector kernels keep
    them in fp32."""
    heads = (128,) if w.cache == "fp8" else (128, 16)
    return (path == 0 and w.dtype == "bf16" and w.n_heads in heads and w.d_latent == 512 and
            w.d_rope == 64 and w.page_size == 64)


def bf16_round(x):
    """Values rounded to bf16 (nearest even), as fp64."""
    return I.bf16_bits_to_f64(I.f32_to_bf16_bits(np.asarray(x, np.float32)))


def rope_base(w):
    """The RoPE ``base`` argument of the oracle for workload ``w``: its base, or the
    oracle's YaRN description when the workload stretches RoPE."""
    import oracle as O
    return O.Yarn(w.rope_base, *w.yarn) if w.yarn else w.rope_base


def host_tensor(w, name, shape, std=1.0, layer=0):
    return I.to_f64(w, I.tensor_values(w, name, shape, std, layer))


def device_tensor(torch, w, name, shape, std=1.0, layer=0, dtype=None):
    dt = dtype or (torch.float32 if w.dtype == "f32" else torch.bfloat16)
    t = torch.empty(shape, dtype=dt, device="cuda")
    I.fill_device(t, I.stream_key(w.seed, name, layer), std)
    return t
