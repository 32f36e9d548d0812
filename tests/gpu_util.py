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
        note(f"  {what}: max|err|/rms {err / rms:.4f} (bound {BF16_REL_RMS})")
        assert err <= BF16_REL_RMS * rms, f"{what}: max|err| {err:.3e} > {BF16_REL_RMS} * rms {rms:.3e}"
    return err


def assert_partials_within_weight_rounding(got, ref, q_lat, q_pe, rows, length, num_splits,
                                           page, tau, d_latent, what=""):
    """Split partials of a bf16 MFMA path, element by element.  That path rounds
    each softmax weight p_j to bf16 (relative error <= 2^-9) before the product
    with the latent rows, while the normaliser sum_j p_j is kept in fp32, so
    output element (i, k) of split s may be off by up to
    2^-9 * sum_j p_j |c_jk| / sum_j p_j.  The bound taken is twice that (2^-8,
    leaving room for the fp32 rounding of scores and sums) with the weighted mean
    of |c| computed here from fp64 scores, plus 1e-6.  Queries must be exactly
    representable in bf16.  A wrong row, scale or index lands far outside."""
    import oracle as O
    rows = np.asarray(rows, np.float64)[:length]
    for s, (a, b) in enumerate(O.split_bounds(length, num_splits, page)):
        if a >= b:
            continue
        c = rows[a:b, :d_latent]
        sc = tau * (c @ q_lat.T + rows[a:b, d_latent:] @ q_pe.T)        # [tokens, heads]
        p = np.exp(sc - sc.max(axis=0))
        bound = 2.0 ** -8 * (p.T @ np.abs(c)) / p.sum(axis=0)[:, None] + 1e-6
        err = np.abs(np.asarray(got[s], np.float64) - ref[s])
        worst = (err / bound).max()
        note(f"  o_part {what} split {s}: max err / bound {worst:.3f}")
        assert worst <= 1.0, f"o_part {what} split {s}: error {worst:.2f}x the weight-rounding bound"


def host_tensor(w, name, shape, std=1.0, layer=0):
    return I.to_f64(w, I.tensor_values(w, name, shape, std, layer))


def device_tensor(torch, w, name, shape, std=1.0, layer=0, dtype=None):
    dt = dtype or (torch.float32 if w.dtype == "f32" else torch.bfloat16)
    t = torch.empty(shape, dtype=dt, device="cuda")
    I.fill_device(t, I.stream_key(w.seed, name, layer), std)
    return t
