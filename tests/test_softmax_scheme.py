"""The single-reference softmax the matrix-core attention kernels use, modelled
on the host in fp32 and pinned against the fp64 oracle.

The kernels accumulate a split's rows tile by tile with one exponent reference
per head, fixed at the maximum score of the split's first tile (log2 units), so
the accumulated output is never rescaled; the score chain is free to exceed
the reference by up to 2^64 (fp32 and bf16 both have the range), and a split
whose largest score lies further above it is accumulated once more with that
largest score as the reference.  This file states that scheme in plain numpy
and checks that it gives the softmax of [Report] §2.4 of
"《DeepSeek-V2》深度解读报告" (the sum of the content and RoPE scores) for
ordinary scores, for a spike far past the headroom, for one just under it and
for a first tile with no valid row.
"""
import math

import numpy as np

import oracle as O

TILE = 32
HEADROOM = 64.0
LOG2E = 1.0 / math.log(2.0)


def _scheme(scores, values, tile=TILE):
    """scores [n] (natural units, -inf = masked), values [n, d] -> (o, lse, passes)
    by the single-reference accumulation in fp32."""
    x = (np.asarray(scores, np.float64) * LOG2E).astype(np.float32)     # log2 units
    v = np.asarray(values, np.float32)
    ref = np.float32(np.max(x[:tile]))
    for passes in (1, 2):
        mr = np.float32(max(ref, np.float32(-1e30)))
        acc = np.zeros(v.shape[1], np.float32)
        tot = np.float32(0)
        seen = np.float32(-np.inf)
        pmax = np.float32(0)
        for a in range(0, len(x), tile):
            xs = x[a:a + tile]
            seen = max(seen, np.float32(xs.max()))
            p = np.exp2(xs - mr).astype(np.float32)
            pmax = max(pmax, np.float32(p.max()))
            acc += p @ v[a:a + tile]
            tot += np.float32(p.sum())
        if not seen > ref + HEADROOM:
            # the pass kept: no weight above 2^64, so sums of up to 2^60 rows of
            # magnitude up to 2^10 stay inside fp32's range
            assert pmax <= np.float32(2.0 ** HEADROOM)
            break
        ref = seen
    return acc / tot, (float(ref) + math.log2(float(tot))) * math.log(2.0), passes


def _oracle(scores, values):
    """Plain two-pass softmax average and log-sum-exp in fp64."""
    s = np.asarray(scores, np.float64)
    m = s.max()
    w = np.exp(s - m)
    return (w @ np.asarray(values, np.float64)) / w.sum(), m + math.log(w.sum())


def _check(scores, values, want_passes):
    o, lse, passes = _scheme(scores, values)
    ro, rl = _oracle(scores, values)
    assert passes == want_passes
    np.testing.assert_allclose(o, ro, rtol=0, atol=2e-5 * np.abs(ro).max() + 1e-6)
    assert abs(lse - rl) <= 1e-5 * max(1.0, abs(rl))


def test_ordinary_scores_take_one_pass():
    rng = np.random.default_rng(1)
    for n in (1, 31, 32, 33, 1000):
        _check(rng.standard_normal(n), rng.standard_normal((n, 8)), 1)


def test_spike_past_the_headroom_takes_a_second_pass():
    rng = np.random.default_rng(2)
    s = rng.standard_normal(500)
    s[300] = s[:TILE].max() + 90.0 / LOG2E            # 90 log2 units above the first tile
    _check(s, rng.standard_normal((500, 8)), 2)


def test_spike_just_under_the_headroom_stays_in_one_pass():
    rng = np.random.default_rng(3)
    s = rng.standard_normal(500)
    s[300] = s[:TILE].max() + 60.0 / LOG2E            # 2^60: representable, no second pass
    _check(s, rng.standard_normal((500, 8)), 1)


def test_first_tile_without_a_valid_row():
    """A first tile that is masked entirely (an unusable page): the reference is
    -inf, clamped for the exponent; the second pass takes the real maximum."""
    rng = np.random.default_rng(4)
    s = rng.standard_normal(200)
    s[:64] = -np.inf
    v = rng.standard_normal((200, 8))
    o, lse, passes = _scheme(s, v)
    ro, rl = _oracle(s[64:], v[64:])
    assert passes == 2
    np.testing.assert_allclose(o, ro, rtol=0, atol=2e-5)
    assert abs(lse - rl) <= 1e-5 * abs(rl) + 1e-6


def test_the_scheme_agrees_with_the_oracle_split_partials():
    """Latent rows and queries as the attention call sees them: the scheme on
    each split's scores equals the oracle's split partials (scores from the
    oracle's own definition s = tau (q_lat . c + q_pe . k^R))."""
    rng = np.random.default_rng(5)
    d_c, d_r, L, S = 32, 8, 300, 3
    rows = rng.standard_normal((L, d_c + d_r))
    q_lat, q_pe = rng.standard_normal((2, d_c)) * 0.5, rng.standard_normal((2, d_r))
    rows[250, :d_c] = 40.0 * np.sign(q_lat[1])        # spike for head 1 in a later tile
    tau = 1.0 / math.sqrt(24)
    ro, rl = O.attention_partials(q_lat, q_pe, rows, S, d_c, d_r, tau, 16)
    for s, (a, b) in enumerate(O.split_bounds(L, S, 16)):
        for i in range(2):
            sc = tau * (rows[a:b, :d_c] @ q_lat[i] + rows[a:b, d_c:] @ q_pe[i])
            o, lse, _ = _scheme(sc, rows[a:b, :d_c])
            np.testing.assert_allclose(o, ro[s, i], rtol=0, atol=3e-5 * np.abs(ro[s, i]).max())
            assert abs(lse - rl[s, i]) <= 1e-5 * max(1.0, abs(rl[s, i]))
