"""Host checks of the seeded input generator (no GPU)."""
import math

import numpy as np
import pytest

from mla_latent_kv_dkv_amd import inputs as I


def test_splitmix64_published_first_outputs():
    # SplitMix64 seeded with 0: the first outputs of the published generator
    got = [int(x) for x in I.words(0, 0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_counter_based_random_access():
    key = I.stream_key(7, "pool", 3)
    whole = I.normal_f32(key, 0, 5000)
    np.testing.assert_array_equal(I.normal_f32(key, 1234, 100), whole[1234:1334])
    assert I.stream_key(7, "pool", 3) != I.stream_key(7, "pool", 4) != I.stream_key(8, "pool", 3)


def test_normal_statistics():
    v = I.normal_f32(I.stream_key(1, "x"), 0, 1 << 20, std=0.5).astype(np.float64)
    assert abs(v.mean()) < 3e-3 and abs(v.std() - 0.5) < 3e-3
    assert np.abs(v).max() <= 0.5 * 131070 / (math.sqrt(4 * (65536.0 ** 2 - 1) / 12)) + 1e-6


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.concatenate([I.normal_f32(I.stream_key(2, "y"), 0, 100000, 3.0),
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(I.f32_to_bf16_bits(x), ref)
    np.testing.assert_allclose(I.bf16_bits_to_f64(ref), torch.from_numpy(x).to(torch.bfloat16)
                               .double().numpy(), rtol=0, atol=0)


@pytest.mark.parametrize("name", list(I.WORKLOADS))
def test_page_tables_are_valid(name):
    w = I.WORKLOADS[name]
    lens = I.seq_lengths(w)
    bt, total = I.page_table(w, lens)
    pages = (lens + w.page_size - 1) // w.page_size
    used = np.concatenate([bt[b, :pages[b]] for b in range(w.batch)])
    assert sorted(used.tolist()) == list(range(total))
    if not w.permute_pages:
        np.testing.assert_array_equal(used, np.arange(total))
    if w.ragged:
        lo, hi = w.ragged
        assert lens.min() >= lo and lens.max() <= hi and len(set(lens.tolist())) > w.batch // 2


def test_pool_rows_follow_the_page_table():
    w = I.Workload("t", 16, 2, 4, 8, 4, "bf16", 3, 150, 99, page_size=16)
    lens = I.seq_lengths(w)
    bt, total = I.page_table(w, lens)
    flat = I.tensor_values(w, "pool", (total * w.page_size, w.row))
    for b in range(w.batch):
        rows = I.pool_rows(w, bt, b, int(lens[b]))
        for j in (0, 15, 16, 149):
            np.testing.assert_array_equal(rows[j], flat[bt[b, j // 16] * 16 + j % 16])
