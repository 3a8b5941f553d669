"""The seeded input generator: determinism, shapes, moments, spikes, samples."""

import numpy as np

from exact_attention_121_amd.inputs import WORKLOADS, make_inputs, make_qkv, sample_rows


def test_workload_table():
    w = WORKLOADS
    assert (w[1].B, w[1].Hq, w[1].N, w[1].d, w[1].causal) == (1, 1, 128, 64, False)
    assert (w[2].B, w[2].Hq, w[2].Hkv, w[2].N, w[2].d, w[2].causal) == (2, 32, 32, 2048, 128, False)
    assert (w[3].B, w[3].Hq, w[3].N, w[3].d, w[3].causal, w[3].spike_mult) == (8, 16, 4096, 64, True, 8.0)
    assert (w[4].Hq, w[4].Hkv, w[4].N, w[4].d, w[4].causal) == (32, 8, 8192, 256, True)
    assert (w[5].Hq, w[5].Hkv, w[5].N, w[5].d, w[5].sigma, w[5].sample_rows) == (32, 1, 131072, 128, 0.5, 256)
    assert w[2].scale == np.float32(1 / np.sqrt(128))
    assert w[2].flops == 4 * 128 * 2 * 32 * 2048 * 2048
    assert w[3].pairs == 8 * 16 * 4096 * 4097 // 2


def test_deterministic_and_seed_sensitive():
    a = make_qkv(1, 4, 2, 33, 64, seed=5)
    b = make_qkv(1, 4, 2, 33, 64, seed=5)
    c = make_qkv(1, 4, 2, 33, 64, seed=6)
    for x, y in zip(a, b):
        assert x.dtype == np.float16 and np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])
    assert a[0].shape == (1, 4, 33, 64) and a[1].shape == (1, 2, 33, 64) and a[2].shape == (1, 2, 33, 64)


def test_moments_and_sigma():
    q, k, v = make_qkv(1, 2, 2, 4096, 64, seed=3, sigma=0.5)
    for x in (q, k, v):
        x = x.astype(np.float64)
        assert abs(x.mean()) < 0.01 and abs(x.std() - 0.5) < 0.01


def test_tiny_workload_matches_recipe():
    q, k, v = make_inputs(WORKLOADS[1])
    rng = np.random.default_rng(1001)
    want_q = rng.standard_normal((128, 64), dtype=np.float32).astype(np.float16)
    assert np.array_equal(q[0, 0], want_q)


def test_spike_rows_exact_count():
    B, H, N, d = 2, 3, 500, 64
    q, k, v = make_qkv(B, H, H, N, d, seed=11, spike_frac=0.01, spike_mult=8.0)
    plain_q, plain_k, plain_v = make_qkv(B, H, H, N, d, seed=11)
    count = round(0.01 * B * H * N)
    # Q is drawn first from the same stream, so its unspiked values coincide.
    ratio = q.astype(np.float32).reshape(-1, d) / np.where(plain_q == 0, 1, plain_q).astype(np.float32).reshape(-1, d)
    spiked = np.isclose(np.median(ratio, axis=1), 8.0, rtol=1e-2)
    assert spiked.sum() == count
    assert np.array_equal(q.reshape(-1, d)[~spiked], plain_q.reshape(-1, d)[~spiked])
    assert np.abs(k.astype(np.float32)).max() > 5 * np.abs(v.astype(np.float32)).max() / 2


def test_sample_rows():
    w = WORKLOADS[5]
    r = sample_rows(w)
    assert r.shape == (1, 32, 256)
    for h in range(32):
        row = r[0, h]
        assert row[0] == 0 and row[-1] == w.N - 1
        assert len(np.unique(row)) == 256 and np.all(np.diff(row) > 0)
    assert not np.array_equal(r[0, 0], r[0, 1])
    assert np.array_equal(r, sample_rows(w))
    small = sample_rows(WORKLOADS[1], count=1000)
    assert np.array_equal(small[0, 0], np.arange(128))


def test_bf16_rounding_matches_torch():
    """round_to_bf16 is round-to-nearest-even to bfloat16: torch's own fp32 ->
    bf16 conversion gives the same values (ties included)."""
    import numpy as np
    import torch

    from exact_attention_121_amd.inputs import round_to_bf16
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-8, 8, 20000),
                        # exact ties between two bf16 values, both parities
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.0 - 2.0 ** -7, 0.0], np.float32)])
    assert np.array_equal(round_to_bf16(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())
