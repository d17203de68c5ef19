"""The seeded input generator: determinism, shapes and distributions."""

import numpy as np
import pytest

from chunked_kda_prefill_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -0.0, 65504.0,
                                  1e-30, -3.3895314e38], dtype=np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_tiny_is_deterministic_and_well_formed():
    a, b = wl.tiny(), wl.tiny()
    for name in ("q", "k", "v", "g", "beta"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    assert a.q.shape == (256, 2, 128) and a.q.dtype == np.uint16
    assert a.g.dtype == np.float32 and a.beta.shape == (256, 2)
    assert a.initial_state.shape == (1, 2, 128, 128)
    assert not a.initial_state.any()
    assert list(a.cu_seqlens) == [0, 256]
    assert a.num_chunks() == 4
    g = a.g
    assert g.max() <= 0.0 and g.min() >= -5.0
    k = wl.bf16_bits_to_f32(a.k).astype(np.float64)
    nrm = np.linalg.norm(k, axis=-1)
    assert np.allclose(nrm, 1.0, atol=5e-3)
    q = wl.bf16_bits_to_f32(a.q).astype(np.float64)
    assert abs(np.std(q) * np.sqrt(128) - 1.0) < 0.05
    assert 0.0 < a.beta.min() and a.beta.max() < 1.0


def test_sharegpt_like_lengths():
    rng = np.random.default_rng(2)
    L = wl.sharegpt_like_lengths(rng, 64)
    assert L.shape == (64,)
    assert L.min() >= 15 and L.max() <= 8192
    assert not np.any(L % 64 == 0)
    assert 300 < np.median(L) < 1200


def test_pinned_channels_sit_at_the_lower_bound():
    w = wl.make_workload("p", [100], H=3, seed=5, pinned_fraction=0.10)
    for h in range(3):
        pinned = np.all(w.g[:, h, :] == -5.0, axis=0)
        assert pinned.sum() == 13


def test_batch_workload_has_nonzero_initial_state():
    w = wl.make_workload("b", [64, 64], H=2, seed=9, h0="normal")
    assert w.initial_state.shape == (2, 2, 128, 128)
    assert abs(float(np.std(w.initial_state)) - 0.1) < 0.01


def test_algorithmic_counts():
    w = wl.tiny()
    assert wl.algorithmic_bytes(w) == 256 * 2 * 1540 + 2 * 1 * 2 * 65536
    assert wl.algorithmic_flops(w) == 256 * 2 * 154624
