"""Pins of the oracle's conversions, LM-head product and row statistics."""
import numpy as np
import pytest
import scipy.special

from oracle import bf16, rules


def torch_bf16_bits(x32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_matches_torch_random():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    assert np.array_equal(bf16.f64_to_bf16(x.astype(np.float64)), torch_bf16_bits(x))


def test_bf16_halfway_cases():
    # 1 + k/256 lies exactly halfway between bf16 neighbours for odd k
    ks = np.arange(-255, 256)
    x = (1.0 + ks / 256.0).astype(np.float32) * np.float32(3.0)
    got = bf16.f64_to_bf16(x.astype(np.float64))
    assert np.array_equal(got, torch_bf16_bits(x))
    # explicit values: 1 + 1/256 -> 1 (even), 1 + 3/256 -> 1 + 4/256
    assert bf16.round_bf16(np.array([1 + 1 / 256]))[0] == 1.0
    assert bf16.round_bf16(np.array([1 + 3 / 256]))[0] == 1 + 4 / 256
    assert bf16.round_bf16(np.array([-(1 + 3 / 256)]))[0] == -(1 + 4 / 256)
    # mantissa overflow carries into the exponent
    assert bf16.round_bf16(np.array([2 - 1 / 512]))[0] == 2.0


def test_bf16_roundtrip():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16.bf16_to_f64(bits)
    finite = np.isfinite(vals) & (np.abs(vals) > 1e-37)
    assert np.array_equal(bf16.f64_to_bf16(vals[finite]), bits[finite])


def test_lm_head_one_hot_selects_column():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((50, 16))
    h = np.zeros((3, 16))
    h[0, 4] = 1.0
    h[1, 15] = 1.0
    h[2, 0] = 1.0
    out = rules.lm_head_logits(h, w)
    assert np.array_equal(out[0], w[:, 4])
    assert np.array_equal(out[1], w[:, 15])
    assert np.array_equal(out[2], w[:, 0])


def test_lm_head_brute_force_integers():
    rng = np.random.default_rng(2)
    w = rng.integers(-8, 9, (13, 7)).astype(np.float64)
    h = rng.integers(-8, 9, (2, 3, 7)).astype(np.float64)
    out = rules.lm_head_logits(h, w)
    for a in range(2):
        for b in range(3):
            for v in range(13):
                assert out[a, b, v] == sum(h[a, b, k] * w[v, k] for k in range(7))


@pytest.mark.parametrize("T", [0.3, 0.7, 1.0, 2.5])
def test_target_probs_matches_scipy(T):
    rng = np.random.default_rng(3)
    l = (rng.standard_normal((4, 5, 1000)) * 3).astype(np.float32)
    p = rules.target_probs(l, T)
    ref = scipy.special.softmax(l.astype(np.float64) / T, axis=-1)
    assert np.allclose(p, ref, rtol=1e-6, atol=0)
    assert p.dtype == np.float32


def test_target_probs_rejects_bad_temperature():
    with pytest.raises(ValueError):
        rules.target_probs(np.zeros((1, 3), np.float32), 0.0)
    with pytest.raises(ValueError):
        rules.target_probs(np.zeros((1, 3), np.float32), float("nan"))


def test_argmax_lowest_index_on_ties():
    l = np.array([[[0.0, 2.0, 1.0, 2.0], [5.0, 5.0, 5.0, 5.0]]], dtype=np.float32)
    am, gap = rules.top2(l)
    assert am.tolist() == [[1, 0]]
    assert gap.tolist() == [[0.0, 0.0]]
    # brute scan
    rng = np.random.default_rng(4)
    x = rng.integers(0, 4, (200, 9)).astype(np.float32)
    am, _ = rules.top2(x)
    for r in range(200):
        best = 0
        for j in range(9):
            if x[r, j] > x[r, best]:
                best = j
        assert am[r] == best
