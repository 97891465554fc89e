"""Pins of the oracle's activation + dropout ([ActPage] sections 3-5): the
generator against its published known-answer vectors, the mask against the
binomial law and its invariances, and the backward against finite
differences of the forward with the mask held fixed."""
import json
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_philox_known_answers(orc):
    kat = json.load(open(os.path.join(HERE, "golden", "philox4x32_10_kat.json")))
    for case in kat["cases"]:
        ctr = [int(v, 16) for v in case["ctr"]]
        key = [int(v, 16) for v in case["key"]]
        assert orc.philox4x32_10(ctr, key) == [int(v, 16) for v in case["out"]]


def test_threshold_rounding(orc):
    assert orc.dropout_threshold(0.0) == 0
    assert orc.dropout_threshold(1.0) == 1 << 16
    assert orc.dropout_threshold(0.5) == 1 << 15
    assert orc.dropout_threshold(0.25) == 1 << 14
    # round to nearest: 0.1 * 2^16 = 6553.6, 0.3 * 2^16 = 19660.8, 0.7 * 2^16 = 45875.2
    assert orc.dropout_threshold(0.1) == 6554
    assert orc.dropout_threshold(0.3) == 19661
    assert orc.dropout_threshold(0.7) == 45875


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_keep_fraction_is_binomial(orc, p):
    n = 1 << 20
    keep = orc.dropout_keep(n, p, seed=20240611)
    q = 1.0 - orc.dropout_threshold(p) / float(1 << 16)
    sd = np.sqrt(q * (1 - q) / n)
    assert abs(keep.mean() - q) < 5 * sd
    # Pairs of neighbours are independent too (a stuck word would show).
    both = (keep[0::2] & keep[1::2]).mean()
    assert abs(both - q * q) < 5 * np.sqrt(q * q * (1 - q * q) / (n // 2))


def test_edge_probabilities(orc):
    x = np.linspace(-3, 3, 1001)
    assert (orc.dropout_keep(1001, 0.0, 7) == 1).all()
    assert (orc.dropout_keep(1001, 1.0, 7) == 0).all()
    np.testing.assert_array_equal(orc.act_dropout_fwd(x, "gelu", 0.0, seed=7), orc.act("gelu", x))
    assert (orc.act_dropout_fwd(x, "gelu", 1.0, seed=7) == 0).all()


def test_offset_and_seed_words(orc):
    n, k = 4096, 1 << 34  # an offset past 2^32 blocks exercises the counter's high word
    a = orc.dropout_keep(n + 64, 0.5, seed=99, offset=0)
    b = orc.dropout_keep(n, 0.5, seed=99, offset=64)
    np.testing.assert_array_equal(a[64:], b)
    assert (orc.dropout_keep(n, 0.5, 99, offset=k) != orc.dropout_keep(n, 0.5, 99, 0)).any()
    # The seed's high word is part of the key.
    assert (orc.dropout_keep(n, 0.5, 5 + (1 << 32)) != orc.dropout_keep(n, 0.5, 5)).any()
    # Different seeds agree on about q^2 + (1 - q)^2 of the elements.
    m = (orc.dropout_keep(1 << 18, 0.5, 1) == orc.dropout_keep(1 << 18, 0.5, 2)).mean()
    assert abs(m - 0.5) < 0.01


@pytest.mark.parametrize("act", ["none", "gelu", "silu", "tanh", "sigmoid"])
def test_forward_is_unbiased(orc, act):
    rng = np.random.default_rng(3)
    x = rng.standard_normal(1 << 19)
    y = orc.act_dropout_fwd(x, act, 0.3, seed=11)
    a = orc.act(act, x)
    keep = orc.dropout_keep(x.size, 0.3, 11)
    np.testing.assert_allclose(y[keep == 1], a[keep == 1] / 0.7, rtol=1e-15)
    assert (y[keep == 0] == 0).all()
    # E[y] = E[act(x)]: the scaled survivors' mean matches within sampling error.
    se = np.std(a) / np.sqrt(x.size) * 2.0
    assert abs(y.mean() - a.mean()) < 5 * se


@pytest.mark.parametrize("act,param", [("gelu", 0.0), ("silu", 0.0), ("mish", 0.0), ("elu", 0.5),
                                       ("softplus", 0.0)])
def test_backward_is_the_derivative(orc, act, param):
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4000) * 2
    dy = rng.standard_normal(4000)
    x[np.abs(x) < 1e-3] += 0.01  # keep the finite differences off elu's kink
    dx = orc.act_dropout_bwd(dy, x, act, 0.2, seed=123, offset=8, act_param=param)
    h = 1e-6
    f = lambda v: orc.act_dropout_fwd(v, act, 0.2, seed=123, offset=8, act_param=param)
    fd = dy * (f(x + h) - f(x - h)) / (2 * h)
    np.testing.assert_allclose(dx, fd, rtol=1e-6, atol=1e-8)


def test_mask_layout_known_answer(orc):
    """Elements 0..7 under seed 0 use the eight 16-bit halves of
    Philox4x32-10 at counter 0 and key 0 -- the first published
    known-answer vector -- low half first, so their keep flags at a set of
    thresholds are fixed by those words (a different counter, word or half
    assignment changes the pattern)."""
    kat = json.load(open(os.path.join(HERE, "golden", "philox4x32_10_kat.json")))["cases"][0]
    assert kat["ctr"] == ["00000000"] * 4 and kat["key"] == ["00000000"] * 2
    words = [int(v, 16) for v in kat["out"]]
    halves = [h for w in words for h in (w & 0xFFFF, w >> 16)]
    cuts = sorted(set(halves))
    # thresholds below, between and above the eight 16-bit values
    ts = [0, cuts[0] // 2] + [(a + b) // 2 + 1 for a, b in zip(cuts, cuts[1:])] + [cuts[-1] + 1]
    for t in ts:
        p = t / float(1 << 16)
        assert orc.dropout_threshold(p) == t
        expect = np.array([1 if v >= t else 0 for v in halves], dtype=np.uint8)
        np.testing.assert_array_equal(orc.dropout_keep(8, p, seed=0, offset=0), expect)


def test_mask_next_counter(orc):
    """Elements 8..15 take counter 1 (the generator itself is pinned by its
    known-answer vectors above); an offset of 8 starts at that counter."""
    words = orc.philox4x32_10([1, 0, 0, 0], [0, 0])
    halves = np.array([h for w in words for h in (w & 0xFFFF, w >> 16)])
    for t in (int(np.median(halves)), int(halves.min()) + 1, int(halves.max())):
        p = t / float(1 << 16)
        expect = (halves >= t).astype(np.uint8)
        np.testing.assert_array_equal(orc.dropout_keep(16, p, seed=0, offset=0)[8:], expect)
        np.testing.assert_array_equal(orc.dropout_keep(8, p, seed=0, offset=8), expect)
