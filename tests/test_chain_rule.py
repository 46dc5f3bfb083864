"""The near-tie rule of the chained-decode parity check (tests/gpu_util.chained_routing), on
hand-made oracle traces: it must accept a flip only at a genuine near-tie, only between the tied
pair, and stop there; any other difference is an error."""
import numpy as np
import pytest

from tests import gpu_util as gu

K, N = 4, 60


def _trace(rng, n, tie_layer=None, gap=1e-6):
    out = []
    for L in range(n):
        lg = rng.standard_normal(512) * 8.0
        if L == tie_layer:
            o = np.argsort(-lg, kind="stable")
            lg[o[K]] = lg[o[K - 1]] - gap * np.std(lg)  # (k+1)-th just below the k-th
        ids = np.argsort(-lg, kind="stable")[:K]
        out.append({"logits": lg, "ids": ids})
    return out


def test_identical_routing_never_parts():
    tr = _trace(np.random.default_rng(1), N)
    got = np.stack([r["ids"] for r in tr])
    assert gu.chained_routing(got, tr, 1e-6, K, N) is None


def test_flip_at_a_near_tie_parts_there():
    tr = _trace(np.random.default_rng(2), N, tie_layer=50, gap=1e-5)
    got = np.stack([r["ids"] for r in tr])
    o = np.argsort(-tr[50]["logits"], kind="stable")
    got[50] = np.concatenate([o[:K - 1], o[K:K + 1]])  # 5th instead of the 4th
    got[51:] = -1  # whatever follows is not compared
    assert gu.chained_routing(got, tr, 1e-6, K, N) == 50


def test_flip_without_a_near_tie_fails():
    tr = _trace(np.random.default_rng(3), N)
    got = np.stack([r["ids"] for r in tr])
    o = np.argsort(-tr[10]["logits"], kind="stable")
    got[10] = np.concatenate([o[:K - 1], o[K:K + 1]])
    with pytest.raises(AssertionError):
        gu.chained_routing(got, tr, 1e-6, K, N)


def test_wrong_expert_at_a_near_tie_fails():
    tr = _trace(np.random.default_rng(4), N, tie_layer=40, gap=1e-5)
    got = np.stack([r["ids"] for r in tr])
    o = np.argsort(-tr[40]["logits"], kind="stable")
    got[40] = np.concatenate([o[1:K], o[K + 3:K + 4]])  # drops the best, takes the 8th
    with pytest.raises(AssertionError):
        gu.chained_routing(got, tr, 1e-6, K, N)
