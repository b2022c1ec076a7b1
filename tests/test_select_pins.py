"""Pins of the selection oracle (oracle/tree_select_oracle.py) against what
the pages and the mathematics fix, independently of the oracle's own
ranking code:

* [DT] Appendix B: on tie-free inputs with W = B, the ledger's global top B
  is the sequential best-first heap's tree -- here node for node in pop
  order, at batch sizes 1, 2, 5 and 32 (the sizes the page reports);
* [DAR] Lemma 1: the same with a non-positive depth bonus, and a positive
  bonus breaks ancestor closure (a negative control);
* order statistics: the chosen keys are exactly the B largest (numpy sort);
* tree invariants: parents precede children, keys never rise along a path,
  dead-leaf padding of short ledgers, bad-ledger reports;
* a ledger small enough to rank by hand.
"""
import numpy as np
import pytest

from oracle import tree_select_oracle as S


def test_hand_ranked_ledger():
    """D = 2, L = 2.  Level 1: a (-0.1, tok 10), b (-0.5, tok 11).  Level 2:
    a's children c (-0.3, tok 20) and d (-0.9, tok 21) in slots 0, 1.  By hand
    the ranking is a, c, b, d; with budget 3: a, c, b -> parents [-1, 0, -1]."""
    score = np.array([[-0.1, -0.5], [-0.3, -0.9]], np.float32)
    parent = np.array([[-1, -1], [0, 0]], np.int32)
    token = np.array([[10, 11], [20, 21]], np.int32)
    tp, tt, n, bad = S.select_one(score, parent, token, 3, 0.0)
    assert tp.tolist() == [-1, 0, -1] and tt.tolist() == [10, 20, 11] and n == 3 and not bad
    # budget 5 > 4 candidates: one dead leaf
    tp, tt, n, bad = S.select_one(score, parent, token, 5, 0.0)
    assert tp.tolist() == [-1, 0, -1, 0, -1] and tt.tolist() == [10, 20, 11, 21, -1] and n == 4
    # a depth bonus of -0.5 per level: keys a -0.6, b -1.0, c -1.3, d -1.9 -> a, b, c
    tp, tt, n, bad = S.select_one(score, parent, token, 3, -0.5)
    assert tp.tolist() == [-1, -1, 0] and tt.tolist() == [10, 11, 20]


@pytest.mark.parametrize("batch", [1, 2, 5, 32])
def test_frontier_topb_equals_best_first_heap(batch):
    """[DT] Appendix B: W = B makes the ledger's global top B the heap's tree."""
    D, k, B = 8, 3, 12
    score = np.zeros((batch, D, B * k), np.float32)
    parent = np.zeros_like(score, dtype=np.int32)
    token = np.zeros_like(parent)
    heaps = []
    for b in range(batch):
        sc = S.PathScorer(seed=1000 + b, k=k)
        score[b], parent[b], token[b] = S.frontier_ledger(sc, D, B)
        heaps.append(S.heap_tree(sc, D, B))
    tp, tt, nr, err = S.select_topb(score, parent, token, B)
    assert err == 0 and (nr == B).all()
    for b in range(batch):
        assert tp[b].tolist() == heaps[b][0].tolist(), b
        assert tt[b].tolist() == heaps[b][1].tolist(), b


@pytest.mark.parametrize("beta", [0.0, -0.05, -0.5])
def test_nonpositive_depth_bonus_keeps_heap_equivalence(beta):
    """[DAR] Lemma 1: with beta <= 0 the global top B equals the heap on the
    bonus-adjusted key (deep, narrow trees: D 16, k 4, B 64)."""
    D, k, B = 16, 4, 64
    for seed in (7, 8):
        sc = S.PathScorer(seed=seed, k=k)
        score, parent, token = S.frontier_ledger(sc, D, B)
        tp, tt, n, bad = S.select_one(score, parent, token, B, beta)
        hp, ht = S.heap_tree(sc, D, B, beta)
        assert not bad and tp.tolist() == hp.tolist() and tt.tolist() == ht.tolist()


def test_positive_depth_bonus_breaks_closure():
    """Negative control: a large positive bonus ranks deep candidates above
    their own parents, so the top B is no longer a tree and is reported."""
    sc = S.PathScorer(seed=3, k=4)
    score, parent, token = S.frontier_ledger(sc, 8, 16)
    _, _, _, bad = S.select_one(score, parent, token, 16, 5.0)
    assert bad
    tp, tt, nr, err = S.select_topb(score[None], parent[None], token[None], 16, 5.0)
    assert err == (S.ERR_BAD_LEDGER << 24) | 0


def _random_monotone_ledger(rng, D, W, k, p_empty=0.1, ties=False):
    """Random ledger with non-increasing scores along every parent pointer."""
    L = W * k
    score = np.full((D, L), -np.inf, np.float32)
    parent = np.full((D, L), -1, np.int32)
    token = rng.integers(0, 1000, (D, L)).astype(np.int32)
    for t in range(D):
        for e in range(L):
            if rng.random() < p_empty:
                continue
            step = np.float32(rng.integers(0, 4) * 0.25 if ties else rng.exponential(0.5))
            if t == 0:
                score[t, e] = -step
            else:
                live = np.flatnonzero(np.isfinite(score[t - 1]))
                if live.size == 0:
                    continue
                p = int(rng.choice(live))
                parent[t, e] = p
                score[t, e] = np.float32(score[t - 1, p] - step)
    return score, parent, token


@pytest.mark.parametrize("ties", [False, True])
def test_selection_is_the_b_largest_and_a_tree(ties):
    rng = np.random.default_rng(11 if ties else 12)
    for _ in range(20):
        D, W, k = int(rng.integers(1, 6)), int(rng.integers(1, 5)), int(rng.integers(1, 4))
        B = int(rng.integers(1, 3 * D * W * k))
        score, parent, token = _random_monotone_ledger(rng, D, W, k, ties=ties)
        L = W * k
        tp, tt, n, bad = S.select_one(score, parent, token, B, 0.0)
        assert not bad
        finite = np.sort(score[np.isfinite(score)].astype(np.float64))[::-1]
        assert n == min(B, finite.size)
        # the chosen scores are the n largest, in non-increasing order
        keys = []
        ok = np.isfinite(score)
        flat_s = score.reshape(-1)
        chosen_idx = []
        # recover each chosen entry from (parent position, token) by walking the ranking
        ranking = sorted(np.flatnonzero(ok.reshape(-1)), key=lambda e: (-float(flat_s[e]), e))
        chosen_idx = ranking[:n]
        keys = [float(flat_s[e]) for e in chosen_idx]
        assert np.array_equal(np.array(keys), finite[:n])
        # parents precede children, every parent is chosen, tokens carried over
        for i in range(n):
            assert tp[i] < i
            e = chosen_idx[i]
            t, s = divmod(e, L)
            assert tt[i] == token[t, s]
            if t == 0:
                assert tp[i] == -1
            else:
                assert chosen_idx[tp[i]] == (t - 1) * L + parent[t, s]
        assert (tp[n:] == -1).all() and (tt[n:] == -1).all()


def test_bad_parent_slot_is_reported():
    score = np.array([[-0.1, -0.2], [-0.3, -0.4]], np.float32)
    parent = np.array([[-1, -1], [7, 0]], np.int32)   # slot 7 does not exist
    token = np.array([[1, 2], [3, 4]], np.int32)
    tp, tt, n, bad = S.select_one(score, parent, token, 4, 0.0)
    assert bad and tt.tolist() == [1, 2, -1, 4] and tp.tolist() == [-1, -1, -1, 0]
    score[0, 1] = np.nan   # an empty slot may not be anybody's parent either
    parent[1, 0] = 1
    tp, tt, n, bad = S.select_one(score, parent, token, 4, 0.0)
    assert bad and n == 3 and tt.tolist() == [1, -1, 4, -1]
