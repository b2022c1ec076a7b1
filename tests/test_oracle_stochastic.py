"""Pins of the oracle's stochastic acceptance ([TSD] "Verification and
Acceptance Algorithms", "Exact Sampling Equivalence") against what the pages
and the mathematics fix, not against the oracle itself:

* the method's claim: the first token emitted from a node is distributed
  exactly as the target's distribution there, whatever the drafter's q and
  however many sibling candidates were drawn from it (seeded Monte Carlo,
  five-sigma binomial bound);
* a point-mass target distribution (one logit dominant, so exp underflows
  every other weight to 0) must give the greedy walk of tree_accept_greedy
  exactly, for any q and any uniforms;
* q equal to p accepts every first candidate: the walk follows first
  children to a leaf and draws the next token there by the plain inverse
  transform of target_sample.
"""
import numpy as np
import pytest

from oracle import tree_verify_oracle as O


def _first_token_freq(p_logits, q, k, trials, seed, temperature=1.0):
    """Empirical distribution of the first emitted token at the root with k
    candidate children drawn i.i.d. from q (each a leaf)."""
    V = len(q)
    rng = np.random.default_rng(seed)
    parent = np.full(k, -1, np.int32)
    node_logits = np.zeros((k, V))
    node_q = np.full((k, V), 1.0 / V)
    counts = np.zeros(V)
    for _ in range(trials):
        draft = rng.choice(V, size=k, p=q).astype(np.int32)
        ua = rng.random(k)
        uf = rng.random()
        path, nxt = O.accept_stochastic_one(parent, draft, p_logits, node_logits, temperature, q, node_q, ua, uf, 8)
        counts[draft[path[0]] if path else nxt] += 1
    return counts / trials


@pytest.mark.parametrize("k,seed", [(1, 0), (3, 1), (4, 2)])
def test_first_token_follows_target(k, seed):
    rng = np.random.default_rng(100 + seed)
    V = 5
    logits = rng.normal(0, 1.5, V)
    q = rng.dirichlet(np.full(V, 0.7))
    p = np.exp(logits - logits.max())
    p /= p.sum()
    trials = 60000
    freq = _first_token_freq(logits, q, k, trials, seed)
    sigma = np.sqrt(p * (1 - p) / trials)
    assert np.all(np.abs(freq - p) <= 5 * sigma + 1e-4), (freq, p)
    # and the test would see a sampler that ignored the target: q != p here
    assert np.max(np.abs(q - p)) > 10 * sigma.max()


def test_first_token_follows_target_with_temperature():
    rng = np.random.default_rng(7)
    V = 6
    logits = rng.normal(0, 2.0, V)
    q = rng.dirichlet(np.ones(V))
    T = 0.7
    y = logits / T
    p = np.exp(y - y.max())
    p /= p.sum()
    trials = 60000
    freq = _first_token_freq(logits, q, 3, trials, 3, temperature=T)
    sigma = np.sqrt(p * (1 - p) / trials)
    assert np.all(np.abs(freq - p) <= 5 * sigma + 1e-4), (freq, p)


def _random_forest(rng, n):
    parent = np.empty(n, np.int32)
    for i in range(n):
        parent[i] = rng.integers(-1, i) if i else -1
    return parent


@pytest.mark.parametrize("seed", range(6))
def test_point_mass_target_is_the_greedy_walk(seed):
    rng = np.random.default_rng(seed)
    B, V, D = 3, 40, 6
    sizes = rng.integers(1, 25, B)
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = int(cu[-1])
    parent = np.concatenate([_random_forest(rng, int(s)) for s in sizes]).astype(np.int32)
    root_logits = rng.normal(0, 1, (B, V))
    node_logits = rng.normal(0, 1, (T, V))
    root_star = rng.integers(0, V, B)
    node_star = rng.integers(0, V, T)
    root_logits[np.arange(B), root_star] = 2000.0       # exp(-2000) underflows: p is one-hot
    node_logits[np.arange(T), node_star] = 2000.0
    # drafts: often the target's choice, sometimes not, some dead leaves
    draft = np.where(rng.random(T) < 0.6, np.where(parent < 0, root_star[np.searchsorted(cu, np.arange(T), side="right") - 1],
                                                   node_star[np.maximum(parent + cu[np.searchsorted(cu, np.arange(T), side="right") - 1], 0)]),
                     rng.integers(0, V, T)).astype(np.int32)
    draft[rng.random(T) < 0.1] = -1
    root_q = rng.dirichlet(np.ones(V), B)
    node_q = rng.dirichlet(np.ones(V), T)
    ua, uf = rng.random(T), rng.random(B)
    got = O.accept_stochastic(parent, draft, cu, root_logits, node_logits, 1.0, root_q, node_q, ua, uf, D)
    want = O.accept_greedy(parent, draft, node_star.astype(np.int32), root_star.astype(np.int32), cu, D)
    for g, w in zip(got, want):
        assert np.array_equal(np.asarray(g), np.asarray(w))


@pytest.mark.parametrize("seed", range(4))
def test_draft_equal_to_target_accepts_first_children(seed):
    rng = np.random.default_rng(50 + seed)
    V, D, n = 30, 5, 20
    parent = _random_forest(rng, n)
    draft = rng.integers(0, V, n).astype(np.int32)
    root_logits = rng.normal(0, 1, V)
    node_logits = rng.normal(0, 1, (n, V))
    T = 0.9
    root_q = O._softmax64(root_logits, T)
    node_q = np.stack([O._softmax64(r, T) for r in node_logits])
    ua, uf = rng.random(n), float(rng.random())
    path, nxt = O.accept_stochastic_one(parent, draft, root_logits, node_logits, T, root_q, node_q, ua, uf, D)
    cur, want = -1, []
    while len(want) < D:
        kids = [j for j in range(n) if parent[j] == cur]
        if not kids:
            break
        want.append(kids[0])
        cur = kids[0]
    assert path == want
    last = root_logits[None] if not want else node_logits[want[-1]][None]
    assert nxt == int(O.target_sample(last, T, [uf])[0])
