"""Pins of the Gated-DeltaNet tree-verification oracle ([DT] section 4.5.4,
"Tree-aware recurrent verification") against closed forms, numpy's
convolution, the chain-over-the-path invariant, and the failure the page
describes (a chain recurrence over the flattened tree corrupts the state)."""
import numpy as np
import pytest

from oracle import tree_gdn_oracle as G
from tree_attention_verification_bitmask_amd import workloads as W


def ancestors_or_self(parent, j):
    out = [j]
    while parent[out[-1]] >= 0:
        out.append(int(parent[out[-1]]))
    return out


def small(rng, parents, hk=2, hv=4, dk=8, dv=6, K=4):
    return W.gdn_inputs(rng, parents, hk=hk, hv=hv, dk=dk, dv=dv, conv_k=K, state_std=0.5)


def verify(gi, parent=None, scale=0.7, l2norm=True, **kw):
    p = gi.parent if parent is None else parent
    args = dict(q=gi.q, k=gi.k, v=gi.v, g=gi.g, beta=gi.beta, S0=gi.state)
    args.update(kw)
    return G.gdn_tree_verify(args["q"], args["k"], args["v"], args["g"], args["beta"], args["S0"],
                             p, gi.cu_nodes, scale, l2norm)


def test_step_closed_forms():
    rng = np.random.default_rng(0)
    S0 = rng.normal(size=(4, 3))
    q, k, v = rng.normal(size=3), rng.normal(size=3), rng.normal(size=4)
    S, o = G.gdn_step(S0, q, k, v, 0.0, 0.0)                 # no decay, no write
    assert np.array_equal(S, S0) and np.allclose(o, S0 @ q)
    S, o = G.gdn_step(S0, q, k, v, np.log(0.25), 0.0)        # pure decay
    assert np.allclose(S, 0.25 * S0)
    S, o = G.gdn_step(np.zeros((4, 3)), q, k, v, -0.3, 0.5)  # empty state: one rank-1 write
    assert np.allclose(S, 0.5 * np.outer(v, k)) and np.allclose(o, 0.5 * v * (k @ q))
    kn = k / np.linalg.norm(k)                               # beta 1, unit key: S k^ becomes v
    S, _ = G.gdn_step(S0, q, kn, v, 0.0, 1.0)
    assert np.allclose(S @ kn, v)
    # leading head axis: the same as per head
    Sh = rng.normal(size=(2, 4, 3))
    qh, kh, vh = rng.normal(size=(2, 3)), rng.normal(size=(2, 3)), rng.normal(size=(2, 4))
    Sb, ob = G.gdn_step(Sh, qh, kh, vh, np.array([-0.1, -0.2]), np.array([0.3, 0.6]))
    for h in range(2):
        S1, o1 = G.gdn_step(Sh[h], qh[h], kh[h], vh[h], [-0.1, -0.2][h], [0.3, 0.6][h])
        assert np.allclose(Sb[h], S1) and np.allclose(ob[h], o1)


@pytest.mark.parametrize("seed", [1, 2])
def test_orthonormal_keys_closed_form(seed):
    """With orthonormal keys (distinct basis vectors, no normalisation) the
    erase term of a write never touches the other writes, so
      o_t = e^{G_t} S0 D_t q^_t + sum_{s in path(t)} e^{G_t - G_s} beta_s v_s q^_t[key(s)]
    with G the summed log decay along the path and D_t scaling the columns of
    the path's keys by (1 - beta_s).  Pins the ancestor sets, the decay
    cumulation and the per-head key sharing."""
    rng = np.random.default_rng(seed)
    n = 12
    parent = W.best_first_tree(rng, n, 5)
    gi = small(rng, [parent], hk=2, hv=4, dk=n, dv=5)
    keyof = np.stack([rng.permutation(n) for _ in range(2)], 1)   # [T, Hk] distinct basis index per head
    k = np.zeros((n, 2, n), np.float32)
    for t in range(n):
        for hh in range(2):
            k[t, hh, keyof[t, hh]] = 1.0
    scale = 0.9
    o = G.gdn_tree_verify(gi.q, k, gi.v, gi.g, gi.beta, gi.state, parent, gi.cu_nodes, scale, False)
    for t in range(n):
        path = ancestors_or_self(parent, t)
        for h in range(4):
            hk = h // 2
            q = gi.q[t, hk].astype(np.float64) * scale
            Gt = sum(float(gi.g[s, h]) for s in path)
            d = np.ones(n)
            for s in path:
                d[keyof[s, hk]] = 1.0 - float(gi.beta[s, h])
            want = np.exp(Gt) * gi.state[0, h].astype(np.float64) @ (d * q)
            for s in path:
                Gs = sum(float(gi.g[r, h]) for r in ancestors_or_self(parent, s))
                want = want + np.exp(Gt - Gs) * float(gi.beta[s, h]) * gi.v[s, h] * q[keyof[s, hk]]
            np.testing.assert_allclose(o[t, h], want, rtol=1e-10, atol=1e-12)


def test_node_equals_chain_over_its_own_path():
    """Each node's output is the recurrence over exactly its root->node tokens:
    the oracle on a chain made of those tokens gives the same output."""
    rng = np.random.default_rng(3)
    parent = W.random_tree(rng, 10, 6)
    gi = small(rng, [parent])
    o = verify(gi)
    for t in range(10):
        path = ancestors_or_self(parent, t)[::-1]
        sub = G.gdn_tree_verify(gi.q[path], gi.k[path], gi.v[path], gi.g[path], gi.beta[path], gi.state,
                                W.chain_tree(len(path)), np.array([0, len(path)]), 0.7, True)
        np.testing.assert_allclose(o[t], sub[-1], rtol=1e-12, atol=1e-12)


def test_flattening_the_tree_corrupts_the_state():
    """Negative control ([DT] 4.5.4): node 2 is node 0's child and node 1 is
    node 0's sibling.  A chain recurrence over the flattened order lets node 1
    write into node 2's state; the tree recurrence does not."""
    rng = np.random.default_rng(4)
    tree = np.array([-1, -1, 0], np.int32)
    gi = small(rng, [tree])
    o_tree = verify(gi)
    o_flat = verify(gi, parent=W.chain_tree(3))
    np.testing.assert_allclose(o_tree[0], o_flat[0], rtol=1e-12)     # the first node agrees
    assert np.abs(o_tree[2] - o_flat[2]).max() > 1e-3                # the grandchild does not
    # node 1 is a root child in the tree: it sees only itself
    solo = G.gdn_tree_verify(gi.q[1:2], gi.k[1:2], gi.v[1:2], gi.g[1:2], gi.beta[1:2], gi.state,
                             np.array([-1]), np.array([0, 1]), 0.7, True)
    np.testing.assert_allclose(o_tree[1], solo[0], rtol=1e-12)


def test_conv_chain_equals_numpy_convolution():
    """A chain tree's windows are the ordinary causal convolution of (conv
    state, inputs): numpy's full convolution with the reversed taps."""
    rng = np.random.default_rng(5)
    T, K = 9, 4
    gi = small(rng, [W.chain_tree(T)], K=K)
    y = G.gdn_conv_tree(gi.x, gi.conv_state, gi.conv_w, gi.parent, gi.cu_nodes)
    for c in range(gi.x.shape[1]):
        seq = np.concatenate([gi.conv_state[0, :, c], gi.x[:, c]]).astype(np.float64)
        z = np.convolve(seq, gi.conv_w[c, ::-1].astype(np.float64))[K - 1:K - 1 + T]
        np.testing.assert_allclose(y[:, c], z / (1 + np.exp(-z)), rtol=1e-12, atol=1e-14)


def test_conv_window_reads_ancestors_then_conv_state():
    """Star tree (every node a root child): each window is the conv state
    followed by the node itself.  Deep tree: a node at level >= K sees only
    its K nearest ancestors-or-self."""
    rng = np.random.default_rng(6)
    K = 4
    star = np.full(5, -1, np.int32)
    gi = small(rng, [star], K=K)
    y = G.gdn_conv_tree(gi.x, gi.conv_state, gi.conv_w, star, gi.cu_nodes)
    w = gi.conv_w.astype(np.float64)
    for t in range(5):
        z = (w[:, :K - 1] * gi.conv_state[0].T).sum(1) + w[:, K - 1] * gi.x[t]
        np.testing.assert_allclose(y[t], z / (1 + np.exp(-z)), rtol=1e-12, atol=1e-14)
    tree = np.array([-1, 0, 1, -1, 2, 4, 3], np.int32)   # node 5: path 0,1,2,4,5 (level 5)
    gi = small(rng, [tree], K=K)
    w = gi.conv_w.astype(np.float64)
    y = G.gdn_conv_tree(gi.x, gi.conv_state, gi.conv_w, tree, gi.cu_nodes)
    z = sum(w[:, K - 1 - j] * gi.x[a] for j, a in enumerate([5, 4, 2, 1]))
    np.testing.assert_allclose(y[5], z / (1 + np.exp(-z)), rtol=1e-12, atol=1e-14)
    # node 6 (level 2: 3 -> 6) reaches two conv-state rows
    z = w[:, 3] * gi.x[6] + w[:, 2] * gi.x[3] + w[:, 1] * gi.conv_state[0, 2] + w[:, 0] * gi.conv_state[0, 1]
    np.testing.assert_allclose(y[6], z / (1 + np.exp(-z)), rtol=1e-12, atol=1e-14)


def test_commit_continues_the_accepted_path():
    """After committing a path, a new token verified from the committed state
    and conv state gets the same conv output and layer output as that token
    placed under the path's last node in the original tree."""
    rng = np.random.default_rng(7)
    parent = W.best_first_tree(rng, 11, 5)
    last = int(np.argmax(np.array([len(ancestors_or_self(parent, t)) for t in range(11)])))
    path = ancestors_or_self(parent, last)[::-1]
    ext = np.concatenate([parent, [last]]).astype(np.int32)           # node 11: child of `last`
    gi = small(rng, [ext])
    alen = np.array([len(path)], np.int32)
    aidx = np.zeros((1, 8), np.int32)
    aidx[0, :len(path)] = path
    S, cs = G.gdn_commit(gi.state, gi.conv_state, gi.x, gi.k, gi.v, gi.g, gi.beta,
                         np.array([0, 11]), alen, aidx)
    y_ext = G.gdn_conv_tree(gi.x, gi.conv_state, gi.conv_w, ext, gi.cu_nodes)
    y_new = G.gdn_conv_tree(gi.x[11:], cs, gi.conv_w, np.array([-1]), np.array([0, 1]))
    np.testing.assert_allclose(y_new[0], y_ext[11], rtol=1e-12, atol=1e-14)
    o_ext = verify(gi, parent=ext)
    o_new = G.gdn_tree_verify(gi.q[11:], gi.k[11:], gi.v[11:], gi.g[11:], gi.beta[11:], S,
                              np.array([-1]), np.array([0, 1]), 0.7, True)
    np.testing.assert_allclose(o_new[0], o_ext[11], rtol=1e-10, atol=1e-12)
    # nothing accepted: both states unchanged
    S0, cs0 = G.gdn_commit(gi.state, gi.conv_state, gi.x, gi.k, gi.v, gi.g, gi.beta,
                           np.array([0, 11]), np.zeros(1, np.int32), aidx)
    assert np.array_equal(S0, gi.state) and np.array_equal(cs0, gi.conv_state)


def test_l2norm_and_scale():
    """The normalisation makes the output independent of the size of q and k
    (up to eps), and scale multiplies the output linearly."""
    rng = np.random.default_rng(8)
    parent = W.random_tree(rng, 6, 4)
    gi = small(rng, [parent])
    o = verify(gi)
    o2 = verify(gi, q=gi.q * 3.0, k=gi.k * 5.0)
    np.testing.assert_allclose(o, o2, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(verify(gi, scale=1.4), 2.0 * o, rtol=1e-12)
