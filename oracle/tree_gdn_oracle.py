"""CPU oracle for tree-aware recurrent verification of a Gated-DeltaNet layer.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module; the product path (the HIP
library and its Python binding) never does and shares no code with it.

Page followed:
  [DT]  "DominoTree: Conditional Tree-Structured Drafting with Domino for
        Speculative Decoding" (arXiv 2607.08642), section 4.5.4 "Scaling to a
        27B hybrid-attention target", paragraph "Tree-aware recurrent
        verification": an ancestor mask is not enough for a recurrent layer;
        each node needs the state of its own root path and a dense convolution
        window per node, and only the accepted path's state is committed.
        Flattening the tree into a chain corrupts the state.

Everything here is float64 and literal: a node's output is the recurrence
replayed from the committed state over the node's own root path, one token at
a time (no chunking, no WY/UT transform).

Parity pins (tests/test_gdn_pins.py): one-step closed forms, the orthogonal-key
closed form (with orthonormal keys the erase term vanishes and the output is
decayed linear attention over the node's ancestors), a chain tree against
numpy's convolution, the flattening negative control, and the commit against
the verify output at the last accepted node.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------------------
# O-gdn: tree-aware recurrent verification for a Gated-DeltaNet layer ([DT]
# section 4.5.4, "Tree-aware recurrent verification": each node's recurrent
# state and short-convolution window follow the node's own root path, since
# a chain recurrence over the flattened tree lets rejected siblings write into
# the state later nodes read; only the accepted path's state is committed).
# The page names the layer, not its formulas; the readings below follow the
# published gated delta rule:
#   k^ = k / sqrt(|k|^2 + eps), q^ = scale * q / sqrt(|q|^2 + eps)
#   S  <- exp(g) * S (I - beta k^ k^T) + beta v k^T,   o = S q^
# with S [dv, dk] per value head, v-head h reading q/k head h // (Hv / Hk),
# and a depthwise causal convolution of width K with SiLU on the layer's
# inputs, whose window for a node is the committed conv state (the K - 1 most
# recent inputs, oldest first) followed by the inputs along the node's path.
# ---------------------------------------------------------------------------

GDN_EPS = 1e-6


def _l2n(x, eps=GDN_EPS):
    x = np.asarray(x, np.float64)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def gdn_step(S, q, k, v, g, beta):
    """One step of the gated delta rule on already-normalised q, k.  S
    [..., dv, dk]; q, k [..., dk]; v [..., dv]; g, beta [...] (leading axes are
    heads).  Returns (new S, output S q)."""
    a = np.exp(np.asarray(g, np.float64))[..., None, None]
    b = np.asarray(beta, np.float64)[..., None, None]
    Sk = np.einsum("...ij,...j->...i", S, k)
    S = a * (S - b * Sk[..., :, None] * k[..., None, :]) + b * v[..., :, None] * k[..., None, :]
    return S, np.einsum("...ij,...j->...i", S, q)


def _root_path(parent, lo, j):
    path = []
    u = j
    while u >= 0:
        path.append(u)
        u = int(parent[lo + u])
    return path[::-1]


def _heads(q, k, v, g, beta, scale, l2norm):
    """Normalised q^, k^ expanded to the value heads, as float64."""
    Hk, Hv = np.asarray(q).shape[1], np.asarray(v).shape[1]
    rep = Hv // Hk
    qn = _l2n(q) if l2norm else np.asarray(q, np.float64)
    kn = _l2n(k) if l2norm else np.asarray(k, np.float64)
    qn = np.repeat(qn, rep, axis=1) * scale
    kn = np.repeat(kn, rep, axis=1)
    return qn, kn, np.asarray(v, np.float64), np.asarray(g, np.float64), np.asarray(beta, np.float64)


def gdn_tree_verify(q, k, v, g, beta, S0, parent, cu_nodes, scale: float, l2norm: bool = True):
    """Per node: the recurrence run from the request's committed state S0
    [B, Hv, dv, dk] over the tokens of the node's root->node path, and the
    node's output.  q, k [T, Hk, dk]; v [T, Hv, dv]; g, beta [T, Hv].
    Returns o [T, Hv, dv] (float64)."""
    qn, kn, v, g, beta = _heads(q, k, v, g, beta, scale, l2norm)
    S0 = np.asarray(S0, np.float64)
    T, Hv, dv = v.shape
    o = np.zeros((T, Hv, dv))
    cu = np.asarray(cu_nodes)
    for b in range(cu.shape[0] - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for j in range(hi - lo):
            S = S0[b].copy()
            for u in _root_path(parent, lo, j):
                t = lo + u
                S, out = gdn_step(S, qn[t], kn[t], v[t], g[t], beta[t])
            o[lo + j] = out
    return o


def gdn_conv_tree(x, conv_state, weight, parent, cu_nodes):
    """Depthwise causal convolution with SiLU over each node's own window: the
    request's conv_state [B, K-1, C] (oldest first) followed by the inputs x
    [T, C] along the node's root path, the last K entries taken; weight [C, K]
    (weight[:, K-1] multiplies the node's own input).  Returns y [T, C]."""
    x = np.asarray(x, np.float64)
    cs = np.asarray(conv_state, np.float64)
    w = np.asarray(weight, np.float64)
    K = w.shape[1]
    y = np.zeros_like(x)
    cu = np.asarray(cu_nodes)
    for b in range(cu.shape[0] - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        for j in range(hi - lo):
            seq = [cs[b, p] for p in range(K - 1)] + [x[lo + u] for u in _root_path(parent, lo, j)]
            win = np.stack(seq[-K:])                   # [K, C]
            z = (w.T * win).sum(0)
            y[lo + j] = z / (1.0 + np.exp(-z))
    return y


def gdn_commit(S0, conv_state, x, k, v, g, beta, cu_nodes, accept_len, accept_idx,
               l2norm: bool = True):
    """The recurrent state each request keeps after acceptance: S0 advanced
    by the accepted tokens in path order, and the conv state holding the last
    K - 1 inputs of (old conv state, accepted inputs).  Nothing accepted keeps
    both unchanged.  Returns (S [B, Hv, dv, dk], conv_state [B, K-1, C])."""
    _, kn, v, g, beta = _heads(k, k, v, g, beta, 1.0, l2norm)
    S = np.array(S0, dtype=np.float64, copy=True)
    cs = np.array(conv_state, dtype=np.float64, copy=True)
    x = np.asarray(x, np.float64)
    cu = np.asarray(cu_nodes)
    km1 = cs.shape[1]
    for b in range(cu.shape[0] - 1):
        lo = int(cu[b])
        rows = [lo + int(accept_idx[b, j]) for j in range(int(accept_len[b]))]
        for t in rows:
            S[b], _ = gdn_step(S[b], kn[t], kn[t], v[t], g[t], beta[t])
        if km1 > 0 and rows:
            seq = [cs[b, p] for p in range(km1)] + [x[t] for t in rows]
            cs[b] = np.stack(seq[-km1:])
    return S, cs
