"""CPU oracle for the tree-verification pass.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module; the product path (the HIP
library and its Python binding) never does and shares no code with it.

It is deliberately plain and slow: Python sets and loops for the tree logic,
numpy float64 for attention, one (node, head) at a time, no blocking, no
fusion, no reordering beyond what the definitions state.

Pages followed:
  [TSD] "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
        Tree Attention Accelerate LLM Serving" (llms.blog), sections
        "Tree Representation of Speculative Candidates", "The Tree Attention
        Mechanism" (parts 1 Tree Flattening, 2 2D Causal Tree Mask,
        3 Tree Positional IDs), "Verification and Acceptance Algorithms"
        (Greedy Tree Verification) and "KV Cache Rollback".
  [DT]  "DominoTree: Conditional Tree-Structured Drafting with Domino for
        Speculative Decoding" (arXiv 2607.08642), section 2.1 and Appendix B.

Readings taken where the pages leave a step open (each is also listed in the
design notes):
  * parent[i] == -1 means "child of the implicit root", the last verified
    token; parents must precede children (parent[i] < i).
  * level(i) = number of nodes on the root->i path (1 for a root child);
    PosID(root) = P_b - 1 with 0-based positions, so pos[i] = P_b + level(i) - 1.
  * the ancestor mask is packed LSB-first: bit (j & 63) of word (j >> 6) of
    node i's row is set iff node j is i or an ancestor of i.
  * tree node j's K/V live at cache row kv_start[b] + P_b + j (appended after
    the prefix); a query head h reads KV head h // (Hq/Hkv).
  * the greedy walk takes the lowest-index matching child; a negative draft
    token (a dead leaf) never matches.
  * compaction writes the accepted path's K/V to rows P_b .. P_b+L-1, in path
    order, and leaves every other row untouched.

Parity pins: every function here is checked in tests/test_oracle_pins.py
against closed forms, hand-made fixtures from the pages' worked example,
brute force on small inputs and invariants the pages fix.
"""
from __future__ import annotations

import numpy as np

# device-error encoding shared by contract with the C ABI: (code << 24) | index
ERR_BAD_PARENT = 1   # parent[v] not in [-1, v)
ERR_TOO_DEEP = 2     # level(i) > max_depth
ERR_BAD_REQUEST = 3  # request sizes inconsistent with the host maxima / buffers


def _enc(code: int, index: int) -> int:
    return (code << 24) | (index & 0xFFFFFF)


# ---------------------------------------------------------------------------
# O-mask: ancestor sets, levels, position ids  ([TSD] "2D Causal Tree Mask",
# "Tree Positional IDs")
# ---------------------------------------------------------------------------

def ancestor_set(parent, i: int) -> set:
    """anc(i) = {i} U anc(parent[i]), anc(-1) = {} -- the set of tree nodes
    node i may attend to ([TSD] "2D Causal Tree Mask": an ancestor or itself)."""
    out = set()
    v = int(i)
    while v >= 0:
        out.add(v)
        v = int(parent[v])
    return out


def mask_build(parent, cu_nodes, prefix_len, max_nodes: int, max_depth: int):
    """Packed ancestor bitmask, levels and position ids for a batch of trees.

    Returns (anc uint64 [T, W], level int32 [T], pos int32 [T], err int) with
    W = ceil(max_nodes / 64).  err is 0, or the largest encoded error
    (code << 24 | global node index) over all nodes, where a node's walk to
    the root reports the first bad parent it meets, or ERR_TOO_DEEP when its
    level would exceed max_depth.  A request with more than max_nodes nodes
    reports (ERR_BAD_REQUEST, b) and gets no outputs.
    """
    parent = np.asarray(parent)
    cu = np.asarray(cu_nodes)
    B = cu.shape[0] - 1
    T = int(cu[-1]) if B >= 0 else 0
    W = (max_nodes + 63) // 64
    anc = np.zeros((T, W), dtype=np.uint64)
    level = np.zeros(T, dtype=np.int32)
    pos = np.zeros(T, dtype=np.int32)
    err = 0
    for b in range(B):
        lo, hi = int(cu[b]), int(cu[b + 1])
        n = hi - lo
        if n < 0 or n > max_nodes:
            err = max(err, _enc(ERR_BAD_REQUEST, b))
            continue
        par = parent[lo:hi]
        for i in range(n):
            # the walk toward the root, checking each parent pointer it follows
            members = []
            v = i
            bad = None
            while True:
                members.append(v)
                if len(members) > max_depth:
                    bad = _enc(ERR_TOO_DEEP, lo + i)
                    break
                p = int(par[v])
                if not (-1 <= p < v):
                    bad = _enc(ERR_BAD_PARENT, lo + v)
                    break
                if p < 0:
                    break
                v = p
            if bad is not None:
                err = max(err, bad)
                continue
            words = [0] * W
            for j in members:
                words[j >> 6] |= 1 << (j & 63)
            anc[lo + i] = np.array(words, dtype=np.uint64)
            level[lo + i] = len(members)
            pos[lo + i] = int(prefix_len[b]) + len(members) - 1
    return anc, level, pos, err


def unpack_mask(anc_row, n: int) -> np.ndarray:
    """Bool vector of length n from one packed row (LSB-first words)."""
    out = np.zeros(n, dtype=bool)
    for j in range(n):
        out[j] = (int(anc_row[j >> 6]) >> (j & 63)) & 1
    return out


# ---------------------------------------------------------------------------
# O-attn: per-node tree attention  ([TSD] "The Tree Attention Mechanism")
# ---------------------------------------------------------------------------

def key_rows(parent, b_kv_start: int, b_prefix: int, i: int) -> np.ndarray:
    """Cache rows node i attends to: the whole prefix, then its own
    ancestors-or-self among the tree rows appended after the prefix."""
    tree = sorted(ancestor_set(parent, i))
    return np.array(list(range(b_kv_start, b_kv_start + b_prefix))
                    + [b_kv_start + b_prefix + j for j in tree], dtype=np.int64)


def attention_row(q_vec, k_rows, v_rows, scale: float) -> np.ndarray:
    """softmax_t(scale * q . k_t) weighted sum of v_t, all in float64."""
    q = np.asarray(q_vec, dtype=np.float64)
    K = np.asarray(k_rows, dtype=np.float64)
    V = np.asarray(v_rows, dtype=np.float64)
    s = scale * (K @ q)
    s = s - s.max()
    p = np.exp(s)
    p = p / p.sum()
    return p @ V


def tree_attention(q, k, v, parent, cu_nodes, kv_start, prefix_len, scale: float,
                   rows=None) -> np.ndarray:
    """o[t, h] for every global node t and query head h (or only for the
    (t, h) pairs listed in `rows`, returned in that order as [len(rows), d]).

    q [T, Hq, d]; k, v [kv_rows, Hkv, d]; KV head of h is h // (Hq // Hkv).
    """
    q = np.asarray(q)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    cu = np.asarray(cu_nodes)
    owner = np.searchsorted(cu, np.arange(T), side="right") - 1
    if rows is None:
        rows = [(t, h) for t in range(T) for h in range(Hq)]
        out = np.zeros((T, Hq, d), dtype=np.float64)
        full = True
    else:
        out = np.zeros((len(rows), d), dtype=np.float64)
        full = False
    cache = {}
    for n, (t, h) in enumerate(rows):
        b = int(owner[t])
        i = int(t - cu[b])
        g = h // G
        key = (t, g)
        if key not in cache:
            cache.clear()
            idx = key_rows(parent[int(cu[b]):int(cu[b + 1])], int(kv_start[b]), int(prefix_len[b]), i)
            cache[key] = (np.asarray(k[idx, g, :], np.float64), np.asarray(v[idx, g, :], np.float64))
        K, V = cache[key]
        o = attention_row(q[t, h, :], K, V, scale)
        if full:
            out[t, h] = o
        else:
            out[n] = o
    return out


# ---------------------------------------------------------------------------
# O-accept: greedy acceptance  ([TSD] "Verification and Acceptance
# Algorithms", Greedy Tree Verification)
# ---------------------------------------------------------------------------

def accept_walk_one(parent, draft, target, root_target: int, max_depth: int):
    """The greedy walk for one request: starting at the implicit root with the
    target's choice there, repeatedly look for a child (lowest index first)
    whose draft token equals the target's current choice; stop when none does
    or the node is a leaf.  Returns (path node indices, next token)."""
    n = len(parent)
    want = int(root_target)
    cur = -1
    path = []
    while len(path) < max_depth:
        kids = [j for j in range(n) if int(parent[j]) == cur]
        match = None
        for c in kids:                      # ascending index
            if int(draft[c]) >= 0 and int(draft[c]) == want:
                match = c
                break
        if match is None:
            break
        path.append(match)
        cur = match
        want = int(target[match])
    return path, want


def accept_bruteforce_one(parent, draft, target, root_target: int):
    """Independent formulation: a node is 'valid' iff every node u on its
    root->node path carries the token the target chose at u's parent (the
    root's choice for a root child).  The accepted node is the deepest valid
    node, lowest index among equals; next token = its target (or the root's
    choice when nothing is valid).  With distinct sibling tokens the valid set
    is a chain and this equals the walk."""
    n = len(parent)
    best = None
    best_len = 0
    for v in range(n):
        chain = []
        u = v
        while u >= 0:
            chain.append(u)
            u = int(parent[u])
        chain.reverse()
        ok = True
        for u in chain:
            p = int(parent[u])
            want = int(root_target) if p < 0 else int(target[p])
            if int(draft[u]) < 0 or int(draft[u]) != want:
                ok = False
                break
        if ok and len(chain) > best_len:
            best, best_len = chain, len(chain)
    if best is None:
        return [], int(root_target)
    return best, int(target[best[-1]])


def accept_greedy(parent, draft, target, root_target, cu_nodes, max_depth: int):
    """Batched walk.  Returns (accept_len [B], accept_idx [B, max_depth] padded
    with -1, next_token [B]); indices are request-local."""
    cu = np.asarray(cu_nodes)
    B = cu.shape[0] - 1
    alen = np.zeros(B, dtype=np.int32)
    aidx = np.full((B, max_depth), -1, dtype=np.int32)
    nxt = np.zeros(B, dtype=np.int32)
    for b in range(B):
        lo, hi = int(cu[b]), int(cu[b + 1])
        path, tok = accept_walk_one(parent[lo:hi], draft[lo:hi], target[lo:hi],
                                    int(root_target[b]), max_depth)
        alen[b] = len(path)
        aidx[b, :len(path)] = path
        nxt[b] = tok
    return alen, aidx, nxt


# ---------------------------------------------------------------------------
# O-compact: KV rollback as a physical gather  ([TSD] "KV Cache Rollback")
# ---------------------------------------------------------------------------

def kv_compact(k, v, kv_start, prefix_len, accept_len, accept_idx):
    """Copy of the caches where, for each request, row P+j (j < L) holds what
    row P+idx[j] held before the call; every other row is unchanged.
    Returns (k', v', new_kv_len [B])."""
    k2 = np.array(k, copy=True)
    v2 = np.array(v, copy=True)
    B = len(prefix_len)
    new_len = np.zeros(B, dtype=np.int32)
    for b in range(B):
        base = int(kv_start[b]) + int(prefix_len[b])
        L = int(accept_len[b])
        for j in range(L):
            src = base + int(accept_idx[b][j])
            k2[base + j] = k[src]
            v2[base + j] = v[src]
        new_len[b] = int(prefix_len[b]) + L
    return k2, v2, new_len


# ---------------------------------------------------------------------------
# O-argmax: the target's choice at each node ([TSD] "Verification and
# Acceptance Algorithms", greedy tree verification: the target prediction at
# a node is the argmax of its logits)
# ---------------------------------------------------------------------------

def target_argmax(logits) -> np.ndarray:
    """Row-wise argmax of logits [rows, vocab] (fp32, or bf16 widened exactly
    to fp32 by the caller).  Readings: the lowest index wins a tie (-0 and +0
    are equal); a NaN ranks above every number, so a row holding NaN returns
    its first NaN.  numpy's argmax implements exactly this rule and serves as
    the step."""
    x = np.asarray(logits, dtype=np.float64)
    if x.shape[1] == 0:
        raise ValueError("vocab must be at least 1")
    return np.argmax(x, axis=1).astype(np.int32)


def target_sample(logits, temperature: float, u) -> np.ndarray:
    """The target's sampled choice at every node, for verification at
    temperature T > 0 with a deterministic draft ([DT] section 4.1: the target
    is sampled while the draft stays deterministic; with a point-mass draft
    distribution, [TSD]'s min(1, p/q) rule accepts a child exactly when the
    target's sample equals its token).  Row r's token is drawn from
    softmax(logits[r] / T) by inverse transform with the caller's uniform
    u[r] in [0, 1): with y = x * (1/T), M = max y and w = exp(y - M) (float64),
    the token is the smallest index whose cumulative weight exceeds u * sum(w);
    if rounding leaves none, the last index with w > 0.  Readings for
    non-finite rows: a NaN gives the first NaN, else +inf the first +inf, and a
    row of -inf gives index 0."""
    x = np.asarray(logits, dtype=np.float64)
    if x.shape[1] == 0:
        raise ValueError("vocab must be at least 1")
    inv_t = 1.0 / float(temperature)
    out = np.zeros(x.shape[0], dtype=np.int32)
    for r in range(x.shape[0]):
        row = x[r]
        if np.isnan(row).any():
            out[r] = int(np.flatnonzero(np.isnan(row))[0])
            continue
        if np.isposinf(row).any():
            out[r] = int(np.flatnonzero(np.isposinf(row))[0])
            continue
        y = row * inv_t
        m = y.max()
        if m == -np.inf:
            out[r] = 0
            continue
        w = np.exp(y - m)
        c = np.cumsum(w)
        i = int(np.searchsorted(c, float(u[r]) * c[-1], side="right"))
        out[r] = i if i < row.shape[0] else int(np.flatnonzero(w > 0)[-1])
    return out


# ---------------------------------------------------------------------------
# O-rope: rotary embedding at tree position ids ([TSD] "Tree Positional
# IDs": PosID(v) = PosID(root) + depth(v) is what RoPE sees)
# ---------------------------------------------------------------------------

def rope_rotate(x, pos, base: float) -> np.ndarray:
    """Rotate the last axis of x [..., d] by position pos (broadcast over the
    leading axes).  Reading (the pages name RoPE without its formula): the
    rotate-half layout, channel i paired with channel i + d/2, angle
    pos * base**(-2i/d) for i < d/2; float64 throughout."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    inv = base ** (-2.0 * np.arange(h, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def tree_rope(q, k, pos, cu_nodes, kv_start, prefix_len, base: float):
    """q [T, Hq, d] rotated by pos[t]; the tree's K rows (cache row
    kv_start[b] + P_b + j for node j of request b) rotated by the same
    position; every other cache row unchanged.  Returns (q', k')."""
    q2 = rope_rotate(q, np.asarray(pos)[:, None], base)
    k2 = np.asarray(k, dtype=np.float64).copy()
    cu = np.asarray(cu_nodes)
    for b in range(cu.shape[0] - 1):
        lo, hi = int(cu[b]), int(cu[b + 1])
        r0 = int(kv_start[b]) + int(prefix_len[b])
        for j in range(hi - lo):
            k2[r0 + j] = rope_rotate(k2[r0 + j], np.full(k2.shape[1], pos[lo + j]), base)
    return q2, k2


# ---------------------------------------------------------------------------
# Stochastic acceptance ([TSD] "Verification and Acceptance Algorithms",
# section "Exact Sampling Equivalence": a candidate x proposed with draft
# probability q(x) is accepted with probability min(1, p(x)/q(x)); after a
# rejection a replacement is drawn from (p - q)+ normalised)
# ---------------------------------------------------------------------------

def _softmax64(logits_row, temperature: float) -> np.ndarray:
    """softmax(x / T) in float64: y = x * (1/T), w = exp(y - max y), w / sum w."""
    y = np.asarray(logits_row, dtype=np.float64) * (1.0 / float(temperature))
    w = np.exp(y - y.max())
    return w / w.sum()


def _draw(weights, u: float) -> int:
    """Inverse transform over unnormalised weights (index order): the smallest
    i whose cumulative weight exceeds u * total; if rounding leaves none, the
    last index with positive weight."""
    c = np.cumsum(np.asarray(weights, dtype=np.float64))
    i = int(np.searchsorted(c, float(u) * c[-1], side="right"))
    return i if i < len(c) else int(np.flatnonzero(np.asarray(weights) > 0)[-1])


def accept_stochastic_one(parent, draft, root_logits, node_logits, temperature: float, root_q, node_q,
                          u_accept, u_final: float, max_depth: int):
    """The stochastic walk for one request (float64 throughout).

    At the current node v (first the implicit root) the target distribution
    is p = softmax(logits_v / T) and the drafter's is q_v (the distribution
    v's children were drawn from).  The children are tried in ascending index
    with r = p: child c with token x is accepted iff u_accept[c] < min(1,
    r(x) / q_v(x)) (a token with q_v(x) = 0 is accepted iff r(x) > 0); after a
    rejection r becomes (r - q_v)+ / sum (r - q_v)+ (if that sum is 0, r is
    kept).  An accepted child becomes the current node (the walk stops after
    max_depth accepted nodes); when no child is accepted, or v has none, the
    next token is drawn from r with u_final by inverse transform.  Children
    with a negative draft token (dead leaves) are skipped.
    Returns (path node indices, next token)."""
    n = len(parent)
    cur = -1
    path = []
    while True:
        p = _softmax64(root_logits if cur < 0 else node_logits[cur], temperature)
        q = np.asarray(root_q if cur < 0 else node_q[cur], dtype=np.float64)
        r = p
        kids = [j for j in range(n) if int(parent[j]) == cur] if len(path) < max_depth else []
        accepted = None
        for c in kids:                      # ascending index
            x = int(draft[c])
            if x < 0:
                continue
            a = min(1.0, r[x] / q[x]) if q[x] > 0 else (1.0 if r[x] > 0 else 0.0)
            if float(u_accept[c]) < a:
                accepted = c
                break
            res = np.maximum(r - q, 0.0)
            tot = res.sum()
            if tot > 0:
                r = res / tot
        if accepted is None:
            return path, _draw(r, u_final)
        path.append(accepted)
        cur = accepted


def accept_stochastic(parent, draft, cu_nodes, root_logits, node_logits, temperature: float, root_q, node_q,
                      u_accept, u_final, max_depth: int):
    """accept_stochastic_one per request; node arrays are global [T, ...],
    parents request-local.  Returns (accept_len [B], accept_idx [B, max_depth]
    (-1 padded), next_token [B])."""
    cu = np.asarray(cu_nodes)
    B = cu.shape[0] - 1
    alen = np.zeros(B, np.int32)
    aidx = np.full((B, max_depth), -1, np.int32)
    nxt = np.zeros(B, np.int32)
    for b in range(B):
        lo, hi = int(cu[b]), int(cu[b + 1])
        path, t = accept_stochastic_one(parent[lo:hi], draft[lo:hi], root_logits[b], node_logits[lo:hi],
                                        temperature, root_q[b], node_q[lo:hi], u_accept[lo:hi],
                                        float(u_final[b]), max_depth)
        alen[b] = len(path)
        aidx[b, :len(path)] = path
        nxt[b] = t
    return alen, aidx, nxt


# ---------------------------------------------------------------------------
# O-rollback by token table ([TSD] "KV Cache Rollback": unaccepted nodes are
# discarded by "page table updates" in paged caches)
# ---------------------------------------------------------------------------

def token_table_rollback(req_to_token, tree_slots, cu_nodes, prefix_len, accept_len, accept_idx):
    """Paged cache with one token per page: req_to_token[b, p] is the slot of
    position p of request b, and node j of request b was written to slot
    tree_slots[lo + j].  After acceptance, positions P_b .. P_b + L_b - 1
    point at the accepted nodes' slots in path order; no K/V moves.  Returns
    (table', new_len [B], freed [T] (each request's unaccepted slots in node
    order, from its own offset lo; the rest of its region is -1), n_freed [B])."""
    tab = np.array(req_to_token, dtype=np.int32, copy=True)
    cu = np.asarray(cu_nodes)
    B = cu.shape[0] - 1
    T = int(cu[-1]) if B > 0 else 0
    new_len = np.zeros(B, np.int32)
    freed = np.full(T, -1, np.int32)
    n_freed = np.zeros(B, np.int32)
    for b in range(B):
        lo, hi = int(cu[b]), int(cu[b + 1])
        P, L = int(prefix_len[b]), int(accept_len[b])
        path = [int(x) for x in accept_idx[b, :L]]
        for j, node in enumerate(path):
            tab[b, P + j] = tree_slots[lo + node]
        new_len[b] = P + L
        rest = [tree_slots[lo + i] for i in range(hi - lo) if i not in set(path)]
        freed[lo:lo + len(rest)] = rest
        n_freed[b] = len(rest)
    return tab, new_len, freed, n_freed
