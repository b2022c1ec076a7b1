"""CPU oracle for the one-shot selection of a draft tree from a frontier ledger.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module; the product path (the HIP
library and its Python binding) never does and shares no code with it.

Pages followed:
  [DT]  "DominoTree: Conditional Tree-Structured Drafting with Domino for
        Speculative Decoding" (arXiv 2607.08642), section 3.3 and Appendix B.
        In short: the drafter keeps W frontier lanes per request and grows
        them one depth at a time; each candidate it scores is recorded once
        (its path log-probability and the slot of its parent), and only after
        the last depth is the tree picked, in one step, as the B best records
        overall.  The picked records are then renumbered so that every parent
        comes before its children, the parent slots are translated into the
        new numbering, and a request with fewer than B usable records is
        filled up with leaves that can never be accepted.  Because extending
        a path never raises its log-probability, the B best records already
        contain every ancestor of each one they contain, which is why (with
        W = B) the pick agrees with a best-first heap.
  [DAR] "DARTree: Speculative Diffusion Decoding with Autoregressive Draft
        Trees" (gist.science), Technical Summary, "2. Deferred Best-First
        Pruning": one global top-B over the fixed-width supertree, equal to
        the sequential max-heap's choice when a non-positive depth bonus
        beta is added (Lemma 1).

Readings taken where the pages leave a step open (each is also listed in the
design notes):
  * ledger layout [batch, D, L] with L = W*k slots per depth; depth index t
    holds candidates at tree level t + 1.  parent[b, 0, e] == -1 (children of
    the root); for t > 0, parent[b, t, e] is the slot index (0..L-1) of the
    parent candidate at depth t - 1.  A slot with a non-finite score is empty.
  * the selection key is score + beta * level, evaluated in float64 (the
    float32 score and beta widen exactly; beta * level is exact; one
    rounding in the sum).  Keys compare in descending order; equal keys go
    by depth, then by slot (the frontier's tie rule in [DT] Appendix B),
    i.e. by flat entry index t * L + e ascending.
  * output order = that ranking, so with non-increasing keys along every
    path parents precede children, and on tie-free inputs it is the heap's
    pop order.
  * dead leaves: parent -1 (a root child) and token -1, which the greedy
    walk never accepts.
  * a selected candidate whose parent slot is out of range, not selected, or
    ranked after it (possible only when keys rise along a path, e.g.
    beta > 0) is reported as a bad ledger and emitted as a dead leaf, so the
    output always lists parents before children.

Parity pins (tests/test_select_pins.py): selection against a brute-force
ranking written independently, the heap equivalence on tie-free inputs at
batch sizes 1, 2, 5 and 32 ([DT] Appendix B), ancestor closure, the dead-leaf
padding and the bad-ledger report.
"""
from __future__ import annotations

import heapq
import zlib

import numpy as np

ERR_BAD_LEDGER = 5  # a selected candidate's parent is out of range, unselected or ranked later


def _enc(code: int, index: int) -> int:
    return (code << 24) | (index & 0xFFFFFF)


# ---------------------------------------------------------------------------
# Selection: global top B of a ledger ([DT] Appendix B; [DAR] "Deferred
# Best-First Pruning")
# ---------------------------------------------------------------------------

def selection_keys(score, beta: float) -> np.ndarray:
    """key[t, e] = score[t, e] + beta * (t + 1) in float64, -inf for an empty
    slot (non-finite score)."""
    s = np.asarray(score, dtype=np.float32).astype(np.float64)
    D = s.shape[0]
    lev = np.arange(1, D + 1, dtype=np.float64)[:, None]
    key = s + np.float64(np.float32(beta)) * lev
    key[~np.isfinite(key)] = -np.inf
    return key


def select_one(score, parent, token, budget: int, beta: float):
    """One request.  score/parent/token: [D, L].  Returns (tree_parent
    [budget], tree_token [budget], n_real, bad) where bad is True if some
    selected candidate had to be emitted as a dead leaf."""
    score = np.asarray(score)
    D, L = score.shape
    key = selection_keys(score, beta)
    flat = key.reshape(-1)
    cand = [e for e in range(D * L) if np.isfinite(flat[e])]
    # descending key; equal keys by depth then slot = by flat index ascending
    cand.sort(key=lambda e: (-flat[e], e))
    chosen = cand[:budget]
    pos = {e: i for i, e in enumerate(chosen)}
    tp = np.full(budget, -1, dtype=np.int32)
    tt = np.full(budget, -1, dtype=np.int32)
    bad = False
    for i, e in enumerate(chosen):
        t, slot = divmod(e, L)
        p = int(parent[t, slot])
        if t == 0:
            ok = p == -1
            pp = -1
        else:
            # the parent must be chosen and ranked before its child
            ok = 0 <= p < L and pos.get((t - 1) * L + p, i) < i
            pp = pos[(t - 1) * L + p] if ok else -1
        if not ok:
            bad = True
            continue  # dead leaf: parent -1, token -1
        tp[i] = pp
        tt[i] = int(token[t, slot])
    return tp, tt, len(chosen), bad


def select_topb(score, parent, token, budget: int, beta: float = 0.0):
    """Batched selection.  score/parent/token: [batch, D, L].  Returns
    (tree_parent [batch, budget], tree_token [batch, budget], n_real [batch],
    err) with err 0 or the largest (ERR_BAD_LEDGER << 24 | b)."""
    score = np.asarray(score)
    Bt = score.shape[0]
    tp = np.zeros((Bt, budget), np.int32)
    tt = np.zeros((Bt, budget), np.int32)
    nr = np.zeros(Bt, np.int32)
    err = 0
    for b in range(Bt):
        tp[b], tt[b], nr[b], bad = select_one(score[b], parent[b], token[b], budget, beta)
        if bad:
            err = max(err, _enc(ERR_BAD_LEDGER, b))
    return tp, tt, nr, err


# ---------------------------------------------------------------------------
# A synthetic drafter, the frontier builder and the sequential heap ([DT]
# section 3.3 and Appendix B).  The scorer stands in for the drafter's
# conditional correction: node u's k children get probabilities
# p_r ~ gamma_u^r (r = 0..k-1, normalised), gamma_u ~ U(0.2, 0.8) drawn from a
# seed keyed by u's root path, as in the best-first tree shapes of the
# workloads; child tokens are distinct among siblings.
# ---------------------------------------------------------------------------

class PathScorer:
    def __init__(self, seed: int, k: int, vocab: int = 151936):
        self.seed = int(seed)
        self.k = int(k)
        self.vocab = int(vocab)

    def children(self, path: tuple):
        """(log p float32 [k], token int [k]) for the node at `path` (a tuple
        of child ranks from the root; () is the root)."""
        h = zlib.crc32(np.asarray((self.seed,) + tuple(path), dtype=np.int64).tobytes())
        rng = np.random.default_rng(h)
        gamma = rng.uniform(0.2, 0.8)
        w = gamma ** np.arange(self.k, dtype=np.float64)
        logp = np.log(w / w.sum()).astype(np.float32)
        tok = rng.choice(self.vocab, size=self.k, replace=False).astype(np.int64)
        return logp, tok


def frontier_ledger(scorer: PathScorer, D: int, W: int):
    """The frontier builder for one request ([DT] section 3.3): depth 1 scores
    the root's k children; every later depth scores the k children of each of
    the W lanes kept from the previous depth, then keeps the top W by
    cumulative log-probability (float32 sums; ties by slot).  Every scored
    candidate goes to the ledger.  Returns (score float32 [D, W*k], parent
    int32 [D, W*k], token int32 [D, W*k])."""
    k = scorer.k
    L = W * k
    score = np.full((D, L), -np.inf, np.float32)
    parent = np.full((D, L), -1, np.int32)
    token = np.full((D, L), -1, np.int32)
    # lanes: (slot at previous depth, path, cumulative score)
    lanes = [(-1, (), np.float32(0.0))]
    for t in range(D):
        cands = []
        for li, (pslot, path, s0) in enumerate(lanes):
            logp, tok = scorer.children(path)
            for r in range(k):
                e = li * k + r
                sc = np.float32(s0 + logp[r])
                score[t, e] = sc
                parent[t, e] = pslot if t > 0 else -1
                token[t, e] = tok[r]
                cands.append((e, path + (r,), sc))
        cands.sort(key=lambda c: (-float(c[2]), c[0]))
        lanes = [(e, p, s) for (e, p, s) in cands[:W]]
    return score, parent, token


def heap_tree(scorer: PathScorer, D: int, B: int, beta: float = 0.0):
    """Sequential best-first expansion ([DT] Appendix B): a max-heap on the
    selection key, seeded with the root's children; pop the best node, append
    it to the tree, push its children unless it is at level D; B pops.  Ties
    go by insertion order.  Returns (tree_parent [B], tree_token [B]) in pop
    order, dead-leaf padded if fewer than B nodes exist."""
    bk = np.float64(np.float32(beta))
    heap = []
    counter = 0

    def push(path, sc, par_pos, tok):
        nonlocal counter
        key = np.float64(sc) + bk * len(path)
        heapq.heappush(heap, (-key, counter, path, sc, par_pos, tok))
        counter += 1

    logp, tok = scorer.children(())
    for r in range(scorer.k):
        push((r,), np.float32(logp[r]), -1, int(tok[r]))
    tp = np.full(B, -1, np.int32)
    tt = np.full(B, -1, np.int32)
    for i in range(B):
        if not heap:
            break
        _, _, path, sc, par_pos, tk = heapq.heappop(heap)
        tp[i] = par_pos
        tt[i] = tk
        if len(path) < D:
            logp, tok = scorer.children(path)
            for r in range(scorer.k):
                push(path + (r,), np.float32(sc + logp[r]), i, int(tok[r]))
    return tp, tt
