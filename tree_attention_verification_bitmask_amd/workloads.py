"""Seeded synthetic inputs for the tree-verification pass.

This module only *draws* inputs: tree shapes (parent arrays), draft and target
token ids, prefix lengths, cache layout and Q/K/V values.  It computes none of
the pass's outputs (no ancestor mask, no position ids, no attention, no
acceptance, no compaction), so both the CPU oracle and the HIP path can take
their inputs from here without sharing any of the method's arithmetic.

Pages the shapes follow:
  [TSD]  "Tree-Structured Speculative Decoding: How Multi-Candidate Trees and
         Tree Attention Accelerate LLM Serving" (llms.blog).
  [DT]   "DominoTree: Conditional Tree-Structured Drafting with Domino for
         Speculative Decoding" (arXiv 2607.08642).

Tree encoding (the flattening of [TSD] "The Tree Attention Mechanism", part 1
"Tree Flattening"): node i of a request is a draft token; ``parent[i]`` is a
request-local index smaller than i, or -1 when the node hangs directly under
the implicit root, which is the last verified context token ([TSD] "Tree
Representation of Speculative Candidates").  Parents precede children, as
[DT] Appendix B ("Frontier ledger and selection") orders its selected trees.

The five named workloads:
  c1  tiny fp32 correctness case (random recursive tree, depth <= 8);
  c2  Qwen3-4B-shaped layer (best-first tree of 64 nodes, prefix 1024);
  c3  Qwen3-8B-shaped layer (best-first tree of 128 nodes, prefix 4096);
  c4  long-context layer (width-first 16 x 16 tree, prefix 8192);
  c5  8 concurrent requests, ragged prefixes 2048..8192, random trees 32..128.

Every draw uses numpy's PCG64 ``default_rng(seed)``; a call with the same
arguments returns bit-identical arrays.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field

import numpy as np

QWEN3_VOCAB = 151936

# name -> static description.  'tree' selects the shape generator.
CONFIGS = {
    "c1": dict(desc="tiny fp32: B1, Hq2/Hkv1, d64, prefix 128, random tree of 16 nodes, depth<=8",
               dtype="f32", batch=1, hq=2, hkv=1, d=64, prefix=(128, 128), nodes=(16, 16),
               max_depth=8, tree="random", vocab=1000, values="unit"),
    "c2": dict(desc="Qwen3-4B-shaped layer: B1, bf16, Hq32/Hkv8, d128, prefix 1024, best-first tree of 64",
               dtype="bf16", batch=1, hq=32, hkv=8, d=128, prefix=(1024, 1024), nodes=(64, 64),
               max_depth=16, tree="best_first", vocab=QWEN3_VOCAB, values="qwen"),
    "c3": dict(desc="Qwen3-8B-shaped layer: B1, bf16, Hq32/Hkv8, d128, prefix 4096, best-first tree of 128",
               dtype="bf16", batch=1, hq=32, hkv=8, d=128, prefix=(4096, 4096), nodes=(128, 128),
               max_depth=16, tree="best_first", vocab=QWEN3_VOCAB, values="qwen"),
    "c4": dict(desc="long-context layer: B1, bf16, Hq32/Hkv8, d128, prefix 8192, width-first 16x16 tree",
               dtype="bf16", batch=1, hq=32, hkv=8, d=128, prefix=(8192, 8192), nodes=(256, 256),
               max_depth=16, tree="width_first", vocab=QWEN3_VOCAB, values="qwen"),
    "c5": dict(desc="concurrent: B8, bf16, Hq32/Hkv8, d128, prefix U{2048..8192}, random trees of U{32..128}",
               dtype="bf16", batch=8, hq=32, hkv=8, d=128, prefix=(2048, 8192), nodes=(32, 128),
               max_depth=16, tree="random", vocab=QWEN3_VOCAB, values="qwen"),
}


@dataclass
class Workload:
    """One batch of inputs for the four calls, as host numpy arrays.

    Layouts (all C-contiguous):
      parent     int32 [T]            request-local parent index or -1
      cu_nodes   int32 [B+1]          request b owns nodes cu_nodes[b]:cu_nodes[b+1]
      prefix_len int32 [B]            P_b, cached tokens before the tree
      kv_start   int32 [B]            first cache row of request b
      q          float32 [T, Hq, d]   (bf16-representable when dtype == 'bf16')
      k, v       float32 [kv_rows, Hkv, d]; request b's prefix is rows
                 kv_start[b] + [0, P_b), its tree node j is row kv_start[b] + P_b + j
      draft      int32 [T]            draft token of each node (negative = dead leaf)
      target     int32 [T]            target model's greedy choice after each node
      root_target int32 [B]           target's greedy choice at the implicit root
    """
    name: str
    dtype: str
    hq: int
    hkv: int
    d: int
    max_depth: int
    parent: np.ndarray
    cu_nodes: np.ndarray
    prefix_len: np.ndarray
    kv_start: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    draft: np.ndarray
    target: np.ndarray
    root_target: np.ndarray
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.cu_nodes.shape[0] - 1)

    @property
    def total_nodes(self) -> int:
        return int(self.cu_nodes[-1])

    @property
    def kv_rows(self) -> int:
        return int(self.k.shape[0])

    @property
    def max_nodes(self) -> int:
        return int(np.max(np.diff(self.cu_nodes))) if self.batch else 0

    @property
    def max_prefix(self) -> int:
        return int(np.max(self.prefix_len)) if self.batch else 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def nodes_of(self, b: int) -> slice:
        return slice(int(self.cu_nodes[b]), int(self.cu_nodes[b + 1]))


# ----------------------------------------------------------------------------
# value helpers
# ----------------------------------------------------------------------------

def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as
    float32 so that both sides see exactly the same bf16-representable numbers.
    Non-finite inputs are not expected here."""
    u = np.array(x, dtype=np.float32, copy=True, order="C").view(np.uint32)
    lsb = u >> 16
    lsb &= 1
    u += np.uint32(0x7FFF)
    u += lsb
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of bf16-representable float32 values (as uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float32 values."""
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# tree shapes
# ----------------------------------------------------------------------------

def random_tree(rng: np.random.Generator, n: int, max_depth: int) -> np.ndarray:
    """parent[i] uniform over {-1, 0, .., i-1}, redrawn while it would put node i
    deeper than max_depth (so: uniform over the admissible parents)."""
    parent = np.empty(n, dtype=np.int32)
    depth = np.empty(n, dtype=np.int64)  # generator bookkeeping only
    for i in range(n):
        while True:
            p = int(rng.integers(-1, i)) if i > 0 else -1
            dp = 1 if p < 0 else depth[p] + 1
            if dp <= max_depth:
                break
        parent[i] = p
        depth[i] = dp
    return parent


def best_first_tree(rng: np.random.Generator, n: int, max_depth: int, m: int = 4) -> np.ndarray:
    """Shape of a best-first (max-heap) draft tree, as DDTree / DominoTree build
    it ([DT] section 2.4 and Appendix B): each expanded node (and the implicit
    root) offers m children whose probabilities decay geometrically,
    p_r proportional to gamma^r with gamma ~ U(0.2, 0.8) drawn per node; a
    node's score is the sum of log-probabilities on its path; the highest
    score is popped next (ties by insertion order) until n nodes are placed.
    Children of nodes at max_depth are not offered.  Node index = pop order,
    so parents precede children."""
    parent = np.empty(n, dtype=np.int32)
    heap: list = []
    counter = 0

    def offer(par_idx: int, par_score: float, par_depth: int):
        nonlocal counter
        if par_depth >= max_depth:
            return
        gamma = float(rng.uniform(0.2, 0.8))
        w = gamma ** np.arange(m, dtype=np.float64)
        logp = np.log(w / w.sum())
        for r in range(m):
            heapq.heappush(heap, (-(par_score + logp[r]), counter, par_idx, par_depth + 1))
            counter += 1

    offer(-1, 0.0, 0)
    for i in range(n):
        neg_score, _, par, dep = heapq.heappop(heap)
        parent[i] = par
        offer(i, -neg_score, dep)
    return parent


def width_first_tree(rng: np.random.Generator, levels: int, width: int) -> np.ndarray:
    """Fixed-width tree: `levels` levels of `width` nodes, level-major indices;
    level-1 nodes hang under the implicit root, every deeper node picks its
    parent uniformly among the previous level's nodes."""
    parent = np.empty(levels * width, dtype=np.int32)
    parent[:width] = -1
    for lev in range(1, levels):
        lo = (lev - 1) * width
        parent[lev * width:(lev + 1) * width] = rng.integers(lo, lo + width, size=width)
    return parent


def chain_tree(n: int) -> np.ndarray:
    """A chain: node i's parent is i-1 (a linear draft)."""
    return np.arange(-1, n - 1, dtype=np.int32)


def star_tree(n: int, rooted: bool) -> np.ndarray:
    """All nodes under the implicit root (rooted=False) or under node 0."""
    if rooted:
        p = np.zeros(n, dtype=np.int32)
        p[0] = -1
        return p
    return np.full(n, -1, dtype=np.int32)


def _depths(parent: np.ndarray) -> np.ndarray:
    # generator bookkeeping (used to pick a deepest node for forced acceptance)
    dep = np.empty(parent.shape[0], dtype=np.int64)
    for i, p in enumerate(parent):
        dep[i] = 1 if p < 0 else dep[p] + 1
    return dep


# ----------------------------------------------------------------------------
# tokens
# ----------------------------------------------------------------------------

def draw_tokens(rng: np.random.Generator, parent: np.ndarray, vocab: int,
                force_path: bool = False):
    """Draft tokens distinct among siblings; target tokens by the 50% rule: for
    the implicit root and every node with children, with probability 1/2 the
    target's choice equals the draft token of a uniformly chosen child, else it
    is uniform over the vocabulary.  With force_path the targets along one
    root-to-deepest-node path are set so that the whole path matches.
    Returns (draft[N], target[N], root_target)."""
    n = parent.shape[0]
    children: list[list[int]] = [[] for _ in range(n + 1)]  # slot n = implicit root
    for i in range(n):
        children[n if parent[i] < 0 else parent[i]].append(i)
    draft = np.empty(n, dtype=np.int32)
    for kids in children:
        if kids:
            while True:  # distinct among siblings: redraw on a collision
                toks = rng.integers(0, vocab, size=len(kids))
                if len(np.unique(toks)) == len(kids):
                    break
            draft[kids] = toks
    target = rng.integers(0, vocab, size=n + 1).astype(np.int32)
    for slot, kids in enumerate(children):
        if kids and rng.random() < 0.5:
            target[slot] = draft[kids[int(rng.integers(0, len(kids)))]]
    if force_path and n:
        dep = _depths(parent)
        node = int(np.argmax(dep))
        path = [node]
        while parent[path[-1]] >= 0:
            path.append(int(parent[path[-1]]))
        path.reverse()
        target[n] = draft[path[0]]
        for a, b in zip(path[:-1], path[1:]):
            target[a] = draft[b]
    return draft, target[:n].copy(), int(target[n])


# ----------------------------------------------------------------------------
# full workloads
# ----------------------------------------------------------------------------

def _draw_values(rng, shape, kind: str, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if kind == "qwen":
        x *= np.float32(1.0 / math.sqrt(128.0))
    if dtype == "bf16":
        x = round_to_bf16(x)
    return x


def make_workload(name: str, seed: int = 0, force_path: bool = False,
                  values: str | None = None, **override) -> Workload:
    """Build one of the named workloads (see CONFIGS) with the given seed.

    values: None = the config's own distribution; 'sensitive' = the
    mask-sensitivity recipe (Q, K ~ N(0,1) so logits have unit spread, and
    every tree node's V row carries a large node-specific offset, so that
    attending one wrong tree key moves the output by O(1)).
    override: replace any CONFIGS field (e.g. prefix=(0, 0), nodes=(7, 7)).
    """
    cfg = dict(CONFIGS[name])
    cfg.update(override)
    rng = np.random.default_rng(seed)
    B, hq, hkv, d = cfg["batch"], cfg["hq"], cfg["hkv"], cfg["d"]
    D = cfg["max_depth"]
    lo, hi = cfg["prefix"]
    prefix = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    nlo, nhi = cfg["nodes"]
    parents, drafts, targets, roots = [], [], [], []
    for b in range(B):
        n = int(rng.integers(nlo, nhi + 1))
        shape = cfg["tree"]
        if shape == "random":
            par = random_tree(rng, n, D)
        elif shape == "best_first":
            par = best_first_tree(rng, n, D, m=cfg.get("m", 4))
        elif shape == "width_first":
            width = cfg.get("width", 16)
            assert n % width == 0
            par = width_first_tree(rng, n // width, width)
        elif shape == "chain":
            par = chain_tree(n)
        elif shape == "star":
            par = star_tree(n, rooted=False)
        else:
            raise ValueError(shape)
        dr, tg, rt = draw_tokens(rng, par, cfg["vocab"], force_path=force_path)
        parents.append(par)
        drafts.append(dr)
        targets.append(tg)
        roots.append(rt)
    sizes = np.array([p.shape[0] for p in parents], dtype=np.int64)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(sizes)
    kv_len = prefix.astype(np.int64) + sizes
    kv_start = np.zeros(B, dtype=np.int32)
    kv_start[1:] = np.cumsum(kv_len)[:-1]
    kv_rows = int(kv_len.sum())
    T = int(cu[-1])
    kind = values or cfg["values"]
    dtype = cfg["dtype"]
    if kind == "sensitive":
        q = _draw_values(rng, (T, hq, d), "unit", dtype)
        k = _draw_values(rng, (kv_rows, hkv, d), "unit", dtype)
        v = _draw_values(rng, (kv_rows, hkv, d), "qwen", dtype)
        for b in range(B):
            n = int(sizes[b])
            for j in range(n):
                row = int(kv_start[b]) + int(prefix[b]) + j
                off = np.float32(10.0 * (j + 1) / max(n, 1))
                v[row, :, j % d] += off
        if dtype == "bf16":
            v = round_to_bf16(v)
    else:
        q = _draw_values(rng, (T, hq, d), kind, dtype)
        k = _draw_values(rng, (kv_rows, hkv, d), kind, dtype)
        v = _draw_values(rng, (kv_rows, hkv, d), kind, dtype)
    return Workload(
        name=name, dtype=dtype, hq=hq, hkv=hkv, d=d, max_depth=D,
        parent=np.concatenate(parents).astype(np.int32) if parents else np.zeros(0, np.int32),
        cu_nodes=cu, prefix_len=prefix, kv_start=kv_start,
        q=q, k=k, v=v,
        draft=np.concatenate(drafts).astype(np.int32) if drafts else np.zeros(0, np.int32),
        target=np.concatenate(targets).astype(np.int32) if targets else np.zeros(0, np.int32),
        root_target=np.array(roots, dtype=np.int32),
        seed=seed, meta=dict(cfg=cfg, values=kind, force_path=force_path),
    )


def make_from_trees(parents: list, prefix_len: list, hq: int, hkv: int, d: int,
                    dtype: str, seed: int = 0, max_depth: int = 16, vocab: int = 1000,
                    values: str = "unit") -> Workload:
    """A workload over caller-given parent arrays (one per request), with the
    same token and value recipes as make_workload."""
    rng = np.random.default_rng(seed)
    B = len(parents)
    drafts, targets, roots = [], [], []
    for par in parents:
        dr, tg, rt = draw_tokens(rng, np.asarray(par, dtype=np.int32), vocab)
        drafts.append(dr)
        targets.append(tg)
        roots.append(rt)
    sizes = np.array([len(p) for p in parents], dtype=np.int64)
    prefix = np.asarray(prefix_len, dtype=np.int32)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(sizes)
    kv_len = prefix.astype(np.int64) + sizes
    kv_start = np.zeros(B, dtype=np.int32)
    if B:
        kv_start[1:] = np.cumsum(kv_len)[:-1]
    kv_rows = int(kv_len.sum())
    T = int(cu[-1])
    q = _draw_values(rng, (T, hq, d), values, dtype)
    k = _draw_values(rng, (kv_rows, hkv, d), values, dtype)
    v = _draw_values(rng, (kv_rows, hkv, d), values, dtype)
    return Workload(
        name="custom", dtype=dtype, hq=hq, hkv=hkv, d=d, max_depth=max_depth,
        parent=np.concatenate([np.asarray(p, np.int32) for p in parents]) if B else np.zeros(0, np.int32),
        cu_nodes=cu, prefix_len=prefix, kv_start=kv_start, q=q, k=k, v=v,
        draft=np.concatenate(drafts).astype(np.int32) if B else np.zeros(0, np.int32),
        target=np.concatenate(targets).astype(np.int32) if B else np.zeros(0, np.int32),
        root_target=np.array(roots, dtype=np.int32), seed=seed, meta=dict(values=values),
    )


# ---------------------------------------------------------------------------
# Frontier ledgers: the input of tree_select_topb ([DT] section 3.3 and
# Appendix B: [batch, D, W*k] slots, each a cumulative log-probability, a
# parent slot at the previous depth and a draft token).
# ---------------------------------------------------------------------------

def random_ledger(rng: np.random.Generator, batch: int, depth: int, width: int, k: int,
                  p_empty: float = 0.0, tie_step: float = 0.0):
    """A ledger whose scores never rise along a parent pointer: slot e of
    depth t (lane e // k, child e % k) hangs under a random live slot of depth
    t - 1 and scores its parent's score minus a positive step (an exponential
    draw, or a multiple of ``tie_step`` -- zero included -- when it is set, to
    make ties).  A fraction ``p_empty`` of slots is empty (score -inf).
    Returns (score float32, parent int32, token int32), each [batch, depth,
    width * k]."""
    L = width * k
    score = np.full((batch, depth, L), -np.inf, np.float32)
    parent = np.full((batch, depth, L), -1, np.int32)
    token = rng.integers(0, 151936, (batch, depth, L)).astype(np.int32)
    for b in range(batch):
        for t in range(depth):
            if tie_step > 0:
                step = (rng.integers(0, 4, L) * tie_step).astype(np.float32)
            else:
                step = rng.exponential(0.7, L).astype(np.float32)
            live = rng.random(L) >= p_empty
            if t == 0:
                score[b, 0, live] = -step[live]
                continue
            prev = np.flatnonzero(np.isfinite(score[b, t - 1]))
            if prev.size == 0:
                continue
            par = prev[rng.integers(0, prev.size, L)]
            parent[b, t] = par
            s = (score[b, t - 1, par] - step).astype(np.float32)
            score[b, t, live] = s[live]
    return score, parent, token


def frontier_shaped_ledger(rng: np.random.Generator, batch: int, depth: int, width: int, k: int):
    """A ledger with the frontier builder's shape ([DT] section 3.3): depth 1
    holds the root's k children; at every later depth the `width` best slots
    of the previous depth (by score; ties by slot) are the lanes, and lane l's
    k children fill slots l*k .. l*k+k-1 with probabilities p_r ~ gamma^r
    (gamma ~ U(0.2, 0.8) per lane, normalised) added to the lane's score in
    float32.  Slots of lanes that do not exist stay empty.  Returns (score
    float32, parent int32, token int32), each [batch, depth, width * k]."""
    L = width * k
    score = np.full((batch, depth, L), -np.inf, np.float32)
    parent = np.full((batch, depth, L), -1, np.int32)
    token = np.full((batch, depth, L), -1, np.int32)
    r = np.arange(k)
    for b in range(batch):
        lane_slot = np.array([-1])
        lane_score = np.zeros(1, np.float32)
        for t in range(depth):
            nl = lane_slot.size
            gamma = rng.uniform(0.2, 0.8, nl)
            w = gamma[:, None] ** r[None, :]
            logp = np.log(w / w.sum(axis=1, keepdims=True)).astype(np.float32)
            slots = (np.arange(nl)[:, None] * k + r[None, :]).reshape(-1)
            score[b, t, slots] = (lane_score[:, None] + logp).reshape(-1).astype(np.float32)
            parent[b, t, slots] = np.repeat(lane_slot, k) if t > 0 else -1
            for li in range(nl):
                token[b, t, li * k:(li + 1) * k] = rng.choice(151936, size=k, replace=False)
            live = np.flatnonzero(np.isfinite(score[b, t]))
            order = live[np.lexsort((live, -score[b, t, live].astype(np.float64)))]
            lane_slot = order[:width].astype(np.int32)
            lane_score = score[b, t, lane_slot]
    return score, parent, token


# ---------------------------------------------------------------------------
# Gated-DeltaNet layer inputs for tree-aware recurrent verification.  The
# layer shape is a stand-in (the page names a hybrid Gated-DeltaNet target but
# prints no layer sizes): 16 query/key heads and 32 value heads of 128
# channels, a width-4 short convolution over the 2*16*128 + 32*128 = 8192
# mixed channels.
# ---------------------------------------------------------------------------

GDN_LAYER = dict(hk=16, hv=32, dk=128, dv=128, conv_k=4)


@dataclass
class GdnInputs:
    parent: np.ndarray       # int32 [T], per-request local parents
    cu_nodes: np.ndarray     # int32 [B+1]
    x: np.ndarray            # float32 [T, C], bf16-representable: the layer's mixed inputs
    conv_state: np.ndarray   # float32 [B, K-1, C], bf16-representable, oldest first
    conv_w: np.ndarray       # float32 [C, K], bf16-representable
    q: np.ndarray            # float32 [T, Hk, dk], bf16-representable
    k: np.ndarray            # float32 [T, Hk, dk]
    v: np.ndarray            # float32 [T, Hv, dv]
    g: np.ndarray            # float32 [T, Hv], log decay (<= 0)
    beta: np.ndarray         # float32 [T, Hv], write strength in (0, 1)
    state: np.ndarray        # float32 [B, Hv, dv, dk], the committed recurrent state
    max_depth: int


def gdn_inputs(rng: np.random.Generator, parents: list, hk: int = 16, hv: int = 32, dk: int = 128,
               dv: int = 128, conv_k: int = 4, state_std: float = 0.1) -> GdnInputs:
    """Seeded synthetic inputs for one Gated-DeltaNet layer over a batch of
    draft trees (one parent array per request).  x, conv_state, q, k, v ~
    N(0, 1) and the conv weights ~ N(0, 1/4), all rounded to bf16; the log
    decay g ~ -U(0.01, 0.5) and beta ~ U(0.05, 0.95); the committed state ~
    N(0, state_std) in float32."""
    B = len(parents)
    sizes = np.array([len(p) for p in parents], dtype=np.int64)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(sizes)
    T = int(cu[-1])
    C = 2 * hk * dk + hv * dv
    depth = max([int(_depths(np.asarray(p)).max()) if len(p) else 1 for p in parents] + [1])
    nrm = lambda *s: round_to_bf16(rng.standard_normal(size=s, dtype=np.float32))
    return GdnInputs(
        parent=np.concatenate([np.asarray(p, np.int32) for p in parents]) if T else np.zeros(0, np.int32),
        cu_nodes=cu,
        x=nrm(T, C),
        conv_state=nrm(B, conv_k - 1, C),
        conv_w=round_to_bf16(rng.standard_normal(size=(C, conv_k), dtype=np.float32) * np.float32(0.5)),
        q=nrm(T, hk, dk),
        k=nrm(T, hk, dk),
        v=nrm(T, hv, dv),
        g=-rng.uniform(0.01, 0.5, size=(T, hv)).astype(np.float32),
        beta=rng.uniform(0.05, 0.95, size=(T, hv)).astype(np.float32),
        state=(rng.standard_normal(size=(B, hv, dv, dk), dtype=np.float32) * np.float32(state_std)),
        max_depth=depth,
    )
