"""tree_accept_stochastic on the GPU against the oracle, through the C ABI.

The accepted path, its length and the next token are integers decided in
float64 on both sides (only the order of additions differs), so they must
match the oracle exactly.  Inputs: random forests, each node's children drawn
from that node's draft distribution (so acceptances and rejections both
occur), independent target logits, seeded uniforms; vocabularies from 40 (many
rejections per node) to 151936 (the Qwen3 vocabulary); fp32 and bf16 logits.
Also: a point-mass target gives tree_accept_greedy's walk, max_depth cuts the
walk, and bad parents, tokens and request ranges are reported per request.
"""
import numpy as np
import pytest

from oracle import tree_verify_oracle as O
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tree_attention_verification_bitmask_amd import binding
    binding.lib()   # raises if the HIP library is missing: no fallback
    return binding


def B():
    from tree_attention_verification_bitmask_amd import binding
    return binding


def _round_bf16(x):
    f = np.asarray(x, np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)


def make_case(seed, batch, nodes, V, dead=0.05, spread=3.0, q_noise=1.0, logit_dtype="f32", root_kids=None):
    """Random forests; each node's children drawn from its q; target logits
    independent of q.  root_kids: the first root_kids nodes of each request
    are the root's children and the others hang below them."""
    rng = np.random.default_rng(seed)
    sizes = rng.integers(nodes[0], nodes[1] + 1, batch)
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    T = int(cu[-1])
    parent = np.empty(T, np.int32)
    for b in range(batch):
        lo = int(cu[b])
        for i in range(int(sizes[b])):
            if root_kids is not None:
                parent[lo + i] = -1 if i < root_kids else int(rng.integers(0, i))
            else:
                parent[lo + i] = -1 if i == 0 else int(rng.integers(-1, i))
    root_logits = rng.normal(0, spread, (batch, V)).astype(np.float32)
    node_logits = rng.normal(0, spread, (T, V)).astype(np.float32)
    if logit_dtype == "bf16":
        root_logits, node_logits = _round_bf16(root_logits), _round_bf16(node_logits)
    # draft distributions: the target's logits plus noise (a drafter that
    # roughly agrees with the target), so candidates are often but not always
    # accepted
    def qdist(logits):
        z = logits.astype(np.float64) + rng.normal(0, q_noise, logits.shape)
        z = np.exp(z - z.max(axis=1, keepdims=True))
        return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)
    root_q, node_q = qdist(root_logits), qdist(node_logits)
    draft = np.empty(T, np.int32)
    for b in range(batch):
        lo = int(cu[b])
        for i in range(int(sizes[b])):
            p = int(parent[lo + i])
            q = root_q[b] if p < 0 else node_q[lo + p]
            q64 = q.astype(np.float64)
            draft[lo + i] = int(rng.choice(V, p=q64 / q64.sum()))
    draft[rng.random(T) < dead] = -1
    u_accept = rng.random(T)
    u_final = rng.random(batch)
    return dict(parent=parent, draft=draft, cu=cu, root_logits=root_logits, node_logits=node_logits,
                root_q=root_q, node_q=node_q, u_accept=u_accept, u_final=u_final)


def run_gpu(c, temperature, max_depth, logit_dtype="f32"):
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()
    f64 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float64)).cuda()
    ldt = torch.bfloat16 if logit_dtype == "bf16" else torch.float32
    lg = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda().to(ldt).contiguous()
    f32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    alen, aidx, nxt, err = B().tree_accept_stochastic(
        i32(c["parent"]), i32(c["draft"]), i32(c["cu"]), lg(c["root_logits"]), lg(c["node_logits"]), temperature,
        f32(c["root_q"]), f32(c["node_q"]), f64(c["u_accept"]), f64(c["u_final"]), max_depth)
    torch.cuda.synchronize()
    return alen.cpu().numpy(), aidx.cpu().numpy(), nxt.cpu().numpy(), int(err.item())


def run_oracle(c, temperature, max_depth):
    return O.accept_stochastic(c["parent"], c["draft"], c["cu"], c["root_logits"].astype(np.float64),
                               c["node_logits"].astype(np.float64), temperature, c["root_q"].astype(np.float64),
                               c["node_q"].astype(np.float64), c["u_accept"], c["u_final"], max_depth)


CASES = [  # seed, batch, nodes, vocab, temperature, max_depth, logits
    (0, 8, (10, 40), 40, 1.0, 16, "f32"),
    (1, 16, (1, 64), 257, 0.7, 8, "f32"),
    (2, 4, (50, 128), 4096, 1.3, 16, "f32"),
    (3, 8, (30, 90), 4096, 1.0, 4, "bf16"),
    (4, 2, (64, 128), 151936, 1.0, 16, "f32"),
    (5, 3, (20, 60), 151936, 0.8, 16, "bf16"),
    (6, 2, (2, 4), 1500000, 1.0, 16, "f32"),     # 733 chunks: more than one block-wide tile of chunk weights
    (7, 3, (20, 40), 3001, 1.0, 16, "bf16"),     # rows not 16-byte aligned: the element-wise loads
    (8, 64, (1, 24), 1000, 0.9, 8, "f32"),       # 64 requests, trees of 1 to 24 nodes
]


@pytest.mark.parametrize("seed,batch,nodes,V,temp,D,ldt", CASES)
def test_stochastic_walk_matches_oracle(seed, batch, nodes, V, temp, D, ldt):
    announce(f"stochastic accept seed {seed} B {batch} V {V} T {temp} D {D} {ldt}")
    c = make_case(seed, batch, nodes, V, logit_dtype=ldt)
    alen, aidx, nxt, err = run_gpu(c, temp, D, ldt)
    ralen, raidx, rnxt = run_oracle(c, temp, D)
    assert err == 0
    assert np.array_equal(alen, ralen), (alen, ralen)
    assert np.array_equal(aidx, raidx)
    assert np.array_equal(nxt, rnxt), (nxt, rnxt)


def test_stochastic_walk_exercises_both_outcomes():
    """The random cases above accept and reject: check the inputs do both
    (on the oracle, so the parity tests are not vacuous)."""
    c = make_case(0, 8, (10, 40), 40)
    alen, _, _ = run_oracle(c, 1.0, 16)
    assert alen.max() >= 2 and (alen < np.diff(c["cu"])).any()


def test_point_mass_target_gives_greedy_walk():
    announce("stochastic accept: point-mass target")
    rng = np.random.default_rng(9)
    c = make_case(9, 6, (5, 50), 300)
    T = c["draft"].shape[0]
    bstar = rng.integers(0, 300, 6)
    nstar = rng.integers(0, 300, T)
    c["root_logits"][np.arange(6), bstar] = 3000.0
    c["node_logits"][np.arange(T), nstar] = 3000.0
    # drafts often equal to the parent's choice
    owner = np.searchsorted(c["cu"], np.arange(T), side="right") - 1
    want = np.where(c["parent"] < 0, bstar[owner], nstar[np.maximum(c["parent"] + c["cu"][owner], 0)])
    c["draft"] = np.where(rng.random(T) < 0.7, want, c["draft"]).astype(np.int32)
    alen, aidx, nxt, err = run_gpu(c, 1.0, 16)
    galen, gaidx, gnxt = O.accept_greedy(c["parent"], c["draft"], nstar.astype(np.int32), bstar.astype(np.int32),
                                         c["cu"], 16)
    assert err == 0
    assert np.array_equal(alen, galen) and np.array_equal(aidx, gaidx) and np.array_equal(nxt, gnxt)
    assert galen.max() >= 2


def test_errors_reported_per_request():
    announce("stochastic accept: errors")
    c = make_case(11, 4, (6, 20), 100, dead=0.0)
    lo1, lo2 = int(c["cu"][1]), int(c["cu"][2])
    c["parent"][lo1 + 3] = 5            # request 1: a parent after its child
    c["draft"][lo2 + 1] = 100           # request 2: a token outside the vocabulary
    alen, aidx, nxt, err = run_gpu(c, 1.0, 16)
    assert err == max((O.ERR_BAD_PARENT << 24) | (lo1 + 3), (B().DEVERR_BAD_TOKEN << 24) | (lo2 + 1))
    for b in (1, 2):
        assert alen[b] == 0 and nxt[b] == -1 and (aidx[b] == -1).all()
    # the good requests are walked as the oracle walks them
    for b in (0, 3):
        lo, hi = int(c["cu"][b]), int(c["cu"][b + 1])
        path, t = O.accept_stochastic_one(c["parent"][lo:hi], c["draft"][lo:hi], c["root_logits"][b].astype(np.float64),
                                          c["node_logits"][lo:hi].astype(np.float64), 1.0,
                                          c["root_q"][b].astype(np.float64), c["node_q"][lo:hi].astype(np.float64),
                                          c["u_accept"][lo:hi], float(c["u_final"][b]), 16)
        assert alen[b] == len(path) and list(aidx[b, :len(path)]) == path and nxt[b] == t


def test_many_candidates_at_one_node():
    """Roots with 40 children and a drafter far from the target, so that most
    tests reject: tests past the fourth at a node take the per-row
    continuation after the whole-GPU passes."""
    announce("stochastic accept: 40 root children")
    deep = 0
    for seed, ldt in ((21, "f32"), (22, "bf16"), (23, "f32")):
        c = make_case(seed, 3, (60, 90), 3000, q_noise=4.0, logit_dtype=ldt, root_kids=40)
        alen, aidx, nxt, err = run_gpu(c, 1.0, 16, ldt)
        ralen, raidx, rnxt = run_oracle(c, 1.0, 16)
        assert err == 0
        assert np.array_equal(alen, ralen) and np.array_equal(aidx, raidx) and np.array_equal(nxt, rnxt)
        # how far down the root's candidate list each request went
        for b in range(3):
            lo, hi = int(c["cu"][b]), int(c["cu"][b + 1])
            live = [i for i in range(hi - lo) if c["parent"][lo + i] == -1 and c["draft"][lo + i] >= 0]
            tried = live.index(int(raidx[b, 0])) + 1 if ralen[b] > 0 else len(live)
            deep += tried > 5
    assert deep >= 2, "the cases should reach the continuation"


def test_zero_residual_sum_keeps_r():
    """Target and draft the same point mass, every candidate a token the
    drafter gives probability 0: each test rejects, (r - q)+ sums to 0 so r
    stays p, and the next token is the point mass (also past the fourth
    candidate)."""
    announce("stochastic accept: zero residual sum")
    rng = np.random.default_rng(31)
    V, B = 500, 4
    c = make_case(31, B, (8, 12), V, dead=0.0, root_kids=7)
    T = c["draft"].shape[0]
    star_r = rng.integers(0, V, B)
    star_n = rng.integers(0, V, T)
    c["root_logits"][np.arange(B), star_r] = 3000.0
    c["node_logits"][np.arange(T), star_n] = 3000.0
    c["root_q"][:] = 0.0
    c["root_q"][np.arange(B), star_r] = 1.0
    c["node_q"][:] = 0.0
    c["node_q"][np.arange(T), star_n] = 1.0
    owner = np.searchsorted(c["cu"], np.arange(T), side="right") - 1
    want = np.where(c["parent"] < 0, star_r[owner], star_n[np.maximum(c["parent"] + c["cu"][owner], 0)])
    c["draft"] = ((want + 1 + rng.integers(0, V - 1, T)) % V).astype(np.int32)   # never the point mass
    alen, aidx, nxt, err = run_gpu(c, 1.0, 16)
    ralen, raidx, rnxt = run_oracle(c, 1.0, 16)
    assert err == 0
    assert (ralen == 0).all() and np.array_equal(rnxt, star_r)
    assert np.array_equal(alen, ralen) and np.array_equal(aidx, raidx) and np.array_equal(nxt, rnxt)


@pytest.mark.parametrize("nodes,D", [((0, 3), 1), ((0, 3), 16), ((0, 0), 4)])
def test_empty_trees_and_depth_one(nodes, D):
    """Requests with no nodes draw the next token from the root's p; a batch
    with no nodes at all passes empty node arrays; max_depth 1 tests only
    the root's children."""
    announce(f"stochastic accept: nodes {nodes} D {D}")
    c = make_case(41, 12, nodes, 500)
    alen, aidx, nxt, err = run_gpu(c, 1.0, D)
    ralen, raidx, rnxt = run_oracle(c, 1.0, D)
    assert err == 0
    assert np.array_equal(alen, ralen) and np.array_equal(aidx, raidx) and np.array_equal(nxt, rnxt)


@pytest.mark.parametrize("case", range(20))
def test_stochastic_random_shapes(case):
    """Seeded random shapes: 1 to 9 requests of 0 to 85 nodes, vocabularies
    from 2 to 40000 (chunk edges 2048 and 2049 included), temperatures 0.3 to
    4, max_depth 1 to 64, drafters near and far from the target, and roots
    with up to 11 children."""
    rng = np.random.default_rng(5000 + case)
    batch = int(rng.integers(1, 10))
    lo_n = int(rng.choice([0, 1, 5]))
    hi_n = lo_n + int(rng.choice([0, 3, 20, 80]))
    V = int(rng.choice([2, 3, 17, 100, 1000, 2048, 2049, 5000, 40000]))
    temp = float(rng.choice([0.3, 0.7, 1.0, 1.5, 4.0]))
    D = int(rng.choice([1, 2, 4, 16, 64]))
    ldt = "bf16" if rng.random() < 0.4 else "f32"
    qn = float(rng.choice([0.3, 1.0, 4.0]))
    rk = None if rng.random() < 0.7 else int(rng.integers(1, 12))
    announce(f"stochastic random {case}: B {batch} nodes {lo_n}-{hi_n} V {V} T {temp} D {D} {ldt} root_kids {rk}")
    c = make_case(10000 + case, batch, (lo_n, hi_n), V, q_noise=qn, logit_dtype=ldt, root_kids=rk)
    alen, aidx, nxt, err = run_gpu(c, temp, D, ldt)
    ralen, raidx, rnxt = run_oracle(c, temp, D)
    assert err == 0
    assert np.array_equal(alen, ralen) and np.array_equal(aidx, raidx) and np.array_equal(nxt, rnxt)
