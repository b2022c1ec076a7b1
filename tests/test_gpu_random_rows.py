"""tree_mask_build and tree_accept_commit on random forests against the
oracle, through the C ABI, bit for bit.

Thirty seeded cases: batches of 1 to 12 requests whose trees are empty,
random (up to 300 nodes, depth up to 24), chains, stars or 4-ary heaps;
max_depth 4 to 64, so some trees are too deep and report their errors
([TSD] "The Tree Attention Mechanism", parts 2 and 3, for the mask, levels
and position ids); most drafts set to their parent's target (siblings may
then share a token: the lowest index wins), so accepted paths run deep
([TSD] greedy verification),
and the accepted rows of a bf16 or fp32 cache with 1 to 8 KV heads and head
dim 64 or 128 gathered into place ([TSD] "KV Cache Rollback").
"""
import numpy as np
import pytest

from oracle import tree_verify_oracle as O
from tree_attention_verification_bitmask_amd import workloads as W
from tests.gpu_util import announce, dev_workload, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tree_attention_verification_bitmask_amd import binding
    binding.lib()   # raises if the HIP library is missing: no fallback
    return binding


def forest(rng):
    batch = int(rng.integers(1, 13))
    trees = []
    for _ in range(batch):
        kind = int(rng.integers(5))
        n = int(rng.integers(0, 300)) if kind != 4 else 0
        if kind == 0:
            t = W.random_tree(rng, n, 24) if n else np.zeros(0, np.int32)
        elif kind == 1:
            t = W.chain_tree(min(n, 70))
        elif kind == 2:
            t = W.star_tree(max(n % 40, 1), rooted=bool(rng.integers(2)))   # siblings need distinct drafts
        elif kind == 3:
            t = ((np.arange(n) - 1) // 4).astype(np.int32)
            t[:1] = -1
        else:
            t = np.zeros(0, np.int32)
        trees.append(np.asarray(t, np.int32))
    prefixes = [int(x) for x in rng.integers(0, 500, batch)]
    return trees, prefixes


@pytest.mark.parametrize("case", range(30))
def test_mask_and_commit_random_forests(case):
    from tree_attention_verification_bitmask_amd import binding as B
    rng = np.random.default_rng(9000 + case)
    trees, prefixes = forest(rng)
    hkv = int(rng.choice([1, 2, 8]))
    d = int(rng.choice([64, 128]))
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    md = int(rng.choice([4, 8, 16, 24, 64]))
    announce(f"mask/commit random {case}: nodes {[len(t) for t in trees]} hkv {hkv} d {d} {dtype} max_depth {md}")
    wl = W.make_from_trees(trees, prefixes, hq=hkv, hkv=hkv, d=d, dtype=dtype, seed=case, vocab=1000)
    for b in range(wl.batch):   # most drafts carry the token their parent's target chose (ties: lowest index)
        s = wl.nodes_of(b)
        p = wl.parent[s]
        want = np.where(p < 0, wl.root_target[b], wl.target[s][np.maximum(p, 0)])
        wl.draft[s] = np.where(rng.random(len(p)) < 0.7, want, wl.draft[s])
    dv = dev_workload(wl)
    mn = max(1, wl.max_nodes)
    # the mask, levels and position ids, errors included
    anc, lev, pos, err = B.tree_mask_build(dv["parent"], dv["cu"], dv["P"], mn, md)
    torch.cuda.synchronize()
    ranc, rlev, rpos, rerr = O.mask_build(wl.parent, wl.cu_nodes, wl.prefix_len, mn, md)
    assert int(err.item()) == rerr
    assert np.array_equal(to_np(anc).view(np.uint64), ranc)
    assert np.array_equal(to_np(lev), rlev) and np.array_equal(to_np(pos), rpos)
    # the walk and the gather in one call
    k0, v0 = to_np(dv["k"]), to_np(dv["v"])
    alen, aidx, nxt, nl, cerr = B.tree_accept_commit(dv["parent"], dv["draft"], dv["target"], dv["root"], dv["cu"],
                                                     dv["ks"], dv["P"], dv["k"], dv["v"], md)
    torch.cuda.synchronize()
    assert int(cerr.item()) == 0
    ralen, raidx, rnxt = O.accept_greedy(wl.parent, wl.draft, wl.target, wl.root_target, wl.cu_nodes, md)
    rk, rv, rnl = O.kv_compact(k0, v0, wl.kv_start, wl.prefix_len, ralen, raidx)
    assert np.array_equal(to_np(alen), ralen) and np.array_equal(to_np(aidx), raidx)
    assert np.array_equal(to_np(nxt), rnxt) and np.array_equal(to_np(nl), rnl)
    assert np.array_equal(to_np(dv["k"]).view(np.uint32), rk.view(np.uint32))
    assert np.array_equal(to_np(dv["v"]).view(np.uint32), rv.view(np.uint32))
