"""tree_attn_verify on random shapes against the oracle, through the C ABI.

Forty seeded cases: batches of 1 to 8 requests whose trees are empty, tiny
(fewer than 32 rows per KV head) or up to 89 nodes (chains of at most 64, so
that every level stays within max_depth 64), prefixes from 0 to 9000 keys,
1 to 8 KV heads with GQA groups of 1 to 8, head dim 64 or 128, bf16 (the
matrix-core kernel in whichever order the plan picks) and fp32 (the vector
kernel).  The oracle is float64 attention straight from the parent arrays
([TSD] "The Tree Attention Mechanism", parts 1 and 2); large cases are
compared on a sample of (node, head) rows.
"""
import numpy as np
import pytest

from oracle import tree_verify_oracle as O
from tree_attention_verification_bitmask_amd import workloads as W
from tests.gpu_util import announce, assert_attn_close, dev_workload, sample_rows, to_np

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tree_attention_verification_bitmask_amd import binding
    binding.lib()   # raises if the HIP library is missing: no fallback
    return binding


def random_case(rng):
    batch = int(rng.choice([1, 1, 2, 3, 5, 8]))
    small = rng.random() < 0.5
    trees, prefixes = [], []
    for _ in range(batch):
        n = int(rng.integers(0, 8)) if small else int(rng.integers(1, 90))
        kind = int(rng.integers(3))
        if kind == 0:
            t = W.chain_tree(min(n, 64))
        else:
            t = W.random_tree(rng, n, 16) if n else np.zeros(0, np.int32)
        trees.append(np.asarray(t, np.int32))
        prefixes.append(int(rng.choice([0, 1, 17, 300, 1500, 4100, 9000])))
    if sum(len(t) for t in trees) == 0:
        trees[0] = W.chain_tree(1)
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 4, 8]))
    d = int(rng.choice([64, 128]))
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    return trees, prefixes, hkv, G, d, dtype


@pytest.mark.parametrize("case", range(40))
def test_attn_random_shapes(case):
    from tree_attention_verification_bitmask_amd import binding as B
    trees, prefixes, hkv, G, d, dtype = random_case(np.random.default_rng(7000 + case))
    announce(f"attn random {case}: nodes {[len(t) for t in trees]} P {prefixes} hkv {hkv} G {G} d {d} {dtype}")
    wl = W.make_from_trees(trees, prefixes, hq=hkv * G, hkv=hkv, d=d, dtype=dtype, seed=case, values="qwen")
    dv = dev_workload(wl)
    mn = max(1, wl.max_nodes)
    anc, _, _, merr = B.tree_mask_build(dv["parent"], dv["cu"], dv["P"], mn, 64)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = B.tree_attn_verify(dv["q"], dv["k"], dv["v"], dv["cu"], dv["ks"], dv["P"], anc, mn, wl.max_prefix, err=err)
    torch.cuda.synchronize()
    assert int(merr.item()) == 0 and int(err.item()) == 0
    rows = sample_rows(wl, 160, case) if wl.total_nodes * wl.hq > 2000 else None
    ref = O.tree_attention(wl.q, wl.k, wl.v, wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len, wl.scale, rows=rows)
    ref_abs = O.tree_attention(wl.q, wl.k, np.abs(wl.v), wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len,
                               wl.scale, rows=rows)
    o = to_np(out)
    if rows is not None:
        o = np.stack([o[t, h] for t, h in rows])
    assert_attn_close(o, ref, ref_abs, dtype, stated=True, what=f"random {case}")


def random_fp32_case(rng):
    """fp32 shapes for the vector kernel's tiles: GQA groups of 1 to 16 (tiles
    of 1 to 8 query heads, several tiles per KV head when the group exceeds 8)
    and trees of up to 160 nodes, so that tiles of 4, 2 and 1 nodes all occur,
    with ragged last tiles."""
    batch = int(rng.choice([1, 1, 2, 4]))
    trees, prefixes = [], []
    for _ in range(batch):
        n = int(rng.integers(1, 161))
        t = W.chain_tree(min(n, 64)) if rng.random() < 0.2 else W.random_tree(rng, n, 16)
        trees.append(np.asarray(t, np.int32))
        prefixes.append(int(rng.choice([0, 5, 130, 1100, 4100])))
    hkv = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
    d = int(rng.choice([64, 128]))
    return trees, prefixes, hkv, G, d


@pytest.mark.parametrize("case", range(24))
def test_attn_random_fp32_groups(case):
    from tree_attention_verification_bitmask_amd import binding as B
    trees, prefixes, hkv, G, d = random_fp32_case(np.random.default_rng(7500 + case))
    announce(f"attn fp32 random {case}: nodes {[len(t) for t in trees]} P {prefixes} hkv {hkv} G {G} d {d}")
    wl = W.make_from_trees(trees, prefixes, hq=hkv * G, hkv=hkv, d=d, dtype="f32", seed=case, values="qwen")
    dv = dev_workload(wl)
    anc, _, _, merr = B.tree_mask_build(dv["parent"], dv["cu"], dv["P"], wl.max_nodes, 64)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = B.tree_attn_verify(dv["q"], dv["k"], dv["v"], dv["cu"], dv["ks"], dv["P"], anc, wl.max_nodes,
                             wl.max_prefix, err=err)
    torch.cuda.synchronize()
    assert int(merr.item()) == 0 and int(err.item()) == 0
    rows = sample_rows(wl, 160, case) if wl.total_nodes * wl.hq > 2000 else None
    ref = O.tree_attention(wl.q, wl.k, wl.v, wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len, wl.scale, rows=rows)
    ref_abs = O.tree_attention(wl.q, wl.k, np.abs(wl.v), wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len,
                               wl.scale, rows=rows)
    o = to_np(out)
    if rows is not None:
        o = np.stack([o[t, h] for t, h in rows])
    assert_attn_close(o, ref, ref_abs, "f32", stated=True, what=f"fp32 random {case}")


@pytest.mark.parametrize("splits", [2, 3, 7, 40, 1000])
def test_attn_fp32_forced_slices(splits):
    """The vector kernel's key-axis slices and their merge, at slice counts the
    plan override fixes (1000 is clamped to the number of 64-key chunks):
    two requests whose key axes end inside different slices, one of them
    with no prefix, so that some slices hold no key a row sees."""
    from tree_attention_verification_bitmask_amd import binding as B
    trees = [W.random_tree(np.random.default_rng(81), 45, 16), W.chain_tree(20)]
    wl = W.make_from_trees(trees, [700, 0], hq=12, hkv=4, d=64, dtype="f32", seed=splits, values="qwen")
    plan = B.tree_attn_verify_plan(wl.batch, wl.total_nodes, wl.max_nodes, wl.max_prefix, wl.hq, wl.hkv, wl.d,
                                   B.TV_F32, splits=splits)
    announce(f"attn fp32 slices {splits}: plan {plan}")
    span, S, kps = 700 + 45, plan["splits"], plan["keys_per_split"]
    # whole 64-key chunks per slice, no empty slice past the longest key axis
    assert plan["mfma"] == 0 and 1 < S <= min(splits, (span + 63) // 64) and kps % 64 == 0
    assert (S - 1) * kps < span <= S * kps
    dv = dev_workload(wl)
    anc, _, _, merr = B.tree_mask_build(dv["parent"], dv["cu"], dv["P"], wl.max_nodes, 64)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = B.tree_attn_verify(dv["q"], dv["k"], dv["v"], dv["cu"], dv["ks"], dv["P"], anc, wl.max_nodes,
                             wl.max_prefix, err=err, splits=splits)
    torch.cuda.synchronize()
    assert int(merr.item()) == 0 and int(err.item()) == 0
    ref = O.tree_attention(wl.q, wl.k, wl.v, wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len, wl.scale)
    ref_abs = O.tree_attention(wl.q, wl.k, np.abs(wl.v), wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len,
                               wl.scale)
    assert_attn_close(to_np(out), ref, ref_abs, "f32", stated=True, what=f"fp32 slices {splits}")
