"""tree_attn_verify_noalloc against tree_attn_verify, through the C ABI: the
allocation-free call (static per-GPU scratch instead of a workspace) must
give the plain call's output bit for bit, on two calls in a row, the second
with a smaller input (the scratch keeps the first call's contents)."""
import numpy as np
import pytest

from tree_attention_verification_bitmask_amd import workloads as W
from tests.gpu_util import announce, dev_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tree_attention_verification_bitmask_amd import binding
    binding.lib()   # raises if the HIP library is missing: no fallback
    return binding


def _both(wl):
    from tree_attention_verification_bitmask_amd import binding as B
    d = dev_workload(wl)
    anc, _, _, e = B.tree_mask_build(d["parent"], d["cu"], d["P"], wl.max_nodes, 64)
    assert int(e.item()) == 0
    err1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref = B.tree_attn_verify(d["q"], d["k"], d["v"], d["cu"], d["ks"], d["P"], anc, wl.max_nodes, wl.max_prefix,
                             err=err1)
    err2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = B.tree_attn_verify_noalloc(d["q"], d["k"], d["v"], d["cu"], d["ks"], d["P"], anc, wl.max_nodes,
                                     wl.max_prefix, err=err2)
    torch.cuda.synchronize()
    assert int(err1.item()) == 0 and int(err2.item()) == 0
    return got, ref


@pytest.mark.parametrize("first,second", [("c5", "c3"), ("c4", "c2")])
def test_noalloc_matches_workspace_call(first, second):
    """Two calls in a row on one GPU, the second smaller; each bit-identical to
    the call that brings its own workspace."""
    for name in (first, second):
        announce(f"noalloc {name} (after {first})")
        wl = W.make_workload(name, seed=4)
        got, ref = _both(wl)
        assert np.array_equal(got.view(torch.int16).cpu().numpy(), ref.view(torch.int16).cpu().numpy()), name


def test_noalloc_fp32_and_single_slice():
    """Plans that need no scratch (an unsliced vector-kernel call) go through too."""
    announce("noalloc c1 fp32")
    wl = W.make_workload("c1", seed=2)
    got, ref = _both(wl)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))


def test_noalloc_fp32_slices():
    """fp32 calls whose key axis the vector kernel cuts into slices keep their
    partials in the scratch: two such calls in a row, the second smaller,
    each bit-identical to the call with its own workspace."""
    from tree_attention_verification_bitmask_amd import binding as B
    cases = [([W.random_tree(np.random.default_rng(90), 7, 16)], [8192]),
             ([W.chain_tree(3)], [3000])]
    for i, (trees, prefixes) in enumerate(cases):
        wl = W.make_from_trees(trees, prefixes, hq=32, hkv=8, d=128, dtype="f32", seed=i, values="qwen")
        plan = B.tree_attn_verify_plan(wl.batch, wl.total_nodes, wl.max_nodes, wl.max_prefix, wl.hq, wl.hkv,
                                       wl.d, B.TV_F32)
        announce(f"noalloc fp32 slices case {i}: plan {plan}")
        assert plan["splits"] > 1 and plan["workspace_bytes"] > 0
        got, ref = _both(wl)
        assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32)), i
