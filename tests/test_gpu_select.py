"""tree_select_topb on the GPU against the selection oracle, through the C
ABI.  Every output is integer, so every comparison is exact: tree parents,
tokens, the real-node counts and the error word."""
import numpy as np
import pytest

from oracle import tree_select_oracle as S
from tree_attention_verification_bitmask_amd import workloads as W
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


def run_select(score, parent, token, budget, beta=0.0):
    dev = lambda x, dt: torch.from_numpy(np.ascontiguousarray(x, dtype=dt)).cuda()
    tp, tt, nr, err = B().tree_select_topb(dev(score, np.float32), dev(parent, np.int32),
                                           dev(token, np.int32), budget, beta)
    torch.cuda.synchronize()
    return tp.cpu().numpy(), tt.cpu().numpy(), nr.cpu().numpy(), int(err.item())


def check(score, parent, token, budget, beta=0.0, expect_err=None):
    got = run_select(score, parent, token, budget, beta)
    ref = S.select_topb(score, parent, token, budget, beta)
    assert np.array_equal(got[0], ref[0]), "tree_parent"
    assert np.array_equal(got[1], ref[1]), "tree_token"
    assert np.array_equal(got[2], ref[2]), "n_real"
    assert got[3] == ref[3], (hex(got[3]), hex(ref[3]))
    if expect_err is not None:
        assert (got[3] != 0) == expect_err
    return got


@pytest.mark.parametrize("batch", [1, 2, 5, 32])
def test_select_frontier_equals_heap(batch):
    """[DT] Appendix B at the page's batch sizes: the selected tree is the
    sequential best-first heap's, node for node (D 16, k 4, W = B = 64)."""
    announce(f"select frontier batch {batch}")
    D, k, Bn = 16, 4, 64
    L = Bn * k
    score = np.zeros((batch, D, L), np.float32)
    parent = np.zeros((batch, D, L), np.int32)
    token = np.zeros((batch, D, L), np.int32)
    heaps = []
    for b in range(batch):
        sc = S.PathScorer(seed=500 + b, k=k)
        score[b], parent[b], token[b] = S.frontier_ledger(sc, D, Bn)
        heaps.append(S.heap_tree(sc, D, Bn))
    tp, tt, nr, err = check(score, parent, token, Bn, expect_err=False)
    for b in range(batch):
        assert tp[b].tolist() == heaps[b][0].tolist() and tt[b].tolist() == heaps[b][1].tolist()


@pytest.mark.parametrize("beta", [-0.2, -1.0])
def test_select_depth_bonus(beta):
    announce(f"select depth bonus {beta}")
    sc = S.PathScorer(seed=77, k=4)
    score, parent, token = S.frontier_ledger(sc, 16, 128)
    tp, tt, _, _ = check(score[None], parent[None], token[None], 128, beta, expect_err=False)
    hp, ht = S.heap_tree(sc, 16, 128, beta)
    assert tp[0].tolist() == hp.tolist() and tt[0].tolist() == ht.tolist()


@pytest.mark.parametrize("shape", [(3, 16, 64, 4), (2, 8, 128, 8), (4, 64, 32, 4), (1, 1, 1, 1),
                                   (1, 64, 128, 1), (6, 5, 3, 2)])
def test_select_frontier_shaped(shape):
    batch, D, Wd, k = shape
    announce(f"select frontier-shaped {shape}")
    rng = np.random.default_rng(sum(shape))
    score, parent, token = W.frontier_shaped_ledger(rng, batch, D, Wd, k)
    for budget in sorted({1, min(Wd, 1024), min(Wd * k, 1024), 1024}):
        check(score, parent, token, budget, expect_err=False)


@pytest.mark.parametrize("tie_step,p_empty", [(0.0, 0.0), (0.25, 0.0), (0.25, 0.3), (0.0, 0.9)])
def test_select_random_ledgers(tie_step, p_empty):
    """Random monotone ledgers, with many exact ties (zero steps included)
    and empty slots: ties go by depth, then slot, and parents stay first."""
    announce(f"select random ties={tie_step} empty={p_empty}")
    rng = np.random.default_rng(int(tie_step * 100) + int(p_empty * 10))
    score, parent, token = W.random_ledger(rng, 8, 12, 16, 4, p_empty=p_empty, tie_step=tie_step)
    for budget in (1, 7, 64, 500, 1024):
        check(score, parent, token, budget, expect_err=False)


def test_select_all_equal_scores():
    """Every key equal: the order is the slot order, depth by depth."""
    announce("select all equal")
    D, L = 4, 8
    score = np.zeros((1, D, L), np.float32)
    score[0, 0, ::2] = -0.0           # -0 and +0 are one key
    parent = np.zeros((1, D, L), np.int32)
    parent[0, 0] = -1
    token = np.arange(D * L, dtype=np.int32).reshape(1, D, L)
    tp, tt, nr, err = check(score, parent, token, 20, expect_err=False)
    assert tt[0].tolist() == list(range(20))


def test_select_short_and_empty_ledgers():
    announce("select short and empty")
    score = np.full((3, 4, 8), -np.inf, np.float32)
    parent = np.full((3, 4, 8), -1, np.int32)
    token = np.ones((3, 4, 8), np.int32)
    score[1, 0, 3] = -1.0                  # one candidate
    score[2, 0, :] = np.nan                # NaN slots are empty too
    score[2, 0, 0] = np.inf
    tp, tt, nr, err = check(score, parent, token, 16, expect_err=False)
    assert nr.tolist() == [0, 1, 0] and (tp[0] == -1).all() and (tt[0] == -1).all()


def test_select_largest_ledger():
    """64 depths x 128 slots (8192, the limit), budget 1024."""
    announce("select largest ledger")
    rng = np.random.default_rng(4)
    score, parent, token = W.frontier_shaped_ledger(rng, 2, 64, 32, 4)
    assert score.shape[1] * score.shape[2] == B().TV_MAX_LEDGER
    check(score, parent, token, 1024, expect_err=False)
    s3, p3, t3 = W.random_ledger(rng, 2, 64, 32, 4, p_empty=0.1)
    check(s3, p3, t3, 1024, expect_err=False)


def test_select_bad_ledgers_reported():
    """A positive depth bonus ranks children above their parents, and a
    parent slot out of range: both reported, and the outputs equal the
    oracle's (those candidates become dead leaves)."""
    announce("select bad ledgers")
    sc = S.PathScorer(seed=3, k=4)
    score, parent, token = S.frontier_ledger(sc, 8, 16)
    check(score[None], parent[None], token[None], 16, 5.0, expect_err=True)
    s, p, t = W.random_ledger(np.random.default_rng(9), 3, 6, 8, 2)
    p[2, 3, :] = 999                        # request 2: slots pointing nowhere
    got = check(s, p, t, 64, expect_err=True)
    assert got[3] == (B().DEVERR_BAD_LEDGER << 24) | 2
