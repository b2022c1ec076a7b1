"""tree_target_sample on the GPU against the oracle, through the C ABI: the
sampled token of every row equals the oracle's inverse-transform sample for
the same uniforms, for fp32 and bf16 logits, at the Qwen3 vocabulary and at
ragged sizes, several temperatures, the edge uniforms and the special values.

Both sides decide in float64; only the order of the additions differs.  A row
whose threshold u * S lies within 1e-12 * S of a cumulative boundary could
therefore go either way: there the GPU's token only has to be valid (its
cumulative interval must hold the threshold to that tolerance), and the test
reports how many such rows it met (none, at these seeds)."""
import numpy as np
import pytest

from oracle import tree_verify_oracle as O
from tree_attention_verification_bitmask_amd import workloads as W
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REL_TIE = 1e-12


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


def _interval_ok(row, t, u, g):
    """g's cumulative interval [c[g-1], c[g]) holds u * S to REL_TIE * S."""
    y = np.asarray(row, np.float64) * (1.0 / t)
    c = np.cumsum(np.exp(y - y.max()))
    S = c[-1]
    thr = u * S
    lo = c[g - 1] if g > 0 else 0.0
    return c[g] > 0 and lo - REL_TIE * S <= thr < c[g] + REL_TIE * S


def _margin(row, t, u, g):
    """Distance of u * S from the nearest boundary of g's interval, over S."""
    y = np.asarray(row, np.float64) * (1.0 / t)
    c = np.cumsum(np.exp(y - y.max()))
    S = c[-1]
    lo = c[g - 1] if g > 0 else 0.0
    return min(abs(u * S - lo), abs(c[g] - u * S)) / S


def check(x32, dtype, t, u):
    """x32: float32 numpy logits (bf16-representable for 'bf16'); u float64."""
    x = torch.from_numpy(np.ascontiguousarray(x32)).cuda()
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
        assert np.array_equal(x.float().cpu().numpy(), x32, equal_nan=True)
    ut = torch.from_numpy(np.ascontiguousarray(u, np.float64)).cuda()
    got = B().tree_target_sample(x.contiguous(), float(np.float32(t)), ut).cpu().numpy()
    torch.cuda.synchronize()
    ref = O.target_sample(x32, float(np.float32(t)), u)
    bad = np.flatnonzero(got != ref)
    ties = 0
    for r in bad:
        finite = np.isfinite(x32[r]).all() and 0.0 <= u[r] < 1.0
        # a mismatch is allowed only on a boundary tie, and then must be valid
        assert finite and _margin(x32[r], np.float32(t), u[r], ref[r]) < REL_TIE, (r, got[r], ref[r])
        assert _interval_ok(x32[r], np.float32(t), u[r], got[r]), (r, got[r], ref[r])
        ties += 1
    return ties


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vocab", [(129, 151936), (65, 151936), (3, 151937), (5, 7), (1, 1),
                                        (2, 8193), (4, 2048), (3, 6144)])
@pytest.mark.parametrize("t", [0.7, 1.0])
def test_sample_random(dtype, rows, vocab, t):
    announce(f"sample {dtype} {rows}x{vocab} T={t}")
    rng = np.random.default_rng(rows * 7 + vocab)
    x = W.round_to_bf16(rng.normal(0, 3, (rows, vocab)).astype(np.float32))
    u = rng.random(rows)
    assert check(x, dtype, t, u) == 0


@pytest.mark.parametrize("t", [1e-3, 0.25, 4.0, 100.0])
def test_sample_temperatures(t):
    announce(f"sample temperatures T={t}")
    rng = np.random.default_rng(11)
    x = rng.normal(0, 2, (33, 151936)).astype(np.float32)
    u = rng.random(33)
    assert check(x, "f32", t, u) == 0


def test_sample_edge_uniforms():
    """u = 0 gives the first index with a positive weight; u just below 1 the
    last; u = 1 and u outside [0, 1) take the stated fallbacks."""
    announce("sample edge uniforms")
    rng = np.random.default_rng(5)
    V = 151936
    x = rng.normal(0, 1, (8, V)).astype(np.float32)
    x[:, :3] = -np.inf             # leading zero weights: u = 0 must skip them
    x[:, V - 5:] = -np.inf         # trailing zero weights: fallbacks must skip them
    u = np.array([0.0, np.nextafter(1.0, 0.0), 1.0, 1.5, -0.25, np.nan, 0.5, 1e-300])
    got_ref = O.target_sample(x, 1.0, u)
    assert got_ref[0] == 3 and got_ref[1] == V - 6 and got_ref[2] == V - 6
    assert check(x, "f32", 1.0, u) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sample_specials(dtype):
    announce(f"sample specials {dtype}")
    rng = np.random.default_rng(3)
    V = 151936
    x = W.round_to_bf16(rng.normal(0, 1, (10, V)).astype(np.float32))
    x[1, :] = -np.inf                                           # -> 0
    x[2, 100000] = np.nan                                       # NaN wins
    x[2, 5] = np.inf
    x[3, 77] = np.inf
    x[3, 78] = np.inf                                           # first +inf
    x[4, :] = -np.inf
    x[4, V - 1] = 2.0                                           # one finite logit, the last
    x[5, :] = 0.0                                               # uniform row
    x[6, 5] = np.nan
    x[6, 4] = np.nan                                            # first NaN
    x[7, ::2] = -np.inf                                         # half the vocabulary masked
    x[8, :] = 80.0                                              # large equal logits
    x[9, 1234] = 200.0                                          # one dominant logit
    u = rng.random(10)
    assert check(x, dtype, 1.0, u) == 0


def test_sample_distribution_on_a_grid():
    """Many rows of one small distribution, u on a uniform grid: every token
    equals the oracle's, so the frequencies are the softmax to one grid step."""
    announce("sample grid")
    rng = np.random.default_rng(0)
    x1 = rng.normal(0, 1.5, size=(1, 3000)).astype(np.float32)
    N = 4096
    u = (np.arange(N) + 0.5) / N
    x = np.repeat(x1, N, 0)
    assert check(x, "f32", 0.8, u) == 0


def test_sample_feeds_acceptance():
    """The c3 pipeline at T > 0: tokens sampled on the GPU feed the walk, which
    accepts the same path as the walk over the oracle's samples."""
    announce("sample feeds acceptance")
    wl = W.make_workload("c3", seed=0, force_path=True)
    V = 151936
    rng = np.random.default_rng(1)
    rows = wl.total_nodes + wl.batch
    x = rng.normal(0, 1, (rows, V)).astype(np.float32)
    want = np.concatenate([wl.target, wl.root_target]).astype(np.int64)
    x[np.arange(rows), want] = 14.0          # most of the mass on the forced tokens
    u = rng.random(rows)
    xt = torch.from_numpy(x).cuda()
    tok = B().tree_target_sample(xt, 1.0, torch.from_numpy(u).cuda()).cpu().numpy()
    ref = O.target_sample(x, 1.0, u)
    assert np.array_equal(tok, ref)
    T = wl.total_nodes
    dev = torch.device("cuda")
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)  # noqa: E731
    alen, aidx, nxt, _ = B().tree_accept_greedy(i32(wl.parent), i32(wl.draft), i32(tok[:T]), i32(tok[T:]),
                                                i32(wl.cu_nodes), wl.max_depth)
    ra = O.accept_greedy(wl.parent, wl.draft, ref[:T], ref[T:], wl.cu_nodes, wl.max_depth)
    assert np.array_equal(alen.cpu().numpy(), ra[0]) and np.array_equal(aidx.cpu().numpy(), ra[1])
    assert np.array_equal(nxt.cpu().numpy(), ra[2])


def test_sample_workspace_reuse():
    """Two calls in a row on one workspace, the second smaller: the second
    result does not depend on what the first left behind."""
    announce("sample workspace reuse")
    rng = np.random.default_rng(9)
    big = rng.normal(0, 2, (40, 151936)).astype(np.float32)
    small = rng.normal(0, 2, (7, 5000)).astype(np.float32)
    ws = torch.empty(B().tree_target_sample_workspace_size(40, 151936), dtype=torch.uint8, device="cuda")
    ub, us = rng.random(40), rng.random(7)
    g1 = B().tree_target_sample(torch.from_numpy(big).cuda(), 1.0, torch.from_numpy(ub).cuda(), workspace=ws)
    g2 = B().tree_target_sample(torch.from_numpy(small).cuda(), 1.0, torch.from_numpy(us).cuda(), workspace=ws)
    assert np.array_equal(g1.cpu().numpy(), O.target_sample(big, 1.0, ub))
    assert np.array_equal(g2.cpu().numpy(), O.target_sample(small, 1.0, us))
