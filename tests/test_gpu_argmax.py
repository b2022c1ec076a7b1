"""tree_target_argmax on the GPU against the oracle, through the C ABI:
bit-exact indices for fp32 and bf16 logits, at the Qwen3 vocabulary and at
ragged sizes, with ties, infinities, NaN and signed zeros."""
import numpy as np
import pytest

from oracle import tree_verify_oracle as O
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


def check(x32, dtype):
    """x32: float32 numpy logits; dtype 'f32' or 'bf16' (x32 must then hold
    bf16-representable values)."""
    t = torch.from_numpy(np.ascontiguousarray(x32)).cuda()
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
        assert np.array_equal(t.float().cpu().numpy(), x32, equal_nan=True)
    got = B().tree_target_argmax(t.contiguous())
    torch.cuda.synchronize()
    ref = O.target_argmax(x32)
    assert np.array_equal(got.cpu().numpy(), ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vocab", [(129, 151936), (65, 151936), (3, 151937), (5, 7), (1, 1), (2, 8193)])
def test_argmax_random(dtype, rows, vocab):
    announce(f"argmax {dtype} {rows}x{vocab}")
    rng = np.random.default_rng(rows + vocab)
    x = W.round_to_bf16(rng.normal(0, 3, (rows, vocab)).astype(np.float32))
    check(x, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_argmax_ties_and_specials(dtype):
    announce(f"argmax specials {dtype}")
    rng = np.random.default_rng(3)
    V = 151936
    x = rng.integers(-4, 4, (12, V)).astype(np.float32)        # ties everywhere
    x[1, :] = -np.inf                                           # -> 0
    x[2, 100000] = np.nan                                       # NaN wins
    x[3, 77] = np.inf
    x[3, 78] = np.inf                                           # first +inf
    x[4, :] = 0.0
    x[4, :50] = -0.0                                            # -0 ties +0 -> 0
    x[5, V - 1] = 9.0                                           # last element
    x[6, 5] = np.nan
    x[6, 4] = np.nan                                            # first NaN
    x[7, :] = 1.0                                               # all equal -> 0
    check(x, dtype)


def test_argmax_feeds_acceptance():
    """The c3 pipeline's target tokens from logits: argmax over one-hot-ish
    logits reproduces the chosen tokens, and the walk accepts the same path
    as with the tokens given directly."""
    announce("argmax feeds acceptance")
    wl = W.make_workload("c3", seed=0, force_path=True)
    V = 151936
    rng = np.random.default_rng(0)
    rows = wl.total_nodes + wl.batch
    x = rng.normal(0, 1, (rows, V)).astype(np.float32)
    want = np.concatenate([wl.target, wl.root_target]).astype(np.int64)
    x[np.arange(rows), want] = 50.0
    t = torch.from_numpy(x).cuda()
    tok = B().tree_target_argmax(t).cpu().numpy()
    assert np.array_equal(tok, want)
