"""Pins of the oracle's sampled target choice (temperature T > 0, deterministic
draft; [DT] section 4.1, [TSD] "Verification and Acceptance Algorithms",
stochastic verification): the inverse transform against the exact
distribution, its limits, and losslessness of the tree walk it feeds."""
import numpy as np
import pytest

from oracle import tree_verify_oracle as O
from tree_attention_verification_bitmask_amd import workloads as W


def softmax(x, t):
    y = np.asarray(x, np.float64) / t
    e = np.exp(y - y.max())
    return e / e.sum()


@pytest.mark.parametrize("t", [0.5, 1.0, 2.0])
def test_inverse_transform_reproduces_the_distribution(t):
    """u on a fine uniform grid: the frequency of each token is its softmax
    probability to within one grid step (the inverse-CDF property)."""
    rng = np.random.default_rng(0)
    x = rng.normal(0, 1.5, size=(1, 50)).astype(np.float32)
    N = 20000
    u = (np.arange(N) + 0.5) / N
    toks = O.target_sample(np.repeat(x, N, 0), t, u)
    freq = np.bincount(toks, minlength=50) / N
    assert np.abs(freq - softmax(x[0], t)).max() <= 1.0 / N + 1e-12
    # tokens are non-decreasing in u (the transform is monotone)
    assert (np.diff(toks) >= 0).all()


def test_chi_square_with_random_uniforms():
    rng = np.random.default_rng(1)
    x = rng.normal(0, 1.0, size=(1, 20)).astype(np.float32)
    N = 40000
    toks = O.target_sample(np.repeat(x, N, 0), 0.8, rng.random(N))
    obs = np.bincount(toks, minlength=20)
    exp = softmax(x[0], 0.8) * N
    chi2 = ((obs - exp) ** 2 / exp).sum()
    assert chi2 < 45.3       # chi-square(19) 99.9th percentile 43.8, plus slack


def test_limits_and_edges():
    x = np.array([[1.0, 3.0, 3.0, 2.0, -np.inf]], np.float32)
    # low temperature: the argmax (ties: the lowest index takes all the mass of u < 1/2)
    assert O.target_sample(x, 1e-3, [0.3])[0] == 1 and O.target_sample(x, 1e-3, [0.7])[0] == 2
    # u = 0: the first index with positive weight; u just below 1: the last
    assert O.target_sample(x, 1.0, [0.0])[0] == 0
    assert O.target_sample(x, 1.0, [np.nextafter(1.0, 0.0)])[0] == 3
    # -inf never drawn; NaN / +inf / all -inf readings
    assert O.target_sample(np.array([[0.0, np.nan, np.nan]], np.float32), 1.0, [0.5])[0] == 1
    assert O.target_sample(np.array([[0.0, 1.0, np.inf, np.inf]], np.float32), 1.0, [0.1])[0] == 2
    assert O.target_sample(np.full((1, 4), -np.inf, np.float32), 1.0, [0.5])[0] == 0
    # a single token is always drawn
    assert O.target_sample(np.array([[7.0]], np.float32), 0.5, [0.99])[0] == 0


def test_sampled_walk_is_lossless_at_the_root():
    """The first token a round emits -- the accepted root child, else the
    target's sample itself -- is distributed as the target's softmax at the
    root: sampling the root row with every u on a grid and walking the tree
    gives each token its probability (to one grid step)."""
    rng = np.random.default_rng(2)
    V = 12
    parent = np.array([-1, -1, -1, 0, 0, 1], np.int32)      # root children 0, 1, 2
    draft = np.array([3, 7, 9, 1, 2, 5], np.int32)
    x = rng.normal(0, 1.0, size=(1, V)).astype(np.float32)
    N = 12000
    first = np.zeros(V, np.int64)
    for k in range(N):
        u = (k + 0.5) / N
        root_tok = O.target_sample(x, 0.7, [u])[0]
        tgt = np.full(6, 11, np.int32)                        # deeper nodes never match
        alen, aidx, nxt = O.accept_greedy(parent, draft, tgt, np.array([root_tok]), np.array([0, 6]), 4)
        tok = draft[aidx[0, 0]] if alen[0] > 0 else nxt[0]
        first[tok] += 1
    assert np.abs(first / N - softmax(x[0], 0.7)).max() <= 1.0 / N + 1e-12


def test_bf16_rows_and_large_vocab():
    """bf16-representable logits over the Qwen3 vocabulary: the drawn token's
    cumulative-weight interval holds u * Z, and over many rows the drawn
    tokens' mean log-probability matches the softmax entropy's sign of scale
    (the draws concentrate where the mass is)."""
    rng = np.random.default_rng(3)
    x = W.round_to_bf16(rng.normal(0, 3, size=(4, 151936)).astype(np.float32))
    u = rng.random(4)
    toks = O.target_sample(x, 0.9, u)
    for r in range(4):
        y = x[r].astype(np.float64) / 0.9
        w = np.exp(y - y.max())
        c = np.cumsum(w)
        t = int(toks[r])
        before = c[t - 1] if t > 0 else 0.0
        assert before <= u[r] * c[-1] < c[t]
        # the drawn token carries well above the median probability
        assert w[t] > np.median(w)
