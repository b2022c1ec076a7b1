"""Tree-aware Gated-DeltaNet verification on the GPU ([DT] section 4.5.4)
against the oracle, through the C ABI: the per-node conv window, the
per-node recurrent output, and the commit of the accepted path's state.

Tolerances (derived from the arithmetic; the oracle is float64):
  * conv output y is bf16, computed in float32 and rounded once to nearest:
    within half a bf16 ulp of the exact value, |err| <= 2^-8 |y| (1 + 2^-10)
    + 1e-7 (the float32 sum and SiLU add a few 2^-24).
  * verify output o is float32.  The dominant term is the committed state
    entering the bf16 matrix products as hi + lo: |S0 - hi - lo| <= 2^-18 |S0|
    per element, so S0 x errs by <= 2^-18 |S0_i|_2 |x|_2, about 4.4e-6 for
    unit x and the state scale used here (N(0, 0.1), 128 columns).  It enters
    o through e^G S0 q^ and through each r_s weighted by z (|e^G| <= 1, the
    weights summing to at most ~2 on these inputs): <= 1e-5.  Float32
    rounding adds ~1e-6.  The check is |err| <= 1e-5 (1 + |o|); the observed
    worst case is 7e-7, and a wrong ancestor moves o by 1e-2 .. 1 (the
    negative control checks that).
  * commit: the state stays float32, one step per accepted token with at most
    three roundings per updated entry, over <= 16 steps here: |err| <=
    3e-6 (1 + |S|) (observed 1e-7).  The conv state is moved bit-exactly.
"""
import numpy as np
import pytest

from oracle import tree_gdn_oracle as G
from tree_attention_verification_bitmask_amd import workloads as W
from tests.gpu_util import announce

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

O_REL = 1e-5
S_REL = 3e-6


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


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda().to(torch.bfloat16)


def f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def mixed(gi):
    """q | k | v of every node in one [T, 2*hk*128 + hv*128] bf16 buffer."""
    T = gi.q.shape[0]
    return np.concatenate([gi.q.reshape(T, -1), gi.k.reshape(T, -1), gi.v.reshape(T, -1)], axis=1)


def run_verify(gi, scale, l2norm=True, parent=None, max_depth=None):
    hk, hv = gi.q.shape[1], gi.v.shape[1]
    y = bf16(mixed(gi))
    q, k, v = B().gdn_split(y, hk, hv)
    par = gi.parent if parent is None else parent
    out, err = B().tree_gdn_verify(q, k, v, f32(gi.g), f32(gi.beta), f32(gi.state), i32(par), i32(gi.cu_nodes),
                                   gi.max_depth if max_depth is None else max_depth, scale, l2norm)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(err.item())


def check_o(got, ref, what=""):
    ratio = float((np.abs(got - ref) / (1.0 + np.abs(ref))).max()) if got.size else 0.0
    print(f"[err] {what}: max |err| / (1 + |o|) = {ratio:.3e}", flush=True)
    bad = np.abs(got - ref) > O_REL * (1.0 + np.abs(ref))
    assert not bad.any(), (what, int(bad.sum()), float(np.abs(got - ref).max()))


def trees(kind, rng):
    if kind == "c2":
        return [W.best_first_tree(rng, 64, 16)]
    if kind == "c3":
        return [W.best_first_tree(rng, 128, 16)]
    if kind == "c4":
        return [W.width_first_tree(rng, 16, 16)]
    if kind == "c5":
        return [W.best_first_tree(rng, int(rng.integers(32, 129)), 16) for _ in range(8)]
    if kind == "ragged":
        return [W.random_tree(rng, n, 8) for n in (1, 33, 0, 70, 5)]
    if kind == "chain64":
        return [W.chain_tree(64)]
    if kind == "star":
        return [np.full(40, -1, np.int32)]
    raise ValueError(kind)


# ---------------------------------------------------------------------------
# tree_gdn_conv
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,K,hk,hv", [("c2", 4, 16, 32), ("ragged", 4, 2, 4), ("ragged", 3, 1, 2),
                                          ("chain64", 2, 2, 2), ("star", 4, 1, 1), ("c5", 4, 2, 4)])
def test_conv_parity(kind, K, hk, hv):
    announce(f"gdn conv {kind} K={K} hk={hk} hv={hv}")
    rng = np.random.default_rng(sum(map(ord, kind)) + K)
    gi = W.gdn_inputs(rng, trees(kind, rng), hk=hk, hv=hv, conv_k=K)
    y, err = B().tree_gdn_conv(bf16(gi.x), bf16(gi.conv_state), bf16(gi.conv_w), i32(gi.parent), i32(gi.cu_nodes))
    torch.cuda.synchronize()
    got = y.float().cpu().numpy()
    ref = G.gdn_conv_tree(gi.x, gi.conv_state, gi.conv_w, gi.parent, gi.cu_nodes)
    print(f"[err] conv: max |err| / (2^-8 |y| + 1e-7) = "
          f"{float((np.abs(got - ref) / (2.0 ** -8 * np.abs(ref) + 1e-7)).max()):.3f}", flush=True)
    assert int(err.item()) == 0
    bad = np.abs(got - ref) > 2.0 ** -8 * (1 + 2.0 ** -10) * np.abs(ref) + 1e-7
    assert not bad.any(), (int(bad.sum()), float(np.abs(got - ref).max()))


def test_conv_bad_parent_reported():
    announce("gdn conv bad parent")
    rng = np.random.default_rng(3)
    gi = W.gdn_inputs(rng, [W.random_tree(rng, 10, 5)], hk=1, hv=1)
    par = gi.parent.copy()
    par[6] = 9                                  # points forward
    _, err = B().tree_gdn_conv(bf16(gi.x), bf16(gi.conv_state), bf16(gi.conv_w), i32(par), i32(gi.cu_nodes))
    torch.cuda.synchronize()
    assert int(err.item()) == (B().DEVERR_BAD_PARENT << 24) | 6


# ---------------------------------------------------------------------------
# tree_gdn_verify
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("kind,hk,hv,l2norm", [("c2", 16, 32, True), ("c3", 4, 8, True), ("c4", 2, 4, True),
                                               ("c5", 2, 4, True), ("ragged", 2, 6, True), ("ragged", 3, 3, False),
                                               ("chain64", 1, 2, True), ("star", 1, 4, True)])
def test_verify_parity(kind, hk, hv, l2norm):
    announce(f"gdn verify {kind} hk={hk} hv={hv} l2norm={l2norm}")
    rng = np.random.default_rng(len(kind) * 7 + hk * 3 + hv)
    gi = W.gdn_inputs(rng, trees(kind, rng), hk=hk, hv=hv)
    if not l2norm:
        # the rule assumes |k| <= 1 (else I - beta k k^T amplifies): unit rows
        gi.k = W.round_to_bf16(gi.k / np.linalg.norm(gi.k, axis=-1, keepdims=True))
        gi.q = W.round_to_bf16(gi.q / np.linalg.norm(gi.q, axis=-1, keepdims=True))
    scale = 128 ** -0.5
    got, err = run_verify(gi, scale, l2norm)
    assert err == 0
    ref = G.gdn_tree_verify(gi.q, gi.k, gi.v, gi.g, gi.beta, gi.state, gi.parent, gi.cu_nodes, scale, l2norm)
    check_o(got, ref, kind)


def correlated(rng, gi, spread=0.3):
    """Queries and keys near one common direction per head, so q^ . k^ is
    near 1 and every ancestor's write moves the output by O(0.1..1)."""
    T, hk, d = gi.q.shape
    base = rng.standard_normal((1, hk, d)).astype(np.float32)
    gi.q = W.round_to_bf16(base + spread * rng.standard_normal((T, hk, d)).astype(np.float32))
    gi.k = W.round_to_bf16(base + spread * rng.standard_normal((T, hk, d)).astype(np.float32))
    return gi


@pytest.mark.parametrize("kind", ["c3", "c4"])
def test_verify_sensitive_and_negative_control(kind):
    """Correlated q/k and scale 1: the tree output is matched, and the
    output of the same nodes under the flattened chain (what a chain
    recurrence would compute) is far outside the tolerance."""
    announce(f"gdn verify sensitive {kind}")
    rng = np.random.default_rng(11)
    gi = correlated(rng, W.gdn_inputs(rng, trees(kind, rng), hk=2, hv=4))
    got, err = run_verify(gi, 1.0)
    assert err == 0
    ref = G.gdn_tree_verify(gi.q, gi.k, gi.v, gi.g, gi.beta, gi.state, gi.parent, gi.cu_nodes, 1.0, True)
    check_o(got, ref, "tree")
    T = gi.q.shape[0]
    flat = G.gdn_tree_verify(gi.q, gi.k, gi.v, gi.g, gi.beta, gi.state, W.chain_tree(T), gi.cu_nodes, 1.0, True)

    def path(t):
        out = [t]
        while gi.parent[out[-1]] >= 0:
            out.append(int(gi.parent[out[-1]]))
        return sorted(out)

    branchy = [t for t in range(T) if path(t) != list(range(t + 1))]
    assert len(branchy) > T // 2
    gap = np.abs(got[branchy] - flat[branchy]).max()
    assert gap > 100 * O_REL * (1 + np.abs(flat[branchy]).max()), gap


def test_verify_full_layer_c3():
    """The full layer (16 q/k heads, 32 v heads) on the 128-node best-first tree."""
    announce("gdn verify full layer c3")
    rng = np.random.default_rng(5)
    gi = W.gdn_inputs(rng, trees("c3", rng))
    got, err = run_verify(gi, 128 ** -0.5)
    assert err == 0
    ref = G.gdn_tree_verify(gi.q, gi.k, gi.v, gi.g, gi.beta, gi.state, gi.parent, gi.cu_nodes, 128 ** -0.5, True)
    check_o(got, ref, "c3 full")


def test_verify_limits_and_errors():
    announce("gdn verify limits and errors")
    rng = np.random.default_rng(6)
    # 257 nodes in one request: LIMIT for that request only
    gi = W.gdn_inputs(rng, [W.random_tree(rng, 257, 8), W.random_tree(rng, 20, 8)], hk=1, hv=1)
    _, err = run_verify(gi, 0.1)
    assert err == (B().DEVERR_LIMIT << 24) | 0
    # 100 nodes with max_depth 64: 6400 table entries > 4096
    gi = W.gdn_inputs(rng, [W.random_tree(rng, 100, 8)], hk=1, hv=1)
    _, err = run_verify(gi, 0.1, max_depth=64)
    assert err == (B().DEVERR_LIMIT << 24) | 0
    # exactly at the limits: 256 nodes x 16 levels, 64-deep chain x 64
    for par, D in ((W.width_first_tree(rng, 16, 16), 16), (W.chain_tree(64), 64)):
        gi = W.gdn_inputs(rng, [par], hk=1, hv=2)
        got, err = run_verify(gi, 0.1, max_depth=D)
        assert err == 0
        check_o(got, G.gdn_tree_verify(gi.q, gi.k, gi.v, gi.g, gi.beta, gi.state, gi.parent, gi.cu_nodes,
                                       0.1, True), f"limit D={D}")
    # a node deeper than max_depth, and a bad parent
    gi = W.gdn_inputs(rng, [W.chain_tree(10)], hk=1, hv=1)
    _, err = run_verify(gi, 0.1, max_depth=6)
    assert err >> 24 == B().DEVERR_TOO_DEEP
    par = gi.parent.copy()
    par[4] = 7
    _, err = run_verify(gi, 0.1, parent=par)
    assert err == (B().DEVERR_BAD_PARENT << 24) | 4


# ---------------------------------------------------------------------------
# tree_gdn_commit, and the whole layer step
# ---------------------------------------------------------------------------

def accepted_paths(rng, parents, D):
    """A random root->node path per request (possibly empty)."""
    alen = np.zeros(len(parents), np.int32)
    aidx = np.zeros((len(parents), D), np.int32)
    for b, par in enumerate(parents):
        if len(par) == 0 or rng.random() < 0.15:
            continue
        t = int(rng.integers(0, len(par)))
        path = [t]
        while par[path[-1]] >= 0:
            path.append(int(par[path[-1]]))
        path = path[::-1]
        alen[b] = len(path)
        aidx[b, :len(path)] = path
    return alen, aidx


@pytest.mark.parametrize("kind,K", [("c5", 4), ("ragged", 3), ("chain64", 2), ("c2", 4)])
def test_commit_parity(kind, K):
    announce(f"gdn commit {kind} K={K}")
    rng = np.random.default_rng(len(kind) + K)
    pars = trees(kind, rng)
    gi = W.gdn_inputs(rng, pars, hk=2, hv=4, conv_k=K)
    D = max(gi.max_depth, 1)
    alen, aidx = accepted_paths(rng, pars, D)
    y = bf16(mixed(gi))
    _, k, v = B().gdn_split(y, 2, 4)
    x, cs = bf16(gi.x), bf16(gi.conv_state)
    st = f32(gi.state)
    err = B().tree_gdn_commit(st, cs, x, k, v, f32(gi.g), f32(gi.beta), i32(gi.cu_nodes), i32(alen), i32(aidx), D)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    S_ref, cs_ref = G.gdn_commit(gi.state, gi.conv_state, gi.x, gi.k, gi.v, gi.g, gi.beta, gi.cu_nodes,
                                 alen, aidx)
    S = st.cpu().numpy()
    print(f"[err] commit state: {float((np.abs(S - S_ref) / (1 + np.abs(S_ref))).max()):.3e}", flush=True)
    assert (np.abs(S - S_ref) <= S_REL * (1 + np.abs(S_ref))).all(), float(np.abs(S - S_ref).max())
    assert np.array_equal(cs.float().cpu().numpy(), cs_ref.astype(np.float32))
    for b in range(len(pars)):
        if alen[b] == 0:
            assert np.array_equal(S[b], gi.state[b])


def test_commit_bad_path_untouched():
    announce("gdn commit bad path")
    rng = np.random.default_rng(9)
    pars = [W.random_tree(rng, 12, 6), W.random_tree(rng, 9, 6)]
    gi = W.gdn_inputs(rng, pars, hk=1, hv=2)
    y = bf16(mixed(gi))
    _, k, v = B().gdn_split(y, 1, 2)
    x, cs = bf16(gi.x), bf16(gi.conv_state)
    cs0 = cs.clone()
    alen = np.array([2, 3], np.int32)
    aidx = np.zeros((2, 6), np.int32)
    aidx[0, :2] = [0, 12]                       # 12 is outside request 0
    aidx[1, :3] = [0, 1, 2]
    st = f32(gi.state)
    err = B().tree_gdn_commit(st, cs, x, k, v, f32(gi.g), f32(gi.beta), i32(gi.cu_nodes), i32(alen), i32(aidx), 6)
    torch.cuda.synchronize()
    assert int(err.item()) == (B().DEVERR_BAD_PATH << 24) | 0
    assert np.array_equal(st.cpu().numpy()[0], gi.state[0])
    assert torch.equal(cs[0], cs0[0]) and not torch.equal(cs[1], cs0[1])


def test_layer_step_pipeline():
    """conv -> verify -> greedy acceptance -> commit, all on the GPU; then one
    more token verified from the committed state equals that token placed
    under the accepted path's last node in the original tree."""
    announce("gdn layer step pipeline")
    rng = np.random.default_rng(21)
    hk, hv = 2, 4
    par = W.best_first_tree(rng, 48, 10)
    draft, target, root = W.draw_tokens(rng, par, 1000, force_path=True)
    cu = np.array([0, 48], np.int32)
    gi = W.gdn_inputs(rng, [par], hk=hk, hv=hv)
    D = gi.max_depth
    x = bf16(gi.x)
    y, err = B().tree_gdn_conv(x, bf16(gi.conv_state), bf16(gi.conv_w), i32(par), i32(cu))
    q, k, v = B().gdn_split(y, hk, hv)
    g_, b_ = f32(gi.g), f32(gi.beta)
    out, err = B().tree_gdn_verify(q, k, v, g_, b_, f32(gi.state), i32(par), i32(cu), D, 128 ** -0.5, True,
                                   err=err)
    alen, aidx, nxt, err = B().tree_accept_greedy(i32(par), i32(draft), i32(target), i32(np.array([root])), i32(cu),
                                                  D, err=err)
    torch.cuda.synchronize()
    L = int(alen[0].item())
    assert L >= 1 and int(err.item()) == 0
    last = int(aidx[0, L - 1].item())
    x_new = W.round_to_bf16(rng.standard_normal((1, gi.x.shape[1])).astype(np.float32))
    ext = np.concatenate([par, [last]]).astype(np.int32)
    ye = G.gdn_conv_tree(np.concatenate([gi.x, x_new]), gi.conv_state, gi.conv_w, ext, np.array([0, 49]))
    ge = np.concatenate([gi.g, -rng.uniform(0.01, 0.5, (1, hv)).astype(np.float32)])
    be = np.concatenate([gi.beta, rng.uniform(0.05, 0.95, (1, hv)).astype(np.float32)])
    # device: commit, then the new token alone from the committed state
    st, cs = f32(gi.state), bf16(gi.conv_state)
    err = B().tree_gdn_commit(st, cs, x, k, v, g_, b_, i32(cu), alen, aidx, D, err=err)
    y1, err = B().tree_gdn_conv(bf16(x_new), cs, bf16(gi.conv_w), i32(np.array([-1])), i32(np.array([0, 1])),
                                err=err)
    q1, k1, v1 = B().gdn_split(y1, hk, hv)
    o1, err = B().tree_gdn_verify(q1, k1, v1, f32(ge[48:]), f32(be[48:]), st, i32(np.array([-1])),
                                  i32(np.array([0, 1])), 1, 128 ** -0.5, True, err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # the conv output of the new token: its window is the same either way
    y1h = y1.float().cpu().numpy()
    assert (np.abs(y1h[0] - ye[48]) <= 2.0 ** -8 * (1 + 2.0 ** -10) * np.abs(ye[48]) + 1e-7).all()
    # the layer output: the oracle on the extended tree, fed the device's own
    # bf16 conv outputs (so only the state path is compared)
    yall = np.concatenate([y.float().cpu().numpy(), y1h])
    qe, ke, ve = (a.reshape(49, -1, 128) for a in np.split(yall, [hk * 128, 2 * hk * 128], axis=1))
    oe = G.gdn_tree_verify(qe, ke, ve, ge, be, gi.state, ext, np.array([0, 49]), 128 ** -0.5, True)
    check_o(o1.cpu().numpy()[0], oe[48], "continued token")
    check_o(out.cpu().numpy(), oe[:48], "tree nodes")
