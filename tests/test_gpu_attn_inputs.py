"""tree_attn_verify_ex's optional inputs on the GPU, through the C ABI.

Token table: the cache rows live scattered in a larger pool and the call reads
them through req_to_token.  The output must equal the contiguous call's bit for
bit (same plan, same arithmetic, only the addresses differ) and the oracle's
attention over the rows the table names, within the attention bound.  Table
entries past a request's P_b + N_b positions hold out-of-range values, so any
read of them would show up as a BAD_SLOT error.

RoPE inside the call: q and the tree's K rows arrive unrotated.  The oracle
rotates them (float64), the K rows are rounded to the cache's element type
(double -> float -> bf16, nearest-even, as the cache stores them), and the
oracle's attention over that must match the call's output within the attention
bound.  The cache's tree K rows afterwards must be bit for bit what
tree_rope_apply writes and within one ulp of the oracle's rotation; q and every
other cache row are untouched.
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


def B():
    from tree_attention_verification_bitmask_amd import binding
    return binding


def i32(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.int32)).cuda()


def mask(d, wl):
    anc, _, pos, err = B().tree_mask_build(d["parent"], d["cu"], d["P"], max(1, wl.max_nodes), 64)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return anc, pos


# Workloads beside the named configs: bf16 trees of fewer than 32 rows per KV
# head (the matrix-core kernel with one partly filled row block) and fp32
# over a long prefix (the vector kernel with the key axis cut into slices).
EXTRA = {
    "tiny_bf16": ([W.chain_tree(1), W.chain_tree(3), W.random_tree(np.random.default_rng(60), 5, 16)],
                  [2000, 7000, 33], 32, 8, 128, "bf16"),
    "fp32_long": ([W.random_tree(np.random.default_rng(61), 6, 16)], [5000], 8, 2, 128, "f32"),
}


def workload(name, seed):
    if name in EXTRA:
        parents, prefixes, hq, hkv, d, dtype = EXTRA[name]
        return W.make_from_trees(parents, prefixes, hq=hq, hkv=hkv, d=d, dtype=dtype, seed=seed, values="qwen")
    return W.make_workload(name, seed=seed)


def paged_pool(wl, d, seed):
    """Scatter the cache rows into a pool 1.5x larger (random distinct slots,
    random values elsewhere) and build req_to_token [B, stride]: position p of
    request b -> the slot of contiguous row kv_start[b] + p; positions past
    P_b + N_b hold out-of-range entries."""
    rows = d["k"].shape[0]
    pool = rows * 3 // 2 + 17
    rng = np.random.default_rng(seed)
    slot_of_row = rng.permutation(pool)[:rows].astype(np.int64)
    g = torch.Generator(device="cpu").manual_seed(seed)
    kp = torch.randn((pool,) + tuple(d["k"].shape[1:]), generator=g).to(d["k"].dtype).cuda()
    vp = torch.randn((pool,) + tuple(d["v"].shape[1:]), generator=g).to(d["v"].dtype).cuda()
    idx = torch.from_numpy(slot_of_row).cuda()
    kp[idx] = d["k"]
    vp[idx] = d["v"]
    sizes = np.diff(wl.cu_nodes).astype(np.int64)
    lens = wl.prefix_len.astype(np.int64) + sizes
    stride = int(lens.max()) + 5 if wl.batch else 1
    table = np.full((wl.batch, stride), -7, np.int64)
    table[:, -1] = pool + 3
    for b in range(wl.batch):
        ks = int(wl.kv_start[b])
        table[b, :lens[b]] = slot_of_row[ks:ks + lens[b]]
    return kp, vp, table.astype(np.int32), slot_of_row


PAGED_CASES = [("c1", 0, {}), ("c2", 1, {}), ("c3", 2, {}), ("c4", 0, {}), ("c5", 0, {}),
               ("c3", 3, dict(waves=8)), ("c2", 4, dict(waves=4, splits=1)),
               ("c5", 1, dict(order=1)), ("c5", 2, dict(splits=3)), ("tiny_bf16", 0, {}), ("fp32_long", 0, {})]


@pytest.mark.parametrize("name,seed,override", PAGED_CASES)
def test_paged_equals_contiguous(name, seed, override):
    announce(f"paged {name} seed {seed} {override}")
    wl = workload(name, seed)
    d = dev_workload(wl)
    anc, _ = mask(d, wl)
    kp, vp, table, _ = paged_pool(wl, d, seed + 100)
    tab = i32(table)
    e1 = torch.zeros(1, dtype=torch.int32, device="cuda")
    e2 = torch.zeros(1, dtype=torch.int32, device="cuda")
    ref = B().tree_attn_verify(d["q"], d["k"], d["v"], d["cu"], d["ks"], d["P"], anc, wl.max_nodes, wl.max_prefix,
                               err=e1, **override)
    got = B().tree_attn_verify(d["q"], kp, vp, d["cu"], None, d["P"], anc, wl.max_nodes, wl.max_prefix, err=e2,
                               req_to_token=tab, **override)
    torch.cuda.synchronize()
    assert int(e1.item()) == 0 and int(e2.item()) == 0, (int(e1.item()), int(e2.item()))
    if got.dtype == torch.bfloat16:
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    else:
        assert torch.equal(got.view(torch.int32), ref.view(torch.int32))


@pytest.mark.parametrize("name,seed", [("c1", 5), ("c2", 5), ("c5", 5)])
def test_paged_matches_oracle(name, seed):
    """The oracle's attention over the rows the table names (gathered from
    the pool on the host)."""
    announce(f"paged vs oracle {name} seed {seed}")
    wl = workload(name, seed)
    d = dev_workload(wl)
    anc, _ = mask(d, wl)
    kp, vp, table, _ = paged_pool(wl, d, seed)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = B().tree_attn_verify(d["q"], kp, vp, d["cu"], None, d["P"], anc, wl.max_nodes, wl.max_prefix, err=err,
                               req_to_token=i32(table))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # contiguous view of what the table names: request b's position p at
    # row kv_start[b] + p
    kpool, vpool = to_np(kp), to_np(vp)
    kc = np.zeros_like(wl.k)
    vc = np.zeros_like(wl.v)
    for b in range(wl.batch):
        n = int(wl.prefix_len[b] + wl.cu_nodes[b + 1] - wl.cu_nodes[b])
        ks = int(wl.kv_start[b])
        kc[ks:ks + n] = kpool[table[b, :n]]
        vc[ks:ks + n] = vpool[table[b, :n]]
    rows = sample_rows(wl, 160, seed) if name == "c5" else None
    ref = O.tree_attention(wl.q, kc, vc, wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len, wl.scale, rows=rows)
    ref_abs = O.tree_attention(wl.q, kc, np.abs(vc), wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len,
                               wl.scale, rows=rows)
    o = to_np(out)
    if rows is not None:
        o = np.stack([o[t, h] for t, h in rows])
    assert_attn_close(o, ref, ref_abs, wl.dtype, what=f"paged {name}")


def test_paged_bad_slot_and_short_table():
    """An entry outside the pool -> BAD_SLOT for its request (row 0 read in
    its place, no fault); a table row shorter than P_b + N_b -> BAD_REQUEST."""
    announce("paged errors")
    for name in ("c5", "c1"):
        wl = W.make_workload(name, seed=6)
        d = dev_workload(wl)
        anc, _ = mask(d, wl)
        kp, vp, table, _ = paged_pool(wl, d, 7)
        bad = table.copy()
        b = wl.batch - 1
        bad[b, int(wl.prefix_len[b]) // 2] = kp.shape[0] + 11
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        B().tree_attn_verify(d["q"], kp, vp, d["cu"], None, d["P"], anc, wl.max_nodes, wl.max_prefix, err=err,
                             req_to_token=i32(bad))
        torch.cuda.synchronize()
        assert int(err.item()) == (B().DEVERR_BAD_SLOT << 24) | b, (name, hex(int(err.item())))
        # the stride cuts off request 0's last tree position
        n0 = int(wl.prefix_len[0] + wl.cu_nodes[1] - wl.cu_nodes[0])
        short = np.ascontiguousarray(table[:, :n0 - 1])
        err.zero_()
        B().tree_attn_verify(d["q"], kp, vp, d["cu"], None, d["P"], anc, wl.max_nodes, wl.max_prefix, err=err,
                             req_to_token=i32(short))
        torch.cuda.synchronize()
        code = int(err.item())
        assert code >> 24 == B().DEVERR_BAD_REQUEST, (name, hex(code))


def round_like_cache(x, dtype):
    """double -> float -> element type, nearest-even (how the cache stores a
    rotated element)."""
    f = np.asarray(x, np.float64).astype(np.float32)
    if dtype == "f32":
        return f
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


ROPE_CASES = [("c1", 0, 1e4, False), ("c2", 0, 1e6, False), ("c3", 1, 1e6, False), ("c5", 0, 1e6, False),
              ("c2", 2, 1e6, True), ("c5", 3, 1e6, True), ("c1", 4, 1e4, True), ("tiny_bf16", 1, 1e6, False),
              ("tiny_bf16", 2, 1e6, True), ("fp32_long", 3, 1e4, True)]


@pytest.mark.parametrize("name,seed,base,paged", ROPE_CASES)
def test_rope_inside_attention(name, seed, base, paged):
    announce(f"rope inside attention {name} seed {seed} base {base} paged={paged}")
    wl = workload(name, seed)
    d = dev_workload(wl)
    anc, pos = mask(d, wl)
    q0 = d["q"].clone()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    if paged:
        kp, vp, table, slot_of_row = paged_pool(wl, d, seed + 50)
        k_in, v_in, ks_in, tab = kp, vp, None, i32(table)
    else:
        k_in, v_in, ks_in, tab = d["k"], d["v"], d["ks"], None
    k_before = k_in.clone()
    out = B().tree_attn_verify(d["q"], k_in, v_in, d["cu"], ks_in, d["P"], anc, wl.max_nodes, wl.max_prefix,
                               err=err, pos_ids=pos, rope_base=base, req_to_token=tab)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(d["q"], q0)                       # q is not written
    # the cache's tree rows: bit for bit tree_rope_apply's, the rest untouched
    kc = k_before.clone()
    if paged:
        # tree_rope_apply rotates contiguous rows: run it on the contiguous
        # cache and compare the tree rows through the slot map
        kr = d["k"].clone()
        qr = d["q"].clone()
        e = B().tree_rope_apply(qr, kr, pos, d["cu"], d["ks"], d["P"], base)
        torch.cuda.synchronize()
        assert int(e.item()) == 0
        kc[torch.from_numpy(slot_of_row).cuda()] = kr
    else:
        qr = d["q"].clone()
        e = B().tree_rope_apply(qr, kc, pos, d["cu"], d["ks"], d["P"], base)
        torch.cuda.synchronize()
        assert int(e.item()) == 0
    assert torch.equal(k_in.view(torch.int16 if k_in.dtype == torch.bfloat16 else torch.int32),
                       kc.view(torch.int16 if kc.dtype == torch.bfloat16 else torch.int32))
    # the oracle: rotate (float64), store K rows as the cache does, attend
    anc_o, lev_o, pos_o, err_o = O.mask_build(wl.parent, wl.cu_nodes, wl.prefix_len, max(1, wl.max_nodes), 64)
    assert err_o == 0 and np.array_equal(pos_o, pos.cpu().numpy())
    q2, k2 = O.tree_rope(wl.q, wl.k, pos_o, wl.cu_nodes, wl.kv_start, wl.prefix_len, base)
    k2 = round_like_cache(k2, wl.dtype)
    rows = sample_rows(wl, 160, seed) if name == "c5" else None
    ref = O.tree_attention(q2, k2, wl.v, wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len, wl.scale, rows=rows)
    ref_abs = O.tree_attention(q2, k2, np.abs(wl.v), wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len,
                               wl.scale, rows=rows)
    o = to_np(out)
    if rows is not None:
        o = np.stack([o[t, h] for t, h in rows])
    assert_attn_close(o, ref, ref_abs, wl.dtype, what=f"rope {name}")
    # and the rotated rows within one ulp of the oracle's rotation
    if not paged:
        got = to_np(k_in).astype(np.float64)
        rel = 2.0 ** -8 if wl.dtype == "bf16" else 2.0 ** -24
        _, k2x = O.tree_rope(wl.q, wl.k, pos_o, wl.cu_nodes, wl.kv_start, wl.prefix_len, base)
        assert np.all(np.abs(got - k2x) <= rel * np.abs(k2x) * 1.0001 + 1e-12)
