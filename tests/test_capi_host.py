"""The C-ABI library on the host: it loads, exports every function the header
declares, and rejects bad arguments before enqueuing anything (these checks
never reach the HIP runtime, so they run without a GPU).  Pointers passed
here are never dereferenced: every call either fails a host check or has an
empty batch."""
import ctypes as C
import os

import pytest

from tree_attention_verification_bitmask_amd import binding as BND

OK, NULL, SHAPE, DTYPE, LIMIT, WS, LAUNCH, ALIGN = range(8)
FAKE = C.c_void_p(0x10000)      # aligned, never dereferenced
FAKE_ODD = C.c_void_p(0x10004)  # 4-byte aligned only


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(BND.LIB_PATH):
        from tree_attention_verification_bitmask_amd import build
        build.build()
    return BND.lib()


def test_exports_every_declared_symbol(L):
    names = BND.header_functions()
    assert set(names) >= {"tree_mask_build", "tree_attn_verify", "tree_accept_greedy",
                          "kv_compact_path", "tree_attn_verify_workspace_size",
                          "tv_status_string", "tv_abi_version"}
    for n in names:
        assert hasattr(L, n), n
    assert L.tv_abi_version() == 1
    assert L.tv_status_string(0) == b"TV_OK"
    assert b"NULL" in L.tv_status_string(NULL)


def mask(L, parent=FAKE, cu=FAKE, P=FAKE, B=1, T=16, max_nodes=16, max_depth=8, anc=FAKE,
         lev=FAKE, pos=FAKE):
    return L.tree_mask_build(parent, cu, P, B, T, max_nodes, max_depth, anc, lev, pos, None, None)


def test_mask_build_host_checks(L):
    assert mask(L, cu=None) == NULL
    assert mask(L, parent=None) == NULL
    assert mask(L, anc=None) == NULL
    assert mask(L, B=-1) == SHAPE
    assert mask(L, T=-1) == SHAPE
    assert mask(L, max_nodes=0) == SHAPE
    assert mask(L, max_depth=0) == SHAPE
    assert mask(L, max_nodes=1025) == LIMIT
    assert mask(L, max_depth=65) == LIMIT
    assert mask(L, T=1 << 24) == LIMIT
    assert mask(L, anc=FAKE_ODD) == ALIGN
    assert mask(L, B=0) == OK                    # empty batch: nothing to do
    assert mask(L, parent=None, anc=None, lev=None, pos=None, T=0) == OK


def attn(L, q=FAKE, k=FAKE, v=FAKE, cu=FAKE, ks=FAKE, P=FAKE, anc=FAKE, B=1, T=128, max_nodes=128,
         max_prefix=4096, rows=4224, hq=32, hkv=8, d=128, scale=0.088, dtype=1, out=FAKE, ws=FAKE,
         ws_bytes=1 << 40):
    return L.tree_attn_verify(q, k, v, cu, ks, P, anc, B, T, max_nodes, max_prefix, rows, hq, hkv, d,
                              scale, dtype, out, ws, ws_bytes, None, None)


def test_attn_host_checks(L):
    assert attn(L, q=None) == NULL
    assert attn(L, out=None) == NULL
    assert attn(L, anc=None) == NULL
    assert attn(L, k=None) == NULL
    assert attn(L, cu=None) == NULL
    assert attn(L, hq=30) == SHAPE               # hq % hkv != 0
    assert attn(L, hkv=0) == SHAPE
    assert attn(L, scale=0.0) == SHAPE
    assert attn(L, scale=float("nan")) == SHAPE
    assert attn(L, max_prefix=-1) == SHAPE
    assert attn(L, rows=-5) == SHAPE
    assert attn(L, d=96) == DTYPE
    assert attn(L, dtype=7) == DTYPE
    assert attn(L, max_nodes=2048) == LIMIT
    # MFMA grid or merge waves past int range (65535 requests x 1024 KV heads)
    assert attn(L, B=65535, T=65535 * 8, max_nodes=8, hq=4096, hkv=1024) == LIMIT
    assert attn(L, q=FAKE_ODD) == ALIGN
    assert attn(L, out=FAKE_ODD) == ALIGN
    need = L.tree_attn_verify_workspace_size(1, 128, 128, 4096, 32, 8, 128, 1)
    assert need > 0
    assert attn(L, ws=None, ws_bytes=0) == WS
    assert attn(L, ws_bytes=need - 1) == WS
    assert attn(L, ws=C.c_void_p(0x10010), ws_bytes=need) == ALIGN
    assert attn(L, B=0, T=0) == OK


def test_workspace_sizes(L):
    # fp32 takes the vector kernel, which needs no workspace; a bf16 tree of
    # 4 rows per KV head over a short prefix is one slice (no partials), over
    # a long one it is cut into slices like any other
    assert L.tree_attn_verify_workspace_size(1, 16, 16, 128, 2, 1, 64, 0) == 0
    assert L.tree_attn_verify_workspace_size(1, 4, 4, 128, 8, 8, 128, 1) == 0
    assert L.tree_attn_verify_workspace_size(1, 1, 1, 8192, 32, 8, 128, 1) > 0
    # bf16 Qwen3-shaped layers split the key axis: bf16 partials (256 B per
    # row and slice) and fp32 (m, l) per row and slice
    for B, T, n, P in ((1, 64, 64, 1024), (1, 128, 128, 4096), (1, 256, 256, 8192), (8, 1024, 128, 8192)):
        ws = L.tree_attn_verify_workspace_size(B, T, n, P, 32, 8, 128, 1)
        assert ws % 8 == 0 and ws >= 8 * 4 * n * 264
    # fp32 grids of few tiles over a long key axis are cut into key-axis
    # slices: (max, sum) and d outputs per (node, query head, slice), in whole
    # 64-key chunks; one node at 32/8 heads over 8192 keys takes 26 slices of
    # 320 keys (8 head tiles x 26 = 208 workgroups)
    for B, T, n, P, d, S in ((1, 1, 1, 8192, 128, 26), (1, 3, 3, 16384, 128, 29), (1, 6, 6, 5000, 64, 16)):
        rows = T * 32 * S
        assert L.tree_attn_verify_workspace_size(B, T, n, P, 32, 8, d, 0) == (rows * 8 + 255) // 256 * 256 + rows * d * 4
    info = (C.c_int32 * 8)()
    assert L.tree_attn_verify_plan(1, 1, 1, 8192, 32, 8, 128, 0, None, info) == OK
    assert list(info) == [0, 0, 0, 26, 320, 0, 0, 432640]
    # invalid sizes report 0
    assert L.tree_attn_verify_workspace_size(1, 16, 16, 128, 3, 2, 64, 1) == 0


def test_attn_plan_is_a_function_of_its_arguments(L, monkeypatch):
    """The plan (and so the workspace size) depends on the host sizes and the
    explicit override only: the process environment plays no part."""
    sizes = (1, 128, 128, 4096, 32, 8, 128, BND.TV_BF16)
    base = BND.tree_attn_verify_plan(*sizes)
    ws = L.tree_attn_verify_workspace_size(*sizes)
    assert base["mfma"] == 1 and base["workspace_bytes"] == ws
    for name in ("TV_MFMA_SPLITS", "TV_MFMA_PLAN"):
        monkeypatch.setenv(name, "3")
    assert BND.tree_attn_verify_plan(*sizes) == base
    assert L.tree_attn_verify_workspace_size(*sizes) == ws
    # the override changes the plan, and the _ex size follows it
    p3 = BND.tree_attn_verify_plan(*sizes, splits=3)
    assert p3["splits"] == 3 and p3["keys_per_split"] * 3 >= 4096 + 128
    assert BND.tree_attn_verify_workspace_size(*sizes, splits=3) == p3["workspace_bytes"] < ws
    # batches: balanced order by default, the others on request; fixed
    # splits keep the sliced orders
    bsz = (8, 634, 128, 7275, 32, 8, 128, BND.TV_BF16)
    bal = BND.tree_attn_verify_plan(*bsz)
    assert bal["planned"] == 2 and bal["splits"] == 0 and bal["keys_per_split"] == 0
    assert BND.tree_attn_verify_plan(*bsz, order=BND.TV_ORDER_BALANCED) == bal
    assert BND.tree_attn_verify_plan(*bsz, order=BND.TV_ORDER_PLANNED)["planned"] == 1
    assert BND.tree_attn_verify_plan(*bsz, order=BND.TV_ORDER_STATIC)["planned"] == 0
    assert BND.tree_attn_verify_plan(*bsz, splits=4)["planned"] == 1
    # beyond the balanced planner (more than 1024 requests, or more than 8
    # row tiles per request and KV head): the longest-first order
    assert BND.tree_attn_verify_plan(1025, 1025, 1, 64, 32, 1, 128, BND.TV_BF16)["planned"] != 2
    assert BND.tree_attn_verify_plan(2, 2048, 1024, 64, 32, 8, 128, BND.TV_BF16,
                                     order=BND.TV_ORDER_BALANCED)["planned"] == 1
    # one request: the balanced order does not apply
    assert BND.tree_attn_verify_plan(*sizes, order=BND.TV_ORDER_BALANCED) == base


def test_attn_override_checked(L):
    ov = BND.PlanOverride(0, 0)
    info = (C.c_int32 * 8)()
    args = (1, 128, 128, 4096, 32, 8, 128, 1)
    assert L.tree_attn_verify_plan(*args, C.byref(ov), info) == OK
    assert L.tree_attn_verify_plan(*args, C.byref(ov), None) == NULL
    assert L.tree_attn_verify_plan(*args, None, info) == OK
    bads = (BND.PlanOverride(-1, 0), BND.PlanOverride(0, 4), BND.PlanOverride(0, 0, 0, (C.c_int32 * 5)(1)),
            BND.PlanOverride(0, 0, 5), BND.PlanOverride(0, 0, 2))
    for bad in bads:
        assert L.tree_attn_verify_plan(*args, C.byref(bad), info) == SHAPE
        assert L.tree_attn_verify_workspace_size_ex(*args, None, C.byref(bad)) == 0
    # 32 rows per wave: 4 or 8 waves per workgroup
    d64 = (1, 128, 128, 4096, 16, 4, 64, 1)
    for a in (args, d64):
        assert BND.tree_attn_verify_plan(*a, waves=4)["rows_per_tile"] == 128
        assert BND.tree_attn_verify_plan(*a, waves=8)["rows_per_tile"] == 256
    # the plain call's checks are the _ex call's checks
    assert L.tree_attn_verify_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 128, 128, 4096, 4224, 30, 8, 128,
                                 0.088, 1, None, FAKE, FAKE, 1 << 40, None, None, None) == SHAPE
    assert L.tree_attn_verify_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0, 128, 4096, 4224, 32, 8, 128,
                                 0.088, 1, None, FAKE, FAKE, 1 << 40, None, C.byref(ov), None) == OK


def test_attn_inputs_checked(L):
    """tv_attn_inputs: RoPE and token-table options are checked on the host,
    and RoPE adds the nodes' (cos, sin) pairs to the workspace."""
    T, d = 128, 128
    sizes = (1, T, 128, 4096, 32, 8, d, 1)

    def ex(inp, ks=FAKE, B=1, T_=T, rows=4224, ws=1 << 40):
        return L.tree_attn_verify_ex(FAKE, FAKE, FAKE, FAKE, ks, FAKE, FAKE, B, T_, 128, 4096, rows, 32, 8, d, 0.088,
                                     1, C.byref(inp) if inp is not None else None, FAKE, FAKE, ws, None, None, None)

    FA = FAKE.value

    def inp(pos=FA, tab=None, stride=0, base=0.0, res=0):
        r = (C.c_int32 * 5)()
        r[2] = res
        return BND.AttnInputs(pos, tab, stride, base, r)
    assert ex(inp(res=1)) == SHAPE                       # reserved field set
    assert ex(inp(base=-1.0)) == SHAPE
    assert ex(inp(base=float("nan"))) == SHAPE
    assert ex(inp(base=float("inf"))) == SHAPE
    assert ex(inp(tab=FA, stride=0)) == SHAPE          # a table needs a stride
    assert ex(inp(pos=None, base=1e6)) == NULL           # RoPE needs positions
    assert ex(inp(tab=None), ks=None) == NULL            # contiguous rows need kv_start
    assert ex(inp(tab=FA + 2, stride=4224), ks=None) == ALIGN
    assert ex(inp(tab=FA, stride=4224), ks=None, rows=0) == SHAPE   # row 0 must exist
    assert ex(inp(pos=None, base=1e6), B=0, T_=0) == OK  # nothing to do: nothing read
    # workspace: the plan's, then T * d/2 (cos, sin) pairs at a 256-byte boundary
    base = L.tree_attn_verify_workspace_size(*sizes)
    rope = L.tree_attn_verify_workspace_size_ex(*sizes, C.byref(inp(base=1e6)), None)
    assert rope == ((base + 255) // 256 * 256) + T * (d // 2) * 8
    assert L.tree_attn_verify_workspace_size_ex(*sizes, C.byref(inp(tab=FA, stride=9000)), None) == base
    assert L.tree_attn_verify_workspace_size_ex(*sizes, C.byref(inp(res=1)), None) == 0
    assert ex(inp(base=1e6), ws=rope - 1) == WS
    # the vector path (fp32): its key-axis slice partials (c3's 256 tiles take 3
    # slices), then the pairs at a 256-byte boundary
    f32 = (1, T, 128, 4096, 32, 8, d, 0)
    base32 = L.tree_attn_verify_workspace_size(*f32)
    assert base32 == (T * 32 * 3 * 8 + 255) // 256 * 256 + T * 32 * 3 * d * 4
    assert L.tree_attn_verify_workspace_size_ex(*f32, C.byref(inp(base=1e6)), None) == \
        ((base32 + 255) // 256 * 256) + T * (d // 2) * 8


def test_attn_noalloc_host_checks(L):
    """The allocation-free call checks its arguments like tree_attn_verify and
    refuses plans larger than its static scratch before touching the GPU."""
    def call(B=1, T=128, max_nodes=128, max_prefix=4096, hq=32, hkv=8, d=128, q=FAKE, out=FAKE):
        return L.tree_attn_verify_noalloc(q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, B, T, max_nodes, max_prefix,
                                          max_prefix + max_nodes, hq, hkv, d, 0.088, 1, out, None, None)
    assert call(q=None) == NULL
    assert call(hq=30) == SHAPE
    assert call(d=96) == DTYPE
    assert call(out=FAKE_ODD) == ALIGN
    assert call(B=0, T=0) == OK
    # a batch whose split partials exceed the static buffer: 125 requests of
    # 32 nodes x 8 KV heads are 1000 one-tile tasks, which the planner cuts
    # into two key slices (2000 x 256 rows x 264 bytes of partials)
    big = (125, 125 * 32, 32, 4096, 32, 8, 128, 1)
    assert L.tree_attn_verify_workspace_size(*big) > BND.TV_NOALLOC_SCRATCH_BYTES
    assert call(*big[:7]) == 8            # TV_ERR_SCRATCH
    assert b"SCRATCH" in L.tv_status_string(8)
    # every configuration of the benchmark fits
    for B, T, n, P in ((1, 64, 64, 1024), (1, 128, 128, 4096), (1, 256, 256, 8192), (8, 1024, 128, 8192)):
        assert L.tree_attn_verify_workspace_size(B, T, n, P, 32, 8, 128, 1) <= BND.TV_NOALLOC_SCRATCH_BYTES


def accept(L, parent=FAKE, dr=FAKE, tg=FAKE, root=FAKE, cu=FAKE, B=1, T=16, D=16, alen=FAKE,
           aidx=FAKE, nxt=FAKE):
    return L.tree_accept_greedy(parent, dr, tg, root, cu, B, T, D, alen, aidx, nxt, None, None)


def test_accept_host_checks(L):
    assert accept(L, parent=None) == NULL
    assert accept(L, root=None) == NULL
    assert accept(L, aidx=None) == NULL
    assert accept(L, D=0) == SHAPE
    assert accept(L, D=65) == LIMIT
    assert accept(L, B=-2) == SHAPE
    assert accept(L, B=0) == OK


def compact(L, k=FAKE, v=FAKE, cu=FAKE, ks=FAKE, P=FAKE, alen=FAKE, aidx=FAKE, B=1, T=16, D=16,
            rows=1000, hkv=8, d=128, dtype=1, nl=FAKE):
    return L.kv_compact_path(k, v, cu, ks, P, alen, aidx, B, T, D, rows, hkv, d, dtype, nl, None, None)


def test_compact_host_checks(L):
    assert compact(L, k=None) == NULL
    assert compact(L, aidx=None) == NULL
    assert compact(L, nl=None) == NULL
    assert compact(L, d=80) == DTYPE
    assert compact(L, dtype=5) == DTYPE
    assert compact(L, D=0) == SHAPE
    assert compact(L, D=100) == LIMIT
    assert compact(L, k=FAKE_ODD) == ALIGN
    assert compact(L, B=0) == OK


def commit(L, parent=FAKE, dr=FAKE, tg=FAKE, root=FAKE, cu=FAKE, ks=FAKE, P=FAKE, B=1, T=16, D=16,
           rows=1000, hkv=8, d=128, dtype=1, k=FAKE, v=FAKE, alen=FAKE, aidx=FAKE, nxt=FAKE, nl=FAKE):
    return L.tree_accept_commit(parent, dr, tg, root, cu, ks, P, B, T, D, rows, hkv, d, dtype, k, v,
                                alen, aidx, nxt, nl, None, None)


def test_accept_commit_host_checks(L):
    assert commit(L, parent=None) == NULL
    assert commit(L, root=None) == NULL
    assert commit(L, ks=None) == NULL
    assert commit(L, k=None) == NULL
    assert commit(L, aidx=None) == NULL
    assert commit(L, nxt=None) == NULL
    assert commit(L, nl=None) == NULL
    assert commit(L, d=80) == DTYPE
    assert commit(L, dtype=5) == DTYPE
    assert commit(L, D=0) == SHAPE
    assert commit(L, hkv=0) == SHAPE
    assert commit(L, rows=-1) == SHAPE
    assert commit(L, D=65) == LIMIT
    assert commit(L, hkv=65536) == LIMIT
    assert commit(L, B=-2) == SHAPE
    assert commit(L, v=FAKE_ODD) == ALIGN
    assert commit(L, B=0) == OK
    assert commit(L, B=0, T=0, parent=None, dr=None, tg=None) == OK


def test_binding_refuses_cpu_tensors(L):
    import torch
    x = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        BND.tree_mask_build(x, x, x, 4, 4)


def test_binding_constants_match_header():
    """The binding's copies of the header's limits and codes are the header's."""
    import re
    text = open(os.path.join(os.path.dirname(__file__), "..", "include", "treeverify.h")).read()
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define (TV_\w+) (\d+)", text)}
    assert defs["TV_MAX_NODES"] == BND.TV_MAX_NODES
    assert defs["TV_MAX_DEPTH"] == BND.TV_MAX_DEPTH
    assert defs["TV_MAX_LEDGER"] == BND.TV_MAX_LEDGER
    assert defs["TV_MAX_VOCAB"] == BND.TV_MAX_VOCAB
    for name in ("BAD_PARENT", "TOO_DEEP", "BAD_REQUEST", "BAD_PATH", "BAD_LEDGER", "LIMIT"):
        assert defs["TV_DEVERR_" + name] == getattr(BND, "DEVERR_" + name)
    for name in ("TV_GDN_HEAD_DIM", "TV_GDN_MAX_NODES", "TV_GDN_MAX_TABLE"):
        assert defs[name] == getattr(BND, name)


def select(L, score=FAKE, parent=FAKE, token=FAKE, B=1, D=4, Ln=8, budget=16, beta=0.0, tp=FAKE,
           tt=FAKE, nr=FAKE):
    return L.tree_select_topb(score, parent, token, B, D, Ln, budget, beta, tp, tt, nr, None, None)


def test_select_host_checks(L):
    assert select(L, B=-1) == SHAPE
    assert select(L, D=0) == SHAPE
    assert select(L, Ln=0) == SHAPE
    assert select(L, budget=0) == SHAPE
    assert select(L, D=65) == LIMIT
    assert select(L, budget=1025) == LIMIT
    assert select(L, D=64, Ln=129) == LIMIT          # 8256 slots > TV_MAX_LEDGER
    assert select(L, beta=float("nan")) == SHAPE
    assert select(L, beta=float("inf")) == SHAPE
    assert select(L, tp=None) == NULL
    assert select(L, score=None) == NULL
    assert select(L, B=0, score=None, parent=None, token=None) == OK
    assert select(L, B=0, D=64, Ln=128, budget=1024) == OK   # largest sizes, empty batch


def test_argmax_host_checks(L):
    am = lambda logits=FAKE, rows=4, vocab=100, dt=1, tok=FAKE: L.tree_target_argmax(logits, rows, vocab, dt, tok, None)
    assert am(rows=-1) == SHAPE
    assert am(vocab=0) == SHAPE
    assert am(vocab=16777217) == LIMIT
    assert am(rows=16777216) == LIMIT
    assert am(dt=7) == DTYPE
    assert am(tok=None) == NULL
    assert am(logits=None) == NULL
    assert am(logits=FAKE_ODD) == ALIGN
    assert am(rows=0, logits=None, tok=None) == OK


def test_sample_host_checks(L):
    ws_need = L.tree_target_sample_workspace_size(4, 100)
    assert ws_need == 4 * 1 * 24                                   # 24 bytes per 2048-logit chunk
    assert L.tree_target_sample_workspace_size(3, 2049) == 3 * 2 * 24
    assert L.tree_target_sample_workspace_size(-1, 5) == 0

    def sm(logits=FAKE, rows=4, vocab=100, dt=1, T=1.0, u=FAKE, tok=FAKE, ws=FAKE, wsb=ws_need):
        return L.tree_target_sample(logits, rows, vocab, dt, T, u, tok, ws, wsb, None)
    assert sm(rows=-1) == SHAPE
    assert sm(vocab=0) == SHAPE
    assert sm(T=0.0) == SHAPE
    assert sm(T=-1.0) == SHAPE
    assert sm(T=float("inf")) == SHAPE
    assert sm(T=float("nan")) == SHAPE
    assert sm(vocab=16777217) == LIMIT
    assert sm(rows=16777216) == LIMIT
    assert sm(rows=262144, vocab=16777216, wsb=1 << 44) == LIMIT  # 2^31 chunk workgroups
    assert sm(dt=7) == DTYPE
    assert sm(tok=None) == NULL
    assert sm(u=None) == NULL
    assert sm(ws=None) == NULL
    assert sm(logits=None) == NULL
    assert sm(logits=FAKE_ODD) == ALIGN
    assert sm(u=FAKE_ODD) == ALIGN
    assert sm(wsb=ws_need - 1) == WS
    assert sm(rows=0, logits=None, u=None, tok=None, ws=None, wsb=0) == OK


def test_rope_and_rollback_host_checks(L):
    rope = lambda q=FAKE, k=FAKE, pos=FAKE, cu=FAKE, ks=FAKE, P=FAKE, B=1, T=16, rows=100, hq=8, hkv=2, d=128, \
        base=1e6, dt=1: L.tree_rope_apply(q, k, pos, cu, ks, P, B, T, rows, hq, hkv, d, base, dt, None, None)
    assert rope(hq=0) == SHAPE
    assert rope(rows=-1) == SHAPE
    assert rope(base=0.0) == SHAPE
    assert rope(base=float("nan")) == SHAPE
    assert rope(d=96) == DTYPE
    assert rope(dt=5) == DTYPE
    assert rope(pos=None) == NULL
    assert rope(q=FAKE_ODD) == ALIGN
    assert rope(B=0, T=0, q=None, k=None, pos=None) == OK
    rb = lambda tab=FAKE, stride=64, slots=FAKE, cu=FAKE, P=FAKE, al=FAKE, ai=FAKE, B=1, T=16, D=16, nl=FAKE, \
        fr=FAKE, nf=FAKE: L.kv_rollback_token_table(tab, stride, slots, cu, P, al, ai, B, T, D, nl, fr, nf, None, None)
    assert rb(D=0) == SHAPE
    assert rb(stride=0) == SHAPE
    assert rb(D=65) == LIMIT
    assert rb(tab=None) == NULL
    assert rb(fr=None) == NULL
    assert rb(B=0) == OK


def test_gdn_host_checks(L):
    conv = lambda x=FAKE, cs=FAKE, w=FAKE, par=FAKE, cu=FAKE, B=1, T=16, Cc=8192, K=4, y=FAKE: \
        L.tree_gdn_conv(x, cs, w, par, cu, B, T, Cc, K, y, None, None)
    assert conv(Cc=12) == SHAPE
    assert conv(Cc=0) == SHAPE
    assert conv(K=1) == SHAPE
    assert conv(K=5) == SHAPE
    assert conv(B=-1) == SHAPE
    assert conv(y=None) == NULL
    assert conv(w=FAKE_ODD) == ALIGN
    assert conv(T=0, x=None, cs=None, w=None, par=None, y=None) == OK
    ver = lambda q=FAKE, k=FAKE, v=FAKE, rs=8192, g=FAKE, be=FAKE, st=FAKE, par=FAKE, cu=FAKE, B=1, T=64, D=16, \
        hk=16, hv=32, d=128, scale=0.088, l2=1, out=FAKE: \
        L.tree_gdn_verify(q, k, v, rs, g, be, st, par, cu, B, T, D, hk, hv, d, scale, l2, out, None, None)
    assert ver(hv=24) == SHAPE                     # hv % hk != 0
    assert ver(hk=0) == SHAPE
    assert ver(D=0) == SHAPE
    assert ver(D=65) == LIMIT
    assert ver(d=64) == DTYPE
    assert ver(rs=8190) == ALIGN
    assert ver(q=FAKE_ODD) == ALIGN
    assert ver(st=FAKE_ODD) == ALIGN
    assert ver(scale=float("nan")) == SHAPE
    assert ver(l2=2) == SHAPE
    assert ver(out=None) == NULL
    assert ver(B=0, T=0, q=None, k=None, v=None, g=None, be=None, st=None, par=None, out=None) == OK
    com = lambda st=FAKE, cs=FAKE, x=FAKE, k=FAKE, v=FAKE, rs=8192, g=FAKE, be=FAKE, cu=FAKE, al=FAKE, ai=FAKE, \
        B=1, T=64, D=16, hk=16, hv=32, d=128, Cc=8192, K=4, l2=1: \
        L.tree_gdn_commit(st, cs, x, k, v, rs, g, be, cu, al, ai, B, T, D, hk, hv, d, Cc, K, l2, None, None)
    assert com(st=None) == NULL
    assert com(cs=None) == NULL
    assert com(K=5) == SHAPE
    assert com(hv=20) == SHAPE
    assert com(d=256) == DTYPE
    assert com(D=65) == LIMIT
    assert com(cs=FAKE_ODD) == ALIGN
    assert com(B=0) == OK


def test_accept_stochastic_host_checks(L):
    B, T, V = 2, 10, 1000
    def ws_size(B, T, V):
        # ten 256-byte-aligned segments over B + T rows and 2048-logit
        # chunks: chunk statistics (16 B), six slots of residual chunk sums
        # (8 B each), then per row (M, Z) 16 B, four pass records of 64 B, the
        # final residual 24 B, candidate range 8 B, decision 4 B, first
        # candidate 24 B; a 24-byte record per candidate node and a 4-byte
        # flag per request
        nch, rows = -(-V // 2048), B + T
        off = 0
        for size in (rows * nch * 16, 6 * rows * nch * 8, rows * 16, 4 * rows * 64, rows * 24, rows * 8, rows * 4,
                     rows * 24, T * 24, B * 4):
            off = -(-off // 256) * 256 + size
        return -(-off // 256) * 256
    need = L.tree_accept_stochastic_workspace_size(B, T, V)
    assert need == ws_size(B, T, V)
    assert L.tree_accept_stochastic_workspace_size(1, 2, 4097) == ws_size(1, 2, 4097) == 3328
    assert L.tree_accept_stochastic_workspace_size(1, 128, 151936) == ws_size(1, 128, 151936)
    assert L.tree_accept_stochastic_workspace_size(-1, T, V) == 0
    assert L.tree_accept_stochastic_workspace_size(B, T, 0) == 0

    def st(parent=FAKE, draft=FAKE, cu=FAKE, B=B, T=T, D=8, rl=FAKE, nl=FAKE, dt=0, temp=1.0, rq=FAKE, nq=FAKE,
           V=V, ua=FAKE, uf=FAKE, alen=FAKE, aidx=FAKE, nxt=FAKE, ws=FAKE, wsb=need):
        return L.tree_accept_stochastic(parent, draft, cu, B, T, D, rl, nl, dt, temp, rq, nq, V, ua, uf, alen, aidx,
                                        nxt, ws, wsb, None, None)
    assert st(B=-1) == SHAPE
    assert st(D=0) == SHAPE
    assert st(V=0) == SHAPE
    for bad_t in (0.0, -1.0, float("inf"), float("nan")):
        assert st(temp=bad_t) == SHAPE
    assert st(D=65) == LIMIT
    assert st(V=16777217) == LIMIT
    assert st(dt=4) == DTYPE
    assert st(rq=None) == NULL
    assert st(uf=None) == NULL
    assert st(nxt=None) == NULL
    assert st(nl=None) == NULL
    assert st(ua=None) == NULL
    assert st(ua=FAKE_ODD) == ALIGN                         # float64 uniforms
    assert st(rl=C.c_void_p(0x10002)) == ALIGN              # fp32 logits
    assert st(ws=None) == WS
    assert st(wsb=need - 1) == WS
    assert st(ws=C.c_void_p(0x10080)) == ALIGN
    assert st(B=0, T=0, ws=None, wsb=0) == OK
