"""Negative controls for the attention check used by the GPU parity tests:
outputs with a plausible mistake, computed on the CPU from the oracle's own
per-row routine with a wrong key set or head, must fail the check, while
the oracle's own output passes it.  Nothing here touches a GPU."""
import numpy as np
import pytest

from oracle import tree_verify_oracle as O
from tree_attention_verification_bitmask_amd import workloads as W
from tests.gpu_util import attn_errors, sample_rows


def _rows_fn(kind, wl, R, b=0):
    P = int(wl.prefix_len[b])
    n = int(wl.cu_nodes[b + 1] - wl.cu_nodes[b])
    base = int(wl.kv_start[b])

    def keys(i):
        if kind == "prefix_only":
            tree = []
        elif kind == "transposed":          # descendants-or-self instead of ancestors
            tree = [j for j in range(n) if R[j, i]]
        elif kind == "flattened":           # every earlier node, as a chain would see them
            tree = list(range(i + 1))
        else:
            tree = [j for j in range(n) if R[i, j]]
        return [base + t for t in range(P)] + [base + P + j for j in tree]
    return keys


def _closure(parent):
    n = len(parent)
    R = np.eye(n, dtype=bool)
    for i in range(n):
        p = int(parent[i])
        if p >= 0:
            R[i] |= R[p]
    return R


def _mutant(kind, wl, rows):
    par = wl.parent[wl.nodes_of(0)]
    R = _closure(par)
    keys = _rows_fn(kind, wl, R)
    G = wl.hq // wl.hkv
    out = []
    for t, h in rows:
        g = (h % wl.hkv) if kind == "wrong_gqa" else h // G
        idx = keys(t)
        out.append(O.attention_row(wl.q[t, h], wl.k[idx, g], wl.v[idx, g], wl.scale))
    return np.array(out)


@pytest.mark.parametrize("P", [0, 64])
def test_negative_controls_fail_on_sensitive_suite(P):
    wl = W.make_workload("c2", seed=7, values="sensitive", prefix=(P, P))
    rows = sample_rows(wl, 200, 0)
    ref = O.tree_attention(wl.q, wl.k, wl.v, wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len, wl.scale, rows=rows)
    ref_abs = O.tree_attention(wl.q, wl.k, np.abs(wl.v), wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len,
                               wl.scale, rows=rows)
    # the oracle itself, rounded to bf16 as the kernel's output is, passes
    _, ok_ratio = attn_errors(W.round_to_bf16(ref.astype(np.float32)), ref, ref_abs, "bf16")
    assert ok_ratio <= 0.5
    kinds = ["zero", "transposed", "flattened", "wrong_gqa"] + (["prefix_only"] if P else [])
    for kind in kinds:
        bad = np.zeros_like(ref) if kind == "zero" else _mutant(kind, wl, rows)
        _, ratio = attn_errors(bad, ref, ref_abs, "bf16")
        assert ratio > 1.0, f"{kind} passed the check (ratio {ratio:.3f})"


def test_zero_output_fails_on_qwen_values():
    """With the Qwen-shaped value distribution (outputs ~1e-3) an all-zero
    output passes the stated 1e-2 alone, but not the per-element bound."""
    wl = W.make_workload("c3", seed=0)
    rows = sample_rows(wl, 64, 0)
    ref = O.tree_attention(wl.q, wl.k, wl.v, wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len, wl.scale, rows=rows)
    ref_abs = O.tree_attention(wl.q, wl.k, np.abs(wl.v), wl.parent, wl.cu_nodes, wl.kv_start, wl.prefix_len,
                               wl.scale, rows=rows)
    mx, ratio = attn_errors(np.zeros_like(ref), ref, ref_abs, "bf16")
    assert mx < 1e-2          # the stated tolerance alone would accept it
    assert ratio > 1.0
