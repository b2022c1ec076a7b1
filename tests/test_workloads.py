"""The seeded input generators: determinism, shapes and the recipe each
workload states (no GPU, no oracle arithmetic needed)."""
import numpy as np
import pytest

from tree_attention_verification_bitmask_amd import workloads as W


def _small(name, seed=0, **kw):
    # full tree shapes, shortened prefixes so the test stays fast
    over = dict(prefix=(8, 64)) if name in ("c2", "c3", "c4", "c5") else {}
    over.update(kw)
    return W.make_workload(name, seed=seed, **over)


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_deterministic_per_seed(name):
    a, b, c = _small(name, 3), _small(name, 3), _small(name, 4)
    for f in ("parent", "cu_nodes", "prefix_len", "kv_start", "q", "k", "v", "draft", "target", "root_target"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    assert not np.array_equal(a.q, c.q)


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_shapes_and_tree_rules(name):
    cfg = W.CONFIGS[name]
    wl = _small(name, 1)
    B = cfg["batch"]
    assert wl.batch == B and wl.q.shape == (wl.total_nodes, cfg["hq"], cfg["d"])
    assert wl.k.shape == (wl.kv_rows, cfg["hkv"], cfg["d"]) == wl.v.shape
    sizes = np.diff(wl.cu_nodes)
    assert np.all((sizes >= cfg["nodes"][0]) & (sizes <= cfg["nodes"][1]))
    assert np.array_equal(wl.kv_start[1:], np.cumsum(wl.prefix_len + sizes)[:-1])
    for b in range(B):
        par = wl.parent[wl.nodes_of(b)]
        n = len(par)
        assert np.all(par < np.arange(n)) and np.all(par >= -1)
        dep = W._depths(par)
        assert dep.max() <= cfg["max_depth"]
        # siblings carry distinct draft tokens
        dr = wl.draft[wl.nodes_of(b)]
        for p in set(par.tolist()):
            kids = dr[par == p]
            assert len(set(kids.tolist())) == len(kids)
        assert np.all((dr >= 0) & (dr < cfg["vocab"]))
    if cfg["dtype"] == "bf16":
        for x in (wl.q, wl.k, wl.v):
            assert np.array_equal(W.round_to_bf16(x), x)


def test_width_first_shape():
    wl = _small("c4", 2)
    par = wl.parent
    assert np.all(par[:16] == -1)
    for lev in range(1, 16):
        blk = par[lev * 16:(lev + 1) * 16]
        assert np.all((blk >= (lev - 1) * 16) & (blk < lev * 16))
    assert W._depths(par).max() == 16


def test_best_first_is_prefix_closed_and_deep():
    rng = np.random.default_rng(0)
    par = W.best_first_tree(rng, 128, 16)
    assert par[0] == -1 and np.all(par < np.arange(128))
    assert W._depths(par).max() > 4          # best-first grows deep along good paths


def test_round_to_bf16_matches_torch():
    import torch
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 100
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(W.round_to_bf16(x), ref)
    bits = W.to_bf16_bits(ref)
    assert np.array_equal(W.from_bf16_bits(bits), ref)


def test_fifty_percent_target_rule():
    rng = np.random.default_rng(7)
    hits = total = 0
    for _ in range(300):
        par = W.random_tree(rng, 20, 16)
        dr, tg, root = W.draw_tokens(rng, par, 151936)
        for slot in range(-1, 20):
            kids = np.nonzero(par == slot)[0]
            if len(kids) == 0:
                continue
            want = root if slot < 0 else tg[slot]
            hits += int(want in set(dr[kids].tolist()))
            total += 1
    assert 0.45 < hits / total < 0.55


def test_sensitive_values_offset_tree_rows():
    wl = W.make_workload("c2", seed=0, prefix=(64, 64), values="sensitive")
    P = int(wl.prefix_len[0])
    n = wl.total_nodes
    col = np.arange(n) % wl.d
    offs = wl.v[P + np.arange(n), 0, col]
    assert np.all(np.diff(10.0 * (np.arange(n) + 1) / n) > 0)
    assert np.corrcoef(offs, 10.0 * (np.arange(n) + 1) / n)[0, 1] > 0.99
