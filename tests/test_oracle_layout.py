"""Pins of the oracle's dispatch layout (counts, aligned offsets, stable
placement, expert_ids, src_info, overflow flag).

What pins it, none of it the oracle's own code:
  * hand-worked layouts (tests/golden/layout_hand_examples.json);
  * library routines: numpy bincount (counts), cumsum (offsets) and a stable
    argsort (placement order);
  * brute force on tiny inputs: a slot's rank is the number of earlier slots
    in its group;
  * invariants: every kept (token, slot) appears exactly once, the counts sum
    to the number of valid slots, offsets are monotone and aligned, and
    src_info / expert_ids invert token_row.

Sources: NeMo AutoModel token_dispatcher page (_align_up,
moe_router_expert_pad_multiple, _assert_no_hybridep_overflow); NeMo AutoModel
fused_a2a page (HybridEPDispatch.forward: -1 marks unused slots, rows grouped
by local expert); MAX DistributedEPDispatchBlockScaledNVDynGlobalScales page
(row_offsets, expert_ids, src_info, fused_shared_expert).
"""

import itertools
import json
import os

import numpy as np
import pytest

from combine_ep_dispatch_amd import workload as wl


def load_cases(golden_dir):
    with open(os.path.join(golden_dir, "layout_hand_examples.json")) as f:
        return json.load(f)


def test_hand_examples(orc, golden_dir):
    doc = load_cases(golden_dir)
    ids = np.array(doc["topk_ids"], np.int32)
    for case in doc["cases"]:
        cfg = orc.Cfg(**case["cfg"])
        L = orc.layout(cfg, ids)
        assert L["counts"].tolist() == case["counts"], case["name"]
        assert L["row_offsets"].tolist() == case["row_offsets"], case["name"]
        assert L["scales_offsets"].tolist() == case["row_offsets"], case["name"]
        assert L["seg_base"].tolist() == case["seg_base"], case["name"]
        assert L["token_row"].tolist() == case["token_row"], case["name"]
        n = len(case["expert_ids"])
        assert L["expert_ids"][:n].tolist() == case["expert_ids"], case["name"]
        assert L["src_info"][:n].tolist() == case["src_info"], case["name"]
        assert int(L["flags"][0]) == case["flags"], case["name"]
        # rows past the used rows are not written
        assert np.all(L["expert_ids"][n:] == orc.SENTINEL_I32)


def group_of(cfg, ids):
    """Group key of every routed slot (numpy), -1 when masked or invalid."""
    E_loc = cfg.E // cfg.S
    e = ids.astype(np.int64)
    valid = (e >= 0) & (e < cfg.E)
    g = np.where(valid, (e // E_loc) * cfg.G + cfg.shared + (e % E_loc), -1)
    return g


def numpy_layout(cfg, ids):
    """The same layout from numpy library routines (bincount, cumsum, stable argsort)."""
    T, K, Kp, G, S, A = cfg.T, cfg.K, cfg.Kp, cfg.G, cfg.S, cfg.A
    g = group_of(cfg, ids)
    if cfg.shared:
        g = np.concatenate([g, np.full((T, 1), cfg.src_seg * G, np.int64)], axis=1)
    flat = g.reshape(-1)
    counts = np.bincount(flat[flat >= 0], minlength=S * G).reshape(S, G)
    al = -(-counts // A) * A
    off = np.concatenate([np.zeros((S, 1), np.int64), np.cumsum(al, axis=1)], axis=1)
    if cfg.C > 0:
        row_offsets = np.minimum(off, cfg.C)
        seg_base = np.arange(S + 1) * cfg.C
    else:
        row_offsets = off
        seg_base = np.concatenate([[0], np.cumsum(off[:, -1])])
    valid = np.nonzero(flat >= 0)[0]
    order = valid[np.argsort(flat[valid], kind="stable")]
    sorted_g = flat[order]
    first = np.searchsorted(sorted_g, np.arange(S * G))
    rank = np.arange(order.size) - first[sorted_g]
    pos = off.reshape(-1)[(sorted_g // G) * (G + 1) + sorted_g % G] + rank
    token_row = np.full(T * Kp, -1, np.int64)
    keep = (pos < cfg.C) if cfg.C > 0 else np.ones_like(pos, bool)
    token_row[order[keep]] = seg_base[sorted_g[keep] // G] + pos[keep]
    return counts, row_offsets, seg_base, token_row.reshape(T, Kp), bool((~keep).any())


def random_cfg(rng, tiny=False):
    S = int(rng.integers(1, 4 if tiny else 9))
    E_loc = int(rng.integers(1, 4 if tiny else 17))
    E = S * E_loc
    K = int(rng.integers(1, min(E, 3 if tiny else 9) + 1))
    T = int(rng.integers(0, 7 if tiny else 300))
    A = int(rng.choice([1, 2, 3, 4, 16] if tiny else [1, 4, 16, 128]))
    shared = int(rng.integers(0, 2))
    src = int(rng.integers(0, S))
    return T, E, S, K, A, shared, src


def random_ids(rng, T, E, K, mask_p=0.1, bad_p=0.0, distinct=True):
    if distinct:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]) if T else np.zeros((0, K), int)
    else:
        ids = rng.integers(0, E, (T, K))
    ids = np.where(rng.random((T, K)) < mask_p, -1, ids)
    if bad_p > 0:
        bad = rng.random((T, K)) < bad_p
        ids = np.where(bad, rng.choice([-7, -2, E, E + 5], (T, K)), ids)
    return ids.astype(np.int32)


@pytest.mark.parametrize("seed", range(40))
def test_matches_numpy_library_routines(orc, seed):
    rng = np.random.default_rng(1000 + seed)
    T, E, S, K, A, shared, src = random_cfg(rng)
    ids = random_ids(rng, T, E, K, mask_p=0.1, bad_p=0.02 if seed % 4 == 0 else 0.0,
                     distinct=seed % 3 != 0)
    cfg = orc.Cfg(T=T, H=8, E=E, S=S, K=K, A=A, shared=shared, src_seg=src)
    if seed % 5 == 1:  # capacity mode
        load = max(1, T * (K + shared) // S)
        cfg.C = int(rng.integers(1, 2 * load + 2))
    cfg.recv_rows = orc.min_recv_rows(cfg)
    L = orc.layout(cfg, ids)
    counts, row_offsets, seg_base, token_row, dropped = numpy_layout(cfg, ids)
    assert np.array_equal(L["counts"], counts)
    assert np.array_equal(L["row_offsets"], row_offsets)
    assert np.array_equal(L["seg_base"], seg_base)
    assert np.array_equal(L["token_row"], token_row)
    bad = bool(((ids < -1) | (ids >= E)).any())
    assert int(L["flags"][0]) == (1 if dropped else 0) | (2 if bad else 0)


@pytest.mark.parametrize("seed", range(60))
def test_brute_force_tiny(orc, seed):
    rng = np.random.default_rng(seed)
    T, E, S, K, A, shared, src = random_cfg(rng, tiny=True)
    ids = random_ids(rng, T, E, K, mask_p=0.2, distinct=seed % 2 == 0)
    C = int(rng.integers(1, 6)) if seed % 3 == 0 else 0
    cfg = orc.Cfg(T=T, H=8, E=E, S=S, K=K, A=A, C=C, shared=shared, src_seg=src)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    L = orc.layout(cfg, ids)
    G, Kp, E_loc = cfg.G, cfg.Kp, E // S

    def grp(t, k):
        if k == K:
            return src * G
        e = int(ids[t, k])
        return -1 if e < 0 else (e // E_loc) * G + shared + e % E_loc

    slots = [(t, k) for t in range(T) for k in range(Kp)]
    cnt = {}
    for t, k in slots:
        if grp(t, k) >= 0:
            cnt[grp(t, k)] = cnt.get(grp(t, k), 0) + 1

    def aligned(n):
        return -(-n // A) * A

    for t, k in slots:
        g = grp(t, k)
        if g < 0:
            assert L["token_row"][t, k] == -1
            continue
        s, gl = divmod(g, G)
        # brute force: rank = earlier slots of the same group
        rank = sum(1 for (t2, k2) in slots if (t2, k2) < (t, k) and grp(t2, k2) == g)
        start = sum(aligned(cnt.get(s * G + j, 0)) for j in range(gl))
        pos = start + rank
        if C and pos >= C:
            assert L["token_row"][t, k] == -1
            assert int(L["flags"][0]) & 1
            continue
        base = s * C if C else sum(aligned(cnt.get(s2 * G + j, 0)) for s2 in range(s) for j in range(G))
        assert L["token_row"][t, k] == base + pos, (t, k)


def check_invariants(orc, cfg, ids, L):
    T, K, Kp, G, S, A = cfg.T, cfg.K, cfg.Kp, cfg.G, cfg.S, cfg.A
    tr = L["token_row"]
    valid = np.zeros((T, Kp), bool)
    valid[:, :K] = (ids >= 0) & (ids < cfg.E)
    if cfg.shared:
        valid[:, K] = True
    # counts sum to the number of valid slots
    assert L["counts"].sum() == valid.sum()
    # offsets monotone, aligned (below capacity), last = used rows
    ro = L["row_offsets"]
    assert np.all(np.diff(ro, axis=1) >= 0)
    if cfg.C == 0:
        assert np.all(ro % A == 0)
        assert np.array_equal(np.diff(L["seg_base"]), ro[:, -1])
    else:
        assert np.all((ro % A == 0) | (ro == cfg.C))
    # every kept slot appears exactly once
    kept = tr[tr >= 0]
    assert np.unique(kept).size == kept.size
    assert np.all(tr[~valid] == -1)
    if cfg.C == 0:
        assert np.all(tr[valid] >= 0)
    # src_info and expert_ids invert token_row
    tt, kk = np.nonzero(tr >= 0)
    rows = tr[tt, kk]
    assert np.array_equal(L["src_info"][rows, 0], tt)
    assert np.array_equal(L["src_info"][rows, 1], kk)
    eid = np.where(kk < K, ids[tt, np.minimum(kk, K - 1)], cfg.E)
    assert np.array_equal(L["expert_ids"][rows], eid)
    # every used row is either a kept slot or a pad row (-1 metadata)
    used = np.zeros(cfg.recv_rows, bool)
    for s in range(S):
        used[L["seg_base"][s]: L["seg_base"][s] + ro[s, -1]] = True
    pad = used.copy()
    pad[rows] = False
    assert np.all(L["expert_ids"][pad] == -1)
    assert np.all(L["src_info"][pad] == -1)
    assert np.all(L["expert_ids"][~used] == orc.SENTINEL_I32)
    assert set(rows.tolist()) <= set(np.nonzero(used)[0].tolist())
    return int(used.sum())


@pytest.mark.parametrize("name", list(wl.CONFIGS))
def test_invariants_on_workloads(orc, name):
    w = wl.CONFIGS[name]
    d = wl.make_workload(w, with_x=False)
    cfg = orc.Cfg(T=w.T, H=w.H, E=w.E, S=w.S, K=w.K, A=w.align, C=w.capacity,
                  shared=w.shared_expert, src_seg=w.src_segment)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    L = orc.layout(cfg, d["topk_ids"])
    used = check_invariants(orc, cfg, d["topk_ids"], L)
    # seed-0 fingerprints of the generator + layout
    want_used = {"tiny": 304, "dsv3": 48000, "skewed": 72576, "nvfp4": 52096, "capacity": 45784}
    assert used == want_used[name]
    if name == "capacity":
        assert int(L["flags"][0]) == 1
        assert int((L["token_row"] >= 0).sum()) == 45784
    else:
        assert int(L["flags"][0]) == 0


def test_all_masked_and_empty(orc):
    cfg = orc.Cfg(T=5, H=8, E=4, S=2, K=2, A=4)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    L = orc.layout(cfg, np.full((5, 2), -1, np.int32))
    assert L["counts"].sum() == 0 and np.all(L["token_row"] == -1)
    assert np.all(L["row_offsets"] == 0) and np.all(L["seg_base"] == 0)
    cfg0 = orc.Cfg(T=0, H=8, E=4, S=2, K=2, A=4, C=3, recv_rows=6)
    L0 = orc.layout(cfg0, np.zeros((0, 2), np.int32))
    assert L0["seg_base"].tolist() == [0, 3, 6] and L0["counts"].sum() == 0


def test_invalid_ids_are_masked_and_flagged(orc):
    ids = np.array([[0, 9], [-3, 1], [2, -1]], np.int32)
    cfg = orc.Cfg(T=3, H=8, E=4, S=2, K=2, A=1)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    L = orc.layout(cfg, ids)
    assert L["token_row"].tolist() == [[0, -1], [-1, 1], [2, -1]]
    assert int(L["flags"][0]) == 2


def test_duplicate_ids_in_a_token_keep_slot_order(orc):
    ids = np.array([[1, 1], [1, 0]], np.int32)
    cfg = orc.Cfg(T=2, H=8, E=2, S=1, K=2, A=1)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    L = orc.layout(cfg, ids)
    # group 0 (expert 0): (1,1); group 1 (expert 1): (0,0), (0,1), (1,0)
    assert L["token_row"].tolist() == [[1, 2], [3, 0]]


def test_min_recv_rows_is_attained(orc):
    # worst case: every slot in a group of its own with A-1 pad rows
    T, E, K, A = 3, 8, 2, 5
    ids = np.array([[0, 1], [2, 3], [4, 5]], np.int32)
    cfg = orc.Cfg(T=T, H=8, E=E, S=2, K=K, A=A)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    L = orc.layout(cfg, ids)
    assert L["seg_base"][-1] == cfg.recv_rows == T * K * A
    for combo in itertools.islice(itertools.permutations(range(E), K), 5):
        ids = np.array([combo] * T, np.int32)
        assert orc.layout(cfg, ids)["seg_base"][-1] <= cfg.recv_rows
