"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.

Bar: bit-exact for counts, offsets, token_row, expert_ids, src_info, flags,
the bf16 dispatch copy, NVFP4 codes / scales / rowscales and the combine
backward; the combine and dispatch backward reductions must be within
|gpu - oracle| <= 1e-2 + 2e-2 |oracle| and, since both sides add in the same
order without contraction, are also checked bit for bit.

Cases: the five named workloads at full size, the launch configuration the
benchmark times included; seeded random shapes (ragged tiles, partial hidden
pieces, masked / invalid / duplicate ids, shared expert, capacity); edge
cases (no tokens, everything masked, the largest group count, tile
boundaries, K = 1, one expert per segment, tiny capacities).
"""

import dataclasses
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import gpu_cases as gc

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.init()
    return gc


NAMED = ["tiny", "dsv3", "skewed", "nvfp4", "capacity"]


@pytest.mark.parametrize("name", NAMED)
def test_named_workload_full_size(G, name):
    c = G.workload_case(name)
    lay = G.check_layout(c, name)
    f = int(lay.flags.item())
    assert f & 4 == 0
    if name == "nvfp4":
        G.check_nvfp4(c, lay, name)
    if c.cfg.hidden % 128 == 0:
        G.check_fp8(c, lay, name)
    G.check_dispatch(c, lay, name)
    G.check_combine(c, lay, name, weighted=True)
    G.check_dispatch_bwd(c, lay, name)
    G.check_combine_bwd(c, lay, name, weighted=True)
    G.check_probs_grad(c, lay, name)
    G.check_combine_nvfp4(c, lay, name, weighted=True)
    if name == "nvfp4":  # the dispatch's own NVFP4 rows, combined back
        tr = c.L["token_row"]
        G.check_combine_nvfp4(c, lay, name + " round trip", weighted=True,
                              rows=G.orc.dispatch_nvfp4(c.oc, tr, c.x))
    if name == "capacity":
        assert f == 1  # overflow flag raised, nothing else
    else:
        assert f == 0


# Wider sweeps: EPX_GPU_SEEDS=2000 (about 3 minutes on the MI355X) and
# EPX_GPU_LARGE_SEEDS=50 (6.5-10.8 s per large seed, at most 9 minutes);
# EPX_GPU_SEED_BASE shifts both seed ranges to explore new cases.
SEED_BASE = int(os.environ.get("EPX_GPU_SEED_BASE", "0"))
SEEDS = int(os.environ.get("EPX_GPU_SEEDS", "128"))
LARGE_SEEDS = int(os.environ.get("EPX_GPU_LARGE_SEEDS", "4"))
HUGE_SEEDS = int(os.environ.get("EPX_GPU_HUGE_SEEDS", "2"))


@pytest.mark.parametrize("seed", range(SEED_BASE, SEED_BASE + SEEDS))
def test_random_shapes(G, seed):
    rng = np.random.default_rng(seed)
    kw = {}
    if seed % 4 == 1:
        kw["distinct"] = False
    if seed % 6 == 2:
        kw["bad_p"] = 0.05
    c = G.random_case(100 + seed, **kw)
    if seed % 5 == 3:
        load = max(1, c.cfg.num_tokens * c.cfg.kp // c.cfg.num_segments)
        c.cfg.seg_capacity = int(rng.integers(1, load + 2))
        c.cfg.recv_rows = G.epx.ep_query(c.cfg).min_recv_rows
        c = G.Case(c.cfg, c.ids, c.probs, c.x, c.seed)
    name = f"random{seed}"
    lay = G.check_layout(c, name)
    G.check_dispatch(c, lay, name)
    if seed % 2 == 0:
        G.check_dispatch_with_layout(c, name)
    elif c.cfg.hidden % 16 == 0:
        G.check_dispatch_nvfp4_with_layout(c, name)
    if seed % 3 == 0 and c.cfg.hidden % 128 == 0:
        G.check_dispatch_fp8_with_layout(c, name)
    if c.cfg.hidden % 16 == 0:
        G.check_nvfp4(c, lay, name)
    if c.cfg.hidden % 128 == 0:
        G.check_fp8(c, lay, name)
    G.check_combine(c, lay, name, weighted=seed % 2 == 0)
    G.check_dispatch_bwd(c, lay, name)
    G.check_combine_bwd(c, lay, name, weighted=seed % 3 != 0)
    G.check_probs_grad(c, lay, name)
    if c.cfg.hidden % 16 == 0:
        G.check_combine_nvfp4(c, lay, name, weighted=seed % 2 == 1)


@pytest.mark.parametrize("seed", range(SEED_BASE, SEED_BASE + LARGE_SEEDS))
def test_large_random_shapes(G, seed):
    """Multi-tile layouts (direct and look-back paths), bench-like hidden
    sizes, capacity drops and the shared expert at T = 1000..20000."""
    rng = np.random.default_rng(10_000 + seed)
    S = int(rng.choice([1, 2, 4, 8]))
    E_loc = int(rng.choice([1, 4, 16, 32, 64]))
    K = int(rng.integers(1, min(S * E_loc, 8) + 1))
    kw = dict(T=int(rng.integers(1000, 20001)), H=int(rng.choice([512, 2048, 4096, 7168])), S=S, E_loc=E_loc, K=K,
              A=int(rng.choice([1, 16, 128])), shared=int(rng.integers(0, 2)), src=int(rng.integers(0, S)),
              mask_p=float(rng.choice([0.0, 0.01])), bad_p=float(rng.choice([0.0, 0.001])))
    if kw["T"] * kw["H"] > 60_000_000:
        kw["H"] = 2048
    c = G.random_case(20_000 + seed, **kw)
    if seed % 3 == 1:
        load = max(1, c.cfg.num_tokens * c.cfg.kp // c.cfg.num_segments)
        c.cfg.seg_capacity = int(rng.integers(load // 2, load + 2))
        c.cfg.recv_rows = G.epx.ep_query(c.cfg).min_recv_rows
        c = G.Case(c.cfg, c.ids, c.probs, c.x, c.seed)
    name = f"large{seed}"
    lay = G.check_layout(c, name)
    G.check_dispatch(c, lay, name)
    if c.cfg.hidden % 16 == 0:
        G.check_nvfp4(c, lay, name)
    if c.cfg.hidden % 128 == 0:
        G.check_fp8(c, lay, name)
    G.check_combine(c, lay, name, weighted=seed % 2 == 0)
    G.check_dispatch_bwd(c, lay, name)
    G.check_combine_bwd(c, lay, name, weighted=seed % 3 != 0)
    G.check_probs_grad(c, lay, name)
    G.check_combine_nvfp4(c, lay, name, weighted=seed % 2 == 0)


@pytest.mark.parametrize("seed", range(SEED_BASE, SEED_BASE + HUGE_SEEDS))
def test_huge_random_layouts(G, seed):
    """Layouts past one chunk of 256 two-kernel tiles: T = 70 000..400 000
    (up to 3.2 M routed slots, up to 7 chunks), random group counts up to
    2048, repeated ids, masks, bad ids, capacity drops and the shared expert;
    the bf16 movers at narrow rows."""
    rng = np.random.default_rng(30_000 + seed)
    S = int(rng.choice([1, 2, 4, 8]))
    E_loc = int(rng.choice([3, 16, 21, 64, 255]))
    K = int(rng.integers(1, min(S * E_loc, 8) + 1))
    kw = dict(T=int(rng.integers(70_000, 400_001)), H=int(rng.choice([16, 48, 128])), S=S, E_loc=E_loc, K=K,
              A=int(rng.choice([1, 4, 128])), shared=int(rng.integers(0, 2)), src=int(rng.integers(0, S)),
              mask_p=float(rng.choice([0.0, 0.02])), bad_p=float(rng.choice([0.0, 0.001])), distinct=False)
    c = G.random_case(40_000 + seed, **kw)
    if seed % 3 == 1:
        load = max(1, c.cfg.num_tokens * c.cfg.kp // c.cfg.num_segments)
        c.cfg.seg_capacity = int(rng.integers(load // 2, load + 2))
        c.cfg.recv_rows = G.epx.ep_query(c.cfg).min_recv_rows
        c = G.Case(c.cfg, c.ids, c.probs, c.x, c.seed)
    name = f"huge{seed}"
    lay = G.check_layout(c, name)
    G.check_dispatch(c, lay, name)
    G.check_combine(c, lay, name, weighted=seed % 2 == 0)
    G.check_dispatch_bwd(c, lay, name)
    G.check_combine_bwd(c, lay, name, weighted=seed % 2 == 1)


EDGE = {
    "no_tokens": dict(T=0),
    "all_masked": dict(T=300, mask_p=1.0),
    "one_token": dict(T=1, K=3, E_loc=4, S=2),
    "max_groups": dict(T=600, S=8, E_loc=255, K=8, shared=1, A=4),
    "max_groups_flat": dict(T=400, S=1, E_loc=2048, K=6, shared=0, A=2),
    "tile_exact": dict(T=2048, K=2, S=2, E_loc=8),
    "tile_plus_one": dict(T=2049, K=2, S=2, E_loc=8),
    "tile_minus_one_slot": dict(T=683, K=3, S=4, E_loc=5),
    "k1": dict(T=500, K=1),
    "one_expert_per_segment": dict(T=700, S=8, E_loc=1, K=4),
    "align_one": dict(T=700, A=1),
    "big_align": dict(T=300, A=256, S=3, E_loc=3, K=2),
    "many_tiles": dict(T=9000, S=4, E_loc=16, K=8, A=16, H=16),
    "hot_expert": dict(T=4000, S=2, E_loc=1, K=1, H=32, A=8),
    "spt1_157_tiles": dict(T=5001, S=8, E_loc=8, K=8, H=16, A=4),        # 1 slot/thread, ragged last tile
    "spt1_at_cap": dict(T=4096, S=4, E_loc=32, K=8, H=16, A=8),           # 128 groups: 128 tiles, one batch
    "spt2_past_cap": dict(T=4097, S=4, E_loc=32, K=8, H=16, A=8),         # one slot more: 2 slots/thread
    "spt4_157_tiles": dict(T=20011, S=4, E_loc=16, K=8, H=16, A=2),       # 4 slots/thread
    "direct_four_batches": dict(T=25000, S=8, E_loc=32, K=8, H=16, A=2),  # 256 groups, 196 tiles: 4 load batches
    "direct_254_tiles": dict(T=65000, S=4, E_loc=16, K=8, H=16, A=2, bad_p=0.01),  # direct path, near its tile limit
    # past 256 two-kernel tiles: 274 tiles, two chunks of tile-count sums (68 groups: 16-byte column loads)
    "direct_274_tiles_chunked": dict(T=70001, S=4, E_loc=16, K=8, H=16, A=2, shared=1, src=3, bad_p=0.01),
    # 293 tiles, a ragged second chunk, 21 groups (one group per load, 8 lanes per group)
    "direct_293_tiles_ragged_chunk": dict(T=100001, S=3, E_loc=7, K=6, H=16, A=4, mask_p=0.05),
    # 4096 tiles in 16 chunks, 16 groups (16-byte loads)
    "direct_16_chunks": dict(T=1 << 20, S=2, E_loc=8, K=8, H=16, A=8, distinct=False),
    "single_pass_max_groups": dict(T=128, S=8, E_loc=255, K=8, shared=1, A=4, H=32),  # 2048 groups, one launch
    "single_pass_1024": dict(T=128, S=8, E_loc=32, K=8, H=64, A=128, shared=1, src=5),  # 1024 slots: count path
    "single_pass_1023": dict(T=1023, S=4, E_loc=8, K=1, H=16, A=4),                   # count path, ragged tile
    "direct_1025": dict(T=1025, S=4, E_loc=8, K=1, H=16, A=4, bad_p=0.01),            # count path, 5 tiles
    "direct_2048": dict(T=256, S=8, E_loc=32, K=8, H=64, A=128, shared=1, src=5),     # decode batch, count path
    "single_pass_256": dict(T=64, S=2, E_loc=16, K=4, H=32, A=8, mask_p=0.1),         # 1 slot/thread bound
    "single_pass_257": dict(T=257, S=4, E_loc=4, K=1, H=32, A=2),                     # 2 slots/thread
    "single_pass_512": dict(T=128, S=2, E_loc=16, K=4, H=32, A=8, bad_p=0.02),        # small path bound
    "single_pass_513": dict(T=171, S=3, E_loc=5, K=3, H=32, A=2, mask_p=0.2),         # one past it: count path
    "count_8192": dict(T=1024, S=8, E_loc=32, K=8, H=64, A=128, mask_p=0.05),        # count path bound
    "direct_8193": dict(T=8193, S=4, E_loc=8, K=1, H=16, A=4, bad_p=0.01),            # one past it: two kernels
    # the largest layout call: 2^24 routed slots, 264 groups; by default two
    # kernels over 8192 tiles in 32 chunks, forced: 8192 single-pass tiles
    "max_routed_slots": dict(T=1 << 21, S=8, E_loc=32, K=8, H=16, A=128, shared=1, src=3, mask_p=0.01,
                             distinct=False),
    "slots_64": dict(T=300, S=1, E_loc=64, K=63, shared=1, src=0, H=64, A=4),  # K' = 64: 16 scatter slot blocks
    "hidden_8": dict(T=500, S=2, E_loc=4, K=3, H=8),                          # one ragged piece per row
    "hidden_16k": dict(T=300, S=2, E_loc=4, K=4, H=16384, A=8),               # 8 full pieces, 16 NVFP4 blocks per lane
    "fused_wide_row": dict(T=5, S=2, E_loc=4, K=2, H=16392, A=4, shared=1),   # one-call bf16 copy past 16384 elements
    # quantizing dispatch, one workgroup per token: K' = 9 (a wave stores two slot rows), masks, bad ids
    "quant_wg_k9": dict(T=700, S=4, E_loc=8, K=8, shared=1, src=1, H=7168, A=4, mask_p=0.1, bad_p=0.01),
    "quant_wg_capacity": dict(T=900, S=2, E_loc=16, K=6, H=4096, A=2, C=1500),       # capacity drops
}


@pytest.mark.parametrize("edge", sorted(EDGE))
def test_edge_cases(G, edge):
    c = G.random_case(7, **dict(EDGE[edge]))
    lay = G.check_layout(c, edge)
    G.check_dispatch(c, lay, edge)
    G.check_dispatch_with_layout(c, edge)
    if c.cfg.hidden % 16 == 0:
        G.check_nvfp4(c, lay, edge)
        G.check_dispatch_nvfp4_with_layout(c, edge)
    if c.cfg.hidden % 128 == 0:
        G.check_dispatch_fp8_with_layout(c, edge)
    if c.cfg.hidden % 128 == 0:
        G.check_fp8(c, lay, edge)
    G.check_combine(c, lay, edge)
    G.check_dispatch_bwd(c, lay, edge)
    G.check_combine_bwd(c, lay, edge)
    G.check_probs_grad(c, lay, edge)
    if c.cfg.hidden % 16 == 0:
        G.check_combine_nvfp4(c, lay, edge)


@pytest.mark.parametrize("C", [1, 2, 7, 64])
def test_tiny_capacities(G, C):
    c = G.random_case(55, T=400, S=4, E_loc=4, K=4, A=4, shared=1, src=2, C=C, H=256)
    c.cfg.recv_rows = G.epx.ep_query(c.cfg).min_recv_rows
    c = G.Case(c.cfg, c.ids, c.probs, c.x, c.seed)
    lay = G.check_layout(c, f"cap{C}")
    assert int(lay.flags.item()) & 1
    G.check_dispatch(c, lay, f"cap{C}")
    G.check_nvfp4(c, lay, f"cap{C}")
    if c.cfg.hidden % 128 == 0:
        G.check_fp8(c, lay, f"cap{C}")
    G.check_combine(c, lay, f"cap{C}")
    G.check_combine_bwd(c, lay, f"cap{C}")
    G.check_probs_grad(c, lay, f"cap{C}")


@pytest.mark.parametrize("H", [1040, 4096, 16384])
def test_nvfp4_special_rows(G, H):
    """Zero tokens, negative zeros, subnormal bf16 values, huge outliers,
    tiny blocks next to a large one (E4M3-subnormal and zero block scales).
    H = 1040: 65 blocks, the second block column of a lane is ragged (four
    waves per token); 4096 and 16384: one workgroup per token, with one and
    two blocks per lane."""
    rng = np.random.default_rng(3)
    T = 64
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[0] = 0
    x[1] = -0.0
    x[2] = 1e-39                                   # bf16 subnormals
    x[3, :] = 1e-5 * rng.standard_normal(H)
    x[3, 17] = 250.0                               # tiny blocks beside a big one
    x[4] *= 3e4
    x[5] = rng.uniform(-6, 6, H)
    x[6, ::2] = 0.0
    x[7] = 10.0 ** rng.uniform(-30, 30, H) * np.sign(rng.standard_normal(H))
    xb = G.wl.bf16_bits(x)
    c = G.random_case(9, T=T, H=H, S=2, E_loc=4, K=2, A=4, shared=1, src=0, mask_p=0.0)
    c = G.Case(c.cfg, c.ids, c.probs, xb, c.seed)
    lay = G.check_layout(c, "nvfp4_special")
    G.check_nvfp4(c, lay, "nvfp4_special")
    if H % 128 == 0:
        G.check_fp8(c, lay, "fp8_special")


@pytest.mark.parametrize("H", [1040, 4096])
def test_combine_nvfp4_special_rows(G, H):
    """NVFP4 combine over rows with every E4M3 scale byte (the NaN codes 0x7F
    and 0xFF included), every code byte, and rowscales 0, -0, bf16
    subnormals, the largest finite bf16, infinity and NaN.  Outputs that are
    NaN must be NaN in both; all others equal bit for bit.  H = 1040: 65
    blocks, the second piece of a token holds one block."""
    rng = np.random.default_rng(5)
    T = 64
    c = G.random_case(12, T=T, H=H, S=2, E_loc=4, K=3, A=4, shared=1, src=0, mask_p=0.1)
    lay = G.check_layout(c, "nvfp4_combine_special")
    R = c.cfg.recv_rows
    codes = rng.integers(0, 256, (R, H // 2), dtype=np.uint8)
    scales = (np.arange(R * (H // 16)) % 256).astype(np.uint8).reshape(R, H // 16)
    rng.shuffle(scales, axis=1)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0],
                        np.uint16)
    rs = G.wl.bf16_bits(np.exp2(rng.uniform(-20, 20, R)).astype(np.float32))
    rs[: specials.size] = specials
    rng.shuffle(rs)
    probs = c.probs
    y = G.bf16_filled(T, H, G.orc.SENTINEL_U16)
    G.epx.ep_combine_nvfp4(c.cfg, lay, torch.from_numpy(codes.reshape(-1)).to(G.DEV),
                           torch.from_numpy(scales.reshape(-1)).to(G.DEV), G.u16_tensor(rs),
                           torch.from_numpy(probs.reshape(-1)).to(G.DEV), y)
    torch.cuda.synchronize()
    got = G.bits_of(y).reshape(-1)
    want = G.orc.combine_nvfp4(c.oc, c.L["token_row"], codes, scales, rs, probs).reshape(-1)
    nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    assert np.array_equal(nan(got), nan(want)), np.nonzero(nan(got) != nan(want))[0][:8]
    assert nan(want).any() and (~nan(want)).any()
    G.assert_bits_equal(got[~nan(want)], want[~nan(want)], "combine_nvfp4 special rows")


def test_fp8_special_rows(G):
    """FP8 blocks with zeros, -0, bf16 subnormals, huge and tiny magnitudes,
    ties at E4M3 midpoints, and a ragged last block group (H/128 = 9)."""
    rng = np.random.default_rng(4)
    T, H = 48, 1152
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[0] = 0
    x[1] = -0.0
    x[2, :128] = 1e-39
    x[3] = (rng.standard_normal(H) * 10.0 ** rng.uniform(-20, 20, H)).astype(np.float32)
    x[4, :128] = 7.0 * rng.integers(-64, 65, 128) / 64  # values on the E4M3 grid and midpoints
    x[5, ::3] = 0.0
    xb = G.wl.bf16_bits(x)
    c = G.random_case(11, T=T, H=H, S=2, E_loc=4, K=2, A=4, shared=1, src=1, mask_p=0.0)
    c = G.Case(c.cfg, c.ids, c.probs, xb, c.seed)
    lay = G.check_layout(c, "fp8_special")
    G.check_fp8(c, lay, "fp8_special")


def sp_header(ws):
    """(generation, ticket, departure word) of a single-pass workspace."""
    h = ws[:16].cpu().numpy().view(np.uint64)
    return int(h[0]) >> 32, int(h[0]) & 0xFFFFFFFF, int(h[1])


def test_single_pass_workspace_reuse(G):
    """One zeroed workspace serves a sequence of single-pass layouts of
    different shapes (more tiles, fewer, more groups, capacity drops, bad
    ids): every call matches the oracle, and each leaves the header with the
    ticket and the departure word reset and the generation one higher, so stale descriptors of earlier calls are never taken for
    current ones."""
    seq = [G.workload_case("dsv3"), G.random_case(5, T=300, S=2, E_loc=3, K=2, A=4),
           G.workload_case("skewed", T=5000), G.random_case(6, T=2000, S=8, E_loc=256, K=6, A=1, shared=0),
           G.workload_case("capacity", T=3000), G.random_case(7, T=4000, S=4, E_loc=8, K=4, bad_p=0.05),
           G.workload_case("dsv3")]
    nbytes = max(G.epx.ep_query(c.cfg).workspace_bytes for c in seq)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=G.DEV)
    gen0 = sp_header(ws)[0]
    for i, c in enumerate(seq + seq):
        path = "single-pass" if i < len(seq) else "single-pass-barrier"
        lay = G.gpu_layout(c.cfg, c.ids, ws=ws, path=path)
        G.assert_layout_equal(G.layout_np(lay), c.L, f"reuse call {i} ({path})")
        gen, ticket, depart = sp_header(ws)
        assert (gen, ticket, depart) == (gen0 + i + 1, 0, 0), (i, gen, ticket, depart)
    # two-kernel calls in between write tile counts into the same workspace:
    # the next single-pass call must not take them for descriptors
    c = G.workload_case("skewed", T=3000)
    G.gpu_layout(c.cfg, c.ids, ws=ws, path="two-kernel")
    G.assert_layout_equal(G.layout_np(G.gpu_layout(c.cfg, c.ids, ws=ws, path="single-pass")), c.L, "after 2k")


def test_concurrent_streams(G):
    """Calls on two streams at once, each with its own workspace and output
    buffers, do not interfere: layouts (the single pass keeps a ticket and a
    generation in its workspace) and bf16 dispatches of two different
    shapes, enqueued alternately on two default-priority streams, match the
    oracle on every round."""
    cases = [G.workload_case("skewed", T=3000), G.random_case(11, T=2500, S=4, E_loc=16, K=6, A=16, H=256)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    paths = [G.epx.EP_LAYOUT_LOOKBACK, 0, G.epx.EP_LAYOUT_BARRIER]
    for rnd in range(3):
        cfgs = [dataclasses.replace(c.cfg, flags=paths[(rnd + i) % 3]) for i, c in enumerate(cases)]
        ids = [torch.from_numpy(np.ascontiguousarray(c.ids, np.int32).reshape(-1)).to(G.DEV) for c in cases]
        xs = [G.u16_tensor(c.x) for c in cases]
        lays = [G.sentinel_layout(cfg) for cfg in cfgs]
        wss = [G.epx.workspace_for(cfg, G.DEV) for cfg in cfgs]
        recvs = [G.bf16_filled(cfg.recv_rows, cfg.hidden, G.orc.SENTINEL_U16) for cfg in cfgs]
        torch.cuda.synchronize()
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                G.epx.ep_dispatch_layout(cfgs[i], ids[i], wss[i], lays[i])
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                G.epx.ep_dispatch(cfgs[i], lays[i], xs[i], recvs[i])
        torch.cuda.synchronize()
        for i, c in enumerate(cases):
            G.assert_layout_equal(G.layout_np(lays[i]), c.L, f"stream {i} round {rnd}")
            G.assert_bits_equal(G.bits_of(recvs[i]), G.orc.dispatch(c.oc, c.L["token_row"], c.x),
                                f"stream {i} round {rnd}: recv")


def test_determinism(G):
    c = G.workload_case("skewed", T=3000)
    for path in G.LAYOUT_PATHS:
        a = G.layout_np(G.gpu_layout(c.cfg, c.ids, path=path))
        b = G.layout_np(G.gpu_layout(c.cfg, c.ids, path=path))
        for k in a:
            assert np.array_equal(a[k], b[k]), (path, k)
        G.assert_layout_equal(a, c.L, f"skewed3000 {path}")


def test_dispatch_with_layout_matches_separate_calls(G):
    """ep_dispatch_with_layout gives the bytes of ep_dispatch_layout then
    ep_dispatch, and ep_dispatch_nvfp4_with_layout those of
    ep_dispatch_layout then ep_dispatch_nvfp4, pad rows zeroed or untouched,
    on the fused small path
    (up to 512 routed slots: 1, 300 and 512 slots, shared expert, capacity
    drops, masked and bad ids) and past it (513 slots)."""
    cases = [dict(T=1, S=2, E_loc=4, K=1, H=16, A=8),
             dict(T=100, S=3, E_loc=5, K=3, A=16, H=64, shared=1, src=1, mask_p=0.05, bad_p=0.02),
             dict(T=64, S=8, E_loc=32, K=8, A=128, H=1040, shared=1, src=5),
             dict(T=170, S=3, E_loc=5, K=3, A=2, H=48, C=40, shared=1),
             dict(T=171, S=3, E_loc=5, K=3, A=2, H=48, C=40)]
    for i, kw in enumerate(cases):
        c = G.random_case(60 + i, **kw)
        for flags in (0, G.epx.EP_ZERO_PAD_ROWS):
            cfg = dataclasses.replace(c.cfg, flags=flags)
            ids_t = torch.from_numpy(np.ascontiguousarray(c.ids, np.int32).reshape(-1)).to(G.DEV)
            x = G.u16_tensor(c.x)
            lay1, lay2 = G.sentinel_layout(cfg), G.sentinel_layout(cfg)
            r1 = G.bf16_filled(cfg.recv_rows, cfg.hidden, 0x7FA5)
            r2 = G.bf16_filled(cfg.recv_rows, cfg.hidden, 0x7FA5)
            G.epx.ep_dispatch_layout(cfg, ids_t, G.epx.workspace_for(cfg, G.DEV), lay1)
            G.epx.ep_dispatch(cfg, lay1, x, r1)
            G.epx.ep_dispatch_with_layout(cfg, ids_t, G.epx.workspace_for(cfg, G.DEV), lay2, x, r2)
            torch.cuda.synchronize()
            G.assert_layout_equal(G.layout_np(lay2), G.layout_np(lay1), f"case {i} flags {flags}")
            G.assert_bits_equal(G.bits_of(r2), G.bits_of(r1), f"case {i} flags {flags}: recv")
            G.assert_layout_equal(G.layout_np(lay2), c.L, f"case {i} flags {flags} (oracle)")
            # the NVFP4 form against ep_dispatch_nvfp4 on the separate layout
            R, H = cfg.recv_rows, cfg.hidden
            q1 = [torch.full((R * H // 2,), 0xA5, dtype=torch.uint8, device=G.DEV),
                  torch.full((R * H // 16,), 0xA5, dtype=torch.uint8, device=G.DEV), G.bf16_filled(R, 1, 0x7FA5)]
            q2 = [t.clone() for t in q1]
            lay3 = G.sentinel_layout(cfg)
            G.epx.ep_dispatch_nvfp4(cfg, lay1, x, *q1)
            G.epx.ep_dispatch_nvfp4_with_layout(cfg, ids_t, G.epx.workspace_for(cfg, G.DEV), lay3, x, *q2)
            torch.cuda.synchronize()
            G.assert_layout_equal(G.layout_np(lay3), G.layout_np(lay1), f"case {i} flags {flags} (nvfp4)")
            for n, a_, b_ in zip(("codes", "scales", "rowscale"), q2, q1):
                G.assert_bits_equal(a_.view(torch.uint8).cpu().numpy(), b_.view(torch.uint8).cpu().numpy(),
                                    f"case {i} flags {flags}: {n}")


def test_dispatch_fp8_with_layout_matches_separate_calls(G):
    """ep_dispatch_fp8_with_layout gives the bytes of ep_dispatch_layout then
    ep_dispatch_fp8, pad rows zeroed or untouched: one kernel at 1, 300, 510
    and 512 routed slots (shared expert, capacity drops, masked and bad ids;
    rows of 1, 2 and 7 iterations of 8 128-element blocks, the last two
    ragged) and the layout launches then the FP8 dispatch at 513."""
    cases = [dict(T=1, S=2, E_loc=4, K=1, H=128, A=8),
             dict(T=100, S=3, E_loc=5, K=3, A=16, H=7168, shared=1, src=1, mask_p=0.05, bad_p=0.02),
             dict(T=64, S=8, E_loc=32, K=8, A=128, H=1152, shared=1, src=5),
             dict(T=170, S=3, E_loc=5, K=3, A=2, H=256, C=40, shared=1),
             dict(T=171, S=3, E_loc=5, K=3, A=2, H=256, C=40)]
    for i, kw in enumerate(cases):
        c = G.random_case(80 + i, **kw)
        for flags in (0, G.epx.EP_ZERO_PAD_ROWS):
            cfg = dataclasses.replace(c.cfg, flags=flags)
            R, H = cfg.recv_rows, cfg.hidden
            ids_t = torch.from_numpy(np.ascontiguousarray(c.ids, np.int32).reshape(-1)).to(G.DEV)
            x = G.u16_tensor(c.x)
            lay1, lay2 = G.sentinel_layout(cfg), G.sentinel_layout(cfg)
            q1 = [torch.full((R * H,), 0xA5, dtype=torch.uint8, device=G.DEV),
                  torch.full((R * (H // 128),), 0x7FA5A5A5, dtype=torch.int32, device=G.DEV).view(torch.float32)]
            q2 = [t.clone() for t in q1]
            G.epx.ep_dispatch_layout(cfg, ids_t, G.epx.workspace_for(cfg, G.DEV), lay1)
            G.epx.ep_dispatch_fp8(cfg, lay1, x, *q1)
            G.epx.ep_dispatch_fp8_with_layout(cfg, ids_t, G.epx.workspace_for(cfg, G.DEV), lay2, x, *q2)
            torch.cuda.synchronize()
            G.assert_layout_equal(G.layout_np(lay2), G.layout_np(lay1), f"case {i} flags {flags} (fp8)")
            G.assert_layout_equal(G.layout_np(lay2), c.L, f"case {i} flags {flags} (fp8, oracle)")
            for n, a_, b_ in zip(("codes", "scales"), q2, q1):
                G.assert_bits_equal(a_.view(torch.uint8).cpu().numpy(), b_.view(torch.uint8).cpu().numpy(),
                                    f"case {i} flags {flags}: fp8 {n}")


def test_zero_pad_rows_flag(G):
    c = G.random_case(21, T=333, S=3, E_loc=5, K=3, A=16, H=64, shared=1, src=1)
    c.cfg.flags = G.epx.EP_ZERO_PAD_ROWS
    lay = G.check_layout(c, "zero_pad")
    cfg = c.cfg
    tr = c.L["token_row"]
    used = np.zeros(cfg.recv_rows, bool)
    for s in range(cfg.num_segments):
        used[c.L["seg_base"][s]: c.L["seg_base"][s] + c.L["row_offsets"][s, -1]] = True
    pad = used.copy()
    pad[tr[tr >= 0]] = False
    assert pad.any()
    recv = G.bf16_filled(cfg.recv_rows, cfg.hidden, 0x7FA5)
    G.epx.ep_dispatch(cfg, lay, G.u16_tensor(c.x), recv)
    codes = torch.full((cfg.recv_rows * cfg.hidden // 2,), 0xA5, dtype=torch.uint8, device=G.DEV)
    scales = torch.full((cfg.recv_rows * cfg.hidden // 16,), 0xA5, dtype=torch.uint8, device=G.DEV)
    rowscale = G.bf16_filled(cfg.recv_rows, 1, 0x7FA5)
    G.epx.ep_dispatch_nvfp4(cfg, lay, G.u16_tensor(c.x), codes, scales, rowscale)
    gy = G.wl.make_tensor_like_rows(cfg.num_tokens, cfg.hidden, 5)
    go = G.bf16_filled(cfg.recv_rows, cfg.hidden, 0x7FA5)
    G.epx.ep_combine_bwd(cfg, lay, G.u16_tensor(gy), torch.from_numpy(c.probs.reshape(-1)).to(G.DEV), go)
    torch.cuda.synchronize()
    r = G.bits_of(recv).reshape(cfg.recv_rows, cfg.hidden)
    assert np.all(r[pad] == 0) and np.all(r[~used] == 0x7FA5)
    # the layout and dispatch in one call (layout launch then scatter at this size) zero the same pad rows
    lay2 = G.sentinel_layout(cfg)
    recv2 = G.bf16_filled(cfg.recv_rows, cfg.hidden, 0x7FA5)
    ids_t = torch.from_numpy(np.ascontiguousarray(c.ids, np.int32).reshape(-1)).to(G.DEV)
    G.epx.ep_dispatch_with_layout(cfg, ids_t, G.epx.workspace_for(cfg, G.DEV), lay2, G.u16_tensor(c.x), recv2)
    torch.cuda.synchronize()
    assert np.array_equal(G.bits_of(recv2), G.bits_of(recv))
    G.assert_layout_equal(G.layout_np(lay2), c.L, "zero_pad (with layout)")
    assert np.array_equal(r[tr[tr >= 0]], G.orc.dispatch(c.oc, tr, c.x)[tr[tr >= 0]])
    cd = codes.cpu().numpy().reshape(cfg.recv_rows, -1)
    sc = scales.cpu().numpy().reshape(cfg.recv_rows, -1)
    rs = G.bits_of(rowscale)
    assert np.all(cd[pad] == 0) and np.all(sc[pad] == 0) and np.all(rs[pad] == 0)
    assert np.all(cd[~used] == 0xA5) and np.all(rs[~used] == 0x7FA5)
    g = G.bits_of(go).reshape(cfg.recv_rows, cfg.hidden)
    assert np.all(g[pad] == 0) and np.all(g[~used] == 0x7FA5)


def test_assert_no_overflow(G):
    c = G.workload_case("capacity", T=2000)
    lay = G.gpu_layout(c.cfg, c.ids)
    with pytest.raises(G.epx.EpError):
        G.epx.assert_no_overflow(lay, capacity=c.cfg.seg_capacity)
    c2 = G.workload_case("tiny")
    G.epx.assert_no_overflow(G.gpu_layout(c2.cfg, c2.ids))


def test_combine_of_dispatch_is_identity_on_gpu(G):
    """combine(dispatch(x)) with identity experts and probabilities summing
    to 1 returns x exactly (the shared expert, weight 1, doubles it)."""
    for name in ("dsv3", "nvfp4"):
        c = G.workload_case(name, T=512)
        cfg = c.cfg
        lay = G.gpu_layout(cfg, c.ids)
        recv = G.bf16_filled(cfg.recv_rows, cfg.hidden, 0x7FC1)  # pad rows stay NaN
        G.epx.ep_dispatch(cfg, lay, G.u16_tensor(c.x), recv)
        y = G.bf16_filled(cfg.num_tokens, cfg.hidden, 0)
        G.epx.ep_combine(cfg, lay, recv, torch.from_numpy(c.probs.reshape(-1)).to(G.DEV), y)
        torch.cuda.synchronize()
        want = c.x if not cfg.shared_expert else G.wl.bf16_bits(2.0 * G.f32(c.x))
        assert np.array_equal(G.bits_of(y).reshape(cfg.num_tokens, -1), want), name


def test_graph_replays_match_eager(G):
    """The whole step captured into a HIP graph: every replay (with eager
    work and output clearing in between) reproduces the eager results and
    the oracle's layout."""
    c = G.workload_case("nvfp4", T=1024)
    cfg = c.cfg
    epx, DEV = G.epx, G.DEV
    R, T, H = cfg.recv_rows, cfg.num_tokens, cfg.hidden
    ids = torch.from_numpy(c.ids.reshape(-1)).to(DEV)
    x = G.u16_tensor(c.x)
    probs = torch.from_numpy(c.probs.reshape(-1)).to(DEV)
    out = G.u16_tensor(c.rows(1))
    lay = epx.Layout.empty(cfg, DEV)
    ws = epx.workspace_for(cfg, DEV)
    bufs = {"recv": torch.empty(R * H, dtype=torch.bfloat16, device=DEV),
            "codes": torch.empty(R * H // 2, dtype=torch.uint8, device=DEV),
            "scales": torch.empty(R * H // 16, dtype=torch.uint8, device=DEV),
            "rowscale": torch.empty(R, dtype=torch.bfloat16, device=DEV),
            "y": torch.empty(T * H, dtype=torch.bfloat16, device=DEV),
            "gout": torch.empty(R * H, dtype=torch.bfloat16, device=DEV),
            "gx": torch.empty(T * H, dtype=torch.bfloat16, device=DEV)}

    def step():
        epx.ep_dispatch_layout(cfg, ids, ws, lay)
        epx.ep_dispatch(cfg, lay, x, bufs["recv"])
        epx.ep_dispatch_nvfp4(cfg, lay, x, bufs["codes"], bufs["scales"], bufs["rowscale"])
        epx.ep_combine(cfg, lay, out, probs, bufs["y"])
        epx.ep_combine_bwd(cfg, lay, bufs["y"], probs, bufs["gout"])
        epx.ep_dispatch_bwd(cfg, lay, out, bufs["gx"])

    def clear():
        for t in list(bufs.values()) + [lay.token_row, lay.expert_ids, lay.src_info, lay.counts, lay.flags]:
            t.view(torch.uint8).fill_(0x5A)

    clear()
    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in bufs.items()}
    ref_tr = lay.token_row.clone()
    assert np.array_equal(ref_tr.cpu().numpy(), c.L["token_row"])

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = G.random_case(3, T=200, H=256)
    for i in range(4):
        clear()
        torch.cuda.synchronize()
        G.check_layout(other, f"eager between replays {i}")  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lay.token_row, ref_tr), i
        for k, v in bufs.items():
            if k in ("recv", "codes", "scales", "rowscale", "gout"):
                # only the used rows are defined
                used = torch.from_numpy(np.unique(c.L["token_row"][c.L["token_row"] >= 0])).to(DEV).long()
                a, b = v.view(R, -1)[used], ref[k].view(R, -1)[used]
            else:
                a, b = v, ref[k]
            assert torch.equal(a, b), (i, k)


def test_graph_replays_of_decode_step_with_fused_dispatch(G):
    """A decode-sized step (T=16 at DeepSeek-V3 dims: the layout and the
    dispatch in one kernel, then combine) captured into a HIP graph: every
    replay, with its outputs cleared and unrelated eager work in between,
    gives the eager results, and those equal the oracle's."""
    c = G.workload_case("dsv3", T=16)
    cfg = dataclasses.replace(c.cfg, flags=G.epx.EP_ZERO_PAD_ROWS)
    epx, DEV = G.epx, G.DEV
    R, T, H = cfg.recv_rows, cfg.num_tokens, cfg.hidden
    ids = torch.from_numpy(np.ascontiguousarray(c.ids, np.int32).reshape(-1)).to(DEV)
    x = G.u16_tensor(c.x)
    probs = torch.from_numpy(c.probs.reshape(-1)).to(DEV)
    out = G.u16_tensor(c.rows(2))
    lay = epx.Layout.empty(cfg, DEV)
    ws = epx.workspace_for(cfg, DEV)
    recv = torch.empty(R * H, dtype=torch.bfloat16, device=DEV)
    y = torch.empty(T * H, dtype=torch.bfloat16, device=DEV)

    def step():
        epx.ep_dispatch_with_layout(cfg, ids, ws, lay, x, recv)
        epx.ep_combine(cfg, lay, out, probs, y)

    def clear():
        # the oracle's sentinel bytes: rows past the used ones stay unwritten
        for t in (recv, y, lay.token_row, lay.expert_ids, lay.src_info, lay.counts, lay.row_offsets, lay.flags):
            t.view(torch.uint8).fill_(int(G.orc.SENTINEL_U8))

    clear()
    step()
    torch.cuda.synchronize()
    G.assert_layout_equal(G.layout_np(lay), c.L, "decode step (eager)")
    want_recv = G.orc.dispatch(c.oc, c.L["token_row"], c.x)
    used = np.zeros(R, bool)
    for sg in range(cfg.num_segments):
        used[c.L["seg_base"][sg]: c.L["seg_base"][sg] + c.L["row_offsets"][sg, -1]] = True
    tr = c.L["token_row"]
    kept = np.zeros(R, bool)
    kept[tr[tr >= 0]] = True
    got = G.bits_of(recv).reshape(R, H)
    assert (used & ~kept).any()
    assert np.array_equal(got[kept], want_recv.reshape(R, H)[kept])
    assert np.all(got[used & ~kept] == 0)  # pad rows zeroed
    G.assert_bits_equal(G.bits_of(y), G.orc.combine(c.oc, c.L["token_row"], c.rows(2), c.probs), "decode y")
    ref_recv, ref_y, ref_tr = recv.clone(), y.clone(), lay.token_row.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    other = G.random_case(5, T=40, H=64)
    u = torch.from_numpy(np.nonzero(used)[0]).to(DEV).long()
    for i in range(4):
        clear()
        torch.cuda.synchronize()
        G.check_dispatch_with_layout(other, f"eager between replays {i}")  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lay.token_row, ref_tr), i
        assert torch.equal(recv.view(R, H)[u], ref_recv.view(R, H)[u]), i
        assert torch.equal(y, ref_y), i


def test_autograd_dispatch_with_ids_matches_route_then_dispatch(G):
    """EpDispatcher.dispatch(x, topk_ids) (layout and dispatch in one call,
    one kernel at 64 routed slots) gives the receive rows and the input
    gradient of route(topk_ids) then dispatch(x), bit for bit, and the
    oracle's receive rows."""
    from combine_ep_dispatch_amd.autograd import EpDispatcher

    c = G.random_case(45, T=16, S=4, E_loc=8, K=4, H=256, A=8, shared=1, src=1, mask_p=0.1)
    T, H = c.cfg.num_tokens, c.cfg.hidden
    ids = torch.from_numpy(c.ids).to(G.DEV)
    gr = G.u16_tensor(G.wl.make_tensor_like_rows(c.cfg.recv_rows, H, 6)).view(-1, H)
    out = []
    for one_call in (True, False):
        cfg = G.epx.EpConfig(num_tokens=T, hidden=H, num_experts=c.cfg.num_experts, num_segments=c.cfg.num_segments,
                             top_k=c.cfg.top_k, align=c.cfg.align, shared_expert=1, src_segment=1)
        d = EpDispatcher(cfg, G.DEV)
        x = G.u16_tensor(c.x).view(T, H).clone().requires_grad_(True)
        if one_call:
            recv = d.dispatch(x, ids)
        else:
            d.route(ids)
            recv = d.dispatch(x)
        (recv.float() * gr.float()).sum().backward()
        torch.cuda.synchronize()
        out.append((G.bits_of(recv.detach()), G.bits_of(x.grad), G.layout_np(d.layout)))
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][1], out[1][1])
    for k in ("counts", "row_offsets", "seg_base", "token_row", "flags"):  # written whole (rows past the used
        assert np.array_equal(out[0][2][k], c.L[k]), k                    # ones stay as Layout.empty left them)
    tr = c.L["token_row"]
    kept = np.zeros(c.cfg.recv_rows, bool)
    kept[tr[tr >= 0]] = True
    want = G.orc.dispatch(c.oc, tr, c.x).reshape(c.cfg.recv_rows, H)
    assert np.array_equal(out[0][0].reshape(-1, H)[kept], want[kept])


def test_autograd_dispatcher_matches_fp64_reference(G):
    """EpDispatcher: dispatch -> (x2) -> combine with autograd, against torch
    fp64 autograd of an index_select / index_add formulation on the oracle's
    layout (CPU).  Gradients pass through bf16 roundings on the GPU path,
    hence the 2^-7 relative tolerance."""
    from combine_ep_dispatch_amd.autograd import EpDispatcher

    c = G.random_case(41, T=300, S=4, E_loc=6, K=4, H=256, A=8, shared=1, src=2, mask_p=0.1)
    cfg = G.epx.EpConfig(num_tokens=c.cfg.num_tokens, hidden=c.cfg.hidden, num_experts=c.cfg.num_experts,
                         num_segments=c.cfg.num_segments, top_k=c.cfg.top_k, align=c.cfg.align,
                         shared_expert=1, src_segment=2)
    d = EpDispatcher(cfg, G.DEV)
    T, H, K = cfg.num_tokens, cfg.hidden, cfg.top_k
    x = G.u16_tensor(c.x).view(T, H).clone().requires_grad_(True)
    probs = torch.from_numpy(c.probs).to(G.DEV).requires_grad_(True)
    ids = torch.from_numpy(c.ids).to(G.DEV)
    recv = d.dispatch(x, ids)
    expert_out = recv * 2.0
    y = d.combine(expert_out, probs)
    gy = G.u16_tensor(G.wl.make_tensor_like_rows(T, H, 9)).view(T, H)
    (y.float() * gy.float()).sum().backward()
    torch.cuda.synchronize()
    assert np.array_equal(d.layout.token_row.cpu().numpy(), c.L["token_row"])

    tr = torch.from_numpy(c.L["token_row"].astype(np.int64))
    xr = torch.from_numpy(G.f32(c.x).astype(np.float64)).requires_grad_(True)
    pr = torch.from_numpy(c.probs.astype(np.float64)).requires_grad_(True)
    yr = torch.zeros(T, H, dtype=torch.float64)
    for k in range(cfg.kp):
        ok = tr[:, k] >= 0
        w = pr[:, k] if k < K else torch.ones(T, dtype=torch.float64)
        yr = yr + torch.where(ok[:, None], w[:, None] * 2.0 * xr, torch.zeros(()))
    (yr * torch.from_numpy(G.f32(G.bits_of(gy)).reshape(T, H).astype(np.float64))).sum().backward()
    assert np.allclose(y.detach().float().cpu().numpy(), yr.detach().numpy(), rtol=2 ** -7, atol=1e-5)
    assert np.allclose(x.grad.float().cpu().numpy(), xr.grad.numpy(), rtol=2 ** -6, atol=1e-4)
    assert np.allclose(probs.grad.cpu().numpy(), pr.grad.numpy(), rtol=1e-3, atol=1e-3)


def test_autograd_backward_keeps_the_layout_of_its_forward(G):
    """Routing the next batch before this batch's backward must not change
    this batch's gradients: every forward node keeps the layout it ran with.
    The gradients with a second routing in between equal those without, bit
    for bit."""
    from combine_ep_dispatch_amd.autograd import EpDispatcher

    c = G.random_case(43, T=200, S=2, E_loc=8, K=4, H=128, A=4, shared=0, mask_p=0.05)
    other = G.random_case(44, T=200, S=2, E_loc=8, K=4, H=128, A=4, shared=0, mask_p=0.05)
    T, H = c.cfg.num_tokens, c.cfg.hidden

    def grads(reroute):
        cfg = G.epx.EpConfig(num_tokens=T, hidden=H, num_experts=c.cfg.num_experts,
                             num_segments=c.cfg.num_segments, top_k=c.cfg.top_k, align=c.cfg.align)
        d = EpDispatcher(cfg, G.DEV)
        x = G.u16_tensor(c.x).view(T, H).clone().requires_grad_(True)
        probs = torch.from_numpy(c.probs).to(G.DEV).requires_grad_(True)
        y = d.combine(d.dispatch(x, torch.from_numpy(c.ids).to(G.DEV)) * 2.0, probs)
        if reroute:
            d.route(torch.from_numpy(other.ids).to(G.DEV))
        gy = G.u16_tensor(G.wl.make_tensor_like_rows(T, H, 5)).view(T, H)
        (y.float() * gy.float()).sum().backward()
        torch.cuda.synchronize()
        return G.bits_of(x.grad), probs.grad.cpu().numpy().view(np.uint32)

    gx0, gp0 = grads(False)
    gx1, gp1 = grads(True)
    assert np.array_equal(gx0, gx1)
    assert np.array_equal(gp0, gp1)
