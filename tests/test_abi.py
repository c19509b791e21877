"""The C ABI on the host (no GPU needed): the library loads, exports every
symbol include/epx.h declares, sizes buffers as documented and rejects every
host-checkable invalid argument with EP_EINVAL before touching the device.

No call here reaches a kernel launch: each one fails validation first.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def layout_tiles(routed, ng):
    """Layout tiles: 256 threads x spt slots.  spt is 1 when every lane of
    the direct column sums then covers its tiles in one 64-load batch (at
    most 256 tiles), else the smallest of 2, 4, 8 giving at most 256 tiles,
    else 8."""
    lanes = 1
    while lanes < 64 and ng * lanes * 2 <= 256:
        lanes *= 2

    def tiles_at(spt):
        return max(1, -(-routed // (256 * spt)))

    if tiles_at(1) <= min(256, 64 * lanes):
        return tiles_at(1)
    for spt in (2, 4):
        if tiles_at(spt) <= 256:
            return tiles_at(spt)
    return tiles_at(8)


def sp_tiles(routed):
    """Single-pass layout tiles: 256 x spt slots, spt the smallest of 1, 2,
    4, 8 giving at most 32 tiles (else 8)."""
    for spt in (1, 2, 4):
        if routed <= 256 * spt * 32:
            return max(1, -(-routed // (256 * spt)))
    return max(1, -(-routed // (256 * 8)))


def workspace_bytes(routed, ng):
    """A 256-byte header, then the larger of the two paths' tables: 32-bit
    tile counts plus, past 256 tiles, 32-bit sums of each chunk of 256 tiles
    (two-kernel path), or two arrays of 64-bit descriptors (single pass)."""
    tiles = layout_tiles(routed, ng)
    chunks = 0 if tiles <= 256 else -(-tiles // 256)
    return 256 + max((tiles + chunks) * ng * 4, sp_tiles(routed) * ng * 16)


def test_layout_tiles_rule():
    # DeepSeek-V3 share (256 groups): one lane per group, 64 tiles per batch
    assert layout_tiles(4096 * 8, 256) == 64          # 2 slots per thread (1 would need 2 batches)
    assert layout_tiles(1024 * 8, 256) == 32          # 1 slot per thread
    assert layout_tiles(16384 * 6, 68) == 192         # 2 slots per thread, 2 batches of 2 lanes
    assert layout_tiles(4096 * 6, 68) == 96           # 1 slot per thread, 2 lanes per group
    assert layout_tiles(70001 * 8, 64) == 274         # past one chunk of 256 tiles: two chunks
    assert layout_tiles(0, 8) == 1


@pytest.fixture(scope="module")
def L():
    from combine_ep_dispatch_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from combine_ep_dispatch_amd import build

        build.build()
    return _lib.lib()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "epx.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    from combine_ep_dispatch_amd import _lib

    names = declared_functions()
    assert set(names) == set(_lib.SYMBOLS), names
    for n in names:
        assert hasattr(L, n), n
    assert L.ep_abi_version() == 1
    assert L.ep_strerror(-1) == b"invalid argument"
    assert L.ep_strerror(0) == b"ok"
    assert b"ep_dispatch_layout_noalloc" in L.ep_strerror(-4)


def test_noalloc_layout_rejects_oversized_problems_before_any_launch(L):
    """The built-in scratch of ep_dispatch_layout_noalloc holds
    EP_NOALLOC_SCRATCH_BYTES; a configuration whose workspace_bytes exceeds
    it gets EP_ESCRATCH (-4) before anything is enqueued, and argument errors
    keep EP_EINVAL."""
    from combine_ep_dispatch_amd._lib import EP_NOALLOC_SCRATCH_BYTES, EpLayout

    fake = 0x10000  # never dereferenced: every call below fails validation first
    lay = EpLayout(*([fake] * 8))
    big = cfg(num_tokens=1 << 21, num_experts=2048, num_segments=8, top_k=8, align=1)
    st, rows, ws, _ = query(L, big)
    assert st == 0 and ws > EP_NOALLOC_SCRATCH_BYTES
    big.recv_rows = rows
    cc = big.to_c()
    assert L.ep_dispatch_layout_noalloc(ctypes.byref(cc), fake, ctypes.byref(lay), None) == -4
    bad = cfg(num_tokens=-1).to_c()
    assert L.ep_dispatch_layout_noalloc(ctypes.byref(bad), fake, ctypes.byref(lay), None) == -1
    small = cfg()
    st, rows, ws, _ = query(L, small)
    assert ws <= EP_NOALLOC_SCRATCH_BYTES
    small.recv_rows = rows - 1
    cs = small.to_c()
    assert L.ep_dispatch_layout_noalloc(ctypes.byref(cs), fake, ctypes.byref(lay), None) == -1
    small.recv_rows = rows
    cs = small.to_c()
    assert L.ep_dispatch_layout_noalloc(ctypes.byref(cs), None, ctypes.byref(lay), None) == -1
    assert L.ep_dispatch_layout_noalloc(ctypes.byref(cs), fake, None, None) == -1


def test_header_and_binding_structs_agree():
    from combine_ep_dispatch_amd._lib import EpCfg, EpLayout

    assert ctypes.sizeof(EpCfg) == 10 * 4 + 8 + 2 * 4
    assert EpCfg.recv_rows.offset == 40
    assert ctypes.sizeof(EpLayout) == 8 * 8


def cfg(**kw):
    from combine_ep_dispatch_amd import EpConfig

    base = dict(num_tokens=128, hidden=256, num_experts=8, num_segments=2, top_k=2, align=16)
    base.update(kw)
    return EpConfig(**base)


def query(L, c):
    from combine_ep_dispatch_amd._lib import EpCfg  # noqa: F401

    rows, ws, g = ctypes.c_int64(-1), ctypes.c_int64(-1), ctypes.c_int32(-1)
    cc = c.to_c()
    st = L.ep_query(ctypes.byref(cc), ctypes.byref(rows), ctypes.byref(ws), ctypes.byref(g))
    return st, rows.value, ws.value, g.value


def test_query_sizes(L, orc):
    import numpy as np

    for kw in [dict(), dict(align=1), dict(shared_expert=1, src_segment=1),
               dict(seg_capacity=100), dict(num_tokens=0), dict(num_tokens=4096, hidden=7168,
               num_experts=256, num_segments=8, top_k=8, align=128),
               # past 256 two-kernel tiles (chunk sums) and at the 2^24-slot layout limit
               dict(num_tokens=70_000, num_experts=64, num_segments=4, top_k=8, align=16),
               dict(num_tokens=1 << 21, num_experts=256, num_segments=8, top_k=8, align=128, shared_expert=1)]:
        c = cfg(**kw)
        st, rows, ws, g = query(L, c)
        assert st == 0
        oc = orc.Cfg(T=c.num_tokens, H=c.hidden, E=c.num_experts, S=c.num_segments, K=c.top_k,
                     A=c.align, C=c.seg_capacity, shared=c.shared_expert, src_seg=c.src_segment)
        assert rows == orc.min_recv_rows(oc)
        assert g == c.num_experts // c.num_segments + c.shared_expert
        routed = c.num_tokens * c.top_k
        ng = c.num_segments * g
        assert ws == workspace_bytes(routed, ng)
    # the bound is reached by some routing and never exceeded (oracle layout)
    rng = np.random.default_rng(0)
    c = cfg(num_tokens=9, num_experts=12, num_segments=3, top_k=3, align=5, shared_expert=1)
    _, rows, _, _ = query(L, c)
    oc = orc.Cfg(T=9, H=8, E=12, S=3, K=3, A=5, shared=1, recv_rows=rows)
    for _ in range(50):
        ids = np.stack([rng.permutation(12)[:3] for _ in range(9)]).astype(np.int32)
        assert orc.layout(oc, ids)["seg_base"][-1] <= rows


INVALID = [
    dict(num_tokens=-1), dict(hidden=0), dict(hidden=12), dict(num_experts=0), dict(num_segments=0),
    dict(num_experts=9), dict(top_k=0), dict(top_k=9), dict(align=0), dict(seg_capacity=-1),
    dict(shared_expert=2), dict(shared_expert=1, src_segment=2), dict(shared_expert=1, src_segment=-1),
    dict(flags=6), dict(flags=7), dict(flags=10), dict(flags=12), dict(flags=14), dict(flags=18), dict(flags=20),
    dict(flags=24), dict(flags=32),
    dict(flags=16, num_tokens=(1 << 15) + 1, top_k=8),  # forced count path past 2^18 routed slots
    dict(num_experts=4096, num_segments=2),  # > EP_MAX_GROUPS groups
    dict(num_tokens=1 << 28, top_k=4),  # 2^30 slots
    # capacity mode: the unclamped aligned offsets (summed in int32 before the
    # clamp to C) would reach 2^31 although S * C is small
    dict(num_tokens=4, num_experts=4, num_segments=1, top_k=4, align=1 << 30, seg_capacity=100),
    dict(num_tokens=64, num_experts=8, num_segments=2, top_k=2, align=1 << 28, seg_capacity=1000),
]


@pytest.mark.parametrize("kw", INVALID, ids=[str(k) for k in INVALID])
def test_query_rejects_invalid_config(L, kw):
    assert query(L, cfg(**kw))[0] == -1


@pytest.mark.parametrize("flags", [0, 1, 2, 3, 4, 5, 8, 9, 16, 17])
def test_query_accepts_documented_flags(L, flags):
    """EP_ZERO_PAD_ROWS (1) with at most one of the layout path bits
    EP_LAYOUT_LOOKBACK (2), EP_LAYOUT_DIRECT (4), EP_LAYOUT_BARRIER (8),
    EP_LAYOUT_COUNT (16)."""
    from combine_ep_dispatch_amd import (EP_LAYOUT_BARRIER, EP_LAYOUT_COUNT, EP_LAYOUT_DIRECT, EP_LAYOUT_LOOKBACK,
                                         EP_ZERO_PAD_ROWS)

    assert (EP_ZERO_PAD_ROWS, EP_LAYOUT_LOOKBACK, EP_LAYOUT_DIRECT, EP_LAYOUT_BARRIER, EP_LAYOUT_COUNT) == (1, 2, 4, 8, 16)
    assert query(L, cfg(flags=flags))[0] == 0


def test_forced_count_path_bound(L):
    """EP_LAYOUT_COUNT takes at most 2^18 routed slots (its cost grows with
    the square of the batch); the default choice has no such bound."""
    assert query(L, cfg(flags=16, num_tokens=1 << 15, top_k=8))[0] == 0
    assert query(L, cfg(flags=16, num_tokens=(1 << 15) + 1, top_k=8))[0] == -1
    assert query(L, cfg(flags=0, num_tokens=(1 << 15) + 1, top_k=8))[0] == 0


def test_layout_rejects_more_than_2_24_routed_slots(L):
    """A layout call takes at most 2^24 routed slots (T*K); ep_query and the
    movers take larger batches.  Only batches past the limit are passed: at
    or below it these fake pointers would reach a launch."""
    from combine_ep_dispatch_amd._lib import EpLayout

    fake = 0x10000
    lay = EpLayout(*([fake] * 8))
    for T, K in (((1 << 21) + 1, 8), ((1 << 24) + 1, 1), (1 << 20, 17)):
        c = cfg(num_tokens=T, top_k=K, num_experts=64, num_segments=8, hidden=256)
        st, rows, ws, _ = query(L, c)
        assert st == 0 and T * K > 1 << 24
        c.recv_rows = rows
        cc = c.to_c()
        assert L.ep_dispatch_layout(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), None) == -1
        assert L.ep_dispatch_layout_noalloc(ctypes.byref(cc), fake, ctypes.byref(lay), None) == -1


def test_forced_barrier_path_bound(L):
    """EP_LAYOUT_BARRIER takes at most 2^20 routed slots (every workgroup
    reads every tile's counts); the look-back and the default have no such
    bound below the 2^24-slot layout limit."""
    big = dict(num_tokens=(1 << 17) + 1, top_k=8, num_experts=64, num_segments=8)
    assert query(L, cfg(flags=8, num_tokens=1 << 17, top_k=8, num_experts=64, num_segments=8))[0] == 0
    assert query(L, cfg(flags=8, **big))[0] == -1
    assert query(L, cfg(flags=2, **big))[0] == 0
    assert query(L, cfg(flags=0, **big))[0] == 0


def test_null_config_and_reserved_fields(L):
    assert L.ep_query(None, None, None, None) == -1
    c = cfg().to_c()
    c.reserved0 = 1
    assert L.ep_query(ctypes.byref(c), None, None, None) == -1
    c = cfg().to_c()
    c.reserved1 = 7
    assert L.ep_query(ctypes.byref(c), None, None, None) == -1


def test_calls_reject_bad_arguments_before_any_launch(L):
    from combine_ep_dispatch_amd._lib import EpLayout

    c = cfg()
    st, rows, ws, g = query(L, c)
    fake = 0x10000  # never dereferenced: every call below fails validation first
    lay = EpLayout(*([fake] * 8))
    # recv_rows below the bound
    c.recv_rows = rows - 1
    cc = c.to_c()
    assert L.ep_dispatch_layout(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), None) == -1
    assert L.ep_dispatch(ctypes.byref(cc), ctypes.byref(lay), fake, fake, None) == -1
    assert L.ep_combine(ctypes.byref(cc), ctypes.byref(lay), fake, None, fake, None) == -1
    assert L.ep_dispatch_bwd(ctypes.byref(cc), ctypes.byref(lay), fake, fake, None) == -1
    assert L.ep_combine_bwd(ctypes.byref(cc), ctypes.byref(lay), fake, None, fake, None) == -1
    assert L.ep_dispatch_nvfp4(ctypes.byref(cc), ctypes.byref(lay), fake, fake, fake, fake, None) == -1
    c.recv_rows = rows
    cc = c.to_c()
    # workspace too small / misaligned / missing
    assert L.ep_dispatch_layout(ctypes.byref(cc), fake, fake, ws - 1, ctypes.byref(lay), None) == -1
    assert L.ep_dispatch_layout(ctypes.byref(cc), fake, fake + 4, ws, ctypes.byref(lay), None) == -1
    assert L.ep_dispatch_layout(ctypes.byref(cc), fake, None, ws, ctypes.byref(lay), None) == -1
    # missing or misaligned buffers
    assert L.ep_dispatch_layout(ctypes.byref(cc), None, fake, ws, ctypes.byref(lay), None) == -1
    assert L.ep_dispatch_layout(ctypes.byref(cc), fake, fake, ws, None, None) == -1
    for field in ("counts", "seg_base", "row_offsets", "scales_offsets", "token_row", "expert_ids",
                  "src_info", "flags"):
        bad = EpLayout(*([fake] * 8))
        setattr(bad, field, None)
        assert L.ep_dispatch_layout(ctypes.byref(cc), fake, fake, ws, ctypes.byref(bad), None) == -1, field
        setattr(bad, field, fake + 2)
        assert L.ep_dispatch_layout(ctypes.byref(cc), fake, fake, ws, ctypes.byref(bad), None) == -1, field
    assert L.ep_dispatch(ctypes.byref(cc), ctypes.byref(lay), fake + 8, fake, None) == -1
    assert L.ep_dispatch(ctypes.byref(cc), ctypes.byref(lay), fake, None, None) == -1
    assert L.ep_dispatch(ctypes.byref(cc), None, fake, fake, None) == -1
    assert L.ep_combine(ctypes.byref(cc), ctypes.byref(lay), fake, fake + 2, fake, None) == -1
    assert L.ep_combine_bwd(ctypes.byref(cc), ctypes.byref(lay), fake, fake + 1, fake, None) == -1
    assert L.ep_dispatch_bwd(ctypes.byref(cc), ctypes.byref(lay), None, fake, None) == -1
    # NVFP4 needs H % 16 == 0 and H <= 16384
    c24 = cfg(hidden=24)
    c24.recv_rows = rows
    cc = c24.to_c()
    assert L.ep_dispatch_nvfp4(ctypes.byref(cc), ctypes.byref(lay), fake, fake, fake, fake, None) == -1
    cbig = cfg(hidden=16384 + 16)
    cbig.recv_rows = rows
    cc = cbig.to_c()
    assert L.ep_dispatch_nvfp4(ctypes.byref(cc), ctypes.byref(lay), fake, fake, fake, fake, None) == -1


def test_dispatch_with_layout_rejects_bad_arguments_before_any_launch(L):
    from combine_ep_dispatch_amd._lib import EpLayout

    c = cfg()
    st, rows, ws, g = query(L, c)
    fake = 0x10000  # never dereferenced: every call below fails validation first
    lay = EpLayout(*([fake] * 8))
    c.recv_rows = rows - 1
    cc = c.to_c()
    assert L.ep_dispatch_with_layout(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake, fake, None) == -1
    c.recv_rows = rows
    cc = c.to_c()
    assert L.ep_dispatch_with_layout(ctypes.byref(cc), fake, fake, ws - 1, ctypes.byref(lay), fake, fake, None) == -1
    assert L.ep_dispatch_with_layout(ctypes.byref(cc), fake, None, ws, ctypes.byref(lay), fake, fake, None) == -1
    assert L.ep_dispatch_with_layout(ctypes.byref(cc), None, fake, ws, ctypes.byref(lay), fake, fake, None) == -1
    assert L.ep_dispatch_with_layout(ctypes.byref(cc), fake, fake, ws, None, fake, fake, None) == -1
    assert L.ep_dispatch_with_layout(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake + 8, fake, None) == -1
    assert L.ep_dispatch_with_layout(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake, None, None) == -1
    assert L.ep_dispatch_with_layout(None, fake, fake, ws, ctypes.byref(lay), fake, fake, None) == -1


def test_dispatch_nvfp4_with_layout_rejects_bad_arguments_before_any_launch(L):
    from combine_ep_dispatch_amd._lib import EpLayout

    c = cfg()
    st, rows, ws, g = query(L, c)
    fake = 0x10000  # never dereferenced: every call below fails validation first
    lay = EpLayout(*([fake] * 8))
    cc = c.to_c()
    f = L.ep_dispatch_nvfp4_with_layout
    assert f(ctypes.byref(cc), fake, fake, ws - 1, ctypes.byref(lay), fake, fake, fake, fake, None) == -1
    assert f(ctypes.byref(cc), fake, fake, ws, None, fake, fake, fake, fake, None) == -1
    assert f(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake + 8, fake, fake, fake, None) == -1  # x
    assert f(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake, fake + 8, fake, fake, None) == -1  # codes
    assert f(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake, fake, None, fake, None) == -1
    assert f(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake, fake, fake, fake + 1, None) == -1
    for H in (24, 16384 + 16):  # not a whole number of 16-element blocks; past the NVFP4 row limit
        c2 = cfg()
        c2.hidden = H
        c2.recv_rows = rows
        cc2 = c2.to_c()
        assert f(ctypes.byref(cc2), fake, fake, ws, ctypes.byref(lay), fake, fake, fake, fake, None) == -1


def test_dispatch_fp8_with_layout_rejects_bad_arguments_before_any_launch(L):
    from combine_ep_dispatch_amd._lib import EpLayout

    fake = 0x10000  # never dereferenced: every call below fails validation first
    lay = EpLayout(*([fake] * 8))
    f = L.ep_dispatch_fp8_with_layout
    c = cfg()
    c.hidden = 256
    st, rows, ws, g = query(L, c)
    c.recv_rows = rows
    cc = c.to_c()
    assert f(ctypes.byref(cc), fake, fake, ws - 1, ctypes.byref(lay), fake, fake, fake, None) == -1
    assert f(ctypes.byref(cc), fake, fake, ws, None, fake, fake, fake, None) == -1
    assert f(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake + 8, fake, fake, None) == -1  # x
    assert f(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake, fake + 8, fake, None) == -1  # codes
    assert f(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake, fake, fake + 2, None) == -1  # scales
    assert f(ctypes.byref(cc), fake, fake, ws, ctypes.byref(lay), fake, fake, None, None) == -1
    for H in (192, 16384 + 128):  # not whole 128-element blocks; past the FP8 row limit
        c2 = cfg()
        c2.hidden = H
        c2.recv_rows = rows
        cc2 = c2.to_c()
        assert f(ctypes.byref(cc2), fake, fake, ws, ctypes.byref(lay), fake, fake, fake, None) == -1


def test_binding_rejects_cpu_tensors():
    import torch

    import combine_ep_dispatch_amd as epx

    c = cfg()
    c.recv_rows = epx.ep_query(c).min_recv_rows
    with pytest.raises(ValueError):
        epx.ep_dispatch_layout(c, torch.zeros(c.num_tokens * c.top_k, dtype=torch.int32),
                               torch.zeros(64, dtype=torch.uint8), None)


def test_product_package_does_not_touch_the_oracle():
    pkg = os.path.join(ROOT, "combine_ep_dispatch_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "liboracle" not in text, f


def test_new_entry_points_reject_bad_arguments(L):
    from combine_ep_dispatch_amd._lib import EpLayout

    c = cfg(hidden=256)
    st, rows, ws, g = query(L, c)
    fake = 0x10000  # never dereferenced: every call below fails validation first
    lay = EpLayout(*([fake] * 8))
    c.recv_rows = rows
    cc = c.to_c()
    # combine_bwd_probs: missing / misaligned buffers, too few rows
    assert L.ep_combine_bwd_probs(ctypes.byref(cc), ctypes.byref(lay), fake, fake, None, None) == -1
    assert L.ep_combine_bwd_probs(ctypes.byref(cc), ctypes.byref(lay), fake + 2, fake, fake, None) == -1
    assert L.ep_combine_bwd_probs(ctypes.byref(cc), ctypes.byref(lay), fake, fake, fake + 2, None) == -1
    assert L.ep_combine_bwd_probs(ctypes.byref(cc), None, fake, fake, fake, None) == -1
    # fp8 dispatch: H must be a multiple of 128 and at most 16384
    assert L.ep_dispatch_fp8(ctypes.byref(cc), ctypes.byref(lay), fake, fake, None, None) == -1
    assert L.ep_dispatch_fp8(ctypes.byref(cc), ctypes.byref(lay), fake, fake + 8, fake, None) == -1
    for h in (192, 16384 + 128):
        ch = cfg(hidden=h)
        ch.recv_rows = rows
        cch = ch.to_c()
        assert L.ep_dispatch_fp8(ctypes.byref(cch), ctypes.byref(lay), fake, fake, fake, None) == -1
    short = cfg(hidden=256)
    short.recv_rows = rows - 1
    cs = short.to_c()
    assert L.ep_dispatch_fp8(ctypes.byref(cs), ctypes.byref(lay), fake, fake, fake, None) == -1
    assert L.ep_combine_bwd_probs(ctypes.byref(cs), ctypes.byref(lay), fake, fake, fake, None) == -1
    # combine over NVFP4 rows: H % 16, 8-byte aligned codes, buffers present, enough rows
    assert L.ep_combine_nvfp4(ctypes.byref(cc), ctypes.byref(lay), fake + 4, fake, fake, None, fake, None) == -1
    assert L.ep_combine_nvfp4(ctypes.byref(cc), ctypes.byref(lay), fake, None, fake, None, fake, None) == -1
    assert L.ep_combine_nvfp4(ctypes.byref(cc), ctypes.byref(lay), fake, fake, fake + 1, None, fake, None) == -1
    assert L.ep_combine_nvfp4(ctypes.byref(cc), ctypes.byref(lay), fake, fake, fake, fake + 2, fake, None) == -1
    assert L.ep_combine_nvfp4(ctypes.byref(cc), ctypes.byref(lay), fake, fake, fake, None, fake + 8, None) == -1
    assert L.ep_combine_nvfp4(ctypes.byref(cc), None, fake, fake, fake, None, fake, None) == -1
    assert L.ep_combine_nvfp4(ctypes.byref(cs), ctypes.byref(lay), fake, fake, fake, None, fake, None) == -1
    c24 = cfg(hidden=24)
    c24.recv_rows = rows
    cc24 = c24.to_c()
    assert L.ep_combine_nvfp4(ctypes.byref(cc24), ctypes.byref(lay), fake, fake, fake, None, fake, None) == -1
    # routing-map conversions: dense probabilities need compact ones and vice versa
    assert L.ep_indices_to_multihot(ctypes.byref(cc), None, None, fake, None, None) == -1
    assert L.ep_indices_to_multihot(ctypes.byref(cc), fake, None, None, None, None) == -1
    assert L.ep_indices_to_multihot(ctypes.byref(cc), fake, None, fake, fake, None) == -1
    assert L.ep_indices_to_multihot(ctypes.byref(cc), fake + 1, fake, fake, fake, None) == -1
    assert L.ep_multihot_to_indices(ctypes.byref(cc), None, None, fake, None, None, None) == -1
    assert L.ep_multihot_to_indices(ctypes.byref(cc), fake, None, fake, fake, None, None) == -1
    assert L.ep_multihot_to_indices(ctypes.byref(cc), fake, fake, fake, fake, fake + 2, None) == -1
    assert L.ep_multihot_to_indices(None, fake, fake, fake, fake, None, None) == -1


def test_single_grid_calls_reject_batches_past_the_grid_limit(L):
    """A HIP grid dimension holds at most 2^32 - 1 work-items.  The calls that
    launch one grid per batch reject a batch whose grid would not fit: one
    wave per token for the quantizing dispatches and the routing-map
    conversions (T >= 2^26 - 16), one 256-thread workgroup per token for the
    probability gradient (T >= 2^24 - 4).  The configurations themselves are
    valid (ep_query accepts them), so the grid rule is what rejects them.
    Only batches at the limit are passed: below it these fake pointers would
    reach a launch."""
    from combine_ep_dispatch_amd._lib import EpLayout

    fake = 0x10000
    lay = EpLayout(*([fake] * 8))
    for T, calls in ((2 ** 26 - 16, ("nvfp4", "fp8", "to_multihot", "to_indices")), (2 ** 24 - 4, ("probs",))):
        c = cfg(num_tokens=T, hidden=256, align=1)
        st, rows, _, _ = query(L, c)
        assert st == 0
        c.recv_rows = rows
        cc = c.to_c()
        for name in calls:
            if name == "nvfp4":
                rc = L.ep_dispatch_nvfp4(ctypes.byref(cc), ctypes.byref(lay), fake, fake, fake, fake, None)
            elif name == "fp8":
                rc = L.ep_dispatch_fp8(ctypes.byref(cc), ctypes.byref(lay), fake, fake, fake, None)
            elif name == "to_multihot":
                rc = L.ep_indices_to_multihot(ctypes.byref(cc), fake, None, fake, None, None)
            elif name == "to_indices":
                rc = L.ep_multihot_to_indices(ctypes.byref(cc), fake, None, fake, None, None, None)
            else:
                rc = L.ep_combine_bwd_probs(ctypes.byref(cc), ctypes.byref(lay), fake, fake, fake, None)
            assert rc == -1, (name, T)
