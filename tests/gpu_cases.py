"""Shared machinery of the GPU parity tests: run the HIP path (through the
C ABI, via the Python binding) and the CPU oracle on the same seeded inputs
and return both results as numpy arrays.

Every GPU output buffer is pre-filled with the sentinels the oracle uses for
"not written", so whole arrays are compared: a value the kernel should not
have written shows up as a mismatch too.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import combine_ep_dispatch_amd as epx
import oracle as orc
from combine_ep_dispatch_amd import workload as wl

DEV = torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ocfg(cfg: epx.EpConfig) -> "orc.Cfg":
    return orc.Cfg(T=cfg.num_tokens, H=cfg.hidden, E=cfg.num_experts, S=cfg.num_segments, K=cfg.top_k,
                   A=cfg.align, C=cfg.seg_capacity, shared=cfg.shared_expert, src_seg=cfg.src_segment,
                   recv_rows=cfg.recv_rows)


def cfg_of(w: wl.Workload, T=None, extra_rows=0, flags=0) -> epx.EpConfig:
    cfg = epx.EpConfig(num_tokens=w.T if T is None else T, hidden=w.H, num_experts=w.E,
                       num_segments=w.S, top_k=w.K, align=w.align, seg_capacity=w.capacity,
                       shared_expert=w.shared_expert, src_segment=w.src_segment, flags=flags)
    cfg.recv_rows = epx.ep_query(cfg).min_recv_rows + extra_rows
    return cfg


def i32_filled(n, dev=DEV):
    return torch.full((n,), int(orc.SENTINEL_I32), dtype=torch.int32, device=dev)


def sentinel_layout(cfg: epx.EpConfig) -> epx.Layout:
    S, G, R, T = cfg.num_segments, cfg.groups_per_segment, cfg.recv_rows, cfg.num_tokens
    f = lambda *shape: i32_filled(int(np.prod(shape))).view(*shape)  # noqa: E731
    return epx.Layout(f(S, G), f(S + 1), f(S, G + 1), f(S, G + 1), f(T, cfg.kp), f(R), f(R, 2), f(1))


# The layout paths a test can force (cfg.flags bits); 0 = the default choice.
LAYOUT_PATHS = {"single-pass": epx.EP_LAYOUT_LOOKBACK, "single-pass-barrier": epx.EP_LAYOUT_BARRIER,
                "two-kernel": epx.EP_LAYOUT_DIRECT, "count": epx.EP_LAYOUT_COUNT, "default": 0}
PATH_FLAGS = epx.EP_LAYOUT_LOOKBACK | epx.EP_LAYOUT_DIRECT | epx.EP_LAYOUT_BARRIER | epx.EP_LAYOUT_COUNT
COUNT_FORCED_MAX_SLOTS = 1 << 18  # routed slots EP_LAYOUT_COUNT accepts
BARRIER_FORCED_MAX_SLOTS = 1 << 20  # routed slots EP_LAYOUT_BARRIER accepts


def gpu_layout(cfg: epx.EpConfig, ids: np.ndarray, ws=None, path=None) -> epx.Layout:
    """Layout into sentinel-filled arrays; a fresh zeroed workspace unless one
    is given; `path` (a LAYOUT_PATHS key) overrides cfg's path bits."""
    saved = cfg.flags
    if path is not None:
        cfg.flags = (saved & ~PATH_FLAGS) | LAYOUT_PATHS[path]
    try:
        lay = sentinel_layout(cfg)
        if ws is None:
            ws = epx.workspace_for(cfg, DEV)
        ids_t = torch.from_numpy(np.ascontiguousarray(ids, np.int32).reshape(-1)).to(DEV)
        epx.ep_dispatch_layout(cfg, ids_t, ws, lay)
        torch.cuda.synchronize()
    finally:
        cfg.flags = saved
    return lay


def layout_np(lay: epx.Layout) -> dict:
    return {k: getattr(lay, k).cpu().numpy() for k in
            ("counts", "seg_base", "row_offsets", "scales_offsets", "token_row", "expert_ids",
             "src_info", "flags")}


def assert_layout_equal(g: dict, o: dict, name=""):
    for k in ("counts", "seg_base", "row_offsets", "scales_offsets", "token_row", "flags",
              "expert_ids", "src_info"):
        a, b = g[k].reshape(-1), o[k].reshape(-1)
        if not np.array_equal(a, b):
            bad = np.nonzero(a != b)[0]
            raise AssertionError(f"{name}: layout.{k} differs at {bad.size} places, first {bad[:8].tolist()}: "
                                 f"gpu {a[bad[:8]].tolist()} oracle {b[bad[:8]].tolist()}")


def u16_tensor(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).to(DEV).view(torch.bfloat16)


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_filled(rows, H, bits):
    return torch.full((rows * H,), int(np.int16(np.uint16(bits).view(np.int16))), dtype=torch.int16,
                      device=DEV).view(torch.bfloat16)


def f32(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def assert_bits_equal(gpu: np.ndarray, ora: np.ndarray, name: str):
    a, b = gpu.reshape(-1), ora.reshape(-1)
    if not np.array_equal(a, b):
        bad = np.nonzero(a != b)[0]
        raise AssertionError(f"{name}: {bad.size} of {a.size} differ, first at {bad[:6].tolist()}: "
                             f"gpu {a[bad[:6]].tolist()} oracle {b[bad[:6]].tolist()}")


def assert_close_bf16(gpu_bits: np.ndarray, ora_bits: np.ndarray, name: str):
    """The combine tolerance: |gpu - oracle| <= 1e-2 + 2e-2 |oracle| element-wise."""
    g = f32(gpu_bits).astype(np.float64).reshape(-1)
    o = f32(ora_bits).astype(np.float64).reshape(-1)
    err = np.abs(g - o)
    ok = err <= 1e-2 + 2e-2 * np.abs(o)
    if not ok.all():
        bad = np.nonzero(~ok)[0]
        raise AssertionError(f"{name}: {bad.size} elements outside tolerance, max err {err.max()}")


class Case:
    """Inputs of one parity case and the oracle's answers (computed lazily)."""

    def __init__(self, cfg: epx.EpConfig, ids, probs, x=None, seed=1):
        self.cfg, self.ids, self.probs, self.x, self.seed = cfg, ids, probs, x, seed
        self.oc = ocfg(cfg)
        self._L = None

    @property
    def L(self):
        if self._L is None:
            self._L = orc.layout(self.oc, self.ids)
        return self._L

    def rows(self, seed_offset, nan_pad=False):
        """Stand-in expert outputs / gradients for every receive row (bf16 bits)."""
        out = wl.make_tensor_like_rows(self.cfg.recv_rows, self.cfg.hidden, self.seed * 1000 + seed_offset)
        if nan_pad:
            used = np.zeros(self.cfg.recv_rows, bool)
            tr = self.L["token_row"]
            used[tr[tr >= 0]] = True
            out[~used] = np.uint16(0x7FC1)
        return out


def random_case(seed: int, **over) -> Case:
    rng = np.random.default_rng(seed)
    S = over.pop("S", int(rng.integers(1, 9)))
    E_loc = over.pop("E_loc", int(rng.integers(1, 33)))
    E = S * E_loc
    K = over.pop("K", int(rng.integers(1, min(E, 9) + 1)))
    T = over.pop("T", int(rng.integers(0, 700)))
    H = over.pop("H", int(rng.choice([16, 48, 128, 256, 528, 1040, 2064])))
    A = over.pop("A", int(rng.choice([1, 2, 4, 16, 128])))
    shared = over.pop("shared", int(rng.integers(0, 2)))
    src = over.pop("src", int(rng.integers(0, S)))
    mask_p = over.pop("mask_p", float(rng.choice([0.0, 0.05, 0.3])))
    bad_p = over.pop("bad_p", 0.0)
    distinct = over.pop("distinct", True)
    C = over.pop("C", 0)
    assert not over, over
    if distinct:
        ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]) if T else np.zeros((0, K), np.int64)
    else:
        ids = rng.integers(0, E, (T, K))
    ids = np.where(rng.random((T, K)) < mask_p, -1, ids)
    if bad_p > 0:
        ids = np.where(rng.random((T, K)) < bad_p, rng.choice([-9, -2, E, E + 3], (T, K)), ids)
    ids = ids.astype(np.int32)
    logits = rng.standard_normal((T, K))
    p = np.exp(logits - (logits.max(1, keepdims=True) if T else 0))
    probs = (p / (p.sum(1, keepdims=True) if T else 1)).astype(np.float32)
    x = wl.bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    cfg = epx.EpConfig(num_tokens=T, hidden=H, num_experts=E, num_segments=S, top_k=K, align=A,
                       seg_capacity=C, shared_expert=shared, src_segment=src if shared else 0)
    cfg.recv_rows = epx.ep_query(cfg).min_recv_rows
    return Case(cfg, ids, probs, x, seed)


def workload_case(name: str, T=None) -> Case:
    w = wl.CONFIGS[name]
    if T is not None:
        w = w.at_tokens(T)
    d = wl.make_workload(w)
    cfg = cfg_of(w)
    return Case(cfg, d["topk_ids"], d["probs"], d["x"], seed=7)


# --------------------------------------------------------------------------
# One parity check per hot-path step; each runs the GPU op and the oracle.
# --------------------------------------------------------------------------

def check_layout(c: Case, name: str) -> epx.Layout:
    say(f"[gpu] layout {name}: T={c.cfg.num_tokens} E={c.cfg.num_experts} S={c.cfg.num_segments} "
        f"K={c.cfg.top_k} A={c.cfg.align} C={c.cfg.seg_capacity} shared={c.cfg.shared_expert} "
        f"R={c.cfg.recv_rows}")
    # Every layout path (single pass, two kernels, count, and whichever the
    # size selects by default) must give the oracle's layout; the default
    # one is returned.  The count path takes at most 2^18 routed slots, the
    # single pass's barrier flavour 2^20.
    routed = c.cfg.num_tokens * c.cfg.top_k
    paths = ["single-pass", "two-kernel"]
    if routed <= BARRIER_FORCED_MAX_SLOTS:
        paths.append("single-pass-barrier")
    if routed <= COUNT_FORCED_MAX_SLOTS:
        paths.append("count")
    for path in paths:
        assert_layout_equal(layout_np(gpu_layout(c.cfg, c.ids, path=path)), c.L, f"{name} ({path})")
    lay = gpu_layout(c.cfg, c.ids)
    assert_layout_equal(layout_np(lay), c.L, name)
    return lay


def check_dispatch(c: Case, lay: epx.Layout, name: str):
    say(f"[gpu] dispatch {name}: H={c.cfg.hidden}")
    cfg = c.cfg
    recv = bf16_filled(cfg.recv_rows, cfg.hidden, orc.SENTINEL_U16)
    epx.ep_dispatch(cfg, lay, u16_tensor(c.x), recv)
    torch.cuda.synchronize()
    want = orc.dispatch(c.oc, c.L["token_row"], c.x)
    assert_bits_equal(bits_of(recv), want, f"{name}: recv")


def check_dispatch_with_layout(c: Case, name: str):
    """ep_dispatch_with_layout (one kernel for up to 512 routed slots, the
    layout launches and the scatter above) against the oracle's layout and
    dispatch, into sentinel-filled buffers."""
    say(f"[gpu] dispatch_with_layout {name}: T={c.cfg.num_tokens} K={c.cfg.top_k} H={c.cfg.hidden}")
    cfg = c.cfg
    lay = sentinel_layout(cfg)
    ws = epx.workspace_for(cfg, DEV)
    ids_t = torch.from_numpy(np.ascontiguousarray(c.ids, np.int32).reshape(-1)).to(DEV)
    recv = bf16_filled(cfg.recv_rows, cfg.hidden, orc.SENTINEL_U16)
    epx.ep_dispatch_with_layout(cfg, ids_t, ws, lay, u16_tensor(c.x), recv)
    torch.cuda.synchronize()
    assert_layout_equal(layout_np(lay), c.L, f"{name} (with layout)")
    assert_bits_equal(bits_of(recv), orc.dispatch(c.oc, c.L["token_row"], c.x), f"{name}: recv (with layout)")


def check_dispatch_nvfp4_with_layout(c: Case, name: str):
    """ep_dispatch_nvfp4_with_layout (one kernel for up to 512 routed slots,
    the layout launches and the NVFP4 dispatch above) against the oracle's
    layout and NVFP4 dispatch, into sentinel-filled buffers."""
    say(f"[gpu] dispatch_nvfp4_with_layout {name}: T={c.cfg.num_tokens} K={c.cfg.top_k} H={c.cfg.hidden}")
    cfg = c.cfg
    R, H = cfg.recv_rows, cfg.hidden
    lay = sentinel_layout(cfg)
    ws = epx.workspace_for(cfg, DEV)
    ids_t = torch.from_numpy(np.ascontiguousarray(c.ids, np.int32).reshape(-1)).to(DEV)
    codes = torch.full((R * H // 2,), int(orc.SENTINEL_U8), dtype=torch.uint8, device=DEV)
    scales = torch.full((R * H // 16,), int(orc.SENTINEL_U8), dtype=torch.uint8, device=DEV)
    rowscale = bf16_filled(R, 1, orc.SENTINEL_U16)
    epx.ep_dispatch_nvfp4_with_layout(cfg, ids_t, ws, lay, u16_tensor(c.x), codes, scales, rowscale)
    torch.cuda.synchronize()
    assert_layout_equal(layout_np(lay), c.L, f"{name} (nvfp4 with layout)")
    wc, wsc, wr = orc.dispatch_nvfp4(c.oc, c.L["token_row"], c.x)
    assert_bits_equal(codes.cpu().numpy(), wc, f"{name}: codes (with layout)")
    assert_bits_equal(scales.cpu().numpy(), wsc, f"{name}: scales (with layout)")
    assert_bits_equal(bits_of(rowscale), wr, f"{name}: rowscale (with layout)")


def check_nvfp4(c: Case, lay: epx.Layout, name: str, x=None):
    say(f"[gpu] nvfp4 {name}: H={c.cfg.hidden}")
    cfg = c.cfg
    x = c.x if x is None else x
    R, H = cfg.recv_rows, cfg.hidden
    codes = torch.full((R * H // 2,), int(orc.SENTINEL_U8), dtype=torch.uint8, device=DEV)
    scales = torch.full((R * H // 16,), int(orc.SENTINEL_U8), dtype=torch.uint8, device=DEV)
    rowscale = bf16_filled(R, 1, orc.SENTINEL_U16)
    epx.ep_dispatch_nvfp4(cfg, lay, u16_tensor(x), codes, scales, rowscale)
    torch.cuda.synchronize()
    wc, ws, wr = orc.dispatch_nvfp4(c.oc, c.L["token_row"], x)
    assert_bits_equal(codes.cpu().numpy(), wc, f"{name}: codes")
    assert_bits_equal(scales.cpu().numpy(), ws, f"{name}: scales")
    assert_bits_equal(bits_of(rowscale), wr, f"{name}: rowscale")


def check_combine(c: Case, lay: epx.Layout, name: str, weighted=True):
    say(f"[gpu] combine {name}: weighted={weighted}")
    cfg = c.cfg
    out = c.rows(1, nan_pad=True)
    probs = c.probs if weighted else None
    y = bf16_filled(cfg.num_tokens, cfg.hidden, orc.SENTINEL_U16)
    pt = None if probs is None else torch.from_numpy(probs.reshape(-1)).to(DEV)
    epx.ep_combine(cfg, lay, u16_tensor(out), pt, y)
    torch.cuda.synchronize()
    want = orc.combine(c.oc, c.L["token_row"], out, probs)
    got = bits_of(y)
    assert_close_bf16(got, want, f"{name}: combine")
    # same op order, no contraction: the kernel reproduces the oracle bit for bit
    assert_bits_equal(got, want, f"{name}: combine (bitwise)")


def check_dispatch_bwd(c: Case, lay: epx.Layout, name: str):
    say(f"[gpu] dispatch_bwd {name}")
    cfg = c.cfg
    g = c.rows(2, nan_pad=True)
    gx = bf16_filled(cfg.num_tokens, cfg.hidden, orc.SENTINEL_U16)
    epx.ep_dispatch_bwd(cfg, lay, u16_tensor(g), gx)
    torch.cuda.synchronize()
    want = orc.dispatch_bwd(c.oc, c.L["token_row"], g)
    got = bits_of(gx)
    assert_close_bf16(got, want, f"{name}: dispatch_bwd")
    assert_bits_equal(got, want, f"{name}: dispatch_bwd (bitwise)")


def check_combine_bwd(c: Case, lay: epx.Layout, name: str, weighted=True):
    say(f"[gpu] combine_bwd {name}: weighted={weighted}")
    cfg = c.cfg
    gy = wl.make_tensor_like_rows(cfg.num_tokens, cfg.hidden, c.seed * 1000 + 3)
    probs = c.probs if weighted else None
    go = bf16_filled(cfg.recv_rows, cfg.hidden, orc.SENTINEL_U16)
    pt = None if probs is None else torch.from_numpy(probs.reshape(-1)).to(DEV)
    epx.ep_combine_bwd(cfg, lay, u16_tensor(gy), pt, go)
    torch.cuda.synchronize()
    want = orc.combine_bwd(c.oc, c.L["token_row"], gy, probs)
    assert_bits_equal(bits_of(go), want, f"{name}: combine_bwd")


def check_probs_grad(c: Case, lay: epx.Layout, name: str):
    """grad_probs against the oracle's float64 dot products, within the bound
    of the kernel's fp32 summation: each thread adds 8*ceil(H/2048) products
    in order, then 6 butterfly levels and 4 wave partials, one product
    rounding each: (8*ceil(H/2048) + 10) * 2^-24 * sum |terms|."""
    say(f"[gpu] combine_bwd_probs {name}")
    cfg = c.cfg
    T, H, K = cfg.num_tokens, cfg.hidden, cfg.top_k
    gy = wl.make_tensor_like_rows(T, H, c.seed * 1000 + 3)
    out = c.rows(1, nan_pad=True)
    gp = torch.full((T * K,), float("nan"), dtype=torch.float32, device=DEV)
    epx.ep_combine_bwd_probs(cfg, lay, u16_tensor(gy), u16_tensor(out), gp)
    torch.cuda.synchronize()
    got = gp.cpu().numpy().reshape(T, K).astype(np.float64)
    gp2 = torch.full((T * K,), float("nan"), dtype=torch.float32, device=DEV)
    epx.ep_combine_bwd_probs(cfg, lay, u16_tensor(gy), u16_tensor(out), gp2)
    torch.cuda.synchronize()
    assert torch.equal(gp.view(torch.int32), gp2.view(torch.int32)), f"{name}: not deterministic"
    tr = c.L["token_row"]
    want = orc.combine_bwd_probs(c.oc, tr, gy, out)
    gyf = np.abs(f32(gy).reshape(T, H).astype(np.float64))
    mag = np.zeros((T, K))
    for k in range(K):
        ok = tr[:, k] >= 0
        if ok.any():
            mag[ok, k] = (gyf[ok] * np.abs(f32(out[tr[ok, k]]).astype(np.float64))).sum(1)
    bound = (8 * -(-H // 2048) + 10) * 2.0 ** -24 * mag + 1e-30
    err = np.abs(got - want)
    if not np.all(err <= bound):
        i = np.argmax(err - bound)
        raise AssertionError(f"{name}: grad_probs err {err.flat[i]} > bound {bound.flat[i]}")
    masked = tr[:, :K] < 0
    assert np.all(got[masked] == 0), f"{name}: masked slots not zero"


def check_fp8(c: Case, lay: epx.Layout, name: str, x=None):
    say(f"[gpu] fp8 {name}: H={c.cfg.hidden}")
    cfg = c.cfg
    x = c.x if x is None else x
    R, H = cfg.recv_rows, cfg.hidden
    codes = torch.full((R * H,), int(orc.SENTINEL_U8), dtype=torch.uint8, device=DEV)
    scales = torch.full((R * (H // 128),), int(np.int32(orc.SENTINEL_F32_BITS.view(np.int32))),
                        dtype=torch.int32, device=DEV).view(torch.float32)
    epx.ep_dispatch_fp8(cfg, lay, u16_tensor(x), codes, scales)
    torch.cuda.synchronize()
    wc, wsc = orc.dispatch_fp8(c.oc, c.L["token_row"], x)
    assert_bits_equal(codes.cpu().numpy(), wc, f"{name}: fp8 codes")
    assert_bits_equal(scales.view(torch.int32).cpu().numpy(), wsc.view(np.int32), f"{name}: fp8 scales")


def check_dispatch_fp8_with_layout(c: Case, name: str):
    """ep_dispatch_fp8_with_layout (one kernel for up to 512 routed slots, the
    layout launches and the FP8 dispatch above) against the oracle's layout
    and FP8 dispatch, into sentinel-filled buffers."""
    say(f"[gpu] dispatch_fp8_with_layout {name}: T={c.cfg.num_tokens} K={c.cfg.top_k} H={c.cfg.hidden}")
    cfg = c.cfg
    R, H = cfg.recv_rows, cfg.hidden
    lay = sentinel_layout(cfg)
    ws = epx.workspace_for(cfg, DEV)
    ids_t = torch.from_numpy(np.ascontiguousarray(c.ids, np.int32).reshape(-1)).to(DEV)
    codes = torch.full((R * H,), int(orc.SENTINEL_U8), dtype=torch.uint8, device=DEV)
    scales = torch.full((R * (H // 128),), int(np.int32(orc.SENTINEL_F32_BITS.view(np.int32))),
                        dtype=torch.int32, device=DEV).view(torch.float32)
    epx.ep_dispatch_fp8_with_layout(cfg, ids_t, ws, lay, u16_tensor(c.x), codes, scales)
    torch.cuda.synchronize()
    assert_layout_equal(layout_np(lay), c.L, f"{name} (fp8 with layout)")
    wc, wsc = orc.dispatch_fp8(c.oc, c.L["token_row"], c.x)
    assert_bits_equal(codes.cpu().numpy(), wc, f"{name}: fp8 codes (with layout)")
    assert_bits_equal(scales.view(torch.int32).cpu().numpy(), wsc.view(np.int32), f"{name}: fp8 scales (with layout)")


def nvfp4_rows(c: Case, seed_offset: int):
    """Stand-in NVFP4 expert outputs for every receive row: random codes,
    E4M3 scales (some negative) and bf16 rowscales over 2^-40..2^40.  Rows no
    kept slot uses are poisoned (codes 0x77, scale 0x7E, rowscale 2^100), so
    a read of them shows up in the result."""
    rng = np.random.default_rng(c.seed * 1000 + seed_offset)
    R, H = c.cfg.recv_rows, c.cfg.hidden
    codes = rng.integers(0, 256, (R, H // 2), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (R, H // 16), dtype=np.uint8)
    scales[rng.random((R, H // 16)) < 0.05] |= 0x80
    rs = wl.bf16_bits(np.exp2(rng.uniform(-40, 40, R)).astype(np.float32))
    used = np.zeros(R, bool)
    tr = c.L["token_row"]
    used[tr[tr >= 0]] = True
    codes[~used] = 0x77
    scales[~used] = 0x7E
    rs[~used] = wl.bf16_bits(np.array([2.0 ** 100], np.float32))[0]
    return codes, scales, rs


def check_combine_nvfp4(c: Case, lay: epx.Layout, name: str, weighted=True, rows=None):
    """ep_combine_nvfp4 against the oracle, bit for bit (same op order, no
    contraction); `rows` = (codes, scales, rowscale bits), random by default."""
    say(f"[gpu] combine_nvfp4 {name}: weighted={weighted}")
    cfg = c.cfg
    codes, scales, rs = nvfp4_rows(c, 4) if rows is None else rows
    probs = c.probs if weighted else None
    y = bf16_filled(cfg.num_tokens, cfg.hidden, orc.SENTINEL_U16)
    pt = None if probs is None else torch.from_numpy(probs.reshape(-1)).to(DEV)
    epx.ep_combine_nvfp4(cfg, lay, torch.from_numpy(codes.reshape(-1)).to(DEV),
                         torch.from_numpy(scales.reshape(-1)).to(DEV), u16_tensor(rs.reshape(-1)), pt, y)
    torch.cuda.synchronize()
    want = orc.combine_nvfp4(c.oc, c.L["token_row"], codes, scales, rs, probs)
    got = bits_of(y)
    assert_close_bf16(got, want, f"{name}: combine_nvfp4")
    assert_bits_equal(got, want, f"{name}: combine_nvfp4 (bitwise)")
