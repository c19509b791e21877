"""Guard bands and determinism for every entry point, through the C ABI.

Each output buffer is a slice of a larger allocation whose head and tail
(1024 elements each) hold a sentinel: after the call the guards must be
untouched, so no kernel writes before or past its buffer.  Every op is run
twice, each time into fresh sentinel-filled buffers, and must give the same
bytes (rows a call leaves unwritten keep the sentinel both times)."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

GUARD = 1024  # elements; keeps 16-byte alignment for every dtype used here
FILL = {torch.uint8: np.uint8(0xA5), torch.int32: np.uint32(0xA5A5A5A5),
        torch.float32: np.uint32(0x7FA5A5A5), torch.bfloat16: np.uint16(0x7FA5)}


@pytest.fixture(scope="module")
def G():
    import gpu_cases as gc

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return gc


class Guarded:
    """A device buffer of n elements between two sentinel-filled guards."""

    def __init__(self, n, dtype):
        self.n = n
        self.full = torch.empty(n + 2 * GUARD, dtype=dtype, device="cuda:0")
        bits = FILL[dtype]
        if dtype == torch.uint8:
            self.full.fill_(int(bits))
        elif dtype == torch.bfloat16:
            self.full.view(torch.int16).fill_(int(bits.view(np.int16)))
        else:
            self.full.view(torch.int32).fill_(int(bits.view(np.int32)))
        self.guard_bytes = self.full[:GUARD].view(torch.uint8).clone()
        self.view = self.full[GUARD:GUARD + n]

    def check(self, name):
        assert torch.equal(self.full[:GUARD].view(torch.uint8), self.guard_bytes), f"{name}: write before the buffer"
        assert torch.equal(self.full[GUARD + self.n:].view(torch.uint8), self.guard_bytes), \
            f"{name}: write past the buffer"
        return self.view.contiguous().view(torch.uint8).cpu().numpy().copy()


CASES = [
    dict(T=700, S=4, E_loc=8, K=4, H=528, A=8, shared=1, src=2, mask_p=0.1, bad_p=0.02),  # ragged H, shared
    dict(T=400, S=4, E_loc=4, K=4, H=256, A=4, shared=1, src=1, C=40),                    # capacity drops
    dict(T=3000, S=8, E_loc=16, K=8, H=1024, A=16),                                        # direct layout path
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_guards_and_determinism(G, case):
    c = G.random_case(100 + case, **dict(CASES[case]))
    cfg = c.cfg
    T, H, R, K, E = cfg.num_tokens, cfg.hidden, cfg.recv_rows, cfg.top_k, cfg.num_experts
    S, Gs = cfg.num_segments, cfg.groups_per_segment
    G.say(f"[gpu] guards case {case}: T={T} H={H} R={R} K={K} shared={cfg.shared_expert} C={cfg.seg_capacity}")
    ids = torch.from_numpy(np.ascontiguousarray(c.ids, np.int32).reshape(-1)).to(G.DEV)
    probs = torch.from_numpy(np.ascontiguousarray(c.probs, np.float32).reshape(-1)).to(G.DEV)
    x = G.u16_tensor(c.x).view(-1)
    out = G.u16_tensor(c.rows(1)).view(-1)
    gy = G.u16_tensor(G.wl.make_tensor_like_rows(T, H, c.seed * 1000 + 3)).view(-1)
    rm_np, dp_np = G.orc.indices_to_multihot(c.oc, c.ids, c.probs)
    cq_np, sq_np, rq_np = G.nvfp4_rows(c, 4)
    cq = torch.from_numpy(cq_np.reshape(-1)).to(G.DEV)
    sq = torch.from_numpy(sq_np.reshape(-1)).to(G.DEV)
    rq = G.u16_tensor(rq_np.reshape(-1))
    rm = torch.from_numpy(rm_np.reshape(-1)).to(G.DEV)
    dp = torch.from_numpy(dp_np.reshape(-1)).to(G.DEV)

    def run_all():
        outs = {}
        # the single-pass layout first, with its workspace between guards too
        wsg = Guarded(G.epx.ep_query(cfg).workspace_bytes, torch.uint8)
        wsg.view.zero_()
        sp = G.gpu_layout(cfg, c.ids, ws=wsg.view, path="single-pass")
        wsg.check("workspace")
        G.assert_layout_equal(G.layout_np(sp), c.L, f"guards case {case} single-pass")
        ws = G.epx.workspace_for(cfg, G.DEV)
        shapes = {"counts": (S, Gs), "seg_base": (S + 1,), "row_offsets": (S, Gs + 1),
                  "scales_offsets": (S, Gs + 1), "token_row": (T, cfg.kp), "expert_ids": (R,),
                  "src_info": (R, 2), "flags": (1,)}
        lb = {k: Guarded(int(np.prod(s)), torch.int32) for k, s in shapes.items()}
        lay = G.epx.Layout(**{k: lb[k].view.view(*shapes[k]) for k in shapes})
        G.epx.ep_dispatch_layout(cfg, ids, ws, lay)
        torch.cuda.synchronize()
        for k, b in lb.items():
            outs[f"layout.{k}"] = b.check(f"layout.{k}")

        def op(name, fn, *specs):
            bufs = [Guarded(n, dt) for n, dt in specs]
            fn(*[b.view for b in bufs])
            torch.cuda.synchronize()
            for i, b in enumerate(bufs):
                outs[f"{name}[{i}]"] = b.check(f"{name}[{i}]")

        op("dispatch", lambda r: G.epx.ep_dispatch(cfg, lay, x, r), (R * H, torch.bfloat16))
        op("nvfp4", lambda a, b, r: G.epx.ep_dispatch_nvfp4(cfg, lay, x, a, b, r),
           (R * H // 2, torch.uint8), (R * H // 16, torch.uint8), (R, torch.bfloat16))
        if H % 128 == 0:
            op("fp8", lambda a, b: G.epx.ep_dispatch_fp8(cfg, lay, x, a, b),
               (R * H, torch.uint8), (R * (H // 128), torch.float32))
        op("combine", lambda o: G.epx.ep_combine(cfg, lay, out, probs, o), (T * H, torch.bfloat16))
        op("dispatch_bwd", lambda o: G.epx.ep_dispatch_bwd(cfg, lay, out, o), (T * H, torch.bfloat16))
        op("combine_bwd", lambda o: G.epx.ep_combine_bwd(cfg, lay, gy, probs, o), (R * H, torch.bfloat16))
        op("probs_grad", lambda o: G.epx.ep_combine_bwd_probs(cfg, lay, gy, out, o), (T * K, torch.float32))
        op("combine_nvfp4", lambda o: G.epx.ep_combine_nvfp4(cfg, lay, cq, sq, rq, probs, o), (T * H, torch.bfloat16))
        op("to_multihot", lambda m, d: G.epx.ep_indices_to_multihot(cfg, ids, probs, m, d),
           (T * E, torch.uint8), (T * E, torch.float32))
        op("to_indices", lambda i, p, f: G.epx.ep_multihot_to_indices(cfg, rm, dp, i, p, f),
           (T * K, torch.int32), (T * K, torch.float32), (1, torch.int32))
        return outs

    first = run_all()
    second = run_all()
    assert first.keys() == second.keys()
    for k in first:
        assert np.array_equal(first[k], second[k]), f"{k}: two runs differ"
    # the layout in the guarded buffers is the oracle's
    assert np.array_equal(first["layout.token_row"].view(np.int32), c.L["token_row"].reshape(-1))
    assert np.array_equal(first["layout.flags"].view(np.int32), c.L["flags"].reshape(-1))
