"""Pins of the oracle's payload steps: bf16 dispatch, fp32 weighted combine,
dispatch backward (sum over slots) and combine backward (redispatch).

What pins them:
  * dispatch rows equal the source token's row (src_info);
  * combine of dispatch with identity experts and probabilities summing to 1
    returns the input bit for bit (with a shared expert of weight 1: 2x);
  * the fp64 closed form y = sum_k w_k out[row(t,k)], within the fp32
    accumulation bound plus half a bf16 ulp;
  * adjoint identities <D x, g> = <x, D^T g> and <C o, gy> = <o, C^T gy>
    within the rounding bound;
  * torch CPU autograd of an index_select / index_add formulation in fp64.

Sources: NeMo AutoModel fused_a2a page (HybridEPDispatch.backward combines
gradients; HybridEPCombine.backward redispatches them); NeMo AutoModel
token_dispatcher page (TokenDispatcherConfig.moe_router_dtype: fp32 weighted
averaging of expert outputs).
"""

import numpy as np
import pytest
import torch

from combine_ep_dispatch_amd import workload as wl


def f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def make_case(orc, seed, T=37, H=24, E=12, S=3, K=4, A=4, shared=0, C=0, mask_p=0.1):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    ids = np.where(rng.random((T, K)) < mask_p, -1, ids).astype(np.int32)
    logits = rng.standard_normal((T, K))
    p = np.exp(logits - logits.max(1, keepdims=True))
    probs = (p / p.sum(1, keepdims=True)).astype(np.float32)
    x = wl.bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    cfg = orc.Cfg(T=T, H=H, E=E, S=S, K=K, A=A, C=C, shared=shared, src_seg=S - 1)
    cfg.recv_rows = orc.min_recv_rows(cfg)
    L = orc.layout(cfg, ids)
    return cfg, ids, probs, x, L, rng


def test_dispatch_rows_equal_source_rows(orc):
    cfg, ids, probs, x, L, _ = make_case(orc, 1, shared=1)
    recv = orc.dispatch(cfg, L["token_row"], x)
    tr = L["token_row"]
    tt, kk = np.nonzero(tr >= 0)
    assert np.array_equal(recv[tr[tt, kk]], x[tt])
    unused = np.ones(cfg.recv_rows, bool)
    unused[tr[tt, kk]] = False
    assert np.all(recv[unused] == orc.SENTINEL_U16)


@pytest.mark.parametrize("shared", [0, 1])
def test_combine_of_dispatch_is_identity(orc, shared):
    cfg, ids, probs, x, L, _ = make_case(orc, 2, T=64, H=64, shared=shared, mask_p=0.0)
    recv = orc.dispatch(cfg, L["token_row"], x)
    y = orc.combine(cfg, L["token_row"], recv, probs)
    if shared:
        want = wl.bf16_bits(2.0 * f32(x))
    else:
        want = x
    assert np.array_equal(y, want)


def closed_form(cfg, token_row, out, probs):
    T, K, Kp = cfg.T, cfg.K, cfg.Kp
    y = np.zeros((T, cfg.H))
    mag = np.zeros((T, cfg.H))
    for k in range(Kp):
        rows = token_row[:, k]
        w = np.ones(T) if (probs is None or k >= K) else probs[:, k].astype(np.float64)
        ok = rows >= 0
        v = np.zeros((T, cfg.H))
        v[ok] = f32(out[rows[ok]]).astype(np.float64)
        y += w[:, None] * v
        mag += np.abs(w[:, None] * v)
    return y, mag


@pytest.mark.parametrize("weighted", [True, False])
@pytest.mark.parametrize("shared", [0, 1])
def test_combine_matches_fp64_closed_form(orc, weighted, shared):
    cfg, ids, probs, x, L, rng = make_case(orc, 3, shared=shared)
    out = wl.bf16_bits(rng.standard_normal((cfg.recv_rows, cfg.H), dtype=np.float32))
    pr = probs if weighted else None
    y = orc.combine(cfg, L["token_row"], out, pr)
    y64, mag = closed_form(cfg, L["token_row"], out, pr)
    # fp32: each of <= K' products and sums rounds once (2*K'*2^-24 * sum|terms|);
    # final bf16 rounding: half an ulp, at most 2^-8 |y| (plus the fp32 error)
    bound = 2 * cfg.Kp * 2.0 ** -24 * mag
    bound = bound + 2.0 ** -8 * (np.abs(y64) + bound) + 1e-30
    assert np.all(np.abs(f32(y).astype(np.float64) - y64) <= bound)
    # masked-out tokens give exact zeros
    none = np.all(L["token_row"] < 0, axis=1)
    assert np.all(y[none] == 0)


def test_adjoint_identities(orc):
    cfg, ids, probs, x, L, rng = make_case(orc, 4, shared=1, A=8)
    tr = L["token_row"]
    g = wl.bf16_bits(rng.standard_normal((cfg.recv_rows, cfg.H), dtype=np.float32))
    gy = wl.bf16_bits(rng.standard_normal((cfg.T, cfg.H), dtype=np.float32))
    out = wl.bf16_bits(rng.standard_normal((cfg.recv_rows, cfg.H), dtype=np.float32))
    used = np.zeros(cfg.recv_rows, bool)
    used[tr[tr >= 0]] = True
    # <D x, g> == <x, D^T g>
    recv = orc.dispatch(cfg, tr, x)
    lhs = np.sum(f32(recv[used]).astype(np.float64) * f32(g[used]))
    gx = orc.dispatch_bwd(cfg, tr, g)
    rhs = np.sum(f32(x).astype(np.float64) * f32(gx))
    # D^T g is rounded to bf16 (2^-8 relative) after fp32 sums
    gmag = np.zeros((cfg.T, cfg.H))
    for k in range(cfg.Kp):
        ok = tr[:, k] >= 0
        gmag[ok] += np.abs(f32(g[tr[ok, k]]))
    tol = np.sum(np.abs(f32(x)) * gmag) * (2.0 ** -8 + 2 * cfg.Kp * 2.0 ** -24)
    assert abs(lhs - rhs) <= tol
    # <C o, gy> == <o, C^T gy>
    y = orc.combine(cfg, tr, out, probs)
    go = orc.combine_bwd(cfg, tr, gy, probs)
    lhs = np.sum(f32(y).astype(np.float64) * f32(gy))
    rhs = np.sum(f32(out[used]).astype(np.float64) * f32(go[used]))
    y64, mag = closed_form(cfg, tr, out, probs)
    tol = np.sum((np.abs(y64) + mag) * np.abs(f32(gy))) * (2.0 ** -8 + 2 * cfg.Kp * 2.0 ** -24)
    assert abs(lhs - rhs) <= tol
    # pad and unused rows of grad_out are not written
    assert np.all(go[~used] == orc.SENTINEL_U16)


def test_backward_matches_torch_autograd(orc):
    cfg, ids, probs, x, L, rng = make_case(orc, 5, shared=1, A=2)
    tr = torch.from_numpy(L["token_row"].astype(np.int64))
    T, H, K, Kp, R = cfg.T, cfg.H, cfg.K, cfg.Kp, cfg.recv_rows
    w = torch.ones(T, Kp, dtype=torch.float64)
    w[:, :K] = torch.from_numpy(probs.astype(np.float64))
    ok = tr >= 0
    tt, kk = torch.nonzero(ok, as_tuple=True)
    rows = tr[tt, kk]
    # dispatch: recv = scatter of x rows; combine: y[t] = sum_k w out[row]
    xt = torch.from_numpy(f32(x).astype(np.float64)).requires_grad_(True)
    recv = torch.zeros(R, H, dtype=torch.float64).index_copy(0, rows, xt.index_select(0, tt))
    g = torch.from_numpy(f32(wl.bf16_bits(rng.standard_normal((R, H), dtype=np.float32))).astype(np.float64))
    (recv * g).sum().backward()
    gx_ref = xt.grad.numpy()
    gx = f32(orc.dispatch_bwd(cfg, L["token_row"], wl.bf16_bits(g.numpy().astype(np.float32))))
    assert np.allclose(gx, gx_ref, rtol=2 ** -8, atol=1e-6)

    ot = torch.from_numpy(f32(wl.bf16_bits(rng.standard_normal((R, H), dtype=np.float32))).astype(np.float64))
    ot.requires_grad_(True)
    y = torch.zeros(T, H, dtype=torch.float64).index_add(0, tt, ot.index_select(0, rows) * w[tt, kk][:, None])
    gy = torch.from_numpy(f32(wl.bf16_bits(rng.standard_normal((T, H), dtype=np.float32))).astype(np.float64))
    (y * gy).sum().backward()
    go_ref = ot.grad.numpy()
    go = f32(orc.combine_bwd(cfg, L["token_row"], wl.bf16_bits(gy.numpy().astype(np.float32)), probs))
    used = rows.numpy()
    assert np.allclose(go[used], go_ref[used], rtol=2 ** -8, atol=1e-30)


def test_dropped_slots_contribute_zero(orc):
    cfg, ids, probs, x, L, rng = make_case(orc, 6, T=40, E=8, S=2, K=3, A=1, C=20, mask_p=0.0)
    assert int(L["flags"][0]) == 1
    tr = L["token_row"]
    out = wl.bf16_bits(rng.standard_normal((cfg.recv_rows, cfg.H), dtype=np.float32))
    y = orc.combine(cfg, tr, out, probs)
    y64, mag = closed_form(cfg, tr, out, probs)
    assert np.all(np.abs(f32(y) - y64) <= 2.0 ** -8 * np.abs(y64) + 4 * cfg.Kp * 2.0 ** -24 * mag + 1e-30)
    none = np.all(tr < 0, axis=1)
    assert none.any() and np.all(y[none] == 0)


def test_probability_gradient_matches_torch_autograd(orc):
    """grad_probs (NeMo AutoModel fused_a2a page, HybridEPDispatch.backward:
    a probability gradient beside the hidden-state gradient) is the
    derivative of combine's weighted sum with respect to the weights."""
    cfg, ids, probs, x, L, rng = make_case(orc, 8, shared=1, A=4, mask_p=0.15)
    T, H, K, R = cfg.T, cfg.H, cfg.K, cfg.recv_rows
    tr = torch.from_numpy(L["token_row"].astype(np.int64))
    out = wl.bf16_bits(rng.standard_normal((R, H), dtype=np.float32))
    gy = wl.bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    p = torch.from_numpy(probs.astype(np.float64)).requires_grad_(True)
    ot = torch.from_numpy(f32(out).astype(np.float64))
    y = torch.zeros(T, H, dtype=torch.float64)
    for k in range(cfg.Kp):
        ok = tr[:, k] >= 0
        w = p[:, k] if k < K else torch.ones(T, dtype=torch.float64)
        y = y + torch.where(ok[:, None], w[:, None] * ot[tr[:, k].clamp(min=0)], torch.zeros(()))
    (y * torch.from_numpy(f32(gy).astype(np.float64))).sum().backward()
    want = p.grad.numpy()
    got = orc.combine_bwd_probs(cfg, L["token_row"], gy, out)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    masked = L["token_row"][:, :K] < 0
    assert masked.any() and np.all(got[masked] == 0)
