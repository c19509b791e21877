"""GPU parity of the compact <-> dense routing conversions (NeMo AutoModel
token_dispatcher page, _HybridEPManager._indices_to_multihot; NeMo AutoModel
fused_a2a page, HybridEPDispatch.forward takes a routing map or indices),
bit for bit against the CPU oracle."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def G():
    import gpu_cases as gc

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return gc


CASES = [  # T, E, K, distinct, mask_p, bad_p
    (0, 8, 2, True, 0.0, 0.0),
    (1, 8, 8, True, 0.0, 0.0),
    (300, 37, 5, True, 0.1, 0.0),
    (513, 256, 8, True, 0.0, 0.0),
    (200, 100, 6, False, 0.2, 0.05),
    (64, 2048, 16, True, 0.05, 0.02),
    (4096, 256, 8, True, 0.0, 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[0]}_E{c[1]}_K{c[2]}" for c in CASES])
def test_indices_to_multihot(G, case):
    T, E, K, distinct, mask_p, bad_p = case
    rng = np.random.default_rng(T + E + K)
    ids = (np.stack([rng.permutation(E)[:K] for _ in range(T)]) if distinct and T else
           rng.integers(0, E, (T, K)))
    ids = np.where(rng.random((T, K)) < mask_p, -1, ids)
    ids = np.where(rng.random((T, K)) < bad_p, rng.choice([-3, E, E + 9], (T, K)), ids).astype(np.int32)
    probs = rng.random((T, K)).astype(np.float32)
    cfg = G.epx.EpConfig(num_tokens=T, hidden=8, num_experts=E, num_segments=1, top_k=K)
    G.say(f"[gpu] indices_to_multihot T={T} E={E} K={K}")
    rm = torch.full((T * E,), 0xA5, dtype=torch.uint8, device=G.DEV)
    dp = torch.full((T * E,), float("nan"), dtype=torch.float32, device=G.DEV)
    ids_t = torch.from_numpy(ids.reshape(-1)).to(G.DEV)
    pr_t = torch.from_numpy(probs.reshape(-1)).to(G.DEV)
    G.epx.ep_indices_to_multihot(cfg, ids_t, pr_t, rm, dp)
    torch.cuda.synchronize()
    oc = G.orc.Cfg(T=T, H=8, E=E, S=1, K=K)
    wrm, wdp = G.orc.indices_to_multihot(oc, ids, probs)
    G.assert_bits_equal(rm.cpu().numpy(), wrm, "routing_map")
    G.assert_bits_equal(dp.view(torch.int32).cpu().numpy(), wdp.view(np.int32), "dense_probs")
    # map only (no dense probabilities)
    rm2 = torch.full((T * E,), 0xA5, dtype=torch.uint8, device=G.DEV)
    G.epx.ep_indices_to_multihot(cfg, ids_t, None, rm2, None)
    torch.cuda.synchronize()
    G.assert_bits_equal(rm2.cpu().numpy(), wrm, "routing_map (no probs)")


MAPS = [  # T, E, K, density
    (0, 8, 2, 0.5),
    (300, 37, 5, 0.08),
    (513, 256, 8, 0.03),
    (200, 100, 6, 0.2),       # many rows overflow K
    (64, 2048, 16, 0.004),
    (100, 64, 64, 0.9),       # K at its largest, E an exact chunk
    (4096, 256, 8, 0.031),
]


@pytest.mark.parametrize("case", MAPS, ids=[f"T{c[0]}_E{c[1]}_K{c[2]}_d{c[3]}" for c in MAPS])
def test_multihot_to_indices(G, case):
    T, E, K, dens = case
    rng = np.random.default_rng(T * 7 + E)
    rm = ((rng.random((T, E)) < dens) * rng.integers(1, 256, (T, E))).astype(np.uint8)
    dp = rng.random((T, E)).astype(np.float32)
    cfg = G.epx.EpConfig(num_tokens=T, hidden=8, num_experts=E, num_segments=1, top_k=K)
    G.say(f"[gpu] multihot_to_indices T={T} E={E} K={K} density={dens}")
    ids = torch.full((T * K,), -7, dtype=torch.int32, device=G.DEV)
    pr = torch.full((T * K,), float("nan"), dtype=torch.float32, device=G.DEV)
    flags = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    G.epx.ep_multihot_to_indices(cfg, torch.from_numpy(rm.reshape(-1)).to(G.DEV),
                                 torch.from_numpy(dp.reshape(-1)).to(G.DEV), ids, pr, flags)
    torch.cuda.synchronize()
    oc = G.orc.Cfg(T=T, H=8, E=E, S=1, K=K)
    wids, wpr, wflags = G.orc.multihot_to_indices(oc, rm, dp)
    G.assert_bits_equal(ids.cpu().numpy(), wids, "topk_ids")
    G.assert_bits_equal(pr.view(torch.int32).cpu().numpy(), wpr.view(np.int32), "probs")
    assert int(flags.item()) == wflags


def test_map_routed_dispatch_matches_oracle(G):
    """A dense routing map converted on the GPU feeds the layout and combine:
    the same result as the oracle run on the oracle's conversion."""
    c0 = G.random_case(31, T=700, S=4, E_loc=8, K=4, H=256, A=8, mask_p=0.1)
    cfg = c0.cfg
    T, E, K = cfg.num_tokens, cfg.num_experts, cfg.top_k
    oc = G.orc.Cfg(T=T, H=8, E=E, S=cfg.num_segments, K=K)
    rm, dp = G.orc.indices_to_multihot(oc, c0.ids, c0.probs)
    ids = torch.empty(T * K, dtype=torch.int32, device=G.DEV)
    pr = torch.empty(T * K, dtype=torch.float32, device=G.DEV)
    G.epx.ep_multihot_to_indices(cfg, torch.from_numpy(rm.reshape(-1)).to(G.DEV),
                                 torch.from_numpy(dp.reshape(-1)).to(G.DEV), ids, pr)
    torch.cuda.synchronize()
    wids, wpr, _ = G.orc.multihot_to_indices(oc, rm, dp)
    c = G.Case(cfg, wids, wpr, c0.x, c0.seed)
    lay = G.check_layout(c, "map_routed")
    assert np.array_equal(ids.cpu().numpy().reshape(T, K), wids)
    G.check_dispatch(c, lay, "map_routed")
    G.check_combine(c, lay, "map_routed")
