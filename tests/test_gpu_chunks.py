"""The movers' chunked launches, on the GPU: a HIP grid holds at most 2^32 - 1
work-items, so the bf16 scatter (dispatch, combine backward) and the gathers
(combine, dispatch backward) split larger batches into token chunks.  With
H = 8 (one 16-byte vector per row, one piece) the split is reachable:

  * scatter, K' = 64: 1 048 560 tokens per launch (one wave per
    (token, piece, slot), 8-wave workgroups);
  * gathers, K' = 1: 67 108 862 tokens per launch (one wave per
    (token, piece), 2-wave workgroups).

Each test runs a batch just past the first chunk, so the second launch
starts at a nonzero token offset, and compares the whole output with the
oracle bit for bit.  The receive rows come from the oracle's layout (the
movers only read token_row), uploaded as the layout's token_row.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

SCATTER_CHUNK = 1_048_560   # ((2^32 - 1) // 512 - 8) // 64 * 8 - 8
GATHER_CHUNK = 67_108_862   # (2^32 - 1) // 128 * 2


@pytest.fixture(scope="module")
def G():
    import gpu_cases as gc

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.cuda.init()
    return gc


def layout_from_oracle(G, cfg, ids):
    """The oracle's layout of `ids`, as a device Layout (only token_row is
    read by the movers; the other arrays are left empty)."""
    oc = G.ocfg(cfg)
    L = G.orc.layout(oc, ids)
    lay = G.epx.Layout.empty(cfg, G.DEV)
    lay.token_row.copy_(torch.from_numpy(L["token_row"]))
    return oc, L["token_row"], lay


def test_scatter_past_one_launch(G):
    T, K, H = SCATTER_CHUNK + 333, 64, 8
    G.say(f"[gpu] chunked scatter: T={T} K'={K} H={H}")
    cfg = G.epx.EpConfig(num_tokens=T, hidden=H, num_experts=K, num_segments=1, top_k=K)
    cfg.recv_rows = G.epx.ep_query(cfg).min_recv_rows
    rng = np.random.default_rng(3)
    ids = np.broadcast_to(np.arange(K, dtype=np.int32), (T, K)).copy()
    ids[rng.random((T, K)) < 0.01] = -1  # a few masked slots
    oc, tr, lay = layout_from_oracle(G, cfg, ids)
    x = G.wl.bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    recv = G.bf16_filled(cfg.recv_rows, H, G.orc.SENTINEL_U16)
    G.epx.ep_dispatch(cfg, lay, G.u16_tensor(x), recv)
    torch.cuda.synchronize()
    G.assert_bits_equal(G.bits_of(recv), G.orc.dispatch(oc, tr, x), "chunked dispatch")
    del recv
    probs = rng.random((T, K), dtype=np.float32)
    gout = G.bf16_filled(cfg.recv_rows, H, G.orc.SENTINEL_U16)
    G.epx.ep_combine_bwd(cfg, lay, G.u16_tensor(x), torch.from_numpy(probs.reshape(-1)).to(G.DEV), gout)
    torch.cuda.synchronize()
    G.assert_bits_equal(G.bits_of(gout), G.orc.combine_bwd(oc, tr, x, probs), "chunked combine_bwd")


def test_gathers_past_one_launch(G):
    T, H = GATHER_CHUNK + 77, 8
    G.say(f"[gpu] chunked gathers: T={T} K'=1 H={H}")
    cfg = G.epx.EpConfig(num_tokens=T, hidden=H, num_experts=2, num_segments=1, top_k=1)
    cfg.recv_rows = G.epx.ep_query(cfg).min_recv_rows
    rng = np.random.default_rng(4)
    ids = rng.integers(0, 2, (T, 1), dtype=np.int32)
    ids[rng.random((T, 1)) < 0.001] = -1
    oc, tr, lay = layout_from_oracle(G, cfg, ids)
    out = G.wl.bf16_bits(rng.standard_normal((cfg.recv_rows, H), dtype=np.float32))
    probs = rng.random((T, 1), dtype=np.float32)
    y = G.bf16_filled(T, H, G.orc.SENTINEL_U16)
    G.epx.ep_combine(cfg, lay, G.u16_tensor(out), torch.from_numpy(probs.reshape(-1)).to(G.DEV), y)
    torch.cuda.synchronize()
    G.assert_bits_equal(G.bits_of(y), G.orc.combine(oc, tr, out, probs), "chunked combine")
    gx = G.bf16_filled(T, H, G.orc.SENTINEL_U16)
    G.epx.ep_dispatch_bwd(cfg, lay, G.u16_tensor(out), gx)
    torch.cuda.synchronize()
    G.assert_bits_equal(G.bits_of(gx), G.orc.dispatch_bwd(oc, tr, out), "chunked dispatch_bwd")
