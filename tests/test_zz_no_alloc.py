"""ep_dispatch_layout_noalloc against ep_dispatch_layout on the GPU, through
the C ABI: the same layout, bit for bit, on consecutive calls that share the
library's built-in scratch (the second and third smaller than the first, the
third on the other prefix path).

Both calls write into sentinel-filled buffers, so whole arrays are compared:
rows that one call leaves untouched must be left untouched by the other.
"""

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


def _both(G, c, name):
    cfg = c.cfg
    G.say(f"[gpu] noalloc layout {name}: T={cfg.num_tokens} E={cfg.num_experts} S={cfg.num_segments} "
          f"K={cfg.top_k} A={cfg.align} C={cfg.seg_capacity} shared={cfg.shared_expert} flags={cfg.flags}")
    ref = G.gpu_layout(cfg, c.ids)
    lay = G.sentinel_layout(cfg)
    ids = torch.from_numpy(np.ascontiguousarray(c.ids, np.int32).reshape(-1)).to(G.DEV)
    G.epx.ep_dispatch_layout_noalloc(cfg, ids, lay)
    torch.cuda.synchronize()
    G.assert_layout_equal(G.layout_np(lay), G.layout_np(ref), name)
    return lay


def test_noalloc_layout_matches_the_workspace_entry_point(G):
    big = G.workload_case("dsv3")
    assert G.epx.ep_query(big.cfg).workspace_bytes <= G.epx.EP_NOALLOC_SCRATCH_BYTES
    _both(G, big, "dsv3")
    smaller = G.workload_case("skewed", T=1000)
    smaller.cfg.flags |= G.epx.EP_LAYOUT_LOOKBACK
    _both(G, smaller, "skewed T=1000 look-back")
    tiny = G.workload_case("dsv3", T=16)
    _both(G, tiny, "dsv3 T=16")
    # the oracle agrees as well (the workspace entry point is checked against
    # it everywhere else)
    G.assert_layout_equal(G.layout_np(_both(G, tiny, "dsv3 T=16 again")), tiny.L, "dsv3 T=16 vs oracle")


def test_noalloc_layout_rejects_oversized_problems(G):
    """A configuration whose workspace exceeds the built-in scratch gets
    EP_ESCRATCH before anything is enqueued (the pointers are valid device
    addresses but far too small: no kernel may run)."""
    import ctypes

    cfg = G.epx.EpConfig(num_tokens=1 << 21, hidden=256, num_experts=2048, num_segments=8, top_k=8)
    q = G.epx.ep_query(cfg)
    assert q.workspace_bytes > G.epx.EP_NOALLOC_SCRATCH_BYTES
    cfg.recv_rows = q.min_recv_rows
    buf = torch.zeros(64, dtype=torch.int32, device=G.DEV)
    lay = G.epx.Layout(*([buf] * 8)).to_c()
    c = cfg.to_c()
    rc = G.epx._lib.lib().ep_dispatch_layout_noalloc(ctypes.byref(c), buf.data_ptr(), ctypes.byref(lay), None)
    torch.cuda.synchronize()
    assert rc == -4
    assert int(buf.abs().sum().item()) == 0
