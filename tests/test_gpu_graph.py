"""The device inject path under HIP graph capture.

inject_topk_device enqueues only kernels (no memset, no copy), so a serving
loop can capture it once and replay it.  Each replay must reproduce the
eager result bit for bit; eager work (cache resets, synchronisations) runs
between the replays.
"""

import numpy as np
import pytest
import torch

from pre_rope_kv_amd import harness, workloads

from test_gpu_parity import _release_device_memory, _say  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["tiny_L1_H2_D64", "llama3_8b_k5"])
def test_device_inject_graph_replays_match_eager(name):
    w = workloads.make(name)
    dw = harness.DeviceWorkload(w, gen_device="cpu" if name.startswith("tiny") else "cuda")
    dw.setup_device_batch()
    blocks = w.listed_blocks()
    dw.inject_device()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    want_k, want_v = dw.listed_blocks_host(blocks)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    dw.reset_cache()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    old_stream = dw.stream
    with torch.cuda.graph(g, stream=side):
        dw.stream = torch.cuda.current_stream()
        dw.inject_device()
    dw.stream = old_stream
    torch.cuda.synchronize()
    for rep in range(3):
        dw.reset_cache()                 # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_k, got_v = dw.listed_blocks_host(blocks)
        _say(f"{name}: replay {rep} equal to eager")
        assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v), rep
    assert int(dw.status.item()) == 0
