"""The device inject path, and the whole serving step, under HIP graph
capture.

inject_topk_device, retrieve_topk and attend_paged enqueue only kernels (no
memset, no copy), so a serving loop can capture them once and replay them.
Each replay must reproduce the eager result bit for bit; eager work (cache
resets, synchronisations) runs between the replays.
"""

import math

import numpy as np
import pytest
import torch

from pre_rope_kv_amd import harness, prkv, workloads

from test_gpu_parity import _release_device_memory, _say  # noqa: F401
from test_gpu_retrieve import _embeddings

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


@pytest.mark.parametrize("name", ["tiny_L1_H2_D64", "llama3_8b_k50"])
def test_serving_step_graph_replays_match_eager(name):
    """retrieve_topk -> inject_topk_device (on the retrieved ids, written
    straight into the device batch) -> attend_paged (the context's last
    positions as the query), captured as one graph."""
    w = workloads.make(name)
    sp = w.spec
    gen = "cpu" if name.startswith("tiny") else "cuda"
    embs, emb = _embeddings(w)
    q_emb = w.query_embeddings("cuda", emb=embs)
    dw = harness.DeviceWorkload(w, gen_device=gen, host_mapping=False)
    dw.setup_device_batch()
    ws_bytes = prkv.retrieve_workspace_bytes(sp.n_requests, sp.facts_per_store)
    rws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    d_rs = torch.as_tensor(w.req_store(), device="cuda")
    q_len, hq, D = 4, 4 * sp.num_kv_heads, sp.head_dim
    ctxs = [int(w.prefix[r]) + sum(w.length_of(f) for f in ids)
            for r, ids in enumerate(w.retrieved)]
    g = torch.Generator(device="cpu")
    g.manual_seed(5)
    q = torch.randn((sp.n_requests, q_len, hq, D), generator=g).to(torch.bfloat16) \
        .view(torch.int16).cuda()
    q_start = torch.as_tensor([c - q_len for c in ctxs], dtype=torch.int32, device="cuda")
    out = torch.empty((sp.num_layers, sp.n_requests, q_len, hq, D), dtype=torch.float32,
                      device="cuda")
    ab = prkv.attn_batch(sp.n_requests, q_len, hq, dw.d_bt.shape[1], q, q_start, dw.d_bt,
                         dw.d_bt_len, out)
    blocks = w.listed_blocks()

    def step(stream):
        prkv.retrieve_topk(emb, sp.n_requests, sp.facts_per_store, sp.emb_dim, q_emb, d_rs,
                           sp.n_requests, sp.k, dw.d_ids, rws, ws_bytes, d_status=dw.status,
                           stream=stream)
        prkv.inject_topk_device(dw.store, dw.fact_table, dw.batch, dw.k_layers(), dw.v_layers(),
                                sp.block_size, w.num_blocks, dw.workspace, dw.ws_bytes,
                                d_status=dw.status, stream=stream)
        prkv.attend_paged(dw.store, ab, dw.k_layers(), dw.v_layers(), sp.block_size,
                          w.num_blocks, 1.0 / math.sqrt(D), d_status=dw.status, stream=stream)

    def reset():
        # eager work: the prefix and query slots read as zeros, ids and
        # output poisoned so that a replay that skips a kernel shows
        dw.k_cache.zero_()
        dw.v_cache.zero_()
        dw.d_ids.fill_(-1)
        out.fill_(float("nan"))
        torch.cuda.synchronize()

    reset()
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    want_ids = dw.d_ids.cpu().numpy().copy()
    assert sorted(want_ids.tolist()) == sorted(f for ids in w.retrieved for f in ids)
    want_k, want_v = dw.listed_blocks_host(blocks)
    want_out = out.cpu().numpy().copy()
    assert np.all(np.isfinite(want_out))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(3):
        reset()
        graph.replay()
        torch.cuda.synchronize()
        got_k, got_v = dw.listed_blocks_host(blocks)
        assert np.array_equal(dw.d_ids.cpu().numpy(), want_ids), rep
        assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v), rep
        assert np.array_equal(out.cpu().numpy(), want_out), rep
        _say(f"{name}: serving-step replay {rep} equal to eager")
    assert int(dw.status.item()) == 0


def test_checked_device_inject_graph_replays_match_eager():
    """The device step with the duplicate-slot check (a clear kernel, not a
    memset, empties its slot set) on a batch whose two requests share a
    block, captured once: every replay skips the same tokens, reports the
    same status and writes the same cache as the eager step."""
    import dataclasses

    from test_gpu_device_path import _shared_block_workload
    w = _shared_block_workload("graph_dup")
    dw = harness.DeviceWorkload(w, host_mapping=False)
    dw.setup_device_batch(flags=prkv.BATCH_CHECK_SLOTS)
    blocks = w.listed_blocks()
    dw.status.zero_()
    dw.inject_device()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 128
    want_k, want_v = dw.listed_blocks_host(blocks)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
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
        dw.status.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(dw.status.item()) == 128, rep
        got_k, got_v = dw.listed_blocks_host(blocks)
        assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v), rep
    assert dataclasses.is_dataclass(w)
