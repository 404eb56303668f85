"""inject_topk_device_noalloc: the device-side retrieve-and-inject step on the
library's own per-GPU scratch array instead of a caller workspace.

Checked against inject_topk_device on the same batch (caches and status bit
for bit) and against the oracle at the parity bar, on three calls in a row
that share the scratch array: a batch of 400 facts, then a smaller one of
270 (both through the plan and mapping kernels, which use the workspace),
then a 5-fact batch (the fused single launch); and with the duplicate-slot
check, whose slot set lives in the array too.  A batch whose bounds do not
fit the array is rejected before anything is enqueued.
"""

import numpy as np
import pytest
import torch

from pre_rope_kv_amd import harness, prkv, workloads
from test_gpu_parity import (_release_device_memory, compare, custom_workload,  # noqa: F401
                             oracle_images, written_mask)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _workload(name, n_facts, seed):
    rng = np.random.default_rng(seed)
    pool = n_facts + 20
    facts = {f: int(rng.integers(1, 40)) for f in range(pool)}
    ids = [int(x) for x in rng.permutation(pool)[:n_facts]]
    cut = sorted(int(c) for c in rng.choice(np.arange(1, n_facts), 2, replace=False))
    reqs = [(ids[:cut[0]], 5), (ids[cut[0]:cut[1]], 17), (ids[cut[1]:], 0)]
    return custom_workload(name, 3, 8, 128, 16, facts, reqs, theta=5e5, num_blocks=4096)


def _noalloc(dw):
    prkv.inject_topk_device_noalloc(dw.store, dw.fact_table, dw.batch, dw.k_layers(),
                                    dw.v_layers(), dw.w.spec.block_size, dw.w.num_blocks,
                                    d_status=dw.status, stream=dw.stream)


def _check_against_workspace_path(w, max_facts):
    _say(f"no-alloc: {w.spec.name}, {sum(len(i) for i in w.retrieved)} facts, "
         f"{w.n_tokens} tokens, max_facts bound {max_facts}")
    dw = harness.DeviceWorkload(w)
    dw.setup_device_batch(max_facts=max_facts)
    blocks = w.listed_blocks()
    dw.status.zero_()
    dw.inject_device()
    torch.cuda.synchronize()
    ref_status = int(dw.status.item())
    ref_k, ref_v = dw.listed_blocks_host(blocks)
    dw.reset_cache()
    dw.status.zero_()
    _noalloc(dw)
    torch.cuda.synchronize()
    assert int(dw.status.item()) == ref_status == 0
    got_k, got_v = dw.listed_blocks_host(blocks)
    assert np.array_equal(got_k, ref_k) and np.array_equal(got_v, ref_v)
    img_k, img_v, n = oracle_images(w, "cuda")
    assert n == w.n_tokens
    compare(img_k, img_v, got_k, got_v, written_mask(w, blocks))
    sp = w.spec
    assert dw.count_non_sentinel() == 2 * sp.num_layers * w.n_tokens * sp.num_kv_heads * \
        sp.head_dim
    return dw


def test_noalloc_equals_workspace_path_on_consecutive_calls():
    # > 256 facts: the plan and per-token mapping kernels, which keep the
    # plan and the mapping in the workspace (here: the scratch array)
    _check_against_workspace_path(_workload("noalloc_400", 400, 1), 400)
    # a smaller batch right after: the array still holds the first call's data
    _check_against_workspace_path(_workload("noalloc_270", 270, 2), 270)
    # a small batch: the fused launch, which writes its plan and mapping there too
    _check_against_workspace_path(workloads.make("tiny_L1_H2_D64"), None)


def test_noalloc_with_the_duplicate_slot_check():
    """The checked step (slot set in the scratch array too) on a batch whose
    two requests share a block: the same skipped tokens, status and cache as
    inject_topk_device with a caller workspace."""
    import dataclasses
    w = _workload("noalloc_dup", 300, 4)
    bts = [t.copy() for t in w.block_tables]
    bts[1][1] = bts[0][1]      # request 1 injects from position 17: its block 1 collides
    w = dataclasses.replace(w, block_tables=bts)
    blocks = sorted(set(int(b) for t in bts for b in t))
    dw = harness.DeviceWorkload(w, host_mapping=False)
    dw.setup_device_batch(max_facts=300, flags=prkv.BATCH_CHECK_SLOTS)
    dw.status.zero_()
    dw.inject_device()
    torch.cuda.synchronize()
    ref_status = int(dw.status.item())
    ref_k, ref_v = dw.listed_blocks_host(blocks)
    dw.reset_cache()
    dw.status.zero_()
    side = torch.cuda.Stream()            # a stream of its own: the scratch of its device
    side.wait_stream(dw.stream)
    prkv.inject_topk_device_noalloc(dw.store, dw.fact_table, dw.batch, dw.k_layers(),
                                    dw.v_layers(), w.spec.block_size, w.num_blocks,
                                    d_status=dw.status, stream=side)
    torch.cuda.synchronize()
    assert int(dw.status.item()) == ref_status == 128
    got_k, got_v = dw.listed_blocks_host(blocks)
    assert np.array_equal(got_k, ref_k) and np.array_equal(got_v, ref_v)


def test_noalloc_rejects_bounds_beyond_the_scratch():
    w = _workload("noalloc_reject", 300, 3)
    dw = harness.DeviceWorkload(w)
    # bounds whose workspace exceeds the 16 MiB array (about 1.4 M tokens)
    dw.setup_device_batch(max_facts=300, max_tokens=2_000_000)
    assert prkv.inject_device_workspace_bytes(300, 2_000_000) > prkv.NOALLOC_SCRATCH_BYTES
    dw.status.zero_()
    with pytest.raises(prkv.PrkvError) as err:
        _noalloc(dw)
    assert err.value.name == "BUFFER_TOO_SMALL"
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    assert dw.count_non_sentinel() == 0
