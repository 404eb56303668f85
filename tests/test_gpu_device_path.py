"""GPU tests specific to the device-resident path (inject_topk_device):
validation on the device never faults, reports what it skipped, and
everything it did not skip matches the oracle bit for bit (V, untouched
slots) or within 2 ulp (K).

Expected images come from the oracle over the same requests, with the slots
of the tokens the device must skip put back to the sentinel.
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import paged
from pre_rope_kv_amd import harness, workloads

from test_gpu_parity import (_release_device_memory, compare, custom_workload,  # noqa: F401
                             oracle_images, written_mask)

pytestmark = pytest.mark.gpu

SENT = workloads.SENTINEL_BF16


def _device_run(w, setup=None, patch=None, **batch_kw):
    dw = harness.DeviceWorkload(w, host_mapping=False)
    dw.setup_device_batch(**batch_kw)
    if patch is not None:
        patch(dw)
    dw.status.zero_()
    dw.inject_device()
    torch.cuda.synchronize()
    return dw


def _expect(w_oracle, blocks_of, skip_slots=()):
    """Oracle images over blocks_of's listed blocks, skipped slots reset."""
    img_k, img_v, _ = oracle_images(w_oracle, "cuda")
    for s in skip_slots:
        for layer in range(w_oracle.spec.num_layers):
            img_k.row(layer, s)[...] = SENT
            img_v.row(layer, s)[...] = SENT
    mask = written_mask(w_oracle, blocks_of)
    for s in skip_slots:
        b, o = divmod(s, w_oracle.spec.block_size)
        mask[blocks_of.index(b), o] = False
    return img_k, img_v, mask


def _check(dw, w_oracle, skip_slots=()):
    blocks = dw.w.listed_blocks()
    assert blocks == w_oracle.listed_blocks()
    img_k, img_v, mask = _expect(w_oracle, blocks, skip_slots)
    gk, gv = dw.listed_blocks_host(blocks)
    compare(img_k, img_v, gk, gv, mask)
    sp = dw.w.spec
    injected = int(mask.sum())
    assert dw.count_non_sentinel() == 2 * sp.num_layers * injected * sp.num_kv_heads * sp.head_dim


FACTS = {0: 9, 1: 14, 2: 5}


@pytest.mark.parametrize("bad_id", [999, -1])
def test_unknown_fact_is_dropped(bad_id):
    """An unknown id contributes no tokens; the next fact follows directly."""
    w = custom_workload("unknown", 2, 8, 128, 16, FACTS, [([0, 1, 2], 7)])
    dw = _device_run(w, patch=lambda dw: dw.d_ids.__setitem__(1, bad_id))
    assert int(dw.status.item()) == 8
    _check(dw, dataclasses.replace(w, retrieved=[[0, 2]]))


def test_position_out_of_range_is_skipped():
    w = custom_workload("pos_oob", 2, 8, 128, 16, FACTS, [([0, 1, 2], 40)], max_position=64)
    dw = _device_run(w)
    assert int(dw.status.item()) == 2
    _, pos, slot = paged.token_mapping(w.requests(), w.fact_rows, 16)
    skip = [s for p, s in zip(pos, slot) if p >= 64]
    assert len(skip) == 4
    _check(dw, w, skip)


def test_short_block_table_is_skipped():
    w = custom_workload("bt_short", 2, 8, 128, 16, FACTS, [([0, 1, 2], 7)])
    nb = len(w.block_tables[0])
    dw = _device_run(w, patch=lambda dw: dw.d_bt_len.__setitem__(0, nb - 1))
    assert int(dw.status.item()) == 4
    _, pos, slot = paged.token_mapping(w.requests(), w.fact_rows, 16)
    skip = [s for p, s in zip(pos, slot) if p // 16 >= nb - 1]
    assert skip
    _check(dw, w, skip)


def test_block_id_out_of_range_is_skipped():
    w = custom_workload("bt_bad_id", 2, 8, 128, 16, FACTS, [([0, 1, 2], 7)])
    dw = _device_run(w, patch=lambda dw: dw.d_bt.__setitem__((0, 1), w.num_blocks + 3))
    assert int(dw.status.item()) == 4
    _, pos, slot = paged.token_mapping(w.requests(), w.fact_rows, 16)
    skip = [s for p, s in zip(pos, slot) if p // 16 == 1]
    _check(dw, w, skip)


def test_max_tokens_drops_the_excess():
    w = custom_workload("max_tok", 2, 8, 128, 16, FACTS, [([0, 1, 2], 7)])
    n = w.n_tokens
    dw = _device_run(w, max_tokens=n - 5)
    assert int(dw.status.item()) == 16
    _, _, slot = paged.token_mapping(w.requests(), w.fact_rows, 16)
    assert dw.device_mapping()[0] == n - 5
    _check(dw, w, slot[n - 5:])


def test_max_facts_drops_the_excess():
    w = custom_workload("max_facts", 2, 8, 128, 16, FACTS, [([0, 1, 2], 7)])
    dw = _device_run(w, max_facts=2)
    assert int(dw.status.item()) == 32
    _check(dw, dataclasses.replace(w, retrieved=[[0, 1]]))


def test_two_batches_reuse_store_and_workspace():
    """Two different batches through one store and one workspace."""
    facts = {0: 9, 1: 14, 2: 5, 3: 21}
    w1 = custom_workload("batch_a", 3, 8, 128, 16, facts, [([3, 0], 5), ([1, 2, 1], 11)])
    dw = _device_run(w1, max_tokens=200, max_facts=8)
    assert int(dw.status.item()) == 0
    _check(dw, w1)
    # second batch: other order and prefix, same blocks
    w2 = dataclasses.replace(w1, retrieved=[[2, 3], [0]], prefix=np.array([0, 30]))
    dw.w = w2
    dw.reset_cache()
    dw.setup_device_batch(max_tokens=200, max_facts=8)
    dw.status.zero_()
    dw.inject_device()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    _check(dw, w2)
