"""GPU tests specific to the device-resident path (inject_topk_device):
validation on the device never faults, reports what it skipped, and
everything it did not skip matches the oracle bit for bit (V, untouched
slots) or within 2 ulp (K).  Each runs on both device mappings: the fused
single launch (batches of at most 256 facts and 256 requests) and the
plan + mapping + inject kernels (forced by a larger max_facts bound); the two
must also agree with each other bit for bit, workspace included.

Expected images come from the oracle over the same requests, with the slots
of the tokens the device must skip put back to the sentinel.
"""

import dataclasses
from collections import Counter

import numpy as np
import pytest
import torch

from oracle import paged
from pre_rope_kv_amd import harness, prkv, workloads

from test_gpu_parity import (_release_device_memory, compare, custom_workload,  # noqa: F401
                             oracle_images, run_full, written_mask)

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
FUSE_LIMIT = 256           # the library's bound for the fused mapping
MAPPINGS = {"fused": {}, "kernels": {"max_facts": FUSE_LIMIT + 44}}
mapping = pytest.mark.parametrize("kw", list(MAPPINGS.values()), ids=list(MAPPINGS))


@mapping
@pytest.mark.parametrize("bad_id", [999, -1])
def test_unknown_fact_is_dropped(bad_id, kw):
    """An unknown id contributes no tokens; the next fact follows directly."""
    w = custom_workload("unknown", 2, 8, 128, 16, FACTS, [([0, 1, 2], 7)])
    dw = _device_run(w, patch=lambda dw: dw.d_ids.__setitem__(1, bad_id), **kw)
    assert int(dw.status.item()) == 8
    _check(dw, dataclasses.replace(w, retrieved=[[0, 2]]))


@mapping
def test_position_out_of_range_is_skipped(kw):
    w = custom_workload("pos_oob", 2, 8, 128, 16, FACTS, [([0, 1, 2], 40)], max_position=64)
    dw = _device_run(w, **kw)
    assert int(dw.status.item()) == 2
    _, pos, slot = paged.token_mapping(w.requests(), w.fact_rows, 16)
    skip = [s for p, s in zip(pos, slot) if p >= 64]
    assert len(skip) == 4
    _check(dw, w, skip)


@mapping
def test_short_block_table_is_skipped(kw):
    w = custom_workload("bt_short", 2, 8, 128, 16, FACTS, [([0, 1, 2], 7)])
    nb = len(w.block_tables[0])
    dw = _device_run(w, patch=lambda dw: dw.d_bt_len.__setitem__(0, nb - 1), **kw)
    assert int(dw.status.item()) == 4
    _, pos, slot = paged.token_mapping(w.requests(), w.fact_rows, 16)
    skip = [s for p, s in zip(pos, slot) if p // 16 >= nb - 1]
    assert skip
    _check(dw, w, skip)


@mapping
def test_block_id_out_of_range_is_skipped(kw):
    w = custom_workload("bt_bad_id", 2, 8, 128, 16, FACTS, [([0, 1, 2], 7)])
    dw = _device_run(w, patch=lambda dw: dw.d_bt.__setitem__((0, 1), w.num_blocks + 3), **kw)
    assert int(dw.status.item()) == 4
    _, pos, slot = paged.token_mapping(w.requests(), w.fact_rows, 16)
    skip = [s for p, s in zip(pos, slot) if p // 16 == 1]
    _check(dw, w, skip)


@mapping
def test_max_tokens_drops_the_excess(kw):
    w = custom_workload("max_tok", 2, 8, 128, 16, FACTS, [([0, 1, 2], 7)])
    n = w.n_tokens
    dw = _device_run(w, max_tokens=n - 5, **kw)
    assert int(dw.status.item()) == 16
    _, _, slot = paged.token_mapping(w.requests(), w.fact_rows, 16)
    assert dw.device_mapping()[0] == n - 5
    _check(dw, w, slot[n - 5:])


@mapping
@pytest.mark.parametrize("heads", [8, 1])
def test_loose_max_tokens_bound(heads, kw):
    """max_tokens far above the batch's count: the grid is sized for the bound
    and the kernel spreads the real tokens over it (split count chosen on the
    device); every token is still injected exactly once."""
    w = custom_workload(f"loose_h{heads}", 6, heads, 128, 16, FACTS, [([2, 0, 1], 3), ([1], 20)],
                        num_blocks=4096)
    dw = _device_run(w, max_tokens=64 * w.n_tokens, **kw)
    assert int(dw.status.item()) == 0
    assert dw.device_mapping()[0] == w.n_tokens
    _check(dw, w)


@mapping
def test_expected_count_far_too_low(kw):
    """The grid is sized for max_facts facts of the store's mean length; a
    batch of the one long fact (mean length ~7, batch 600 tokens) is ~25 x
    that, covered by the grid stride."""
    facts = {0: 200, **{i: 1 for i in range(1, 31)}}
    w = custom_workload("long_fact", 4, 8, 128, 16, facts, [([0, 0, 0], 5)], num_blocks=1024)
    dw = _device_run(w, **kw)
    assert int(dw.status.item()) == 0
    assert dw.device_mapping()[0] == 600
    _check(dw, w)


@pytest.mark.parametrize("bound", [2, FUSE_LIMIT, FUSE_LIMIT + 1])
def test_max_facts_drops_the_excess(bound):
    """More facts than max_facts: the excess facts are dropped (the first two
    bounds take the fused mapping, the last the separate kernels)."""
    ids = [0, 1, 2] * ((bound + 2) // 3 + 1)            # repeats are legal
    w = custom_workload(f"max_facts_{bound}", 2, 8, 128, 16, FACTS, [(ids, 7)],
                        num_blocks=2048)
    dw = _device_run(w, max_facts=bound)
    assert int(dw.status.item()) == 32
    _check(dw, dataclasses.replace(w, retrieved=[ids[:bound]]))


@pytest.mark.parametrize("max_facts", [8, FUSE_LIMIT + 1], ids=["fused", "kernels"])
def test_two_batches_reuse_store_and_workspace(max_facts):
    """Two different batches through one store and one workspace."""
    facts = {0: 9, 1: 14, 2: 5, 3: 21}
    w1 = custom_workload("batch_a", 3, 8, 128, 16, facts, [([3, 0], 5), ([1, 2, 1], 11)])
    dw = _device_run(w1, max_tokens=200, max_facts=max_facts)
    assert int(dw.status.item()) == 0
    _check(dw, w1)
    # second batch: other order and prefix, same blocks
    w2 = dataclasses.replace(w1, retrieved=[[2, 3], [0]], prefix=np.array([0, 30]))
    dw.w = w2
    dw.reset_cache()
    dw.setup_device_batch(max_tokens=200, max_facts=max_facts)
    dw.status.zero_()
    dw.inject_device()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    _check(dw, w2)


def _workspace_parts(dw):
    """Header, plan and per-token mapping the device path left in its workspace."""
    ws = dw.workspace.cpu().numpy()
    lay = dw.ws_layout
    n_tok = int(ws[0:8].view(np.int64)[0])
    n_facts = int(ws[8:12].view(np.int32)[0])
    plan = ws[lay["plan"]:lay["plan"] + 16 * n_facts].view(np.int32).reshape(n_facts, 4)
    arr = [ws[lay[k]:lay[k] + 4 * n_tok].view(np.int32).copy() for k in ("src_row", "pos", "slot")]
    return n_tok, n_facts, plan.copy(), arr


AGREE = [
    ("tiny_L1_H2_D64", {}),
    ("llama3_8b_k5", {}),
    ("llama3_8b_k50", {}),
    ("llama3_8b_k5", {"rope_style": 1, "key_layout": 1}),          # interleaved, chunk-local
    ("llama3_8b_k5", {"num_kv_heads": 1}),                          # 8 tokens per wave
]


@pytest.mark.parametrize("name,changes", AGREE,
                         ids=[n + "".join(f"_{k}{v}" for k, v in c.items()) for n, c in AGREE])
def test_fused_mapping_equals_separate_kernels(name, changes):
    w = workloads.make(workloads.with_spec(name, **changes))
    dw = harness.DeviceWorkload(w, host_mapping=False, gen_device="cuda")
    results = []
    for kw in MAPPINGS.values():
        dw.reset_cache()
        dw.setup_device_batch(**kw)
        dw.status.zero_()
        dw.inject_device()
        torch.cuda.synchronize()
        gk, gv = dw.listed_blocks_host(w.listed_blocks())
        results.append((int(dw.status.item()), _workspace_parts(dw), gk, gv,
                        dw.count_non_sentinel()))
    (s1, (n1, f1, p1, m1), k1, v1, c1), (s2, (n2, f2, p2, m2), k2, v2, c2) = results
    assert s1 == s2 == 0
    assert n1 == n2 == w.n_tokens and f1 == f2
    assert np.array_equal(p1, p2)
    assert all(np.array_equal(a, b) for a, b in zip(m1, m2))
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2) and c1 == c2
    sp = w.spec
    assert c1 == 2 * sp.num_layers * w.n_tokens * sp.num_kv_heads * sp.head_dim


@pytest.mark.parametrize("n_req", [FUSE_LIMIT, FUSE_LIMIT + 1])
def test_many_requests_at_the_fused_limit(n_req):
    """256 requests of one fact each fill the fused plan's request and fact
    arrays exactly; 257 take the separate kernels.  Both must meet the oracle
    and equal the host library's mapping."""
    facts = {f: 1 + f % 5 for f in range(16)}
    reqs = [([r % 16], r % 7) for r in range(n_req)]
    w = custom_workload(f"req{n_req}", 2, 2, 64, 16, facts, reqs, num_blocks=4096)
    dw = _device_run(w)
    assert int(dw.status.item()) == 0
    n, src, pos, slot = dw.device_mapping()
    req_ptr, ids, start, bt, bt_len = w.csr()
    host = prkv.build_slot_mapping(dw.store, req_ptr, ids, start, bt, bt_len, 16, w.num_blocks)
    assert n == w.n_tokens
    assert all(np.array_equal(a, b) for a, b in zip((src, pos, slot), host))
    _check(dw, w)


SHAPES = [(2, 1, 16), (3, 2, 64), (2, 8, 128)]      # (layers, KV heads, head_dim)
FAULTS = [None, "unknown_id", "short_table", "bad_block"]


@pytest.mark.parametrize("seed", range(64))
def test_random_small_batches_both_mappings(seed):
    """Seeded random small batches (repeated and absent ids, empty requests,
    block sizes 1-32, three head shapes), a quarter of them valid and the
    rest with one planted fault.  Valid: both device mappings equal the host
    library's build_slot_mapping and the caches meet the oracle.  Always:
    the fused and the separate-kernel mappings agree bit for bit (cache,
    workspace, status)."""
    rng = np.random.default_rng(5000 + seed)
    L, H, D = SHAPES[seed % len(SHAPES)]
    fault = FAULTS[(seed // len(SHAPES)) % len(FAULTS)]
    n_facts = int(rng.integers(1, 12))
    facts = {f: int(rng.integers(1, 40)) for f in range(n_facts)}
    reqs = []
    for r in range(int(rng.integers(1, 6))):
        k = int(rng.integers(1 if r == 0 else 0, 6))
        reqs.append(([int(x) for x in rng.integers(0, n_facts, size=k)], int(rng.integers(0, 100))))
    bs = int(rng.choice([1, 4, 16, 32]))
    w = custom_workload(f"rand{seed}", L, H, D, bs, facts, reqs, num_blocks=4096)

    def plant(dw):
        if fault == "unknown_id":
            dw.d_ids[int(rng.integers(0, len(dw.d_ids)))] = n_facts + 7
        elif fault == "short_table":
            dw.d_bt_len[0] = max(0, int(dw.d_bt_len[0].item()) - 1)
        elif fault == "bad_block":              # the block of request 0's first fact token
            dw.d_bt[0, reqs[0][1] // bs] = w.num_blocks + 1

    runs = []
    for kw in MAPPINGS.values():
        rng_state = rng.bit_generator.state
        dw = _device_run(w, patch=plant, **kw)
        rng.bit_generator.state = rng_state          # the same fault for both mappings
        gk, gv = dw.listed_blocks_host(w.listed_blocks())
        runs.append((int(dw.status.item()), _workspace_parts(dw), gk, gv, dw))
    (s1, (n1, f1, p1, m1), k1, v1, dw1), (s2, (n2, f2, p2, m2), k2, v2, _) = runs
    assert s1 == s2 and n1 == n2 and f1 == f2 and np.array_equal(p1, p2)
    assert all(np.array_equal(a, b) for a, b in zip(m1, m2))
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    if fault is None:
        assert s1 == 0 and n1 == w.n_tokens
        req_ptr, ids, start, bt, bt_len = w.csr()
        host = prkv.build_slot_mapping(dw1.store, req_ptr, ids, start, bt, bt_len, bs,
                                       w.num_blocks)
        assert all(np.array_equal(a, b) for a, b in zip(m1, host))
        _check(dw1, w)
    else:
        assert s1 != 0


def test_two_streams_inject_concurrently():
    """Two batches (the two halves of a batch's requests) injected at once on
    two HIP streams, host-mapped through inject_topk and device-mapped
    through inject_topk_device with separate workspaces: the cache equals one
    launch of the whole batch, bit for bit, and matches the oracle."""
    rng = np.random.default_rng(21)
    facts = {f: int(rng.integers(5, 60)) for f in range(60)}
    reqs = [([int(x) for x in rng.choice(60, size=int(rng.integers(3, 12)), replace=False)],
             int(rng.integers(0, 100))) for _ in range(6)]
    w = custom_workload("two_streams", 4, 8, 128, 16, facts, reqs, theta=5e5, num_blocks=1024)
    dw, rep, (img_k, img_v, want_k, want_v) = run_full(w, path="host")
    blocks = w.listed_blocks()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    n0 = sum(w.length_of(f) for ids, _ in reqs[:3] for f in ids)
    n = dw.n_tokens
    src, pos, slot = dw.d_map

    # host-mapped: tokens of requests 0-2 on one stream, 3-5 on the other
    dw.reset_cache()
    torch.cuda.synchronize()
    prkv.inject_topk(dw.store, n0, src[:n0], pos[:n0], slot[:n0], dw.k_layers(), dw.v_layers(),
                     16, w.num_blocks, d_status=dw.status, stream=s1)
    prkv.inject_topk(dw.store, n - n0, src[n0:], pos[n0:], slot[n0:], dw.k_layers(),
                     dw.v_layers(), 16, w.num_blocks, d_status=dw.status, stream=s2)
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    got_k, got_v = dw.listed_blocks_host(blocks)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)

    # device-mapped: each half its own device batch and workspace
    halves = []
    for r0 in (0, 3):
        part = reqs[r0:r0 + 3]
        sub = custom_workload("two_streams", 4, 8, 128, 16, facts, part, theta=5e5,
                              num_blocks=1024)
        req_ptr, ids, start, _, _ = sub.csr()
        bt = np.ascontiguousarray(dw.bt[r0:r0 + 3])
        btl = np.ascontiguousarray(dw.bt_len[r0:r0 + 3])
        d = [torch.from_numpy(np.ascontiguousarray(a)).cuda()
             for a in (req_ptr, ids, start, bt, btl)]
        max_tok = len(ids) * 60
        ws_b = prkv.inject_device_workspace_bytes(len(ids), max_tok)
        ws = torch.zeros(ws_b, dtype=torch.uint8, device="cuda")
        b = prkv.device_batch(3, bt.shape[1], len(ids), max_tok, *d)
        halves.append((b, ws, ws_b, d))
    dw.setup_device_batch()
    dw.reset_cache()
    torch.cuda.synchronize()
    for (b, ws, ws_b, _), s in zip(halves, (s1, s2)):
        prkv.inject_topk_device(dw.store, dw.fact_table, b, dw.k_layers(), dw.v_layers(), 16,
                                w.num_blocks, ws, ws_b, d_status=dw.status, stream=s)
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    got_k, got_v = dw.listed_blocks_host(blocks)
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)


@dataclasses.dataclass
class _SharedBlocks(workloads.Workload):
    """A workload whose block tables share blocks (listed once each)."""

    def listed_blocks(self):
        return sorted(set(super().listed_blocks()))


def _shared_block_workload(name, L=2, H=8, D=128):
    """Two requests; request 1's first block is request 0's second block, so
    positions 16 + o of request 0 and o of request 1 land in one slot."""
    facts = {0: 9, 1: 14, 2: 5, 3: 20}
    w = custom_workload(name, L, H, D, 16, facts, [([0, 1], 7), ([2, 3], 3)])
    bt0, bt1 = w.block_tables
    bt1 = bt1.copy()
    bt1[0] = bt0[1]
    fields = {f.name: getattr(w, f.name) for f in dataclasses.fields(w)}
    fields["block_tables"] = [bt0, bt1]
    return _SharedBlocks(**fields)


@pytest.mark.parametrize("max_facts", [None, FUSE_LIMIT + 44], ids=["small", "kernels"])
def test_duplicate_slots_detected_with_check_flag(max_facts):
    """With PRKV_BATCH_CHECK_SLOTS, tokens whose slot another token of the
    batch also maps to are all skipped (neither is written), status gets 128,
    and everything else matches the oracle; the host builder rejects the same
    batch with DUPLICATE_SLOT."""
    w = _shared_block_workload("dup_slots")
    dw = harness.DeviceWorkload(w, host_mapping=False)
    req_ptr, ids, start, bt, bt_len = w.csr()
    with pytest.raises(prkv.PrkvError) as err:
        prkv.build_slot_mapping(dw.store, req_ptr, ids, start, bt, bt_len, 16, w.num_blocks)
    assert err.value.name == "DUPLICATE_SLOT"
    dw.setup_device_batch(max_facts=max_facts, flags=prkv.BATCH_CHECK_SLOTS)
    dw.status.zero_()
    dw.inject_device()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 128
    src, _, slot = paged.token_mapping(w.requests(), w.fact_rows, 16)
    dups = sorted(s for s, c in Counter(slot).items() if c > 1)
    assert len(dups) == 11          # request 0's positions 19..29, request 1's 3..13
    # the device mapping marks exactly the colliding tokens as skipped
    n, d_src, _, d_slot = dw.device_mapping()
    assert n == len(slot) and np.array_equal(d_slot, np.array(slot, np.int32))
    skipped = {t for t, s in enumerate(slot) if s in set(dups)}
    assert all((d_src[t] == -1) == (t in skipped) for t in range(n))
    blocks = w.listed_blocks()
    img_k, img_v, mask = _expect(w, blocks, dups)
    gk, gv = dw.listed_blocks_host(blocks)
    compare(img_k, img_v, gk, gv, mask)
    sp = w.spec
    assert dw.count_non_sentinel() == \
        2 * sp.num_layers * int(mask.sum()) * sp.num_kv_heads * sp.head_dim


@pytest.mark.parametrize("name", ["tiny_L1_H2_D64", "llama3_8b_k5"])
def test_check_flag_on_a_valid_batch_changes_nothing(name):
    """A batch without duplicates: with the check the cache, status and
    mapping equal those of the unchecked step, bit for bit."""
    w = workloads.make(name)
    dw = harness.DeviceWorkload(w, host_mapping=False, gen_device="cuda")
    out = []
    for flags in (0, prkv.BATCH_CHECK_SLOTS):
        dw.reset_cache()
        dw.setup_device_batch(flags=flags)
        dw.status.zero_()
        dw.inject_device()
        torch.cuda.synchronize()
        gk, gv = dw.listed_blocks_host(w.listed_blocks())
        n, src, pos, slot = dw.device_mapping()
        out.append((int(dw.status.item()), n, src.copy(), pos.copy(), slot.copy(), gk, gv))
    a, b = out
    assert a[0] == b[0] == 0 and a[1] == b[1] == w.n_tokens
    assert all(np.array_equal(x, y) for x, y in zip(a[2:], b[2:]))
    _check(dw, w)


def test_check_flag_many_duplicates():
    """Two requests with identical block tables and prefixes: every position
    of request 0 (39 tokens) collides with request 1's (41 tokens), so only
    request 1's last two tokens and the third request are written."""
    facts = {f: 10 + 3 * f for f in range(8)}
    w = custom_workload("dup_all", 3, 4, 64, 16, facts,
                        [([0, 1, 2], 5), ([3, 4], 5), ([5, 6, 7], 2)], num_blocks=512)
    bts = list(w.block_tables)
    bts[1] = bts[0].copy()            # request 1 shares request 0's blocks
    fields = {f.name: getattr(w, f.name) for f in dataclasses.fields(w)}
    fields["block_tables"] = bts
    w = _SharedBlocks(**fields)
    dw = harness.DeviceWorkload(w, host_mapping=False)
    dw.setup_device_batch(flags=prkv.BATCH_CHECK_SLOTS)
    dw.status.zero_()
    dw.inject_device()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 128
    _, _, slot = paged.token_mapping(w.requests(), w.fact_rows, 16)
    dups = sorted(s for s, c in Counter(slot).items() if c > 1)
    assert len(dups) == sum(facts[f] for f in (0, 1, 2))
    blocks = w.listed_blocks()
    img_k, img_v, mask = _expect(w, blocks, dups)
    gk, gv = dw.listed_blocks_host(blocks)
    compare(img_k, img_v, gk, gv, mask)


@pytest.mark.parametrize("seed", range(16))
def test_random_shared_blocks_with_check(seed):
    """Seeded random small batches in which one request's block-table entry
    is replaced by a block of another request (so some of their slots may
    collide, or none if their offsets do not meet), through the checked
    device step (small and separate-kernel bounds alternate): exactly the
    colliding tokens are skipped, status is 128 iff there is a collision,
    and everything else meets the oracle."""
    rng = np.random.default_rng(7000 + seed)
    L, H, D = SHAPES[seed % len(SHAPES)]
    n_facts = int(rng.integers(2, 12))
    facts = {f: int(rng.integers(1, 40)) for f in range(n_facts)}
    reqs = [([int(x) for x in rng.integers(0, n_facts, size=int(rng.integers(1, 6)))],
             int(rng.integers(0, 60))) for _ in range(int(rng.integers(2, 5)))]
    bs = int(rng.choice([1, 4, 16, 32]))
    w = custom_workload(f"shared{seed}", L, H, D, bs, facts, reqs, num_blocks=4096)
    bts = [t.copy() for t in w.block_tables]
    r1, r2 = (int(x) for x in rng.choice(len(bts), 2, replace=False))
    bts[r2][int(rng.integers(0, len(bts[r2])))] = bts[r1][int(rng.integers(0, len(bts[r1])))]
    fields = {f.name: getattr(w, f.name) for f in dataclasses.fields(w)}
    fields["block_tables"] = bts
    w = _SharedBlocks(**fields)
    dw = harness.DeviceWorkload(w, host_mapping=False)
    dw.setup_device_batch(max_facts=None if seed % 2 else FUSE_LIMIT + 44,
                          flags=prkv.BATCH_CHECK_SLOTS)
    dw.status.zero_()
    dw.inject_device()
    torch.cuda.synchronize()
    _, _, slot = paged.token_mapping(w.requests(), w.fact_rows, bs)
    dups = sorted(s for s, c in Counter(slot).items() if c > 1)
    assert int(dw.status.item()) == (128 if dups else 0)
    n, d_src, _, _ = dw.device_mapping()
    assert n == len(slot)
    assert all((d_src[t] == -1) == (s in set(dups)) for t, s in enumerate(slot))
    blocks = w.listed_blocks()
    img_k, img_v, mask = _expect(w, blocks, dups)
    gk, gv = dw.listed_blocks_host(blocks)
    compare(img_k, img_v, gk, gv, mask)
