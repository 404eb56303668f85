"""GPU query-prefill attention over the injected paged cache (attend_paged),
Theorem 3 end to end.

Each request's whole context goes through the inject path: a prefix "fact"
at position 0, the retrieved facts, then the query's own K/V as a last
"fact", so every position the query attends to was written by inject.  The
expected output is the oracle's brute-force float64 attention over the same
prompt encoded in place (each key rotated at its absolute position, the
query rotated in float64).

Tolerance, from the arithmetic: the kernel's q and probabilities enter the
matrix cores as bf16 hi + lo pairs (relative error ~2^-16 per product) with
fp32 accumulation over <= ~2k keys, so against attention over the SAME cache
contents the error is ~1e-5 (bound used: 2e-4).  Against the in-place
prompt, K may also differ by 1 bf16 ulp in a few elements (the inject bar),
which moves a score by <= ~4e-4; bound used: 3e-3.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention, bf16, inject, rope
from pre_rope_kv_amd import harness, prkv, workloads

from test_gpu_parity import (_release_device_memory, _say, custom_workload,  # noqa: F401
                             rope_kwargs)

pytestmark = pytest.mark.gpu

TOL_SAME_CACHE = 2e-4
TOL_IN_PLACE = 3e-3


def context_workload(name, L, H, D, bs, prefix, fact_lens, q_len, n_req=1, seed=0, theta=5e5):
    """Request r: [prefix fact, its facts..., query fact], start position 0.
    q_len: the query fact's length, or a list of them per request (0: none)."""
    rng = np.random.default_rng(seed)
    facts, reqs, fid = {}, [], 0
    for r in range(n_req):
        ids = []
        ql = q_len[r] if isinstance(q_len, (list, tuple)) else q_len
        for ln in [prefix] + [int(x) for x in fact_lens[r]] + ([ql] if ql > 0 else []):
            facts[fid] = ln
            ids.append(fid)
            fid += 1
        reqs.append((ids, 0))
    # put order shuffled so rows are scattered in the arena
    order = list(facts)
    rng.shuffle(order)
    w = custom_workload(name, L, H, D, bs, {f: facts[f] for f in order}, reqs, theta=theta,
                        num_blocks=max(512, 4 * sum(facts.values()) // bs))
    return w


def expected(w, q_bits, q_len, hq, layers, gen):
    """Oracle attention over the prompt encoded in place: [len(layers)][n_req][Q][Hq][D]."""
    sp = w.spec
    out = np.zeros((len(layers), sp.n_requests, q_len, hq, sp.head_dim))
    for r, ids in enumerate(w.retrieved):
        ks, vs = [], []
        for f in ids:
            k, v = w.fact_kv(f, device=gen)
            ks.append(k.cpu().numpy().view(np.uint16))
            vs.append(v.cpu().numpy().view(np.uint16))
        k_all = np.concatenate(ks, 1)          # [L][ctx][H][D]
        v_all = np.concatenate(vs, 1)
        ctx = k_all.shape[1]
        pos = np.arange(ctx)
        q_pos = np.arange(ctx - q_len, ctx)
        q_rot = rope.rotate(bf16.bf16_bits_to_f64(q_bits[r]), q_pos[:, None], sp.rope_theta,
                            **rope_kwargs(sp))
        for li, l in enumerate(layers):
            kk = bf16.bf16_bits_to_f64(inject.rotate_k_bits(k_all[l], pos[:, None], sp.rope_theta,
                                                            **rope_kwargs(sp)))
            vv = bf16.bf16_bits_to_f64(v_all[l])
            out[li, r] = attention.causal_gqa(q_rot, q_pos, kk, vv, pos,
                                               1.0 / math.sqrt(sp.head_dim))
    return out


def from_cache(dw, q_bits, q_len, layers):
    """Oracle attention over the GPU cache's own K/V (isolates the kernel)."""
    sp = dw.w.spec
    out = np.zeros((len(layers), sp.n_requests, q_len, q_bits.shape[2], sp.head_dim))
    for r, ids in enumerate(dw.w.retrieved):
        ctx = sum(dw.w.length_of(f) for f in ids)
        bt = dw.w.block_tables[r]
        slots = torch.as_tensor([int(bt[p // sp.block_size]) * sp.block_size + p % sp.block_size
                                 for p in range(ctx)], device=dw.device)
        kr = dw.slot_rows(dw.k_cache, slots)   # [L][ctx][H][D] in either cache layout
        vr = dw.slot_rows(dw.v_cache, slots)
        pos = np.arange(ctx)
        q_pos = np.arange(ctx - q_len, ctx)
        q_rot = rope.rotate(bf16.bf16_bits_to_f64(q_bits[r]), q_pos[:, None], sp.rope_theta,
                            **rope_kwargs(sp))
        for li, l in enumerate(layers):
            kk = bf16.bf16_bits_to_f64(kr[l].cpu().numpy().view(np.uint16))
            vv = bf16.bf16_bits_to_f64(vr[l].cpu().numpy().view(np.uint16))
            out[li, r] = attention.causal_gqa(q_rot, q_pos, kk, vv, pos,
                                               1.0 / math.sqrt(sp.head_dim))
    return out


def run_attention(w, q_len, hq, gen="cuda", layers=None, seed=1, mutate_bt=None,
                  mutate_q_start=None):
    sp = w.spec
    dw = harness.DeviceWorkload(w, gen_device=gen)
    dw.inject()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q_bits = torch.randn((sp.n_requests, q_len, hq, sp.head_dim), generator=g) \
        .to(torch.bfloat16).view(torch.int16)
    ctxs = [sum(w.length_of(f) for f in ids) for ids in w.retrieved]
    q_start = torch.as_tensor([c - q_len for c in ctxs], dtype=torch.int32, device="cuda")
    bt = torch.from_numpy(np.ascontiguousarray(dw.bt)).cuda()
    bt_len = torch.from_numpy(dw.bt_len).cuda()
    if mutate_bt is not None:
        mutate_bt(bt, bt_len)
    if mutate_q_start is not None:
        mutate_q_start(q_start)
    q = q_bits.cuda()
    out = torch.full((sp.num_layers, sp.n_requests, q_len, hq, sp.head_dim), float("nan"),
                     dtype=torch.float32, device="cuda")
    batch = prkv.attn_batch(sp.n_requests, q_len, hq, bt.shape[1], q, q_start, bt, bt_len, out)
    dw.status.zero_()
    prkv.attend_paged(dw.store, batch, dw.k_layers(), dw.v_layers(), sp.block_size, w.num_blocks,
                      1.0 / math.sqrt(sp.head_dim), d_status=dw.status)
    torch.cuda.synchronize()
    layers = list(range(sp.num_layers)) if layers is None else layers
    got = out[layers].cpu().numpy().astype(np.float64)
    return dw, q_bits.numpy().view(np.uint16), got, layers


def check(dw, q_bits, got, q_len, hq, layers, gen):
    assert np.all(np.isfinite(got))
    same = from_cache(dw, q_bits, q_len, layers)
    place = expected(dw.w, q_bits, q_len, hq, layers, gen)
    e_same = float(np.max(np.abs(got - same)))
    e_place = float(np.max(np.abs(got - place)))
    _say(f"attention: max |gpu - oracle over gpu cache| = {e_same:.3g}, "
         f"max |gpu - oracle in place| = {e_place:.3g}, mean {np.mean(np.abs(got - place)):.3g}")
    assert e_same <= TOL_SAME_CACHE
    assert e_place <= TOL_IN_PLACE


def test_attention_tiny_shape():
    # tiny workload's shape: 1 layer, 2 KV heads, D 64, 8 query heads, 4 query tokens
    w = context_workload("attn_tiny", 1, 2, 64, 16, 32, [[17, 9, 30, 8, 21]], 4)
    dw, qb, got, layers = run_attention(w, 4, 8, gen="cpu")
    assert int(dw.status.item()) == 0
    check(dw, qb, got, 4, 8, layers, "cpu")


@pytest.mark.parametrize("bs", [16, 32])
def test_attention_llama_shape(bs):
    # Llama-3-8B per-layer shape (8 KV heads, 32 query heads, D 128), 16 query tokens
    rng = np.random.default_rng(bs)
    lens = [rng.integers(20, 61, size=10), rng.integers(20, 61, size=3)]
    w = context_workload(f"attn_llama_bs{bs}", 3, 8, 128, bs, 64, lens, 16, n_req=2, seed=bs)
    dw, qb, got, layers = run_attention(w, 16, 32)
    assert int(dw.status.item()) == 0
    check(dw, qb, got, 16, 32, layers, "cuda")


def test_attention_long_context_k50():
    # one request with 50 facts (~2k keys), two of its layers checked
    rng = np.random.default_rng(50)
    w = context_workload("attn_k50", 4, 8, 128, 16, 64, [rng.integers(20, 61, size=50)], 16,
                         seed=50)
    dw, qb, got, layers = run_attention(w, 16, 32, layers=[0, 3])
    assert int(dw.status.item()) == 0
    check(dw, qb, got, 16, 32, layers, "cuda")


def test_attention_missing_block_is_masked_and_reported():
    rng = np.random.default_rng(7)
    w = context_workload("attn_missing", 2, 8, 128, 16, 64, [rng.integers(20, 61, size=4)], 16)

    def drop_last(bt, bt_len):
        bt_len[0] -= 1

    dw, qb, got, layers = run_attention(w, 16, 32, mutate_bt=drop_last)
    assert int(dw.status.item()) == 4
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("bs,prefix,lens,q_len,hq,D", [
    (24, 40, [[7, 33, 12, 50]], 8, 8, 128),      # block size not a power of two
    (12, 5, [[9, 3]], 4, 4, 64),                 # context shorter than one key tile
    (16, 20, [[12]], 32, 2, 64),                 # context of exactly one 64-key span
    (16, 17, [[30, 31], [5]], 5, 6, 128),        # 15 rows per KV head (group 3), ragged
])
def test_attention_edge_shapes(bs, prefix, lens, q_len, hq, D):
    w = context_workload(f"attn_edge_{bs}_{D}_{q_len}", 2, 2, D, bs, prefix, lens, q_len,
                         n_req=len(lens), seed=bs + D)
    dw, qb, got, layers = run_attention(w, q_len, hq, gen="cpu")
    assert int(dw.status.item()) == 0
    check(dw, qb, got, q_len, hq, layers, "cpu")


@pytest.mark.parametrize("bs,D,H,hq,q_len,lens", [
    (16, 128, 2, 8, 40, [[30, 12, 41]]),       # 160 rows: three row blocks, the last 32 rows
    (24, 64, 2, 4, 33, [[9, 50], [17]]),       # 66 rows: a second block of 2 rows, ragged
    (16, 128, 8, 32, 64, [[35, 22, 48, 20]]),  # Llama-3-8B grouping, a 64-token question
    (32, 64, 3, 3, 100, [[60, 7]]),            # group 1: 100 rows, two blocks
])
def test_attention_long_queries(bs, D, H, hq, q_len, lens):
    """Queries longer than one workgroup's 64 (query token, query head) rows:
    the rows are split into blocks, each reading the keys up to its last
    query token."""
    w = context_workload(f"attn_long_{bs}_{D}_{H}_{q_len}", 2, H, D, bs, 20, lens, q_len,
                         n_req=len(lens), seed=q_len)
    dw, qb, got, layers = run_attention(w, q_len, hq, gen="cpu")
    assert int(dw.status.item()) == 0
    check(dw, qb, got, q_len, hq, layers, "cpu")


@pytest.mark.parametrize("bs,prefix,lens", [(1, 2000, [[40, 30]]), (2, 4100, [[57, 9]])])
def test_attention_block_table_beyond_lds(bs, prefix, lens):
    """Block tables longer than the 2048 entries staged in LDS are read from
    device memory (contexts of ~2,080 and ~4,170 positions at block sizes 1
    and 2: 2,078 and 2,087 table entries)."""
    w = context_workload(f"attn_longbt_{bs}", 2, 2, 64, bs, prefix, lens, 8, seed=bs)
    dw, qb, got, layers = run_attention(w, 8, 8, gen="cpu")
    assert dw.bt.shape[1] > 2048
    assert int(dw.status.item()) == 0
    check(dw, qb, got, 8, 8, layers, "cpu")


@pytest.mark.parametrize("H,hq,q_len,theta", [
    (4, 28, 12, 1e6),   # Qwen2.5-7B grouping (7 query heads per KV head): 84 rows, the
                        # 64-row block boundary falls inside query token 9's heads
    (8, 32, 16, 1e6),   # Mistral-7B grouping and RoPE base
])
def test_attention_evaluated_model_shapes(H, hq, q_len, theta):
    """Query prefill in the KV shapes of the other models the InferScale page
    evaluates (Qwen2.5-7B, Mistral-7B; D 128)."""
    rng = np.random.default_rng(H * 100 + hq)
    lens = [rng.integers(20, 61, size=6), rng.integers(20, 61, size=3)]
    w = context_workload(f"attn_models_{H}_{hq}", 2, H, 128, 16, 64, lens, q_len, n_req=2,
                         seed=hq, theta=theta)
    dw, qb, got, layers = run_attention(w, q_len, hq, gen="cpu")
    assert int(dw.status.item()) == 0
    check(dw, qb, got, q_len, hq, layers, "cpu")


def test_attention_ragged_query_lengths():
    """Per-request query lengths (q_lens) inside a padded q_len: each
    request's own rows against the oracle over the same cache, the padding
    rows exactly 0; a q_lens value out of range sets bit 8, is clamped, and
    leaves the other requests' outputs bit for bit unchanged."""
    qls = [16, 5, 0, 9, 1]
    rng = np.random.default_rng(77)
    lens = [rng.integers(5, 50, size=int(rng.integers(1, 5))) for _ in qls]
    L, H, D, bs, Q, hq = 2, 2, 128, 16, max(qls), 8
    w = context_workload("attn_ragged", L, H, D, bs, 20, lens, qls, n_req=len(qls), seed=77)
    dw = harness.DeviceWorkload(w, gen_device="cpu")
    dw.inject()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    ctxs = [sum(w.length_of(f) for f in ids) for ids in w.retrieved]
    g = torch.Generator(device="cpu")
    g.manual_seed(78)
    q_bits = torch.randn((len(qls), Q, hq, D), generator=g).to(torch.bfloat16).view(torch.int16)
    q_start = torch.as_tensor([c - ql for c, ql in zip(ctxs, qls)], dtype=torch.int32,
                              device="cuda")
    bt = torch.from_numpy(np.ascontiguousarray(dw.bt)).cuda()
    bt_len = torch.from_numpy(dw.bt_len).cuda()
    q = q_bits.cuda()

    def run(q_lens):
        out = torch.full((L, len(qls), Q, hq, D), float("nan"), dtype=torch.float32,
                         device="cuda")
        d_ql = torch.as_tensor(q_lens, dtype=torch.int32, device="cuda")
        ab = prkv.attn_batch(len(qls), Q, hq, bt.shape[1], q, q_start, bt, bt_len, out,
                             q_lens=d_ql)
        dw.status.zero_()
        prkv.attend_paged(dw.store, ab, dw.k_layers(), dw.v_layers(), bs, w.num_blocks,
                          1.0 / math.sqrt(D), d_status=dw.status)
        torch.cuda.synchronize()
        return out.cpu().numpy().astype(np.float64), int(dw.status.item())

    got, st = run(qls)
    assert st == 0
    worst = 0.0
    for r, (ql, ctx) in enumerate(zip(qls, ctxs)):
        assert np.all(got[:, r, ql:] == 0), r
        if ql == 0:
            continue
        b = w.block_tables[r]
        slots = torch.as_tensor([int(b[p // bs]) * bs + p % bs for p in range(ctx)],
                                device=dw.device)
        kr = dw.slot_rows(dw.k_cache, slots)
        vr = dw.slot_rows(dw.v_cache, slots)
        q_pos = np.arange(ctx - ql, ctx)
        q_rot = rope.rotate(bf16.bf16_bits_to_f64(q_bits[r, :ql].numpy().view(np.uint16)),
                            q_pos[:, None], 5e5)
        for l in range(L):
            want = attention.causal_gqa(q_rot, q_pos,
                                        bf16.bf16_bits_to_f64(kr[l].cpu().numpy().view(np.uint16)),
                                        bf16.bf16_bits_to_f64(vr[l].cpu().numpy().view(np.uint16)),
                                        np.arange(ctx), 1.0 / math.sqrt(D))
            worst = max(worst, float(np.max(np.abs(got[l, r, :ql] - want))))
    _say(f"ragged queries: max |gpu - oracle over gpu cache| = {worst:.3g}")
    assert worst <= TOL_SAME_CACHE
    bad, st = run([-1] + qls[1:])
    assert st == 8
    assert np.all(bad[:, 0] == 0)
    assert np.array_equal(bad[:, 1:], got[:, 1:])


@pytest.mark.parametrize("D,H,hq,q_len", [(64, 8, 32, 16), (128, 8, 32, 7)])
def test_attention_one_key_group_grids(D, H, hq, q_len):
    """Grids of more than one workgroup per CU (here 2 layers x 20 requests x
    8 KV heads = 320) take the one-key-group kernel; small grids, as in most
    tests here, take three key groups."""
    rng = np.random.default_rng(D + q_len)
    lens = [rng.integers(3, 40, size=int(rng.integers(1, 4))) for _ in range(20)]
    w = context_workload(f"attn_kg1_{D}_{q_len}", 2, H, D, 16, 9, lens, q_len, n_req=20,
                         seed=D + q_len)
    dw, qb, got, layers = run_attention(w, q_len, hq, gen="cpu")
    assert int(dw.status.item()) == 0
    check(dw, qb, got, q_len, hq, layers, "cpu")


def random_attention_case(seed):
    """A seeded random attention shape: head dim, KV heads, group size, block
    size (powers of two and not), layers, requests, prefix and fact lengths,
    query length, RoPE base and cache layout.  Odd seeds have grids of more
    than one workgroup per CU (the one-key-group kernel), even seeds small
    ones (three key groups); tile counts take every value modulo the ring
    depth."""
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.choice([64, 128]))
    group = int(rng.choice([1, 2, 3, 4, 7]))
    bs = int(rng.choice([1, 2, 3, 5, 8, 16, 24, 32]))
    if seed % 2:     # at least 3 x 11 x 8 = 264 workgroups: the one-key-group kernel
        H, L, n_req = 8, int(rng.integers(3, 5)), int(rng.integers(11, 15))
    else:
        H, L, n_req = int(rng.choice([1, 2, 4, 8])), int(rng.integers(1, 5)), int(rng.integers(1, 7))
    q_len = int(rng.integers(1, 25))
    prefix = int(rng.integers(1, 200))
    lens = [rng.integers(1, 81, size=int(rng.integers(0, 7))) for _ in range(n_req)]
    theta = float(rng.choice([1e4, 5e5]))
    layout = int(rng.integers(0, 2))
    w = context_workload(f"attn_rand_{seed}", L, H, D, bs, prefix, lens, q_len, n_req=n_req,
                         seed=seed, theta=theta)
    if layout:
        w = workloads.dataclasses.replace(
            w, spec=workloads.dataclasses.replace(w.spec, cache_layout=prkv.CACHE_HND))
    return w, q_len, H * group


@pytest.mark.parametrize("seed", range(12))
def test_attention_random_shapes(seed):
    w, q_len, hq = random_attention_case(seed)
    sp = w.spec
    grid = sp.num_layers * sp.n_requests * sp.num_kv_heads * -(-q_len * (hq // sp.num_kv_heads) // 64)
    _say(f"seed {seed}: D {sp.head_dim}, H {sp.num_kv_heads}, {hq} query heads, bs "
         f"{sp.block_size}, L {sp.num_layers}, {sp.n_requests} requests, q_len {q_len}, "
         f"layout {'HND' if sp.cache_layout else 'NHD'}, grid {grid}")
    dw, qb, got, layers = run_attention(w, q_len, hq, gen="cpu", seed=seed)
    assert int(dw.status.item()) == 0
    check(dw, qb, got, q_len, hq, layers, "cpu")


def test_attention_query_positions_out_of_range_are_reported():
    # request 0 starts past max_position - q_len, request 1 before 0: both are
    # reported (bit 2) and produce 0; request 2 is unaffected
    rng = np.random.default_rng(3)
    lens = [rng.integers(5, 40, size=4) for _ in range(3)]
    w = context_workload("attn_qpos", 2, 2, 128, 16, 20, lens, 8, n_req=3, seed=3)
    _, qb0, ref, layers = run_attention(w, 8, 8, gen="cpu")
    max_pos = w.spec.max_position

    def bad_starts(q_start):
        q_start[0] = max_pos - 8 + 1
        q_start[1] = -1

    dw, qb, got, _ = run_attention(w, 8, 8, gen="cpu", mutate_q_start=bad_starts)
    assert int(dw.status.item()) == 2
    assert np.all(got[:, :2] == 0)
    assert np.array_equal(got[:, 2], ref[:, 2])


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name,layers,layout", [("llama3_8b_batch64_k50", (0, 11, 22, 31), 0),
                                                ("llama3_70b_batch16_k50", (0, 26, 53, 79), 0),
                                                ("llama3_8b_batch64_k50", (5, 17, 29), 1)])
def test_attention_full_size(name, layers, layout):
    """The launch the bench times: the whole batch injected by the device
    path into a zeroed cache, then one attend_paged over every request's
    whole context (16 query tokens = the context's last 16 positions, 4 query
    heads per KV head, all layers); the outputs of every request at the
    listed layers (first, last and between) against the oracle's attention
    over the same cache contents (one layer's K and V gathered at a time,
    (layer, request) pairs spread over host threads).  layout 1: the HND
    cache layout."""
    from concurrent.futures import ThreadPoolExecutor

    from test_gpu_parity import _oracle_threads
    spec = workloads.dataclasses.replace(workloads.SPECS[name], cache_layout=layout)
    w0 = workloads.make(spec)
    nb = harness.fit_num_blocks(spec, 2 * w0.capacity_rows * spec.num_layers * spec.row_bytes +
                                (3 << 30))
    w = w0 if nb == spec.num_blocks else workloads.make(spec, num_blocks=nb)
    dw = harness.DeviceWorkload(w, host_mapping=False)
    dw.setup_device_batch()
    dw.k_cache.zero_()
    dw.v_cache.zero_()
    dw.inject_device()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    q_len, hq, D, L = 16, 4 * spec.num_kv_heads, spec.head_dim, spec.num_layers
    ctxs = [int(w.prefix[r]) + sum(w.length_of(f) for f in ids)
            for r, ids in enumerate(w.retrieved)]
    g = torch.Generator(device="cpu")
    g.manual_seed(17)
    q_bits = torch.randn((spec.n_requests, q_len, hq, D), generator=g) \
        .to(torch.bfloat16).view(torch.int16)
    q_start = torch.as_tensor([c - q_len for c in ctxs], dtype=torch.int32, device="cuda")
    out = torch.full((L, spec.n_requests, q_len, hq, D), float("nan"), dtype=torch.float32,
                     device="cuda")
    batch = prkv.attn_batch(spec.n_requests, q_len, hq, dw.d_bt.shape[1], q_bits.cuda(), q_start,
                            dw.d_bt, dw.d_bt_len, out)
    dw.status.zero_()
    prkv.attend_paged(dw.store, batch, dw.k_layers(), dw.v_layers(), spec.block_size,
                      w.num_blocks, 1.0 / math.sqrt(D), d_status=dw.status)
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    assert bool(torch.isfinite(out).all())
    # every request's context positions, as cache slots, concatenated
    bs = spec.block_size
    starts = np.concatenate([[0], np.cumsum(ctxs)])
    slots = np.concatenate([np.asarray(w.block_tables[r], np.int64)[np.arange(c) // bs] * bs +
                            np.arange(c) % bs for r, c in enumerate(ctxs)])
    d_slots = torch.as_tensor(slots, device=dw.device)
    q_rot = [rope.rotate(bf16.bf16_bits_to_f64(q_bits[r].numpy().view(np.uint16)),
                         np.arange(c - q_len, c)[:, None], spec.rope_theta, **rope_kwargs(spec))
             for r, c in enumerate(ctxs)]
    kv = {l: (dw.slot_rows_layer(dw.k_cache, l, d_slots).cpu().numpy().view(np.uint16),
              dw.slot_rows_layer(dw.v_cache, l, d_slots).cpu().numpy().view(np.uint16),
              out[l].cpu().numpy().astype(np.float64)) for l in layers}

    def one(pair):
        l, r = pair
        kl, vl, got = kv[l]
        a, b, c = starts[r], starts[r + 1], ctxs[r]
        want = attention.causal_gqa(q_rot[r], np.arange(c - q_len, c),
                                    bf16.bf16_bits_to_f64(kl[a:b]), bf16.bf16_bits_to_f64(vl[a:b]),
                                    np.arange(c), 1.0 / math.sqrt(D))
        return float(np.max(np.abs(got[r] - want)))

    pairs = [(l, r) for l in layers for r in range(spec.n_requests)]
    with ThreadPoolExecutor(_oracle_threads()) as pool:
        worst = max(pool.map(one, pairs))
    _say(f"{name}: {len(pairs)} (layer, request) outputs (every request at layers {layers}), "
         f"max |gpu - oracle over gpu cache| = {worst:.3g}")
    assert worst <= TOL_SAME_CACHE
