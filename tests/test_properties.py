"""Property tests (hypothesis) on random small batches and RoPE shapes, plus
determinism of the seeded input generator.

* the oracle's positions and slots obey the invariants of their definition
  (injective, one slot per fact token, inside the request's listed blocks,
  contiguous positions after the prefix in list order; chunk-local rotation
  position + index in fact = serving position);
* the host library's build_slot_mapping equals the oracle bit for bit, for
  pre-RoPE and chunk-local stores;
* RoPE keeps every pair's norm, composes relocations, is the identity at
  position 0, and its two pairings are conjugate by the even/odd permutation.
"""

import math

import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from oracle import paged, rope
from pre_rope_kv_amd import prkv, workloads

SETTINGS = settings(max_examples=60, deadline=None,
                    suppress_health_check=[HealthCheck.too_slow])


@st.composite
def batches(draw):
    n_facts = draw(st.integers(1, 10))
    lengths = draw(st.lists(st.integers(1, 20), min_size=n_facts, max_size=n_facts))
    bs = draw(st.sampled_from([1, 2, 3, 7, 16, 32, 63, 64, 65, 100, 130]))
    n_req = draw(st.integers(1, 3))
    order = draw(st.permutations(list(range(n_facts))))   # arena order of the facts
    rows, r = {}, 0
    for f in order:
        rows[f] = (r, lengths[f])
        r += lengths[f]
    reqs = []
    free = draw(st.permutations(list(range(400))))
    cur = 0
    for _ in range(n_req):
        ids = draw(st.lists(st.integers(0, n_facts - 1), max_size=5))   # repeats are legal
        prefix = draw(st.integers(0, 40))
        need = -(-(prefix + sum(lengths[f] for f in ids)) // bs)
        table = list(free[cur:cur + need])
        cur += need
        reqs.append((ids, prefix, table))
    return rows, reqs, bs, r


@SETTINGS
@given(batches())
def test_oracle_mapping_invariants(case):
    rows, reqs, bs, _ = case
    src, pos, slot = paged.token_mapping(reqs, rows, bs)
    local = paged.rotation_positions(reqs, rows, chunk_local=True)
    assert len(slot) == len(set(slot)) == sum(rows[f][1] for ids, _, _ in reqs for f in ids)
    t = 0
    for ids, prefix, table in reqs:
        p = prefix
        for f in ids:
            r0, ln = rows[f]
            for i in range(ln):
                assert src[t] == r0 + i and pos[t] == p + i
                assert slot[t] // bs in table and slot[t] % bs == (p + i) % bs
                assert local[t] + i == pos[t]
                t += 1
            p += ln
    assert paged.rotation_positions(reqs, rows, chunk_local=False) == pos


@SETTINGS
@given(batches(), st.booleans())
def test_library_mapping_equals_oracle(case, chunk_local):
    rows, reqs, bs, cap = case
    n_facts = len(rows)
    d = prkv.desc(1, 1, 16, n_facts, max(cap, 1), 16384, 1e4,
                  key_layout=prkv.KEYS_CHUNK_LOCAL if chunk_local else prkv.KEYS_PRE_ROPE)
    store = prkv.store_create(d)
    for f in sorted(rows, key=lambda f: rows[f][0]):        # puts in arena order
        prkv.store_put_fact(store, f, rows[f][1])
    stride = max(1, max(len(t) for _, _, t in reqs))
    bt = np.zeros((len(reqs), stride), np.int32)
    for i, (_, _, t) in enumerate(reqs):
        bt[i, :len(t)] = t
    req_ptr = np.cumsum([0] + [len(ids) for ids, _, _ in reqs]).astype(np.int32)
    ids = np.array([f for ids, _, _ in reqs for f in ids], np.int32)
    starts = np.array([p for _, p, _ in reqs], np.int32)
    bt_len = np.array([len(t) for _, _, t in reqs], np.int32)
    src, pos, slot = prkv.build_slot_mapping(store, req_ptr, ids, starts, bt, bt_len, bs, 400)
    o_src, _, o_slot = paged.token_mapping(reqs, rows, bs)
    o_pos = paged.rotation_positions(reqs, rows, chunk_local)
    assert src.tolist() == o_src and pos.tolist() == o_pos and slot.tolist() == o_slot


@SETTINGS
@given(st.sampled_from([2, 4, 8, 16, 32, 64]),
       st.floats(2.0, 1e6),
       st.lists(st.integers(0, 16383), min_size=1, max_size=6),
       st.integers(0, 16383),
       st.sampled_from([rope.HALF_SPLIT, rope.INTERLEAVED]),
       st.booleans(),
       st.integers(0, 2**32 - 1))
def test_rope_invariants(d, base, positions, delta, style, scaled, seed):
    scaling = rope.LLAMA31 if scaled else None
    x = np.random.default_rng(seed).standard_normal((len(positions), d))
    pos = np.array(positions)
    y = rope.rotate(x, pos, base, style=style, scaling=scaling)
    first, second = rope.pair_indices(d, style)
    assert np.allclose(np.hypot(y[:, first], y[:, second]), np.hypot(x[:, first], x[:, second]),
                       rtol=1e-12, atol=0)
    two = rope.rotate(y, np.full_like(pos, delta), base, style=style, scaling=scaling)
    one = rope.rotate(x, pos + delta, base, style=style, scaling=scaling)
    assert np.allclose(two, one, rtol=0, atol=1e-10 * math.sqrt(d))
    assert np.array_equal(rope.rotate(x, np.zeros_like(pos), base, style=style,
                                      scaling=scaling), x)
    if style == rope.INTERLEAVED:
        perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
        z = np.empty_like(x)
        z[:, perm] = rope.rotate(x[:, perm], pos, base, scaling=scaling)
        assert np.array_equal(y, z)


def test_generator_is_deterministic():
    for name in ("tiny_L1_H2_D64", "llama3_70b_batch16_k50"):
        a, b = workloads.make(name), workloads.make(name)
        assert np.array_equal(a.lengths, b.lengths) and np.array_equal(a.prefix, b.prefix)
        assert a.retrieved == b.retrieved and a.put_order == b.put_order
        assert all(np.array_equal(x, y) for x, y in zip(a.block_tables, b.block_tables))
    w = workloads.make("tiny_L1_H2_D64")
    for f in w.put_order[:5]:
        k1, v1 = w.fact_kv(f, device="cpu")
        k2, v2 = w.fact_kv(f, device="cpu")
        assert np.array_equal(k1.numpy(), k2.numpy()) and np.array_equal(v1.numpy(), v2.numpy())
