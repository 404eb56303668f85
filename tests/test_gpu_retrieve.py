"""GPU exact top-k retrieval against the oracle, and retrieve -> inject end
to end.

Scores are float64 sums of exact bf16 products on both sides; the ranking is
compared id for id.  Where two oracle scores are closer than 1e-12 (a near
tie that float64 rounding may order either way) only the set is compared and
the order is checked to be valid.
"""

import dataclasses

import numpy as np
import pytest
import torch

from oracle import retrieve
from pre_rope_kv_amd import harness, prkv, workloads

from test_gpu_parity import (_full_size, _release_device_memory, check_device_mapping,  # noqa: F401
                             compare, oracle_images, written_mask, _say)

pytestmark = pytest.mark.gpu

TIE = 1e-12


def run_retrieve(emb, q, req_store, F, k, dim, n_stores):
    """emb: device int16 [n_stores*F][dim]; q: device int16 [n_req][dim]."""
    n_req = q.shape[0]
    ids = torch.full((n_req * k,), -7, dtype=torch.int32, device="cuda")
    sc = torch.zeros(n_req * k, dtype=torch.float64, device="cuda")
    ws_bytes = prkv.retrieve_workspace_bytes(n_req, F)
    ws = torch.empty(max(ws_bytes, 8), dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_rs = torch.as_tensor(req_store, dtype=torch.int32, device="cuda")
    prkv.retrieve_topk(emb, n_stores, F, dim, q, d_rs, n_req, k, ids, ws, ws_bytes, d_scores=sc,
                       d_status=status)
    torch.cuda.synchronize()
    return ids.view(n_req, k).cpu().numpy(), sc.view(n_req, k).cpu().numpy(), int(status.item())


def check_against_oracle(emb_h, q_h, req_store, F, k, ids, sc):
    """emb_h [n_stores][F][dim], q_h [n_req][dim] (uint16 bits)."""
    for r in range(q_h.shape[0]):
        s = int(req_store[r])
        score = retrieve.scores(q_h[r], emb_h[s])
        want = retrieve.topk(score, k)
        got = ids[r] - s * F
        assert np.allclose(sc[r], score[want], rtol=0, atol=1e-13 * (1 + np.abs(score[want])))
        if np.array_equal(got, want):
            continue
        # near ties only: same set of best scores, order valid
        boundary = score[want[-1]]
        gs = score[got]
        assert np.all(np.diff(gs) <= TIE), "GPU ranking not in score order"
        assert set(got[gs > boundary + TIE]) == set(want[score[want] > boundary + TIE])
        assert np.all(np.abs(gs - score[want]) <= TIE)


def _embeddings(w, device="cuda"):
    embs = [w.store_embeddings(s, device) for s in range(w.spec.n_requests)]
    return embs, torch.cat(embs, 0).contiguous()


@pytest.mark.parametrize("name", workloads.ORDER)
def test_retrieve_matches_oracle(name):
    w = workloads.make(name)
    sp = w.spec
    embs, emb = _embeddings(w)
    q = w.query_embeddings("cuda", emb=embs)
    ids, sc, st = run_retrieve(emb, q, w.req_store(), sp.facts_per_store, sp.k, sp.emb_dim,
                               sp.n_requests)
    assert st == 0
    emb_h = emb.cpu().numpy().view(np.uint16).reshape(sp.n_requests, sp.facts_per_store, -1)
    check_against_oracle(emb_h, q.cpu().numpy().view(np.uint16), w.req_store(),
                         sp.facts_per_store, sp.k, ids, sc)
    # the synthetic queries are built around the drawn facts: same set retrieved
    same = sum(set(ids[r]) == set(w.retrieved[r]) for r in range(sp.n_requests))
    _say(f"{name}: {same}/{sp.n_requests} requests retrieve exactly their drawn facts")
    assert same == sp.n_requests


@pytest.mark.parametrize("F,k,dim", [(1, 1, 512), (1003, 64, 512), (777, 7, 4096),
                                     (64, 64, 1024), (5000, 50, 2560),
                                     # widths that are not multiples of 512: a partial
                                     # last chunk (384, 768, 1000, 8) or a single one
                                     (2000, 50, 384), (1500, 20, 768), (300, 64, 1000),
                                     (100, 10, 8), (257, 5, 4088),
                                     # more than 2,048 scores per top-k workgroup (16
                                     # slices of 2,500 / 4,375): the waves run 3-5
                                     # chunk rounds before the lists are merged
                                     (40000, 50, 512), (70000, 64, 256)])
def test_retrieve_shapes(F, k, dim):
    g = torch.Generator(device="cuda")
    g.manual_seed(F * 131 + k * 7 + dim)
    n_stores, n_req = 3, 5
    emb = (torch.randn((n_stores * F, dim), generator=g, device="cuda") / dim ** 0.5)
    emb = emb.to(torch.bfloat16).view(torch.int16)
    q = (torch.randn((n_req, dim), generator=g, device="cuda") / dim ** 0.5)
    q = q.to(torch.bfloat16).view(torch.int16)
    req_store = np.array([0, 2, 1, 2, 0], np.int32)
    ids, sc, st = run_retrieve(emb, q, req_store, F, k, dim, n_stores)
    assert st == 0
    check_against_oracle(emb.cpu().numpy().view(np.uint16).reshape(n_stores, F, dim),
                         q.cpu().numpy().view(np.uint16), req_store, F, k, ids, sc)


@pytest.mark.parametrize("F", [300, 16384])
def test_retrieve_exact_ties_order_by_id(F):
    """Duplicate embeddings score identically: the smaller fact id ranks first
    (F = 16384: one request's scores are split over 16 top-k workgroups, and
    the duplicates fall in different slices)."""
    dim, k = 512, 20
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    base = (torch.randn((F, dim), generator=g, device="cuda") / dim ** 0.5).to(torch.bfloat16)
    h = F // 2
    base[h:2 * h] = base[:h]         # fact f and f + F/2 are identical
    q = base[10:11].clone()          # query equals fact 10 (and 10 + F/2)
    emb = base.view(torch.int16).contiguous()
    ids, sc, st = run_retrieve(emb, q.view(torch.int16), np.array([0], np.int32), F, k, dim, 1)
    assert ids[0][0] == 10 and ids[0][1] == 10 + h
    check_against_oracle(emb.cpu().numpy().view(np.uint16)[None], q.view(torch.int16).cpu()
                         .numpy().view(np.uint16), [0], F, k, ids, sc)


@pytest.mark.parametrize("F", [50, 8192])
def test_retrieve_bad_store_reports(F):
    dim, k = 512, 5
    emb = torch.zeros((F, dim), dtype=torch.int16, device="cuda")
    q = torch.zeros((2, dim), dtype=torch.int16, device="cuda")
    ids, sc, st = run_retrieve(emb, q, np.array([0, 3], np.int32), F, k, dim, 1)
    assert st == 64
    assert np.all(ids[1] == -1)
    assert list(ids[0]) == [0, 1, 2, 3, 4]   # all scores 0: id order


def _oracle_ids_of(sp, emb, q):
    """The oracle's top-k of each request's own store (request r searches
    store r) for device embeddings and queries: global fact ids, best first."""
    emb_h = emb.cpu().numpy().view(np.uint16).reshape(sp.n_requests, sp.facts_per_store, -1)
    q_h = q.cpu().numpy().view(np.uint16)
    return [[int(r * sp.facts_per_store + f)
             for f in retrieve.topk(retrieve.scores(q_h[r], emb_h[r]), sp.k)]
            for r in range(sp.n_requests)]


def _oracle_ids(w):
    """The oracle's top-k for the workload's own embeddings and queries."""
    embs, emb = _embeddings(w)
    q = w.query_embeddings("cuda", emb=embs)
    del embs
    return _oracle_ids_of(w.spec, emb, q)


def _retrieve_then_inject(dw, w_drawn):
    """retrieve_topk over the embeddings of w_drawn (the workload as drawn:
    its embeddings and queries depend on the rank order of its facts) writes
    the fact ids into the device batch, inject_topk_device injects them: the
    ids must be dw's (the oracle's top-k order, set by the caller), the
    device mapping the oracle's."""
    w, sp = dw.w, dw.w.spec
    embs, emb = _embeddings(w_drawn)
    q = w_drawn.query_embeddings("cuda", emb=embs)
    del embs
    dw.setup_device_batch()
    dw.d_ids.fill_(-1)
    ws_bytes = prkv.retrieve_workspace_bytes(sp.n_requests, sp.facts_per_store)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    d_rs = torch.as_tensor(w.req_store(), device="cuda")
    prkv.retrieve_topk(emb, sp.n_requests, sp.facts_per_store, sp.emb_dim, q, d_rs,
                       sp.n_requests, sp.k, dw.d_ids, ws, ws_bytes, d_status=dw.status)
    dw.inject_device()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    got = dw.d_ids.cpu().numpy().reshape(sp.n_requests, sp.k)
    assert [list(map(int, row)) for row in got] == [list(map(int, r)) for r in w.retrieved]
    check_device_mapping(dw)


@pytest.mark.parametrize("name", ["tiny_L1_H2_D64", "llama3_8b_k50"])
def test_retrieve_then_inject(name):
    """retrieve_topk writes the fact ids straight into the device batch;
    inject_topk_device then injects them.  Expected: the oracle's own top-k
    (from the embeddings) injected by the oracle."""
    w = workloads.make(name)
    sp = w.spec
    gen = "cpu" if name.startswith("tiny") else "cuda"
    embs, emb = _embeddings(w)
    q = w.query_embeddings("cuda", emb=embs)
    assert list(w.req_store()) == list(range(sp.n_requests))   # request r searches store r
    oracle_ids = _oracle_ids_of(sp, emb, q)
    dw = harness.DeviceWorkload(w, gen_device=gen, host_mapping=False)
    dw.setup_device_batch()
    dw.d_ids.fill_(-1)
    ws_bytes = prkv.retrieve_workspace_bytes(sp.n_requests, sp.facts_per_store)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    d_rs = torch.as_tensor(w.req_store(), device="cuda")
    prkv.retrieve_topk(emb, sp.n_requests, sp.facts_per_store, sp.emb_dim, q, d_rs,
                       sp.n_requests, sp.k, dw.d_ids, ws, ws_bytes, d_status=dw.status)
    dw.inject_device()
    torch.cuda.synchronize()
    assert int(dw.status.item()) == 0
    w_oracle = dataclasses.replace(w, retrieved=oracle_ids)
    assert w_oracle.n_tokens == w.n_tokens
    blocks = w.listed_blocks()
    img_k, img_v, _ = oracle_images(w_oracle, gen)
    gk, gv = dw.listed_blocks_host(blocks)
    compare(img_k, img_v, gk, gv, written_mask(w_oracle, blocks))
    assert dw.count_non_sentinel() == 2 * sp.num_layers * w.n_tokens * sp.num_kv_heads * sp.head_dim


@pytest.mark.timeout(900)
def test_retrieve_then_inject_batch64_full_size():
    """The 64-request batch end to end at full size: retrieve_topk's ids (the
    oracle's top-k and the drawn facts) injected by inject_topk_device, every
    K and V element of every request checked against the oracle."""
    drawn = {}

    def in_retrieval_order(w):
        # the queries are built around the drawn facts: the oracle retrieves
        # exactly those sets (checked), in the order of their scores
        ids = _oracle_ids(w)
        assert [sorted(r) for r in ids] == [sorted(map(int, r)) for r in w.retrieved]
        drawn["w"] = w
        return dataclasses.replace(w, retrieved=ids)

    _full_size("llama3_8b_batch64_k50", paths=("retrieve",), prepare=in_retrieval_order,
               via=lambda dw, path: _retrieve_then_inject(dw, drawn["w"]))


@pytest.mark.parametrize("seed", range(12))
def test_retrieve_random_shapes(seed):
    """Seeded random shapes: requests, stores, facts per store (1 to 12,000),
    k (1 to min(64, F)), width (a multiple of 8 up to 2,048), duplicated
    embeddings (exact ties across the store) and the store each request
    reads; ids and scores against the oracle's, request by request."""
    rng = np.random.default_rng(1000 + seed)
    n_stores = int(rng.integers(1, 4))
    F = int(np.exp(rng.uniform(0, np.log(12000))))
    F = max(1, min(F, 12000))
    k = int(rng.integers(1, min(64, F) + 1))
    dim = 8 * int(rng.integers(1, 257))
    n_req = int(rng.integers(1, 25))
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    emb = (torch.randn((n_stores * F, dim), generator=g, device="cuda") / dim ** 0.5)
    emb = emb.to(torch.bfloat16)
    if F >= 4:   # a quarter of each store's rows duplicated elsewhere in it: exact ties
        for s in range(n_stores):
            src = torch.as_tensor(rng.integers(0, F, F // 4), device="cuda") + s * F
            dst = torch.as_tensor(rng.integers(0, F, F // 4), device="cuda") + s * F
            emb[dst] = emb[src]
    emb = emb.view(torch.int16).contiguous()
    req_store = rng.integers(0, n_stores, n_req).astype(np.int32)
    # queries: a stored row plus noise, so each request has clear leaders
    rows = torch.as_tensor(req_store.astype(np.int64) * F + rng.integers(0, F, n_req),
                           device="cuda")
    q = emb.view(torch.bfloat16)[rows].float() + \
        0.3 * torch.randn((n_req, dim), generator=g, device="cuda") / dim ** 0.5
    q = q.to(torch.bfloat16).view(torch.int16).contiguous()
    ids, sc, st = run_retrieve(emb, q, req_store, F, k, dim, n_stores)
    assert st == 0
    check_against_oracle(emb.cpu().numpy().view(np.uint16).reshape(n_stores, F, dim),
                         q.cpu().numpy().view(np.uint16), req_store, F, k, ids, sc)


def test_retrieve_nan_scores_rank_last():
    """Facts whose embedding holds a NaN score NaN: they rank below every
    number, among themselves by id (the oracle's sort puts NaN last the same
    way), and their scores come back NaN."""
    F, dim, k = 100, 64, 20
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    emb = (torch.randn((F, dim), generator=g, device="cuda") / dim ** 0.5).to(torch.bfloat16)
    emb = emb.view(torch.int16).contiguous()
    emb[:90, 7] = 0x7FC0                 # bf16 quiet NaN in rows 0..89
    q = (torch.randn((1, dim), generator=g, device="cuda") / dim ** 0.5).to(torch.bfloat16)
    q = q.view(torch.int16).contiguous()
    ids, sc, st = run_retrieve(emb, q, np.array([0], np.int32), F, k, dim, 1)
    assert st == 0
    score = retrieve.scores(q.cpu().numpy().view(np.uint16)[0], emb.cpu().numpy().view(np.uint16))
    want = retrieve.topk(score, k)
    assert np.isnan(score[:90]).all() and np.isfinite(score[90:]).all()
    assert list(want) == list(np.argsort(-score[90:], kind="stable") + 90) + list(range(10))
    assert list(ids[0]) == list(want)
    assert np.allclose(sc[0][:10], score[want[:10]], rtol=0, atol=1e-13)
    assert np.isnan(sc[0][10:]).all()
