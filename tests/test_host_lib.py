"""CPU tests of libprkv.so's host half: exports, fact table, slot mapping,
RoPE table and every error path that can be forced without a GPU.

None of these make a HIP compute call: stores are metadata-only (NULL device
pointers), and device-side entry points are only driven into argument errors
that are raised before anything touches the HIP runtime.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from oracle import paged, rope
from pre_rope_kv_amd import prkv, workloads

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "prkv.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|void|char)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_header_function():
    names = header_functions()
    assert "inject_topk" in names and "build_slot_mapping" in names
    L = prkv.lib()
    for n in names:
        assert hasattr(L, n), f"libprkv.so does not export {n}"
    assert sorted(prkv.EXPORTS) == names


def test_error_codes_match_header():
    text = open(HEADER).read()
    for name, code in re.findall(r"PRKV_ERR_(\w+)\s*=\s*(-\d+)", text):
        assert prkv.ERRORS[int(code)] == name


def _desc(**kw):
    base = dict(num_layers=2, num_kv_heads=2, head_dim=64, max_facts=16, capacity_rows=100,
                max_position=256, rope_theta=1e4)
    base.update(kw)
    return prkv.desc(**base)


def test_required_bytes():
    d = _desc()
    arena, table = prkv.store_required_bytes(d)
    assert arena == 2 * 100 * 2 * 64 * 2
    assert table == 256 * 32 * 16


LLAMA31 = (8.0, 1.0, 4.0, 8192)


@pytest.mark.parametrize("bad", [
    dict(num_layers=0), dict(num_layers=129), dict(num_kv_heads=0), dict(head_dim=96),
    dict(head_dim=8), dict(head_dim=2048), dict(max_facts=0), dict(capacity_rows=0),
    dict(capacity_rows=2**31), dict(max_position=0), dict(rope_theta=1.0),
    dict(rope_theta=float("nan")), dict(rope_style=2), dict(rope_style=-1),
    dict(key_layout=2), dict(llama3_scaling=(0.5, 1.0, 4.0, 8192)),
    dict(llama3_scaling=(8.0, 4.0, 1.0, 8192)), dict(llama3_scaling=(8.0, 0.0, 4.0, 8192)),
    dict(llama3_scaling=(8.0, 1.0, 4.0, 0)), dict(llama3_scaling=(float("inf"), 1.0, 4.0, 8192)),
    dict(raw=("rope_scaling", 2)), dict(raw=("cache_layout", 2)),
])
def test_bad_descriptor(bad):
    raw = bad.pop("raw", None)
    d = _desc(**bad)
    if raw:
        setattr(d, *raw)
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.store_create(d)
    assert ei.value.name == "INVALID_ARG"


def test_variant_descriptors_accepted():
    for kw in (dict(rope_style=1), dict(key_layout=1), dict(llama3_scaling=LLAMA31),
               dict(rope_style=1, key_layout=1, llama3_scaling=LLAMA31)):
        prkv.store_destroy(prkv.store_create(_desc(**kw)))


def test_store_create_pointer_rules():
    d = _desc()
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.lib()  # partial device pointers
        h = ctypes.c_void_p()
        prkv._check(prkv.lib().store_create(ctypes.byref(d), 4096, None, None, None,
                                            ctypes.byref(h)), "store_create")
    assert ei.value.name == "INVALID_ARG"
    with pytest.raises(prkv.PrkvError) as ei:
        h = ctypes.c_void_p()
        prkv._check(prkv.lib().store_create(ctypes.byref(d), 4104, 4096, 4096, None,
                                            ctypes.byref(h)), "store_create")
    assert ei.value.name == "ALIGNMENT"


def test_fact_table_and_put_errors():
    st = prkv.store_create(_desc())
    prkv.store_put_fact(st, 3, 10)
    prkv.store_put_fact(st, 0, 5)
    assert prkv.store_fact_info(st, 3) == (0, 10)
    assert prkv.store_fact_info(st, 0) == (10, 5)
    cases = [((3, 4), "DUPLICATE_FACT"), ((16, 4), "CAPACITY"), ((-1, 4), "CAPACITY"),
             ((5, 0), "INVALID_ARG"), ((5, 86), "CAPACITY")]
    for (fid, ln), name in cases:
        with pytest.raises(prkv.PrkvError) as ei:
            prkv.store_put_fact(st, fid, ln)
        assert ei.value.name == name
    # a failed put leaves the table unchanged
    prkv.store_put_fact(st, 5, 85)
    assert prkv.store_fact_info(st, 5) == (15, 85)
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.store_fact_info(st, 7)
    assert ei.value.name == "UNKNOWN_FACT"
    # sources given to a metadata-only store
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.store_put_fact(st, 9, 1, k_src=4096, v_src=4096, stream=0)
    assert ei.value.name == "CAPACITY"  # capacity is checked first (100 rows used)


def test_put_sources_need_device_store():
    st = prkv.store_create(_desc())
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.store_put_fact(st, 1, 2, k_src=4096, v_src=4096, stream=0)
    assert ei.value.name == "NO_DEVICE"
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.store_put_fact(st, 1, 2, k_src=4096, v_src=None, stream=0)
    assert ei.value.name == "INVALID_ARG"


def test_inject_rejects_metadata_only_store():
    st = prkv.store_create(_desc())
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.inject_topk(st, 1, 4096, 4096, 4096, [4096, 4096], [4096, 4096], 16, 4, stream=0)
    assert ei.value.name == "NO_DEVICE"


def _load_workload_store(w):
    sp = w.spec
    d = prkv.desc(sp.num_layers, sp.num_kv_heads, sp.head_dim, w.max_facts, w.capacity_rows,
                  sp.max_position, sp.rope_theta)
    st = prkv.store_create(d)
    for f in w.put_order:
        prkv.store_put_fact(st, f, w.length_of(f))
    return st


@pytest.mark.parametrize("name", workloads.ORDER)
def test_slot_mapping_matches_oracle(name):
    w = workloads.make(name)
    st = _load_workload_store(w)
    for f in w.put_order[:50]:
        assert prkv.store_fact_info(st, f) == w.fact_rows[f]
    req_ptr, ids, start, bt, bt_len = w.csr()
    src, pos, slot = prkv.build_slot_mapping(st, req_ptr, ids, start, bt, bt_len,
                                             w.spec.block_size, w.num_blocks)
    o_src, o_pos, o_slot = paged.token_mapping(w.requests(), w.fact_rows, w.spec.block_size)
    assert len(src) == w.n_tokens
    assert np.array_equal(src, np.array(o_src, np.int32))
    assert np.array_equal(pos, np.array(o_pos, np.int32))
    assert np.array_equal(slot, np.array(o_slot, np.int32))


@pytest.mark.parametrize("name", ["tiny_L1_H2_D64", "llama3_8b_k50", "llama3_70b_batch16_k50"])
def test_slot_mapping_chunk_local_rotation_positions(name):
    w = workloads.make(name)
    d = prkv.desc(w.spec.num_layers, w.spec.num_kv_heads, w.spec.head_dim, w.max_facts,
                  w.capacity_rows, w.spec.max_position, w.spec.rope_theta,
                  key_layout=prkv.KEYS_CHUNK_LOCAL)
    st = prkv.store_create(d)
    for f in w.put_order:
        prkv.store_put_fact(st, f, w.length_of(f))
    req_ptr, ids, start, bt, bt_len = w.csr()
    src, pos, slot = prkv.build_slot_mapping(st, req_ptr, ids, start, bt, bt_len,
                                             w.spec.block_size, w.num_blocks)
    o_src, _, o_slot = paged.token_mapping(w.requests(), w.fact_rows, w.spec.block_size)
    o_rot = paged.rotation_positions(w.requests(), w.fact_rows, chunk_local=True)
    assert np.array_equal(src, np.array(o_src, np.int32))
    assert np.array_equal(pos, np.array(o_rot, np.int32))
    assert np.array_equal(slot, np.array(o_slot, np.int32))


def _small_mapping_case():
    d = _desc(max_facts=8, capacity_rows=64, max_position=64)
    st = prkv.store_create(d)
    prkv.store_put_fact(st, 7, 2)   # rows 0..1
    prkv.store_put_fact(st, 3, 3)   # rows 2..4
    return st


def test_slot_mapping_small_golden():
    st = _small_mapping_case()
    bt = np.array([[5, 2, 7, 0], [3, 1, -1, -1]], np.int32)
    src, pos, slot = prkv.build_slot_mapping(st, [0, 2, 4], [7, 3, 3, 7], [3, 0], bt, [4, 2],
                                             4, 8)
    assert src.tolist() == [0, 1, 2, 3, 4, 2, 3, 4, 0, 1]
    assert pos.tolist() == [3, 4, 5, 6, 7, 0, 1, 2, 3, 4]
    assert slot.tolist() == [23, 8, 9, 10, 11, 12, 13, 14, 15, 4]


@pytest.mark.parametrize("case,name", [
    (dict(ids=[7, 5]), "UNKNOWN_FACT"),
    (dict(ids=[7, -2]), "UNKNOWN_FACT"),
    (dict(bt_len=[1]), "OUT_OF_RANGE"),                 # table too short
    (dict(bt=[[5, 9, 7, 0]]), "OUT_OF_RANGE"),          # block id >= num_blocks
    (dict(bt=[[5, -1, 7, 0]]), "OUT_OF_RANGE"),         # negative block id
    (dict(start=[60]), "OUT_OF_RANGE"),                 # position >= max_position
    (dict(bt=[[5, 5, 7, 0]], start=[0]), "DUPLICATE_SLOT"),
    (dict(ids=[7, 7, 3], bt=[[1, 1, 1, 1]], start=[0]), "DUPLICATE_SLOT"),
    (dict(start=[-1]), "INVALID_ARG"),
    (dict(bt_len=[5]), "INVALID_ARG"),                  # longer than the stride
    (dict(ptr=[1, 2]), "INVALID_ARG"),
    (dict(ptr=[0, 3, 2]), "INVALID_ARG"),
    (dict(block_size=0), "INVALID_ARG"),
    (dict(num_blocks=2**30, block_size=4), "INVALID_ARG"),
])
def test_slot_mapping_errors(case, name):
    st = _small_mapping_case()
    ids = case.get("ids", [7, 3])
    ptr = case.get("ptr", [0, len(ids)])
    bt = np.array(case.get("bt", [[5, 2, 7, 0]]), np.int32)
    n_req = len(ptr) - 1
    start = case.get("start", [3] * n_req)
    bt_len = case.get("bt_len", [4] * n_req)
    if len(bt) < n_req:
        bt = np.repeat(bt, n_req, axis=0)
    outs = tuple(np.full(32, -7, np.int32) for _ in range(3))
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.build_slot_mapping(st, ptr, ids, start, bt, bt_len, case.get("block_size", 4),
                                case.get("num_blocks", 8), out=outs)
    assert ei.value.name == name
    for o in outs:
        assert np.all(o == -7), "outputs must be untouched on error"


def test_slot_mapping_buffer_too_small_reports_count():
    st = _small_mapping_case()
    outs = tuple(np.full(3, -7, np.int32) for _ in range(3))
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.build_slot_mapping(st, [0, 2], [7, 3], [3], np.array([[5, 2, 7, 0]], np.int32),
                                [4], 4, 8, out=outs)
    assert ei.value.name == "BUFFER_TOO_SMALL"
    assert all(np.all(o == -7) for o in outs)


def test_slot_mapping_empty_and_reuse():
    st = _small_mapping_case()
    src, pos, slot = prkv.build_slot_mapping(st, [0], [], [], np.zeros((0, 0), np.int32), [],
                                             4, 8)
    assert len(src) == 0
    # after a duplicate-slot failure the next call is clean (scratch is reset)
    with pytest.raises(prkv.PrkvError):
        prkv.build_slot_mapping(st, [0, 3], [7, 7, 3], [0],
                                np.array([[1, 1, 1, 1]], np.int32), [4], 4, 8)
    src, pos, slot = prkv.build_slot_mapping(st, [0, 1], [7], [0],
                                             np.array([[1, 1, 1, 1]], np.int32), [4], 4, 8)
    assert slot.tolist() == [4, 5]


@pytest.mark.parametrize("d_model,theta,scaled", [(64, 1e4, False), (128, 5e5, False),
                                                  (16, 10.0, False), (128, 5e5, True),
                                                  (64, 5e5, True)])
def test_rope_table_hi_lo(d_model, theta, scaled):
    d = prkv.desc(1, 1, d_model, 1, 1, 16384, theta,
                  llama3_scaling=LLAMA31 if scaled else None)
    t = prkv.rope_table_fill(d).astype(np.float64)
    pos = np.arange(16384)
    w = rope.rotation_factors(pos, d_model, theta,     # float64 cos + i sin
                              rope.Llama3Scaling(*LLAMA31) if scaled else None)
    ch, cl, sh, sl = t[..., 0], t[..., 1], t[..., 2], t[..., 3]
    # hi parts are the float32 roundings; hi + lo carries ~48 bits
    assert np.array_equal(ch, w.real.astype(np.float32).astype(np.float64))
    assert np.array_equal(sh, w.imag.astype(np.float32).astype(np.float64))
    assert np.max(np.abs(ch + cl - w.real)) < 2.0 ** -46
    assert np.max(np.abs(sh + sl - w.imag)) < 2.0 ** -46
    # position 0 is the identity rotation exactly
    assert np.all(ch[0] == 1) and np.all(cl[0] == 0) and np.all(sh[0] == 0) and np.all(sl[0] == 0)


def test_same_fact_twice_is_legal():
    st = _small_mapping_case()
    src, pos, slot = prkv.build_slot_mapping(st, [0, 2], [7, 7], [0],
                                             np.array([[1, 2]], np.int32), [2], 4, 8)
    assert src.tolist() == [0, 1, 0, 1]
    assert pos.tolist() == [0, 1, 2, 3]
    assert slot.tolist() == [4, 5, 6, 7]


@pytest.mark.parametrize("facts,tokens", [(1, 1), (50, 2000), (3200, 192000), (0, 0), (7, 13)])
def test_device_workspace_size_matches_layout(facts, tokens):
    assert prkv.inject_device_workspace_bytes(facts, tokens) == \
        prkv.workspace_layout(facts, tokens)["total"]


def test_device_workspace_size_rejects_bad_bounds():
    for facts, tokens in ((-1, 5), (5, -1), (5, 2**31)):
        with pytest.raises(prkv.PrkvError) as ei:
            prkv.inject_device_workspace_bytes(facts, tokens)
        assert ei.value.name == "INVALID_ARG"


def test_upload_fact_table_argument_errors():
    st = prkv.store_create(_desc(max_facts=16))
    L = prkv.lib()
    for ptr, nbytes, name in ((None, 256, "INVALID_ARG"), (4100, 256, "ALIGNMENT"),
                              (4096, 8 * 16 - 8, "BUFFER_TOO_SMALL")):
        with pytest.raises(prkv.PrkvError) as ei:
            prkv._check(L.store_upload_fact_table(st.handle, ptr, nbytes, None), "upload")
        assert ei.value.name == name


def test_inject_device_rejects_metadata_store_and_bad_batches():
    st = prkv.store_create(_desc())
    b = prkv.device_batch(1, 4, 2, 10, 4096, 4096, 4096, 4096, 4096)
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.inject_topk_device(st, 4096, b, [4096, 4096], [4096, 4096], 16, 4, 4096, 1 << 20,
                                stream=0)
    assert ei.value.name == "NO_DEVICE"


@pytest.mark.parametrize("kw,name", [
    (dict(k=0), "INVALID_ARG"), (dict(k=65), "INVALID_ARG"), (dict(k=101), "INVALID_ARG"),
    (dict(dim=1004), "INVALID_ARG"), (dict(dim=0), "INVALID_ARG"), (dict(dim=4104), "INVALID_ARG"),
    (dict(dim=4608), "INVALID_ARG"),
    (dict(n_stores=0), "INVALID_ARG"), (dict(fact_emb=None), "INVALID_ARG"),
    (dict(fact_emb=4104), "ALIGNMENT"), (dict(ws_bytes=8), "BUFFER_TOO_SMALL"),
])
def test_retrieve_argument_errors(kw, name):
    a = dict(fact_emb=4096, n_stores=2, F=100, dim=1536, query=8192, req_store=12288, n_req=2,
             k=5, ids=16384, ws=20480, ws_bytes=2 * 100 * 8)
    a.update(kw)
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.retrieve_topk(a["fact_emb"], a["n_stores"], a["F"], a["dim"], a["query"],
                           a["req_store"], a["n_req"], a["k"], a["ids"], a["ws"], a["ws_bytes"],
                           stream=0)
    assert ei.value.name == name


def test_retrieve_workspace_bytes():
    assert prkv.retrieve_workspace_bytes(64, 2000) == 64 * 2000 * 8
    # few requests with many facts: 16 score slices each, partial top-64
    # lists (8-byte keys, then 4-byte ids, 256-byte aligned) after the scores
    scores = 16 * 20000 * 8
    n = 16 * 16 * 64
    assert prkv.retrieve_workspace_bytes(16, 20000) == scores + n * 8 + n * 4
    assert prkv.retrieve_workspace_bytes(1, 1023) == 1023 * 8   # slices need >= 1024 scores


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no fallback: without libprkv.so every entry point raises
    monkeypatch.setattr(prkv, "LIB_PATH", str(tmp_path / "libprkv.so"))
    monkeypatch.setattr(prkv, "_lib", None)
    with pytest.raises(ImportError, match="no fallback"):
        prkv.lib()
    with pytest.raises(ImportError):
        prkv.store_required_bytes(_desc())
    with pytest.raises(ImportError):
        prkv.store_create(_desc())


def _wide_block_store():
    d = _desc(max_facts=4, capacity_rows=1000, max_position=1024)
    st = prkv.store_create(d)
    prkv.store_put_fact(st, 0, 150)   # rows 0..149
    prkv.store_put_fact(st, 1, 90)    # rows 150..239
    return st


def test_slot_mapping_block_wider_than_a_bitmap_word():
    """block_size 100: a run of one fact inside a block covers several
    64-slot words of the duplicate bitmap; the mapping is still the closed
    form slot = bt[p // bs] * bs + p % bs."""
    st = _wide_block_store()
    bt = np.array([[3, 0, 5], [2, 4, -1]], np.int32)
    src, pos, slot = prkv.build_slot_mapping(st, [0, 1, 2], [0, 1], [37, 5], bt, [3, 2], 100, 8)
    want_pos = list(range(37, 187)) + list(range(5, 95))
    want_row = list(range(0, 150)) + list(range(150, 240))
    want_slot = [int(bt[0][q // 100]) * 100 + q % 100 for q in range(37, 187)] + \
                [int(bt[1][q // 100]) * 100 + q % 100 for q in range(5, 95)]
    assert pos.tolist() == want_pos and src.tolist() == want_row and slot.tolist() == want_slot


@pytest.mark.parametrize("start0,start1,first_dup", [(37, 63, 263), (37, 0, 237), (70, 0, 270)])
def test_duplicate_slot_reports_the_first_one(start0, start1, first_dup):
    """Two requests share block 2 (slots 200..299).  Request 0 takes slots
    200 + start0 .. 299 with its fact 0; request 1 writes fact 1 from position
    start1 in block 2, so its first clash is the lowest slot both cover, in
    token order (270: request 1's run starts in bitmap word 3, the clash is in
    word 4)."""
    st = _wide_block_store()
    bt = np.array([[2, 7, 6], [2, 5, -1]], np.int32)
    outs = tuple(np.full(400, -7, np.int32) for _ in range(3))
    with pytest.raises(prkv.PrkvError) as ei:
        prkv.build_slot_mapping(st, [0, 1, 2], [0, 1], [start0, start1], bt, [3, 2], 100, 8,
                                out=outs)
    assert ei.value.name == "DUPLICATE_SLOT"
    assert f"slot {first_dup} written twice" in str(ei.value)
    assert all(np.all(o == -7) for o in outs)
    # every bit set before the failure was cleared: the same blocks map cleanly now
    src, pos, slot = prkv.build_slot_mapping(st, [0, 1], [1], [start1], bt[1:], [2], 100, 8)
    assert slot.tolist() == [200 + q if q < 100 else 500 + q - 100 for q in range(start1, start1 + 90)]


def test_build_slot_mapping_concurrent_calls_on_one_store():
    """build_slot_mapping is documented safe to call concurrently on one store:
    eight threads (ctypes releases the GIL during the call) map different
    batches at once, some invalid; every valid result equals the same call
    made alone, and every invalid one fails with its own error message
    (last_error_string is per thread)."""
    import threading

    d = _desc(max_facts=400, capacity_rows=400 * 60, max_position=16384)
    st = prkv.store_create(d)
    rng = np.random.default_rng(11)
    lengths = {}
    for f in range(400):
        lengths[f] = int(rng.integers(1, 60))
        prkv.store_put_fact(st, f, lengths[f])

    def batch(seed):
        r = np.random.default_rng(seed)
        n_req = int(r.integers(1, 6))
        ptr, ids, start, tables, bt_len = [0], [], [], [], []
        free = r.permutation(20000)
        used = 0
        for _ in range(n_req):
            k = int(r.integers(1, 30))
            fid = [int(x) for x in r.choice(400, size=k, replace=False)]
            pre = int(r.integers(0, 200))
            need = -(-(pre + sum(lengths[f] for f in fid)) // 16)
            ids += fid
            ptr.append(len(ids))
            start.append(pre)
            tables.append(free[used:used + need])
            bt_len.append(need)
            used += need
        stride = max(bt_len)
        bt = np.zeros((n_req, stride), np.int32)
        for i, t in enumerate(tables):
            bt[i, :len(t)] = t
        bad = seed % 3 == 0
        if bad:
            ids[0] = 399 + 1000     # an id never stored
        return (ptr, ids, start, bt, bt_len), bad

    cases = [batch(s) for s in range(48)]
    expected = []
    for args, bad in cases:
        if bad:
            expected.append(None)
        else:
            expected.append(prkv.build_slot_mapping(st, *args, 16, 20000))

    results = [None] * len(cases)

    def worker(w):
        for i in range(w, len(cases), 8):
            args, bad = cases[i]
            for _ in range(5):
                try:
                    got = prkv.build_slot_mapping(st, *args, 16, 20000)
                    results[i] = ("ok", got)
                except prkv.PrkvError as e:
                    results[i] = ("err", e.name, str(e))

    threads = [threading.Thread(target=worker, args=(w,)) for w in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for i, ((args, bad), want) in enumerate(zip(cases, expected)):
        if bad:
            assert results[i][0] == "err" and results[i][1] == "UNKNOWN_FACT", i
            assert "1399" in results[i][2], results[i][2]
        else:
            assert results[i][0] == "ok", results[i]
            for g, e in zip(results[i][1], want):
                assert np.array_equal(g, e), i


def test_stage_facts_needs_device_backed_stores():
    """store_stage_facts between metadata-only stores: NO_DEVICE, no HIP call."""
    a = prkv.store_create(_desc(), None, None, None)
    b = prkv.store_create(_desc(), None, None, None)
    prkv.store_put_fact(a, 0, 5)
    with pytest.raises(prkv.PrkvError) as err:
        prkv.store_stage_facts(a, b, [0], stream=0)    # the null stream: no torch device needed
    assert err.value.name == "NO_DEVICE"
    assert prkv.lib().store_stage_facts(None, b.handle, 0, None, None) == prkv.CODES["INVALID_ARG"]


def test_chunk_facts_covers_the_batch_in_order():
    """The staging injector's chunks: consecutive, covering every token once,
    each piece's facts in order (a fact repeated inside a piece listed once),
    at most the asked number of pieces, and close to equal token counts."""
    from pre_rope_kv_amd import harness
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(1, 60))
        facts = [int(x) for x in rng.integers(0, 40, size=n)]
        lens = [int(x) for x in rng.integers(1, 300, size=n)]
        chunks = int(rng.integers(1, 20))
        pieces = harness.chunk_facts(facts, lens, chunks)
        assert 1 <= len(pieces) <= min(chunks, n)
        assert pieces[0][1] == 0 and pieces[-1][2] == sum(lens)
        for (_, _, e), (_, s, _) in zip(pieces[:-1], pieces[1:]):
            assert e == s
        # rebuild the fact list from the token ranges
        ends = np.cumsum(lens)
        i = 0
        for fs, t0, t1 in pieces:
            j = int(np.searchsorted(ends, t1, side="left")) + 1
            assert ends[j - 1] == t1 and (i == 0 or ends[i - 1] == t0)
            assert fs == list(dict.fromkeys(facts[i:j]))
            i = j
        assert i == n
        if len(pieces) == chunks and n >= 4 * chunks:
            biggest = max(t1 - t0 for _, t0, t1 in pieces)
            assert biggest <= sum(lens) / chunks + max(lens)
    assert harness.chunk_facts([], [], 4) == []
