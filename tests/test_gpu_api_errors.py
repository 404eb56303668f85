"""Host-side argument errors of the entry points that need a device-backed
store (inject_topk, inject_topk_device, attend_paged): each bad argument is
rejected with its documented code and nothing is enqueued, so the cache
stays at the sentinel, the status word at 0 and the attention output
untouched.  Every case here is one the host code checks before any launch."""

import ctypes

import pytest
import torch

from pre_rope_kv_amd import harness, prkv

from test_gpu_parity import custom_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dw():
    w = custom_workload("api_errors", 2, 8, 128, 16, {0: 9, 1: 14}, [([0, 1], 5)])
    d = harness.DeviceWorkload(w)
    d.setup_device_batch()
    torch.cuda.synchronize()
    d.status.zero_()
    return d


def _code(fn, *args, **kw):
    with pytest.raises(prkv.PrkvError) as ei:
        fn(*args, **kw)
    return ei.value.name


def _untouched(dw):
    torch.cuda.synchronize()
    assert dw.count_non_sentinel() == 0 and int(dw.status.item()) == 0


def test_inject_topk_argument_errors(dw):
    w, (src, pos, slot) = dw.w, dw.d_map
    K, V = list(dw.k_layers()), list(dw.v_layers())
    bs, nb, n = w.spec.block_size, w.num_blocks, dw.n_tokens

    def call(n_tokens=n, s=src, p=pos, sl=slot, k=K, v=V, block_size=bs, num_blocks=nb,
             status=dw.status):
        prkv.inject_topk(dw.store, n_tokens, s, p, sl, k, v, block_size, num_blocks,
                         d_status=status, stream=dw.stream)

    assert _code(call, n_tokens=-1) == "INVALID_ARG"
    assert _code(call, n_tokens=nb * bs + 1) == "INVALID_ARG"
    assert _code(call, s=None) == "INVALID_ARG"
    assert _code(call, p=pos.data_ptr() + 2) == "ALIGNMENT"
    assert _code(call, status=dw.status.data_ptr() + 1) == "ALIGNMENT"
    assert _code(call, block_size=0) == "INVALID_ARG"
    assert _code(call, num_blocks=1 << 28) == "INVALID_ARG"          # 2^32 slots
    assert _code(call, k=[K[0], None]) == "INVALID_ARG"
    assert _code(call, v=[V[0], V[1].data_ptr() + 2]) == "ALIGNMENT"
    _untouched(dw)


def test_inject_topk_device_argument_errors(dw):
    base = list(dw.inject_device_args())
    lib = prkv.lib()
    b = dw.batch

    def code(**changes):
        a = list(base)
        for i, v in changes.items():
            a[int(i[1:])] = v
        rc = lib.inject_topk_device(*a)
        return prkv.ERRORS.get(rc, rc) if rc else "OK"

    def with_batch(**fields):
        nb = prkv.DeviceBatch.from_buffer_copy(b)
        for k, v in fields.items():
            setattr(nb, k, v)
        return nb

    assert code(a8=base[8] - 1) == "BUFFER_TOO_SMALL"
    assert code(a7=base[7] + 16) == "ALIGNMENT"
    assert code(a1=base[1] + 4) == "ALIGNMENT"
    assert code(a1=None) == "INVALID_ARG"
    assert code(a7=None) == "INVALID_ARG"
    keep = []
    for fields, want in ((dict(max_tokens=dw.w.num_blocks * dw.w.spec.block_size + 1),
                          "INVALID_ARG"),
                         (dict(n_req=-1), "INVALID_ARG"),
                         (dict(flags=2), "INVALID_ARG"),          # unknown flag bit
                         (dict(flags=-1), "INVALID_ARG"),
                         (dict(fact_ids=None), "INVALID_ARG"),
                         (dict(start_pos=b.start_pos + 2), "ALIGNMENT")):
        nbatch = with_batch(**fields)
        keep.append(nbatch)
        assert code(a2=ctypes.byref(nbatch)) == want, fields
    _untouched(dw)


def test_attend_paged_argument_errors(dw):
    w = dw.w
    n_req, q_len, hq, D = w.spec.n_requests, 4, 32, w.spec.head_dim
    q = torch.zeros((n_req, 17, hq, D), dtype=torch.bfloat16, device="cuda")
    q_start = torch.full((n_req,), 5, dtype=torch.int32, device="cuda")
    out = torch.full((w.spec.num_layers, n_req, 17, hq, D), float("nan"), device="cuda")
    K, V = list(dw.k_layers()), list(dw.v_layers())
    stride = dw.d_bt.shape[1]

    def call(q_len=q_len, heads=hq, bt_stride=stride, qp=q, bt_len=dw.d_bt_len, scale=0.1,
             block_size=w.spec.block_size, k=K):
        ab = prkv.attn_batch(n_req, q_len, heads, bt_stride, qp, q_start, dw.d_bt, bt_len, out)
        prkv.attend_paged(dw.store, ab, k, V, block_size, w.num_blocks, scale,
                          d_status=dw.status, stream=dw.stream)

    assert _code(call, heads=12) == "INVALID_ARG"                 # not a multiple of 8
    assert _code(call, q_len=w.spec.max_position + 1) == "INVALID_ARG"   # past every position
    assert _code(call, scale=0.0) == "INVALID_ARG"
    assert _code(call, scale=float("nan")) == "INVALID_ARG"
    assert _code(call, qp=q.data_ptr() + 8) == "ALIGNMENT"
    assert _code(call, bt_len=None) == "INVALID_ARG"
    assert _code(call, block_size=0) == "INVALID_ARG"
    assert _code(call, k=[K[0].data_ptr() + 2, K[1]]) == "ALIGNMENT"
    torch.cuda.synchronize()
    assert bool(torch.isnan(out).all())
    _untouched(dw)


def test_attend_paged_rejects_head_dim_16():
    w = custom_workload("api_errors_d16", 1, 1, 16, 16, {0: 5}, [([0], 2)])
    d = harness.DeviceWorkload(w)
    d.setup_device_batch()
    q = torch.zeros((1, 1, 4, 16), dtype=torch.bfloat16, device="cuda")
    qs = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.zeros((1, 1, 1, 4, 16), device="cuda")
    ab = prkv.attn_batch(1, 1, 4, d.d_bt.shape[1], q, qs, d.d_bt, d.d_bt_len, out)
    assert _code(prkv.attend_paged, d.store, ab, list(d.k_layers()), list(d.v_layers()), 16,
                 w.num_blocks, 0.25, stream=d.stream) == "INVALID_ARG"


def test_store_stage_facts_errors(dw):
    """Staging between stores: every bad argument is rejected before
    anything is copied (the destination's arenas keep their fill)."""
    w = dw.w
    sp = w.spec
    # room for 20 rows: fact 0 (9 rows) fits, facts 0 and 1 (9 + 14) do not
    dst_desc = prkv.desc(sp.num_layers, sp.num_kv_heads, sp.head_dim, w.max_facts, 20,
                         sp.max_position, sp.rope_theta)
    k = torch.full((sp.num_layers, 20, sp.num_kv_heads, sp.head_dim), 7, dtype=torch.int16,
                   device="cuda")
    v = torch.full_like(k, 7)
    rope = torch.empty(prkv.store_required_bytes(dst_desc)[1] // 4, dtype=torch.float32,
                       device="cuda")
    dst = prkv.store_create(dst_desc, k, v, rope)
    assert _code(prkv.store_stage_facts, dw.store, dst, [5]) == "UNKNOWN_FACT"
    assert _code(prkv.store_stage_facts, dw.store, dst, [-1]) == "UNKNOWN_FACT"
    assert _code(prkv.store_stage_facts, dw.store, dst, [0, 1]) == "CAPACITY"
    prkv.store_put_fact(dst, 1, 3)                 # fact 1 reserved with another length
    assert _code(prkv.store_stage_facts, dw.store, dst, [1]) == "INVALID_ARG"
    other = prkv.desc(sp.num_layers, sp.num_kv_heads, 64, w.max_facts, 20, sp.max_position,
                      sp.rope_theta)
    k2 = torch.zeros((sp.num_layers, 20, sp.num_kv_heads, 64), dtype=torch.int16, device="cuda")
    rope2 = torch.empty(prkv.store_required_bytes(other)[1] // 4, dtype=torch.float32,
                        device="cuda")
    dst2 = prkv.store_create(other, k2, k2.clone(), rope2)
    assert _code(prkv.store_stage_facts, dw.store, dst2, [0]) == "INVALID_ARG"    # head_dim
    assert _code(prkv.store_stage_facts, dw.store, dw.store, [0]) == "INVALID_ARG"  # one store
    meta = prkv.store_create(dst_desc, None, None, None)
    assert _code(prkv.store_stage_facts, dw.store, meta, [0]) == "NO_DEVICE"
    torch.cuda.synchronize()
    assert bool((k == 7).all()) and bool((v == 7).all())
    prkv.store_stage_facts(dw.store, dst, [0])      # a valid call for contrast
    torch.cuda.synchronize()
    assert not bool((k == 7).all())
    _untouched(dw)
