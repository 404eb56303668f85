"""CPU tests of libprkv_ceiling.so, the bench's measuring sticks: its exports
and the argument checks of every entry point, which return before anything
touches the HIP runtime.  The addresses passed are aligned stand-ins that the
host never dereferences; each bad case changes one argument of an otherwise
valid call, so a missing check would reach a launch.  Without a GPU such a
launch fails with an error (and the test with it); where a GPU is visible the
argument-check tests are skipped, so a stray launch can never read the
stand-in addresses.
"""

import ctypes
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402

P = ctypes.c_void_p(1 << 20)   # 16-byte aligned, never dereferenced on the host
ODD = ctypes.c_void_p((1 << 20) + 8)


def lib():
    return bench.ceiling_lib()


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0     # counts devices without initialising one
    except Exception:
        return False


no_gpu = pytest.mark.skipif(_gpu_visible(), reason="a missing check would launch on the GPU")


def test_exports():
    L = lib()
    for name in ("ceiling_gather_scatter", "ceiling_read", "ceiling_gather_kv", "ceiling_empty"):
        assert hasattr(L, name)


# a valid call: 2 layers, 8 KV heads of 128 dims, 64 blocks of 16 slots, 3 requests
GOOD = dict(k=P, v=P, layer_bytes=64 * 16 * 8 * 128 * 2, layers=2, heads=8, dim=128, bt=P,
            bt_stride=5, bt_len=P, ctx=P, n_req=3, bs=16, nblocks=64, hg=1, sink=P, passes=1,
            nt=0)


def gather(**kw):
    a = dict(GOOD, **kw)
    return lib().ceiling_gather_kv(a["k"], a["v"], a["layer_bytes"], a["layers"], a["heads"],
                                   a["dim"], a["bt"], a["bt_stride"], a["bt_len"], a["ctx"],
                                   a["n_req"], a["bs"], a["nblocks"], a["hg"], a["sink"],
                                   a["passes"], a["nt"], None)


@pytest.mark.parametrize("kw", [
    dict(k=None), dict(v=None), dict(bt=None), dict(bt_len=None), dict(ctx=None),
    dict(sink=None), dict(k=ODD), dict(v=ODD),
    dict(dim=96), dict(dim=256), dict(layers=0), dict(heads=0), dict(n_req=0),
    dict(bt_stride=0), dict(bs=0), dict(nblocks=0), dict(layer_bytes=64 * 16 * 8 * 128 * 2 + 8),
    # a layer must hold every slot of every block
    dict(layer_bytes=64 * 16 * 8 * 128 * 2 - 16), dict(nblocks=65),
    dict(nblocks=1 << 27, bs=16, layer_bytes=1 << 50),
    # head groups must divide the heads and fill 256 lanes evenly
    dict(hg=0), dict(hg=3), dict(hg=16), dict(hg=32, heads=32, layer_bytes=1 << 30),
    dict(hg=3, heads=24, dim=64, layer_bytes=1 << 30),
    # passes other than 1, 2, 4 or 8
    dict(passes=0), dict(passes=3), dict(passes=16), dict(passes=3, nt=1),
    dict(passes=5, dim=64), dict(passes=3, hg=8), dict(passes=3, hg=4, dim=64),
], ids=repr)
@no_gpu
def test_gather_kv_rejects_bad_arguments(kw):
    assert gather(**kw) == -1


@no_gpu
def test_read_and_copy_reject_bad_arguments():
    L = lib()
    assert L.ceiling_read(None, 1024, P, 1, 8, None) == -1
    assert L.ceiling_read(P, 1000, P, 1, 8, None) == -1       # not a multiple of 16
    assert L.ceiling_read(ODD, 1024, P, 1, 8, None) == -1
    assert L.ceiling_read(P, 1024, P, 3, 8, None) == -1       # per_lane 1, 2, 4 or 8
    assert L.ceiling_read(P, 1024, P, 1, 0, None) == -1
    assert L.ceiling_read(P, 0, P, 1, 8, None) == 0           # nothing to read, no launch
    assert L.ceiling_empty(0, None) == -1
