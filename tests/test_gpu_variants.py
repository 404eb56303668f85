"""GPU parity of the RoPE table variants against the CPU oracle.

Variants (each a store-descriptor option, the kernels' arithmetic unchanged):
  interleaved   pairs (2j, 2j+1), RoFormer's block-diagonal form (GPT-J style)
  llama31       Llama 3.1's long-context frequency rule (factor 8, 1, 4, 8192)
  chunk_local   the store holds keys already rotated at positions 0 .. len-1 of
                their fact; injection relocates them by R(s), s = the fact's
                serving start (Theorem 6's axiom R_a^T R_b = R_{b-a})
  hnd           paged cache blocks laid out [H][block_size][D] instead of
                [block_size][H][D] (slots and block tables unchanged; the
                comparison reads the cache back in the logical slot order)
Same bar as the base path: V and untouched slots bit-exact, K within 2 bf16
ulp with mean error < 1e-3, the device-built mapping bit-equal to the
oracle's.  Attention is checked with the interleaved and scaled tables (the
query is rotated in-kernel with the store's pairing and frequencies) and over
an HND cache.
"""

import gc

import numpy as np
import pytest
import torch

from pre_rope_kv_amd import prkv, workloads

import test_gpu_attention as att
from test_gpu_parity import (EDGE, _full_size, _release_device_memory,  # noqa: F401
                             custom_workload, run_full)

pytestmark = pytest.mark.gpu

LLAMA31 = (8.0, 1.0, 4.0, 8192)
VARIANTS = {
    "interleaved": dict(rope_style=prkv.ROPE_INTERLEAVED),
    "llama31": dict(llama3_scaling=LLAMA31),
    "chunk_local": dict(key_layout=prkv.KEYS_CHUNK_LOCAL),
    "all_three": dict(rope_style=prkv.ROPE_INTERLEAVED, llama3_scaling=LLAMA31,
                      key_layout=prkv.KEYS_CHUNK_LOCAL),
    "hnd": dict(cache_layout=prkv.CACHE_HND),
}


def variant_workload(name, variant):
    spec = workloads.dataclasses.replace(workloads.SPECS[name], **VARIANTS[variant])
    return workloads.make(spec)


@pytest.mark.parametrize("path", ["host", "device"])
@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("name", ["tiny_L1_H2_D64", "llama3_8b_k5"])
def test_variant_full_compare(name, variant, path):
    w = variant_workload(name, variant)
    dw, rep, _ = run_full(w, gen_device="cpu" if name.startswith("tiny") else "cuda", path=path)
    sp = w.spec
    expect = 2 * sp.num_layers * w.n_tokens * sp.num_kv_heads * sp.head_dim
    assert dw.count_non_sentinel() == expect


def test_variant_llama8b_k50_interleaved_scaled():
    w = variant_workload("llama3_8b_k50", "all_three")
    run_full(w, path="device")


def test_variant_llama8b_k50_hnd():
    run_full(variant_workload("llama3_8b_k50", "hnd"), path="device")


@pytest.mark.timeout(900)
def test_variant_batch64_full_size():
    _full_size("llama3_8b_batch64_k50", paths=("device",), **VARIANTS["all_three"])


@pytest.mark.timeout(900)
def test_variant_batch64_full_size_hnd():
    _full_size("llama3_8b_batch64_k50", paths=("device",), **VARIANTS["hnd"])


@pytest.mark.timeout(900)
def test_variant_llama70b_full_size_hnd():
    # block size 32, fact starts that straddle blocks
    _full_size("llama3_70b_batch16_k50", paths=("device",), **VARIANTS["hnd"])


HND_EDGE = ["prefix0_len1", "len256_straddle_bs32", "dup_fact_in_request", "h1_d64", "h1_d16",
            "h1_d512", "h3_d128", "h2_d1024", "bs1", "250_facts"]


@pytest.mark.parametrize("path", ["host", "device"])
@pytest.mark.parametrize("name", HND_EDGE)
def test_hnd_edge_case(name, path):
    _, L, H, D, bs, facts, reqs = next(c for c in EDGE if c[0] == name)
    nb = 2048 if name == "250_facts" else 512
    w = custom_workload(name + "_hnd", L, H, D, bs, facts, reqs, theta=5e5, num_blocks=nb)
    w = workloads.dataclasses.replace(
        w, spec=workloads.dataclasses.replace(w.spec, **VARIANTS["hnd"]))
    dw, rep, _ = run_full(w, gen_device="cuda", path=path)
    assert dw.hnd
    assert dw.count_non_sentinel() == 2 * L * w.n_tokens * H * D


@pytest.mark.parametrize("variant", ["interleaved", "llama31", "hnd"])
@pytest.mark.parametrize("D", [64, 128])
def test_variant_attention(variant, D):
    rng = np.random.default_rng(D)
    w = att.context_workload(f"attn_{variant}_{D}", 2, 2, D, 16, 40,
                             [rng.integers(5, 60, size=6), rng.integers(5, 60, size=9)],
                             q_len=8, n_req=2, seed=D)
    w.spec = workloads.dataclasses.replace(w.spec, **VARIANTS[variant])
    q_len, hq = 8, 8
    dw, q_bits, got, layers = att.run_attention(w, q_len, hq, gen="cpu")
    assert int(dw.status.item()) == 0
    att.check(dw, q_bits, got, q_len, hq, layers, "cpu")


@pytest.mark.parametrize("bs,D,q_len,hq", [(24, 128, 16, 32), (12, 64, 4, 4), (32, 128, 16, 32)])
def test_hnd_attention_block_sizes(bs, D, q_len, hq):
    # block sizes that are and are not powers of two, over an HND cache
    rng = np.random.default_rng(bs * D)
    lens = [rng.integers(5, 60, size=7), rng.integers(5, 60, size=3)]
    w = att.context_workload(f"attn_hnd_{bs}_{D}", 2, hq // 4, D, bs, 30,
                             lens, q_len=q_len, n_req=2, seed=bs + D)
    w.spec = workloads.dataclasses.replace(w.spec, **VARIANTS["hnd"])
    dw, q_bits, got, layers = att.run_attention(w, q_len, hq, gen="cpu")
    assert dw.hnd
    assert int(dw.status.item()) == 0
    att.check(dw, q_bits, got, q_len, hq, layers, "cpu")


@pytest.mark.parametrize("name", ["tiny_L1_H2_D64", "llama3_8b_k5"])
def test_hnd_cache_equals_nhd_cache(name):
    # only addresses differ between the layouts: read back in slot order,
    # the two caches are bit-identical (K included)
    got = []
    for variant in (None, "hnd"):
        w = workloads.make(name) if variant is None else variant_workload(name, variant)
        dw, _, _ = run_full(w, gen_device="cpu" if name.startswith("tiny") else "cuda",
                            path="device")
        got.append(dw.listed_blocks_host(w.listed_blocks()))
        del dw
        gc.collect()
        torch.cuda.empty_cache()
    (k0, v0), (k1, v1) = got
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
