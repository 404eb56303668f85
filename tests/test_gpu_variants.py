"""GPU parity of the RoPE table variants against the CPU oracle.

Variants (each a store-descriptor option, the kernels' arithmetic unchanged):
  interleaved   pairs (2j, 2j+1), RoFormer's block-diagonal form (GPT-J style)
  llama31       Llama 3.1's long-context frequency rule (factor 8, 1, 4, 8192)
  chunk_local   the store holds keys already rotated at positions 0 .. len-1 of
                their fact; injection relocates them by R(s), s = the fact's
                serving start (Theorem 6's axiom R_a^T R_b = R_{b-a})
Same bar as the base path: V and untouched slots bit-exact, K within 2 bf16
ulp with mean error < 1e-3, the device-built mapping bit-equal to the
oracle's.  Attention is checked with the interleaved and scaled tables (the
query is rotated in-kernel with the store's pairing and frequencies).
"""

import numpy as np
import pytest

from pre_rope_kv_amd import prkv, workloads

import test_gpu_attention as att
from test_gpu_parity import _full_size, _release_device_memory, run_full  # noqa: F401

pytestmark = pytest.mark.gpu

LLAMA31 = (8.0, 1.0, 4.0, 8192)
VARIANTS = {
    "interleaved": dict(rope_style=prkv.ROPE_INTERLEAVED),
    "llama31": dict(llama3_scaling=LLAMA31),
    "chunk_local": dict(key_layout=prkv.KEYS_CHUNK_LOCAL),
    "all_three": dict(rope_style=prkv.ROPE_INTERLEAVED, llama3_scaling=LLAMA31,
                      key_layout=prkv.KEYS_CHUNK_LOCAL),
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


def test_variant_batch64_full_size_sampled():
    _full_size("llama3_8b_batch64_k50", 256, seed=5, path="device", **VARIANTS["all_three"])


@pytest.mark.parametrize("variant", ["interleaved", "llama31"])
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
