"""GPU parity on seeded random combinations of store shape and options: layer
count, KV heads, head_dim, pairing, Llama 3.1 frequency rule, chunk-local
keys, cache layout (NHD or HND), block size, facts and requests drawn
together, so that combinations
no hand-written case names (several options on a row narrower than a wave,
a fused device mapping on a ragged head count...) meet the oracle.  Same bar
as every parity test: V and untouched slots bit-exact, K within 2 bf16 ulp
with mean error < 1e-3."""

import dataclasses

import numpy as np
import pytest

from pre_rope_kv_amd import prkv

from test_gpu_parity import _release_device_memory, custom_workload, run_full  # noqa: F401

pytestmark = pytest.mark.gpu

LLAMA31 = (8.0, 1.0, 4.0, 8192)


@pytest.mark.parametrize("seed", range(64))
def test_random_shape_and_options(seed):
    rng = np.random.default_rng(9000 + seed)
    L = int(rng.integers(1, 7))
    H = int(rng.choice([1, 2, 3, 4, 8]))
    D = int(rng.choice([16, 32, 64, 128, 256]))
    bs = int(rng.choice([1, 8, 16, 32]))
    n_facts = int(rng.integers(1, 9))
    facts = {f: int(rng.integers(1, 50)) for f in range(n_facts)}
    reqs = [([int(x) for x in rng.integers(0, n_facts, size=int(rng.integers(1, 5)))],
             int(rng.integers(0, 300))) for _ in range(int(rng.integers(1, 4)))]
    w = custom_workload(f"shape{seed}", L, H, D, bs, facts, reqs,
                        theta=float(rng.choice([1e4, 5e5])), num_blocks=2048)
    options = dict(rope_style=int(rng.integers(0, 2)),
                   llama3_scaling=LLAMA31 if rng.integers(0, 2) else None,
                   key_layout=int(rng.integers(0, 2)),
                   cache_layout=int(rng.integers(0, 2)))
    w = dataclasses.replace(w, spec=dataclasses.replace(w.spec, **options))
    assert options["rope_style"] in (prkv.ROPE_HALF_SPLIT, prkv.ROPE_INTERLEAVED)
    path = "device" if seed % 2 else "host"
    dw, rep, _ = run_full(w, path=path)
    sp = w.spec
    assert dw.count_non_sentinel() == 2 * sp.num_layers * w.n_tokens * sp.num_kv_heads * sp.head_dim
