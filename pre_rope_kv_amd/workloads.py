"""Seeded synthetic inputs for retrieve-and-inject.

This module only DRAWS inputs: fact lengths, retrieved fact ids, prefix
lengths, block allocation and the pre-RoPE K/V values.  It holds none of the
method's arithmetic (no positions, no slots, no rotation), so both the CPU
oracle's tests and the HIP path can be fed from it.

The pages' workload is LoCoMo personal memory (InferScale review, "Referee
Report", Summary).  Its conversations and extracted facts are not used: the
five workloads below stand in for them with synthetic facts of stated length
distributions, N(0,1) bfloat16 K/V, and randomly placed cache blocks.

Draw order (fixed, per workload):
  store stream  (seed = store_seed):   1. every fact length, store by store
  request stream (seed = request_seed): 2. k distinct fact ids per request,
                                           order kept (retrieval rank order)
                                        3. prefix lengths (when drawn)
                                        4. one shuffled free list of blocks,
                                           handed out in request order
                                        5. put order of resident facts
  K/V values: per fact, from SeedSequence([store_seed, store, fact]) so they do
  not depend on which facts are resident or where they sit in the arena.
"""

from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass

import numpy as np

SENTINEL_BF16 = 0x7F7F  # finite bf16 (about 3.39e38) marking never-written cache


@dataclass(frozen=True)
class Spec:
    name: str
    num_layers: int
    num_kv_heads: int
    head_dim: int
    rope_theta: float
    n_requests: int           # each request has its own store of facts
    facts_per_store: int
    length_dist: tuple        # ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi)
    k: int                    # retrieved facts per request
    prefix: tuple             # ("fixed", P) | ("uniform", lo, hi)
    block_size: int
    num_blocks: int
    resident: str             # "all" facts put in the store, or only "retrieved" ones
    store_seed: int
    request_seed: int
    query_len: int = 0        # query tokens given blocks after the facts
    num_q_heads: int = 0      # only for the attention-equivalence check
    max_position: int = 16384
    emb_dim: int = 1536       # retrieval embedding width
    rope_style: int = 0       # 0 half-split pairs, 1 interleaved pairs
    llama3_scaling: tuple = None  # (factor, low, high, original max position) or None
    key_layout: int = 0       # 0 pre-RoPE keys, 1 keys rotated at chunk-local positions
    cache_layout: int = 0     # 0 NHD [block][bs][H][D], 1 HND [block][H][bs][D]

    @property
    def row_bytes(self):
        return self.num_kv_heads * self.head_dim * 2

    @property
    def bytes_per_token(self):
        """Algorithmic HBM bytes per injected token: read K,V rows, write K,V rows."""
        return self.num_layers * 4 * self.row_bytes


SPECS = {
    "tiny_L1_H2_D64": Spec(
        name="tiny_L1_H2_D64", num_layers=1, num_kv_heads=2, head_dim=64,
        rope_theta=1.0e4, n_requests=1, facts_per_store=100,
        length_dist=("uniform", 8, 32), k=5, prefix=("fixed", 32),
        block_size=16, num_blocks=64, resident="all",
        store_seed=0, request_seed=0, query_len=4, num_q_heads=8),
    "llama3_8b_k5": Spec(
        name="llama3_8b_k5", num_layers=32, num_kv_heads=8, head_dim=128,
        rope_theta=5.0e5, n_requests=1, facts_per_store=2000,
        length_dist=("uniform", 20, 60), k=5, prefix=("fixed", 64),
        block_size=16, num_blocks=4096, resident="all",
        store_seed=1, request_seed=1),
    "llama3_8b_k50": Spec(
        name="llama3_8b_k50", num_layers=32, num_kv_heads=8, head_dim=128,
        rope_theta=5.0e5, n_requests=1, facts_per_store=2000,
        length_dist=("uniform", 20, 60), k=50, prefix=("fixed", 64),
        block_size=16, num_blocks=4096, resident="all",
        store_seed=1, request_seed=2),          # same store as llama3_8b_k5
    "llama3_8b_batch64_k50": Spec(
        name="llama3_8b_batch64_k50", num_layers=32, num_kv_heads=8, head_dim=128,
        rope_theta=5.0e5, n_requests=64, facts_per_store=2000,
        length_dist=("uniform", 20, 60), k=50, prefix=("fixed", 64),
        block_size=16, num_blocks=131072, resident="retrieved",
        store_seed=3, request_seed=3),
    # one tensor-parallel rank's share of the 64-request batch (1 of 8 KV heads)
    "llama3_8b_batch64_k50_h1": Spec(
        name="llama3_8b_batch64_k50_h1", num_layers=32, num_kv_heads=1, head_dim=128,
        rope_theta=5.0e5, n_requests=64, facts_per_store=2000,
        length_dist=("uniform", 20, 60), k=50, prefix=("fixed", 64),
        block_size=16, num_blocks=131072, resident="retrieved",
        store_seed=3, request_seed=3),
    "llama3_70b_batch16_k50": Spec(
        name="llama3_70b_batch16_k50", num_layers=80, num_kv_heads=8, head_dim=128,
        rope_theta=5.0e5, n_requests=16, facts_per_store=20000,
        length_dist=("lognormal", 40.0, 1.0, 4, 256), k=50, prefix=("uniform", 16, 512),
        block_size=32, num_blocks=8192, resident="retrieved",
        store_seed=4, request_seed=4),
}

ORDER = list(SPECS)  # small to large


def _draw_lengths(rng, spec, n):
    kind = spec.length_dist[0]
    if kind == "uniform":
        _, lo, hi = spec.length_dist
        return rng.integers(lo, hi + 1, size=n).astype(np.int64)
    if kind == "lognormal":
        _, median, sigma, lo, hi = spec.length_dist
        raw = rng.lognormal(mean=math.log(median), sigma=sigma, size=n)
        return np.clip(np.rint(raw), lo, hi).astype(np.int64)
    raise ValueError(kind)


@dataclass
class Workload:
    spec: Spec
    num_blocks: int                 # physical blocks in the cache actually allocated
    lengths: np.ndarray             # [n_requests][facts_per_store] every fact's length
    retrieved: list                 # per request: global fact ids, rank order
    prefix: np.ndarray              # [n_requests] prefix length per request
    block_tables: list              # per request: int64 array of physical block ids
    put_order: list                 # global fact ids in the order they are put
    fact_rows: dict                 # global fact id -> (first arena row, length)
    capacity_rows: int              # arena rows needed for the resident facts

    # ---- id helpers ----------------------------------------------------
    def store_of(self, fact_id):
        return divmod(int(fact_id), self.spec.facts_per_store)

    def length_of(self, fact_id):
        s, f = self.store_of(fact_id)
        return int(self.lengths[s, f])

    @property
    def max_facts(self):
        return self.spec.n_requests * self.spec.facts_per_store

    @property
    def n_tokens(self):
        return int(sum(self.length_of(f) for ids in self.retrieved for f in ids))

    # ---- arrays in the form the C ABI takes ----------------------------
    def csr(self):
        """(req_ptr, fact_ids, start_pos, block_tables[n_req][stride], bt_len), int32."""
        n = self.spec.n_requests
        req_ptr = np.zeros(n + 1, np.int32)
        req_ptr[1:] = np.cumsum([len(ids) for ids in self.retrieved])
        fact_ids = np.concatenate([np.asarray(ids, np.int32) for ids in self.retrieved])
        stride = max(len(bt) for bt in self.block_tables)
        bt = np.full((n, stride), -1, np.int32)
        bt_len = np.zeros(n, np.int32)
        for r, t in enumerate(self.block_tables):
            bt[r, :len(t)] = t
            bt_len[r] = len(t)
        return req_ptr, fact_ids, self.prefix.astype(np.int32), bt, bt_len

    def requests(self):
        """[(fact_ids, prefix, block_table)] per request, plain Python values."""
        return [([int(f) for f in ids], int(p), [int(b) for b in bt])
                for ids, p, bt in zip(self.retrieved, self.prefix, self.block_tables)]

    def listed_blocks(self):
        return sorted(int(b) for bt in self.block_tables for b in bt)

    # ---- K/V values ----------------------------------------------------
    def fact_seed(self, fact_id):
        s, f = self.store_of(fact_id)
        st = np.random.SeedSequence([self.spec.store_seed, s, f]).generate_state(2, np.uint32)
        return (int(st[0]) | (int(st[1]) << 32)) & ((1 << 63) - 1)

    def fact_kv(self, fact_id, device="cpu"):
        """Pre-RoPE (K, V) of one fact as int16 tensors [L][len][H][D] of bf16 bits.

        Values are N(0,1) float32 rounded to bfloat16 by torch; the generator
        is torch's for the given device, so values depend on the device type.
        """
        import torch
        sp = self.spec
        g = torch.Generator(device=device)
        g.manual_seed(self.fact_seed(fact_id))
        shape = (2, sp.num_layers, self.length_of(fact_id), sp.num_kv_heads, sp.head_dim)
        kv = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        kv = kv.to(torch.bfloat16).view(torch.int16)
        return kv[0].contiguous(), kv[1].contiguous()

    # ---- retrieval embeddings -------------------------------------------
    def _gen(self, device, *key):
        import torch
        st = np.random.SeedSequence([self.spec.store_seed, *key]).generate_state(2, np.uint32)
        g = torch.Generator(device=device)
        g.manual_seed((int(st[0]) | (int(st[1]) << 32)) & ((1 << 63) - 1))
        return g

    def _topic(self, r, device):
        """Unit direction standing for what request r asks about."""
        import torch
        E = self.spec.emb_dim
        u = torch.randn(E, generator=self._gen(device, 3_000_017, r), device=device,
                        dtype=torch.float32)
        return u / torch.linalg.vector_norm(u)

    def store_embeddings(self, store, device="cpu"):
        """Retrieval embeddings of one store's facts, int16 bf16 bits [F][E].

        Every fact: N(0, 1/E) per element (norm close to 1).  The facts the
        store's request drew are made relevant to that request's topic u:
        the i-th drawn fact gets + a_i u with a_i = 0.5 - 0.25 i / k, so a
        query along u finds exactly those facts (their scores are >= 0.25,
        every other fact's is N(0, 1/E), about 0.026 per sigma)."""
        import torch
        sp = self.spec
        E = sp.emb_dim
        x = torch.randn((sp.facts_per_store, E), generator=self._gen(device, 2_000_003, store),
                        device=device, dtype=torch.float32) / math.sqrt(E)
        if store < len(self.retrieved):
            ids = self.retrieved[store]
            u = self._topic(store, device)
            for i, f in enumerate(ids):
                x[f - store * sp.facts_per_store] += (0.5 - 0.25 * i / len(ids)) * u
        return x.to(torch.bfloat16).view(torch.int16).contiguous()

    def query_embeddings(self, device="cpu", emb=None):
        """One query per request, int16 bf16 bits [n_req][E]: the request's
        topic direction plus N(0, 0.05^2 / E) noise.  (`emb` is accepted for
        callers that hold the store embeddings; it is not needed.)"""
        import torch
        sp = self.spec
        E = sp.emb_dim
        out = torch.empty((sp.n_requests, E), dtype=torch.float32, device=device)
        for r in range(sp.n_requests):
            noise = torch.randn(E, generator=self._gen(device, 4_000_037, r), device=device,
                                dtype=torch.float32)
            out[r] = self._topic(r, device) + 0.05 / math.sqrt(E) * noise
        return out.to(torch.bfloat16).view(torch.int16).contiguous()

    def req_store(self):
        """Store searched by each request: request r owns store r."""
        return np.arange(self.spec.n_requests, dtype=np.int32)

    def extras_kv(self, tag, shape, device="cpu"):
        """Extra seeded N(0,1) bf16 tensor (prefix / query content), int16 bits."""
        import torch
        st = np.random.SeedSequence([self.spec.store_seed, 1_000_003, tag]).generate_state(2, np.uint32)
        g = torch.Generator(device=device)
        g.manual_seed((int(st[0]) | (int(st[1]) << 32)) & ((1 << 63) - 1))
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return x.to(torch.bfloat16).view(torch.int16).contiguous()


def make(spec_or_name, num_blocks=None):
    """Draw the workload.  num_blocks overrides the cache size (it changes the draw)."""
    spec = SPECS[spec_or_name] if isinstance(spec_or_name, str) else spec_or_name
    nb = int(num_blocks or spec.num_blocks)
    rs = np.random.Generator(np.random.PCG64(np.random.SeedSequence([spec.store_seed])))
    rq = np.random.Generator(np.random.PCG64(np.random.SeedSequence([spec.request_seed, 7])))
    n, F = spec.n_requests, spec.facts_per_store

    # 1. lengths of every fact in every store
    lengths = np.stack([_draw_lengths(rs, spec, F) for _ in range(n)])
    # 2. k distinct ids per request, rank order kept; ids are global (store * F + local)
    retrieved = [[int(r * F + f) for f in rq.choice(F, size=spec.k, replace=False)]
                 for r in range(n)]
    # 3. prefix lengths
    if spec.prefix[0] == "fixed":
        prefix = np.full(n, spec.prefix[1], np.int64)
    else:
        prefix = rq.integers(spec.prefix[1], spec.prefix[2] + 1, size=n).astype(np.int64)
    # 4. one shuffled free list, handed out in request order
    free = rq.permutation(nb)
    block_tables, cursor = [], 0
    for r in range(n):
        used = int(prefix[r]) + sum(int(lengths[divmod(f, F)]) for f in retrieved[r])
        need = -(-(used + spec.query_len) // spec.block_size)
        if cursor + need > nb:
            raise ValueError(f"{spec.name}: {nb} blocks are too few")
        block_tables.append(free[cursor:cursor + need].astype(np.int64))
        cursor += need
    # 5. resident facts and their put order
    if spec.resident == "all":
        put_order = list(range(n * F))
    else:
        flat = [f for ids in retrieved for f in ids]
        put_order = [flat[i] for i in rq.permutation(len(flat))]
    fact_rows, row = {}, 0
    for f in put_order:
        ln = int(lengths[divmod(f, F)])
        fact_rows[f] = (row, ln)
        row += ln
    return Workload(spec=spec, num_blocks=nb, lengths=lengths, retrieved=retrieved,
                    prefix=prefix, block_tables=block_tables, put_order=put_order,
                    fact_rows=fact_rows, capacity_rows=row)


def with_spec(name, **changes):
    """A variant of a named workload (edge cases: other H, D, block size...)."""
    return dataclasses.replace(SPECS[name], **changes)
