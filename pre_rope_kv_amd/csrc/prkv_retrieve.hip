// Exact top-k retrieval on gfx950: inner products of a request's query
// embedding with every fact embedding of the request's store, then the k best
// facts in rank order.  Output is the fact-id list the inject path consumes.
//
// Source (page "InferScale: GPU-Native KV Injection for Personalized LLM
// Serving", Pith review of arXiv 2607.27090): "Referee Report", Summary --
// facts are retrieved at serving time through a GPU index and their ids then
// resolve to pre-RoPE KV; Figure 2 caption -- each fact has a retrieval
// embedding in the GPU vector store under the same fact_id; "Circularity
// Check" -- the index backend changes latency, not which facts are found.
// Exact search stands in for the approximate index.
//
// score_kernel: one wave per group of facts of one request (8 facts, or 2
// when 8 would leave fewer than two workgroups per CU, e.g. one request: then
// the store's rows are read by four times as many waves).  The query is
// read once per wave; lane l owns elements [8l + 512j, 8l + 512j + 8) of the
// embedding (lanes past the width take zeros in the last, partial chunk), so
// every 16-byte load of a fact row is coalesced.  Products of
// two bf16 values are exact; they are accumulated in float64 and reduced
// across the wave with a butterfly (lane exchanges in the VALU, no LDS round
// trips), so a score differs from the exact inner product by ~1e-16
// relative.  HBM bound (the embeddings are read once);
// no MFMA: one query per store is a matrix-vector product.
//
// topk_kernel: 1024-lane workgroups, one per request, or up to 16 per
// request when few requests have many facts (each takes a slice of the
// scores).  Each wave loads two 64-score chunks at a time, sorts each with an
// in-register bitonic network and merges them into its running top-64 (the
// lane-wise better of a best-first and a worst-first list, then a bitonic
// merge); the 16 wave lists are merged in LDS as a tree (4 rounds).  With
// several slices, topk_merge_kernel merges their top-64 lists the same way
// (k <= 64, so the request's best k are among them).  The partner exchanges
// of the networks stay in the VALU (DPP row permutations for lane xor 1, 2,
// 4, 8; the permlane swaps for xor 16 and 32) and every compare-exchange is
// branch-free, so the kernel is bound by the VALU work of its 16 waves on
// one CU rather than by LDS round trips.
// Order: higher score first, then smaller fact id, so ties are deterministic.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "prkv_device_common.h"
#include "prkv_internal.h"

namespace {

using prkv_dev::xor_lane;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kScoreWaves = 4;
constexpr int kFactsPerWave = 8;        // facts per wave when the grid fills the chip
constexpr int kFactsPerWaveSmall = 2;   // otherwise
constexpr int kTopkThreads = 1024;
constexpr int kMaxK = 64;
constexpr int kMaxList = 64;   // candidates per partial list (one per lane)

struct ScoreParams {
  const uint16_t* fact_emb;   // [n_stores][F][dim]
  const uint16_t* query_emb;  // [n_req][dim]
  const int32_t* req_store;   // [n_req]
  double* scores;             // [n_req][F]
  int32_t* status;
  int32_t n_req, n_stores, facts_per_store, dim, groups_per_req, facts_per_wave;
};

__device__ __forceinline__ double bf16_lo(unsigned w) {
  return double(__uint_as_float(w << 16));
}
__device__ __forceinline__ double bf16_hi(unsigned w) {
  return double(__uint_as_float(w & 0xffff0000u));
}

// A double from lane (lane ^ M) of the wave, both halves through the lane
// exchanges of prkv_dev::xor_lane (every lane active).
template <int M>
__device__ __forceinline__ double xor_double(double x, int lane) {
  const uint64_t b = uint64_t(__double_as_longlong(x));
  const uint32_t lo = xor_lane<M>(uint32_t(b), lane);
  const uint32_t hi = xor_lane<M>(uint32_t(b >> 32), lane);
  return __longlong_as_double(int64_t((uint64_t(hi) << 32) | lo));
}

template <int CHUNKS>  // ceil(dim / 512); dim is a multiple of 8
__global__ __launch_bounds__(kWave * kScoreWaves) void score_kernel(ScoreParams p) {
  const int gw = blockIdx.x * kScoreWaves + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int r = gw / p.groups_per_req;
  if (r >= p.n_req) return;
  const int f0 = (gw - r * p.groups_per_req) * p.facts_per_wave;
  const int s = p.req_store[r];
  if (s < 0 || s >= p.n_stores) {
    if (lane == 0 && f0 == 0 && p.status) atomicOr(p.status, 64);
    return;
  }
  // The last 512-element chunk may be partial: a lane whose 8 elements lie
  // past dim takes zeros (dim is a multiple of 8, so a lane's piece is
  // wholly inside or wholly outside).
  const bool tail_in = lane * 8 + 512 * (CHUNKS - 1) < p.dim;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 q[CHUNKS];
  const uint16_t* qrow = p.query_emb + int64_t(r) * p.dim + lane * 8;
#pragma unroll
  for (int j = 0; j < CHUNKS; ++j)
    q[j] = (j < CHUNKS - 1 || tail_in) ? *reinterpret_cast<const u32x4*>(qrow + 512 * j) : zero;
  const uint16_t* base = p.fact_emb + (int64_t(s) * p.facts_per_store) * p.dim + lane * 8;
  const int f1 = min(f0 + p.facts_per_wave, p.facts_per_store);
  // G facts' rows are loaded together before any is reduced, so G rows per
  // wave are in flight (G * CHUNKS * 4 VGPRs)
  constexpr int G = CHUNKS <= 2 ? 8 : (CHUNKS <= 4 ? 4 : 2);
  for (int g0 = f0; g0 < f1; g0 += G) {
    u32x4 e[G][CHUNKS];
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const uint16_t* row = base + int64_t(g0 + i < f1 ? g0 + i : f0) * p.dim;
#pragma unroll
      for (int j = 0; j < CHUNKS; ++j)
        e[i][j] = (j < CHUNKS - 1 || tail_in)
                      ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row + 512 * j))
                      : zero;
    }
#pragma unroll
    for (int i = 0; i < G; ++i) {
      double acc = 0.0;
#pragma unroll
      for (int j = 0; j < CHUNKS; ++j) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc = __builtin_fma(bf16_lo(q[j][d]), bf16_lo(e[i][j][d]), acc);
          acc = __builtin_fma(bf16_hi(q[j][d]), bf16_hi(e[i][j][d]), acc);
        }
      }
      // butterfly across the wave (lane exchanges, no LDS round trips)
      acc += xor_double<32>(acc, lane);
      acc += xor_double<16>(acc, lane);
      acc += xor_double<8>(acc, lane);
      acc += xor_double<4>(acc, lane);
      acc += xor_double<2>(acc, lane);
      acc += xor_double<1>(acc, lane);
      if (lane == 0 && g0 + i < f1) p.scores[int64_t(r) * p.facts_per_store + g0 + i] = acc;
    }
  }
}

// Order key: larger is better.  Monotone map of a double to uint64.
__device__ __forceinline__ uint64_t order_key(double x) {
  const uint64_t b = __double_as_longlong(x);
  if (x != x) return 0;  // NaN ranks last
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ double key_value(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double(int64_t(b));
}

struct Cand {
  uint64_t key;
  int32_t id;
};

__device__ __forceinline__ bool better(const Cand& a, const Cand& b) {
  return a.key > b.key || (a.key == b.key && a.id < b.id);
}

template <int M>
__device__ __forceinline__ Cand xor_cand(const Cand& c, int lane) {
  Cand o;
  const uint32_t lo = xor_lane<M>(uint32_t(c.key), lane);
  const uint32_t hi = xor_lane<M>(uint32_t(c.key >> 32), lane);
  o.key = (uint64_t(hi) << 32) | lo;
  o.id = int32_t(xor_lane<M>(uint32_t(c.id), lane));
  return o;
}

// Bitonic compare-exchange with the partner lane ^ ST: within blocks of BLK
// lanes the lower lane keeps the better candidate when the block runs
// best-first.  Blocks alternate direction by the BLK bit of the lane (BLK =
// 128: one block, the whole wave); DESC flips every direction, so a network
// built from these steps sorts worst-first instead.
template <int ST, int BLK, bool DESC>
__device__ __forceinline__ Cand cx(const Cand& v, int lane) {
  const Cand o = xor_cand<ST>(v, lane);
  // the lane keeps the worse of the pair where it is the upper lane of a
  // best-first block or the lower lane of a worst-first one
  const bool flip = ((lane & ST) == 0) != (((lane & BLK) == 0) != DESC);
  const bool ob = (o.key > v.key) | ((o.key == v.key) & (o.id < v.id));
  const bool take = ob != flip;
  Cand r;
  r.key = take ? o.key : v.key;
  r.id = take ? o.id : v.id;
  return r;
}

// Bitonic merge of a bitonic sequence over the wave: strides 32, 16, ..., 1.
template <int BLK, bool DESC>
__device__ __forceinline__ Cand bitonic_merge(Cand v, int lane) {
  v = cx<32, BLK, DESC>(v, lane);
  v = cx<16, BLK, DESC>(v, lane);
  v = cx<8, BLK, DESC>(v, lane);
  v = cx<4, BLK, DESC>(v, lane);
  v = cx<2, BLK, DESC>(v, lane);
  return cx<1, BLK, DESC>(v, lane);
}

// The wave's 64 candidates sorted best-first (DESC: worst-first): bitonic
// sort, blocks of 2, 4, ..., 64 lanes.
template <bool DESC>
__device__ __forceinline__ Cand sort64(Cand v, int lane) {
  v = cx<1, 2, DESC>(v, lane);
  v = cx<2, 4, DESC>(v, lane);
  v = cx<1, 4, DESC>(v, lane);
  v = cx<4, 8, DESC>(v, lane);
  v = cx<2, 8, DESC>(v, lane);
  v = cx<1, 8, DESC>(v, lane);
  v = cx<8, 16, DESC>(v, lane);
  v = cx<4, 16, DESC>(v, lane);
  v = cx<2, 16, DESC>(v, lane);
  v = cx<1, 16, DESC>(v, lane);
  v = cx<16, 32, DESC>(v, lane);
  v = cx<8, 32, DESC>(v, lane);
  v = cx<4, 32, DESC>(v, lane);
  v = cx<2, 32, DESC>(v, lane);
  v = cx<1, 32, DESC>(v, lane);
  return bitonic_merge<128, DESC>(v, lane);
}

// a sorted best-first, b worst-first: the 64 best of both, best-first.  The
// lane-wise better of the two is a bitonic sequence that holds them.
__device__ __forceinline__ Cand merge64(const Cand& a, const Cand& b, int lane) {
  return bitonic_merge<128, false>(better(b, a) ? b : a, lane);
}

struct TopkParams {
  const double* scores;  // [n_req][F]
  const int32_t* req_store;
  int32_t* fact_ids;     // [n_req][k]
  double* out_scores;    // [n_req][k], optional
  uint64_t* part_key;    // [n_req][parts][64] partial lists (parts > 1), workspace
  int32_t* part_id;
  int32_t n_req, n_stores, facts_per_store, k;
  int32_t parts;         // workgroups per request in the first pass
};

// Score slices per request for the first top-k pass: enough workgroups to
// spread a few large requests over the chip (up to 16, at least 1024 scores
// each); one when the requests alone fill it.
inline int topk_parts(int64_t n_req, int64_t facts_per_store) {
  if (n_req <= 0) return 1;
  int parts = int(std::min<int64_t>(16, (256 + n_req - 1) / n_req));
  while (parts > 1 && facts_per_store / parts < 1024) parts /= 2;
  return parts < 1 ? 1 : parts;
}

// Byte offsets of the parts of the retrieval workspace: scores at 0, then
// the partial keys and ids (256-byte aligned), and the total.
struct RetrieveWs {
  size_t keys, ids, total;
  RetrieveWs(int64_t n_req, int64_t facts_per_store) {
    auto up = [](size_t v) { return (v + 255u) / 256u * 256u; };
    const size_t scores = size_t(n_req) * size_t(facts_per_store) * sizeof(double);
    const int parts = topk_parts(n_req, facts_per_store);
    const size_t n = parts > 1 ? size_t(n_req) * size_t(parts) * kMaxList : 0;
    keys = up(scores);
    ids = keys + up(n * sizeof(uint64_t));
    total = parts > 1 ? ids + n * sizeof(int32_t) : scores;
  }
};

// The waves' sorted lists (one Cand per lane, best first) merged in LDS as a
// tree; wave 0 returns the best 64 of the workgroup, best first (the other
// waves return their last list).  In each round wave w < half merges in the
// list of wave w + half, read back to front so that it runs worst-first; it
// writes only its own slots, which no wave reads in that round.
__device__ Cand block_merge(Cand best, uint64_t* s_key, int32_t* s_id) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  constexpr int nw = kTopkThreads / kWave;
  s_key[threadIdx.x] = best.key;
  s_id[threadIdx.x] = best.id;
  __syncthreads();
  for (int half = nw / 2; half >= 1; half /= 2) {
    if (wave < half) {
      const int o = (wave + half) * kWave + (kWave - 1 - lane);
      best = merge64(best, Cand{s_key[o], s_id[o]}, lane);
      s_key[threadIdx.x] = best.key;
      s_id[threadIdx.x] = best.id;
    }
    __syncthreads();
  }
  return best;
}

// Lane i < k of wave 0 writes the request's i-th best fact (global id) and
// score.
__device__ void write_topk(const TopkParams& p, int r, int s, bool ok, const Cand& acc) {
  const int lane = threadIdx.x % kWave;
  if (threadIdx.x < kWave && lane < p.k) {
    const int64_t o = int64_t(r) * p.k + lane;
    const bool real = ok && acc.id != INT32_MAX;
    p.fact_ids[o] = real ? s * p.facts_per_store + acc.id : -1;
    if (p.out_scores) p.out_scores[o] = real ? key_value(acc.key) : 0.0;
  }
}

// First pass: workgroup (r, part) keeps the best 64 of its slice of request
// r's scores; with one part it writes the result, otherwise its list.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkParams p) {
  __shared__ uint64_t s_key[kTopkThreads];
  __shared__ int32_t s_id[kTopkThreads];
  const int r = blockIdx.x / p.parts, part = blockIdx.x % p.parts;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int nw = kTopkThreads / kWave;
  const int s = p.req_store[r];
  const bool ok = s >= 0 && s < p.n_stores;
  const double* sc = p.scores + int64_t(r) * p.facts_per_store;
  const Cand worst = {0, INT32_MAX};
  // The score row's address depends only on r, so its loads issue together
  // with that of req_store; a request whose store is out of range takes no
  // candidate (its row in the workspace exists but was not written).
  const int F = p.facts_per_store;
  const int lo = int(int64_t(F) * part / p.parts), hi = int(int64_t(F) * (part + 1) / p.parts);
  // Two 64-score chunks per round, both loaded before either is sorted.  In
  // the first round the chunks are sorted in opposite directions and merged
  // into the running list directly; later rounds sort both worst-first and
  // merge each into it.
  const int64_t step = nw * kWave;
  Cand best = worst;
  for (int64_t c0 = lo + wave * kWave; c0 < hi; c0 += 2 * step) {
    const int64_t f = c0 + lane, g = c0 + step + lane;
    Cand a = worst, b = worst;
    if (f < hi) a = Cand{order_key(sc[f]), int32_t(f)};
    if (g < hi) b = Cand{order_key(sc[g]), int32_t(g)};
    if (!ok) a = b = worst;
    const bool two = c0 + step < hi;
    if (c0 == lo + wave * kWave) {
      best = two ? merge64(sort64<false>(a, lane), sort64<true>(b, lane), lane)
                 : sort64<false>(a, lane);
    } else {
      best = merge64(best, sort64<true>(a, lane), lane);
      if (two) best = merge64(best, sort64<true>(b, lane), lane);
    }
  }
  const Cand acc = block_merge(best, s_key, s_id);
  if (p.parts == 1) {
    write_topk(p, r, s, ok, acc);
  } else if (threadIdx.x < kWave) {
    const int64_t o = (int64_t(r) * p.parts + part) * kMaxList + lane;
    p.part_key[o] = acc.key;
    p.part_id[o] = acc.id;
  }
}

// Second pass (parts > 1): one workgroup per request; wave w < parts loads
// list w (sorted best first) and the lists are merged as in the first pass.
__global__ __launch_bounds__(kTopkThreads) void topk_merge_kernel(TopkParams p) {
  __shared__ uint64_t s_key[kTopkThreads];
  __shared__ int32_t s_id[kTopkThreads];
  const int r = blockIdx.x;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int s = p.req_store[r];
  const bool ok = s >= 0 && s < p.n_stores;
  Cand best = {0, INT32_MAX};
  if (wave < p.parts) {
    const int64_t o = (int64_t(r) * p.parts + wave) * kMaxList + lane;
    best.key = p.part_key[o];
    best.id = p.part_id[o];
  }
  write_topk(p, r, s, ok, block_merge(best, s_key, s_id));
}

template <int CHUNKS>
hipError_t launch_scores(const ScoreParams& p, hipStream_t s) {
  const int64_t waves = int64_t(p.n_req) * p.groups_per_req;
  const int64_t grid = (waves + kScoreWaves - 1) / kScoreWaves;
  hipLaunchKernelGGL(score_kernel<CHUNKS>, dim3(unsigned(grid)), dim3(kWave * kScoreWaves), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int retrieve_workspace_bytes(int32_t n_req, int32_t facts_per_store, size_t* bytes) {
  prkv::clear_error();
  if (!bytes) return prkv::fail(PRKV_ERR_INVALID_ARG, "bytes is NULL");
  if (n_req < 0 || facts_per_store < 0)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "negative size");
  *bytes = RetrieveWs(n_req, facts_per_store).total;
  return PRKV_OK;
}

int retrieve_topk(const void* d_fact_emb, int32_t n_stores, int32_t facts_per_store,
                  int32_t dim, const void* d_query_emb, const int32_t* d_req_store,
                  int32_t n_req, int32_t k, int32_t* d_fact_ids, double* d_scores,
                  void* d_workspace, size_t workspace_bytes, int32_t* d_status, void* stream) {
  prkv::clear_error();
  if (n_req < 0 || n_stores < 1 || facts_per_store < 1)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "bad sizes (n_req %d, n_stores %d, facts %d)", n_req,
                      n_stores, facts_per_store);
  if (k < 1 || k > kMaxK || k > facts_per_store)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "k %d not in [1, min(64, facts_per_store)]", k);
  if (dim < 8 || dim % 8 != 0 || dim > 4096)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "dim %d must be a multiple of 8 in [8, 4096]", dim);
  if (int64_t(n_stores) * facts_per_store > INT32_MAX)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "n_stores * facts_per_store exceeds 2^31-1");
  if (n_req == 0) return PRKV_OK;
  if (!d_fact_emb || !d_query_emb || !d_req_store || !d_fact_ids || !d_workspace)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "NULL pointer argument");
  if ((reinterpret_cast<uintptr_t>(d_fact_emb) | reinterpret_cast<uintptr_t>(d_query_emb)) & 15u)
    return prkv::fail(PRKV_ERR_ALIGNMENT, "embeddings must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(d_workspace) | reinterpret_cast<uintptr_t>(d_scores)) & 7u ||
      (reinterpret_cast<uintptr_t>(d_req_store) | reinterpret_cast<uintptr_t>(d_fact_ids) |
       reinterpret_cast<uintptr_t>(d_status)) & 3u)
    return prkv::fail(PRKV_ERR_ALIGNMENT, "workspace/scores 8-byte, int32 arrays 4-byte aligned");
  const RetrieveWs wl(n_req, facts_per_store);
  const size_t need = wl.total;
  if (workspace_bytes < need)
    return prkv::fail(PRKV_ERR_BUFFER_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                      workspace_bytes);
  ScoreParams sp;
  sp.fact_emb = static_cast<const uint16_t*>(d_fact_emb);
  sp.query_emb = static_cast<const uint16_t*>(d_query_emb);
  sp.req_store = d_req_store;
  sp.scores = static_cast<double*>(d_workspace);
  sp.status = d_status;
  sp.n_req = n_req;
  sp.n_stores = n_stores;
  sp.facts_per_store = facts_per_store;
  sp.dim = dim;
  // fewer facts per wave when the default would leave CUs idle
  const int64_t wgs_default =
      (int64_t(n_req) * ((facts_per_store + kFactsPerWave - 1) / kFactsPerWave) + kScoreWaves - 1) /
      kScoreWaves;
  sp.facts_per_wave =
      wgs_default < 2 * int64_t(prkv::compute_units()) ? kFactsPerWaveSmall : kFactsPerWave;
  sp.groups_per_req = (facts_per_store + sp.facts_per_wave - 1) / sp.facts_per_wave;
  if (int64_t(n_req) * sp.groups_per_req / kScoreWaves + 1 > INT32_MAX)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "grid too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch ((dim + 511) / 512) {
    case 1: e = launch_scores<1>(sp, s); break;
    case 2: e = launch_scores<2>(sp, s); break;
    case 3: e = launch_scores<3>(sp, s); break;
    case 4: e = launch_scores<4>(sp, s); break;
    case 5: e = launch_scores<5>(sp, s); break;
    case 6: e = launch_scores<6>(sp, s); break;
    case 7: e = launch_scores<7>(sp, s); break;
    case 8: e = launch_scores<8>(sp, s); break;
    default: return prkv::fail(PRKV_ERR_INVALID_ARG, "dim %d unsupported", dim);
  }
  if (e != hipSuccess)
    return prkv::fail(PRKV_ERR_HIP, "score launch: %s", hipGetErrorString(e));
  TopkParams tp;
  tp.scores = static_cast<const double*>(d_workspace);
  tp.req_store = d_req_store;
  tp.fact_ids = d_fact_ids;
  tp.out_scores = d_scores;
  tp.n_req = n_req;
  tp.n_stores = n_stores;
  tp.facts_per_store = facts_per_store;
  tp.k = k;
  tp.parts = topk_parts(n_req, facts_per_store);
  if (int64_t(n_req) * tp.parts > INT32_MAX)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "top-k grid too large");
  tp.part_key = reinterpret_cast<uint64_t*>(static_cast<char*>(d_workspace) + wl.keys);
  tp.part_id = reinterpret_cast<int32_t*>(static_cast<char*>(d_workspace) + wl.ids);
  hipLaunchKernelGGL(topk_kernel, dim3(unsigned(int64_t(n_req) * tp.parts)), dim3(kTopkThreads), 0,
                     s, tp);
  if (tp.parts > 1)
    hipLaunchKernelGGL(topk_merge_kernel, dim3(unsigned(n_req)), dim3(kTopkThreads), 0, s, tp);
  e = hipGetLastError();
  if (e != hipSuccess) return prkv::fail(PRKV_ERR_HIP, "top-k launch: %s", hipGetErrorString(e));
  return PRKV_OK;
}

}  // extern "C"
