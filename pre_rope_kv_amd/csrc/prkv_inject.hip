// Device half of libprkv.so for gfx950 (MI355X): store creation and fact
// upload (HIP runtime copies), and the inject kernel.
//
// Operation (page "InferScale: GPU-Native KV Injection for Personalized LLM
// Serving", Pith review of arXiv 2607.27090): "What carries the argument" --
// keys stored before rotary encoding are re-rotated to serving-time positions
// on injection into the paged cache; "Referee Report", Summary -- retrieved
// facts' KV are scatter-copied into vLLM's paged KV cache; Theorem 6 (ledger
// axiom R_a^T R_b = R_{b-a}) -- rotating at injection is an exact relocation.
//
// The kernel is a pure HBM-bound gather-rotate-scatter: per (token, layer) it
// reads one K row and one V row (H*D bf16 each) from the arenas and writes
// them to the token's slot of that layer's K and V cache.  No MFMA: the
// rotation is a few fp32 VALU operations per element, far below the ridge.
//
// Work layout
//  - A workgroup is 4 waves (256 lanes) and owns a tile of 4 consecutive
//    tokens, one per wave, and a contiguous share ("split") of each token's
//    chunk range, i.e. a range of layers.  There are at least 8 splits, one
//    per XCD (split = workgroup id % splits, and workgroups are dealt to the
//    XCDs round robin), and small batches use more so the grid still covers
//    the chip.  (Measured on MI355X: one token per wave beats 2, 4 or 8 per
//    wave, and 4-wave groups beat 8- or 16-wave groups on the large
//    batches.)
//  - A token's work is L*H*D/16 "chunks"; chunk (l, h, c) covers 8 RoPE
//    pairs: 16 bytes at element h*D + 8c (first half of the head) and 16
//    bytes at h*D + D/2 + 8c (second half).  With half-split pairing these
//    hold x1 and x2 of pairs 8c .. 8c+7; with interleaved pairing each holds
//    4 whole pairs.  Either way a lane owns whole pairs, so no cross-lane
//    exchange is needed.  Lanes take chunks lane, lane+64, ...;
//    since 64 is a multiple of D/16, a lane's c is fixed (lane % (D/16)) and
//    its 8 (cos, sin) pairs are loaded once per token and kept in VGPRs for
//    every layer.
//  - When a (token, layer) row has fewer than 64 chunks (H * D/16 < 64 and
//    dividing it), a wave instead covers 64 / (H * D/16) consecutive tokens
//    of one layer per iteration (a tile is then 4 waves x that many tokens),
//    so every load and store instruction still spans whole consecutive rows
//    (a separate instantiation, MULTI).
//  - Token metadata for the tile is gathered with one coalesced load per
//    lane; each token's cos/sin row (read once per (position, pair) per tile)
//    is staged in LDS, laid out so lanes with consecutive c read consecutive
//    16-byte words.
//  - Rotation: x1' = x1 c - x2 s, x2' = x2 c + x1 s with c = c_hi + c_lo and
//    s = s_hi + s_lo (float32 hi/lo of the float64 value).  The two products
//    with the hi parts are exact as p + e and q + f (FMA error terms); their
//    difference a = p - q is rounded once to float32, which is exact when
//    the products nearly cancel (Sterbenz) -- the case that needs the
//    compensation -- and otherwise costs at most half an ulp of a; the error
//    terms and the lo products are summed in float32 and added to a with one
//    more rounding.  So before the bf16 rounding the value is within about
//    one float32 ulp of the exact rotation, and the bf16 result is the
//    correctly rounded one except near a bf16 rounding boundary, where it
//    can be the neighbour (1 bf16 ulp).  Rounding to bf16 is nearest-even
//    (v_cvt_pk_bf16_f32).
//  - 16-byte nontemporal loads and stores; 64-bit addressing (one layer of
//    a large cache exceeds 4 GiB).  The cache is NHD ([block][bs][H][D]: a
//    token's K row is H * D contiguous elements, like the arena's) or HND
//    ([block][H][bs][D]: each head's D elements land block_size * D apart);
//    only the store address differs.
//  - With the mapping built on the device the token count is known only to
//    the kernel: the host sizes the grid for an expected count (the store's
//    mean fact length), the kernel covers more tokens by its grid stride and
//    gives a small batch more splits; small batches (up to 256 facts and
//    ~4k tokens) build the mapping inside this kernel (fused_plan below),
//    one launch in all.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <mutex>
#include <vector>

#include "prkv_device_common.h"
#include "prkv_internal.h"

// Workspace of inject_topk_device_noalloc, for callers that cannot allocate
// device memory: one array per GPU, held until the process ends.  Host code
// never passes this name to a kernel (on the host it is only a stand-in); it
// uses the device address hipGetSymbolAddress returns (scratch_address).
static __device__ __align__(256) unsigned char scratch[PRKV_NOALLOC_SCRATCH_BYTES];

namespace {
using namespace prkv_dev;


constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;
constexpr int kThreads = kWave * kWavesPerGroup;
constexpr int kUnroll = 2;
constexpr int kXcds = 8;

struct LayerPtrs {
  uint16_t* p[prkv::kMaxLayers];
};

struct FactPlan {
  int32_t tok_start, row0, len, pad;
};

struct DeviceBatch {
  const int32_t* req_fact_ptr;
  const int32_t* fact_ids;
  const int32_t* start_pos;
  const int32_t* block_tables;
  const int32_t* bt_len;
  const int2* fact_table;      // [store max_facts] (first row or -1, length)
  FactPlan* plan;              // workspace
  int64_t* n_tokens_out;       // workspace header
  int32_t* n_facts_out;        // workspace header
  int32_t* src_row;            // workspace, [max_tokens]
  int32_t* pos;
  int32_t* slot;
  int32_t* status;
  uint32_t* slot_table;        // workspace: open-addressing set of slots, or NULL (no check)
  uint32_t table_mask;         // capacity - 1 (capacity a power of two)
  int64_t max_tokens;
  int64_t num_blocks;
  int32_t n_req;
  int32_t bt_stride;
  int32_t max_facts_batch;
  int32_t store_max_facts;
  int32_t block_size;
  int32_t max_position;
  int32_t chunk_local;         // rotation position = the fact's first position
};

struct InjectParams {
  const uint16_t* k_arena;
  const uint16_t* v_arena;
  const f32x4* rope;  // [max_position][D/2] (cos_hi, cos_lo, sin_hi, sin_lo)
  const int32_t* src_row;
  const int32_t* pos;
  const int32_t* slot;
  int32_t* status;
  const int64_t* n_tokens_dev;  // when set, the token count is min(*n_tokens_dev, n_tokens)
  int64_t n_tokens;
  int64_t capacity_rows;
  int64_t num_slots;
  int32_t max_position;
  int32_t num_layers;
  int32_t num_heads;
  int32_t n_splits;          // workgroups per tile
  int32_t iters_per_split;   // 64-chunk iterations (layers when tpw > 1) per split
  int32_t tpw;               // tokens per wave: 64 / (H * D/16) when that divides 64, else 1
  int32_t want_waves;        // waves that cover the chip
  int32_t block_size;
  int32_t hnd;               // cache layout HND ([block][H][bs][D]) instead of NHD
};

// Element offset of (slot, head 0, dim 0) in a layer's cache, and the
// distance between consecutive heads of one slot.  NHD [block][bs][H][D]:
// slot * H * D and D.  HND [block][H][bs][D]: with slot = b * bs + o,
// (b * H * bs + o) * D = ((slot - o) * H + o) * D and bs * D.
template <int D>
__device__ __forceinline__ int64_t cache_slot_base(const InjectParams& p, int slot) {
  if (!p.hnd) return int64_t(slot) * p.num_heads * D;
  const int o = slot % p.block_size;
  return (int64_t(slot - o) * p.num_heads + o) * D;
}

// Half-split pairing: lo holds x1 of pairs 0..7, hi holds x2 of pairs 0..7.
__device__ __forceinline__ void rotate8(u32x4& lo, u32x4& hi, const f32x4 (&cs)[8]) {
  u32x4 olo, ohi;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float a0 = lo_bf16(lo[d]), a1 = hi_bf16(lo[d]);
    const float b0 = lo_bf16(hi[d]), b1 = hi_bf16(hi[d]);
    olo[d] = pack_bf16(rot_first(a0, b0, cs[2 * d]), rot_first(a1, b1, cs[2 * d + 1]));
    ohi[d] = pack_bf16(rot_second(a0, b0, cs[2 * d]), rot_second(a1, b1, cs[2 * d + 1]));
  }
  lo = olo;
  hi = ohi;
}

// Interleaved pairing: word d of `a` is pair 0..3 as (x1, x2), word d of `b`
// is pair 4..7.
__device__ __forceinline__ void rotate8_interleaved(u32x4& a, u32x4& b, const f32x4 (&cs)[8]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const float a1 = lo_bf16(a[d]), a2 = hi_bf16(a[d]);
    const float b1 = lo_bf16(b[d]), b2 = hi_bf16(b[d]);
    a[d] = pack_bf16(rot_first(a1, a2, cs[d]), rot_second(a1, a2, cs[d]));
    b[d] = pack_bf16(rot_first(b1, b2, cs[4 + d]), rot_second(b1, b2, cs[4 + d]));
  }
}

// LDS index of pair j's (cos, sin) within a token's row: the pairs lane c
// needs are k*CPH + c, k = 0..7.  Half-split: the two 16-byte chunks at 8c
// and D/2 + 8c hold pairs 8c .. 8c+7.  Interleaved: the chunk at 8c holds
// pairs 4c .. 4c+3 and the chunk at D/2 + 8c pairs D/4 + 4c .. D/4 + 4c + 3.
template <int D, int STYLE>
__device__ __forceinline__ int pair_slot(int j) {
  constexpr int CPH = D / 16;
  if (STYLE == PRKV_ROPE_HALF_SPLIT) return (j & 7) * CPH + (j >> 3);
  const int hi = j >= D / 4;
  const int jj = j - hi * (D / 4);
  return (4 * hi + (jj & 3)) * CPH + (jj >> 2);
}

__device__ __forceinline__ void flag(int32_t* status, int bits) {
  if (status) atomicOr(status, bits);
}

constexpr uint32_t kSlotEmpty = 0xFFFFFFFFu;   // never a slot (slots are < 2^31 - 1)
constexpr uint32_t kSlotDup = 0x80000000u;
constexpr int kStatusDuplicateSlot = 128;

__device__ __forceinline__ uint32_t slot_hash(uint32_t slot, uint32_t mask) {
  return (slot * 0x9E3779B1u) & mask;   // Fibonacci hashing; slots are not
}                                       // multiples of the capacity in general

// Inserts `slot` into the set; on finding it present, marks it as duplicate.
__device__ __forceinline__ void slot_insert(const DeviceBatch& b, uint32_t slot) {
  uint32_t h = slot_hash(slot, b.table_mask);
  for (uint64_t probe = 0; probe <= uint64_t(b.table_mask); ++probe) {
    const uint32_t prev = atomicCAS(b.slot_table + h, kSlotEmpty, slot);
    if (prev == kSlotEmpty) return;
    if ((prev & ~kSlotDup) == slot) {
      if (!(prev & kSlotDup)) atomicOr(b.slot_table + h, kSlotDup);
      flag(b.status, kStatusDuplicateSlot);
      return;
    }
    h = (h + 1) & b.table_mask;
  }
}

// Whether `slot` (inserted by this call's mapping) is marked duplicate.
__device__ __forceinline__ bool slot_marked(const DeviceBatch& b, uint32_t slot) {
  uint32_t h = slot_hash(slot, b.table_mask);
  for (uint64_t probe = 0; probe <= uint64_t(b.table_mask); ++probe) {
    const uint32_t e = b.slot_table[h];
    if (e == kSlotEmpty) return false;
    if ((e & ~kSlotDup) == slot) return (e & kSlotDup) != 0;
    h = (h + 1) & b.table_mask;
  }
  return false;
}

// ---------------------------------------------------------------------------
// Fused mapping for small batches (at most kFuseFacts facts, kFuseReqs
// requests and kFuseTokens expected tokens): every workgroup of the inject
// kernel rebuilds the batch plan in LDS (one fact per thread) and maps its
// own tile's tokens, so the whole device-side step is one launch instead of
// plan + mapping + inject.  The
// plan, the per-token mapping and every status bit are exactly those of
// plan_kernel and materialize_kernel below; workgroup 0 writes the plan and
// the header to the workspace, and the workgroup with split 0 of each tile
// writes that tile's mapping.
// ---------------------------------------------------------------------------

constexpr int kFuseFacts = kThreads;
constexpr int kFuseReqs = kThreads;
// Above ~4k expected tokens every workgroup rebuilding the plan costs more
// than the two extra launches (measured on MI355X: fused 4 % faster at 50
// facts / 1.9k tokens, 0.5-2 % slower from 100 facts / 3.8k tokens up).
constexpr int64_t kFuseTokens = 4096;
// Up to this many expected tokens the fused grid is capped at one round of
// resident workgroups (launch_inject).
constexpr int64_t kFuseCapTokens = 1024;

struct FusedLds {
  int64_t pos0[kFuseFacts];      // serving position of the fact's first token
  int32_t tok[kFuseFacts];       // first token of the fact (clamped to max_tokens)
  int32_t row0[kFuseFacts];
  int32_t req[kFuseFacts];
  int32_t reqptr[kFuseReqs + 1];
  int32_t start[kFuseReqs];      // per request: prefix length
  int32_t btlen[kFuseReqs];      // per request: block-table length
  int32_t n_facts;
  int64_t wsum[kWavesPerGroup];
};

// Builds the plan in LDS; returns the batch's token count.
__device__ int64_t fused_plan(const DeviceBatch& b, FusedLds& s) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const bool lead = blockIdx.x == 0;
  // the per-request arrays are staged together, so later steps read LDS
  for (int i = tid; i <= b.n_req; i += kThreads) {
    s.reqptr[i] = b.req_fact_ptr[i];
    if (i < b.n_req) {
      s.start[i] = b.start_pos[i];
      s.btlen[i] = b.bt_len[i];
    }
  }
  __syncthreads();
  int n_facts = s.reqptr[b.n_req];
  if (n_facts < 0 || n_facts > b.max_facts_batch) {
    if (lead && tid == 0) flag(b.status, 32);
    n_facts = n_facts < 0 ? 0 : b.max_facts_batch;
  }
  int len = 0, row0 = -1;
  if (tid < n_facts) {
    const int f = b.fact_ids[tid];
    if (f >= 0 && f < b.store_max_facts) {
      const int2 e = b.fact_table[f];
      if (e.x >= 0 && e.y > 0) {
        row0 = e.x;
        len = e.y;
      }
    }
    if (len == 0 && lead) flag(b.status, 8);
  }
  // inclusive scan within the wave (DPP, no LDS round trips), then across
  // the 4 waves
  const int64_t x = prkv_dev::wave_scan_incl(int64_t(len));
  if (lane == kWave - 1) s.wsum[wave] = x;
  __syncthreads();
  int64_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWavesPerGroup; ++w) {
    before += w < wave ? s.wsum[w] : 0;
    total += s.wsum[w];
  }
  const int64_t excl = before + x - len;
  const int32_t tok = int32_t(excl < b.max_tokens ? excl : b.max_tokens);
  if (tid < n_facts) {
    s.tok[tid] = tok;
    s.row0[tid] = row0;
  }
  if (tid == 0) s.n_facts = n_facts;
  __syncthreads();
  if (tid < n_facts) {
    int lo = 0, hi = b.n_req - 1;  // the last request r with reqptr[r] <= tid
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (s.reqptr[mid] <= tid) lo = mid; else hi = mid - 1;
    }
    int first = s.reqptr[lo];
    if (first < 0 || first > tid) first = tid;
    s.req[tid] = lo;
    s.pos0[tid] = int64_t(s.start[lo]) + (tok - s.tok[first]);
    if (lead) {
      FactPlan pl;
      pl.tok_start = tok;
      pl.row0 = row0;
      pl.len = len;
      pl.pad = 0;
      b.plan[tid] = pl;
    }
  }
  const int64_t n_tokens = total < b.max_tokens ? total : b.max_tokens;
  if (lead && tid == 0) {
    if (total > b.max_tokens) flag(b.status, 16);
    *b.n_tokens_out = n_tokens;
    *b.n_facts_out = n_facts;
  }
  __syncthreads();
  return n_tokens;
}

// Token t < n_tokens of a fused batch, in two parts so that the block-table
// load can stay in flight while the tile's K/V rows and cos/sin are loaded.
// fused_map_token: from the plan in LDS, the arena row, the rotation
// position, the request, the serving position ps and bad = 2 when ps is out
// of range; it issues the block-table load and returns the block id (-1:
// none).  fused_finish: the slot from that block id (bad = 4 when the table
// is too short or the id out of range) and, with `report`, the status bits
// and the workspace mapping exactly as materialize_kernel writes them (a
// token that fails gets row -1, position 0, slot 0).
__device__ __forceinline__ int64_t fused_map_token(const DeviceBatch& b, const FusedLds& s,
                                                   int64_t t, int& row, int& pos, int64_t& ps,
                                                   int& bad) {
  int lo = 0, hi = s.n_facts - 1;  // the fact of t: the last f with tok[f] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (s.tok[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int off = int(t - s.tok[lo]);
  const int r = s.req[lo];
  ps = s.pos0[lo] + off;
  row = s.row0[lo] + off;
  bad = (ps < 0 || ps >= b.max_position) ? 2 : 0;
  pos = bad ? 0 : int32_t(b.chunk_local ? s.pos0[lo] : ps);
  if (bad) return -1;
  const int64_t bi = ps / b.block_size;
  return bi < s.btlen[r] && bi < b.bt_stride
             ? int64_t(b.block_tables[int64_t(r) * b.bt_stride + bi]) : -1;
}

__device__ __forceinline__ int fused_finish(const DeviceBatch& b, int64_t t, bool report,
                                            int row, int pos, int64_t ps, int64_t blk, int bad) {
  int slot = 0;
  if (!bad) {
    if (blk < 0 || blk >= b.num_blocks) bad = 4;
    else slot = int32_t(blk * b.block_size + ps % b.block_size);
  }
  if (report) {
    if (bad) flag(b.status, bad);
    b.src_row[t] = bad ? -1 : row;
    b.pos[t] = bad ? 0 : pos;
    b.slot[t] = bad ? 0 : slot;
  }
  return bad ? -1 : slot;
}

template <int D, int STYLE, bool MULTI, bool FUSED>
__global__ __launch_bounds__(kThreads) void inject_kernel(InjectParams p, LayerPtrs kc,
                                                          LayerPtrs vc, DeviceBatch fb) {
  constexpr int CPH = D / 16;   // 16-byte chunks per half head
  constexpr int HALF = D / 2;   // pairs per head
  extern __shared__ f32x4 smem[];

  const int tpw = MULTI ? p.tpw : 1;
  const int tile_tokens = kWavesPerGroup * tpw;
  int* meta = reinterpret_cast<int*>(smem + tile_tokens * HALF);  // row, pos, slot
  int64_t n_tokens = p.n_tokens;
  FusedLds* fused = nullptr;
  if constexpr (FUSED) {
    // after meta, 16-byte aligned
    fused = reinterpret_cast<FusedLds*>(smem + tile_tokens * HALF + (3 * tile_tokens + 3) / 4);
    const int64_t planned = fused_plan(fb, *fused);
    n_tokens = planned < n_tokens ? planned : n_tokens;
  } else if (p.n_tokens_dev) {
    const int64_t dev = *p.n_tokens_dev;
    n_tokens = dev < n_tokens ? (dev < 0 ? 0 : dev) : n_tokens;
  }
  const int64_t n_tiles = (n_tokens + tile_tokens - 1) / tile_tokens;

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int c = lane % CPH;
  const int H = p.num_heads;
  const int nc = H * CPH;                 // chunks per (token, layer) row
  const int total = p.num_layers * nc;    // chunks per token
  const int max_it = tpw > 1 ? p.num_layers : (total + kWave - 1) / kWave;

  // When the count is only known here (device mapping), the host sized the
  // grid for an estimate of it: a larger batch is covered by the grid
  // stride, and a small one gets more splits, with the host's rule, so it
  // does not leave most of the grid idle.
  int n_splits = p.n_splits, per = p.iters_per_split;
  if (FUSED || p.n_tokens_dev) {
    int sp = n_splits;
    while (sp < max_it && n_tiles * sp * 2 <= int64_t(gridDim.x) &&
           n_tiles * sp * kWavesPerGroup < p.want_waves)
      sp *= 2;
    if (sp > max_it) sp = max_it;
    if (sp != n_splits) {
      per = (max_it + sp - 1) / sp;
      per = (per + kUnroll - 1) / kUnroll * kUnroll;
      n_splits = (max_it + per - 1) / per;
    }
  }
  const int split = blockIdx.x % n_splits;
  const int64_t tile_stride = gridDim.x / n_splits;
  const int64_t first_tile =
      blockIdx.x < tile_stride * n_splits ? blockIdx.x / n_splits : n_tiles;  // spare: none
  const int it0 = split * per;
  int it1 = it0 + per;
  if (it1 > max_it) it1 = max_it;
  const int64_t row_elems = int64_t(H) * D;
  const int64_t layer_elems = p.capacity_rows * row_elems;
  const int64_t head_stride = p.hnd ? int64_t(p.block_size) * D : D;  // in the cache

  for (int64_t tile = first_tile; tile < n_tiles; tile += tile_stride) {
    const int64_t tok0 = tile * tile_tokens;
    __syncthreads();  // LDS of the previous tile is no longer read

    // 1. Wave-wide gather of the tile's (row, pos, slot), thread i for token
    //    i (tile_tokens <= kThreads); a row of -1 marks a token to skip,
    //    other out-of-range tokens are reported and skipped.  A fused batch
    //    leaves the slot for step 3: its block-table load is in flight
    //    meanwhile (a slot of -1 then marks a token to skip).
    int f_row = 0, f_pos = 0, f_bad = 0;
    int64_t f_ps = 0, f_blk = -1;
    const bool own_token = int(threadIdx.x) < tile_tokens && tok0 + threadIdx.x < n_tokens;
    if (int(threadIdx.x) < tile_tokens) {
      const int i = threadIdx.x;
      const int64_t t = tok0 + i;
      int row = -1, pos = 0, slot = 0;
      if (own_token) {
        if constexpr (FUSED) {
          f_blk = fused_map_token(fb, *fused, t, f_row, f_pos, f_ps, f_bad);
          row = f_bad ? -1 : f_row;
          pos = f_pos;
        } else {
          row = p.src_row[t];
          pos = p.pos[t];
          slot = p.slot[t];
        }
        const int bad = row == -1 ? 0
                        : ((row < 0 || row >= p.capacity_rows) ? 1 : 0) |
                          ((pos < 0 || pos >= p.max_position) ? 2 : 0) |
                          ((!FUSED && (slot < 0 || slot >= p.num_slots)) ? 4 : 0);
        if (bad) {
          if (p.status && split == 0) atomicOr(p.status, bad);
          row = -1;
        }
      }
      meta[3 * i + 0] = row;
      meta[3 * i + 1] = pos;
      meta[3 * i + 2] = slot;
    }
    __syncthreads();

    // 2. One token per wave: the wave's first layer group is loaded now,
    //    before the cos/sin staging below, so both loads are in flight
    //    together (the K/V rows need only the arena row).
    u32x4 ka[kUnroll], kb[kUnroll], va[kUnroll], vb[kUnroll];
    int lay[kUnroll], hd[kUnroll];
    bool live[kUnroll];
    const int wrow = MULTI ? -1 : __builtin_amdgcn_readfirstlane(meta[3 * wave + 0]);
    auto load_group = [&](int it) {
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int e = (it + u) * kWave + lane;
        live[u] = (it + u) < it1 && e < total;
        const int l = e / nc;
        const int r = e - l * nc;
        lay[u] = l;
        hd[u] = r / CPH;
        if (live[u]) {
          const int64_t aoff = int64_t(l) * layer_elems + int64_t(wrow) * row_elems +
                               int64_t(hd[u]) * D + c * 8;
          ka[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.k_arena + aoff));
          kb[u] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(p.k_arena + aoff + HALF));
          va[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.v_arena + aoff));
          vb[u] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(p.v_arena + aoff + HALF));
        }
      }
    };
    if (!MULTI && wrow >= 0 && it0 < it1) load_group(it0);

    // 3. Stage each token's cos/sin row in LDS, ordered so that lane c reads
    //    its 8 pairs at k*CPH + c (pair_slot).
    for (int e = threadIdx.x; e < tile_tokens * HALF; e += kThreads) {
      const int i = e / HALF, j = e - (e / HALF) * HALF;
      if (meta[3 * i] < 0) continue;
      const f32x4 v = p.rope[int64_t(meta[3 * i + 1]) * HALF + j];
      smem[i * HALF + pair_slot<D, STYLE>(j)] = v;
    }
    if constexpr (FUSED) {
      // the slot from the block id loaded in step 1 (only the slot entry is
      // written here; the loop above reads rows and positions)
      if (own_token)
        meta[3 * threadIdx.x + 2] =
            fused_finish(fb, tok0 + threadIdx.x, split == 0, f_row, f_pos, f_ps, f_blk, f_bad);
    }
    __syncthreads();

    // 4a. Rows narrower than a wave (H * D/16 < 64 chunks): the wave covers
    //     tpw consecutive tokens of the tile, one layer per iteration, so its
    //     loads and stores cover whole consecutive rows.
    if constexpr (MULTI) {
      const int j = wave * tpw + lane / nc;     // the lane's token in the tile
      const int h = (lane % nc) / CPH;
      const int row = meta[3 * j + 0];
      const int slot = meta[3 * j + 2];   // -1: a fused token whose block failed
      f32x4 cs[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) cs[k] = smem[j * HALF + k * CPH + c];
      const int64_t in_row = int64_t(h) * D + c * 8;
      const int64_t a0 = int64_t(row) * row_elems + in_row;
      const int64_t s0 = cache_slot_base<D>(p, slot) + int64_t(h) * head_stride + c * 8;
      if (row >= 0 && slot >= 0) {
        for (int l0 = it0; l0 < it1; l0 += kUnroll) {
          u32x4 ka[kUnroll], kb[kUnroll], va[kUnroll], vb[kUnroll];
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            if (l0 + u < it1) {
              const int64_t aoff = int64_t(l0 + u) * layer_elems + a0;
              ka[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.k_arena + aoff));
              kb[u] = __builtin_nontemporal_load(
                  reinterpret_cast<const u32x4*>(p.k_arena + aoff + HALF));
              va[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p.v_arena + aoff));
              vb[u] = __builtin_nontemporal_load(
                  reinterpret_cast<const u32x4*>(p.v_arena + aoff + HALF));
            }
          }
#pragma unroll
          for (int u = 0; u < kUnroll; ++u) {
            if (l0 + u >= it1) continue;
            if (STYLE == PRKV_ROPE_HALF_SPLIT) rotate8(ka[u], kb[u], cs);
            else rotate8_interleaved(ka[u], kb[u], cs);
            uint16_t* kd = kc.p[l0 + u] + s0;
            uint16_t* vd = vc.p[l0 + u] + s0;
            __builtin_nontemporal_store(ka[u], reinterpret_cast<u32x4*>(kd));
            __builtin_nontemporal_store(kb[u], reinterpret_cast<u32x4*>(kd + HALF));
            __builtin_nontemporal_store(va[u], reinterpret_cast<u32x4*>(vd));
            __builtin_nontemporal_store(vb[u], reinterpret_cast<u32x4*>(vd + HALF));
          }
        }
      }
    } else {
    // 4b. Otherwise each wave streams its one token through every layer of
    //     its split.
    const int row = __builtin_amdgcn_readfirstlane(meta[3 * wave + 0]);
    const int slot = __builtin_amdgcn_readfirstlane(meta[3 * wave + 2]);
    if (row >= 0 && slot >= 0) {   // slot -1: a fused token whose block failed
      const int64_t slot_base = cache_slot_base<D>(p, slot);

      f32x4 cs[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) cs[k] = smem[wave * HALF + k * CPH + c];

      for (int it = it0; it < it1; it += kUnroll) {
        if (it != it0) load_group(it);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          if (!live[u]) continue;
          if (STYLE == PRKV_ROPE_HALF_SPLIT) rotate8(ka[u], kb[u], cs);
          else rotate8_interleaved(ka[u], kb[u], cs);
          const int64_t soff = slot_base + int64_t(hd[u]) * head_stride + c * 8;
          uint16_t* kd = kc.p[lay[u]] + soff;
          uint16_t* vd = vc.p[lay[u]] + soff;
          __builtin_nontemporal_store(ka[u], reinterpret_cast<u32x4*>(kd));
          __builtin_nontemporal_store(kb[u], reinterpret_cast<u32x4*>(kd + HALF));
          __builtin_nontemporal_store(va[u], reinterpret_cast<u32x4*>(vd));
          __builtin_nontemporal_store(vb[u], reinterpret_cast<u32x4*>(vd + HALF));
        }
      }
    }
    }  // MULTI
  }
}


// ---------------------------------------------------------------------------
// Device-side slot mapping (fact ids and block tables resident in HBM).
//
// plan_kernel (one workgroup): per fact of the batch, in request and rank
// order, look up (first row, length) in the device fact table and scan the
// lengths: tok_start = number of injected tokens before the fact.
// materialize_kernel (one wave per fact): find the fact's request, place it
// after the request's prefix and earlier facts (dynamic top-k assembly),
// and write each token's (arena row, position, slot) with full validation;
// a token that fails is written with row -1 (skipped by the inject kernel).
// ---------------------------------------------------------------------------

constexpr int kPlanThreads = 1024;

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(DeviceBatch b) {
  __shared__ int wave_sums[kPlanThreads / kWave];
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  int n_facts = b.n_req > 0 ? b.req_fact_ptr[b.n_req] : 0;
  if (n_facts < 0 || n_facts > b.max_facts_batch) {
    if (tid == 0) flag(b.status, 32);
    n_facts = n_facts < 0 ? 0 : b.max_facts_batch;
  }
  int64_t carry = 0;
  for (int base = 0; base < n_facts; base += kPlanThreads) {
    const int i = base + tid;
    int len = 0, row0 = -1;
    if (i < n_facts) {
      const int f = b.fact_ids[i];
      if (f >= 0 && f < b.store_max_facts) {
        const int2 e = b.fact_table[f];
        if (e.x >= 0 && e.y > 0) {
          row0 = e.x;
          len = e.y;
        }
      }
      if (len == 0) flag(b.status, 8);
    }
    const int x = prkv_dev::wave_scan_incl(int32_t(len));  // inclusive, within the wave
    if (lane == kWave - 1) wave_sums[wave] = x;
    __syncthreads();
    if (wave == 0) {
      static_assert(kPlanThreads / kWave == 16, "the wave sums fill one 16-lane row");
      int s = lane < kPlanThreads / kWave ? wave_sums[lane] : 0;
      s = prkv_dev::row_scan_incl(s);
      if (lane < kPlanThreads / kWave) wave_sums[lane] = s;
    }
    __syncthreads();
    const int64_t excl = carry + (wave > 0 ? wave_sums[wave - 1] : 0) + x - len;
    if (i < n_facts) {
      FactPlan pl;
      pl.tok_start = int32_t(excl < b.max_tokens ? excl : b.max_tokens);
      pl.row0 = row0;
      pl.len = len;
      pl.pad = 0;
      b.plan[i] = pl;
    }
    carry += wave_sums[kPlanThreads / kWave - 1];
    __syncthreads();  // wave_sums is reused by the next chunk
  }
  if (tid == 0) {
    if (carry > b.max_tokens) flag(b.status, 16);
    *b.n_tokens_out = carry < b.max_tokens ? carry : b.max_tokens;
    *b.n_facts_out = n_facts;
  }
}

__global__ __launch_bounds__(kThreads) void materialize_kernel(DeviceBatch b) {
  const int fi = blockIdx.x * kWavesPerGroup + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (fi >= *b.n_facts_out) return;
  const FactPlan pl = b.plan[fi];
  if (pl.len <= 0) return;
  // request of fact fi: the last r with req_fact_ptr[r] <= fi
  int lo = 0, hi = b.n_req - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (b.req_fact_ptr[mid] <= fi) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  int first = b.req_fact_ptr[r];
  if (first < 0 || first > fi) first = fi;
  const int64_t pos0 = int64_t(b.start_pos[r]) + (pl.tok_start - b.plan[first].tok_start);
  const int32_t* bt = b.block_tables + int64_t(r) * b.bt_stride;
  const int nb = b.bt_len[r];
  for (int t = lane; t < pl.len; t += kWave) {
    const int64_t tok = int64_t(pl.tok_start) + t;
    if (tok >= b.max_tokens) break;
    const int64_t ps = pos0 + t;
    int row = pl.row0 + t, slot = 0, bad = 0;
    if (ps < 0 || ps >= b.max_position) {
      bad = 2;
    } else {
      const int64_t bi = ps / b.block_size;
      const int64_t blk = bi < nb && bi < b.bt_stride ? int64_t(bt[bi]) : -1;
      if (blk < 0 || blk >= b.num_blocks) bad = 4;
      else slot = int32_t(blk * b.block_size + ps % b.block_size);
    }
    if (bad) {
      flag(b.status, bad);
      row = -1;
    } else if (b.slot_table) {
      slot_insert(b, slot);
    }
    b.src_row[tok] = row;
    b.pos[tok] = bad ? 0 : int32_t(b.chunk_local ? pos0 : ps);
    b.slot[tok] = slot;
  }
}

// Duplicate-slot check (optional, PRKV_BATCH_CHECK_SLOTS): the mapping
// kernel inserts every valid token's slot into an open-addressing set in the
// workspace (capacity a power of two >= 2 * max_tokens, so an empty entry is
// always found); a slot found already present is marked with the top bit
// (slots are < 2^31) and status bit 128 is set.  resolve_kernel then turns
// every token whose slot is marked into a skipped token (row -1), so neither
// of two colliding tokens is written, as the host builder rejects the batch.
// The set is cleared at the start of every call (clear_table_kernel).

__global__ __launch_bounds__(kThreads) void clear_table_kernel(u32x4* table, int64_t n_vec) {
  const u32x4 empty = {kSlotEmpty, kSlotEmpty, kSlotEmpty, kSlotEmpty};
  for (int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x; i < n_vec;
       i += int64_t(gridDim.x) * kThreads)
    table[i] = empty;
}

__global__ __launch_bounds__(kThreads) void resolve_kernel(DeviceBatch b) {
  const int64_t n = *b.n_tokens_out;
  for (int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x; t < n;
       t += int64_t(gridDim.x) * kThreads) {
    if (b.src_row[t] < 0) continue;
    if (slot_marked(b, uint32_t(b.slot[t]))) b.src_row[t] = -1;
  }
}

int hip_fail(hipError_t e, const char* what) {
  return prkv::fail(PRKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

template <int D, int STYLE, bool MULTI>
void launch_one(const InjectParams& p, const LayerPtrs& kc, const LayerPtrs& vc,
                const DeviceBatch* fused, int64_t grid, size_t lds, hipStream_t s) {
  if (fused)
    hipLaunchKernelGGL((inject_kernel<D, STYLE, MULTI, true>), dim3(unsigned(grid)),
                       dim3(kThreads), lds, s, p, kc, vc, *fused);
  else
    hipLaunchKernelGGL((inject_kernel<D, STYLE, MULTI, false>), dim3(unsigned(grid)),
                       dim3(kThreads), lds, s, p, kc, vc, DeviceBatch{});
}

template <int D>
hipError_t launch(const InjectParams& p, const LayerPtrs& kc, const LayerPtrs& vc,
                  const DeviceBatch* fused, int64_t grid, size_t lds, int style, hipStream_t s) {
  const bool multi = p.tpw > 1;
  if (style == PRKV_ROPE_INTERLEAVED) {
    if (multi) launch_one<D, PRKV_ROPE_INTERLEAVED, true>(p, kc, vc, fused, grid, lds, s);
    else launch_one<D, PRKV_ROPE_INTERLEAVED, false>(p, kc, vc, fused, grid, lds, s);
  } else {
    if (multi) launch_one<D, PRKV_ROPE_HALF_SPLIT, true>(p, kc, vc, fused, grid, lds, s);
    else launch_one<D, PRKV_ROPE_HALF_SPLIT, false>(p, kc, vc, fused, grid, lds, s);
  }
  return hipGetLastError();
}


// Workspace of inject_topk_device: header (n_tokens int64 at 0, n_facts
// int32 at 8), the per-fact plan at 256, then src_row, pos and slot arrays of
// max_tokens int32 each, then the duplicate-slot set (table_entries uint32,
// a power of two >= 2 * max_tokens and >= 64), every part 256-byte aligned.
struct Workspace {
  size_t plan, src_row, pos, slot, table, total;
  uint64_t table_entries;   // <= 2^32 (max_tokens <= 2^31 - 1)
  Workspace(int64_t max_facts, int64_t max_tokens) {
    auto up = [](size_t v) { return (v + 255u) / 256u * 256u; };
    plan = 256;
    src_row = plan + up(size_t(max_facts) * sizeof(FactPlan));
    pos = src_row + up(size_t(max_tokens) * 4u);
    slot = pos + up(size_t(max_tokens) * 4u);
    table = slot + up(size_t(max_tokens) * 4u);
    table_entries = 64;
    while (table_entries < 2 * uint64_t(max_tokens)) table_entries *= 2;
    total = table + size_t(table_entries) * 4u;
  }
};

int check_cache_args(const prkv_store* st, int32_t block_size, int64_t num_blocks,
                     void* const* k_cache_layers, void* const* v_cache_layers) {
  if (!st) return prkv::fail(PRKV_ERR_INVALID_ARG, "store is NULL");
  if (!st->device_backed()) return prkv::fail(PRKV_ERR_NO_DEVICE, "metadata-only store");
  if (block_size < 1 || num_blocks < 1)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "block_size and num_blocks must be >= 1");
  const int64_t num_slots = num_blocks * int64_t(block_size);
  if (num_blocks > INT32_MAX || num_slots > INT32_MAX)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "num_blocks * block_size exceeds 2^31-1");
  if (!k_cache_layers || !v_cache_layers)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "cache pointer arrays are NULL");
  for (int l = 0; l < st->desc.num_layers; ++l) {
    if (!k_cache_layers[l] || !v_cache_layers[l])
      return prkv::fail(PRKV_ERR_INVALID_ARG, "cache pointer of layer %d is NULL", l);
    if (!aligned16(k_cache_layers[l]) || !aligned16(v_cache_layers[l]))
      return prkv::fail(PRKV_ERR_ALIGNMENT, "cache pointer of layer %d not 16-byte aligned", l);
  }
  return PRKV_OK;
}

// Enqueues the inject kernel for up to n_tokens tokens (the exact count is
// *n_tokens_dev when that is set, and the grid is then sized for
// expect_tokens).  With `fused` set, the kernel maps the batch itself (small
// batches, see fused_plan).  Arguments are already validated.
int launch_inject(const prkv_store* st, int64_t n_tokens, const int64_t* n_tokens_dev,
                  const int32_t* d_src_row, const int32_t* d_pos, const int32_t* d_slot,
                  void* const* k_cache_layers, void* const* v_cache_layers, int32_t block_size,
                  int64_t num_blocks, int32_t* d_status, hipStream_t s,
                  const DeviceBatch* fused = nullptr, int64_t expect_tokens = -1) {
  const prkv_store_desc& d = st->desc;
  LayerPtrs kc{}, vc{};
  for (int l = 0; l < d.num_layers; ++l) {
    kc.p[l] = static_cast<uint16_t*>(k_cache_layers[l]);
    vc.p[l] = static_cast<uint16_t*>(v_cache_layers[l]);
  }
  // Launch shape: tiles of 4 waves x tpw tokens; split each token's work
  // across workgroups until the grid holds enough waves to cover the chip.
  const int D = d.head_dim;
  const int nc = d.num_kv_heads * (D / 16);   // 16-byte chunk pairs per (token, layer)
  const int tpw = (nc < kWave && kWave % nc == 0) ? kWave / nc : 1;
  const int64_t chunks = int64_t(d.num_layers) * nc;
  const int iters = tpw > 1 ? d.num_layers : int((chunks + kWave - 1) / kWave);
  const int64_t want_waves = int64_t(prkv::compute_units()) * 16;
  const int64_t tile_tokens = int64_t(kWavesPerGroup) * tpw;
  const bool device_count = n_tokens_dev || fused;
  const int64_t sized_for =
      device_count && expect_tokens >= 0 && expect_tokens < n_tokens ? expect_tokens : n_tokens;
  const int64_t tiles = std::max<int64_t>(1, (sized_for + tile_tokens - 1) / tile_tokens);
  const int64_t tiles_bound = (n_tokens + tile_tokens - 1) / tile_tokens;
  // At least one split per XCD: workgroups are dealt to the 8 XCDs round
  // robin, so split = blockIdx % 8 gives each XCD's L2 and translation caches
  // one range of layers (measured on MI355X: 2-3 % faster than whole tokens
  // per workgroup on the 32- and 80-layer batches).
  int n_splits = kXcds;
  while (n_splits < iters && tiles * n_splits * kWavesPerGroup < want_waves) n_splits *= 2;
  if (n_splits > iters) n_splits = iters;
  int per = (iters + n_splits - 1) / n_splits;
  per = (per + kUnroll - 1) / kUnroll * kUnroll;
  n_splits = (iters + per - 1) / per;
  // at most 2^20 workgroups; each loops over tiles with a grid stride
  const int64_t grid_tiles = tiles < (int64_t(1) << 20) / n_splits ? tiles
                                                                    : (int64_t(1) << 20) / n_splits;
  int64_t grid = grid_tiles * n_splits;
  if (device_count) {
    // The grid is sized for the expected count rather than the bound: a
    // spare workgroup still loads the count before it can exit, and spare
    // ones run last, so a grid sized for a loose bound costs ~0.6 ns per
    // spare workgroup at the end of the kernel (measured: +8 % at 4 x the
    // count).  At least enough workgroups for the kernel to spread a small
    // batch over the chip (its rule stops below 2 * want_waves / 4), which
    // also keeps the chip covered if the estimate is far too low.
    const int64_t spread =
        std::min<int64_t>(want_waves / kWavesPerGroup * 2, tiles_bound * iters);
    if (grid < spread) grid = spread;
  }
  // A fused launch's workgroups each rebuild the batch plan before they know
  // whether a tile is left for them, so a small batch gets at most one
  // residency round of them (four per CU); its tiles are then walked by the
  // grid stride (same-process A/B: k = 5 -8 %, k = 10 -1.4 %, k = 20 -2.9 %;
  // at k = 50, 2k tokens, +1 %, so larger batches keep the wider grid).
  if (fused && expect_tokens >= 0 && expect_tokens <= kFuseCapTokens) {
    const int64_t cap = int64_t(prkv::compute_units()) * 4;
    if (grid > cap) grid = cap;
  }
  size_t lds = size_t(tile_tokens) * (size_t(D / 2) * 16 + 12);
  if (fused)  // the plan follows the metadata at the next 16-byte boundary
    lds = size_t(tile_tokens) * size_t(D / 2) * 16 + size_t((3 * tile_tokens + 3) / 4) * 16 +
          sizeof(FusedLds);

  InjectParams p;
  p.k_arena = static_cast<const uint16_t*>(st->k_arena);
  p.v_arena = static_cast<const uint16_t*>(st->v_arena);
  p.rope = static_cast<const f32x4*>(st->rope);
  p.src_row = d_src_row;
  p.pos = d_pos;
  p.slot = d_slot;
  p.status = d_status;
  p.n_tokens_dev = n_tokens_dev;
  p.n_tokens = n_tokens;
  p.capacity_rows = d.capacity_rows;
  p.num_slots = num_blocks * int64_t(block_size);
  p.max_position = d.max_position;
  p.num_layers = d.num_layers;
  p.num_heads = d.num_kv_heads;
  p.n_splits = n_splits;
  p.iters_per_split = per;
  p.tpw = tpw;
  p.want_waves = int32_t(want_waves);
  p.block_size = block_size;
  p.hnd = d.cache_layout == PRKV_CACHE_HND;

  hipError_t e;
  switch (D) {
    case 16: e = launch<16>(p, kc, vc, fused, grid, lds, d.rope_style, s); break;
    case 32: e = launch<32>(p, kc, vc, fused, grid, lds, d.rope_style, s); break;
    case 64: e = launch<64>(p, kc, vc, fused, grid, lds, d.rope_style, s); break;
    case 128: e = launch<128>(p, kc, vc, fused, grid, lds, d.rope_style, s); break;
    case 256: e = launch<256>(p, kc, vc, fused, grid, lds, d.rope_style, s); break;
    case 512: e = launch<512>(p, kc, vc, fused, grid, lds, d.rope_style, s); break;
    case 1024: e = launch<1024>(p, kc, vc, fused, grid, lds, d.rope_style, s); break;
    default: return prkv::fail(PRKV_ERR_INVALID_ARG, "head_dim %d unsupported", D);
  }
  if (e != hipSuccess) return hip_fail(e, "inject launch");
  return PRKV_OK;
}

}  // namespace

extern "C" {

int store_create(const prkv_store_desc* desc, void* k_arena, void* v_arena, void* rope_table,
                 void* stream, prkv_store** out) {
  prkv::clear_error();
  if (int rc = prkv::validate_desc(desc)) return rc;
  if (!out) return prkv::fail(PRKV_ERR_INVALID_ARG, "out is NULL");
  const bool any = k_arena || v_arena || rope_table;
  const bool all = k_arena && v_arena && rope_table;
  if (any && !all)
    return prkv::fail(PRKV_ERR_INVALID_ARG,
                      "k_arena, v_arena and rope_table must be all set or all NULL");
  if (all && (!aligned16(k_arena) || !aligned16(v_arena) || !aligned16(rope_table)))
    return prkv::fail(PRKV_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  prkv_store* st = nullptr;
  if (int rc = prkv::store_new(desc, &st)) return rc;
  if (all) {
    std::vector<float> table;
    try {
      table.resize(prkv::rope_bytes(*desc) / sizeof(float));
    } catch (const std::bad_alloc&) {
      store_destroy(st);
      return prkv::fail(PRKV_ERR_NO_MEMORY, "rope table staging");
    }
    if (int rc = rope_table_fill(desc, table.data(), table.size() * sizeof(float))) {
      store_destroy(st);
      return rc;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(rope_table, table.data(), prkv::rope_bytes(*desc),
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      store_destroy(st);
      return hip_fail(e, "rope table upload");
    }
    st->k_arena = k_arena;
    st->v_arena = v_arena;
    st->rope = rope_table;
  }
  *out = st;
  return PRKV_OK;
}

int store_put_fact(prkv_store* st, int32_t fact_id, int32_t len, const void* k_src,
                   const void* v_src, void* stream) {
  prkv::clear_error();
  if (int rc = prkv::check_put(st, fact_id, len)) return rc;
  if ((k_src == nullptr) != (v_src == nullptr))
    return prkv::fail(PRKV_ERR_INVALID_ARG, "k_src and v_src must both be set or both NULL");
  if (k_src) {
    if (!st->device_backed())
      return prkv::fail(PRKV_ERR_NO_DEVICE, "metadata-only store cannot take fact data");
    const prkv_store_desc& d = st->desc;
    const size_t row_bytes = size_t(prkv::row_elems(d)) * 2u;
    const size_t width = size_t(len) * row_bytes;
    const size_t dpitch = size_t(d.capacity_rows) * row_bytes;
    const size_t doff = size_t(st->rows_used) * row_bytes;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpy2DAsync(static_cast<char*>(st->k_arena) + doff, dpitch, k_src, width,
                                    width, size_t(d.num_layers), hipMemcpyDefault, s);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(static_cast<char*>(st->v_arena) + doff, dpitch, v_src, width, width,
                           size_t(d.num_layers), hipMemcpyDefault, s);
    if (e != hipSuccess) return hip_fail(e, "fact upload");
  }
  prkv::commit_put(st, fact_id, len);
  return PRKV_OK;
}

int store_stage_facts(const prkv_store* src, prkv_store* dst, int32_t n_facts,
                      const int32_t* fact_ids, void* stream) {
  prkv::clear_error();
  if (!src || !dst) return prkv::fail(PRKV_ERR_INVALID_ARG, "store is NULL");
  if (src == dst) return prkv::fail(PRKV_ERR_INVALID_ARG, "source and destination are one store");
  if (!src->device_backed() || !dst->device_backed())
    return prkv::fail(PRKV_ERR_NO_DEVICE, "metadata-only store");
  const prkv_store_desc& a = src->desc;
  const prkv_store_desc& b = dst->desc;
  if (a.num_layers != b.num_layers || a.num_kv_heads != b.num_kv_heads ||
      a.head_dim != b.head_dim || a.key_layout != b.key_layout)
    return prkv::fail(PRKV_ERR_INVALID_ARG,
                      "stores differ in layers, KV heads, head_dim or key layout");
  if (n_facts < 0 || (n_facts > 0 && !fact_ids))
    return prkv::fail(PRKV_ERR_INVALID_ARG, "bad fact list");
  // Validate everything before enqueueing: each fact is in the source; in
  // the destination it is either present with the same length (its rows are
  // refreshed) or absent (appended; a fact listed twice is appended once).
  std::vector<int64_t> rows;
  std::vector<std::pair<int32_t, int64_t>> appended;   // (fact, row), in order
  try {
    rows.resize(size_t(n_facts));
  } catch (const std::bad_alloc&) {
    return prkv::fail(PRKV_ERR_NO_MEMORY, "staging plan");
  }
  int64_t next = dst->rows_used;
  for (int32_t i = 0; i < n_facts; ++i) {
    const int32_t f = fact_ids[i];
    if (f < 0 || f >= a.max_facts || src->first_row[f] < 0)
      return prkv::fail(PRKV_ERR_UNKNOWN_FACT, "fact %d not in the source store", f);
    if (f >= b.max_facts)
      return prkv::fail(PRKV_ERR_CAPACITY, "fact id %d outside the destination's [0, %d)", f,
                        b.max_facts);
    const int32_t len = src->length[f];
    if (dst->first_row[f] >= 0) {
      if (dst->length[f] != len)
        return prkv::fail(PRKV_ERR_INVALID_ARG, "fact %d has length %d in the destination, %d "
                          "in the source", f, dst->length[f], len);
      rows[i] = dst->first_row[f];
      continue;
    }
    int64_t row = -1;
    for (const auto& pa : appended)
      if (pa.first == f) row = pa.second;
    if (row < 0) {
      if (next + len > b.capacity_rows)
        return prkv::fail(PRKV_ERR_CAPACITY, "fact %d: %d rows exceed the destination's "
                          "capacity", f, len);
      row = next;
      next += len;
      try {
        appended.emplace_back(f, row);
      } catch (const std::bad_alloc&) {
        return prkv::fail(PRKV_ERR_NO_MEMORY, "staging plan");
      }
    }
    rows[i] = row;
  }
  const size_t row_bytes = size_t(prkv::row_elems(a)) * 2u;
  const size_t spitch = size_t(a.capacity_rows) * row_bytes;
  const size_t dpitch = size_t(b.capacity_rows) * row_bytes;
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int32_t i = 0; i < n_facts; ++i) {
    const int32_t f = fact_ids[i];
    const size_t width = size_t(src->length[f]) * row_bytes;
    const size_t soff = size_t(src->first_row[f]) * row_bytes;
    const size_t doff = size_t(rows[i]) * row_bytes;
    hipError_t e = hipMemcpy2DAsync(static_cast<char*>(dst->k_arena) + doff, dpitch,
                                    static_cast<const char*>(src->k_arena) + soff, spitch, width,
                                    size_t(a.num_layers), hipMemcpyDefault, s);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(static_cast<char*>(dst->v_arena) + doff, dpitch,
                           static_cast<const char*>(src->v_arena) + soff, spitch, width,
                           size_t(a.num_layers), hipMemcpyDefault, s);
    if (e != hipSuccess) return hip_fail(e, "fact staging copy");
  }
  for (const auto& pa : appended) prkv::commit_put(dst, pa.first, src->length[pa.first]);
  return PRKV_OK;
}

int inject_topk(const prkv_store* st, int64_t n_tokens, const int32_t* d_src_row,
                const int32_t* d_pos, const int32_t* d_slot, void* const* k_cache_layers,
                void* const* v_cache_layers, int32_t block_size, int64_t num_blocks,
                int32_t* d_status, void* stream) {
  prkv::clear_error();
  if (int rc = check_cache_args(st, block_size, num_blocks, k_cache_layers, v_cache_layers))
    return rc;
  if (n_tokens < 0) return prkv::fail(PRKV_ERR_INVALID_ARG, "n_tokens < 0");
  const int64_t num_slots = num_blocks * int64_t(block_size);
  if (n_tokens > num_slots)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "n_tokens %lld exceeds the cache's %lld slots",
                      (long long)n_tokens, (long long)num_slots);
  if (n_tokens == 0) return PRKV_OK;
  if (!d_src_row || !d_pos || !d_slot)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "NULL pointer argument");
  if ((reinterpret_cast<uintptr_t>(d_src_row) | reinterpret_cast<uintptr_t>(d_pos) |
       reinterpret_cast<uintptr_t>(d_slot) | reinterpret_cast<uintptr_t>(d_status)) & 3u)
    return prkv::fail(PRKV_ERR_ALIGNMENT, "int32 arrays must be 4-byte aligned");
  return launch_inject(st, n_tokens, nullptr, d_src_row, d_pos, d_slot, k_cache_layers,
                       v_cache_layers, block_size, num_blocks, d_status,
                       static_cast<hipStream_t>(stream));
}

int store_upload_fact_table(const prkv_store* st, void* d_table, size_t table_bytes,
                            void* stream) {
  prkv::clear_error();
  if (!st) return prkv::fail(PRKV_ERR_INVALID_ARG, "store is NULL");
  if (!d_table) return prkv::fail(PRKV_ERR_INVALID_ARG, "d_table is NULL");
  if (reinterpret_cast<uintptr_t>(d_table) & 7u)
    return prkv::fail(PRKV_ERR_ALIGNMENT, "d_table must be 8-byte aligned");
  const size_t need = size_t(st->desc.max_facts) * 8u;
  if (table_bytes < need)
    return prkv::fail(PRKV_ERR_BUFFER_TOO_SMALL, "fact table needs %zu bytes, got %zu", need,
                      table_bytes);
  std::vector<int32_t> host;
  try {
    host.resize(size_t(st->desc.max_facts) * 2u);
  } catch (const std::bad_alloc&) {
    return prkv::fail(PRKV_ERR_NO_MEMORY, "fact table staging");
  }
  for (int32_t f = 0; f < st->desc.max_facts; ++f) {
    host[2 * size_t(f)] = int32_t(st->first_row[f]);   // -1 when absent
    host[2 * size_t(f) + 1] = st->length[f];
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(d_table, host.data(), need, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "fact table upload");
  return PRKV_OK;
}

int inject_device_workspace_bytes(int32_t max_facts_batch, int64_t max_tokens, size_t* bytes) {
  prkv::clear_error();
  if (!bytes) return prkv::fail(PRKV_ERR_INVALID_ARG, "bytes is NULL");
  if (max_facts_batch < 0 || max_tokens < 0 || max_tokens > INT32_MAX)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "bad bounds");
  *bytes = Workspace(max_facts_batch, max_tokens).total;
  return PRKV_OK;
}

}  // extern "C"

namespace {

// inject_topk_device's work on a given workspace (the caller's, or the
// library's scratch array for inject_topk_device_noalloc).
int inject_device_impl(const prkv_store* st, const void* d_fact_table,
                       const prkv_device_batch* batch, void* const* k_cache_layers,
                       void* const* v_cache_layers, int32_t block_size, int64_t num_blocks,
                       void* d_workspace, size_t workspace_bytes, int32_t* d_status,
                       void* stream) {
  if (int rc = check_cache_args(st, block_size, num_blocks, k_cache_layers, v_cache_layers))
    return rc;
  if (!batch) return prkv::fail(PRKV_ERR_INVALID_ARG, "batch is NULL");
  const prkv_device_batch& b = *batch;
  if (b.n_req < 0 || b.max_facts < 0 || b.max_tokens < 0 || b.bt_stride < 0)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "negative batch size");
  if (b.flags & ~int32_t(PRKV_BATCH_CHECK_SLOTS))
    return prkv::fail(PRKV_ERR_INVALID_ARG, "unknown batch flags 0x%x", unsigned(b.flags));
  if (b.max_tokens > INT32_MAX) return prkv::fail(PRKV_ERR_INVALID_ARG, "max_tokens > 2^31-1");
  const int64_t num_slots = num_blocks * int64_t(block_size);
  if (b.max_tokens > num_slots)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "max_tokens %lld exceeds the cache's %lld slots",
                      (long long)b.max_tokens, (long long)num_slots);
  if (b.n_req == 0 || b.max_facts == 0 || b.max_tokens == 0) return PRKV_OK;
  if (!d_fact_table || !b.req_fact_ptr || !b.fact_ids || !b.start_pos || !b.bt_len ||
      (!b.block_tables && b.bt_stride > 0) || !d_workspace)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "NULL pointer argument");
  if ((reinterpret_cast<uintptr_t>(d_fact_table) & 7u) ||
      (reinterpret_cast<uintptr_t>(d_workspace) & 255u) ||
      ((reinterpret_cast<uintptr_t>(b.req_fact_ptr) | reinterpret_cast<uintptr_t>(b.fact_ids) |
        reinterpret_cast<uintptr_t>(b.start_pos) | reinterpret_cast<uintptr_t>(b.bt_len) |
        reinterpret_cast<uintptr_t>(b.block_tables) | reinterpret_cast<uintptr_t>(d_status)) &
       3u))
    return prkv::fail(PRKV_ERR_ALIGNMENT,
                      "fact table 8-byte, workspace 256-byte, int32 arrays 4-byte aligned");
  const Workspace ws(b.max_facts, b.max_tokens);
  if (workspace_bytes < ws.total)
    return prkv::fail(PRKV_ERR_BUFFER_TOO_SMALL, "workspace needs %zu bytes, got %zu", ws.total,
                      workspace_bytes);

  char* base = static_cast<char*>(d_workspace);
  DeviceBatch db;
  db.req_fact_ptr = b.req_fact_ptr;
  db.fact_ids = b.fact_ids;
  db.start_pos = b.start_pos;
  db.block_tables = b.block_tables;
  db.bt_len = b.bt_len;
  db.fact_table = static_cast<const int2*>(d_fact_table);
  db.plan = reinterpret_cast<FactPlan*>(base + ws.plan);
  db.n_tokens_out = reinterpret_cast<int64_t*>(base);
  db.n_facts_out = reinterpret_cast<int32_t*>(base + 8);
  db.src_row = reinterpret_cast<int32_t*>(base + ws.src_row);
  db.pos = reinterpret_cast<int32_t*>(base + ws.pos);
  db.slot = reinterpret_cast<int32_t*>(base + ws.slot);
  db.status = d_status;
  db.max_tokens = b.max_tokens;
  db.num_blocks = num_blocks;
  db.n_req = b.n_req;
  db.bt_stride = b.bt_stride;
  db.max_facts_batch = b.max_facts;
  db.store_max_facts = st->desc.max_facts;
  db.block_size = block_size;
  db.max_position = st->desc.max_position;
  db.chunk_local = st->desc.key_layout == PRKV_KEYS_CHUNK_LOCAL;
  const bool check = (b.flags & PRKV_BATCH_CHECK_SLOTS) != 0;
  db.slot_table = check ? reinterpret_cast<uint32_t*>(base + ws.table) : nullptr;
  db.table_mask = uint32_t(ws.table_entries - 1);

  // Expected token count: max_facts facts of the store's mean length, plus
  // 10 %.  The kernels stay correct for any count up to max_tokens.
  int64_t expect = b.max_tokens;
  if (st->facts_put > 0) {
    const double mean = double(st->rows_used) / double(st->facts_put);
    expect = std::min<int64_t>(b.max_tokens, int64_t(1.1 * mean * b.max_facts) + 1);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one launch for small batches; the duplicate check needs the whole
  // mapping before any write, so it always takes the separate kernels
  if (!check && b.max_facts <= kFuseFacts && b.n_req <= kFuseReqs && expect <= kFuseTokens)
    return launch_inject(st, b.max_tokens, nullptr, nullptr, nullptr, nullptr, k_cache_layers,
                         v_cache_layers, block_size, num_blocks, d_status, s, &db, expect);
  hipError_t e;
  if (check) {
    const int64_t n_vec = int64_t(ws.table_entries / 4);
    const int64_t cgrid = std::min<int64_t>((n_vec + kThreads - 1) / kThreads, 1024);
    hipLaunchKernelGGL(clear_table_kernel, dim3(unsigned(cgrid)), dim3(kThreads), 0, s,
                       reinterpret_cast<u32x4*>(db.slot_table), n_vec);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "slot table clear launch");
  }
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, db);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "plan launch");
  const int64_t mgrid = (int64_t(b.max_facts) + kWavesPerGroup - 1) / kWavesPerGroup;
  hipLaunchKernelGGL(materialize_kernel, dim3(unsigned(mgrid)), dim3(kThreads), 0, s, db);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "materialize launch");
  if (check) {
    const int64_t rgrid =
        std::max<int64_t>(1, std::min<int64_t>((expect + kThreads - 1) / kThreads, 2048));
    hipLaunchKernelGGL(resolve_kernel, dim3(unsigned(rgrid)), dim3(kThreads), 0, s, db);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "duplicate-slot resolve launch");
  }
  return launch_inject(st, b.max_tokens, db.n_tokens_out, db.src_row, db.pos, db.slot,
                       k_cache_layers, v_cache_layers, block_size, num_blocks, d_status, s,
                       nullptr, expect);
}

// Device address of this library's scratch array on the device that runs
// `stream`, looked up once per device with that device current (each GPU
// holds its own copy of the array at its own address; the array's name in
// host code is only a host-side stand-in).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_address(hipStream_t stream, void** out) {
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDevice_t dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "device %d beyond the %d the library tracks",
                      int(dev), kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u))
      return prkv::fail(PRKV_ERR_HIP, "scratch array has no 256-byte aligned device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PRKV_OK;
}

}  // namespace

extern "C" {

int inject_topk_device(const prkv_store* st, const void* d_fact_table,
                       const prkv_device_batch* batch, void* const* k_cache_layers,
                       void* const* v_cache_layers, int32_t block_size, int64_t num_blocks,
                       void* d_workspace, size_t workspace_bytes, int32_t* d_status,
                       void* stream) {
  prkv::clear_error();
  return inject_device_impl(st, d_fact_table, batch, k_cache_layers, v_cache_layers, block_size,
                            num_blocks, d_workspace, workspace_bytes, d_status, stream);
}

int inject_topk_device_noalloc(const prkv_store* st, const void* d_fact_table,
                               const prkv_device_batch* batch, void* const* k_cache_layers,
                               void* const* v_cache_layers, int32_t block_size,
                               int64_t num_blocks, int32_t* d_status, void* stream) {
  prkv::clear_error();
  if (!batch) return prkv::fail(PRKV_ERR_INVALID_ARG, "batch is NULL");
  if (batch->max_facts < 0 || batch->max_tokens < 0 || batch->max_tokens > INT32_MAX)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "negative or oversized batch bounds");
  const size_t need = Workspace(batch->max_facts, batch->max_tokens).total;
  if (need > size_t(PRKV_NOALLOC_SCRATCH_BYTES))
    return prkv::fail(PRKV_ERR_BUFFER_TOO_SMALL,
                      "batch bounds (max_facts %d, max_tokens %lld) need %zu workspace bytes; "
                      "the library's scratch holds %zu",
                      batch->max_facts, (long long)batch->max_tokens, need,
                      size_t(PRKV_NOALLOC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (int rc = scratch_address(static_cast<hipStream_t>(stream), &ws)) return rc;
  return inject_device_impl(st, d_fact_table, batch, k_cache_layers, v_cache_layers, block_size,
                            num_blocks, ws, size_t(PRKV_NOALLOC_SCRATCH_BYTES), d_status, stream);
}

}  // extern "C"

namespace prkv {

int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int v = cached[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    n = 256;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace prkv
