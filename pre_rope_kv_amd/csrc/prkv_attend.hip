// Query-prefill attention over the injected paged cache, gfx950 (MI355X).
//
// The step after injection: with the retrieved facts' K/V in the paged cache,
// only the query is prefilled, attending causally to the prefix, the
// injected facts and itself.  Source (page "InferScale: GPU-Native KV
// Injection for Personalized LLM Serving", Pith review of arXiv 2607.27090):
// "The pith" (only the query is prefilled), "Core claim" and Theorem 3
// (injected KV at the intended positions is equivalent to prompt-injecting
// the same tokens), reference [1] (grouped-query attention).
//
// The cache is NHD ([block][bs][H][D]: a key's head rows are 256 B apart
// from those of the other heads) or HND ([block][H][bs][D]: one head's keys
// of a block are contiguous); only the address of a key's row differs.
//
// Work unit: one workgroup per (layer, request, KV head, row block).  The
// rows are the q_len query tokens x the `group` query heads sharing that KV
// head, in blocks of 64 (16 per wave); a row block reads the keys up to its
// last query token.  Keys stream in tiles of 32 positions through an LDS
// ring of three tiles: while tile t is computed, tiles t+1 and t+2's K and V
// rows travel from the paged cache straight into LDS (global_load_lds_dwordx4,
// no register staging), gathered through the block table (kept in LDS; the
// slot and cache-row offset of every key are computed once, three tiles
// ahead, by one wave in turn).  Per tile each wave computes
//   S^T = K Q^T - m (v_mfma_f32_16x16x32_bf16 from accumulators that start
//                  at minus the row's running reference m; the accumulator
//                  then holds, per lane, scores of the lane's own query row)
//   online softmax in fp32 (exp2, lazily rescaled running max, running sum)
//   O^T += V^T P^T (same MFMA; S^T's accumulator layout is exactly the B
//                  operand layout P^T needs; the V^T A operand comes from
//                  row-major V through transposing LDS reads,
//                  ds_read_b64_tr_b16)
// Rows are stored unpadded with XOR-swizzled 16-byte chunks so both operand
// reads are free of bank conflicts.  The rotated query and the
// probabilities are split into bf16 hi + lo parts and multiplied twice, so
// the products carry ~16 significant bits and the result is accurate to
// fp32 rounding; K and V are the cache's bf16 values.  At 16 query tokens
// the kernel does about 64 flop per byte of cache (128 with the doubled
// products), below the MFMA ridge: it is bound by reading the cache.
// A three-tile LDS ring (50 KB with the slot and offset buffers, plus the
// block table): three workgroups per CU, each with two tiles in flight while
// it computes the third.  The tile loop is unrolled over the three ring
// slots, so every LDS address of a tile is an immediate offset and the
// per-tile vector-ALU work (which three waves per SIMD share with the matrix
// products) stays small.  Measured on MI355X, this reads the cache at 82-88 %
// of a plain gather of the same rows in the same workgroup split; it is 2 %
// faster than two tiles at four workgroups per CU, and 16-key tiles in a
// six-tile ring (more bytes in flight, twice the barriers) are 13-19 %
// slower.  What a tile costs between its arrival and the reuse of its ring
// slot (the matrix products, softmax, operand reads and the barrier) sets
// the rate, more than the bytes in flight.
//
// The query is rotated in-kernel with the store's RoPE table and pairing
// (compensated fp32, as in injection).  Keys outside [0, q_start + q_len),
// keys after the row's own position (causal), and keys whose block is
// missing from the table (reported in status bit 4) are masked.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "prkv_device_common.h"
#include "prkv_internal.h"

namespace {
using namespace prkv_dev;

constexpr int kWave = 64;
constexpr int kTile = 32;       // keys per tile
constexpr int kStages = 3;      // LDS ring of tiles; kStages - 1 are in flight
constexpr int kSlotRing = 4;    // slot buffers (>= kStages + 1, a power of two)
constexpr int kMaxRows = 64;    // query rows per workgroup
constexpr int kThreads = kMaxRows / 16 * kWave;
constexpr int kBtLds = 2048;    // block-table entries kept in LDS

// a ring slot known at compile time
template <int X>
using Slot = std::integral_constant<int, X>;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;

struct LayerCPtrs {
  const uint16_t* p[prkv::kMaxLayers];
};

struct AttnParams {
  const uint16_t* q;       // [n_req][q_len][Hq][D] pre-RoPE bf16
  const int32_t* q_start;  // [n_req]
  const int32_t* q_lens;   // [n_req] query tokens per request (<= q_len), or null: all q_len
  const int32_t* bt;       // [n_req][bt_stride]
  const int32_t* bt_len;   // [n_req]
  const f32x4* rope;       // [max_position][D/2]
  float* out;              // [L][n_req][q_len][Hq][D]
  int32_t* status;
  int64_t num_blocks;
  float scale_log2;        // softmax scale * log2(e)
  int32_t n_req, q_len, num_q_heads, num_kv_heads, group, rows;
  int32_t row_blocks;      // ceil(rows / kMaxRows) workgroups per (layer, request, KV head)
  int32_t bt_stride, block_size, max_position;
  int32_t bs_shift;        // log2(block_size) when it is a power of two, else -1
  int32_t hnd;             // cache layout HND ([block][H][bs][D]) instead of NHD
};

__device__ __forceinline__ bf16x8 load8(const unsigned char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// A float from lane (lane ^ M) of the wave (every lane active).
template <int M>
__device__ __forceinline__ float xor_f(float x) {
  return __uint_as_float(prkv_dev::xor_lane<M>(__float_as_uint(x), int(threadIdx.x % kWave)));
}

// Transposing LDS read (ds_read_b64_tr_b16): in each group of 16 lanes, lane
// i receives element i % 4 of the 8-byte words addressed by lanes i / 4,
// i / 4 + 4, i / 4 + 8, i / 4 + 12 of its group.
__device__ __forceinline__ uint2 read_tr(const unsigned char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).
constexpr unsigned vmcnt_imm(unsigned n) {
  return (n & 15u) | ((n >> 4) << 14) | (7u << 4) | (15u << 8);
}

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16 l (lds is wave-uniform; the compiler puts it in M0, the s_nop covers the
// M0-to-LDS-DMA hazard).  Written as inline
// assembly on purpose: the compiler then does not track these loads, so it
// does not make every later LDS read wait for them (it cannot tell that they
// fill the other buffer).  The caller waits for them explicitly
// (s_waitcnt vmcnt(0) before the barrier that publishes the tile).
__device__ __forceinline__ void load_lds16(const void* src, uint32_t lds_addr) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(src), "{m0}"(m0)
               : "memory");
}

// BT_LDS: the request's block table is staged in LDS (bt_stride <= kBtLds);
// otherwise it is read from device memory.
// KG: key groups.  With KG > 1 (a grid too small to fill the chip, e.g. one
// request) the workgroup has KG groups of 4 waves with the same rows; group
// g takes key tiles g, g + KG, ... through its own LDS ring, and the groups'
// (max, sum, O) are merged in LDS at the end, so a CU has KG times as many
// tiles in flight for the one workgroup it holds.
template <int D, int STYLE, bool BT_LDS, int KG>
__global__ __launch_bounds__(kThreads * KG) __attribute__((amdgpu_waves_per_eu(3))) void
attend_kernel(AttnParams p, LayerCPtrs kc, LayerCPtrs vc) {
  constexpr int NT = kThreads * KG;      // threads of the workgroup
  constexpr int KB = D / 32;            // 32-wide k-blocks of Q K^T
  constexpr int MT = D / 16;            // 16-dim tiles of O^T
  constexpr int ROWB = D * 2;           // bytes per K or V row
  constexpr int DC = D / 8;             // 16-byte chunks per row
  constexpr int TILEB = kTile * ROWB;   // bytes per K or V tile
  // a ring of tiles of K and V, row-major, 16-byte chunks XOR-swizzled per row
  __shared__ __align__(1024) unsigned char s_kv[KG][kStages][2][TILEB];
  // per key: slot, -1 beyond ctx, -2 missing; and the byte offset of its head
  // row in a layer's cache (0 for a masked key: a valid address)
  __shared__ __align__(16) int s_slots[KG][kSlotRing][kTile];
  __shared__ __align__(16) int64_t s_offs[KG][kSlotRing][kTile];
  extern __shared__ int s_bt[];         // the request's block table (bt_stride <= kBtLds)

  // XCD-aware order: workgroups are dealt round-robin over the 8 XCDs, so
  // logical id (b % 8) * (grid / 8) + b / 8 gives each XCD a contiguous run
  // of (layer, request, head, row block) work: the heads of one cache row,
  // and the row blocks that read the same keys, share an L2.
  const int nwg = gridDim.x;
  const int bid = (nwg % 8 == 0) ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : blockIdx.x;
  const int rb = bid % p.row_blocks;
  const int unit = bid / p.row_blocks;
  const int g = unit % p.num_kv_heads;
  const int r = (unit / p.num_kv_heads) % p.n_req;
  const int layer = unit / (p.num_kv_heads * p.n_req);
  const int lane = threadIdx.x % kWave;
  const int kg = int(threadIdx.x) / kThreads;     // key group
  const int lt = int(threadIdx.x) % kThreads;     // thread within the group
  const int wave = lt / kWave;                    // wave within the group
  const int a = lane / 16, c16 = lane % 16;
  // This request's query tokens: q_lens[r] (a value outside [0, q_len] is
  // reported, status bit 8, and clamped), else q_len.
  int qlen_r = p.q_len;
  if (p.q_lens) {
    const int v = p.q_lens[r];
    if ((v < 0 || v > p.q_len) && threadIdx.x == 0 && p.status) atomicOr(p.status, 8);
    qlen_r = v < 0 ? 0 : (v > p.q_len ? p.q_len : v);
  }
  const int rows_r = qlen_r * p.group;
  // rows (query token, query head of the group) rb * 64 .. rb * 64 + 63;
  // rows past this request's query (but inside q_len) get output 0
  const int row = rb * kMaxRows + wave * 16 + c16;
  const bool row_ok = row < rows_r;
  const bool row_out = row < p.rows;
  const int qi = row_out ? row / p.group : 0;
  const int hq = g * p.group + (row_out ? row % p.group : 0);
  // The query's positions must lie in [0, max_position); a request whose
  // do not is reported (status bit 2) and attends to nothing (output 0).
  const int q_first = p.q_start[r];
  const bool req_ok = q_first >= 0 && q_first <= p.max_position - qlen_r;
  if (!req_ok && threadIdx.x == 0 && p.status) atomicOr(p.status, 2);
  const int q0 = req_ok ? q_first : 0;
  const int qpos = q0 + qi;
  // the row block's first and last query tokens: its keys are [0, ctx), and
  // tiles that end at or before its first query position need no mask; a
  // block with no row of this request reads nothing
  const int qi_first = rb * kMaxRows / p.group;
  const bool block_live = req_ok && rows_r > rb * kMaxRows;
  const int qi_last = block_live ? (min(rows_r, (rb + 1) * kMaxRows) - 1) / p.group : 0;
  const int q_block0 = q0 + qi_first;
  const int ctx = block_live ? q0 + qi_last + 1 : 0;

  // The first kThreads block-table entries are loaded now, so that their
  // latency overlaps the query's (the host checks bt_stride >= 1).
  const int32_t* btr = p.bt + int64_t(r) * p.bt_stride;
  const int bt_first = btr[min(int(threadIdx.x), p.bt_stride - 1)];
  const int nb = min(p.bt_len[r], p.bt_stride);

  // 1. The lane's dims 32kb + 8a + e of its rotated query row, as hi + lo bf16.
  bf16x8 qh[KB] = {}, ql[KB] = {};
  // With several key groups only group 0 loads and rotates the query rows;
  // it hands them to the others through LDS (below).
  if (KG == 1 || kg == 0) {
    float x[KB][8];
    const uint16_t* qr = p.q + ((int64_t(r) * p.q_len + qi) * p.num_q_heads + hq) * D;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qr + 32 * kb + 8 * a);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        x[kb][2 * d] = lo_bf16(w[d]);
        x[kb][2 * d + 1] = hi_bf16(w[d]);
      }
    }
    // The (cos, sin) entries of the lane's D/8 pairs (its D/4 dims), loaded
    // unconditionally (the row index is clamped into the table) so all loads
    // are in flight together; every index is < D/2, inside the position's
    // row.  An out-of-range position rotates by the identity.
    const bool pos_ok = qpos >= 0 && qpos < p.max_position;
    const f32x4* rrow = p.rope + int64_t(pos_ok ? qpos : 0) * (D / 2);
    constexpr int NCS = D / 8;
    f32x4 cs[NCS];
#pragma unroll
    for (int n = 0; n < NCS; ++n) {
      // half split: n = 8kb + e -> pair 32kb + 8a + e; interleaved: n = 4kb + m
      // -> pair 16kb + 4a + m
      const int j = STYLE == PRKV_ROPE_HALF_SPLIT ? 32 * (n / 8) + 8 * a + n % 8
                                                  : 16 * (n / 4) + 4 * a + n % 4;
      cs[n] = rrow[j];
    }
#pragma unroll
    for (int n = 0; n < NCS; ++n) cs[n] = pos_ok ? cs[n] : f32x4{1.f, 0.f, 0.f, 0.f};
    if (STYLE == PRKV_ROPE_HALF_SPLIT) {
#pragma unroll
      for (int kb = 0; kb < KB / 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          // pair 32kb + 8a + e: elements of k-blocks kb and kb + KB/2
          const f32x4 c = cs[8 * kb + e];
          const float x1 = x[kb][e], x2 = x[kb + KB / 2][e];
          x[kb][e] = rot_first(x1, x2, c);
          x[kb + KB / 2][e] = rot_second(x1, x2, c);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          // pair 16kb + 4a + m: dims 2j, 2j + 1 = e 2m, 2m + 1 of k-block kb
          const f32x4 c = cs[4 * kb + m];
          const float x1 = x[kb][2 * m], x2 = x[kb][2 * m + 1];
          x[kb][2 * m] = rot_first(x1, x2, c);
          x[kb][2 * m + 1] = rot_second(x1, x2, c);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = row_ok ? x[kb][e] * p.scale_log2 : 0.f;  // scores come out in log2 units
        const __bf16 h = (__bf16)v;
        qh[kb][e] = h;
        ql[kb][e] = (__bf16)(v - (float)h);
      }
    }
  }
  // Pin the query rotation (and the waits for its loads) here, ahead of the
  // direct tile loads, whose completion the compiler does not track: a wait
  // for the query's loads placed after them would also wait for the tiles.
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) asm volatile("" ::"v"(qh[kb]), "v"(ql[kb]));

  f32x4 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Per row: the reference m_run (-inf until a finite score), m_use the same
  // but 0 while there is none, negm = -m_use in all four accumulator lanes
  // (the score products start from it, so scores come out relative to the
  // reference), thr the relative score that moves the reference.
  float m_run = -INFINITY, l_run = 0.f, m_use = 0.f, thr = -INFINITY;
  f32x4 negm = {0.f, 0.f, 0.f, 0.f};

  const uint16_t* kl = kc.p[layer];
  const uint16_t* vl = vc.p[layer];
  const int64_t row_elems = int64_t(p.num_kv_heads) * D;
  const int ntiles = ctx > 0 ? (ctx + kTile - 1) / kTile : 0;

  // The table is staged in LDS when it fits (nb <= bt_stride <= kBtLds, the
  // dynamic LDS size); a longer one (contexts beyond kBtLds blocks) is read
  // from global memory, where the slots are computed kStages tiles ahead.
  // group 0's rotated query rows for the other key groups, in the first
  // ring (free until the first tile is issued, after two more barriers)
  u32x4* q_share = reinterpret_cast<u32x4*>(&s_kv[0][0][0][0]);
  if constexpr (KG > 1) {
    if (kg == 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        q_share[(2 * kb) * kThreads + lt] = __builtin_bit_cast(u32x4, qh[kb]);
        q_share[(2 * kb + 1) * kThreads + lt] = __builtin_bit_cast(u32x4, ql[kb]);
      }
    }
  }
  if constexpr (BT_LDS) {
    if (int(threadIdx.x) < nb) s_bt[threadIdx.x] = bt_first;
    for (int i = threadIdx.x + NT; i < nb; i += NT) s_bt[i] = btr[i];
  }
  __syncthreads();
  if constexpr (KG > 1) {
    if (kg > 0) {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        qh[kb] = __builtin_bit_cast(bf16x8, q_share[(2 * kb) * kThreads + lt]);
        ql[kb] = __builtin_bit_cast(bf16x8, q_share[(2 * kb + 1) * kThreads + lt]);
      }
    }
  }
  // Slot of position pos < ctx, or -2 when its block is missing from the table.
  auto slot_of = [&](int pos) -> int {
    const int bi = p.bs_shift >= 0 ? pos >> p.bs_shift : pos / p.block_size;
    const int off = pos - bi * p.block_size;
    const int bj = bi < nb ? bi : 0;   // nb <= bt_stride and bt_stride >= 1
    const int64_t blk = BT_LDS ? s_bt[bj] : btr[bj];
    const bool inb = bi < nb && blk >= 0 && blk < p.num_blocks;
    return inb ? int(blk * p.block_size + off) : -2;
  };
  // Is any block of the context missing?  Its keys are masked and reported;
  // with none, a tile that ends at or before the first query position needs
  // no mask at all (every key is visible to every row).
  int bad = 0;
  const int nblk = ctx > 0 ? (ctx - 1) / p.block_size + 1 : 0;
  for (int i = threadIdx.x; i < nblk; i += NT) {
    const int64_t blk = i < nb ? (BT_LDS ? s_bt[i] : btr[i]) : -1;
    bad |= blk < 0 || blk >= p.num_blocks;
  }
  const bool any_missing = __syncthreads_or(bad) != 0;
  if (any_missing && threadIdx.x == 0 && p.status) atomicOr(p.status, 4);

  // LDS layout of a tile: row k (key) of K or V is ROWB contiguous bytes;
  // its logical 16-byte chunk c sits at chunk position c ^ swz(k).  The
  // swizzles make the MFMA operand reads conflict-free without padding
  // (padding is impossible: a direct load fills 1 KB contiguously):
  //   K, read 16 rows x one chunk per 16 lanes: swk spreads the 16 rows over
  //     all 64 banks;
  //   V, read transposed (4 rows x 32 bytes per 16 lanes, 8 rows per 32):
  //     swv moves each row's 32-byte piece to its own bank group.
  auto swk = [](int k) { return D == 128 ? k % 16 : (k / 2) % 8; };
  auto swv = [](int k) { return D == 128 ? 2 * (k % 8) : 2 * ((k / 2) % 4); };

  // Group kg's i-th tile is key tile i * KG + kg; group-local index i runs
  // its ring.  Each key's slot and the byte offset of its head row in a
  // layer's cache (0 for a masked key) are looked up kStages tiles ahead,
  // into a ring of kSlotRing buffers, by the first kTile lanes of the
  // group's wave i % 4, so the work rotates over the SIMDs.
  auto fill_slots = [&](int i) {
    if (wave == (i & 3) && lane < kTile) {
      const int pos = (i * KG + kg) * kTile + lane;
      const int sk = pos < ctx ? slot_of(pos) : -1;
      // element offset of (slot sk, head g): NHD sk * H * D + g * D; HND
      // (with sk = b * bs + o) ((sk - o) * H + o) * D + g * bs * D
      int64_t off = 0;
      if (sk >= 0) {
        if (p.hnd) {
          const int o = p.bs_shift >= 0 ? (sk & (p.block_size - 1)) : sk % p.block_size;
          off = (int64_t(sk - o) * p.num_kv_heads + o) * D + int64_t(g) * p.block_size * D;
        } else {
          off = int64_t(sk) * row_elems + g * D;
        }
      }
      s_slots[kg][i % kSlotRing][lane] = sk;
      s_offs[kg][i % kSlotRing][lane] = 2 * off;
    }
  };
  // Issue the direct loads of tile t into ring slot SLOT (t % kStages, a
  // compile-time constant).  Instruction n of the tile fills 1 KB = rows
  // n * RPI .. n * RPI + RPI - 1; lane l takes row n * RPI + l / DC, chunk
  // position l % DC, i.e. logical chunk (l % DC) ^ swizzle.  Masked keys load
  // from offset 0 (the layer's first cache row, a valid address) and are
  // zeroed before use.
  constexpr int RPI = 64 / DC;                  // rows per load instruction
  constexpr int NI = kTile * DC / 64 / 4;       // instructions per wave per tile, for K and for V
  constexpr unsigned LPT = 2 * NI;              // loads per wave per tile
  static_assert(NI >= 1 && kTile * DC % 256 == 0, "a tile must split over the 4 waves");
  const uint32_t kv_lds =
      uint32_t(reinterpret_cast<uintptr_t>((lds_void*)(&s_kv[kg][0][0][0])));
  // this wave's 1 KB piece of ring slot 0, a scalar: the destination of each
  // load adds a constant to it
  const uint32_t lds_w = __builtin_amdgcn_readfirstlane(kv_lds + uint32_t(wave) * 1024u);
  auto issue = [&](int ti, auto SLOT) {
    constexpr int slot = decltype(SLOT)::value;
    const int64_t* so = s_offs[kg][ti % kSlotRing];
    const uint32_t kd = lds_w + uint32_t(slot) * (2 * TILEB);
    const uint32_t vd = kd + TILEB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = i * 4 + wave;
      const int k = n * RPI + lane / DC;
      const int pk = lane % DC;
      const int64_t off = so[k];
      load_lds16(reinterpret_cast<const char*>(kl + 8 * (pk ^ swk(k))) + off, kd + i * 4096);
      load_lds16(reinterpret_cast<const char*>(vl + 8 * (pk ^ swv(k))) + off, vd + i * 4096);
    }
  };
  // Zero the K and V rows of masked keys of the group's tile in buffer `buf`.
  auto zero_masked = [&](const int* sl, auto SLOT) {
    constexpr int buf = decltype(SLOT)::value;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int e = lt; e < kTile * DC; e += kThreads) {
      const int k = e / DC;
      if (sl[k] < 0) {
        *reinterpret_cast<u32x4*>(s_kv[kg][buf][0] + k * ROWB + 16 * (e % DC)) = zero;
        *reinterpret_cast<u32x4*>(s_kv[kg][buf][1] + k * ROWB + 16 * (e % DC)) = zero;
      }
    }
  };
  // One 64-key tile; `masked` (uniform) applies the causal, context and
  // missing-block mask from the tile's slots.
  auto compute = [&](const unsigned char* kt_lds, const unsigned char* vt_lds, int base,
                     const int* sl, bool masked) {
    constexpr int KT = kTile / 16;      // 16-key blocks of the tile
    // S^T = K Q^T - m_use: lane holds keys 16kt + 4a + i of its row
    f32x4 s[KT];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      s[kt] = negm;
      const int k = 16 * kt + c16;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 ka = load8(kt_lds + k * ROWB + 16 * ((4 * kb + a) ^ swk(k)));
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh[kb], s[kt], 0, 0, 0);
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[kb], s[kt], 0, 0, 0);
      }
    }
    // mask, online softmax (scores are already scaled to log2 units)
    float mt_max = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      if (masked) {
        const int k0 = 16 * kt + 4 * a;
        const int4 s4 = *reinterpret_cast<const int4*>(sl + k0);
        const int sk[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = row_ok & (base + k0 + i <= qpos) & (sk[i] >= 0);
          s[kt][i] = ok ? s[kt][i] : -INFINITY;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) mt_max = fmaxf(mt_max, s[kt][i]);
    }
    // across the lanes holding the same rows, by permlane swaps (no LDS
    // round trip in the tile's dependency chain)
    mt_max = fmaxf(mt_max, xor_f<16>(mt_max));
    mt_max = fmaxf(mt_max, xor_f<32>(mt_max));
    // Lazy rescale: the reference m_run only moves (and O, l are rescaled)
    // when some row of the wave sees a score more than 2^kLazy above it;
    // otherwise the probabilities are taken against the old reference and
    // may exceed 1 (by at most 2^kLazy), which the final division by l
    // cancels exactly.
    // (Scores and mt_max are relative to m_use; the first finite score of a
    // row always sets its reference.)
    constexpr float kLazy = 8.f;
    if (__builtin_amdgcn_ballot_w64(mt_max > thr) != 0) {
      const float m_new = fmaxf(m_run, m_use + mt_max);
      const float alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
      m_run = m_new;
      const float m_use_new = m_new == -INFINITY ? 0.f : m_new;
      const float d = m_use_new - m_use;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) s[kt] -= d;
      m_use = m_use_new;
      negm = f32x4{-m_use, -m_use, -m_use, -m_use};
      thr = m_new == -INFINITY ? -INFINITY : kLazy;
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(s[kt][i]);
        s[kt][i] = e;
        l_run += e;
      }
    }
    // O^T += V^T P^T over two 32-key halves.  The B operand P^T of lane
    // (a, c16) holds keys 32kk + 4a + i and 32kk + 16 + 4a + i (i = 0..3,
    // straight from the S^T accumulators); the A operand V^T needs the same
    // keys for dim c16 of the 16-dim tile, which two transposing reads
    // deliver: source lane c16 addresses key 32kk + 4a + c16 / 4 (+16), dims
    // 16mt + 4 (c16 % 4) .. + 3.
#pragma unroll
    for (int kk = 0; kk < KT / 2; ++kk) {
      // hi parts rounded in pairs; each lo part is the value minus its hi
      // part read back from the packed word
      u32x4 phw, plw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v0 = j < 2 ? s[2 * kk][2 * j] : s[2 * kk + 1][2 * j - 4];
        const float v1 = j < 2 ? s[2 * kk][2 * j + 1] : s[2 * kk + 1][2 * j - 3];
        const unsigned hw = pack_bf16(v0, v1);
        phw[j] = hw;
        plw[j] = pack_bf16(v0 - lo_bf16(hw), v1 - hi_bf16(hw));
      }
      const bf16x8 ph = __builtin_bit_cast(bf16x8, phw);
      const bf16x8 pl = __builtin_bit_cast(bf16x8, plw);
      const int k = 32 * kk + 4 * a + c16 / 4;   // swv(k + 16) == swv(k)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const unsigned char* vp =
            vt_lds + k * ROWB + 16 * ((2 * mt + (c16 % 4) / 2) ^ swv(k)) + 8 * (c16 % 2);
        const uint2 lo4 = read_tr(vp);
        const uint2 hi4 = read_tr(vp + 16 * ROWB);
        const u32x4 packed = {lo4.x, lo4.y, hi4.x, hi4.y};
        const bf16x8 va = __builtin_bit_cast(bf16x8, packed);
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph, o[mt], 0, 0, 0);
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, o[mt], 0, 0, 0);
      }
    }
  };

  if constexpr (KG == 1) {
    // Pipeline: tiles t+1 .. t+kStages-1 stream into the ring while tile t
    // is computed; slots run kStages tiles ahead.
    static_assert(kStages == 3, "the loops below are unrolled over the ring");
    if (ntiles > 0) {
      for (int u = 0; u < kStages && u < ntiles; ++u) fill_slots(u);
      __syncthreads();
      issue(0, Slot<0>{});
      if (ntiles > 1) issue(1, Slot<1>{});
    }
    // Tile t in ring slot SLOT = t % 3 (a constant in each unrolled copy, so
    // the slot's LDS addresses are immediate offsets).
    auto step = [&](int t, auto SLOT) {
      constexpr int rs = decltype(SLOT)::value;
      const int base = t * kTile;
      // this wave's loads of tile t have landed (tile t+1's may still fly)
      if (t + 1 < ntiles) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPT));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();                 // ... and every wave's; tile t-1 is consumed
      __asm__ volatile("" ::: "memory");
      if (t + 2 < ntiles) issue(t + 2, Slot<(rs + 2) % 3>{});
      if (t + 3 < ntiles) fill_slots(t + 3);
      const int* sl = s_slots[0][t % kSlotRing];
      const bool masked = any_missing || base + kTile - 1 > q_block0;
      if (masked) {
        zero_masked(sl, SLOT);
        __syncthreads();
      }
      compute(s_kv[0][rs][0], s_kv[0][rs][1], base, sl, masked);
    };
    for (int t = 0; t < ntiles; t += 3) {
      step(t, Slot<0>{});
      if (t + 1 < ntiles) step(t + 1, Slot<1>{});
      if (t + 2 < ntiles) step(t + 2, Slot<2>{});
    }
  } else {
    // Pipeline (per key group, on its own tiles): tiles i+1 .. i+kStages-1
    // stream into the group's ring while tile i is computed; slots run kStages
    // tiles ahead.  Every group runs n_iter iterations so that the barriers
    // match; a group whose tiles have run out only takes part in them.
    const int n_mine = ntiles > kg ? (ntiles - kg + KG - 1) / KG : 0;   // this group's tiles
    const int n_iter = (ntiles + KG - 1) / KG;
    static_assert(kStages == 3, "the loops below are unrolled over the ring");
    if (n_iter > 0) {
      for (int u = 0; u < kStages && u < n_mine; ++u) fill_slots(u);
      __syncthreads();
      if (n_mine > 0) issue(0, Slot<0>{});
      if (n_mine > 1) issue(1, Slot<1>{});
    }
    auto step = [&](int i, auto SLOT) {
      constexpr int rs = decltype(SLOT)::value;
      const int base = (i * KG + kg) * kTile;
      const bool mine = i < n_mine;
      // this wave's loads of tile i have landed (tile i+1's may still fly)
      if (mine && i + 1 < n_mine) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPT));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();                 // ... and every wave's; tile i-1 is consumed
      __asm__ volatile("" ::: "memory");
      if (i + 2 < n_mine) issue(i + 2, Slot<(rs + 2) % 3>{});
      if (i + 3 < n_mine) fill_slots(i + 3);
      const int* sl = s_slots[kg][i % kSlotRing];
      // Zeroing masked rows is decided for the whole workgroup (the barrier
      // after it must be reached by every wave): by the iteration's last tile.
      const bool any_masked = any_missing || (i + 1) * KG * kTile - 1 > q_block0;
      if (any_masked) {
        if (mine) zero_masked(sl, SLOT);
        __syncthreads();
      }
      const bool masked = any_missing || base + kTile - 1 > q_block0;
      if (mine) compute(s_kv[kg][rs][0], s_kv[kg][rs][1], base, sl, masked);
    };
    for (int i = 0; i < n_iter; i += 3) {
      step(i, Slot<0>{});
      if (i + 1 < n_iter) step(i + 1, Slot<1>{});
      if (i + 2 < n_iter) step(i + 2, Slot<2>{});
    }

  }

  // normalise and write O[layer][r][qi][hq][d], d = 16mt + 4a + i
  float l_tot = l_run + xor_f<16>(l_run);
  l_tot += xor_f<32>(l_tot);
  if constexpr (KG > 1) {
    // Groups 1.. hand (max, sum, O) to group 0 through LDS (the rings are
    // free: every group has waited for and consumed its last tile), and
    // group 0 rescales all to the largest reference and adds them up.
    constexpr int NF = 2 + 4 * MT;                 // floats per thread
    static_assert(sizeof(s_kv) >= size_t(KG - 1) * NF * kThreads * sizeof(float),
                  "merge scratch must fit in the rings");
    float* scratch = reinterpret_cast<float*>(&s_kv[0][0][0][0]);
    __syncthreads();
    if (kg > 0) {
      float* my = scratch + size_t(kg - 1) * NF * kThreads;
      my[lt] = m_run;
      my[kThreads + lt] = l_tot;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) my[(2 + 4 * mt + e) * kThreads + lt] = o[mt][e];
    }
    __syncthreads();
    if (kg > 0) return;
    float m_all = m_run;
#pragma unroll
    for (int g2 = 1; g2 < KG; ++g2)
      m_all = fmaxf(m_all, scratch[size_t(g2 - 1) * NF * kThreads + lt]);
    const float w0 = m_all == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_all);
    l_tot *= w0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] *= w0;
#pragma unroll
    for (int g2 = 1; g2 < KG; ++g2) {
      const float* other = scratch + size_t(g2 - 1) * NF * kThreads;
      const float wg = m_all == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(other[lt] - m_all);
      l_tot += wg * other[kThreads + lt];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[mt][e] += wg * other[(2 + 4 * mt + e) * kThreads + lt];
    }
  }
  if (row_out) {
    const float inv = row_ok && l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = p.out + (((int64_t(layer) * p.n_req + r) * p.q_len + qi) * p.num_q_heads + hq) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4*>(orow + 16 * mt + 4 * a) =
          row_ok ? o[mt] * inv : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

template <int D, int STYLE, int KG>
void launch_attend_kg(const AttnParams& p, const LayerCPtrs& kc, const LayerCPtrs& vc,
                      int64_t grid, hipStream_t s) {
  // the block table is the dynamic LDS: a short table leaves room for more
  // workgroups per CU
  if (p.bt_stride <= kBtLds)
    hipLaunchKernelGGL((attend_kernel<D, STYLE, true, KG>), dim3(unsigned(grid)),
                       dim3(kThreads * KG),
                       size_t(p.bt_stride > 0 ? p.bt_stride : 1) * sizeof(int32_t), s, p, kc, vc);
  else
    hipLaunchKernelGGL((attend_kernel<D, STYLE, false, KG>), dim3(unsigned(grid)),
                       dim3(kThreads * KG), sizeof(int32_t), s, p, kc, vc);
}

template <int D, int STYLE>
void launch_attend_style(const AttnParams& p, const LayerCPtrs& kc, const LayerCPtrs& vc,
                         int64_t grid, hipStream_t s) {
  // A grid of at most one workgroup per CU (e.g. one request: L x H
  // workgroups) leaves each CU one workgroup's tiles in flight: there, three
  // key groups per workgroup (12 waves, three LDS rings) triple them.
  if (grid <= prkv::compute_units())
    launch_attend_kg<D, STYLE, 3>(p, kc, vc, grid, s);
  else
    launch_attend_kg<D, STYLE, 1>(p, kc, vc, grid, s);
}

template <int D>
hipError_t launch_attend(const AttnParams& p, const LayerCPtrs& kc, const LayerCPtrs& vc,
                         int64_t grid, int style, hipStream_t s) {
  if (style == PRKV_ROPE_INTERLEAVED)
    launch_attend_style<D, PRKV_ROPE_INTERLEAVED>(p, kc, vc, grid, s);
  else
    launch_attend_style<D, PRKV_ROPE_HALF_SPLIT>(p, kc, vc, grid, s);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int attend_paged(const prkv_store* st, const prkv_attn_batch* b, void* const* k_cache_layers,
                 void* const* v_cache_layers, int32_t block_size, int64_t num_blocks,
                 float softmax_scale, int32_t* d_status, void* stream) {
  prkv::clear_error();
  if (!st || !b) return prkv::fail(PRKV_ERR_INVALID_ARG, "store or batch is NULL");
  if (!st->device_backed()) return prkv::fail(PRKV_ERR_NO_DEVICE, "metadata-only store");
  const prkv_store_desc& d = st->desc;
  if (d.head_dim != 64 && d.head_dim != 128)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "attention supports head_dim 64 or 128, not %d",
                      d.head_dim);
  if (b->n_req < 0 || b->q_len < 0 || b->num_q_heads < 1 || b->bt_stride < 0)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "bad batch sizes");
  if (b->n_req > 0 && b->q_len > 0 && b->bt_stride < 1)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "bt_stride must be >= 1");
  if (b->num_q_heads % d.num_kv_heads != 0)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "num_q_heads %d not a multiple of %d KV heads",
                      b->num_q_heads, d.num_kv_heads);
  const int group = b->num_q_heads / d.num_kv_heads;
  if (b->q_len > d.max_position)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "q_len %d exceeds max_position %d", b->q_len,
                      d.max_position);
  const int64_t rows = int64_t(b->q_len) * group;
  if (rows > INT32_MAX - kMaxRows)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "q_len * heads per KV head = %lld too large",
                      (long long)rows);
  const int64_t row_blocks = (rows + kMaxRows - 1) / kMaxRows;
  if (block_size < 1 || num_blocks < 1 || num_blocks * int64_t(block_size) > INT32_MAX)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "bad cache shape");
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return prkv::fail(PRKV_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (b->n_req == 0 || b->q_len == 0) return PRKV_OK;
  if (!b->q || !b->q_start || !b->block_tables || !b->bt_len || !b->out || !k_cache_layers ||
      !v_cache_layers)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "NULL pointer argument");
  if ((reinterpret_cast<uintptr_t>(b->q) | reinterpret_cast<uintptr_t>(b->out)) & 15u ||
      (reinterpret_cast<uintptr_t>(b->q_start) | reinterpret_cast<uintptr_t>(b->block_tables) |
       reinterpret_cast<uintptr_t>(b->bt_len) | reinterpret_cast<uintptr_t>(b->q_lens) |
       reinterpret_cast<uintptr_t>(d_status)) & 3u)
    return prkv::fail(PRKV_ERR_ALIGNMENT, "q/out 16-byte, int32 arrays 4-byte aligned");
  LayerCPtrs kc{}, vc{};
  for (int l = 0; l < d.num_layers; ++l) {
    if (!k_cache_layers[l] || !v_cache_layers[l])
      return prkv::fail(PRKV_ERR_INVALID_ARG, "cache pointer of layer %d is NULL", l);
    if ((reinterpret_cast<uintptr_t>(k_cache_layers[l]) |
         reinterpret_cast<uintptr_t>(v_cache_layers[l])) & 15u)
      return prkv::fail(PRKV_ERR_ALIGNMENT, "cache pointer of layer %d not 16-byte aligned", l);
    kc.p[l] = static_cast<const uint16_t*>(k_cache_layers[l]);
    vc.p[l] = static_cast<const uint16_t*>(v_cache_layers[l]);
  }
  const int64_t grid = int64_t(d.num_layers) * b->n_req * d.num_kv_heads * row_blocks;
  if (grid > INT32_MAX) return prkv::fail(PRKV_ERR_INVALID_ARG, "grid too large");
  AttnParams p;
  p.q = b->q;
  p.q_start = b->q_start;
  p.q_lens = b->q_lens;
  p.bt = b->block_tables;
  p.bt_len = b->bt_len;
  p.rope = static_cast<const f32x4*>(st->rope);
  p.out = b->out;
  p.status = d_status;
  p.num_blocks = num_blocks;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.n_req = b->n_req;
  p.q_len = b->q_len;
  p.num_q_heads = b->num_q_heads;
  p.num_kv_heads = d.num_kv_heads;
  p.group = group;
  p.rows = int32_t(rows);
  p.row_blocks = int32_t(row_blocks);
  p.bt_stride = b->bt_stride;
  p.block_size = block_size;
  p.bs_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz(uint32_t(block_size)) : -1;
  p.max_position = d.max_position;
  p.hnd = d.cache_layout == PRKV_CACHE_HND;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = d.head_dim == 64 ? launch_attend<64>(p, kc, vc, grid, d.rope_style, s)
                                        : launch_attend<128>(p, kc, vc, grid, d.rope_style, s);
  if (e != hipSuccess) return prkv::fail(PRKV_ERR_HIP, "attend launch: %s", hipGetErrorString(e));
  return PRKV_OK;
}

}  // extern "C"
