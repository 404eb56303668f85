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
// Work unit: one workgroup per (layer, request, KV head).  Its rows are the
// q_len query tokens x the `group` query heads sharing that KV head (at most
// 64 rows, 16 per wave).  Keys stream in tiles of 128 positions: the K rows
// of the tile are gathered through the block table (kept in LDS) into
// registers while the previous tile is computed, then written to LDS
// (row-major, padded), V transposed on the way in.  Per 64-key step of a tile
// each wave computes
//   S^T = K Q^T   (v_mfma_f32_16x16x32_bf16; the accumulator then holds, per
//                  lane, 16 scores of the lane's own query row)
//   online softmax in fp32 (exp2, running max and sum per row)
//   O^T += V^T P^T (same MFMA; S^T's accumulator layout is exactly the B
//                  operand layout P^T needs, with the key order permuted the
//                  same way in V^T's A operand)
// The rotated query and the probabilities are split into bf16 hi + lo parts
// and multiplied twice, so the products carry ~16 significant bits and the
// result is accurate to fp32 rounding; K and V are the cache's bf16 values.
// At 16 query tokens the kernel reads each cache row once per 64 rows of
// work (about 64 flop/B), below the MFMA ridge: it is bound by reading the
// cache, and the doubled MFMAs cost nothing.
//
// The query is rotated in-kernel with the store's RoPE table and pairing
// (compensated fp32, as in injection).  Keys outside [0, q_start + q_len), keys after the
// row's own position (causal), and keys whose block is missing from the
// table (reported in status bit 4) are masked.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "prkv_device_common.h"
#include "prkv_internal.h"

namespace {
using namespace prkv_dev;

constexpr int kWave = 64;
constexpr int kKeys = 64;       // keys per compute step
constexpr int kTile = 128;      // keys staged per tile (two compute steps)
constexpr int kMaxRows = 64;    // query rows per workgroup
constexpr int kThreads = kMaxRows / 16 * kWave;
constexpr int kBtLds = 2048;    // block-table entries kept in LDS
constexpr int kVLanes = 8;      // lanes per run in the V staging
constexpr int kVPad = 8;        // pad bytes per V^T row in LDS

struct LayerCPtrs {
  const uint16_t* p[prkv::kMaxLayers];
};

struct AttnParams {
  const uint16_t* q;       // [n_req][q_len][Hq][D] pre-RoPE bf16
  const int32_t* q_start;  // [n_req]
  const int32_t* bt;       // [n_req][bt_stride]
  const int32_t* bt_len;   // [n_req]
  const f32x4* rope;       // [max_position][D/2]
  float* out;              // [L][n_req][q_len][Hq][D]
  int32_t* status;
  int64_t num_blocks;
  float scale_log2;        // softmax scale * log2(e)
  int32_t n_req, q_len, num_q_heads, num_kv_heads, group, rows;
  int32_t bt_stride, block_size, max_position;
};

__device__ __forceinline__ bf16x8 load8(const unsigned char* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

template <int D, int STYLE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2))) void attend_kernel(AttnParams p, LayerCPtrs kc,
                                                          LayerCPtrs vc) {
  constexpr int KB = D / 32;            // 32-wide k-blocks of Q K^T
  constexpr int MT = D / 16;            // 16-dim tiles of O^T
  constexpr int KROW = D * 2 + 16;      // bytes per K row in LDS (padded)
  constexpr int VROW = kTile * 2 + kVPad;  // bytes per V^T row in LDS (padded)
  constexpr int DC = D / 8;             // 16-byte chunks per head row
  __shared__ __align__(16) unsigned char s_k[kTile * KROW];
  __shared__ __align__(16) unsigned char s_vt[D * VROW];
  __shared__ int s_slot[kTile];         // slot of each key of the tile, -1 if masked
  __shared__ int s_bt[kBtLds];          // the request's block table (first kBtLds entries)

  const int g = blockIdx.x % p.num_kv_heads;
  const int r = (blockIdx.x / p.num_kv_heads) % p.n_req;
  const int layer = blockIdx.x / (p.num_kv_heads * p.n_req);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int a = lane / 16, c16 = lane % 16;
  const int row = wave * 16 + c16;
  const bool row_ok = row < p.rows;
  const int qi = row_ok ? row / p.group : 0;
  const int hq = g * p.group + (row_ok ? row % p.group : 0);
  const int q0 = p.q_start[r];
  const int qpos = q0 + qi;
  const int ctx = q0 + p.q_len;  // keys [0, ctx)

  // 1. The lane's dims 32kb + 8a + e of its rotated query row, as hi + lo bf16.
  bf16x8 qh[KB], ql[KB];
  {
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
    const bool pos_ok = qpos >= 0 && qpos < p.max_position;
    const f32x4* rrow = p.rope + int64_t(pos_ok ? qpos : 0) * (D / 2);
    if (STYLE == PRKV_ROPE_HALF_SPLIT) {
#pragma unroll
      for (int kb = 0; kb < KB / 2; ++kb) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 32 * kb + 8 * a + e;  // pairs with j + D/2 (k-block kb + KB/2)
          const f32x4 cs = pos_ok ? rrow[j] : f32x4{1.f, 0.f, 0.f, 0.f};
          const float x1 = x[kb][e], x2 = x[kb + KB / 2][e];
          x[kb][e] = rot_first(x1, x2, cs);
          x[kb + KB / 2][e] = rot_second(x1, x2, cs);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int j = 16 * kb + 4 * a + m;  // dims 2j, 2j + 1 = e 2m, 2m + 1
          const f32x4 cs = pos_ok ? rrow[j] : f32x4{1.f, 0.f, 0.f, 0.f};
          const float x1 = x[kb][2 * m], x2 = x[kb][2 * m + 1];
          x[kb][2 * m] = rot_first(x1, x2, cs);
          x[kb][2 * m + 1] = rot_second(x1, x2, cs);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = row_ok ? x[kb][e] : 0.f;
        const __bf16 h = (__bf16)v;
        qh[kb][e] = h;
        ql[kb][e] = (__bf16)(v - (float)h);
      }
    }
  }

  f32x4 o[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int32_t* btr = p.bt + int64_t(r) * p.bt_stride;
  const int nb = min(p.bt_len[r], p.bt_stride);
  const uint16_t* kl = kc.p[layer];
  const uint16_t* vl = vc.p[layer];
  const int64_t row_elems = int64_t(p.num_kv_heads) * D;
  const int ntiles = ctx > 0 ? (ctx + kTile - 1) / kTile : 0;

  // Staging of a 128-key tile by the workgroup's lanes: K as kTile x DC
  // 16-byte chunks (KI per lane), V as kTile/4 x DC items of 4 keys x 8 dims
  // (VI per lane).  The loads of tile t+1 are issued into registers before
  // tile t is computed and written to LDS after the next barrier.
  constexpr int KI = kTile * DC / kThreads;
  constexpr int VITEMS = (kTile / 4) * DC;
  constexpr int VI = (VITEMS + kThreads - 1) / kThreads;
  static_assert(KI >= 1 && kTile * DC % kThreads == 0, "K staging must tile the workgroup");
  static_assert(KI + 4 * VI <= 32, "validity bits");
  // (the host checks bt_stride <= kBtLds, so nb <= kBtLds)
  for (int i = threadIdx.x; i < nb; i += kThreads) s_bt[i] = btr[i];
  __syncthreads();
  // Slot of position pos: -1 beyond the context, -2 block missing from the
  // table.  Branch-free, so the prefetch below is straight-line code.
  auto slot_of = [&](int pos) -> int {
    const int bi = pos / p.block_size;
    const int64_t blk = s_bt[bi < nb ? bi : 0];
    const bool inb = bi < nb && blk >= 0 && blk < p.num_blocks;
    const int slot = int(blk * p.block_size + pos % p.block_size);
    return pos >= ctx ? -1 : (inb ? slot : -2);
  };
  // V item -> (key quad, dims chunk): runs of kVLanes consecutive lanes share
  // a dims chunk and take consecutive key quads.  A run writes 64 contiguous
  // bytes of each V^T row it touches, and the next run (next chunk, 8 rows
  // down, 8 * VROW bytes = 16 banks over) lands beside it, so the transposed
  // writes of a half-wave hit distinct banks; in global memory a wave reads
  // 128 contiguous bytes of each of 32 rows.
  static_assert((kTile / 4) % kVLanes == 0, "key quads must tile the lane runs");
  auto v_kq = [](int item) { return item % kVLanes + kVLanes * (item / kVLanes / DC); };
  auto v_dc = [](int item) { return (item / kVLanes) % DC; };
  // Masked keys load slot 0 (always a valid address, a cache hit) and are
  // zeroed at commit; `valid` holds one bit per load.
  u32x4 pk[KI], pv[VI][4];
  uint32_t valid = 0;
  bool missing = false;  // some key's block is missing from the table
  auto prefetch = [&](int base) {
    valid = 0;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const int sk = slot_of(base + c / DC);
      valid |= uint32_t(sk >= 0) << i;
      pk[i] = *reinterpret_cast<const u32x4*>(kl + int64_t(sk >= 0 ? sk : 0) * row_elems +
                                              g * D + 8 * (c % DC));
    }
#pragma unroll
    for (int h = 0; h < VI; ++h) {
      const int item = threadIdx.x + kThreads * h;
      const int it = item < VITEMS ? item : 0;
      const int kq = v_kq(it), dc = v_dc(it);
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const int sv = slot_of(base + 4 * kq + k4);
        valid |= uint32_t(sv >= 0 && item < VITEMS) << (KI + 4 * h + k4);
        pv[h][k4] = *reinterpret_cast<const u32x4*>(vl + int64_t(sv >= 0 ? sv : 0) * row_elems +
                                                    g * D + 8 * dc);
      }
    }
  };
  // registers -> LDS for the tile starting at `base` (call between barriers)
  auto commit = [&](int base) {
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if (threadIdx.x < kTile) {
      const int sl = slot_of(base + threadIdx.x);
      missing |= sl == -2;
      s_slot[threadIdx.x] = sl;
    }
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int c = threadIdx.x + kThreads * i;
      *reinterpret_cast<u32x4*>(s_k + (c / DC) * KROW + (c % DC) * 16) =
          (valid >> i) & 1u ? pk[i] : zero;
    }
#pragma unroll
    for (int h = 0; h < VI; ++h) {
      const int item = threadIdx.x + kThreads * h;
      if (item < VITEMS) {
        const int kq = v_kq(item), dc = v_dc(item);
        u32x4 w[4];
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) w[k4] = (valid >> (KI + 4 * h + k4)) & 1u ? pv[h][k4] : zero;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint2 even, odd;  // dims 8dc + 2d and 8dc + 2d + 1, keys 4kq .. 4kq + 3
          even.x = (w[0][d] & 0xffffu) | (w[1][d] << 16);
          even.y = (w[2][d] & 0xffffu) | (w[3][d] << 16);
          odd.x = (w[0][d] >> 16) | (w[1][d] & 0xffff0000u);
          odd.y = (w[2][d] >> 16) | (w[3][d] & 0xffff0000u);
          *reinterpret_cast<uint2*>(s_vt + (8 * dc + 2 * d) * VROW + 8 * kq) = even;
          *reinterpret_cast<uint2*>(s_vt + (8 * dc + 2 * d + 1) * VROW + 8 * kq) = odd;
        }
      }
    }
  };
  // one 64-key step at key offset `ko` of the staged tile starting at `base`
  auto compute = [&](int base, int ko) {
    // S^T = K Q^T: lane holds keys 16kt + 4a + i of its row
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const bf16x8 ka = load8(s_k + (ko + 16 * kt + c16) * KROW + (32 * kb + 8 * a) * 2);
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh[kb], s[kt], 0, 0, 0);
        s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[kb], s[kt], 0, 0, 0);
      }
    }
    // mask, scale, online softmax
    float mt_max = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = ko + 16 * kt + 4 * a + i;
        const int sk = s_slot[key];
        const bool ok = row_ok & (base + key <= qpos) & (sk >= 0);
        const float v = ok ? s[kt][i] * p.scale_log2 : -INFINITY;
        s[kt][i] = v;
        mt_max = fmaxf(mt_max, v);
      }
    }
    mt_max = fmaxf(mt_max, __shfl_xor(mt_max, 16, kWave));
    mt_max = fmaxf(mt_max, __shfl_xor(mt_max, 32, kWave));
    const float m_new = fmaxf(m_run, mt_max);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    l_run *= alpha;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[mt] *= alpha;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = __builtin_amdgcn_exp2f(s[kt][i] - m_use);
        s[kt][i] = e;
        l_run += e;
      }
    }
    m_run = m_new;
    // O^T += V^T P^T over two 32-key steps
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 ph, pl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = j < 4 ? s[2 * kk][j] : s[2 * kk + 1][j - 4];
        const __bf16 h = (__bf16)v;
        ph[j] = h;
        pl[j] = (__bf16)(v - (float)h);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const unsigned char* vr = s_vt + (16 * mt + c16) * VROW;
        const uint2 lo4 = *reinterpret_cast<const uint2*>(vr + (ko + 32 * kk + 4 * a) * 2);
        const uint2 hi4 = *reinterpret_cast<const uint2*>(vr + (ko + 32 * kk + 16 + 4 * a) * 2);
        const u32x4 packed = {lo4.x, lo4.y, hi4.x, hi4.y};
        const bf16x8 va = __builtin_bit_cast(bf16x8, packed);
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, ph, o[mt], 0, 0, 0);
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pl, o[mt], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) prefetch(0);
  for (int t = 0; t < ntiles; ++t) {
    const int base = t * kTile;
    __syncthreads();  // the previous tile is consumed
    commit(base);
    __syncthreads();
    if (t + 1 < ntiles) prefetch(base + kTile);
    compute(base, 0);
    if (base + kKeys < ctx) compute(base, kKeys);
  }

  if (missing && p.status) atomicOr(p.status, 4);

  // normalise and write O[layer][r][qi][hq][d], d = 16mt + 4a + i
  float l_tot = l_run + __shfl_xor(l_run, 16, kWave);
  l_tot += __shfl_xor(l_tot, 32, kWave);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = p.out + (((int64_t(layer) * p.n_req + r) * p.q_len + qi) * p.num_q_heads + hq) * D;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      *reinterpret_cast<f32x4*>(orow + 16 * mt + 4 * a) = o[mt] * inv;
  }
}

template <int D>
hipError_t launch_attend(const AttnParams& p, const LayerCPtrs& kc, const LayerCPtrs& vc,
                         int64_t grid, int style, hipStream_t s) {
  if (style == PRKV_ROPE_INTERLEAVED)
    hipLaunchKernelGGL((attend_kernel<D, PRKV_ROPE_INTERLEAVED>), dim3(unsigned(grid)),
                       dim3(kThreads), 0, s, p, kc, vc);
  else
    hipLaunchKernelGGL((attend_kernel<D, PRKV_ROPE_HALF_SPLIT>), dim3(unsigned(grid)),
                       dim3(kThreads), 0, s, p, kc, vc);
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
  if (b->bt_stride > kBtLds)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "bt_stride %d exceeds %d block-table entries",
                      b->bt_stride, kBtLds);
  if (b->num_q_heads % d.num_kv_heads != 0)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "num_q_heads %d not a multiple of %d KV heads",
                      b->num_q_heads, d.num_kv_heads);
  const int group = b->num_q_heads / d.num_kv_heads;
  if (int64_t(b->q_len) * group > kMaxRows)
    return prkv::fail(PRKV_ERR_INVALID_ARG, "q_len * heads per KV head = %lld exceeds %d",
                      (long long)b->q_len * group, kMaxRows);
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
       reinterpret_cast<uintptr_t>(b->bt_len) | reinterpret_cast<uintptr_t>(d_status)) & 3u)
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
  const int64_t grid = int64_t(d.num_layers) * b->n_req * d.num_kv_heads;
  if (grid > INT32_MAX) return prkv::fail(PRKV_ERR_INVALID_ARG, "grid too large");
  AttnParams p;
  p.q = b->q;
  p.q_start = b->q_start;
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
  p.rows = b->q_len * group;
  p.bt_stride = b->bt_stride;
  p.block_size = block_size;
  p.max_position = d.max_position;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t e = d.head_dim == 64 ? launch_attend<64>(p, kc, vc, grid, d.rope_style, s)
                                        : launch_attend<128>(p, kc, vc, grid, d.rope_style, s);
  if (e != hipSuccess) return prkv::fail(PRKV_ERR_HIP, "attend launch: %s", hipGetErrorString(e));
  return PRKV_OK;
}

}  // extern "C"
