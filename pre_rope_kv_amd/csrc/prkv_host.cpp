// Host half of libprkv.so: descriptor validation, the fact table, the
// slot-mapping builder and the RoPE table builder.  Plain C++17; no HIP calls.
//
// Operation sources (page "InferScale: GPU-Native KV Injection for
// Personalized LLM Serving", Pith review of arXiv 2607.27090):
//  - fact table keyed by fact_id: Figure 2 caption (each fact encoded once
//    under a shared fact_id) and the ledger's read-mostly-store axiom
//    (Proposition 5): append-only, no delete.
//  - slot mapping: "If this is right" bullet 2 and "invented entities:
//    Chunked RoPE" (dynamic top-k placement at arbitrary positions) and the
//    KV-connector axiom, section 3.4 (prefix external, blocks allocated
//    without prefill, then scatter-copy).
//  - RoPE table: ledger axiom R_a^T R_b = R_{b-a} (Theorem 6, section 5.1);
//    frequencies of RoFormer (reference [20]) with half-split pairing.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <new>
#include <string>

#include "prkv_internal.h"

namespace prkv {

static thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

void clear_error() { g_error.clear(); }

static bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int validate_desc(const prkv_store_desc* d) {
  if (!d) return fail(PRKV_ERR_INVALID_ARG, "descriptor is NULL");
  if (d->num_layers < 1 || d->num_layers > kMaxLayers)
    return fail(PRKV_ERR_INVALID_ARG, "num_layers %d not in [1, %d]", d->num_layers, kMaxLayers);
  if (d->num_kv_heads < 1)
    return fail(PRKV_ERR_INVALID_ARG, "num_kv_heads %d < 1", d->num_kv_heads);
  if (!pow2(d->head_dim) || d->head_dim < 16 || d->head_dim > 1024)
    return fail(PRKV_ERR_INVALID_ARG, "head_dim %d must be a power of two in [16, 1024]",
                d->head_dim);
  if (d->max_facts < 1) return fail(PRKV_ERR_INVALID_ARG, "max_facts %d < 1", d->max_facts);
  if (d->capacity_rows < 1 || d->capacity_rows > std::numeric_limits<int32_t>::max())
    return fail(PRKV_ERR_INVALID_ARG, "capacity_rows %lld not in [1, 2^31-1]",
                (long long)d->capacity_rows);
  if (d->max_position < 1) return fail(PRKV_ERR_INVALID_ARG, "max_position %d < 1", d->max_position);
  if (d->rope_style != PRKV_ROPE_HALF_SPLIT && d->rope_style != PRKV_ROPE_INTERLEAVED)
    return fail(PRKV_ERR_INVALID_ARG, "rope_style %d unsupported", d->rope_style);
  if (!(d->rope_theta > 1.0) || !std::isfinite(d->rope_theta))
    return fail(PRKV_ERR_INVALID_ARG, "rope_theta must be finite and > 1");
  if (d->key_layout != PRKV_KEYS_PRE_ROPE && d->key_layout != PRKV_KEYS_CHUNK_LOCAL)
    return fail(PRKV_ERR_INVALID_ARG, "key_layout %d unsupported", d->key_layout);
  if (d->rope_scaling == PRKV_SCALING_LLAMA3) {
    const double f = d->scaling_factor, lo = d->low_freq_factor, hi = d->high_freq_factor;
    if (!(f >= 1.0) || !std::isfinite(f))
      return fail(PRKV_ERR_INVALID_ARG, "scaling_factor must be finite and >= 1");
    if (!(lo > 0.0) || !(hi > lo) || !std::isfinite(hi))
      return fail(PRKV_ERR_INVALID_ARG, "need 0 < low_freq_factor < high_freq_factor < inf");
    if (d->original_max_position < 1)
      return fail(PRKV_ERR_INVALID_ARG, "original_max_position %d < 1",
                  d->original_max_position);
  } else if (d->rope_scaling != PRKV_SCALING_NONE) {
    return fail(PRKV_ERR_INVALID_ARG, "rope_scaling %d unsupported", d->rope_scaling);
  }
  if (d->cache_layout != PRKV_CACHE_NHD && d->cache_layout != PRKV_CACHE_HND)
    return fail(PRKV_ERR_INVALID_ARG, "cache_layout %d unsupported", d->cache_layout);
  const double heads_dim = double(d->num_kv_heads) * d->head_dim;
  if (heads_dim * d->capacity_rows * d->num_layers * 2.0 > 9.0e18)
    return fail(PRKV_ERR_INVALID_ARG, "arena size overflows");
  return PRKV_OK;
}

size_t arena_bytes(const prkv_store_desc& d) {
  return size_t(d.num_layers) * size_t(d.capacity_rows) * size_t(row_elems(d)) * 2u;
}

size_t rope_bytes(const prkv_store_desc& d) {
  return size_t(d.max_position) * size_t(d.head_dim / 2) * 16u;
}

int store_new(const prkv_store_desc* d, prkv_store** out) {
  prkv_store* st = new (std::nothrow) prkv_store();
  if (!st) return fail(PRKV_ERR_NO_MEMORY, "out of host memory");
  st->desc = *d;
  try {
    st->first_row.assign(size_t(d->max_facts), -1);
    st->length.assign(size_t(d->max_facts), 0);
  } catch (const std::bad_alloc&) {
    delete st;
    return fail(PRKV_ERR_NO_MEMORY, "fact table of %d entries", d->max_facts);
  }
  *out = st;
  return PRKV_OK;
}

int check_put(const prkv_store* st, int32_t fact_id, int32_t len) {
  if (!st) return fail(PRKV_ERR_INVALID_ARG, "store is NULL");
  if (fact_id < 0 || fact_id >= st->desc.max_facts)
    return fail(PRKV_ERR_CAPACITY, "fact id %d outside [0, %d)", fact_id, st->desc.max_facts);
  if (len < 1) return fail(PRKV_ERR_INVALID_ARG, "fact %d: length %d < 1", fact_id, len);
  if (st->first_row[fact_id] >= 0)
    return fail(PRKV_ERR_DUPLICATE_FACT, "fact %d already stored", fact_id);
  if (st->rows_used + len > st->desc.capacity_rows)
    return fail(PRKV_ERR_CAPACITY, "fact %d: %d rows exceed capacity (%lld of %lld used)",
                fact_id, len, (long long)st->rows_used, (long long)st->desc.capacity_rows);
  return PRKV_OK;
}

void commit_put(prkv_store* st, int32_t fact_id, int32_t len) {
  st->first_row[fact_id] = st->rows_used;
  st->length[fact_id] = len;
  st->rows_used += len;
  st->facts_put += 1;
}

}  // namespace prkv

using namespace prkv;

extern "C" {

const char* last_error_string(void) { return g_error.c_str(); }

int store_required_bytes(const prkv_store_desc* desc, size_t* arena_bytes_each,
                         size_t* rope_table_bytes) {
  clear_error();
  if (int rc = validate_desc(desc)) return rc;
  if (!arena_bytes_each || !rope_table_bytes)
    return fail(PRKV_ERR_INVALID_ARG, "output pointer is NULL");
  *arena_bytes_each = arena_bytes(*desc);
  *rope_table_bytes = rope_bytes(*desc);
  return PRKV_OK;
}

int store_fact_info(const prkv_store* st, int32_t fact_id, int64_t* first_row, int32_t* len) {
  clear_error();
  if (!st || !first_row || !len) return fail(PRKV_ERR_INVALID_ARG, "NULL argument");
  if (fact_id < 0 || fact_id >= st->desc.max_facts || st->first_row[fact_id] < 0)
    return fail(PRKV_ERR_UNKNOWN_FACT, "fact %d not stored", fact_id);
  *first_row = st->first_row[fact_id];
  *len = st->length[fact_id];
  return PRKV_OK;
}

void store_destroy(prkv_store* st) { delete st; }

int rope_table_fill(const prkv_store_desc* desc, float* out, size_t out_bytes) {
  clear_error();
  if (int rc = validate_desc(desc)) return rc;
  if (!out) return fail(PRKV_ERR_INVALID_ARG, "output is NULL");
  const size_t need = rope_bytes(*desc);
  if (out_bytes < need)
    return fail(PRKV_ERR_BUFFER_TOO_SMALL, "rope table needs %zu bytes, got %zu", need, out_bytes);
  const int half = desc->head_dim / 2;
  // f_j in extended precision (with the frequency rule), then one rounding
  // to double
  std::vector<double> inv(half);
  for (int j = 0; j < half; ++j) {
    long double f = std::pow((long double)desc->rope_theta,
                             -(2.0L * j) / (long double)desc->head_dim);
    if (desc->rope_scaling == PRKV_SCALING_LLAMA3) {
      const long double pi = 3.14159265358979323846264338327950288L;
      const long double W = desc->original_max_position;
      const long double lo = desc->low_freq_factor, hi = desc->high_freq_factor;
      const long double factor = desc->scaling_factor;
      const long double wavelen = 2.0L * pi / f;
      if (wavelen > W / lo) {
        f = f / factor;
      } else if (wavelen >= W / hi) {
        const long double m = (W / wavelen - lo) / (hi - lo);
        f = (1.0L - m) * f / factor + m * f;
      }
    }
    inv[j] = double(f);
  }
  for (int64_t p = 0; p < desc->max_position; ++p) {
    float* row = out + p * int64_t(half) * 4;
    for (int j = 0; j < half; ++j) {
      const double a = double(p) * inv[j];
      const double c = std::cos(a), s = std::sin(a);
      const float ch = float(c), sh = float(s);
      row[4 * j + 0] = ch;
      row[4 * j + 1] = float(c - double(ch));
      row[4 * j + 2] = sh;
      row[4 * j + 3] = float(s - double(sh));
    }
  }
  return PRKV_OK;
}

int build_slot_mapping(const prkv_store* st, int32_t n_req, const int32_t* req_fact_ptr,
                       const int32_t* fact_ids, const int32_t* start_pos,
                       const int32_t* block_tables, int32_t bt_stride, const int32_t* bt_len,
                       int32_t block_size, int64_t num_blocks, int32_t* src_row, int32_t* pos,
                       int32_t* slot, int64_t capacity, int64_t* n_tokens) {
  clear_error();
  if (!st) return fail(PRKV_ERR_INVALID_ARG, "store is NULL");
  if (!n_tokens) return fail(PRKV_ERR_INVALID_ARG, "n_tokens is NULL");
  if (n_req < 0) return fail(PRKV_ERR_INVALID_ARG, "n_req %d < 0", n_req);
  if (block_size < 1) return fail(PRKV_ERR_INVALID_ARG, "block_size %d < 1", block_size);
  if (num_blocks < 1) return fail(PRKV_ERR_INVALID_ARG, "num_blocks %lld < 1", (long long)num_blocks);
  const int64_t num_slots = num_blocks * int64_t(block_size);
  if (num_blocks > std::numeric_limits<int32_t>::max() ||
      num_slots > std::numeric_limits<int32_t>::max())
    return fail(PRKV_ERR_INVALID_ARG, "num_blocks * block_size exceeds 2^31-1");
  if (n_req == 0) {
    *n_tokens = 0;
    return PRKV_OK;
  }
  if (!req_fact_ptr || !start_pos || !bt_len)
    return fail(PRKV_ERR_INVALID_ARG, "request arrays must not be NULL");
  if (req_fact_ptr[0] != 0) return fail(PRKV_ERR_INVALID_ARG, "req_fact_ptr[0] must be 0");
  if (bt_stride < 0) return fail(PRKV_ERR_INVALID_ARG, "bt_stride %d < 0", bt_stride);
  for (int32_t r = 0; r < n_req; ++r) {
    if (req_fact_ptr[r + 1] < req_fact_ptr[r])
      return fail(PRKV_ERR_INVALID_ARG, "req_fact_ptr decreases at request %d", r);
    if (bt_len[r] < 0 || bt_len[r] > bt_stride)
      return fail(PRKV_ERR_INVALID_ARG, "request %d: bt_len %d not in [0, bt_stride=%d]", r,
                  bt_len[r], bt_stride);
    if (start_pos[r] < 0) return fail(PRKV_ERR_INVALID_ARG, "request %d: start_pos < 0", r);
  }
  if (req_fact_ptr[n_req] > 0 && !fact_ids) return fail(PRKV_ERR_INVALID_ARG, "fact_ids is NULL");
  if (!block_tables && bt_stride > 0) return fail(PRKV_ERR_INVALID_ARG, "block_tables is NULL");

  // Pass 1: resolve, place and validate, run by run (a run = consecutive
  // tokens of one fact inside one block: one division, one table lookup and
  // one or two bitmap words per run).  Duplicate slots are found with a
  // bitmap over all slots; a run's bits are set only once its whole range
  // is free, and every run set is cleared again before returning.  Nothing
  // is written to the outputs unless the whole batch is valid.
  struct Run {
    int64_t s0;
    int32_t len;
  };
  static thread_local std::vector<uint64_t> seen;
  static thread_local std::vector<Run> runs;
  runs.clear();
  const size_t words = size_t((num_slots + 63) / 64);
  if (seen.size() < words) seen.resize(words, 0);
  const prkv_store_desc& d = st->desc;
  const bool chunk_local = d.key_layout == PRKV_KEYS_CHUNK_LOCAL;
  // first slot in [s0, s0 + n) already taken, or -1
  auto first_taken = [&](int64_t s0, int64_t n) -> int64_t {
    for (int64_t s = s0; s < s0 + n;) {
      const int64_t b0 = s & 63, take = std::min<int64_t>(64 - b0, s0 + n - s);
      const uint64_t mask = (take == 64 ? ~uint64_t(0) : ((uint64_t(1) << take) - 1)) << b0;
      const uint64_t hit = seen[size_t(s >> 6)] & mask;
      if (hit) return (s & ~int64_t(63)) + __builtin_ctzll(hit);
      s += take;
    }
    return -1;
  };
  auto mark = [&](int64_t s0, int64_t n, bool set) {
    for (int64_t s = s0; s < s0 + n;) {
      const int64_t b0 = s & 63, take = std::min<int64_t>(64 - b0, s0 + n - s);
      const uint64_t mask = (take == 64 ? ~uint64_t(0) : ((uint64_t(1) << take) - 1)) << b0;
      if (set) seen[size_t(s >> 6)] |= mask;
      else seen[size_t(s >> 6)] &= ~mask;
      s += take;
    }
  };
  int rc = PRKV_OK;
  int64_t total = 0;
  for (int32_t r = 0; r < n_req && rc == PRKV_OK; ++r) {
    const int32_t* bt = block_tables + int64_t(r) * bt_stride;
    int64_t p = start_pos[r];
    for (int32_t i = req_fact_ptr[r]; i < req_fact_ptr[r + 1] && rc == PRKV_OK; ++i) {
      const int32_t f = fact_ids[i];
      if (f < 0 || f >= d.max_facts || st->first_row[f] < 0) {
        rc = fail(PRKV_ERR_UNKNOWN_FACT, "request %d, fact %d: id %d not stored", r,
                  i - req_fact_ptr[r], f);
        break;
      }
      const int32_t len = st->length[f];
      if (p + len > d.max_position) {
        rc = fail(PRKV_ERR_OUT_OF_RANGE, "request %d: position %lld >= max_position %d", r,
                  (long long)(p + len - 1), d.max_position);
        break;
      }
      for (int32_t t = 0; t < len;) {
        const int64_t bi = p / block_size;
        const int64_t off = p - bi * block_size;
        if (bi >= bt_len[r]) {
          rc = fail(PRKV_ERR_OUT_OF_RANGE,
                    "request %d: position %lld needs block index %lld, table has %d", r,
                    (long long)p, (long long)bi, bt_len[r]);
          break;
        }
        const int64_t b = bt[bi];
        if (b < 0 || b >= num_blocks) {
          rc = fail(PRKV_ERR_OUT_OF_RANGE, "request %d: block id %lld outside [0, %lld)", r,
                    (long long)b, (long long)num_blocks);
          break;
        }
        const int32_t run = int32_t(std::min<int64_t>(block_size - off, len - t));
        const int64_t s0 = b * block_size + off;
        const int64_t dup = first_taken(s0, run);
        if (dup >= 0) {
          rc = fail(PRKV_ERR_DUPLICATE_SLOT, "request %d: slot %lld written twice", r,
                    (long long)dup);
          break;
        }
        mark(s0, run, true);
        runs.push_back(Run{s0, run});
        total += run;
        t += run;
        p += run;
      }
    }
  }
  for (const Run& u : runs) mark(u.s0, u.len, false);
  if (rc != PRKV_OK) return rc;
  *n_tokens = total;
  if (total > capacity)
    return fail(PRKV_ERR_BUFFER_TOO_SMALL, "%lld tokens, capacity %lld", (long long)total,
                (long long)capacity);
  if (total == 0) return PRKV_OK;  // nothing to write; the outputs may be NULL
  if (!src_row || !pos || !slot)
    return fail(PRKV_ERR_INVALID_ARG, "output arrays must not be NULL");

  // Pass 2: the batch is valid; write (arena row, rotation position, slot)
  // per token in request, fact-list and token order, run by run.
  int64_t k = 0;
  size_t u = 0;
  for (int32_t r = 0; r < n_req; ++r) {
    int64_t p = start_pos[r];
    for (int32_t i = req_fact_ptr[r]; i < req_fact_ptr[r + 1]; ++i) {
      const int32_t f = fact_ids[i];
      const int64_t row0 = st->first_row[f];
      const int32_t len = st->length[f];
      const int64_t fact_start = p;
      for (int32_t t = 0; t < len; ++u) {
        const Run& run = runs[u];
        for (int32_t j = 0; j < run.len; ++j, ++k) {
          src_row[k] = int32_t(row0 + t + j);
          pos[k] = int32_t(chunk_local ? fact_start : p + j);
          slot[k] = int32_t(run.s0 + j);
        }
        t += run.len;
        p += run.len;
      }
    }
  }
  return PRKV_OK;
}

}  // extern "C"
