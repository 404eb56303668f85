// Internal declarations shared by the host (C++) and device (HIP) halves of
// libprkv.so.  Not part of the public ABI; see include/prkv.h.
#pragma once

#include <cstdint>
#include <vector>

#include "prkv.h"

struct prkv_store {
  prkv_store_desc desc;
  void* k_arena = nullptr;  // device, [L][capacity_rows][H][D] bf16
  void* v_arena = nullptr;
  void* rope = nullptr;     // device, [max_position][D/2] x (cos_hi, cos_lo, sin_hi, sin_lo)
  int64_t rows_used = 0;
  int64_t facts_put = 0;
  std::vector<int64_t> first_row;  // per fact id; -1 when absent
  std::vector<int32_t> length;     // per fact id
  bool device_backed() const { return k_arena != nullptr; }
};

namespace prkv {

// Records the message for last_error_string() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

int validate_desc(const prkv_store_desc* d);
inline int64_t row_elems(const prkv_store_desc& d) {
  return int64_t(d.num_kv_heads) * d.head_dim;
}
size_t arena_bytes(const prkv_store_desc& d);
size_t rope_bytes(const prkv_store_desc& d);

// Host-side halves used by the HIP file.
int store_new(const prkv_store_desc* d, prkv_store** out);
int check_put(const prkv_store* st, int32_t fact_id, int32_t len);
void commit_put(prkv_store* st, int32_t fact_id, int32_t len);

constexpr int kMaxLayers = 128;

// Compute units of the current device (cached per device; 256 if unknown).
// Defined with the device code.
int compute_units();

}  // namespace prkv
