// Exercises the host half of libprkv.so (descriptor validation, the fact
// table, build_slot_mapping, rope_table_fill) on seeded random inputs,
// valid and invalid, so that an AddressSanitizer / UndefinedBehaviorSanitizer
// build can catch memory and UB errors in it.  Built and run by
// tests/test_host_sanitizers.py with g++ (no device code involved).
// Exit status 0 = every call returned a documented code and every
// successful mapping was self-consistent.

#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "prkv_internal.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int i) {
  if (!ok) {
    std::fprintf(stderr, "case %d: %s\n", i, what);
    ++failures;
  }
}

bool documented(int rc) { return rc <= 0 && rc >= PRKV_ERR_NO_MEMORY; }

prkv_store_desc random_desc(std::mt19937& rng, bool valid) {
  std::uniform_int_distribution<int> u(0, 99);
  prkv_store_desc d{};
  const int dims[] = {16, 32, 64, 128};
  d.num_layers = 1 + u(rng) % 4;
  d.num_kv_heads = 1 + u(rng) % 3;
  d.head_dim = dims[u(rng) % 4];
  d.max_facts = 1 + u(rng) % 40;
  d.capacity_rows = 1 + u(rng) % 400;
  d.max_position = 1 + u(rng) % 300;
  d.rope_style = u(rng) % 2;
  d.rope_theta = 10000.0;
  d.key_layout = u(rng) % 2;
  d.cache_layout = u(rng) % 2;
  if (u(rng) % 2) {
    d.rope_scaling = PRKV_SCALING_LLAMA3;
    d.scaling_factor = 8.0;
    d.low_freq_factor = 1.0;
    d.high_freq_factor = 4.0;
    d.original_max_position = 64;
  }
  if (!valid) {
    switch (u(rng) % 8) {
      case 0: d.num_layers = 0; break;
      case 1: d.head_dim = 48; break;
      case 2: d.max_facts = -3; break;
      case 3: d.capacity_rows = 0; break;
      case 4: d.rope_style = 7; break;
      case 5: d.rope_theta = 0.5; break;
      case 6: d.rope_scaling = 1; d.high_freq_factor = 0.5; break;
      default: d.cache_layout = 2; break;
    }
  }
  return d;
}

}  // namespace

int main() {
  std::mt19937 rng(1234);
  std::uniform_int_distribution<int> u(0, 1 << 20);

  for (int i = 0; i < 300; ++i) {
    const bool valid = u(rng) % 4 != 0;
    prkv_store_desc d = random_desc(rng, valid);
    const int rc = prkv::validate_desc(&d);
    expect(valid ? rc == PRKV_OK : rc == PRKV_ERR_INVALID_ARG, "validate_desc", i);
    if (rc != PRKV_OK) continue;

    // RoPE table: exact size, then one float short
    size_t arena = 0, table = 0;
    expect(store_required_bytes(&d, &arena, &table) == PRKV_OK, "required bytes", i);
    std::vector<float> tab(table / sizeof(float));
    expect(rope_table_fill(&d, tab.data(), table) == PRKV_OK, "rope_table_fill", i);
    expect(tab[0] == 1.0f && tab[1] == 0.0f && tab[2] == 0.0f && tab[3] == 0.0f,
           "position 0 is the identity", i);
    expect(rope_table_fill(&d, tab.data(), table - 4) == PRKV_ERR_BUFFER_TOO_SMALL,
           "short rope buffer", i);

    // a metadata-only store with random puts (some rejected)
    prkv_store* st = nullptr;
    expect(prkv::store_new(&d, &st) == PRKV_OK, "store_new", i);
    std::vector<int> lens(d.max_facts, 0);
    for (int f = 0; f < d.max_facts + 3; ++f) {
      const int fid = u(rng) % (d.max_facts + 2) - 1;
      const int len = u(rng) % 20 - 2;
      const int prc = prkv::check_put(st, fid, len);
      expect(documented(prc), "check_put code", i);
      if (prc == PRKV_OK) {
        prkv::commit_put(st, fid, len);
        lens[fid] = len;
      }
    }
    int64_t row = 0;
    int32_t len = 0;
    for (int f = 0; f < d.max_facts; ++f) {
      const int irc = store_fact_info(st, f, &row, &len);
      expect(lens[f] > 0 ? (irc == PRKV_OK && len == lens[f]) : irc == PRKV_ERR_UNKNOWN_FACT,
             "store_fact_info", i);
    }

    // random batches through build_slot_mapping
    for (int b = 0; b < 8; ++b) {
      const int n_req = u(rng) % 4;
      const int sizes[] = {1, 2, 5, 16, 63, 64, 65, 100, 130};
      const int bs = sizes[u(rng) % 9];   // runs up to 130 slots span several bitmap words
      const int64_t num_blocks = 1 + u(rng) % 64;
      const int stride = u(rng) % 24;
      std::vector<int32_t> ptr(n_req + 1, 0), start(n_req), bt_len(n_req);
      std::vector<int32_t> ids, bt(size_t(n_req) * stride + 1);
      for (int r = 0; r < n_req; ++r) {
        const int k = u(rng) % 5;
        for (int j = 0; j < k; ++j) ids.push_back(u(rng) % (d.max_facts + 2) - 1);
        ptr[r + 1] = int32_t(ids.size());
        start[r] = u(rng) % 40 - (u(rng) % 10 == 0 ? 5 : 0);
        bt_len[r] = stride ? u(rng) % (stride + 1) : 0;
        for (int e = 0; e < stride; ++e)
          bt[size_t(r) * stride + e] = u(rng) % (int(num_blocks) + 4) - 2;
      }
      ids.push_back(0);  // keep the pointer valid when the batch is empty
      int64_t n = -1;
      int mrc = build_slot_mapping(st, n_req, ptr.data(), ids.data(), start.data(), bt.data(),
                                   stride, bt_len.data(), bs, num_blocks, nullptr, nullptr,
                                   nullptr, 0, &n);
      expect(documented(mrc), "mapping code (count)", i);
      if (mrc == PRKV_OK || mrc == PRKV_ERR_BUFFER_TOO_SMALL) {
        const int64_t cap = n + int64_t(u(rng) % 3) - 1;  // one short, exact or one over
        std::vector<int32_t> src(cap > 0 ? cap : 1), pos(src.size()), slot(src.size());
        mrc = build_slot_mapping(st, n_req, ptr.data(), ids.data(), start.data(), bt.data(),
                                 stride, bt_len.data(), bs, num_blocks, src.data(), pos.data(),
                                 slot.data(), cap < 0 ? 0 : cap, &n);
        expect(documented(mrc), "mapping code", i);
        if (mrc == PRKV_OK) {
          int64_t want = 0;
          for (int r = 0; r < n_req; ++r)
            for (int j = ptr[r]; j < ptr[r + 1]; ++j) want += lens[ids[j]];
          expect(n == want, "token count", i);
          for (int64_t t = 0; t < n; ++t) {
            expect(slot[t] >= 0 && slot[t] < num_blocks * bs, "slot range", i);
            expect(pos[t] >= 0 && pos[t] < d.max_position, "position range", i);
            expect(src[t] >= 0 && src[t] < d.capacity_rows, "row range", i);
          }
        }
      }
    }
    store_destroy(st);
  }
  std::printf("host sanitizer driver: %d failures\n", failures);
  return failures == 0 ? 0 : 1;
}
