// Drives the host side of the library (the block-list builders, the schedule
// builder, status strings) over seeded random patterns, valid and invalid, so
// that a build with AddressSanitizer and UndefinedBehaviorSanitizer checks
// every access they make.  Compiled and run by tests/test_host_sanitize.py with
// the host compiler; the device code is not part of it.
//
// Usage: host_sanitize <iterations> <seed>; prints "ok <cases>" and exits 0,
// or prints the failed invariant and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "bsvf.h"

namespace {

int failures = 0;

void expect(bool cond, const char* what, long it) {
  if (!cond) {
    std::printf("FAILED: %s (iteration %ld)\n", what, it);
    ++failures;
  }
}

// Two-call protocol of a builder: sizes first, then the arrays at exactly
// that capacity; also one call with the capacity one short.
struct Lists {
  std::vector<int32_t> q_tiles, kv_ptr, kv_iv, kv_flag;
  int32_t n_qt = 0, nnz = 0;
  int64_t useful = 0;
};

int build(const attn_pattern_t& p, int32_t granule, int32_t bq, Lists& out, long it) {
  int32_t n_qt = 0, nnz = 0;
  int64_t useful = 0;
  int st = granule ? attn_build_blocks_granular(&p, granule, bq, nullptr, nullptr, nullptr, nullptr, &useful, &n_qt, &nnz)
                   : attn_build_blocks(&p, bq, nullptr, nullptr, nullptr, &useful, &n_qt, &nnz);
  if (st != ATTN_OK) return st;
  expect(n_qt > 0 && nnz > 0, "sizes positive", it);
  out.q_tiles.assign(2 * (size_t)n_qt, -7);
  out.kv_ptr.assign((size_t)n_qt + 1, -7);
  out.kv_iv.assign(2 * (size_t)nnz, -7);
  out.kv_flag.assign((size_t)nnz, -7);
  if (nnz > 1) {  // one short of the needed capacity: ATTN_E_SIZE, nothing past the arrays
    int32_t cq = n_qt, cn = nnz - 1;
    const int s2 = granule ? attn_build_blocks_granular(&p, granule, bq, out.q_tiles.data(), out.kv_ptr.data(),
                                                        out.kv_iv.data(), out.kv_flag.data(), &useful, &cq, &cn)
                           : attn_build_blocks(&p, bq, out.q_tiles.data(), out.kv_ptr.data(), out.kv_iv.data(),
                                               &useful, &cq, &cn);
    expect(s2 == ATTN_E_SIZE, "short capacity reported", it);
  }
  out.n_qt = n_qt;
  out.nnz = nnz;
  st = granule ? attn_build_blocks_granular(&p, granule, bq, out.q_tiles.data(), out.kv_ptr.data(), out.kv_iv.data(),
                                            out.kv_flag.data(), &out.useful, &out.n_qt, &out.nnz)
               : attn_build_blocks(&p, bq, out.q_tiles.data(), out.kv_ptr.data(), out.kv_iv.data(), &out.useful,
                                   &out.n_qt, &out.nnz);
  expect(st == ATTN_OK && out.n_qt == n_qt && out.nnz == nnz && out.useful == useful, "second call agrees", it);
  return st;
}

void check_lists(const attn_pattern_t& p, const Lists& L, long it) {
  const int64_t N = (int64_t)p.num_frames * p.tokens_per_frame;
  int64_t rows = 0;
  expect(L.kv_ptr[0] == 0 && L.kv_ptr[L.n_qt] == L.nnz, "kv_ptr ends", it);
  for (int32_t t = 0; t < L.n_qt; ++t) {
    const int32_t qs = L.q_tiles[2 * t], nr = L.q_tiles[2 * t + 1];
    expect(qs == rows && nr > 0 && nr % 16 == 0, "tiles cover the rows in order", it);
    rows += nr;
    expect(L.kv_ptr[t] <= L.kv_ptr[t + 1], "kv_ptr ascending", it);
    int64_t last = -1;
    for (int32_t e = L.kv_ptr[t]; e < L.kv_ptr[t + 1]; ++e) {
      const int32_t ks = L.kv_iv[2 * e], kl = L.kv_iv[2 * e + 1];
      expect(ks % 16 == 0 && kl > 0 && kl % 16 == 0 && ks + (int64_t)kl <= N && ks > last, "intervals valid", it);
      last = ks;
    }
  }
  expect(rows == N, "every row in a tile", it);
}

void check_schedule(const Lists& L, int32_t batch, int32_t heads, int32_t group, int32_t nx, long it) {
  int32_t n_work = 0;
  int st = attn_build_schedule(L.q_tiles.data(), L.kv_ptr.data(), L.kv_iv.data(), L.n_qt, batch, heads, group, nx,
                               nullptr, &n_work);
  expect(st == ATTN_OK && n_work > 0, "schedule size", it);
  if (st != ATTN_OK) return;
  std::vector<int32_t> order((size_t)n_work + 1, -9);
  if (n_work > 1) {
    int32_t cap = n_work - 1;
    expect(attn_build_schedule(L.q_tiles.data(), L.kv_ptr.data(), L.kv_iv.data(), L.n_qt, batch, heads, group, nx,
                               order.data(), &cap) == ATTN_E_SIZE && cap == n_work,
           "schedule short capacity", it);
  }
  int32_t cap = n_work;
  st = attn_build_schedule(L.q_tiles.data(), L.kv_ptr.data(), L.kv_iv.data(), L.n_qt, batch, heads, group, nx,
                           order.data(), &cap);
  expect(st == ATTN_OK && cap == n_work && order[(size_t)n_work] == -9, "schedule written in bounds", it);
  const int64_t items = (int64_t)L.n_qt * batch * heads;
  std::vector<char> seen((size_t)items, 0);
  int64_t real = 0;
  for (int32_t i = 0; i < n_work; ++i) {
    const int32_t w = order[i];
    if (w < 0) {
      expect(w == -1, "padding is -1", it);
      continue;
    }
    expect(w < items && !seen[(size_t)w], "a permutation", it);
    if (w < items) seen[(size_t)w] = 1;
    ++real;
  }
  expect(real == items, "every item scheduled", it);
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 500;
  const unsigned seed = argc > 2 ? (unsigned)std::atol(argv[2]) : 1u;
  std::mt19937 rng(seed);
  auto pick = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  long cases = 0;
  for (long it = 0; it < iters; ++it) {
    std::vector<int32_t> globals;
    const int F = pick(1, 12);
    for (int g = pick(0, 3); g > 0; --g) globals.push_back(pick(0, F - 1));
    attn_pattern_t p{F, 16 * pick(1, 40), pick(0, 3), pick(0, 3), (int32_t)globals.size(),
                     globals.empty() ? nullptr : globals.data()};
    const int32_t bq = 16 * pick(1, 16);
    // occasionally invalid: the builders must refuse without touching memory
    const int bad = pick(0, 9);
    if (bad == 0) p.tokens_per_frame += 8;
    if (bad == 1) p.win_before = -1;
    if (bad == 2 && p.num_global > 0) globals[0] = F;
    Lists L;
    const int st = build(p, 0, bad == 3 ? bq + 8 : bq, L, it);
    if (bad <= 3 && !(bad == 2 && p.num_global == 0)) {
      expect(st != ATTN_OK, "invalid input refused", it);
      expect(attn_status_str(st) != nullptr && attn_last_error() != nullptr, "error strings", it);
      continue;
    }
    if (st != ATTN_OK) {
      // a pattern in which some frame attends nothing is refused as such
      expect(st == ATTN_E_PATTERN, "only pattern errors on valid sizes", it);
      continue;
    }
    check_lists(p, L, it);
    const int32_t batch = pick(1, 2), heads = pick(1, 6), nx = pick(1, 16);
    check_schedule(L, batch, heads, 0, nx, it);
    check_schedule(L, batch, heads, pick(1, 40), nx, it);
    if (p.tokens_per_frame >= 64) {
      Lists G;
      const int32_t granule = 64 * pick(1, 3);
      if (build(p, granule, bq, G, it) == ATTN_OK) {
        check_lists(p, G, it);
        for (int32_t e = 0; e < G.nnz; ++e) expect(G.kv_flag[e] == 0 || G.kv_flag[e] == 1, "flags 0 or 1", it);
        check_schedule(G, batch, heads, 0, nx, it);
      }
    }
    ++cases;
  }
  // NULL and out-of-range arguments
  int32_t a = 0, b = 0;
  int64_t u = 0;
  expect(attn_build_blocks(nullptr, 16, nullptr, nullptr, nullptr, &u, &a, &b) == ATTN_E_INVAL, "NULL pattern", -1);
  expect(attn_build_schedule(nullptr, nullptr, nullptr, 1, 1, 1, 0, 8, nullptr, &a) == ATTN_E_INVAL, "NULL lists", -1);
  expect(attn_status_str(12345) != nullptr, "unknown status string", -1);
  if (failures) return 1;
  std::printf("ok %ld\n", cases);
  return 0;
}
