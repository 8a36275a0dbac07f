// Host side of the bsvf C ABI: status strings, per-thread error messages, the
// integer block-list builder and the launch-order (schedule) builder.
//
// Block lists follow the frame-aligned 16-token blocking of vatt-ghern.pages.dev
// "deep-heygen-avatar-iv-trillium-tpu", section 把 block 縮到 16 (also bytechap
// "How it works", cloudcurated Wall 2): every tile and every key interval starts
// and ends on a multiple of 16 tokens that is also a frame edge, so the kernel
// needs no mask predicate, no extra scan and no padding.
#include <algorithm>
#include <cstring>
#include <numeric>
#include <string>
#include <vector>

#include "bsvf_internal.h"

namespace bsvf {

static thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = std::string(attn_status_str(status)) + ": " + msg;
  return status;
}

int ok() {
  g_last_error.clear();
  return ATTN_OK;
}

int check_tensor(const char* name, const void* p, const int64_t* s,
                 int32_t B, int32_t H, int32_t N, int32_t D) {
  std::string n(name);
  if (!p) return fail(ATTN_E_INVAL, n + " is NULL");
  if (!s) return fail(ATTN_E_INVAL, n + " strides are NULL");
  if (!aligned16(p)) return fail(ATTN_E_ALIGN, n + " is not 16-byte aligned");
  for (int i = 0; i < 3; ++i) {
    if (s[i] <= 0) return fail(ATTN_E_ALIGN, n + " strides must be positive");
    if (s[i] % 8) return fail(ATTN_E_ALIGN, n + " strides must be multiples of 8 elements (16 bytes)");
  }
  if (s[2] < D) return fail(ATTN_E_ALIGN, n + " n-stride is smaller than head_dim");
  // element offset of the last row start inside one head, plus the row
  const long double span = (long double)s[2] * (N - 1) + D;
  if (span >= 2147483647.0L) return fail(ATTN_E_SIZE, n + " spans more than 2^31 elements within a head");
  const long double total = (long double)s[0] * (B - 1) + (long double)s[1] * (H - 1) + span;
  if (total >= 9.0e18L) return fail(ATTN_E_SIZE, n + " offsets overflow int64");
  return ATTN_OK;
}

}  // namespace bsvf

using bsvf::fail;

extern "C" {

int attn_abi_version(void) { return BSVF_ABI_VERSION; }

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_E_INVAL: return "ATTN_E_INVAL";
    case ATTN_E_ALIGN: return "ATTN_E_ALIGN";
    case ATTN_E_PATTERN: return "ATTN_E_PATTERN";
    case ATTN_E_SIZE: return "ATTN_E_SIZE";
    case ATTN_E_UNSUPPORTED: return "ATTN_E_UNSUPPORTED";
    case ATTN_E_HIP: return "ATTN_E_HIP";
    default: return "ATTN_E_UNKNOWN";
  }
}

const char* attn_last_error(void) { return bsvf::g_last_error.c_str(); }

int attn_build_blocks(const attn_pattern_t* p, int32_t block_q, int32_t* q_tiles,
                      int32_t* kv_ptr, int32_t* kv_iv, int64_t* useful_pairs,
                      int32_t* n_qt, int32_t* nnz) {
  if (!p || !n_qt || !nnz) return fail(ATTN_E_INVAL, "pattern, n_qt and nnz must not be NULL");
  const int64_t F = p->num_frames, T = p->tokens_per_frame;
  if (F < 1) return fail(ATTN_E_PATTERN, "num_frames must be >= 1");
  if (T <= 0 || T % 16) return fail(ATTN_E_ALIGN, "tokens_per_frame must be a positive multiple of 16");
  if (block_q <= 0 || block_q % 16) return fail(ATTN_E_ALIGN, "block_q must be a positive multiple of 16");
  if (p->win_before < 0 || p->win_after < 0) return fail(ATTN_E_PATTERN, "windows must be >= 0");
  if (p->num_global < 0) return fail(ATTN_E_PATTERN, "num_global must be >= 0");
  if (p->num_global > 0 && !p->global_frames) return fail(ATTN_E_INVAL, "global_frames is NULL");
  if (F * T > 2147483647LL) return fail(ATTN_E_SIZE, "num_frames * tokens_per_frame exceeds INT32_MAX");

  std::vector<char> is_global(F, 0);
  for (int32_t i = 0; i < p->num_global; ++i) {
    const int32_t g = p->global_frames[i];
    if (g < 0 || g >= F) return fail(ATTN_E_PATTERN, "global frame out of range");
    is_global[g] = 1;
  }

  // Runs of attended key frames per query frame: frames in ascending order,
  // adjacent frames merged into one run [first, last + 1).
  std::vector<std::vector<std::pair<int64_t, int64_t>>> runs(F);
  for (int64_t f = 0; f < F; ++f) {
    for (int64_t g = 0; g < F; ++g) {
      const bool in_window = (g - f >= -(int64_t)p->win_before) && (g - f <= (int64_t)p->win_after);
      if (!in_window && !is_global[g]) continue;
      auto& r = runs[f];
      if (!r.empty() && r.back().second == g) r.back().second = g + 1;
      else r.emplace_back(g, g + 1);
    }
    if (runs[f].empty()) return fail(ATTN_E_PATTERN, "a query frame attends no key frame");
  }

  const int64_t full = T / block_q, tail = T % block_q;
  const int64_t tiles_per_frame = full + (tail ? 1 : 0);
  int64_t need_qt = F * tiles_per_frame, need_nnz = 0, useful = 0;
  for (int64_t f = 0; f < F; ++f) {
    int64_t keys = 0;
    for (auto& r : runs[f]) keys += (r.second - r.first) * T;
    need_nnz += (int64_t)runs[f].size() * tiles_per_frame;
    useful += T * keys;  // all rows of the frame, every attended key
  }
  if (need_qt > 2147483647LL / 2 || need_nnz > 2147483647LL / 2)
    return fail(ATTN_E_SIZE, "block list too large");
  if (useful_pairs) *useful_pairs = useful;

  if (!q_tiles && !kv_ptr && !kv_iv) {
    *n_qt = (int32_t)need_qt;
    *nnz = (int32_t)need_nnz;
    return bsvf::ok();
  }
  if (!q_tiles || !kv_ptr || !kv_iv)
    return fail(ATTN_E_INVAL, "q_tiles, kv_ptr and kv_iv must be all NULL or all non-NULL");
  if (*n_qt < need_qt || *nnz < need_nnz) {
    *n_qt = (int32_t)need_qt;
    *nnz = (int32_t)need_nnz;
    return fail(ATTN_E_SIZE, "output capacity too small");
  }

  int64_t t = 0, e = 0;
  kv_ptr[0] = 0;
  for (int64_t f = 0; f < F; ++f) {
    for (int64_t i = 0; i < tiles_per_frame; ++i) {
      const int64_t start = f * T + i * block_q;
      const int64_t rows = (i < full) ? block_q : tail;
      q_tiles[2 * t] = (int32_t)start;
      q_tiles[2 * t + 1] = (int32_t)rows;
      for (auto& r : runs[f]) {
        kv_iv[2 * e] = (int32_t)(r.first * T);
        kv_iv[2 * e + 1] = (int32_t)((r.second - r.first) * T);
        ++e;
      }
      ++t;
      kv_ptr[t] = (int32_t)e;
    }
  }
  *n_qt = (int32_t)need_qt;
  *nnz = (int32_t)need_nnz;
  return bsvf::ok();
}

int attn_build_blocks_granular(const attn_pattern_t* p, int32_t granule, int32_t block_q,
                               int32_t* q_tiles, int32_t* kv_ptr, int32_t* kv_iv, int32_t* kv_flag,
                               int64_t* useful_pairs, int32_t* n_qt, int32_t* nnz) {
  if (!p || !n_qt || !nnz) return fail(ATTN_E_INVAL, "pattern, n_qt and nnz must not be NULL");
  const int64_t F = p->num_frames, T = p->tokens_per_frame;
  if (F < 1) return fail(ATTN_E_PATTERN, "num_frames must be >= 1");
  if (T <= 0 || T % 16) return fail(ATTN_E_ALIGN, "tokens_per_frame must be a positive multiple of 16");
  if (granule <= 0 || granule % 64) return fail(ATTN_E_ALIGN, "granule must be a positive multiple of 64");
  if (block_q <= 0 || block_q % 16) return fail(ATTN_E_ALIGN, "block_q must be a positive multiple of 16");
  if (p->win_before < 0 || p->win_after < 0) return fail(ATTN_E_PATTERN, "windows must be >= 0");
  if (p->num_global < 0) return fail(ATTN_E_PATTERN, "num_global must be >= 0");
  if (p->num_global > 0 && !p->global_frames) return fail(ATTN_E_INVAL, "global_frames is NULL");
  if (F * T > 2147483647LL) return fail(ATTN_E_SIZE, "num_frames * tokens_per_frame exceeds INT32_MAX");
  std::vector<char> is_global(F, 0);
  for (int32_t i = 0; i < p->num_global; ++i) {
    const int32_t g = p->global_frames[i];
    if (g < 0 || g >= F) return fail(ATTN_E_PATTERN, "global frame out of range");
    is_global[g] = 1;
  }
  auto attends = [&](int64_t f, int64_t g) {
    return (g - f >= -(int64_t)p->win_before && g - f <= (int64_t)p->win_after) || is_global[g];
  };
  const int64_t N = F * T;
  // Blocks of one tile: 0 none, 1 every (row, key) pair attended, 2 some.
  auto block_kind = [&](int64_t qs, int64_t qe, int64_t ks, int64_t ke) {
    bool any = false, all = true;
    for (int64_t f = qs / T; f <= (qe - 1) / T; ++f)
      for (int64_t g = ks / T; g <= (ke - 1) / T; ++g) {
        const bool a = attends(f, g);
        any |= a;
        all &= a;
      }
    return any ? (all ? 1 : 2) : 0;
  };
  int64_t useful = 0;
  for (int64_t f = 0; f < F; ++f)
    for (int64_t g = 0; g < F; ++g)
      if (attends(f, g)) useful += T * T;
  if (useful_pairs) *useful_pairs = useful;

  const bool fill = q_tiles || kv_ptr || kv_iv || kv_flag;
  if (fill && (!q_tiles || !kv_ptr || !kv_iv || !kv_flag))
    return fail(ATTN_E_INVAL, "q_tiles, kv_ptr, kv_iv and kv_flag must be all NULL or all non-NULL");
  const int64_t cap_qt = *n_qt, cap_nnz = *nnz;
  int64_t t = 0, e = 0;
  if (fill && cap_qt >= 1) kv_ptr[0] = 0;
  for (int64_t qs = 0; qs < N; qs += block_q, ++t) {
    const int64_t qe = std::min<int64_t>(qs + block_q, N);
    bool empty = true;
    int64_t run_s = -1, run_kind = 0;
    auto close = [&](int64_t end) {
      if (run_s < 0) return;
      if (fill && e < cap_nnz) {
        kv_iv[2 * e] = (int32_t)run_s;
        kv_iv[2 * e + 1] = (int32_t)(end - run_s);
        kv_flag[e] = run_kind == 2 ? 1 : 0;
      }
      ++e;
      run_s = -1;
    };
    for (int64_t ks = 0; ks < N; ks += granule) {
      const int64_t ke = std::min<int64_t>(ks + granule, N);
      const int kind = block_kind(qs, qe, ks, ke);
      if (kind == 0 || kind != run_kind) close(ks);
      if (kind != 0) {
        empty = false;
        if (run_s < 0) { run_s = ks; run_kind = kind; }
      }
      run_kind = kind == 0 ? 0 : run_kind;
    }
    close(N);
    if (empty) return fail(ATTN_E_PATTERN, "a query tile attends no key");
    if (fill && t < cap_qt) {
      q_tiles[2 * t] = (int32_t)qs;
      q_tiles[2 * t + 1] = (int32_t)(qe - qs);
      kv_ptr[t + 1] = (int32_t)e;
    }
    if (t > 2147483647LL / 2 || e > 2147483647LL / 2) return fail(ATTN_E_SIZE, "block list too large");
  }
  const bool short_cap = fill && (cap_qt < t || cap_nnz < e);
  *n_qt = (int32_t)t;
  *nnz = (int32_t)e;
  if (short_cap) return fail(ATTN_E_SIZE, "output capacity too small");
  return bsvf::ok();
}

int attn_build_schedule(const int32_t* q_tiles, const int32_t* kv_ptr, const int32_t* kv_iv,
                        int32_t n_qt, int32_t batch, int32_t heads, int32_t group,
                        int32_t num_xcd, int32_t* work_order, int32_t* n_work) {
  if (!q_tiles || !kv_ptr || !kv_iv || !n_work) return fail(ATTN_E_INVAL, "NULL argument");
  if (n_qt <= 0 || batch <= 0 || heads <= 0) return fail(ATTN_E_INVAL, "sizes must be positive");
  if (group < 0 || num_xcd < 1) return fail(ATTN_E_INVAL, "group must be >= 0 and num_xcd >= 1");
  const int64_t items = (int64_t)n_qt * heads * batch;
  if (items > 2147483647LL) return fail(ATTN_E_SIZE, "too many work items");

  // Cost of a tile: attended keys x max(rows, R/2), R the largest tile's
  // rows.  A tile's run time follows its key count; a short tile saves time
  // only once it leaves half of its workgroup's waves idle.  A tile of at most
  // R/4 rows (the kernel walks it with all its waves on a quarter of the
  // rows' work each) costs about a third of a full one: keys x R/3.
  int64_t max_rows = 1;
  for (int32_t t = 0; t < n_qt; ++t) max_rows = std::max<int64_t>(max_rows, q_tiles[2 * t + 1]);
  std::vector<int64_t> cost(n_qt);
  std::vector<char> is_short(n_qt);
  for (int32_t t = 0; t < n_qt; ++t) {
    int64_t keys = 0;
    for (int32_t e = kv_ptr[t]; e < kv_ptr[t + 1]; ++e) keys += kv_iv[2 * e + 1];
    const int64_t rows = q_tiles[2 * t + 1];
    is_short[t] = 4 * rows <= max_rows;
    cost[t] = keys * (is_short[t] ? max_rows / 3 : std::max<int64_t>(rows, max_rows / 2));
  }

  // One queue of items per die; workgroup slot*num_xcd + x takes item
  // queue[x][slot].
  std::vector<std::vector<int32_t>> queue(num_xcd);
  if (group > 0) {
    // Items by decreasing cost (stable), dealt to the dies in groups of `group`.
    std::vector<int32_t> order(items);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
      return cost[a % n_qt] > cost[b % n_qt];
    });
    for (int64_t i = 0; i < items; ++i) queue[(i / group) % num_xcd].push_back(order[i]);
  } else {
    // Tiles of one (batch, head) with the same key intervals (the tiles of one
    // query frame) read the same K and V: keep each such set together on one
    // die, so its tiles stream those keys through that die's L2 at the same
    // time.  Sets of neighbouring frames share most of their keys (the
    // window, the global frames), so the sets in (batch, head, frame) order
    // are cut into num_xcd contiguous runs of about equal cost: a die works
    // through whole heads, or long stretches of one, frame after frame.
    // Short tiles stay out of the sets (a walk of few rows runs ahead of the
    // set's full tiles and would fetch the keys alone): each goes to its
    // set's die, after all of that die's sets, in the same order, where the
    // short tiles of neighbouring frames run together.
    struct Unit { int64_t cost; std::vector<int32_t> items, shorts; };
    std::vector<Unit> units;
    int64_t total = 0;
    for (int64_t bh = 0; bh < (int64_t)batch * heads; ++bh) {
      int32_t t = 0;
      while (t < n_qt) {
        Unit un{0, {}, {}};
        int32_t u = t;
        for (; u < n_qt; ++u) {
          const int32_t n0 = kv_ptr[t + 1] - kv_ptr[t], n1 = kv_ptr[u + 1] - kv_ptr[u];
          if (n0 != n1 || !std::equal(kv_iv + 2 * kv_ptr[t], kv_iv + 2 * kv_ptr[t + 1], kv_iv + 2 * kv_ptr[u]))
            break;
          (is_short[u] ? un.shorts : un.items).push_back((int32_t)(bh * n_qt + u));
          un.cost += cost[u];
        }
        total += un.cost;
        units.push_back(std::move(un));
        t = u;
      }
    }
    // unit j goes to the die whose share of the total cost holds its midpoint
    std::vector<std::vector<int32_t>> tail(num_xcd);
    int64_t before = 0;
    for (const Unit& un : units) {
      int x = 0;
      if (total > 0) {
        const long double mid = (long double)before + (long double)un.cost / 2;
        x = (int)std::min<long double>(num_xcd - 1, mid * num_xcd / total);
      }
      before += un.cost;
      queue[x].insert(queue[x].end(), un.items.begin(), un.items.end());
      tail[x].insert(tail[x].end(), un.shorts.begin(), un.shorts.end());
    }
    for (int x = 0; x < num_xcd; ++x) queue[x].insert(queue[x].end(), tail[x].begin(), tail[x].end());
  }
  size_t depth = 0;
  for (const auto& q : queue) depth = std::max(depth, q.size());
  if (group > 0) depth = (size_t)((depth + group - 1) / group * group);
  const int64_t need = (int64_t)depth * num_xcd;
  if (need > 2147483647LL) return fail(ATTN_E_SIZE, "too many work items");
  if (!work_order) {
    *n_work = (int32_t)need;
    return bsvf::ok();
  }
  if (*n_work < need) {
    *n_work = (int32_t)need;
    return fail(ATTN_E_SIZE, "work_order capacity too small");
  }
  for (int64_t i = 0; i < need; ++i) work_order[i] = -1;
  for (int x = 0; x < num_xcd; ++x)
    for (size_t slot = 0; slot < queue[x].size(); ++slot) work_order[slot * num_xcd + x] = queue[x][slot];
  *n_work = (int32_t)need;
  return bsvf::ok();
}

}  // extern "C"
