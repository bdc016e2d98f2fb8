// Randomised checks of the host half of libzl (worklist builder and worklist
// validation), built with g++ under AddressSanitizer and UBSan by
// tests/test_host_sanitizers.py. No HIP: zl_host.cpp is plain C++17.
//
// For random problems and item tables (empty, ragged, overlapping and
// out-of-range items, key splits, any slot count) it checks that the builder
// either rejects the input with the documented status or returns a worklist
// that the validator accepts and whose sections cover the work exactly:
//   - forward tiles: every (query row, head, key) of every item once (key
//     chunks of split items included), outputs redirected to disjoint
//     workspace rows for chunks;
//   - dQ tiles: the unsplit cut, every (query row, head) once;
//   - backward tiles: every (key, head) of every item with queries once;
//   - slot offsets: monotone, ending at the tile count.
// Corrupted headers must be rejected by the validator.

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cmath>
#include <cstring>
#include <map>
#include <random>
#include <set>
#include <tuple>
#include <vector>

#include "zl.h"
#include "zl_internal.h"

#define CHECK(cond)                                                              \
  do {                                                                           \
    if (!(cond)) {                                                               \
      std::fprintf(stderr, "check failed at line %d: %s (case %d)\n", __LINE__, #cond, g_case); \
      std::exit(1);                                                              \
    }                                                                            \
  } while (0)

static int g_case = 0;

struct Built {
  std::vector<uint64_t> buf;  // 8-byte aligned storage
  const zl_worklist_header* h() const { return reinterpret_cast<const zl_worklist_header*>(buf.data()); }
  template <typename T>
  const T* at(uint64_t off) const { return reinterpret_cast<const T*>(reinterpret_cast<const char*>(buf.data()) + off); }
};

static int build(const zl_problem& p, const std::vector<zl_item>& items, int n_slots, Built* out) {
  size_t bytes = 0;
  int rc = zl_build_worklist(&p, items.empty() ? nullptr : items.data(), int32_t(items.size()), n_slots,
                             nullptr, &bytes);
  if (rc) return rc;
  out->buf.assign(bytes / 8 + 1, 0);
  size_t bytes2 = bytes;
  rc = zl_build_worklist(&p, items.empty() ? nullptr : items.data(), int32_t(items.size()), n_slots,
                         out->buf.data(), &bytes2);
  if (rc == 0) CHECK(bytes2 == bytes);
  return rc;
}

static void check_slots(const int32_t* slots, int n_slots, int n_tiles) {
  CHECK(slots[0] == 0 && slots[n_slots] == n_tiles);
  for (int s = 0; s < n_slots; ++s) CHECK(slots[s] <= slots[s + 1]);
}

static void verify(const zl_problem& p, const std::vector<zl_item>& items, int n_slots, const Built& b) {
  const zl_worklist_header* h = b.h();
  const zl_worklist_header* hv = nullptr;
  CHECK(zl::check_worklist(h, &hv) == ZL_OK && hv == h);
  CHECK(h->n_items == int32_t(items.size()) && h->n_slots == n_slots && h->kv_chunk == p.kv_chunk);
  const int n = int(items.size());
  const zl_outmap* om = b.at<zl_outmap>(h->outmap_offset);
  const zl_merge* mg = b.at<zl_merge>(h->merges_offset);
  // chunk item -> original item, from the merge list (items in order)
  std::vector<int> owner(size_t(h->n_vitems), -1);
  for (int i = 0; i < n; ++i) owner[size_t(i)] = i;
  {
    int v = n, m = 0;
    int64_t ws = 0;
    for (int i = 0; i < n; ++i) {
      const zl_item& it = items[size_t(i)];
      if (m < h->n_merges && mg[m].q_off == it.q_off && mg[m].q_len == it.q_len &&
          mg[m].head_begin == it.head_begin && mg[m].head_cnt == it.head_cnt && it.q_len > 0 &&
          p.kv_chunk > 0 && it.kv_len > p.kv_chunk) {
        CHECK(mg[m].ws_row0 == ws && mg[m].n_parts >= 2);
        for (int k = 0; k < mg[m].n_parts; ++k, ++v) {
          owner[size_t(v)] = i;
          CHECK(om[v].to_workspace == 1);
          CHECK(om[v].o_shift == ws + int64_t(k) * it.q_len - it.q_off);
        }
        ws += int64_t(mg[m].n_parts) * it.q_len;
        ++m;
      }
    }
    CHECK(m == h->n_merges && v == h->n_vitems && ws == h->ws_rows);
  }
  for (int i = 0; i < n; ++i) CHECK(om[i].to_workspace == 0 && om[i].o_shift == 0);

  // forward tiles: (item, row, head) -> key ranges, disjoint and complete
  const zl_tile* ft = b.at<zl_tile>(h->tiles_offset);
  std::map<std::tuple<int, int64_t, int>, std::vector<std::pair<int64_t, int64_t>>> keys;
  for (int t = 0; t < h->n_tiles; ++t) {
    const zl_tile& x = ft[t];
    CHECK(x.item >= 0 && x.item < h->n_vitems);
    const int i = owner[size_t(x.item)];
    const zl_item& it = items[size_t(i)];
    CHECK(x.q_rows >= 1 && x.q_rows <= h->block_m);
    CHECK(x.q_row0 >= it.q_off && x.q_row0 + x.q_rows <= it.q_off + it.q_len);
    CHECK(x.head >= it.head_begin && x.head < it.head_begin + it.head_cnt);
    CHECK(x.kv_len >= 0 && x.kv_row0 >= it.kv_off && x.kv_row0 + x.kv_len <= it.kv_off + it.kv_len);
    CHECK((x.q_row0 - it.q_off) % h->block_m == 0);
    keys[{i, x.q_row0, x.head}].push_back({x.kv_row0, x.kv_row0 + x.kv_len});
  }
  int64_t want_blocks = 0;
  for (int i = 0; i < n; ++i) {
    const zl_item& it = items[size_t(i)];
    want_blocks += int64_t(it.head_cnt) * ((int64_t(it.q_len) + h->block_m - 1) / h->block_m);
    for (int hd = it.head_begin; hd < it.head_begin + it.head_cnt; ++hd)
      for (int64_t r0 = it.q_off; r0 < it.q_off + it.q_len; r0 += h->block_m) {
        auto f = keys.find({i, r0, hd});
        CHECK(f != keys.end());
        auto v = f->second;
        std::sort(v.begin(), v.end());
        int64_t pos = it.kv_off;
        for (auto& r : v) {
          CHECK(r.first == pos);
          pos = r.second;
        }
        CHECK(pos == it.kv_off + it.kv_len);
      }
  }
  CHECK(int64_t(keys.size()) == want_blocks);
  if (n_slots > 0) check_slots(b.at<int32_t>(h->slots_offset), n_slots, h->n_tiles);

  // dQ tiles: the unsplit cut
  const zl_tile* qt = b.at<zl_tile>(h->dq_tiles_offset);
  std::set<std::tuple<int, int64_t, int>> qcov;
  for (int t = 0; t < h->n_dq_tiles; ++t) {
    const zl_tile& x = qt[t];
    CHECK(x.item >= 0 && x.item < n);
    const zl_item& it = items[size_t(x.item)];
    CHECK(x.kv_row0 == it.kv_off && x.kv_len == it.kv_len);
    CHECK(qcov.insert({x.item, x.q_row0, x.head}).second);
  }
  CHECK(int64_t(qcov.size()) == want_blocks);
  if (n_slots > 0) check_slots(b.at<int32_t>(h->dq_slots_offset), n_slots, h->n_dq_tiles);

  // backward tiles: every (key block, head) of items with queries once
  const zl_tile* bt = b.at<zl_tile>(h->bwd_tiles_offset);
  std::set<std::tuple<int, int64_t, int>> bcov;
  int64_t want_bwd = 0;
  for (int i = 0; i < n; ++i) {
    const zl_item& it = items[size_t(i)];
    if (it.q_len > 0)
      want_bwd += int64_t(it.head_cnt) * ((int64_t(it.kv_len) + h->block_n_bwd - 1) / h->block_n_bwd);
  }
  for (int t = 0; t < h->n_bwd_tiles; ++t) {
    const zl_tile& x = bt[t];
    CHECK(x.item >= 0 && x.item < n);
    const zl_item& it = items[size_t(x.item)];
    CHECK(x.q_row0 == it.q_off && x.q_rows == it.q_len);
    CHECK(x.kv_len >= 1 && x.kv_len <= h->block_n_bwd);
    CHECK(x.kv_row0 >= it.kv_off && x.kv_row0 + x.kv_len <= it.kv_off + it.kv_len);
    CHECK(bcov.insert({x.item, x.kv_row0, x.head}).second);
  }
  CHECK(int64_t(bcov.size()) == want_bwd && h->n_bwd_tiles == want_bwd);
  if (n_slots > 0) check_slots(b.at<int32_t>(h->bwd_slots_offset), n_slots, h->n_bwd_tiles);

  // corrupted copies are rejected
  const size_t nb = b.buf.size();
  std::vector<uint64_t> bad(b.buf);
  auto* bh = reinterpret_cast<zl_worklist_header*>(bad.data());
  bh->total_bytes = 8;
  CHECK(zl::check_worklist(bad.data(), &hv) == ZL_ERR_WORKLIST);
  std::memcpy(bad.data(), b.buf.data(), nb * 8);
  bh->n_tiles = h->n_tiles + 1000000;
  CHECK(zl::check_worklist(bad.data(), &hv) == ZL_ERR_WORKLIST);
  std::memcpy(bad.data(), b.buf.data(), nb * 8);
  bh->head_dim = 96;
  CHECK(zl::check_worklist(bad.data(), &hv) == ZL_ERR_WORKLIST);
  std::memcpy(bad.data(), b.buf.data(), nb * 8);
  bh->n_merges = h->n_merges + 1000000;
  CHECK(zl::check_worklist(bad.data(), &hv) == ZL_ERR_WORKLIST);
  std::memcpy(bad.data(), b.buf.data(), nb * 8);
  bh->ws_rows = h->n_merges > 0 ? 0 : 64;  // merge list and workspace disagree
  CHECK(zl::check_worklist(bad.data(), &hv) == ZL_ERR_WORKLIST);
  std::memcpy(bad.data(), b.buf.data(), nb * 8);
  bh->tiles_offset = h->tiles_offset + 8;  // misaligned section
  CHECK(zl::check_worklist(bad.data(), &hv) == ZL_ERR_WORKLIST);
  std::memcpy(bad.data(), b.buf.data(), nb * 8);
  bh->softmax_scale = std::nanf("");  // a NaN scale must not pass validation
  CHECK(zl::check_worklist(bad.data(), &hv) == ZL_ERR_WORKLIST);
  std::memcpy(bad.data(), b.buf.data(), nb * 8);
  bh->num_heads = int32_t((zl::kMaxRowElems / bh->head_dim) + 1);  // rows past 2^21 elements
  CHECK(zl::check_worklist(bad.data(), &hv) == ZL_ERR_WORKLIST);
}

int main(int argc, char** argv) {
  const int cases = argc > 1 ? std::atoi(argv[1]) : 400;
  std::mt19937_64 rng(12345);
  auto uni = [&](int a, int b) { return std::uniform_int_distribution<int>(a, b)(rng); };
  int ok = 0, rejected = 0;
  for (g_case = 0; g_case < cases; ++g_case) {
    zl_problem p{};
    p.num_heads = uni(1, 9);
    p.head_dim = uni(0, 1) ? 128 : 64;
    p.softmax_scale = 0.f;
    p.kv_chunk = uni(0, 2) == 0 ? 0 : uni(1, 700);
    const int n_items = uni(0, 9);
    std::vector<zl_item> items;
    int64_t q = 0, kv = 0;
    const bool make_bad = uni(0, 5) == 0;
    for (int i = 0; i < n_items; ++i) {
      zl_item it{};
      it.q_len = uni(0, 3) == 0 ? 0 : uni(1, 900);
      it.kv_len = uni(0, 4) == 0 ? 0 : uni(1, 2500);
      it.head_begin = uni(0, p.num_heads - 1);
      it.head_cnt = uni(0, p.num_heads - it.head_begin);
      it.q_off = q;
      it.kv_off = uni(0, 2) == 0 && kv > 0 ? uni(0, int(kv) - 1) : kv;  // shared keys allowed
      q += it.q_len;
      kv = std::max(kv, it.kv_off + it.kv_len);
      items.push_back(it);
    }
    p.q_rows = q + uni(0, 50);
    p.kv_rows = kv + uni(0, 50);
    int expect = ZL_OK;
    if (make_bad && !items.empty()) {
      const int k = uni(0, 2);
      zl_item& it = items[size_t(uni(0, int(items.size()) - 1))];
      if (k == 0) {  // rows past the buffer
        it.q_off = p.q_rows - it.q_len + 1;
        expect = ZL_ERR_RANGE;
      } else if (k == 1) {  // heads past H
        it.head_begin = p.num_heads;
        it.head_cnt = 1;
        expect = ZL_ERR_RANGE;
      } else if (items.size() >= 2 && items[0].q_len > 0 && items[0].head_cnt > 0) {  // overlap
        zl_item dup = items[0];
        dup.kv_len = 5;
        items.push_back(dup);
        expect = ZL_ERR_OVERLAP;
      }
    }
    const int n_slots = uni(0, 3) == 0 ? 0 : uni(1, 300);
    Built b;
    const int rc = build(p, items, n_slots, &b);
    if (expect != ZL_OK) {
      CHECK(rc == expect || (rc == ZL_ERR_RANGE && expect == ZL_ERR_OVERLAP));
      ++rejected;
      continue;
    }
    CHECK(rc == ZL_OK);
    verify(p, items, n_slots, b);
    ++ok;
  }
  // argument errors
  zl_problem p{};
  p.num_heads = 2;
  p.head_dim = 64;
  p.q_rows = p.kv_rows = 10;
  size_t bytes = 0;
  CHECK(zl_build_worklist(nullptr, nullptr, 0, 0, nullptr, &bytes) == ZL_ERR_NULL);
  CHECK(zl_build_worklist(&p, nullptr, -1, 0, nullptr, &bytes) == ZL_ERR_ARG);
  CHECK(zl_build_worklist(&p, nullptr, 0, -1, nullptr, &bytes) == ZL_ERR_ARG);
  p.kv_chunk = -5;
  CHECK(zl_build_worklist(&p, nullptr, 0, 0, nullptr, &bytes) == ZL_ERR_ARG);
  p.kv_chunk = 0;
  p.softmax_scale = std::nanf("");
  CHECK(zl_build_worklist(&p, nullptr, 0, 0, nullptr, &bytes) == ZL_ERR_ARG);
  p.softmax_scale = 0.f;
  p.num_heads = int32_t(zl::kMaxRowElems / 64) + 1;
  CHECK(zl_build_worklist(&p, nullptr, 0, 0, nullptr, &bytes) == ZL_ERR_SHAPE);
  CHECK(zl::check_worklist(nullptr, nullptr) == ZL_ERR_NULL);
  std::printf("host fuzz: %d worklists verified, %d rejected as expected\n", ok, rejected);
  return 0;
}
