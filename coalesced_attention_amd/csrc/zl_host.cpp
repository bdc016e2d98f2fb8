// Host half of libzl.so: status strings, thread-local error text, argument
// validation and the stable LPT worklist builder. Plain C++17 with no HIP
// headers, so it builds with hipcc for the library and with g++ (under
// sanitizers) for host-only checks.
//
// Scheduling reading: the engine places whole sequences and shards on one
// rank with a stable schedule (pith.science review of arXiv 2608.01150,
// "What carries the argument"). Tiles are cut per (item, head, query block),
// sorted by cost with a total order that keeps equal costs in cut order (a
// stable sort), and placed longest first on the least-loaded slot.

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "zl.h"
#include "zl_internal.h"

namespace zl {

namespace {
// fixed storage: reporting an error never allocates, so no exception can
// leave an entry point through it
thread_local char g_error[512];
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_error[0] = '\0'; }

int check_worklist(const void* h_wl, const zl_worklist_header** hdr) {
  if (!h_wl) return fail(ZL_ERR_NULL, "host worklist is NULL");
  const auto* h = static_cast<const zl_worklist_header*>(h_wl);
  if (h->magic != ZL_WORKLIST_MAGIC) return fail(ZL_ERR_WORKLIST, "worklist magic mismatch");
  if (h->abi_version != ZL_ABI_VERSION)
    return fail(ZL_ERR_WORKLIST, "worklist built for ABI %u, library is %d", h->abi_version,
                ZL_ABI_VERSION);
  if ((h->head_dim != 64 && h->head_dim != 128) || h->num_heads < 1 ||
      int64_t(h->num_heads) * h->head_dim > kMaxRowElems || h->n_tiles < 0 ||
      h->n_slots < 0 || h->n_slots > kMaxSlots || h->block_m != kFwdBlockM ||
      !(h->softmax_scale > 0.f) || h->q_rows < 0 || h->kv_rows < 0)
    return fail(ZL_ERR_WORKLIST, "worklist header fields out of range");
  if (h->block_n_bwd != kBwdBlockN || h->n_bwd_tiles < 0)
    return fail(ZL_ERR_WORKLIST, "worklist backward fields out of range");
  uint64_t need = h->tiles_offset + uint64_t(h->n_tiles) * sizeof(zl_tile);
  if (h->n_slots > 0) {
    if (h->slots_offset < need) return fail(ZL_ERR_WORKLIST, "worklist slot table overlaps tiles");
    need = h->slots_offset + uint64_t(h->n_slots + 1) * sizeof(int32_t);
  }
  if (h->bwd_tiles_offset < need) return fail(ZL_ERR_WORKLIST, "worklist sections overlap");
  need = h->bwd_tiles_offset + uint64_t(h->n_bwd_tiles) * sizeof(zl_tile);
  if (h->n_slots > 0) {
    if (h->bwd_slots_offset < need) return fail(ZL_ERR_WORKLIST, "worklist sections overlap");
    need = h->bwd_slots_offset + uint64_t(h->n_slots + 1) * sizeof(int32_t);
  }
  if (h->kv_chunk < ZL_KV_CHUNK_AUTO || h->n_vitems < h->n_items || h->n_merges < 0 || h->n_dq_tiles < 0 ||
      h->ws_rows < 0 || (h->n_merges > 0) != (h->ws_rows > 0))
    return fail(ZL_ERR_WORKLIST, "worklist split fields out of range");
  if (h->outmap_offset < need) return fail(ZL_ERR_WORKLIST, "worklist sections overlap");
  need = h->outmap_offset + uint64_t(h->n_vitems) * sizeof(zl_outmap);
  if (h->merges_offset < need) return fail(ZL_ERR_WORKLIST, "worklist sections overlap");
  need = h->merges_offset + uint64_t(h->n_merges) * sizeof(zl_merge);
  if (h->n_merges == 0) {
    if (h->dq_tiles_offset != h->tiles_offset || h->dq_slots_offset != h->slots_offset ||
        h->n_dq_tiles != h->n_tiles)
      return fail(ZL_ERR_WORKLIST, "worklist dQ section must alias the forward one");
  } else {
    if (h->dq_tiles_offset < need) return fail(ZL_ERR_WORKLIST, "worklist sections overlap");
    need = h->dq_tiles_offset + uint64_t(h->n_dq_tiles) * sizeof(zl_tile);
    if (h->n_slots > 0) {
      if (h->dq_slots_offset < need) return fail(ZL_ERR_WORKLIST, "worklist sections overlap");
      need = h->dq_slots_offset + uint64_t(h->n_slots + 1) * sizeof(int32_t);
    }
  }
  if (h->tiles_offset < sizeof(zl_worklist_header) || (h->tiles_offset & 15u) ||
      (h->slots_offset & 15u) || (h->bwd_tiles_offset & 15u) || (h->bwd_slots_offset & 15u) ||
      (h->outmap_offset & 15u) || (h->merges_offset & 15u) || (h->dq_tiles_offset & 15u) ||
      (h->dq_slots_offset & 15u) || need > h->total_bytes)
    return fail(ZL_ERR_WORKLIST, "worklist offsets inconsistent with its size");
  *hdr = h;
  return ZL_OK;
}

}  // namespace zl

using namespace zl;

extern "C" int zl_abi_version(void) { return ZL_ABI_VERSION; }

extern "C" const char* zl_status_string(int status) {
  switch (status) {
    case ZL_OK: return "ok";
    case ZL_ERR_NULL: return "null pointer";
    case ZL_ERR_SHAPE: return "unsupported shape";
    case ZL_ERR_RANGE: return "item out of range";
    case ZL_ERR_OVERLAP: return "items overlap";
    case ZL_ERR_BUFSIZE: return "buffer too small";
    case ZL_ERR_ALIGN: return "pointer not 16-byte aligned";
    case ZL_ERR_WORKLIST: return "invalid worklist";
    case ZL_ERR_HIP: return "HIP error";
    case ZL_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

extern "C" const char* zl_last_error(void) { return g_error; }

namespace {

constexpr uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

int validate_items(const zl_problem& p, const zl_item* items, int32_t n_items) {
  for (int32_t i = 0; i < n_items; ++i) {
    const zl_item& it = items[i];
    if (it.q_len < 0 || it.kv_len < 0 || it.head_cnt < 0 || it.q_off < 0 || it.kv_off < 0 ||
        it.head_begin < 0)
      return fail(ZL_ERR_RANGE, "item %d has a negative field", i);
    if (it.q_off + it.q_len > p.q_rows || it.kv_off + it.kv_len > p.kv_rows ||
        int64_t(it.head_begin) + it.head_cnt > p.num_heads)
      return fail(ZL_ERR_RANGE, "item %d lies outside the packed buffers or heads", i);
  }
  // Two items may share query rows only on disjoint heads.
  std::vector<int32_t> order;
  order.reserve(n_items);
  for (int32_t i = 0; i < n_items; ++i)
    if (items[i].q_len > 0 && items[i].head_cnt > 0) order.push_back(i);
  std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return items[a].q_off != items[b].q_off ? items[a].q_off < items[b].q_off : a < b;
  });
  for (size_t x = 0; x < order.size(); ++x) {
    const zl_item& a = items[order[x]];
    for (size_t y = x + 1; y < order.size(); ++y) {
      const zl_item& b = items[order[y]];
      if (b.q_off >= a.q_off + a.q_len) break;
      if (b.head_begin < a.head_begin + a.head_cnt && a.head_begin < b.head_begin + b.head_cnt)
        return fail(ZL_ERR_OVERLAP, "items %d and %d write the same (row, head)", order[x],
                    order[y]);
    }
  }
  return ZL_OK;
}

struct TileKey {
  zl_tile t;
  int64_t cost;
};

// Stable LPT: order by cost, largest first, equal costs in cut order -- a
// total order, so std::sort gives the stable result. Forward tiles are cut
// in (item, head, first query row) order; backward tiles (kv_first) in
// (item, first key row, head) order.
// With n_slots == 0 the order itself is written; otherwise each tile goes to
// the least-loaded slot (lowest index on ties) and the tiles are written slot
// by slot with offsets [n_slots + 1].
int schedule(std::vector<TileKey>& tiles, int32_t n_slots, zl_tile* out, int32_t* slots,
             int64_t* total_cost, int64_t* makespan, bool kv_first = false) {
  std::sort(tiles.begin(), tiles.end(), [kv_first](const TileKey& a, const TileKey& b) {
    if (a.cost != b.cost) return a.cost > b.cost;
    if (a.t.item != b.t.item) return a.t.item < b.t.item;
    if (kv_first && a.t.kv_row0 != b.t.kv_row0) return a.t.kv_row0 < b.t.kv_row0;
    if (a.t.head != b.t.head) return a.t.head < b.t.head;
    if (a.t.q_row0 != b.t.q_row0) return a.t.q_row0 < b.t.q_row0;
    return a.t.kv_row0 < b.t.kv_row0;
  });
  const int32_t n = int32_t(tiles.size());
  *total_cost = 0;
  *makespan = 0;
  for (const TileKey& k : tiles) *total_cost += k.cost;
  if (n_slots == 0) {
    for (int32_t t = 0; t < n; ++t) out[t] = tiles[size_t(t)].t;
    return ZL_OK;
  }
  try {
    // Least-loaded slot, lowest index on ties: a binary heap ordered by
    // (load, slot); then a stable counting sort lays the tiles out by slot.
    std::vector<std::pair<int64_t, int32_t>> heap;
    std::vector<int32_t> slot_of(static_cast<size_t>(n));
    std::vector<int32_t> count(static_cast<size_t>(n_slots) + 1, 0);
    std::vector<int64_t> load(static_cast<size_t>(n_slots), 0);
    heap.reserve(size_t(n_slots));
    for (int32_t s = 0; s < n_slots; ++s) heap.emplace_back(0, s);
    auto cmp = [](const std::pair<int64_t, int32_t>& a, const std::pair<int64_t, int32_t>& b) {
      return a > b;  // min-heap on (load, slot)
    };
    std::make_heap(heap.begin(), heap.end(), cmp);
    for (int32_t t = 0; t < n; ++t) {
      std::pop_heap(heap.begin(), heap.end(), cmp);
      const int32_t s = heap.back().second;
      heap.back().first += tiles[size_t(t)].cost;
      slot_of[size_t(t)] = s;
      load[size_t(s)] = heap.back().first;
      ++count[size_t(s) + 1];
      std::push_heap(heap.begin(), heap.end(), cmp);
    }
    for (int32_t s = 0; s < n_slots; ++s) count[size_t(s) + 1] += count[size_t(s)];
    for (int32_t s = 0; s <= n_slots; ++s) slots[s] = count[size_t(s)];
    std::vector<int32_t> fill(count.begin(), count.end() - 1);
    for (int32_t t = 0; t < n; ++t) out[fill[size_t(slot_of[size_t(t)])]++] = tiles[size_t(t)].t;
    for (int64_t l : load) *makespan = std::max(*makespan, l);
  } catch (const std::bad_alloc&) {
    return fail(ZL_ERR_ARG, "out of host memory scheduling %d tiles", n);
  }
  return ZL_OK;
}

}  // namespace

extern "C" int zl_build_worklist(const zl_problem* problem, const zl_item* items, int32_t n_items,
                                 int32_t n_slots, void* host_buf, size_t* bytes) {
  clear_error();
  if (!problem || !bytes) return fail(ZL_ERR_NULL, "problem and bytes must be non-NULL");
  if (n_items < 0) return fail(ZL_ERR_ARG, "n_items < 0");
  if (n_items > 0 && !items) return fail(ZL_ERR_NULL, "items is NULL");
  if (n_slots < 0 || n_slots > kMaxSlots) return fail(ZL_ERR_ARG, "n_slots out of range");
  const zl_problem& p = *problem;
  if ((p.head_dim != 64 && p.head_dim != 128) || p.num_heads < 1 || p.q_rows < 0 ||
      p.kv_rows < 0)
    return fail(ZL_ERR_SHAPE, "head_dim must be 64 or 128 and sizes non-negative");
  if (int64_t(p.num_heads) * p.head_dim > kMaxRowElems)
    return fail(ZL_ERR_SHAPE, "num_heads * head_dim exceeds %lld", (long long)kMaxRowElems);
  if (p.kv_chunk < ZL_KV_CHUNK_AUTO)
    return fail(ZL_ERR_ARG, "problem.kv_chunk must be >= 0 or ZL_KV_CHUNK_AUTO");
  if (!(p.softmax_scale <= 0.f || std::isfinite(p.softmax_scale)))
    return fail(ZL_ERR_ARG, "softmax_scale must be finite");
  int rc = validate_items(p, items, n_items);
  if (rc) return rc;

  const int block_m = kFwdBlockM;
  // Key split: item i has parts[i] chunks of chunk[i] keys (the last one
  // shorter); only items with queries, heads and more than kv_chunk keys.
  std::vector<int32_t> parts, chunk;
  try {
    parts.assign(size_t(n_items), 1);
    chunk.assign(size_t(n_items), 0);
  } catch (const std::bad_alloc&) {
    return fail(ZL_ERR_ARG, "out of host memory for %d items", n_items);
  }
  int64_t n_unsplit64 = 0, n_tiles64 = 0, n_vitems64 = n_items, ws_rows = 0;
  int32_t n_merges = 0;
  for (int32_t i = 0; i < n_items; ++i) {
    const zl_item& it = items[i];
    const int64_t qblocks = (int64_t(it.q_len) + block_m - 1) / block_m;
    n_unsplit64 += int64_t(it.head_cnt) * qblocks;
    // ZL_KV_CHUNK_AUTO: only items above the automatic threshold, in chunks
    // of at most ZL_KV_CHUNK_AUTO_KEYS keys
    const int32_t kc = p.kv_chunk != ZL_KV_CHUNK_AUTO ? p.kv_chunk
                       : it.kv_len > ZL_KV_CHUNK_AUTO_MIN_KEYS ? ZL_KV_CHUNK_AUTO_KEYS
                                                               : 0;
    if (kc > 0 && it.q_len > 0 && it.head_cnt > 0 && it.kv_len > kc) {
      const int64_t n = (int64_t(it.kv_len) + kc - 1) / kc;
      const int64_t c = ((int64_t(it.kv_len) + n - 1) / n + 63) / 64 * 64;
      parts[size_t(i)] = int32_t((it.kv_len + c - 1) / c);
      chunk[size_t(i)] = int32_t(c);
    }
    if (parts[size_t(i)] > 1) {
      n_vitems64 += parts[size_t(i)];
      ws_rows += int64_t(parts[size_t(i)]) * it.q_len;
      ++n_merges;
    }
    n_tiles64 += int64_t(it.head_cnt) * qblocks * parts[size_t(i)];
  }
  int64_t n_bwd64 = 0;
  for (int32_t i = 0; i < n_items; ++i) {
    const zl_item& it = items[i];
    if (it.q_len > 0)
      n_bwd64 += int64_t(it.head_cnt) * ((int64_t(it.kv_len) + kBwdBlockN - 1) / kBwdBlockN);
  }
  if (n_tiles64 > INT32_MAX || n_bwd64 > INT32_MAX || n_vitems64 > INT32_MAX)
    return fail(ZL_ERR_ARG, "too many tiles");
  const int32_t n_tiles = int32_t(n_tiles64), n_bwd_tiles = int32_t(n_bwd64);
  const int32_t n_unsplit = int32_t(n_unsplit64), n_vitems = int32_t(n_vitems64);
  const bool split = n_merges > 0;
  const uint64_t slot_bytes = n_slots > 0 ? uint64_t(n_slots + 1) * 4 : 0;
  const uint64_t tiles_off = align_up(sizeof(zl_worklist_header), 256);
  const uint64_t slots_off = align_up(tiles_off + uint64_t(n_tiles) * sizeof(zl_tile), 256);
  const uint64_t bwd_tiles_off = align_up(slots_off + slot_bytes, 256);
  const uint64_t bwd_slots_off = align_up(bwd_tiles_off + uint64_t(n_bwd_tiles) * sizeof(zl_tile), 256);
  const uint64_t outmap_off = align_up(bwd_slots_off + slot_bytes, 256);
  const uint64_t merges_off = align_up(outmap_off + uint64_t(n_vitems) * sizeof(zl_outmap), 256);
  uint64_t end = align_up(merges_off + uint64_t(n_merges) * sizeof(zl_merge), 256);
  uint64_t dq_tiles_off = tiles_off, dq_slots_off = n_slots > 0 ? slots_off : 0;
  if (split) {
    dq_tiles_off = end;
    dq_slots_off = align_up(dq_tiles_off + uint64_t(n_unsplit) * sizeof(zl_tile), 256);
    end = align_up(dq_slots_off + slot_bytes, 256);
    if (n_slots == 0) dq_slots_off = 0;
  }
  const uint64_t total = end;
  if (!host_buf) {
    *bytes = size_t(total);
    return ZL_OK;
  }
  if (*bytes < total) return fail(ZL_ERR_BUFSIZE, "worklist needs %llu bytes", (unsigned long long)total);
  if (reinterpret_cast<uintptr_t>(host_buf) & 7u) return fail(ZL_ERR_ALIGN, "host_buf must be 8-byte aligned");

  char* base = static_cast<char*>(host_buf);
  std::memset(base, 0, size_t(total));
  auto* hdr = reinterpret_cast<zl_worklist_header*>(base);

  // Forward tiles: block_m query rows x one head x the item's key range --
  // the unsplit items first, in (item, head, query block) order, then the
  // key chunks of split items as items n_items, n_items + 1, ... in (item,
  // chunk, head, query block) order. The dQ pass uses the unsplit cut.
  const int64_t c0 = int64_t(block_m) * kCostC0PerRow;
  auto* outmap = reinterpret_cast<zl_outmap*>(base + outmap_off);
  auto* merges = reinterpret_cast<zl_merge*>(base + merges_off);
  std::vector<TileKey> tiles, dq_tiles;
  try {
    tiles.reserve(size_t(n_tiles));
    auto cut = [&](std::vector<TileKey>& out, int32_t i, int32_t vitem, int32_t k0, int32_t keys) {
      const zl_item& it = items[i];
      for (int32_t h = it.head_begin; h < it.head_begin + it.head_cnt; ++h)
        for (int32_t r0 = 0; r0 < it.q_len; r0 += block_m) {
          const int32_t rows = std::min(block_m, it.q_len - r0);
          out.push_back(TileKey{zl_tile{it.q_off + r0, it.kv_off + k0, rows, keys, h, vitem},
                                int64_t(rows) * keys + c0});
        }
    };
    for (int32_t i = 0; i < n_items; ++i) {
      outmap[i] = zl_outmap{0, 0, 0};
      if (parts[size_t(i)] == 1) cut(tiles, i, i, 0, items[i].kv_len);
    }
    int32_t vitem = n_items, m = 0;
    int64_t ws_row = 0;
    for (int32_t i = 0; i < n_items; ++i) {
      if (parts[size_t(i)] == 1) continue;
      const zl_item& it = items[i];
      merges[m++] = zl_merge{it.q_off, ws_row, it.q_len, it.head_begin, it.head_cnt, parts[size_t(i)]};
      for (int32_t pidx = 0; pidx < parts[size_t(i)]; ++pidx, ++vitem) {
        const int32_t k0 = pidx * chunk[size_t(i)];
        outmap[vitem] = zl_outmap{ws_row + int64_t(pidx) * it.q_len - it.q_off, 1, 0};
        cut(tiles, i, vitem, k0, std::min(chunk[size_t(i)], it.kv_len - k0));
      }
      ws_row += int64_t(parts[size_t(i)]) * it.q_len;
    }
    if (split) {
      dq_tiles.reserve(size_t(n_unsplit));
      for (int32_t i = 0; i < n_items; ++i) cut(dq_tiles, i, i, 0, items[i].kv_len);
    }
  } catch (const std::bad_alloc&) {
    return fail(ZL_ERR_ARG, "out of host memory for %d tiles", n_tiles);
  }
  int64_t total_cost = 0, makespan = 0;
  rc = schedule(tiles, n_slots, reinterpret_cast<zl_tile*>(base + tiles_off),
                reinterpret_cast<int32_t*>(base + slots_off), &total_cost, &makespan);
  if (rc) return rc;
  if (split) {
    int64_t dq_total = 0, dq_makespan = 0;
    rc = schedule(dq_tiles, n_slots, reinterpret_cast<zl_tile*>(base + dq_tiles_off),
                  reinterpret_cast<int32_t*>(base + (n_slots > 0 ? dq_slots_off : dq_tiles_off)),
                  &dq_total, &dq_makespan);
    if (rc) return rc;
  }

  // Backward tiles: block_n_bwd keys x one head x all of the item's queries.
  const int64_t c0_bwd = int64_t(kBwdBlockN) * kCostC0PerRow;
  std::vector<TileKey> btiles;
  try {
    btiles.reserve(size_t(n_bwd_tiles));
    for (int32_t i = 0; i < n_items; ++i) {
      const zl_item& it = items[i];
      if (it.q_len == 0) continue;
      for (int32_t k0 = 0; k0 < it.kv_len; k0 += kBwdBlockN) {
        const int32_t keys = std::min(kBwdBlockN, it.kv_len - k0);
        for (int32_t h = it.head_begin; h < it.head_begin + it.head_cnt; ++h)
          btiles.push_back(TileKey{zl_tile{it.q_off, it.kv_off + k0, it.q_len, keys, h, i},
                                   int64_t(keys) * it.q_len + c0_bwd});
      }
    }
  } catch (const std::bad_alloc&) {
    return fail(ZL_ERR_ARG, "out of host memory for %d backward tiles", n_bwd_tiles);
  }
  int64_t bwd_total = 0, bwd_makespan = 0;
  rc = schedule(btiles, n_slots, reinterpret_cast<zl_tile*>(base + bwd_tiles_off),
                reinterpret_cast<int32_t*>(base + bwd_slots_off), &bwd_total, &bwd_makespan, true);
  if (rc) return rc;

  hdr->magic = ZL_WORKLIST_MAGIC;
  hdr->abi_version = ZL_ABI_VERSION;
  hdr->total_bytes = total;
  hdr->q_rows = p.q_rows;
  hdr->kv_rows = p.kv_rows;
  hdr->num_heads = p.num_heads;
  hdr->head_dim = p.head_dim;
  hdr->softmax_scale = p.softmax_scale > 0.f ? p.softmax_scale
                                             : float(1.0 / std::sqrt(double(p.head_dim)));
  hdr->block_m = block_m;
  hdr->n_items = n_items;
  hdr->n_tiles = n_tiles;
  hdr->n_slots = n_slots;
  hdr->cost_c0 = int32_t(c0);
  hdr->tiles_offset = tiles_off;
  hdr->slots_offset = n_slots > 0 ? slots_off : 0;
  hdr->total_cost = total_cost;
  hdr->max_slot_cost = makespan;
  hdr->block_n_bwd = kBwdBlockN;
  hdr->n_bwd_tiles = n_bwd_tiles;
  hdr->bwd_tiles_offset = bwd_tiles_off;
  hdr->bwd_slots_offset = n_slots > 0 ? bwd_slots_off : 0;
  hdr->bwd_max_slot_cost = bwd_makespan;
  hdr->kv_chunk = p.kv_chunk;
  hdr->n_vitems = n_vitems;
  hdr->outmap_offset = outmap_off;
  hdr->n_merges = n_merges;
  hdr->n_dq_tiles = split ? n_unsplit : n_tiles;
  hdr->merges_offset = merges_off;
  hdr->dq_tiles_offset = dq_tiles_off;
  hdr->dq_slots_offset = dq_slots_off;
  hdr->ws_rows = ws_rows;
  *bytes = size_t(total);
  return ZL_OK;
}
