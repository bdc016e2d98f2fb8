/*
 * zl.h - C ABI of the MI355X (gfx950) coalesced attention library, libzl.so.
 *
 * What it computes
 *   One GPU runs one rank's share of a mixed image/video batch: whole short
 *   sequences side by side with distributed-attention shards, all in one
 *   launch (the "coalesced attention engine" of the newx.sg page "Zellige:
 *   Moldable Sequence Placement for Mixed Image-Video DiT Training",
 *   Abstract). A shard is one split theta = (q, h, k) of a sequence's
 *   queries, heads and key/value states (pith.science review of arXiv
 *   2608.01150, "What carries the argument"); on one GPU it is simply a work
 *   item with a query row range, a head range and a key/value row range.
 *   Each item is dense, exact, non-causal softmax attention (same review,
 *   "Assumptions", paper Sec. II, after FlashAttention [7]).
 *
 * Conventions
 *   - Q is [q_rows, num_heads, head_dim] bf16, K and V are
 *     [kv_rows, num_heads, head_dim] bf16, row-major and contiguous.
 *   - O is [q_rows, num_heads, head_dim] fp32 and LSE is [q_rows, num_heads]
 *     fp32; LSE is the natural log of sum_j exp(scale * q.k_j).
 *   - The caller owns every buffer, host and device. The library never
 *     allocates device memory, never synchronises, and launches only on the
 *     stream it is given (a hipStream_t passed as void*; NULL = the null
 *     stream). Device pointers must be 16-byte aligned.
 *   - Every call returns ZL_OK (0) or a negative ZL_ERR_* code; no C++
 *     exception crosses the ABI. zl_last_error() gives a thread-local text.
 *   - All argument checks run on the host before any HIP call, so a bad
 *     argument never reaches a kernel.
 *   - Precondition on the data: Q, K, V and dO hold finite values (no NaN,
 *     no infinity). The kernels are built on that assumption (maxima taken
 *     without NaN propagation); with non-finite inputs the outputs are
 *     unspecified, though every launch still runs to completion. The host
 *     side validates its own float arguments with full IEEE semantics (a
 *     NaN softmax scale is rejected).
 */
#ifndef ZL_H_
#define ZL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZL_ABI_VERSION 3
#define ZL_WORKLIST_MAGIC 0x31574c5au /* "ZLW1" little-endian */

enum zl_status {
  ZL_OK = 0,
  ZL_ERR_NULL = -1,     /* a required pointer is NULL */
  ZL_ERR_SHAPE = -2,    /* head_dim not 64/128, num_heads < 1 or too large, negative sizes */
  ZL_ERR_RANGE = -3,    /* an item lies outside the rows or heads */
  ZL_ERR_OVERLAP = -4,  /* two items write the same (query row, head) */
  ZL_ERR_BUFSIZE = -5,  /* host buffer too small */
  ZL_ERR_ALIGN = -6,    /* a device pointer is not 16-byte aligned */
  ZL_ERR_WORKLIST = -7, /* bad magic, version or header in a worklist */
  ZL_ERR_HIP = -8,      /* a HIP call failed; detail in zl_last_error() */
  ZL_ERR_ARG = -9       /* any other invalid argument */
};

/* One work item: query rows [q_off, q_off+q_len) attend to key/value rows
 * [kv_off, kv_off+kv_len) on heads [head_begin, head_begin+head_cnt).
 * A whole sequence of length L is (q_len = L, kv_len = L, all heads); a
 * theta = (q, h, k) shard holds about L/q queries, H/h heads, L/k keys.
 * q_len = 0 or head_cnt = 0 is a no-op; kv_len = 0 gives O = 0 and
 * LSE = -inf on the item's rows. 32 bytes. The six fields are the ones the
 * work-item table names (q_off, q_len, kv_off, kv_len, head_begin, head_cnt);
 * they are stored with the two 64-bit offsets first so that the record has
 * no padding (the Python binding takes them in the table's order). */
typedef struct zl_item {
  int64_t q_off;
  int64_t kv_off;
  int32_t q_len;
  int32_t kv_len;
  int32_t head_begin;
  int32_t head_cnt;
} zl_item;

/* Shapes shared by every item of one launch. softmax_scale <= 0 selects
 * 1/sqrt(head_dim).
 * kv_chunk > 0 splits, inside the forward launch, every item with more than
 * kv_chunk keys into n = ceil(kv_len / kv_chunk) key chunks of equal length
 * (rounded up to a multiple of 64; the last one shorter): each chunk is
 * computed as its own partial (O_p, LSE_p) in a caller workspace and the
 * partials are then merged exactly as zl_merge_partials does (a theta k
 * split done inside one rank: pith.science review, "What carries the
 * argument"). This shortens the longest tiles, so the static schedule
 * balances better. kv_chunk = 0: no split.
 * kv_chunk = ZL_KV_CHUNK_AUTO splits only the items with more than
 * ZL_KV_CHUNK_AUTO_MIN_KEYS keys, each into chunks of at most
 * ZL_KV_CHUNK_AUTO_KEYS keys (as kv_chunk = ZL_KV_CHUNK_AUTO_KEYS would);
 * shorter items stay whole. */
#define ZL_KV_CHUNK_AUTO (-1)
#define ZL_KV_CHUNK_AUTO_MIN_KEYS 131072
#define ZL_KV_CHUNK_AUTO_KEYS 65536
typedef struct zl_problem {
  int64_t q_rows;
  int64_t kv_rows;
  int32_t num_heads;
  int32_t head_dim;
  float softmax_scale;
  int32_t kv_chunk; /* >= 0, or ZL_KV_CHUNK_AUTO */
} zl_problem;

/* Worklist buffer = header, then sections at the header's offsets (each
 * 256-byte aligned): forward tiles and slot offsets, backward tiles and slot
 * offsets, the output map, the merge list, and (when items are split) the
 * unsplit forward tiles and slot offsets for the dQ pass.
 * A forward tile is block_m query rows of one item on one head, against the
 * item's whole key range (or one key chunk of it, see kv_chunk). Tiles are
 * ordered by the stable LPT rule: cost = q_rows * kv_len + cost_c0, sorted by
 * cost, largest first, ties kept in cut order: the unsplit items' tiles in
 * (item, head, query block) order, then the chunks' tiles in (item, chunk,
 * head, query block) order; with n_slots > 0 each tile in that order
 * goes to the least-loaded slot (lowest index on ties) and the tile array
 * is stored slot by slot, slot s owning tiles [slots[s], slots[s+1]). With
 * n_slots == 0 the tile array is the LPT order and the launch has one
 * workgroup per tile. When n_slots is a multiple of 8, slot s runs on
 * workgroup w with s = (w % 8) * (n_slots / 8) + w / 8: workgroups are
 * dispatched round-robin over the 8 XCDs, so consecutive slots (the query
 * blocks of one item and head, which read the same K/V) share an L2. */
typedef struct zl_tile {
  int64_t q_row0;  /* first query row (packed) */
  int64_t kv_row0; /* first key/value row (packed) */
  int32_t q_rows;  /* 1..block_m */
  int32_t kv_len;  /* >= 0 */
  int32_t head;
  int32_t item;    /* item, or n_items + k for the k-th key chunk of a split item */
} zl_tile;

/* Where a forward tile writes: rows q_row0 .. of O / LSE (to_workspace = 0)
 * or of the workspace partials (to_workspace = 1), shifted by o_shift rows.
 * One entry per item and per key chunk of a split item (indexed by
 * zl_tile.item). 16 bytes. */
typedef struct zl_outmap {
  int64_t o_shift;
  int32_t to_workspace;
  int32_t reserved;
} zl_outmap;

/* One split item: its n_parts partials sit at workspace rows
 * ws_row0 + p * q_len (p = 0 .. n_parts-1) and are merged into O / LSE rows
 * q_off .. q_off + q_len on heads [head_begin, head_begin + head_cnt).
 * 32 bytes. */
typedef struct zl_merge {
  int64_t q_off;
  int64_t ws_row0;
  int32_t q_len;
  int32_t head_begin;
  int32_t head_cnt;
  int32_t n_parts;
} zl_merge;

typedef struct zl_worklist_header {
  uint32_t magic;       /* ZL_WORKLIST_MAGIC */
  uint32_t abi_version; /* ZL_ABI_VERSION */
  uint64_t total_bytes;
  int64_t q_rows;
  int64_t kv_rows;
  int32_t num_heads;
  int32_t head_dim;
  float softmax_scale; /* resolved (> 0) */
  int32_t block_m;     /* query rows per forward tile */
  int32_t n_items;
  int32_t n_tiles;
  int32_t n_slots;
  int32_t cost_c0;
  uint64_t tiles_offset; /* bytes from the start of the buffer */
  uint64_t slots_offset; /* int32_t[n_slots + 1]; unused when n_slots == 0 */
  int64_t total_cost;
  int64_t max_slot_cost; /* makespan of the static schedule (0 if n_slots == 0) */
  /* Backward tiles: block_n_bwd keys of one item on one head, against all of
   * the item's query rows; same LPT rule (cost = q_rows * kv_len + c0), with
   * equal costs kept in (item, key block, head) order, and the same slot
   * count, stored slot by slot at bwd_tiles_offset with int32 offsets
   * [n_slots + 1] at bwd_slots_offset. Slot s runs on workgroup s. Items with
   * no queries or no keys have no backward tiles. */
  int32_t block_n_bwd;
  int32_t n_bwd_tiles;
  uint64_t bwd_tiles_offset;
  uint64_t bwd_slots_offset;
  int64_t bwd_max_slot_cost;
  /* In-launch key split (problem.kv_chunk). The forward tiles above then
   * include the chunks' tiles; the backward's query-major dQ pass uses the
   * unsplit forward schedule at dq_tiles_offset (n_dq_tiles tiles, int32
   * slot offsets at dq_slots_offset), which is the forward section itself
   * when nothing is split. outmap: n_vitems zl_outmap entries; merges:
   * n_merges zl_merge entries; ws_rows: rows of the forward workspace. */
  int32_t kv_chunk;
  int32_t n_vitems;
  uint64_t outmap_offset;
  int32_t n_merges;
  int32_t n_dq_tiles;
  uint64_t merges_offset;
  uint64_t dq_tiles_offset;
  uint64_t dq_slots_offset;
  int64_t ws_rows;
  uint8_t pad[8];
} zl_worklist_header; /* 192 bytes */

int zl_abi_version(void);
const char* zl_status_string(int status);
/* Thread-local detail of the last failing call on this thread ("" if none). */
const char* zl_last_error(void);

/* Build the tile schedule for one launch on the host. Two calls: with
 * host_buf == NULL only *bytes is set to the size needed; then, with a
 * buffer of at least that many bytes (8-byte aligned), the worklist is
 * written there and *bytes is set to its size. Host memory only (temporary
 * vectors); no device allocation and no HIP call.
 * The caller copies the buffer to device memory unchanged; a worklist is
 * immutable and can serve any number of launches (every layer of a step).
 * Errors: ZL_ERR_NULL, ZL_ERR_SHAPE (head_dim not 64 or 128, num_heads < 1,
 * num_heads * head_dim > 2^20, negative row counts), ZL_ERR_RANGE,
 * ZL_ERR_OVERLAP, ZL_ERR_BUFSIZE, ZL_ERR_ARG (n_items < 0, n_slots < 0 or
 * > 1<<20, kv_chunk < 0 other than ZL_KV_CHUNK_AUTO, softmax_scale NaN or
 * infinite).
 * The schedule is a stable LPT list schedule: the reading taken of the
 * engine's stable scheduling of whole sequences and shards on one rank
 * (pith.science review of arXiv 2608.01150, "What carries the argument"). */
int zl_build_worklist(const zl_problem* problem, const zl_item* items, int32_t n_items,
                      int32_t n_slots, void* host_buf, size_t* bytes);

/* Coalesced forward: for every item, head and query row,
 *   O = softmax(scale * q K^T) V,  LSE = ln sum_j exp(scale * q.k_j),
 * non-causal, over the item's own key range (exact attention: pith.science
 * review, "Assumptions", Sec. II / FlashAttention [7]; whole sequences and
 * shards in one launch: newx.sg page, Abstract).
 * h_wl: the worklist in host memory (read for the launch shape); d_wl: the
 * same bytes in device memory. q, k, v: bf16 device buffers; o, lse: fp32
 * device buffers. Only (row, head) pairs that some item covers are written.
 * workspace: fp32 device buffer of ws_rows * num_heads * (head_dim + 1)
 * floats (partial O [ws_rows, H, d], then partial LSE [ws_rows, H]) when the
 * worklist splits items (header ws_rows > 0), else ignored (may be NULL);
 * owned by the caller, overwritten. Split items cost one more launch (the
 * merge) on the same stream. Asynchronous on `stream`. Errors: ZL_ERR_NULL,
 * ZL_ERR_WORKLIST, ZL_ERR_ALIGN, ZL_ERR_HIP. */
int zl_coalesced_attn_fwd(const void* h_wl, const void* d_wl, const void* q, const void* k,
                          const void* v, float* o, float* lse, float* workspace, void* stream);

/* Merge of KV-split partials. A k-split shard computes attention of the
 * same queries against disjoint key ranges (pith.science review, "What
 * carries the argument": theta splits key/value states); the exact result
 * over the union follows from the parts' LSE: with M = max_p LSE_p,
 * w_p = exp(LSE_p - M), W = sum_p w_p:  LSE = M + ln W,
 * O = sum_p (w_p / W) O_p. If every part has LSE = -inf: O = 0, LSE = -inf.
 * Part p's rows start p * part_row_stride rows after o_parts / lse_parts;
 * every buffer is laid out [rows, num_heads, head_dim] (O) and
 * [rows, num_heads] (LSE); only heads [head_begin, head_begin+head_cnt) are
 * read and written. o_out / lse_out must not overlap the parts.
 * Errors: ZL_ERR_NULL, ZL_ERR_SHAPE, ZL_ERR_RANGE, ZL_ERR_ARG (n_parts < 1
 * or > 64, part_row_stride < rows, overlapping output), ZL_ERR_ALIGN,
 * ZL_ERR_HIP. */
int zl_merge_partials(int32_t n_parts, int64_t rows, int32_t num_heads, int32_t head_begin,
                      int32_t head_cnt, int32_t head_dim, const float* o_parts,
                      const float* lse_parts, int64_t part_row_stride, float* o_out,
                      float* lse_out, void* stream);

/* Backward of the coalesced forward, recomputing the probabilities from the
 * saved LSE (exact attention, pith.science review "Assumptions", Sec. II /
 * FlashAttention [7]; the split of the dK / dV work over key/value blocks
 * follows the theta k axis, "What carries the argument"). For every item and
 * head, with P = exp(scale * q K^T - LSE):
 *   D    = rowsum(dO * O)                 (scale * D is written to d_ws,
 *                                          [q_rows, H] fp32)
 *   dV  += P^T dO,   dS = P * (dO V^T - D)
 *   dQ  += scale * dS K,   dK += scale * dS^T Q
 * dq [q_rows, H, d], dk and dv [kv_rows, H, d] are fp32 and ACCUMULATED
 * (the caller zeroes them); q, k, v, dout are bf16; o and lse are the
 * forward's outputs. Two launches on `stream`: dQ and D over the forward
 * tiles (each (row, head) has one writer: deterministic), then dK / dV over
 * the backward tiles, added with fp32 atomics because items may share
 * key/value rows (where they do, the order of those sums is not fixed).
 * Errors: ZL_ERR_NULL, ZL_ERR_WORKLIST, ZL_ERR_ALIGN, ZL_ERR_HIP. */
int zl_coalesced_attn_bwd(const void* h_wl, const void* d_wl, const void* q, const void* k,
                          const void* v, const float* o, const float* lse, const void* dout,
                          float* dq, float* dk, float* dv, float* d_ws, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). Same computation, arguments and errors as
 * zl_coalesced_attn_fwd, except that the key-chunk partials of a worklist
 * built with a key split go to a scratch array that the library holds in
 * device memory (ZL_NOALLOC_SCRATCH_BYTES on each GPU it runs on, kept until
 * the process ends) instead of a caller workspace. It calls no hipMalloc,
 * hipFree or allocating routine.
 * - A worklist whose partials need more than ZL_NOALLOC_SCRATCH_BYTES
 *   (ws_rows * num_heads * (head_dim + 1) * 4 bytes) is rejected with
 *   ZL_ERR_BUFSIZE before any HIP call.
 * - The scratch of a GPU is looked up on the first call that needs it, with
 *   that GPU current; `stream` must belong to the current device
 *   (ZL_ERR_ARG otherwise).
 * - Every call on one GPU shares that GPU's scratch and it keeps the last
 *   call's contents: calls that overlap in time on one GPU (different
 *   streams, or host threads) race and give undefined results; calls in
 *   order on one stream are safe. Nothing needs clearing: each partial is
 *   written in full before the merge reads it. */
#define ZL_NOALLOC_SCRATCH_BYTES (64ll << 20)
int zl_coalesced_attn_fwd_noalloc(const void* h_wl, const void* d_wl, const void* q,
                                  const void* k, const void* v, float* o, float* lse,
                                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ZL_H_ */
