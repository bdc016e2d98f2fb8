// Internal declarations shared by the host code and the HIP entry points of
// libzl.so. Not part of the ABI.
#ifndef ZL_INTERNAL_H_
#define ZL_INTERNAL_H_

#include <stdint.h>

#include "zl.h"

namespace zl {

// Forward tile: kFwdWaves waves x 32 query rows, streaming kFwdBlockN keys
// per step. The key block can be overridden at build time
// (-DZL_FWD_BLOCK_N=32) to compare shapes.
#ifndef ZL_FWD_WAVES
#define ZL_FWD_WAVES 8
#endif
#ifndef ZL_FWD_BLOCK_N
#define ZL_FWD_BLOCK_N 64
#endif
constexpr int kFwdWaves = ZL_FWD_WAVES;
constexpr int kFwdBlockM = kFwdWaves * 32;
constexpr int kFwdBlockN = ZL_FWD_BLOCK_N;
static_assert(kFwdBlockM == 256, "the worklist cuts 256-row tiles");
static_assert(sizeof(zl_worklist_header) == 192 && sizeof(zl_tile) == 32 &&
                  sizeof(zl_outmap) == 16 && sizeof(zl_merge) == 32,
              "ABI record sizes");
// dK/dV backward tile: 8 waves x 32 keys, streaming 32 query rows per step.
constexpr int kBwdWaves = 8;
constexpr int kBwdBlockN = kBwdWaves * 32;
constexpr int kBwdBlockM = 32;

// Per-tile fixed cost in (query row x key) units used by the LPT rule: the
// prologue and epilogue of a tile cost about as much as 64 keys of work.
constexpr int kCostC0PerRow = 64;
// Largest static slot count accepted by zl_build_worklist.
constexpr int kMaxSlots = 1 << 20;
// Largest num_heads * head_dim (elements of one packed row). The kernels form
// byte offsets of up to 256 rows inside a buffer resource in 32-bit
// arithmetic: 256 rows * 2^20 elements * 4 bytes (fp32 O) = 2^30 stays clear
// of overflow.
constexpr int64_t kMaxRowElems = int64_t(1) << 20;

// Merge the key-chunk partials of every split item of a worklist (its merge
// list) from the forward workspace into O / LSE, one launch on `stream`.
// Defined with the merge kernel; h is the host header, d_wl the device copy.
int launch_merge_list(const zl_worklist_header* h, const char* d_wl, const float* ws_o,
                      const float* ws_lse, float* o, float* lse, void* stream);

// Record a printf-style detail for zl_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the thread-local error text.
void clear_error();
// Validate a host copy of a worklist; on success *hdr points into it.
int check_worklist(const void* h_wl, const zl_worklist_header** hdr);
// True if p is non-null and 16-byte aligned.
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace zl

#endif  // ZL_INTERNAL_H_
