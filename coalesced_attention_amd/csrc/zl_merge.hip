// Merge of KV-split partials for gfx950.
//
// A theta = (q, h, k) shard with k > 1 computes the same queries against k
// disjoint key ranges (pith.science review of arXiv 2608.01150, "What
// carries the argument"). Each partial carries its softmax average O_p and
// its log-sum-exp LSE_p; the exact attention over the union of the key
// ranges (the review's "Assumptions", Sec. II, exact attention after
// FlashAttention [7]) weights part p by exp(LSE_p - LSE).
//
// The kernel is a pure stream over HBM: each thread owns 4 consecutive
// head_dim elements of one (row, head) and reads them from every part with
// 128-bit non-temporal loads (the partials are read once), writing the result
// with a non-temporal store; consecutive threads cover consecutive addresses.
// The part weights are recomputed per thread from the n_parts LSE values,
// which hit in cache after the first thread of the (row, head).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "zl.h"
#include "zl_internal.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxParts = 64;
constexpr int kThreads = 256;

// One (row, head, 4 head_dim elements) of a merge: parts at o_parts /
// lse_parts (already offset to the row and head), part p a further p *
// o_part / lse_part elements on.
template <int D>
__device__ __forceinline__ void merge_one(int n_parts, const float* __restrict__ o_parts,
                                          const float* __restrict__ lse_parts, int64_t o_part,
                                          int64_t lse_part, float* __restrict__ o_out,
                                          float* __restrict__ lse_out, bool write_lse) {
  float m = -INFINITY;
  for (int p = 0; p < n_parts; ++p) m = fmaxf(m, lse_parts[p * lse_part]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse;
  if (m == -INFINITY) {
    lse = -INFINITY;  // no keys in any part: O = 0
  } else {
    float wsum = 0.f;
    for (int p = 0; p < n_parts; ++p) {
      const float w = __expf(lse_parts[p * lse_part] - m);
      wsum += w;
      const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(o_parts + p * o_part));
      acc += w * x;
    }
    const float inv = 1.f / wsum;
    acc *= inv;
    lse = m + __logf(wsum);
  }
  __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(o_out));
  if (write_lse) *lse_out = lse;
}

template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(
    int n_parts, int64_t rows, int H, int head_begin, int head_cnt,
    const float* __restrict__ o_parts, const float* __restrict__ lse_parts,
    int64_t part_row_stride, float* __restrict__ o_out, float* __restrict__ lse_out) {
  constexpr int kVec = D / 4;
  const int64_t total = rows * head_cnt * kVec;
  for (int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x; gid < total;
       gid += int64_t(gridDim.x) * kThreads) {
    const int vec = int(gid % kVec);
    const int64_t rh = gid / kVec;
    const int head = head_begin + int(rh % head_cnt);
    const int64_t row = rh / head_cnt;
    const int64_t lse_idx = row * H + head;
    const int64_t o_idx = lse_idx * D + vec * 4;
    const int64_t lse_part = part_row_stride * H;
    merge_one<D>(n_parts, o_parts + o_idx, lse_parts + lse_idx, lse_part * D, lse_part,
                 o_out + o_idx, lse_out + lse_idx, vec == 0);
  }
}

// The merge list of a worklist: blockIdx.y (striding by gridDim.y) picks a
// split item, the x dimension strides over its (row, head, 4 elements); the
// partials sit in the forward workspace, part p of item m at rows
// ws_row0 + p * q_len.
template <int D>
__global__ __launch_bounds__(kThreads) void merge_list_kernel(
    const zl_merge* __restrict__ merges, int n_merges, const float* __restrict__ ws_o,
    const float* __restrict__ ws_lse, float* __restrict__ O, float* __restrict__ LSE, int H) {
  constexpr int kVec = D / 4;
  for (int mi = blockIdx.y; mi < n_merges; mi += gridDim.y) {
    const zl_merge m = merges[mi];
    const int64_t total = int64_t(m.q_len) * m.head_cnt * kVec;
    for (int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x; gid < total;
         gid += int64_t(gridDim.x) * kThreads) {
      const int vec = int(gid % kVec);
      const int64_t rh = gid / kVec;
      const int head = m.head_begin + int(rh % m.head_cnt);
      const int64_t r = rh / m.head_cnt;
      const int64_t src = (m.ws_row0 + r) * H + head;
      const int64_t dst = (m.q_off + r) * H + head;
      const int64_t lse_part = int64_t(m.q_len) * H;
      merge_one<D>(m.n_parts, ws_o + src * D + vec * 4, ws_lse + src, lse_part * D, lse_part,
                   O + dst * D + vec * 4, LSE + dst, vec == 0);
    }
  }
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

}  // namespace

extern "C" int zl_merge_partials(int32_t n_parts, int64_t rows, int32_t num_heads,
                                 int32_t head_begin, int32_t head_cnt, int32_t head_dim,
                                 const float* o_parts, const float* lse_parts,
                                 int64_t part_row_stride, float* o_out, float* lse_out,
                                 void* stream) {
  zl::clear_error();
  if (!o_parts || !lse_parts || !o_out || !lse_out)
    return zl::fail(ZL_ERR_NULL, "merge buffers must be non-NULL");
  if ((head_dim != 64 && head_dim != 128) || num_heads < 1 || rows < 0 || head_cnt < 0)
    return zl::fail(ZL_ERR_SHAPE, "head_dim must be 64 or 128, sizes non-negative");
  if (head_begin < 0 || int64_t(head_begin) + head_cnt > num_heads)
    return zl::fail(ZL_ERR_RANGE, "head range outside [0, num_heads)");
  if (n_parts < 1 || n_parts > kMaxParts) return zl::fail(ZL_ERR_ARG, "n_parts must be in [1, 64]");
  if (part_row_stride < rows) return zl::fail(ZL_ERR_ARG, "part_row_stride < rows: parts overlap");
  if (!zl::aligned16(o_parts) || !zl::aligned16(o_out))
    return zl::fail(ZL_ERR_ALIGN, "O buffers must be 16-byte aligned");
  if (rows == 0 || head_cnt == 0) return ZL_OK;
  const size_t o_row = size_t(num_heads) * head_dim * 4, l_row = size_t(num_heads) * 4;
  const size_t o_parts_bytes = size_t(part_row_stride) * o_row * size_t(n_parts - 1) + size_t(rows) * o_row;
  const size_t l_parts_bytes = size_t(part_row_stride) * l_row * size_t(n_parts - 1) + size_t(rows) * l_row;
  const size_t o_out_bytes = size_t(rows) * o_row, l_out_bytes = size_t(rows) * l_row;
  if (ranges_overlap(o_out, o_out_bytes, o_parts, o_parts_bytes) ||
      ranges_overlap(o_out, o_out_bytes, lse_parts, l_parts_bytes) ||
      ranges_overlap(lse_out, l_out_bytes, o_parts, o_parts_bytes) ||
      ranges_overlap(lse_out, l_out_bytes, lse_parts, l_parts_bytes) ||
      ranges_overlap(o_out, o_out_bytes, lse_out, l_out_bytes))
    return zl::fail(ZL_ERR_ARG, "merge output overlaps an input or itself");

  const int64_t total = rows * head_cnt * (head_dim / 4);
  // a grid-stride loop over at most 16 workgroups per CU
  const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, 256 * 16);
  if (blocks > INT32_MAX) return zl::fail(ZL_ERR_ARG, "merge too large for one launch");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, n_parts,
                       rows, num_heads, head_begin, head_cnt, o_parts, lse_parts, part_row_stride,
                       o_out, lse_out);
  else
    hipLaunchKernelGGL(merge_kernel<64>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, n_parts,
                       rows, num_heads, head_begin, head_cnt, o_parts, lse_parts, part_row_stride,
                       o_out, lse_out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return zl::fail(ZL_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
  return ZL_OK;
}

namespace zl {

int launch_merge_list(const zl_worklist_header* h, const char* d_wl, const float* ws_o,
                      const float* ws_lse, float* o, float* lse, void* stream) {
  if (h->n_merges == 0) return ZL_OK;
  // enough blocks along x to cover the largest split item's elements a few
  // times over the chip, at most 65535 items along y (the kernel strides)
  const zl_merge* hm = reinterpret_cast<const zl_merge*>(reinterpret_cast<const char*>(h) + h->merges_offset);
  int64_t most = 0;
  for (int32_t i = 0; i < h->n_merges; ++i)
    most = std::max(most, int64_t(hm[i].q_len) * hm[i].head_cnt * (h->head_dim / 4));
  const unsigned gx = unsigned(std::max<int64_t>(1, std::min<int64_t>((most + kThreads - 1) / kThreads, 4096)));
  const unsigned gy = unsigned(std::min<int32_t>(h->n_merges, 65535));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const zl_merge* dm = reinterpret_cast<const zl_merge*>(d_wl + h->merges_offset);
  if (h->head_dim == 128)
    hipLaunchKernelGGL(merge_list_kernel<128>, dim3(gx, gy), dim3(kThreads), 0, s, dm, h->n_merges,
                       ws_o, ws_lse, o, lse, h->num_heads);
  else
    hipLaunchKernelGGL(merge_list_kernel<64>, dim3(gx, gy), dim3(kThreads), 0, s, dm, h->n_merges,
                       ws_o, ws_lse, o, lse, h->num_heads);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZL_ERR_HIP, "split merge launch: %s", hipGetErrorString(e));
  return ZL_OK;
}

}  // namespace zl
