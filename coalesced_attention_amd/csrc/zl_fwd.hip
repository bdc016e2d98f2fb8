// Coalesced varlen attention forward for gfx950 (CDNA4).
//
// One launch runs every tile of a worklist: a tile is up to 256 query rows
// of one work item on one head, against that item's whole key range. Whole
// sequences and theta = (q, h, k) shards differ only in their row and head
// ranges, so they share the launch (newx.sg page "Zellige: Moldable
// Sequence Placement for Mixed Image-Video DiT Training", Abstract; shards
// per the pith.science review of arXiv 2608.01150, "What carries the
// argument"). The attention is exact softmax attention computed block by
// block with a running maximum and sum (the IO-aware exact method the
// review's "Assumptions" section cites as FlashAttention [7]).
//
// Work decomposition (per workgroup of 8 waves, one tile at a time):
//   - wave w owns query rows [32w, 32w+32) of the tile; lane l owns query
//     row l%32 and half h = l/32 of that row's keys in every 32-key block.
//   - scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in registers).
//     In the accumulator layout a lane then holds 16 keys of ONE query, so
//     the row max is an in-lane reduction plus one v_permlane32_swap, and
//     the running sum needs no exchange until the epilogue.
//   - the output is also accumulated transposed, O^T += V^T P^T (A = V^T read
//     from a row-major LDS tile with ds_read_b64_tr_b16, B = P^T straight
//     from the score registers converted to bf16), so the rescale factor of
//     a query multiplies registers of the same lane.
//   - K/V tiles of 64 keys are double-buffered in LDS; the next tile's
//     global loads are in flight while the current one is consumed.
//   - the running max is only raised when a row's new maximum exceeds the
//     one in use by more than 2^8 (in exp2 units): the probabilities are
//     then at most 256, the final O / l and LSE are unchanged in exact
//     arithmetic, and most blocks skip the O rescale.

#include <hip/hip_runtime.h>

#include <cmath>

#include "zl.h"
#include "zl_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define ZL_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int D>
struct Fwd {
  static constexpr int kWaves = zl::kFwdWaves;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBlockM = zl::kFwdBlockM;
  static constexpr int kBN = 64;              // keys per block
  static constexpr int kKB = kBN / 32;        // 32-key MFMA blocks per key block
  static constexpr int kDS = D / 16;          // 16-wide steps over head_dim
  static constexpr int kDB = D / 32;          // 32-wide output blocks over head_dim
  static constexpr int kKP = D * 2 + 16;      // K row pitch (bytes): 16-lane b128 reads hit distinct banks
  static constexpr int kVP = D * 2 + 64;      // V row pitch (bytes): 4-row transpose reads hit distinct banks
  static constexpr int kKBytes = kBN * kKP;
  static constexpr int kVBytes = kBN * kVP;
  static constexpr int kStage = kKBytes + kVBytes;
  static constexpr int kLdsBytes = 2 * kStage;
  static constexpr int kChunksPerRow = D / 8;  // 16-byte chunks per row
  static constexpr int kChunks = kBN * kChunksPerRow;
  static constexpr int kCPT = kChunks / kThreads;  // chunks per thread per tensor
  static_assert(kChunks % kThreads == 0, "tile load must divide evenly");
};

__device__ __forceinline__ float swap_halves_max(float x) {
  // v_permlane32_swap exchanges lanes l and l^32; one of the two results is
  // the lane's own value and the other its partner's.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float swap_halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const char ZL_LDS* p) {
  return *reinterpret_cast<const bf16x8 ZL_LDS*>(p);
}

__device__ __forceinline__ i16x4 lds_read_tr16(const char ZL_LDS* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<i16x4 ZL_LDS*>(const_cast<char ZL_LDS*>(p)));
}

template <int D>
__device__ __forceinline__ void run_tile(const zl_tile& tile, const __bf16* __restrict__ Q,
                                         const __bf16* __restrict__ K,
                                         const __bf16* __restrict__ V, float* __restrict__ O,
                                         float* __restrict__ LSE, int H, float c,
                                         char ZL_LDS* smem) {
  using C = Fwd<D>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int64_t rs = int64_t(H) * D;  // elements between consecutive rows

  // ---- Q^T fragments: query row `qr`, head_dim [ds*16 + 8*half, +8)
  const int qr = wave * 32 + l32;
  const bool qvalid = qr < tile.q_rows;
  bf16x8 qf[C::kDS];
  {
    const __bf16* qp = Q + (tile.q_row0 + (qvalid ? qr : 0)) * rs + int64_t(tile.head) * D + 8 * half;
#pragma unroll
    for (int ds = 0; ds < C::kDS; ++ds) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(qp + ds * 16);
      qf[ds] = qvalid ? x : bf16x8{};
    }
  }

  const int kv_len = tile.kv_len;
  const int nblk = (kv_len + C::kBN - 1) / C::kBN;
  const __bf16* kbase = K + tile.kv_row0 * rs + int64_t(tile.head) * D;
  const __bf16* vbase = V + tile.kv_row0 * rs + int64_t(tile.head) * D;

  u32x4 kreg[C::kCPT], vreg[C::kCPT];
  auto gload = [&](int blk) {
#pragma unroll
    for (int i = 0; i < C::kCPT; ++i) {
      const int ch = tid + i * C::kThreads;
      const int row = ch / C::kChunksPerRow, col = ch % C::kChunksPerRow;
      const int key = blk * C::kBN + row;
      if (key < kv_len) {
        kreg[i] = *reinterpret_cast<const u32x4*>(kbase + int64_t(key) * rs + col * 8);
        vreg[i] = *reinterpret_cast<const u32x4*>(vbase + int64_t(key) * rs + col * 8);
      } else {
        kreg[i] = u32x4{0, 0, 0, 0};
        vreg[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int stage) {
    char ZL_LDS* kb = smem + stage * C::kStage;
    char ZL_LDS* vb = kb + C::kKBytes;
#pragma unroll
    for (int i = 0; i < C::kCPT; ++i) {
      const int ch = tid + i * C::kThreads;
      const int row = ch / C::kChunksPerRow, col = ch % C::kChunksPerRow;
      *reinterpret_cast<u32x4 ZL_LDS*>(kb + row * C::kKP + col * 16) = kreg[i];
      *reinterpret_cast<u32x4 ZL_LDS*>(vb + row * C::kVP + col * 16) = vreg[i];
    }
  };

  f32x16 oacc[C::kDB];
#pragma unroll
  for (int i = 0; i < C::kDB; ++i) oacc[i] = f32x16{};
  float m_use = -INFINITY;  // running max in use, in exp2 units (score * c)
  float l_part = 0.f;       // this lane's partial row sum (its half of the keys)

  if (nblk > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  // Per-lane byte offsets inside a stage.
  const int k_off = l32 * C::kKP + half * 16;
  const int tr_row = 4 * half + ((lane & 15) >> 2);
  const int tr_col = (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;

  for (int j = 0; j < nblk; ++j) {
    if (j + 1 < nblk) gload(j + 1);
    const char ZL_LDS* kb = smem + (j & 1) * C::kStage;
    const char ZL_LDS* vb = kb + C::kKBytes;

    // ---- S^T = K Q^T for 64 keys x 32 queries
    f32x16 s[C::kKB];
#pragma unroll
    for (int b = 0; b < C::kKB; ++b) {
      s[b] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < C::kDS; ++ds) {
        bf16x8 a = lds_read_b128(kb + b * 32 * C::kKP + k_off + ds * 32);
        s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], s[b], 0, 0, 0);
      }
    }

    // ---- mask keys past the item's end (last block only)
    if ((j + 1) * C::kBN > kv_len) {
#pragma unroll
      for (int b = 0; b < C::kKB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * C::kBN + b * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= kv_len) s[b][r] = -INFINITY;
        }
    }

    // ---- row max over the block, both halves
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < C::kKB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
    mx = swap_halves_max(mx) * c;

    // ---- raise the max in use only when it grew by more than the slack
    if (mx > m_use + kRescaleSlack) {
      const float alpha = __builtin_amdgcn_exp2f(m_use - mx);
      m_use = mx;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < C::kDB; ++i) oacc[i] *= alpha;
    }

    // ---- P = exp2(S c - m), partial row sums, bf16 B operands
    bf16x8 pf[C::kKB][2];
    float lsum = 0.f;
#pragma unroll
    for (int b = 0; b < C::kKB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[b][r], c, -m_use));
        lsum += p;
        pf[b][r >> 3][r & 7] = (__bf16)p;
      }
    l_part += lsum;

    // ---- O^T += V^T P^T
    // k-slot e of the B operand (b, u) in half `half` holds key
    // b*32 + 16u + 8(e/4) + 4*half + e%4: the lane's own registers 8u..8u+7.
    // The A operand reads the same keys of V transposed, 4 keys per read.
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int b = 0; b < C::kKB; ++b)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const char ZL_LDS* vp = vb + (b * 32 + 16 * u + tr_row) * C::kVP + db * 64 + tr_col;
          const i16x4 lo = lds_read_tr16(vp);
          const i16x4 hi = lds_read_tr16(vp + 8 * C::kVP);
          // whole-vector concatenation: per-element inserts of bf16 lanes
          // were lowered to a lossy permute by the compiler
          const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 a = __builtin_bit_cast(bf16x8, cat);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[b][u], oacc[db], 0, 0, 0);
        }

    if (j + 1 < nblk) lstore((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l)
  const float l_tot = swap_halves_sum(l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? kLn2 * (m_use + __builtin_amdgcn_logf(l_tot)) : -INFINITY;
  if (qvalid) {
    float* op = O + (tile.q_row0 + qr) * rs + int64_t(tile.head) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < C::kDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 x = {oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                   oacc[db][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(op + db * 32 + 8 * g) = x;
      }
    if (half == 0) LSE[(tile.q_row0 + qr) * H + tile.head] = lse;
  }
}

template <int D>
__global__ __launch_bounds__(Fwd<D>::kThreads, 1) void fwd_kernel(
    const zl_tile* __restrict__ tiles, const int32_t* __restrict__ slots, int n_slots,
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int H, float c) {
  __shared__ __attribute__((aligned(16))) char smem_raw[Fwd<D>::kLdsBytes];
  char ZL_LDS* smem = (char ZL_LDS*)(smem_raw);  // generic -> LDS address space
  int t0, t1;
  if (n_slots > 0) {
    t0 = slots[blockIdx.x];
    t1 = slots[blockIdx.x + 1];
  } else {
    t0 = blockIdx.x;
    t1 = t0 + 1;
  }
  for (int t = t0; t < t1; ++t) {
    const zl_tile tile = tiles[t];
    run_tile<D>(tile, Q, K, V, O, LSE, H, c, smem);
    __syncthreads();  // LDS is reused by the next tile
  }
}

template <int D>
int launch_fwd(const zl_worklist_header* h, const char* d_wl, const void* q, const void* k,
               const void* v, float* o, float* lse, hipStream_t stream) {
  const int grid = h->n_slots > 0 ? h->n_slots : h->n_tiles;
  if (grid == 0 || h->n_tiles == 0) return ZL_OK;
  const float c = h->softmax_scale * kLog2e;
  hipLaunchKernelGGL(fwd_kernel<D>, dim3(grid), dim3(Fwd<D>::kThreads), 0, stream,
                     reinterpret_cast<const zl_tile*>(d_wl + h->tiles_offset),
                     reinterpret_cast<const int32_t*>(d_wl + h->slots_offset), h->n_slots,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), o, lse, h->num_heads, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return zl::fail(ZL_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return ZL_OK;
}

}  // namespace

extern "C" int zl_coalesced_attn_fwd(const void* h_wl, const void* d_wl, const void* q,
                                     const void* k, const void* v, float* o, float* lse,
                                     void* stream) {
  zl::clear_error();
  const zl_worklist_header* h = nullptr;
  int rc = zl::check_worklist(h_wl, &h);
  if (rc) return rc;
  if (!d_wl || !q || !k || !v || !o || !lse)
    return zl::fail(ZL_ERR_NULL, "device pointers must be non-NULL");
  if (!zl::aligned16(d_wl) || !zl::aligned16(q) || !zl::aligned16(k) || !zl::aligned16(v) ||
      !zl::aligned16(o) || !zl::aligned16(lse))
    return zl::fail(ZL_ERR_ALIGN, "device pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* dw = static_cast<const char*>(d_wl);
  return h->head_dim == 128 ? launch_fwd<128>(h, dw, q, k, v, o, lse, s)
                            : launch_fwd<64>(h, dw, q, k, v, o, lse, s);
}
