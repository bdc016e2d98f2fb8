// Backward of the coalesced attention for gfx950 (CDNA4), recomputing the
// probabilities from the forward's log-sum-exp.
//
// For every item and head, with s the softmax scale, P = exp(s q K^T - LSE):
//   D  = rowsum(dO * O)                              (bwd_preprocess)
//   dV += P^T dO,  dS = P * (dO V^T - D)
//   dK += s dS^T Q,  dQ += s dS K                     (bwd_kernel)
// The attention is the dense exact attention of the pith.science review of
// arXiv 2608.01150 ("Assumptions", Sec. II, after FlashAttention [7]); the
// work is split over key/value blocks, the axis a theta k split cuts ("What
// carries the argument").
//
// bwd_kernel: one tile = 128 keys of one item on one head, against all of the
// item's queries, 4 waves (one per SIMD) x 32 keys. A wave keeps its keys' K
// and V rows in registers (as the B operands of S = Q K^T and dP = dO V^T) and
// its dK^T and dV^T accumulators; the item's queries stream through LDS in
// steps of 64 rows (Q, dO, and their LSE and D), double-buffered with
// direct-to-LDS loads. Per step and wave:
//   S  = Q K^T, dP = dO V^T                    (A = Q / dO rows from LDS)
//   P  = exp2(S c - LSE2), dS = s P (dP - D)   (lane = key, registers = queries)
//   dV^T += dO^T P, dK^T += Q^T dS             (A = dO^T / Q^T transpose reads)
//   dS^T -> LDS, barrier
//   dQ[64 x 32-wide d slice] = dS K over all 128 keys -> fp32 atomics
// At the end dK^T / dV^T go through LDS to coalesced fp32 atomics (items may
// share key/value rows, whose gradients add up).

#include <hip/hip_runtime.h>

#include <cmath>

#include "zl.h"
#include "zl_device.h"
#include "zl_internal.h"

namespace {

using namespace zl::dev;

template <int D>
struct Bwd {
  static constexpr int kWaves = zl::kBwdWaves;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBN = zl::kBwdBlockN;  // keys per tile, 32 per wave
  static constexpr int kBM = zl::kBwdBlockM;  // query rows per step
  static constexpr int kQB = kBM / 32;
  static constexpr int kDS = D / 16;
  static constexpr int kDB = D / 32;
  // bf16 tiles with D columns use the forward's group layout: kG rows of
  // 1 KB stored chunk-column-major, each group padded by 16*kG bytes.
  static constexpr int kG = 512 / D;
  static constexpr int kGB = 1024 + 16 * kG;
  static constexpr int kQTile = (kBM / kG) * kGB;  // Q or dO rows of one step
  static constexpr int kKTile = (kBN / kG) * kGB;  // K rows of the tile
  // dS^T tile: kBN keys (rows) x kBM queries (columns), same scheme.
  static constexpr int kG2 = 512 / kBM;
  static constexpr int kGB2 = 1024 + 16 * kG2;
  static constexpr int kSTile = (kBN / kG2) * kGB2;
  static constexpr int kOffQ = 0;                   // 2 stages
  static constexpr int kOffDO = 2 * kQTile;         // 2 stages
  static constexpr int kOffK = 4 * kQTile;
  static constexpr int kOffS = kOffK + kKTile;
  static constexpr int kOffL = kOffS + kSTile;      // 2 stages x (LSE2[kBM], D[kBM]) fp32
  static constexpr int kLdsBytes = kOffL + 2 * 2 * kBM * 4;
  // dK^T / dV^T flush: [kBN][D] fp32 with a 16-byte row pad, over the Q/dO area
  static constexpr int kFlushPitch = D * 4 + 16;
  static constexpr int kUnits = kDB * kQB;           // dQ (d slice, query block) units
  static_assert(kBN == kWaves * 32 && kBM % 32 == 0, "shapes");
  static_assert(kBN * kFlushPitch <= 4 * kQTile, "flush buffer fits the Q/dO stages");
  static_assert(kUnits % kWaves == 0 || kWaves % kUnits == 0, "dQ units spread evenly");
};

// Byte offset of the 16-byte chunk holding (row, col) in a group-layout tile
// with G rows per group, GB bytes per group; col is a multiple of 8.
__device__ __forceinline__ int grp_off(int row, int col, int G, int GB) {
  return (row / G) * GB + ((col / 8) * G + row % G) * 16;
}

// ---------------------------------------------------------------- preprocess
// D[row, head] = sum_c dO[row, head, c] * O[row, head, c] over the forward
// tiles (256 rows x 1 head each): one thread per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess(const zl_tile* __restrict__ tiles,
                                                      const __bf16* __restrict__ dO,
                                                      const float* __restrict__ O,
                                                      float* __restrict__ Dws, int H) {
  const zl_tile t = uniform_tile(tiles[blockIdx.x]);
  const int r = threadIdx.x;
  if (r >= t.q_rows) return;
  const int64_t row = t.q_row0 + r;
  const __bf16* g = dO + (row * H + t.head) * D;
  const float* o = O + (row * H + t.head) * D;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D; c += 8) {
    const bf16x8 gv = *reinterpret_cast<const bf16x8*>(g + c);
    const f32x4 o0 = *reinterpret_cast<const f32x4*>(o + c);
    const f32x4 o1 = *reinterpret_cast<const f32x4*>(o + c + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(float(gv[e]), o0[e], acc);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = fmaf(float(gv[4 + e]), o1[e], acc);
  }
  Dws[row * H + t.head] = acc;
}

// ---------------------------------------------------------------- main
template <int D>
__device__ __forceinline__ void bwd_tile(const zl_tile& tile, const __bf16* __restrict__ Q,
                                         const __bf16* __restrict__ K,
                                         const __bf16* __restrict__ V,
                                         const __bf16* __restrict__ dO,
                                         const float* __restrict__ LSE,
                                         const float* __restrict__ Dws, float* __restrict__ dQ,
                                         float* __restrict__ dK, float* __restrict__ dV, int H,
                                         float scale, char ZL_LDS* smem) {
  using C = Bwd<D>;
  constexpr int DS = C::kDS, DB = C::kDB, QB = C::kQB, G = C::kG, GB = C::kGB;
  constexpr int G2 = C::kG2, GB2 = C::kGB2;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int64_t rs = int64_t(H) * D;
  const float c = scale * kLog2e;

  // ---- this lane's key: K^T / V^T operands (k = head_dim, j = key)
  const int key = wave * 32 + l32;
  const bool kvalid = key < tile.kv_len;
  bf16x8 kf[DS], vf[DS];
  {
    const int64_t kr = tile.kv_row0 + (kvalid ? key : 0);
    const __bf16* kp = K + kr * rs + int64_t(tile.head) * D + 8 * half;
    const __bf16* vp = V + kr * rs + int64_t(tile.head) * D + 8 * half;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kp + ds * 16);
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(vp + ds * 16);
      kf[ds] = kvalid ? a : bf16x8{};
      vf[ds] = kvalid ? b : bf16x8{};
    }
  }

  // ---- direct-to-LDS loads of `nrows` rows starting at packed row `row0`;
  // rows at or past `valid` read as zero. Lane l carries row l % G, chunk l / G
  // of a 1 KB group; wave w fills groups w, w + 4, ...
  const int ld_lane = (lane % G) * int(rs) * 2 + (lane / G) * 16;
  auto issue_rows = [&](const __bf16* base, int64_t row0, int valid, int nrows, int lds_off)
                        __attribute__((always_inline)) {
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(nrows, valid)));
    const int64_t addr = uniform_i64(reinterpret_cast<int64_t>(base + row0 * rs + int64_t(tile.head) * D));
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<__bf16*>(addr), 0,
                                                        rows * int(rs) * 2, kBufferFlags);
    for (int gi = wave; gi < nrows / G; gi += C::kWaves)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void ZL_LDS*)(smem + lds_off + gi * GB), 16,
                                               ld_lane,
                                               __builtin_amdgcn_readfirstlane(gi * G * int(rs) * 2),
                                               0, 0);
  };
  // LSE2 = LSE * log2 e (+inf past the item: P = 0) and D for a step, loaded
  // into registers by threads 0..2*kBM-1 and stored to LDS later.
  auto load_ld = [&](int step) __attribute__((always_inline)) {
    float x = 0.f;
    if (tid < 2 * C::kBM) {
      const int r = step * C::kBM + (tid % C::kBM);
      const int64_t idx = (tile.q_row0 + r) * H + tile.head;
      if (r < tile.q_rows)
        x = tid < C::kBM ? LSE[idx] * kLog2e : Dws[idx];
      else
        x = tid < C::kBM ? INFINITY : 0.f;
    }
    return x;
  };
  auto store_ld = [&](int stage, float x) __attribute__((always_inline)) {
    if (tid < 2 * C::kBM)
      *reinterpret_cast<float ZL_LDS*>(smem + C::kOffL + stage * 2 * C::kBM * 4 + tid * 4) = x;
  };

  // ---- per-lane LDS offsets
  // row reads (A of S and dP): row qb*32 + l32, chunk 2*ds + half
  const int a_lane = grp_off(l32, 8 * half, G, GB);
  // transpose reads of Q^T / dO^T (A of dK^T / dV^T): rows in the order the
  // S accumulator keeps them, 4*half + e and 8 + 4*half + e
  const int e_l = (lane & 15) >> 2;
  const int c_l = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tq_lane = ((4 * half + e_l) / G) * GB + (c_l * G + (4 * half + e_l) % G) * 16 + (lane & 1) * 8;
  // transpose reads in natural order (dQ GEMM): rows 8*half + e (+4)
  const int tk_lane = ((8 * half + e_l) / G) * GB + (c_l * G + (8 * half + e_l) % G) * 16 + (lane & 1) * 8;
  const int ts_lane = ((8 * half + e_l) / G2) * GB2 + (c_l * G2 + (8 * half + e_l) % G2) * 16 + (lane & 1) * 8;

  auto tr8 = [&](const char ZL_LDS* p0, const char ZL_LDS* p1) __attribute__((always_inline)) {
    const i16x4 lo = lds_read_tr16(p0);
    const i16x4 hi = lds_read_tr16(p1);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Row r0 + 8 in a group layout is (8 / G) groups and (8 % G) rows further.
  constexpr int kPlus8 = (8 / G) * GB + (8 % G) * 16;
  constexpr int kPlus4 = (4 / G) * GB + (4 % G) * 16;
  constexpr int kPlus4S = (4 / G2) * GB2 + (4 % G2) * 16;

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  const int nsteps = (tile.q_rows + C::kBM - 1) / C::kBM;
  // ---- prologue: K tile, step 0 of Q / dO / LSE / D
  issue_rows(K, tile.kv_row0, tile.kv_len, C::kBN, C::kOffK);
  issue_rows(Q, tile.q_row0, tile.q_rows, C::kBM, C::kOffQ);
  issue_rows(dO, tile.q_row0, tile.q_rows, C::kBM, C::kOffDO);
  store_ld(0, load_ld(0));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const bool ragged_keys = tile.kv_len < C::kBN;
  for (int step = 0; step < nsteps; ++step) {
    const int st = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) {
      const int64_t r1 = tile.q_row0 + int64_t(step + 1) * C::kBM;
      const int v1 = tile.q_rows - (step + 1) * C::kBM;
      issue_rows(Q, r1, v1, C::kBM, C::kOffQ + (st ^ 1) * C::kQTile);
      issue_rows(dO, r1, v1, C::kBM, C::kOffDO + (st ^ 1) * C::kQTile);
    }
    // issued after the direct loads: waiting for it waits for them too
    const float ld_next = more ? load_ld(step + 1) : 0.f;

    const char ZL_LDS* qs = smem + C::kOffQ + st * C::kQTile;
    const char ZL_LDS* gs = smem + C::kOffDO + st * C::kQTile;
    const char ZL_LDS* ls = smem + C::kOffL + st * 2 * C::kBM * 4;

    // ---- S = Q K^T and dP = dO V^T (lane = key, registers = queries)
    f32x16 s[QB], dp[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const int off = (qb * 32 / G) * GB + a_lane + ds * 2 * G * 16;
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(qs + off), kf[ds], s[qb], 0, 0, 0);
        dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(gs + off), vf[ds], dp[qb], 0, 0, 0);
      }
    }

    // ---- P and dS; register r holds query qb*32 + 8*(r/4) + 4*half + r%4
    bf16x8 pf[QB][2], sf[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qo = (qb * 32 + 8 * g + 4 * half) * 4;
        const f32x4 l2 = *reinterpret_cast<const f32x4 ZL_LDS*>(ls + qo);
        const f32x4 dd = *reinterpret_cast<const f32x4 ZL_LDS*>(ls + C::kBM * 4 + qo);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float p = __builtin_amdgcn_exp2f(fmaf(s[qb][r], c, -l2[e]));
          if (ragged_keys && !kvalid) p = 0.f;
          const float dsv = scale * p * (dp[qb][r] - dd[e]);
          pf[qb][r >> 3][r & 7] = (__bf16)p;
          sf[qb][r >> 3][r & 7] = (__bf16)dsv;
        }
      }
    }

    // ---- dV^T += dO^T P, dK^T += Q^T dS; k-slot e of operand (qb, u) in
    // half h is query qb*32 + 16u + 8(e/4) + 4h + e%4 (the S register order)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int off = ((qb * 32 + 16 * u) / G) * GB + tq_lane + db * 4 * G * 16;
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr8(gs + off, gs + off + kPlus8), pf[qb][u],
                                                           dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr8(qs + off, qs + off + kPlus8), sf[qb][u],
                                                           dk[db], 0, 0, 0);
        }

    // ---- dS^T -> LDS: row = key; elements 0-3 / 4-7 of sf[qb][u] are the
    // queries qb*32 + 16u + 4h .. +3 / qb*32 + 16u + 8 + 4h .. +3. The halves
    // are split with whole-vector shuffles: building the stored vector from
    // single bf16 elements is lowered to a lossy byte permute.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const i16x8 all = __builtin_bit_cast(i16x8, sf[qb][u]);
        const i16x4 lo = __builtin_shufflevector(all, all, 0, 1, 2, 3);
        const i16x4 hi = __builtin_shufflevector(all, all, 4, 5, 6, 7);
        const int off = grp_off(key, qb * 32 + 16 * u, G2, GB2) + half * 8;
        *reinterpret_cast<i16x4 ZL_LDS*>(smem + C::kOffS + off) = lo;
        *reinterpret_cast<i16x4 ZL_LDS*>(smem + C::kOffS + off + G2 * 16) = hi;  // next chunk
      }
    // The next step's direct loads were issued before this step's MFMAs; every
    // wave waits for its own before the barrier, so after it they are all in LDS.
    __builtin_amdgcn_s_waitcnt(kWaitLoads);
    __syncthreads();

    // ---- dQ = dS K for (d slice, query block) units, over all 128 keys
    const char ZL_LDS* ks = smem + C::kOffK;
    const char ZL_LDS* ss = smem + C::kOffS;
#pragma unroll
    for (int n = 0; n < (C::kUnits + C::kWaves - 1) / C::kWaves; ++n) {
      const int unit = wave + n * C::kWaves;
      if (C::kUnits % C::kWaves != 0 && unit >= C::kUnits) break;
      const int db = unit % DB, qb = unit / DB;
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < C::kBN / 16; ++kk) {
        const int koff = ((kk * 16) / G) * GB + tk_lane + db * 4 * G * 16;
        const int soff = ((kk * 16) / G2) * GB2 + ts_lane + qb * 4 * G2 * 16;
        const bf16x8 a = tr8(ss + soff, ss + soff + kPlus4S);
        const bf16x8 b = tr8(ks + koff, ks + koff + kPlus4);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      }
      // lane = d column db*32 + l32, register r = query qb*32 + 8(r/4) + 4h + r%4
      const int d = db * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qr = step * C::kBM + qb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (qr < tile.q_rows)
          atomicAdd(dQ + ((tile.q_row0 + qr) * H + tile.head) * D + d, acc[r]);
      }
    }
    if (more) store_ld(st ^ 1, ld_next);
    __syncthreads();
  }

  // ---- dK, dV: registers -> LDS [key][d] fp32 -> coalesced atomics
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  auto flush = [&](const f32x16 (&acc)[DB], float* __restrict__ out) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
        *reinterpret_cast<f32x4 ZL_LDS*>(smem + key * C::kFlushPitch + (db * 32 + 8 * g + 4 * half) * 4) = x;
      }
    __syncthreads();
    for (int idx = tid; idx < tile.kv_len * D; idx += C::kThreads) {
      const int kr = idx / D, col = idx % D;
      const float x = *reinterpret_cast<const float ZL_LDS*>(smem + kr * C::kFlushPitch + col * 4);
      atomicAdd(out + ((tile.kv_row0 + kr) * H + tile.head) * D + col, x);
    }
    __syncthreads();
  };
  flush(dk, dK);
  flush(dv, dV);
}

template <int D>
__global__ __launch_bounds__(Bwd<D>::kThreads, 1) void bwd_kernel(
    const zl_tile* __restrict__ tiles, const int32_t* __restrict__ slots, int n_slots,
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dws,
    float* __restrict__ dQ, float* __restrict__ dK, float* __restrict__ dV, int H, float scale) {
  __shared__ __attribute__((aligned(16))) char smem_raw[Bwd<D>::kLdsBytes];
  char ZL_LDS* smem = (char ZL_LDS*)(smem_raw);  // generic -> LDS address space
  int t0, t1;
  if (n_slots > 0) {
    // same XCD-aware slot mapping as the forward
    const int w = blockIdx.x;
    const int s = n_slots % kXcds == 0 ? (w % kXcds) * (n_slots / kXcds) + w / kXcds : w;
    t0 = slots[s];
    t1 = slots[s + 1];
  } else {
    t0 = blockIdx.x;
    t1 = t0 + 1;
  }
  t0 = __builtin_amdgcn_readfirstlane(t0);
  t1 = __builtin_amdgcn_readfirstlane(t1);
  for (int t = t0; t < t1; ++t) {
    const zl_tile tile = uniform_tile(tiles[t]);
    bwd_tile<D>(tile, Q, K, V, dO, LSE, Dws, dQ, dK, dV, H, scale, smem);
    __syncthreads();
  }
}

template <int D>
int launch_bwd(const zl_worklist_header* h, const char* d_wl, const void* q, const void* k,
               const void* v, const float* o, const float* lse, const void* dout, float* dq,
               float* dk, float* dv, float* d_ws, hipStream_t stream) {
  if (h->n_tiles > 0) {
    hipLaunchKernelGGL(bwd_preprocess<D>, dim3(h->n_tiles), dim3(256), 0, stream,
                       reinterpret_cast<const zl_tile*>(d_wl + h->tiles_offset),
                       static_cast<const __bf16*>(dout), o, d_ws, h->num_heads);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return zl::fail(ZL_ERR_HIP, "backward preprocess launch: %s", hipGetErrorString(e));
  }
  const int grid = h->n_slots > 0 ? h->n_slots : h->n_bwd_tiles;
  if (grid == 0 || h->n_bwd_tiles == 0) return ZL_OK;
  hipLaunchKernelGGL(bwd_kernel<D>, dim3(grid), dim3(Bwd<D>::kThreads), 0, stream,
                     reinterpret_cast<const zl_tile*>(d_wl + h->bwd_tiles_offset),
                     reinterpret_cast<const int32_t*>(d_wl + h->bwd_slots_offset), h->n_slots,
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), static_cast<const __bf16*>(dout), lse, d_ws,
                     dq, dk, dv, h->num_heads, h->softmax_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return zl::fail(ZL_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return ZL_OK;
}

}  // namespace

extern "C" int zl_coalesced_attn_bwd(const void* h_wl, const void* d_wl, const void* q,
                                     const void* k, const void* v, const float* o,
                                     const float* lse, const void* dout, float* dq, float* dk,
                                     float* dv, float* d_ws, void* stream) {
  zl::clear_error();
  const zl_worklist_header* h = nullptr;
  int rc = zl::check_worklist(h_wl, &h);
  if (rc) return rc;
  if (!d_wl || !q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !d_ws)
    return zl::fail(ZL_ERR_NULL, "device pointers must be non-NULL");
  const void* ptrs[] = {d_wl, q, k, v, o, lse, dout, dq, dk, dv, d_ws};
  for (const void* p : ptrs)
    if (!zl::aligned16(p)) return zl::fail(ZL_ERR_ALIGN, "device pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* dw = static_cast<const char*>(d_wl);
  return h->head_dim == 128 ? launch_bwd<128>(h, dw, q, k, v, o, lse, dout, dq, dk, dv, d_ws, s)
                            : launch_bwd<64>(h, dw, q, k, v, o, lse, dout, dq, dk, dv, d_ws, s);
}
