// Backward of the coalesced attention for gfx950 (CDNA4), recomputing the
// probabilities from the forward's log-sum-exp.
//
// For every item and head, with s the softmax scale, P = exp(s q K^T - LSE):
//   D  = rowsum(dO * O),  dS = s P (dO V^T - D)
//   dQ += dS K                       (dq_kernel, one owner per query row)
//   dV += P^T dO,  dK += dS^T Q      (dkdv_kernel, one owner per key block)
// The attention is the dense exact attention of the pith.science review of
// arXiv 2608.01150 ("Assumptions", Sec. II, after FlashAttention [7]); the
// dK/dV work is split over key/value blocks, the axis a theta k split cuts
// ("What carries the argument").
//
// Two kernels, no atomics on dQ: S and dP are recomputed by both (7 GEMMs in
// all instead of 5), which costs less than summing a partial dQ from every
// key block through device-scope fp32 atomics, and makes dQ deterministic.
//
// dq_kernel runs the forward's tiles (up to 256 query rows of one item on one
// head, 8 waves x 32 rows) with the forward's layout (64-key LDS tiles): per
// 32-key half-block,
//   S^T = K Q^T, dP^T = V dO^T       (A = K / V rows from LDS, B = Q^T / dO^T
//                                     held in registers; lane = query)
//   dS^T = s P^T (dP^T - D)          (in the accumulator registers)
//   dQ^T += K^T dS^T                 (A = K^T transpose reads, B = dS^T)
// software-pipelined over the halves: the dS arithmetic of one half runs
// beside the S / dP MFMAs of the next and the dQ MFMAs of the previous.
// It also computes D for its rows and stores it for dkdv_kernel.
//
// dkdv_kernel: one tile = 256 keys of one item on one head, against all of
// the item's queries, streamed through LDS 32 rows at a time (Q, dO, LSE, D;
// direct-to-LDS loads, a 4-step ring, two steps ahead). Each of the 8 waves
// (two per SIMD) owns 32 keys and runs all four products for them:
//   S = Q K^T, dP = dO V^T          (A = Q / dO rows from LDS; B = the wave's
//                                    K rows held in registers, V rows read
//                                    from the tile's V staged once in LDS;
//                                    lane = key)
//   P = exp2(S c - LSE log2 e), dS = P (s dP - s D), packed to bf16 in place
//   dV^T += dO^T P, dK^T += Q^T dS  (A = dO^T / Q^T transpose reads whose
//                                    query order matches the accumulator's)
// so no operand leaves the wave, and the exponentials of one wave run beside
// the MFMAs of the other wave on its SIMD. One barrier per two steps. At the end
// dK^T / dV^T go through LDS to coalesced fp32 atomics (items may share
// key/value rows, whose gradients add up).

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
  static constexpr int kDS = D / 16;
  static constexpr int kDB = D / 32;
  // bf16 tiles with D columns use the forward's group layout: kG rows of
  // 1 KB stored chunk-column-major, each group padded by 16*kG bytes.
  static constexpr int kG = 512 / D;
  static constexpr int kGB = 1024 + 16 * kG;
  static constexpr int kQGroups = kBM / kG;           // groups of one step's Q (or dO)
  static constexpr int kQTile = kQGroups * kGB;
  static constexpr int kRing = 4;                     // steps held in LDS
  static constexpr int kOffQ = 0;                     // kRing stages
  static constexpr int kOffDO = kRing * kQTile;       // kRing stages
  static constexpr int kLSlot = 512;                  // LSE[64] then D[64], fp32
  static constexpr int kOffL = 2 * kRing * kQTile;    // kRing slots
  static constexpr int kVGroups = kBN / kG;           // the tile's V rows
  static constexpr int kOffV = kOffL + kRing * kLSlot;
  static constexpr int kLdsBytes = kOffV + kVGroups * kGB;
  // per wave and step: Q and dO groups spread over all waves, and one more
  // load (LSE or D) on the last two waves; per wave and tile: its share of V
  static constexpr int kLoadsPerWave = 2 * kQGroups / kWaves;
  static constexpr int kVLoadsPerWave = kVGroups / kWaves;
  // dK^T / dV^T flush: [kBN][D] fp32 with a 16-byte row pad, over the whole LDS
  static constexpr int kFlushPitch = D * 4 + 16;
  static_assert(kBN == kWaves * 32 && kBM == 32, "shapes");
  static_assert((2 * kQGroups) % kWaves == 0 && kVGroups % kWaves == 0, "loads spread evenly");
  static_assert(kBN * kFlushPitch <= kLdsBytes, "flush buffer fits the LDS");
};

// dq_kernel: the forward's tile shape and LDS layout, 64-key blocks.
template <int D>
struct BwdQ {
  static constexpr int kWaves = zl::kFwdWaves;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBN = 64;
  static constexpr int kDS = D / 16;
  static constexpr int kDB = D / 32;
  static constexpr int kG = 512 / D;
  static constexpr int kGB = 1024 + 16 * kG;
  static constexpr int kGroups = kBN / kG;
  static constexpr int kTileBytes = kGroups * kGB;
  // The key loop runs over 32-key halves of the 64-key LDS tiles. K(x) is
  // last read by the dQ of half (x, 1), which runs in half (x+1, 0), and V(x)
  // by the S, dP of half (x, 1), which run in half (x, 0). The barrier between
  // the halves of block J publishes block J+1 and issues K(J+3), V(J+3), into
  // the stages of K(J-1) and V(J).
  static constexpr int kKStages = 4;
  static constexpr int kVStages = 3;
  static constexpr int kAhead = 3;
  static_assert(kAhead == kKStages - 1 && kAhead == kVStages, "stage reuse distance");
  static constexpr int kLdsBytes = (kKStages + kVStages) * kTileBytes;
  static constexpr int kGroupsPerWave = (kGroups + kWaves - 1) / kWaves;
  static_assert(zl::kFwdBlockM == kWaves * 32, "forward tiles hold 32 rows per wave");
};

// ---------------------------------------------------------------- dQ
template <int D>
__device__ __forceinline__ void dq_tile(const zl_tile& tile, const __bf16* __restrict__ Q,
                                        const __bf16* __restrict__ K,
                                        const __bf16* __restrict__ V,
                                        const __bf16* __restrict__ dO,
                                        const float* __restrict__ O,
                                        const float* __restrict__ LSE, float* __restrict__ Dws,
                                        float* __restrict__ dQ, int H, float scale,
                                        char ZL_LDS* smem) {
  using C = BwdQ<D>;
  constexpr int DS = C::kDS, DB = C::kDB, G = C::kG, GB = C::kGB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int64_t rs = int64_t(H) * D;
  const float c = scale * kLog2e;

  // ---- this lane's query row: Q^T and dO^T fragments (head_dim
  // [ds*16 + 8*half, +8)), s * D with D = rowsum(dO * O), and LSE in exp2 units
  const int qr = wave * 32 + l32;
  const bool qvalid = qr < tile.q_rows;
  const int64_t row = tile.q_row0 + (qvalid ? qr : 0);
  bf16x8 qf[DS], gf[DS];
  float dpart = 0.f;
  {
    const int64_t off = row * rs + int64_t(tile.head) * D + 8 * half;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(Q + off + ds * 16);
      const bf16x8 g = *reinterpret_cast<const bf16x8*>(dO + off + ds * 16);
      const f32x4 o0 = *reinterpret_cast<const f32x4*>(O + off + ds * 16);
      const f32x4 o1 = *reinterpret_cast<const f32x4*>(O + off + ds * 16 + 4);
      qf[ds] = qvalid ? x : bf16x8{};
      gf[ds] = qvalid ? g : bf16x8{};
#pragma unroll
      for (int e = 0; e < 4; ++e) dpart = fmaf(float(g[e]), o0[e], dpart);
#pragma unroll
      for (int e = 0; e < 4; ++e) dpart = fmaf(float(g[4 + e]), o1[e], dpart);
    }
  }
  // sD = s * D: dS = s P (dP - D) = P (s dP - sD) is then one fma and a multiply
  const float drow = qvalid ? scale * swap_halves_sum(dpart) : 0.f;
  const float l2 = qvalid ? LSE[row * H + tile.head] * kLog2e : INFINITY;
  if (qvalid && half == 0) Dws[row * H + tile.head] = drow;

  const int kv_len = tile.kv_len;
  const int nblk = (kv_len + C::kBN - 1) / C::kBN;
  const __bf16* kbase = K + tile.kv_row0 * rs + int64_t(tile.head) * D;
  const __bf16* vbase = V + tile.kv_row0 * rs + int64_t(tile.head) * D;

  // ---- direct-to-LDS loads of key block `blk` (rows past kv_len, and every
  // row of block -1, read as 0)
  const int ld_lane = (lane % G) * int(rs) * 2 + (lane / G) * 16;
  const int row_bytes = __builtin_amdgcn_readfirstlane(int(rs) * 2);
  auto issue_tile = [&](const __bf16* base, int stage_off, int blk) __attribute__((always_inline)) {
    // keys of the block inside the item, on the scalar unit: the opaque
    // step keeps the clamp from becoming a vector med3
    int rows = kv_len - blk * C::kBN;
    rows = rows < C::kBN ? rows : C::kBN;
    asm volatile("" : "+s"(rows));
    rows = (blk < 0 || rows < 0) ? 0 : rows;
    const int64_t addr = uniform_i64(reinterpret_cast<int64_t>(base + int64_t(max(blk, 0)) * C::kBN * rs));
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<__bf16*>(addr), 0,
                                                        rows * row_bytes, kBufferFlags);
#pragma unroll
    for (int i = 0; i < C::kGroupsPerWave; ++i) {
      const int gi = wave * C::kGroupsPerWave + i;
      if (C::kGroups % (C::kWaves * C::kGroupsPerWave) != 0 && gi >= C::kGroups) break;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (void ZL_LDS*)(smem + stage_off + gi * GB), 16, ld_lane,
          __builtin_amdgcn_readfirstlane(gi * G * int(rs) * 2), 0, 0);
    }
  };
  constexpr int kLoadsPerTile = C::kGroupsPerWave;
  auto kstage = [&](int blk) { return ((blk + C::kKStages) % C::kKStages) * C::kTileBytes; };
  auto vstage = [&](int blk) { return (C::kKStages + blk % C::kVStages) * C::kTileBytes; };

  // row fragment (A of S^T and dP^T): row b*32 + l32, chunk 2*ds + half
  const int r_lane = (l32 / G) * GB + (half * G + l32 % G) * 16;
  // K^T fragment by transpose reads (A of dQ^T), as the forward's V^T
  const int rr = 4 * half + ((lane & 15) >> 2);
  const int c_l = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int t_lane = (rr / G) * GB + (c_l * G + rr % G) * 16 + (lane & 1) * 8;
  auto opaque = [&](int a) __attribute__((always_inline)) {
    asm volatile("" : "+v"(a));
    return (const char ZL_LDS*)(smem + a);
  };
  auto read_row = [&](const char ZL_LDS* base, int b, int ds) __attribute__((always_inline)) {
    return lds_read_b128(base + (b * 32 / G) * GB + ds * 2 * G * 16);
  };
  auto read_tr = [&](const char ZL_LDS* base, int b, int u, int db) __attribute__((always_inline)) {
    const char ZL_LDS* p = base + ((b * 32 + 16 * u) / G) * GB + db * 4 * G * 16;
    const i16x4 lo = lds_read_tr16(p);
    const i16x4 hi = lds_read_tr16(p + (8 / G) * GB + (8 % G) * 16);  // 8 rows further
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 dq[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) dq[i] = f32x16{};

  if (nblk > 0) {
    // ---- software pipeline over 32-key halves t = 2J + h of the key blocks.
    // Half t computes, in two windows of 16 keys each,
    //   dS(t) from S(t), dP(t)                          (VALU)
    //   S(t+1) = K Q^T, dP(t+1) = V dO^T                 (MFMA, K/V rows)
    //   dQ^T += K(t-1)^T dS(t-1)                         (MFMA, K transpose reads)
    // so the exponentials of one half run beside the MFMAs of its neighbours.
    // The prologue loads a zero block -1 for the empty dQ of half 0.
    issue_tile(kbase, kstage(-1), -1);
#pragma unroll
    for (int b = 0; b < C::kAhead; ++b) {
      issue_tile(kbase, kstage(b), b);
      issue_tile(vbase, vstage(b), b);
    }
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(4 * kLoadsPerTile));  // K(-1), K(0), V(0) landed
    lds_barrier();
    f32x16 s_a = f32x16{}, d_a = f32x16{}, s_b, d_b;
    bf16x8 x_a[2], x_b[2] = {bf16x8{}, bf16x8{}};
    {
      const char ZL_LDS* kr = opaque(kstage(0) + r_lane);
      const char ZL_LDS* vr = opaque(vstage(0) + r_lane);
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        s_a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row(kr, 0, ds), qf[ds], s_a, 0, 0, 0);
        d_a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_row(vr, 0, ds), gf[ds], d_a, 0, 0, 0);
      }
    }
    const bool ragged = (kv_len % C::kBN) != 0;
    // half (J, h): S(t), dP(t) in sc, dc; S(t+1), dP(t+1) into sn, dn; dS(t)
    // into xc; dS(t-1) from xp
    auto half_step = [&](int J, int h, f32x16& sc, const f32x16& dc, f32x16& sn, f32x16& dn,
                         bf16x8 (&xc)[2], const bf16x8 (&xp)[2]) __attribute__((always_inline)) {
      const int jn = h ? J + 1 : J, bn = h ? 0 : 1;  // block and half of t+1
      const int jp = h ? J : J - 1, bp = h ? 0 : 1;  // block and half of t-1
      const char ZL_LDS* kr = opaque(kstage(jn) + r_lane);
      const char ZL_LDS* vr = opaque(vstage(jn) + r_lane);
      const char ZL_LDS* kt = opaque(kstage(jp) + t_lane);
      // Keys at or past kv_len (only in the last block) get a score of -inf,
      // so P = 0 there. Their K rows are zero, but P = exp2(-LSE log2 e)
      // could still overflow for a row with a very negative LSE.
      if (ragged && J + 1 == nblk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = J * C::kBN + h * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= kv_len) sc[r] = -INFINITY;
        }
      }
      // four windows (u, q): elements 4q..4q+3 of operand u, a quarter of
      // the S / dP d-steps and half of the dQ column blocks each
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        u32x4 packed;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          constexpr int NS = DS / 4, NQ = DB / 2;
          bf16x8 kf[NS], vf[NS], tf[NQ];
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            kf[i] = read_row(kr, bn, u * (DS / 2) + q * NS + i);
            vf[i] = read_row(vr, bn, u * (DS / 2) + q * NS + i);
          }
#pragma unroll
          for (int i = 0; i < NQ; ++i) tf[i] = read_tr(kt, bp, u, q * NQ + i);
          // k-slot e of operand u is key 32h + 16u + 8(e/4) + 4*half + e%4
          float ds4[4];
#pragma unroll
          for (int e4 = 0; e4 < 4; ++e4) {
            const int r = 8 * u + 4 * q + e4;
            const float p = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -l2));
            ds4[e4] = fmaf(dc[r], scale, -drow) * p;
          }
          packed[2 * q] = pack_bf16x2(ds4[0], ds4[1]);
          packed[2 * q + 1] = pack_bf16x2(ds4[2], ds4[3]);
          pin(packed[2 * q]);
          pin(packed[2 * q + 1]);
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            const int ds = u * (DS / 2) + q * NS + i;
            sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[ds], ds == 0 ? f32x16{} : sn, 0, 0, 0);
            dn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], gf[ds], ds == 0 ? f32x16{} : dn, 0, 0, 0);
          }
#pragma unroll
          for (int i = 0; i < NQ; ++i)
            dq[q * NQ + i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[i], xp[u], dq[q * NQ + i], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        xc[u] = __builtin_bit_cast(bf16x8, packed);
      }
    };
    for (int J = 0; J < nblk; ++J) {
      half_step(J, 0, s_a, d_a, s_b, d_b, x_a, x_b);
      // K(J+1), V(J+1) landed: only the two loads of the previous barrier may fly
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(2 * kLoadsPerTile));
      lds_barrier();
      issue_tile(kbase, kstage(J + C::kAhead), J + C::kAhead);
      issue_tile(vbase, vstage(J + C::kAhead), J + C::kAhead);
      half_step(J, 1, s_b, d_b, s_a, d_a, x_b, x_a);
    }
    // ---- drain: dQ^T += K(nblk-1, half 1)^T dS
    const char ZL_LDS* kt = opaque(kstage(nblk - 1) + t_lane);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr(kt, 1, u, db), x_b[u], dq[db], 0, 0, 0);
  }

  // ---- dQ += dQ^T (lane = query, register r = d db*32 + 8(r/4) + 4*half + r%4);
  // the tile is the only writer of these (row, head) pairs
  if (qvalid) {
    float* qp = dQ + row * rs + int64_t(tile.head) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4* p = reinterpret_cast<f32x4*>(qp + db * 32 + 8 * g);
        const f32x4 a = {dq[db][4 * g], dq[db][4 * g + 1], dq[db][4 * g + 2], dq[db][4 * g + 3]};
        *p = *p + a;
      }
  }
}

template <int D>
__global__ __launch_bounds__(BwdQ<D>::kThreads, 1) void dq_kernel(
    const zl_tile* __restrict__ tiles, const int32_t* __restrict__ slots, int n_slots,
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ Dws, float* __restrict__ dQ, int H, float scale) {
  __shared__ __attribute__((aligned(16))) char smem_raw[BwdQ<D>::kLdsBytes];
  char ZL_LDS* smem = (char ZL_LDS*)(smem_raw);
  int t0, t1;
  if (n_slots > 0) {
    // the forward's XCD-aware slot mapping: the query blocks of one (item,
    // head), which read the same K/V, share an L2
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
    dq_tile<D>(tile, Q, K, V, dO, O, LSE, Dws, dQ, H, scale, smem);
    __builtin_amdgcn_s_waitcnt(0);  // the zero-filled prefetches of blocks past the end
    __syncthreads();
  }
}

// ---------------------------------------------------------------- main
template <int D>
__device__ __forceinline__ void dkdv_tile(const zl_tile& tile, const __bf16* __restrict__ Q,
                                          const __bf16* __restrict__ K,
                                          const __bf16* __restrict__ V,
                                          const __bf16* __restrict__ dO,
                                          const float* __restrict__ LSE,
                                          const float* __restrict__ Dws, float* __restrict__ dK,
                                          float* __restrict__ dV, int H, float scale,
                                          char ZL_LDS* smem) {
  using C = Bwd<D>;
  constexpr int DS = C::kDS, DB = C::kDB, G = C::kG, GB = C::kGB;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int64_t rs = int64_t(H) * D;
  const int nsteps = (tile.q_rows + C::kBM - 1) / C::kBM;
  const float c = scale * kLog2e;

  // ---- direct-to-LDS loads of step `step`: Q and dO rows (rows at or past
  // the item's end read as zero), and on waves 6 / 7 the LSE / D values
  const int ld_lane = (lane % G) * int(rs) * 2 + (lane / G) * 16;
  const int l_lane = lane * H * 4;
  auto issue_step = [&](int step) __attribute__((always_inline)) {
    const int slot = step % C::kRing;
    const int valid = tile.q_rows - step * C::kBM;
    const int64_t row0 = tile.q_row0 + int64_t(step) * C::kBM;
#pragma unroll
    for (int i = 0; i < C::kLoadsPerWave; ++i) {
      const int gi = wave + i * C::kWaves;  // over [Q groups, dO groups]
      const bool is_q = gi < C::kQGroups;
      const int g = is_q ? gi : gi - C::kQGroups;
      const __bf16* base = (is_q ? Q : dO) + row0 * rs + int64_t(tile.head) * D;
      const int64_t addr = uniform_i64(reinterpret_cast<int64_t>(base));
      const int rows = __builtin_amdgcn_readfirstlane(min(C::kBM, valid));
      const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<__bf16*>(addr), 0,
                                                          rows * int(rs) * 2, kBufferFlags);
      const int off = (is_q ? C::kOffQ : C::kOffDO) + slot * C::kQTile + g * GB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void ZL_LDS*)(smem + off), 16, ld_lane,
                                               __builtin_amdgcn_readfirstlane(g * G * int(rs) * 2),
                                               0, 0);
    }
    if (wave >= C::kWaves - 2) {
      const bool is_lse = wave == C::kWaves - 2;
      const float* base = (is_lse ? LSE : Dws) + row0 * H + tile.head;
      const int64_t addr = uniform_i64(reinterpret_cast<int64_t>(base));
      const int rows = __builtin_amdgcn_readfirstlane(min(64, valid));
      const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<float*>(addr), 0,
                                                          rows * H * 4, kBufferFlags);
      const int off = C::kOffL + slot * C::kLSlot + (is_lse ? 0 : 256);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void ZL_LDS*)(smem + off), 4, l_lane,
                                               0, 0, 0);
    }
  };
  // ---- this lane's key: K row in registers (B of S = Q K^T: k = head_dim,
  // j = key), V rows of the whole tile in LDS (B of dP = dO V^T)
  const int key = wave * 32 + l32;
  const bool kvalid = key < tile.kv_len;
  bf16x8 kf[DS];
  {
    const int64_t kr = tile.kv_row0 + (kvalid ? key : 0);
    const int64_t off = kr * rs + int64_t(tile.head) * D + 8 * half;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(K + off + ds * 16);
      kf[ds] = kvalid ? a : bf16x8{};
    }
  }
  {
    const __bf16* base = V + tile.kv_row0 * rs + int64_t(tile.head) * D;
    const int64_t addr = uniform_i64(reinterpret_cast<int64_t>(base));
    const int rows = __builtin_amdgcn_readfirstlane(min(C::kBN, tile.kv_len));
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<__bf16*>(addr), 0,
                                                        rows * int(rs) * 2, kBufferFlags);
#pragma unroll
    for (int i = 0; i < C::kVLoadsPerWave; ++i) {
      const int g = wave * C::kVLoadsPerWave + i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (void ZL_LDS*)(smem + C::kOffV + g * GB), 16,
                                               ld_lane,
                                               __builtin_amdgcn_readfirstlane(g * G * int(rs) * 2),
                                               0, 0);
    }
  }
  // prologue: V, steps 0 and 1. The workgroup meets after every odd step:
  // that barrier waits for every load issued so far, i.e. the rows of the
  // next two steps. Step x's loads go out at the top of step x - 2 into the
  // ring slot of step x - 4, whose last readers finished before the barrier
  // that follows step x - 4 or x - 3, whichever is odd.
  issue_step(0);
  if (nsteps > 1) issue_step(1);
  __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  lds_barrier();

  // row reads (A of S and dP, B of dP): row l32, chunk 2*ds + half
  const int a_lane = (l32 / G) * GB + (half * G + l32 % G) * 16;
  const int v_lane = C::kOffV + (wave * 32 / G) * GB + a_lane;
  // transpose reads of Q^T / dO^T (A of dK^T / dV^T): rows in the order the
  // S accumulator keeps them, 4*half + e and 8 + 4*half + e
  const int e_l = (lane & 15) >> 2;
  const int c_l = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int tq_lane = ((4 * half + e_l) / G) * GB + (c_l * G + (4 * half + e_l) % G) * 16 + (lane & 1) * 8;
  constexpr int kPlus8 = (8 / G) * GB + (8 % G) * 16;  // 8 rows further
  auto tr8 = [&](int a) __attribute__((always_inline)) {
    const i16x4 lo = lds_read_tr16(smem + a);
    const i16x4 hi = lds_read_tr16(smem + a + kPlus8);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  for (int j = 0; j < nsteps; ++j) {
    const bool issue = j + 2 < nsteps;
    if (issue) issue_step(j + 2);
    const int slot = j % C::kRing;
    int qa = C::kOffQ + slot * C::kQTile + a_lane;
    int ga = C::kOffDO + slot * C::kQTile + a_lane;
    int va = v_lane;
    asm volatile("" : "+v"(qa), "+v"(ga), "+v"(va));
    // S = Q K^T, dP = dO V^T (lane = key; register r holds query 8*(r/4) + 4*half + r%4)
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(smem + qa + ds * 2 * G * 16), kf[ds], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read_b128(smem + ga + ds * 2 * G * 16),
                                                   lds_read_b128(smem + va + ds * 2 * G * 16), dp, 0, 0, 0);
    }
    // P = exp2(S c - LSE log2 e), dS = P (s dP - s D), packed as the B operands
    // of dV^T += dO^T P and dK^T += Q^T dS. Keys at or past kv_len have zero
    // K / V rows; their P and dS only reach dV / dK columns of those keys,
    // which are not stored.
    const char ZL_LDS* ls = smem + C::kOffL + slot * C::kLSlot;
    u32x4 pk[2], sk[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 lse = *reinterpret_cast<const f32x4 ZL_LDS*>(ls + (8 * g + 4 * half) * 4);
      const f32x4 dd = *reinterpret_cast<const f32x4 ZL_LDS*>(ls + 256 + (8 * g + 4 * half) * 4);
      float p[4], d[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = __builtin_amdgcn_exp2f(fmaf(s[4 * g + e], c, -lse[e] * kLog2e));
        d[e] = fmaf(dp[4 * g + e], scale, -dd[e]) * p[e];
      }
      pk[g >> 1][2 * (g & 1)] = pack_bf16x2(p[0], p[1]);
      pk[g >> 1][2 * (g & 1) + 1] = pack_bf16x2(p[2], p[3]);
      sk[g >> 1][2 * (g & 1)] = pack_bf16x2(d[0], d[1]);
      sk[g >> 1][2 * (g & 1) + 1] = pack_bf16x2(d[2], d[3]);
    }
    int qt = C::kOffQ + slot * C::kQTile + tq_lane;
    int gt = C::kOffDO + slot * C::kQTile + tq_lane;
    asm volatile("" : "+v"(qt), "+v"(gt));
    // k-slot e of operand u in half h is query 16u + 8(e/4) + 4h + e%4
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pk[u]);
      const bf16x8 sf = __builtin_bit_cast(bf16x8, sk[u]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int off = ((16 * u) / G) * GB + db * 4 * G * 16;
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr8(gt + off), pf, dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr8(qt + off), sf, dk[db], 0, 0, 0);
      }
    }
    if (j & 1) {
      __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
      lds_barrier();
    }
  }
  lds_barrier();  // every wave is done with the ring and V

  // ---- dK^T then dV^T -> LDS [key][d] fp32 (over the whole LDS, no longer
  // read; register r of block db is d = db*32 + 8(r/4) + 4*half + r%4), then
  // every thread adds a strided share with coalesced fp32 atomics (items may
  // share key/value rows, whose gradients add up)
#pragma unroll
  for (int kind = 0; kind < 2; ++kind) {
    const f32x16 (&acc)[DB] = kind == 0 ? dk : dv;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = {acc[db][4 * g], acc[db][4 * g + 1], acc[db][4 * g + 2], acc[db][4 * g + 3]};
        *reinterpret_cast<f32x4 ZL_LDS*>(smem + key * C::kFlushPitch + (db * 32 + 8 * g + 4 * half) * 4) = x;
      }
    __syncthreads();
    float* __restrict__ out = kind == 0 ? dK : dV;
    for (int idx = tid; idx < tile.kv_len * D; idx += C::kThreads) {
      const int kr = idx / D, col = idx % D;
      const float x = *reinterpret_cast<const float ZL_LDS*>(smem + kr * C::kFlushPitch + col * 4);
      atomicAdd(out + ((tile.kv_row0 + kr) * H + tile.head) * D + col, x);
    }
    __syncthreads();
  }
}

template <int D>
__global__ __launch_bounds__(Bwd<D>::kThreads, 1) void dkdv_kernel(
    const zl_tile* __restrict__ tiles, const int32_t* __restrict__ slots, int n_slots,
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dws,
    float* __restrict__ dK, float* __restrict__ dV, int H, float scale) {
  __shared__ __attribute__((aligned(16))) char smem_raw[Bwd<D>::kLdsBytes];
  char ZL_LDS* smem = (char ZL_LDS*)(smem_raw);  // generic -> LDS address space
  int t0, t1;
  if (n_slots > 0) {
    // Slot = workgroup. Workgroups go round-robin to the 8 XCDs, and equal-cost
    // backward tiles are cut key block by key block with the heads innermost,
    // so when the head count and the slot count are multiples of 8, XCD x runs
    // every key block of heads x, x + 8, ...: the Q / dO rows those tiles
    // stream stay in one L2.
    const int s = blockIdx.x;
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
    dkdv_tile<D>(tile, Q, K, V, dO, LSE, Dws, dK, dV, H, scale, smem);
    __syncthreads();
  }
}

template <int D>
int launch_bwd(const zl_worklist_header* h, const char* d_wl, const void* q, const void* k,
               const void* v, const float* o, const float* lse, const void* dout, float* dq,
               float* dk, float* dv, float* d_ws, hipStream_t stream) {
  const __bf16* Q = static_cast<const __bf16*>(q);
  const __bf16* K = static_cast<const __bf16*>(k);
  const __bf16* V = static_cast<const __bf16*>(v);
  const __bf16* G = static_cast<const __bf16*>(dout);
  // dQ and D over the unsplit forward tiles and slots, then dK / dV (which
  // read D)
  const int qgrid = h->n_slots > 0 ? h->n_slots : h->n_dq_tiles;
  if (qgrid > 0 && h->n_dq_tiles > 0) {
    hipLaunchKernelGGL(dq_kernel<D>, dim3(qgrid), dim3(BwdQ<D>::kThreads), 0, stream,
                       reinterpret_cast<const zl_tile*>(d_wl + h->dq_tiles_offset),
                       reinterpret_cast<const int32_t*>(d_wl + h->dq_slots_offset), h->n_slots, Q, K,
                       V, G, o, lse, d_ws, dq, h->num_heads, h->softmax_scale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return zl::fail(ZL_ERR_HIP, "backward dQ launch: %s", hipGetErrorString(e));
  }
  const int grid = h->n_slots > 0 ? h->n_slots : h->n_bwd_tiles;
  if (grid == 0 || h->n_bwd_tiles == 0) return ZL_OK;
  hipLaunchKernelGGL(dkdv_kernel<D>, dim3(grid), dim3(Bwd<D>::kThreads), 0, stream,
                     reinterpret_cast<const zl_tile*>(d_wl + h->bwd_tiles_offset),
                     reinterpret_cast<const int32_t*>(d_wl + h->bwd_slots_offset), h->n_slots, Q,
                     K, V, G, lse, d_ws, dk, dv, h->num_heads, h->softmax_scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return zl::fail(ZL_ERR_HIP, "backward dK/dV launch: %s", hipGetErrorString(e));
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
