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
#include <type_traits>

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
// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
// Buffer resource word 3 for raw (untyped) dword loads on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;

template <int D>
struct Fwd {
  static constexpr int kWaves = zl::kFwdWaves;
  static constexpr int kQB = zl::kFwdQueryBlocks;  // 32-query MFMA blocks per wave
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBlockM = zl::kFwdBlockM;
  static constexpr int kBN = zl::kFwdBlockN;  // keys per block
  static constexpr int kKB = kBN / 32;        // 32-key MFMA blocks per key block
  static constexpr int kDS = D / 16;          // 16-wide steps over head_dim
  static constexpr int kDB = D / 32;          // 32-wide output blocks over head_dim
  static constexpr int kKP = D * 2 + 16;      // K row pitch (bytes): 16-lane b128 reads hit distinct banks
  static constexpr int kVP = D * 2 + 64;      // V row pitch (bytes): 4-row transpose reads hit distinct banks
  static constexpr int kKBytes = kBN * kKP;
  static constexpr int kVBytes = kBN * kVP;
  static constexpr int kLdsBytes = 2 * (kKBytes + kVBytes);
  static constexpr int kChunksPerRow = D / 8;  // 16-byte chunks per row
  static constexpr int kChunks = kBN * kChunksPerRow;
  // chunks per thread per tensor (the last round may leave threads idle)
  static constexpr int kCPT = (kChunks + kThreads - 1) / kThreads;
  static_assert(kChunks % kThreads == 0 || kCPT == 1, "partial rounds only when one round");
  static_assert(kBlockM == kWaves * 32 * kQB, "tile rows");
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

// The tile record is the same for every lane; readfirstlane tells the
// compiler so, which keeps the derived addresses and the buffer resources in
// scalar registers.
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ zl_tile uniform_tile(const zl_tile& t) {
  zl_tile u;
  u.q_row0 = uniform_i64(t.q_row0);
  u.kv_row0 = uniform_i64(t.kv_row0);
  u.q_rows = __builtin_amdgcn_readfirstlane(t.q_rows);
  u.kv_len = __builtin_amdgcn_readfirstlane(t.kv_len);
  u.head = __builtin_amdgcn_readfirstlane(t.head);
  u.item = __builtin_amdgcn_readfirstlane(t.item);
  return u;
}

template <int D>
__device__ __forceinline__ void run_tile(const zl_tile& tile, const __bf16* __restrict__ Q,
                                         const __bf16* __restrict__ K,
                                         const __bf16* __restrict__ V, float* __restrict__ O,
                                         float* __restrict__ LSE, int H, float c,
                                         char ZL_LDS* smem) {
  using C = Fwd<D>;
  constexpr int QB = C::kQB, KB = C::kKB, DS = C::kDS, DB = C::kDB, CPT = C::kCPT;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int64_t rs = int64_t(H) * D;  // elements between consecutive rows

  // ---- Q^T fragments: query rows wave*32*QB + 32*qb + l32,
  // head_dim [ds*16 + 8*half, +8)
  bf16x8 qf[QB][DS];
  bool qvalid[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qr = (wave * QB + qb) * 32 + l32;
    qvalid[qb] = qr < tile.q_rows;
    const __bf16* qp =
        Q + (tile.q_row0 + (qvalid[qb] ? qr : 0)) * rs + int64_t(tile.head) * D + 8 * half;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      bf16x8 x = *reinterpret_cast<const bf16x8*>(qp + ds * 16);
      qf[qb][ds] = qvalid[qb] ? x : bf16x8{};
    }
  }

  const int kv_len = tile.kv_len;
  const int nblk = (kv_len + C::kBN - 1) / C::kBN;
  const __bf16* kbase = K + tile.kv_row0 * rs + int64_t(tile.head) * D;
  const __bf16* vbase = V + tile.kv_row0 * rs + int64_t(tile.head) * D;

  // LDS: K stages 0,1 then V stages 0,1.
  char ZL_LDS* const kst[2] = {smem, smem + C::kKBytes};
  char ZL_LDS* const vst[2] = {smem + 2 * C::kKBytes, smem + 2 * C::kKBytes + C::kVBytes};

  // Global -> register -> LDS staging with raw buffer loads. The buffer of
  // block `blk` starts at its first key row and ends at the item's last key,
  // so rows past kv_len read as zero without a branch. Thread `tid` always
  // moves the same 16-byte chunks (row, column) of a 64-key tile.
  int ld_off[CPT];
  int st_k[CPT], st_v[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    // threads past the tile's chunk count re-load and re-store chunk 0 of
    // their row 0 copy: the same bytes the owning thread writes
    const int ch = (tid + i * C::kThreads) % C::kChunks;
    const int row = ch / C::kChunksPerRow, col = ch % C::kChunksPerRow;
    ld_off[i] = int(row * rs + col * 8) * 2;  // < 64 rows of one tile
    st_k[i] = row * C::kKP + col * 16;
    st_v[i] = row * C::kVP + col * 16;
  }
  u32x4 kreg[CPT], vreg[CPT];
  auto gload = [&](const __bf16* base, u32x4 (&reg)[CPT], int blk) __attribute__((always_inline)) {
    // wave-uniform by construction; readfirstlane keeps the descriptor in
    // scalar registers (a vector descriptor would need a waterfall loop)
    const int rows = __builtin_amdgcn_readfirstlane(min(C::kBN, max(0, kv_len - blk * C::kBN)));
    const int64_t addr = uniform_i64(reinterpret_cast<int64_t>(base + int64_t(blk) * C::kBN * rs));
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<__bf16*>(addr), 0,
                                                        rows * int(rs) * 2, kBufferFlags);
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      reg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, ld_off[i], 0, 0));
  };
  auto lstore = [&](char ZL_LDS* dst, const u32x4 (&reg)[CPT], const int (&off)[CPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) *reinterpret_cast<u32x4 ZL_LDS*>(dst + off[i]) = reg[i];
  };

  // Per-lane LDS byte offsets.
  const int k_off = l32 * C::kKP + half * 16;
  const int tr_row = 4 * half + ((lane & 15) >> 2);
  const int tr_col = (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;

  // S^T = K Q^T for one 64-key block; each K fragment feeds every query block.
  auto qk = [&](const char ZL_LDS* kb, f32x16 (&s)[QB][KB]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < KB; ++b) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][b] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const bf16x8 a = lds_read_b128(kb + b * 32 * C::kKP + k_off + ds * 32);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ds], s[qb][b], 0, 0, 0);
      }
    }
  };
  // Keys at or past kv_len (only in the last block) get -inf.
  auto mask = [&](f32x16 (&s)[QB][KB], int blk) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int b = 0; b < KB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = blk * C::kBN + b * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= kv_len) s[qb][b][r] = -INFINITY;
        }
  };
  // Row max over both halves of the block, in exp2 units.
  auto rowmax = [&](const f32x16 (&s)[KB]) __attribute__((always_inline)) {
    float m0 = fmaxf(s[0][0], s[0][1]), m1 = fmaxf(s[0][2], s[0][3]);
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int r = (b == 0 ? 4 : 0); r < 16; r += 4) {
        m0 = fmaxf(m0, fmaxf(s[b][r], s[b][r + 1]));
        m1 = fmaxf(m1, fmaxf(s[b][r + 2], s[b][r + 3]));
      }
    return swap_halves_max(fmaxf(m0, m1)) * c;
  };
  // O^T += V^T P^T for one 64-key block; each V^T fragment feeds every query block.
  auto pv = [&](const char ZL_LDS* vb, const bf16x8 (&pf)[QB][KB][2], f32x16 (&o)[QB][DB]) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const char ZL_LDS* vp = vb + (b * 32 + 16 * u + tr_row) * C::kVP + db * 64 + tr_col;
          const i16x4 lo = lds_read_tr16(vp);
          const i16x4 hi = lds_read_tr16(vp + 8 * C::kVP);
          // whole-vector concatenation: per-element inserts of bf16 lanes
          // were lowered to a lossy permute by the compiler
          const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 a = __builtin_bit_cast(bf16x8, cat);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb][b][u], o[qb][db], 0, 0, 0);
        }
  };

  f32x16 oacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[qb][i] = f32x16{};
  float m_use[QB], l_part[QB];  // max in use (exp2 units) and this lane's partial row sum
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_use[qb] = -INFINITY;
    l_part[qb] = 0.f;
  }
  f32x16 s_a[QB][KB], s_b[QB][KB];

  // ---- prologue: K(0), V(0), K(1) to LDS; S(0) and its max
  if (nblk > 0) {
    gload(kbase, kreg, 0);
    gload(vbase, vreg, 0);
    lstore(kst[0], kreg, st_k);
    lstore(vst[0], vreg, st_v);
    gload(kbase, kreg, 1);
    lstore(kst[1], kreg, st_k);
  }
  __syncthreads();
  if (nblk > 0) {
    qk(kst[0], s_a);
    if (nblk == 1) mask(s_a, 0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m_use[qb] = rowmax(s_a[qb]);
  }
  __syncthreads();  // K stage 0 is refilled by the first iteration

  // ---- one 64-key block. Iteration j turns S(j) (in `sc`) into P(j) in
  // place and accumulates O += V(j)^T P(j)^T, while computing S(j+1) into
  // `sn`. The work is issued as short windows in program order, each a
  // vector-ALU chunk followed by the matrix-core chunk it does not depend
  // on, so the MFMAs of one window run under the vector work of the next:
  //   phase A, 4 windows: exponentials of 16 scores of S(j) | 8 MFMAs of S(j+1)
  //   phase B, 4 windows: bf16 pack + row sums of 16 probabilities and part
  //                       of the max of S(j+1) | 8 MFMAs of O += V^T P^T
  // K runs two blocks ahead of V so each LDS stage is rewritten only after
  // the barrier that ends its last reader.
  // The last iteration also runs the S(j+1) MFMAs, on a K stage holding
  // zeros (the loads past the last block return zero); its result is unused.
  const bool ragged = (kv_len % C::kBN) != 0;
  auto iteration = [&](int j, f32x16 (&sc)[QB][KB], f32x16 (&sn)[QB][KB])
      __attribute__((always_inline)) {
    const bool has_next = j + 1 < nblk;
    constexpr int kWin = 2 * KB;              // windows per phase
    constexpr int kPer = QB * KB * 16 / kWin;  // scores per phase-A window
    gload(kbase, kreg, j + 2);  // all zero past the last block
    gload(vbase, vreg, j + 1);
    // Keys past kv_len exist only in the last block; mask them just before
    // they are exponentiated. (The max of S(j+1) taken in phase B may see
    // the zero scores of the zero-filled rows: that only raises the max in
    // use, which the normalisation cancels.)
    if (ragged && j + 1 == nblk) mask(sc, j);
    const char ZL_LDS* kb = kst[(j + 1) & 1];
    // phase A
#pragma unroll
    for (int w = 0; w < kWin; ++w) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int idx = w * kPer + e;
        const int qb = idx / (KB * 16), b = (idx / 16) % KB, r = idx % 16;
        sc[qb][b][r] = __builtin_amdgcn_exp2f(fmaf(sc[qb][b][r], c, -m_use[qb]));
      }
      {
        const int b = w / 2, ds0 = (w % 2) * (DS / 2);
#pragma unroll
        for (int ds = ds0; ds < ds0 + DS / 2; ++ds) {
          const bf16x8 a = lds_read_b128(kb + b * 32 * C::kKP + k_off + ds * 32);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            sn[qb][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                a, qf[qb][ds], ds == 0 ? f32x16{} : sn[qb][b], 0, 0, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase B
    const char ZL_LDS* vb = vst[j & 1];
    float mx0[QB], mx1[QB];
#pragma unroll
    for (int w = 0; w < kWin; ++w) {
      const int b = w / 2, u = w % 2;
      bf16x8 pf[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float ls = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = sc[qb][b][8 * u + e];
          ls += pe;
          pf[qb][e] = (__bf16)pe;
        }
        l_part[qb] += ls;
        {
          // max over the 8 scores of S(j+1) at the same positions
          const f32x16& t = sn[qb][b];
          const float m4 = fmaxf(fmaxf(t[8 * u], t[8 * u + 1]), fmaxf(t[8 * u + 2], t[8 * u + 3]));
          const float m8 = fmaxf(fmaxf(t[8 * u + 4], t[8 * u + 5]), fmaxf(t[8 * u + 6], t[8 * u + 7]));
          if (w == 0) {
            mx0[qb] = m4;
            mx1[qb] = m8;
          } else {
            mx0[qb] = fmaxf(mx0[qb], m4);
            mx1[qb] = fmaxf(mx1[qb], m8);
          }
        }
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char ZL_LDS* vp = vb + (b * 32 + 16 * u + tr_row) * C::kVP + db * 64 + tr_col;
        const i16x4 lo = lds_read_tr16(vp);
        const i16x4 hi = lds_read_tr16(vp + 8 * C::kVP);
        // whole-vector concatenation: per-element inserts of bf16 lanes
        // were lowered to a lossy permute by the compiler
        const i16x8 cat = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        const bf16x8 a = __builtin_bit_cast(bf16x8, cat);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb], oacc[qb][db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lstore(kst[j & 1], kreg, st_k);
    lstore(vst[(j + 1) & 1], vreg, st_v);
    __syncthreads();
    if (has_next) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mx = swap_halves_max(fmaxf(mx0[qb], mx1[qb])) * c;
        // Raise the max in use only when a row grew past the slack. The
        // branch is taken by the whole wave or not at all, so the O
        // accumulators are only touched when some row needs it.
        const bool grow = mx > m_use[qb] + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float alpha = grow ? __builtin_amdgcn_exp2f(m_use[qb] - mx) : 1.f;
          m_use[qb] = grow ? mx : m_use[qb];
          l_part[qb] *= alpha;
#pragma unroll
          for (int i = 0; i < DB; ++i) oacc[qb][i] *= alpha;
        }
      }
    }
  };
  for (int j = 0; j < nblk; j += 2) {
    iteration(j, s_a, s_b);
    if (j + 1 < nblk) iteration(j + 1, s_b, s_a);
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = swap_halves_sum(l_part[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse = l_tot > 0.f ? kLn2 * (m_use[qb] + __builtin_amdgcn_logf(l_tot)) : -INFINITY;
    if (qvalid[qb]) {
      const int qr = (wave * QB + qb) * 32 + l32;
      float* op = O + (tile.q_row0 + qr) * rs + int64_t(tile.head) * D + 4 * half;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& a = oacc[qb][db];
          f32x4 x = {a[4 * g] * inv, a[4 * g + 1] * inv, a[4 * g + 2] * inv, a[4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(op + db * 32 + 8 * g) = x;
        }
      if (half == 0) LSE[(tile.q_row0 + qr) * H + tile.head] = lse;
    }
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
  t0 = __builtin_amdgcn_readfirstlane(t0);
  t1 = __builtin_amdgcn_readfirstlane(t1);
  for (int t = t0; t < t1; ++t) {
    const zl_tile tile = uniform_tile(tiles[t]);
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
