// Coalesced varlen attention forward for gfx950 (CDNA4).
//
// One launch runs every tile of a worklist: a tile is up to 256 query rows
// of one work item on one head, against that item's whole key range. Whole
// sequences and theta = (q, h, k) shards differ only in their row and head
// ranges, so they share the launch (newx.sg page "Zellige: Moldable
// Sequence Placement for Mixed Image-Video DiT Training", Abstract; shards
// per the pith.science review of arXiv 2608.01150, "What carries the
// argument"). The attention is exact softmax attention computed block by
// block with a running shift and sum (the IO-aware exact method the
// review's "Assumptions" section cites as FlashAttention [7]).
//
// Work decomposition (per workgroup of 8 waves, two per SIMD, one tile at a
// time):
//   - wave w owns query rows [32w, 32w+32) of the tile; lane l owns query
//     row l%32 and half h = l/32 of that row's keys in every 32-key block.
//   - scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in registers;
//     the tile's Q rows arrive through LDS with the same direct loads as K/V).
//     In the accumulator layout a lane then holds 16 keys of ONE query, so
//     the row max is an in-lane reduction plus one v_permlane32_swap, and
//     the running sum needs no exchange until the epilogue.
//   - the output is also accumulated transposed, O^T += V^T P^T (A = V^T read
//     from the LDS tile with ds_read_b64_tr_b16, B = P^T straight from the
//     score registers converted to bf16), so the rescale factor of a query
//     multiplies registers of the same lane.
//   - K/V tiles of 64 keys go from HBM straight into LDS with buffer loads
//     (no staging registers), four stages each, K three blocks ahead of
//     its use and V one; each wave works on three blocks at once (see the
//     iteration below) and the workgroup meets one barrier per two blocks.
//   - the shift of a row's exponentials is the maximum of its first key
//     block, and it is raised only when a lane's running sum of weights
//     passes 2^32 (or overflows): weights above 1 are exact in floating
//     point and cancel in O / l and LSE, so the key loop computes no block
//     maxima; the rare raise recomputes the block from its scores.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "zl.h"
#include "zl_device.h"
#include "zl_internal.h"

namespace {

using namespace zl::dev;

// Bound on a lane's running sum of weights before the shift is raised.
constexpr float kSumLimit = 4294967296.0f;  // 2^32

template <int D>
struct Fwd {
  static constexpr int kWaves = zl::kFwdWaves;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBlockM = zl::kFwdBlockM;
  static constexpr int kBN = zl::kFwdBlockN;  // keys per block
  static constexpr int kKB = kBN / 32;        // 32-key MFMA blocks per key block
  static constexpr int kDS = D / 16;          // 16-wide steps over head_dim
  static constexpr int kDB = D / 32;          // 32-wide output blocks over head_dim
  // LDS tiles are groups of kG rows (1 KB of bf16) stored chunk-column-major:
  // 16-byte chunk c of row r' of a group sits at byte (c * kG + r') * 16.
  // A direct-to-LDS load of one wave fills one group. Padding a group by
  // 16 * kG bytes puts the 16 rows read by a 16-lane K fragment load, and
  // the 4 rows x 32 bytes of a V transpose read, in distinct banks.
  static constexpr int kG = 512 / D;
  static constexpr int kGroupBytes = 1024 + 16 * kG;
  static constexpr int kGroups = kBN / kG;
  static constexpr int kTileBytes = kGroups * kGroupBytes;
  // LDS stages and load distances (in key blocks). Iteration j reads K(j+1)
  // and V(j-1) and issues K(j + kKAhead) and V(j + kVAhead). The workgroup
  // meets a barrier after every odd iteration (and after the last one); it
  // waits for every load issued so far and publishes K and V for the next
  // two iterations. A stage may be refilled once a barrier after its last
  // reader has passed: K(x) is last read in iteration x-1 and V(x) in
  // iteration x+1, and an even iteration's last barrier lies two iterations
  // back.
  static constexpr int kKStages = 4;
  static constexpr int kVStages = 4;
  static constexpr int kKAhead = 3;
  static constexpr int kVAhead = 1;
  static_assert(kKAhead <= kKStages - 1 && kVAhead <= kVStages - 3, "stage reuse distance");
  static constexpr int kLdsBytes = (kKStages + kVStages) * kTileBytes;
  static constexpr int kGroupsPerWave = (kGroups + kWaves - 1) / kWaves;
  static_assert(kBlockM == kWaves * 32, "one 32-row MFMA block per wave");
  static_assert(kBN % 32 == 0 && (D == 64 || D == 128), "shapes");
};

// O / LSE rows of the tile start at out_row0 (q_row0, or a workspace row for
// a key chunk of a split item).
template <int D>
__device__ __forceinline__ void run_tile(const zl_tile& tile, const __bf16* __restrict__ Q,
                                         const __bf16* __restrict__ K,
                                         const __bf16* __restrict__ V, float* __restrict__ O,
                                         float* __restrict__ LSE, int64_t out_row0, int H,
                                         float c, char ZL_LDS* smem) {
  using C = Fwd<D>;
  constexpr int KB = C::kKB, DS = C::kDS, DB = C::kDB, G = C::kG, GB = C::kGroupBytes;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int64_t rs = int64_t(H) * D;  // elements between consecutive rows

  // ---- Q^T fragments (read in the prologue): query row wave*32 + l32,
  // head_dim [ds*16 + 8*half, +8)
  const int qr = wave * 32 + l32;
  const bool qvalid = qr < tile.q_rows;
  bf16x8 qf[DS];

  const int kv_len = tile.kv_len;
  const int nblk = (kv_len + C::kBN - 1) / C::kBN;
  const __bf16* kbase = K + tile.kv_row0 * rs + int64_t(tile.head) * D;
  const __bf16* vbase = V + tile.kv_row0 * rs + int64_t(tile.head) * D;

  // ---- direct-to-LDS tile loads. The buffer of block `blk` starts at its
  // first key row and holds only the rows before kv_len, so rows past the
  // item (and every row of a block outside [0, nblk)) arrive as zeros.
  // Lane l of a group load carries row (l % G), chunk (l / G) of the group.
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
  constexpr int kLoadsPerTile = C::kGroupsPerWave;  // per wave, per tensor
  auto kstage = [&](int blk) { return (blk % C::kKStages) * C::kTileBytes; };
  auto vstage = [&](int blk) { return (C::kKStages + (blk + C::kVStages) % C::kVStages) * C::kTileBytes; };

  // ---- per-lane LDS offsets (the rest are compile-time immediates)
  // K fragment (A of S^T): row b*32 + l32, chunk 2*ds + half.
  const int k_lane = (l32 / G) * GB + (half * G + l32 % G) * 16;
  // V^T fragment via transpose reads: row R0 + rr with rr = 4*half + e_l,
  // chunk db*4 + c_l, byte (lane & 1) * 8 within the chunk.
  const int rr = 4 * half + ((lane & 15) >> 2);
  const int c_l = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int v_lane = (rr / G) * GB + (c_l * G + rr % G) * 16 + (lane & 1) * 8;

  // Per-stage base addresses are formed once per block and kept opaque, so
  // the compiler does not hoist one register per (stage, fragment) pair
  // (stage offsets exceed the 16-bit DS immediate).
  auto k_base = [&](int stage_off) __attribute__((always_inline)) {
    int a = stage_off + k_lane;
    asm volatile("" : "+v"(a));
    return (const char ZL_LDS*)(smem + a);
  };
  auto v_base = [&](int stage_off) __attribute__((always_inline)) {
    int a = stage_off + v_lane;
    asm volatile("" : "+v"(a));
    return (const char ZL_LDS*)(smem + a);
  };
  auto read_k = [&](const char ZL_LDS* kb, int b, int ds) __attribute__((always_inline)) {
    return lds_read_b128(kb + (b * 32 / G) * GB + ds * 2 * G * 16);
  };
  auto read_v = [&](const char ZL_LDS* vb, int b, int u, int db) __attribute__((always_inline)) {
    const char ZL_LDS* p = vb + ((b * 32 + 16 * u) / G) * GB + db * 4 * G * 16;
    const i16x4 lo = lds_read_tr16(p);
    const i16x4 hi = lds_read_tr16(p + (8 / G) * GB + (8 % G) * 16);  // 8 rows further
    // whole-vector concatenation: per-element inserts of bf16 lanes were
    // lowered to a lossy permute by the compiler
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // Keys at or past kv_len (only in the last block) get -inf.
  auto mask = [&](f32x16 (&s)[KB], int blk) __attribute__((always_inline)) {
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = blk * C::kBN + b * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (key >= kv_len) s[b][r] = -INFINITY;
      }
  };
  // max of 16 scores and a running value as a tree of three-input maxima
  // (8 v_max3_f32)
  auto max3 = [](float a, float b, float d) __attribute__((always_inline)) { return fmaxf(fmaxf(a, b), d); };
  auto max16 = [&](const f32x16& t, float run) __attribute__((always_inline)) {
    const float a = max3(t[0], t[1], t[2]);
    const float b = max3(t[3], t[4], t[5]);
    const float d = max3(t[6], t[7], t[8]);
    const float e = max3(t[9], t[10], t[11]);
    const float f = max3(t[12], t[13], t[14]);
    return max3(max3(a, b, d), max3(e, f, t[15]), run);
  };

  f32x16 oacc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) oacc[i] = f32x16{};
  float m_use = -INFINITY;  // the row's shift (exp2 units): its first block's max, raised on overflow
  float l_part = 0.f;       // this lane's partial row sum, relative to m_use

  if (nblk > 0) {
    // ---- prologue: K(0), the Q rows, K(1), V(0), K(2); S(0) and its max.
    // Only K(0) and Q are waited for before S(0); the other loads land while
    // its MFMAs run.
    static_assert(C::kKAhead == 3 && C::kVAhead == 1, "prologue load order");
    // Q rows go through LDS with direct loads, into the four stages the
    // prologue does not fill: K stage 3 and V stages 1..3 (groups of kG rows
    // in the K/V layout). V stage 3 is also iteration 0's V(-1), which is
    // multiplied by P(-1) = 0; Q rows are finite, so that adds zeros.
    static_assert(C::kKStages == 4 && C::kVStages == 4, "Q staging stages");
    constexpr int kQGroupsPerWave = C::kBlockM / G / C::kWaves;
    auto q_group_off = [&](int g) __attribute__((always_inline)) {
      return g < C::kGroups ? 3 * C::kTileBytes + g * GB
                            : (C::kKStages + 1) * C::kTileBytes + (g - C::kGroups) * GB;
    };
    issue_tile(kbase, kstage(0), 0);
    {
      const int64_t qaddr = uniform_i64(reinterpret_cast<int64_t>(Q + tile.q_row0 * rs + int64_t(tile.head) * D));
      const auto qrsrc = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<__bf16*>(qaddr), 0,
                                                           tile.q_rows * row_bytes, kBufferFlags);
#pragma unroll
      for (int i = 0; i < kQGroupsPerWave; ++i) {
        const int g = wave * kQGroupsPerWave + i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            qrsrc, (void ZL_LDS*)(smem + q_group_off(g)), 16, ld_lane,
            __builtin_amdgcn_readfirstlane(g * G * int(rs) * 2), 0, 0);
      }
    }
    issue_tile(kbase, kstage(1), 1);
    issue_tile(vbase, vstage(0), 0);
    issue_tile(kbase, kstage(2), 2);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(3 * kLoadsPerTile));  // K(0) and Q landed
    lds_barrier();
    {
      // Q^T fragments: row qr, chunk 2*ds + half (the K fragment pattern)
      const int g0 = (wave * 32) / G;
      int qo = q_group_off(g0) + ((qr % 32) / G) * GB + (half * G + qr % G) * 16;
      asm volatile("" : "+v"(qo));
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) qf[ds] = lds_read_b128(smem + qo + ds * 2 * G * 16);
    }
    f32x16 s_a[KB], s_b[KB];
    bf16x8 p_a[KB][2], p_b[KB][2];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      s_a[b] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        s_a[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_k(k_base(kstage(0)), b, ds), qf[ds], s_a[b], 0, 0, 0);
      p_b[b][0] = bf16x8{};
      p_b[b][1] = bf16x8{};
    }
    if (nblk == 1) mask(s_a, 0);
    {
      float mx = max16(s_a[0], -INFINITY);
#pragma unroll
      for (int b = 1; b < KB; ++b) mx = max16(s_a[b], mx);
      m_use = swap_halves_max(mx) * c;
    }
    __syncthreads();  // the prologue's loads land; K stage 0 is refilled in iteration 1

    // ---- iteration j, three blocks in flight:
    //   exponentials, row sums and bf16 packing of S(j) -> P(j)     (VALU)
    //   S(j+1) = K(j+1) Q^T                                          (MFMA)
    //   O += V(j-1)^T P(j-1)^T                                       (MFMA)
    // issued as 4*KB windows; the two windows of pair (b, u) each
    // exponentiate 4 of the 8 scores that form P(j)'s operand (b, u), run a
    // quarter of S(j+1)'s MFMAs for key block b, and half of the PV MFMAs for
    // operand (b, u) of P(j-1), alternating a dependent S MFMA with an
    // independent PV MFMA. Loads run ahead: K(j+3)
    // and V(j+1) are issued at the top; the barrier at the bottom of every
    // odd iteration publishes them for the next two iterations.
    const bool ragged = (kv_len % C::kBN) != 0;
    auto iteration = [&](int j, f32x16 (&sc)[KB], f32x16 (&sn)[KB], bf16x8 (&pc)[KB][2],
                         const bf16x8 (&pp)[KB][2], bool bar) __attribute__((always_inline)) {
      issue_tile(kbase, kstage(j + C::kKAhead), j + C::kKAhead);
      issue_tile(vbase, vstage(j + C::kVAhead), j + C::kVAhead);
      if (ragged && j + 1 == nblk) mask(sc, j);
      const char ZL_LDS* kb = k_base(kstage(j + 1));
      const char ZL_LDS* vb = v_base(vstage(j - 1));
      const float l_prev = l_part;
#pragma unroll
      for (int w = 0; w < 2 * KB; ++w) {
        const int b = w / 2, u = w % 2;
        u32x4 packed;
        // two sub-windows of 4 scores, 2 S MFMAs and 2 PV MFMAs each
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          constexpr int NS = DS / 4, NV = DB / 2;
          bf16x8 kf[NS], vf[NV];
#pragma unroll
          for (int i = 0; i < NS; ++i) kf[i] = read_k(kb, b, u * (DS / 2) + hw * NS + i);
#pragma unroll
          for (int i = 0; i < NV; ++i) vf[i] = read_v(vb, b, u, hw * NV + i);
          float pe[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(sc[b][8 * u + 4 * hw + e], c, -m_use));
          l_part += (pe[0] + pe[1]) + (pe[2] + pe[3]);
          packed[2 * hw] = pack_bf16x2(pe[0], pe[1]);
          packed[2 * hw + 1] = pack_bf16x2(pe[2], pe[3]);
          pin(packed[2 * hw]);
          pin(packed[2 * hw + 1]);
          pin(l_part);
#pragma unroll
          for (int i = 0; i < NS; ++i) {
            const int ds = u * (DS / 2) + hw * NS + i;
            sn[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[ds], ds == 0 ? f32x16{} : sn[b], 0, 0, 0);
            if (i < NV) oacc[hw * NV + i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pp[b][u], oacc[hw * NV + i], 0, 0, 0);
          }
#pragma unroll
          for (int i = NS; i < NV; ++i)
            oacc[hw * NV + i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pp[b][u], oacc[hw * NV + i], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        pc[b][u] = __builtin_bit_cast(bf16x8, packed);
      }
      if (bar) __syncthreads();
      // P(j) was taken relative to m_use. Weights above 1 are exact in
      // floating point, so the shift only has to keep exp2 and the sums far
      // from overflow: a lane whose running sum left [0, 2^32] (or became
      // inf) sends its wave down this rare path, which shifts each row by the
      // maximum of its block and redoes P(j) from the scores, still in
      // registers. O, which holds P(0..j-1), and l are scaled to match.
      if (__builtin_amdgcn_ballot_w64(!(l_part <= kSumLimit)) != 0) {
        float mx = -INFINITY;
#pragma unroll
        for (int b2 = 0; b2 < KB; ++b2) mx = max16(sc[b2], mx);
        const float m_new = fmaxf(m_use, swap_halves_max(mx) * c);
        const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
        float bs = 0.f;
#pragma unroll
        for (int b2 = 0; b2 < KB; ++b2)
#pragma unroll
          for (int u2 = 0; u2 < 2; ++u2)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pv = __builtin_amdgcn_exp2f(fmaf(sc[b2][8 * u2 + e], c, -m_new));
              bs += pv;
              pc[b2][u2][e] = (__bf16)pv;
            }
        l_part = fmaf(l_prev, alpha, bs);
#pragma unroll
        for (int i = 0; i < DB; ++i) oacc[i] *= alpha;
        m_use = m_new;
      }
    };
    int j = 0;
    for (; j + 1 < nblk; j += 2) {
      iteration(j, s_a, s_b, p_a, p_b, false);
      iteration(j + 1, s_b, s_a, p_b, p_a, true);
    }
    if (j < nblk) iteration(j, s_a, s_b, p_a, p_b, true);
    // ---- drain: O += V(nblk-1)^T P(nblk-1)^T
    const bf16x8 (&pl)[KB][2] = (nblk & 1) ? p_a : p_b;
    const char ZL_LDS* vb = v_base(vstage(nblk - 1));
#pragma unroll
    for (int b = 0; b < KB; ++b)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_v(vb, b, u, db), pl[b][u], oacc[db], 0, 0, 0);
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 * (m + log2 l)
  const float l_tot = swap_halves_sum(l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? kLn2 * (m_use + __builtin_amdgcn_logf(l_tot)) : -INFINITY;
  if (qvalid) {
    float* op = O + (out_row0 + qr) * rs + int64_t(tile.head) * D + 4 * half;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& a = oacc[db];
        f32x4 x = {a[4 * g] * inv, a[4 * g + 1] * inv, a[4 * g + 2] * inv, a[4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(op + db * 32 + 8 * g) = x;
      }
    if (half == 0) LSE[(out_row0 + qr) * H + tile.head] = lse;
  }
}

template <int D>
__global__ __launch_bounds__(Fwd<D>::kThreads, 1) void fwd_kernel(
    const zl_tile* __restrict__ tiles, const int32_t* __restrict__ slots, int n_slots,
    const zl_outmap* __restrict__ outmap, const __bf16* __restrict__ Q,
    const __bf16* __restrict__ K, const __bf16* __restrict__ V, float* __restrict__ O,
    float* __restrict__ LSE, float* __restrict__ ws_o, float* __restrict__ ws_lse, int H,
    float c) {
  __shared__ __attribute__((aligned(16))) char smem_raw[Fwd<D>::kLdsBytes];
  char ZL_LDS* smem = (char ZL_LDS*)(smem_raw);  // generic -> LDS address space
  int t0, t1;
  if (n_slots > 0) {
    // Workgroups are dispatched round-robin over the XCDs (w -> XCD w % 8),
    // each with its own L2. Consecutive slots receive consecutive tiles of
    // the LPT order, i.e. the query blocks of one (item, head) that read the
    // same K/V, so slot s runs on a workgroup of XCD s / (n_slots / 8).
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
    const zl_outmap om = outmap[tile.item];
    const bool to_ws = __builtin_amdgcn_readfirstlane(om.to_workspace) != 0;
    const int64_t out_row0 = tile.q_row0 + uniform_i64(om.o_shift);
    run_tile<D>(tile, Q, K, V, to_ws ? ws_o : O, to_ws ? ws_lse : LSE, out_row0, H, c, smem);
    __syncthreads();  // LDS is reused by the next tile
  }
}

template <int D>
int launch_fwd(const zl_worklist_header* h, const char* d_wl, const void* q, const void* k,
               const void* v, float* o, float* lse, float* ws, hipStream_t stream) {
  const int grid = h->n_slots > 0 ? h->n_slots : h->n_tiles;
  if (grid == 0 || h->n_tiles == 0) return ZL_OK;
  const float c = h->softmax_scale * kLog2e;
  float* ws_o = ws;
  float* ws_lse = ws ? ws + h->ws_rows * int64_t(h->num_heads) * D : nullptr;
  hipLaunchKernelGGL(fwd_kernel<D>, dim3(grid), dim3(Fwd<D>::kThreads), 0, stream,
                     reinterpret_cast<const zl_tile*>(d_wl + h->tiles_offset),
                     reinterpret_cast<const int32_t*>(d_wl + h->slots_offset), h->n_slots,
                     reinterpret_cast<const zl_outmap*>(d_wl + h->outmap_offset),
                     static_cast<const __bf16*>(q), static_cast<const __bf16*>(k),
                     static_cast<const __bf16*>(v), o, lse, ws_o, ws_lse, h->num_heads, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return zl::fail(ZL_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  if (h->n_merges > 0)
    return zl::launch_merge_list(h, d_wl, ws_o, ws_lse, o, lse, stream);
  return ZL_OK;
}

}  // namespace

extern "C" int zl_coalesced_attn_fwd(const void* h_wl, const void* d_wl, const void* q,
                                     const void* k, const void* v, float* o, float* lse,
                                     float* workspace, void* stream) {
  zl::clear_error();
  const zl_worklist_header* h = nullptr;
  int rc = zl::check_worklist(h_wl, &h);
  if (rc) return rc;
  if (!d_wl || !q || !k || !v || !o || !lse)
    return zl::fail(ZL_ERR_NULL, "device pointers must be non-NULL");
  if (h->ws_rows > 0 && !workspace)
    return zl::fail(ZL_ERR_NULL, "the worklist splits items: workspace must be non-NULL");
  if (!zl::aligned16(d_wl) || !zl::aligned16(q) || !zl::aligned16(k) || !zl::aligned16(v) ||
      !zl::aligned16(o) || !zl::aligned16(lse) || (h->ws_rows > 0 && !zl::aligned16(workspace)))
    return zl::fail(ZL_ERR_ALIGN, "device pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* dw = static_cast<const char*>(d_wl);
  float* ws = h->ws_rows > 0 ? workspace : nullptr;
  return h->head_dim == 128 ? launch_fwd<128>(h, dw, q, k, v, o, lse, ws, s)
                            : launch_fwd<64>(h, dw, q, k, v, o, lse, ws, s);
}

// ---- allocation-free variant: the key-chunk partials live in a file-scope
// device array instead of a caller workspace. The array name is a host-side
// stand-in in host code; its device address is looked up once per device
// with hipGetSymbolAddress and only that address is handed to kernels.
namespace {

constexpr int64_t kScratchBytes = ZL_NOALLOC_SCRATCH_BYTES;
constexpr int64_t kScratchFloats = kScratchBytes / int64_t(sizeof(float));
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) float scratch[kScratchFloats];

std::atomic<float*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the first
// call made with that device current, then cached).
int scratch_address(int dev, float** out) {
  float* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !addr)
        return zl::fail(ZL_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
      p = static_cast<float*>(addr);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ZL_OK;
}

}  // namespace

extern "C" int zl_coalesced_attn_fwd_noalloc(const void* h_wl, const void* d_wl, const void* q,
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
  const int64_t need = h->ws_rows * int64_t(h->num_heads) * (h->head_dim + 1);
  if (need > kScratchFloats)
    return zl::fail(ZL_ERR_BUFSIZE,
                    "the worklist's key-chunk partials need %lld bytes; the allocation-free entry "
                    "point holds %lld (use zl_coalesced_attn_fwd with a caller workspace)",
                    (long long)(need * int64_t(sizeof(float))), (long long)kScratchBytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const char* dw = static_cast<const char*>(d_wl);
  float* ws = nullptr;
  if (need > 0) {
    int cur = -1, sdev = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess) e = hipStreamGetDevice(s, &sdev);
    if (e != hipSuccess) return zl::fail(ZL_ERR_HIP, "device query: %s", hipGetErrorString(e));
    if (sdev != cur)
      return zl::fail(ZL_ERR_ARG, "stream belongs to device %d but device %d is current", sdev, cur);
    if (cur < 0 || cur >= kMaxDevices)
      return zl::fail(ZL_ERR_ARG, "device %d is beyond the %d the library tracks", cur, kMaxDevices);
    rc = scratch_address(cur, &ws);
    if (rc) return rc;
  }
  return h->head_dim == 128 ? launch_fwd<128>(h, dw, q, k, v, o, lse, ws, s)
                            : launch_fwd<64>(h, dw, q, k, v, o, lse, ws, s);
}
