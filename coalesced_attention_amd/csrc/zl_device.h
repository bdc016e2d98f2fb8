// Device-side helpers shared by the HIP kernels of libzl.so (gfx950).
#ifndef ZL_DEVICE_H_
#define ZL_DEVICE_H_

#include <hip/hip_runtime.h>

#include <cstdint>

#include "zl.h"

namespace zl {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define ZL_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;               // accelerator complex dies of an MI355X
// s_waitcnt immediate that waits until at most n vector-memory operations
// of this wave are outstanding (lgkmcnt and expcnt left at their maximum).
// vmcnt is six bits on gfx9-family parts, split over bits [3:0] and [15:14].
__host__ __device__ constexpr int wait_vmcnt(int n) {
  return (n & 0xF) | ((n >> 4) << 14) | 0x0F70;
}
static_assert(wait_vmcnt(0) == 0x0F70 && wait_vmcnt(17) == 0x4F71 && wait_vmcnt(63) == 0xCF7F,
              "vmcnt encoding");
// Buffer resource word 3 for raw (untyped) dword loads on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;


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

// Workgroup barrier for the LDS hand-offs inside pipelined loops.
// __syncthreads() carries a workgroup-scope fence, for which the compiler
// drains every outstanding vector-memory operation -- including direct-to-LDS
// prefetches meant for later iterations. This barrier waits only for this
// wave's own LDS reads and writes (lgkmcnt 0) and then meets the other waves;
// a wave waits for the direct loads the next iteration needs with an explicit
// vmcnt before it. The "memory" clobber keeps the compiler from moving any
// memory access across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// An empty asm that reads `x`: x must be computed before this point.
template <typename T>
__device__ __forceinline__ void pin(const T& x) {
  asm volatile("" ::"v"(x));
}

// Two floats rounded to bf16 (RNE) in one dword, a in the low half.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(unsigned, v);
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

}  // namespace dev
}  // namespace zl

#endif  // ZL_DEVICE_H_
