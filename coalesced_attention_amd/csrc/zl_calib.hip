// Attainable matrix-core rate of the calling GPU on a given kind of bf16
// operand: a register-only stream of v_mfma_f32_32x32x16_bf16, timed with HIP
// events. A measurement aid beside the attention kernels, declared in
// zl_calib.h.
#include <hip/hip_runtime.h>

#include <vector>

#include "zl_calib.h"
#include "zl_internal.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 512;          // 8 waves, two per SIMD
constexpr int kOperandVectors = 65536;  // 1 MiB of bf16x8 operands
constexpr int kMaxIters = 1 << 24;

// Each wave keeps four operand fragments and four accumulators in registers
// and issues 8 MFMAs per round, every accumulator updated twice per round
// with a different operand pair. The per-thread checksum keeps the compiler
// from dropping the loop.
__global__ __launch_bounds__(kThreads, 1) void mfma_stream(const bf16x8* __restrict__ in,
                                                           float* __restrict__ out, int iters) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  const bf16x8 a0 = in[(4 * t + 0) & (kOperandVectors - 1)];
  const bf16x8 a1 = in[(4 * t + 1) & (kOperandVectors - 1)];
  const bf16x8 b0 = in[(4 * t + 2) & (kOperandVectors - 1)];
  const bf16x8 b1 = in[(4 * t + 3) & (kOperandVectors - 1)];
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c3, 0, 0, 0);
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b1, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += (c0[r] + c1[r]) + (c2[r] + c3[r]);
  out[t] = s;
}

// bf16 bit patterns: random sign, biased exponent 120..127 (2^-7 .. 2^0),
// random 7-bit mantissa, from a 32-bit linear congruential sequence; or 1.0.
std::vector<uint16_t> operand_bits(int operands) {
  std::vector<uint16_t> h(size_t(kOperandVectors) * 8);
  uint32_t x = 12345u;
  for (auto& v : h) {
    x = x * 1664525u + 1013904223u;
    const uint32_t sign = (x >> 31) << 15;
    const uint32_t exp = 120u + ((x >> 20) & 7u);
    const uint32_t man = (x >> 9) & 0x7fu;
    v = operands == ZL_CALIB_CONSTANT ? uint16_t(0x3f80) : uint16_t(sign | (exp << 7) | man);
  }
  return h;
}

}  // namespace

extern "C" int zl_calib_mfma(int operands, int iters, double* tflops, void* stream) {
  zl::clear_error();
  if (!tflops) return zl::fail(ZL_ERR_NULL, "tflops must be non-NULL");
  if (operands != ZL_CALIB_RANDOM && operands != ZL_CALIB_CONSTANT)
    return zl::fail(ZL_ERR_ARG, "operands must be ZL_CALIB_RANDOM or ZL_CALIB_CONSTANT");
  if (iters < 1 || iters > kMaxIters) return zl::fail(ZL_ERR_ARG, "iters must be in [1, 2^24]");
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus < 1)
    return zl::fail(ZL_ERR_HIP, "device query: %s", hipGetErrorString(e));
  const std::vector<uint16_t> h = operand_bits(operands);
  auto s = static_cast<hipStream_t>(stream);
  bf16x8* din = nullptr;
  float* dout = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  float ms = 0.f;
  e = hipMalloc(&din, h.size() * sizeof(uint16_t));
  if (e == hipSuccess) e = hipMalloc(&dout, size_t(cus) * kThreads * sizeof(float));
  if (e == hipSuccess) e = hipMemcpy(din, h.data(), h.size() * sizeof(uint16_t), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(mfma_stream, dim3(cus), dim3(kThreads), 0, s, din, dout,
                       iters / 10 > 0 ? iters / 10 : 1);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) {
    hipLaunchKernelGGL(mfma_stream, dim3(cus), dim3(kThreads), 0, s, din, dout, iters);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  // nothing is freed while a launch of this call may still run
  const hipError_t es = hipStreamSynchronize(s);
  if (e == hipSuccess) e = es;
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (din) (void)hipFree(din);
  if (dout) (void)hipFree(dout);
  if (e != hipSuccess) return zl::fail(ZL_ERR_HIP, "calibration: %s", hipGetErrorString(e));
  if (!(ms > 0.f)) return zl::fail(ZL_ERR_HIP, "calibration: no elapsed time");
  const double flops = 32768.0 * 8.0 * double(iters) * double(cus) * (kThreads / 64);
  *tflops = flops / (double(ms) * 1e-3) / 1e12;
  return ZL_OK;
}
