// Measurement probes: the chip's achievable dense MFMA rate (and the shader
// clock it runs at) and its achievable streaming-read bandwidth, so that the
// operator's figures can be set against measured peaks as well as nominal ones.
// Not part of the operator.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "flp_launch.h"

namespace flp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeWG = 2048;  // workgroups of the MFMA probe (8 per compute unit)

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// bf16 with a random sign, exponent in [-7, 0] and mantissa: |x| in [2^-7, 2).
__device__ __forceinline__ uint16_t random_bf16(uint32_t h) {
  return uint16_t(((h & 1u) << 15) | ((120u + ((h >> 1) & 7u)) << 7) | ((h >> 4) & 0x7Fu));
}

// Eight operand pairs cycled through 16 independent accumulator chains of
// v_mfma_f32_16x16x32_bf16; wave 0 records the shader-clock and real-time
// counters around the loop.  out[wg] keeps the sums alive; clk[2 wg + 0/1] are
// the two counter deltas.
__global__ __launch_bounds__(256) void k_probe_mfma(int64_t iters, int zero, float* __restrict__ out,
                                                    uint64_t* __restrict__ clk) {
  const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
  bf16x8_t A[8], B[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    u16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t h = mix(gid * 131u + uint32_t(s) * 17u + uint32_t(e));
      a[e] = zero ? uint16_t(0) : random_bf16(h);
      b[e] = zero ? uint16_t(0) : random_bf16(mix(h));
    }
    A[s] = __builtin_bit_cast(bf16x8_t, a);
    B[s] = __builtin_bit_cast(bf16x8_t, b);
  }
  f32x4_t acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[s], B[(s + j) & 7], acc[j], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) r += (acc[j][0] + acc[j][1]) + (acc[j][2] + acc[j][3]);
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  r += __shfl_xor(r, 1);
  if (threadIdx.x == 0) {
    out[blockIdx.x] = r;
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Streaming read: every thread xors 16-byte words with a grid stride, eight loads
// in flight; one value per workgroup is written.
__global__ __launch_bounds__(256) void k_probe_read(const u32x4* __restrict__ src, int64_t n,
                                                    uint32_t* __restrict__ out) {
  uint32_t x = 0;
  const int64_t stride = int64_t(gridDim.x) * 256;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= (v[u][0] ^ v[u][1]) ^ (v[u][2] ^ v[u][3]);
  }
  for (; i < n; i += stride) {
    const u32x4 a = src[i];
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  x ^= __shfl_xor(x, 1);
  if (threadIdx.x == 0) out[blockIdx.x] = x;
}

}  // namespace

size_t probe_scratch_bytes() { return size_t(kProbeWG) * (4 + 16); }

hipError_t probe_mfma(int zero, int64_t iters, void* scratch, hipStream_t s, double* tflops,
                      double* clock_ghz) {
  float* out = static_cast<float*>(scratch);
  uint64_t* clk = reinterpret_cast<uint64_t*>(static_cast<char*>(scratch) + size_t(kProbeWG) * 4);
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) {
    // one untimed launch brings the clock to its sustained state
    hipLaunchKernelGGL(k_probe_mfma, dim3(kProbeWG), dim3(256), 0, s, iters, zero, out, clk);
    e = hipEventRecord(a, s);
    hipLaunchKernelGGL(k_probe_mfma, dim3(kProbeWG), dim3(256), 0, s, iters, zero, out, clk);
    if (e == hipSuccess) e = hipEventRecord(b, s);
    if (e == hipSuccess) e = hipGetLastError();
  }
  std::vector<uint64_t> host(2 * size_t(kProbeWG));
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (e == hipSuccess)
    e = hipMemcpyAsync(host.data(), clk, host.size() * 8, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  int dev = 0, wall_khz = 0;
  if (e == hipSuccess) e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (a != nullptr) (void)hipEventDestroy(a);
  if (b != nullptr) (void)hipEventDestroy(b);
  if (e != hipSuccess) return e;
  const double flops = double(kProbeWG) * 4.0 * double(iters) * 128.0 * (16.0 * 16.0 * 32.0 * 2.0);
  *tflops = flops / (double(ms) * 1e-3) / 1e12;
  std::vector<double> ratio;
  for (int w = 0; w < kProbeWG; ++w)
    if (host[2 * w + 1] > 0) ratio.push_back(double(host[2 * w]) / double(host[2 * w + 1]));
  std::sort(ratio.begin(), ratio.end());
  *clock_ghz = ratio.empty() ? 0.0 : ratio[ratio.size() / 2] * double(wall_khz) * 1e3 / 1e9;
  return hipSuccess;
}

hipError_t probe_read(const void* buf, size_t bytes, void* scratch, hipStream_t s, double* gbs) {
  const int64_t n = int64_t(bytes / 16);
  const unsigned grid = 256 * 8;
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  float ms = 0.f;
  if (e == hipSuccess) {
    hipLaunchKernelGGL(k_probe_read, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(buf), n,
                       static_cast<uint32_t*>(scratch));
    e = hipEventRecord(a, s);
    for (int r = 0; r < 5; ++r)
      hipLaunchKernelGGL(k_probe_read, dim3(grid), dim3(256), 0, s, static_cast<const u32x4*>(buf),
                         n, static_cast<uint32_t*>(scratch));
    if (e == hipSuccess) e = hipEventRecord(b, s);
    if (e == hipSuccess) e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (a != nullptr) (void)hipEventDestroy(a);
  if (b != nullptr) (void)hipEventDestroy(b);
  if (e != hipSuccess) return e;
  *gbs = double(n) * 16.0 * 5.0 / (double(ms) * 1e-3) / 1e9;
  return hipSuccess;
}

}  // namespace flp
