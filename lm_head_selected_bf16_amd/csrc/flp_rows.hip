// Row selection for the indexed variants (PR #547 page, section "What",
// indexed semantics: full output row shape, a duplicated id selects its row
// once, an id outside the batch is ignored, rows left out get zero results and
// zero gradients).
//
// A list of row ids becomes a byte mask over the batch (k_mark: every listed
// in-range id writes 1 to its row's byte, so duplicates are idempotent by
// construction).  The linear variants then compact the mask into the
// ascending list of selected rows (k_compact, one workgroup), copy those rows
// and their per-row inputs into a dense block (k_gather), run the dense
// kernels on the block and put the results back in full shape with zeros for
// the rows left out (k_scatter_rows, k_scatter_hidden).  The operator on
// materialised logits reads the mask directly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flp_launch.h"

namespace flp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t load_id(const void* ids, bool i64, int64_t i) {
  return i64 ? reinterpret_cast<const int64_t*>(ids)[i]
             : int64_t(reinterpret_cast<const int32_t*>(ids)[i]);
}

constexpr int kStrideBlocks = 4096;  // grid cap of the grid-stride kernels

__global__ __launch_bounds__(256) void k_zero_words(uint32_t* __restrict__ dst, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    dst[i] = 0u;
}

__global__ __launch_bounds__(256) void k_mark(const void* __restrict__ rows, int r64, int64_t n_rows,
                                              int64_t N, uint8_t* __restrict__ mask) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n_rows;
       i += int64_t(gridDim.x) * 256) {
    const int64_t r = load_id(rows, r64 != 0, i);
    if (r >= 0 && r < N) mask[r] = 1;
  }
}

// One workgroup of 1024 threads walks the mask in blocks of 4096 rows (four
// consecutive rows per thread): a wave-level inclusive scan of the per-thread
// counts, the 16 wave totals through LDS, then every selected row gets its
// compact position and is entered in sel.  Rows left out get position -1; sel
// entries past the count are set to -1.
__global__ __launch_bounds__(1024) void k_compact(const uint8_t* __restrict__ mask, int64_t N,
                                                  int32_t* __restrict__ pos,
                                                  int32_t* __restrict__ sel, int64_t cap) {
  __shared__ int32_t wsum[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int64_t base = 0;
  for (int64_t r0 = 0; r0 < N; r0 += 4096) {
    const int64_t r = r0 + 4 * int64_t(t);
    int m[4];
    int c = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      m[k] = (r + k < N) ? int(mask[r + k] != 0) : 0;
      c += m[k];
    }
    int x = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[w] = x;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int s = wsum[j];
      before += (j < w) ? s : 0;
      total += s;
    }
    int64_t p = base + before + (x - c);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (r + k >= N) break;
      pos[r + k] = m[k] ? int32_t(p) : -1;
      if (m[k]) sel[p++] = int32_t(r + k);
    }
    base += total;
    __syncthreads();  // wsum is rewritten by the next block
  }
  for (int64_t j = base + t; j < cap; j += 1024) sel[j] = -1;
}

// One workgroup per compact row j: copy hidden row sel[j] (zeros for a padding
// entry) and the row's per-row inputs.  A padding entry gets target -1, so the
// dense kernels treat it as an ignored row.
__global__ __launch_bounds__(256) void k_gather(GatherArgs a) {
  const int64_t j = blockIdx.x;
  const int32_t r = a.sel[j];
  const int64_t nvec = a.row_bytes / 16;
  u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(a.h_c) + j * a.row_bytes);
  if (r >= 0) {
    const u32x4* src =
        reinterpret_cast<const u32x4*>(static_cast<const char*>(a.hidden) + int64_t(r) * a.row_bytes);
    for (int64_t i = threadIdx.x; i < nvec; i += 256) dst[i] = src[i];
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = threadIdx.x; i < nvec; i += 256) dst[i] = z;
  }
  if (threadIdx.x == 0) {
    a.t_c[j] = r >= 0 ? load_id(a.targets, a.t64 != 0, r) : int64_t(-1);
    if (a.temp_c != nullptr) a.temp_c[j] = r >= 0 ? a.temperature[r] : 1.0f;
    if (a.g_c != nullptr) a.g_c[j] = r >= 0 ? a.grad_out[r] : 0.0f;
    if (a.lse_c != nullptr) a.lse_c[j] = r >= 0 ? a.lse[r] : 0.0f;
  }
}

__global__ __launch_bounds__(256) void k_scatter_rows(const int32_t* __restrict__ pos, int64_t N,
                                                      const float* __restrict__ logp_c,
                                                      const float* __restrict__ lse_c,
                                                      float* __restrict__ logp,
                                                      float* __restrict__ lse) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= N) return;
  const int32_t p = pos[i];
  logp[i] = p >= 0 ? logp_c[p] : 0.0f;
  if (lse != nullptr) lse[i] = p >= 0 ? lse_c[p] : 0.0f;
}

// One workgroup per output row.
__global__ __launch_bounds__(256) void k_scatter_hidden(const int32_t* __restrict__ pos,
                                                        const u32x4* __restrict__ dh_c,
                                                        int64_t nvec, u32x4* __restrict__ dh) {
  const int64_t r = blockIdx.x;
  const int32_t p = pos[r];
  u32x4* dst = dh + r * nvec;
  if (p >= 0) {
    const u32x4* src = dh_c + int64_t(p) * nvec;
    for (int64_t i = threadIdx.x; i < nvec; i += 256) dst[i] = src[i];
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = threadIdx.x; i < nvec; i += 256) dst[i] = z;
  }
}

unsigned stride_grid(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return unsigned(b < kStrideBlocks ? (b > 0 ? b : 1) : kStrideBlocks);
}

}  // namespace

hipError_t launch_zero(void* dst, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  ProfScope ps(FLP_K_ROWS, s);
  const int64_t n = int64_t(bytes / 4);
  hipLaunchKernelGGL(k_zero_words, dim3(stride_grid(n)), dim3(256), 0, s,
                     static_cast<uint32_t*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_select(const void* rows, bool r64, int64_t n_rows, int64_t N, uint8_t* mask,
                         int32_t* pos, int32_t* sel, int64_t cap, hipStream_t s) {
  hipError_t e = launch_zero(mask, align_up(size_t(N)), s);
  if (e != hipSuccess) return e;
  ProfScope ps(FLP_K_ROWS, s);
  if (n_rows > 0)
    hipLaunchKernelGGL(k_mark, dim3(stride_grid(n_rows)), dim3(256), 0, s, rows, int(r64), n_rows,
                       N, mask);
  if (pos != nullptr)
    hipLaunchKernelGGL(k_compact, dim3(1), dim3(1024), 0, s, mask, N, pos, sel, cap);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, int64_t cap, hipStream_t s) {
  if (cap <= 0) return hipSuccess;
  ProfScope ps(FLP_K_ROWS, s);
  hipLaunchKernelGGL(k_gather, dim3(unsigned(cap)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const int32_t* pos, int64_t N, const float* logp_c,
                               const float* lse_c, float* logp, float* lse, hipStream_t s) {
  ProfScope ps(FLP_K_ROWS, s);
  hipLaunchKernelGGL(k_scatter_rows, dim3(unsigned((N + 255) / 256)), dim3(256), 0, s, pos, N,
                     logp_c, lse_c, logp, lse);
  return hipGetLastError();
}

hipError_t launch_scatter_hidden(const int32_t* pos, int64_t N, const void* dh_c, size_t row_bytes,
                                 void* dh, hipStream_t s) {
  ProfScope ps(FLP_K_ROWS, s);
  hipLaunchKernelGGL(k_scatter_hidden, dim3(unsigned(N)), dim3(256), 0, s, pos,
                     static_cast<const u32x4*>(dh_c), int64_t(row_bytes / 16),
                     static_cast<u32x4*>(dh));
  return hipGetLastError();
}

}  // namespace flp
