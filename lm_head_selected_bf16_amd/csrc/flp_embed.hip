// Untied embedding lookup and its deterministic grad_weight ("Feat/nemotron h
// lm head logprob cuda", PR #555 summary bullets: an untied embedding lookup
// whose grad_weight is a sorted-segment deterministic reduction; its Known
// issues note that the pages' version accumulates repeated ids in BF16 and
// misses FP64 parity, so here every segment accumulates in fp32 and rounds
// once).
//
//   out[i]      = E[ids[i]]                 (a zero row for ids outside [0, V))
//   d_E[v]      = sum over tokens i with ids[i] == v of grad[i], in ascending i
//
// The backward sorts the (id, token) pairs by id with a stable LSD radix sort
// (8-bit digits, blocks of 256 keys; ranks inside a block come from an
// in-order count, so the sort is deterministic) and finds each id's segment in
// the sorted list.  The sorted list is then cut into fixed groups of 32
// positions, one workgroup each, so a frequent id does not serialise on one
// wave: inside a group every run of equal ids is summed in fp32 in token order;
// a segment that spans several groups adds its per-group pieces in group order.
// Every order is fixed by the sorted list: the output is bitwise reproducible.
//
// The rows of ids that do not occur are most of d_E's bytes.  The sort's
// scatter passes occupy few compute units, so their launches (and the group
// pass) carry extra "rider" workgroups that write those zero rows alongside;
// the first sort pass marks the ids that occur before any rider runs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flp_launch.h"

namespace flp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSortBlock = int(kEmbSortBlock);  // keys per block of a radix pass (one per thread)

__device__ __forceinline__ int64_t load_id(const void* ids, bool i64, int64_t i) {
  return i64 ? reinterpret_cast<const int64_t*>(ids)[i]
             : int64_t(reinterpret_cast<const int32_t*>(ids)[i]);
}

// One wave per token row, four rows per workgroup: 16-byte copies.
__global__ __launch_bounds__(256) void k_embed_fwd(const u32x4* __restrict__ weight,
                                                   const void* __restrict__ ids, int i64,
                                                   int64_t N, int64_t V, int64_t row_vec,
                                                   u32x4* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t i = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (i >= N) return;
  const int64_t v = load_id(ids, i64 != 0, i);
  u32x4* dst = out + i * row_vec;
  if (v >= 0 && v < V) {
    const u32x4* src = weight + v * row_vec;
    for (int64_t c = lane; c < row_vec; c += 64) dst[c] = src[c];
  } else {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t c = lane; c < row_vec; c += 64) dst[c] = z;
  }
}

// Zero rows of ids that do not occur, written by workgroups appended to another
// kernel's grid: workgroup r of the riders clears rows v0 + 4 r .. v0 + 4 r + 3 of
// [v0, v1) (one wave per row) whose id is unmarked.  seg_end[v] != 0 marks an id
// that occurs (set by the first sort pass, later overwritten by its segment end,
// which is never 0).
struct ZeroRider {
  u32x4* dW;               // d_E [V][row_vec]
  const int32_t* seg_end;  // [V]
  int64_t v0, v1;          // rows of this launch
  int64_t row_vec;         // 16-byte chunks per d_E row
  int64_t blocks() const { return (v1 - v0 + 3) / 4; }
};

__device__ __forceinline__ void ride(const ZeroRider& z, int64_t r) {
  const int64_t v = z.v0 + r * 4 + (threadIdx.x >> 6);
  if (v >= z.v1 || z.seg_end[v] != 0) return;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4* row = z.dW + v * z.row_vec;
  for (int64_t c = threadIdx.x & 63; c < z.row_vec; c += 64) __builtin_nontemporal_store(zero, row + c);
}

// Sort keys: the id, or V for an id outside [0, V) (those sort last and are
// dropped); values: the token index.  The same grid clears the [V] segment
// bounds (an id that does not occur keeps an empty segment).
__global__ __launch_bounds__(256) void k_sort_init(const void* __restrict__ ids, int i64, int64_t N,
                                                   int64_t V, uint32_t* __restrict__ keys,
                                                   int32_t* __restrict__ vals,
                                                   int32_t* __restrict__ seg_begin,
                                                   int32_t* __restrict__ seg_end) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < V) {
    seg_begin[i] = 0;
    seg_end[i] = 0;
  }
  if (i >= N) return;
  const int64_t v = load_id(ids, i64 != 0, i);
  keys[i] = (v >= 0 && v < V) ? uint32_t(v) : uint32_t(V);
  vals[i] = int32_t(i);
}

// Per-block digit counts, stored digit-major: hist[d * n_blocks + b].  With
// `mark` set (the first pass), also marks every id that occurs: mark[id] = 1.
__global__ __launch_bounds__(256) void k_sort_hist(const uint32_t* __restrict__ keys, int64_t n,
                                                   int shift, int64_t n_blocks,
                                                   int32_t* __restrict__ hist,
                                                   int32_t* __restrict__ mark, int64_t V) {
  __shared__ int32_t cnt[256];
  const int t = threadIdx.x;
  const int64_t b = blockIdx.x;
  cnt[t] = 0;
  __syncthreads();
  for (int k = t; k < kSortBlock; k += 256) {
    const int64_t i = b * kSortBlock + k;
    if (i < n) {
      const uint32_t key = keys[i];
      atomicAdd(&cnt[(key >> shift) & 255u], 1);
      if (mark != nullptr && int64_t(key) < V) mark[key] = 1;
    }
  }
  __syncthreads();
  hist[int64_t(t) * n_blocks + b] = cnt[t];
}

// Stable scatter of one radix pass.  A block holds 256 consecutive keys.  Its
// offset for digit d is the count of all keys with a smaller digit plus the
// count of keys with digit d in earlier blocks (thread d sums its digit's
// counts, then an exclusive scan over the 256 digit totals in LDS); a key's
// place adds the number of keys before it in the block with the same digit.
__global__ __launch_bounds__(256) void k_sort_scatter(const uint32_t* __restrict__ kin,
                                                      const int32_t* __restrict__ vin, int64_t n,
                                                      int shift, int64_t n_blocks,
                                                      const int32_t* __restrict__ hist,
                                                      uint32_t* __restrict__ kout,
                                                      int32_t* __restrict__ vout, ZeroRider z) {
  if (int64_t(blockIdx.x) >= n_blocks) {
    ride(z, int64_t(blockIdx.x) - n_blocks);
    return;
  }
  __shared__ int32_t tot[256];
  __shared__ int32_t run[256];
  __shared__ int32_t dig[256];
  const int t = threadIdx.x;
  const int64_t b = blockIdx.x;
  int32_t before = 0, all = 0;
  const int32_t* h = hist + int64_t(t) * n_blocks;
  for (int64_t q0 = 0; q0 < n_blocks; q0 += 8) {  // eight counts in flight
    int32_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = (q0 + u < n_blocks) ? h[q0 + u] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      before += (q0 + u < b) ? c[u] : 0;
      all += c[u];
    }
  }
  tot[t] = all;
  __syncthreads();
  if (t < 64) {  // exclusive scan of the 256 digit totals by one wave, 4 per lane
    int32_t x[4], sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = tot[4 * t + k];
      sum += x[k];
    }
    int32_t inc = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t y = __shfl_up(inc, off);
      if (t >= off) inc += y;
    }
    int32_t p = inc - sum;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      run[4 * t + k] = p;
      p += x[k];
    }
  }
  __syncthreads();
  run[t] += before;
  const int64_t i = b * kSortBlock + t;
  const bool valid = i < n;
  const uint32_t key = valid ? kin[i] : 0u;
  const int d = valid ? int((key >> shift) & 255u) : -1;
  dig[t] = d;
  __syncthreads();
  int r = 0;
  for (int u = 0; u < t; ++u) r += (dig[u] == d) ? 1 : 0;
  if (valid) {
    const int32_t pos = run[d] + r;
    kout[pos] = key;
    vout[pos] = vin[i];
  }
}

// Segment of each id in the sorted keys: [seg_begin[v], seg_end[v]) (both
// zero-filled before, so an id that does not occur has an empty segment).
__global__ __launch_bounds__(256) void k_seg_bounds(const uint32_t* __restrict__ keys, int64_t n,
                                                    int64_t V, int32_t* __restrict__ seg_begin,
                                                    int32_t* __restrict__ seg_end) {
  const int64_t p = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (p >= n) return;
  const uint32_t k = keys[p];
  if (int64_t(k) >= V) return;
  if (p == 0 || keys[p - 1] != k) seg_begin[k] = int32_t(p);
  if (p == n - 1 || keys[p + 1] != k) seg_end[k] = int32_t(p + 1);
}

template <int SIZE>
__device__ __forceinline__ void unpack_chunk(const u32x4& v, float* x, bool f16);

template <>
__device__ __forceinline__ void unpack_chunk<2>(const u32x4& v, float* x, bool f16) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (f16) {
      x[2 * k] = float(__builtin_bit_cast(_Float16, uint16_t(v[k] & 0xFFFFu)));
      x[2 * k + 1] = float(__builtin_bit_cast(_Float16, uint16_t(v[k] >> 16)));
    } else {
      x[2 * k] = __uint_as_float(v[k] << 16);
      x[2 * k + 1] = __uint_as_float(v[k] & 0xFFFF0000u);
    }
  }
}

template <>
__device__ __forceinline__ void unpack_chunk<4>(const u32x4& v, float* x, bool) {
#pragma unroll
  for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(v[k]);
}

__device__ __forceinline__ uint32_t round_bf16(float f) {  // round to nearest even
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0xFFFFu) ? 0x40u : 0u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t round_16(float f, bool f16) {
  return f16 ? uint32_t(__builtin_bit_cast(uint16_t, _Float16(f))) : round_bf16(f);
}

template <int XS, bool OUT_F32>
__device__ __forceinline__ void store_chunk(const float* acc, void* dW, int64_t v, int64_t row_vec,
                                            int64_t c, bool f16) {
  constexpr int EPC = 16 / XS;
  if constexpr (OUT_F32) {
    float* out = static_cast<float*>(dW) + (v * row_vec + c) * EPC;
#pragma unroll
    for (int k = 0; k < EPC; k += 4) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) w[j] = __float_as_uint(acc[k + j]);
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(out + k));
    }
  } else {
    u32x4 w;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = round_16(acc[2 * k], f16) | (round_16(acc[2 * k + 1], f16) << 16);
    __builtin_nontemporal_store(w, static_cast<u32x4*>(dW) + v * row_vec + c);
  }
}

// Pass A: one workgroup per group of kSegGroup consecutive sorted positions.  The
// group is cut into runs of equal id; each run is summed in fp32 in sorted
// (= ascending token) order.  A run that is its id's whole segment is written to
// d_W at once; a run that starts at the group's first position goes to the
// group's head slot, any other run that reaches past the group to its tail slot
// (a group holds at most one of each).  Thread t owns the 16-byte chunks
// t, t + 256, ... of a row.
constexpr int kSegGroup = int(kEmbSegGroup);

template <int XS, bool OUT_F32>
__device__ __forceinline__ void finish_run(const float* acc, int64_t j, int a, bool whole,
                                           uint32_t k, float* head, float* tail, void* dW,
                                           int64_t row_vec, int64_t c, bool f16) {
  constexpr int EPC = 16 / XS;
  if (whole) {
    store_chunk<XS, OUT_F32>(acc, dW, int64_t(k), row_vec, c, f16);
  } else {
    float* slot = (a == 0 ? head : tail) + (j * row_vec + c) * EPC;
#pragma unroll
    for (int q = 0; q < EPC; q += 4) {
      u32x4 w;
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = __float_as_uint(acc[q + u]);
      *reinterpret_cast<u32x4*>(slot + q) = w;
    }
  }
}

template <int XS, bool OUT_F32>
__global__ __launch_bounds__(256) void k_embed_runs(const u32x4* __restrict__ grad, int f16,
                                                    const uint32_t* __restrict__ keys,
                                                    const int32_t* __restrict__ tok,
                                                    const int32_t* __restrict__ seg_begin,
                                                    const int32_t* __restrict__ seg_end, int64_t N,
                                                    int64_t V, int64_t row_vec,
                                                    float* __restrict__ head,
                                                    float* __restrict__ tail, void* __restrict__ dW,
                                                    int64_t n_groups, ZeroRider z) {
  if (int64_t(blockIdx.x) >= n_groups) {
    ride(z, int64_t(blockIdx.x) - n_groups);
    return;
  }
  constexpr int EPC = 16 / XS;
  __shared__ uint32_t skey[kSegGroup];
  __shared__ int32_t stok[kSegGroup];
  __shared__ uint8_t whole[kSegGroup];  // the run ending before position p is its whole segment
  const int64_t j = blockIdx.x;
  const int64_t s0 = j * kSegGroup;
  const int n = int((N - s0) < kSegGroup ? (N - s0) : kSegGroup);
  if (threadIdx.x < kSegGroup) {
    // positions past the batch and dropped ids read as key V (never summed)
    const bool in = int(threadIdx.x) < n;
    const uint32_t k = in ? keys[s0 + threadIdx.x] : uint32_t(V);
    const bool live = in && int64_t(k) < V;
    skey[threadIdx.x] = k;
    stok[threadIdx.x] = live ? tok[s0 + threadIdx.x] : -1;
    // a run inside the group is the whole segment iff the segment starts at or after
    // the group start and ends at or before the group end
    whole[threadIdx.x] =
        live ? uint8_t(seg_begin[k] >= s0 && seg_end[k] <= s0 + kSegGroup) : uint8_t(0);
  }
  __syncthreads();
  // summed positions: the prefix of the group with ids in [0, V) (dropped ids sort last)
  int m = 0;
  while (m < n && int64_t(skey[m]) < V) ++m;
  for (int64_t c = threadIdx.x; c < row_vec; c += 256) {
    // every row of the group in flight at once, then the runs in order
    u32x4 x4[kSegGroup];
#pragma unroll
    for (int p = 0; p < kSegGroup; ++p) {
      const int32_t t = stok[p];
      x4[p] = grad[int64_t(t < 0 ? 0 : t) * row_vec + c];
    }
    float acc[EPC];
#pragma unroll
    for (int q = 0; q < EPC; ++q) acc[q] = 0.0f;
    int a = 0;
#pragma unroll
    for (int p = 0; p < kSegGroup; ++p) {
      if (p < m) {
        if (p > a && skey[p] != skey[p - 1]) {
          finish_run<XS, OUT_F32>(acc, j, a, whole[a] != 0, skey[p - 1], head, tail, dW,
                                  row_vec, c, f16 != 0);
#pragma unroll
          for (int q = 0; q < EPC; ++q) acc[q] = 0.0f;
          a = p;
        }
        float x[EPC];
        unpack_chunk<XS>(x4[p], x, f16 != 0);
#pragma unroll
        for (int q = 0; q < EPC; ++q) acc[q] += x[q];
      }
    }
    if (m > a)  // the group's last run
      finish_run<XS, OUT_F32>(acc, j, a, whole[a] != 0, skey[a], head, tail, dW, row_vec, c,
                              f16 != 0);
  }
}

// Pass B: an id whose segment spans several groups adds its pieces in group
// order (the first group's head or tail slot, then the head slots of the
// following groups); an id inside one group was written by pass A, and an id
// that does not occur by a zero-row rider.  Workgroup b of B tests the ids b,
// b + B, ..., one per thread (the stride spreads frequent ids, which are often
// neighbours, over many workgroups), lists the spanning ones in LDS, then
// combines them one after another with all 256 threads, eight pieces in flight.
template <int XS, bool OUT_F32>
__global__ __launch_bounds__(256) void k_embed_rows(const int32_t* __restrict__ seg_begin,
                                                    const int32_t* __restrict__ seg_end,
                                                    int64_t V, int64_t row_vec,
                                                    const float* __restrict__ head,
                                                    const float* __restrict__ tail, int f16,
                                                    void* __restrict__ dW) {
  constexpr int EPC = 16 / XS;
  __shared__ int32_t list[256];
  __shared__ int32_t count;
  const int t = threadIdx.x;
  const int64_t v_t = int64_t(blockIdx.x) + int64_t(t) * gridDim.x;
  if (t == 0) count = 0;
  __syncthreads();
  if (v_t < V) {
    const int32_t b = seg_begin[v_t], e = seg_end[v_t];
    if (e > b && b / kSegGroup != (e - 1) / kSegGroup) list[atomicAdd(&count, 1)] = t;
  }
  __syncthreads();
  const int n = count;
  for (int k = 0; k < n; ++k) {
    const int64_t v = int64_t(blockIdx.x) + int64_t(list[k]) * gridDim.x;
    const int64_t b = seg_begin[v], e = seg_end[v];
    const int64_t g0 = b / kSegGroup, g1 = (e - 1) / kSegGroup;
    const float* first = (b == g0 * kSegGroup) ? head : tail;
    for (int64_t c = t; c < row_vec; c += 256) {
      float acc[EPC];
      const float* f = first + (g0 * row_vec + c) * EPC;
#pragma unroll
      for (int q = 0; q < EPC; ++q) acc[q] = f[q];
      int64_t g = g0 + 1;
      for (; g + 8 <= g1 + 1; g += 8) {  // eight pieces in flight, added in group order
        float x[8][EPC];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float* h = head + ((g + u) * row_vec + c) * EPC;
#pragma unroll
          for (int q = 0; q < EPC; ++q) x[u][q] = h[q];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int q = 0; q < EPC; ++q) acc[q] += x[u][q];
      }
      for (; g <= g1; ++g) {
        const float* h = head + (g * row_vec + c) * EPC;
#pragma unroll
        for (int q = 0; q < EPC; ++q) acc[q] += h[q];
      }
      store_chunk<XS, OUT_F32>(acc, dW, v, row_vec, c, f16 != 0);
    }
  }
}

}  // namespace

int embed_sort_passes(int64_t V) {
  int bits = 0;
  while ((uint64_t(V) >> bits) != 0) ++bits;  // keys run up to V (the dropped-id key)
  return (bits + 7) / 8;
}

hipError_t launch_embedding_forward(flp_dtype x, const void* weight, const void* ids, bool i64,
                                    int64_t N, int64_t D, int64_t V, void* out, hipStream_t s) {
  ProfScope ps(FLP_K_EMBEDDING, s);
  const int64_t row_vec = D * int64_t(dtype_size(x)) / 16;
  hipLaunchKernelGGL(k_embed_fwd, dim3(unsigned((N + 3) / 4)), dim3(256), 0, s,
                     static_cast<const u32x4*>(weight), ids, int(i64), N, V, row_vec,
                     static_cast<u32x4*>(out));
  return hipGetLastError();
}

hipError_t launch_embedding_backward(const EmbedBwdArgs& a, hipStream_t s) {
  ProfScope ps(FLP_K_EMBEDDING, s);
  const int64_t N = a.N, V = a.V;
  const int64_t n_blocks = (N + kSortBlock - 1) / kSortBlock;
  const int64_t init_n = N > V ? N : V;
  hipLaunchKernelGGL(k_sort_init, dim3(unsigned((init_n + 255) / 256)), dim3(256), 0, s, a.ids,
                     int(a.i64), N, V, a.keys[0], a.vals[0], a.seg_begin, a.seg_end);
  const int passes = embed_sort_passes(V);
  // Zero rows ride on the scatter launches (latency-bound, with most compute
  // units idle) and on the group pass: the group pass takes the upper half of
  // the rows, the scatters share the lower half evenly.
  ZeroRider z{};
  z.dW = static_cast<u32x4*>(a.d_weight);
  z.seg_end = a.seg_end;
  z.row_vec = a.D * int64_t(dtype_size(a.dw)) / 16;
  const int64_t lower = V - V / 2;
  const int n_sort_slices = passes;
  int slice = 0;
  auto next_slice = [&]() {
    ZeroRider r = z;
    r.v0 = lower * slice / n_sort_slices;
    r.v1 = lower * (slice + 1) / n_sort_slices;
    ++slice;
    return r;
  };
  for (int p = 0; p < passes; ++p) {
    const int src = p & 1, dst = src ^ 1;
    hipLaunchKernelGGL(k_sort_hist, dim3(unsigned(n_blocks)), dim3(256), 0, s, a.keys[src], N,
                       8 * p, n_blocks, a.hist, p == 0 ? a.seg_end : nullptr, V);
    const ZeroRider zs = next_slice();
    hipLaunchKernelGGL(k_sort_scatter, dim3(unsigned(n_blocks + zs.blocks())), dim3(256), 0, s,
                       a.keys[src], a.vals[src], N, 8 * p, n_blocks, a.hist, a.keys[dst],
                       a.vals[dst], zs);
  }
  const int fin = passes & 1;
  hipLaunchKernelGGL(k_seg_bounds, dim3(unsigned((N + 255) / 256)), dim3(256), 0, s, a.keys[fin],
                     N, V, a.seg_begin, a.seg_end);
  const int64_t row_vec = a.D * int64_t(dtype_size(a.x)) / 16;
  const int64_t n_groups = (N + kSegGroup - 1) / kSegGroup;
  ZeroRider zr = z;
  zr.v0 = lower;
  zr.v1 = V;
  const dim3 ga(unsigned(n_groups + zr.blocks())), gb(unsigned((V + 255) / 256));
  const int f16 = a.x == FLP_F16 ? 1 : 0;
  const u32x4* g = static_cast<const u32x4*>(a.grad);
  const uint32_t* keys = a.keys[fin];
  const int32_t* tok = a.vals[fin];
  if (a.x == FLP_F32) {
    hipLaunchKernelGGL((k_embed_runs<4, true>), ga, dim3(256), 0, s, g, 0, keys, tok, a.seg_begin,
                       a.seg_end, N, V, row_vec, a.head, a.tail, a.d_weight, n_groups, zr);
    hipLaunchKernelGGL((k_embed_rows<4, true>), gb, dim3(256), 0, s, a.seg_begin, a.seg_end, V,
                       row_vec, a.head, a.tail, 0, a.d_weight);
  } else if (a.dw == FLP_F32) {
    hipLaunchKernelGGL((k_embed_runs<2, true>), ga, dim3(256), 0, s, g, f16, keys, tok,
                       a.seg_begin, a.seg_end, N, V, row_vec, a.head, a.tail, a.d_weight,
                       n_groups, zr);
    hipLaunchKernelGGL((k_embed_rows<2, true>), gb, dim3(256), 0, s, a.seg_begin, a.seg_end, V,
                       row_vec, a.head, a.tail, f16, a.d_weight);
  } else {
    hipLaunchKernelGGL((k_embed_runs<2, false>), ga, dim3(256), 0, s, g, f16, keys, tok,
                       a.seg_begin, a.seg_end, N, V, row_vec, a.head, a.tail, a.d_weight,
                       n_groups, zr);
    hipLaunchKernelGGL((k_embed_rows<2, false>), gb, dim3(256), 0, s, a.seg_begin, a.seg_end, V,
                       row_vec, a.head, a.tail, f16, a.d_weight);
  }
  return hipGetLastError();
}

}  // namespace flp
