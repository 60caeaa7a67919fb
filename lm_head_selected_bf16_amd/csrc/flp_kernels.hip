// gfx950 (CDNA4) kernels of the fused linear selected-token log-probability.
//
// Forward ("Fused Linear LogP" docs page, sections "Backends" and "Reference
// Semantics"): each workgroup computes one [BM x 256] tile of scaled logits
// z = (h W^T + b) / T with bf16 (or fp32) MFMA and fp32 accumulation, then
// folds the tile into a per-row (max, sum of exp) pair and picks up the target
// logit; a merge kernel folds the pairs of all vocabulary tiles in ascending
// order into lse and logp.  The [N, V] logits never reach HBM.
//
// Backward (PR #234, "Implementation details"; PR #555 summary): per row
// chunk, a dlogits kernel recomputes the same logit tiles and writes
// dz = G (onehot - exp(z - lse)) / T; two MFMA GEMMs give d_hidden = dz W and
// d_weight += dz^T hidden with a fixed ascending K order; d_bias partials are
// folded in ascending row-tile order.  No atomics anywhere.
//
// Register layout.  Every MFMA is issued as mfma(A = N-side fragment,
// B = M-side fragment), so lane l of a wave holds output row (l % 16) of a
// 16-row block and four consecutive output columns 4*(l / 16) + 0..3 of a
// 16-column block.  Both operand fragments are 16 bytes of K read from LDS at
// (row l % 16, 16-byte chunk l / 16).
//
// Batch invariance.  For every logit the MFMA chain over K is the same
// (ascending 128-byte stages, same instruction, same lane placement of K), and
// the per-row reductions over a 256-column vocabulary tile use one fixed tree
// defined by column positions only: within a lane over its 4 columns and 4
// column blocks, across the four 16-lane groups by xor-butterfly, then across
// the four 64-column waves in ascending order.  No kernel's per-row arithmetic
// depends on N, the row tile size or the row's position.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <math.h>

#include "flp_launch.h"

namespace flp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kStageBytes = 128;  // bytes of K per operand row per pipeline stage
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kGroupM = 8;        // row tiles per scheduling group

struct BF16 {
  static constexpr int kSize = 2;
};
struct F32 {
  static constexpr int kSize = 4;
};

// LDS tiles hold rows of 8 16-byte chunks (one 128-byte stage of K).  Chunk c
// of row r lives at chunk position c ^ f(r) to spread MFMA fragment reads and
// transposed writes over the banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 64 bytes of K per lane quad: one bf16 16x16x32 MFMA, or four fp32 16x16x4
// MFMAs over the same 16 bytes per lane (K index 4g + t in instruction t).
template <class E>
__device__ __forceinline__ void mma64(f32x4_t& c, const u32x4& a, const u32x4& b);

template <>
__device__ __forceinline__ void mma64<BF16>(f32x4_t& c, const u32x4& a, const u32x4& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                               __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma64<F32>(f32x4_t& c, const u32x4& a, const u32x4& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Store four consecutive fp32 values as the element type.
template <class E>
__device__ __forceinline__ void store4(void* base, int64_t idx, const f32x4_t& v);

template <>
__device__ __forceinline__ void store4<BF16>(void* base, int64_t idx, const f32x4_t& v) {
  u32x2 w;
  w.x = bf16_bits_rne(v.x) | (bf16_bits_rne(v.y) << 16);
  w.y = bf16_bits_rne(v.z) | (bf16_bits_rne(v.w) << 16);
  *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + idx) = w;
}

template <>
__device__ __forceinline__ void store4<F32>(void* base, int64_t idx, const f32x4_t& v) {
  *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(base) + idx) = v;
}

__device__ __forceinline__ int64_t load_target(const void* t, int t64, int64_t i) {
  return t64 ? reinterpret_cast<const int64_t*>(t)[i] : int64_t(reinterpret_cast<const int32_t*>(t)[i]);
}

// Workgroup id -> (row tile, column tile).  Workgroups are dispatched
// round-robin over the 8 XCDs, so ids are first regrouped so that each XCD
// receives a contiguous run of logical tiles (sharing its L2), then the run is
// walked in groups of kGroupM row tiles, row tile fastest, so that the
// workgroups resident at one time share both operand tiles.
__device__ __forceinline__ void tile_of(int bid, int nbm, int nbn, int& tm, int& tn) {
  const int total = nbm * nbn;
  const int per = total >> 3;
  int lin = bid;
  if (bid < per * 8) lin = (bid & 7) * per + (bid >> 3);
  const int width = kGroupM * nbn;
  const int grp = lin / width;
  const int first = grp * kGroupM;
  const int gm = min(nbm - first, kGroupM);
  const int in = lin - grp * width;
  tm = first + in % gm;
  tn = in / gm;
}

// ---- global -> LDS staging ------------------------------------------------------------

// Operand stored K-contiguous: row r at base + r * ld, K bytes [kb0, kb0 + 128).
template <int ROWS, int NT>
struct LoadK {
  static constexpr int kChunks = ROWS * 8;
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  u32x4 v[kPer];

  __device__ __forceinline__ void load(const void* base, int64_t ld, int64_t row0, int64_t nrows,
                                       int64_t kb0, int64_t kbytes, int tid) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + j * NT;
      const int r = idx >> 3, c = idx & 7;
      const int64_t row = row0 + r;
      const int64_t kb = kb0 + c * 16;
      u32x4 x = {0u, 0u, 0u, 0u};
      if ((kChunks % NT == 0 || idx < kChunks) && row < nrows && kb < kbytes)
        x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + row * ld + kb);
      v[j] = x;
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + j * NT;
      if (kChunks % NT == 0 || idx < kChunks) {
        const int r = idx >> 3, c = idx & 7;
        lds[r * 8 + swz(r, c)] = v[j];
      }
    }
  }
};

// Operand stored M-contiguous ([K][M] in memory): each thread reads an 8 x 8
// (bf16) or 4 x 4 (fp32) block of K rows x M columns and transposes it in
// registers so that LDS holds M rows of contiguous K, as for LoadK.
template <class E, int ROWS, int NT>
struct LoadT;

template <int ROWS, int NT>
struct LoadT<BF16, ROWS, NT> {
  static constexpr int kMC = ROWS / 8;            // 8-column chunks of M
  static constexpr int kBlocks = kMC * 8;         // x 8 groups of 8 K rows (64 K per stage)
  static constexpr int kPer = (kBlocks + NT - 1) / NT;
  u32x4 v[kPer][8];

  __device__ __forceinline__ void load(const void* base, int64_t ld, int64_t m0, int64_t mvalid,
                                       int64_t k0, int64_t kvalid, int tid) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + j * NT;
      const int mc = idx % kMC, kg = idx / kMC;
      const int64_t m = m0 + mc * 8;
      const bool live = (kBlocks % NT == 0 || idx < kBlocks) && m < mvalid;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t k = k0 + kg * 8 + q;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (live && k < kvalid)
          x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + k * ld + m * 2);
        v[j][q] = x;
      }
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + j * NT;
      if (kBlocks % NT == 0 || idx < kBlocks) {
        const int mc = idx % kMC, kg = idx / kMC;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int d = q >> 1;
          const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
          u32x4 o;
          o.x = __builtin_amdgcn_perm(v[j][1][d], v[j][0][d], sel);
          o.y = __builtin_amdgcn_perm(v[j][3][d], v[j][2][d], sel);
          o.z = __builtin_amdgcn_perm(v[j][5][d], v[j][4][d], sel);
          o.w = __builtin_amdgcn_perm(v[j][7][d], v[j][6][d], sel);
          const int r = mc * 8 + q;
          lds[r * 8 + swz(r, kg)] = o;
        }
      }
    }
  }
};

template <int ROWS, int NT>
struct LoadT<F32, ROWS, NT> {
  static constexpr int kMC = ROWS / 4;            // 4-column chunks of M
  static constexpr int kBlocks = kMC * 8;         // x 8 groups of 4 K rows (32 K per stage)
  static constexpr int kPer = (kBlocks + NT - 1) / NT;
  u32x4 v[kPer][4];

  __device__ __forceinline__ void load(const void* base, int64_t ld, int64_t m0, int64_t mvalid,
                                       int64_t k0, int64_t kvalid, int tid) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + j * NT;
      const int mc = idx % kMC, kg = idx / kMC;
      const int64_t m = m0 + mc * 4;
      const bool live = (kBlocks % NT == 0 || idx < kBlocks) && m < mvalid;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t k = k0 + kg * 4 + q;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (live && k < kvalid)
          x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) + k * ld + m * 4);
        v[j][q] = x;
      }
    }
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int idx = tid + j * NT;
      if (kBlocks % NT == 0 || idx < kBlocks) {
        const int mc = idx % kMC, kg = idx / kMC;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x4 o;
          o.x = v[j][0][q];
          o.y = v[j][1][q];
          o.z = v[j][2][q];
          o.w = v[j][3][q];
          const int r = mc * 4 + q;
          lds[r * 8 + swz(r, kg)] = o;
        }
      }
    }
  }
};

// ---- the MFMA K loop ----------------------------------------------------------------------

template <class E, int WMB, int WNB>
__device__ __forceinline__ void compute_stage(f32x4_t (&acc)[WMB][WNB], const u32x4* As,
                                              const u32x4* Bs, int arow0, int brow0, int i, int g) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4 af[WMB], bf[WNB];
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      const int r = arow0 + mb * 16 + i;
      af[mb] = As[r * 8 + swz(r, h * 4 + g)];
    }
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      const int r = brow0 + nb * 16 + i;
      bf[nb] = Bs[r * 8 + swz(r, h * 4 + g)];
    }
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) mma64<E>(acc[mb][nb], bf[nb], af[mb]);
  }
}

// Two LDS buffers per operand; global loads for stage s+1 are in flight in
// registers while stage s is multiplied.  One barrier per stage.
template <class E, int WMB, int WNB, class LoadFn, class StoreFn>
__device__ __forceinline__ void kloop(f32x4_t (&acc)[WMB][WNB], int nst, u32x4* sA0, u32x4* sA1,
                                      u32x4* sB0, u32x4* sB1, int arow0, int brow0, int lane,
                                      LoadFn&& load, StoreFn&& store) {
  const int i = lane & 15, g = lane >> 4;
  load(0);
  store(sA0, sB0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const bool more = st + 1 < nst;
    if (more) load(st + 1);
    const bool odd = st & 1;
    compute_stage<E, WMB, WNB>(acc, odd ? sA1 : sA0, odd ? sB1 : sB0, arow0, brow0, i, g);
    if (more) store(odd ? sA0 : sA1, odd ? sB0 : sB1);
    __syncthreads();
  }
}

// ---- logits tile shared by the forward and dlogits kernels ---------------------------------
//
// Workgroup = WAVES_M x 4 waves; wave (wm, wn) owns rows [wm*RW, wm*RW + RW) and the
// 64 vocabulary columns [wn*64, wn*64 + 64) of the BM x 256 tile.
template <class E, int BM, int WAVES_M>
struct LogitTile {
  static constexpr int NT = 256 * WAVES_M;
  static constexpr int BN = 256;
  static constexpr int RW = BM / WAVES_M;
  static constexpr int WMB = RW / 16;
  static constexpr int WNB = 4;
  static constexpr size_t kLds = size_t(2) * (BM + BN) * kStageBytes;
  static_assert(RW % 16 == 0, "rows per wave must be a multiple of 16");

  __device__ __forceinline__ static void run(f32x4_t (&acc)[WMB][WNB], const void* hidden,
                                             const void* weight, int64_t row0, int64_t nrows,
                                             int64_t col0, int64_t V, int64_t D, u32x4* smem) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 3, wm = wave >> 2;
    const int64_t kbytes = D * E::kSize;
    const int nst = int((kbytes + kStageBytes - 1) / kStageBytes);
    u32x4* sA0 = smem;
    u32x4* sA1 = smem + BM * 8;
    u32x4* sB0 = smem + 2 * BM * 8;
    u32x4* sB1 = sB0 + BN * 8;
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    LoadK<BM, NT> la;
    LoadK<BN, NT> lb;
    kloop<E, WMB, WNB>(
        acc, nst, sA0, sA1, sB0, sB1, wm * RW, wn * 64, lane,
        [&](int st) {
          la.load(hidden, kbytes, row0, nrows, int64_t(st) * kStageBytes, kbytes, tid);
          lb.load(weight, kbytes, col0, V, int64_t(st) * kStageBytes, kbytes, tid);
        },
        [&](u32x4* a, u32x4* b) {
          la.store(a, tid);
          lb.store(b, tid);
        });
  }
};

// ---- forward: logits tile -> per-row (max, sum of exp) partial + target logit -------------
template <class E, int BM, int WAVES_M>
__global__ __launch_bounds__(256 * WAVES_M) void k_fwd(FwdArgs p) {
  using Tile = LogitTile<E, BM, WAVES_M>;
  constexpr int RW = Tile::RW, WMB = Tile::WMB, WNB = Tile::WNB, NT = Tile::NT;
  extern __shared__ u32x4 smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 3, wm = wave >> 2, i = lane & 15, g = lane >> 4;
  const int nbm = int((p.N + BM - 1) / BM);
  const int nbn = int((p.V + 255) / 256);
  int tm, tn;
  tile_of(blockIdx.x, nbm, nbn, tm, tn);
  const int64_t row0 = int64_t(tm) * BM, col0 = int64_t(tn) * 256;

  f32x4_t acc[WMB][WNB];
  Tile::run(acc, p.hidden, p.weight, row0, p.N, col0, p.V, p.D, smem);

  float* red = reinterpret_cast<float*>(smem);  // [4][BM] row max, then [4][BM] row sums
  const int64_t cw = col0 + wn * 64;
  float bcol[WNB][4];
  bool cval[WNB][4];
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t c = cw + nb * 16 + 4 * g + r;
      cval[nb][r] = c < p.V;
      bcol[nb][r] = (p.bias != nullptr && c < p.V) ? p.bias[c] : 0.f;
    }

#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int rl = wm * RW + mb * 16 + i;
    const int64_t row = row0 + rl;
    const float invT = (p.temperature != nullptr && row < p.N) ? 1.0f / p.temperature[row] : 1.0f;
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float z = (acc[mb][nb][r] + bcol[nb][r]) * invT;
        z = cval[nb][r] ? z : -INFINITY;
        acc[mb][nb][r] = z;
        mx = fmaxf(mx, z);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (g == 0) red[wn * BM + rl] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int rl = wm * RW + mb * 16 + i;
    const int64_t row = row0 + rl;
    const float M = fmaxf(fmaxf(red[rl], red[BM + rl]), fmaxf(red[2 * BM + rl], red[3 * BM + rl]));
    float sb[WNB];
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      const float e0 = fast_exp2((acc[mb][nb][0] - M) * kLog2e);
      const float e1 = fast_exp2((acc[mb][nb][1] - M) * kLog2e);
      const float e2 = fast_exp2((acc[mb][nb][2] - M) * kLog2e);
      const float e3 = fast_exp2((acc[mb][nb][3] - M) * kLog2e);
      sb[nb] = (e0 + e1) + (e2 + e3);
    }
    float s = (sb[0] + sb[1]) + (sb[2] + sb[3]);
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (g == 0) red[4 * BM + wn * BM + rl] = s;
    if (row < p.N) {
      const int64_t t = load_target(p.targets, p.t64, row);
      const int64_t rel = t - cw;
      if (t >= 0 && t < p.V && rel >= 0 && rel < 64 && int((rel & 15) >> 2) == g) {
        const int tnb = int(rel >> 4), tr = int(rel & 3);
        float zt = 0.f;
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) zt = (nb == tnb && r == tr) ? acc[mb][nb][r] : zt;
        p.zt[row] = zt;
      }
    }
  }
  __syncthreads();
  for (int rl = tid; rl < BM; rl += NT) {
    const int64_t row = row0 + rl;
    if (row < p.N) {
      const float M = fmaxf(fmaxf(red[rl], red[BM + rl]), fmaxf(red[2 * BM + rl], red[3 * BM + rl]));
      const float* sr = red + 4 * BM;
      const float S = ((sr[rl] + sr[BM + rl]) + sr[2 * BM + rl]) + sr[3 * BM + rl];
      p.part[int64_t(tn) * p.N + row] = make_float2(M, S);
    }
  }
}

// ---- merge: ascending fold of the per-tile pairs -> lse, logp --------------------------------
//
// 256 threads = 32 rows x 8 segments of vocabulary tiles.  Each thread folds its
// segment in ascending order, then one thread per row folds the 8 segment
// results in ascending order.  The topology depends on V only.
__device__ __forceinline__ void fold(float& M, float& S, float m, float s) {
  if (m == -INFINITY) return;
  const float Mn = fmaxf(M, m);
  const float a = S * fast_exp2((M - Mn) * kLog2e);
  const float b = s * fast_exp2((m - Mn) * kLog2e);
  S = a + b;
  M = Mn;
}

__global__ __launch_bounds__(256) void k_merge(MergeArgs p) {
  __shared__ float sm[8][32], ss[8][32];
  const int rl = threadIdx.x & 31, seg = threadIdx.x >> 5;
  const int64_t row = int64_t(blockIdx.x) * 32 + rl;
  const int64_t seglen = (p.n_vt + 7) / 8;
  float M = -INFINITY, S = 0.f;
  if (row < p.N) {
    const int64_t v0 = seg * seglen, v1 = min(p.n_vt, v0 + seglen);
    for (int64_t v = v0; v < v1; ++v) {
      const float2 q = p.part[v * p.N + row];
      fold(M, S, q.x, q.y);
    }
  }
  sm[seg][rl] = M;
  ss[seg][rl] = S;
  __syncthreads();
  if (seg == 0 && row < p.N) {
    float M2 = -INFINITY, S2 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) fold(M2, S2, sm[k][rl], ss[k][rl]);
    const float ls = logf(S2);
    const int64_t t = load_target(p.targets, p.t64, row);
    const bool valid = t >= 0 && t < p.V;
    p.logp[row] = valid ? (p.zt[row] - M2) - ls : 0.0f;
    if (p.lse != nullptr) p.lse[row] = M2 + ls;
  }
}

// ---- dlogits: recompute the logit tile, dz = G (onehot - p) / T, d_bias partials ------------
//
// dz is written row-major ([token][vocab], for d_hidden = dz W) and transposed
// ([vocab][token], for d_weight = dz^T hidden) so that both GEMMs read K-contiguous
// operands.  The transposed copy goes through LDS in passes of CPP columns so
// that every vocabulary row receives BM contiguous tokens.
template <class E>
__device__ __forceinline__ void lds_put(char* base, int idx, float v);
template <>
__device__ __forceinline__ void lds_put<BF16>(char* base, int idx, float v) {
  reinterpret_cast<uint16_t*>(base)[idx] = uint16_t(bf16_bits_rne(v));
}
template <>
__device__ __forceinline__ void lds_put<F32>(char* base, int idx, float v) {
  reinterpret_cast<float*>(base)[idx] = v;
}

template <class E, int BM, int WAVES_M>
__global__ __launch_bounds__(256 * WAVES_M) void k_dz(DzArgs p) {
  using Tile = LogitTile<E, BM, WAVES_M>;
  constexpr int RW = Tile::RW, WMB = Tile::WMB, WNB = Tile::WNB, NT = Tile::NT;
  extern __shared__ u32x4 smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave & 3, wm = wave >> 2, i = lane & 15, g = lane >> 4;
  const int nbm = int((p.rows + BM - 1) / BM);
  const int nbn = int((p.V + 255) / 256);
  int tm, tn;
  tile_of(blockIdx.x, nbm, nbn, tm, tn);
  const int64_t row0 = int64_t(tm) * BM, col0 = int64_t(tn) * 256;

  f32x4_t acc[WMB][WNB];
  Tile::run(acc, p.hidden, p.weight, row0, p.rows, col0, p.V, p.D, smem);

  const int64_t cw = col0 + wn * 64;
  float bcol[WNB][4];
  bool cval[WNB][4];
  f32x4_t csum[WNB];
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb) {
    csum[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t c = cw + nb * 16 + 4 * g + r;
      cval[nb][r] = c < p.V;
      bcol[nb][r] = (p.bias != nullptr && c < p.V) ? p.bias[c] : 0.f;
    }
  }
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int64_t row = row0 + wm * RW + mb * 16 + i;
    const bool rv = row < p.rows;
    const float invT = (p.temperature != nullptr && rv) ? 1.0f / p.temperature[row] : 1.0f;
    const int64_t t = rv ? load_target(p.targets, p.t64, row) : -1;
    const bool valid = t >= 0 && t < p.V;
    const float G = valid ? p.grad_out[row] * invT : 0.f;
    const float L = rv ? p.lse[row] : 0.f;
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      f32x4_t d;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t c = cw + nb * 16 + 4 * g + r;
        const float z = (acc[mb][nb][r] + bcol[nb][r]) * invT;
        const float pr = fast_exp2((z - L) * kLog2e);
        const float oh = (c == t) ? 1.0f : 0.0f;
        float v = G * (oh - pr);
        v = (valid && cval[nb][r]) ? v : 0.0f;
        d[r] = v;
      }
      acc[mb][nb] = d;
      csum[nb] += d;
      if (p.dz != nullptr) store4<E>(p.dz, row * p.ldz + cw + nb * 16 + 4 * g, d);
    }
  }

  char* lds = reinterpret_cast<char*>(smem);
  if (p.dzT != nullptr) {
    // LDS tile [CPP columns][BM tokens], each column row padded by 16 bytes.
    constexpr int CPP = E::kSize == 2 ? 256 : 128;
    constexpr int kRowB = BM * E::kSize + 16;
    constexpr int kPitch = kRowB / E::kSize;
    constexpr int kChunksPerCol = BM * E::kSize / 16;
    constexpr int kTokPerChunk = 16 / E::kSize;
    for (int pass = 0; pass < 256 / CPP; ++pass) {
      __syncthreads();
      if (wn * 64 >= pass * CPP && wn * 64 < (pass + 1) * CPP) {
#pragma unroll
        for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
          for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int c = wn * 64 + nb * 16 + 4 * g + r - pass * CPP;
              const int tok = wm * RW + mb * 16 + i;
              lds_put<E>(lds, c * kPitch + tok, acc[mb][nb][r]);
            }
      }
      __syncthreads();
      for (int idx = tid; idx < CPP * kChunksPerCol; idx += NT) {
        const int c = idx / kChunksPerCol, ch = idx % kChunksPerCol;
        const u32x4 v = *reinterpret_cast<const u32x4*>(lds + c * kRowB + ch * 16);
        const int64_t vcol = col0 + pass * CPP + c;
        const int64_t tok = row0 + ch * kTokPerChunk;
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(p.dzT) +
                                  (vcol * p.ldt + tok) * E::kSize) = v;
      }
    }
  }
  if (p.dbias_part == nullptr) return;
  // Column sums over the tile's rows: in-lane over row blocks, then a butterfly
  // over the 16 lanes holding the other rows, then ascending over row waves.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [WAVES_M][256]
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = csum[nb][r];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      if (i == 0) red[wm * 256 + wn * 64 + nb * 16 + 4 * g + r] = x;
    }
  __syncthreads();
  for (int c = tid; c < 256; c += NT) {
    float s = red[c];
#pragma unroll
    for (int w = 1; w < WAVES_M; ++w) s += red[w * 256 + c];
    p.dbias_part[int64_t(tm) * p.ldz + col0 + c] = s;
  }
}

// ---- tiled transpose (hidden chunk -> hidden^T for the d_weight GEMM) -------------------------
// dst[c][r] = src[r][c]; tokens r in [rows, rows_pad) are written as zeros so that
// 16-byte loads straddling the end of the chunk read zeros.
template <class T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ src, int64_t rows,
                                                   int64_t rows_pad, int64_t cols, int64_t ld_src,
                                                   T* __restrict__ dst, int64_t ld_dst) {
  __shared__ T tile[64][65];
  const int64_t r0 = int64_t(blockIdx.y) * 64, c0 = int64_t(blockIdx.x) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int k = ty; k < 64; k += 4) {
    const int64_t r = r0 + k, c = c0 + tx;
    tile[k][tx] = (r < rows && c < cols) ? src[r * ld_src + c] : T(0);
  }
  __syncthreads();
  for (int k = ty; k < 64; k += 4) {
    const int64_t c = c0 + k, r = r0 + tx;
    if (r < rows_pad && c < cols) dst[c * ld_dst + r] = tile[tx][k];
  }
}

// ---- GEMMs of the backward ----------------------------------------------------------------
//
// C[M x N] (+)= sum_k A(m, k) B(n, k).  A is the M-side operand, B the N-side one;
// AT / BT mark an operand stored [K][M] (M-contiguous) instead of [M][K].
//   d_hidden: M = tokens, N = D, K = V; A = dz [tok][V], B = W [V][D] (BT).
//   d_weight: M = V, N = D, K = tokens; A = dz^T [V][tok], B = hidden^T [D][tok].
template <class E, int ROWS, int NT, bool T>
struct Loader;
template <class E, int ROWS, int NT>
struct Loader<E, ROWS, NT, false> {
  LoadK<ROWS, NT> l;
  __device__ __forceinline__ void load(const void* base, int64_t ld, int64_t r0, int64_t rvalid,
                                       int64_t st, int64_t K, int tid) {
    l.load(base, ld, r0, rvalid, st * kStageBytes, K * E::kSize, tid);
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const { l.store(lds, tid); }
};
template <class E, int ROWS, int NT>
struct Loader<E, ROWS, NT, true> {
  LoadT<E, ROWS, NT> l;
  __device__ __forceinline__ void load(const void* base, int64_t ld, int64_t r0, int64_t rvalid,
                                       int64_t st, int64_t K, int tid) {
    l.load(base, ld, r0, rvalid, st * (kStageBytes / E::kSize), K, tid);
  }
  __device__ __forceinline__ void store(u32x4* lds, int tid) const { l.store(lds, tid); }
};

// LOAD: start from the fp32 accumulator p.acc; STORE: 0 = element type to p.out,
// 1 = fp32 to p.acc.
template <class E, int BM, int BN, int WAVES_M, int WAVES_N, bool AT, bool BT, bool LOAD, int STORE>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void k_gemm(GemmArgs p) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int RW = BM / WAVES_M, CW = BN / WAVES_N;
  constexpr int WMB = RW / 16, WNB = CW / 16;
  static_assert(RW % 16 == 0 && CW % 16 == 0, "wave tile must be a multiple of 16");
  extern __shared__ u32x4 smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M, i = lane & 15, g = lane >> 4;
  const int nbm = int((p.M + BM - 1) / BM), nbn = int((p.N + BN - 1) / BN);
  int tm, tn;
  tile_of(blockIdx.x, nbm, nbn, tm, tn);
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;

  // Row pointers of this lane's output rows; columns are then immediate offsets.
  const int64_t nl = n0 + wn * CW + 4 * g;
  f32x4_t acc[WMB][WNB];
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int64_t m = m0 + wm * RW + mb * 16 + i;
    const float* arow = p.acc + (m < p.M ? m : 0) * p.N + nl;
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      f32x4_t x = {0.f, 0.f, 0.f, 0.f};
      if (LOAD && m < p.M && nl + nb * 16 < p.N) x = *reinterpret_cast<const f32x4_t*>(arow + nb * 16);
      acc[mb][nb] = x;
    }
  }

  const int64_t kst = kStageBytes / E::kSize;
  const int nst = int((p.K + kst - 1) / kst);
  u32x4* sA0 = smem;
  u32x4* sA1 = smem + BM * 8;
  u32x4* sB0 = smem + 2 * BM * 8;
  u32x4* sB1 = sB0 + BN * 8;
  Loader<E, BM, NT, AT> la;
  Loader<E, BN, NT, BT> lb;
  kloop<E, WMB, WNB>(
      acc, nst, sA0, sA1, sB0, sB1, wm * RW, wn * CW, lane,
      [&](int st) {
        la.load(p.a, p.lda_b, m0, AT ? p.lda_b / E::kSize : p.M, st, p.K, tid);
        lb.load(p.b, p.ldb_b, n0, p.N, st, p.K, tid);
      },
      [&](u32x4* a, u32x4* b) {
        la.store(a, tid);
        lb.store(b, tid);
      });

#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int64_t m = m0 + wm * RW + mb * 16 + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      if (nl + nb * 16 >= p.N) continue;
      if (STORE == 1)
        *reinterpret_cast<f32x4_t*>(p.acc + m * p.N + nl + nb * 16) = acc[mb][nb];
      else
        store4<E>(p.out, m * p.ldo + nl + nb * 16, acc[mb][nb]);
    }
  }
}

// ---- d_bias: ascending fold of the per-row-tile partials --------------------------------------
__global__ __launch_bounds__(256) void k_dbias_fold(const float* part, int64_t n_parts, int64_t ldz,
                                                    int64_t V, float* d_bias, int init) {
  const int64_t v = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (v >= V) return;
  float s = init ? 0.0f : d_bias[v];
  for (int64_t r = 0; r < n_parts; ++r) s += part[r * ldz + v];
  d_bias[v] = s;
}

// ---- launch helpers ----------------------------------------------------------------------------

template <class K>
hipError_t prepare(K kernel, size_t lds) {
  // Dynamic LDS above 64 KiB must be opted into once per kernel.
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
}

template <class E, int BM, int WM>
hipError_t fwd_cfg(const FwdArgs& a, hipStream_t s) {
  using Tile = LogitTile<E, BM, WM>;
  static hipError_t once = prepare(k_fwd<E, BM, WM>, Tile::kLds);
  if (once != hipSuccess) return once;
  const int64_t blocks = ((a.N + BM - 1) / BM) * ((a.V + 255) / 256);
  hipLaunchKernelGGL((k_fwd<E, BM, WM>), dim3(unsigned(blocks)), dim3(Tile::NT), Tile::kLds, s, a);
  return hipGetLastError();
}

template <class E>
hipError_t fwd_dispatch(const FwdArgs& a, hipStream_t s) {
  if (a.N <= 32) return fwd_cfg<E, 32, 1>(a, s);
  if (a.N <= 64) return fwd_cfg<E, 64, 1>(a, s);
  if (a.N <= 128) return fwd_cfg<E, 128, 1>(a, s);
  return fwd_cfg<E, 256, 2>(a, s);
}

template <class E>
hipError_t dz_dispatch(const DzArgs& a, hipStream_t s) {
  constexpr int BM = int(kDzRowTile), WM = 1;
  using Tile = LogitTile<E, BM, WM>;
  static hipError_t once = prepare(k_dz<E, BM, WM>, Tile::kLds);
  if (once != hipSuccess) return once;
  const int64_t blocks = ((a.rows + BM - 1) / BM) * ((a.V + 255) / 256);
  hipLaunchKernelGGL((k_dz<E, BM, WM>), dim3(unsigned(blocks)), dim3(Tile::NT), Tile::kLds, s, a);
  return hipGetLastError();
}

template <class E, int BM, int BN, int WM, int WN, bool AT, bool BT, bool LOAD, int STORE>
hipError_t gemm_cfg(const GemmArgs& a, hipStream_t s) {
  constexpr size_t lds = size_t(2) * (BM + BN) * kStageBytes;
  static hipError_t once = prepare(k_gemm<E, BM, BN, WM, WN, AT, BT, LOAD, STORE>, lds);
  if (once != hipSuccess) return once;
  const int64_t blocks = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm<E, BM, BN, WM, WN, AT, BT, LOAD, STORE>), dim3(unsigned(blocks)),
                     dim3(64 * WM * WN), lds, s, a);
  return hipGetLastError();
}

// The per-element MFMA chain does not depend on the tile shape, so the variants
// below may use different tiles and still give the same bits.  The fp32
// accumulator variants use a narrower tile to stay within the register file.
template <class E>
hipError_t dw_dispatch(const GemmArgs& a, hipStream_t s);

template <>
hipError_t dw_dispatch<BF16>(const GemmArgs& a, hipStream_t s) {
  if (a.load_acc) {
    if (a.store_acc) return gemm_cfg<BF16, 256, 128, 2, 2, false, false, true, 1>(a, s);
    return gemm_cfg<BF16, 256, 128, 2, 2, false, false, true, 0>(a, s);
  }
  if (a.store_acc) return gemm_cfg<BF16, 256, 128, 2, 2, false, false, false, 1>(a, s);
  return gemm_cfg<BF16, 256, 192, 2, 2, false, false, false, 0>(a, s);
}

template <>
hipError_t dw_dispatch<F32>(const GemmArgs& a, hipStream_t s) {
  if (a.load_acc) {
    if (a.store_acc) return gemm_cfg<F32, 128, 128, 2, 2, false, false, true, 1>(a, s);
    return gemm_cfg<F32, 128, 128, 2, 2, false, false, true, 0>(a, s);
  }
  if (a.store_acc) return gemm_cfg<F32, 128, 128, 2, 2, false, false, false, 1>(a, s);
  return gemm_cfg<F32, 128, 128, 2, 2, false, false, false, 0>(a, s);
}

}  // namespace

hipError_t launch_forward(flp_dtype x, const FwdArgs& a, hipStream_t s) {
  return x == FLP_BF16 ? fwd_dispatch<BF16>(a, s) : fwd_dispatch<F32>(a, s);
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_merge, dim3(unsigned((a.N + 31) / 32)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dz(flp_dtype x, const DzArgs& a, hipStream_t s) {
  return x == FLP_BF16 ? dz_dispatch<BF16>(a, s) : dz_dispatch<F32>(a, s);
}

hipError_t launch_dx(flp_dtype x, const GemmArgs& a, hipStream_t s) {
  if (x == FLP_BF16) return gemm_cfg<BF16, 256, 192, 2, 2, false, true, false, 0>(a, s);
  return gemm_cfg<F32, 128, 128, 2, 2, false, true, false, 0>(a, s);
}

hipError_t launch_dw(flp_dtype x, const GemmArgs& a, hipStream_t s) {
  return x == FLP_BF16 ? dw_dispatch<BF16>(a, s) : dw_dispatch<F32>(a, s);
}

hipError_t launch_transpose(flp_dtype x, const void* src, int64_t rows, int64_t rows_pad, int64_t cols,
                            int64_t ld_src, void* dst, int64_t ld_dst, hipStream_t s) {
  const dim3 grid(unsigned((cols + 63) / 64), unsigned((rows_pad + 63) / 64));
  if (x == FLP_BF16)
    hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(src), rows, rows_pad, cols, ld_src,
                       static_cast<uint16_t*>(dst), ld_dst);
  else
    hipLaunchKernelGGL(k_transpose<float>, grid, dim3(256), 0, s, static_cast<const float*>(src),
                       rows, rows_pad, cols, ld_src, static_cast<float*>(dst), ld_dst);
  return hipGetLastError();
}

hipError_t launch_dbias_fold(const float* part, int64_t n_parts, int64_t ldz, int64_t V,
                             float* d_bias, int init, hipStream_t s) {
  hipLaunchKernelGGL(k_dbias_fold, dim3(unsigned((V + 255) / 256)), dim3(256), 0, s, part, n_parts,
                     ldz, V, d_bias, init);
  return hipGetLastError();
}

const char* kernel_ids() {
  return "k_fwd<bf16|f32, BM 32/64/128/256, BN 256, mfma_f32_16x16x32_bf16|16x16x4f32>; "
         "k_merge<32 rows x 8 segments>; k_dz<BM 128, BN 256>; "
         "k_gemm dX<256x192, W transposed in registers>; k_gemm dW<256x192, fp32 acc>; "
         "k_transpose; k_dbias_fold";
}

}  // namespace flp
