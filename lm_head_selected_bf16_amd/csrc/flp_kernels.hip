// gfx950 (CDNA4) kernels of the fused linear selected-token log-probability.
//
// Forward ("Fused Linear LogP" docs page, sections "Backends" and "Reference
// Semantics"): each workgroup computes one [BM x 256] tile of scaled logits
// z = (h W^T + b) / T with bf16 (or fp32) MFMA and fp32 accumulation, folds
// the tile into a per-row (max, sum of exp) pair and picks up the target
// logit; a merge kernel folds the pairs of all vocabulary tiles into lse and
// logp.  The [N, V] logits never reach HBM.
//
// Backward (PR #234, "Implementation details"; PR #555 summary): per row
// chunk, a dlogits kernel recomputes the same logit tiles and writes
// dz = G (onehot - exp(z - lse)) / T row-major and transposed; two GEMMs give
// d_hidden = dz W and d_weight (+)= dz^T hidden, each with one fixed ascending
// K order; d_bias partials are folded in ascending row-tile order.  No atomics.
//
// One MFMA engine serves all four contractions.  Every operand is stored
// K-contiguous (W is transposed once per backward for d_hidden; hidden per
// chunk for d_weight) and streamed by direct global->LDS loads
// (buffer_load_dwordx4 ... lds, no register staging, whole 128-byte lines) into two
// LDS stages of 128 bytes of K per row.  Waves form a WM x WN grid; each wave
// owns a (BM/WM) x (BN/WN) block of 16 x 16 MFMA tiles with fp32 accumulators,
// and double-buffers its operand fragments across the two 64-byte halves of a
// stage.
//
// Register layout: every MFMA is issued as mfma(A = N-side fragment,
// B = M-side fragment), so lane l holds output row (l % 16) of a 16-row block
// and four consecutive output columns 4 (l / 16) + 0..3 of a 16-column block.
// Both fragments are 16 bytes of K read from LDS at (row l % 16, chunk l / 16).
//
// Batch invariance: every logit has the same MFMA chain over K (ascending
// 64-byte steps, same instruction, same lane placement of K) and every
// per-row reduction over a 256-column vocabulary tile uses one fixed tree
// defined by column positions only: in-lane over the 4 columns x 8 column
// blocks a lane holds of each 128-column half, across the four 16-lane groups
// by xor-butterfly (16, then 32), then half 0 + half 1.  No per-row arithmetic
// depends on N, the row tile or the row's position.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include <math.h>

#include "flp_launch.h"

namespace flp {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kStageBytes = 64;   // bytes of K per operand row per pipeline stage
constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kGroupM = 8;        // row tiles per scheduling group
constexpr int kTileCols = 256;    // vocabulary tile of the logits kernels
constexpr int kHalfCols = 128;    // columns per wave column in the logits kernels

struct BF16 {
  static constexpr int kSize = 2;
};
struct F16 {
  static constexpr int kSize = 2;
};
struct F32 {
  static constexpr int kSize = 4;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Both halves of a 16-lane (32-lane) exchange: every lane gets the values of lanes
// l and l ^ 16 (l ^ 32), lower row first (v_permlane16_swap / v_permlane32_swap, a
// VALU move).  A commutative combine of the two equals the xor-butterfly step.
__device__ __forceinline__ f32x2_t pair16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2_t{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ f32x2_t pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return f32x2_t{__uint_as_float(r[0]), __uint_as_float(r[1])};
}

// x of lane l ^ m.  For m = 1 and 2 a DPP quad permutation ([1, 0, 3, 2] and
// [2, 3, 0, 1]) and for m = 8 a rotation by 8 within the 16-lane row do it as a
// VALU move; other distances go through ds_bpermute.
__device__ __forceinline__ float lane_xor(float x, int m) {
  const int b = __float_as_int(x);
  if (m == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true));
  if (m == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true));
  if (m == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, true));
  return __shfl_xor(x, m);
}

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
__device__ __forceinline__ void mma64<F16>(f32x4_t& c, const u32x4& a, const u32x4& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                              __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma64<F32>(f32x4_t& c, const u32x4& a, const u32x4& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
}

// Bits of a 16-bit element type, rounded to nearest even.  gfx950 converts fp32
// to bf16 in hardware (v_cvt_pk_bf16_f32, round to nearest even, denormals kept:
// bit for bit the rounding (u + 0x7FFF + ((u >> 16) & 1)) >> 16 of the fp32 bits
// for every finite value).
template <class E>
__device__ __forceinline__ uint32_t bits16(float f);
template <>
__device__ __forceinline__ uint32_t bits16<BF16>(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
template <>
__device__ __forceinline__ uint32_t bits16<F16>(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}
template <class E>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return bits16<E>(lo) | (bits16<E>(hi) << 16);
}
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Store four consecutive fp32 values as the element type.
template <class E>
__device__ __forceinline__ void store4(void* base, int64_t idx, const f32x4_t& v) {
  static_assert(E::kSize == 2, "16-bit element types");
  u32x2 w;
  w.x = pack2<E>(v.x, v.y);
  w.y = pack2<E>(v.z, v.w);
  *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + idx) = w;
}

template <>
__device__ __forceinline__ void store4<F32>(void* base, int64_t idx, const f32x4_t& v) {
  *reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(base) + idx) = v;
}

// K-blocked layout of the backward GEMM operands (dz, dz^T, W^T, hidden^T):
// element (r, k) of a matrix with `rows` rows sits at ((k / KB) * rows + r) * KB
// + k % KB, KB = 128 bytes of K.  One 128-byte pipeline stage of a GEMM tile is
// then a contiguous block of tile rows x 128 bytes.
template <int KB>
__device__ __forceinline__ int64_t kblk(int64_t r, int64_t k, int64_t rows) {
  return ((k / KB) * rows + r) * KB + (k % KB);
}

__device__ __forceinline__ int64_t load_target(const void* t, int t64, int64_t i) {
  return t64 ? reinterpret_cast<const int64_t*>(t)[i] : int64_t(reinterpret_cast<const int32_t*>(t)[i]);
}

// Workgroup id -> (row tile, column tile).  Workgroups are dispatched
// round-robin over the 8 XCDs, so ids are first regrouped so that each XCD
// receives a contiguous run of logical tiles (sharing its L2), then the run is
// walked in groups of GM row tiles, row tile fastest, so that the workgroups
// resident at one time share both operand tiles.  Logits tiles use GM = 8
// (8 row tiles x 4 vocabulary tiles per XCD at a time; 4 and 16 measured slower);
// the backward GEMMs use GM = 1, the 12 column tiles of one row tile in turn
// (measured best of 1, 2, 4, 8 and 16 with their split LDS ring).
template <int GM = kGroupM>
__device__ __forceinline__ void tile_of(int bid, int nbm, int nbn, int& tm, int& tn) {
  const int total = nbm * nbn;
  const int per = total >> 3;
  int lin = bid;
  if (bid < per * 8) lin = (bid & 7) * per + (bid >> 3);
  const int width = GM * nbn;
  const int grp = lin / width;
  const int first = grp * GM;
  const int gm = min(nbm - first, GM);
  const int in = lin - grp * width;
  tm = first + in % gm;
  tn = in / gm;
}

// ---- direct global -> LDS staging of one operand tile --------------------------------------
//
// A pipeline stage holds 128 bytes of K per operand row (two 64-byte MFMA steps),
// so that every load covers whole 128-byte cache lines.  In LDS a row is 8
// 16-byte chunks; logical chunk c of row r sits at position c ^ ((r >> 1) & 7),
// which puts the 16 rows of a fragment read on 16 distinct bank groups.  One wave
// instruction fills 64 consecutive LDS chunks (lane l -> chunk base + l): it
// covers rows 8 inst + l / 8 at positions l % 8.  Rows past the end of the
// operand read a clamped (valid) row whose results are never used; in a last,
// half stage (64 bytes of K left) the upper four chunks repeat the lower four.
template <int ROWS, int NW>
struct DTile {
  static constexpr int kInsts = ROWS / 8;
  static constexpr int kPer = (kInsts + NW - 1) / NW;
  // Wave w issues instructions w*kPer .. min(kInsts, (w+1)*kPer) - 1, so the last
  // waves may issue fewer: count(w) per stage.
  static constexpr int count(int w) {
    return kInsts - w * kPer <= 0 ? 0 : (kInsts - w * kPer > kPer ? kPer : kInsts - w * kPer);
  }
  static_assert(ROWS % 16 == 0, "tile rows must be a multiple of 16");
  int q;                // row within the instruction's 8 rows
  int c0, c1;           // logical chunk loaded by this lane for even / odd instructions
  int64_t ld, ks, rows_valid;  // row stride, stage stride (bytes), rows that exist
  bool full;            // every row of the tile is valid: no clamping

  __device__ __forceinline__ void init(int64_t ld_, int64_t ks_, int64_t rows_valid_, int lane) {
    ld = ld_;
    ks = ks_;
    rows_valid = rows_valid_;
    full = rows_valid_ >= ROWS;
    q = lane >> 3;
    c0 = (lane & 7) ^ (q >> 1);
    c1 = c0 ^ 4;
  }
  __device__ __forceinline__ void issue(const char* base, int stage, bool half, u32x4* lds,
                                        int wave) const {
    // A raw buffer resource based at the stage keeps the per-lane part a 32-bit
    // offset that does not change from stage to stage.
    const char* sb = base + int64_t(stage) * ks;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)sb, (short)0, 0x7FFFFFFF, 0x00020000);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int inst = wave * kPer + j;
      if (kInsts % NW == 0 || inst < kInsts) {
        int c = (inst & 1) ? c1 : c0;
        c = half ? (c & 3) : c;
        int64_t r = int64_t(inst) * 8 + q;
        if (!full) r = r < rows_valid ? r : rows_valid - 1;
        const uint32_t off = uint32_t(r * ld) + uint32_t(c * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(lds + inst * 64), 16, int(off), 0, 0, 0);
      }
    }
  }
};

// Wait until at most N of this wave's vector-memory loads are outstanding and its
// LDS reads have completed, then barrier the workgroup.  The direct loads
// complete in issue order.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_own() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// ---- the MFMA engine -------------------------------------------------------------------------
//
// A ring of NS LDS buffers of one 128-byte stage each (two for the large tiles);
// stage t lives in buffer t % NS and holds the MFMA steps 2t (chunks 0-3) and
// 2t + 1 (chunks 4-7).  Every MFMA step multiplies fragments read from LDS during
// the previous step.  The workgroup synchronises once per stage, between its two
// steps: stage t + 1 must have landed (its loads were issued NS - 1 stages
// earlier) and every wave must be done reading stage t, whose buffer then receives
// the loads of stage t + NS.  Small tiles do little work per stage, so they use a
// deeper ring to keep enough loads in flight.
// What a peeled pipeline stage does at its barrier (a compile-time tag).
template <int M>
using Mode = std::integral_constant<int, M>;

template <class E, int BM, int BN, int WM, int WN, int NS = 2, int NSA = NS>
struct Engine {
  using TileA = DTile<BM, WM * WN>;
  static constexpr int NW = WM * WN;
  static constexpr int NT = 64 * NW;
  static constexpr int RW = BM / WM;
  static constexpr int CW = BN / WN;
  static constexpr int WMB = RW / 16;
  static constexpr int WNB = CW / 16;
  static constexpr int kSlots = (BM + BN) * 8;  // 16-byte LDS chunks per stage
  // NSA buffers of the A operand, NS of B (NSA = NS: one ring of both).
  static constexpr size_t kLds = (size_t(NSA) * BM + size_t(NS) * BN) * 128;
  static_assert(NS >= 2, "at least two LDS stages");
  static_assert(NSA == NS || (NS == 2 && NSA == 3), "A ring one deeper than B: 3 and 2 buffers");
  static_assert(RW % 16 == 0 && CW % 16 == 0, "wave tile must be a multiple of 16");

  struct Frag {
    u32x4 a[WMB], b[WNB];
  };

  // Fragments of one MFMA step from the buffer at `st`: per-lane base chunks fa,
  // fb; the 16-row blocks are immediate offsets (128 chunks apart).
  __device__ __forceinline__ static void read(Frag& f, const u32x4* st, int fa, int fb) {
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) f.a[mb] = st[fa + mb * 128];
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) f.b[nb] = st[BM * 8 + fb + nb * 128];
  }

  // The same with the A and B fragments in separate buffers.
  __device__ __forceinline__ static void read2(Frag& f, const u32x4* sa, const u32x4* sb, int fa,
                                               int fb) {
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) f.a[mb] = sa[fa + mb * 128];
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) f.b[nb] = sb[fb + nb * 128];
  }

  __device__ __forceinline__ static void mmas(f32x4_t (&acc)[WMB][WNB], const Frag& f) {
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) mma64<E>(acc[mb][nb], f.b[nb], f.a[mb]);
  }

  // Keep the reads of the next step spread among the MFMAs of this one, starting
  // with MFMAs: the wait for this step's fragments then precedes every new read
  // (LDS reads complete in order, so a read issued first would be waited for too).
  __device__ __forceinline__ static void interleave() {
    constexpr int kR = WMB + WNB, kM = WMB * WNB * (E::kSize == 2 ? 1 : 4);
    constexpr int kStep = kM / kR > 0 ? kM / kR : 1;
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, kStep, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (kM > kStep * kR) __builtin_amdgcn_sched_group_barrier(0x008, kM - kStep * kR, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // acc (+)= A[rows, K] . B[rows, K]^T over kbytes of K (a multiple of 64; ODD when
  // kbytes / 64 is odd).  a and b point at the first row of the tile; rows past
  // *_rows_valid are clamped.
  template <bool ODD>
  __device__ __forceinline__ static void run(f32x4_t (&acc)[WMB][WNB], const char* a, int64_t lda,
                                             int64_t a_rows_valid, const char* b, int64_t ldb,
                                             int64_t b_rows_valid, int64_t kbytes, u32x4* smem) {
    run<ODD>(acc, a, lda, 128, a_rows_valid, b, ldb, 128, b_rows_valid, kbytes, smem);
  }
  // The same with explicit stage strides (bytes from one 128-byte K stage of a row
  // to the next): 128 for row-major operands, rows x 128 for K-blocked ones.
  template <bool ODD>
  __device__ __forceinline__ static void run(f32x4_t (&acc)[WMB][WNB], const char* a, int64_t lda,
                                             int64_t a_ks, int64_t a_rows_valid, const char* b,
                                             int64_t ldb, int64_t b_ks, int64_t b_rows_valid,
                                             int64_t kbytes, u32x4* smem) {
    const int tid = threadIdx.x, lane = tid & 63;
    // Wave-uniform, so that the LDS destinations of the direct loads (M0) are scalar.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WM, wn = wave / WM, i = lane & 15, g = lane >> 4;
    const int nsteps = int(kbytes / kStageBytes);
    const int nst = (nsteps + 1) / 2;
    TileA ta;
    DTile<BN, NW> tb;
    ta.init(lda, a_ks, a_rows_valid, lane);
    tb.init(ldb, b_ks, b_rows_valid, lane);
    // Chunk of the even step for this lane; the odd step's is pos ^ 4.
    const int pos = g ^ ((i >> 1) & 7);
    const int fa = (wm * RW + i) * 8 + pos;
    const int fb = (wn * CW + i) * 8 + pos;
    auto issue = [&](int t) {
      u32x4* dst = smem + (t % NS) * kSlots;
      const bool half = ODD && t == nst - 1;
      ta.issue(a, t, half, dst, wave);
      tb.issue(b, t, half, dst + BM * 8, wave);
    };
    if constexpr (NSA != NS) {
      static_assert(!ODD, "the split ring serves the GEMMs, whose K is whole 128-byte stages");
      split(acc, nst, ta, tb, a, b, fa, fb, smem, wave);
      return;
    } else if constexpr (NS > 2) {
      deep<ODD>(acc, nst, issue, fa, fb, smem, wave);
      return;
    }
    issue(0);
    if (nst > 1) {
      issue(1);
      wait_stages<1>(wave);
      barrier_only();
    } else {
      wait_barrier<0>();
    }
    Frag f0, f1;
    read(f0, smem, fa, fb);
    // Stage t: step 2t from f0 (read one step earlier) while reading step 2t + 1
    // into f1; synchronise; step 2t + 1 from f1 while reading step 2t + 2 into
    // f0.  After the last stage the other buffer still holds consumed data that
    // no load overwrites any more; reading it (unused) keeps the body free of
    // branches around the fragment reads.
    //
    // The stages that issue loads run in a loop of their own whose body has no
    // branches (one block the scheduler orders as a whole); the last two stages
    // (barrier only, then neither barrier nor loads) are peeled off.
    auto stage = [&](int t, auto mode) {
      constexpr int kMode = decltype(mode)::value;  // 0: barrier + loads, 1: barrier, 2: none
      read(f1, smem + (t & 1) * kSlots, fa ^ 4, fb ^ 4);
      mmas(acc, f0);
      interleave();
      if constexpr (kMode <= 1) wait_barrier<0>();
      if constexpr (kMode == 0) issue(t + 2);
      read(f0, smem + ((t + 1) & 1) * kSlots, fa, fb);
      mmas(acc, f1);
      interleave();
    };
    for (int t = 0; t + 2 < nst; ++t) stage(t, Mode<0>{});
    if (nst >= 2) stage(nst - 2, Mode<1>{});
    if (!ODD) stage(nst - 1, Mode<2>{});
    if constexpr (ODD) mmas(acc, f0);
  }

  // The ring of NS > 2 stages: the first NS stages are issued up front; at the
  // barrier of stage t, stages t + 2 .. t + NS - 1 may still be in flight (every
  // stage issues the same number of loads per wave, a half stage included), and
  // near the end of the K walk everything is waited for.  Waves may issue
  // different numbers of loads per stage (the instructions of a tile are split
  // over the waves in runs of kPer), so each wave waits on its own count: a
  // wave-uniform branch picks the immediate, and every wave then reaches the one
  // barrier.
  static_assert(NS == 2 || (NS - 1) * (TileA::kPer + DTile<BN, NW>::kPer) <= 63,
                "the loads in flight must fit the vmcnt counter");
  static constexpr int loads_of(int w) { return TileA::count(w) + DTile<BN, NW>::count(w); }
  // Last wave of the run of waves from w on that issue as many loads as wave w.
  static constexpr int run_end(int w) {
    return w + 1 < NW && loads_of(w + 1) == loads_of(w) ? run_end(w + 1) : w;
  }
  template <int Stages, int W = 0>
  __device__ __forceinline__ static void wait_stages(int wave) {
    constexpr int Last = run_end(W);
    if constexpr (Last + 1 < NW) {
      if (wave <= Last) {
        wait_own<Stages * loads_of(W)>();
        return;
      }
      wait_stages<Stages, Last + 1>(wave);
    } else {
      wait_own<Stages * loads_of(W)>();
    }
  }
  // Per-wave wait until at most KA stages of its A loads and KB stages of its B
  // loads are outstanding.
  static constexpr int mix_of(int w, int ka, int kb) {
    return ka * TileA::count(w) + kb * DTile<BN, NW>::count(w);
  }
  static constexpr int mix_end(int w, int ka, int kb) {
    return w + 1 < NW && mix_of(w + 1, ka, kb) == mix_of(w, ka, kb) ? mix_end(w + 1, ka, kb) : w;
  }
  template <int KA, int KB, int W = 0>
  __device__ __forceinline__ static void wait_mix(int wave) {
    constexpr int Last = mix_end(W, KA, KB);
    if constexpr (Last + 1 < NW) {
      if (wave <= Last) {
        wait_own<mix_of(W, KA, KB)>();
        return;
      }
      wait_mix<KA, KB, Last + 1>(wave);
    } else {
      wait_own<mix_of(W, KA, KB)>();
    }
  }

  // The split ring: three buffers of the A operand, two of B.  The GEMMs stream
  // their A operand (dz, dz^T) from HBM once, while B (W^T, hidden^T) is shared by
  // many workgroups through the caches, so the A loads get two stages of time to
  // land and the B loads one.  At the barrier of stage t the buffers of stage t
  // are free and receive B(t + 2), then A(t + 3), in that order: the direct loads
  // complete in issue order, so waiting until only this wave's A(t + 2) loads may
  // be outstanding (issued at the previous barrier, after B(t + 1)) guarantees
  // that all of stage t + 1 has landed.
  template <class TA, class TB>
  __device__ __forceinline__ static void split(f32x4_t (&acc)[WMB][WNB], int nst, const TA& ta,
                                               const TB& tb, const char* a, const char* b, int fa,
                                               int fb, u32x4* smem, int wave) {
    u32x4* const sa = smem;
    u32x4* const sb = smem + NSA * BM * 8;
    auto issue_a = [&](int t, int buf) { ta.issue(a, t, false, sa + buf * BM * 8, wave); };
    auto issue_b = [&](int t, int buf) { tb.issue(b, t, false, sb + buf * BN * 8, wave); };
    issue_a(0, 0);
    issue_b(0, 0);
    if (nst > 1) {
      issue_a(1, 1);
      issue_b(1, 1);
    }
    if (nst > 2) {
      issue_a(2, 2);
      wait_mix<2, 1>(wave);  // A(1), B(1), A(2) may be in flight
    } else if (nst > 1) {
      wait_mix<1, 1>(wave);
    } else {
      wait_own<0>();
    }
    barrier_only();
    Frag f0, f1;
    read2(f0, sa, sb, fa, fb);
    int ca = 0, cb = 0;  // buffers of stage t
    // As in the two-stage ring, the stages that issue both loads run in a loop
    // without branches, and the last three stages are peeled off.
    auto stage = [&](int t, auto mode) {
      // 0: barrier + B(t + 2) + A(t + 3), 1: barrier + B(t + 2), 2: barrier, 3: none
      constexpr int kMode = decltype(mode)::value;
      const int na = ca == 2 ? 0 : ca + 1, nb = cb ^ 1;
      read2(f1, sa + ca * BM * 8, sb + cb * BN * 8, fa ^ 4, fb ^ 4);
      mmas(acc, f0);
      interleave();
      if constexpr (kMode <= 1)
        wait_mix<1, 0>(wave);  // only A(t + 2) may be in flight
      else if constexpr (kMode == 2)
        wait_own<0>();
      if constexpr (kMode <= 2) barrier_only();
      if constexpr (kMode <= 1) issue_b(t + 2, cb);
      if constexpr (kMode == 0) issue_a(t + 3, ca);
      read2(f0, sa + na * BM * 8, sb + nb * BN * 8, fa, fb);
      mmas(acc, f1);
      interleave();
      ca = na;
      cb = nb;
    };
    int t = 0;
    for (; t + 3 < nst; ++t) stage(t, Mode<0>{});
    if (t + 2 < nst) stage(t++, Mode<1>{});
    if (t + 1 < nst) stage(t++, Mode<2>{});
    stage(t, Mode<3>{});
  }

  template <bool ODD, class Issue>
  __device__ __forceinline__ static void deep(f32x4_t (&acc)[WMB][WNB], int nst, Issue& issue,
                                              int fa, int fb, u32x4* smem, int wave) {
    for (int t = 0; t < NS && t < nst; ++t) issue(t);
    if (nst >= NS) {
      wait_stages<NS - 1>(wave);
      barrier_only();
    } else {
      wait_barrier<0>();
    }
    Frag f0, f1;
    read(f0, smem, fa, fb);
    int cur = 0;  // buffer of stage t
    // 0: wait + barrier + loads of stage t + NS, 1: wait + barrier, 2: wait for all
    // + barrier, 3: none; the load-issuing stages again form a loop of their own.
    auto stage = [&](int t, auto mode) {
      constexpr int kMode = decltype(mode)::value;
      const int nxt = cur + 1 == NS ? 0 : cur + 1;
      read(f1, smem + cur * kSlots, fa ^ 4, fb ^ 4);
      mmas(acc, f0);
      interleave();
      if constexpr (kMode <= 1) {
        wait_stages<NS - 2>(wave);
        barrier_only();
      } else if constexpr (kMode == 2) {
        wait_barrier<0>();
      }
      if constexpr (kMode == 0) issue(t + NS);
      read(f0, smem + nxt * kSlots, fa, fb);
      mmas(acc, f1);
      interleave();
      cur = nxt;
    };
    int t = 0;
    for (; t + NS < nst; ++t) stage(t, Mode<0>{});
    if (t + NS - 1 < nst) stage(t++, Mode<1>{});
    for (; t + 1 < nst; ++t) stage(t, Mode<2>{});
    if (!ODD) stage(t, Mode<3>{});
    if constexpr (ODD) mmas(acc, f0);
  }
};

// ---- forward: logits tile -> per-row (max, sum of exp) partial + target logit -------------
//
// Workgroup = WM x 2 waves; wave (wm, wn) owns rows [wm*RW, wm*RW + RW) and the 128
// vocabulary columns [wn*128, wn*128 + 128) of the BM x 256 tile.
template <class E, int BM, int WM, int NS = 2>
using LogitEngine = Engine<E, BM, kTileCols, WM, 2, NS>;

// The fixed per-row tree over the 32 values one lane holds of a wave's 128 columns.
template <int WNB>
__device__ __forceinline__ float lane_sum(const float (&e)[WNB][4]) {
  static_assert(WNB == 8, "the reduction tree is defined for 8 column blocks per wave");
  float s[WNB];
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb) s[nb] = (e[nb][0] + e[nb][1]) + (e[nb][2] + e[nb][3]);
  return ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
}

template <class E, int BM, int WM, bool ODD, int NS = 2>
__global__ __launch_bounds__(128 * WM) void k_fwd(FwdArgs p) {
  using Eng = LogitEngine<E, BM, WM, NS>;
  constexpr int RW = Eng::RW, WMB = Eng::WMB, WNB = Eng::WNB, NT = Eng::NT;
  extern __shared__ u32x4 smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile tests become scalar
  const int wm = wave % WM, wn = wave / WM, i = lane & 15, g = lane >> 4;
  const int nbm = int((p.N + BM - 1) / BM);
  const int nbn = int((p.V + kTileCols - 1) / kTileCols);
  int tm, tn;
  tile_of(blockIdx.x, nbm, nbn, tm, tn);
  const int64_t row0 = int64_t(tm) * BM, col0 = int64_t(tn) * kTileCols;
  const int64_t kbytes = p.D * E::kSize;

  f32x4_t acc[WMB][WNB];
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  Eng::template run<ODD>(acc, reinterpret_cast<const char*>(p.hidden) + row0 * kbytes, kbytes, p.N - row0,
           reinterpret_cast<const char*>(p.weight) + col0 * kbytes, kbytes, p.V - col0, kbytes,
           smem);
  // Waves still reading their last fragments after the last stage barrier may read
  // either buffer (buffer 0 when the stage count is odd): LDS is reused below.
  __syncthreads();

  // [2][BM] row max of y = h W^T + b per wave column, [2][BM] row sums, [BM] row max of z
  static_assert(5 * BM * sizeof(float) <= Eng::kLds, "the row reductions fit the operand ring");
  float* red = reinterpret_cast<float*>(smem);
  const int64_t cw = col0 + wn * kHalfCols;
  // Columns of this wave at or past lim are vocabulary padding (lim < 128 only in
  // the last vocabulary tile).
  const int lim = int(p.V - cw < kHalfCols ? p.V - cw : kHalfCols);
  float bcol[WNB][4];
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) bcol[nb][r] = 0.f;
  if (p.bias != nullptr) {
    const float* bw = p.bias + cw + 4 * g;
    if (lim == kHalfCols) {  // wave-uniform: every column of the wave exists
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) bcol[nb][r] = bw[nb * 16 + r];
    } else {
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb * 16 + 4 * g + r < lim) bcol[nb][r] = bw[nb * 16 + r];
    }
  }

  // The logits are z = y / T with y = h W^T + b; the accumulators become y and 1/T
  // enters through the exp argument's FMA.
  // The row max of z is the row max of y times 1/T, bit for bit: rounding is
  // monotone, so max_j fl(y_j / T) = fl(max_j(y_j) / T).
  float invT[WMB];
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int rl = wm * RW + mb * 16 + i;
    const int64_t row = row0 + rl;
    invT[mb] = (p.temperature != nullptr && row < p.N) ? 1.0f / p.temperature[row] : 1.0f;
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[mb][nb][r] += bcol[nb][r];
    if (lim < kHalfCols) {  // the last vocabulary tile: padding columns drop out
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb * 16 + 4 * g + r >= lim) acc[mb][nb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, acc[mb][nb][r]);
    f32x2_t q = pair16(mx);
    mx = fmaxf(q.x, q.y);
    q = pair32(mx);
    mx = fmaxf(q.x, q.y);
    if (g == 0) red[wn * BM + rl] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int rl = wm * RW + mb * 16 + i;
    const int64_t row = row0 + rl;
    const float M = fmaxf(red[rl], red[BM + rl]) * invT[mb];  // row max of z
    const float Ml = M * kLog2e;
    const float k = invT[mb] * kLog2e;
    if (wn == 0 && g == 0) red[4 * BM + rl] = M;
    // exp(z - M) = 2^(y (log2 e / T) - M log2 e): one FMA per logit
    float e[WNB][4];
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) e[nb][r] = fast_exp2(fmaf(acc[mb][nb][r], k, -Ml));
    float s = lane_sum<WNB>(e);
    f32x2_t q = pair16(s);
    s = q.x + q.y;
    q = pair32(s);
    s = q.x + q.y;
    if (g == 0) red[2 * BM + wn * BM + rl] = s;
    if (row < p.N) {
      const int64_t t = load_target(p.targets, p.t64, row) - p.t_off;
      const int64_t rel = t - cw;
      if (t >= 0 && t < p.V && rel >= 0 && rel < kHalfCols && int((rel & 15) >> 2) == g) {
        const int tnb = int(rel >> 4), tr = int(rel & 3);
        float yt = 0.f;
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r) yt = (nb == tnb && r == tr) ? acc[mb][nb][r] : yt;
        p.zt[row] = yt * invT[mb];
      }
    }
  }
  __syncthreads();
  for (int rl = tid; rl < BM; rl += NT) {
    const int64_t row = row0 + rl;
    if (row < p.N) {
      const float M = red[4 * BM + rl];
      const float S = red[2 * BM + rl] + red[3 * BM + rl];
      p.part[int64_t(tn) * p.N + row] = make_float2(M, S);
    }
  }
}

// ---- merge: per-tile pairs -> lse, logp ------------------------------------------------------
//
// The row max M is the largest tile max (exact in any order).  The sum
// S = sum_t s_t 2^((m_t - M) log2 e) runs over 256 leaves: leaf j adds the tiles
// [j L, j L + L) (L = ceil(n_vt / 256)) in ascending order, and the leaves are
// added by a complete binary tree (pairs, pairs of pairs, ...).  Both depend on the
// vocabulary only, so a row gets the same bits whatever the batch and whichever
// of the two workgroup shapes below merges it: R = 1 row per workgroup (one leaf
// per thread, for small batches) or R = 8 rows (eight leaves per thread).  The tree
// levels inside a wave are xor butterflies over the lanes of one row (addition is
// commutative, so both partners hold the same bits), the last two levels combine
// the four waves.  LL = tiles per leaf when they fit in registers (1 or 2), else 0:
// the tiles are then read twice (max, then sum).
constexpr int kMergeLeaves = 256;
constexpr int64_t kMergeRowMax = 2048;  // batches up to this size: one row per workgroup

__device__ __forceinline__ float merge_term(float2 q, float M) {
  return q.x == -INFINITY ? 0.f : q.y * fast_exp2((q.x - M) * kLog2e);
}

template <int R, int LL>
__global__ __launch_bounds__(256) void k_merge(MergeArgs p) {
  constexpr int P = kMergeLeaves / (256 / R);  // leaves per thread
  __shared__ float sm[4][R], ss[4][R];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rl = tid % R, c = tid / R;  // row in the workgroup, thread of the row
  const int64_t row = int64_t(blockIdx.x) * R + rl;
  const bool live = row < p.N;
  const int64_t L = (p.n_vt + kMergeLeaves - 1) / kMergeLeaves;
  const int64_t v0 = int64_t(c) * P * L, v1 = min(p.n_vt, v0 + P * L);
  const bool fin = c == 0 && live;
  int64_t t = -1;
  float zt = 0.f;
  if (fin) {
    t = load_target(p.targets, p.t64, row);
    zt = p.zt[row];
  }
  auto tile = [&](int64_t v) {
    return (live && v < v1) ? p.part[v * p.N + row] : make_float2(-INFINITY, 0.f);
  };
  float2 q[LL > 0 ? P * LL : 1];
  float m = -INFINITY;
  if constexpr (LL > 0) {
#pragma unroll
    for (int u = 0; u < P * LL; ++u) q[u] = tile(v0 + u);
#pragma unroll
    for (int u = 0; u < P * LL; ++u) m = fmaxf(m, q[u].x);
  } else {
    for (int64_t v = v0; v < v1; ++v) m = fmaxf(m, tile(v).x);
  }
#pragma unroll
  for (int k = R; k < 64; k <<= 1) m = fmaxf(m, lane_xor(m, k));
  if (lane < R) sm[wave][rl] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(sm[0][rl], sm[1][rl]), fmaxf(sm[2][rl], sm[3][rl]));
  float l[P];
#pragma unroll
  for (int k = 0; k < P; ++k) {
    if constexpr (LL > 0) {
      l[k] = merge_term(q[k * LL], M);
#pragma unroll
      for (int j = 1; j < LL; ++j) l[k] += merge_term(q[k * LL + j], M);
    } else {
      l[k] = 0.f;
      for (int64_t v = v0 + k * L; v < v0 + (k + 1) * L; ++v) l[k] += merge_term(tile(v), M);
    }
  }
  float sum;
  if constexpr (P == 8)
    sum = ((l[0] + l[1]) + (l[2] + l[3])) + ((l[4] + l[5]) + (l[6] + l[7]));
  else
    sum = l[0];
#pragma unroll
  for (int k = R; k < 64; k <<= 1) sum += lane_xor(sum, k);
  if (lane < R) ss[wave][rl] = sum;
  __syncthreads();
  if (fin) {
    const float S = (ss[0][rl] + ss[1][rl]) + (ss[2][rl] + ss[3][rl]);
    const float ls = logf(S);
    const bool valid = t >= 0 && t < p.V;
    p.logp[row] = valid ? (zt - M) - ls : 0.0f;
    if (p.lse != nullptr) p.lse[row] = M + ls;
  }
}

__global__ __launch_bounds__(256) void k_fill(float* dst, int64_t n, float value) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) dst[i] = value;
}

// ---- the operator on materialised logits ----------------------------------------------------
//
// One wave per row, four rows per workgroup.  Lane l owns the 16-byte chunks
// l, l + 64, l + 128, ... of its row and keeps an online (max, sum of exp) over
// them in chunk order; the 64 lane pairs are then combined by a xor butterfly
// whose combine step is symmetric, so every lane ends with the same bits.  The
// row is read once with streaming loads, four chunks per lane in flight.

template <class E>
__device__ __forceinline__ void unpack8(const u32x4& v, float (&x)[8]);
template <>
__device__ __forceinline__ void unpack8<BF16>(const u32x4& v, float (&x)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = __uint_as_float(v[k] << 16);
    x[2 * k + 1] = __uint_as_float(v[k] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void unpack8<F16>(const u32x4& v, float (&x)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    x[2 * k] = float(__builtin_bit_cast(_Float16, uint16_t(v[k] & 0xFFFFu)));
    x[2 * k + 1] = float(__builtin_bit_cast(_Float16, uint16_t(v[k] >> 16)));
  }
}

template <class E>
__device__ __forceinline__ float load_elem(const void* base, int64_t i);
template <>
__device__ __forceinline__ float load_elem<BF16>(const void* base, int64_t i) {
  return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(base)[i]) << 16);
}
template <>
__device__ __forceinline__ float load_elem<F16>(const void* base, int64_t i) {
  return float(reinterpret_cast<const _Float16*>(base)[i]);
}
template <>
__device__ __forceinline__ float load_elem<F32>(const void* base, int64_t i) {
  return reinterpret_cast<const float*>(base)[i];
}

template <class E>
__global__ __launch_bounds__(256) void k_logits_fwd(LogitsArgs p) {
  constexpr int EPC = 16 / E::kSize;  // elements per 16-byte chunk
  constexpr int kBatch = 4;
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= p.N) return;
  if (p.mask != nullptr && p.mask[row] == 0) {  // a row left out by an indexed call
    if (lane == 0) {
      p.logp[row] = 0.0f;
      if (p.lse_out != nullptr) p.lse_out[row] = 0.0f;
    }
    return;
  }
  const int64_t nch = p.V / EPC;
  const u32x4* src =
      reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(p.logits) + row * p.V * E::kSize);
  float M = -INFINITY, S = 0.f;
  for (int64_t c0 = lane; c0 < nch; c0 += 64 * kBatch) {
    u32x4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (c0 + u * 64 < nch) v[u] = __builtin_nontemporal_load(src + c0 + u * 64);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (c0 + u * 64 >= nch) break;
      float x[EPC];
      if constexpr (E::kSize == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(v[u][k]);
      } else {
        unpack8<E>(v[u], x);
      }
      float cm = x[0];
#pragma unroll
      for (int k = 1; k < EPC; ++k) cm = fmaxf(cm, x[k]);
      const float Mn = fmaxf(M, cm);
      float e = 0.f;
#pragma unroll
      for (int k = 0; k < EPC; ++k) e += fast_exp2((x[k] - Mn) * kLog2e);
      S = S * fast_exp2((M - Mn) * kLog2e) + e;
      M = Mn;
    }
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float Mo = __shfl_xor(M, off), So = __shfl_xor(S, off);
    const float Mn = fmaxf(M, Mo);
    const float a = (M == -INFINITY) ? 0.f : S * fast_exp2((M - Mn) * kLog2e);
    const float b = (Mo == -INFINITY) ? 0.f : So * fast_exp2((Mo - Mn) * kLog2e);
    S = a + b;
    M = Mn;
  }
  if (lane != 0) return;
  const float ls = logf(S);
  const int64_t t = load_target(p.targets, p.t64, row);
  const bool valid = t >= 0 && t < p.V;
  const float zt = valid ? load_elem<E>(p.logits, row * p.V + t) : 0.f;
  p.logp[row] = valid ? (zt - M) - ls : 0.0f;
  if (p.lse_out != nullptr) p.lse_out[row] = M + ls;
}

template <class E>
__global__ __launch_bounds__(256) void k_logits_bwd(LogitsArgs p) {
  constexpr int EPC = 16 / E::kSize;
  constexpr int kBatch = 4;
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= p.N) return;
  const int64_t nch = p.V / EPC;
  const u32x4* src =
      reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(p.logits) + row * p.V * E::kSize);
  u32x4* dst = reinterpret_cast<u32x4*>(reinterpret_cast<char*>(p.d_logits) + row * p.V * E::kSize);
  if (p.mask != nullptr && p.mask[row] == 0) {  // a row left out by an indexed call: zero gradient
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t c = lane; c < nch; c += 64) __builtin_nontemporal_store(z, dst + c);
    return;
  }
  const int64_t t = load_target(p.targets, p.t64, row);
  const bool valid = t >= 0 && t < p.V;
  const float G = valid ? p.grad_out[row] : 0.f;
  const float L = p.lse[row];
  for (int64_t c0 = lane; c0 < nch; c0 += 64 * kBatch) {
    u32x4 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (c0 + u * 64 < nch) v[u] = __builtin_nontemporal_load(src + c0 + u * 64);
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t c = c0 + u * 64;
      if (c >= nch) break;
      float x[EPC], d[EPC];
      if constexpr (E::kSize == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) x[k] = __uint_as_float(v[u][k]);
      } else {
        unpack8<E>(v[u], x);
      }
#pragma unroll
      for (int k = 0; k < EPC; ++k) {
        const float pr = fast_exp2((x[k] - L) * kLog2e);
        const float oh = (c * EPC + k == t) ? 1.0f : 0.0f;
        d[k] = valid ? G * (oh - pr) : 0.0f;
      }
      u32x4 w;
      if constexpr (E::kSize == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = __float_as_uint(d[k]);
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = pack2<E>(d[2 * k], d[2 * k + 1]);
      }
      __builtin_nontemporal_store(w, dst + c);
    }
  }
}

// ---- dlogits: recompute the logit tile, dz = G (onehot - p) / T, d_bias partials ------------
//
// dz is written token-major (the A operand of d_hidden = dz W) and transposed (the
// A operand of d_weight = dz^T hidden), both in the K-blocked layout of the GEMM
// operands.  16-bit inputs write them straight from the registers, every wave
// store instruction one contiguous 1 KB run (8 rows x one 128-byte K block).
//
// K order.  Within every 32-wide block of K, the 16-bit backward GEMMs take their K
// positions in the order
//   K position 32 b + 8 g + 4 h + r  <->  index 32 b + 16 h + 4 g + r
// (g, r = 0..3; h = 0, 1) of the vocabulary (d_hidden) or token (d_weight)
// dimension: the order in which a lane of the logit tile holds its values, so that
// each lane's eight values of two adjacent 16-column blocks form one 16-byte chunk
// of K.  The transposes of W and of hidden (k_transpose16) apply the same order, so
// every product pairs the same dz, W and hidden entries as in the natural order.

template <class E, int BM, int WM, bool ODD>
__global__ __launch_bounds__(128 * WM) void k_dz(DzArgs p) {
  using Eng = LogitEngine<E, BM, WM>;
  constexpr int RW = Eng::RW, WMB = Eng::WMB, WNB = Eng::WNB, NT = Eng::NT;
  constexpr bool kDirect = E::kSize == 2;  // 16-bit: stores straight from the registers
  static_assert(!kDirect || (BM == kTileCols && WM == 4), "the 16-bit store path is laid out for "
                                                          "the 256 x 256 tile with 4 x 2 waves");
  extern __shared__ u32x4 smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile tests become scalar
  const int wm = wave % WM, wn = wave / WM, i = lane & 15, g = lane >> 4;
  const int nbm = int((p.rows + BM - 1) / BM);
  const int nbn = int((p.V + kTileCols - 1) / kTileCols);
  int tm, tn;
  tile_of(blockIdx.x, nbm, nbn, tm, tn);
  const int64_t row0 = int64_t(tm) * BM, col0 = int64_t(tn) * kTileCols;
  const int64_t kbytes = p.D * E::kSize;

  f32x4_t acc[WMB][WNB];
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  Eng::template run<ODD>(acc, reinterpret_cast<const char*>(p.hidden) + row0 * kbytes, kbytes, p.rows - row0,
           reinterpret_cast<const char*>(p.weight) + col0 * kbytes, kbytes, p.V - col0, kbytes,
           smem);

  const int64_t cw = col0 + wn * kHalfCols;
  // Columns of this wave at or past lim are vocabulary padding (lim < 128 only in
  // the last vocabulary tile).
  const int lim = int(p.V - cw < kHalfCols ? p.V - cw : kHalfCols);
  f32x4_t csum[WNB];
  // The per-row inputs of the wave's rows and the bias are all loaded before the
  // first of them is used (rows past the batch read the last row, whose values are
  // then not used), so the epilogue waits for one memory round trip, not one per
  // input and row block.  The branches are wave-uniform and outside the row loops.
  auto rowc = [&](int mb) {
    const int64_t row = row0 + wm * RW + mb * 16 + i;
    return row < p.rows ? row : p.rows - 1;
  };
  float rtemp[WMB], rgrad[WMB], rlse[WMB];
  int64_t rt64[WMB];
  int32_t rt32[WMB];
  if (p.t64) {
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      rt64[mb] = reinterpret_cast<const int64_t*>(p.targets)[rowc(mb)];
      rt32[mb] = 0;
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
      rt32[mb] = reinterpret_cast<const int32_t*>(p.targets)[rowc(mb)];
      rt64[mb] = 0;
    }
  }
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    rgrad[mb] = p.grad_out[rowc(mb)];
    rlse[mb] = p.lse[rowc(mb)];
    rtemp[mb] = 1.0f;
  }
  if (p.temperature != nullptr) {
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) rtemp[mb] = p.temperature[rowc(mb)];
  }
  float bcol[WNB][4];
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb) {
    csum[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) bcol[nb][r] = 0.f;
  }
  if (p.bias != nullptr) {
    const float* bw = p.bias + cw + 4 * g;
    if (lim == kHalfCols) {  // wave-uniform: every column of the wave exists
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) bcol[nb][r] = bw[nb * 16 + r];
    } else {
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (nb * 16 + 4 * g + r < lim) bcol[nb][r] = bw[nb * 16 + r];
    }
  }
  // Nothing computed from the per-row inputs may move above this point (it would
  // wait for them in front of the bias loads).
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb)
    asm volatile("" : "+v"(rt32[mb]), "+v"(rt64[mb]), "+v"(rtemp[mb]), "+v"(rgrad[mb]), "+v"(rlse[mb]));
  // Per row block: k = log2(e) / T, L log2(e), G = grad / T (0 for an ignored target)
  // and the target's column within the wave (-1: not among its columns, -2: ignored).
  float rk[WMB], rl[WMB], rg[WMB];
  int rtc[WMB];
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int64_t row = row0 + wm * RW + mb * 16 + i;
    const bool rv = row < p.rows;
    const float invT = (p.temperature != nullptr && rv) ? 1.0f / rtemp[mb] : 1.0f;
    const int64_t t = !rv ? -1 : p.t64 ? rt64[mb] : int64_t(rt32[mb]);
    const bool valid = t >= 0 && t < p.V;
    rg[mb] = valid ? rgrad[mb] * invT : 0.f;
    rl[mb] = (rv ? rlse[mb] : 0.f) * kLog2e;
    rk[mb] = invT * kLog2e;
    const int64_t trel = t - cw;
    rtc[mb] = !valid ? -2 : (trel >= 0 && trel < kHalfCols) ? int(trel) : -1;
  }
  {
    // dz = G (onehot - exp(z - lse)) / T, kept in the accumulator registers, with
    // z = y / T, y = h W^T + b: the accumulators become y, and
    // exp(z - lse) = 2^(y (log2 e / T) - lse log2 e) is one FMA and one exp2 per logit.
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mb][nb][r] += bcol[nb][r];
      const int64_t row = row0 + wm * RW + mb * 16 + i;
      const float G = rg[mb], k = rk[mb], Ll = rl[mb];
      const bool valid = rtc[mb] != -2;
      const int tcol = rtc[mb] >= 0 ? rtc[mb] : -1;
      // Every kept logit is G (0 - p) = (-G) p (bit for bit, except that a p that
      // underflows to 0 gives a zero of the other sign); the target's entry,
      // G (1 - p), is taken from the row's logit before the tile is overwritten.
      // Few rows of a wave have their target among its 128 columns, so that part
      // runs under a branch most waves skip.
      float vt = 0.f;
      if (tcol >= 0) {
        float yt = 0.f;
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb * 16 + 4 * g + r == tcol) yt = acc[mb][nb][r];
        vt = G * (1.0f - fast_exp2(fmaf(yt, k, -Ll)));
      }
      const float nG = -G;
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mb][nb][r] = nG * fast_exp2(fmaf(acc[mb][nb][r], k, -Ll));
      if (tcol >= 0) {
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb * 16 + 4 * g + r == tcol) acc[mb][nb][r] = vt;
      }
      // Rows with an ignored target and the vocabulary padding get zeros (+0).
      if (!valid) {
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
      if (lim < kHalfCols) {  // wave-uniform: the last vocabulary tile only
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nb * 16 + 4 * g + r >= lim) acc[mb][nb][r] = 0.f;
      }
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) {
        const f32x4_t d = acc[mb][nb];
        csum[nb] += d;
        if constexpr (!kDirect) {
          constexpr int KB = 128 / E::kSize;
          const int64_t c = cw + nb * 16 + 4 * g;
          if (p.dz != nullptr) store4<E>(p.dz, kblk<KB>(row, c, p.ldt), d);
          if (p.dzT != nullptr) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int64_t at = kblk<KB>(c + r, row, p.ldz);
              if constexpr (E::kSize == 4)
                reinterpret_cast<float*>(p.dzT)[at] = d[r];
              else
                reinterpret_cast<uint16_t*>(p.dzT)[at] = uint16_t(bits16<E>(d[r]));
            }
          }
        }
      }
    }
  }
  if constexpr (kDirect) {
    // Lane (i, g) holds, for row block mb and the column blocks 2 c, 2 c + 1 of its
    // wave, token i at the vocabulary columns 32 c + 16 h + 4 g + r: in the K order
    // above, chunk g of the 32-wide step c of that token (16 bytes).
    //
    // dz^T: an MFMA multiplies such a chunk by a 0/1 matrix selecting 16 of its 32
    // columns (column 16 e + n for output column n), which lays the 16 x 16 block out
    // column-wise: lane (n, g) gets column 16 e + n at tokens 4 g + r.  A 16-bit value
    // times 1 plus zeros is exact in fp32, so these are the same bits.  The row blocks
    // 2 q and 2 q + 1 together give the tokens 32 q + 16 h + 4 g + r of one column:
    // chunk g of its 32-wide token step q.
    //
    // Stores.  A 128-byte K block is two such steps.  Lane i < 8 holds chunk g of
    // step 0 (X) for row i, lane i + 8 the same for row i + 8; their step-1 chunks
    // (Y) are swapped between the two lanes (lane i ^ 8, a DPP row rotation), after
    // which one store covers rows 0..7 (lanes i < 8: X at chunk g, lanes i >= 8: the
    // partner's Y at chunk 4 + g) and another rows 8..15: 8 rows x 128 bytes each.
    constexpr uint32_t kOne = std::is_same<E, F16>::value ? 0x3C00u : 0x3F80u;  // 1.0
    // The selection B operand: lane (n, g) supplies rows 8 g .. 8 g + 7 of column n,
    // and column n selects K slot 8 (n >> 2) + 4 e + (n & 3).
    u32x4 sel[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int jj = g == (i >> 2) ? 4 * e + (i & 3) : -1;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        sel[e][w] = (jj == 2 * w ? kOne : 0u) | (jj == 2 * w + 1 ? kOne << 16 : 0u);
    }
    const bool lo = i < 8;
    // Element offsets, within one 16-row block and one 128-byte K block, of this
    // lane's 16 bytes in the store of rows 0..7 (o0) and of rows 8..15 (o1).
    const int o0 = (i & 7) * 64 + (lo ? g : 4 + g) * 8;
    const int o1 = o0 + 8 * 64 + (lo ? 32 : -32);
    // The swap is a DPP row rotation by 8 whose bank mask writes only the lanes that
    // take the partner's value (banks 2 and 3 = lanes 8..15 for the first store,
    // banks 0 and 1 for the second); the other lanes keep x.
    auto store_pair = [&](uint16_t* base, const u32x4& x, const u32x4& y) {
      u32x4 s0, s1;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s0[w] = uint32_t(__builtin_amdgcn_update_dpp(int(x[w]), int(y[w]), 0x128, 0xF, 0xC, false));
        s1[w] = uint32_t(__builtin_amdgcn_update_dpp(int(x[w]), int(y[w]), 0x128, 0xF, 0x3, false));
      }
      __builtin_nontemporal_store(s0, reinterpret_cast<u32x4*>(base + o0));
      __builtin_nontemporal_store(s1, reinterpret_cast<u32x4*>(base + o1));
    };
    uint16_t* const dz = reinterpret_cast<uint16_t*>(p.dz);
    uint16_t* const dzT = reinterpret_cast<uint16_t*>(p.dzT);
    const int64_t tw = row0 + wm * RW;  // first token of this wave's rows (a multiple of 64)
#pragma unroll
    for (int b = 0; b < WNB / 4; ++b) {  // the two 128-byte K blocks of the wave's 128 columns
      u32x4 f[WMB][2];
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int nb = 4 * b + 2 * cc;
          f[mb][cc].x = pack2<E>(acc[mb][nb][0], acc[mb][nb][1]);
          f[mb][cc].y = pack2<E>(acc[mb][nb][2], acc[mb][nb][3]);
          f[mb][cc].z = pack2<E>(acc[mb][nb + 1][0], acc[mb][nb + 1][1]);
          f[mb][cc].w = pack2<E>(acc[mb][nb + 1][2], acc[mb][nb + 1][3]);
        }
      if (dz != nullptr) {
        const int64_t kb = (cw + 64 * b) / 64;  // K block of columns cw + 64 b .. + 63
#pragma unroll
        for (int mb = 0; mb < WMB; ++mb)
          store_pair(dz + (kb * p.ldt + tw + mb * 16) * 64, f[mb][0], f[mb][1]);
      }
      if (dzT != nullptr) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            u32x4 t[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              f32x4_t u0 = {0.f, 0.f, 0.f, 0.f}, u1 = {0.f, 0.f, 0.f, 0.f};
              mma64<E>(u0, f[2 * q][cc], sel[e]);
              mma64<E>(u1, f[2 * q + 1][cc], sel[e]);
              t[q] = u32x4{pack2<E>(u0[0], u0[1]), pack2<E>(u0[2], u0[3]), pack2<E>(u1[0], u1[1]),
                           pack2<E>(u1[2], u1[3])};
            }
            // rows: vocabulary columns cw + 64 b + 32 cc + 16 e + 0..15; K block: the
            // wave's 64 tokens
            const int64_t vrow = cw + 64 * b + 32 * cc + 16 * e;
            store_pair(dzT + ((tw / 64) * p.ldz + vrow) * 64, t[0], t[1]);
          }
      }
    }
  }
  if (p.dbias_part == nullptr) return;
  // Column sums over the tile's rows: in-lane over row blocks, then over the 16
  // lanes holding the other rows, then ascending over row waves.  The 16-lane step
  // is a reduce-scatter: a lane holds 32 column values (j = 4 nb + r); at the step
  // over lane bit m it keeps the half of its values that bit selects and adds the
  // partner's copy of that half, so after the four steps lane i holds the finished
  // sums of columns j = 2i and 2i + 1 (30 exchanges instead of 128).
  static_assert(WNB == 8, "the column reduction is laid out for 32 values per lane");
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [WM][256]
  {
    float v[4 * WNB];
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[4 * nb + r] = csum[nb][r];
#pragma unroll
    for (int h = 2 * WNB, m = 8; h >= 2; h >>= 1, m >>= 1) {
      const bool up = (i & m) != 0;
#pragma unroll
      for (int k = 0; k < h; ++k) {
        const float send = up ? v[k] : v[k + h];
        const float keep = up ? v[k + h] : v[k];
        v[k] = keep + lane_xor(send, m);
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int j = 2 * i + e;
      red[wm * kTileCols + wn * kHalfCols + (j >> 2) * 16 + 4 * g + (j & 3)] = v[e];
    }
  }
  __syncthreads();
  for (int c = tid; c < kTileCols; c += NT) {
    float s = red[c];
#pragma unroll
    for (int w = 1; w < WM; ++w) s += red[w * kTileCols + c];
    p.dbias_part[int64_t(tm) * p.ldz + col0 + c] = s;
  }
}

// ---- GEMMs of the backward ----------------------------------------------------------------
//
// C[M x N] (+)= sum_k A[m][k] B[n][k], both operands in the K-blocked layout.
//   d_hidden: M = tokens, N = D, K = V (padded); A = dz, B = W^T.
//   d_weight: M = V, N = D, K = tokens (padded); A = dz^T, B = hidden^T.
// LOAD: start from the fp32 accumulator p.acc; STORE: 0 = element type to p.out,
// 1 = fp32 to p.acc.
template <class E, int BM, int BN, int WM, int WN, bool LOAD, int STORE, int NS = 2, int NSA = NS>
__global__ __launch_bounds__(64 * WM * WN) void k_gemm(GemmArgs p) {
  using Eng = Engine<E, BM, BN, WM, WN, NS, NSA>;
  constexpr int RW = Eng::RW, CW = Eng::CW, WMB = Eng::WMB, WNB = Eng::WNB;
  extern __shared__ u32x4 smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM, i = lane & 15, g = lane >> 4;
  const int nbm = int((p.M + BM - 1) / BM), nbn = int((p.N + BN - 1) / BN);
  int tm, tn;
  tile_of<1>(blockIdx.x, nbm, nbn, tm, tn);
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t nl = n0 + wn * CW + 4 * g;

  f32x4_t acc[WMB][WNB];
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int64_t m = m0 + wm * RW + mb * 16 + i;
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      f32x4_t x = {0.f, 0.f, 0.f, 0.f};
      if (LOAD && m < p.M && nl + nb * 16 < p.N)
        x = *reinterpret_cast<const f32x4_t*>(p.acc + m * p.N + nl + nb * 16);
      acc[mb][nb] = x;
    }
  }
  Eng::template run<false>(acc, reinterpret_cast<const char*>(p.a) + m0 * p.lda_b, p.lda_b,
                           p.a_ks, p.M - m0, reinterpret_cast<const char*>(p.b) + n0 * p.ldb_b,
                           p.ldb_b, p.b_ks, p.N - n0, p.K * E::kSize, smem);

  if constexpr (STORE == 0 && E::kSize == 2) {
    // 16-bit output: the tile is staged in the operand ring (rows of BN values plus 16
    // bytes) and written as 16-byte chunks of whole output rows.  The output is
    // 16-byte aligned, its row stride (D elements) a multiple of 32 and N = D a
    // multiple of 8, so every chunk lies inside one row.
    constexpr int kRowB = BN * 2 + 16;
    constexpr int kCh = BN * 2 / 16;  // 16-byte chunks per tile row
    static_assert(size_t(BM) * kRowB <= Eng::kLds, "the staged tile fits the operand ring");
    char* lds = reinterpret_cast<char*>(smem);
    __syncthreads();  // every wave is done reading the operand ring
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) {
        const int rl = wm * RW + mb * 16 + i;
        const int cl = wn * CW + nb * 16 + 4 * g;
        u32x2 w;
        w.x = pack2<E>(acc[mb][nb][0], acc[mb][nb][1]);
        w.y = pack2<E>(acc[mb][nb][2], acc[mb][nb][3]);
        *reinterpret_cast<u32x2*>(lds + rl * kRowB + cl * 2) = w;
      }
    __syncthreads();
    for (int idx = tid; idx < BM * kCh; idx += Eng::NT) {
      const int rl = idx / kCh, ch = idx - rl * kCh;
      const int64_t m = m0 + rl, n = n0 + ch * 8;
      if (m < p.M && n < p.N)
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + m * p.ldo + n) =
            *reinterpret_cast<const u32x4*>(lds + rl * kRowB + ch * 16);
    }
    return;
  }

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

// ---- tiled transpose ---------------------------------------------------------------------------
// dst = src^T in the K-blocked layout (dst has `cols` rows and K = rows_pad);
// entries r in [rows, rows_pad) are written as zeros.
template <class T>
__global__ __launch_bounds__(256) void k_transpose(const T* __restrict__ src, int64_t rows,
                                                   int64_t rows_pad, int64_t cols, int64_t ld_src,
                                                   T* __restrict__ dst) {
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
    if (r < rows_pad && c < cols) dst[kblk<128 / sizeof(T)>(c, r, cols)] = tile[tx][k];
  }
}

// The same for 16-bit elements with 16-byte global accesses on both sides: a
// 64 x 64 tile is read as 8 16-byte chunks per source row and written as 8
// 16-byte chunks per destination row (one 128-byte K block).  Requires
// 16-byte aligned source rows and rows_pad a multiple of 64.  The destination's K
// positions take the fragment-major order of the 16-bit backward GEMMs: K
// position 32 b + 8 g + 4 h + r holds source row 32 b + 16 h + 4 g + r.
__global__ __launch_bounds__(256) void k_transpose16(const uint16_t* __restrict__ src, int64_t rows,
                                                     int64_t rows_pad, int64_t cols, int64_t ld_src,
                                                     uint16_t* __restrict__ dst) {
  __shared__ uint32_t tile[64][33];  // [row][column pair], 132-byte rows
  const int64_t r0 = int64_t(blockIdx.y) * 64, c0 = int64_t(blockIdx.x) * 64;
  const int t = threadIdx.x, j = t & 7, q = t >> 3;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int rl = q + 32 * p;
    const int64_t r = r0 + rl, c = c0 + 8 * j;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r < rows && c < cols) v = *reinterpret_cast<const u32x4*>(src + r * ld_src + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[rl][4 * j + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int cl = q + 32 * p;
    const int64_t c = c0 + cl, r = r0 + 8 * j;
    // K positions 8 j + k of the tile: block j >> 2, g = j & 3, h = k >> 2, r = k & 3.
    uint32_t h[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int src = 32 * (j >> 2) + 16 * (k >> 2) + 4 * (j & 3) + (k & 3);
      h[k] = (tile[src][cl >> 1] >> (16 * (cl & 1))) & 0xFFFFu;
    }
    const u32x4 w = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                     h[6] | (h[7] << 16)};
    if (c < cols && r < rows_pad) *reinterpret_cast<u32x4*>(dst + kblk<64>(c, r, cols)) = w;
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

// Dynamic LDS above 64 KiB must be opted into per kernel and device.  Each launch
// site keeps a per-device record of having done so; two threads that race on the
// first launch both set the same attribute.
constexpr int kMaxDevices = 64;
template <class K>
hipError_t prepare(K kernel, size_t lds, std::atomic<int> (&ready)[kMaxDevices]) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool tracked = dev >= 0 && dev < kMaxDevices;
  if (tracked && ready[dev].load(std::memory_order_acquire) != 0) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e == hipSuccess && tracked) ready[dev].store(1, std::memory_order_release);
  return e;
}

template <class E, int BM, int WM, bool ODD, int NS = 2>
hipError_t fwd_cfg(const FwdArgs& a, hipStream_t s) {
  using Eng = LogitEngine<E, BM, WM, NS>;
  static std::atomic<int> ready[kMaxDevices];
  const hipError_t e = prepare(k_fwd<E, BM, WM, ODD, NS>, Eng::kLds, ready);
  if (e != hipSuccess) return e;
  const int64_t blocks = ((a.N + BM - 1) / BM) * ((a.V + kTileCols - 1) / kTileCols);
  hipLaunchKernelGGL((k_fwd<E, BM, WM, ODD, NS>), dim3(unsigned(blocks)), dim3(Eng::NT), Eng::kLds,
                     s, a);
  return hipGetLastError();
}

// Number of 64-byte K stages of a logits tile is odd (D * element size / 64).
template <class E>
bool odd_stages(int64_t D) {
  return ((D * E::kSize) / kStageBytes) % 2 == 1;
}

template <class E, bool ODD>
hipError_t fwd_rows(const FwdArgs& a, hipStream_t s) {
  if (a.N <= 32) {
    // Over at most 256 vocabulary tiles (a vocabulary shard) the few workgroups each
    // wait out a load latency per stage with two stages, so they keep three in flight
    // (four LDS stages, 147 KB).  Over the full vocabulary the 2-stage tiles, two
    // workgroups per compute unit, stream W faster.
    const int64_t vt = (a.V + kTileCols - 1) / kTileCols;
    if (vt <= 256) return fwd_cfg<E, 32, 2, ODD, 4>(a, s);
    return fwd_cfg<E, 32, 2, ODD>(a, s);
  }
  if (a.N <= 64) return fwd_cfg<E, 64, 2, ODD>(a, s);
  if (a.N <= 128) return fwd_cfg<E, 128, 2, ODD>(a, s);
  return fwd_cfg<E, 256, 4, ODD>(a, s);
}

template <class E>
hipError_t fwd_dispatch(const FwdArgs& a, hipStream_t s) {
  return odd_stages<E>(a.D) ? fwd_rows<E, true>(a, s) : fwd_rows<E, false>(a, s);
}

template <class E, int BM, int WM, bool ODD>
hipError_t dz_cfg(const DzArgs& a, hipStream_t s) {
  using Eng = LogitEngine<E, BM, WM>;
  constexpr size_t lds = Eng::kLds;
  static std::atomic<int> ready[kMaxDevices];
  const hipError_t e = prepare(k_dz<E, BM, WM, ODD>, lds, ready);
  if (e != hipSuccess) return e;
  const int64_t blocks = ((a.rows + BM - 1) / BM) * ((a.V + kTileCols - 1) / kTileCols);
  hipLaunchKernelGGL((k_dz<E, BM, WM, ODD>), dim3(unsigned(blocks)), dim3(Eng::NT), lds, s, a);
  return hipGetLastError();
}

template <class E, int BM, int BN, int WM, int WN, bool LOAD, int STORE, int NS = 2, int NSA = NS>
hipError_t gemm_cfg(const GemmArgs& a, hipStream_t s) {
  using Eng = Engine<E, BM, BN, WM, WN, NS, NSA>;
  static std::atomic<int> ready[kMaxDevices];
  const hipError_t e = prepare(k_gemm<E, BM, BN, WM, WN, LOAD, STORE, NS, NSA>, Eng::kLds, ready);
  if (e != hipSuccess) return e;
  const int64_t blocks = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm<E, BM, BN, WM, WN, LOAD, STORE, NS, NSA>), dim3(unsigned(blocks)),
                     dim3(Eng::NT), Eng::kLds, s, a);
  return hipGetLastError();
}

// A-operand ring depth of the 256 x 224 backward GEMM tiles (B keeps two buffers):
// the split ring of Engine::split (d_hidden and d_weight 2 % faster than one ring of
// two stages, same bits).
constexpr int kGemmNSA = 3;

// The per-element MFMA chain does not depend on the tile shape, so the GEMM
// variants may use different tiles and still give the same bits.
//
// d_hidden walks the whole vocabulary for every tile and cannot split K without
// changing the bits, so a batch of few rows has few tiles: there the tiles shrink
// (more workgroups stream W^T side by side) and the LDS ring deepens.  Thresholds
// measured on the 16-bit training shape (D = 2688, V = 131072): 64 x 16 tiles are
// fastest up to 64 rows, 64 x 32 up to 128, 128 x 64 up to 512, 128 x 128 up to
// 1024, and the 256 x 224 tile from 2048 rows on.
template <class E>
hipError_t dx_tiles16(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 64) return gemm_cfg<E, 64, 16, 4, 1, false, 0, 8>(a, s);
  if (a.M <= 128) return gemm_cfg<E, 64, 32, 4, 1, false, 0, 8>(a, s);
  if (a.M <= 512) return gemm_cfg<E, 128, 64, 2, 2, false, 0, 4>(a, s);
  if (a.M <= 1024) return gemm_cfg<E, 128, 128, 2, 2, false, 0, 3>(a, s);
  return gemm_cfg<E, 256, 224, 4, 2, false, 0, 2, kGemmNSA>(a, s);
}
template <class E>
hipError_t dx_dispatch(const GemmArgs& a, hipStream_t s);
template <>
hipError_t dx_dispatch<BF16>(const GemmArgs& a, hipStream_t s) {
  return dx_tiles16<BF16>(a, s);
}
template <>
hipError_t dx_dispatch<F16>(const GemmArgs& a, hipStream_t s) {
  return dx_tiles16<F16>(a, s);
}
template <>
hipError_t dx_dispatch<F32>(const GemmArgs& a, hipStream_t s) {
  return gemm_cfg<F32, 128, 128, 2, 2, false, 0>(a, s);
}

template <class E>
hipError_t dw_dispatch(const GemmArgs& a, hipStream_t s);
template <>
hipError_t dw_dispatch<BF16>(const GemmArgs& a, hipStream_t s) {
  if (a.load_acc) {
    if (a.store_acc) return gemm_cfg<BF16, 256, 224, 4, 2, true, 1, 2, kGemmNSA>(a, s);
    return gemm_cfg<BF16, 256, 224, 4, 2, true, 0, 2, kGemmNSA>(a, s);
  }
  if (a.store_acc) return gemm_cfg<BF16, 256, 224, 4, 2, false, 1, 2, kGemmNSA>(a, s);
  return gemm_cfg<BF16, 256, 224, 4, 2, false, 0, 2, kGemmNSA>(a, s);
}
template <>
hipError_t dw_dispatch<F16>(const GemmArgs& a, hipStream_t s) {
  if (a.load_acc) {
    if (a.store_acc) return gemm_cfg<F16, 256, 224, 4, 2, true, 1, 2, kGemmNSA>(a, s);
    return gemm_cfg<F16, 256, 224, 4, 2, true, 0, 2, kGemmNSA>(a, s);
  }
  if (a.store_acc) return gemm_cfg<F16, 256, 224, 4, 2, false, 1, 2, kGemmNSA>(a, s);
  return gemm_cfg<F16, 256, 224, 4, 2, false, 0, 2, kGemmNSA>(a, s);
}
template <>
hipError_t dw_dispatch<F32>(const GemmArgs& a, hipStream_t s) {
  if (a.load_acc) {
    if (a.store_acc) return gemm_cfg<F32, 128, 128, 2, 2, true, 1>(a, s);
    return gemm_cfg<F32, 128, 128, 2, 2, true, 0>(a, s);
  }
  if (a.store_acc) return gemm_cfg<F32, 128, 128, 2, 2, false, 1>(a, s);
  return gemm_cfg<F32, 128, 128, 2, 2, false, 0>(a, s);
}

}  // namespace

hipError_t launch_forward(flp_dtype x, const FwdArgs& a, hipStream_t s) {
  ProfScope ps(FLP_K_FORWARD, s);
  if (x == FLP_BF16) return fwd_dispatch<BF16>(a, s);
  if (x == FLP_F16) return fwd_dispatch<F16>(a, s);
  return fwd_dispatch<F32>(a, s);
}

template <int R>
void merge_rows(const MergeArgs& a, hipStream_t s) {
  const dim3 grid(unsigned((a.N + R - 1) / R));
  const int64_t L = (a.n_vt + kMergeLeaves - 1) / kMergeLeaves;
  if (L == 1)
    hipLaunchKernelGGL((k_merge<R, 1>), grid, dim3(256), 0, s, a);
  else if (L == 2)
    hipLaunchKernelGGL((k_merge<R, 2>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((k_merge<R, 0>), grid, dim3(256), 0, s, a);
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t s) {
  ProfScope ps(FLP_K_MERGE, s);
  // One row per workgroup while that still gives a few workgroups per compute unit.
  if (a.N <= kMergeRowMax)
    merge_rows<1>(a, s);
  else
    merge_rows<8>(a, s);
  return hipGetLastError();
}

hipError_t launch_fill(float* dst, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, dst, n, value);
  return hipGetLastError();
}

hipError_t launch_logits_forward(flp_dtype x, const LogitsArgs& a, hipStream_t s) {
  ProfScope ps(FLP_K_LOGITS_FORWARD, s);
  const dim3 grid(unsigned((a.N + 3) / 4));
  if (x == FLP_BF16)
    hipLaunchKernelGGL(k_logits_fwd<BF16>, grid, dim3(256), 0, s, a);
  else if (x == FLP_F16)
    hipLaunchKernelGGL(k_logits_fwd<F16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_logits_fwd<F32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_logits_backward(flp_dtype x, const LogitsArgs& a, hipStream_t s) {
  ProfScope ps(FLP_K_LOGITS_BACKWARD, s);
  const dim3 grid(unsigned((a.N + 3) / 4));
  if (x == FLP_BF16)
    hipLaunchKernelGGL(k_logits_bwd<BF16>, grid, dim3(256), 0, s, a);
  else if (x == FLP_F16)
    hipLaunchKernelGGL(k_logits_bwd<F16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_logits_bwd<F32>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dz(flp_dtype x, const DzArgs& a, hipStream_t s) {
  ProfScope ps(FLP_K_DLOGITS, s);
  if (x == FLP_BF16)
    return odd_stages<BF16>(a.D) ? dz_cfg<BF16, int(kDzRowTile), 4, true>(a, s)
                                 : dz_cfg<BF16, int(kDzRowTile), 4, false>(a, s);
  if (x == FLP_F16)
    return odd_stages<F16>(a.D) ? dz_cfg<F16, int(kDzRowTile), 4, true>(a, s)
                                : dz_cfg<F16, int(kDzRowTile), 4, false>(a, s);
  return odd_stages<F32>(a.D) ? dz_cfg<F32, int(kDzRowTile), 4, true>(a, s)
                              : dz_cfg<F32, int(kDzRowTile), 4, false>(a, s);
}

hipError_t launch_dx(flp_dtype x, const GemmArgs& a, hipStream_t s) {
  ProfScope ps(FLP_K_DHIDDEN, s);
  if (x == FLP_BF16) return dx_dispatch<BF16>(a, s);
  if (x == FLP_F16) return dx_dispatch<F16>(a, s);
  return dx_dispatch<F32>(a, s);
}

hipError_t launch_dw(flp_dtype x, const GemmArgs& a, hipStream_t s) {
  ProfScope ps(FLP_K_DWEIGHT, s);
  if (x == FLP_BF16) return dw_dispatch<BF16>(a, s);
  if (x == FLP_F16) return dw_dispatch<F16>(a, s);
  return dw_dispatch<F32>(a, s);
}

hipError_t launch_transpose(flp_dtype x, const void* src, int64_t rows, int64_t rows_pad, int64_t cols,
                            int64_t ld_src, void* dst, hipStream_t s) {
  ProfScope ps(FLP_K_TRANSPOSE, s);
  const dim3 grid(unsigned((cols + 63) / 64), unsigned((rows_pad + 63) / 64));
  if (x != FLP_F32)
    hipLaunchKernelGGL(k_transpose16, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src),
                       rows, rows_pad, cols, ld_src, static_cast<uint16_t*>(dst));
  else
    hipLaunchKernelGGL(k_transpose<float>, grid, dim3(256), 0, s, static_cast<const float*>(src),
                       rows, rows_pad, cols, ld_src, static_cast<float*>(dst));
  return hipGetLastError();
}

hipError_t launch_dbias_fold(const float* part, int64_t n_parts, int64_t ldz, int64_t V,
                             float* d_bias, int init, hipStream_t s) {
  ProfScope ps(FLP_K_DBIAS, s);
  hipLaunchKernelGGL(k_dbias_fold, dim3(unsigned((V + 255) / 256)), dim3(256), 0, s, part, n_parts,
                     ldz, V, d_bias, init);
  return hipGetLastError();
}

const char* kernel_ids() {
  return "engine: direct global->LDS (buffer_load_dwordx4 lds, whole lines), 2 LDS stages x 128 B of K "
         "(3-8 for the small dX tiles), "
         "mfma_f32_16x16x32_bf16 | 16x16x32_f16 | 16x16x4f32; k_fwd<BM 32/64/128 x BN 256 2x2 waves (BM 32: 4 stages over <= 256 vocabulary tiles), "
         "BM 256 4x2 waves>; k_merge<1 or 8 rows; 256 leaves, fixed tree>; k_dz<BM 256 x BN 256, 4x2 waves>; "
         "k_gemm dX, dW<256x224, 4x2 waves, K-blocked operands; dX for <= 1024 rows: 64x16, "
         "64x32, 128x64, 128x128>; k_transpose (K-blocked); "
         "k_dbias_fold; k_fill; k_logits_fwd, k_logits_bwd<one wave per row>; "
         "rows: k_mark, k_compact, k_gather, k_scatter_rows, k_scatter_hidden; "
         "embedding: k_embed_fwd, radix sort (k_sort_init, k_sort_hist, k_sort_scatter; zero-row "
         "riders), k_seg_bounds, k_embed_runs<32-position groups>, k_embed_rows";
}

}  // namespace flp
