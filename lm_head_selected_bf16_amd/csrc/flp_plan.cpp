// Workspace layouts and fail-closed argument validation for the C ABI.
// Pure host arithmetic: no HIP call, no pointer is ever dereferenced, so every
// gate can be exercised on a machine without a GPU.
#include "flp_plan.h"

#include <algorithm>
#include <limits>

namespace flp {

namespace {

constexpr int64_t kMaxIndex = std::numeric_limits<int64_t>::max() / 16;

bool mul_ok(int64_t a, int64_t b) { return a == 0 || b <= kMaxIndex / a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Span {
  uintptr_t lo = 0, hi = 0;
  bool live() const { return hi > lo; }
};

Span span(const void* p, size_t bytes) {
  Span s;
  if (p != nullptr && bytes > 0) {
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + bytes;
  }
  return s;
}

bool overlap(const Span& a, const Span& b) {
  return a.live() && b.live() && a.lo < b.hi && b.lo < a.hi;
}

// Every output span must be disjoint from every input span and from every other
// output span.
bool any_alias(const Span* outs, int n_out, const Span* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = 0; j < n_in; ++j)
      if (overlap(outs[i], ins[j])) return true;
    for (int j = i + 1; j < n_out; ++j)
      if (overlap(outs[i], outs[j])) return true;
  }
  return false;
}

// An empty batch writes only d_weight and d_bias, as zeros (sums over no rows).
flp_status validate_empty_sums(int64_t D, int64_t V, size_t xs, const void* weight,
                               const float* bias, const void* d_weight, flp_dtype dw,
                               const float* d_bias) {
  if (!aligned(d_weight, 16) || !aligned(d_bias, 4)) return FLP_MISALIGNED;
  const Span ins[] = {span(weight, size_t(V) * D * xs), span(bias, size_t(V) * 4)};
  const Span outs[] = {span(d_weight, size_t(V) * D * dtype_size(dw)), span(d_bias, size_t(V) * 4)};
  return any_alias(outs, 2, ins, 2) ? FLP_INVALID_ARGUMENT : FLP_OK;
}

flp_status check_dims(int64_t N, int64_t D, int64_t V, flp_dtype x, flp_dtype t) {
  if (N < 0 || D < 1 || V < 1) return FLP_INVALID_ARGUMENT;
  if (x != FLP_BF16 && x != FLP_F16 && x != FLP_F32) return FLP_UNSUPPORTED_DTYPE;
  if (t != FLP_I64 && t != FLP_I32) return FLP_UNSUPPORTED_DTYPE;
  if (D % 32 != 0) return FLP_UNSUPPORTED_SHAPE;
  // The logit-tile kernels address the rows of a hidden / weight tile through a
  // buffer resource with 32-bit offsets (row r of at most 256 at r * D * size,
  // plus the chunk within the 128-byte stage): every such offset must stay below
  // the resource's 2^31 - 1 records.
  if (D > kMaxIndex / 256 || D * int64_t(dtype_size(x)) * 256 >= (int64_t(1) << 31))
    return FLP_UNSUPPORTED_SHAPE;
  const int64_t rows = std::max<int64_t>(round_up(std::max<int64_t>(N, 1), kRowQuantum), 1);
  const int64_t ldz = round_up(V, kVocabTile);
  if (!mul_ok(rows, D) || !mul_ok(ldz, D) || !mul_ok(rows, ldz) ||
      !mul_ok(ceil_div(V, kVocabTile), rows))
    return FLP_UNSUPPORTED_SHAPE;
  // Grid limits: row tiles x vocab tiles and the output tiles of the GEMMs.
  if (ceil_div(rows, 16) * ceil_div(V, kVocabTile) > (int64_t(1) << 31) - 1) return FLP_UNSUPPORTED_SHAPE;
  return FLP_OK;
}

}  // namespace

FwdLayout fwd_layout(int64_t N, int64_t /*D*/, int64_t V) {
  FwdLayout L;
  L.n_vt = ceil_div(V, kVocabTile);
  L.part_off = 0;
  L.zt_off = align_up(size_t(L.n_vt) * size_t(N) * 8);
  L.total = L.zt_off + align_up(size_t(N) * 4);
  return L;
}

BwdLayout bwd_layout_for_chunk(int64_t N, int64_t D, int64_t V, flp_dtype x, flp_dtype dw,
                               int64_t chunk, bool need_dh, bool need_dw, bool need_db) {
  BwdLayout L;
  const int64_t full = round_up(std::max<int64_t>(N, 1), kRowQuantum);
  chunk = std::min(round_up(std::max<int64_t>(chunk, 1), kRowQuantum), full);
  const size_t xs = dtype_size(x);
  L.chunk = chunk;
  L.n_chunks = ceil_div(std::max<int64_t>(N, 1), chunk);
  L.ldz = round_up(V, kVocabTile);
  L.ldt = chunk;
  size_t off = 0;
  L.dz_off = off;
  if (need_dh) off += align_up(size_t(chunk) * size_t(L.ldz) * xs);
  L.wt_off = off;  // W^T [D][ldz], zero-padded past V
  if (need_dh) off += align_up(size_t(D) * size_t(L.ldz) * xs);
  L.dzt_off = off;
  if (need_dw) off += align_up(size_t(L.ldz) * size_t(chunk) * xs);
  L.ht_off = off;
  if (need_dw) off += align_up(size_t(D) * size_t(chunk) * xs);
  L.dbp_off = off;
  if (need_db) off += align_up(size_t(chunk / kDzRowTile) * size_t(L.ldz) * 4);
  L.acc_off = off;
  L.use_acc = need_dw && dw != FLP_F32 && L.n_chunks > 1;
  if (L.use_acc) off += align_up(size_t(V) * size_t(D) * 4);
  L.total = std::max<size_t>(off, kAlign);
  return L;
}

BwdLayout bwd_layout_for_bytes(int64_t N, int64_t D, int64_t V, flp_dtype x, flp_dtype dw,
                               size_t bytes, bool need_dh, bool need_dw, bool need_db) {
  const int64_t full = round_up(std::max<int64_t>(N, 1), kRowQuantum);
  BwdLayout L = bwd_layout_for_chunk(N, D, V, x, dw, full, need_dh, need_dw, need_db);
  if (L.total <= bytes) return L;
  // Several chunks: the fp32 accumulator (if any) plus per-chunk buffers.
  const size_t ldz = size_t(round_up(V, kVocabTile));
  const size_t xs = dtype_size(x);
  const size_t q = size_t(kRowQuantum);
  const size_t per_quantum = (need_dh ? q * ldz * xs : 0) + (need_dw ? q * (ldz + size_t(D)) * xs : 0) +
                             (need_db ? (q / size_t(kDzRowTile)) * ldz * 4 : 0);
  const size_t fixed = ((need_dw && dw != FLP_F32) ? align_up(size_t(V) * size_t(D) * 4) : 0) +
                       (need_dh ? align_up(size_t(D) * ldz * xs) : 0);
  // The layout of nq quanta takes fixed + nq * per_quantum bytes plus alignment
  // padding, so this nq is an upper bound; step down to the first that fits.
  int64_t nq = 0;
  if (per_quantum > 0 && bytes > fixed) nq = int64_t((bytes - fixed) / per_quantum);
  nq = std::min<int64_t>(nq, full / kRowQuantum);
  if (need_dh && nq > 0) {
    // Round the chunk down to a whole number of d_hidden waves when that is possible.
    const bool f32 = x == FLP_F32;
    const int64_t tm = f32 ? kGemmTile32 : kGemmTileM16, tn = f32 ? kGemmTile32 : kGemmTileN16;
    const int64_t ct = ceil_div(D, tn);
    int64_t a = ct, b = kNumCUs;  // gcd
    while (b != 0) {
      const int64_t r = a % b;
      a = b;
      b = r;
    }
    const int64_t wave_rows = (kNumCUs / a) * tm;
    if (wave_rows % kRowQuantum == 0) {
      const int64_t wq = wave_rows / kRowQuantum;
      if (nq >= wq) nq = nq / wq * wq;
    }
  }
  for (; nq >= 1; --nq) {
    L = bwd_layout_for_chunk(N, D, V, x, dw, nq * kRowQuantum, need_dh, need_dw, need_db);
    if (L.total <= bytes) return L;
  }
  L = BwdLayout();
  return L;
}

SelLayout sel_layout(int64_t N, int64_t n_rows) {
  SelLayout L;
  L.cap = std::max<int64_t>(std::min(n_rows, N), 0);
  size_t off = 0;
  L.mask_off = off;
  off += align_up(size_t(std::max<int64_t>(N, 0)));
  L.pos_off = off;
  off += align_up(size_t(std::max<int64_t>(N, 0)) * 4);
  L.sel_off = off;
  off += align_up(size_t(L.cap) * 4);
  L.total = std::max<size_t>(off, kAlign);
  return L;
}

IdxLayout idx_layout(int64_t N, int64_t D, int64_t n_rows, flp_dtype x, bool backward,
                     bool need_dh) {
  IdxLayout L;
  L.sel = sel_layout(N, n_rows);
  const size_t c = size_t(L.sel.cap);
  const size_t row_bytes = size_t(D) * dtype_size(x);
  size_t off = L.sel.total;
  L.h_off = off;
  off += align_up(c * row_bytes);
  L.t_off = off;
  off += align_up(c * 8);
  L.temp_off = off;
  off += align_up(c * 4);
  if (backward) {
    L.g_off = off;
    off += align_up(c * 4);
    L.lse_in_off = off;
    off += align_up(c * 4);
    L.dh_off = off;
    if (need_dh) off += align_up(c * row_bytes);
  } else {
    L.logp_off = off;
    off += align_up(c * 4);
    L.lse_off = off;
    off += align_up(c * 4);
  }
  L.dense_off = off;
  return L;
}

EmbLayout emb_layout(int64_t N, int64_t D, int64_t V) {
  EmbLayout L;
  const size_t n = size_t(std::max<int64_t>(N, 0));
  L.n_blocks = ceil_div(std::max<int64_t>(N, 1), kEmbSortBlock);
  size_t off = 0;
  for (int k = 0; k < 2; ++k) {
    L.keys_off[k] = off;
    off += align_up(n * 4);
    L.vals_off[k] = off;
    off += align_up(n * 4);
  }
  L.hist_off = off;
  off += align_up(size_t(256) * size_t(L.n_blocks) * 4);
  L.seg_begin_off = off;
  off += align_up(size_t(V) * 4);
  L.seg_end_off = off;
  off += align_up(size_t(V) * 4);
  const size_t groups = size_t(ceil_div(std::max<int64_t>(N, 1), kEmbSegGroup));
  L.head_off = off;
  off += align_up(groups * size_t(D) * 4);
  L.tail_off = off;
  off += align_up(groups * size_t(D) * 4);
  L.total = off;
  return L;
}

flp_status validate_rows(int64_t N, const void* rows, flp_dtype r, int64_t n_rows) {
  if (N < 0 || n_rows < 0) return FLP_INVALID_ARGUMENT;
  if (r != FLP_I64 && r != FLP_I32) return FLP_UNSUPPORTED_DTYPE;
  if (N > kMaxIndexedRows || n_rows > kMaxIndex / 8) return FLP_UNSUPPORTED_SHAPE;
  if (n_rows > 0 && rows == nullptr) return FLP_INVALID_ARGUMENT;
  if (!aligned(rows, dtype_size(r))) return FLP_MISALIGNED;
  return FLP_OK;
}

namespace {
// The forward's gates.  own_scratch: the workspace is the library's own fixed
// array (the allocation-free entry point), which cannot overlap a caller's
// buffer, so only its size is checked.
flp_status forward_gates(int64_t N, int64_t D, int64_t V, flp_dtype x, const void* hidden,
                         const void* weight, const float* bias, const void* targets, flp_dtype t,
                         const float* temperature, const float* out_logp, const float* out_lse,
                         const void* workspace, size_t workspace_bytes, bool own_scratch) {
  flp_status st = check_dims(N, D, V, x, t);
  if (st != FLP_OK) return st;
  if (N == 0) return FLP_OK;
  if (!hidden || !weight || !targets || !out_logp || (!own_scratch && !workspace))
    return FLP_INVALID_ARGUMENT;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || (!own_scratch && !aligned(workspace, 16)) ||
      !aligned(bias, 4) || !aligned(temperature, 4) || !aligned(out_logp, 4) ||
      !aligned(out_lse, 4) || !aligned(targets, dtype_size(t)))
    return FLP_MISALIGNED;
  const size_t xs = dtype_size(x);
  const Span ins[] = {span(hidden, size_t(N) * D * xs), span(weight, size_t(V) * D * xs),
                      span(bias, size_t(V) * 4), span(targets, size_t(N) * dtype_size(t)),
                      span(temperature, size_t(N) * 4)};
  const Span outs[] = {span(out_logp, size_t(N) * 4), span(out_lse, size_t(N) * 4),
                       own_scratch ? Span() : span(workspace, workspace_bytes)};
  if (any_alias(outs, 3, ins, 5)) return FLP_INVALID_ARGUMENT;
  if (workspace_bytes < fwd_layout(N, D, V).total) return FLP_WORKSPACE_TOO_SMALL;
  return FLP_OK;
}
}  // namespace

flp_status validate_forward(int64_t N, int64_t D, int64_t V, flp_dtype x, const void* hidden,
                            const void* weight, const float* bias, const void* targets,
                            flp_dtype t, const float* temperature, const float* out_logp,
                            const float* out_lse, const void* workspace,
                            size_t workspace_bytes) {
  return forward_gates(N, D, V, x, hidden, weight, bias, targets, t, temperature, out_logp,
                       out_lse, workspace, workspace_bytes, false);
}

flp_status validate_forward_noalloc(int64_t N, int64_t D, int64_t V, flp_dtype x,
                                    const void* hidden, const void* weight, const float* bias,
                                    const void* targets, flp_dtype t, const float* temperature,
                                    const float* out_logp, const float* out_lse,
                                    size_t scratch_bytes) {
  return forward_gates(N, D, V, x, hidden, weight, bias, targets, t, temperature, out_logp,
                       out_lse, nullptr, scratch_bytes, true);
}

flp_status validate_forward_partial(int64_t N, int64_t D, int64_t V_local, int64_t vocab_start,
                                    int64_t V_total, flp_dtype x, const void* hidden,
                                    const void* weight, const float* bias, const void* targets,
                                    flp_dtype t, const float* temperature, const void* partial,
                                    const float* zt) {
  flp_status st = check_dims(N, D, V_local, x, t);
  if (st != FLP_OK) return st;
  if (vocab_start < 0 || V_total < 1 || vocab_start > V_total - V_local) return FLP_INVALID_ARGUMENT;
  // Shard boundaries on vocabulary-tile boundaries keep every tile, and so every
  // partial, identical to the unsharded one.
  if (vocab_start % kVocabTile != 0) return FLP_UNSUPPORTED_SHAPE;
  if (V_local % kVocabTile != 0 && vocab_start + V_local != V_total) return FLP_UNSUPPORTED_SHAPE;
  if (N == 0) return FLP_OK;
  if (!hidden || !weight || !targets || !partial || !zt) return FLP_INVALID_ARGUMENT;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(partial, 16) || !aligned(zt, 4) ||
      !aligned(bias, 4) || !aligned(temperature, 4) || !aligned(targets, dtype_size(t)))
    return FLP_MISALIGNED;
  const size_t xs = dtype_size(x);
  const Span ins[] = {span(hidden, size_t(N) * D * xs), span(weight, size_t(V_local) * D * xs),
                      span(bias, size_t(V_local) * 4), span(targets, size_t(N) * dtype_size(t)),
                      span(temperature, size_t(N) * 4)};
  const Span outs[] = {span(partial, size_t(ceil_div(V_local, kVocabTile)) * size_t(N) * 8),
                       span(zt, size_t(N) * 4)};
  if (any_alias(outs, 2, ins, 5)) return FLP_INVALID_ARGUMENT;
  return FLP_OK;
}

flp_status validate_merge(int64_t N, int64_t V_total, const void* partials, const float* zt,
                          const void* targets, flp_dtype t, const float* out_logp,
                          const float* out_lse) {
  if (N < 0 || V_total < 1) return FLP_INVALID_ARGUMENT;
  if (t != FLP_I64 && t != FLP_I32) return FLP_UNSUPPORTED_DTYPE;
  const int64_t n_vt = ceil_div(V_total, kVocabTile);
  if (!mul_ok(n_vt, std::max<int64_t>(N, 1)) || !mul_ok(n_vt * std::max<int64_t>(N, 1), 8))
    return FLP_UNSUPPORTED_SHAPE;
  if (N == 0) return FLP_OK;
  if (!partials || !zt || !targets || !out_logp) return FLP_INVALID_ARGUMENT;
  if (!aligned(partials, 16) || !aligned(zt, 4) || !aligned(out_logp, 4) || !aligned(out_lse, 4) ||
      !aligned(targets, dtype_size(t)))
    return FLP_MISALIGNED;
  const Span ins[] = {span(partials, size_t(n_vt) * size_t(N) * 8), span(zt, size_t(N) * 4),
                      span(targets, size_t(N) * dtype_size(t))};
  const Span outs[] = {span(out_logp, size_t(N) * 4), span(out_lse, size_t(N) * 4)};
  if (any_alias(outs, 2, ins, 3)) return FLP_INVALID_ARGUMENT;
  return FLP_OK;
}

namespace {

flp_status check_logits_dims(int64_t N, int64_t V, flp_dtype x, flp_dtype t) {
  if (N < 0 || V < 1) return FLP_INVALID_ARGUMENT;
  if (x != FLP_BF16 && x != FLP_F16 && x != FLP_F32) return FLP_UNSUPPORTED_DTYPE;
  if (t != FLP_I64 && t != FLP_I32) return FLP_UNSUPPORTED_DTYPE;
  // Rows are streamed in 16-byte chunks.
  if ((V * int64_t(dtype_size(x))) % 16 != 0) return FLP_UNSUPPORTED_SHAPE;
  const int64_t n = std::max<int64_t>(N, 1);
  if (!mul_ok(n, V) || !mul_ok(n * V, 8) || ceil_div(n, 4) > (int64_t(1) << 31) - 1)
    return FLP_UNSUPPORTED_SHAPE;
  return FLP_OK;
}

}  // namespace

flp_status validate_logits_forward(int64_t N, int64_t V, flp_dtype x, const void* logits,
                                   const void* targets, flp_dtype t, const float* out_logp,
                                   const float* out_lse) {
  flp_status st = check_logits_dims(N, V, x, t);
  if (st != FLP_OK || N == 0) return st;
  if (!logits || !targets || !out_logp) return FLP_INVALID_ARGUMENT;
  if (!aligned(logits, 16) || !aligned(out_logp, 4) || !aligned(out_lse, 4) ||
      !aligned(targets, dtype_size(t)))
    return FLP_MISALIGNED;
  const Span ins[] = {span(logits, size_t(N) * size_t(V) * dtype_size(x)),
                      span(targets, size_t(N) * dtype_size(t))};
  const Span outs[] = {span(out_logp, size_t(N) * 4), span(out_lse, size_t(N) * 4)};
  if (any_alias(outs, 2, ins, 2)) return FLP_INVALID_ARGUMENT;
  return FLP_OK;
}

flp_status validate_logits_backward(int64_t N, int64_t V, flp_dtype x, const float* grad_out,
                                    const float* lse, const void* logits, const void* targets,
                                    flp_dtype t, const void* d_logits) {
  flp_status st = check_logits_dims(N, V, x, t);
  if (st != FLP_OK || N == 0) return st;
  if (!grad_out || !lse || !logits || !targets || !d_logits) return FLP_INVALID_ARGUMENT;
  if (!aligned(logits, 16) || !aligned(d_logits, 16) || !aligned(grad_out, 4) ||
      !aligned(lse, 4) || !aligned(targets, dtype_size(t)))
    return FLP_MISALIGNED;
  const Span ins[] = {span(grad_out, size_t(N) * 4), span(lse, size_t(N) * 4),
                      span(logits, size_t(N) * size_t(V) * dtype_size(x)),
                      span(targets, size_t(N) * dtype_size(t))};
  const Span outs[] = {span(d_logits, size_t(N) * size_t(V) * dtype_size(x))};
  if (any_alias(outs, 1, ins, 4)) return FLP_INVALID_ARGUMENT;
  return FLP_OK;
}

flp_status validate_backward(int64_t N, int64_t D, int64_t V, flp_dtype x, const float* grad_out,
                             const float* lse, const void* hidden, const void* weight,
                             const float* bias, const void* targets, flp_dtype t,
                             const float* temperature, const void* d_hidden,
                             const void* d_weight, flp_dtype dw, const float* d_bias,
                             const void* workspace, size_t workspace_bytes) {
  flp_status st = check_dims(N, D, V, x, t);
  if (st != FLP_OK) return st;
  if (dw != x && dw != FLP_F32) return FLP_UNSUPPORTED_DTYPE;
  if (N == 0) return validate_empty_sums(D, V, dtype_size(x), weight, bias, d_weight, dw, d_bias);
  if (!grad_out || !lse || !hidden || !weight || !targets) return FLP_INVALID_ARGUMENT;
  if (!d_hidden && !d_weight && !d_bias) return FLP_OK;
  if (!workspace) return FLP_INVALID_ARGUMENT;
  const size_t xs = dtype_size(x);
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 16) ||
      !aligned(grad_out, 4) || !aligned(lse, 4) || !aligned(bias, 4) ||
      !aligned(temperature, 4) || !aligned(targets, dtype_size(t)) ||
      !aligned(d_hidden, 16) || !aligned(d_weight, 16) || !aligned(d_bias, 4))
    return FLP_MISALIGNED;
  const Span ins[] = {span(grad_out, size_t(N) * 4), span(lse, size_t(N) * 4),
                      span(hidden, size_t(N) * D * xs), span(weight, size_t(V) * D * xs),
                      span(bias, size_t(V) * 4), span(targets, size_t(N) * dtype_size(t)),
                      span(temperature, size_t(N) * 4)};
  const Span outs[] = {span(d_hidden, size_t(N) * D * xs),
                       span(d_weight, size_t(V) * D * dtype_size(dw)),
                       span(d_bias, size_t(V) * 4), span(workspace, workspace_bytes)};
  if (any_alias(outs, 4, ins, 7)) return FLP_INVALID_ARGUMENT;
  const BwdLayout L = bwd_layout_for_bytes(N, D, V, x, dw, workspace_bytes, d_hidden != nullptr,
                                           d_weight != nullptr, d_bias != nullptr);
  if (L.chunk == 0) return FLP_WORKSPACE_TOO_SMALL;
  return FLP_OK;
}

flp_status validate_forward_indexed(int64_t N, int64_t D, int64_t V, flp_dtype x,
                                    const void* hidden, const void* weight, const float* bias,
                                    const void* targets, flp_dtype t, const float* temperature,
                                    const void* rows, flp_dtype r, int64_t n_rows,
                                    const float* out_logp, const float* out_lse,
                                    const void* workspace, size_t workspace_bytes) {
  flp_status st = check_dims(N, D, V, x, t);
  if (st != FLP_OK) return st;
  if ((st = validate_rows(N, rows, r, n_rows)) != FLP_OK) return st;
  if (N == 0) return FLP_OK;
  if (!hidden || !weight || !targets || !out_logp || !workspace) return FLP_INVALID_ARGUMENT;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 16) ||
      !aligned(bias, 4) || !aligned(temperature, 4) || !aligned(out_logp, 4) ||
      !aligned(out_lse, 4) || !aligned(targets, dtype_size(t)))
    return FLP_MISALIGNED;
  const size_t xs = dtype_size(x);
  const Span ins[] = {span(hidden, size_t(N) * D * xs), span(weight, size_t(V) * D * xs),
                      span(bias, size_t(V) * 4), span(targets, size_t(N) * dtype_size(t)),
                      span(temperature, size_t(N) * 4), span(rows, size_t(n_rows) * dtype_size(r))};
  const Span outs[] = {span(out_logp, size_t(N) * 4), span(out_lse, size_t(N) * 4),
                       span(workspace, workspace_bytes)};
  if (any_alias(outs, 3, ins, 6)) return FLP_INVALID_ARGUMENT;
  const IdxLayout L = idx_layout(N, D, n_rows, x, false, false);
  const size_t need = L.dense_off + (L.sel.cap > 0 ? fwd_layout(L.sel.cap, D, V).total : 0);
  if (workspace_bytes < need) return FLP_WORKSPACE_TOO_SMALL;
  return FLP_OK;
}

flp_status validate_backward_indexed(int64_t N, int64_t D, int64_t V, flp_dtype x,
                                     const float* grad_out, const float* lse, const void* hidden,
                                     const void* weight, const float* bias, const void* targets,
                                     flp_dtype t, const float* temperature, const void* rows,
                                     flp_dtype r, int64_t n_rows, const void* d_hidden,
                                     const void* d_weight, flp_dtype dw, const float* d_bias,
                                     const void* workspace, size_t workspace_bytes) {
  flp_status st = check_dims(N, D, V, x, t);
  if (st != FLP_OK) return st;
  if (dw != x && dw != FLP_F32) return FLP_UNSUPPORTED_DTYPE;
  if ((st = validate_rows(N, rows, r, n_rows)) != FLP_OK) return st;
  if (N == 0) return validate_empty_sums(D, V, dtype_size(x), weight, bias, d_weight, dw, d_bias);
  if (!grad_out || !lse || !hidden || !weight || !targets) return FLP_INVALID_ARGUMENT;
  if (!d_hidden && !d_weight && !d_bias) return FLP_OK;
  if (!workspace) return FLP_INVALID_ARGUMENT;
  const size_t xs = dtype_size(x);
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(workspace, 16) ||
      !aligned(grad_out, 4) || !aligned(lse, 4) || !aligned(bias, 4) ||
      !aligned(temperature, 4) || !aligned(targets, dtype_size(t)) ||
      !aligned(d_hidden, 16) || !aligned(d_weight, 16) || !aligned(d_bias, 4))
    return FLP_MISALIGNED;
  const Span ins[] = {span(grad_out, size_t(N) * 4), span(lse, size_t(N) * 4),
                      span(hidden, size_t(N) * D * xs), span(weight, size_t(V) * D * xs),
                      span(bias, size_t(V) * 4), span(targets, size_t(N) * dtype_size(t)),
                      span(temperature, size_t(N) * 4), span(rows, size_t(n_rows) * dtype_size(r))};
  const Span outs[] = {span(d_hidden, size_t(N) * D * xs),
                       span(d_weight, size_t(V) * D * dtype_size(dw)),
                       span(d_bias, size_t(V) * 4), span(workspace, workspace_bytes)};
  if (any_alias(outs, 4, ins, 8)) return FLP_INVALID_ARGUMENT;
  const IdxLayout L = idx_layout(N, D, n_rows, x, true, d_hidden != nullptr);
  if (workspace_bytes < L.dense_off) return FLP_WORKSPACE_TOO_SMALL;
  if (L.sel.cap > 0 &&
      bwd_layout_for_bytes(L.sel.cap, D, V, x, dw, workspace_bytes - L.dense_off,
                           d_hidden != nullptr, d_weight != nullptr, d_bias != nullptr)
              .chunk == 0)
    return FLP_WORKSPACE_TOO_SMALL;
  return FLP_OK;
}

flp_status validate_logits_indexed(int64_t N, int64_t V, flp_dtype x, bool backward,
                                   const float* grad_out, const float* lse, const void* logits,
                                   const void* targets, flp_dtype t, const void* rows,
                                   flp_dtype r, int64_t n_rows, const void* out_a,
                                   const void* out_b, const void* workspace,
                                   size_t workspace_bytes) {
  flp_status st = check_logits_dims(N, V, x, t);
  if (st != FLP_OK) return st;
  if ((st = validate_rows(N, rows, r, n_rows)) != FLP_OK) return st;
  if (N == 0) return FLP_OK;
  if (!logits || !targets || !out_a || !workspace) return FLP_INVALID_ARGUMENT;
  if (backward && (!grad_out || !lse)) return FLP_INVALID_ARGUMENT;
  const size_t row_out = backward ? size_t(V) * dtype_size(x) : 4;
  if (!aligned(logits, 16) || !aligned(out_a, backward ? 16 : 4) || !aligned(out_b, 4) ||
      !aligned(grad_out, 4) || !aligned(lse, 4) || !aligned(targets, dtype_size(t)))
    return FLP_MISALIGNED;
  const Span ins[] = {span(logits, size_t(N) * size_t(V) * dtype_size(x)),
                      span(targets, size_t(N) * dtype_size(t)), span(grad_out, size_t(N) * 4),
                      span(lse, size_t(N) * 4), span(rows, size_t(n_rows) * dtype_size(r))};
  const Span outs[] = {span(out_a, size_t(N) * row_out), span(out_b, size_t(N) * 4),
                       span(workspace, workspace_bytes)};
  if (any_alias(outs, 3, ins, 5)) return FLP_INVALID_ARGUMENT;
  if (workspace_bytes < align_up(size_t(N))) return FLP_WORKSPACE_TOO_SMALL;
  return FLP_OK;
}

namespace {

flp_status check_embedding_dims(int64_t N, int64_t D, int64_t V, flp_dtype x, flp_dtype id) {
  if (N < 0 || D < 1 || V < 1) return FLP_INVALID_ARGUMENT;
  if (x != FLP_BF16 && x != FLP_F16 && x != FLP_F32) return FLP_UNSUPPORTED_DTYPE;
  if (id != FLP_I64 && id != FLP_I32) return FLP_UNSUPPORTED_DTYPE;
  // rows move in 16-byte chunks; token indices, sort keys (ids and the dropped-id
  // key V) and segment bounds are 32-bit
  if ((D * int64_t(dtype_size(x))) % 16 != 0) return FLP_UNSUPPORTED_SHAPE;
  if (N > kMaxIndexedRows || V > kMaxIndexedRows - 1) return FLP_UNSUPPORTED_SHAPE;
  if (!mul_ok(std::max<int64_t>(N, 1), D) || !mul_ok(V, D) || !mul_ok(V * D, 8))
    return FLP_UNSUPPORTED_SHAPE;
  return FLP_OK;
}

}  // namespace

flp_status validate_embedding_forward(int64_t N, int64_t D, int64_t V, flp_dtype x,
                                      const void* weight, const void* ids, flp_dtype id,
                                      const void* out) {
  flp_status st = check_embedding_dims(N, D, V, x, id);
  if (st != FLP_OK || N == 0) return st;
  if (!weight || !ids || !out) return FLP_INVALID_ARGUMENT;
  if (!aligned(weight, 16) || !aligned(out, 16) || !aligned(ids, dtype_size(id)))
    return FLP_MISALIGNED;
  const size_t xs = dtype_size(x);
  const Span ins[] = {span(weight, size_t(V) * D * xs), span(ids, size_t(N) * dtype_size(id))};
  const Span outs[] = {span(out, size_t(N) * D * xs)};
  if (any_alias(outs, 1, ins, 2)) return FLP_INVALID_ARGUMENT;
  return FLP_OK;
}

flp_status validate_embedding_backward(int64_t N, int64_t D, int64_t V, flp_dtype x,
                                       const void* grad, const void* ids, flp_dtype id,
                                       const void* d_weight, flp_dtype dw, const void* workspace,
                                       size_t workspace_bytes) {
  flp_status st = check_embedding_dims(N, D, V, x, id);
  if (st != FLP_OK) return st;
  if (dw != x && dw != FLP_F32) return FLP_UNSUPPORTED_DTYPE;
  if (!d_weight) return FLP_INVALID_ARGUMENT;
  if (N == 0) return validate_empty_sums(D, V, dtype_size(x), nullptr, nullptr, d_weight, dw, nullptr);
  if (!grad || !ids || !workspace) return FLP_INVALID_ARGUMENT;
  if (!aligned(grad, 16) || !aligned(d_weight, 16) || !aligned(workspace, 16) ||
      !aligned(ids, dtype_size(id)))
    return FLP_MISALIGNED;
  const size_t xs = dtype_size(x);
  const Span ins[] = {span(grad, size_t(N) * D * xs), span(ids, size_t(N) * dtype_size(id))};
  const Span outs[] = {span(d_weight, size_t(V) * D * dtype_size(dw)),
                       span(workspace, workspace_bytes)};
  if (any_alias(outs, 2, ins, 2)) return FLP_INVALID_ARGUMENT;
  if (workspace_bytes < emb_layout(N, D, V).total) return FLP_WORKSPACE_TOO_SMALL;
  return FLP_OK;
}

}  // namespace flp
