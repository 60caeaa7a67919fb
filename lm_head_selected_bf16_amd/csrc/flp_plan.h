// Host-side planning shared by the C-ABI layer and the kernels: the numeric
// constants of the reduction topology, workspace layouts and argument
// validation.  Plain C++, no HIP dependency, never dereferences a pointer.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/flp.h"

namespace flp {

// Vocabulary tile width of the forward and dlogits kernels.  It fixes the
// reduction topology of every row (online max / sum-of-exp per 256-column
// tile, then an ascending fold over tiles), so it is a constant of the
// numerics, not a tuning knob.
constexpr int64_t kVocabTile = 256;
// Row granularity of backward chunks (multiple of every row tile and K step).
constexpr int64_t kRowQuantum = 256;
// Row tile of the dlogits kernel: one d_bias partial row per tile.
constexpr int64_t kDzRowTile = 256;
// K of the d_weight GEMM (tokens) is padded with zeros to a multiple of this.
constexpr int64_t kTokPad = 64;
// Output tiles of the backward GEMMs: 256 x 224 for 16-bit inputs, 128 x 128 for fp32.
constexpr int64_t kGemmTileM16 = 256, kGemmTileN16 = 224, kGemmTile32 = 128;
// Compute units of the targeted device (MI355X).  A backward that needs several
// row chunks prefers chunks whose d_hidden GEMM fills whole waves of workgroups:
// every d_hidden tile runs over all of K = V, so a nearly empty last wave costs
// a full tile time.
constexpr int64_t kNumCUs = 256;
constexpr size_t kAlign = 256;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
inline size_t align_up(size_t a) { return (a + kAlign - 1) / kAlign * kAlign; }

inline size_t dtype_size(flp_dtype t) {
  switch (t) {
    case FLP_BF16: return 2;
    case FLP_F16: return 2;
    case FLP_F32: return 4;
    case FLP_I64: return 8;
    case FLP_I32: return 4;
  }
  return 0;
}

// ---- forward workspace: [n_vt][N] (max, sum) pairs, then [N] target logits ----
struct FwdLayout {
  int64_t n_vt = 0;
  size_t part_off = 0, zt_off = 0, total = 0;
};
FwdLayout fwd_layout(int64_t N, int64_t D, int64_t V);

// ---- backward workspace: dz chunk, d_bias partials, fp32 d_weight accumulator ----
struct BwdLayout {
  int64_t chunk = 0;      // rows per chunk (multiple of kRowQuantum)
  int64_t n_chunks = 0;
  int64_t ldz = 0;        // row stride of dz in elements (V rounded up to kVocabTile)
  int64_t ldt = 0;        // row stride of dz^T and hidden^T in elements (= chunk)
  size_t dz_off = 0, wt_off = 0, dzt_off = 0, ht_off = 0, dbp_off = 0, acc_off = 0, total = 0;
  bool use_acc = false;   // fp32 d_weight accumulator in the workspace
};
// Size for a given chunk; need_* say which outputs are requested.
BwdLayout bwd_layout_for_chunk(int64_t N, int64_t D, int64_t V, flp_dtype x, flp_dtype dw,
                               int64_t chunk, bool need_dh, bool need_dw, bool need_db);
// Largest chunk that fits `bytes` (chunk = 0 in the result when nothing fits).
BwdLayout bwd_layout_for_bytes(int64_t N, int64_t D, int64_t V, flp_dtype x, flp_dtype dw,
                               size_t bytes, bool need_dh, bool need_dw, bool need_db);

// ---- indexed variants: row selection and the gathered copy of the selected rows ----
// Largest N the indexed variants take (compact positions are int32).
constexpr int64_t kMaxIndexedRows = (int64_t(1) << 31) - 1;
// Selection: [N] byte mask, [N] int32 compact positions, [cap] int32 selected row
// ids in ascending order (-1 past the count), with cap = min(n_rows, N).
struct SelLayout {
  int64_t cap = 0;
  size_t mask_off = 0, pos_off = 0, sel_off = 0, total = 0;
};
SelLayout sel_layout(int64_t N, int64_t n_rows);
// Linear variants: the selection, then the gathered rows (hidden [cap][D] x,
// targets [cap] int64, temperature [cap], grad_out [cap], lse [cap]), the
// compact outputs (logp, lse, d_hidden [cap][D]), then the dense workspace.
struct IdxLayout {
  SelLayout sel;
  size_t h_off = 0, t_off = 0, temp_off = 0, g_off = 0, lse_in_off = 0;
  size_t logp_off = 0, lse_off = 0, dh_off = 0, dense_off = 0;
};
IdxLayout idx_layout(int64_t N, int64_t D, int64_t n_rows, flp_dtype x, bool backward,
                     bool need_dh);

// ---- embedding backward: radix-sort buffers and the per-id segments ----
constexpr int64_t kEmbSortBlock = 256;  // keys per block of a radix pass
constexpr int64_t kEmbSegGroup = 32;    // sorted positions per group of the segment sums
struct EmbLayout {
  int64_t n_blocks = 0;   // radix-sort blocks of kEmbSortBlock keys
  size_t keys_off[2] = {0, 0}, vals_off[2] = {0, 0};
  size_t hist_off = 0, seg_begin_off = 0, seg_end_off = 0;
  size_t head_off = 0, tail_off = 0, total = 0;  // fp32 [ceil(N / kEmbSegGroup)][D] each
};
EmbLayout emb_layout(int64_t N, int64_t D, int64_t V);

// ---- validation (pure host logic; never dereferences a pointer) ----
flp_status validate_forward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                            const void* hidden, const void* weight, const float* bias,
                            const void* targets, flp_dtype t_dtype, const float* temperature,
                            const float* out_logp, const float* out_lse,
                            const void* workspace, size_t workspace_bytes);
// The allocation-free forward: the forward's gates on everything the caller passes,
// and its workspace size against the library's fixed scratch array.
flp_status validate_forward_noalloc(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                    const void* hidden, const void* weight, const float* bias,
                                    const void* targets, flp_dtype t_dtype,
                                    const float* temperature, const float* out_logp,
                                    const float* out_lse, size_t scratch_bytes);
// Vocabulary-shard forward and the merge of the shards' partials.
flp_status validate_forward_partial(int64_t N, int64_t D, int64_t V_local, int64_t vocab_start,
                                    int64_t V_total, flp_dtype x_dtype, const void* hidden,
                                    const void* weight, const float* bias, const void* targets,
                                    flp_dtype t_dtype, const float* temperature,
                                    const void* partial, const float* zt);
flp_status validate_merge(int64_t N, int64_t V_total, const void* partials, const float* zt,
                          const void* targets, flp_dtype t_dtype, const float* out_logp,
                          const float* out_lse);
// The operator on materialised logits.
flp_status validate_logits_forward(int64_t N, int64_t V, flp_dtype x_dtype, const void* logits,
                                   const void* targets, flp_dtype t_dtype, const float* out_logp,
                                   const float* out_lse);
flp_status validate_logits_backward(int64_t N, int64_t V, flp_dtype x_dtype, const float* grad_out,
                                    const float* lse, const void* logits, const void* targets,
                                    flp_dtype t_dtype, const void* d_logits);
// The row list of an indexed call (shared by every indexed variant).
flp_status validate_rows(int64_t N, const void* rows, flp_dtype r_dtype, int64_t n_rows);
flp_status validate_backward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                             const float* grad_out, const float* lse,
                             const void* hidden, const void* weight, const float* bias,
                             const void* targets, flp_dtype t_dtype, const float* temperature,
                             const void* d_hidden, const void* d_weight, flp_dtype dw_dtype,
                             const float* d_bias, const void* workspace, size_t workspace_bytes);

// Indexed variants: the dense gates plus the row list and the indexed workspace.
flp_status validate_forward_indexed(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                    const void* hidden, const void* weight, const float* bias,
                                    const void* targets, flp_dtype t_dtype,
                                    const float* temperature, const void* rows,
                                    flp_dtype r_dtype, int64_t n_rows, const float* out_logp,
                                    const float* out_lse, const void* workspace,
                                    size_t workspace_bytes);
flp_status validate_backward_indexed(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                     const float* grad_out, const float* lse,
                                     const void* hidden, const void* weight, const float* bias,
                                     const void* targets, flp_dtype t_dtype,
                                     const float* temperature, const void* rows,
                                     flp_dtype r_dtype, int64_t n_rows, const void* d_hidden,
                                     const void* d_weight, flp_dtype dw_dtype,
                                     const float* d_bias, const void* workspace,
                                     size_t workspace_bytes);
// Forward (backward = false): out_a = logp [N], out_b = lse [N] or NULL.
// Backward: out_a = d_logits [N, V], out_b = NULL.
flp_status validate_logits_indexed(int64_t N, int64_t V, flp_dtype x_dtype, bool backward,
                                   const float* grad_out, const float* lse, const void* logits,
                                   const void* targets, flp_dtype t_dtype, const void* rows,
                                   flp_dtype r_dtype, int64_t n_rows, const void* out_a,
                                   const void* out_b, const void* workspace,
                                   size_t workspace_bytes);

// Untied embedding lookup (forward) and its grad_weight (backward).
flp_status validate_embedding_forward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                      const void* weight, const void* ids, flp_dtype id_dtype,
                                      const void* out);
flp_status validate_embedding_backward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                       const void* grad, const void* ids, flp_dtype id_dtype,
                                       const void* d_weight, flp_dtype dw_dtype,
                                       const void* workspace, size_t workspace_bytes);

}  // namespace flp
