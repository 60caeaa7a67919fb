// Kernel argument blocks and launchers (implemented in flp_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "flp_plan.h"

namespace flp {

// The current device is a gfx950 (cached per device): FLP_OK, else
// FLP_UNSUPPORTED_DEVICE (or FLP_HIP_ERROR when the device cannot be queried).
flp_status check_device();
// Enqueue the forward (logit tiles, then the ascending merge) on `s` with its
// workspace at `workspace`, laid out as fwd_layout(N, D, V).  The arguments
// have been validated.
flp_status enqueue_forward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype, const void* hidden,
                           const void* weight, const float* bias, const void* targets,
                           flp_dtype t_dtype, const float* temperature, float* out_logp,
                           float* out_lse, void* workspace, hipStream_t s);

struct FwdArgs {
  const void* hidden;
  const void* weight;
  const float* bias;
  const void* targets;
  int t64;
  const float* temperature;
  int64_t N, D, V;
  int64_t t_off;    // vocabulary id of weight row 0 (0 unless a shard)
  float2* part;     // [n_vt][N]
  float* zt;        // [N]
};
struct MergeArgs {
  const float2* part;
  const float* zt;
  const void* targets;
  int t64;
  int64_t N, V, n_vt;
  float* logp;
  float* lse;       // may be null
};
struct DzArgs {
  const void* hidden;   // chunk start
  const void* weight;
  const float* bias;
  const void* targets;  // chunk start
  int t64;
  const float* temperature;  // chunk start or null
  const float* grad_out;     // chunk start
  const float* lse;          // chunk start
  int64_t rows, D, V, ldz, ldt;  // ldz: vocabulary padded; ldt: rows allocated in the chunk
  void* dz;                  // [ldt rows][ldz] K-blocked, or null when d_hidden is not needed
  void* dzT;                 // [ldz rows][ldt] K-blocked, or null when d_weight is not needed
  float* dbias_part;         // [rows_alloc / kDzRowTile][ldz] or null
};
struct LogitsArgs {
  const void* logits;        // [N][V]
  const void* targets;
  int t64;
  int64_t N, V;
  const float* grad_out;     // backward only
  const float* lse;          // backward only
  float* logp;               // forward only
  float* lse_out;            // forward only, may be null
  void* d_logits;            // backward only
  const uint8_t* mask;       // [N] selected rows (indexed variants) or null for all rows
};
struct GatherArgs {
  const int32_t* sel;        // [cap] selected row ids, -1 for padding entries
  const void* hidden;        // [N][D]
  int64_t row_bytes;         // D * element size (a multiple of 16)
  const void* targets;
  int t64;
  const float* temperature;  // may be null
  const float* grad_out;     // may be null
  const float* lse;          // may be null
  void* h_c;                 // [cap][D]
  int64_t* t_c;              // [cap]
  float* temp_c;             // [cap] or null
  float* g_c;                // [cap] or null
  float* lse_c;              // [cap] or null
};
struct GemmArgs {
  const void* a;   // M-side operand
  const void* b;   // N-side operand
  int64_t lda_b, ldb_b;  // row strides in bytes (128 in the K-blocked layout)
  int64_t a_ks, b_ks;    // bytes from one 128-byte K stage to the next (rows x 128)
  int64_t M, N, K;
  void* out;             // output (x dtype or fp32)
  int64_t ldo;           // elements
  float* acc;            // fp32 accumulator [M][N] (dW) or null
  int load_acc;          // continue from acc
  int store_acc;         // store fp32 to acc (else store to out in x dtype)
};

hipError_t launch_forward(flp_dtype x, const FwdArgs& a, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, hipStream_t s);
hipError_t launch_fill(float* dst, int64_t n, float value, hipStream_t s);
hipError_t launch_logits_forward(flp_dtype x, const LogitsArgs& a, hipStream_t s);
hipError_t launch_logits_backward(flp_dtype x, const LogitsArgs& a, hipStream_t s);
hipError_t launch_dz(flp_dtype x, const DzArgs& a, hipStream_t s);
hipError_t launch_dx(flp_dtype x, const GemmArgs& a, hipStream_t s);
hipError_t launch_dw(flp_dtype x, const GemmArgs& a, hipStream_t s);
// dst = src^T for src [rows][cols] (row stride ld_src elements), written K-blocked
// with cols rows and K = rows_pad; K entries in [rows, rows_pad) are zero-filled.
hipError_t launch_transpose(flp_dtype x, const void* src, int64_t rows, int64_t rows_pad, int64_t cols,
                            int64_t ld_src, void* dst, hipStream_t s);
hipError_t launch_dbias_fold(const float* part, int64_t n_parts, int64_t ldz, int64_t V,
                             float* d_bias, int init, hipStream_t s);
const char* kernel_ids();

// Row selection for the indexed variants (flp_rows.hip).  launch_zero clears
// bytes / 4 words.  launch_select builds the mask; with pos != null it also
// compacts it into pos / sel.
hipError_t launch_zero(void* dst, size_t bytes, hipStream_t s);
hipError_t launch_select(const void* rows, bool r64, int64_t n_rows, int64_t N, uint8_t* mask,
                         int32_t* pos, int32_t* sel, int64_t cap, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, int64_t cap, hipStream_t s);
hipError_t launch_scatter_rows(const int32_t* pos, int64_t N, const float* logp_c,
                               const float* lse_c, float* logp, float* lse, hipStream_t s);
hipError_t launch_scatter_hidden(const int32_t* pos, int64_t N, const void* dh_c, size_t row_bytes,
                                 void* dh, hipStream_t s);

// Untied embedding lookup and its sorted-segment grad_weight (flp_embed.hip).
struct EmbedBwdArgs {
  flp_dtype x;               // dtype of grad (and of the embedding)
  flp_dtype dw;              // x or FLP_F32
  const void* grad;          // [N][D]
  const void* ids;           // [N]
  bool i64;
  int64_t N, D, V;
  uint32_t* keys[2];         // [N] radix-sort ping-pong buffers
  int32_t* vals[2];          // [N]
  int32_t* hist;             // [256][ceil(N / kEmbSortBlock)]
  int32_t* seg_begin;        // [V]
  int32_t* seg_end;          // [V]
  float* head;               // [ceil(N / kEmbSegGroup)][D] fp32 pieces of segments that span groups
  float* tail;               // same shape
  void* d_weight;            // [V][D] dw
};
int embed_sort_passes(int64_t V);
hipError_t launch_embedding_forward(flp_dtype x, const void* weight, const void* ids, bool i64,
                                    int64_t N, int64_t D, int64_t V, void* out, hipStream_t s);
hipError_t launch_embedding_backward(const EmbedBwdArgs& a, hipStream_t s);

// Measurement probes (flp_probe.hip); they synchronise the stream.
size_t probe_scratch_bytes();
hipError_t probe_mfma(int zero, int64_t iters, void* scratch, hipStream_t s, double* tflops,
                      double* clock_ghz);
hipError_t probe_read(const void* buf, size_t bytes, void* scratch, hipStream_t s, double* gbs);

// Event brackets around each launch while profiling is enabled (flp_api.cpp).
struct ProfScope {
  ProfScope(int kind, hipStream_t s);
  ~ProfScope();
  int kind;
  hipStream_t stream;
  hipEvent_t a = nullptr;
};

}  // namespace flp
