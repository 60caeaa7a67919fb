// C ABI entry points (include/flp.h): validate synchronously, then enqueue the
// kernels on the caller's stream.  Fail closed: no fallback path exists.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "flp_launch.h"

namespace {

using namespace flp;

// Per-device cache of "is gfx950": 0 = unknown, 1 = yes, 2 = no.
std::atomic<int> g_arch[64];

}  // namespace

flp_status flp::check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FLP_UNSUPPORTED_DEVICE;
  if (dev < 64) {
    const int c = g_arch[dev].load(std::memory_order_relaxed);
    if (c == 1) return FLP_OK;
    if (c == 2) return FLP_UNSUPPORTED_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FLP_HIP_ERROR;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_arch[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FLP_OK : FLP_UNSUPPORTED_DEVICE;
}

namespace {

inline char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }

// The sums over the rows of an empty batch (or an empty selection) are zero.
flp_status zero_sums(void* d_weight, size_t dw_bytes, float* d_bias, int64_t V, hipStream_t s) {
  if (d_weight == nullptr && d_bias == nullptr) return FLP_OK;
  const flp_status st = check_device();
  if (st != FLP_OK) return st;
  if (d_weight != nullptr && launch_zero(d_weight, dw_bytes, s) != hipSuccess) return FLP_HIP_ERROR;
  if (d_bias != nullptr && launch_zero(d_bias, size_t(V) * 4, s) != hipSuccess) return FLP_HIP_ERROR;
  return FLP_OK;
}

// ---- optional per-kernel event timing ----
struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
std::atomic<bool> g_prof_on{false};
std::vector<ProfRec> g_prof_recs;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace flp {

ProfScope::ProfScope(int k, hipStream_t s) : kind(k), stream(s) {
  if (!g_prof_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  a = prof_event();
  if (a != nullptr && hipEventRecord(a, stream) != hipSuccess) {
    g_prof_pool.push_back(a);
    a = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (a == nullptr) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  hipEvent_t b = prof_event();
  if (b == nullptr || hipEventRecord(b, stream) != hipSuccess) {
    g_prof_pool.push_back(a);
    if (b != nullptr) g_prof_pool.push_back(b);
    return;
  }
  g_prof_recs.push_back(ProfRec{kind, a, b});
}

flp_status enqueue_forward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype, const void* hidden,
                           const void* weight, const float* bias, const void* targets,
                           flp_dtype t_dtype, const float* temperature, float* out_logp,
                           float* out_lse, void* workspace, hipStream_t s) {
  const FwdLayout L = fwd_layout(N, D, V);
  FwdArgs f;
  f.hidden = hidden;
  f.weight = weight;
  f.bias = bias;
  f.targets = targets;
  f.t64 = t_dtype == FLP_I64;
  f.temperature = temperature;
  f.N = N;
  f.D = D;
  f.V = V;
  f.t_off = 0;
  f.part = reinterpret_cast<float2*>(at(workspace, L.part_off));
  f.zt = reinterpret_cast<float*>(at(workspace, L.zt_off));
  if (launch_forward(x_dtype, f, s) != hipSuccess) return FLP_HIP_ERROR;
  MergeArgs m;
  m.part = f.part;
  m.zt = f.zt;
  m.targets = targets;
  m.t64 = f.t64;
  m.N = N;
  m.V = V;
  m.n_vt = L.n_vt;
  m.logp = out_logp;
  m.lse = out_lse;
  if (launch_merge(m, s) != hipSuccess) return FLP_HIP_ERROR;
  return FLP_OK;
}

}  // namespace flp

extern "C" {

size_t flp_forward_workspace_bytes(int64_t N, int64_t D, int64_t V) {
  if (N < 0 || D < 1 || V < 1) return 0;
  return fwd_layout(N, D, V).total;
}

flp_status flp_forward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype, const void* hidden,
                       const void* weight, const float* bias, const void* targets,
                       flp_dtype t_dtype, const float* temperature, float* out_logp,
                       float* out_lse, void* workspace, size_t workspace_bytes, void* stream) {
  flp_status st = validate_forward(N, D, V, x_dtype, hidden, weight, bias, targets, t_dtype,
                                   temperature, out_logp, out_lse, workspace, workspace_bytes);
  if (st != FLP_OK || N == 0) return st;
  if ((st = check_device()) != FLP_OK) return st;
  return enqueue_forward(N, D, V, x_dtype, hidden, weight, bias, targets, t_dtype, temperature,
                         out_logp, out_lse, workspace, static_cast<hipStream_t>(stream));
}

size_t flp_forward_partial_bytes(int64_t N, int64_t V_local) {
  if (N < 0 || V_local < 1) return 0;
  return size_t(ceil_div(V_local, kVocabTile)) * size_t(N) * 8;
}

flp_status flp_forward_partial(int64_t N, int64_t D, int64_t V_local, int64_t vocab_start,
                               int64_t V_total, flp_dtype x_dtype, const void* hidden,
                               const void* weight, const float* bias, const void* targets,
                               flp_dtype t_dtype, const float* temperature, void* partial,
                               float* zt, void* stream) {
  flp_status st = validate_forward_partial(N, D, V_local, vocab_start, V_total, x_dtype, hidden,
                                           weight, bias, targets, t_dtype, temperature, partial, zt);
  if (st != FLP_OK || N == 0) return st;
  if ((st = check_device()) != FLP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Rows whose target lies in another shard keep zt = 0.
  if (launch_fill(zt, N, 0.0f, s) != hipSuccess) return FLP_HIP_ERROR;
  FwdArgs f;
  f.hidden = hidden;
  f.weight = weight;
  f.bias = bias;
  f.targets = targets;
  f.t64 = t_dtype == FLP_I64;
  f.temperature = temperature;
  f.N = N;
  f.D = D;
  f.V = V_local;
  f.t_off = vocab_start;
  f.part = static_cast<float2*>(partial);
  f.zt = zt;
  if (launch_forward(x_dtype, f, s) != hipSuccess) return FLP_HIP_ERROR;
  return FLP_OK;
}

flp_status flp_merge(int64_t N, int64_t V_total, const void* partials, const float* zt,
                     const void* targets, flp_dtype t_dtype, float* out_logp, float* out_lse,
                     void* stream) {
  flp_status st = validate_merge(N, V_total, partials, zt, targets, t_dtype, out_logp, out_lse);
  if (st != FLP_OK || N == 0) return st;
  if ((st = check_device()) != FLP_OK) return st;
  MergeArgs m;
  m.part = static_cast<const float2*>(partials);
  m.zt = zt;
  m.targets = targets;
  m.t64 = t_dtype == FLP_I64;
  m.N = N;
  m.V = V_total;
  m.n_vt = ceil_div(V_total, kVocabTile);
  m.logp = out_logp;
  m.lse = out_lse;
  if (launch_merge(m, static_cast<hipStream_t>(stream)) != hipSuccess) return FLP_HIP_ERROR;
  return FLP_OK;
}

flp_status flp_logits_forward(int64_t N, int64_t V, flp_dtype x_dtype, const void* logits,
                              const void* targets, flp_dtype t_dtype, float* out_logp,
                              float* out_lse, void* stream) {
  flp_status st = validate_logits_forward(N, V, x_dtype, logits, targets, t_dtype, out_logp, out_lse);
  if (st != FLP_OK || N == 0) return st;
  if ((st = check_device()) != FLP_OK) return st;
  LogitsArgs a{};
  a.logits = logits;
  a.targets = targets;
  a.t64 = t_dtype == FLP_I64;
  a.N = N;
  a.V = V;
  a.logp = out_logp;
  a.lse_out = out_lse;
  if (launch_logits_forward(x_dtype, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FLP_HIP_ERROR;
  return FLP_OK;
}

flp_status flp_logits_backward(int64_t N, int64_t V, flp_dtype x_dtype, const float* grad_out,
                               const float* lse, const void* logits, const void* targets,
                               flp_dtype t_dtype, void* d_logits, void* stream) {
  flp_status st = validate_logits_backward(N, V, x_dtype, grad_out, lse, logits, targets, t_dtype,
                                           d_logits);
  if (st != FLP_OK || N == 0) return st;
  if ((st = check_device()) != FLP_OK) return st;
  LogitsArgs a{};
  a.logits = logits;
  a.targets = targets;
  a.t64 = t_dtype == FLP_I64;
  a.N = N;
  a.V = V;
  a.grad_out = grad_out;
  a.lse = lse;
  a.d_logits = d_logits;
  if (launch_logits_backward(x_dtype, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FLP_HIP_ERROR;
  return FLP_OK;
}

size_t flp_backward_workspace_bytes(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                    flp_dtype dw_dtype, int64_t chunk_rows) {
  if (N < 0 || D < 1 || V < 1 || chunk_rows < 0) return 0;
  if (x_dtype != FLP_BF16 && x_dtype != FLP_F16 && x_dtype != FLP_F32) return 0;
  if (N == 0) return 0;
  if (chunk_rows > 0)
    return bwd_layout_for_chunk(N, D, V, x_dtype, dw_dtype, chunk_rows, true, true, true).total;
  // The minimum: 256-row chunks, or one chunk of the whole batch when that is smaller
  // (a single chunk needs no fp32 d_W accumulator, which can outweigh its larger buffers).
  const size_t q = bwd_layout_for_chunk(N, D, V, x_dtype, dw_dtype, kRowQuantum, true, true, true).total;
  const size_t one = bwd_layout_for_chunk(N, D, V, x_dtype, dw_dtype, N, true, true, true).total;
  return q < one ? q : one;
}

int64_t flp_backward_chunk_rows(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                flp_dtype dw_dtype, size_t workspace_bytes, int need_d_hidden,
                                int need_d_weight, int need_d_bias) {
  if (N < 1 || D < 1 || V < 1) return 0;
  if (x_dtype != FLP_BF16 && x_dtype != FLP_F16 && x_dtype != FLP_F32) return 0;
  if (dw_dtype != x_dtype && dw_dtype != FLP_F32) return 0;
  if (!need_d_hidden && !need_d_weight && !need_d_bias) return 0;
  return bwd_layout_for_bytes(N, D, V, x_dtype, dw_dtype, workspace_bytes, need_d_hidden != 0,
                              need_d_weight != 0, need_d_bias != 0)
      .chunk;
}

flp_status flp_backward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                        const float* grad_out, const float* lse, const void* hidden,
                        const void* weight, const float* bias, const void* targets,
                        flp_dtype t_dtype, const float* temperature, void* d_hidden,
                        void* d_weight, flp_dtype dw_dtype, float* d_bias, void* workspace,
                        size_t workspace_bytes, void* stream) {
  flp_status st = validate_backward(N, D, V, x_dtype, grad_out, lse, hidden, weight, bias, targets,
                                    t_dtype, temperature, d_hidden, d_weight, dw_dtype, d_bias,
                                    workspace, workspace_bytes);
  if (st != FLP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (N == 0) return zero_sums(d_weight, size_t(V) * D * dtype_size(dw_dtype), d_bias, V, s);
  if (!d_hidden && !d_weight && !d_bias) return FLP_OK;
  if ((st = check_device()) != FLP_OK) return st;
  const BwdLayout L = bwd_layout_for_bytes(N, D, V, x_dtype, dw_dtype, workspace_bytes,
                                           d_hidden != nullptr, d_weight != nullptr,
                                           d_bias != nullptr);
  const size_t xs = dtype_size(x_dtype);
  const size_t ts = dtype_size(t_dtype);
  void* dz = d_hidden ? at(workspace, L.dz_off) : nullptr;
  void* wT = d_hidden ? at(workspace, L.wt_off) : nullptr;
  void* dzT = d_weight ? at(workspace, L.dzt_off) : nullptr;
  void* hT = d_weight ? at(workspace, L.ht_off) : nullptr;
  float* dbp = d_bias ? reinterpret_cast<float*>(at(workspace, L.dbp_off)) : nullptr;
  float* acc = nullptr;
  if (d_weight) {
    if (dw_dtype == FLP_F32)
      acc = static_cast<float*>(d_weight);
    else if (L.use_acc)
      acc = reinterpret_cast<float*>(at(workspace, L.acc_off));
  }
  for (int64_t c = 0; c < L.n_chunks; ++c) {
    const int64_t r0 = c * L.chunk;
    const int64_t rows = (N - r0 < L.chunk) ? N - r0 : L.chunk;
    const bool last = c + 1 == L.n_chunks;
    const void* h_chunk = static_cast<const char*>(hidden) + size_t(r0) * D * xs;
    DzArgs z;
    z.hidden = h_chunk;
    z.weight = weight;
    z.bias = bias;
    z.targets = static_cast<const char*>(targets) + size_t(r0) * ts;
    z.t64 = t_dtype == FLP_I64;
    z.temperature = temperature ? temperature + r0 : nullptr;
    z.grad_out = grad_out + r0;
    z.lse = lse + r0;
    z.rows = rows;
    z.D = D;
    z.V = V;
    z.ldz = L.ldz;
    z.ldt = L.ldt;
    z.dz = dz;
    z.dzT = dzT;
    z.dbias_part = dbp;
    if (launch_dz(x_dtype, z, s) != hipSuccess) return FLP_HIP_ERROR;
    if (d_hidden) {
      // W^T is made once, after the first dlogits: that kernel re-reads hidden, which
      // the forward left in the Infinity Cache and streaming 1.4 GB of W and W^T
      // through it first would evict.
      if (c == 0 && launch_transpose(x_dtype, weight, V, L.ldz, D, D, wT, s) != hipSuccess)
        return FLP_HIP_ERROR;
      GemmArgs g;
      g.a = dz;
      g.b = wT;
      g.lda_b = 128;
      g.ldb_b = 128;
      g.a_ks = L.ldt * 128;
      g.b_ks = D * 128;
      g.M = rows;
      g.N = D;
      g.K = L.ldz;  // dz and W^T are zero past V
      g.out = static_cast<char*>(d_hidden) + size_t(r0) * D * xs;
      g.ldo = D;
      g.acc = nullptr;
      g.load_acc = 0;
      g.store_acc = 0;
      if (launch_dx(x_dtype, g, s) != hipSuccess) return FLP_HIP_ERROR;
    }
    if (d_weight) {
      const int64_t kpad = round_up(rows, kTokPad);  // dz^T and hidden^T are zero past rows
      if (launch_transpose(x_dtype, h_chunk, rows, kpad, D, D, hT, s) != hipSuccess)
        return FLP_HIP_ERROR;
      GemmArgs g;
      g.a = dzT;
      g.b = hT;
      g.lda_b = 128;
      g.ldb_b = 128;
      g.a_ks = L.ldz * 128;
      g.b_ks = D * 128;
      g.M = V;
      g.N = D;
      g.K = kpad;
      g.out = d_weight;
      g.ldo = D;
      g.acc = acc;
      g.load_acc = (acc != nullptr && c > 0) ? 1 : 0;
      g.store_acc = (acc != nullptr && (dw_dtype == FLP_F32 || !last)) ? 1 : 0;
      if (launch_dw(x_dtype, g, s) != hipSuccess) return FLP_HIP_ERROR;
    }
    if (d_bias) {
      if (launch_dbias_fold(dbp, (rows + kDzRowTile - 1) / kDzRowTile, L.ldz, V, d_bias, c == 0,
                            s) != hipSuccess)
        return FLP_HIP_ERROR;
    }
  }
  return FLP_OK;
}

// ---- indexed (row-subset) variants ----

size_t flp_forward_indexed_workspace_bytes(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                           int64_t n_rows) {
  if (N < 0 || D < 1 || V < 1 || n_rows < 0 || dtype_size(x_dtype) == 0) return 0;
  if (N == 0) return 0;
  const IdxLayout L = idx_layout(N, D, n_rows, x_dtype, false, false);
  return L.dense_off + (L.sel.cap > 0 ? fwd_layout(L.sel.cap, D, V).total : 0);
}

flp_status flp_forward_indexed(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                               const void* hidden, const void* weight, const float* bias,
                               const void* targets, flp_dtype t_dtype, const float* temperature,
                               const void* rows, flp_dtype r_dtype, int64_t n_rows,
                               float* out_logp, float* out_lse, void* workspace,
                               size_t workspace_bytes, void* stream) {
  flp_status st = validate_forward_indexed(N, D, V, x_dtype, hidden, weight, bias, targets, t_dtype,
                                           temperature, rows, r_dtype, n_rows, out_logp, out_lse,
                                           workspace, workspace_bytes);
  if (st != FLP_OK || N == 0) return st;
  if ((st = check_device()) != FLP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const IdxLayout L = idx_layout(N, D, n_rows, x_dtype, false, false);
  const int64_t cap = L.sel.cap;
  auto* mask = reinterpret_cast<uint8_t*>(at(workspace, L.sel.mask_off));
  auto* pos = reinterpret_cast<int32_t*>(at(workspace, L.sel.pos_off));
  auto* sel = reinterpret_cast<int32_t*>(at(workspace, L.sel.sel_off));
  if (launch_select(rows, r_dtype == FLP_I64, n_rows, N, mask, pos, sel, cap, s) != hipSuccess)
    return FLP_HIP_ERROR;
  float* logp_c = reinterpret_cast<float*>(at(workspace, L.logp_off));
  float* lse_c = reinterpret_cast<float*>(at(workspace, L.lse_off));
  if (cap > 0) {
    GatherArgs g{};
    g.sel = sel;
    g.hidden = hidden;
    g.row_bytes = D * int64_t(dtype_size(x_dtype));
    g.targets = targets;
    g.t64 = t_dtype == FLP_I64;
    g.temperature = temperature;
    g.h_c = at(workspace, L.h_off);
    g.t_c = reinterpret_cast<int64_t*>(at(workspace, L.t_off));
    g.temp_c = temperature ? reinterpret_cast<float*>(at(workspace, L.temp_off)) : nullptr;
    if (launch_gather(g, cap, s) != hipSuccess) return FLP_HIP_ERROR;
    st = flp_forward(cap, D, V, x_dtype, g.h_c, weight, bias, g.t_c, FLP_I64, g.temp_c, logp_c,
                     lse_c, at(workspace, L.dense_off), workspace_bytes - L.dense_off, stream);
    if (st != FLP_OK) return st;
  }
  if (launch_scatter_rows(pos, N, logp_c, lse_c, out_logp, out_lse, s) != hipSuccess)
    return FLP_HIP_ERROR;
  return FLP_OK;
}

size_t flp_backward_indexed_workspace_bytes(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                            flp_dtype dw_dtype, int64_t n_rows,
                                            int64_t chunk_rows) {
  if (N < 0 || D < 1 || V < 1 || n_rows < 0 || chunk_rows < 0) return 0;
  if (x_dtype != FLP_BF16 && x_dtype != FLP_F16 && x_dtype != FLP_F32) return 0;
  if (N == 0) return 0;
  const IdxLayout L = idx_layout(N, D, n_rows, x_dtype, true, true);
  if (L.sel.cap == 0) return L.dense_off;
  return L.dense_off + flp_backward_workspace_bytes(L.sel.cap, D, V, x_dtype, dw_dtype, chunk_rows);
}

flp_status flp_backward_indexed(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                const float* grad_out, const float* lse, const void* hidden,
                                const void* weight, const float* bias, const void* targets,
                                flp_dtype t_dtype, const float* temperature, const void* rows,
                                flp_dtype r_dtype, int64_t n_rows, void* d_hidden,
                                void* d_weight, flp_dtype dw_dtype, float* d_bias,
                                void* workspace, size_t workspace_bytes, void* stream) {
  flp_status st = validate_backward_indexed(N, D, V, x_dtype, grad_out, lse, hidden, weight, bias,
                                            targets, t_dtype, temperature, rows, r_dtype, n_rows,
                                            d_hidden, d_weight, dw_dtype, d_bias, workspace,
                                            workspace_bytes);
  if (st != FLP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t dw_bytes = size_t(V) * D * dtype_size(dw_dtype);
  if (N == 0) return zero_sums(d_weight, dw_bytes, d_bias, V, s);
  if (!d_hidden && !d_weight && !d_bias) return FLP_OK;
  if ((st = check_device()) != FLP_OK) return st;
  const IdxLayout L = idx_layout(N, D, n_rows, x_dtype, true, d_hidden != nullptr);
  const int64_t cap = L.sel.cap;
  const size_t row_bytes = size_t(D) * dtype_size(x_dtype);
  auto* mask = reinterpret_cast<uint8_t*>(at(workspace, L.sel.mask_off));
  auto* pos = reinterpret_cast<int32_t*>(at(workspace, L.sel.pos_off));
  auto* sel = reinterpret_cast<int32_t*>(at(workspace, L.sel.sel_off));
  if (launch_select(rows, r_dtype == FLP_I64, n_rows, N, mask, pos, sel, cap, s) != hipSuccess)
    return FLP_HIP_ERROR;
  void* dh_c = d_hidden ? at(workspace, L.dh_off) : nullptr;
  if (cap > 0) {
    GatherArgs g{};
    g.sel = sel;
    g.hidden = hidden;
    g.row_bytes = int64_t(row_bytes);
    g.targets = targets;
    g.t64 = t_dtype == FLP_I64;
    g.temperature = temperature;
    g.grad_out = grad_out;
    g.lse = lse;
    g.h_c = at(workspace, L.h_off);
    g.t_c = reinterpret_cast<int64_t*>(at(workspace, L.t_off));
    g.temp_c = temperature ? reinterpret_cast<float*>(at(workspace, L.temp_off)) : nullptr;
    g.g_c = reinterpret_cast<float*>(at(workspace, L.g_off));
    g.lse_c = reinterpret_cast<float*>(at(workspace, L.lse_in_off));
    if (launch_gather(g, cap, s) != hipSuccess) return FLP_HIP_ERROR;
    st = flp_backward(cap, D, V, x_dtype, g.g_c, g.lse_c, g.h_c, weight, bias, g.t_c, FLP_I64,
                      g.temp_c, dh_c, d_weight, dw_dtype, d_bias, at(workspace, L.dense_off),
                      workspace_bytes - L.dense_off, stream);
    if (st != FLP_OK) return st;
  } else if ((st = zero_sums(d_weight, dw_bytes, d_bias, V, s)) != FLP_OK) {
    return st;  // nothing can be selected
  }
  if (d_hidden && launch_scatter_hidden(pos, N, dh_c, row_bytes, d_hidden, s) != hipSuccess)
    return FLP_HIP_ERROR;
  return FLP_OK;
}

size_t flp_logits_indexed_workspace_bytes(int64_t N) {
  return N > 0 ? align_up(size_t(N)) : 0;
}

flp_status flp_logits_forward_indexed(int64_t N, int64_t V, flp_dtype x_dtype,
                                      const void* logits, const void* targets, flp_dtype t_dtype,
                                      const void* rows, flp_dtype r_dtype, int64_t n_rows,
                                      float* out_logp, float* out_lse, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  flp_status st = validate_logits_indexed(N, V, x_dtype, false, nullptr, nullptr, logits, targets,
                                          t_dtype, rows, r_dtype, n_rows, out_logp, out_lse,
                                          workspace, workspace_bytes);
  if (st != FLP_OK || N == 0) return st;
  if ((st = check_device()) != FLP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* mask = static_cast<uint8_t*>(workspace);
  if (launch_select(rows, r_dtype == FLP_I64, n_rows, N, mask, nullptr, nullptr, 0, s) !=
      hipSuccess)
    return FLP_HIP_ERROR;
  LogitsArgs a{};
  a.logits = logits;
  a.targets = targets;
  a.t64 = t_dtype == FLP_I64;
  a.N = N;
  a.V = V;
  a.logp = out_logp;
  a.lse_out = out_lse;
  a.mask = mask;
  if (launch_logits_forward(x_dtype, a, s) != hipSuccess) return FLP_HIP_ERROR;
  return FLP_OK;
}

flp_status flp_logits_backward_indexed(int64_t N, int64_t V, flp_dtype x_dtype,
                                       const float* grad_out, const float* lse,
                                       const void* logits, const void* targets,
                                       flp_dtype t_dtype, const void* rows, flp_dtype r_dtype,
                                       int64_t n_rows, void* d_logits, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  flp_status st = validate_logits_indexed(N, V, x_dtype, true, grad_out, lse, logits, targets,
                                          t_dtype, rows, r_dtype, n_rows, d_logits, nullptr,
                                          workspace, workspace_bytes);
  if (st != FLP_OK || N == 0) return st;
  if ((st = check_device()) != FLP_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* mask = static_cast<uint8_t*>(workspace);
  if (launch_select(rows, r_dtype == FLP_I64, n_rows, N, mask, nullptr, nullptr, 0, s) !=
      hipSuccess)
    return FLP_HIP_ERROR;
  LogitsArgs a{};
  a.logits = logits;
  a.targets = targets;
  a.t64 = t_dtype == FLP_I64;
  a.N = N;
  a.V = V;
  a.grad_out = grad_out;
  a.lse = lse;
  a.d_logits = d_logits;
  a.mask = mask;
  if (launch_logits_backward(x_dtype, a, s) != hipSuccess) return FLP_HIP_ERROR;
  return FLP_OK;
}

// ---- untied embedding lookup ----

flp_status flp_embedding_forward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                 const void* weight, const void* ids, flp_dtype id_dtype,
                                 void* out, void* stream) {
  flp_status st = validate_embedding_forward(N, D, V, x_dtype, weight, ids, id_dtype, out);
  if (st != FLP_OK || N == 0) return st;
  if ((st = check_device()) != FLP_OK) return st;
  if (launch_embedding_forward(x_dtype, weight, ids, id_dtype == FLP_I64, N, D, V, out,
                               static_cast<hipStream_t>(stream)) != hipSuccess)
    return FLP_HIP_ERROR;
  return FLP_OK;
}

size_t flp_embedding_backward_workspace_bytes(int64_t N, int64_t D, int64_t V) {
  if (N < 0 || D < 1 || V < 1) return 0;
  return emb_layout(N, D, V).total;
}

flp_status flp_embedding_backward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                  const void* grad, const void* ids, flp_dtype id_dtype,
                                  void* d_weight, flp_dtype dw_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  flp_status st = validate_embedding_backward(N, D, V, x_dtype, grad, ids, id_dtype, d_weight,
                                              dw_dtype, workspace, workspace_bytes);
  if (st != FLP_OK) return st;
  if (N == 0)
    return zero_sums(d_weight, size_t(V) * D * dtype_size(dw_dtype), nullptr, V,
                     static_cast<hipStream_t>(stream));
  if ((st = check_device()) != FLP_OK) return st;
  const EmbLayout L = emb_layout(N, D, V);
  EmbedBwdArgs a{};
  a.x = x_dtype;
  a.dw = dw_dtype;
  a.grad = grad;
  a.ids = ids;
  a.i64 = id_dtype == FLP_I64;
  a.N = N;
  a.D = D;
  a.V = V;
  for (int k = 0; k < 2; ++k) {
    a.keys[k] = reinterpret_cast<uint32_t*>(at(workspace, L.keys_off[k]));
    a.vals[k] = reinterpret_cast<int32_t*>(at(workspace, L.vals_off[k]));
  }
  a.hist = reinterpret_cast<int32_t*>(at(workspace, L.hist_off));
  a.seg_begin = reinterpret_cast<int32_t*>(at(workspace, L.seg_begin_off));
  a.seg_end = reinterpret_cast<int32_t*>(at(workspace, L.seg_end_off));
  a.head = reinterpret_cast<float*>(at(workspace, L.head_off));
  a.tail = reinterpret_cast<float*>(at(workspace, L.tail_off));
  a.d_weight = d_weight;
  if (launch_embedding_backward(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return FLP_HIP_ERROR;
  return FLP_OK;
}

// ---- measurement probes ----

size_t flp_probe_scratch_bytes(void) { return probe_scratch_bytes(); }

flp_status flp_probe_mfma(int zero_operands, int64_t iters, void* scratch, size_t scratch_bytes,
                          double* out_tflops, double* out_clock_ghz, void* stream) {
  if (iters < 1 || iters > 1000000 || !scratch || !out_tflops || !out_clock_ghz)
    return FLP_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(scratch) % 16 != 0) return FLP_MISALIGNED;
  if (scratch_bytes < probe_scratch_bytes()) return FLP_WORKSPACE_TOO_SMALL;
  flp_status st = check_device();
  if (st != FLP_OK) return st;
  if (probe_mfma(zero_operands != 0 ? 1 : 0, iters, scratch, static_cast<hipStream_t>(stream),
                 out_tflops, out_clock_ghz) != hipSuccess)
    return FLP_HIP_ERROR;
  return FLP_OK;
}

flp_status flp_probe_read(const void* buffer, size_t bytes, void* scratch, size_t scratch_bytes,
                          double* out_gbs, void* stream) {
  if (!buffer || bytes < 16 || bytes % 16 != 0 || !scratch || !out_gbs) return FLP_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(buffer) % 16 != 0 || reinterpret_cast<uintptr_t>(scratch) % 16 != 0)
    return FLP_MISALIGNED;
  if (scratch_bytes < probe_scratch_bytes()) return FLP_WORKSPACE_TOO_SMALL;
  const uintptr_t b0 = reinterpret_cast<uintptr_t>(buffer), s0 = reinterpret_cast<uintptr_t>(scratch);
  if (b0 < s0 + scratch_bytes && s0 < b0 + bytes) return FLP_INVALID_ARGUMENT;
  flp_status st = check_device();
  if (st != FLP_OK) return st;
  if (probe_read(buffer, bytes, scratch, static_cast<hipStream_t>(stream), out_gbs) != hipSuccess)
    return FLP_HIP_ERROR;
  return FLP_OK;
}

void flp_profile_enable(int on) { g_prof_on.store(on != 0); }

flp_status flp_profile_read(double* ms, int64_t* count, int n) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  const int m = n < FLP_K_COUNT ? n : FLP_K_COUNT;
  for (int k = 0; k < m; ++k) {
    ms[k] = 0.0;
    count[k] = 0;
  }
  flp_status st = FLP_OK;
  for (const ProfRec& r : g_prof_recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      st = FLP_HIP_ERROR;
    else if (r.kind < m) {
      ms[r.kind] += double(t);
      count[r.kind] += 1;
    }
    g_prof_pool.push_back(r.a);
    g_prof_pool.push_back(r.b);
  }
  g_prof_recs.clear();
  return st;
}

const char* flp_status_string(flp_status status) {
  switch (status) {
    case FLP_OK: return "FLP_OK";
    case FLP_INVALID_ARGUMENT: return "FLP_INVALID_ARGUMENT: null pointer, negative size or overlapping buffers";
    case FLP_UNSUPPORTED_DTYPE: return "FLP_UNSUPPORTED_DTYPE";
    case FLP_UNSUPPORTED_SHAPE:
      return "FLP_UNSUPPORTED_SHAPE: D must be a multiple of 32 with 256 * D * element size < 2^31, "
             "and sizes must fit the index range";
    case FLP_MISALIGNED: return "FLP_MISALIGNED";
    case FLP_WORKSPACE_TOO_SMALL: return "FLP_WORKSPACE_TOO_SMALL";
    case FLP_UNSUPPORTED_DEVICE: return "FLP_UNSUPPORTED_DEVICE: needs gfx950 (MI355X)";
    case FLP_HIP_ERROR: return "FLP_HIP_ERROR";
  }
  return "FLP_UNKNOWN_STATUS";
}

const char* flp_build_info(void) {
  static const std::string info = [] {
    char buf[1024];
    std::snprintf(buf, sizeof(buf),
                  "flp 0.2 gfx950 fallback=none vocab_tile=%lld row_quantum=%lld git=%s | %s",
                  (long long)kVocabTile, (long long)kRowQuantum,
#ifdef FLP_GIT_HASH
                  FLP_GIT_HASH,
#else
                  "unknown",
#endif
                  kernel_ids());
    return std::string(buf);
  }();
  return info.c_str();
}

}  // extern "C"
