// C ABI of the FMHA forward library (declared in include/fmha.h).
//
// Host-side argument validation happens before any HIP call, so the checks
// run (and are tested) on machines without a GPU. The library allocates
// nothing; launches go to the caller's stream. Its one piece of state is the
// fixed device array below that fmha_bwd_noalloc uses as its workspace, and
// that array's address on each device.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "fmha.h"
#include "fmha_bwd_params.h"
#include "fmha_kernel_params.h"

static_assert(FMHA_TRACE_EVENTS_PER_WAVE == fmha::kTraceEvents, "trace record count");
static_assert(FMHA_TRACE_EV_SLOT == fmha::kEvSlot && FMHA_TRACE_EV_QK_DONE == fmha::kEvQkDone &&
                  FMHA_TRACE_EV_MFMA_DONE == fmha::kEvMfmaDone &&
                  FMHA_TRACE_EV_COPY_ISSUED == fmha::kEvCopyIssued &&
                  FMHA_TRACE_EV_VALU_DONE == fmha::kEvValuDone &&
                  FMHA_TRACE_EV_WAIT_DONE == fmha::kEvWaitDone && FMHA_TRACE_EV_ITEM == fmha::kEvItem,
              "trace event codes");

// Workspace of fmha_bwd_noalloc: a file-scope device array, one copy per GPU,
// held until the process ends. Host code never passes its name to a kernel (on
// the host the name is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[FMHA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Device addresses of `scratch`, one per device, looked up on the first
// fmha_bwd_noalloc call on that device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

hipError_t scratch_address(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return hipSuccess;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by the bf16, fp8 and fp4 P.V entry points. Returns FMHA_OK when the
// arguments describe a launchable problem.
fmha_status_t check_common(const void* q, const void* k, const void* v,
                           const int32_t* cu_q, const int32_t* cu_k, int32_t batch,
                           int32_t total_q, int32_t total_k, int32_t max_q, int32_t max_k,
                           int32_t heads, int32_t head_dim, int32_t causal, float scale,
                           const void* out, const float* lse) {
  if (batch < 0 || total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0) return FMHA_ERR_INVALID_ARG;
  if (heads <= 0) return FMHA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FMHA_ERR_INVALID_ARG;
  if (!(scale > 0.f) || !isfinite(scale)) return FMHA_ERR_INVALID_ARG;
  if ((cu_q == nullptr) != (cu_k == nullptr)) return FMHA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return FMHA_ERR_UNSUPPORTED;
  if (cu_q == nullptr) {
    // dense [batch, seqlen, heads, d]
    if ((int64_t)batch * max_q != total_q || (int64_t)batch * max_k != total_k) return FMHA_ERR_INVALID_ARG;
  }
  // element offsets are computed in 32-bit inside the kernels' inner loops, and
  // a tile copy's per-lane byte offset reaches up to 63 rows past a document's
  // end (those rows read as zeros only while that offset does not wrap)
  const int64_t row = (int64_t)heads * head_dim;
  if (row * ((int64_t)total_q + 64) > INT32_MAX || row * ((int64_t)total_k + 64) > INT32_MAX ||
      (int64_t)heads * total_q > INT32_MAX || batch > 65535 || heads > 65535 ||
      ((int64_t)max_q + 127) / 128 * heads * batch > INT32_MAX)
    return FMHA_ERR_UNSUPPORTED;
  if (total_q > 0 && (q == nullptr || out == nullptr)) return FMHA_ERR_INVALID_ARG;
  if (total_k > 0 && (k == nullptr || v == nullptr)) return FMHA_ERR_INVALID_ARG;
  if ((q && !aligned16(q)) || (k && !aligned16(k)) || (v && !aligned16(v)) ||
      (out && !aligned16(out)) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return FMHA_ERR_INVALID_ARG;
  return FMHA_OK;
}

fmha::FwdParams make_params(const void* q, const void* k, const void* v, const int32_t* cu_q,
                            const int32_t* cu_k, int32_t batch, int32_t total_q,
                            int32_t total_k, int32_t max_q, int32_t max_k, int32_t heads,
                            float scale, void* out, float* lse) {
  fmha::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.cu_q = cu_q;
  p.cu_k = cu_k;
  p.v_scale = nullptr;
  p.num_splits = 1;
  p.out = out;
  p.lse = lse;
  p.batch = batch;
  p.total_q = total_q;
  p.total_k = total_k;
  p.max_seqlen_q = max_q;
  p.max_seqlen_k = max_k;
  p.heads = heads;
  p.scale_log2 = scale * kLog2e;
  return p;
}

}  // namespace

extern "C" {

fmha_status_t fmha_fwd_variant(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t total_q, int32_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t num_heads, int32_t head_dim,
                               int32_t causal, float softmax_scale,
                               void* out, float* lse, int32_t variant, void* stream) {
  fmha_status_t st = check_common(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                                  max_seqlen_q, max_seqlen_k, num_heads, head_dim, causal,
                                  softmax_scale, out, lse);
  if (st != FMHA_OK) return st;
  if (variant < FMHA_VARIANT_AUTO || variant > FMHA_VARIANT_WIDE) return FMHA_ERR_INVALID_ARG;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return FMHA_OK;
  fmha::FwdParams p = make_params(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                                  max_seqlen_q, max_seqlen_k, num_heads, softmax_scale, out, lse);
  hipError_t e = fmha::launch_fwd_bf16(p, head_dim, causal != 0, variant, (hipStream_t)stream);
  return e == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH;
}

fmha_status_t fmha_fwd(const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int32_t batch, int32_t total_q, int32_t total_k,
                       int32_t max_seqlen_q, int32_t max_seqlen_k,
                       int32_t num_heads, int32_t head_dim,
                       int32_t causal, float softmax_scale,
                       void* out, float* lse, void* stream) {
  return fmha_fwd_variant(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                          max_seqlen_q, max_seqlen_k, num_heads, head_dim, causal, softmax_scale,
                          out, lse, FMHA_VARIANT_AUTO, stream);
}

fmha_status_t fmha_fwd_fp8pv_variant(const void* q, const void* k, const uint8_t* v_e4m3,
                                     const float* v_scale,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     int32_t batch, int32_t total_q, int32_t total_k,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     int32_t num_heads, int32_t head_dim,
                                     int32_t causal, float softmax_scale,
                                     void* out, float* lse, int32_t variant, void* stream) {
  fmha_status_t st = check_common(q, k, v_e4m3, cu_seqlens_q, cu_seqlens_k, batch, total_q,
                                  total_k, max_seqlen_q, max_seqlen_k, num_heads, head_dim,
                                  causal, softmax_scale, out, lse);
  if (st != FMHA_OK) return st;
  if (head_dim != 128) return FMHA_ERR_UNSUPPORTED;
  if (variant < FMHA_VARIANT_AUTO || variant > FMHA_VARIANT_WIDE) return FMHA_ERR_INVALID_ARG;
  if (variant == FMHA_VARIANT_PIPELINED || variant == FMHA_VARIANT_WIDE) return FMHA_ERR_UNSUPPORTED;
  if (total_k > 0 && v_scale == nullptr) return FMHA_ERR_INVALID_ARG;
  if (v_scale && (reinterpret_cast<uintptr_t>(v_scale) & 3u)) return FMHA_ERR_INVALID_ARG;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return FMHA_OK;
  fmha::FwdParams p = make_params(q, k, v_e4m3, cu_seqlens_q, cu_seqlens_k, batch, total_q,
                                  total_k, max_seqlen_q, max_seqlen_k, num_heads, softmax_scale,
                                  out, lse);
  p.v_scale = v_scale;
  hipError_t e = fmha::launch_fwd_fp8pv(p, head_dim, causal != 0, variant, (hipStream_t)stream);
  return e == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH;
}

fmha_status_t fmha_fwd_fp8pv(const void* q, const void* k, const uint8_t* v_e4m3,
                             const float* v_scale,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t batch, int32_t total_q, int32_t total_k,
                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int32_t num_heads, int32_t head_dim,
                             int32_t causal, float softmax_scale,
                             void* out, float* lse, void* stream) {
  return fmha_fwd_fp8pv_variant(q, k, v_e4m3, v_scale, cu_seqlens_q, cu_seqlens_k, batch,
                                total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads,
                                head_dim, causal, softmax_scale, out, lse, FMHA_VARIANT_AUTO,
                                stream);
}

fmha_status_t fmha_fwd_fp4pv_variant(const void* q, const void* k, const uint8_t* v_e2m1,
                                     const uint8_t* v_mx_scale,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     int32_t batch, int32_t total_q, int32_t total_k,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     int32_t num_heads, int32_t head_dim,
                                     int32_t causal, float softmax_scale,
                                     void* out, float* lse, int32_t variant, void* stream) {
  fmha_status_t st = check_common(q, k, v_e2m1, cu_seqlens_q, cu_seqlens_k, batch, total_q,
                                  total_k, max_seqlen_q, max_seqlen_k, num_heads, head_dim,
                                  causal, softmax_scale, out, lse);
  if (st != FMHA_OK) return st;
  if (head_dim != 128) return FMHA_ERR_UNSUPPORTED;
  if (variant < FMHA_VARIANT_AUTO || variant > FMHA_VARIANT_WIDE) return FMHA_ERR_INVALID_ARG;
  if (variant == FMHA_VARIANT_PIPELINED || variant == FMHA_VARIANT_WIDE) return FMHA_ERR_UNSUPPORTED;
  if (total_k > 0 && v_mx_scale == nullptr) return FMHA_ERR_INVALID_ARG;
  if (v_mx_scale && (reinterpret_cast<uintptr_t>(v_mx_scale) & 3u)) return FMHA_ERR_INVALID_ARG;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return FMHA_OK;
  fmha::FwdParams p = make_params(q, k, v_e2m1, cu_seqlens_q, cu_seqlens_k, batch, total_q,
                                  total_k, max_seqlen_q, max_seqlen_k, num_heads, softmax_scale,
                                  out, lse);
  p.v_mx_scale = v_mx_scale;
  hipError_t e = fmha::launch_fwd_fp4pv(p, head_dim, causal != 0, variant, (hipStream_t)stream);
  return e == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH;
}

fmha_status_t fmha_fwd_fp4pv(const void* q, const void* k, const uint8_t* v_e2m1,
                             const uint8_t* v_mx_scale,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t batch, int32_t total_q, int32_t total_k,
                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int32_t num_heads, int32_t head_dim,
                             int32_t causal, float softmax_scale,
                             void* out, float* lse, void* stream) {
  return fmha_fwd_fp4pv_variant(q, k, v_e2m1, v_mx_scale, cu_seqlens_q, cu_seqlens_k, batch,
                                total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads,
                                head_dim, causal, softmax_scale, out, lse, FMHA_VARIANT_AUTO,
                                stream);
}

size_t fmha_fwd_splitkv_workspace_size(int32_t total_q, int32_t num_heads, int32_t head_dim,
                                       int32_t num_splits) {
  if (total_q < 0 || num_heads <= 0 || (head_dim != 64 && head_dim != 128) || num_splits < 1 ||
      num_splits > fmha::kMaxSplits)
    return 0;
  if (num_splits == 1) return 0;   // runs the unsplit pass, which needs no workspace
  return (size_t)num_splits * (size_t)total_q * (size_t)num_heads * (size_t)(head_dim + 1) *
         sizeof(float);
}

int32_t fmha_fwd_splitkv_num_splits(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_heads, int32_t causal, int32_t variant) {
  if (batch < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_heads < 0) return -1;
  if (variant < FMHA_VARIANT_AUTO || variant > FMHA_VARIANT_PINGPONG) return -1;
  return fmha::recommended_splits(batch, max_seqlen_q, max_seqlen_k, num_heads, causal != 0,
                                  variant);
}

fmha_status_t fmha_fwd_splitkv(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t total_q, int32_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t num_heads, int32_t head_dim,
                               int32_t causal, float softmax_scale,
                               void* out, float* lse, int32_t num_splits,
                               void* workspace, size_t workspace_bytes,
                               int32_t variant, void* stream) {
  fmha_status_t st = check_common(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                                  max_seqlen_q, max_seqlen_k, num_heads, head_dim, causal,
                                  softmax_scale, out, lse);
  if (st != FMHA_OK) return st;
  if (variant < FMHA_VARIANT_AUTO || variant > FMHA_VARIANT_WIDE) return FMHA_ERR_INVALID_ARG;
  if (variant == FMHA_VARIANT_PIPELINED || variant == FMHA_VARIANT_WIDE) return FMHA_ERR_UNSUPPORTED;
  if (num_splits < 1 || num_splits > fmha::kMaxSplits) return FMHA_ERR_INVALID_ARG;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return FMHA_OK;
  fmha::FwdParams p = make_params(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                                  max_seqlen_q, max_seqlen_k, num_heads, softmax_scale, out, lse);
  if (num_splits == 1) {
    const hipError_t e = fmha::launch_fwd_bf16(p, head_dim, causal != 0, variant,
                                               (hipStream_t)stream);
    return e == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH;
  }
  const size_t need = fmha_fwd_splitkv_workspace_size(total_q, num_heads, head_dim, num_splits);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)
    return FMHA_ERR_INVALID_ARG;
  p.num_splits = num_splits;
  p.o_part = static_cast<float*>(workspace);
  p.lse_part = p.o_part + (size_t)num_splits * total_q * num_heads * head_dim;
  hipError_t e = fmha::launch_fwd_bf16_splitkv(p, head_dim, causal != 0, variant,
                                               (hipStream_t)stream);
  if (e != hipSuccess) return FMHA_ERR_LAUNCH;
  e = fmha::launch_merge_partials(p.o_part, p.lse_part, num_splits, total_q, num_heads, head_dim,
                                  out, lse, (hipStream_t)stream);
  return e == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH;
}

size_t fmha_bwd_workspace_size(int32_t total_q, int32_t num_heads) {
  if (total_q < 0 || num_heads <= 0) return 0;
  return 2 * (size_t)total_q * (size_t)num_heads * sizeof(float);
}

}  // extern "C"

namespace {

// Checks of the backward's arguments other than its workspace.
fmha_status_t check_bwd(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, const int32_t* cu_q,
                        const int32_t* cu_k, int32_t batch, int32_t total_q, int32_t total_k,
                        int32_t max_q, int32_t max_k, int32_t heads, int32_t head_dim,
                        int32_t causal, float scale, const void* dq, const void* dk,
                        const void* dv) {
  fmha_status_t st = check_common(q, k, v, cu_q, cu_k, batch, total_q, total_k, max_q, max_k,
                                  heads, head_dim, causal, scale, out, lse);
  if (st != FMHA_OK) return st;
  if (total_q > 0 && (dout == nullptr || lse == nullptr || dq == nullptr))
    return FMHA_ERR_INVALID_ARG;
  if (total_k > 0 && (dk == nullptr || dv == nullptr)) return FMHA_ERR_INVALID_ARG;
  if ((dout && !aligned16(dout)) || (dq && !aligned16(dq)) || (dk && !aligned16(dk)) ||
      (dv && !aligned16(dv)))
    return FMHA_ERR_INVALID_ARG;
  if (((int64_t)max_k + 127) / 128 * heads * batch > INT32_MAX) return FMHA_ERR_UNSUPPORTED;
  return FMHA_OK;
}

// The two backward launches, with the workspace at `workspace` (checked).
fmha_status_t launch_backward(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, const int32_t* cu_q,
                              const int32_t* cu_k, int32_t batch, int32_t total_q,
                              int32_t total_k, int32_t max_q, int32_t max_k, int32_t heads,
                              int32_t head_dim, int32_t causal, float scale, void* dq, void* dk,
                              void* dv, void* workspace, hipStream_t stream) {
  fmha::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.dout = dout;
  p.lse = lse;
  p.cu_q = cu_q;
  p.cu_k = cu_k;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = static_cast<float*>(workspace);
  p.lse2 = p.delta + (size_t)total_q * heads;
  p.batch = batch;
  p.total_q = total_q;
  p.total_k = total_k;
  p.max_seqlen_q = max_q;
  p.max_seqlen_k = max_k;
  p.heads = heads;
  p.scale = scale;
  p.scale_log2 = scale * kLog2e;
  const hipError_t e = fmha::launch_bwd(p, head_dim, causal != 0, stream);
  return e == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

fmha_status_t fmha_bwd(const void* q, const void* k, const void* v, const void* out,
                       const void* dout, const float* lse,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int32_t batch, int32_t total_q, int32_t total_k,
                       int32_t max_seqlen_q, int32_t max_seqlen_k,
                       int32_t num_heads, int32_t head_dim,
                       int32_t causal, float softmax_scale,
                       void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, void* stream) {
  fmha_status_t st = check_bwd(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, batch,
                               total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads, head_dim,
                               causal, softmax_scale, dq, dk, dv);
  if (st != FMHA_OK) return st;
  const size_t need = fmha_bwd_workspace_size(total_q, num_heads);
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need))
    return FMHA_ERR_INVALID_ARG;
  if (batch == 0 || (total_q == 0 && total_k == 0)) return FMHA_OK;
  return launch_backward(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, batch, total_q,
                         total_k, max_seqlen_q, max_seqlen_k, num_heads, head_dim, causal,
                         softmax_scale, dq, dk, dv, workspace, (hipStream_t)stream);
}

fmha_status_t fmha_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t total_q, int32_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t num_heads, int32_t head_dim,
                               int32_t causal, float softmax_scale,
                               void* dq, void* dk, void* dv, void* stream) {
  fmha_status_t st = check_bwd(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, batch,
                               total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads, head_dim,
                               causal, softmax_scale, dq, dk, dv);
  if (st != FMHA_OK) return st;
  if (fmha_bwd_workspace_size(total_q, num_heads) > (size_t)FMHA_NOALLOC_SCRATCH_BYTES)
    return FMHA_ERR_UNSUPPORTED;
  if (batch == 0 || (total_q == 0 && total_k == 0)) return FMHA_OK;
  // D and LSE * log2(e) go to this device's copy of the fixed array. Every row
  // they are read at is written first by the same call's dQ launch, so the
  // previous call's contents need no clearing.
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return FMHA_ERR_LAUNCH;
  return launch_backward(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, batch, total_q,
                         total_k, max_seqlen_q, max_seqlen_k, num_heads, head_dim, causal,
                         softmax_scale, dq, dk, dv, ws, (hipStream_t)stream);
}

fmha_status_t fmha_merge_partials(const float* o_part, const float* lse_part, int32_t num_parts,
                                  int32_t total_q, int32_t num_heads, int32_t head_dim,
                                  void* out, float* lse, void* stream) {
  if (num_parts < 1 || num_parts > fmha::kMaxSplits || total_q < 0 || num_heads <= 0)
    return FMHA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return FMHA_ERR_UNSUPPORTED;
  if ((int64_t)num_heads * total_q > INT32_MAX) return FMHA_ERR_UNSUPPORTED;
  if (total_q == 0) return FMHA_OK;
  if (o_part == nullptr || lse_part == nullptr || out == nullptr) return FMHA_ERR_INVALID_ARG;
  if (!aligned16(o_part) || (reinterpret_cast<uintptr_t>(lse_part) & 3u) || !aligned16(out) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)))
    return FMHA_ERR_INVALID_ARG;
  hipError_t e = fmha::launch_merge_partials(o_part, lse_part, num_parts, total_q, num_heads,
                                             head_dim, out, lse, (hipStream_t)stream);
  return e == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH;
}

fmha_status_t fmha_fwd_trace(int32_t pv_format, const void* q, const void* k, const void* v,
                             const void* v_scale,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t batch, int32_t total_q, int32_t total_k,
                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int32_t num_heads, int32_t head_dim,
                             int32_t causal, float softmax_scale,
                             void* out, float* lse, int32_t detailed,
                             int32_t traced_workgroups, uint64_t* trace, size_t trace_bytes,
                             void* stream) {
  if (pv_format < FMHA_PV_BF16 || pv_format > FMHA_PV_E2M1) return FMHA_ERR_INVALID_ARG;
  fmha_status_t st = check_common(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                                  max_seqlen_q, max_seqlen_k, num_heads, head_dim, causal,
                                  softmax_scale, out, lse);
  if (st != FMHA_OK) return st;
  if (head_dim != 128 || causal != 1) return FMHA_ERR_UNSUPPORTED;
  if (detailed != 0 && detailed != 1) return FMHA_ERR_INVALID_ARG;
  if (pv_format != FMHA_PV_BF16 && total_k > 0 && v_scale == nullptr) return FMHA_ERR_INVALID_ARG;
  if (v_scale && (reinterpret_cast<uintptr_t>(v_scale) & 3u)) return FMHA_ERR_INVALID_ARG;
  if (traced_workgroups < 1 || traced_workgroups > 4096) return FMHA_ERR_INVALID_ARG;
  const size_t need = (size_t)traced_workgroups * 8 * FMHA_TRACE_EVENTS_PER_WAVE * sizeof(uint64_t);
  if (trace == nullptr || (reinterpret_cast<uintptr_t>(trace) & 7u) || trace_bytes < need)
    return FMHA_ERR_INVALID_ARG;
  if (batch == 0 || total_q == 0 || max_seqlen_q == 0) return FMHA_OK;
  fmha::FwdParams p = make_params(q, k, v, cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k,
                                  max_seqlen_q, max_seqlen_k, num_heads, softmax_scale, out, lse);
  if (pv_format == FMHA_PV_E4M3) p.v_scale = static_cast<const float*>(v_scale);
  if (pv_format == FMHA_PV_E2M1) p.v_mx_scale = static_cast<const uint8_t*>(v_scale);
  p.trace = trace;
  p.trace_wgs = traced_workgroups;
  const int pv = pv_format == FMHA_PV_E4M3 ? fmha::kPvE4m3
                 : pv_format == FMHA_PV_E2M1 ? fmha::kPvE2m1 : fmha::kPvBf16;
  const hipError_t e = fmha::launch_fwd_trace(p, pv, true, detailed != 0, (hipStream_t)stream);
  return e == hipSuccess ? FMHA_OK : FMHA_ERR_LAUNCH;
}

int32_t fmha_fwd_auto_variant(int32_t batch, int32_t max_seqlen_q, int32_t num_heads) {
  if (batch < 0 || max_seqlen_q < 0 || num_heads < 0) return -1;
  return fmha::resolve_variant(fmha::kVariantAuto, batch, max_seqlen_q, num_heads);
}

fmha_status_t fmha_validate_cu_seqlens(const int32_t* host_cu, int32_t batch, int32_t total,
                                       int32_t max_seqlen) {
  if (batch < 0 || total < 0 || max_seqlen < 0) return FMHA_ERR_INVALID_ARG;
  if (host_cu == nullptr) return FMHA_ERR_INVALID_ARG;
  if (host_cu[0] != 0) return FMHA_ERR_INVALID_ARG;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t len = (int64_t)host_cu[b + 1] - host_cu[b];
    if (len < 0 || len > max_seqlen) return FMHA_ERR_INVALID_ARG;
  }
  return host_cu[batch] == total ? FMHA_OK : FMHA_ERR_INVALID_ARG;
}

const char* fmha_status_string(fmha_status_t status) {
  switch (status) {
    case FMHA_OK: return "ok";
    case FMHA_ERR_INVALID_ARG: return "invalid argument";
    case FMHA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FMHA_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

int32_t fmha_abi_version(void) { return FMHA_ABI_VERSION; }

}  // extern "C"
