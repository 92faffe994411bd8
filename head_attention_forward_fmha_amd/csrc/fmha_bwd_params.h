// Parameter block of the backward pass, shared by the host launcher and the
// gfx950 kernels.
#ifndef FMHA_BWD_PARAMS_H_
#define FMHA_BWD_PARAMS_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmha {

// Backward pass. The dQ kernel walks key tiles per query block and also
// computes D_i = dO_i . O_i and LSE_i * log2(e) (+inf for a row that saw no
// key, so that its P is 0) once per row, into the workspace; the dK/dV kernel,
// launched after it, walks query tiles per key block and reads them. Both
// recompute P from the saved LSE.
struct BwdParams {
  const void* q;          // bf16 [total_q, heads, d]
  const void* k;          // bf16 [total_k, heads, d]
  const void* v;          // bf16 [total_k, heads, d]
  const void* out;        // bf16 [total_q, heads, d], the forward's O
  const void* dout;       // bf16 [total_q, heads, d]
  const float* lse;       // fp32 [heads, total_q], the forward's LSE (natural log)
  const int32_t* cu_q;    // [batch + 1] or nullptr (dense)
  const int32_t* cu_k;
  void* dq;               // bf16 [total_q, heads, d]
  void* dk;               // bf16 [total_k, heads, d]
  void* dv;               // bf16 [total_k, heads, d]
  float* delta;           // workspace: fp32 [heads, total_q]
  float* lse2;            // workspace: fp32 [heads, total_q]
  int32_t batch;
  int32_t total_q;
  int32_t total_k;
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  int32_t heads;
  float scale;            // softmax_scale (fp32)
  float scale_log2;       // softmax_scale * log2(e)
  int32_t n_blocks;       // key blocks (dK/dV) or query blocks (dQ) per document
};

hipError_t launch_bwd(const BwdParams& p, int head_dim, bool causal, hipStream_t stream);

}  // namespace fmha

#endif  // FMHA_BWD_PARAMS_H_
