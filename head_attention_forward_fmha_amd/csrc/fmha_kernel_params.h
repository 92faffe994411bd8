// Kernel parameter block shared by the host launcher and the gfx950 kernels.
#ifndef FMHA_KERNEL_PARAMS_H_
#define FMHA_KERNEL_PARAMS_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmha {

struct FwdParams {
  const void* q;          // bf16 [total_q, heads, d]
  const void* k;          // bf16 [total_k, heads, d]
  const void* v;          // bf16 or e4m3 [total_k, heads, d]
  const int32_t* cu_q;    // [batch + 1] or nullptr (dense)
  const int32_t* cu_k;    // [batch + 1] or nullptr (dense)
  const float* v_scale;   // [heads] (fp8 P.V only)
  const uint8_t* v_mx_scale;  // E8M0 [ceil(total_k / 32), heads, d] (fp4 P.V only)
  void* out;              // bf16 [total_q, heads, d]
  float* lse;             // fp32 [heads, total_q] or nullptr
  int32_t batch;
  int32_t total_q;
  int32_t total_k;
  int32_t max_seqlen_q;
  int32_t max_seqlen_k;
  int32_t heads;
  float scale_log2;       // softmax_scale * log2(e)
  int32_t n_mblocks;      // query blocks per document (set by the launcher)
  // split-KV: the key tiles of every work item are cut into num_splits ranges,
  // each writing its own O (fp32, normalised by its own row sum) and LSE
  int32_t num_splits;     // 1 unless launched by launch_fwd_bf16_splitkv
  float* o_part;          // [num_splits, total_q, heads, d]
  float* lse_part;        // [num_splits, heads, total_q]
  // pipeline tracing (launch_fwd_trace only): per traced wave, kTraceEvents
  // 64-bit records (event << 56) | (shader clock counter mod 2^56)
  uint64_t* trace;        // [trace_wgs, 8 waves, kTraceEvents]
  int32_t trace_wgs;      // workgroups (lowest ids) that record
};

constexpr int kTraceEvents = 8192;   // records per traced wave; later events are dropped

// Events of the ping-pong kernel's timeline (launch_fwd_trace). A slot is the
// stretch between two workgroup barriers; in it a wave runs either the MFMA
// phase (Q.K^T, then P.V) or the VALU phase (copies, mask and softmax, wait for
// its copies).
enum TraceEvent : int {
  kEvSlot = 0,        // slot start (after the barrier)
  kEvQkDone = 1,      // MFMA phase: Q.K^T issued (detailed mode)
  kEvMfmaDone = 2,    // MFMA phase done
  kEvCopyIssued = 3,  // VALU phase: copies issued (detailed mode)
  kEvValuDone = 4,    // VALU phase: softmax done
  kEvWaitDone = 5,    // before the barrier (detailed mode)
  kEvItem = 6,        // a work item starts
};

// Number formats of the P.V product: bf16, fp8 e4m3 (one fp32 scale per head
// for V) or fp4 e2m1 (MXFP4 V, per-group power-of-two scales for P).
constexpr int kPvBf16 = 0;
constexpr int kPvE4m3 = 1;
constexpr int kPvE2m1 = 2;

// Kernel variants (the values of fmha.h's FMHA_VARIANT_*).
constexpr int kVariantAuto = 0;      // pick by problem size
constexpr int kVariantFourWave = 1;  // 4 waves, 128 query rows per workgroup
constexpr int kVariantPingPong = 2;  // 8 waves in two phase-shifted groups, 256 rows
constexpr int kVariantPipelined = 3; // 4 waves, each software-pipelined (bf16 only)
constexpr int kVariantWide = 4;      // 4 waves of 64 rows, one per SIMD (bf16 only)

// Query rows per workgroup of each kernel.
constexpr int kRowsFourWave = 128;
constexpr int kRowsPingPong = 256;
constexpr int kRowsPipelined = 128;
constexpr int kRowsWide = 256;

// The kernel a launch runs. Automatic selection takes the 8-wave kernel once the
// problem has at least 128 work items of 256 query rows (half the CUs of an
// MI355X; a split-KV launch has `splits` items per block), else the 4-wave
// kernel, whose smaller blocks spread a small problem over more CUs.
inline int resolve_variant(int variant, int32_t batch, int32_t max_seqlen_q, int32_t heads,
                           int splits = 1) {
  if (variant != kVariantAuto) return variant;
  const long long blocks = ((long long)max_seqlen_q + kRowsPingPong - 1) / kRowsPingPong *
                           heads * batch * splits;
  return blocks >= 128 ? kVariantPingPong : kVariantFourWave;
}

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, bool causal, int variant,
                           hipStream_t stream);
hipError_t launch_fwd_fp8pv(const FwdParams& p, int head_dim, bool causal, int variant,
                            hipStream_t stream);
hipError_t launch_fwd_fp4pv(const FwdParams& p, int head_dim, bool causal, int variant,
                            hipStream_t stream);
// bf16 forward pass with the key tiles of each work item cut into p.num_splits
// ranges: writes p.o_part / p.lse_part, not p.out / p.lse (see launch_merge_partials)
hipError_t launch_fwd_bf16_splitkv(const FwdParams& p, int head_dim, bool causal, int variant,
                                   hipStream_t stream);
// out[t, h, :] = sum_s exp(LSE_s - LSE) O_s[t, h, :] (bf16), LSE = log sum_s exp(LSE_s)
hipError_t launch_merge_partials(const float* o_part, const float* lse_part, int num_parts,
                                 int total_q, int heads, int head_dim, void* out, float* lse,
                                 hipStream_t stream);
// the causal ping-pong kernel (d = 128, P.V format pv) with phase stamps:
// detailed stamps every event, coarse only kEvSlot, kEvMfmaDone, kEvValuDone,
// kEvItem; p.trace_wgs workgroups record into p.trace
hipError_t launch_fwd_trace(const FwdParams& p, int pv, bool causal, bool detailed,
                            hipStream_t stream);
// split count the automatic choice uses for a problem on the current device
int recommended_splits(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                       int32_t heads, bool causal, int variant);
constexpr int kMaxSplits = 64;

}  // namespace fmha

#endif  // FMHA_KERNEL_PARAMS_H_
