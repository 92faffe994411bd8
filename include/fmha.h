/*
 * fmha.h -- C ABI of the MI355X (gfx950) fused multi-head attention forward pass.
 *
 * The operation (sources: "[BUG] Unexpected Slower Performance in C++ CuTe
 * (77_blackwell_fmha) vs Python CuTe DSL (fmha.py) on Jetson Thor", Key
 * Observation 2, the softmax_step listings; "CuTe DSL 4.7/4.8 regression:
 * FlashAttention-4 SM100 forward kernel spills registers", Describe the bug and
 * the benchmark script under Steps/Code to reproduce bug): for every document b
 * and head h,
 *
 *     S   = softmax_scale * Q_b,h K_b,h^T                 (sq x sk)
 *     S_ij = -inf where causal and j > i + (sk - sq)       (bottom-right aligned)
 *     P   = softmax(S) row by row,  O_b,h = P V_b,h,
 *     LSE_i = ln sum_j exp(S_ij)                            (natural log)
 *
 * computed as tiled Q.K^T, an online softmax in the exp2 domain (scale and
 * running row maximum folded into one multiply-add), and P.V with fp32
 * accumulation. A query row that sees no key gets O = 0 and LSE = -inf.
 *
 * Layout. Tokens of all documents are packed: q, k, v, out are contiguous
 * row-major [total_tokens, num_heads, head_dim]. Documents are given by int32
 * prefix arrays cu_seqlens_q / cu_seqlens_k of length batch + 1 (document b
 * owns query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1])), as the benchmark script of the
 * FlashAttention-4 spill issue passes them. When both cu_seqlens pointers are
 * NULL the input is dense [batch, seqlen, num_heads, head_dim] with
 * seqlen_q = max_seqlen_q and seqlen_k = max_seqlen_k, which is byte-identical
 * to the packed layout with uniform documents. lse is fp32 [num_heads, total_q].
 *
 * Ownership. The caller allocates and owns every buffer; all pointers except
 * those documented as host pointers are device pointers on the current HIP
 * device. The library allocates nothing, keeps no mutable state, is reentrant,
 * and enqueues its work on `stream` (a hipStream_t; NULL is the legacy default
 * stream) without synchronising. Outputs are complete once the stream reaches
 * the enqueued kernel.
 *
 * Errors. Argument checks run on the host before any HIP call and return
 * FMHA_ERR_INVALID_ARG (null or misaligned pointers, negative sizes,
 * inconsistent dense sizes, non-finite scale) or FMHA_ERR_UNSUPPORTED (a
 * head_dim other than 64 or 128, or a problem beyond the kernels' 32-bit
 * offsets: heads * head_dim * (total_q + 64) or heads * head_dim * (total_k +
 * 64) above 2^31 - 1, heads * total_q above 2^31 - 1, batch or heads above
 * 65535). A failed launch returns FMHA_ERR_LAUNCH. The
 * contents of cu_seqlens are a precondition (non-decreasing, starting at 0,
 * ending at total, every length <= max_seqlen); they are not read on the host,
 * and fmha_validate_cu_seqlens checks a host copy. Behaviour on violated
 * preconditions is undefined.
 */
#ifndef FMHA_H_
#define FMHA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FMHA_OK = 0,
  FMHA_ERR_INVALID_ARG = 1,
  FMHA_ERR_UNSUPPORTED = 2,
  FMHA_ERR_LAUNCH = 3
} fmha_status_t;

/*
 * bf16 forward pass.
 *   q            bf16 [total_q, num_heads, head_dim], 16-byte aligned
 *   k, v         bf16 [total_k, num_heads, head_dim], 16-byte aligned
 *   cu_seqlens_q int32 [batch + 1] device array, or NULL (dense)
 *   cu_seqlens_k int32 [batch + 1] device array, or NULL (dense); both NULL or both set
 *   batch        number of documents (>= 0)
 *   total_q/k    rows of q and of k/v (dense: batch * max_seqlen_q / _k)
 *   max_seqlen_q longest query document (sizes the launch grid)
 *   max_seqlen_k longest key document
 *   num_heads    > 0
 *   head_dim     64 or 128
 *   causal       0 or 1
 *   softmax_scale fp32 multiplier of Q.K^T (typically 1/sqrt(head_dim))
 *   out          bf16 [total_q, num_heads, head_dim], 16-byte aligned
 *   lse          fp32 [num_heads, total_q], or NULL to skip it
 *   stream       hipStream_t
 */
fmha_status_t fmha_fwd(const void* q, const void* k, const void* v,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int32_t batch, int32_t total_q, int32_t total_k,
                       int32_t max_seqlen_q, int32_t max_seqlen_k,
                       int32_t num_heads, int32_t head_dim,
                       int32_t causal, float softmax_scale,
                       void* out, float* lse, void* stream);

/*
 * Forward pass with P.V in fp8 (OCP e4m3), the FP8 PV variant of "Kernel
 * Bottleneck Tuning (validated on FA4 FP4/FP8 PV, GB300)" (introduction and
 * section 5). Q.K^T stays bf16. V arrives as e4m3 codes with one fp32 scale per
 * head: V[t, h, :] = decode(v_e4m3[t, h, :]) * v_scale[h]. After exp2, P is
 * rounded to e4m3 with a power-of-two scale folded into the exp2 argument (the
 * log-domain refactoring of that page's section 4); the row sum uses the fp32
 * values before rounding, and the epilogue folds v_scale and the inverse P
 * scale into the single normalising multiply.
 *   v_e4m3   uint8 [total_k, num_heads, head_dim], 16-byte aligned
 *   v_scale  fp32 [num_heads] device array
 * Every other argument as for fmha_fwd. head_dim must be 128.
 */
fmha_status_t fmha_fwd_fp8pv(const void* q, const void* k, const uint8_t* v_e4m3,
                             const float* v_scale,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t batch, int32_t total_q, int32_t total_k,
                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int32_t num_heads, int32_t head_dim,
                             int32_t causal, float softmax_scale,
                             void* out, float* lse, void* stream);

/*
 * Forward pass with P.V in fp4 (OCP e2m1 with power-of-two block scales), the
 * FP4 PV variant of "Kernel Bottleneck Tuning (validated on FA4 FP4/FP8 PV,
 * GB300)" (introduction; section 4, log-domain refactoring). Q.K^T stays bf16.
 *
 * V arrives in OCP MXFP4 along the token axis of the packed tensor:
 *   v_e2m1      uint8 [total_k, num_heads, head_dim / 2], 16-byte aligned: two
 *               e2m1 codes per byte, even d in the low nibble;
 *   v_mx_scale  uint8 [ceil(total_k / 32), num_heads, head_dim], 4-byte
 *               aligned: E8M0 exponents, one per 32 consecutive tokens (from
 *               token 0 of the packed tensor), head and d;
 *   V[t, h, d] = e2m1(code[t, h, d]) * 2^(v_mx_scale[t / 32, h, d] - 127).
 * A 32-token block may span two documents; documents may start anywhere.
 *
 * P is quantised per group, a group being the keys of one query row inside one
 * 32-token block: with c = softmax_scale * log2(e) and g the group's largest
 * raw score q.k, E = ceil(c*g - log2 6) and P_hat = 2^E * e2m1(2^(c*q.k - E))
 * (round to nearest even), the division by 2^E being a subtraction inside the
 * exp2 argument. The quantised P depends only on the scores (not on the order
 * in which key tiles are visited). The row sum uses the values before rounding,
 * so LSE is that of the exact scores, and O = sum P_hat V / sum 2^(c q.k).
 * Every other argument as for fmha_fwd; head_dim must be 128; v_mx_scale may be
 * NULL only when total_k == 0.
 */
fmha_status_t fmha_fwd_fp4pv(const void* q, const void* k, const uint8_t* v_e2m1,
                             const uint8_t* v_mx_scale,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t batch, int32_t total_q, int32_t total_k,
                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int32_t num_heads, int32_t head_dim,
                             int32_t causal, float softmax_scale,
                             void* out, float* lse, void* stream);

/*
 * Kernel variant selection, for testing and tuning. FMHA_VARIANT_AUTO (what
 * fmha_fwd, fmha_fwd_fp8pv and fmha_fwd_fp4pv use) takes the 8-wave ping-pong kernel when the
 * problem has at least 128 blocks of 256 query rows, else the 4-wave kernel;
 * fmha_fwd_splitkv counts each block num_splits times.
 * All variants compute the same function. The 4-wave and ping-pong kernels run
 * the same per-row arithmetic in the same key-tile order and give bit-identical
 * results; the pipelined and 64-row-wave kernels take the lazy row-maximum
 * decision per 32 keys and agree with them within rounding, which is all the
 * ABI promises.
 */
#define FMHA_VARIANT_AUTO 0
#define FMHA_VARIANT_FOUR_WAVE 1   /* 4 waves, 128 query rows per workgroup   */
#define FMHA_VARIANT_PINGPONG 2    /* 8 waves in two phase-shifted groups     */
#define FMHA_VARIANT_PIPELINED 3   /* 4 waves, each software-pipelined; bf16
                                      only (fp8/fp4 P.V: FMHA_ERR_UNSUPPORTED) */
#define FMHA_VARIANT_WIDE 4        /* 4 waves of 64 query rows, one per SIMD,
                                      each K/V operand read feeding two MFMAs;
                                      bf16 only (fp8/fp4 P.V, split-KV:
                                      FMHA_ERR_UNSUPPORTED) */

/* fmha_fwd with an explicit kernel variant (any other value: INVALID_ARG). */
fmha_status_t fmha_fwd_variant(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t total_q, int32_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t num_heads, int32_t head_dim,
                               int32_t causal, float softmax_scale,
                               void* out, float* lse, int32_t variant, void* stream);

/* fmha_fwd_fp8pv with an explicit kernel variant (any other value: INVALID_ARG;
 * FMHA_VARIANT_PIPELINED, FMHA_VARIANT_WIDE: FMHA_ERR_UNSUPPORTED). */
fmha_status_t fmha_fwd_fp8pv_variant(const void* q, const void* k, const uint8_t* v_e4m3,
                                     const float* v_scale,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     int32_t batch, int32_t total_q, int32_t total_k,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     int32_t num_heads, int32_t head_dim,
                                     int32_t causal, float softmax_scale,
                                     void* out, float* lse, int32_t variant, void* stream);

/* fmha_fwd_fp4pv with an explicit kernel variant (any other value: INVALID_ARG;
 * FMHA_VARIANT_PIPELINED, FMHA_VARIANT_WIDE: FMHA_ERR_UNSUPPORTED). */
fmha_status_t fmha_fwd_fp4pv_variant(const void* q, const void* k, const uint8_t* v_e2m1,
                                     const uint8_t* v_mx_scale,
                                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                     int32_t batch, int32_t total_q, int32_t total_k,
                                     int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     int32_t num_heads, int32_t head_dim,
                                     int32_t causal, float softmax_scale,
                                     void* out, float* lse, int32_t variant, void* stream);

/*
 * Split-KV forward pass (bf16): the same function as fmha_fwd_variant, for
 * problems with too few query blocks to fill the GPU (short query ranges
 * against long keys). The key tiles each (document, head, query block) visits
 * are cut into num_splits near-equal ranges; each range runs as its own work
 * item and writes its O (fp32, normalised by its own row sum) and LSE into the
 * workspace; a second kernel merges them (as fmha_merge_partials) into out and
 * lse on the same stream.
 *   num_splits       1 .. 64 (fmha_fwd_splitkv_num_splits suggests one); 1 runs
 *                    the unsplit pass (fmha_fwd_variant) and needs no workspace
 *   workspace        device memory, 16-byte aligned, at least
 *                    fmha_fwd_splitkv_workspace_size(...) bytes, owned by the
 *                    caller (NULL allowed when num_splits is 1); contents on
 *                    return when num_splits > 1: O parts fp32
 *                    [num_splits, total_q, num_heads, head_dim], then LSE parts
 *                    fp32 [num_splits, num_heads, total_q]. Calls that share a
 *                    workspace must not overlap.
 *   variant          FMHA_VARIANT_AUTO, _FOUR_WAVE or _PINGPONG (_PIPELINED,
 *                    _WIDE: FMHA_ERR_UNSUPPORTED)
 * Every other argument as for fmha_fwd.
 */
fmha_status_t fmha_fwd_splitkv(const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t total_q, int32_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t num_heads, int32_t head_dim,
                               int32_t causal, float softmax_scale,
                               void* out, float* lse, int32_t num_splits,
                               void* workspace, size_t workspace_bytes,
                               int32_t variant, void* stream);

/* Bytes of workspace fmha_fwd_splitkv needs: num_splits * total_q * num_heads *
 * (head_dim + 1) * 4 when num_splits > 1, 0 when num_splits is 1 or a size is
 * invalid. Host only. */
size_t fmha_fwd_splitkv_workspace_size(int32_t total_q, int32_t num_heads, int32_t head_dim,
                                       int32_t num_splits);

/* The split count that minimises the estimated time of a problem on the current
 * HIP device (1: do not split); -1 for negative sizes or an unknown variant.
 * Queries the device's compute-unit count once; launches nothing. */
int32_t fmha_fwd_splitkv_num_splits(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_heads, int32_t causal, int32_t variant);

/*
 * Merges partial attention results over disjoint key ranges of the same query
 * rows (the combine step of split-KV, and of a key-sharded, context-parallel
 * pass after the parts are gathered):
 *   LSE = log sum_s exp(LSE_s),  out = sum_s exp(LSE_s - LSE) * O_s  (bf16)
 * Parts with LSE_s = -inf (no key) weigh nothing; a row with no key anywhere
 * gets out = 0, LSE = -inf.
 *   o_part    fp32 [num_parts, total_q, num_heads, head_dim], 16-byte aligned
 *   lse_part  fp32 [num_parts, num_heads, total_q] (natural log)
 *   out       bf16 [total_q, num_heads, head_dim], 16-byte aligned
 *   lse       fp32 [num_heads, total_q], or NULL
 *   num_parts 1 .. 64; head_dim 64 or 128
 */
fmha_status_t fmha_merge_partials(const float* o_part, const float* lse_part, int32_t num_parts,
                                  int32_t total_q, int32_t num_heads, int32_t head_dim,
                                  void* out, float* lse, void* stream);

/*
 * Pipeline trace of the forward pass ("Kernel Bottleneck Tuning (validated on
 * FA4 FP4/FP8 PV, GB300)", section 2: trace the real pipeline, coarsely). Runs
 * the causal 8-wave ping-pong kernel on the problem, computing out and lse as
 * the forward entry points do, while every wave of the first
 * traced_workgroups workgroups records its phase boundaries:
 *   trace[wg][wave][i], wg < traced_workgroups, wave < 8, i < FMHA_TRACE_EVENTS_PER_WAVE:
 *     (event << 56) | (shader clock counter mod 2^56), from s_memtime.
 * Records after a wave's FMHA_TRACE_EVENTS_PER_WAVE-th are dropped; entries it
 * did not write keep their contents, so clear the buffer first (a zero word
 * ends a wave's records). Events (FMHA_TRACE_EV_*): a slot is the stretch
 * between two workgroup barriers, in which a wave runs either the MFMA phase
 * (Q.K^T, then P.V) or the VALU phase (copies, mask and softmax, wait for its
 * copies); ITEM marks the start of each work item. detailed = 0 (coarse)
 * records SLOT, MFMA_DONE, VALU_DONE and ITEM; detailed = 1 all of them.
 * Each stamp is a side-effecting scalar instruction that the compiler cannot
 * schedule work across: the coarse mode perturbs the pipeline least; detailed
 * spans are longer than the untraced kernel's and locate time rather than
 * measure it.
 *   pv_format  FMHA_PV_BF16 (v bf16, v_scale NULL), FMHA_PV_E4M3 (v e4m3 codes,
 *              v_scale fp32 [heads]) or FMHA_PV_E2M1 (v MXFP4 codes, v_scale the
 *              E8M0 exponents), as fmha_fwd / _fp8pv / _fp4pv
 *   causal     must be 1; head_dim must be 128 (else FMHA_ERR_UNSUPPORTED)
 *   trace      8-byte aligned, at least traced_workgroups * 8 *
 *              FMHA_TRACE_EVENTS_PER_WAVE * 8 bytes; traced_workgroups 1..4096
 */
#define FMHA_PV_BF16 0
#define FMHA_PV_E4M3 1
#define FMHA_PV_E2M1 2
#define FMHA_TRACE_EVENTS_PER_WAVE 8192
#define FMHA_TRACE_EV_SLOT 0         /* slot start, after the barrier          */
#define FMHA_TRACE_EV_QK_DONE 1      /* MFMA phase: Q.K^T issued (detailed)     */
#define FMHA_TRACE_EV_MFMA_DONE 2    /* MFMA phase done                         */
#define FMHA_TRACE_EV_COPY_ISSUED 3  /* VALU phase: copies issued (detailed)    */
#define FMHA_TRACE_EV_VALU_DONE 4    /* VALU phase: softmax done                */
#define FMHA_TRACE_EV_WAIT_DONE 5    /* copies landed, before the barrier (detailed) */
#define FMHA_TRACE_EV_ITEM 6         /* a work item starts                      */
fmha_status_t fmha_fwd_trace(int32_t pv_format, const void* q, const void* k, const void* v,
                             const void* v_scale,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             int32_t batch, int32_t total_q, int32_t total_k,
                             int32_t max_seqlen_q, int32_t max_seqlen_k,
                             int32_t num_heads, int32_t head_dim,
                             int32_t causal, float softmax_scale,
                             void* out, float* lse, int32_t detailed,
                             int32_t traced_workgroups, uint64_t* trace, size_t trace_bytes,
                             void* stream);

/*
 * Backward pass of fmha_fwd: dQ, dK, dV of the attention given the upstream
 * gradient dO, with P recomputed from the forward's LSE. The step timed in
 * "CuTe DSL 4.7/4.8 regression: FlashAttention-4 SM100 forward kernel spills
 * registers" (Describe the bug; Steps/Code to reproduce bug) is that forward
 * followed by this backward of mean(O^2). For every document and head, with
 * P as defined at the top of this header and tau = softmax_scale:
 *
 *     dV = P^T dO,  dP = dO V^T,  dS_ij = P_ij (dP_ij - D_i),  D_i = dO_i . O_i,
 *     dQ = tau dS K,  dK = tau dS^T Q,
 *
 * (D_i = sum_j P_ij dP_ij, as O_i = sum_j P_ij V_j). Query rows that saw no key
 * (LSE = -inf) contribute nothing and get dQ = 0; keys no query sees get
 * dK = dV = 0. The result is deterministic: every element is summed in a fixed
 * order, without atomics. P and dS are rounded to bf16 as MFMA operands, D is
 * taken from the bf16 O, accumulation is fp32.
 *   q, k, v, cu_seqlens_*, sizes, causal, softmax_scale   as for fmha_fwd
 *   out       bf16 [total_q, num_heads, head_dim], the forward's output
 *   dout      bf16 [total_q, num_heads, head_dim], 16-byte aligned
 *   lse       fp32 [num_heads, total_q], the forward's LSE (required)
 *   dq        bf16 [total_q, num_heads, head_dim], 16-byte aligned
 *   dk, dv    bf16 [total_k, num_heads, head_dim], 16-byte aligned
 *   workspace device memory of at least fmha_bwd_workspace_size(total_q,
 *             num_heads) bytes, 16-byte aligned, owned by the caller; it holds
 *             D and LSE * log2(e) per (head, row) and may be reused once the
 *             stream has passed this call
 * Errors as for fmha_fwd; a missing or short workspace, or a NULL dout, lse,
 * dq, dk or dv for a non-empty problem, gives FMHA_ERR_INVALID_ARG.
 */
size_t fmha_bwd_workspace_size(int32_t total_q, int32_t num_heads);
fmha_status_t fmha_bwd(const void* q, const void* k, const void* v, const void* out,
                       const void* dout, const float* lse,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                       int32_t batch, int32_t total_q, int32_t total_k,
                       int32_t max_seqlen_q, int32_t max_seqlen_k,
                       int32_t num_heads, int32_t head_dim,
                       int32_t causal, float softmax_scale,
                       void* dq, void* dk, void* dv,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * fmha_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid allocation. Same arguments, results and errors
 * as fmha_bwd (bitwise the same dQ, dK, dV). D and LSE * log2(e) go to a
 * fixed device array of FMHA_NOALLOC_SCRATCH_BYTES inside the library, one
 * copy per GPU, which each GPU holds until the process ends; its address is
 * looked up (hipGetSymbolAddress, no allocation) on the first call on a device.
 * The call allocates nothing.
 *   limit     fmha_bwd_workspace_size(total_q, num_heads) <= FMHA_NOALLOC_SCRATCH_BYTES,
 *             i.e. num_heads * total_q <= 2^21 (c4: 2^20); larger problems
 *             return FMHA_ERR_UNSUPPORTED before any HIP call
 *   sharing   every call on a GPU uses that GPU's one array: calls that can
 *             overlap on one GPU (other streams, other threads) race and must
 *             be ordered by the caller; sequential calls on one stream are safe
 *   device    the current device must be the stream's device
 * A failed address lookup returns FMHA_ERR_LAUNCH.
 */
#define FMHA_NOALLOC_SCRATCH_BYTES (16u << 20)
fmha_status_t fmha_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t total_q, int32_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t num_heads, int32_t head_dim,
                               int32_t causal, float softmax_scale,
                               void* dq, void* dk, void* dv, void* stream);

/*
 * The kernel variant FMHA_VARIANT_AUTO resolves to for a problem of `batch`
 * documents, longest query document max_seqlen_q and num_heads heads:
 * FMHA_VARIANT_FOUR_WAVE or FMHA_VARIANT_PINGPONG. Negative sizes give -1.
 * Host only; makes no HIP call.
 */
int32_t fmha_fwd_auto_variant(int32_t batch, int32_t max_seqlen_q, int32_t num_heads);

/*
 * Host-side check of a cu_seqlens array (HOST pointer, batch + 1 entries):
 * starts at 0, is non-decreasing, ends at total, and no document is longer
 * than max_seqlen. Returns FMHA_OK or FMHA_ERR_INVALID_ARG. Makes no HIP call.
 */
fmha_status_t fmha_validate_cu_seqlens(const int32_t* host_cu_seqlens, int32_t batch,
                                       int32_t total, int32_t max_seqlen);

/* Static, NUL-terminated description of a status code. */
const char* fmha_status_string(fmha_status_t status);

/* ABI version of this header: (major << 16) | minor. */
int32_t fmha_abi_version(void);

#define FMHA_ABI_VERSION ((1 << 16) | 5)

#ifdef __cplusplus
}
#endif

#endif /* FMHA_H_ */
