// Merge of split-KV partial results.
//
// A query row's keys split into disjoint ranges s give per-range results
// O_s = sum_{j in s} exp(S_j) V_j / sum_{j in s} exp(S_j) and
// LSE_s = ln sum_{j in s} exp(S_j). Softmax over the union is the same
// rescaling by exp of a maximum difference that the online softmax applies
// tile by tile ("[BUG] Unexpected Slower Performance in C++ CuTe
// (77_blackwell_fmha) vs Python CuTe DSL (fmha.py) on Jetson Thor", Key
// Observation 2, the softmax_step listings), here applied once across ranges:
//   LSE = m + ln sum_s exp(LSE_s - m),  m = max_s LSE_s,
//   O   = sum_s exp(LSE_s - LSE) O_s.
// Ranges that saw no key have LSE_s = -inf and weigh nothing; a row with no key
// at all gets O = 0 and LSE = -inf.
//
// This is HBM-bound work (num_parts * (4d + 4) bytes read and 2d + 4 written
// per row): lanes over d with 16-byte loads, several rows per wave.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fmha_kernel_params.h"

namespace fmha {

namespace {

// Each lane merges 4 consecutive d values of one row (16-byte loads and
// stores); a wave covers 64 * 4 / kD rows, a block kMergeWaves waves.
constexpr int kMergeWaves = 4;

template <int kD>
__global__ __launch_bounds__(64 * kMergeWaves) void fmha_merge_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, int num_parts,
    int total_q, int heads, __bf16* __restrict__ out, float* __restrict__ lse) {
  constexpr int kLanesPerRow = kD / 4;
  constexpr int kRowsPerWave = 64 / kLanesPerRow;
  const int lane = threadIdx.x & 63;
  const long long row = ((long long)blockIdx.x * kMergeWaves + (threadIdx.x >> 6)) * kRowsPerWave +
                        lane / kLanesPerRow;
  const long long n_rows = (long long)total_q * heads;
  if (row >= n_rows) return;
  const int sub = lane % kLanesPerRow;
  const int t = (int)(row / heads);
  const int h = (int)(row - (long long)t * heads);
  const size_t part_stride = (size_t)total_q * heads * kD;   // between parts of O
  const size_t lse_stride = (size_t)heads * total_q;          // between parts of LSE
  const size_t lse_idx = (size_t)h * total_q + t;

  float m = -INFINITY;
  for (int s = 0; s < num_parts; ++s) m = fmaxf(m, lse_part[s * lse_stride + lse_idx]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  if (m != -INFINITY) {
    const float4* src = reinterpret_cast<const float4*>(o_part + (size_t)row * kD) + sub;
#pragma unroll 4
    for (int s = 0; s < num_parts; ++s) {
      const float w = expf(lse_part[s * lse_stride + lse_idx] - m);
      const float4 o = src[s * (part_stride / 4)];
      den += w;
      acc.x += w * o.x;
      acc.y += w * o.y;
      acc.z += w * o.z;
      acc.w += w * o.w;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  bf16x4_t r;
  r[0] = (__bf16)(acc.x * inv);
  r[1] = (__bf16)(acc.y * inv);
  r[2] = (__bf16)(acc.z * inv);
  r[3] = (__bf16)(acc.w * inv);
  *reinterpret_cast<bf16x4_t*>(out + (size_t)row * kD + 4 * sub) = r;
  if (lse != nullptr && sub == 0) lse[lse_idx] = den > 0.f ? m + logf(den) : -INFINITY;
}

}  // namespace

hipError_t launch_merge_partials(const float* o_part, const float* lse_part, int num_parts,
                                 int total_q, int heads, int head_dim, void* out, float* lse,
                                 hipStream_t stream) {
  const long long n_rows = (long long)total_q * heads;
  if (n_rows == 0) return hipSuccess;
  if (head_dim != 128 && head_dim != 64) return hipErrorInvalidValue;
  const long long rows_per_block = (long long)kMergeWaves * (64 * 4 / head_dim);
  const long long blocks = (n_rows + rows_per_block - 1) / rows_per_block;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(64 * kMergeWaves);
  if (head_dim == 128)
    hipLaunchKernelGGL(fmha_merge_kernel<128>, grid, block, 0, stream, o_part, lse_part,
                       num_parts, total_q, heads, (__bf16*)out, lse);
  else
    hipLaunchKernelGGL(fmha_merge_kernel<64>, grid, block, 0, stream, o_part, lse_part,
                       num_parts, total_q, heads, (__bf16*)out, lse);
  return hipGetLastError();
}

}  // namespace fmha
