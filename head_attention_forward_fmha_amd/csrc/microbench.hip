// Instruction-throughput microbenchmarks for gfx950 (MI355X, CDNA4).
//
// "Kernel Bottleneck Tuning (validated on FA4 FP4/FP8 PV, GB300)", section 1:
// measure each instruction's throughput in isolation, with several independent
// dependency chains per thread and a cycle counter around the timed loop, and
// compare the rates with the budget a kernel design assumes. Here every wave
// times itself with s_memtime (the shader clock) between two barriers; the
// host reports the median over all waves of the device.
//
// One workgroup per compute unit: each kernel holds 96 KB of LDS, so a second
// workgroup cannot be resident on the same CU, and a workgroup has 4 * wps
// waves, i.e. wps waves on each of the CU's four SIMDs.
//
// Every LDS access stays inside the first 64 KB of the 96 KB array, and every
// global access is the wave's own result slot (block * 16 + wave, block < grid,
// wave < 16).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "fmha_microbench.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsBytes = 98304;     // forces one workgroup per CU
constexpr int kLdsUsed = 65536;      // the part the LDS benchmarks read
constexpr int kMaxWaves = 16;        // result slots per workgroup
constexpr int kChains = 8;           // independent dependency chains

struct Slot {
  unsigned long long cycles;
  float sink;  // keeps every chain's result live
  float pad;
};

// Softmax-like vector stream (one iteration: 32 scores -> FMA, exp2, row sum,
// bf16 pack), the per-tile work of the attention softmax.
__device__ __forceinline__ float softmax_like(float (&x)[32], int iters) {
  float l = 0.f;
  const float c = 0.1275f, m = -0.5f;
  for (int it = 0; it < iters; ++it) {
    int packed = 0;
#pragma unroll
    for (int i = 0; i < 32; i += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], c, m));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i + 1], c, m));
      l += p0 + p1;
      packed ^= __builtin_bit_cast(int, bf16x2{(__bf16)p0, (__bf16)p1});
      x[i] = __builtin_fmaf(p1, 0.5f, x[i]);
    }
    l += (float)packed;
  }
  return l;
}

// 2^x on the FMA path, for comparing a polynomial exp2 with v_exp_f32 (which
// shares the quarter-rate unit with the P conversions). Cody and Waite's range
// reduction: x = n + f with n = round(x) and |f| <= 1/2, rounding by adding and
// subtracting 1.5 * 2^23 (n then sits in the low mantissa bits of the sum); 2^f
// by a degree-3 polynomial fitted here for relative error on [-1/2, 1/2] (max
// 7.5e-5, about 13.7 bits, evaluated in fp32: more than the 8 bits a bf16 P
// keeps); 2^n by adding n to the exponent field. x is clamped at -125, so that
// the result stays a normal number (the polynomial's value lies in [0.7, 1.42]).
// Eight vector instructions: max, add, sub, sub, three FMAs, shift-and-add (in
// this benchmark a ninth: the compiler quiets a possible NaN with another max,
// since each chain feeds a value built by integer addition back in).
__device__ __forceinline__ float exp2_poly(float x) {
  constexpr float kRound = 12582912.f;   // 1.5 * 2^23
  x = __builtin_fmaxf(x, -125.f);
  const float t = x + kRound;
  const float n = t - kRound;
  const float f = x - n;
  const float p = __builtin_fmaf(
      __builtin_fmaf(__builtin_fmaf(0.05517132207751274f, f, 0.24261054396629333f), f,
                     0.6932609677314758f),
      f, 0.9999281167984009f);
  return __builtin_bit_cast(float, __builtin_bit_cast(int, p) + (__builtin_bit_cast(int, t) << 23));
}

template <int kWhich>
__global__ __launch_bounds__(1024) void microbench_kernel(Slot* out, int iters, int mfma_waves) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int simd_wave = wave >> 2;  // 0 .. wps-1: the wave's index on its SIMD
  if constexpr (kWhich == FMHA_MB_LDS_B128 || kWhich == FMHA_MB_MFMA_LDS_B128) {
    for (int i = threadIdx.x; i < kLdsUsed / 4; i += blockDim.x)
      ((uint32_t*)lds)[i] = (i * 2654435761u) & 0x3f803f80u;  // small bf16 values
  } else if (threadIdx.x == 0) {
    lds[blockIdx.x % kLdsBytes] = 0;  // the array stays allocated
  }
  __syncthreads();
  float sink = 0.f;
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  unsigned long long t_stop = 0;  // set by waves timed over part of their loop

  if constexpr (kWhich == FMHA_MB_EXP2_POLY) {
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = 0.01f * (lane + c);
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < kChains; ++c) x[c] = exp2_poly(-__builtin_fabsf(x[c]));
#pragma unroll
    for (int c = 0; c < kChains; ++c) sink += x[c];
  } else if constexpr (kWhich == FMHA_MB_EXP2_WITH_FMA) {
    // one op: one v_exp_f32 and four v_fma_f32, each on its own chain
    float x[kChains], y[kChains][4];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      x[c] = 0.01f * (lane + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) y[c][j] = 0.02f * (lane + c + j);
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
          x[c] = __builtin_amdgcn_exp2f(-__builtin_fabsf(x[c]));
#pragma unroll
          for (int j = 0; j < 4; ++j) y[c][j] = __builtin_fmaf(y[c][j], 0.999f, 0.001f);
        }
#pragma unroll
    for (int c = 0; c < kChains; ++c) sink += x[c] + y[c][0] + y[c][1] + y[c][2] + y[c][3];
  } else if constexpr (kWhich == FMHA_MB_EXP2 || kWhich == FMHA_MB_FMA) {
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = 0.01f * (lane + c);
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
          if constexpr (kWhich == FMHA_MB_EXP2)
            x[c] = __builtin_amdgcn_exp2f(-__builtin_fabsf(x[c]));  // stays in (0, 1]
          else
            x[c] = __builtin_fmaf(x[c], 0.999f, 0.001f);
        }
#pragma unroll
    for (int c = 0; c < kChains; ++c) sink += x[c];
  } else if constexpr (kWhich == FMHA_MB_CVT_BF16 || kWhich == FMHA_MB_CVT_E4M3 ||
                       kWhich == FMHA_MB_CVT_E2M1 || kWhich == FMHA_MB_EXP2_E4M3) {
    // each chain converts two floats into the packed word that the next
    // conversion reads back as one of its inputs
    int w[kChains];
    float y[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
      w[c] = 0x3c003c00 + lane + c;
      y[c] = 0.25f + 0.01f * c;
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
          const float a = __builtin_bit_cast(float, w[c]);
          if constexpr (kWhich == FMHA_MB_CVT_BF16) {
            w[c] = __builtin_bit_cast(int, bf16x2{(__bf16)a, (__bf16)y[c]});
          } else if constexpr (kWhich == FMHA_MB_CVT_E4M3) {
            w[c] = __builtin_amdgcn_cvt_pk_fp8_f32(a, y[c], w[c], false);
          } else if constexpr (kWhich == FMHA_MB_CVT_E2M1) {
            w[c] = (int)__builtin_amdgcn_cvt_scalef32_pk_fp4_f32((unsigned)w[c], a, y[c], 1.f, 0);
          } else {
            // the fp8 P path: exp2 of two scores, then one packed e4m3 convert
            const float p0 = __builtin_amdgcn_exp2f(-__builtin_fabsf(a));
            const float p1 = __builtin_amdgcn_exp2f(-__builtin_fabsf(y[c]));
            w[c] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, w[c], false);
            y[c] = p0;
          }
        }
#pragma unroll
    for (int c = 0; c < kChains; ++c) sink += (float)w[c] + y[c];
  } else if constexpr (kWhich == FMHA_MB_MFMA_BF16 || kWhich == FMHA_MB_MFMA_E4M3 ||
                       kWhich == FMHA_MB_MFMA_WITH_VALU) {
    const bool mfma = kWhich != FMHA_MB_MFMA_WITH_VALU || simd_wave < mfma_waves;
    if (mfma) {
      // four accumulation chains, 8 MFMAs per chain per iteration
      f32x16 acc[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][i] = 0.f;
      if constexpr (kWhich == FMHA_MB_MFMA_E4M3) {
        i32x8 a8, b8;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a8[i] = 0x38383838 + lane;
          b8[i] = 0x30303030 + i;
        }
        for (int it = 0; it < iters; ++it)
#pragma unroll
          for (int r = 0; r < 32; ++r)
            acc[r & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, acc[r & 3], 0, 0,
                                                                         0, 127, 0, 127);
      } else {
        bf16x8 a, b;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          a[i] = (__bf16)(0.002f * i);
          b[i] = (__bf16)(0.001f * (lane + i));
        }
        for (int it = 0; it < iters; ++it)
#pragma unroll
          for (int r = 0; r < 32; ++r)
            acc[r & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[r & 3], 0, 0, 0);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) sink += acc[a][i];
    } else {
      // timed over its first `iters` iterations, then kept running as long
      // again, so that it overlaps the MFMA wave (about 1000 cycles per
      // iteration) for the whole of both measurements
      float x[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = 0.01f * (lane + i);
      sink = softmax_like(x, iters);
      t_stop = __builtin_amdgcn_s_memtime();
      sink += softmax_like(x, iters);
    }
  } else if constexpr (kWhich == FMHA_MB_SOFTMAX) {
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.01f * (lane + i);
    sink = softmax_like(x, iters);
  } else if constexpr (kWhich == FMHA_MB_LDS_B128 || kWhich == FMHA_MB_MFMA_LDS_B128) {
    // wave w reads the 16 KB window (w % 4) * 16 KB, lane l 16 bytes at
    // l * 16 + t * 1024 (a conflict-free pattern), shifted every iteration
    const int base = (wave & 3) * 16384;
    auto rd = [&](int t, int it) -> bf16x8 {
      return *(const bf16x8*)(lds + base + ((t * 1024 + lane * 16 + it * 16) & 16383));
    };
    if constexpr (kWhich == FMHA_MB_LDS_B128) {
      int xr = 0;
      for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int t = 0; t < 32; ++t) {
          const i32x4 v = __builtin_bit_cast(i32x4, rd(t, it));
          xr ^= v[0] ^ v[1] ^ v[2] ^ v[3];
        }
      sink = (float)xr;
    } else {
      // one 1 KB A operand per MFMA, read a whole set of 16 ahead (double
      // buffer), as the Q.K^T of a 32-row wave consumes them
      f32x16 acc[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][i] = 0.f;
      bf16x8 bq;
#pragma unroll
      for (int i = 0; i < 8; ++i) bq[i] = (__bf16)(0.001f * (lane + i));
      bf16x8 ka[2][16];
#pragma unroll
      for (int t = 0; t < 16; ++t) ka[0][t] = rd(t, 0);
      auto body = [&](bf16x8 (&use)[16], bf16x8 (&fill)[16], int it) {
#pragma unroll
        for (int t = 0; t < 16; ++t) fill[t] = rd(t, it + 1);
#pragma unroll
        for (int t = 0; t < 16; ++t)
          acc[t & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(use[t], bq, acc[t & 3], 0, 0, 0);
      };
      // one loop trip: two sets of 16 MFMAs, each set's reads issued during
      // the other's MFMAs (the last set read is not consumed)
      for (int it = 0; it < iters; ++it) {
        body(ka[0], ka[1], 2 * it);
        body(ka[1], ka[0], 2 * it + 1);
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int i = 0; i < 16; ++i) sink += acc[a][i];
    }
  }

  __builtin_amdgcn_s_waitcnt(0);
  const unsigned long long t1 = t_stop != 0 ? t_stop : __builtin_amdgcn_s_memtime();
  if (lane == 0) {
    Slot& s = out[blockIdx.x * kMaxWaves + wave];
    s.cycles = t1 - t0;
    s.sink = sink;
  }
}

// Instructions (or operations) of the measured kind one wave issues per
// iteration of its timed loop.
double ops_per_iteration(int which) {
  switch (which) {
    case FMHA_MB_EXP2:
    case FMHA_MB_FMA:
    case FMHA_MB_CVT_BF16:
    case FMHA_MB_CVT_E4M3:
    case FMHA_MB_CVT_E2M1:
    case FMHA_MB_EXP2_E4M3:
    case FMHA_MB_EXP2_POLY:
    case FMHA_MB_EXP2_WITH_FMA:
      return 8.0 * kChains;
    case FMHA_MB_MFMA_BF16:
    case FMHA_MB_MFMA_E4M3:
    case FMHA_MB_MFMA_WITH_VALU:
      return 32.0;
    case FMHA_MB_LDS_B128:
      return 32.0;
    case FMHA_MB_MFMA_LDS_B128:
      return 32.0;  // two sets of 16 MFMAs, 16 reads each
    case FMHA_MB_SOFTMAX:
      return 1.0;   // cycles per iteration of the stream
    default:
      return 0.0;
  }
}

template <int kWhich>
hipError_t launch(Slot* out, int grid, int wps, int iters, int mfma_waves, hipStream_t s) {
  hipLaunchKernelGGL(microbench_kernel<kWhich>, dim3(grid), dim3(256 * wps), 0, s, out, iters,
                     mfma_waves);
  return hipGetLastError();
}

hipError_t launch_any(int which, Slot* out, int grid, int wps, int iters, int mfma_waves,
                      hipStream_t s) {
  switch (which) {
    case FMHA_MB_EXP2: return launch<FMHA_MB_EXP2>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_FMA: return launch<FMHA_MB_FMA>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_CVT_BF16: return launch<FMHA_MB_CVT_BF16>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_CVT_E4M3: return launch<FMHA_MB_CVT_E4M3>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_CVT_E2M1: return launch<FMHA_MB_CVT_E2M1>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_EXP2_E4M3:
      return launch<FMHA_MB_EXP2_E4M3>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_MFMA_BF16: return launch<FMHA_MB_MFMA_BF16>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_MFMA_E4M3: return launch<FMHA_MB_MFMA_E4M3>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_LDS_B128: return launch<FMHA_MB_LDS_B128>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_MFMA_LDS_B128:
      return launch<FMHA_MB_MFMA_LDS_B128>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_MFMA_WITH_VALU:
      return launch<FMHA_MB_MFMA_WITH_VALU>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_SOFTMAX: return launch<FMHA_MB_SOFTMAX>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_EXP2_POLY:
      return launch<FMHA_MB_EXP2_POLY>(out, grid, wps, iters, mfma_waves, s);
    case FMHA_MB_EXP2_WITH_FMA:
      return launch<FMHA_MB_EXP2_WITH_FMA>(out, grid, wps, iters, mfma_waves, s);
    default: return hipErrorInvalidValue;
  }
}

double median(std::vector<double> v) {
  if (v.empty()) return 0.0;
  std::sort(v.begin(), v.end());
  return v[v.size() / 2];
}

}  // namespace

extern "C" {

int32_t fmha_microbench_run(int32_t which, int32_t waves_per_simd, int32_t iters,
                            double* result) {
  if (result == nullptr || which < 0 || which >= FMHA_MB_COUNT || waves_per_simd < 1 ||
      waves_per_simd > 4 || iters < 1 || iters > (1 << 20))
    return 1;
  if (which == FMHA_MB_MFMA_WITH_VALU && waves_per_simd != 2) return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 3;
  const int grid = cus;
  const int mfma_waves = 1;  // MFMA_WITH_VALU: SIMD wave 0 runs MFMAs, wave 1 the vector stream
  Slot* d_out = nullptr;
  const size_t bytes = sizeof(Slot) * (size_t)grid * kMaxWaves;
  if (hipMalloc(&d_out, bytes) != hipSuccess) return 3;
  int status = 0;
  std::vector<Slot> h((size_t)grid * kMaxWaves);
  // a warm-up launch (code load, clock ramp), then the measured one
  for (int rep = 0; rep < 2 && status == 0; ++rep) {
    if (hipMemset(d_out, 0, bytes) != hipSuccess ||
        launch_any(which, d_out, grid, waves_per_simd, iters, mfma_waves, nullptr) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
      status = 3;
  }
  if (status == 0 && hipMemcpy(h.data(), d_out, bytes, hipMemcpyDeviceToHost) != hipSuccess)
    status = 3;
  (void)hipFree(d_out);
  if (status != 0) return status;
  const int waves = 4 * waves_per_simd;
  const double trips = (double)iters;
  const double per_trip = ops_per_iteration(which);
  std::vector<double> primary, secondary;
  for (int b = 0; b < grid; ++b)
    for (int w = 0; w < waves; ++w) {
      const double cyc = (double)h[(size_t)b * kMaxWaves + w].cycles;
      const bool valu_wave = which == FMHA_MB_MFMA_WITH_VALU && (w >> 2) >= mfma_waves;
      if (valu_wave)
        secondary.push_back(cyc / trips);            // cycles per softmax-like iteration
      else
        primary.push_back(cyc / (trips * per_trip)); // cycles per instruction
    }
  result[0] = median(primary);
  result[1] = median(secondary);
  return 0;
}

}  // extern "C"
