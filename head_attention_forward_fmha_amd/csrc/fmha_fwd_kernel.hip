// FMHA forward kernels for gfx950 (MI355X, CDNA4).
//
// What is computed: per document and head, O = softmax(scale * Q K^T) V with
// optional bottom-right causal masking, plus LSE = ln sum exp(scale * q.k).
// The pages ("[BUG] Unexpected Slower Performance in C++ CuTe
// (77_blackwell_fmha) vs Python CuTe DSL (fmha.py) on Jetson Thor", Key
// Observation 2; "Kernel Bottleneck Tuning", section 4) describe the method as
// tiled Q.K^T, an online softmax in the exp2 domain whose scale and running row
// maximum are folded into one fused multiply-add, then P.V with fp32
// accumulation. The design below is written for CDNA4 rather than taken from
// the Blackwell kernels those pages discuss.
//
// Work decomposition. One workgroup = 4 waves = 128 query rows of one
// (document, head); each wave owns 32 query rows. The 1-D grid is remapped so
// that each XCD (workgroups are dealt to the 8 XCDs round-robin) runs one
// contiguous range of (document, head) pairs with all their query blocks,
// longest causal block first: the blocks that stream the same K/V run together
// on one XCD and share its L2.
//
// Orientation. Both products are computed transposed so that every lane owns
// one query column of the MFMA result:
//   S^T[key, query] = K . Q^T   (v_mfma_f32_32x32x16_bf16, A = K rows from
//                                LDS, B = Q held in registers)
//   O^T[d, query]  += V^T . P^T (A = V read from LDS with ds_read_b64_tr_b16,
//                                B = P straight from the S^T accumulators)
// A lane (half h = lane/32, column n = lane%32) holds 16 keys of each 32-key
// S^T block for query n. The row max and row sum are therefore in-lane
// reductions plus one v_permlane32_swap between lanes n and n+32, and the
// online-softmax rescale of O is a per-lane scalar. The key order in which P
// leaves the accumulator is matched by the rows each tr16 read fetches.
//
// K/V streaming. K and V tiles of 64 keys are copied HBM -> LDS with
// global_load_lds_dwordx4 (no VGPR staging) into a double buffer; tile j+1 is
// in flight while tile j is computed. Rows are XOR-swizzled in 16-byte chunks
// (see swz) so that both the 16-byte K reads and the 8-byte transposed V reads
// spread over all 64 banks.
// Key rows past the end of a document are clamped to its last row; their
// scores are masked to -inf, so they contribute exactly zero.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fmha_kernel_params.h"

namespace fmha {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBM = kWaves * 32;  // query rows per workgroup
constexpr int kBN = 64;           // keys per K/V tile
constexpr int kXcds = 8;          // accelerator complex dies of an MI355X
// fp8 P.V: P is quantised as e4m3(2^8 * p); 2^8 is the largest power of two
// not above e4m3's maximum 448, so p = 1 maps exactly and small p stay normal.
constexpr float kPScaleLog2 = 8.f;

// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second. With both operands holding x, the two results are
// [x_lo, x_lo] and [x_hi, x_hi], so combining them all-reduces lanes n, n+32.
// The results pass through an empty asm: without it the optimiser folds
// fmaxf/fadd of the two float results into the first result alone.
__device__ __forceinline__ void half_swap(float x, float& lo, float& hi) {
  const int a = __builtin_bit_cast(int, x);
  auto r = __builtin_amdgcn_permlane32_swap(a, a, false, false);
  int r0 = r[0], r1 = r[1];
  asm volatile("" : "+v"(r0), "+v"(r1));
  lo = __builtin_bit_cast(float, r0);
  hi = __builtin_bit_cast(float, r1);
}

__device__ __forceinline__ float wave_half_swap_max(float x) {
  float lo, hi;
  half_swap(x, lo, hi);
  return fmaxf(lo, hi);
}

__device__ __forceinline__ float wave_half_swap_sum(float x) {
  float lo, hi;
  half_swap(x, lo, hi);
  return lo + hi;
}

// Bank-spreading swizzle of 16-byte chunks: chunk c of row r is stored at
// c ^ swz(r). The LDS has 64 4-byte banks (256 bytes). Requirements:
//  * 16 consecutive rows read at one logical chunk (the 16-byte K operand
//    reads) must land on 16 distinct bank groups;
//  * the transposed V reads fetch 4 consecutive rows x 4 consecutive chunks
//    (bf16) or 8 rows x 2 chunks (fp8) per half-wave, which must also be
//    spread over all banks.
// For 256-byte rows (16 chunks) the low two row bits select the high two chunk
// bits; for 128-byte rows (8 chunks, two rows per bank sweep) row bit 1 selects
// chunk bit 2 and row bits 2-3 the low two chunk bits.
template <int kChunksPerRow>
__device__ __forceinline__ int swz(int row) {
  static_assert(kChunksPerRow == 16 || kChunksPerRow == 8, "rows are 128 or 256 bytes");
  if constexpr (kChunksPerRow == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// s_waitcnt immediate that waits until at most n vector-memory ops are in flight
// (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and
// lgkmcnt left at their maxima so they are not waited on).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// s_waitcnt immediate that waits for all LDS/scalar-memory ops (lgkmcnt = 0)
constexpr int waitcnt_lgkm0() { return 0xF | (0x3 << 14) | (0x7 << 4); }

// Buffer resource (V#) for raw byte-addressed loads: base, size in bytes, and
// the gfx9 raw-buffer format word. Loads at offsets >= num_bytes return zero,
// which is how rows past the end of a document are filled.
__device__ __forceinline__ i32x4 make_buffer_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)num_bytes);
  r[3] = 0x00020000;                                                  // 32-bit data format
  return r;
}

// HBM -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane l
// writes LDS bytes [lds + 16*l, lds + 16*l + 16). Written as inline asm so that
// the compiler does not serialise it against unrelated LDS reads; the kernel
// orders it explicitly with s_waitcnt vmcnt + s_barrier. m0 is reserved by the
// compiler and never holds a live value in these kernels.
__device__ __forceinline__ void lds_dma_16(uint32_t lds_addr, int voffset, i32x4 rsrc,
                                           int soffset) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_addr), "v"(voffset), "s"(rsrc), "s"(soffset)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const LDS_AS char*)(const char*)p);
}

// Compiler-only fence: keeps LDS accesses on their side of a barrier.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

template <int kD, bool kCausal, bool kFp8>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void fmha_fwd_kernel(FwdParams p) {
  constexpr int kRowBytes = kD * 2;              // one K row in bytes
  constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per K row
  constexpr int kTileBytes = kBN * kRowBytes;    // one K tile
  constexpr int kLoadsPerWave = kTileBytes / (kThreads * 16);
  constexpr int kVRowBytes = kFp8 ? kD : kD * 2;  // one V row in bytes
  constexpr int kVChunks = kVRowBytes / 16;
  constexpr int kVTileBytes = kBN * kVRowBytes;
  constexpr int kVLoadsPerWave = kVTileBytes / (kThreads * 16);
  constexpr int kKSteps = kD / 16;               // QK^T MFMA steps over d
  constexpr int kDBlocks = kD / 32;              // O^T accumulator blocks
  constexpr int kKeyBlocks = kBN / 32;           // S^T accumulator blocks
  static_assert(kLoadsPerWave * kThreads * 16 == kTileBytes, "K tile must split into lane loads");
  static_assert(kVLoadsPerWave * kThreads * 16 == kVTileBytes, "V tile must split into lane loads");
  static_assert(!kFp8 || kBN == 64, "the fp8 P.V step consumes exactly one 64-key tile");

  __shared__ __attribute__((aligned(1024))) char smem_k[2][kTileBytes];   // [stage]
  __shared__ __attribute__((aligned(1024))) char smem_v[2][kVTileBytes];  // [stage]

  // ---- work item. Workgroups are dealt to the 8 XCDs round-robin (id % 8).
  // Work items are ordered (document, head)-major with query blocks inner,
  // longest (causal) block first, and each XCD takes one contiguous range of
  // them, so the query blocks sharing one K/V stream run together on one XCD
  // and hit in its L2.
  const int n_items = p.batch * p.heads * p.n_mblocks;
  const int wg = blockIdx.x;
  const int xcd = wg % kXcds;
  const int per = n_items / kXcds, extra = n_items % kXcds;
  const int item = xcd * per + min(xcd, extra) + wg / kXcds;
  const int pair = item / p.n_mblocks;
  const int mblock = p.n_mblocks - 1 - (item - pair * p.n_mblocks);
  const int doc = pair / p.heads;
  const int head = pair - doc * p.heads;

  int q_start, q_end, k_start, k_end;
  if (p.cu_q != nullptr) {
    q_start = p.cu_q[doc];
    q_end = p.cu_q[doc + 1];
    k_start = p.cu_k[doc];
    k_end = p.cu_k[doc + 1];
  } else {
    q_start = doc * p.max_seqlen_q;
    q_end = q_start + p.max_seqlen_q;
    k_start = doc * p.max_seqlen_k;
    k_end = k_start + p.max_seqlen_k;
  }
  const int sq = q_end - q_start;
  const int sk = k_end - k_start;
  const int m0 = mblock * kBM;
  if (m0 >= sq) return;  // uniform over the workgroup, before any barrier
  const int causal_off = sk - sq;

  int kend = sk;
  if (kCausal) kend = min(sk, max(0, m0 + kBM + causal_off));
  const int n_tiles = (kend + kBN - 1) / kBN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;    // query column of the MFMA result
  const int half = lane >> 5;   // which half of the 32-key block this lane holds
  const int row_stride = p.heads * kD;  // elements between consecutive tokens
  const int wave_q0 = m0 + wave * 32;   // first query row of this wave (in doc)
  const int qi = wave_q0 + col;         // this lane's query row (in doc)

  // ---- Q: the B operand of S^T = K Q^T, held in registers for the whole loop
  bf16x8 qreg[kKSteps];
  {
    const int qrow = q_start + min(qi, sq - 1);
    const bf16_t* qp = (const bf16_t*)p.q + (size_t)qrow * row_stride + head * kD + 8 * half;
#pragma unroll
    for (int t = 0; t < kKSteps; ++t) qreg[t] = *(const bf16x8*)(qp + 16 * t);
    // Q has landed before the K/V stream starts, so no wait on the stream's
    // vector-memory counter is ever needed for Q inside the tile loop
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }

  // ---- HBM -> LDS copy. Each wave copies 1 KB blocks: lane l lands at byte
  // 16*l of the block, so the swizzle is applied by choosing which global chunk
  // each lane fetches. Offsets are relative to this (document, head); rows past
  // the document end fall outside the buffer and arrive as zeros.
  const uint32_t k_stride = (uint32_t)p.heads * kRowBytes;   // bytes between K tokens
  const uint32_t v_stride = (uint32_t)p.heads * kVRowBytes;  // bytes between V tokens
  const i32x4 k_rsrc = make_buffer_rsrc(
      (const char*)p.k + (size_t)k_start * k_stride + head * kRowBytes, (uint32_t)sk * k_stride);
  const i32x4 v_rsrc = make_buffer_rsrc(
      (const char*)p.v + (size_t)k_start * v_stride + head * kVRowBytes, (uint32_t)sk * v_stride);
  int k_voff[kLoadsPerWave];
#pragma unroll
  for (int r = 0; r < kLoadsPerWave; ++r) {
    const int byte = 1024 * (r * kWaves + wave) + 16 * lane;
    const int row = byte / kRowBytes;
    const int phys = (byte % kRowBytes) / 16;
    k_voff[r] = row * (int)k_stride + (phys ^ swz<kChunks>(row)) * 16;
  }
  int v_voff[kVLoadsPerWave];
#pragma unroll
  for (int r = 0; r < kVLoadsPerWave; ++r) {
    const int byte = 1024 * (r * kWaves + wave) + 16 * lane;
    const int row = byte / kVRowBytes;
    const int phys = (byte % kVRowBytes) / 16;
    v_voff[r] = row * (int)v_stride + (phys ^ swz<kVChunks>(row)) * 16;
  }
  const uint32_t k_lds0 = lds_address(&smem_k[0][1024 * wave]);
  const uint32_t v_lds0 = lds_address(&smem_v[0][1024 * wave]);

  auto issue_tile = [&](int j, int stage) {
    const int kt0 = j * kBN;
#pragma unroll
    for (int r = 0; r < kLoadsPerWave; ++r)
      lds_dma_16(k_lds0 + stage * kTileBytes + 1024 * kWaves * r, k_voff[r], k_rsrc,
                 (int)((uint32_t)kt0 * k_stride));
#pragma unroll
    for (int r = 0; r < kVLoadsPerWave; ++r)
      lds_dma_16(v_lds0 + stage * kVTileBytes + 1024 * kWaves * r, v_voff[r], v_rsrc,
                 (int)((uint32_t)kt0 * v_stride));
  };

  // ---- softmax state (per lane = per query; lanes n and n+32 agree)
  const float c = p.scale_log2;       // softmax_scale * log2(e)
  // bf16 P tolerates p up to 2^8; e4m3 P already spends its range on the
  // 2^kPScaleLog2 scale, so the fp8 path keeps the exact running maximum.
  constexpr float kLazyLog2 = kFp8 ? 0.f : 8.f;
  float m_run = -__builtin_inff();    // running max of raw scores
  float l_run = 0.f;                  // running sum of exp2(c*(s - m_run))
  f32x16 oacc[kDBlocks];
#pragma unroll
  for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;

  // ---- per-lane LDS byte offsets of the MFMA operand reads, relative to a
  // stage's tile. Everything else in an address (stage, key block, 16-key step)
  // is a compile-time immediate, because the swizzle only looks at the low four
  // row bits and the stage is static in the unrolled loop below.
  const int g = lane >> 4;   // 16-lane group of the transposed reads
  const int gi = lane & 15;
  int k_off[kKSteps];        // K rows 32*kb + col, logical chunk 2t + half
#pragma unroll
  for (int t = 0; t < kKSteps; ++t)
    k_off[t] = col * kRowBytes + (((2 * t + half) ^ swz<kChunks>(col)) * 16);
  // bf16 V (tr16): rows 16*ks16 + 8r + 4*half + gi/4, d = 32*db + 16*(g&1) + 4*(gi&3)
  // fp8 V (tr8): rows 32*(r>>1) + 16*(r&1) + 8*(e>>2) + 4*half + (e&3), e = gi/2,
  //              byte column 32*db + 16*(g&1) + 8*(gi&1)
  constexpr int kVReads = kFp8 ? 1 : 2;
  int v_off[kVReads][kDBlocks];
#pragma unroll
  for (int r = 0; r < kVReads; ++r)
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) {
      if constexpr (!kFp8) {
        const int row = 8 * r + 4 * half + gi / 4;
        const int d = 32 * db + 16 * (g & 1) + 4 * (gi & 3);
        v_off[r][db] = row * kVRowBytes + (((d / 8) ^ swz<kVChunks>(row)) * 16) + (d % 8) * 2;
      } else {
        const int e = gi >> 1;
        const int row = 8 * (e >> 2) + 4 * half + (e & 3);
        const int byte_col = 32 * db + 16 * (g & 1) + 8 * (gi & 1);
        v_off[r][db] =
            row * kVRowBytes + (((byte_col / 16) ^ swz<kVChunks>(row)) * 16) + (byte_col % 16);
      }
    }

  // ---- one K/V tile: wait for it, S^T = K Q^T, mask, online softmax, O^T += V^T P^T
  auto step = [&](int j, auto stage_tag) {
    constexpr int stage = decltype(stage_tag)::value;
    // tile j has landed once only tile j+1's copies can still be in flight
    if (j + 1 < n_tiles) {
      issue_tile(j + 1, stage ^ 1);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoadsPerWave + kVLoadsPerWave));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __builtin_amdgcn_s_barrier();
    compiler_fence();

    const int kt0 = j * kBN;
    // tiles entirely above the diagonal for all 32 rows of this wave are skipped
    const bool wave_active = !kCausal || (kt0 <= wave_q0 + 31 + causal_off);
    if (wave_active) {
      const char* ks = smem_k[stage];
      const char* vs = smem_v[stage];

      // ---- S^T = K Q^T for 64 keys x 32 queries
      f32x16 sacc[kKeyBlocks];
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
      // K operands for step t+1 are read while step t's MFMAs run
      bf16x8 ka[2][kKeyBlocks];
      auto read_k = [&](int t, bf16x8* dst) {
#pragma unroll
        for (int kb = 0; kb < kKeyBlocks; ++kb)
          dst[kb] = *(const bf16x8*)(ks + k_off[t] + kb * 32 * kRowBytes);
      };
      read_k(0, ka[0]);
#pragma unroll
      for (int t = 0; t < kKSteps; ++t) {
        if (t + 1 < kKSteps) read_k(t + 1, ka[(t + 1) & 1]);
#pragma unroll
        for (int kb = 0; kb < kKeyBlocks; ++kb)
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t & 1][kb], qreg[t], sacc[kb], 0, 0, 0);
      }

      // ---- masking (only on the diagonal band and on the ragged key tail)
      const bool need_mask = (kt0 + kBN > sk) ||
                             (kCausal && (kt0 + kBN - 1 > wave_q0 + causal_off));
      if (need_mask) {
        const int lim = kCausal ? min(sk - 1, qi + causal_off) : sk - 1;
#pragma unroll
        for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kt0 + 32 * kb + (i / 4) * 8 + 4 * half + (i % 4);
            if (key > lim) sacc[kb][i] = -__builtin_inff();
          }
      }

      // ---- online softmax in the exp2 domain
      // A row's maximum in use (m_run) is only raised when the row sees a
      // score more than kLazyLog2 (base-2 units) above it; the O/l rescale pass
      // then runs for the wave, with alpha = 1 exactly on rows that were not
      // raised, so every row's arithmetic depends on its own scores only.
      // Otherwise p = exp2(c*s - c*m_run) stays <= 2^kLazyLog2. Any m gives
      // the same O and LSE in exact arithmetic; this only bounds p.
      // Four independent partial maxima keep the dependency chains short.
      float mp[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mp[i & 3] = fmaxf(mp[i & 3], sacc[kb][i]);
      float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
      mx = wave_half_swap_max(mx);
      // NaN when both are -inf (a row with nothing visible yet): no raise
      const bool raise = (mx - m_run) * c > kLazyLog2;
      if (__builtin_amdgcn_ballot_w64(raise) != 0) {
        // raise implies mx > m_run and mx finite; alpha = 0 when m_run = -inf
        const float alpha = raise ? __builtin_amdgcn_exp2f((m_run - mx) * c) : 1.f;
        m_run = raise ? mx : m_run;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      }
      // fold: p = exp2(s*c - m_run*c); an all-masked row keeps the fold finite.
      // fp8: P is produced pre-multiplied by 2^kPScaleLog2 inside the exponent.
      const float neg_mc = (m_run == -__builtin_inff()) ? 0.f : -m_run * c;
      const float p_add = kFp8 ? neg_mc + kPScaleLog2 : neg_mc;
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sacc[kb][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], c, p_add));

      // row sum from the fp32 values, four independent chains; l_run holds this
      // lane's half of the keys and the halves are added at the end
      {
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) rs[i & 3] += sacc[kb][i];
        l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
      }

      if constexpr (!kFp8) {
        // P in bf16 (round to nearest even) as the P.V operand
        bf16x8 pb[kBN / 16];
#pragma unroll
        for (int ks16 = 0; ks16 < kBN / 16; ++ks16)
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) pb[ks16][jj] = (bf16_t)sacc[ks16 / 2][8 * (ks16 % 2) + jj];

        // ---- O^T += V^T P^T, 16 keys per MFMA. Lane (half, m) needs
        // V[keys 16*ks16 + 8r + 4*half + 0..3][d = 32*db + m]; source lane gi of
        // group g reads 4 d-values of key row (.. + gi/4).
#pragma unroll
        for (int ks16 = 0; ks16 < kBN / 16; ++ks16)
#pragma unroll
          for (int db = 0; db < kDBlocks; ++db) {
            bf16x4 va[2];
#pragma unroll
            for (int r = 0; r < 2; ++r)
              va[r] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                  (LDS_AS bf16x4*)(vs + v_off[r][db] + 16 * ks16 * kVRowBytes));
            const bf16x8 a = {va[0][0], va[0][1], va[0][2], va[0][3],
                              va[1][0], va[1][1], va[1][2], va[1][3]};
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ks16], oacc[db], 0, 0, 0);
          }
      } else {
        // ---- O^T += V^T P^T in e4m3, all 64 keys of the tile in one MFMA per d block.
        // Byte j of a lane's operand is key kappa(half, j) =
        //   32*(j/16) + 8*((j%16)/4) + 4*half + j%4,
        // which is where the S^T accumulator left P; V is fetched to match.
        i32x8 pb;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const int kb = w / 4, i0 = 4 * (w % 4);
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[kb][i0], sacc[kb][i0 + 1], 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(sacc[kb][i0 + 2], sacc[kb][i0 + 3], word, true);
          pb[w] = word;
        }
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
          i32x8 a;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            // read r delivers bytes 8r..8r+7: keys 32*(r>>1) + 16*(r&1) + ...
            const auto t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (LDS_AS i32x2*)(vs + v_off[0][db] + (32 * (r >> 1) + 16 * (r & 1)) * kVRowBytes));
            a[2 * r] = t[0];
            a[2 * r + 1] = t[1];
          }
          oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb, oacc[db], 0, 0, 0, 127,
                                                                     0, 127);
        }
      }
    }
    // every wave's reads of this stage have returned before it is refilled
    __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
    __builtin_amdgcn_s_barrier();
    compiler_fence();
  };

  if (n_tiles > 0) issue_tile(0, 0);
  int j = 0;
  for (; j + 2 <= n_tiles; j += 2) {
    step(j, std::integral_constant<int, 0>());
    step(j + 1, std::integral_constant<int, 1>());
  }
  if (j < n_tiles) step(j, std::integral_constant<int, 0>());

  // ---- epilogue: O /= l, bf16 store; LSE = scale*m + ln(l)
  l_run = wave_half_swap_sum(l_run);
  if (qi < sq) {
    // fp8: O = v_scale * sum(P_hat V_codes) / l, where l carries the same 2^kPScaleLog2
    const float num_scale = kFp8 ? p.v_scale[head] : 1.f;
    const float inv_l = (l_run > 0.f) ? num_scale / l_run : 0.f;
    bf16_t* op = (bf16_t*)p.out + (size_t)(q_start + qi) * row_stride + head * kD;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int d0 = 32 * db + 8 * ig + 4 * half;
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (bf16_t)(oacc[db][4 * ig + e] * inv_l);
        *(bf16x4*)(op + d0) = o4;
      }
    if (p.lse != nullptr && half == 0) {
      float lse = -__builtin_inff();
      const float lsub = kFp8 ? kPScaleLog2 : 0.f;
      if (l_run > 0.f)
        lse = (m_run * c + (__builtin_amdgcn_logf(l_run) - lsub)) * 0.69314718055994531f;
      p.lse[(size_t)head * p.total_q + q_start + qi] = lse;
    }
  }
}

template <int kD, bool kCausal, bool kFp8>
static hipError_t launch(const FwdParams& p, hipStream_t stream) {
  FwdParams q = p;
  q.n_mblocks = (p.max_seqlen_q + kBM - 1) / kBM;
  const long long n_items = (long long)q.n_mblocks * p.heads * p.batch;
  if (n_items == 0) return hipSuccess;
  if (n_items > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fmha_fwd_kernel<kD, kCausal, kFp8>), dim3((unsigned)n_items), dim3(kThreads),
                     0, stream, q);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, bool causal, hipStream_t stream) {
  if (head_dim == 128)
    return causal ? launch<128, true, false>(p, stream) : launch<128, false, false>(p, stream);
  return causal ? launch<64, true, false>(p, stream) : launch<64, false, false>(p, stream);
}

hipError_t launch_fwd_fp8pv(const FwdParams& p, int head_dim, bool causal, hipStream_t stream) {
  if (head_dim != 128) return hipErrorInvalidValue;
  return causal ? launch<128, true, true>(p, stream) : launch<128, false, true>(p, stream);
}

}  // namespace fmha
