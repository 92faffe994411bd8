// Device-side building blocks of the gfx950 FMHA forward kernels.
//
// The operation (pages: "[BUG] Unexpected Slower Performance in C++ CuTe
// (77_blackwell_fmha) vs Python CuTe DSL (fmha.py) on Jetson Thor", Key
// Observation 2, the softmax_step listings; "Kernel Bottleneck Tuning",
// section 4): per document and head, S = scale * Q K^T, an online softmax in
// the exp2 domain with the scale and the running row maximum folded into one
// fused multiply-add, P.V with fp32 accumulation, and an epilogue that
// normalises O and writes LSE.
//
// Orientation. Both products are computed transposed so that every lane owns
// one query column of the MFMA result:
//   S^T[key, query] = K . Q^T   (v_mfma_f32_32x32x16_bf16, A = K rows from
//                                LDS, B = Q held in registers)
//   O^T[d, query]  += V^T . P^T (A = V read from LDS with ds_read_b64_tr_b16,
//                                _tr_b8 for e4m3 V or _tr_b4 for e2m1 V; B = P
//                                straight from the S^T accumulators)
// A lane (half = lane/32, column n = lane%32) holds 16 keys of each 32-key S^T
// block for query n: keys 8*(i/4) + 4*half + i%4 of accumulator register i.
// The row max and row sum are in-lane reductions plus one v_permlane32_swap
// between lanes n and n+32, and the online-softmax rescale of O is a per-lane
// scalar. The transposed V reads fetch exactly the key order in which P leaves
// the accumulator.
//
// LDS layout. K and V tiles are row-major [key][d] with 16-byte chunks
// XOR-swizzled per row (swz) so that the 16-byte K operand reads and the 8-byte
// transposed V reads both spread over all 64 banks. Tiles are copied
// HBM -> LDS by buffer_load_dwordx4 ... lds, which needs no VGPR staging and
// returns zeros for rows past the end of a document.

#ifndef FMHA_DEVICE_H_
#define FMHA_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fmha_kernel_params.h"

namespace fmha {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int kBN = 64;     // keys per K/V tile
constexpr int kXcds = 8;    // accelerator complex dies of an MI355X
// fp8 P.V: P is quantised as e4m3(2^(c s - A + 5)) with A a running anchor in
// exp2 units (softmax_e4m3), so a key at the anchor scales to 2^5 and the lazy
// raise has a factor 14 of headroom under e4m3's maximum 448; values down to
// 2^-11 of the anchor stay in e4m3's normal range.
constexpr float kPScaleLog2 = 5.f;
constexpr float kE4m3Max = 448.f;

// ---------------------------------------------------------------- primitives

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
// chunk bit 2 and row bits 2-3 the low two chunk bits. For 64-byte rows (e2m1
// V, 4 chunks, four rows per bank sweep) the transposed reads of a half-wave
// fetch rows 8a + b (a, b = 0..3) at one chunk: row bits 0-1 already spread
// them over the sweep, and row bits 3-4 pick the chunk. Only the low five row
// bits matter, so the swizzle repeats every 32 rows.
template <int kChunksPerRow>
__device__ __forceinline__ int swz(int row) {
  static_assert(kChunksPerRow == 16 || kChunksPerRow == 8 || kChunksPerRow == 4,
                "rows are 64, 128 or 256 bytes");
  if constexpr (kChunksPerRow == 16) return ((row & 3) << 2) | ((row >> 2) & 3);
  if constexpr (kChunksPerRow == 4) return (row >> 3) & 3;
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// s_waitcnt immediate that waits until at most n vector-memory ops are in flight
// (gfx9 encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14; expcnt and
// lgkmcnt left at their maxima so they are not waited on).
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }
// s_waitcnt immediate that waits for all LDS/scalar-memory ops (lgkmcnt = 0)
constexpr int waitcnt_lgkm0() { return 0xF | (0x3 << 14) | (0x7 << 4); }

// Buffer resource (V#) for raw byte-addressed loads: base, size in bytes, and
// the gfx9 raw-buffer format word. Loads whose per-lane offset (plus the
// instruction's immediate offset) is >= num_bytes return zero, which is how
// rows past the end of a document are filled; the copies keep the scalar
// offset at zero, so every byte address is covered by that check.
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
// the compiler does not serialise it against unrelated LDS reads; the kernels
// order it explicitly with s_waitcnt vmcnt + s_barrier. The asm writes m0 and,
// through s_add_u32, the scalar condition code; both are declared clobbered, as
// the copies sit between compiler-generated branches.
template <int kLdsOffset>
__device__ __forceinline__ void lds_dma_16(uint32_t lds_base, int voffset, i32x4 rsrc,
                                           int soffset) {
  // m0 = lds_base + kLdsOffset is formed here, so that only the base stays live
  // in a scalar register across the loop
  asm volatile(
      "s_add_u32 m0, %0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_base), "v"(voffset), "s"(rsrc), "s"(soffset), "n"(kLdsOffset)
      : "memory", "scc", "m0");
}

// HBM -> LDS copy of 4 bytes per active lane from a per-lane address
// (global_load_lds_dword): lane l writes LDS bytes [lds + 4*l, lds + 4*l + 4).
// It needs no buffer descriptor in scalar registers; the caller keeps src in
// bounds. Ordered like lds_dma_16.
__device__ __forceinline__ void lds_dma_global_4(uint32_t lds_base, const void* src) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off"
      :
      : "s"(lds_base), "v"(src)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const LDS_AS char*)(const char*)p);
}

// Compiler-only fence: keeps LDS accesses on their side of a barrier.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  [&]<int... I>(std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>()), ...);
  }(std::make_integer_sequence<int, N>());
}

// Wait for every outstanding LDS read, then the workgroup barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(waitcnt_lgkm0());
  __builtin_amdgcn_s_barrier();
  compiler_fence();
}

// ---------------------------------------------------------------- work items

// A (document, head, query block). Keys [k_start, k_start + sk) of the packed
// tensor are the document's, of which those before k_start + key_lo are
// hidden (key_lo > 0 only after align_keys_to_blocks).
struct WorkItem {
  int head, q_start, k_start, sq, sk, m0, key_lo;
};

// The fp4 P.V path keeps its key tiles on the 32-token blocks of the packed
// tensor, which carry V's scales and form P's quantisation groups: a document
// that starts inside a block is widened to the block start, and the extra
// leading keys are masked. The causal offset sk - sq grows by the same amount,
// so every query still sees the same keys.
__device__ __forceinline__ void align_keys_to_blocks(WorkItem& w) {
  const int r = w.k_start & 31;
  w.k_start -= r;
  w.sk += r;
  w.key_lo = r;
}

// Work items are the (document, head, query block) triples, ordered
// (document, head)-major with query blocks inner, longest causal block first,
// and split into kXcds contiguous ranges, one per XCD. Workgroups are dealt to
// the XCDs round-robin (id % kXcds), so the query blocks that stream the same
// K/V run together on one XCD and share its L2.
//
// The kernels are persistent: the launcher sizes the grid to what the chip
// holds at once (a multiple of kXcds), and the W workgroups of an XCD walk its
// range in rounds of W items, alternating direction every round, so that a
// workgroup that drew a long causal block in one round draws a short one in
// the next and the XCD finishes evenly.
struct ItemCursor {
  int start, count, per_xcd, lane, round;
  __device__ __forceinline__ explicit ItemCursor(int n_items) {
    const int xcd = blockIdx.x % kXcds;
    const int per = n_items / kXcds, extra = n_items % kXcds;
    start = xcd * per + min(xcd, extra);
    count = per + (xcd < extra ? 1 : 0);
    per_xcd = gridDim.x / kXcds;
    lane = blockIdx.x / kXcds;
    round = 0;
  }
  // the next item of this workgroup; false when its share is done
  __device__ __forceinline__ bool next(int& item) {
    while (round * per_xcd < count) {
      const int pos = round * per_xcd + ((round & 1) ? per_xcd - 1 - lane : lane);
      ++round;
      if (pos < count) {
        item = start + pos;
        return true;
      }
    }
    return false;
  }
};

// Runs f(p, item) for this workgroup's work items. Persistent launches
// (kPersistent) walk the XCD's range with an ItemCursor, re-reading the
// parameters per item (kernel_params); the others take the single item their
// block index names, with the same XCD-contiguous numbering. Split-KV launches
// (kSplit) have num_splits items per (document, head, query block), adjacent.
template <bool kPersistent, bool kSplit, typename F>
__device__ __forceinline__ void for_each_item(const FwdParams& params, F&& f);

template <bool kSplit>
__device__ __forceinline__ int n_work_items(const FwdParams& p) {
  const int n = p.batch * p.heads * p.n_mblocks;
  if constexpr (kSplit) return n * p.num_splits;
  return n;
}

// The kernel's own FwdParams argument, read from the kernel-argument segment.
// The persistent kernels fetch it afresh for every work item: the pointer passes
// through an empty asm, so the compiler reloads the (invariant) fields where it
// needs them instead of keeping all of them in scalar registers across the loop.
__device__ __forceinline__ const FwdParams& kernel_params() {
  const FwdParams* q = (const FwdParams*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(q));
  return *q;
}

__device__ __forceinline__ WorkItem decode_work_item(const FwdParams& p, int bm, int item) {
  const int pair = item / p.n_mblocks;
  const int mblock = p.n_mblocks - 1 - (item - pair * p.n_mblocks);
  const int doc = pair / p.heads;
  WorkItem w;
  w.head = pair - doc * p.heads;
  int q_end, k_end;
  if (p.cu_q != nullptr) {
    w.q_start = p.cu_q[doc];
    q_end = p.cu_q[doc + 1];
    w.k_start = p.cu_k[doc];
    k_end = p.cu_k[doc + 1];
  } else {
    w.q_start = doc * p.max_seqlen_q;
    q_end = w.q_start + p.max_seqlen_q;
    w.k_start = doc * p.max_seqlen_k;
    k_end = w.k_start + p.max_seqlen_k;
  }
  w.sq = q_end - w.q_start;
  w.sk = k_end - w.k_start;
  w.m0 = mblock * bm;
  w.key_lo = 0;
  return w;
}

template <bool kPersistent, bool kSplit, typename F>
__device__ __forceinline__ void for_each_item(const FwdParams& params, F&& f) {
  if constexpr (kPersistent) {
    ItemCursor cursor(n_work_items<kSplit>(params));
    int item;
    // Items follow each other without a workgroup barrier: every tile loop
    // ends behind an LDS barrier (all reads of its stages done), and an
    // epilogue touches only LDS blocks that the same wave refills first, so
    // the next item's first copies cannot overwrite anything still read, and
    // the previous item's output stores drain while the next item's loads are
    // in flight.
    while (cursor.next(item)) f(kernel_params(), item);
  } else {
    const int n_items = n_work_items<kSplit>(params);
    const int xcd = blockIdx.x % kXcds;
    const int per = n_items / kXcds, extra = n_items % kXcds;
    f(params, xcd * per + min(xcd, extra) + (int)blockIdx.x / kXcds);
  }
}

// ---------------------------------------------------------------- per-wave tile math

// One wave's view of the forward pass: 32 query rows, Q in registers, the
// running softmax state and the O^T accumulators. kWaves is the number of waves
// that copy a tile (it sets how the K/V copies are split among them); kPv is
// the number format of P.V (kPvBf16, kPvE4m3 or kPvE2m1).
template <int kD, bool kCausal, int kPv, int kWaves>
struct WaveTile {
  static constexpr bool kFp8 = kPv == kPvE4m3;
  static constexpr bool kFp4 = kPv == kPvE2m1;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kRowBytes = kD * 2;               // one K row in bytes
  static constexpr int kChunks = kRowBytes / 16;         // 16-byte chunks per K row
  static constexpr int kTileBytes = kBN * kRowBytes;     // one K tile
  static constexpr int kLoadsPerWave = kTileBytes / (kThreads * 16);
  static constexpr int kVRowBytes = kFp4 ? kD / 2 : (kFp8 ? kD : kD * 2);  // one V row
  static constexpr int kVChunks = kVRowBytes / 16;
  static constexpr int kVTileBytes = kBN * kVRowBytes;
  static constexpr int kVLoadsPerWave = kVTileBytes / (kThreads * 16);
  // e2m1 V: the tile's E8M0 exponents, [2 blocks of 32 keys][kD], follow its
  // codes in the same LDS stage; every copying wave fetches all of them (one
  // 4-byte load per lane), writing identical bytes
  static constexpr int kVScaleBytes = kFp4 ? 2 * kD : 0;
  static constexpr int kVStageBytes = kVTileBytes + kVScaleBytes;
  // vector-memory instructions one wave issues to copy a V tile
  static constexpr int kVCopyOps = kVLoadsPerWave + (kFp4 ? 1 : 0);
  static constexpr float kLog2Six = 2.5849625007211562f;   // log2 of e2m1's largest value
  static constexpr int kKSteps = kD / 16;                // QK^T MFMA steps over d
  static constexpr int kDBlocks = kD / 32;               // O^T accumulator blocks
  static constexpr int kKeyBlocks = kBN / 32;            // S^T accumulator blocks
  static constexpr int kVReads = kFp8 ? 1 : 2;
  // bf16 P tolerates p up to 2^8 (lazy maximum); e4m3 P up to its largest
  // finite value (kE4m3Max), with the stepped anchor of softmax_e4m3.
  static constexpr float kLazyLimit = 256.f;  // 2^8: largest p the bf16 path allows
  static_assert(kLoadsPerWave >= 1 && kLoadsPerWave * kThreads * 16 == kTileBytes,
                "K tile must split into whole lane loads");
  static_assert(kVLoadsPerWave >= 1 && kVLoadsPerWave * kThreads * 16 == kVTileBytes,
                "V tile must split into whole lane loads");
  static_assert((!kFp8 && !kFp4) || kBN == 64,
                "the fp8 and fp4 P.V steps consume exactly one 64-key tile");
  static_assert(!kFp4 || kVScaleBytes == 64 * 4, "the exponent image is one 4-byte load per lane");

  // identity
  int lane, col, half, g, gi;
  int wave_q0, qi;       // first query row of this wave / this lane's row (in doc)
  // operands and state
  bf16x8 qreg[kKSteps];
  f32x16 oacc[kDBlocks];
  f32x16 sacc[kKeyBlocks];
  bf16x8 pb[kBN / 16];   // bf16 P of the last softmaxed tile
  i32x8 pb8;             // e4m3 P of the last softmaxed tile
  i32x4 pb4;             // e2m1 P of the last softmaxed tile (32 keys per lane)
  int p_scale;           // its E8M0 group scale for this lane's 32 keys
  float m_run, l_run, c;
  float m_log2;          // e4m3: running anchor; e2m1: integer running maximum (exp2 units)
  int key_lo;            // keys before this are hidden (block-aligned fp4 tiles)
  // per-lane LDS byte offsets of the operand reads within a stage's tile: one
  // per K step, and one per V read and d block. The swizzle only permutes
  // chunk bits that the d block index occupies, so block db's offset is block
  // 0's ^ (kVBlockXor * db).
  static constexpr int kVBlockXor = kFp4 ? 16 : (kFp8 ? 32 : 64);
  int k_off[kKSteps];
  int v_off[kVReads][kDBlocks];
  // HBM -> LDS copy
  i32x4 k_rsrc, v_rsrc;
  uint32_t k_stride, v_stride;
  // Per-lane offset of this wave's first copy instruction of a K (V) tile.
  // Instruction r of the tile reads kCopyRowsK * r rows further on, a step the
  // swizzle does not see (it reads only lower row bits), so its offset is
  // k_copy0 + r * kCopyRowsK * k_stride: the difference is uniform and joins
  // the tile's scalar offset.
  static constexpr int kCopyRowsK = 1024 * kWaves / kRowBytes;
  static constexpr int kCopyRowsV = 1024 * kWaves / kVRowBytes;
  int k_copy0, v_copy0;
  const unsigned char* vs_base;  // e2m1 V exponents: (document start block, head), uniform
  uint32_t vs_stride;
  int vs_last, vs_lds_delta;      // last block (relative); image offset from lds_v0

  // Sets up one wave for work item w: rows 32*row_chunk .. +31 of the item's
  // block, copies split over kWaves waves with this one at index `wave`.
  __device__ __forceinline__ void init(const FwdParams& p, const WorkItem& w, int wave,
                                       int row_chunk) {
    init_lanes(p);
    begin_rows(w, row_chunk);
    load_q(p, w, qi);
    init_read_offsets();
    init_strides(p);
    set_copy_source(p, w);
    init_copy_offsets(wave);
  }

  // What stays the same for every work item of a launch: lane identity, the
  // operand read offsets within a stage, the per-lane copy offsets.
  __device__ __forceinline__ void init_wave(const FwdParams& p, int wave) {
    init_lanes(p);
    init_read_offsets();
    init_strides(p);
    init_copy_offsets(wave);
  }
  __device__ __forceinline__ void init_lanes(const FwdParams& p) {
    lane = threadIdx.x & 63;
    col = lane & 31;
    half = lane >> 5;
    g = lane >> 4;
    gi = lane & 15;
    c = p.scale_log2;
  }
  __device__ __forceinline__ void init_strides(const FwdParams& p) {
    k_stride = (uint32_t)p.heads * kRowBytes;
    v_stride = (uint32_t)p.heads * kVRowBytes;
    if constexpr (kFp4) vs_stride = (uint32_t)p.heads * kD;
  }
  __device__ __forceinline__ void init_read_offsets() {
    // operand read offsets. K rows 32*kb + col at logical chunk 2t + half.
    // bf16 V (tr16): rows 16*ks16 + 8r + 4*half + gi/4, d = 32*db + 16*(g&1) + 4*(gi&3).
    // fp8 V (tr8): rows 32*(r>>1) + 16*(r&1) + 8*(e>>2) + 4*half + (e&3), e = gi/2,
    //              byte column 32*db + 16*(g&1) + 8*(gi&1).
    // fp4 V (tr4): rows 32*half + 8*(gi/4) + 4r + gi%4, byte column 16*db + 8*(g&1)
    //              (d = 32*db + 16*(g&1) + 0..15).
    // Key block, 16-key step and read index only add multiples of 16 rows,
    // which the swizzle ignores, so they are immediates at the read sites.
#pragma unroll
    for (int t = 0; t < kKSteps; ++t)
      k_off[t] = col * kRowBytes + (((2 * t + half) ^ swz<kChunks>(col)) * 16);
#pragma unroll
    for (int r = 0; r < kVReads; ++r) {
      if constexpr (kFp4) {
        const int row = 32 * half + 8 * (gi >> 2) + 4 * r + (gi & 3);
        v_off[r][0] = row * kVRowBytes + ((0 ^ swz<kVChunks>(row)) * 16) + 8 * (g & 1);
      } else if constexpr (!kFp8) {
        const int row = 8 * r + 4 * half + gi / 4;
        const int d = 16 * (g & 1) + 4 * (gi & 3);
        v_off[r][0] = row * kVRowBytes + (((d / 8) ^ swz<kVChunks>(row)) * 16) + (d % 8) * 2;
      } else {
        const int e = gi >> 1;
        const int row = 8 * (e >> 2) + 4 * half + (e & 3);
        const int byte_col = 16 * (g & 1) + 8 * (gi & 1);
        v_off[r][0] =
            row * kVRowBytes + (((byte_col / 16) ^ swz<kVChunks>(row)) * 16) + (byte_col % 16);
      }
#pragma unroll
      for (int db = 1; db < kDBlocks; ++db) v_off[r][db] = v_off[r][0] ^ (kVBlockXor * db);
    }
  }

  // HBM -> LDS copy. Each wave copies 1 KB blocks: lane l lands at byte 16*l
  // of the block, so the swizzle is applied by choosing which global chunk
  // each lane fetches. Offsets are relative to the item's (document, head);
  // rows past the document end fall outside the buffer and arrive as zeros.
  __device__ __forceinline__ void init_copy_offsets(int wave) {
    {
      const int byte = 1024 * wave + 16 * lane;
      const int row = byte / kRowBytes;
      const int phys = (byte % kRowBytes) / 16;
      k_copy0 = row * (int)k_stride + (phys ^ swz<kChunks>(row)) * 16;
    }
    {
      const int byte = 1024 * wave + 16 * lane;
      const int row = byte / kVRowBytes;
      const int phys = (byte % kVRowBytes) / 16;
      v_copy0 = row * (int)v_stride + (phys ^ swz<kVChunks>(row)) * 16;
    }
    if constexpr (kFp4) {
      static_assert(!kFp4 || kD == 128, "the exponent image is [2][128]");
      vs_lds_delta = kVTileBytes - 1024 * wave;
    }
  }

  // The row state of work item w: this wave's rows, an empty running softmax,
  // O = 0. Everything the item's softmax and epilogue read.
  __device__ __forceinline__ void begin_rows(const WorkItem& w, int row_chunk) {
    wave_q0 = w.m0 + 32 * row_chunk;
    qi = wave_q0 + col;
    m_run = -__builtin_inff();
    m_log2 = -__builtin_inff();
    l_run = 0.f;
    key_lo = w.key_lo;
    if constexpr (kFp4) key_lo = __builtin_amdgcn_readfirstlane(key_lo);
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  }

  // The copy state of work item w (buffer descriptors of its K and V, the e2m1
  // exponent rows) and the loads of its Q rows: everything the item's copies
  // and Q.K^T read. A kernel may call this for the next item once the current
  // one has issued its last copy and run its last Q.K^T.
  __device__ __forceinline__ void begin_copies(const FwdParams& p, const WorkItem& w,
                                               int row_chunk) {
    load_q(p, w, w.m0 + 32 * row_chunk + col);
    set_copy_source(p, w);
  }
  // Q: the B operand of S^T = K Q^T, held in registers for the item's tile
  // loop; this lane's row is `row` of the document (clamped to its last row)
  __device__ __forceinline__ void load_q(const FwdParams& p, const WorkItem& w, int row) {
    {
      const int row_stride = p.heads * kD;
      const int qrow = w.q_start + min(row, w.sq - 1);
      const bf16_t* qp = (const bf16_t*)p.q + (size_t)qrow * row_stride + w.head * kD + 8 * half;
#pragma unroll
      for (int t = 0; t < kKSteps; ++t) qreg[t] = *(const bf16x8*)(qp + 16 * t);
      // The kernels wait for Q (vmcnt 0) before their tile loops, after issuing
      // their first K/V copies, so the two HBM round trips overlap and no wait
      // on the stream's counter is ever needed for Q inside the loop.
    }
  }
  __device__ __forceinline__ void set_copy_source(const FwdParams& p, const WorkItem& w) {
    k_rsrc = make_buffer_rsrc((const char*)p.k + (size_t)w.k_start * k_stride + w.head * kRowBytes,
                              (uint32_t)w.sk * k_stride);
    v_rsrc = make_buffer_rsrc((const char*)p.v + (size_t)w.k_start * v_stride + w.head * kVRowBytes,
                              (uint32_t)w.sk * v_stride);
    // e2m1 V exponents: a tile's two 32-key blocks are rows k_start/32 + 2j and
    // + 2j + 1 of [blocks, heads, kD]; lane l copies bytes 4l .. 4l + 3 of the
    // tile's [2][kD] image (block half, d = 4*col .. 4*col + 3). A block past
    // the end of the array (only in a tile's masked tail, whose V codes read
    // as zeros) is replaced by the last block, so every read stays in bounds.
    if constexpr (kFp4) {
      const int blk0 = w.k_start / 32;
      const int n_blocks = (p.total_k + 31) / 32;
      vs_base = p.v_mx_scale + (size_t)blk0 * vs_stride + (size_t)w.head * kD;
      vs_last = max(n_blocks - 1 - blk0, 0);
    }
  }

  // Byte offset of a tile in the copy descriptors' buffers. It is uniform; the
  // persistent (causal) kernels and the fp4 ones say so explicitly, which keeps
  // it in a scalar register there (the buffer loads take it only from one).
  __device__ __forceinline__ static int scalar_offset(int off) {
    if constexpr (kCausal || kFp4) return __builtin_amdgcn_readfirstlane(off);
    return off;
  }

  // The copy descriptors are uniform by construction; readfirstlane tells the
  // compiler so, which keeps them in scalar registers (the buffer loads take
  // them only there).
  __device__ __forceinline__ void pin_copy_state() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k_rsrc[i] = __builtin_amdgcn_readfirstlane(k_rsrc[i]);
      v_rsrc[i] = __builtin_amdgcn_readfirstlane(v_rsrc[i]);
    }
    k_stride = __builtin_amdgcn_readfirstlane(k_stride);
    v_stride = __builtin_amdgcn_readfirstlane(v_stride);
    if constexpr (kFp4) {
      const uint64_t b = reinterpret_cast<uint64_t>(vs_base);
      vs_base = reinterpret_cast<const unsigned char*>(
          ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b));
      vs_stride = __builtin_amdgcn_readfirstlane(vs_stride);
      vs_last = __builtin_amdgcn_readfirstlane(vs_last);
    }
  }

  // This wave's share of the copy of K tile j into K stage kStage (lds_k0 is
  // the LDS address of this wave's first 1 KB block in stage 0): instruction r
  // of kLoadsPerWave, or all of them. V likewise.
  // The tile's byte offset goes into the per-lane offset, not the scalar one:
  // the raw-buffer range check that turns rows past the document end into
  // zeros is made on the per-lane offset, so every byte of the copy is checked
  // against the buffer's size.
  // `base` is a copy of k_copy0 (v_copy0) made where the tile's copy starts,
  // opaque to the compiler, so that the per-instruction sums are formed here
  // and not hoisted out of the tile loop into registers of their own.
  template <int kStage, int kR>
  __device__ __forceinline__ void copy_k_one(int j, uint32_t lds_k0, int base) {
    lds_dma_16<kStage * kTileBytes + 1024 * kWaves * kR>(
        lds_k0, base + scalar_offset((int)((uint32_t)(j * kBN + kR * kCopyRowsK) * k_stride)),
        k_rsrc, 0);
  }
  template <int kStage, int kR>
  __device__ __forceinline__ void copy_v_one(int j, uint32_t lds_v0, int base) {
    lds_dma_16<kStage * kVStageBytes + 1024 * kWaves * kR>(
        lds_v0, base + scalar_offset((int)((uint32_t)(j * kBN + kR * kCopyRowsV) * v_stride)),
        v_rsrc, 0);
  }
  // e2m1 V: tile j's exponent image (the same 256 bytes from every wave)
  template <int kStage>
  __device__ __forceinline__ void copy_v_scales(int j, uint32_t lds_v0) {
    const uint32_t base =
        __builtin_amdgcn_readfirstlane(lds_v0 + vs_lds_delta + kStage * kVStageBytes);
    const int rb = min(2 * j + half, vs_last);
    lds_dma_global_4(base, vs_base + (size_t)(uint32_t)rb * vs_stride + 4 * col);
  }
  template <int kStage>
  __device__ __forceinline__ void copy_k(int j, uint32_t lds_k0) {
    int base = k_copy0;
    asm volatile("" : "+v"(base));
    [&]<int... kR>(std::integer_sequence<int, kR...>) {
      (copy_k_one<kStage, kR>(j, lds_k0, base), ...);
    }(std::make_integer_sequence<int, kLoadsPerWave>());
  }
  template <int kStage>
  __device__ __forceinline__ void copy_v(int j, uint32_t lds_v0) {
    int base = v_copy0;
    asm volatile("" : "+v"(base));
    [&]<int... kR>(std::integer_sequence<int, kR...>) {
      (copy_v_one<kStage, kR>(j, lds_v0, base), ...);
    }(std::make_integer_sequence<int, kVLoadsPerWave>());
    if constexpr (kFp4) copy_v_scales<kStage>(j, lds_v0);
  }

  // Does any of this wave's rows see a key of tile j?
  __device__ __forceinline__ bool active(int j, int causal_off) const {
    return !kCausal || (j * kBN <= wave_q0 + 31 + causal_off);
  }

  // S^T = K Q^T for the 64 keys of the tile at ks (LDS, generic pointer).
  __device__ __forceinline__ void qk(const char* ks) {
#pragma unroll
    for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
    // K operands are read kPrefetch steps ahead of their MFMAs (a ring of
    // kPrefetch + 1 register sets), so the LDS latency hides behind the MFMAs
    // of the steps in between. The scheduling-group barriers keep the compiler
    // from pulling the reads back next to their uses.
    constexpr int kPrefetch = 2;
    bf16x8 ka[kPrefetch + 1][kKeyBlocks];
#pragma unroll
    for (int t = 0; t < kPrefetch && t < kKSteps; ++t)
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
        ka[t][kb] = *(const bf16x8*)(ks + k_off[t] + kb * 32 * kRowBytes);
#pragma unroll
    for (int t = 0; t < kKSteps; ++t) {
      if (t + kPrefetch < kKSteps) {
#pragma unroll
        for (int kb = 0; kb < kKeyBlocks; ++kb)
          ka[(t + kPrefetch) % (kPrefetch + 1)][kb] =
              *(const bf16x8*)(ks + k_off[t + kPrefetch] + kb * 32 * kRowBytes);
      }
#pragma unroll
      for (int kb = 0; kb < kKeyBlocks; ++kb)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % (kPrefetch + 1)][kb], qreg[t],
                                                            sacc[kb], 0, 0, 0);
    }
    // schedule: the first kPrefetch steps' reads, then per step its reads
    // for step t + kPrefetch followed by its MFMAs
    constexpr int kFirstReads = (kPrefetch < kKSteps ? kPrefetch : kKSteps) * kKeyBlocks;
    __builtin_amdgcn_sched_group_barrier(0x100, kFirstReads, 0);
#pragma unroll
    for (int t = 0; t < kKSteps; ++t) {
      if (t + kPrefetch < kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, kKeyBlocks, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, kKeyBlocks, 0);
    }
  }

  // Causal mask (key j visible to query i iff j <= i + sk - sq) and key tail
  // (j < sk), on tiles that need it; the fp4 path also hides keys before key_lo
  // (block alignment). Then the online softmax and P.
  __device__ __forceinline__ void softmax(int j, int sk, int causal_off) {
    const int kt0 = j * kBN;
    bool need_mask = (kt0 + kBN > sk) || (kCausal && (kt0 + kBN - 1 > wave_q0 + causal_off));
    if constexpr (kFp4) need_mask = need_mask || (kt0 < key_lo);
    if (need_mask) {
      const int lim = kCausal ? min(sk - 1, qi + causal_off) : sk - 1;
      // Element (kb, i) holds key kt0 + 4*half + off with the constant
      // off = 32 kb + 8 (i/4) + i%4: each test compares that constant with a
      // per-row bound, opaque to the compiler, and selects -inf; a scheduling
      // barrier after each element keeps its compare next to its select. Left
      // to the compiler, the tests are grouped with one scalar register pair
      // per lane mask, or folded into per-element sums kept in registers
      // across the tile loop.
      int hi_rel = lim - kt0 - 4 * half;   // visible iff off <= hi_rel
      [[maybe_unused]] int lo_rel = key_lo - kt0 - 4 * half;   // fp4: and off >= lo_rel
      asm volatile("" : "+v"(hi_rel), "+v"(lo_rel));
      auto mask_one = [&](auto e_tag) __attribute__((always_inline)) {
        constexpr int e = decltype(e_tag)::value;
        constexpr int kb = e / 16, i = e % 16;
        constexpr int off = 32 * kb + 8 * (i / 4) + (i % 4);
        bool hidden = off > hi_rel;
        if constexpr (kFp4) hidden = hidden || off < lo_rel;
        if (hidden) sacc[kb][i] = -__builtin_inff();
        __builtin_amdgcn_sched_barrier(0);
      };
      [&]<int... kE>(std::integer_sequence<int, kE...>) {
        (mask_one(std::integral_constant<int, kE>()), ...);
      }(std::make_integer_sequence<int, 16 * kKeyBlocks>());
    }
    if constexpr (kFp4) {
      softmax_fp4();
    } else if constexpr (!kFp8) {
      softmax_lazy();
    } else {
      softmax_e4m3();
    }
  }

  // e2m1 P with per-group scales (log-domain quantisation). A lane holds 16
  // keys of each 32-key half of the tile (accumulator kb = key block kb); the
  // keys of one query row in one 32-key block form a quantisation group. exp2
  // is monotonic, so a group's largest p comes from its largest score g, and
  // its power-of-two scale 2^E, E = ceil(c*g - log2 6), keeps every p/2^E <= 6
  // (e2m1's largest value). The division by 2^E is a subtraction inside the
  // exp2 argument: p_hat = exp2(fma(s, c, -E)), one multiply-add per score.
  //
  // The running maximum is an integer M in exp2 units (m_log2), raised only
  // when a tile's p would exceed 2^8, so every O and l rescale is an exact
  // power of two and the quantised P does not depend on M: the codes are a
  // function of the scores alone. E - M (at most 6) is the group's E8M0 scale
  // byte - 127 for the P.V MFMA; the row sum adds the fp32 p_hat * 2^(E - M),
  // the values before rounding.
  __device__ __forceinline__ void softmax_fp4() {
    float ga[kKeyBlocks];
#pragma unroll
    for (int kb = 0; kb < kKeyBlocks; ++kb) {
      float mp[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
      for (int i = 0; i < 16; ++i) mp[i & 3] = fmaxf(mp[i & 3], sacc[kb][i]);
      ga[kb] = wave_half_swap_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
    }
    const float cmx = fmaxf(ga[0], ga[1]) * c;
    // -inf + 8 = -inf: a first finite maximum always raises, an empty row never
    const bool raise = cmx > m_log2 + 8.f;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float m_new = raise ? __builtin_ceilf(cmx) : m_log2;
      // 2^(M_old - M_new): 1 for rows not raised, 0 for a first maximum (the
      // clamp also absorbs -inf and the NaN of -inf - -inf, where O = l = 0)
      const float alpha = __builtin_ldexpf(1.f, (int)fmaxf(m_log2 - m_new, -200.f));
      m_log2 = m_new;
      rescale(alpha);
    }
    const float m_safe = (m_log2 == -__builtin_inff()) ? 0.f : m_log2;
    float rel[kKeyBlocks], add[kKeyBlocks];
#pragma unroll
    for (int kb = 0; kb < kKeyBlocks; ++kb) {
      // an empty group (g = -inf) takes the smallest scale; its p are zero
      const float e = __builtin_ceilf(__builtin_fmaf(ga[kb], c, -kLog2Six));
      rel[kb] = fmaxf(e - m_safe, -127.f);
      add[kb] = -(m_safe + rel[kb]);
    }
    // Packing. Key 32*kb + 8a + 4*half + b (a, b = 0..3) of this lane is
    // rounded into nibble (b) of the 16-bit field a%2 of word[kb][a/2]. One
    // v_permlane32_swap per word pair then leaves lane n (half 0) with the
    // block-0 words of both halves and lane n+32 with the block-1 words, so
    // operand nibble k of a lane is key 32*half + pi(k), with
    // pi = 0-3, 8-11 | 16-19, 24-27 | 4-7, 12-15 | 20-23, 28-31 (words 0..3);
    // the transposed V reads fetch keys in the same order.
    uint32_t word[kKeyBlocks][2] = {{0u, 0u}, {0u, 0u}};
    float rs[kKeyBlocks][2] = {{0.f, 0.f}, {0.f, 0.f}};
    static_for<kKeyBlocks * 8>([&](auto n_tag) {
      constexpr int n = decltype(n_tag)::value;
      constexpr int kb = n / 8, a = (n % 8) / 2, bb = n % 2;
      constexpr int i0 = 4 * a + 2 * bb;
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i0], c, add[kb]));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i0 + 1], c, add[kb]));
      rs[kb][bb] += p0 + p1;
      word[kb][a / 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word[kb][a / 2], p0, p1, 1.f,
                                                                 2 * (a % 2) + bb);
    });
    l_run += __builtin_ldexpf(rs[0][0] + rs[0][1], (int)rel[0]) +
             __builtin_ldexpf(rs[1][0] + rs[1][1], (int)rel[1]);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const auto r = __builtin_amdgcn_permlane32_swap((int)word[0][w], (int)word[1][w], false, false);
      pb4[w] = r[0];
      pb4[2 + w] = r[1];
    }
    // lane n takes group 0's exponent, lane n+32 group 1's (both lanes hold both)
    const auto rs_sel = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, rel[0]),
                                                         __builtin_bit_cast(int, rel[1]), false,
                                                         false);
    p_scale = (int)__builtin_bit_cast(float, rs_sel[0]) + 127;
  }

  // bf16 P: lazy maximum. The maximum in use (m_run) is kept as long as every
  // p = exp2(c*s - c*m_run) of the tile stays <= 2^kLazyLog2, which is checked
  // after the fact on each lane's partial row sum (every p is at most that
  // sum). Only when some row of the wave exceeds it (or has no maximum yet)
  // does the wave compute the tile's row maxima, rescale O and l, and redo p.
  // The scores stay in sacc, so the redo needs no second Q.K^T. Rows whose
  // maximum is not raised see alpha = 1 exactly, so each row's arithmetic
  // depends on its own scores only. Any m gives the same O and LSE in exact
  // arithmetic; m only bounds p.
  __device__ __forceinline__ void softmax_lazy() {
    float rs[4];
    exp_sum_convert(rs);
    float lane_sum = (rs[0] + rs[1]) + (rs[2] + rs[3]);
    // NaN-safe: inf or NaN sums also take the slow path
    const bool raise = (m_run == -__builtin_inff()) || !(lane_sum <= kLazyLimit);
    const uint64_t mask = __builtin_amdgcn_ballot_w64(raise);
    if (mask != 0) {
      // row n is raised if either of its lanes (n, n+32) asked for it
      const uint32_t rows = (uint32_t)mask | (uint32_t)(mask >> 32);
      const bool row_raise = (rows >> col) & 1u;
      const float mx = tile_row_max();
      // rows that see no key yet keep m_run = -inf (their p are all zero);
      // rows not raised recompute bit-identical p
      const bool up = row_raise && (mx > m_run);
      const float alpha = up ? __builtin_amdgcn_exp2f((m_run - mx) * c) : 1.f;
      m_run = up ? mx : m_run;
      rescale(alpha);
      exp_sum_convert(rs);
      lane_sum = (rs[0] + rs[1]) + (rs[2] + rs[3]);
    }
    // l_run holds this lane's half of the keys; the halves are added at the end
    l_run += lane_sum;
  }

  // e4m3 P: a running anchor A in exp2 units, raised lazily by whole steps.
  // The tile's values x = exp2(fma(s, c, 5 - A)) are rounded to e4m3 and summed
  // in fp32; A is kept as long as no x exceeds e4m3's largest value, checked
  // on each lane's partial sum (every x is at most that sum). A row's first
  // maximum sets A = c * (its first tile's row maximum), so that key maps to
  // exactly 2^5; afterwards a row that exceeds the limit raises A by the whole
  // number of steps that brings its tile's maximum under 2^5, and the wave
  // redoes the tile. Every later O and l rescale is then an exact power of
  // two, and because scaling by a power of two commutes with rounding to e4m3
  // in its normal range, the quantised P times 2^(A - 5) is the e4m3-precision
  // rounding of 2^(c s) on the grid that the first anchor fixes, whatever the
  // later steps are: P_hat depends on the scores alone (below 2^-6 of the
  // scale, in e4m3's subnormal range, on the steps as well).
  __device__ __forceinline__ void softmax_e4m3() {
    float rs[4];
    exp_sum_convert(rs);
    float lane_sum = (rs[0] + rs[1]) + (rs[2] + rs[3]);
    // NaN-safe: inf or NaN sums also take the slow path
    const bool raise = (m_log2 == -__builtin_inff()) || !(lane_sum <= kE4m3Max);
    const uint64_t mask = __builtin_amdgcn_ballot_w64(raise);
    if (mask != 0) {
      const uint32_t rows = (uint32_t)mask | (uint32_t)(mask >> 32);
      const bool row_raise = (rows >> col) & 1u;
      const float cmx = tile_row_max() * c;   // -inf for a row that sees no key yet
      const bool first = m_log2 == -__builtin_inff();
      // whole steps for a raised anchor (NaN when both are -inf, never used)
      const float steps = __builtin_ceilf(cmx - m_log2);
      const bool up = row_raise && (first ? cmx > -__builtin_inff() : steps > 0.f);
      // 2^(A_old - A_new): 1 for rows not raised, 0 for a first maximum (O = l = 0)
      float alpha = 1.f;
      if (up) alpha = first ? 0.f : __builtin_ldexpf(1.f, -(int)steps);
      m_log2 = up ? (first ? cmx : m_log2 + steps) : m_log2;
      rescale(alpha);
      exp_sum_convert(rs);
      lane_sum = (rs[0] + rs[1]) + (rs[2] + rs[3]);
    }
    l_run += lane_sum;
  }

  // Row maximum of the tile's scores over both lane halves. Four independent
  // partial maxima keep the dependency chains short.
  __device__ __forceinline__ float tile_row_max() const {
    float mp[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
    for (int kb = 0; kb < kKeyBlocks; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mp[i & 3] = fmaxf(mp[i & 3], sacc[kb][i]);
    return wave_half_swap_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
  }

  __device__ __forceinline__ void rescale(float alpha) {
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
  }

  // p = exp2(fma(s, c, -c*m_run)) for the 32 scores of this lane (the scale and
  // the row maximum folded into one multiply-add), partial row sums of the fp32
  // p in four chains, and P rounded for the P.V operand: bf16 RNE, or e4m3 of
  // exp2(fma(s, c, kPScaleLog2 - A)), the scale and the anchor folded into the
  // addend. The scores in sacc are kept.
  __device__ __forceinline__ void exp_sum_convert(float (&rs)[4]) {
    // an all-masked row keeps the fold finite
    float p_add;
    if constexpr (kFp8) p_add = kPScaleLog2 - ((m_log2 == -__builtin_inff()) ? 0.f : m_log2);
    else p_add = (m_run == -__builtin_inff()) ? 0.f : -m_run * c;
    rs[0] = rs[1] = rs[2] = rs[3] = 0.f;
    if constexpr (!kFp8) {
      static_for<kBN / 16>([&](auto ks_tag) {
        constexpr int ks16 = decltype(ks_tag)::value;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float pv = __builtin_amdgcn_exp2f(
              __builtin_fmaf(sacc[ks16 / 2][8 * (ks16 % 2) + jj], c, p_add));
          rs[jj & 3] += pv;
          pb[ks16][jj] = (bf16_t)pv;
        }
      });
    } else {
      // Byte j of a lane's operand is key kappa(half, j) =
      //   32*(j/16) + 8*((j%16)/4) + 4*half + j%4,
      // which is where the S^T accumulator left P; V is fetched to match.
      static_for<8>([&](auto w_tag) {
        constexpr int w = decltype(w_tag)::value;
        constexpr int kb = w / 4, i0 = 4 * (w % 4);
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i0 + e], c, p_add));
          rs[e] += pv[e];
        }
        int word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
        word = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], word, true);
        pb8[w] = word;
      });
    }
  }

  // O^T += V^T P^T for the tile at vs (LDS, generic pointer).
  __device__ __forceinline__ void pv(const char* vs) {
    if constexpr (kFp4) {
      // all 64 keys of the tile in one e2m1 MFMA per d block; lane (half, m)
      // supplies d row 32*db + m and keys 32*half + pi(0..31), and scales them
      // by the exponent of key block half, column d
      const unsigned char* vsc = (const unsigned char*)(vs + kVTileBytes) + half * kD + col;
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db) {
        const auto lo = __builtin_amdgcn_ds_read_tr4_b64_v2i32((LDS_AS i32x2*)(vs + v_off[0][db]));
        const auto hi = __builtin_amdgcn_ds_read_tr4_b64_v2i32((LDS_AS i32x2*)(vs + v_off[1][db]));
        const int sa = vsc[32 * db];
        const i32x8 a = {lo[0], lo[1], hi[0], hi[1], 0, 0, 0, 0};
        const i32x8 b = {pb4[0], pb4[1], pb4[2], pb4[3], 0, 0, 0, 0};
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, oacc[db], 4, 4, 0, sa,
                                                                   0, p_scale);
      }
    } else if constexpr (!kFp8) {
      // 16 keys per MFMA. Lane (half, m) needs V[keys 16*ks16 + 8r + 4*half
      // + 0..3][d = 32*db + m]; source lane gi of group g reads 4 d-values of
      // key row (.. + gi/4). The A operands of MFMA i + kAhead are read while
      // MFMA i runs (a ring of kAhead + 1 operand sets), which bounds the
      // registers the reads in flight take.
      constexpr int kN = (kBN / 16) * kDBlocks;   // MFMAs per tile
      constexpr int kAhead = 3;
      bf16x8 va[kAhead + 1];
      auto read_v = [&](int i) {
        const int ks16 = i / kDBlocks, db = i % kDBlocks;
        bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4*)(vs + v_off[0][db] + 16 * ks16 * kVRowBytes));
        bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4*)(vs + v_off[1][db] + 16 * ks16 * kVRowBytes));
        va[i % (kAhead + 1)] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
#pragma unroll
      for (int i = 0; i < kAhead; ++i) read_v(i);
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        if (i + kAhead < kN) read_v(i + kAhead);
        const int ks16 = i / kDBlocks, db = i % kDBlocks;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % (kAhead + 1)], pb[ks16], oacc[db],
                                                           0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 1);
#pragma unroll
      for (int i = 0; i < kN; ++i) {
        if (i + kAhead < kN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      }
    } else {
      // all 64 keys of the tile in one e4m3 MFMA per d block
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
        oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb8, oacc[db], 0, 0, 0, 127,
                                                                   0, 127);
      }
    }
  }

  // ---------------------------------------------------------------- software pipeline (bf16)
  //
  // The pipelined kernel walks the keys in half-tiles of 32 (u = 0, 1, ...).
  // Step u of a wave runs three independent pieces of work as one instruction
  // stream: the softmax of half-tile u (VALU), S of half-tile u+1 (Q.K^T MFMAs)
  // and O += P V of half-tile u-1 (P.V MFMAs). A wave thereby keeps its own
  // matrix-core work in flight while it computes exponentials, instead of
  // relying on another wave's opposite phase. S and P of consecutive
  // half-tiles alternate between two register sets (index u & 1). A rescale
  // of O that the softmax of half-tile u asks for (alpha_o) is applied at the
  // start of step u+1, after the P.V of half-tile u-1 and before that of u.
  static constexpr int kHalfQk = kKSteps;        // Q.K^T MFMAs per half-tile
  static constexpr int kHalfPv = 2 * kDBlocks;   // P.V MFMAs per half-tile
  f32x16 hs[2];        // S^T of a half-tile: keys 8*(i/4) + 4*half + i%4 for register i
  bf16x8 hp[2][2];     // bf16 P of a half-tile, per 16-key step
  float alpha_o;       // pending O rescale (1: none)

  // S^T of the half kH of the K tile at ks, into s.
  template <int kH>
  __device__ __forceinline__ void qk_half(const char* ks, f32x16& s) {
    bf16x8 ka[3];
    auto rk = [&](int t) { ka[t % 3] = *(const bf16x8*)(ks + k_off[t] + kH * 32 * kRowBytes); };
    rk(0);
    if (kHalfQk > 1) rk(1);
#pragma unroll
    for (int t = 0; t < kHalfQk; ++t) {
      if (t + 2 < kHalfQk) rk(t + 2);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % 3], qreg[t], t == 0 ? f32x16{} : s, 0, 0, 0);
    }
  }

  // The transposed V operand of P.V MFMA t of half kH of the V tile at vs.
  template <int kH>
  __device__ __forceinline__ bf16x8 read_v_half(const char* vs, int t) const {
    const int l = t / kDBlocks, db = t % kDBlocks;
    const int row0 = 16 * (2 * kH + l);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (LDS_AS bf16x4*)(vs + v_off[0][db] + row0 * kVRowBytes));
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (LDS_AS bf16x4*)(vs + v_off[1][db] + row0 * kVRowBytes));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }

  // O^T += V^T P^T for the half kH of the V tile at vs.
  template <int kH>
  __device__ __forceinline__ void pv_half(const char* vs, const bf16x8 (&p)[2]) {
    bf16x8 va[3];
    va[0] = read_v_half<kH>(vs, 0);
    va[1] = read_v_half<kH>(vs, 1);
#pragma unroll
    for (int t = 0; t < kHalfPv; ++t) {
      if (t + 2 < kHalfPv) va[(t + 2) % 3] = read_v_half<kH>(vs, t + 2);
      oacc[t % kDBlocks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          va[t % 3], p[t / kDBlocks], oacc[t % kDBlocks], 0, 0, 0);
    }
  }

  // Causal mask and key tail of half-tile u, if any of its keys needs it.
  __device__ __forceinline__ void mask_half(f32x16& s, int u, int sk, int causal_off) const {
    const int k0 = 32 * u;
    const bool need = (k0 + 32 > sk) || (kCausal && (k0 + 31 > wave_q0 + causal_off));
    if (need) {
      // constants against one per-row bound, as in softmax()
      const int lim = kCausal ? min(sk - 1, qi + causal_off) : sk - 1;
      int hi_rel = lim - k0 - 4 * half;
      asm volatile("" : "+v"(hi_rel));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (8 * (i / 4) + (i % 4) > hi_rel) s[i] = -__builtin_inff();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // p = exp2(fma(s, c, -c*m_run)) of a half-tile, its bf16 P and this lane's
  // partial row sum (fp32 p, four chains).
  __device__ __forceinline__ float exp_half(const f32x16& s, bf16x8 (&p)[2]) const {
    const float neg_mc = (m_run == -__builtin_inff()) ? 0.f : -m_run * c;
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, neg_mc));
      rs[i & 3] += e;
      p[i / 8][i % 8] = (bf16_t)e;
    }
    return (rs[0] + rs[1]) + (rs[2] + rs[3]);
  }

  // The lazy-maximum check of a half-tile whose p were computed with m_run
  // (see softmax_lazy): rows whose p exceed 2^8, or that have no maximum yet,
  // take the tile's row maximum, and their p, l and pending O rescale follow.
  __device__ __forceinline__ void settle_half(const f32x16& s, bf16x8 (&p)[2], float lane_sum) {
    const bool raise = (m_run == -__builtin_inff()) || !(lane_sum <= kLazyLimit);
    const uint64_t mask = __builtin_amdgcn_ballot_w64(raise);
    if (mask != 0) {
      const uint32_t rows = (uint32_t)mask | (uint32_t)(mask >> 32);
      const bool row_raise = (rows >> col) & 1u;
      float mp[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
#pragma unroll
      for (int i = 0; i < 16; ++i) mp[i & 3] = fmaxf(mp[i & 3], s[i]);
      const float mx = wave_half_swap_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3])));
      const bool up = row_raise && (mx > m_run);
      const float alpha = up ? __builtin_amdgcn_exp2f((m_run - mx) * c) : 1.f;
      m_run = up ? mx : m_run;
      l_run *= alpha;
      alpha_o *= alpha;
      lane_sum = exp_half(s, p);
    }
    l_run += lane_sum;
  }

  // Apply a pending rescale of O (all P.V MFMAs issued so far must have landed).
  __device__ __forceinline__ void settle_o() {
    if (__builtin_amdgcn_ballot_w64(alpha_o != 1.f) != 0) {
#pragma unroll
      for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha_o;
      alpha_o = 1.f;
    }
  }

  // Steady-state step u (kPar = u & 1) as one interleaved stream: softmax of
  // hs[kPar] into hp[kPar]; S of half-tile u+1 (half kPar^1 of the K tile at
  // ks) into hs[kPar^1]; O += P V of half-tile u-1 (hp[kPar^1], half kPar^1 of
  // the V tile at vs). Returns this lane's partial row sum of half-tile u.
  template <int kPar>
  __device__ __forceinline__ float step_interleaved(const char* ks, const char* vs) {
    constexpr int kH = kPar ^ 1;
    static_assert(kHalfQk == kHalfPv, "Q.K^T and P.V steps pair up one to one");
    constexpr int kN = kHalfQk;
    bf16x8 ka[3], va[3];
    auto rk = [&](int t) { ka[t % 3] = *(const bf16x8*)(ks + k_off[t] + kH * 32 * kRowBytes); };
    const float neg_mc = (m_run == -__builtin_inff()) ? 0.f : -m_run * c;
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
    rk(0);
    va[0] = read_v_half<kH>(vs, 0);
    rk(1);
    va[1] = read_v_half<kH>(vs, 1);
#pragma unroll
    for (int t = 0; t < kN; ++t) {
      if (t + 2 < kN) {
        rk(t + 2);
        va[(t + 2) % 3] = read_v_half<kH>(vs, t + 2);
      }
      hs[kH] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % 3], qreg[t],
                                                       t == 0 ? f32x16{} : hs[kH], 0, 0, 0);
      oacc[t % kDBlocks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          va[t % 3], hp[kH][t / kDBlocks], oacc[t % kDBlocks], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(hs[kPar][i], c, neg_mc));
      rs[i & 3] += e;
      hp[kPar][i / 8][i % 8] = (bf16_t)e;
    }
    // order: the first two steps' operand reads; then per step its reads two
    // steps ahead, each MFMA followed by a share of the softmax arithmetic
    constexpr int kValuPerMfma = (56 + 2 * kN - 1) / (2 * kN);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
    for (int t = 0; t < kN; ++t) {
      if (t + 2 < kN) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
    }
    return (rs[0] + rs[1]) + (rs[2] + rs[3]);
  }

  // Split-KV (bf16 path): split `split`'s O, normalised by its own row sum, and
  // its LSE, both fp32, into the partial buffers. A row that saw no key of this
  // split gets O = 0 and LSE = -inf, which the merge weighs by zero.
  __device__ __forceinline__ void epilogue_partial(const FwdParams& p, const WorkItem& w,
                                                   int split) {
    static_assert(!kFp8 && !kFp4, "split-KV runs the bf16 path");
    l_run = wave_half_swap_sum(l_run);
    if (qi >= w.sq) return;
    const float inv_l = (l_run > 0.f) ? 1.f / l_run : 0.f;
    const size_t row = (size_t)split * p.total_q + (size_t)(w.q_start + qi);
    float* op = p.o_part + (row * p.heads + w.head) * kD;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int d0 = 32 * db + 8 * ig + 4 * half;
        float4 o4;
        o4.x = oacc[db][4 * ig + 0] * inv_l;
        o4.y = oacc[db][4 * ig + 1] * inv_l;
        o4.z = oacc[db][4 * ig + 2] * inv_l;
        o4.w = oacc[db][4 * ig + 3] * inv_l;
        *(float4*)(op + d0) = o4;
      }
    if (half == 0) {
      float lse = -__builtin_inff();
      if (l_run > 0.f) lse = (m_run * c + __builtin_amdgcn_logf(l_run)) * 0.69314718055994531f;
      p.lse_part[((size_t)split * p.heads + w.head) * p.total_q + w.q_start + qi] = lse;
    }
  }

  // The epilogue with O written through LDS: each lane's O^T accumulators hold
  // 4 consecutive d of one query per register group, so direct stores write 8
  // bytes per lane into 32 different rows. Here the wave first places its
  // rows' bf16 O, half of d at a time, into a 4 KB LDS region (four 1 KB
  // blocks of 8 rows x 128 bytes at lds + r * kBlockStride, 16-byte chunks
  // XOR-swizzled by (row >> 1) & 7, which leaves at most two lanes on a bank),
  // then reads it back row-major, 16 bytes per lane, and stores 8 rows x 128
  // contiguous bytes per instruction. The region must be one no other wave
  // touches meanwhile: the 4-wave kernel passes blocks of a K stage this wave
  // itself refills first, the 8-wave kernel a private block per wave. LSE as
  // in epilogue().
  template <int kBlockStride>
  __device__ __forceinline__ void epilogue_lds(const FwdParams& p, const WorkItem& w,
                                               uint32_t lds_addr) {
    // the lane-dependent offsets below are formed here, after the tile loop:
    // derived from a lane index the compiler cannot see before this point, so
    // they are not hoisted into the loop, where registers are scarce
    lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
    int ln = lane;
    asm volatile("" : "+s"(lds_addr), "+v"(ln));
    LDS_AS char* lds = (LDS_AS char*)(uintptr_t)lds_addr;
    const int lcol = ln & 31, lhalf = ln >> 5;
    l_run = wave_half_swap_sum(l_run);
    const float num_scale = kFp8 ? p.v_scale[w.head] : 1.f;
    const float inv_l = (l_run > 0.f && qi < w.sq) ? num_scale / l_run : 0.f;
    const int row_stride = p.heads * kD;
    static_assert(kD == 128, "the staging spans a 16 KB K stage: four 1 KB blocks per wave");
    constexpr int kPasses = kD / 64;               // 64 d (128 bytes) per pass
    auto sw = [](int row) { return (row >> 1) & 7; };
    // this lane's write position: row col, block col / 8, row col % 8 inside it
    LDS_AS char* wrow = lds + (lcol >> 3) * kBlockStride + (lcol & 7) * 128;
    // this lane's read position: row R = 8 s + lane / 8 of block s, chunk lane % 8
    const int rr = ln >> 3, rc = ln & 7;
    bf16_t* out0 = (bf16_t*)p.out + (size_t)w.head * kD;
#pragma unroll
    for (int pass = 0; pass < kPasses; ++pass) {
#pragma unroll
      for (int dbp = 0; dbp < 2; ++dbp)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const int db = 2 * pass + dbp;
          bf16x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (bf16_t)(oacc[db][4 * ig + e] * inv_l);
          // d = 32 db + 8 ig + 4 half: 16-byte chunk 4 dbp + ig of the 128-byte row
          *(LDS_AS bf16x4*)(wrow + (((4 * dbp + ig) ^ sw(lcol)) * 16) + 8 * lhalf) = o4;
        }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int row = 8 * s + rr;               // row of this wave's 32
        const bf16x8 v = *(const LDS_AS bf16x8*)(lds + s * kBlockStride + rr * 128 +
                                                 ((rc ^ sw(row)) * 16));
        if (wave_q0 + row < w.sq)
          *(bf16x8*)(out0 + (size_t)(w.q_start + wave_q0 + row) * row_stride + 64 * pass +
                     8 * rc) = v;
      }
    }
    if (p.lse != nullptr && half == 0 && qi < w.sq) {
      float lse = -__builtin_inff();
      const float lsub = kFp8 ? kPScaleLog2 : 0.f;
      const float mlog2 = (kFp4 || kFp8) ? m_log2 : m_run * c;
      if (l_run > 0.f)
        lse = (mlog2 + (__builtin_amdgcn_logf(l_run) - lsub)) * 0.69314718055994531f;
      p.lse[(size_t)w.head * p.total_q + w.q_start + qi] = lse;
    }
  }

  // O /= l -> bf16 store; LSE = scale*m + ln(l) (natural log). A row with no
  // visible key has l = 0: O = 0 and LSE = -inf.
  __device__ __forceinline__ void epilogue(const FwdParams& p, const WorkItem& w) {
    l_run = wave_half_swap_sum(l_run);
    if (qi >= w.sq) return;
    // fp8: O = v_scale * sum(P_hat V_codes) / l, where l carries the same 2^kPScaleLog2
    // (fp4: the block and group scales are applied inside the MFMA)
    const float num_scale = kFp8 ? p.v_scale[w.head] : 1.f;
    const float inv_l = (l_run > 0.f) ? num_scale / l_run : 0.f;
    const int row_stride = p.heads * kD;
    bf16_t* op = (bf16_t*)p.out + (size_t)(w.q_start + qi) * row_stride + w.head * kD;
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
      const float mlog2 = (kFp4 || kFp8) ? m_log2 : m_run * c;
      if (l_run > 0.f)
        lse = (mlog2 + (__builtin_amdgcn_logf(l_run) - lsub)) * 0.69314718055994531f;
      p.lse[(size_t)w.head * p.total_q + w.q_start + qi] = lse;
    }
  }
};

}  // namespace fmha

#endif  // FMHA_DEVICE_H_
