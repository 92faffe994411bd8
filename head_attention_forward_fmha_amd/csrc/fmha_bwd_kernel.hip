// Backward pass of the FMHA forward (gfx950): dQ, dK, dV from the saved LSE.
//
// The step the FlashAttention-4 spill issue times is the varlen causal forward
// followed by the backward of mean(O^2) ("CuTe DSL 4.7/4.8 regression:
// FlashAttention-4 SM100 forward kernel spills registers", Describe the bug and
// Steps/Code to reproduce bug). For one document and head, with
// P_ij = exp(S_ij - LSE_i) recomputed from the forward's LSE:
//
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),   D_i = dO_i . O_i,
//   dQ = tau dS K, dK = tau dS^T Q.
//
// (D_i equals sum_j P_ij dP_ij because O_i = sum_j P_ij V_j.) Two launches:
//
//   1. dQ: a workgroup owns 128 queries, 32 per wave, with Q and dO in
//      registers, and streams 64-key K and V tiles: S^T = K Q^T and
//      dP^T = V dO^T by rows, dQ^T += K^T dS^T transposed. Holding each
//      query's dO row, it also computes D and LSE * log2(e) per (row, head)
//      and writes them to the workspace;
//   2. dK/dV: a workgroup owns 128 keys of one (document, head), 32 per wave
//      position, and streams the document's 64-row Q and dO tiles through a
//      three-stage LDS ring. It is the forward's structure with the roles of
//      queries and keys swapped: S = Q K^T and dP = dO V^T read the streamed
//      tiles by rows (lane = key, registers = queries), and dV^T += dO^T P and
//      dK^T += Q^T dS read them transposed (ds_read_b64_tr_b16), with P and dS
//      as the register operand, exactly as O^T += V^T P^T. Two groups of 4 waves
//      split the work, one computing S, dP, P and dS (holding K and V), the other
//      the transposed products (holding dV and dK), with P and dS passed
//      through LDS; it reads D and LSE * log2(e) of each query tile from the
//      workspace.
//
// Every output element is written by exactly one lane with a fixed summation
// order, so the result is deterministic (no atomics); the price is that S and dP
// are computed twice (seven matrix products instead of five).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fmha_bwd_params.h"
#include "fmha_device.h"

namespace fmha {

namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdRows = 32 * kBwdWaves;   // keys (dK/dV) or queries (dQ) per workgroup
constexpr int kTileRows = 64;              // rows of a streamed tile
constexpr float kLog2eF = 1.4426950408889634f;

// A streamed tile: 64 rows of kD bf16 in LDS, 16-byte chunks swizzled per row
// as in the forward's K/V tiles (so that both the row reads and the transposed
// reads are conflict-free), filled by HBM -> LDS copies.
template <int kD>
struct TileGeom {
  static constexpr int kRowBytes = 2 * kD;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kTileBytes = kTileRows * kRowBytes;
  static constexpr int kKSteps = kD / 16;     // MFMA steps over d
  static constexpr int kDBlocks = kD / 32;    // 32-wide d blocks of an accumulator
  static constexpr int kLoads = kTileBytes / (kBwdWaves * 64 * 16);   // per wave and tile
  static_assert(kLoads * kBwdWaves * 64 * 16 == kTileBytes, "tile splits into lane loads");

  // byte offset of logical 16-byte chunk `chunk` of row `row`
  __device__ __forceinline__ static int at(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz<kChunks>(row)) * 16);
  }
};

// Per-lane operand read offsets and copy offsets of a streamed tile.
template <int kD>
struct TileLane {
  using G = TileGeom<kD>;
  int row_off[G::kKSteps];          // rows read as an A operand: row col, d 16t + 8*half
  int tr_off[2][G::kDBlocks];       // transposed reads (two per 16-row step)
  int copy_off[G::kLoads];          // global byte offset of this lane's chunk per copy

  __device__ __forceinline__ void init(int lane, int wave, uint32_t stride) {
    const int col = lane & 31, half = lane >> 5, g = lane >> 4, gi = lane & 15;
#pragma unroll
    for (int t = 0; t < G::kKSteps; ++t) row_off[t] = G::at(col, 2 * t + half);
    // Lane (half, m) of a transposed read receives the 4 values of d row
    // 32*db + m at tile rows 8r + 4*half + 0..3: lane gi of group g reads 4 d
    // values (32*db + 16*(g&1) + 4*(gi&3)) of row 8r + 4*half + gi/4.
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < G::kDBlocks; ++db) {
        const int row = 8 * r + 4 * half + gi / 4;
        const int d = 32 * db + 16 * (g & 1) + 4 * (gi & 3);
        tr_off[r][db] = G::at(row, d / 8) + (d % 8) * 2;
      }
    // wave w's copy r lands at LDS bytes 1024*(r*kBwdWaves + w) + 16*lane of
    // the tile; the lane fetches the logical chunk stored there
#pragma unroll
    for (int r = 0; r < G::kLoads; ++r) {
      const int byte = 1024 * (r * kBwdWaves + wave) + 16 * lane;
      const int row = byte / G::kRowBytes;
      const int phys = (byte % G::kRowBytes) / 16;
      copy_off[r] = row * (int)stride + (phys ^ swz<G::kChunks>(row)) * 16;
    }
  }

  // copy of the 64 rows from row0 on (relative to the descriptor's base) into
  // the tile at LDS address lds_wave0 + kLdsOffset (lds_wave0: this wave's first
  // 1 KB block of stage 0). The rows' offset goes into the per-lane offset,
  // which the raw-buffer range check covers, so rows past the end read zeros.
  template <int kLdsOffset>
  __device__ __forceinline__ void copy(uint32_t lds_wave0, i32x4 rsrc, int row0,
                                       uint32_t stride) const {
    const int off = __builtin_amdgcn_readfirstlane((int)((uint32_t)row0 * stride));
    static_for<G::kLoads>([&](auto r_tag) {
      constexpr int r = decltype(r_tag)::value;
      lds_dma_16<kLdsOffset + 1024 * kBwdWaves * r>(lds_wave0, copy_off[r] + off, rsrc, 0);
    });
  }
};

// (document, head, block) of a work item; blocks of kBwdRows rows.
struct BwdItem {
  int head, q_start, k_start, sq, sk, block;
};

// Items are numbered through groups of (document, head) pairs, about
// kGroupItems items each, and within a group block by block: a group's longest
// blocks start first, its shortest are dispatched last, and the Q/dO or K/V rows
// that its concurrent workgroups stream are those of a few pairs only. About
// two items per CU of an XCD measured best (fewer pairs per group leave a
// longer tail, more pairs spread the rows over more of the L2). Without a
// causal mask all blocks of a document cost the same, and the items stay in
// pair-major order (one group per pair).
constexpr int kGroupItems = 64;

__device__ __forceinline__ BwdItem decode_bwd_item(const BwdParams& p, int item,
                                                   bool reverse_blocks, bool grouped) {
  const int n_pairs = p.batch * p.heads;
  const int group_pairs = grouped ? max(1, kGroupItems / p.n_blocks) : 1;
  const int base = item / (group_pairs * p.n_blocks) * group_pairs;
  const int g = min(group_pairs, n_pairs - base);   // pairs in this group
  const int r = item - base * p.n_blocks;
  const int b = r / g;
  const int pair = base + (r - b * g);
  BwdItem w;
  w.block = reverse_blocks ? p.n_blocks - 1 - b : b;
  const int doc = pair / p.heads;
  w.head = pair - doc * p.heads;
  if (p.cu_q != nullptr) {
    w.q_start = p.cu_q[doc];
    w.sq = p.cu_q[doc + 1] - w.q_start;
    w.k_start = p.cu_k[doc];
    w.sk = p.cu_k[doc + 1] - w.k_start;
  } else {
    w.q_start = doc * p.max_seqlen_q;
    w.sq = p.max_seqlen_q;
    w.k_start = doc * p.max_seqlen_k;
    w.sk = p.max_seqlen_k;
  }
  return w;
}

// Items are dealt to XCDs in contiguous ranges (workgroup id % 8 picks the XCD),
// so that the blocks of one (document, head), which stream the same tiles, share
// an L2.
__device__ __forceinline__ int xcd_item(int n_items) {
  const int xcd = blockIdx.x % kXcds;
  const int per = n_items / kXcds, extra = n_items % kXcds;
  return xcd * per + min(xcd, extra) + (int)blockIdx.x / kXcds;
}

__device__ __forceinline__ void store_bf16_rows(bf16_t* row, const f32x16* acc, int n_blocks,
                                                float mul, int half) {
  for (int db = 0; db < n_blocks; ++db)
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      bf16x4 v4;
#pragma unroll
      for (int e = 0; e < 4; ++e) v4[e] = (bf16_t)(acc[db][4 * ig + e] * mul);
      *(bf16x4*)(row + 32 * db + 8 * ig + 4 * half) = v4;
    }
}

// ---------------------------------------------------------------- dK and dV

// The dK/dV pass as two groups of 4 waves, two waves per SIMD: 128 keys per
// workgroup, 32 per wave position (sub = wave % 4) as above, but the products
// are split between the groups. Group A holds the position's K and V and turns
// each query tile into S and dP (Q K^T, dO V^T by rows) and from them P and dS;
// group B holds the dV and dK accumulators and runs the transposed products
// dV^T += dO^T P, dK^T += Q^T dS. P and dS pass through LDS (8 KB per position
// and tile). Step s, two barriers:
//   phase 1: A runs S/dP of tile s; B issues the copies of tile s+1 and loads
//            P/dS of tile s-1;
//   phase 2: B runs dV/dK of tile s-1; A computes P/dS of tile s and stores
//            them; B waits for its copies.
// So each SIMD's matrix core is fed by one group at a time while the other
// group's vector work, copies and LDS traffic run beside it, and each group
// needs well under 256 registers where one wave holding everything needed 472
// (one wave per SIMD). Q/dO tiles go through a ring of three stages: in step s
// A reads tile s by rows, B reads tile s-1 transposed, and tile s+1 lands.
template <int kD, bool kCausal>
__global__ __attribute__((amdgpu_flat_work_group_size(2 * kBwdWaves * 64, 2 * kBwdWaves * 64),
                          amdgpu_waves_per_eu(2, 2)))
void fmha_bwd_dkdv_kernel(BwdParams p) {
  using G = TileGeom<kD>;
  __shared__ __attribute__((aligned(1024))) char smem_q[3][G::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char smem_do[3][G::kTileBytes];
  __shared__ __attribute__((aligned(16))) float smem_rows[3][2 * kTileRows];  // LSE*log2e, D
  // P and dS of one tile per wave position: lane l's 16-byte chunk k (P of
  // 16-query steps 0..3, then dS of steps 0..3) at 1024 k + 16 l, so each LDS
  // access of a wave covers 1 KB contiguously
  __shared__ __attribute__((aligned(1024))) char smem_pds[kBwdWaves][8 * 1024];

  const BwdItem w = decode_bwd_item(p, xcd_item(p.batch * p.heads * p.n_blocks), false, kCausal);
  const int n0 = w.block * kBwdRows;
  if (n0 >= w.sk) return;   // uniform over the workgroup
  // readfirstlane: branches on the group are scalar branches, and each group's
  // path gets its own register allocation
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2, sub = wave & 3;
  const int lane = threadIdx.x & 63, col = lane & 31, half = lane >> 5;
  const int kw0 = n0 + 32 * sub;   // this position's first key (in the document)
  const int causal_off = w.sk - w.sq;
  const uint32_t stride = (uint32_t)p.heads * G::kRowBytes;
  const int n_qt = (w.sq + kTileRows - 1) / kTileRows;
  // causal blocks start at the first query tile that sees key n0
  const int t0 = kCausal ? max(0, n0 - causal_off) / kTileRows : 0;
  // tile jt contributes to this position iff some query of it sees its first key
  auto active = [&](int jt) {
    return !kCausal || jt * kTileRows + kTileRows - 1 + causal_off >= kw0;
  };
  LDS_AS char* pds_lds = (LDS_AS char*)(uintptr_t)lds_address(&smem_pds[sub][0]);

  auto run_a = [&]() __attribute__((always_inline)) {
    const float c = p.scale_log2;
    bf16x8 kreg[G::kKSteps], vreg[G::kKSteps];
    {
      const size_t krow = (size_t)(w.k_start + min(kw0 + col, w.sk - 1)) * p.heads * kD +
                          (size_t)w.head * kD + 8 * half;
#pragma unroll
      for (int t = 0; t < G::kKSteps; ++t) {
        kreg[t] = *(const bf16x8*)((const bf16_t*)p.k + krow + 16 * t);
        vreg[t] = *(const bf16x8*)((const bf16_t*)p.v + krow + 16 * t);
      }
    }
    int row_off[G::kKSteps];
#pragma unroll
    for (int t = 0; t < G::kKSteps; ++t) row_off[t] = G::at(col, 2 * t + half);
    const int key = kw0 + col;

    auto step = [&](int jt, auto stage_tag) {
      constexpr int st = decltype(stage_tag)::value;
      const bool on = jt < n_qt && active(jt);
      f32x16 s[2], dp[2];   // the first MFMA of each chain starts from zero
      // ---- phase 1: S = Q K^T and dP = dO V^T (rows 32 kb + 8(r/4) + 4 half + r%4
      // of the tile by this lane's key), operands two steps ahead of their MFMAs
      if (on) {
        const char* qs = smem_q[st];
        const char* dos = smem_do[st];
        __builtin_amdgcn_s_setprio(2);
        static_for<2>([&](auto kb_tag) {
          constexpr int kb = decltype(kb_tag)::value;
          constexpr int kAhead = 2;
          bf16x8 qa[kAhead + 1], da[kAhead + 1];
          auto read_rows = [&](int t) {
            const int off = row_off[t] + kb * 32 * G::kRowBytes;
            qa[t % (kAhead + 1)] = *(const bf16x8*)(qs + off);
            da[t % (kAhead + 1)] = *(const bf16x8*)(dos + off);
          };
#pragma unroll
          for (int t = 0; t < kAhead; ++t) read_rows(t);
#pragma unroll
          for (int t = 0; t < G::kKSteps; ++t) {
            if (t + kAhead < G::kKSteps) read_rows(t + kAhead);
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[t % (kAhead + 1)], kreg[t],
                                                            t == 0 ? f32x16{} : s[kb], 0, 0, 0);
            dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[t % (kAhead + 1)], vreg[t],
                                                             t == 0 ? f32x16{} : dp[kb], 0, 0, 0);
          }
        });
        __builtin_amdgcn_s_setprio(0);
      }
      lds_barrier();
      // ---- phase 2: P = exp2(S c - LSE log2 e), dS = P (dP - D), masked keys
      // P = 0; both rounded to bf16 in the order the forward uses for its P,
      // and stored for group B
      if (on) {
        const float* rows = smem_rows[st];
        const int q0 = jt * kTileRows;
        const bool need_mask = !kCausal ? (q0 + kTileRows > w.sq)
                                        : ((q0 + kTileRows > w.sq) || kw0 + 31 > q0 + causal_off);
        bf16x8 pb[4], dsb[4];
        auto pds = [&](auto mask_tag) {
          constexpr bool kMask = decltype(mask_tag)::value;
          static_for<2>([&](auto kb_tag) {
            constexpr int kb = decltype(kb_tag)::value;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              const int qr = 32 * kb + 8 * g4 + 4 * half;
              const float4 l4 = *(const float4*)(rows + qr);
              const float4 d4 = *(const float4*)(rows + kTileRows + qr);
              const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
              const float dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -lv[e]));
                if constexpr (kMask) {
                  const int i = q0 + qr + e;
                  if (i >= w.sq || (kCausal && key > i + causal_off)) pv = 0.f;
                }
                const float ds = pv * (dp[kb][r] - dl[e]);
                pb[2 * kb + r / 8][r % 8] = (bf16_t)pv;
                dsb[2 * kb + r / 8][r % 8] = (bf16_t)ds;
              }
            }
          });
        };
        if (need_mask) pds(std::true_type());
        else pds(std::false_type());
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          *(LDS_AS bf16x8*)(pds_lds + 1024 * k + 16 * ln) = pb[k];
          *(LDS_AS bf16x8*)(pds_lds + 1024 * (4 + k) + 16 * ln) = dsb[k];
        }
      }
      lds_barrier();
    };
    // the tiles' copies of step t0 (issued by group B) have landed
    lds_barrier();
    int jt = t0;
    for (; jt + 3 <= n_qt + 1; jt += 3) {
      step(jt, std::integral_constant<int, 0>());
      step(jt + 1, std::integral_constant<int, 1>());
      step(jt + 2, std::integral_constant<int, 2>());
    }
    if (jt <= n_qt) step(jt, std::integral_constant<int, 0>());
    if (jt + 1 <= n_qt) step(jt + 1, std::integral_constant<int, 1>());
  };

  auto run_b = [&]() __attribute__((always_inline)) {
    f32x16 dvacc[G::kDBlocks], dkacc[G::kDBlocks];
#pragma unroll
    for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) dvacc[db][i] = dkacc[db][i] = 0.f;
    TileLane<kD> tl;
    tl.init(lane, sub, stride);
    const i32x4 q_rsrc = make_buffer_rsrc(
        (const char*)p.q + (size_t)w.q_start * stride + w.head * G::kRowBytes,
        (uint32_t)w.sq * stride);
    const i32x4 do_rsrc = make_buffer_rsrc(
        (const char*)p.dout + (size_t)w.q_start * stride + w.head * G::kRowBytes,
        (uint32_t)w.sq * stride);
    const uint32_t q_lds0 = lds_address(&smem_q[0][1024 * sub]);
    const uint32_t do_lds0 = lds_address(&smem_do[0][1024 * sub]);
    const uint32_t rows_lds0 = lds_address(&smem_rows[0][0]);
    const size_t row_base = (size_t)w.head * p.total_q + w.q_start;
    // a tile's copies: Q and dO rows, then LSE*log2e and D of its 64 rows (every
    // wave of the group fetches the same 512 bytes)
    auto copy_tile = [&](int jt, auto stage_tag) {
      constexpr int st = decltype(stage_tag)::value;
      tl.template copy<st * G::kTileBytes>(q_lds0, q_rsrc, jt * kTileRows, stride);
      tl.template copy<st * G::kTileBytes>(do_lds0, do_rsrc, jt * kTileRows, stride);
      const size_t r = row_base + min(jt * kTileRows + lane, w.sq - 1);
      const uint32_t rl = __builtin_amdgcn_readfirstlane(rows_lds0 + st * 2 * kTileRows * 4);
      lds_dma_global_4(rl, p.lse2 + r);
      lds_dma_global_4(rl + kTileRows * 4, p.delta + r);
    };

    // step s: stage st holds tile s, (st + 2) % 3 tile s-1, (st + 1) % 3 receives s+1
    auto step = [&](int jt, auto stage_tag) {
      constexpr int st = decltype(stage_tag)::value;
      const bool on = jt - 1 >= t0 && active(jt - 1);
      // ---- phase 1: copies of tile jt+1, P/dS of tile jt-1
      if (jt + 1 < n_qt) copy_tile(jt + 1, std::integral_constant<int, (st + 1) % 3>());
      bf16x8 pb[4], dsb[4];
      if (on) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          pb[k] = *(const LDS_AS bf16x8*)(pds_lds + 1024 * k + 16 * ln);
          dsb[k] = *(const LDS_AS bf16x8*)(pds_lds + 1024 * (4 + k) + 16 * ln);
        }
      }
      lds_barrier();
      // ---- phase 2: dV^T += dO^T P and dK^T += Q^T dS of tile jt-1: pair i
      // (16-query step i / kDBlocks, d block i % kDBlocks) reads the tiles
      // transposed, three pairs ahead
      if (on) {
        const char* qs = smem_q[(st + 2) % 3];
        const char* dos = smem_do[(st + 2) % 3];
        constexpr int kN = 4 * G::kDBlocks;
        constexpr int kAheadT = 3;
        bf16x8 ad[kAheadT + 1], aq[kAheadT + 1];
        auto read_t = [&](int i) {
          const int ks16 = i / G::kDBlocks, db = i % G::kDBlocks;
          const int o0 = tl.tr_off[0][db] + 16 * ks16 * G::kRowBytes;
          const int o1 = tl.tr_off[1][db] + 16 * ks16 * G::kRowBytes;
          const bf16x4 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(dos + o0));
          const bf16x4 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(dos + o1));
          const bf16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(qs + o0));
          const bf16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(qs + o1));
          ad[i % (kAheadT + 1)] =
              bf16x8{dlo[0], dlo[1], dlo[2], dlo[3], dhi[0], dhi[1], dhi[2], dhi[3]};
          aq[i % (kAheadT + 1)] =
              bf16x8{qlo[0], qlo[1], qlo[2], qlo[3], qhi[0], qhi[1], qhi[2], qhi[3]};
        };
        __builtin_amdgcn_s_setprio(2);
#pragma unroll
        for (int i = 0; i < kAheadT; ++i) read_t(i);
#pragma unroll
        for (int i = 0; i < kN; ++i) {
          if (i + kAheadT < kN) read_t(i + kAheadT);
          const int ks16 = i / G::kDBlocks, db = i % G::kDBlocks;
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad[i % (kAheadT + 1)], pb[ks16],
                                                              dvacc[db], 0, 0, 0);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq[i % (kAheadT + 1)], dsb[ks16],
                                                              dkacc[db], 0, 0, 0);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      // the copies of tile jt+1 have landed before the barrier that publishes them
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      lds_barrier();
    };
    if (t0 < n_qt) copy_tile(t0, std::integral_constant<int, 0>());
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
    int jt = t0;
    for (; jt + 3 <= n_qt + 1; jt += 3) {
      step(jt, std::integral_constant<int, 0>());
      step(jt + 1, std::integral_constant<int, 1>());
      step(jt + 2, std::integral_constant<int, 2>());
    }
    if (jt <= n_qt) step(jt, std::integral_constant<int, 0>());
    if (jt + 1 <= n_qt) step(jt + 1, std::integral_constant<int, 1>());

    // dV = sum P^T dO, dK = tau sum dS^T Q for this lane's key
    const int key = kw0 + col;
    if (key < w.sk) {
      const size_t off = (size_t)(w.k_start + key) * p.heads * kD + (size_t)w.head * kD;
      store_bf16_rows((bf16_t*)p.dv + off, dvacc, G::kDBlocks, 1.f, half);
      store_bf16_rows((bf16_t*)p.dk + off, dkacc, G::kDBlocks, p.scale, half);
    }
  };

  if (grp == 0) run_a();
  else run_b();
}

// ---------------------------------------------------------------- dQ

template <int kD, bool kCausal>
__global__ __attribute__((amdgpu_flat_work_group_size(kBwdWaves * 64, kBwdWaves * 64),
                          amdgpu_waves_per_eu(2, 2)))
void fmha_bwd_dq_kernel(BwdParams p) {
  using G = TileGeom<kD>;
  __shared__ __attribute__((aligned(1024))) char smem_k[2][G::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char smem_v[2][G::kTileBytes];

  // causal: the longest query blocks (most keys) first
  const BwdItem w = decode_bwd_item(p, xcd_item(p.batch * p.heads * p.n_blocks), kCausal, kCausal);
  const int m0 = w.block * kBwdRows;
  if (m0 >= w.sq) return;   // uniform over the workgroup
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63, col = lane & 31, half = lane >> 5;
  const int wave_q0 = m0 + 32 * wave;
  const int qi = wave_q0 + col;     // this lane's query (in the document)
  const int causal_off = w.sk - w.sq;
  const uint32_t stride = (uint32_t)p.heads * G::kRowBytes;
  const float c = p.scale_log2;

  // Q and dO rows of this lane's query: the B operands of S^T = K Q^T and
  // dP^T = V dO^T; its LSE*log2e and D
  bf16x8 qreg[G::kKSteps], doreg[G::kKSteps];
  const int qrow = w.q_start + min(qi, w.sq - 1);
  {
    const size_t off = (size_t)qrow * p.heads * kD + (size_t)w.head * kD + 8 * half;
#pragma unroll
    for (int t = 0; t < G::kKSteps; ++t) {
      qreg[t] = *(const bf16x8*)((const bf16_t*)p.q + off + 16 * t);
      doreg[t] = *(const bf16x8*)((const bf16_t*)p.dout + off + 16 * t);
    }
  }
  // LSE*log2e and D = dO . O of this lane's query. D is summed like a tree over
  // 16-byte chunks of the row: each chunk sequentially, then pairs of chunks;
  // lane half h holds chunks 2t + h, so the halves first add each other's chunk
  // sums. The workgroup that owns a query writes both for the dK/dV kernel,
  // which runs after this one.
  const size_t row_idx = (size_t)w.head * p.total_q + qrow;
  const float lse_nat = p.lse[row_idx];
  const float lse2 = (lse_nat == -__builtin_inff()) ? __builtin_inff() : lse_nat * kLog2eF;
  float delta;
  {
    const size_t off = (size_t)qrow * p.heads * kD + (size_t)w.head * kD + 8 * half;
    float part[G::kKSteps];
#pragma unroll
    for (int t = 0; t < G::kKSteps; ++t) {
      const bf16x8 o = *(const bf16x8*)((const bf16_t*)p.out + off + 16 * t);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)doreg[t][e] * (float)o[e];
      part[t] = acc;
    }
#pragma unroll
    for (int t = 0; t < G::kKSteps; ++t) part[t] += __shfl_xor(part[t], 32);
#pragma unroll
    for (int m = 1; m < G::kKSteps; m *= 2) {
      float sum[G::kKSteps];
#pragma unroll
      for (int t = 0; t < G::kKSteps; ++t) sum[t] = part[t] + part[t ^ m];
#pragma unroll
      for (int t = 0; t < G::kKSteps; ++t) part[t] = sum[t];
    }
    delta = part[0];
  }
  if (half == 0 && qi < w.sq) {
    p.delta[row_idx] = delta;
    p.lse2[row_idx] = lse2;
  }
  f32x16 dqacc[G::kDBlocks];
#pragma unroll
  for (int db = 0; db < G::kDBlocks; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dqacc[db][i] = 0.f;

  TileLane<kD> tl;
  tl.init(lane, wave, stride);
  const i32x4 k_rsrc = make_buffer_rsrc(
      (const char*)p.k + (size_t)w.k_start * stride + w.head * G::kRowBytes, (uint32_t)w.sk * stride);
  const i32x4 v_rsrc = make_buffer_rsrc(
      (const char*)p.v + (size_t)w.k_start * stride + w.head * G::kRowBytes, (uint32_t)w.sk * stride);
  const uint32_t k_lds0 = lds_address(&smem_k[0][1024 * wave]);
  const uint32_t v_lds0 = lds_address(&smem_v[0][1024 * wave]);

  int kend = w.sk;
  if (kCausal) kend = min(w.sk, max(0, m0 + kBwdRows + causal_off));
  const int n = (kend + kTileRows - 1) / kTileRows;

  auto compute = [&](int j, auto stage_tag) {
    constexpr int st = decltype(stage_tag)::value;
    const char* ks = smem_k[st];
    const char* vs = smem_v[st];
    const int k0 = j * kTileRows;
    const bool need_mask = (k0 + kTileRows > w.sk) || (kCausal && k0 + kTileRows - 1 > wave_q0 + causal_off);
    // One 32-key block at a time (which keeps two waves per SIMD within their
    // registers): S^T = K Q^T and dP^T = V dO^T for keys 32*kb + 8(r/4) +
    // 4*half + r%4 of the tile by this lane's query, then dS^T in bf16.
    bf16x8 dsb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
      // operands read two steps ahead of their MFMAs (a ring of three), and the
      // scheduling-group barriers keep the reads from being hoisted further
      constexpr int kAhead = 2;
      bf16x8 ka[kAhead + 1], va[kAhead + 1];
      auto read = [&](int t) {
        const int off = tl.row_off[t] + kb * 32 * G::kRowBytes;
        ka[t % (kAhead + 1)] = *(const bf16x8*)(ks + off);
        va[t % (kAhead + 1)] = *(const bf16x8*)(vs + off);
      };
#pragma unroll
      for (int t = 0; t < kAhead; ++t) read(t);
#pragma unroll
      for (int t = 0; t < G::kKSteps; ++t) {
        if (t + kAhead < G::kKSteps) read(t + kAhead);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[t % (kAhead + 1)], qreg[t], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[t % (kAhead + 1)], doreg[t], dp, 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 0);
#pragma unroll
      for (int t = 0; t < G::kKSteps; ++t) {
        if (t + kAhead < G::kKSteps) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lse2));
        if (need_mask) {
          const int key = k0 + 32 * kb + 8 * (r / 4) + 4 * half + (r % 4);
          if (key >= w.sk || (kCausal && key > qi + causal_off)) pv = 0.f;
        }
        dsb[2 * kb + r / 8][r % 8] = (bf16_t)(pv * (dp[r] - delta));
      }
    }
    // dQ^T += K^T dS^T (transposed K tile reads, three MFMAs ahead)
    constexpr int kN = 4 * G::kDBlocks;
    constexpr int kAhead = 3;
    bf16x8 ta[kAhead + 1];
    auto read_t = [&](int i) {
      const int ks16 = i / G::kDBlocks, db = i % G::kDBlocks;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (LDS_AS bf16x4*)(ks + tl.tr_off[0][db] + 16 * ks16 * G::kRowBytes));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (LDS_AS bf16x4*)(ks + tl.tr_off[1][db] + 16 * ks16 * G::kRowBytes));
      ta[i % (kAhead + 1)] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
#pragma unroll
    for (int i = 0; i < kAhead; ++i) read_t(i);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (i + kAhead < kN) read_t(i + kAhead);
      const int ks16 = i / G::kDBlocks, db = i % G::kDBlocks;
      dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[i % (kAhead + 1)], dsb[ks16],
                                                          dqacc[db], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kAhead, 1);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if (i + kAhead < kN) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
    }
  };

  // One barrier per tile: once this wave's copies of tile j have landed and its
  // LDS reads of tile j-1 have returned, the barrier makes tile j visible to
  // every wave and frees tile j-1's stage, which the copies of tile j+1 then
  // fill while tile j is computed.
  auto step = [&](int j, auto stage_tag) {
    constexpr int st = decltype(stage_tag)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
    if (j + 1 < n) {
      tl.template copy<(st ^ 1) * G::kTileBytes>(k_lds0, k_rsrc, (j + 1) * kTileRows, stride);
      tl.template copy<(st ^ 1) * G::kTileBytes>(v_lds0, v_rsrc, (j + 1) * kTileRows, stride);
    }
    // tiles entirely above the diagonal for all 32 rows of this wave are skipped
    if (!kCausal || j * kTileRows <= wave_q0 + 31 + causal_off) compute(j, stage_tag);
  };
  if (n > 0) {
    tl.template copy<0>(k_lds0, k_rsrc, 0, stride);
    tl.template copy<0>(v_lds0, v_rsrc, 0, stride);
  }
  int j = 0;
  for (; j + 2 <= n; j += 2) {
    step(j, std::integral_constant<int, 0>());
    step(j + 1, std::integral_constant<int, 1>());
  }
  if (j < n) step(j, std::integral_constant<int, 0>());

  if (qi < w.sq) {
    const size_t off = (size_t)(w.q_start + qi) * p.heads * kD + (size_t)w.head * kD;
    store_bf16_rows((bf16_t*)p.dq + off, dqacc, G::kDBlocks, p.scale, half);
  }
}

template <int kD, bool kCausal>
hipError_t launch_bwd_t(const BwdParams& p0, hipStream_t stream) {
  BwdParams p = p0;
  // dQ first: its workgroups also write D and LSE*log2e, which dK/dV reads
  p.n_blocks = (p.max_seqlen_q + kBwdRows - 1) / kBwdRows;
  long long items = (long long)p.batch * p.heads * p.n_blocks;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  if (items > 0)
    hipLaunchKernelGGL((fmha_bwd_dq_kernel<kD, kCausal>), dim3((unsigned)items),
                       dim3(kBwdWaves * 64), 0, stream, p);
  p.n_blocks = (p.max_seqlen_k + kBwdRows - 1) / kBwdRows;
  items = (long long)p.batch * p.heads * p.n_blocks;
  if (items > 0x7fffffffLL) return hipErrorInvalidValue;
  if (items > 0)
    hipLaunchKernelGGL((fmha_bwd_dkdv_kernel<kD, kCausal>), dim3((unsigned)items),
                       dim3(2 * kBwdWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdParams& p, int head_dim, bool causal, hipStream_t stream) {
  if (head_dim == 128)
    return causal ? launch_bwd_t<128, true>(p, stream) : launch_bwd_t<128, false>(p, stream);
  if (head_dim == 64)
    return causal ? launch_bwd_t<64, true>(p, stream) : launch_bwd_t<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace fmha
