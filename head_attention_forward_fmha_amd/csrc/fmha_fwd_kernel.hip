// FMHA forward kernels for gfx950 (MI355X, CDNA4) and their launchers.
//
// The per-wave tile math (Q in registers, S^T = K Q^T and O^T += V^T P^T on
// 32x32 MFMA, exp2-domain online softmax) lives in fmha_device.h. This file
// arranges waves, LDS stages and barriers around it in four ways; the first
// two are the ones the automatic choice takes:
//
//  * fmha_fwd_kernel: 4 waves (128 query rows) per workgroup, two workgroups
//    per CU. Each wave runs copy-wait / Q.K^T / softmax / P.V per tile; the
//    other workgroup on the CU fills the gaps. Used for small problems, where
//    128-row blocks give more workgroups to spread over the 256 CUs.
//
//  * fmha_fwd_pingpong_kernel: 8 waves (256 query rows) per workgroup, one
//    workgroup per CU, two waves per SIMD. The waves form two groups that run
//    half a tile apart in lockstep: while group A issues the MFMA phase of a
//    tile (Q.K^T of tile j and P.V of tile j-1), group B runs the VALU phase
//    (mask, online softmax, P conversion of tile j-1), and the next barrier
//    swaps them. The matrix cores and the vector ALUs of each SIMD are
//    therefore kept busy by different waves at the same time, and the K/V
//    tiles are shared by 256 query rows (half the LDS and L2 traffic per
//    FLOP of the 4-wave kernel).
//
//  * fmha_fwd_pipe_kernel: 4 waves of 32 rows, each software-pipelined over
//    half-tiles of 32 keys (its own MFMAs in flight under its own softmax).
//
//  * fmha_fwd_wide_kernel: 4 waves of 64 rows, one per SIMD, each K and V
//    operand read from LDS feeding two MFMAs, Q and O in the accumulation
//    registers; the same per-wave software pipeline.
//
// Causal launches are persistent (each workgroup walks its XCD's share of the
// work items, see for_each_item); every kernel streams K/V tiles of 64 keys
// through a ring of two or three LDS stages with buffer_load ... lds copies,
// ordered by explicit vmcnt waits and barriers.

#include <algorithm>
#include <atomic>

#include "fmha_device.h"

namespace fmha {

// ---------------------------------------------------------------- split-KV

// Split-KV: split s of num_splits takes key tiles [t0, t1) of the n_tiles the
// work item would visit, t0 = s*n/num_splits. The item's key window is moved
// to start at tile t0 (k_start and sk shrink by the same amount, and so does
// the causal offset sk - sq, so every mask keeps its meaning); the split then
// visits t1 - t0 tiles from there. Returns t1 - t0.
__device__ __forceinline__ int take_split(WorkItem& w, int& causal_off, int n_tiles, int split,
                                          int num_splits) {
  const int t0 = (int)((long long)split * n_tiles / num_splits);
  const int t1 = (int)((long long)(split + 1) * n_tiles / num_splits);
  w.k_start += t0 * kBN;
  w.sk -= t0 * kBN;
  causal_off -= t0 * kBN;
  return t1 - t0;
}

// ---------------------------------------------------------------- 4-wave kernel

constexpr int kWaves4 = 4;
constexpr int kBM4 = kWaves4 * 32;  // query rows per workgroup
static_assert(kBM4 == kRowsFourWave, "4-wave block height");

template <int kD, bool kCausal, int kPv, bool kSplit>
__global__ __attribute__((amdgpu_flat_work_group_size(kWaves4 * 64, kWaves4 * 64),
                          amdgpu_waves_per_eu(2, 2)))
void fmha_fwd_kernel(FwdParams params) {
  using WT = WaveTile<kD, kCausal, kPv, kWaves4>;
  __shared__ __attribute__((aligned(1024))) char smem_k[2][WT::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char smem_v[2][WT::kVStageBytes];

  auto run_item = [&](const FwdParams& p, int item) __attribute__((always_inline)) {
  int split = 0;
  if constexpr (kSplit) {
    split = item % p.num_splits;
    item /= p.num_splits;
  }
  WorkItem w = decode_work_item(p, kBM4, item);
  if (w.m0 >= w.sq) return;  // uniform over the workgroup
  if constexpr (WT::kFp4) align_keys_to_blocks(w);
  int causal_off = w.sk - w.sq;
  int kend = w.sk;
  if (kCausal) kend = min(w.sk, max(0, w.m0 + kBM4 + causal_off));
  int n_tiles = (kend + kBN - 1) / kBN;
  if constexpr (kSplit) n_tiles = take_split(w, causal_off, n_tiles, split, p.num_splits);

  const int wave = threadIdx.x >> 6;
  WT t;
  t.init(p, w, wave, wave);
  t.pin_copy_state();
  // Q has landed before the K/V stream starts (its copies are counted by vmcnt)
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  const uint32_t k_lds0 = lds_address(&smem_k[0][1024 * wave]);
  const uint32_t v_lds0 = lds_address(&smem_v[0][1024 * wave]);

  auto step = [&](int j, auto stage_tag) {
    constexpr int stage = decltype(stage_tag)::value;
    // tile j has landed once only tile j+1's copies can still be in flight
    if (j + 1 < n_tiles) {
      t.template copy_k<stage ^ 1>(j + 1, k_lds0);
      t.template copy_v<stage ^ 1>(j + 1, v_lds0);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(WT::kLoadsPerWave + WT::kVCopyOps));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    }
    __builtin_amdgcn_s_barrier();
    compiler_fence();
    // tiles entirely above the diagonal for all 32 rows of this wave are skipped
    if (t.active(j, causal_off)) {
      t.qk(smem_k[stage]);
      t.softmax(j, w.sk, causal_off);
      t.pv(smem_v[stage]);
    }
    // every wave's reads of this stage have returned before it is refilled
    lds_barrier();
  };

  if (n_tiles > 0) {
    t.template copy_k<0>(0, k_lds0);
    t.template copy_v<0>(0, v_lds0);
  }
  int j = 0;
  for (; j + 2 <= n_tiles; j += 2) {
    step(j, std::integral_constant<int, 0>());
    step(j + 1, std::integral_constant<int, 1>());
  }
  if (j < n_tiles) step(j, std::integral_constant<int, 0>());

  // d = 128: O goes out through this wave's own blocks of K stage 1 (its four
  // 1 KB blocks of that 16 KB stage): every wave's reads ended at the last
  // barrier, and the next item writes them first by this wave's own copies of
  // its tile 1. At d = 64 a stage holds only half the staging, so O is stored
  // from registers.
  if constexpr (kSplit) t.epilogue_partial(p, w, split);
  else if constexpr (kD == 128)
    t.template epilogue_lds<1024 * kWaves4>(p, w, lds_address(&smem_k[1][1024 * wave]));
  else t.epilogue(p, w);
  };
  for_each_item<kCausal, kSplit>(params, run_item);
}

// ---------------------------------------------------------------- 8-wave ping-pong kernel

constexpr int kWaves8 = 8;
constexpr int kBM8 = kWaves8 * 32;  // query rows per workgroup
static_assert(kBM8 == kRowsPingPong, "8-wave block height");
constexpr int kStages8 = 3;         // K/V ring depth

// Phase-boundary hooks of the ping-pong kernel. The forward entry points use
// the no-op version; launch_fwd_trace uses StampTrace.
struct NoPhaseTrace {
  __device__ __forceinline__ void begin(const FwdParams& /*p*/, int /*wave*/) {}
  __device__ __forceinline__ void mark(int /*event*/) {}
};

// Pipeline timeline ("Kernel Bottleneck Tuning", section 2: trace the real
// pipeline, coarsely). Each wave of the first p.trace_wgs workgroups records up
// to kTraceEvents words (event << 56) | (s_memtime mod 2^56) from lane 0; the
// waves of other workgroups start full and record nothing. A stamp (s_memtime)
// is a side-effecting instruction the compiler cannot move work across, so every
// stamp perturbs the schedule a little: the coarse mode keeps to slot and phase
// ends; the detailed mode also splits the phases and lengthens them, and is for
// locating time, not for measuring it.
// The record pointer and count are held in vector registers (the empty asm
// statements pin them there), leaving the kernel's scalar registers alone.
template <bool kDetailed>
struct StampTrace {
  uint32_t out_lo, out_hi;
  int idx;
  __device__ __forceinline__ void begin(const FwdParams& p, int wave) {
    const bool on = (int)blockIdx.x < p.trace_wgs;
    const uint64_t o =
        reinterpret_cast<uint64_t>(p.trace + ((size_t)blockIdx.x * kWaves8 + wave) * kTraceEvents);
    out_lo = (uint32_t)o;
    out_hi = (uint32_t)(o >> 32);
    idx = on ? 0 : kTraceEvents;
    asm volatile("" : "+v"(out_lo), "+v"(out_hi), "+v"(idx));
  }
  __device__ __forceinline__ void mark(int event) {
    if (!kDetailed && (event == kEvQkDone || event == kEvCopyIssued || event == kEvWaitDone))
      return;
    const uint64_t t = __builtin_amdgcn_s_memtime();
    if (idx < kTraceEvents && (threadIdx.x & 63) == 0) {
      uint64_t* out = reinterpret_cast<uint64_t*>(((uint64_t)out_hi << 32) | out_lo);
      out[idx] = ((uint64_t)event << 56) | (t & ((1ull << 56) - 1));
    }
    ++idx;
    asm volatile("" : "+v"(idx));
  }
};

// One work item as the ping-pong kernel runs it: the decoded (document, head,
// query block), its share of the key tiles under split-KV, the number of key
// tiles n, and the causal offset; n < 0 for an item with no query rows.
struct ItemPlan {
  WorkItem w;
  int split, n, causal_off;
};

template <bool kCausal, bool kSplit, bool kFp4>
__device__ __forceinline__ ItemPlan plan_item(const FwdParams& p, int item, int bm) {
  ItemPlan it;
  it.split = 0;
  if constexpr (kSplit) {
    it.split = item % p.num_splits;
    item /= p.num_splits;
  }
  it.w = decode_work_item(p, bm, item);
  it.n = -1;
  it.causal_off = 0;
  if (it.w.m0 >= it.w.sq) return it;
  if constexpr (kFp4) align_keys_to_blocks(it.w);
  it.causal_off = it.w.sk - it.w.sq;
  int kend = it.w.sk;
  if (kCausal) kend = min(it.w.sk, max(0, it.w.m0 + bm + it.causal_off));
  it.n = (kend + kBN - 1) / kBN;
  if constexpr (kSplit) it.n = take_split(it.w, it.causal_off, it.n, it.split, p.num_splits);
  return it;
}

template <int kD, bool kCausal, int kPv, bool kSplit, typename Trace = NoPhaseTrace>
__global__ __attribute__((amdgpu_flat_work_group_size(kWaves8 * 64, kWaves8 * 64),
                          amdgpu_waves_per_eu(2, 2)))
void fmha_fwd_pingpong_kernel(FwdParams params) {
  // each group of 4 waves copies whole tiles, so the tile math is set up for 4
  // copying waves
  using WT = WaveTile<kD, kCausal, kPv, 4>;
  // d = 128 stores O through a private 4 KB LDS block per wave (epilogue_lds);
  // d = 64 and split-KV partials store from registers
  constexpr bool kStageO = kD == 128 && !kSplit;
  __shared__ __attribute__((aligned(1024))) char smem_k[kStages8][WT::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char smem_v[kStages8][WT::kVStageBytes];
  __shared__ __attribute__((aligned(1024))) char smem_o[kStageO ? kWaves8 * 4096 : 1024];

  // The wave index is uniform over the wave; readfirstlane says so, which
  // makes every branch on the group a scalar branch (taken as a divergent one,
  // both groups' paths would share one wave's register allocation).
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Trace trace;
  trace.begin(params, wave);
  const int grp = wave >> 2;  // 0: group A, 1: group B (half a tile behind)
  // 32-row chunks alternate between the groups, which evens out the causal work
  const int row_chunk = 2 * (wave & 3) + grp;
  const uint32_t k_lds0 = lds_address(&smem_k[0][1024 * (wave & 3)]);
  const uint32_t v_lds0 = lds_address(&smem_v[0][1024 * (wave & 3)]);

  // The workgroup's items, skipping those without query rows (uniform over the
  // workgroup). Causal launches are persistent and walk the XCD's share with an
  // ItemCursor, re-reading the parameters per item (kernel_params); the others
  // run the single item their block index names.
  // Each group runs its own copy of the item loop (kGrp): the two follow the
  // same sequence of barriers, and neither's values are live in the other's
  // code, which a branch on the group inside one loop would make them.
  auto run_group = [&](auto g_tag) __attribute__((always_inline)) {
    constexpr int kGrp = decltype(g_tag)::value;
    ItemCursor cursor(kCausal ? n_work_items<kSplit>(params) : 0);
    bool single_pending = true;
    auto next_plan = [&](ItemPlan& it) __attribute__((always_inline)) -> bool {
      if constexpr (kCausal) {
        int item;
        while (cursor.next(item)) {
          it = plan_item<kCausal, kSplit, WT::kFp4>(kernel_params(), item, kBM8);
          if (it.n >= 0) return true;
        }
        return false;
      } else {
        if (!single_pending) return false;
        single_pending = false;
        const int n_items = n_work_items<kSplit>(params);
        const int xcd = blockIdx.x % kXcds;
        const int per = n_items / kXcds, extra = n_items % kXcds;
        it = plan_item<kCausal, kSplit, WT::kFp4>(
            params, xcd * per + min(xcd, extra) + (int)blockIdx.x / kXcds, kBM8);
        return it.n >= 0;
      }
    };
    auto item_params = [&]() -> const FwdParams& {
      if constexpr (kCausal) return kernel_params();
      return params;
    };

    ItemPlan cur;
    if (!next_plan(cur)) return;
    trace.mark(kEvItem);
    WT t;
    t.init(item_params(), cur.w, wave & 3, row_chunk);
    if constexpr (kCausal || WT::kFp4) t.pin_copy_state();
    // first item's prologue: K tiles 0 and 1 and V tile 0
    if constexpr (kGrp == 0) {
      if (cur.n > 0) t.template copy_k<0>(0, k_lds0);
      if (cur.n > 0) t.template copy_v<0>(0, v_lds0);
    } else {
      if (cur.n > 1) t.template copy_k<1>(1, k_lds0);
    }

    for (;;) {
      const int n = cur.n, causal_off = cur.causal_off, sk = cur.w.sk;
      // Schedule. Tile j lives in stage j % 3. Slot 2j: group A runs the MFMA phase
      // of tile j (Q.K^T of tile j, P.V of tile j-1) while group B runs the VALU
      // phase of tile j-1 (mask, softmax, P); slot 2j+1 swaps the roles. Copies are
      // issued only at the start of VALU phases, one group at a time: group B
      // copies K of tile j+2 in slot 2j (its stage's previous K was last read in
      // slot 2j-1), group A copies V of tile j+1 in slot 2j+1 (last read in slot
      // 2j-1). Each group waits for its previous copies at the end of its VALU
      // phase, so tile j's K and V are visible from slot 2j-1 and 2j on.
      // The MFMA phase runs at raised wave priority, so that when both waves of a
      // SIMD have an instruction ready the MFMA issues first and the VALU work of
      // the other group fills the cycles in between.
      auto mfma_phase = [&](int j, auto r_tag) {
        constexpr int r = decltype(r_tag)::value;  // j % 3
        __builtin_amdgcn_s_setprio(2);
        if (j < n && t.active(j, causal_off)) t.qk(smem_k[r]);
        trace.mark(kEvQkDone);
        if (j >= 1 && t.active(j - 1, causal_off)) t.pv(smem_v[(r + 2) % 3]);
        __builtin_amdgcn_s_setprio(0);
        trace.mark(kEvMfmaDone);
      };
      auto valu_phase = [&](int j) {
        if (j >= 0 && j < n && t.active(j, causal_off)) t.softmax(j, sk, causal_off);
      };

      auto slot_pair = [&](int j, auto r_tag) {
        constexpr int r = decltype(r_tag)::value;  // j % 3
        // ---- slot 2j
        if constexpr (kGrp == 0) {
          mfma_phase(j, r_tag);
        } else {
          const bool copy = j + 2 < n;
          if (copy) t.template copy_k<(r + 2) % 3>(j + 2, k_lds0);
          trace.mark(kEvCopyIssued);
          valu_phase(j - 1);
          trace.mark(kEvValuDone);
          // the copies of K tile j+1 (issued in slot 2j-2) have landed
          if (copy) __builtin_amdgcn_s_waitcnt(waitcnt_vm(WT::kLoadsPerWave));
          else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        trace.mark(kEvWaitDone);
        lds_barrier();
        trace.mark(kEvSlot);
        // ---- slot 2j+1
        if constexpr (kGrp == 0) {
          const bool copy = j + 1 < n;
          if (copy) t.template copy_v<(r + 1) % 3>(j + 1, v_lds0);
          trace.mark(kEvCopyIssued);
          valu_phase(j);
          trace.mark(kEvValuDone);
          // the copies of V tile j (issued in slot 2j-1) have landed
          if (copy) __builtin_amdgcn_s_waitcnt(waitcnt_vm(WT::kVCopyOps));
          else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        } else {
          mfma_phase(j, r_tag);
        }
        trace.mark(kEvWaitDone);
        lds_barrier();
        trace.mark(kEvSlot);
      };

      // the item's Q and first copies have landed (for a later item: issued
      // during the previous item's last slot pair and epilogue)
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
      lds_barrier();
      trace.mark(kEvSlot);
      int j = 0;
      for (; j + 3 <= n; j += 3) {
        slot_pair(j, std::integral_constant<int, 0>());
        slot_pair(j + 1, std::integral_constant<int, 1>());
        slot_pair(j + 2, std::integral_constant<int, 2>());
      }
      if (j < n) slot_pair(j, std::integral_constant<int, 0>());
      if (j + 1 < n) slot_pair(j + 1, std::integral_constant<int, 1>());

      // The last slot pair, j = n, runs P.V of tile n-1 (and group B's softmax of
      // it). Every copy of this item has landed (each group waited for its last
      // ones in slot 2n-2 or 2n-1) and no K stage is read again, so the next
      // item's Q loads and its K tiles 0 and 1 are issued now and land under
      // this pair and the epilogue; its V tile 0 follows the pair's last barrier,
      // after which no V stage is read. Nothing in this pair waits for them.
      ItemPlan nxt;
      bool more = false;
      if constexpr (kCausal) {
        more = next_plan(nxt);
        if (!more) nxt = cur;
        // The descriptors switch unconditionally (to the current item's when
        // there is no next one): switched under the branch, the merged values
        // would no longer be known to be uniform and the copies could not take
        // them from scalar registers.
        t.set_copy_source(kernel_params(), nxt.w);
        t.pin_copy_state();
        if (more) {
          t.load_q(kernel_params(), nxt.w, nxt.w.m0 + 32 * row_chunk + t.col);
          if constexpr (kGrp == 0) {
            if (nxt.n > 0) t.template copy_k<0>(0, k_lds0);
          } else {
            if (nxt.n > 1) t.template copy_k<1>(1, k_lds0);
          }
        }
      }
      {
        const char* vs = smem_v[(n + 2) % 3];  // tile n-1's V stage
        const bool pv_last = n >= 1 && t.active(n - 1, causal_off);
        // ---- slot 2n
        if constexpr (kGrp == 0) {
          __builtin_amdgcn_s_setprio(2);
          trace.mark(kEvQkDone);
          if (pv_last) t.pv(vs);
          __builtin_amdgcn_s_setprio(0);
          trace.mark(kEvMfmaDone);
        } else {
          trace.mark(kEvCopyIssued);
          valu_phase(n - 1);
          trace.mark(kEvValuDone);
        }
        trace.mark(kEvWaitDone);
        lds_barrier();
        trace.mark(kEvSlot);
        // ---- slot 2n+1
        if constexpr (kGrp == 0) {
          trace.mark(kEvCopyIssued);
          trace.mark(kEvValuDone);
        } else {
          __builtin_amdgcn_s_setprio(2);
          trace.mark(kEvQkDone);
          if (pv_last) t.pv(vs);
          __builtin_amdgcn_s_setprio(0);
          trace.mark(kEvMfmaDone);
        }
        trace.mark(kEvWaitDone);
        lds_barrier();
        trace.mark(kEvSlot);
      }
      if constexpr (kCausal) {
        if (kGrp == 0 && more && nxt.n > 0) t.template copy_v<0>(0, v_lds0);
      }

      if constexpr (kSplit) t.epilogue_partial(item_params(), cur.w, cur.split);
      else if constexpr (kStageO)
        t.template epilogue_lds<1024>(item_params(), cur.w, lds_address(&smem_o[4096 * wave]));
      else t.epilogue(item_params(), cur.w);

      if (!more) break;
      cur = nxt;
      trace.mark(kEvItem);
      t.begin_rows(cur.w, row_chunk);
    }
  };
  if (grp == 0) run_group(std::integral_constant<int, 0>());
  else run_group(std::integral_constant<int, 1>());
}

// ---------------------------------------------------------------- pipelined kernel

// 4 waves (128 query rows) per workgroup, two workgroups per CU, bf16 only.
// Each wave software-pipelines its own work over half-tiles of 32 keys (see
// WaveTile::step_interleaved): iteration i (one barrier) runs steps 2i-1 and
// 2i, which read K tile i (Q.K^T of half-tiles 2i and 2i+1) and V tile i-1
// (P.V of half-tiles 2i-2 and 2i-1), while the copies of K tile i+1 and V
// tile i fill the other LDS stages.
constexpr int kWavesPipe = 4;
constexpr int kBMPipe = kWavesPipe * 32;
static_assert(kBMPipe == kRowsPipelined, "pipelined block height");

template <int kD, bool kCausal>
__global__ __attribute__((amdgpu_flat_work_group_size(kWavesPipe * 64, kWavesPipe * 64),
                          amdgpu_waves_per_eu(2, 2)))
void fmha_fwd_pipe_kernel(FwdParams params) {
  using WT = WaveTile<kD, kCausal, kPvBf16, kWavesPipe>;
  __shared__ __attribute__((aligned(1024))) char smem_k[2][WT::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char smem_v[2][WT::kVTileBytes];

  auto run_item = [&](const FwdParams& p, int item) __attribute__((always_inline)) {
  const WorkItem w = decode_work_item(p, kBMPipe, item);
  if (w.m0 >= w.sq) return;  // uniform over the workgroup
  const int causal_off = w.sk - w.sq;
  int kend = w.sk;
  if (kCausal) kend = min(w.sk, max(0, w.m0 + kBMPipe + causal_off));
  const int n_half = (kend + 31) / 32;
  const int n_tiles = (kend + kBN - 1) / kBN;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  WT t;
  t.init(p, w, wave, wave);
  t.pin_copy_state();
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // Q has landed before the K/V stream starts
  t.alpha_o = 1.f;
  const uint32_t k_lds0 = lds_address(&smem_k[0][1024 * wave]);
  const uint32_t v_lds0 = lds_address(&smem_v[0][1024 * wave]);

  // copies of iteration i: K tile i+1 and V tile i (stage i % 2 each); they
  // land before iteration i+1
  auto copies = [&](int i) __attribute__((always_inline)) {
    const uint32_t kst1 = (uint32_t)((i + 1) & 1), vst = (uint32_t)(i & 1);
    if (i + 1 < n_tiles)
      t.template copy_k<0>(i + 1, __builtin_amdgcn_readfirstlane(k_lds0 + kst1 * WT::kTileBytes));
    if (i < n_tiles)
      t.template copy_v<0>(i, __builtin_amdgcn_readfirstlane(v_lds0 + vst * WT::kVTileBytes));
  };
  auto finish_iteration = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
  };
  // a step with a piece missing (the first and last ones): the pieces run one
  // after another
  auto step_general = [&](int u, auto par_tag, const char* ks, const char* vs)
                          __attribute__((always_inline)) {
    constexpr int par = decltype(par_tag)::value;
    constexpr int h = par ^ 1;
    t.settle_o();
    if (u >= 1 && u - 1 < n_half) t.template pv_half<h>(vs, t.hp[h]);
    if (u + 1 < n_half) t.template qk_half<h>(ks, t.hs[h]);
    if (u >= 0 && u < n_half) {
      t.mask_half(t.hs[par], u, w.sk, causal_off);
      const float ls = t.exp_half(t.hs[par], t.hp[par]);
      t.settle_half(t.hs[par], t.hp[par], ls);
    }
  };
  // iteration i reads K tile i (stage i % 2) and V tile i-1 (the other stage)
  auto iteration_general = [&](int i) __attribute__((always_inline)) {
    copies(i);
    const char* ks = smem_k[i & 1];
    const char* vs = smem_v[(i & 1) ^ 1];
    step_general(2 * i - 1, std::integral_constant<int, 1>(), ks, vs);
    step_general(2 * i, std::integral_constant<int, 0>(), ks, vs);
    finish_iteration();
  };
  // steady state: both steps have all three pieces
  auto iteration_steady = [&](int i, auto kstage_tag) __attribute__((always_inline)) {
    constexpr int kst = decltype(kstage_tag)::value;  // i % 2
    copies(i);
    t.settle_o();
    t.mask_half(t.hs[1], 2 * i - 1, w.sk, causal_off);
    float ls = t.template step_interleaved<1>(smem_k[kst], smem_v[kst ^ 1]);
    t.settle_half(t.hs[1], t.hp[1], ls);
    t.settle_o();
    t.mask_half(t.hs[0], 2 * i, w.sk, causal_off);
    ls = t.template step_interleaved<0>(smem_k[kst], smem_v[kst ^ 1]);
    t.settle_half(t.hs[0], t.hp[0], ls);
    finish_iteration();
  };

  if (n_tiles > 0) {
    t.template copy_k<0>(0, k_lds0);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
    // iterations 0 .. ceil(n_half / 2); the last one holds the final P.V.
    // Iterations 1 .. last_steady have every piece of both steps.
    const int n_iter = (n_half + 1) / 2 + 1;
    const int last_steady = (n_half - 2) / 2;
    iteration_general(0);
    int i = 1;
    for (; i + 1 <= last_steady; i += 2) {
      iteration_steady(i, std::integral_constant<int, 1>());
      iteration_steady(i + 1, std::integral_constant<int, 0>());
    }
    if (i <= last_steady) {
      iteration_steady(i, std::integral_constant<int, 1>());
      ++i;
    }
    for (; i < n_iter; ++i) iteration_general(i);
  }

  t.epilogue(p, w);
  };
  for_each_item<kCausal, false>(params, run_item);
}

// ---------------------------------------------------------------- 64-row-wave kernel

// 4 waves (256 query rows) per workgroup, one workgroup per CU, one wave per
// SIMD with up to 512 registers. Each wave owns two 32-row blocks of the work
// item, blocks w and 7 - w (so that under a causal mask every wave has the
// same work), and gives every K and V operand it reads from LDS to two MFMAs,
// one per block: half the LDS bytes per MFMA of the 32-row kernels. The wave
// software-pipelines its work over half-tiles of 32 keys as the pipelined
// kernel does: step u runs the softmax of half-tile u (vector ALU) beside the
// Q.K^T MFMAs of half-tile u+1 and then the P.V MFMAs of half-tile u-1.
//
// Register files. Q (the B operand of S^T = K Q^T) and O^T (the accumulator
// of O^T += V^T P^T) live in the accumulation registers (AGPRs), S^T and P in
// the vector registers (VGPRs). The MFMAs are inline asm so that each operand
// is read from and written to the file it lives in, without copies between
// the files. The compiler therefore does not see them: the wait states the
// ISA requires between an MFMA and a later instruction that reads or
// overwrites its result, or between a vector write of an operand and the MFMA
// that reads it, come from the schedule (in a steady step, the 16 P.V MFMAs
// issued after the last Q.K^T MFMA of a half-tile keep its S from being read
// before the next step) or from mfma_settle (24 wait states, more than the
// ISA's hazard tables ask for after these MFMAs) where the schedule does not
// provide them.
constexpr int kWavesWide = 4;
constexpr int kBMWide = kWavesWide * 64;  // query rows per workgroup
static_assert(kBMWide == kRowsWide, "64-row-wave block height");
constexpr int kStagesWide = 3;            // K/V ring depth
typedef bf16_t bf16x2 __attribute__((ext_vector_type(2)));

// S^T = K Q^T (first d step: zero accumulator) and S^T += K Q^T
__device__ __forceinline__ void mfma_s_first(f32x16& s, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mfma_s(f32x16& s, const bf16x8& k, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "a"(q));
}
// O^T += V^T P^T, O^T in AGPRs
__device__ __forceinline__ void mfma_o(f32x16& o, const bf16x8& v, const bf16x8& p) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(v), "v"(p));
}

// 24 wait states after the asm MFMAs issued so far, ordered (through the
// operands, which the statement claims to read and write) before every later
// access of the named registers by the compiler's own instructions.
#define FMHA_MFMA_SETTLE "s_nop 7\n\ts_nop 7\n\ts_nop 7"

template <class WT>
__device__ __forceinline__ void mfma_settle_o(WT& a, WT& b) {
  static_assert(WT::kDBlocks == 4 || WT::kDBlocks == 2, "head_dim 128 or 64");
  if constexpr (WT::kDBlocks == 4)
    asm volatile(FMHA_MFMA_SETTLE
                 : "+a"(a.oacc[0]), "+a"(a.oacc[1]), "+a"(a.oacc[2]), "+a"(a.oacc[3]),
                   "+a"(b.oacc[0]), "+a"(b.oacc[1]), "+a"(b.oacc[2]), "+a"(b.oacc[3]));
  else
    asm volatile(FMHA_MFMA_SETTLE
                 : "+a"(a.oacc[0]), "+a"(a.oacc[1]), "+a"(b.oacc[0]), "+a"(b.oacc[1]));
}
template <class WT>
__device__ __forceinline__ void mfma_settle_s(WT& a, WT& b, int set) {
  if (set == 0) asm volatile(FMHA_MFMA_SETTLE : "+v"(a.hs[0]), "+v"(b.hs[0]));
  else asm volatile(FMHA_MFMA_SETTLE : "+v"(a.hs[1]), "+v"(b.hs[1]));
}
// Q (written by the compiler's loads and moves) before the first Q.K^T MFMA of
// an item, and the zeroed O before its first P.V MFMA
template <class WT>
__device__ __forceinline__ void mfma_settle_q(WT& a, WT& b) {
  static_assert(WT::kKSteps == 8 || WT::kKSteps == 4, "head_dim 128 or 64");
  if constexpr (WT::kKSteps == 8) {
    asm volatile(FMHA_MFMA_SETTLE
                 : "+a"(a.qreg[0]), "+a"(a.qreg[1]), "+a"(a.qreg[2]), "+a"(a.qreg[3]),
                   "+a"(a.qreg[4]), "+a"(a.qreg[5]), "+a"(a.qreg[6]), "+a"(a.qreg[7]));
    asm volatile(FMHA_MFMA_SETTLE
                 : "+a"(b.qreg[0]), "+a"(b.qreg[1]), "+a"(b.qreg[2]), "+a"(b.qreg[3]),
                   "+a"(b.qreg[4]), "+a"(b.qreg[5]), "+a"(b.qreg[6]), "+a"(b.qreg[7]));
  } else {
    asm volatile(FMHA_MFMA_SETTLE
                 : "+a"(a.qreg[0]), "+a"(a.qreg[1]), "+a"(a.qreg[2]), "+a"(a.qreg[3]),
                   "+a"(b.qreg[0]), "+a"(b.qreg[1]), "+a"(b.qreg[2]), "+a"(b.qreg[3]));
  }
  mfma_settle_o(a, b);
}

// S^T of half kH of the K tile at ks into hs[kH] of both blocks: one K operand
// read per d step, two MFMAs on it. Reads run two steps ahead.
template <int kH, class WT>
__device__ __forceinline__ void wide_qk(WT& a, WT& b, const char* ks) {
  constexpr int kN = WT::kKSteps;
  bf16x8 ka[3];
  auto rk = [&](int t) {
    ka[t % 3] = *(const bf16x8*)(ks + a.k_off[t] + kH * 32 * WT::kRowBytes);
  };
  rk(0);
  rk(1);
#pragma unroll
  for (int t = 0; t < kN; ++t) {
    if (t + 2 < kN) rk(t + 2);
    if (t == 0) {
      mfma_s_first(a.hs[kH], ka[0], a.qreg[0]);
      mfma_s_first(b.hs[kH], ka[0], b.qreg[0]);
    } else {
      mfma_s(a.hs[kH], ka[t % 3], a.qreg[t]);
      mfma_s(b.hs[kH], ka[t % 3], b.qreg[t]);
    }
  }
}

// O^T += V^T P^T of half kH of the V tile at vs for both blocks (P in hp[kH]):
// one transposed V operand read per (16-key step, d block), two MFMAs on it.
template <int kH, class WT>
__device__ __forceinline__ void wide_pv(WT& a, WT& b, const char* vs) {
  constexpr int kN = WT::kHalfPv;
  bf16x8 va[3];
  va[0] = a.template read_v_half<kH>(vs, 0);
  va[1] = a.template read_v_half<kH>(vs, 1);
#pragma unroll
  for (int t = 0; t < kN; ++t) {
    if (t + 2 < kN) va[(t + 2) % 3] = a.template read_v_half<kH>(vs, t + 2);
    mfma_o(a.oacc[t % WT::kDBlocks], va[t % 3], a.hp[kH][t / WT::kDBlocks]);
    mfma_o(b.oacc[t % WT::kDBlocks], va[t % 3], b.hp[kH][t / WT::kDBlocks]);
  }
}

// A pending rescale of O (alpha_o != 1 in a lane of either block), after every
// P.V MFMA issued so far.
template <class WT>
__device__ __forceinline__ void wide_settle_o(WT& a, WT& b) {
  if (__builtin_amdgcn_ballot_w64(a.alpha_o != 1.f || b.alpha_o != 1.f) != 0) {
    mfma_settle_o(a, b);
#pragma unroll
    for (int db = 0; db < WT::kDBlocks; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        a.oacc[db][i] *= a.alpha_o;
        b.oacc[db][i] *= b.alpha_o;
      }
    mfma_settle_o(a, b);
    a.alpha_o = 1.f;
    b.alpha_o = 1.f;
  }
}

// The softmax arithmetic of one block's 16 scores of a half-tile, cut into
// three stages that a steady step spreads over its MFMAs: stage 0 of score i
// is the folded FMA, stage 1 its exp2, stage 2 the partial sum and, with an
// odd i, the bf16 pack of scores (i-1, i). Slot k runs stage 0 of score k+1,
// stage 1 of score k and stage 2 of score k-1, three independent instructions
// whose inputs were produced a slot (an MFMA) earlier: with one wave per SIMD
// no other wave hides the latency of a dependent chain. The empty asm
// statements keep each result at its slot: left alone, the compiler sinks the
// arithmetic of a block whose results are first used after a branch to behind
// that branch, out of the MFMA stream.
template <int kPar, class WT>
struct ScoreChain {
  WT& t;
  float c, nm;
  float rs[4] = {0.f, 0.f, 0.f, 0.f};
  float x[16];
  float e[16];
  __device__ __forceinline__ ScoreChain(WT& tile, float c_) : t(tile), c(c_) {
    nm = (t.m_run == -__builtin_inff()) ? 0.f : -t.m_run * c;
  }
  __device__ __forceinline__ void fma(int i) {
    x[i] = __builtin_fmaf(t.hs[kPar][i], c, nm);
    asm volatile("" : "+v"(x[i]));
  }
  __device__ __forceinline__ void exp(int i) {
    e[i] = __builtin_amdgcn_exp2f(x[i]);
    asm volatile("" : "+v"(e[i]));
  }
  __device__ __forceinline__ void sum(int i) {
    rs[i & 3] = (i < 4) ? e[i] : rs[i & 3] + e[i];
    asm volatile("" : "+v"(rs[i & 3]));
    if (i & 1) {
      bf16x2 pr = {(bf16_t)e[i - 1], (bf16_t)e[i]};
      asm volatile("" : "+v"(pr));
      t.hp[kPar][i / 8][(i % 8) - 1] = pr[0];
      t.hp[kPar][i / 8][i % 8] = pr[1];
    }
  }
  // slot k of 16 (k = -1: the stage 0 of score 0 before the first slot; k = 16,
  // 17: what remains after the last one)
  __device__ __forceinline__ void slot(int k) {
    if (k + 1 >= 0 && k + 1 < 16) fma(k + 1);
    if (k >= 0 && k < 16) exp(k);
    if (k - 1 >= 0 && k - 1 < 16) sum(k - 1);
  }
  __device__ __forceinline__ float total() const { return (rs[0] + rs[1]) + (rs[2] + rs[3]); }
};

// Steady step u (kPar = u & 1): Q.K^T of half-tile u+1 (half kPar^1 of the K
// tile at ks), then P.V of half-tile u-1 (half kPar^1 of the V tile at vs),
// with the softmax of half-tile u spread over both (ScoreChain), the same
// number of slots of one block after each MFMA of that block. Returns the two
// blocks' partial row sums of half-tile u.
template <int kPar, class WT>
__device__ __forceinline__ float2 wide_step(WT& a, WT& b, const char* ks, const char* vs) {
  constexpr int kH = kPar ^ 1;
  constexpr int kN = WT::kKSteps;
  static_assert(WT::kHalfPv == kN, "Q.K^T and P.V steps pair up one to one");
  constexpr int kR = 8 / kN;   // slots of a block per MFMA of that block
  ScoreChain<kPar, WT> sa(a, a.c), sb(b, b.c);
  auto slots = [&](ScoreChain<kPar, WT>& sc, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int k = k0; k < k0 + kR; ++k) sc.slot(k);
  };
  bf16x8 ka[3], va[3];
  auto rk = [&](int t) {
    ka[t % 3] = *(const bf16x8*)(ks + a.k_off[t] + kH * 32 * WT::kRowBytes);
  };
  auto rv = [&](int t) { va[t % 3] = a.template read_v_half<kH>(vs, t); };
  rk(0);
  rk(1);
  sa.slot(-1);
  sb.slot(-1);
#pragma unroll
  for (int t = 0; t < kN; ++t) {
    if (t + 2 < kN) rk(t + 2);
    if (t == kN - 2) rv(0);
    if (t == kN - 1) rv(1);
    if (t == 0) mfma_s_first(a.hs[kH], ka[0], a.qreg[0]);
    else mfma_s(a.hs[kH], ka[t % 3], a.qreg[t]);
    slots(sa, kR * t);
    __builtin_amdgcn_sched_barrier(0);
    if (t == 0) mfma_s_first(b.hs[kH], ka[0], b.qreg[0]);
    else mfma_s(b.hs[kH], ka[t % 3], b.qreg[t]);
    slots(sb, kR * t);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int t = 0; t < kN; ++t) {
    if (t + 2 < kN) rv(t + 2);
    mfma_o(a.oacc[t % WT::kDBlocks], va[t % 3], a.hp[kH][t / WT::kDBlocks]);
    slots(sa, 8 + kR * t);
    __builtin_amdgcn_sched_barrier(0);
    mfma_o(b.oacc[t % WT::kDBlocks], va[t % 3], b.hp[kH][t / WT::kDBlocks]);
    slots(sb, 8 + kR * t);
    __builtin_amdgcn_sched_barrier(0);
  }
  sa.slot(16);
  sb.slot(16);
  sa.slot(17);
  sb.slot(17);
  return make_float2(sa.total(), sb.total());
}

template <int kD, bool kCausal>
__global__ __attribute__((amdgpu_flat_work_group_size(kWavesWide * 64, kWavesWide * 64),
                          amdgpu_waves_per_eu(1, 1)))
void fmha_fwd_wide_kernel(FwdParams params) {
  using WT = WaveTile<kD, kCausal, kPvBf16, kWavesWide>;
  // d = 128 stores O through a private 4 KB LDS block per wave (epilogue_lds)
  constexpr bool kStageO = kD == 128;
  __shared__ __attribute__((aligned(1024))) char smem_k[kStagesWide][WT::kTileBytes];
  __shared__ __attribute__((aligned(1024))) char smem_v[kStagesWide][WT::kVTileBytes];
  __shared__ __attribute__((aligned(1024))) char smem_o[kStageO ? kWavesWide * 4096 : 1024];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t k_lds0 = lds_address(&smem_k[0][1024 * wave]);
  const uint32_t v_lds0 = lds_address(&smem_v[0][1024 * wave]);

  auto run_item = [&](const FwdParams& p, int item) __attribute__((always_inline)) {
  const WorkItem w = decode_work_item(p, kBMWide, item);
  if (w.m0 >= w.sq) return;  // uniform over the workgroup
  const int causal_off = w.sk - w.sq;
  int kend = w.sk;
  if (kCausal) kend = min(w.sk, max(0, w.m0 + kBMWide + causal_off));
  const int n_half = (kend + 31) / 32;
  const int n_tiles = (kend + kBN - 1) / kBN;

  // block a: rows 32*wave .. +31 of the item (this wave's copies too), block b:
  // rows 32*(7 - wave) .. +31
  WT ta, tb;
  ta.init(p, w, wave, wave);
  ta.pin_copy_state();
  tb.init_lanes(p);
  tb.begin_rows(w, 2 * kWavesWide - 1 - wave);
  tb.load_q(p, w, tb.qi);
  ta.alpha_o = 1.f;
  tb.alpha_o = 1.f;
  // lane-half tests are formed per item, not hoisted out of the item loop into
  // scalar registers held across it
  asm volatile("" : "+v"(ta.half), "+v"(tb.half));

  // the copies of iteration i: K tile i+2 and V tile i+1 (stages (i+2) % 3 and
  // (i+1) % 3, read last in iteration i-1); they land before iteration i+1 ends.
  // Returns the number of copy instructions issued.
  auto copies_rt = [&](int i) __attribute__((always_inline)) -> int {
    int ops = 0;
    if (i + 2 < n_tiles) {
      ta.template copy_k<0>(i + 2, __builtin_amdgcn_readfirstlane(
                                       k_lds0 + (uint32_t)((i + 2) % kStagesWide) * WT::kTileBytes));
      ops += WT::kLoadsPerWave;
    }
    if (i + 1 < n_tiles) {
      ta.template copy_v<0>(i + 1, __builtin_amdgcn_readfirstlane(
                                       v_lds0 + (uint32_t)((i + 1) % kStagesWide) * WT::kVTileBytes));
      ops += WT::kVLoadsPerWave;
    }
    return ops;
  };
  // end of an iteration: this wave's copies from the previous one have landed,
  // then every wave's (and every wave's reads of this iteration are done)
  auto finish_iteration = [&](bool k_copy, bool v_copy) __attribute__((always_inline)) {
    if (k_copy && v_copy) __builtin_amdgcn_s_waitcnt(waitcnt_vm(WT::kLoadsPerWave + WT::kVLoadsPerWave));
    else if (k_copy) __builtin_amdgcn_s_waitcnt(waitcnt_vm(WT::kLoadsPerWave));
    else if (v_copy) __builtin_amdgcn_s_waitcnt(waitcnt_vm(WT::kVLoadsPerWave));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
  };
  // a step with a piece missing (the first and last ones of an item): the
  // pieces one after another, with the MFMA wait states made explicit
  auto step_general = [&](int u, auto par_tag, const char* ks, const char* vs)
                          __attribute__((always_inline)) {
    constexpr int par = decltype(par_tag)::value;
    constexpr int h = par ^ 1;
    wide_settle_o(ta, tb);
    if (u >= 1 && u - 1 < n_half) {
      asm volatile(FMHA_MFMA_SETTLE : "+v"(ta.hp[h][0]), "+v"(ta.hp[h][1]), "+v"(tb.hp[h][0]),
                   "+v"(tb.hp[h][1]));
      wide_pv<h>(ta, tb, vs);
    }
    if (u + 1 < n_half) wide_qk<h>(ta, tb, ks);
    if (u >= 0 && u < n_half) {
      mfma_settle_s(ta, tb, par);
      ta.mask_half(ta.hs[par], u, w.sk, causal_off);
      tb.mask_half(tb.hs[par], u, w.sk, causal_off);
      const float la = ta.exp_half(ta.hs[par], ta.hp[par]);
      const float lb = tb.exp_half(tb.hs[par], tb.hp[par]);
      ta.settle_half(ta.hs[par], ta.hp[par], la);
      tb.settle_half(tb.hs[par], tb.hp[par], lb);
    }
  };
  // iteration i reads K tile i (stage i % 3) and V tile i-1 (stage (i+2) % 3)
  auto iteration_general = [&](int i) __attribute__((always_inline)) {
    const bool k_copy = i + 2 < n_tiles, v_copy = i + 1 < n_tiles;
    copies_rt(i);
    const char* ks = smem_k[i % kStagesWide];
    const char* vs = smem_v[(i + 2) % kStagesWide];
    step_general(2 * i - 1, std::integral_constant<int, 1>(), ks, vs);
    step_general(2 * i, std::integral_constant<int, 0>(), ks, vs);
    finish_iteration(k_copy, v_copy);
  };
  // steady state: both steps have all three pieces; kSt = i % 3
  auto iteration_steady = [&](int i, auto st_tag) __attribute__((always_inline)) {
    constexpr int kSt = decltype(st_tag)::value;
    const bool k_copy = i + 2 < n_tiles, v_copy = i + 1 < n_tiles;
    if (k_copy) ta.template copy_k<(kSt + 2) % kStagesWide>(i + 2, k_lds0);
    if (v_copy) ta.template copy_v<(kSt + 1) % kStagesWide>(i + 1, v_lds0);
    const char* ks = smem_k[kSt];
    const char* vs = smem_v[(kSt + 2) % kStagesWide];
    wide_settle_o(ta, tb);
    ta.mask_half(ta.hs[1], 2 * i - 1, w.sk, causal_off);
    tb.mask_half(tb.hs[1], 2 * i - 1, w.sk, causal_off);
    float2 ls = wide_step<1>(ta, tb, ks, vs);
    ta.settle_half(ta.hs[1], ta.hp[1], ls.x);
    tb.settle_half(tb.hs[1], tb.hp[1], ls.y);
    wide_settle_o(ta, tb);
    ta.mask_half(ta.hs[0], 2 * i, w.sk, causal_off);
    tb.mask_half(tb.hs[0], 2 * i, w.sk, causal_off);
    ls = wide_step<0>(ta, tb, ks, vs);
    ta.settle_half(ta.hs[0], ta.hp[0], ls.x);
    tb.settle_half(tb.hs[0], tb.hp[0], ls.y);
    finish_iteration(k_copy, v_copy);
  };

  if (n_tiles > 0) {
    // prologue: K tiles 0 and 1, V tile 0; Q and K tile 0 land first
    ta.template copy_k<0>(0, k_lds0);
    if (n_tiles > 1) ta.template copy_k<1>(1, k_lds0);
    ta.template copy_v<0>(0, v_lds0);
    if (n_tiles > 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(WT::kLoadsPerWave + WT::kVLoadsPerWave));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(WT::kVLoadsPerWave));
    mfma_settle_q(ta, tb);
    lds_barrier();
    // iterations 0 .. ceil(n_half / 2); the last one holds the final P.V.
    // Iterations 1 .. last_steady have every piece of both steps.
    const int n_iter = (n_half + 1) / 2 + 1;
    const int last_steady = (n_half - 2) / 2;
    iteration_general(0);
    int i = 1;
    for (; i + 2 <= last_steady; i += 3) {
      iteration_steady(i, std::integral_constant<int, 1>());
      iteration_steady(i + 1, std::integral_constant<int, 2>());
      iteration_steady(i + 2, std::integral_constant<int, 0>());
    }
    if (i <= last_steady) {
      iteration_steady(i, std::integral_constant<int, 1>());
      ++i;
    }
    if (i <= last_steady) {
      iteration_steady(i, std::integral_constant<int, 2>());
      ++i;
    }
    for (; i < n_iter; ++i) iteration_general(i);
  }

  mfma_settle_o(ta, tb);
  if constexpr (kStageO) {
    ta.template epilogue_lds<1024>(p, w, lds_address(&smem_o[4096 * wave]));
    tb.template epilogue_lds<1024>(p, w, lds_address(&smem_o[4096 * wave]));
  } else {
    ta.epilogue(p, w);
    tb.epilogue(p, w);
  }
  };
  for_each_item<kCausal, false>(params, run_item);
}

// ---------------------------------------------------------------- launchers

// Compute units of the current device (cached per device; the attribute query
// is a host call).
static int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <int kD, bool kCausal, int kPv, bool kSplit = false>
static hipError_t launch(const FwdParams& p, int variant, hipStream_t stream) {
  FwdParams q = p;
  if (!kSplit) q.num_splits = 1;
  const int variant_run = resolve_variant(variant, p.batch, p.max_seqlen_q, p.heads, q.num_splits);
  const bool use8 = variant_run == kVariantPingPong;
  const bool one_per_cu = use8 || variant_run == kVariantWide;
  const int bm = use8 ? kBM8 : variant_run == kVariantWide ? kBMWide : kBM4;
  q.n_mblocks = (p.max_seqlen_q + bm - 1) / bm;
  const long long n_items = (long long)q.n_mblocks * p.heads * p.batch * q.num_splits;
  if (n_items == 0) return hipSuccess;
  if (n_items > 0x7fffffffLL) return hipErrorInvalidValue;
  // causal kernels are persistent: as many workgroups as the chip holds at once
  // (one per CU for the 8-wave kernel, two for the 4-wave ones), a multiple of
  // the XCD count; the others take one item per workgroup
  const long long resident = (long long)device_cus() * (one_per_cu ? 1 : 2);
  const long long grid =
      kCausal ? (std::min(n_items, resident) + kXcds - 1) / kXcds * kXcds : n_items;
  if (variant_run == kVariantPipelined) {
    if constexpr (kPv == kPvBf16 && !kSplit)
      hipLaunchKernelGGL((fmha_fwd_pipe_kernel<kD, kCausal>), dim3((unsigned)grid),
                         dim3(kWavesPipe * 64), 0, stream, q);
    else
      return hipErrorInvalidValue;
  } else if (variant_run == kVariantWide) {
    if constexpr (kPv == kPvBf16 && !kSplit)
      hipLaunchKernelGGL((fmha_fwd_wide_kernel<kD, kCausal>), dim3((unsigned)grid),
                         dim3(kWavesWide * 64), 0, stream, q);
    else
      return hipErrorInvalidValue;
  } else if (use8)
    hipLaunchKernelGGL((fmha_fwd_pingpong_kernel<kD, kCausal, kPv, kSplit>),
                       dim3((unsigned)grid), dim3(kWaves8 * 64), 0, stream, q);
  else
    hipLaunchKernelGGL((fmha_fwd_kernel<kD, kCausal, kPv, kSplit>), dim3((unsigned)grid),
                       dim3(kWaves4 * 64), 0, stream, q);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdParams& p, int head_dim, bool causal, int variant,
                           hipStream_t stream) {
  if (head_dim == 128)
    return causal ? launch<128, true, kPvBf16>(p, variant, stream)
                  : launch<128, false, kPvBf16>(p, variant, stream);
  return causal ? launch<64, true, kPvBf16>(p, variant, stream)
                : launch<64, false, kPvBf16>(p, variant, stream);
}

hipError_t launch_fwd_fp8pv(const FwdParams& p, int head_dim, bool causal, int variant,
                            hipStream_t stream) {
  if (head_dim != 128) return hipErrorInvalidValue;
  return causal ? launch<128, true, kPvE4m3>(p, variant, stream)
                : launch<128, false, kPvE4m3>(p, variant, stream);
}

hipError_t launch_fwd_fp4pv(const FwdParams& p, int head_dim, bool causal, int variant,
                            hipStream_t stream) {
  if (head_dim != 128) return hipErrorInvalidValue;
  return causal ? launch<128, true, kPvE2m1>(p, variant, stream)
                : launch<128, false, kPvE2m1>(p, variant, stream);
}

hipError_t launch_fwd_trace(const FwdParams& p, int pv, bool causal, bool detailed,
                            hipStream_t stream) {
  FwdParams q = p;
  q.num_splits = 1;
  q.n_mblocks = (p.max_seqlen_q + kBM8 - 1) / kBM8;
  const long long n_items = (long long)q.n_mblocks * p.heads * p.batch;
  if (n_items == 0) return hipSuccess;
  if (n_items > 0x7fffffffLL) return hipErrorInvalidValue;
  const long long grid = (std::min(n_items, (long long)device_cus()) + kXcds - 1) / kXcds * kXcds;
  const dim3 g((unsigned)grid), b(kWaves8 * 64);
#define FMHA_TRACE_LAUNCH(PV, CAUSAL)                                                              \
  do {                                                                                             \
    if (detailed)                                                                                  \
      hipLaunchKernelGGL((fmha_fwd_pingpong_kernel<128, CAUSAL, PV, false, StampTrace<true>>), g, b, \
                         0, stream, q);                                                            \
    else                                                                                           \
      hipLaunchKernelGGL((fmha_fwd_pingpong_kernel<128, CAUSAL, PV, false, StampTrace<false>>), g, \
                         b, 0, stream, q);                                                         \
  } while (0)
  if (!causal) return hipErrorInvalidValue;   // tracing covers the persistent (causal) launches
  if (pv == kPvBf16)
    FMHA_TRACE_LAUNCH(kPvBf16, true);
  else if (pv == kPvE4m3)
    FMHA_TRACE_LAUNCH(kPvE4m3, true);
  else if (pv == kPvE2m1)
    FMHA_TRACE_LAUNCH(kPvE2m1, true);
  else
    return hipErrorInvalidValue;
#undef FMHA_TRACE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_fwd_bf16_splitkv(const FwdParams& p, int head_dim, bool causal, int variant,
                                   hipStream_t stream) {
  if (p.num_splits < 1 || p.num_splits > kMaxSplits) return hipErrorInvalidValue;
  if (head_dim == 128)
    return causal ? launch<128, true, kPvBf16, true>(p, variant, stream)
                  : launch<128, false, kPvBf16, true>(p, variant, stream);
  return causal ? launch<64, true, kPvBf16, true>(p, variant, stream)
                : launch<64, false, kPvBf16, true>(p, variant, stream);
}

// Split count for a problem: the one that minimises the estimated time
//   rounds(S) * (tiles / S + kOverheadTiles) * tile_us + merge_us(S)   (S > 1)
// where rounds(S) is how many times the resident workgroups must be refilled
// to run items * S work items, tile_us the time of one 64-key step of a work
// item with the device full (about 4 TFLOP/s per compute unit), kOverheadTiles
// a work item's prologue and epilogue, and merge_us the merge pass (reading S
// fp32 partial rows at about 5 TB/s). A split must beat the unsplit estimate by
// 15%: a partly idle device runs each busy compute unit faster than the model
// assumes, which favours not splitting.
int recommended_splits(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                       int32_t heads, bool causal, int variant) {
  if (batch <= 0 || max_seqlen_q <= 0 || max_seqlen_k <= 0 || heads <= 0) return 1;
  // a causal item visits half the keys on average
  const double tiles = (double)((max_seqlen_k + kBN - 1) / kBN) / (causal ? 2.0 : 1.0);
  const double d = 128.0;   // tile and merge times both scale with head_dim
  const double rows = (double)batch * max_seqlen_q * heads;
  constexpr double kOverheadTiles = 3.5;
  // estimated time of s splits, on the kernel the launch would pick for them
  auto cost = [&](int s) {
    const int v = resolve_variant(variant, batch, max_seqlen_q, heads, s);
    const bool use8 = v == kVariantPingPong;
    const int bm = use8 ? kBM8 : kBM4;
    const int wgs_per_cu = use8 ? 1 : 2;
    const long long slots = (long long)device_cus() * wgs_per_cu;
    const long long items = (long long)(max_seqlen_q + bm - 1) / bm * heads * batch * s;
    const double tile_us = 4.0 * bm * kBN * d * wgs_per_cu / 4.0e12 * 1e6;
    const double rounds = (double)((items + slots - 1) / slots);
    const double merge_us = s > 1 ? 3.0 + rows * d * 4.0 * (s + 0.5) / 5.0e12 * 1e6 : 0.0;
    return rounds * (tiles / s + kOverheadTiles) * tile_us + merge_us;
  };
  const double unsplit = cost(1);
  int best = 1;
  double best_cost = unsplit;
  for (int s = 2; s <= 16 && s <= tiles; ++s) {
    const double c = cost(s);
    if (c < best_cost && c < 0.85 * unsplit) {
      best = s;
      best_cost = c;
    }
  }
  return best;
}

}  // namespace fmha
