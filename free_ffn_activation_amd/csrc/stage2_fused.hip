// Stage 2 of a batch-1 decode step in one launch on gfx950: the exact up/gate
// gather with the fused activation product, then the sparse down projection,
// joined by an in-kernel grid barrier.
//
// Method ([blog] = deep-dive blog "Prox 完全拆解", section "Stage 2"):
//   u_sp = Pi^out(x, W_up, m_s), h_sp = SiLU(Pi^out(x, W_gate, m_s)),
//   s_sp = u_sp * h_sp, y = Pi^in(s_sp, W_down, m_s)  ([paper] section 2.2)
// (GELU in place of SiLU for a GeGLU layer).  The same mask m_s selects the
// up/gate outputs and the down rows, and it is known from Stage 1 before
// Stage 2 starts; only the values s_j are produced inside Stage 2.
//
// gfx950 design:
//   * one block of 1024 threads per CU: grid = the CU count, launched
//     cooperatively so that every block is resident at once (the host also
//     checks the occupancy first, and every wait below is bounded).  16 waves
//     per block, 4 per SIMD.
//   * phase A is the up/gate kernel's work (s2::upgate_block) over all the
//     grid's waves: s_j by channel index, the ascending index list, k_s, and
//     the zeros of y, all written with agent-coherent stores.
//   * phase B is the down kernel's work: block b takes (column slice, row
//     group) items b, b + G, ...; an item's rows are the kept channels of its
//     channel range, read from the Stage-1 bitmap.  Each block compacts its
//     first item's rows and issues its first batch of W_down loads *before* the
//     grid barrier: the down weight stream overlaps the barrier and the other
//     blocks' up/gate tail, and only the s_j values wait.  (Measured on
//     MI355X: a kernel boundary costs 1.6 us, an in-kernel grid barrier 2.8 us;
//     the barrier pays only if it hides behind those loads.)
//   * ordering: gfx9-family hardware retires vector memory operations in
//     issue order on one counter (vmcnt), so after issuing its W_down loads a
//     thread waits with vmcnt(kDownUnroll) — its phase-A stores are then
//     complete while the loads stay in flight — and the block passes a
//     barrier before its flag store.  Barrier: block b stores flags[b] = its
//     epoch (agent-coherent); one wave of each block with down work polls all
//     flags with agent-coherent loads.  Epochs: every block reads its own flag
//     at the start (all flags are equal between calls, zero in a fresh
//     workspace) and adds one.  s_j is read after the barrier with
//     agent-coherent loads.
//   * a block whose wait exceeds the wait limit (ticks of the 100 MHz real-
//     time clock) gives up: it sets the workspace error word and skips its
//     down work, so the kernel always ends; the host reports the error word
//     (prox_workspace_check).  k_s is published once per launch, by the last
//     block to finish (a completion ticket): -1 if any block gave up.
#include "stage2_common.h"

namespace prox {
namespace {

constexpr int kFusedWaves = kFusedThreads / 64;

template <typename T>
__global__ __launch_bounds__(kFusedThreads) void stage2_fused_kernel(FusedArgs a) {
  typedef typename T::storage S;
  constexpr int kEpl = 16 / sizeof(S);
  constexpr int kCw = 64 * kEpl;  // columns per down column slice
  constexpr int kWaves = kFusedWaves;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_cnt[kWaves];
  __shared__ unsigned s_epoch;
  __shared__ int s_ok;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int G = static_cast<int>(gridDim.x);
  const int blk = static_cast<int>(blockIdx.x);
  const int d = a.ug.d;
  const int f = a.ug.f;
  uint8_t* tws = a.ug.ws_mut;  // batch 1: token 0's workspace slice
  unsigned* flags = reinterpret_cast<unsigned*>(tws + a.off_flags);
  const float* ssp = reinterpret_cast<const float*>(tws + a.ug.off_ssp);
  const uint32_t* bitmap = reinterpret_cast<const uint32_t*>(tws + a.ug.off_bitmap);

  // the first down item of this block and the bitmap word of this thread's
  // channel in it, loaded now so that no load has to be waited for between
  // the end of phase A and the W_down loads
  const int n_items = a.col_slices * a.row_groups;
  const bool has_item = blk < n_items;  // block-uniform
  int cs = has_item ? blk % a.col_slices : 0;
  int c0 = has_item ? (blk / a.col_slices) * a.chan_per_group : 0;
  const uint32_t word0 = has_item ? s2::range_word(bitmap, c0, min(f, c0 + a.chan_per_group)) : 0u;
  if (tid == 0) {
    s_epoch = __hip_atomic_load(&flags[blk], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    s_ok = 1;
  }
  // ---- phase A: up/gate over every wave of the grid (x staged at smem)
  const int ks = s2::upgate_block<T, true, kFusedThreads, false>(a.ug, blk, G, 0, smem);
  __syncthreads();  // x is dead: the region becomes the down reduction buffer

  // ---- phase B set-up: the first item's rows and its first W_down batch
  float* red = reinterpret_cast<float*>(smem);                    // [kWaves][kCw]
  int* jr = reinterpret_cast<int*>(smem + a.red_bytes);           // [max_rows]
  float* sr = reinterpret_cast<float*>(jr + a.max_rows);          // [max_rows]
  const uint8_t* Wd = static_cast<const uint8_t*>(a.w_down);
  const uint32_t row_bytes = static_cast<uint32_t>(d * sizeof(S));
  int n = 0, slot = -1;
  uint4 w[kDownUnroll];
  if (has_item) {
    n = s2::compact_range<kFusedThreads>(word0, c0, min(f, c0 + a.chan_per_group), jr, s_cnt, slot);
    __syncthreads();  // the list is complete
  }
  __builtin_amdgcn_sched_barrier(0);
  if (n > 0) {
    const int col = cs * kCw + lane * kEpl;
    s2::down_batch_loads<kWaves>(Wd, row_bytes, static_cast<uint32_t>((col < d ? col : cs * kCw) * sizeof(S)), jr, n,
                                 wave, w);
    // the phase-A stores precede these kDownUnroll loads in issue order
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kDownUnroll) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
  __syncthreads();  // every thread's phase-A stores are complete

  // ---- grid barrier
  if (tid == 0) __hip_atomic_store(&flags[blk], s_epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (has_item) {  // block-uniform; a block without down work has nothing to wait for
    if (wave == 0) {
      const unsigned epoch = s_epoch;
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (true) {
        bool mine = true;
        for (int i = lane; i < G; i += 64)
          mine = mine && static_cast<int>(__hip_atomic_load(&flags[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                                          epoch) >= 0;
        if (__ballot(!mine) == 0ull) break;
        if (__builtin_amdgcn_s_memrealtime() - t0 > static_cast<uint64_t>(a.wait_ticks)) {
          if (lane == 0) {
            s_ok = 0;
            __hip_atomic_fetch_or(reinterpret_cast<unsigned*>(tws + a.off_err), 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
          }
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    __syncthreads();

    // ---- phase B: the items of this block (skipped if it gave up: y is then invalid)
    float* y = a.ug.y;
    for (int item = blk, first = 1; s_ok && item < n_items; item += G, first = 0) {
      if (!first) {
        cs = item % a.col_slices;
        c0 = (item / a.col_slices) * a.chan_per_group;
        const int c1 = min(f, c0 + a.chan_per_group);
        n = s2::compact_range<kFusedThreads>(s2::range_word(bitmap, c0, c1), c0, c1, jr, s_cnt, slot);
      }
      // s_j of the rows, written by other blocks in phase A
      if (slot >= 0) sr[slot] = __hip_atomic_load(&ssp[c0 + tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (n > 0) {  // block-uniform
        const int col = cs * kCw + lane * kEpl;
        const bool cvalid = col < d;
        const int colc = cvalid ? col : cs * kCw;
        float acc[kEpl];
#pragma unroll
        for (int e = 0; e < kEpl; ++e) acc[e] = 0.f;
        const uint32_t col_bytes = static_cast<uint32_t>(colc * sizeof(S));
        for (int i0 = wave; i0 < n; i0 += kWaves * kDownUnroll) {
          if (!first || i0 != wave) {  // the first batch of the first item is already in w
            s2::down_batch_loads<kWaves>(Wd, row_bytes, col_bytes, jr, n, i0, w);
            __builtin_amdgcn_sched_barrier(0);
          }
          s2::down_batch_fma<T, kWaves>(acc, jr, sr, n, i0, cvalid, w);
        }
        s2::down_reduce_add<kFusedThreads, kCw>(red, acc, kEpl, cs, d, y);
      }
      __syncthreads();  // jr, sr and red are reused by the next item
    }
  }

  // ---- completion ticket: every block adds 1 (plus 1 << 16 if it gave up);
  // the block that draws the last ticket publishes k_s, or -1 if any block of
  // this launch gave up, and resets the counter for the next launch.  k_s has
  // one writer per launch, so a give-up can never be overwritten by it.
  if (tid == 0) {
    unsigned* done = reinterpret_cast<unsigned*>(tws + a.off_done);
    const unsigned mine = 1u + (s_ok ? 0u : 0x10000u);
    const unsigned prev = __hip_atomic_fetch_add(done, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((prev & 0xFFFFu) == static_cast<unsigned>(G - 1)) {
      __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.ug.mask_count, ((prev + mine) >> 16) != 0u ? -1 : ks, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

size_t fused_smem(const FusedArgs& a) {
  return static_cast<size_t>(a.red_bytes) + static_cast<size_t>(a.max_rows) * 8;
}

hipError_t fused_occupancy(int wdtype, size_t smem, int* blocks_per_cu) {
  if (wdtype == PROX_BF16)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, stage2_fused_kernel<Bf16Tag>, kFusedThreads,
                                                       smem);
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, stage2_fused_kernel<F32Tag>, kFusedThreads, smem);
}

// A cooperative launch: the runtime starts it only with every block resident
// at once (or refuses it with hipErrorCooperativeLaunchTooLarge), which is
// what the grid barrier needs; the bounded waits remain as a second guard.
hipError_t launch_stage2_fused(const FusedArgs& a, int wdtype, int grid, hipStream_t s) {
  const size_t smem = fused_smem(a);
  FusedArgs args = a;
  void* params[] = {&args};
  const void* fn = wdtype == PROX_BF16 ? reinterpret_cast<const void*>(stage2_fused_kernel<Bf16Tag>)
                                       : reinterpret_cast<const void*>(stage2_fused_kernel<F32Tag>);
  return hipLaunchCooperativeKernel(fn, dim3(static_cast<unsigned>(grid)), dim3(kFusedThreads), params,
                                    static_cast<unsigned>(smem), s);
}

}  // namespace prox
