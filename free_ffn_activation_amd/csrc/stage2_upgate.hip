// Stage 2, first half, on gfx950: exact up/gate projections of the kept
// channels with the SwiGLU product fused.
//
// Method ([blog] = deep-dive blog "Prox 完全拆解", section "Stage 2"):
//   u_sp = Pi^out(x, W_up, m_s), h_sp = SiLU(Pi^out(x, W_gate, m_s)),
//   s_sp = u_sp * h_sp, with the dense x and the original weights (GELU in
//   place of SiLU for a GeGLU layer).
// The pages fuse the output-sparse up and gate projections into one kernel
// ([blog] section on turning the formulas into GPU work).
//
// gfx950 design:
//   * W_up and W_gate are stored transposed and interleaved per channel
//     ([f][2][d]), so a kept channel is two contiguous d-long runs; only those
//     runs are read (2 * k_s * d * sizeof(w) bytes).
//   * decode mode: every block turns the Stage-1 bitmap into the ascending
//     channel list for its slice of ordinals (block scan of popcounts), so no
//     separate compaction launch is needed; the block owning ordinal 0 also
//     publishes k_s, and every block writes its part of the index list.
//   * one wave per channel: 64 lanes x 16 B per load cover 512 bf16 of a run;
//     up to 8 steps (16 loads, 16 KB per wave) are issued before use.  x lives
//     in LDS.  bf16 products use v_dot2_f32_bf16 (exact products, fp32 sum).
//   * a wave reduction gives u_j and g_j; lane 0 stores s_j = u_j act(g_j).
//   * this kernel also zeroes y, which the down kernel accumulates into.
#include "prox_device.h"
#include "prox_internal.h"

namespace prox {
namespace {

// bitmap words held per thread: d_ff <= 65536 gives 2048 words over 256 threads
constexpr int kMaxWordsPerThread = 8;

// Inclusive block scan of one int per thread; returns the inclusive prefix and
// writes the block total to *total.  `scratch` holds 4 ints.
__device__ __forceinline__ int block_inclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int x = wave_inclusive_scan_int(v);
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += scratch[w];
  *total = scratch[0] + scratch[1] + scratch[2] + scratch[3];
  __syncthreads();
  return base + x;
}

template <typename T, bool kFromBitmap>
__global__ __launch_bounds__(kThreads) void upgate_kernel(UpGateArgs a) {
  typedef typename T::storage S;
  constexpr int kEpl = 16 / sizeof(S);  // elements per 16-byte load
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_scan[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.y;
  const int d = a.d;
  const int f = a.f;
  const int nchunks = d / kEpl;
  const int nw = f / 32;

  uint4* xs = reinterpret_cast<uint4*>(smem);
  int* jl = reinterpret_cast<int*>(smem + static_cast<size_t>(nchunks) * 16);

  // Prologue loads (the bitmap words in decode mode, x) are all issued before
  // the first wait: unconditional loads with clamped indices, then a
  // scheduling barrier, so the prologue costs one memory round trip.
  // Decode mode: each thread keeps a run of consecutive bitmap words in
  // registers; one block scan of their popcounts gives every word's ordinal
  // offset, and the thread then emits the kept channels of its own words that
  // fall in this block's ordinal range.
  constexpr int kXPer = (12288 / kEpl + kThreads - 1) / kThreads;  // d <= 12288
  const u32x4_t* xg = reinterpret_cast<const u32x4_t*>(static_cast<const S*>(a.x) +
                                                     static_cast<size_t>(b) * d);
  u32x4_t* xsv = reinterpret_cast<u32x4_t*>(xs);
  const int per = (nw + kThreads - 1) / kThreads;
  const int w0 = min(nw, tid * per);
  uint32_t wv[kMaxWordsPerThread];
  if (kFromBitmap) {
    const uint32_t* bm = reinterpret_cast<const uint32_t*>(
        a.ws + static_cast<size_t>(b) * a.tok_bytes + a.off_bitmap);
#pragma unroll
    for (int k = 0; k < kMaxWordsPerThread; ++k) wv[k] = bm[min(w0 + k, nw - 1)];
  }
  u32x4_t xv[kXPer];
#pragma unroll
  for (int k = 0; k < kXPer; ++k) xv[k] = xg[min(tid + k * kThreads, nchunks - 1)];
  __builtin_amdgcn_sched_barrier(0);
  // surplus lanes rewrite the last chunk with its own value (no branch)
#pragma unroll
  for (int k = 0; k < kXPer; ++k) xsv[min(tid + k * kThreads, nchunks - 1)] = xv[k];
  // y is accumulated by the down kernel: clear it here
  for (int c = blockIdx.x * kThreads + tid; c < d; c += gridDim.x * kThreads)
    a.y[static_cast<size_t>(b) * d + c] = 0.f;

  int ks = 0;
  int run = 0;
  if (kFromBitmap) {
    int local = 0;
#pragma unroll
    for (int k = 0; k < kMaxWordsPerThread; ++k) {
      if (!(k < per && w0 + k < nw)) wv[k] = 0u;
      local += __popc(wv[k]);
    }
    int total = 0;
    run = block_inclusive_scan(local, s_scan, &total) - local;
    ks = total;
  } else {
    ks = min(max(a.mask_count[b], 0), f);
  }
  const int cpb = (ks + static_cast<int>(gridDim.x) - 1) / static_cast<int>(gridDim.x);
  const int k0 = min(ks, static_cast<int>(blockIdx.x) * cpb);
  const int k1 = min(ks, k0 + cpb);
  const int nloc = k1 - k0;

  if (kFromBitmap) {
    if (blockIdx.x == 0 && tid == 0) a.mask_count[b] = ks;
    int o = run;
#pragma unroll
    for (int k = 0; k < kMaxWordsPerThread; ++k) {
      uint32_t bits = wv[k];
      if (o >= k1 || o + __popc(bits) <= k0) {
        o += __popc(bits);
        continue;
      }
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1u;
        if (o >= k0 && o < k1) jl[o - k0] = (w0 + k) * 32 + bit;
        ++o;
      }
    }
  } else {
    for (int i = tid; i < nloc; i += kThreads) {
      const int j = a.mask_idx[static_cast<size_t>(b) * f + k0 + i];
      jl[i] = (j >= 0 && j < f) ? j : -1;
    }
  }
  __syncthreads();

  const S* W = static_cast<const S*>(a.w_upgate_t);
  float* ssp = reinterpret_cast<float*>(a.ws_mut + static_cast<size_t>(b) * a.tok_bytes + a.off_ssp);
  const int nsteps = (nchunks + 63) / 64;
  for (int i = wave; i < nloc; i += kThreads / 64) {
    const int j = jl[i];
    float su = 0.f, sg = 0.f;
    if (j >= 0) {
      const uint4* wu = reinterpret_cast<const uint4*>(W + static_cast<size_t>(j) * 2 * d);
      const uint4* wg = reinterpret_cast<const uint4*>(W + static_cast<size_t>(j) * 2 * d + d);
      for (int s0 = 0; s0 < nsteps; s0 += kUpGateUnroll) {
        uint4 lu[kUpGateUnroll], lg[kUpGateUnroll];
        // unconditional loads (clamped to the run) so waits pipeline
#pragma unroll
        for (int u = 0; u < kUpGateUnroll; ++u) {
          const int cidx = min((s0 + u) * 64 + lane, nchunks - 1);
          lu[u] = ldg16(wu + cidx);
          lg[u] = ldg16(wg + cidx);
        }
        // keep the whole batch in flight: the scheduler would otherwise sink
        // each load next to its use and serialise the memory round trips
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < kUpGateUnroll; ++u) {
          const int cidx = (s0 + u) * 64 + lane;
          const uint4 xv = xs[min(cidx, nchunks - 1)];
          const float du = dot16<T>(lu[u], xv, 0.f);
          const float dg = dot16<T>(lg[u], xv, 0.f);
          su += cidx < nchunks ? du : 0.f;
          sg += cidx < nchunks ? dg : 0.f;
        }
      }
      su = wave_sum(su);
      sg = wave_sum(sg);
    }
    if (lane == 0) {
      const float sj = (j >= 0) ? su * gate_act(sg, a.act) : 0.f;
      if (kFromBitmap) {
        // decode mode: s by channel index (the down kernel reads it through
        // the bitmap), and the ascending index list for the caller
        ssp[j] = sj;
        a.mask_idx[static_cast<size_t>(b) * f + k0 + i] = j;
      } else {
        ssp[k0 + i] = sj;  // list mode: s by list position
      }
    }
  }
}

}  // namespace

hipError_t launch_upgate(const UpGateArgs& a, int wdtype, int batch, int blocks,
                         bool from_bitmap, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(batch));
  const size_t esz = wdtype == PROX_BF16 ? 2 : 4;
  const size_t smem = static_cast<size_t>(a.d) * esz + static_cast<size_t>(a.max_cpb) * 4;
  if (wdtype == PROX_BF16) {
    if (from_bitmap)
      hipLaunchKernelGGL((upgate_kernel<Bf16Tag, true>), grid, dim3(kThreads), smem, s, a);
    else
      hipLaunchKernelGGL((upgate_kernel<Bf16Tag, false>), grid, dim3(kThreads), smem, s, a);
  } else {
    if (from_bitmap)
      hipLaunchKernelGGL((upgate_kernel<F32Tag, true>), grid, dim3(kThreads), smem, s, a);
    else
      hipLaunchKernelGGL((upgate_kernel<F32Tag, false>), grid, dim3(kThreads), smem, s, a);
  }
  return hipGetLastError();
}

}  // namespace prox
