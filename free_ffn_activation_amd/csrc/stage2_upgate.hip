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
//   * one wave per kept channel: global wave w takes the channels of ordinals
//     w, w + W, w + 2W, ... (W waves in the grid).  Decode mode: every wave
//     holds the Stage-1 bitmap in registers (8 words per lane per 16384
//     channels), counts it with a DPP scan and picks its channel by ordinal
//     itself, so no block-wide scan or list precedes the gather; wave 0 of
//     block 0 publishes k_s, and every wave writes its ordinal's index.  List
//     mode: the channel is read from the caller's list.
//   * 64 lanes x 16 B per load cover 512 bf16 of a run; up to 8 steps (16
//     loads, 16 KB per wave) are issued before use.  x is staged in LDS once
//     per block; the block's one barrier comes after the first weight loads
//     are issued, so it overlaps the gather.  bf16 products use
//     v_dot2_f32_bf16 (exact products, fp32 sum).
//   * a wave reduction gives u_j and g_j; lane 0 stores s_j = u_j act(g_j).
//   * this kernel also zeroes y, which the down kernel accumulates into.
#include <type_traits>

#include "prox_device.h"
#include "prox_internal.h"

namespace prox {
namespace {

// Bitmap chunks of 512 words (16384 channels) held in registers, 8 words per
// lane; larger d_ff reads the further chunks when they are scanned.
constexpr int kChunkWords = 512;
constexpr int kHeldChunks = 2;

// The Stage-1 bitmap of one token as one wave sees it: lane l holds words
// [c * 512 + 8 l, c * 512 + 8 l + 8) of each held chunk c (0 past the end).
struct WaveBitmap {
  const u32x4_t* bm;  // 16-B groups of 4 words
  int n4;             // groups in the bitmap (d_ff / 128)
  int nchunk;
  u32x4_t held[kHeldChunks][2];

  __device__ __forceinline__ void load_chunk(int c, u32x4_t (&w)[2]) const {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int g = c * (kChunkWords / 4) + 2 * lane + h;
      const u32x4_t v = bm[min(g, n4 - 1)];
      w[h] = g < n4 ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void issue(const uint8_t* base, int f) {
    bm = reinterpret_cast<const u32x4_t*>(base);
    n4 = f / 128;
    nchunk = (f / 32 + kChunkWords - 1) / kChunkWords;
#pragma unroll
    for (int c = 0; c < kHeldChunks; ++c) load_chunk(c, held[c]);
  }
  template <bool kHeld = true>
  __device__ __forceinline__ void chunk(int c, u32x4_t (&w)[2]) const {
    if (kHeld && c < kHeldChunks) {  // c is wave-uniform; no dynamic register indexing
      if (c == 1) {
        w[0] = held[1][0];
        w[1] = held[1][1];
      } else {
        w[0] = held[0][0];
        w[1] = held[0][1];
      }
    } else {
      load_chunk(c, w);
    }
  }
  static __device__ __forceinline__ int lane_count(const u32x4_t (&w)[2]) {
    return __popc(w[0].x) + __popc(w[0].y) + __popc(w[0].z) + __popc(w[0].w) + __popc(w[1].x) +
           __popc(w[1].y) + __popc(w[1].z) + __popc(w[1].w);
  }
  // number of set bits (k_s)
  __device__ __forceinline__ int total() const {
    int t = 0;
    for (int c = 0; c < nchunk; ++c) {
      u32x4_t w[2];
      chunk(c, w);
      t += wave_sum_int(lane_count(w));
    }
    return t;
  }
  // channel of the k-th set bit (0-based, k < total()), the same in every
  // lane; kHeld = false reads the words again (they are L2 hits) so that the
  // held registers need not stay live
  template <bool kHeld = true>
  __device__ __forceinline__ int select(int k) const {
    const int lane = threadIdx.x & 63;
    int base = 0;
    for (int c = 0; c < nchunk; ++c) {
      u32x4_t w[2];
      chunk<kHeld>(c, w);
      const int cnt = lane_count(w);
      const int incl = wave_inclusive_scan_int(cnt);
      const int tot = __builtin_amdgcn_readlane(incl, 63);
      if (k < base + tot) {
        const int kp = k - base;
        const int excl = incl - cnt;
        const uint64_t own = __ballot(excl <= kp && kp < incl);  // exactly one lane
        if (own == 0ull) return -1;
        const int owner = static_cast<int>(__builtin_ctzll(own));
        int r = kp - __builtin_amdgcn_readlane(excl, owner);
        const uint32_t ow[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
        uint32_t sel = 0u;
        int m_sel = 0;
        bool found = false;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const uint32_t wm = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ow[m]), owner));
          const int cm = __popc(wm);
          if (!found && r < cm) {
            sel = wm;
            m_sel = m;
            found = true;
          } else if (!found) {
            r -= cm;
          }
        }
        // the r-th set bit of the selected word: lane b tests bit b
        const uint32_t below = lane < 32 ? ((1u << (lane & 31)) - 1u) : 0xFFFFFFFFu;
        const bool hit = lane < 32 && ((sel >> (lane & 31)) & 1u) && __popc(sel & below) == r;
        const uint64_t hits = __ballot(hit);
        if (hits == 0ull) return -1;
        return ((c * kChunkWords + 8 * owner + m_sel) << 5) + static_cast<int>(__builtin_ctzll(hits));
      }
      base += tot;
    }
    return -1;
  }
};

template <typename T, bool kFromBitmap>
__global__ __launch_bounds__(kUgThreads) void upgate_kernel(UpGateArgs a) {
  typedef typename T::storage S;
  constexpr int kEpl = 16 / sizeof(S);  // elements per 16-byte load
  constexpr int kWaves = kUgThreads / 64;
  extern __shared__ __align__(16) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.y;
  const int d = a.d;
  const int f = a.f;
  const int nchunks = d / kEpl;
  const int nsteps = (nchunks + 63) / 64;
  // ordinal gw, gw + nwaves, ...: consecutive ordinals go to consecutive
  // blocks, so the waves left without a channel (ordinals past k_s) spread
  // over every CU instead of filling the last blocks
  const int gw = wave * static_cast<int>(gridDim.x) + static_cast<int>(blockIdx.x);
  const int nwaves = static_cast<int>(gridDim.x) * kWaves;

  // ---- prologue: bitmap (decode mode) or list count, then x; one round trip
  WaveBitmap bmv;
  int ks_list = 0;
  if (kFromBitmap)
    bmv.issue(a.ws + static_cast<size_t>(b) * a.tok_bytes + a.off_bitmap, f);
  else
    ks_list = a.mask_count[b];
  constexpr int kXPer = (12288 / kEpl + kUgThreads - 1) / kUgThreads;  // d <= 12288
  const u32x4_t* xg = reinterpret_cast<const u32x4_t*>(static_cast<const S*>(a.x) +
                                                     static_cast<size_t>(b) * d);
  u32x4_t xv[kXPer];
#pragma unroll
  for (int k = 0; k < kXPer; ++k) xv[k] = xg[min(tid + k * kUgThreads, nchunks - 1)];
  __builtin_amdgcn_sched_barrier(0);
  // y is accumulated by the down kernel: clear it here
  for (int c = blockIdx.x * kUgThreads + tid; c < d; c += gridDim.x * kUgThreads)
    a.y[static_cast<size_t>(b) * d + c] = 0.f;

  const int ks = kFromBitmap ? bmv.total() : min(max(ks_list, 0), f);
  if (kFromBitmap && blockIdx.x == 0 && tid == 0) a.mask_count[b] = ks;
  // channel of ordinal k (-1: past the end, or an out-of-range list entry)
  auto channel_of = [&](int k, auto held) -> int {
    if (k >= ks) return -1;
    if (kFromBitmap) return bmv.template select<decltype(held)::value>(k);
    const int j = __builtin_amdgcn_readfirstlane(a.mask_idx[static_cast<size_t>(b) * f + k]);
    return (j >= 0 && j < f) ? j : -1;
  };

  const S* W = static_cast<const S*>(a.w_upgate_t);
  float* ssp = reinterpret_cast<float*>(a.ws_mut + static_cast<size_t>(b) * a.tok_bytes + a.off_ssp);
  const uint4* xs = reinterpret_cast<const uint4*>(smem);

  // One channel: its first batch of loads is already in lu/lg; returns the
  // wave-reduced (u_j, g_j) in every lane.
  auto finish_channel = [&](int j, uint4 (&lu)[kUpGateUnroll], uint4 (&lg)[kUpGateUnroll], float& su,
                            float& sg) {
    const uint4* wu = reinterpret_cast<const uint4*>(W + static_cast<size_t>(j) * 2 * d);
    const uint4* wg = wu + nchunks;
    su = 0.f;
    sg = 0.f;
    for (int s0 = 0; s0 < nsteps; s0 += kUpGateUnroll) {
      if (s0 > 0) {
#pragma unroll
        for (int u = 0; u < kUpGateUnroll; ++u) {
          const int cidx = min((s0 + u) * 64 + lane, nchunks - 1);
          lu[u] = ldg16(wu + cidx);
          lg[u] = ldg16(wg + cidx);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < kUpGateUnroll; ++u) {
        const int cidx = (s0 + u) * 64 + lane;
        const uint4 xq = xs[min(cidx, nchunks - 1)];
        const float du = dot16<T>(lu[u], xq, 0.f);
        const float dg = dot16<T>(lg[u], xq, 0.f);
        su += cidx < nchunks ? du : 0.f;
        sg += cidx < nchunks ? dg : 0.f;
      }
    }
    su = wave_sum(su);
    sg = wave_sum(sg);
  };
  // the first batch of a channel's loads (unconditional, clamped to the run,
  // all in flight together: the scheduler would otherwise sink each load next
  // to its use and serialise the round trips)
  auto first_loads = [&](int j, uint4 (&lu)[kUpGateUnroll], uint4 (&lg)[kUpGateUnroll]) {
    const uint4* wu = reinterpret_cast<const uint4*>(W + static_cast<size_t>(j) * 2 * d);
    const uint4* wg = wu + nchunks;
#pragma unroll
    for (int u = 0; u < kUpGateUnroll; ++u) {
      const int cidx = min(u * 64 + lane, nchunks - 1);
      lu[u] = ldg16(wu + cidx);
      lg[u] = ldg16(wg + cidx);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto store = [&](int k, int j, float su, float sg) {
    if (lane == 0) {
      const float sj = (j >= 0) ? su * gate_act(sg, a.act) : 0.f;
      if (kFromBitmap) {
        // decode mode: s by channel index (the down kernel reads it through
        // the bitmap), and the ascending index list for the caller
        ssp[j] = sj;
        a.mask_idx[static_cast<size_t>(b) * f + k] = j;
      } else {
        ssp[k] = sj;  // list mode: s by list position
      }
    }
  };

  // first ordinal: x (which arrived with the bitmap) goes to LDS, the
  // channel's first loads go out, then the block's one barrier is passed
  const int j0 = channel_of(gw, std::true_type{});
  {
    uint4* xsw = reinterpret_cast<uint4*>(smem);
#pragma unroll
    for (int q = 0; q < kXPer; ++q)  // surplus lanes rewrite the last chunk with its own value
      xsw[min(tid + q * kUgThreads, nchunks - 1)] = __builtin_bit_cast(uint4, xv[q]);
  }
  uint4 lu[kUpGateUnroll], lg[kUpGateUnroll];
  if (j0 >= 0) first_loads(j0, lu, lg);
  __syncthreads();
  for (int k = gw; k < ks; k += nwaves) {  // wave-uniform
    const int j = (k == gw) ? j0 : channel_of(k, std::false_type{});
    float su = 0.f, sg = 0.f;
    if (j >= 0) {
      if (k != gw) first_loads(j, lu, lg);
      finish_channel(j, lu, lg, su, sg);
    }
    store(k, j, su, sg);
  }
}

}  // namespace

hipError_t launch_upgate(const UpGateArgs& a, int wdtype, int batch, int blocks,
                         bool from_bitmap, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(batch));
  const size_t esz = wdtype == PROX_BF16 ? 2 : 4;
  const size_t smem = static_cast<size_t>(a.d) * esz;
  if (wdtype == PROX_BF16) {
    if (from_bitmap)
      hipLaunchKernelGGL((upgate_kernel<Bf16Tag, true>), grid, dim3(kUgThreads), smem, s, a);
    else
      hipLaunchKernelGGL((upgate_kernel<Bf16Tag, false>), grid, dim3(kUgThreads), smem, s, a);
  } else {
    if (from_bitmap)
      hipLaunchKernelGGL((upgate_kernel<F32Tag, true>), grid, dim3(kUgThreads), smem, s, a);
    else
      hipLaunchKernelGGL((upgate_kernel<F32Tag, false>), grid, dim3(kUgThreads), smem, s, a);
  }
  return hipGetLastError();
}

}  // namespace prox
