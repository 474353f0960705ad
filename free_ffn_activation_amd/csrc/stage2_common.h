// Device code shared by the Stage-2 kernels on gfx950: the up/gate gather
// over kept channels and the down projection over kept rows ([blog] = deep-dive
// blog "Prox 完全拆解", section "Stage 2"; [paper] section 2.2 for Pi^out and
// Pi^in).  Used by the up/gate and down kernels (one launch each) and by the
// fused Stage-2 kernel (both in one launch).
#pragma once

#include <type_traits>

#include "prox_device.h"
#include "prox_internal.h"

namespace prox {
namespace s2 {

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

// The up/gate work of one block of kThreadsPB threads: global wave
// w = wave * nblocks + block takes the kept channels of ordinals w, w + W, ...
// (W = all waves), consecutive ordinals on consecutive blocks so the waves
// left without a channel spread over every CU.  Decode mode (kFromBitmap):
// every wave holds the Stage-1 bitmap in registers and picks its channel by
// ordinal; block 0 publishes k_s (unless kPublishCount is false: the caller
// then publishes it; the function returns k_s); every wave writes its
// ordinal's entry of the ascending index list; s_j is stored by channel index.  List mode: the
// channel comes from the caller's list and s_j is stored by list position.
// kNt: the weight runs are read with the non-temporal hint (a launch over one
// token reads each run once; over several tokens the runs of channels they
// share are read once per token and stay cacheable).  The block also zeroes
// its share of y (the down projection accumulates into it).  s_j and the zeros of y are written with agent-coherent stores, so a
// later phase of the same launch on another XCD can read them once the writer
// has waited for its stores (see the fused kernel).  smem holds x (d elements).
template <typename T, bool kFromBitmap, int kThreadsPB, bool kPublishCount = true, bool kNt = true>
__device__ __forceinline__ int upgate_block(const UpGateArgs& a, int block, int nblocks, int b, uint8_t* smem) {
  typedef typename T::storage S;
  constexpr int kEpl = 16 / sizeof(S);  // elements per 16-byte load
  constexpr int kWaves = kThreadsPB / 64;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int d = a.d;
  const int f = a.f;
  const int nchunks = d / kEpl;
  const int nsteps = (nchunks + 63) / 64;
  const int gw = wave * nblocks + block;
  const int nwaves = nblocks * kWaves;

  // ---- prologue: bitmap (decode mode) or list count, then x; one round trip
  WaveBitmap bmv;
  int ks_list = 0;
  if (kFromBitmap)
    bmv.issue(a.ws + static_cast<size_t>(b) * a.tok_bytes + a.off_bitmap, f);
  else
    ks_list = a.mask_count[b];
  constexpr int kXPer = (12288 / kEpl + kThreadsPB - 1) / kThreadsPB;  // d <= 12288
  const u32x4_t* xg = reinterpret_cast<const u32x4_t*>(static_cast<const S*>(a.x) + static_cast<size_t>(b) * d);
  u32x4_t xv[kXPer];
#pragma unroll
  for (int k = 0; k < kXPer; ++k) xv[k] = xg[min(tid + k * kThreadsPB, nchunks - 1)];
  __builtin_amdgcn_sched_barrier(0);
  // y is accumulated by the down projection: clear it here
  for (int c = block * kThreadsPB + tid; c < d; c += nblocks * kThreadsPB)
    __hip_atomic_store(&a.y[static_cast<size_t>(b) * d + c], 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  const int ks = kFromBitmap ? bmv.total() : min(max(ks_list, 0), f);
  if (kFromBitmap && kPublishCount && block == 0 && tid == 0) a.mask_count[b] = ks;
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
          lu[u] = ldg16_w<kNt>(wu + cidx);
          lg[u] = ldg16_w<kNt>(wg + cidx);
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
      lu[u] = ldg16_w<kNt>(wu + cidx);
      lg[u] = ldg16_w<kNt>(wg + cidx);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto store = [&](int k, int j, float su, float sg) {
    if (lane == 0) {
      const float sj = (j >= 0) ? su * gate_act(sg, a.act) : 0.f;
      if (kFromBitmap) {
        // decode mode: s by channel index (the down projection reads it
        // through the bitmap), and the ascending index list for the caller
        if (j >= 0) __hip_atomic_store(&ssp[j], sj, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.mask_idx[static_cast<size_t>(b) * f + k] = j;
      } else {
        __hip_atomic_store(&ssp[k], sj, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // by list position
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
      xsw[min(tid + q * kThreadsPB, nchunks - 1)] = __builtin_bit_cast(uint4, xv[q]);
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
  return ks;
}

template <typename T>
__device__ __forceinline__ void axpy16(float* acc, float s, uint4 w);

template <>
__device__ __forceinline__ void axpy16<Bf16Tag>(float* acc, float s, uint4 w) {
  acc[0] = fmaf(s, bf16lo(w.x), acc[0]);
  acc[1] = fmaf(s, bf16hi(w.x), acc[1]);
  acc[2] = fmaf(s, bf16lo(w.y), acc[2]);
  acc[3] = fmaf(s, bf16hi(w.y), acc[3]);
  acc[4] = fmaf(s, bf16lo(w.z), acc[4]);
  acc[5] = fmaf(s, bf16hi(w.z), acc[5]);
  acc[6] = fmaf(s, bf16lo(w.w), acc[6]);
  acc[7] = fmaf(s, bf16hi(w.w), acc[7]);
}

template <>
__device__ __forceinline__ void axpy16<F32Tag>(float* acc, float s, uint4 w) {
  acc[0] = fmaf(s, __uint_as_float(w.x), acc[0]);
  acc[1] = fmaf(s, __uint_as_float(w.y), acc[1]);
  acc[2] = fmaf(s, __uint_as_float(w.z), acc[2]);
  acc[3] = fmaf(s, __uint_as_float(w.w), acc[3]);
}

// The Stage-1 bitmap word that holds the calling thread's channel c0 + tid of
// the range [c0, c1) (clamped to the range).
__device__ __forceinline__ uint32_t range_word(const uint32_t* bitmap, int c0, int c1) {
  return bitmap[min(c0 + static_cast<int>(threadIdx.x), c1 - 1) >> 5];
}

// Down projection of one row group: the kept channels of the channel range
// [c0, c1), one thread per channel (`word` = range_word() of that thread),
// compacted in ascending order into the LDS list jr (block ballot).  Returns
// their number (block-uniform); `slot` receives the list position of the
// calling thread's channel (-1 if not kept).  kThreadsPB threads.
template <int kThreadsPB>
__device__ __forceinline__ int compact_range(uint32_t word, int c0, int c1, int* jr, int* s_cnt, int& slot) {
  constexpr int kWaves = kThreadsPB / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int j = c0 + tid;
  const int jc = min(j, c1 - 1);
  const bool kept = j < c1 && ((word >> (jc & 31)) & 1u);
  const uint64_t bal = __ballot(kept);
  if (lane == 0) s_cnt[wave] = __popcll(bal);
  __syncthreads();
  int off = 0, n = 0;
#pragma unroll
  for (int w2 = 0; w2 < kWaves; ++w2) {
    if (w2 < wave) off += s_cnt[w2];
    n += s_cnt[w2];
  }
  slot = kept ? off + __popcll(bal & ((1ull << lane) - 1ull)) : -1;
  if (kept) jr[slot] = j;
  return n;
}

// One batch of W_down rows for wave `wave`: rows i0 + u * kWaves of the list
// (u < kU), loads unconditional (a slot past the end re-reads the
// last row, a lane past the last column reads the slice's first column) so the
// compiler can wait on them one by one.  Wd is the uniform base; row_bytes and
// col_bytes give 32-bit byte offsets (W_down stays below 4 GiB for every
// supported shape: 65536 x 12288 x 4 bytes is 3 GiB).
template <int kWaves, int kU = kDownUnroll>
__device__ __forceinline__ void down_batch_loads(const uint8_t* Wd, uint32_t row_bytes, uint32_t col_bytes,
                                                 const int* jr, int n, int i0, uint4 (&w)[kU]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int i = min(i0 + u * kWaves, n - 1);
    const int j = jr[i];
    w[u] = ldg16(Wd + (static_cast<uint32_t>(j >= 0 ? j : 0) * row_bytes + col_bytes));
  }
}

// down_batch_loads through the buffer resource wr: a slot past the end of the
// list (or a list entry of -1) loads from kWeightOob and costs no memory
// traffic, so a launch over one token reads every row slice once, and then
// (kNt) with the non-temporal hint; over several tokens the rows they share
// are read once per token and stay cacheable.  Measured on MI355X against the clamped re-reads with cacheable
// loads: the down kernel 7.93 -> 7.71 us (Qwen3-8B-shaped layer; decode step
// 30.6 -> 29.8 us) and 16.39 -> 15.57 us (Qwen3-32B-shaped layer).
template <int kWaves, int kU, bool kNt>
__device__ __forceinline__ void down_batch_loads_buf(__amdgpu_buffer_rsrc_t wr, uint32_t row_bytes, uint32_t col_bytes,
                                                     const int* jr, int n, int i0, uint4 (&w)[kU]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int iu = i0 + u * kWaves;
    const int j = jr[min(iu, n - 1)];
    const uint32_t off = (iu < n && j >= 0) ? static_cast<uint32_t>(j) * row_bytes + col_bytes : kWeightOob;
    if constexpr (kNt)
      w[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2 /* nt */));
    else
      w[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 0));
  }
}

template <typename T, int kWaves, int kU = kDownUnroll>
__device__ __forceinline__ void down_batch_fma(float* acc, const int* jr, const float* sr, int n, int i0, bool cvalid,
                                               const uint4 (&w)[kU]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int i = min(i0 + u * kWaves, n - 1);
    const float sv = (i0 + u * kWaves < n && jr[i] >= 0 && cvalid) ? sr[i] : 0.f;
    axpy16<T>(acc, sv, w[u]);
  }
}

// The block's partial rows (one per wave) summed through LDS in fixed wave
// order and added into y with fp32 atomics.
template <int kThreadsPB, int kCw>
__device__ __forceinline__ void down_reduce_add(float* red, const float* acc, int kepl, int cs, int d, float* y) {
  constexpr int kWaves = kThreadsPB / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int e = 0; e < kepl; ++e) red[wave * kCw + lane * kepl + e] = acc[e];
  __syncthreads();
  for (int c = tid; c < kCw; c += kThreadsPB) {
    const int gc = cs * kCw + c;
    if (gc < d) {
      float v = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) v += red[w2 * kCw + c];
      unsafeAtomicAdd(&y[gc], v);
    }
  }
}

}  // namespace s2
}  // namespace prox
