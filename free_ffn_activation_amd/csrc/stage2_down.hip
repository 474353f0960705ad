// Stage 2, second half, on gfx950: the input-sparse down projection.
//
// Method ([blog] = deep-dive blog "Prox 完全拆解", sections on the SwiGLU
// weighted-sum view and "Stage 2"): y = Pi^in(s_sp, W_down, m_s), i.e.
// y = sum over kept j of s_j * W_down[j, :]; the same index j is an up/gate
// output channel and a down input row, so only kept rows of W_down are read.
//
// gfx950 design:
//   * W_down is row-major [f][d]: a kept channel is one contiguous d-long run.
//   * grid = (column slices x row groups, batch).  A column slice is what one
//     wave covers with one 16-B load per lane (512 bf16 / 256 fp32 columns).
//     In decode mode a row group is a fixed range of channels whose kept ones
//     the block finds in the Stage-1 bitmap (s_j is stored by channel index),
//     so no count or list has to be fetched first; with a caller-given list a
//     row group is a contiguous range of that list.  The block stages its
//     (index, s_j) pairs in LDS; each of its 16 waves streams every 16th row
//     with 8 loads in flight and accumulates its columns in registers.
//   * the 16 waves' partial rows are summed through LDS and the block adds its
//     slice into y with fp32 atomics (y was zeroed by the up/gate kernel).
//     Large blocks keep the atomic count (row groups x d) low: fp32 global
//     atomics cost far more per byte than the weight stream.
#include "prox_device.h"
#include "prox_internal.h"

namespace prox {
namespace {

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

template <typename T, bool kFromBitmap>
__global__ __launch_bounds__(kDownThreads) void down_kernel(DownArgs a) {
  typedef typename T::storage S;
  constexpr int kEpl = 16 / sizeof(S);
  constexpr int kCw = 64 * kEpl;  // columns per slice
  constexpr int kWaves = kDownThreads / 64;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_cnt[kWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.y;
  const int d = a.d;
  const int f = a.f;
  const int cs = blockIdx.x % a.col_slices;
  const int rg = blockIdx.x / a.col_slices;
  float* red = reinterpret_cast<float*>(smem);                 // [kWaves][kCw]
  int* jr = reinterpret_cast<int*>(red + kWaves * kCw);        // [max_rows]
  float* sr = reinterpret_cast<float*>(jr + a.max_rows);       // [max_rows]
  const uint8_t* tws = a.ws + static_cast<size_t>(b) * a.tok_bytes;
  const float* ssp = reinterpret_cast<const float*>(tws + a.off_ssp);
  int n = 0;
  if (kFromBitmap) {
    // decode mode: this block's rows are the kept channels of a fixed channel
    // range; the bitmap word and s_j of each channel come in one round trip
    // and a block ballot compacts them in ascending order
    const int c0 = rg * a.chan_per_group;
    const int c1 = min(f, c0 + a.chan_per_group);
    const int j = c0 + tid;
    const int jc = min(j, c1 - 1);
    const uint32_t word = reinterpret_cast<const uint32_t*>(tws + a.off_bitmap)[jc >> 5];
    const float sj = ssp[jc];
    const bool kept = j < c1 && ((word >> (jc & 31)) & 1u);
    const uint64_t bal = __ballot(kept);
    if (lane == 0) s_cnt[wave] = __popcll(bal);
    __syncthreads();
    int off = 0;
    for (int w2 = 0; w2 < kWaves; ++w2) {
      if (w2 < wave) off += s_cnt[w2];
      n += s_cnt[w2];
    }
    if (kept) {
      const int pos = off + __popcll(bal & ((1ull << lane) - 1ull));
      jr[pos] = j;
      sr[pos] = sj;
    }
  } else {
    const int ks = min(max(a.mask_count[b], 0), f);
    const int per = (ks + a.row_groups - 1) / a.row_groups;
    const int r0 = min(ks, rg * per);
    const int r1 = min(ks, r0 + per);
    n = r1 - r0;
    for (int i = tid; i < n; i += kDownThreads) {
      const int j = a.mask_idx[static_cast<size_t>(b) * f + r0 + i];
      const bool ok = j >= 0 && j < f;
      jr[i] = ok ? j : -1;
      sr[i] = ok ? ssp[r0 + i] : 0.f;
    }
  }
  if (n <= 0) return;  // block-uniform
  __syncthreads();

  const int col = cs * kCw + lane * kEpl;
  const bool cvalid = col < d;
  const S* Wd = static_cast<const S*>(a.w_down);
  float acc[kEpl];
#pragma unroll
  for (int e = 0; e < kEpl; ++e) acc[e] = 0.f;
  // Loads are unconditional: a slot past the end (or a skipped index) re-reads
  // a valid row with weight 0, and a lane past the last column reads the
  // slice's first column, so the compiler can wait on the loads one by one.
  const int colc = cvalid ? col : cs * kCw;
  for (int i0 = wave; i0 < n; i0 += kWaves * kDownUnroll) {
    uint4 w[kDownUnroll];
    float sv[kDownUnroll];
#pragma unroll
    for (int u = 0; u < kDownUnroll; ++u) {
      const int i = min(i0 + u * kWaves, n - 1);
      const int j = jr[i];
      sv[u] = (i0 + u * kWaves < n && j >= 0 && cvalid) ? sr[i] : 0.f;
      w[u] = ldg16(Wd + static_cast<size_t>(j >= 0 ? j : 0) * d + colc);
    }
    __builtin_amdgcn_sched_barrier(0);  // the batch stays in flight together
#pragma unroll
    for (int u = 0; u < kDownUnroll; ++u) axpy16<T>(acc, sv[u], w[u]);
  }
#pragma unroll
  for (int e = 0; e < kEpl; ++e) red[wave * kCw + lane * kEpl + e] = acc[e];
  __syncthreads();
  for (int c = tid; c < kCw; c += kDownThreads) {
    const int gc = cs * kCw + c;
    if (gc < d) {
      float v = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < kWaves; ++w2) v += red[w2 * kCw + c];
      unsafeAtomicAdd(&a.y[static_cast<size_t>(b) * d + gc], v);
    }
  }
}

}  // namespace

hipError_t launch_down(const DownArgs& a, int wdtype, int batch, bool from_bitmap, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.col_slices * a.row_groups), static_cast<unsigned>(batch));
  const int cw = wdtype == PROX_BF16 ? 512 : 256;
  const size_t smem = static_cast<size_t>(kDownThreads / 64) * cw * 4 + static_cast<size_t>(a.max_rows) * 8;
  if (wdtype == PROX_BF16) {
    if (from_bitmap)
      hipLaunchKernelGGL((down_kernel<Bf16Tag, true>), grid, dim3(kDownThreads), smem, s, a);
    else
      hipLaunchKernelGGL((down_kernel<Bf16Tag, false>), grid, dim3(kDownThreads), smem, s, a);
  } else {
    if (from_bitmap)
      hipLaunchKernelGGL((down_kernel<F32Tag, true>), grid, dim3(kDownThreads), smem, s, a);
    else
      hipLaunchKernelGGL((down_kernel<F32Tag, false>), grid, dim3(kDownThreads), smem, s, a);
  }
  return hipGetLastError();
}

}  // namespace prox
