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
//     with 8 (or, for its last 4 rows or fewer, 4) loads in flight and
//     accumulates its columns in registers.  The loads go through a buffer
//     resource (with the non-temporal hint when the launch covers one
//     token); batch slots past the list end read past the buffer's records
//     (zeros, no memory access).
//   * the 16 waves' partial rows are summed through LDS and the block adds its
//     slice into y with fp32 atomics (y was zeroed by the up/gate kernel).
//     Large blocks keep the atomic count (row groups x d) low: fp32 global
//     atomics cost far more per byte than the weight stream.
#include <type_traits>

#include "stage2_common.h"

namespace prox {
namespace {

template <typename T, bool kFromBitmap, bool kNt>
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
    // range, compacted from the bitmap; s_j (stored by channel index) of each
    // thread's channel is read in the same round trip
    const int c0 = rg * a.chan_per_group;
    const int c1 = min(f, c0 + a.chan_per_group);
    const float sj = ssp[min(c0 + tid, c1 - 1)];
    int slot;
    n = s2::compact_range<kDownThreads>(s2::range_word(reinterpret_cast<const uint32_t*>(tws + a.off_bitmap), c0, c1),
                                        c0, c1, jr, s_cnt, slot);
    if (slot >= 0) sr[slot] = sj;
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
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc(a.w_down, f, d, static_cast<int>(sizeof(S)));
  float acc[kEpl];
#pragma unroll
  for (int e = 0; e < kEpl; ++e) acc[e] = 0.f;
  const int colc = cvalid ? col : cs * kCw;
  const uint32_t row_bytes = static_cast<uint32_t>(d * sizeof(S));
  const uint32_t col_bytes = static_cast<uint32_t>(colc * sizeof(S));
  auto batch = [&](int i0, auto depth) {
    constexpr int kU = decltype(depth)::value;
    uint4 w[kU];
    s2::down_batch_loads_buf<kWaves, kU, kNt>(wr, row_bytes, col_bytes, jr, n, i0, w);
    __builtin_amdgcn_sched_barrier(0);  // the batch stays in flight together
    s2::down_batch_fma<T, kWaves, kU>(acc, jr, sr, n, i0, cvalid, w);
  };
  // A wave with at most half a batch of rows left issues a half batch (at
  // ~56 kept rows per row group of the Qwen3-8B-shaped layer a wave has 3-4)
  for (int i0 = wave; i0 < n; i0 += kWaves * kDownUnroll) {
    if (i0 + (kDownUnroll / 2) * kWaves >= n)  // wave-uniform
      batch(i0, std::integral_constant<int, kDownUnroll / 2>{});
    else
      batch(i0, std::integral_constant<int, kDownUnroll>{});
  }
  s2::down_reduce_add<kDownThreads, kCw>(red, acc, kEpl, cs, d, a.y + static_cast<size_t>(b) * d);
}

template <typename T, bool kFromBitmap>
void launch_down_t(const DownArgs& a, dim3 grid, size_t smem, hipStream_t s) {
  if (grid.y == 1)  // one token: every row slice is read once (non-temporal loads)
    hipLaunchKernelGGL((down_kernel<T, kFromBitmap, true>), grid, dim3(kDownThreads), smem, s, a);
  else
    hipLaunchKernelGGL((down_kernel<T, kFromBitmap, false>), grid, dim3(kDownThreads), smem, s, a);
}

}  // namespace

hipError_t launch_down(const DownArgs& a, int wdtype, int batch, bool from_bitmap, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.col_slices * a.row_groups), static_cast<unsigned>(batch));
  const int cw = wdtype == PROX_BF16 ? 512 : 256;
  const size_t smem = static_cast<size_t>(kDownThreads / 64) * cw * 4 + static_cast<size_t>(a.max_rows) * 8;
  if (wdtype == PROX_BF16) {
    if (from_bitmap)
      launch_down_t<Bf16Tag, true>(a, grid, smem, s);
    else
      launch_down_t<Bf16Tag, false>(a, grid, smem, s);
  } else {
    if (from_bitmap)
      launch_down_t<F32Tag, true>(a, grid, smem, s);
    else
      launch_down_t<F32Tag, false>(a, grid, smem, s);
  }
  return hipGetLastError();
}

}  // namespace prox
