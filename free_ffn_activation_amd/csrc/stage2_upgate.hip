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
//     loads, 16 KB per wave) are issued before use, with the non-temporal
//     hint when the launch covers one token (each run is then read once).  x is staged in LDS once
//     per block; the block's one barrier comes after the first weight loads
//     are issued, so it overlaps the gather.  bf16 products use
//     v_dot2_f32_bf16 (exact products, fp32 sum).
//   * a wave reduction gives u_j and g_j; lane 0 stores s_j = u_j act(g_j).
//   * this kernel also zeroes y, which the down kernel accumulates into.
// The block's work is s2::upgate_block (stage2_common.h), shared with the
// fused Stage-2 kernel.
#include "stage2_common.h"

namespace prox {
namespace {

template <typename T, bool kFromBitmap, bool kNt>
__global__ __launch_bounds__(kUgThreads) void upgate_kernel(UpGateArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  s2::upgate_block<T, kFromBitmap, kUgThreads, true, kNt>(a, static_cast<int>(blockIdx.x),
                                                          static_cast<int>(gridDim.x),
                                                          static_cast<int>(blockIdx.y), smem);
}

template <typename T, bool kFromBitmap>
void launch_upgate_t(const UpGateArgs& a, dim3 grid, size_t smem, hipStream_t s) {
  if (grid.y == 1)  // one token: every weight run is read once (non-temporal loads)
    hipLaunchKernelGGL((upgate_kernel<T, kFromBitmap, true>), grid, dim3(kUgThreads), smem, s, a);
  else
    hipLaunchKernelGGL((upgate_kernel<T, kFromBitmap, false>), grid, dim3(kUgThreads), smem, s, a);
}

}  // namespace

hipError_t launch_upgate(const UpGateArgs& a, int wdtype, int batch, int blocks,
                         bool from_bitmap, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(batch));
  const size_t esz = wdtype == PROX_BF16 ? 2 : 4;
  const size_t smem = static_cast<size_t>(a.d) * esz;
  if (wdtype == PROX_BF16) {
    if (from_bitmap)
      launch_upgate_t<Bf16Tag, true>(a, grid, smem, s);
    else
      launch_upgate_t<Bf16Tag, false>(a, grid, smem, s);
  } else {
    if (from_bitmap)
      launch_upgate_t<F32Tag, true>(a, grid, smem, s);
    else
      launch_upgate_t<F32Tag, false>(a, grid, smem, s);
  }
  return hipGetLastError();
}

}  // namespace prox
