// Offline kernels: proxy packing, layout transforms, workspace fill and the
// digit histograms used by calibration.
//
// Packing ([blog] = deep-dive blog "Prox 完全拆解", section "Stage 1": the up
// and gate proxies are symmetric per-row INT4 copies kept resident on the GPU;
// W_down has none).  A row is a row of the [d_model, d_ff] matrix, i.e. one
// input coordinate, so Stage 1 reads one contiguous run per kept coordinate.
// Rows are qstride bytes apart (an odd multiple of 128): Stage 1 reads one
// 128-byte column slice from many rows, and a stride with a large power-of-two
// factor would send all of a slice's reads to a few HBM channels.
// scale = fp32(absmax / 7); code = clamp(rint_half_even(fp32(w / scale)),
// -7, 7) with IEEE-rounded fp32 divisions; a zero row has scale 0, codes 0.
#include "prox_device.h"
#include "prox_internal.h"

namespace prox {
namespace {

__device__ __forceinline__ int quant_code(float w, float sc) {
  if (!(sc > 0.f)) return 0;
  const float q = rintf(__fdiv_rn(w, sc));
  return static_cast<int>(fminf(7.f, fmaxf(-7.f, q)));
}

// One block per input row: absmax of the row in both matrices, the two scales,
// then the packed 16-byte groups (8 bytes up codes, 8 bytes gate codes).
template <typename T>
__global__ __launch_bounds__(kThreads) void pack_rows_kernel(const void* wu, const void* wg, int d,
                                                              int f, int qstride, uint8_t* q,
                                                              float* scale) {
  __shared__ float s_max[2][4];
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t rb = static_cast<size_t>(i) * f;
  float mu = 0.f, mg = 0.f;
  for (int c = tid; c < f; c += kThreads) {
    mu = fmaxf(mu, fabsf(load_elem<T>(wu, rb + c)));
    mg = fmaxf(mg, fabsf(load_elem<T>(wg, rb + c)));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    mu = fmaxf(mu, __shfl_xor(mu, m, 64));
    mg = fmaxf(mg, __shfl_xor(mg, m, 64));
  }
  if ((tid & 63) == 0) {
    s_max[0][tid >> 6] = mu;
    s_max[1][tid >> 6] = mg;
  }
  __syncthreads();
  const float au = fmaxf(fmaxf(s_max[0][0], s_max[0][1]), fmaxf(s_max[0][2], s_max[0][3]));
  const float ag = fmaxf(fmaxf(s_max[1][0], s_max[1][1]), fmaxf(s_max[1][2], s_max[1][3]));
  const float su = __fdiv_rn(au, 7.0f);
  const float sg = __fdiv_rn(ag, 7.0f);
  if (tid == 0) {
    scale[i] = su;
    scale[d + i] = sg;
  }
  for (int g = tid; g < f / 16; g += kThreads) {
    uint32_t up[2] = {0u, 0u}, gt[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const size_t c = rb + static_cast<size_t>(g) * 16 + k;
      const uint32_t nu = static_cast<uint32_t>(quant_code(load_elem<T>(wu, c), su) + 8);
      const uint32_t ng = static_cast<uint32_t>(quant_code(load_elem<T>(wg, c), sg) + 8);
      up[k >> 3] |= nu << (4 * (k & 7));
      gt[k >> 3] |= ng << (4 * (k & 7));
    }
    *reinterpret_cast<uint4*>(q + static_cast<size_t>(i) * qstride + static_cast<size_t>(g) * 16) =
        make_uint4(up[0], up[1], gt[0], gt[1]);
  }
  // zero the row's padding bytes (qstride - f, a multiple of 16)
  for (int o = f + tid * 16; o < qstride; o += kThreads * 16)
    *reinterpret_cast<uint4*>(q + static_cast<size_t>(i) * qstride + o) = make_uint4(0u, 0u, 0u, 0u);
}

// dst[j][which][i] = src[i][j] for src [d][f]; 64x64 tiles through LDS.
template <typename S>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const S* __restrict__ src, int d, int f,
                                                              S* __restrict__ dst, int which) {
  __shared__ S tile[64][65];
  const int j0 = blockIdx.x * 64;
  const int i0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63;
  const int ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) tile[r][tx] = src[static_cast<size_t>(i0 + r) * f + j0 + tx];
  __syncthreads();
  for (int r = ty; r < 64; r += 4)
    dst[static_cast<size_t>(j0 + r) * 2 * d + static_cast<size_t>(which) * d + i0 + tx] = tile[tx][r];
}

__global__ void fill_zero_kernel(uint8_t* p, size_t bytes) {
  const size_t n4 = bytes / 4;
  uint32_t* p4 = reinterpret_cast<uint32_t*>(p);
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n4; i += stride)
    p4[i] = 0u;
  if (blockIdx.x == 0 && threadIdx.x < (bytes & 3)) p[n4 * 4 + threadIdx.x] = 0;
}

// Histogram of the 8-bit digit at `shift` of the keys |v| (fp32 bit patterns,
// sign cleared) whose bits under prefix_mask equal prefix.
template <typename T>
__global__ __launch_bounds__(kThreads) void digit_hist_kernel(const void* v, size_t n, uint32_t prefix,
                                                               uint32_t prefix_mask, int shift,
                                                               uint32_t* hist) {
  __shared__ uint32_t h[256];
  h[threadIdx.x] = 0u;
  __syncthreads();
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; i < n; i += stride) {
    const uint32_t key = __float_as_uint(load_elem<T>(v, i)) & 0x7FFFFFFFu;
    if ((key & prefix_mask) == prefix) atomicAdd(&h[(key >> shift) & 255u], 1u);
  }
  __syncthreads();
  if (h[threadIdx.x]) atomicAdd(&hist[threadIdx.x], h[threadIdx.x]);
}

// |v[floor(i N / M)]| for i < M as fp32 (an evenly strided sample), and the
// sample maximum: fp32 bits of non-negative values order as unsigned ints, so
// one atomicMax per block on the bits gives the maximum.
template <typename T>
__global__ __launch_bounds__(kThreads) void sample_abs_kernel(const void* v, uint64_t n, uint32_t m, float* out,
                                                               uint32_t* maxbits) {
  __shared__ uint32_t s_max[kThreads / 64];
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  float a = 0.f;
  if (i < m) {
    a = fabsf(load_elem<T>(v, (static_cast<uint64_t>(i) * n) / m));
    out[i] = a;
  }
  uint32_t bits = __float_as_uint(a);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) bits = max(bits, static_cast<uint32_t>(__shfl_xor(static_cast<int>(bits), o, 64)));
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = bits;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = s_max[0];
    for (int k = 1; k < kThreads / 64; ++k) b = max(b, s_max[k]);
    atomicMax(maxbits, b);
  }
}

// Linear histogram: bin = min(nb - 1, floor(v / w)) with an IEEE fp32
// division, counted in LDS and added to the global counts.
__global__ __launch_bounds__(kThreads) void bin_hist_kernel(const float* v, uint32_t m, float w, int nb,
                                                             uint32_t* hist) {
  extern __shared__ uint32_t h[];
  for (int b = threadIdx.x; b < nb; b += kThreads) h[b] = 0u;
  __syncthreads();
  const uint32_t stride = gridDim.x * kThreads;
  for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < m; i += stride) {
    const float q = __fdiv_rn(v[i], w);
    const int b = q >= static_cast<float>(nb) ? nb - 1 : static_cast<int>(q);
    atomicAdd(&h[b], 1u);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < nb; b += kThreads)
    if (h[b]) atomicAdd(&hist[b], h[b]);
}

}  // namespace

hipError_t launch_sample_abs(const void* v, uint64_t n, int vdtype, uint32_t m, float* out, uint32_t* maxbits,
                             hipStream_t s) {
  const unsigned blocks = (m + kThreads - 1) / kThreads;
  if (vdtype == PROX_BF16)
    hipLaunchKernelGGL((sample_abs_kernel<Bf16Tag>), dim3(blocks), dim3(kThreads), 0, s, v, n, m, out, maxbits);
  else
    hipLaunchKernelGGL((sample_abs_kernel<F32Tag>), dim3(blocks), dim3(kThreads), 0, s, v, n, m, out, maxbits);
  return hipGetLastError();
}

hipError_t launch_bin_hist(const float* v, uint32_t m, float w, int nb, uint32_t* hist, hipStream_t s) {
  unsigned blocks = (m + kThreads - 1) / kThreads;
  if (blocks > 1024) blocks = 1024;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(bin_hist_kernel, dim3(blocks), dim3(kThreads), static_cast<size_t>(nb) * 4, s, v, m, w, nb,
                     hist);
  return hipGetLastError();
}

hipError_t launch_pack(const void* w_up, const void* w_gate, int d, int f, int qstride, int wdtype,
                       uint8_t* proxy_q, float* proxy_scale, void* w_upgate_t, hipStream_t s) {
  const dim3 tgrid(static_cast<unsigned>(f / 64), static_cast<unsigned>(d / 64));
  if (wdtype == PROX_BF16) {
    hipLaunchKernelGGL((pack_rows_kernel<Bf16Tag>), dim3(d), dim3(kThreads), 0, s, w_up, w_gate, d, f,
                       qstride, proxy_q, proxy_scale);
    hipLaunchKernelGGL((transpose_kernel<uint16_t>), tgrid, dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(w_up), d, f, static_cast<uint16_t*>(w_upgate_t), 0);
    hipLaunchKernelGGL((transpose_kernel<uint16_t>), tgrid, dim3(kThreads), 0, s,
                       static_cast<const uint16_t*>(w_gate), d, f, static_cast<uint16_t*>(w_upgate_t), 1);
  } else {
    hipLaunchKernelGGL((pack_rows_kernel<F32Tag>), dim3(d), dim3(kThreads), 0, s, w_up, w_gate, d, f,
                       qstride, proxy_q, proxy_scale);
    hipLaunchKernelGGL((transpose_kernel<float>), tgrid, dim3(kThreads), 0, s,
                       static_cast<const float*>(w_up), d, f, static_cast<float*>(w_upgate_t), 0);
    hipLaunchKernelGGL((transpose_kernel<float>), tgrid, dim3(kThreads), 0, s,
                       static_cast<const float*>(w_gate), d, f, static_cast<float*>(w_upgate_t), 1);
  }
  return hipGetLastError();
}

// 16-bit proxy rows: row i = 16-column groups of {16 up, 16 gate} bf16 values
// (64 bytes), then zero padding up to the row stride.  One thread per 16 bytes.
__global__ __launch_bounds__(kThreads) void pack16_kernel(const uint16_t* wu, const uint16_t* wg, int d, int f,
                                                          int stride, uint8_t* out) {
  const size_t upr = static_cast<size_t>(stride) / 16;  // 16-byte units per row
  const size_t n = static_cast<size_t>(d) * upr;
  for (size_t idx = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x; idx < n;
       idx += static_cast<size_t>(gridDim.x) * kThreads) {
    const size_t i = idx / upr;
    const int u = static_cast<int>(idx - i * upr);
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (u < f / 4) {
      const int c = u >> 2;  // 16-column group
      const int q = u & 3;   // 0, 1: up values 8q..; 2, 3: gate values 8(q-2)..
      const uint16_t* src = (q < 2 ? wu : wg) + i * f + 16 * c + 8 * (q & 1);
      v = *reinterpret_cast<const u32x4_t*>(src);
    }
    *reinterpret_cast<u32x4_t*>(out + i * stride + 16 * static_cast<size_t>(u)) = v;
  }
}

hipError_t launch_pack16(const void* w_up, const void* w_gate, int d, int f, int stride, void* proxy_w16,
                         hipStream_t s) {
  const size_t n = static_cast<size_t>(d) * (stride / 16);
  size_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(pack16_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s,
                     static_cast<const uint16_t*>(w_up), static_cast<const uint16_t*>(w_gate), d, f, stride,
                     static_cast<uint8_t*>(proxy_w16));
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = (bytes / 4 + kThreads - 1) / kThreads;
  if (blocks > 2048) blocks = 2048;
  if (blocks == 0) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s,
                     static_cast<uint8_t*>(p), bytes);
  return hipGetLastError();
}

hipError_t launch_digit_histogram(const void* v, size_t n, int vdtype, uint32_t prefix,
                                  uint32_t prefix_mask, int shift, uint32_t* hist, hipStream_t s) {
  size_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 1024) blocks = 1024;
  if (blocks == 0) blocks = 1;
  if (vdtype == PROX_BF16)
    hipLaunchKernelGGL((digit_hist_kernel<Bf16Tag>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, s, v, n, prefix, prefix_mask, shift, hist);
  else
    hipLaunchKernelGGL((digit_hist_kernel<F32Tag>), dim3(static_cast<unsigned>(blocks)), dim3(kThreads),
                       0, s, v, n, prefix, prefix_mask, shift, hist);
  return hipGetLastError();
}

}  // namespace prox
