// Stage 1 of the Prox decode step with a 16-bit proxy on gfx950: the pages'
// precision ablation, in which the INT4 proxy is replaced by a 16-bit one at
// the same budget ([blog] evidence section, ablation A1).  The proxy is the
// layer's own bf16 weights, stored row-major like the INT4 proxy, so the
// proxy state is the input-sparse projection with the original weights:
//   m_x = 1[|x_i| >= tau_x];  u~ = Pi^in(x, W_up, m_x);
//   s~ = u~ * act(Pi^in(x, W_gate, m_x));  m_s = 1[|s~_j| >= tau_s].
//
// gfx950 design: the batch-1 INT4 kernel with four times the bytes per kept
// row.
//   * grid = (panels x K-splits, batch), split-major; a panel is 128 output
//     columns, a 512-byte run of each kept row: 8 chunks of {16 up, 16 gate}
//     bf16 values.  Each wave compacts the kept rows of a quarter of the
//     split into an LDS list (x_i and the row offset), ascending.
//   * 8 lanes per row, one 64-byte chunk each (four 16-byte loads); a wave
//     keeps 4 rows per lane slot (16 loads) in flight.  bf16 values widen to
//     fp32 exactly; fp32 FMA accumulation.
//   * the K-split partials, the self-resetting ticket and the last block's
//     fixed-order sum, activation and mask bits are the INT4 kernel's.
#include "prox_device.h"
#include "prox_internal.h"

namespace prox {
namespace {

constexpr int kW16Pw = 128;                    // panel width (output columns)
constexpr int kW16Lpr = 8;                     // lanes per row (one 64-byte chunk each)
constexpr int kW16WaveSlots = 64 / kW16Lpr;    // rows per wave step
constexpr int kW16Rows = 4;                    // rows per lane slot in flight
constexpr int kW16RedStride = kThreads + 2;  // conflict-free reduction reads (2 mod 32 words)

__device__ __forceinline__ void acc_bf16x8(float* acc, const u32x4_t& w, float a) {
  acc[0] = fmaf(a, bf16lo(w.x), acc[0]);
  acc[1] = fmaf(a, bf16hi(w.x), acc[1]);
  acc[2] = fmaf(a, bf16lo(w.y), acc[2]);
  acc[3] = fmaf(a, bf16hi(w.y), acc[3]);
  acc[4] = fmaf(a, bf16lo(w.z), acc[4]);
  acc[5] = fmaf(a, bf16hi(w.z), acc[5]);
  acc[6] = fmaf(a, bf16lo(w.w), acc[6]);
  acc[7] = fmaf(a, bf16hi(w.w), acc[7]);
}

template <bool kWriteState>
__global__ __launch_bounds__(kThreads) void stage1_w16_kernel(Stage1Args a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_wave_cnt[4];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.y;
  const int split = blockIdx.x / a.n_panels;
  const int panel = blockIdx.x - split * a.n_panels;
  const int d = a.d;
  const int f = a.f;
  uint8_t* tws = a.ws + static_cast<size_t>(b) * a.tok_bytes;
  unsigned* tickets = reinterpret_cast<unsigned*>(tws + a.off_tickets);
  int* kcount = reinterpret_cast<int*>(tws + a.off_kcount);
  float* partial = reinterpret_cast<float*>(tws + a.off_partial);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(tws + a.off_bitmap);

  // ---- compaction: each wave takes a quarter of this split's rows
  const int row0 = split * a.rows_per_split;
  const int row1 = min(d, row0 + a.rows_per_split);
  const int wchunk = (a.rows_per_split + 3) / 4;
  const int wcap = wchunk + 1;  // one zero-weight sentinel entry per wave
  const int wr0 = min(row1, row0 + wave * wchunk);
  const int wr1 = min(row1, wr0 + wchunk);
  float* ka = reinterpret_cast<float*>(smem) + wave * wcap;
  uint32_t* koff = reinterpret_cast<uint32_t*>(reinterpret_cast<float*>(smem) + 4 * wcap) + wave * wcap;
  const uint16_t* xb = static_cast<const uint16_t*>(a.x) + static_cast<size_t>(b) * d;
  int nkept = 0;
  constexpr int kCompactSteps = 4;
  for (int base = wr0; base < wr1; base += 64 * kCompactSteps) {
    float xv[kCompactSteps];
#pragma unroll
    for (int k = 0; k < kCompactSteps; ++k) xv[k] = bf16_to_f32(xb[min(base + k * 64 + lane, wr1 - 1)]);
#pragma unroll
    for (int k = 0; k < kCompactSteps; ++k) {
      const int i = base + k * 64 + lane;
      const bool keep = i < wr1 && fabsf(xv[k]) >= a.tau_x;
      const uint64_t bal = __ballot(keep);
      if (keep) {
        const int pos = nkept + __popcll(bal & ((1ull << lane) - 1ull));
        ka[pos] = xv[k];
        koff[pos] = static_cast<uint32_t>(i) * static_cast<uint32_t>(a.proxy16_stride);
      }
      nkept += __popcll(bal);
    }
  }
  if (lane == 0) {  // slots past the end read row 0 with weight 0
    ka[nkept] = 0.f;
    koff[nkept] = 0u;
    s_wave_cnt[wave] = nkept;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- main loop: 8 lanes per row, kW16Rows rows per lane slot in flight
  const int wslot = lane / kW16Lpr;
  const int chunk = lane % kW16Lpr;
  const uint8_t* pbase = static_cast<const uint8_t*>(a.proxy_w16) + static_cast<size_t>(panel) * kW16Pw * 4 + chunk * 64;
  float acc_u[16], acc_g[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    acc_u[e] = 0.f;
    acc_g[e] = 0.f;
  }
  for (int r0 = wslot; r0 < nkept; r0 += kW16WaveSlots * kW16Rows) {
    const int rb = r0 - wslot;  // wave-uniform base of this batch
    u32x4_t w[kW16Rows][4];
#pragma unroll
    for (int u = 0; u < kW16Rows; ++u) {
      const uint8_t* p = pbase + koff[min(r0 + u * kW16WaveSlots, nkept)];
#pragma unroll
      for (int q = 0; q < 4; ++q) w[u][q] = *reinterpret_cast<const u32x4_t*>(p + 16 * q);
    }
    __builtin_amdgcn_sched_barrier(0);  // the batch stays in flight together
#pragma unroll
    for (int u = 0; u < kW16Rows; ++u) {
      if (rb + u * kW16WaveSlots < nkept) {
        const float av = ka[min(r0 + u * kW16WaveSlots, nkept)];
        acc_bf16x8(acc_u + 0, w[u][0], av);
        acc_bf16x8(acc_u + 8, w[u][1], av);
        acc_bf16x8(acc_g + 0, w[u][2], av);
        acc_bf16x8(acc_g + 8, w[u][3], av);
      }
    }
  }

  // ---- reduce the row slots (LDS, fixed order)
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    red[e * kW16RedStride + tid] = acc_u[e];
    red[(16 + e) * kW16RedStride + tid] = acc_g[e];
  }
  __syncthreads();
  constexpr int kSlots = kThreads / kW16Lpr;
  const int m = tid / kW16Pw;  // 0 = up, 1 = gate
  const int c = tid % kW16Pw;
  const int ch = c >> 4;
  const int e = c & 15;
  float t = 0.f;
#pragma unroll 8
  for (int sl = 0; sl < kSlots; ++sl) t += red[(m * 16 + e) * kW16RedStride + sl * kW16Lpr + ch];
  const size_t col = static_cast<size_t>(panel) * kW16Pw + c;
  __hip_atomic_store(&partial[(static_cast<size_t>(split) * 2 + m) * f + col], t, __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  if (panel == 0 && tid == 0)
    __hip_atomic_store(&kcount[split], s_wave_cnt[0] + s_wave_cnt[1] + s_wave_cnt[2] + s_wave_cnt[3],
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- last block of this panel: fixed-order sum of the splits, activation, mask
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(&tickets[panel], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == static_cast<unsigned>(a.splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  float* sv = red;  // every thread finished reading red before the ticket barrier
  // k_x: wave 0 of panel 0's last block reads the split counts (stored before
  // the ticket like the partials, one per lane: splits <= 64) right after its
  // first partial loads, so both travel in one round trip
  const bool count_kx = panel == 0 && a.in_count != nullptr && wave == 0;  // wave-uniform
  int kc = 0;
  float tot = 0.f;
  for (int k0 = 0; k0 < a.splits; k0 += 8) {
    float pv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      pv[u] = __hip_atomic_load(&partial[(static_cast<size_t>(min(k0 + u, a.splits - 1)) * 2 + m) * f + col],
                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (k0 == 0 && count_kx)
      kc = __hip_atomic_load(&kcount[min(lane, a.splits - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < a.splits) tot += pv[u];
  }
  sv[tid] = tot;
  __syncthreads();
  if (tid < kW16Pw) {  // waves 0 and 1
    const float st = sv[tid] * gate_act(sv[kW16Pw + tid], a.act);
    const size_t gc = static_cast<size_t>(panel) * kW16Pw + tid;
    if (kWriteState) a.s_tilde[static_cast<size_t>(b) * f + gc] = st;
    const uint64_t bal = __ballot(fabsf(st) >= a.tau_s);
    if (lane == 0) {
      const size_t w0 = (gc - lane) / 32;
      bitmap[w0] = static_cast<uint32_t>(bal);
      bitmap[w0 + 1] = static_cast<uint32_t>(bal >> 32);
    }
  }
  if (tid == 0) __hip_atomic_store(&tickets[panel], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (count_kx) {
    const int t = wave_sum_int(lane < a.splits ? kc : 0);
    if (lane == 0) a.in_count[b] = t;
  }
}

}  // namespace

hipError_t launch_stage1_w16(const Stage1Args& a, int batch, bool write_state, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.n_panels * a.splits), static_cast<unsigned>(batch));
  const size_t kept_bytes = static_cast<size_t>(a.rows_per_split + 4) * (sizeof(float) + sizeof(uint32_t));
  const size_t red_bytes = static_cast<size_t>(32) * kW16RedStride * sizeof(float);
  const size_t smem = kept_bytes > red_bytes ? kept_bytes : red_bytes;
  if (write_state)
    hipLaunchKernelGGL((stage1_w16_kernel<true>), grid, dim3(kThreads), smem, s, a);
  else
    hipLaunchKernelGGL((stage1_w16_kernel<false>), grid, dim3(kThreads), smem, s, a);
  return hipGetLastError();
}

}  // namespace prox
