// Stage 1 of the Prox decode step on gfx950: input-sparse INT4 proxy and the
// shared intermediate-channel mask.
//
// Method ([blog] = deep-dive blog "Prox 完全拆解", section "Stage 1"):
//   m_x = 1[|x_i| >= tau_x];  u~ = Pi^in(x, W~_up, m_x);
//   h~ = SiLU(Pi^in(x, W~_gate, m_x));  s~ = u~ * h~;  m_s = 1[|s~_j| >= tau_s]
// (GELU in place of SiLU for a GeGLU layer: the layer's activation field).
// The pages' kernel ([blog] section on turning the formulas into GPU work) is
// a fused split-N kernel that shares one read of the hidden state between
// the up and gate proxies, skips rejected inputs inside the main loop, unpacks
// INT4 in registers and reduces in FP32, forming s~ and the mask directly.
//
// gfx950 design:
//   * grid = (panels x K-splits, batch).  A panel is 128 output columns, a
//     128-byte run of each kept row (the kernel also builds for 256).  A
//     K-split is a contiguous range of input rows.  Each wave of a block
//     compacts the kept rows of a quarter of that range (ballot + popcount,
//     ascending) into a wave-private LDS list together with a = x_i * scale_i
//     for both proxies, then gathers those rows; no block barrier precedes
//     the gather.
//   * main loop: 8 lanes cover one kept row's 128-byte slice (16 up + 16
//     gate codes per lane, one 16-B load); each lane keeps 16 loads
//     outstanding, so a wave's 128 rows (at 512 rows per split) go out in
//     one batch (with the non-temporal hint when the launch covers one
//     token); x and the two scales of a row are fetched in one round
//     trip.  Rejected rows are never touched, so the bytes read are
//     k_x * panel width per panel.
//   * INT4 unpack: a nibble masked into the low 10 bits of a half word is an
//     f16 subnormal equal to nibble * 2^-24 (or 16 * nibble * 2^-24 for the
//     high nibble of a byte).  v_fma_mix_f32 widens it exactly and fuses the
//     multiply-add with a * 2^24 (or a * 2^20) in fp32: five bit operations
//     and eight FMAs per eight codes.  Codes are stored as code + 8, so the
//     row sums are corrected by 8 * sum(a) once per block.
//   * the K-split partial sums go to the workspace; a self-resetting ticket
//     per panel lets the last block add them in fixed split order (so masks
//     are run-to-run identical), apply the gate activation, ballot |s~| >= tau_s and write
//     the panel's 128 mask bits.
//   * hand-off between blocks without cache-wide maintenance: the partials
//     are written with device-scope stores (sc1: written through to the point
//     of coherence shared by all XCDs), every thread waits for its stores to
//     complete (vmcnt 0) before the block barrier, one thread then bumps the
//     ticket with a device-scope atomic, and the last block reads the
//     partials with device-scope loads (sc1), issued only after its ticket
//     returned.  An agent-scope fence would instead write back and invalidate
//     the whole L2 of the XCD once per wave, which costs far more than the
//     kernel's own traffic.
#include "prox_device.h"
#include "prox_internal.h"

namespace prox {
namespace {

// A kept input row as the gather loop consumes it: a = x_i * scale_i of both
// proxies pre-multiplied by 2^24 and 2^20, and the row's byte offset.
struct KeptA {
  float u24, u20, g24, g20;
};

// Stage-1 block: 4 waves, each taking a quarter of the split's rows;
// kS1Unroll proxy rows per lane per batch.  (8 waves of 8 rows per lane were
// slower: the shorter batches leave less in flight per wave.)
constexpr int kS1Threads = kThreads;
constexpr int kS1Waves = kS1Threads / 64;
constexpr int kS1Unroll = 16;
constexpr int kS1Pw = 128;                       // panel width (output columns)
constexpr int kS1Lpr = kS1Pw / 16;               // lanes per row (16 columns each)
constexpr int kS1WaveSlots = 64 / kS1Lpr;        // rows in flight per wave load
constexpr int kS1BatchRows = kS1WaveSlots * kS1Unroll;
// kept-row lists are sized in whole gather batches
__host__ __device__ constexpr int s1_wave_cap(int rows_per_split) {
  return ((rows_per_split + kS1Waves - 1) / kS1Waves + kS1BatchRows - 1) / kS1BatchRows * kS1BatchRows;
}
constexpr int kS1RedSlots = kS1Threads / kS1Lpr;  // row slots reduced through LDS
// LDS row of the cross-slot reduction: a stride of 2 mod 32 words puts the 32
// reads of a half-wave (16 columns x 2 chunks) in 32 distinct banks
constexpr int kRedStride = kS1RedSlots * kS1Lpr + 2;

// Adds the 8 proxy columns packed in one dword (byte b: column 2b in the low
// nibble, 2b+1 in the high nibble; nibble = code + 8) times `a`, where
// a24 = a * 2^24 and a20 = a * 2^20 (exact power-of-two scalings).
__device__ __forceinline__ void acc_dword(float* acc, uint32_t w, float a24, float a20) {
  const uint32_t t = w >> 8;
  const f16x2_t h0 = __builtin_bit_cast(f16x2_t, w & 0x000F000Fu);  // cols 0 | 4
  const f16x2_t h1 = __builtin_bit_cast(f16x2_t, w & 0x00F000F0u);  // cols 1 | 5
  const f16x2_t h2 = __builtin_bit_cast(f16x2_t, t & 0x000F000Fu);  // cols 2 | 6
  const f16x2_t h3 = __builtin_bit_cast(f16x2_t, t & 0x00F000F0u);  // cols 3 | 7
  acc[0] = fmaf(a24, static_cast<float>(h0.x), acc[0]);
  acc[4] = fmaf(a24, static_cast<float>(h0.y), acc[4]);
  acc[1] = fmaf(a20, static_cast<float>(h1.x), acc[1]);
  acc[5] = fmaf(a20, static_cast<float>(h1.y), acc[5]);
  acc[2] = fmaf(a24, static_cast<float>(h2.x), acc[2]);
  acc[6] = fmaf(a24, static_cast<float>(h2.y), acc[6]);
  acc[3] = fmaf(a20, static_cast<float>(h3.x), acc[3]);
  acc[7] = fmaf(a20, static_cast<float>(h3.y), acc[7]);
}

// kNt: the gather loads carry the non-temporal hint (a launch over one token
// reads each kept row's slice once; over several tokens the rows they share
// are read once per token and stay cacheable).
template <typename T, bool kWriteState, bool kNt>
__global__ __launch_bounds__(kS1Threads) void stage1_kernel(Stage1Args a) {
  constexpr int kPw = kS1Pw;
  constexpr int kLpr = kS1Lpr;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_wave_cnt[kS1Waves];
  __shared__ float s_wave_a[2][kS1Waves];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int b = blockIdx.y;
  // split-major order: blocks dispatched together cover every panel of the
  // same rows (DRAM page locality), and with a panel count divisible by 8 all
  // splits of a panel share an XCD
  const int split = blockIdx.x / a.n_panels;
  const int panel = blockIdx.x - split * a.n_panels;
  const int d = a.d;
  const int f = a.f;
  uint8_t* tws = a.ws + static_cast<size_t>(b) * a.tok_bytes;
  unsigned* tickets = reinterpret_cast<unsigned*>(tws + a.off_tickets);
  int* kcount = reinterpret_cast<int*>(tws + a.off_kcount);
  float* partial = reinterpret_cast<float*>(tws + a.off_partial);
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(tws + a.off_bitmap);

  // ---- compaction: each wave takes a quarter of this split's rows and
  // compacts its kept rows (ascending) into a wave-private LDS list; no block
  // barrier is needed before the gather starts.
  const int row0 = split * a.rows_per_split;
  const int row1 = min(d, row0 + a.rows_per_split);
  constexpr int kWaveSlots = kS1WaveSlots;
  constexpr int kBatchRows = kS1BatchRows;
  const int wchunk = (a.rows_per_split + kS1Waves - 1) / kS1Waves;
  // the lists hold whole batches: positions past the last kept row up to the
  // batch end are zero-weight sentinels that read row 0
  const int wcap = s1_wave_cap(a.rows_per_split);
  const int ucap = wcap / kWaveSlots;
  const int wr0 = min(row1, row0 + wave * wchunk);
  const int wr1 = min(row1, wr0 + wchunk);
  KeptA* ka = reinterpret_cast<KeptA*>(smem) + wave * wcap;
  // row byte offsets, transposed: position p at koff[(p % kWaveSlots) * ucap +
  // p / kWaveSlots], so the offsets a lane gathers in one batch are contiguous
  uint32_t* koff = reinterpret_cast<uint32_t*>(reinterpret_cast<KeptA*>(smem) + kS1Waves * wcap) + wave * wcap;
  constexpr float k2p24 = 16777216.0f;
  constexpr float k2p20 = 1048576.0f;
  int nkept = 0;
  float sum_up = 0.f, sum_gate = 0.f;
  // x and both scales of kCompactSteps 64-row steps are fetched before any is
  // used (one memory round trip for a wave's share at 512 rows per split)
  constexpr int kCompactSteps = 512 / (64 * kS1Waves);
  for (int base = wr0; base < wr1; base += 64 * kCompactSteps) {
    float xv[kCompactSteps], sc_up[kCompactSteps], sc_gate[kCompactSteps];
#pragma unroll
    for (int k = 0; k < kCompactSteps; ++k) {
      const int ii = min(base + k * 64 + lane, wr1 - 1);
      xv[k] = load_elem<T>(a.x, static_cast<size_t>(b) * d + ii);
      sc_up[k] = a.proxy_scale[ii];
      sc_gate[k] = a.proxy_scale[d + ii];
    }
#pragma unroll
    for (int k = 0; k < kCompactSteps; ++k) {
      const int i = base + k * 64 + lane;
      const bool keep = i < wr1 && fabsf(xv[k]) >= a.tau_x;
      const float au = keep ? xv[k] * sc_up[k] : 0.f;
      const float ag = keep ? xv[k] * sc_gate[k] : 0.f;
      const uint64_t bal = __ballot(keep);
      if (keep) {
        const int pos = nkept + __popcll(bal & ((1ull << lane) - 1ull));
        ka[pos] = KeptA{au * k2p24, au * k2p20, ag * k2p24, ag * k2p20};
        koff[(pos % kWaveSlots) * ucap + pos / kWaveSlots] = static_cast<uint32_t>(i) * static_cast<uint32_t>(a.proxy_stride);
      }
      nkept += __popcll(bal);
      sum_up += au;
      sum_gate += ag;
    }
  }
  // sentinels up to the end of the last batch
  for (int p = nkept + lane; p < (nkept + kBatchRows - 1) / kBatchRows * kBatchRows; p += 64) {
    ka[p] = KeptA{0.f, 0.f, 0.f, 0.f};
    koff[(p % kWaveSlots) * ucap + p / kWaveSlots] = 0u;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  sum_up = wave_sum(sum_up);
  sum_gate = wave_sum(sum_gate);
  if (lane == 0) {
    s_wave_a[0][wave] = sum_up;
    s_wave_a[1][wave] = sum_gate;
    s_wave_cnt[wave] = nkept;
  }

  // ---- main loop over the wave's kept rows: kLpr lanes per row
  const int wslot = lane / kLpr;
  const int chunk = lane % kLpr;
  const uint8_t* qbase = a.proxy_q + static_cast<size_t>(panel) * kPw;  // uniform; 32-bit offsets below
  const uint32_t coff = static_cast<uint32_t>(chunk * 16);
  float acc_u[16], acc_g[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    acc_u[e] = 0.f;
    acc_g[e] = 0.f;
  }
  // One batch covers kBatchRows rows, a wave's whole share at 512 rows per
  // split, so every wave makes a single round trip.  The
  // batch's offsets come from LDS as 16-byte vectors, then all its loads are
  // issued (sentinel slots read row 0); a = x_i * scale_i of the next row is
  // read from LDS while the current row is added, and steps with no kept row
  // in any slot are skipped.
  for (int rb = 0; rb < nkept; rb += kBatchRows) {  // wave-uniform
    const uint32_t* ko = koff + wslot * ucap + rb / kWaveSlots;
    uint32_t off[kS1Unroll];
#pragma unroll
    for (int u = 0; u < kS1Unroll; ++u) off[u] = ko[u];
    uint4 w[kS1Unroll];
#pragma unroll
    for (int u = 0; u < kS1Unroll; ++u) w[u] = ldg16_w<kNt>(qbase + (off[u] + coff));
    __builtin_amdgcn_sched_barrier(0);  // the batch stays in flight together
    const KeptA* kb = ka + rb + wslot;
    KeptA cur = kb[0];
#pragma unroll
    for (int u = 0; u < kS1Unroll; ++u) {
      KeptA nxt = cur;
      if (u + 1 < kS1Unroll) nxt = kb[(u + 1) * kWaveSlots];
      if (rb + u * kWaveSlots < nkept) {
        acc_dword(acc_u + 0, w[u].x, cur.u24, cur.u20);
        acc_dword(acc_u + 8, w[u].y, cur.u24, cur.u20);
        acc_dword(acc_g + 0, w[u].z, cur.g24, cur.g20);
        acc_dword(acc_g + 8, w[u].w, cur.g24, cur.g20);
      }
      cur = nxt;
    }
  }

  // ---- reduce the row slots (LDS, fixed order); kept[] is dead now
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    red[e * kRedStride + tid] = acc_u[e];
    red[(16 + e) * kRedStride + tid] = acc_g[e];
  }
  __syncthreads();
  // outputs: threads 0 .. 2 kPw - 1 (up, then gate, of the panel's columns)
  const bool has_out = tid < 2 * kPw;
  const int o = has_out ? tid : 0;
  const int mo = o / kPw;  // 0 = up, 1 = gate
  const size_t col = static_cast<size_t>(panel) * kPw + (o % kPw);
  if (has_out) {
    const int c = o % kPw;
    const int ch = c >> 4;
    const int e = c & 15;
    float t = 0.f;
#pragma unroll 8
    for (int sl = 0; sl < kS1RedSlots; ++sl) t += red[(mo * 16 + e) * kRedStride + sl * kLpr + ch];
    float suma = 0.f;
#pragma unroll
    for (int w = 0; w < kS1Waves; ++w) suma += s_wave_a[mo][w];
    __hip_atomic_store(&partial[(static_cast<size_t>(split) * 2 + mo) * f + col], fmaf(-8.0f, suma, t),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (panel == 0 && tid == 0) {
    int kc = 0;
#pragma unroll
    for (int w = 0; w < kS1Waves; ++w) kc += s_wave_cnt[w];
    __hip_atomic_store(&kcount[split], kc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- last block of this panel: fixed-order sum of the splits, activation, mask
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's stores are complete
  __syncthreads();
  if (tid == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(&tickets[panel], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == static_cast<unsigned>(a.splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!s_last) return;

  // split loads go out in groups of 8 so they travel together; the sums keep
  // the fixed split order
  float* sv = red;  // every thread finished reading red before the ticket barrier
  // k_x: wave 0 of panel 0's last block reads the split counts (stored before
  // the ticket like the partials, one per lane: splits <= 64) right after its
  // first partial loads, so both travel in one round trip
  const bool count_kx = panel == 0 && a.in_count != nullptr && wave == 0;  // wave-uniform
  int kc = 0;
  if (has_out) {
    float tot = 0.f;
    for (int k0 = 0; k0 < a.splits; k0 += 8) {
      float pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int kk = min(k0 + u, a.splits - 1);
        pv[u] = __hip_atomic_load(&partial[(static_cast<size_t>(kk) * 2 + mo) * f + col], __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
      }
      if (k0 == 0 && count_kx)
        kc = __hip_atomic_load(&kcount[min(lane, a.splits - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u < a.splits) tot += pv[u];
    }
    sv[tid] = tot;
  }
  __syncthreads();
  for (int c = tid; c < kPw; c += kS1Threads) {  // wave-uniform trip count
    const float uu = sv[c];
    const float gg = sv[kPw + c];
    const float st = uu * gate_act(gg, a.act);
    const size_t gc = static_cast<size_t>(panel) * kPw + c;
    if (kWriteState) a.s_tilde[static_cast<size_t>(b) * f + gc] = st;
    const uint64_t bal = __ballot(fabsf(st) >= a.tau_s);
    if (lane == 0) {
      const size_t w0 = (gc - lane) / 32;
      bitmap[w0] = static_cast<uint32_t>(bal);
      bitmap[w0 + 1] = static_cast<uint32_t>(bal >> 32);
    }
  }
  // ready for the next stream-ordered call
  if (tid == 0) __hip_atomic_store(&tickets[panel], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (count_kx) {
    const int t = wave_sum_int(lane < a.splits ? kc : 0);
    if (lane == 0) a.in_count[b] = t;
  }
}

template <typename T, bool kWriteState>
void launch_stage1_t(const Stage1Args& a, dim3 grid, size_t smem, hipStream_t s) {
  if (grid.y == 1)  // one token: every kept row's slice is read once (non-temporal loads)
    hipLaunchKernelGGL((stage1_kernel<T, kWriteState, true>), grid, dim3(kS1Threads), smem, s, a);
  else
    hipLaunchKernelGGL((stage1_kernel<T, kWriteState, false>), grid, dim3(kS1Threads), smem, s, a);
}

}  // namespace

hipError_t launch_stage1(const Stage1Args& a, int wdtype, int batch, bool write_state,
                         hipStream_t s) {
  if (a.proxy_kind == PROX_PROXY_W16) return launch_stage1_w16(a, batch, write_state, s);
  const dim3 grid(static_cast<unsigned>(a.n_panels * a.splits), static_cast<unsigned>(batch));
  const size_t kept_bytes =
      static_cast<size_t>(kS1Waves) * s1_wave_cap(a.rows_per_split) * (sizeof(KeptA) + sizeof(uint32_t));
  const size_t red_bytes = static_cast<size_t>(32) * kRedStride * sizeof(float);
  const size_t smem = kept_bytes > red_bytes ? kept_bytes : red_bytes;
  if (wdtype == PROX_BF16) {
    if (write_state)
      launch_stage1_t<Bf16Tag, true>(a, grid, smem, s);
    else
      launch_stage1_t<Bf16Tag, false>(a, grid, smem, s);
  } else {
    if (write_state)
      launch_stage1_t<F32Tag, true>(a, grid, smem, s);
    else
      launch_stage1_t<F32Tag, false>(a, grid, smem, s);
  }
  return hipGetLastError();
}

}  // namespace prox
