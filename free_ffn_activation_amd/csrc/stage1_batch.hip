// Stage 1 of the Prox decode step for a group of 2..8 tokens on gfx950:
// input-sparse INT4 proxy of every token of the group on the matrix cores.
//
// Method ([blog] = deep-dive blog "Prox 完全拆解", section "Stage 1"), per
// token b of the group:
//   m_x,b = 1[|x_b,i| >= tau_x];  u~_b = Pi^in(x_b, W~_up, m_x,b);
//   s~_b = u~_b * act(Pi^in(x_b, W~_gate, m_x,b));  m_s,b = 1[|s~_b,j| >= tau_s]
// The pages study batch 1 and leave larger batches open ([blog] limitations
// section).  Here a group of tokens reads each proxy row once: the union of
// the tokens' kept rows is gathered, and a token that rejects a row gets a
// zero weight for it, so every token still sees exactly its own input mask.
//
// gfx950 design:
//   * grid = panels x K-splits (split-major, as the batch-1 kernel), one
//     block per (panel of 128 output columns, range of input rows), all
//     tokens of the group in the block.
//   * contraction on the matrix cores, v_mfma_f32_16x16x32_f16: the 16 rows
//     of the A operand are (token, part) pairs, the token's weights
//     a = x_b,i * scale_i split into a high and a low f16 part (hi + lo
//     carries ~22 significant bits; products with the small integer codes are
//     exact and accumulate in fp32), after a per-block, per-token power-of-two
//     scaling that puts the largest |a| in [2^14, 2^15).
//   * the B operand comes straight from the row-major codes: a union row's
//     128-byte panel slice is staged in LDS, and ds_read_b64_tr_b4 hands each
//     lane one output column of 16 consecutive staged rows (nibble i = row i),
//     two MFMA operands of 8 rows, turned into signed f16 codes exactly (the
//     high nibble of a byte gives 16 * code, and its A entry is divided by 16).
//   * the K-split partials, the ticket and the last block's fixed-order sum,
//     activation and mask bits are those of the batch-1 kernel, per token.
#include "prox_device.h"
#include "prox_internal.h"

namespace prox {
namespace {

typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2_t;

constexpr int kChunkRows = 512;                  // input rows per pass
constexpr int kTileRows = 64;                    // rows per pair of MFMA K-steps
constexpr int kTiles = kChunkRows / kTileRows;   // 8
constexpr int kPhaseRows = 128;                  // rows staged in LDS at a time
constexpr int kLoads = kChunkRows * 128 / 16 / kThreads;  // 16 B loads per thread per pass
constexpr int kPw = 128;                         // panel width (output columns)
constexpr f32x4_t kZero4 = {0.f, 0.f, 0.f, 0.f};

// LDS: the A operands of one pass [mat][tile][half][k-group][m][8], the staged
// code rows of one phase, the pass's union-row offsets, per-wave statistics.
struct S1BShared {
  _Float16 A[2][kTiles][2][4][16][8];
  uint8_t B[kPhaseRows * kPw];
  uint32_t uoff[kChunkRows];
  float wmax[4][kBatchMax];
  int wkept[4][kBatchMax];
  int wunion[4];
  int sexp[kBatchMax];
  int last;
};

// Eight stored nibbles (code + 8) of one column, rows in the order
// 0, 4, 1, 5, 2, 6, 3, 7 of the dword, as signed f16 codes: a nibble n masked
// under the exponent of 1024 is the f16 1024 + n (1024 + 16 n for a high
// nibble), and one packed f16 subtraction of 1032 (1152) leaves exactly
// n - 8 (16 (n - 8)).  Signed codes keep the matrix core's rounding of each
// product unbiased across columns; offset codes make every product carry the
// sign of the weight a and their rounding would add up over the rows.
__device__ __forceinline__ f16x8_t codes_to_f16(uint32_t w) {
  const uint32_t t = w >> 8;
  const f16x2_t lo_fix = {static_cast<_Float16>(-1032.0f), static_cast<_Float16>(-1032.0f)};
  const f16x2_t hi_fix = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
  const f16x2_t p0 = __builtin_bit_cast(f16x2_t, (w & 0x000F000Fu) | 0x64006400u) + lo_fix;
  const f16x2_t p1 = __builtin_bit_cast(f16x2_t, (w & 0x00F000F0u) | 0x64006400u) + hi_fix;
  const f16x2_t p2 = __builtin_bit_cast(f16x2_t, (t & 0x000F000Fu) | 0x64006400u) + lo_fix;
  const f16x2_t p3 = __builtin_bit_cast(f16x2_t, (t & 0x00F000F0u) | 0x64006400u) + hi_fix;
  return f16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// exponent e with m < 2^e (frexp), clamped so 2^(15-e) and 2^(e-15) stay normal
__device__ __forceinline__ int scale_exponent(float m) {
  if (!(m > 0.f)) return 0;
  int e;
  (void)frexpf(m, &e);
  return max(-111, min(118, e));
}

template <typename T, bool kWriteState>
__global__ __launch_bounds__(kThreads) void stage1_batch_kernel(Stage1Args a) {
  __shared__ __align__(16) S1BShared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int split = blockIdx.x / a.n_panels;
  const int panel = blockIdx.x - split * a.n_panels;
  const int d = a.d;
  const int f = a.f;
  const int nt = a.nt;
  const int row0 = split * a.rows_per_split;
  const int row1 = min(d, row0 + a.rows_per_split);

  // per-lane counts of kept rows per token
  int kept[kBatchMax];
#pragma unroll
  for (int t = 0; t < kBatchMax; ++t) kept[t] = 0;
  // unscaled partial sums of this block, per (chunk of the wave, matrix, token)
  float acc[2][2][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) (&acc[0][0][0])[i] = 0.f;

  const int g = lane >> 4;   // MFMA k-group
  const int mrow = lane & 15;  // A row: token mrow/2, part mrow%2
  constexpr float kInv16 = 0.0625f;

  for (int c0 = row0; c0 < row1; c0 += kChunkRows) {
    const int c1 = min(row1, c0 + kChunkRows);
    // ---- clear the A operands: rows no token keeps, tokens past nt and
    // padding slots stay zero
    {
      u32x4_t* az = reinterpret_cast<u32x4_t*>(&sh.A[0][0][0][0][0][0]);
      constexpr int n16 = static_cast<int>(sizeof(sh.A) / 16);
      const u32x4_t z = {0u, 0u, 0u, 0u};
      for (int i = tid; i < n16; i += kThreads) az[i] = z;
    }
    // ---- input masks of the pass: wave w takes rows c0 + 128w + [0, 128)
    float xv[2][kBatchMax];
    uint32_t keep[2];
    float sc_u[2], sc_g[2];
    float lmax[kBatchMax];
#pragma unroll
    for (int t = 0; t < kBatchMax; ++t) lmax[t] = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = c0 + 128 * wave + 64 * k + lane;
      const int ii = min(i, c1 - 1);
      sc_u[k] = a.proxy_scale[ii];
      sc_g[k] = a.proxy_scale[d + ii];
#pragma unroll
      for (int t = 0; t < kBatchMax; ++t)
        xv[k][t] = load_elem<T>(a.x, static_cast<size_t>(min(t, nt - 1)) * d + ii);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int i = c0 + 128 * wave + 64 * k + lane;
      uint32_t m = 0u;
#pragma unroll
      for (int t = 0; t < kBatchMax; ++t) {
        const bool kp = t < nt && i < c1 && fabsf(xv[k][t]) >= a.tau_x;
        m |= kp ? (1u << t) : 0u;
        if (kp) lmax[t] = fmaxf(lmax[t], fmaxf(fabsf(xv[k][t] * sc_u[k]), fabsf(xv[k][t] * sc_g[k])));
      }
      keep[k] = m;
    }
    const uint64_t bal0 = __ballot(keep[0] != 0u);
    const uint64_t bal1 = __ballot(keep[1] != 0u);
#pragma unroll
    for (int t = 0; t < kBatchMax; ++t) {
      float v = lmax[t];
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
      if (lane == 0) sh.wmax[wave][t] = v;
    }
    if (lane == 0) sh.wunion[wave] = __popcll(bal0) + __popcll(bal1);
    __syncthreads();
    int sexp[kBatchMax];
    float scale[kBatchMax];
#pragma unroll
    for (int t = 0; t < kBatchMax; ++t) {
      const float m = fmaxf(fmaxf(sh.wmax[0][t], sh.wmax[1][t]), fmaxf(sh.wmax[2][t], sh.wmax[3][t]));
      sexp[t] = scale_exponent(m);
      scale[t] = ldexpf(1.0f, 15 - sexp[t]);
    }
    int wbase = 0;
    for (int w = 0; w < wave; ++w) wbase += sh.wunion[w];
    const int nu = sh.wunion[0] + sh.wunion[1] + sh.wunion[2] + sh.wunion[3];
    // ---- union slots (ascending rows) and the A operands
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (keep[k] == 0u) continue;
      const int i = c0 + 128 * wave + 64 * k + lane;
      const int slot = wbase + (k == 0 ? __popcll(bal0 & below) : __popcll(bal0) + __popcll(bal1 & below));
      sh.uoff[slot] = static_cast<uint32_t>(i) * static_cast<uint32_t>(a.proxy_stride);
      const int tile = slot / kTileRows;
      const int gg = (slot >> 4) & 3;
      const int h = (slot >> 3) & 1;
      const int r = slot & 7;
      const int e = 2 * (r & 3) + (r >> 2);
      const float rs = (r & 1) ? kInv16 : 1.0f;  // odd rows pair with high nibbles
#pragma unroll
      for (int t = 0; t < kBatchMax; ++t) {
        if (!((keep[k] >> t) & 1u)) continue;
        ++kept[t];
#pragma unroll
        for (int mat = 0; mat < 2; ++mat) {
          const float av = xv[k][t] * (mat == 0 ? sc_u[k] : sc_g[k]);
          const float v = av * scale[t] * rs;
          const _Float16 hi = static_cast<_Float16>(v);
          const _Float16 lo = static_cast<_Float16>(v - static_cast<float>(hi));
          sh.A[mat][tile][h][gg][2 * t][e] = hi;
          sh.A[mat][tile][h][gg][2 * t + 1][e] = lo;
        }
      }
    }
    if (tid < kBatchMax) sh.sexp[tid] = sexp[tid];
    __syncthreads();

    // ---- gather the union rows' panel slices: thread -> (row tid/8 + 32u, 16-B chunk tid%8)
    const int ntile = (nu + kTileRows - 1) / kTileRows;
    const int rows_pad = ntile * kTileRows;
    const int chunk = tid & 7;
    const uint8_t* pbase = a.proxy_q + static_cast<size_t>(panel) * kPw + chunk * 16;
    u32x4_t wld[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      wld[u] = u32x4_t{0u, 0u, 0u, 0u};
      if (u * 32 < rows_pad) {  // block-uniform (rows_pad is a multiple of 64)
        const int rs = u * 32 + (tid >> 3);
        wld[u] = *reinterpret_cast<const u32x4_t*>(pbase + sh.uoff[min(rs, nu - 1)]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    f32x4_t C[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) (&C[0][0])[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < kChunkRows / kPhaseRows; ++q) {
      if (q * kPhaseRows >= rows_pad) break;  // block-uniform
      // stage 128 rows: row r, chunk c at 16 * (c ^ (r & 7)), halves swapped
      // when bit 3 of r is set (conflict-free transposed reads)
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        const int r = uu * 32 + (tid >> 3);
        u32x4_t v = wld[q * 4 + uu];
        if ((r >> 3) & 1) v = u32x4_t{v.z, v.w, v.x, v.y};
        *reinterpret_cast<u32x4_t*>(&sh.B[r * kPw + 16 * (chunk ^ (r & 7))]) = v;
      }
      __syncthreads();
#pragma unroll
      for (int tl = 0; tl < kPhaseRows / kTileRows; ++tl) {
        if (q * kPhaseRows + tl * kTileRows >= rows_pad) break;  // block-uniform
        const int tile = q * (kPhaseRows / kTileRows) + tl;
        const f16x8_t au0 = *reinterpret_cast<const f16x8_t*>(&sh.A[0][tile][0][g][mrow][0]);
        const f16x8_t au1 = *reinterpret_cast<const f16x8_t*>(&sh.A[0][tile][1][g][mrow][0]);
        const f16x8_t ag0 = *reinterpret_cast<const f16x8_t*>(&sh.A[1][tile][0][g][mrow][0]);
        const f16x8_t ag1 = *reinterpret_cast<const f16x8_t*>(&sh.A[1][tile][1][g][mrow][0]);
        const int r = tl * kTileRows + 16 * g + (lane & 15);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int c = 2 * wave + cc;
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int off = r * kPw + 16 * (c ^ (r & 7)) + 8 * (hf ^ ((r >> 3) & 1));
            const i32x2_t v = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                (__attribute__((address_space(3))) i32x2_t*)((__attribute__((address_space(3))) uint8_t*)(sh.B) + off));
            const f16x8_t b0 = codes_to_f16(static_cast<uint32_t>(v[0]));
            const f16x8_t b1 = codes_to_f16(static_cast<uint32_t>(v[1]));
            // each pair of K-steps starts from zero and is added with a VALU
            // add: the matrix core aligns its products to the largest term,
            // and a large running sum would cost the small products bits
            f32x4_t t = __builtin_amdgcn_mfma_f32_16x16x32_f16(hf == 0 ? au0 : ag0, b0, kZero4, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_16x16x32_f16(hf == 0 ? au1 : ag1, b1, t, 0, 0, 0);
            C[cc][hf] += t;
          }
        }
      }
      __syncthreads();  // the staging buffer is rewritten by the next phase
    }
    // ---- fold the pass into unscaled fp32 sums: rows 4g..4g+3 of C are
    // tokens 2g (hi, lo) and 2g+1 (hi, lo)
    const int e0 = sh.sexp[2 * g];
    const int e1 = sh.sexp[2 * g + 1];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        acc[cc][hf][0] += ldexpf(C[cc][hf][0] + C[cc][hf][1], e0 - 15);
        acc[cc][hf][1] += ldexpf(C[cc][hf][2] + C[cc][hf][3], e1 - 15);
      }
    __syncthreads();  // sexp, wmax and A are rewritten by the next pass
  }

  // ---- block totals of the kept counts per token
#pragma unroll
  for (int t = 0; t < kBatchMax; ++t) {
    const int kc = wave_sum_int(kept[t]);
    if (lane == 0) sh.wkept[wave][t] = kc;
  }
  __syncthreads();

  // ---- partials: lane (g, n) holds tokens 2g, 2g+1 of column n of its chunks
  const int n = lane & 15;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = 2 * g + tt;
    if (t >= nt) continue;
    float* partial = reinterpret_cast<float*>(a.ws + static_cast<size_t>(t) * a.tok_bytes + a.off_partial);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int col = panel * kPw + (2 * wave + cc) * 16 + n;
        __hip_atomic_store(&partial[(static_cast<size_t>(split) * 2 + hf) * f + col], acc[cc][hf][tt],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (panel == 0 && tid < nt) {
    int* kcount = reinterpret_cast<int*>(a.ws + static_cast<size_t>(tid) * a.tok_bytes + a.off_kcount);
    __hip_atomic_store(&kcount[split], (sh.wkept[0][tid] + sh.wkept[1][tid]) + (sh.wkept[2][tid] + sh.wkept[3][tid]),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- last block of this panel: fixed-order sum of the splits per token,
  // activation, mask bits (the group's tickets live in its first token's slice)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  unsigned* tickets = reinterpret_cast<unsigned*>(a.ws + a.off_tickets);
  if (tid == 0) {
    const unsigned prev =
        __hip_atomic_fetch_add(&tickets[panel], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sh.last = (prev == static_cast<unsigned>(a.splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!sh.last) return;

  float* sv = reinterpret_cast<float*>(sh.B);
  const int mm = tid / kPw;  // 0 = up, 1 = gate
  const int cl = tid % kPw;
  const size_t col = static_cast<size_t>(panel) * kPw + cl;
  for (int t = 0; t < nt; ++t) {
    uint8_t* tws = a.ws + static_cast<size_t>(t) * a.tok_bytes;
    const float* partial = reinterpret_cast<const float*>(tws + a.off_partial);
    float tot = 0.f;
    for (int k0 = 0; k0 < a.splits; k0 += 8) {
      float pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int kk = min(k0 + u, a.splits - 1);
        pv[u] = __hip_atomic_load(&partial[(static_cast<size_t>(kk) * 2 + mm) * f + col],
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u < a.splits) tot += pv[u];
    }
    sv[tid] = tot;
    __syncthreads();
    if (tid < kPw) {  // waves 0 and 1
      const float st = sv[tid] * gate_act(sv[kPw + tid], a.act);
      const size_t gc = static_cast<size_t>(panel) * kPw + tid;
      if (kWriteState) a.s_tilde[static_cast<size_t>(t) * f + gc] = st;
      const uint64_t bal = __ballot(fabsf(st) >= a.tau_s);
      if (lane == 0) {
        uint32_t* bitmap = reinterpret_cast<uint32_t*>(tws + a.off_bitmap);
        const size_t w0 = (gc - lane) / 32;
        bitmap[w0] = static_cast<uint32_t>(bal);
        bitmap[w0 + 1] = static_cast<uint32_t>(bal >> 32);
      }
    }
    __syncthreads();  // sv is rewritten for the next token
  }
  if (tid == 0) {
    __hip_atomic_store(&tickets[panel], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (panel == 0 && a.in_count != nullptr) {
      for (int t = 0; t < nt; ++t) {
        const int* kcount = reinterpret_cast<const int*>(a.ws + static_cast<size_t>(t) * a.tok_bytes + a.off_kcount);
        int s = 0;
        for (int k = 0; k < a.splits; ++k)
          s += __hip_atomic_load(&kcount[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        a.in_count[t] = s;
      }
    }
  }
}

}  // namespace

hipError_t launch_stage1_batch(const Stage1Args& a, int wdtype, bool write_state, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.n_panels * a.splits));
  if (wdtype == PROX_BF16) {
    if (write_state)
      hipLaunchKernelGGL((stage1_batch_kernel<Bf16Tag, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((stage1_batch_kernel<Bf16Tag, false>), grid, dim3(kThreads), 0, s, a);
  } else {
    if (write_state)
      hipLaunchKernelGGL((stage1_batch_kernel<F32Tag, true>), grid, dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((stage1_batch_kernel<F32Tag, false>), grid, dim3(kThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace prox
