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
//     256-thread block per (panel of 128 output columns, range of input rows),
//     all tokens of the group in the block; each of the 4 waves owns two
//     16-column chunks of the panel (up and gate).  Three blocks fit on a CU
//     (LDS ~52 KB, at most 168 VGPRs), so the 768 blocks of a Qwen3-8B-shaped
//     layer are all resident at once: a block's chain of memory round trips
//     (x, gather, partials, ticket) is paid once, not once per round of
//     blocks.
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
#include "stage1_mfma.h"

namespace prox {
namespace {

typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2_t;

constexpr int kS1bThreads = 256;                 // 4 waves, two 16-column chunks each
constexpr int kS1bWaves = kS1bThreads / 64;
constexpr int kChunkRows = 512;                  // input rows per pass (two per thread)
constexpr int kRowGroups = kChunkRows / 64;      // 64-row groups of a pass, one wave's rows each
constexpr int kWaveChunks = (128 / 16) / kS1bWaves;  // 16-column chunks per wave
constexpr int kTileRows = 64;                    // rows per pair of MFMA K-steps
constexpr int kTiles = kChunkRows / kTileRows;   // 8
constexpr int kPhaseRows = 128;                  // rows staged in LDS at a time
constexpr int kPw = 128;                         // panel width (output columns)
constexpr int kRowsPerLoad = kS1bThreads / 8;    // 32 rows per load round (8 threads x 16 B per row)
constexpr int kLoads = kChunkRows / kRowsPerLoad;  // 16 loads of 16 B per thread per pass
constexpr int kLoadsPerPhase = kPhaseRows / kRowsPerLoad;  // 4

static_assert(kChunkRows == 2 * kS1bThreads, "the mask step gives each thread two rows of a pass");
static_assert(kLoads % 4 == 0, "a thread's gather offsets are read as 16-byte vectors");
static_assert(2 * kPw == kS1bThreads, "the last block loads one output (up or gate column) per thread");
static_assert(kBatchMax % kS1bWaves == 0, "the last block's waves form the tokens' states in turn");

// LDS: the A operands of one pass [mat][tile][half][k-group][m][8], the staged
// code rows of one phase, the pass's union-row offsets, per-wave statistics.
struct S1BShared {
  _Float16 A[2][kTiles][2][4][16][8];
  uint8_t B[kPhaseRows * kPw];
  uint32_t uoff[kChunkRows];  // union-row byte offsets, transposed (uoff_pos)
  float wmax[kRowGroups][kBatchMax];
  int wkept[kS1bWaves][kBatchMax];
  int wunion[kRowGroups];
  int sexp[kBatchMax];
  int last;
};

// Union slot p's offset lives at uoff[uoff_pos(p)]: the kLoads slots one
// thread gathers (p = kRowsPerLoad u + tid / 8) are contiguous.
__device__ __forceinline__ int uoff_pos(int p) { return (p & (kRowsPerLoad - 1)) * kLoads + p / kRowsPerLoad; }

template <typename T, bool kWriteState>
__global__ __launch_bounds__(kS1bThreads) __attribute__((amdgpu_waves_per_eu(3))) void stage1_batch_kernel(Stage1Args a) {
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

  int kept[kBatchMax];  // per-wave counts of kept rows per token (wave-uniform)
#pragma unroll
  for (int t = 0; t < kBatchMax; ++t) kept[t] = 0;
  float acc[kWaveChunks][2][2];  // unscaled sums of this block: [chunk][matrix][token 2g + i]
#pragma unroll
  for (int i = 0; i < 4 * kWaveChunks; ++i) (&acc[0][0][0])[i] = 0.f;

  const int g = lane >> 4;     // MFMA k-group
  const int mrow = lane & 15;  // A row: token mrow/2, part mrow%2
  const int chunk = tid & 7;   // 16-B chunk this thread gathers
  constexpr float kInv16 = 0.0625f;

  for (int c0 = row0; c0 < row1; c0 += kChunkRows) {
    const int c1 = min(row1, c0 + kChunkRows);
    // ---- clear the A operands: rows no token keeps, tokens past nt and
    // padding slots stay zero
    {
      u32x4_t* az = reinterpret_cast<u32x4_t*>(&sh.A[0][0][0][0][0][0]);
      constexpr int n16 = static_cast<int>(sizeof(sh.A) / 16);
      const u32x4_t z = {0u, 0u, 0u, 0u};
      for (int i = tid; i < n16; i += kS1bThreads) az[i] = z;
    }
    // ---- input masks of the pass: row group h * kS1bWaves + wave holds rows
    // c0 + 64 (h * kS1bWaves + wave) + lane, h = 0, 1
    int iv[2];
    float xv[2][kBatchMax], sc_u[2], sc_g[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      iv[h] = c0 + 64 * (h * kS1bWaves + wave) + lane;
      const int ii = min(iv[h], c1 - 1);
      sc_u[h] = a.proxy_scale[ii];
      sc_g[h] = a.proxy_scale[d + ii];
#pragma unroll
      for (int t = 0; t < kBatchMax; ++t)
        xv[h][t] = load_elem<T>(a.x, static_cast<size_t>(min(t, nt - 1)) * d + ii);
    }
    __builtin_amdgcn_sched_barrier(0);
    uint32_t keep[2];
    uint64_t bal[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      keep[h] = 0u;
      float lmax[kBatchMax];
#pragma unroll
      for (int t = 0; t < kBatchMax; ++t) {
        const bool kp = t < nt && iv[h] < c1 && fabsf(xv[h][t]) >= a.tau_x;
        keep[h] |= kp ? (1u << t) : 0u;
        lmax[t] = kp ? fmaxf(fabsf(xv[h][t] * sc_u[h]), fabsf(xv[h][t] * sc_g[h])) : 0.f;
      }
      bal[h] = __ballot(keep[h] != 0u);
#pragma unroll
      for (int t = 0; t < kBatchMax; ++t) {
        const float v = wave_max_nonneg(lmax[t]);
        if (lane == 0) sh.wmax[h * kS1bWaves + wave][t] = v;
        kept[t] += __popcll(__ballot((keep[h] >> t) & 1u));
      }
      if (lane == 0) sh.wunion[h * kS1bWaves + wave] = __popcll(bal[h]);
    }
    __syncthreads();
    int sexp[kBatchMax];
    float scale[kBatchMax];
#pragma unroll
    for (int t = 0; t < kBatchMax; ++t) {
      float m = 0.f;
#pragma unroll
      for (int w = 0; w < kRowGroups; ++w) m = fmaxf(m, sh.wmax[w][t]);
      sexp[t] = scale_exponent(m);
      scale[t] = ldexpf(1.0f, 15 - sexp[t]);
    }
    int nu = 0;
#pragma unroll
    for (int w = 0; w < kRowGroups; ++w) nu += sh.wunion[w];
    // ---- union slots (ascending rows); slots past the union read row 0
    int slot[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rg = h * kS1bWaves + wave;
      int wbase = 0;
#pragma unroll
      for (int w = 0; w < kRowGroups; ++w) wbase += w < rg ? sh.wunion[w] : 0;
      slot[h] = wbase + __popcll(bal[h] & ((1ull << lane) - 1ull));
      if (keep[h] != 0u)
        sh.uoff[uoff_pos(slot[h])] = static_cast<uint32_t>(iv[h]) * static_cast<uint32_t>(a.proxy_stride);
      const int pz = h * kS1bThreads + tid;
      if (pz >= nu) sh.uoff[uoff_pos(pz)] = 0u;
    }
    if (tid < kBatchMax) sh.sexp[tid] = sexp[tid];
    __syncthreads();

    // ---- gather the union rows' panel slices (thread -> row tid/8 + 32u,
    // 16-B chunk tid%8), issued before the A operands are written so the two
    // overlap.  All loads are issued unconditionally (slots past the union
    // re-read row 0, which the phases below never use), so each phase waits
    // only for its own loads.
    const int ntile = (nu + kTileRows - 1) / kTileRows;
    const int rows_pad = ntile * kTileRows;
    const uint8_t* pbase = a.proxy_q + static_cast<size_t>(panel) * kPw + chunk * 16;
    uint32_t offs[kLoads];
    {
      const u32x4_t* uo = reinterpret_cast<const u32x4_t*>(&sh.uoff[(tid >> 3) * kLoads]);
#pragma unroll
      for (int k = 0; k < kLoads / 4; ++k) {
        const u32x4_t o = uo[k];
        offs[4 * k] = o.x;
        offs[4 * k + 1] = o.y;
        offs[4 * k + 2] = o.z;
        offs[4 * k + 3] = o.w;
      }
    }
    u32x4_t wld[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) wld[u] = *reinterpret_cast<const u32x4_t*>(pbase + offs[u]);
    __builtin_amdgcn_sched_barrier(0);

    // ---- A operands: (token, hi/lo) rows in the slot order of the staged rows
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (keep[h] == 0u) continue;
      const int sl = slot[h];
      const int tile = sl / kTileRows;
      const int gg = (sl >> 4) & 3;
      const int hh = (sl >> 3) & 1;
      const int r = sl & 7;
      const int e = 2 * (r & 3) + (r >> 2);
      const float rs = (r & 1) ? kInv16 : 1.0f;  // odd rows pair with high nibbles
#pragma unroll
      for (int t = 0; t < kBatchMax; ++t) {
        if (!((keep[h] >> t) & 1u)) continue;
#pragma unroll
        for (int mat = 0; mat < 2; ++mat) {
          const float v = xv[h][t] * (mat == 0 ? sc_u[h] : sc_g[h]) * scale[t] * rs;
          const _Float16 hi = static_cast<_Float16>(v);
          const _Float16 lo = static_cast<_Float16>(v - static_cast<float>(hi));
          sh.A[mat][tile][hh][gg][2 * t][e] = hi;
          sh.A[mat][tile][hh][gg][2 * t + 1][e] = lo;
        }
      }
    }
    __syncthreads();

    f32x4_t C[kWaveChunks][2];
#pragma unroll
    for (int j = 0; j < kWaveChunks; ++j) C[j][0] = C[j][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < kChunkRows / kPhaseRows; ++q) {
      if (q * kPhaseRows >= rows_pad) break;  // block-uniform
      // stage 128 rows: row r, chunk c at 16 * (c ^ (r & 7)), halves swapped
      // when bit 3 of r is set (conflict-free transposed reads)
#pragma unroll
      for (int uu = 0; uu < kLoadsPerPhase; ++uu) {
        const int r = uu * kRowsPerLoad + (tid >> 3);
        u32x4_t v = wld[q * kLoadsPerPhase + uu];
        if ((r >> 3) & 1) v = u32x4_t{v.z, v.w, v.x, v.y};
        *reinterpret_cast<u32x4_t*>(&sh.B[r * kPw + 16 * (chunk ^ (r & 7))]) = v;
      }
      __syncthreads();
#pragma unroll
      for (int tl = 0; tl < kPhaseRows / kTileRows; ++tl) {
        if (q * kPhaseRows + tl * kTileRows >= rows_pad) break;  // block-uniform
        const int tile = q * (kPhaseRows / kTileRows) + tl;
        const int r = tl * kTileRows + 16 * g + (lane & 15);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const f16x8_t a0 = *reinterpret_cast<const f16x8_t*>(&sh.A[hf][tile][0][g][mrow][0]);
          const f16x8_t a1 = *reinterpret_cast<const f16x8_t*>(&sh.A[hf][tile][1][g][mrow][0]);
#pragma unroll
          for (int j = 0; j < kWaveChunks; ++j) {
            const int cw = wave + kS1bWaves * j;
            const int off = r * kPw + 16 * (cw ^ (r & 7)) + 8 * (hf ^ ((r >> 3) & 1));
            const i32x2_t v = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
                (__attribute__((address_space(3))) i32x2_t*)((__attribute__((address_space(3))) uint8_t*)(sh.B) + off));
            C[j][hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, codes_to_f16(static_cast<uint32_t>(v[0])), C[j][hf], 0, 0, 0);
            C[j][hf] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, codes_to_f16(static_cast<uint32_t>(v[1])), C[j][hf], 0, 0, 0);
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
    for (int j = 0; j < kWaveChunks; ++j)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        acc[j][hf][0] += ldexpf(C[j][hf][0] + C[j][hf][1], e0 - 15);
        acc[j][hf][1] += ldexpf(C[j][hf][2] + C[j][hf][3], e1 - 15);
      }
    __syncthreads();  // sexp, wmax and A are rewritten by the next pass
  }

  // ---- block totals of the kept counts per token
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < kBatchMax; ++t) sh.wkept[wave][t] = kept[t];
  }
  __syncthreads();

  // ---- partials: lane (g, n) holds tokens 2g, 2g+1 of column n of each of
  // the wave's chunks
  const int n = lane & 15;
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = 2 * g + tt;
    if (t >= nt) continue;
    float* partial = reinterpret_cast<float*>(a.ws + static_cast<size_t>(t) * a.tok_bytes + a.off_partial);
#pragma unroll
    for (int j = 0; j < kWaveChunks; ++j) {
      const int col = panel * kPw + (wave + kS1bWaves * j) * 16 + n;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        __hip_atomic_store(&partial[(static_cast<size_t>(split) * 2 + hf) * f + col], acc[j][hf][tt],
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (panel == 0 && tid < nt) {
    int* kcount = reinterpret_cast<int*>(a.ws + static_cast<size_t>(tid) * a.tok_bytes + a.off_kcount);
    int kc = 0;
#pragma unroll
    for (int w = 0; w < kS1bWaves; ++w) kc += sh.wkept[w][tid];
    __hip_atomic_store(&kcount[split], kc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

  // thread o loads output o (up, then gate, of the panel's columns) of every
  // token for 8 splits at a time (fixed split order in the sums); then wave w
  // forms the state and mask bits of tokens w and w + 4
  static_assert(sizeof(float) * kBatchMax * 2 * kPw <= sizeof(S1BShared::B), "split sums fit the staging buffer");
  float* sv = reinterpret_cast<float*>(sh.B);  // [token][2 * kPw]
  const int o = tid;
  const int mm = o / kPw;  // 0 = up, 1 = gate
  const size_t ocol = static_cast<size_t>(panel) * kPw + (o % kPw);
  // k_x: wave 0 of panel 0's last block (lane t: token t) reads the first 8
  // split counts (stored before the ticket like the partials) right after its
  // first partial loads, so both travel in one round trip
  const bool count_kx = panel == 0 && a.in_count != nullptr && wave == 0;  // wave-uniform
  const int* kcount = reinterpret_cast<const int*>(a.ws + static_cast<size_t>(min(lane, nt - 1)) * a.tok_bytes +
                                                   a.off_kcount);
  int kv0[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) kv0[u] = 0;
  float tot[kBatchMax];
#pragma unroll
  for (int t = 0; t < kBatchMax; ++t) tot[t] = 0.f;
  for (int k0 = 0; k0 < a.splits; k0 += 8) {
    float pv[kBatchMax][8];
#pragma unroll
    for (int t = 0; t < kBatchMax; ++t) {
      const float* partial = reinterpret_cast<const float*>(
          a.ws + static_cast<size_t>(min(t, nt - 1)) * a.tok_bytes + a.off_partial);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int kk = min(k0 + u, a.splits - 1);
        pv[t][u] = __hip_atomic_load(&partial[(static_cast<size_t>(kk) * 2 + mm) * f + ocol], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (k0 == 0 && count_kx) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        kv0[u] = __hip_atomic_load(&kcount[min(u, a.splits - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int t = 0; t < kBatchMax; ++t)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u < a.splits) tot[t] += pv[t][u];
  }
#pragma unroll
  for (int t = 0; t < kBatchMax; ++t)
    if (t < nt) sv[t * 2 * kPw + o] = tot[t];
  __syncthreads();
#pragma unroll
  for (int tw = 0; tw < kBatchMax / kS1bWaves; ++tw) {
    const int t = wave + kS1bWaves * tw;
    if (t >= nt) continue;  // wave-uniform
    uint32_t* bitmap = reinterpret_cast<uint32_t*>(a.ws + static_cast<size_t>(t) * a.tok_bytes + a.off_bitmap);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int c = hh * 64 + lane;
      const float st = sv[t * 2 * kPw + c] * gate_act(sv[t * 2 * kPw + kPw + c], a.act);
      const size_t gc = static_cast<size_t>(panel) * kPw + c;
      if (kWriteState) a.s_tilde[static_cast<size_t>(t) * f + gc] = st;
      const uint64_t bal = __ballot(fabsf(st) >= a.tau_s);
      if (lane == 0) {
        const size_t w0 = (gc - lane) / 32;
        bitmap[w0] = static_cast<uint32_t>(bal);
        bitmap[w0 + 1] = static_cast<uint32_t>(bal >> 32);
      }
    }
  }
  if (tid == 0) __hip_atomic_store(&tickets[panel], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (count_kx && lane < nt) {
    int kx_sum = 0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < a.splits) kx_sum += kv0[u];
    for (int k0 = 8; k0 < a.splits; k0 += 8) {  // more than 8 splits (narrow layers)
      int kv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        kv[u] = __hip_atomic_load(&kcount[min(k0 + u, a.splits - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u < a.splits) kx_sum += kv[u];
    }
    a.in_count[lane] = kx_sum;
  }
}

}  // namespace

hipError_t launch_stage1_batch(const Stage1Args& a, int wdtype, bool write_state, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.n_panels * a.splits));
  const dim3 block(kS1bThreads);
  if (wdtype == PROX_BF16) {
    if (write_state)
      hipLaunchKernelGGL((stage1_batch_kernel<Bf16Tag, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((stage1_batch_kernel<Bf16Tag, false>), grid, block, 0, s, a);
  } else {
    if (write_state)
      hipLaunchKernelGGL((stage1_batch_kernel<F32Tag, true>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((stage1_batch_kernel<F32Tag, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace prox
