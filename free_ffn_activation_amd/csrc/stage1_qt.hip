// Stage 1 of the Prox decode step for a group of 1..8 tokens on gfx950, from
// the channel-major copy of the INT4 proxy (prox_layer.proxy_qt).
//
// Method ([blog] = deep-dive blog "Prox 完全拆解", section "Stage 1"), per
// token b of the group:
//   m_x,b = 1[|x_b,i| >= tau_x];  u~_b = Pi^in(x_b, W~_up, m_x,b);
//   s~_b = u~_b * act(Pi^in(x_b, W~_gate, m_x,b));  m_s,b = 1[|s~_b,j| >= tau_s]
// The pages study batch 1 and leave larger batches open ([blog] limitations
// section).  Between them, the tokens of a group keep nearly every input row
// (eight tokens that each keep half of the rows leave under 1% unkept), so
// this kernel reads every proxy row once and gives a token a zero weight on
// each row it rejects: every token still sees exactly its own input mask.
//
// gfx950 design:
//   * proxy_qt holds, per 16-channel group and 128-row chunk of the inputs,
//     the up codes and then the gate codes as two 1 KB images of the MFMA B
//     operand (lane l: channel l % 16, rows 32 (l / 16) .. + 31), so a wave
//     streams its channels in contiguous 1 KB loads whose addresses do not
//     depend on x: the weight stream starts with the kernel.  The images are
//     stored chunk-major (chunk k of every group, then chunk k + 1), so the
//     blocks, which advance through their chunks together, read one
//     contiguous span at a time.
//   * one 1024-thread block per CU owns a range of 16-channel groups over the
//     whole input range: no K-split partials, no hand-off between blocks.  A
//     group's input range is cut into `parts` ranges, one streaming wave per
//     (group, part) unit (two units when a block holds more than 14), and the
//     parts are added in LDS in a fixed order.
//   * x of the group's tokens (rejected rows set to 0) and all proxy scales
//     are staged in LDS once, at the start.  Each chunk's A operand, rows
//     (token, hi/lo) of a = x_i scale_i after a per-token power-of-two
//     scaling that bounds |a| by 2^15 (from the token's largest |x| and the
//     largest proxy scale), split into two f16 parts (~22 significant bits;
//     products with the small integer codes are exact, sums in fp32), is
//     built from there into a double-buffered LDS image by all 1024 threads,
//     one 16-byte entry (8 rows of one token, projection and part) each.  A
//     token's staged row is rotated by 16 elements per token and the image's
//     entries are xor-swizzled, so the builders' LDS reads and writes spread
//     over the banks.  One block barrier per chunk hands a built image to
//     the streaming waves.  Groups whose x and scales do not fit the LDS run
//     the union-of-rows Stage 1 (qt_fits).
//   * codes, x and scales are read with buffer loads: an out-of-range offset
//     returns zero without a memory request, so tails and absent tokens need
//     no branches and every load is issued in a fixed order.
#include <atomic>

#include "prox_device.h"
#include "prox_internal.h"
#include "stage1_mfma.h"

namespace prox {
namespace {

constexpr int kQtWaves = 16;
constexpr int kQtThreads = 64 * kQtWaves;
constexpr int kQtMaxParts = 4;
constexpr int kQtChunkBytes = 2048;          // up then gate image of one (group, chunk)
constexpr uint32_t kOob = 0x80000000u;       // past every buffer's records: the load returns 0
constexpr int kRsrcWord3 = 0x00020000;       // raw buffer, 32-bit data (gfx9 family)

// Dynamic LDS (bytes):
//   [0, 2 P 8192)    the A image: buffer b, part p at (b P + p) 8192; in it the
//                    fragment of k-step s, up/gate pr at (2 s + pr) 1024, whose
//                    16-byte slot (16 q + m) ^ (s & 1) holds A row m for lane
//                    group q (8 f16; the xor spreads the builders' writes over
//                    the banks).  The epilogue's part sums [group][part][up/
//                    gate][token][16] fp32 reuse it (<= 16 groups x P x 1 KB).
//                    Buffer 1's first 192 bytes hold the pre-pass statistics
//                    (per wave: largest |x| of its token's half, kept inputs of
//                    it, largest proxy scale), read before buffer 1 is first built.
//   then x           [nt][d] in the layer dtype, rows the token rejects set to
//                    0, token t's row rotated by 16 t elements (element r at
//                    (r + 16 t) mod d, so the eight tokens' reads of one row
//                    octet fall in different banks)
//   then the scales  [2][d] fp32
size_t qt_smem_bytes(int parts, int nt, int d, int es) {
  return static_cast<size_t>(2) * parts * 8192 + (static_cast<size_t>(nt) * d * es + 15) / 16 * 16 +
         static_cast<size_t>(8) * d;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0), static_cast<int>(bytes),
                                           kRsrcWord3);
}
__device__ __forceinline__ u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
// the code stream: cache-policy operand 2 is the non-temporal hint (each code
// chunk is read once per launch; x and the scales, which every block reads,
// keep the default policy)
__device__ __forceinline__ u32x4_t bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left free): the streaming waves end
// their branch with it, so the second branch starts with no code load in
// flight as the compiler sees it (the last ones read past the end of the
// buffer and cost nothing).
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// the 8 values of a 16-byte (bf16) or 32-byte (fp32) vector of x
template <typename T>
__device__ __forceinline__ void unpack8(const u32x4_t* v, float* out);
template <>
__device__ __forceinline__ void unpack8<Bf16Tag>(const u32x4_t* v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = bf16lo(v[0][i]);
    out[2 * i + 1] = bf16hi(v[0][i]);
  }
}
template <>
__device__ __forceinline__ void unpack8<F32Tag>(const u32x4_t* v, float* out) {
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = __uint_as_float(v[i / 4][i % 4]);
}

// the same vector with the elements a token rejects (|x| < tau_x) set to 0
template <typename T>
__device__ __forceinline__ void mask8(u32x4_t* v, float tau_x);
template <>
__device__ __forceinline__ void mask8<Bf16Tag>(u32x4_t* v, float tau_x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[0][i];
    const uint32_t lo = fabsf(bf16lo(w)) >= tau_x ? 0x0000FFFFu : 0u;
    const uint32_t hi = fabsf(bf16hi(w)) >= tau_x ? 0xFFFF0000u : 0u;
    v[0][i] = w & (lo | hi);
  }
}
template <>
__device__ __forceinline__ void mask8<F32Tag>(u32x4_t* v, float tau_x) {
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i / 4][i % 4] = fabsf(__uint_as_float(v[i / 4][i % 4])) >= tau_x ? v[i / 4][i % 4] : 0u;
}

// two f32 values as the f16 pair (hi) and the pair of their remainders (lo).
// hi + lo carries ~22 significant bits of a only if the stored hi is the hi
// that lo was taken from: hi comes from v_cvt_pkrtz_f16_f32 (round toward
// zero), an intrinsic the compiler does not fuse with the multiply that
// produced a (a plain f16 conversion it turns into v_fma_mixlo_f16, which
// rounds the exact product, and may then use that for lo but the fp32-rounded
// product for the stored hi: one f16 ulp apart at near-ties).
__device__ __forceinline__ void split_pair(float a0, float a1, uint32_t& hi, uint32_t& lo) {
  const f16x2_t h = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(a0, a1));
  const _Float16 l0 = static_cast<_Float16>(a0 - static_cast<float>(h[0]));
  const _Float16 l1 = static_cast<_Float16>(a1 - static_cast<float>(h[1]));
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, f16x2_t{l0, l1});
}

template <typename T, bool kWriteState, int kUpw>
__global__ __launch_bounds__(kQtThreads) void stage1_qt_kernel(QtArgs a) {
  extern __shared__ __align__(16) u32x4_t qt_smem[];
  constexpr int kEs = static_cast<int>(sizeof(typename T::storage));
  constexpr int kXl = kEs == 2 ? 1 : 2;  // 16-byte vectors per 8 values of x
  constexpr int kD = 4 / kUpw;           // chunks of codes in flight per unit
  // pre-pass: x and scale vectors per thread and round (one round up to
  // d = 5120 for bf16 layers with one unit per streaming wave)
  constexpr int kXv = kXl == 2 ? 2 : (kUpw == 1 ? 5 : 4);
  constexpr int kSv = kXl == 2 ? 1 : (kUpw == 1 ? 3 : 2);
  static_assert(kD % 2 == 0, "the chunk loop's unroll keeps the A buffer index static");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform as the compiler sees it, so the split into streaming and
  // other waves is a scalar branch
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int d = a.d;
  const int nt = a.nt;
  const int P = a.parts;
  const int ncp = a.ncp;
  const int nck = a.nck;
  const int ncp_pad = (ncp + kD - 1) / kD * kD;  // chunk rounds of every wave
  const int g0 = static_cast<int>(static_cast<int64_t>(blockIdx.x) * a.ng / a.nb);
  const int gb = static_cast<int>(static_cast<int64_t>(blockIdx.x + 1) * a.ng / a.nb) - g0;
  const bool streamer = wave < a.s_waves;  // wave-uniform
  // an opaque copy of the split for the second of the two wave-kind branches
  // below, so the compiler cannot fold them back into one if/else
  int s_waves_b;
  asm volatile("s_mov_b32 %0, %1" : "=s"(s_waves_b) : "s"(a.s_waves));

  // LDS views (layout above)
  u32x4_t* const aimg = qt_smem;
  float* const st_wmax = reinterpret_cast<float*>(aimg + P * 512);
  int* const st_wcnt = reinterpret_cast<int*>(st_wmax + kQtWaves);
  float* const st_smax = st_wmax + 2 * kQtWaves;
  uint8_t* const xs = reinterpret_cast<uint8_t*>(aimg + 2 * P * 512);
  float* const ss = reinterpret_cast<float*>(xs + (nt * d * kEs + 15) / 16 * 16);

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, static_cast<uint32_t>(nt * d * kEs));
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.proxy_scale, static_cast<uint32_t>(2 * d * 4));
  const __amdgpu_buffer_rsrc_t qr =
      make_rsrc(a.proxy_qt, static_cast<uint32_t>(static_cast<size_t>(a.ng) * nck * kQtChunkBytes));

  // ---- pre-pass, issued before any weight load: x of token wave / 2 (waves
  // 2t and 2t + 1 split it) and every proxy scale, into LDS (x masked and
  // rotated) with the statistics of the token scales and k_x
  const int xt = wave >> 1;
  const int nvec = d / 8;  // 8-element vectors per token
  const int nsv = d / 2;   // 16-byte vectors of the 2d scales
  const int rounds = max((nvec + 128 * kXv - 1) / (128 * kXv), (nsv + kQtThreads * kSv - 1) / (kQtThreads * kSv));
  u32x4_t xv[kXv][kXl], sv[kSv];
  float lxmax = 0.f, lsmax = 0.f;
  int lcnt = 0;
  auto issue_pre = [&](int r) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kXv; ++j) {
      const int v = r * 128 * kXv + 128 * j + (wave & 1) * 64 + lane;
      const uint32_t off = (xt < nt && v < nvec) ? static_cast<uint32_t>((xt * d + 8 * v) * kEs) : kOob;
#pragma unroll
      for (int l = 0; l < kXl; ++l) xv[j][l] = bload16(xr, off + 16 * l);
    }
#pragma unroll
    for (int j = 0; j < kSv; ++j) {
      const int v = r * kQtThreads * kSv + kQtThreads * j + tid;
      sv[j] = bload16(sr, v < nsv ? static_cast<uint32_t>(16 * v) : kOob);
    }
  };
  auto use_pre = [&](int r) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kXv; ++j) {
      const int v = r * 128 * kXv + 128 * j + (wave & 1) * 64 + lane;
      const bool ok = xt < nt && v < nvec;
      float e[8];
      unpack8<T>(xv[j], e);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        lxmax = fmaxf(lxmax, fabsf(e[i]));  // out-of-range vectors read 0
        lcnt += (ok && fabsf(e[i]) >= a.tau_x) ? 1 : 0;
      }
      if (ok) {
        mask8<T>(xv[j], a.tau_x);
        const int pos = (8 * v + 16 * xt) % d;  // rotated row
#pragma unroll
        for (int l = 0; l < kXl; ++l)
          *reinterpret_cast<u32x4_t*>(xs + (xt * d + pos) * kEs + 16 * l) = xv[j][l];
      }
    }
#pragma unroll
    for (int j = 0; j < kSv; ++j) {
      const int v = r * kQtThreads * kSv + kQtThreads * j + tid;
      if (v < nsv) reinterpret_cast<u32x4_t*>(ss)[v] = sv[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) lsmax = fmaxf(lsmax, fabsf(__uint_as_float(sv[j][i])));
    }
  };
  auto finish_pre = [&]() __attribute__((always_inline)) {
    use_pre(0);
    for (int r = 1; r < rounds; ++r) {  // larger d only
      issue_pre(r);
      use_pre(r);
    }
    const float wx = wave_max_nonneg(lxmax);
    const int wc = wave_sum_int(lcnt);
    const float ws = wave_max_nonneg(lsmax);
    if (lane == 0) {
      st_wmax[wave] = wx;
      st_wcnt[wave] = wc;
      st_smax[wave] = ws;
    }
  };
  // per-token scale 2^(15 - e): |x_i scale_i| < 2^e for every row of the token
  auto token_exp = [&](int t) __attribute__((always_inline)) {
    float smax = 0.f;
#pragma unroll
    for (int w = 0; w < kQtWaves; ++w) smax = fmaxf(smax, st_smax[w]);
    return scale_exponent(fmaxf(st_wmax[2 * t], st_wmax[2 * t + 1]) * smax);
  };

  // ---- A-image entry of this thread, built by every wave: token bt, rows
  // 8 bs .. 8 bs + 7 of lane group bq's 32-row band, projection bp, part bpt
  const int bt = tid & 7;
  const int bs = (tid >> 3) & 3;
  const int bp = (tid >> 5) & 1;
  const int bq = (tid >> 6) & 3;
  const int bpt = tid >> 8;
  const bool bval = bpt < P;
  const int brot = (16 * bt) % d;                // rotation of token bt's staged row
  const int bxrow = (bt < nt ? bt : 0) * d;      // its staged row (token 0's for absent tokens)
  float bsc = 0.f;  // 2^(15 - e) of token bt
  auto build_chunk = [&](int buf, int c) __attribute__((always_inline)) {
    if (!bval) return;
    // rows past d, padding chunks and absent tokens read a valid staged row
    // and scale the entry by 0 (staged x is finite or a kept infinity,
    // which makes every channel infinite or NaN in any case)
    const int r0 = (bpt * ncp + c) * 128 + 32 * bq + 8 * bs;
    const bool ok = bt < nt && c < ncp && r0 < d;
    const int rr = ok ? r0 : 0;
    int pos = rr + brot;
    pos = pos >= d ? pos - d : pos;
    u32x4_t xw[kXl];
#pragma unroll
    for (int l = 0; l < kXl; ++l) xw[l] = *reinterpret_cast<const u32x4_t*>(xs + (bxrow + pos) * kEs + 16 * l);
    const u32x4_t* sp = reinterpret_cast<const u32x4_t*>(ss + bp * d + rr);
    const u32x4_t s0 = sp[0];
    const u32x4_t s1 = sp[1];
    const float f_lo = ok ? bsc : 0.f;
    const float f_hi = ok ? bsc * 0.0625f : 0.f;
    float xe[8];
    unpack8<T>(xw, xe);
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      // elements 2, 3, 6, 7 meet the high nibbles, read as 16 x code
      const float f = (i & 2) ? f_hi : f_lo;
      const float sa = __uint_as_float((i < 4 ? s0 : s1)[i % 4]);
      const float sb = __uint_as_float((i < 4 ? s0 : s1)[i % 4 + 1]);
      split_pair(xe[i] * f * sa, xe[i + 1] * f * sb, hi[i / 2], lo[i / 2]);
    }
    u32x4_t* frag = aimg + (buf * P + bpt) * 512 + (2 * bs + bp) * 64;
    const int sw = bs & 1;
    frag[(16 * bq + 2 * bt) ^ sw] = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
    frag[(16 * bq + 2 * bt + 1) ^ sw] = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
  };

  issue_pre(0);
  __builtin_amdgcn_sched_barrier(0);

  float* red = reinterpret_cast<float*>(aimg);  // [group][part][up/gate][token][16]
  // Two sequential branches, not if/else: the compiler's tracking of loads
  // in flight then starts the streaming waves from the loads issued above
  // (an if/else joins the sides, and its second side would wait for loads
  // only the first kind of wave issued); barriers pair up across them.
  if (streamer) {
    // ---- streaming waves: unit k = (group gl, part p) of this block
    int upart[kUpw], ugl[kUpw];
    uint32_t ubase[kUpw];
    bool uval[kUpw];
#pragma unroll
    for (int k = 0; k < kUpw; ++k) {
      const int u = wave * kUpw + k;
      uval[k] = u < gb * P;
      ugl[k] = uval[k] ? u / P : 0;
      upart[k] = uval[k] ? u - ugl[k] * P : 0;
      ubase[k] = static_cast<uint32_t>((upart[k] * ncp * a.ng + g0 + ugl[k]) * kQtChunkBytes + 16 * lane);
    }
    const uint32_t cstride = static_cast<uint32_t>(a.ng * kQtChunkBytes);  // chunk k to k + 1
    auto code_off = [&](int k, int c, int pr) __attribute__((always_inline)) -> uint32_t {
      return (uval[k] && c < ncp && upart[k] * ncp + c < nck)
                 ? ubase[k] + static_cast<uint32_t>(c) * cstride + static_cast<uint32_t>(pr * 1024)
                 : kOob;
    };
    // the first half of the chunks in flight go out before the pre-pass
    // completes, the rest after it: with all of them ahead, the pre-pass's
    // x and scale misses queue behind the whole burst of code misses (the
    // kernel measured ~15% slower on the 8B and 32B layers at 8 tokens)
    u32x4_t cw[kD][kUpw][2];
#pragma unroll
    for (int c = 0; c < kD / 2; ++c)
#pragma unroll
      for (int k = 0; k < kUpw; ++k)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) cw[c][k][pr] = bload16_nt(qr, code_off(k, c, pr));
    __builtin_amdgcn_sched_barrier(0);
    finish_pre();
    __syncthreads();  // staged x, scales and statistics in LDS
#pragma unroll
    for (int c = kD / 2; c < kD; ++c)
#pragma unroll
      for (int k = 0; k < kUpw; ++k)
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) cw[c][k][pr] = bload16_nt(qr, code_off(k, c, pr));
    const int q = lane >> 4;
    const float un0 = ldexpf(1.0f, token_exp(2 * q) - 15);
    const float un1 = ldexpf(1.0f, token_exp(2 * q + 1) - 15);
    bsc = ldexpf(1.0f, 15 - token_exp(bt));
    build_chunk(0, 0);
    f32x4_t C[kUpw][2];
#pragma unroll
    for (int k = 0; k < kUpw; ++k) C[k][0] = C[k][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    __syncthreads();  // A image of chunk 0 built
    // the loop runs a whole number of unrolled rounds (padding chunks read
    // zeros): an exit from inside a round would reach the loop head with fewer
    // loads in flight, and the compiler would then drain them every round
    for (int c0 = 0; c0 < ncp_pad; c0 += kD) {
#pragma unroll
      for (int kk = 0; kk < kD; ++kk) {
        const int c = c0 + kk;
        // this wave's share of the next image first, so that its temporaries
        // are dead before the matrix-core operands of this chunk are read
        build_chunk((kk + 1) & 1, c + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < kUpw; ++k) {
          const u32x4_t* af = aimg + ((kk & 1) * P + upart[k]) * 512 + lane;
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const u32x4_t w = cw[kk][k][pr];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const f16x8_t av = __builtin_bit_cast(f16x8_t, af[(2 * s + pr) * 64 + ((lane ^ (s & 1)) - lane)]);
              C[k][pr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, codes_to_f16(w[s]), C[k][pr], 0, 0, 0);
            }
            cw[kk][k][pr] = bload16_nt(qr, code_off(k, c + kD, pr));
          }
        }
        __syncthreads();  // this image read, the next one built
      }
    }
    // ---- unscaled part sums: lane (q, n) holds tokens 2q (hi, lo) and
    // 2q + 1 (hi, lo) of channel n
    const int n = lane & 15;
#pragma unroll
    for (int k = 0; k < kUpw; ++k) {
      if (!uval[k]) continue;
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        float* rp = red + ((ugl[k] * P + upart[k]) * 2 + pr) * (kBatchMax * 16);
        rp[(2 * q) * 16 + n] = (C[k][pr][0] + C[k][pr][1]) * un0;
        rp[(2 * q + 1) * 16 + n] = (C[k][pr][2] + C[k][pr][3]) * un1;
      }
    }
    wait_all_loads();
  }
  if (wave >= s_waves_b) {
    // ---- the other waves: they only build A-image entries
    finish_pre();
    __syncthreads();  // staged x, scales and statistics in LDS
    bsc = ldexpf(1.0f, 15 - token_exp(bt));
    if (blockIdx.x == 0 && tid - 64 * a.s_waves < nt && a.in_count != nullptr) {
      const int t = tid - 64 * a.s_waves;
      a.in_count[t] = st_wcnt[2 * t] + st_wcnt[2 * t + 1];
    }
    build_chunk(0, 0);
    __syncthreads();  // A image of chunk 0 built
    // same rounds as the streaming waves; chunks from ncp on build zeros (the
    // last one into the buffer the last round does not read)
    for (int c0 = 0; c0 < ncp_pad; c0 += 2) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        build_chunk((kk + 1) & 1, c0 + kk + 1);
        __syncthreads();  // this image read, the next one built
      }
    }
  }
  __syncthreads();  // part sums in LDS

  // ---- fixed-order sum of the parts, activation, mask bits: a wave holds
  // four (token, group) pairs of 16 channels; lane 16i writes pair i's bits
  const int gmax = (a.ng + a.nb - 1) / a.nb;
  const int items = kBatchMax * gmax * 16;
  for (int it0 = 0; it0 < items; it0 += kQtThreads) {  // block-uniform
    const int it = it0 + tid;
    const int t = it / (gmax * 16);
    const int gl = (it >> 4) % gmax;
    const int n = it & 15;
    const bool ok = it < items && t < nt && gl < gb;
    bool kept = false;
    if (ok) {
      float u = 0.f, g = 0.f;
      for (int p = 0; p < P; ++p) {
        u += red[((gl * P + p) * 2 + 0) * (kBatchMax * 16) + t * 16 + n];
        g += red[((gl * P + p) * 2 + 1) * (kBatchMax * 16) + t * 16 + n];
      }
      const float st = u * gate_act(g, a.act);
      kept = fabsf(st) >= a.tau_s;
      if (kWriteState) a.s_tilde[static_cast<size_t>(t) * a.f + 16 * (g0 + gl) + n] = st;
    }
    const uint64_t bal = __ballot(kept);
    if (ok && n == 0) {
      uint16_t* bm = reinterpret_cast<uint16_t*>(a.ws + static_cast<size_t>(t) * a.tok_bytes + a.off_bitmap);
      bm[g0 + gl] = static_cast<uint16_t>(bal >> (lane & 48));
    }
  }
}

// proxy_q (row-major, 16-column groups of 8 up then 8 gate bytes, low nibble
// first) -> proxy_qt: one thread per dword of 8 codes.  Images are stored
// chunk-major, (chunk k, group g) at (k * ng + g) * 2048.  Dword s of lane l
// of the (chunk k, group g, up/gate pr) image holds channel 16 g + l % 16,
// rows 128 k + 32 (l / 16) + 8 s + e, e = 0..7, element e in nibble
// {0, 4, 1, 5, 2, 6, 3, 7}[e] (the order codes_to_f16 returns); rows past d
// hold code 0 (nibble 8).
__global__ void pack_qt_kernel(const uint8_t* __restrict__ q, int qstride, int d, int ng, size_t total,
                               uint32_t* __restrict__ qt) {
  const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int s = static_cast<int>(i & 3);
  const int l = static_cast<int>((i >> 2) & 63);
  const int pr = static_cast<int>((i >> 8) & 1);
  const size_t rest = i >> 9;
  const size_t g = rest % static_cast<size_t>(ng);
  const int k = static_cast<int>(rest / static_cast<size_t>(ng));
  const int n = l & 15;
  const size_t col = 16 * g + 8 * pr + (n >> 1);
  const int shift = (n & 1) * 4;
  const int rbase = 128 * k + 32 * (l >> 4) + 8 * s;
  constexpr int kPos[8] = {0, 4, 1, 5, 2, 6, 3, 7};
  uint32_t w = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int r = rbase + e;
    const uint32_t nib = r < d ? (q[static_cast<size_t>(r) * qstride + col] >> shift) & 15u : 8u;
    w |= nib << (4 * kPos[e]);
  }
  qt[i] = w;
}

}  // namespace

QtArgs qt_plan(int d, int f, int blocks) {
  QtArgs a{};
  a.d = d;
  a.f = f;
  a.nck = (d + 127) / 128;
  a.ng = f / 16;
  a.nb = std::max(1, std::min(a.ng, blocks));
  const int gmax = (a.ng + a.nb - 1) / a.nb;
  // parts per group: 8 to 14 (group, part) units per block, one streaming
  // wave each (two units per wave from 15 on), so that most waves keep codes
  // in flight and at least one wave of 16 only builds operands
  int parts = gmax <= 3 ? 4 : (gmax <= 7 ? 2 : 1);
  parts = std::min(parts, a.nck);
  a.parts = parts;
  a.ncp = (a.nck + parts - 1) / parts;
  const int units = gmax * parts;
  a.upw = units <= 14 ? 1 : 2;
  a.s_waves = (units + a.upw - 1) / a.upw;
  return a;
}

size_t proxy_qt_bytes(int d, int f) {
  return static_cast<size_t>(f / 16) * static_cast<size_t>((d + 127) / 128) * kQtChunkBytes;
}

namespace {

constexpr int kMaxDevices = 64;  // per-device state below (device ids past it share slot 0)

int current_device() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices ? dev : 0;
}

template <typename T, bool kW, int kU>
hipError_t qt_go(const QtArgs& a, size_t smem, hipStream_t s) {
  // dynamic LDS past 64 KB must be allowed once per kernel and device
  static std::atomic<size_t> allowed[kMaxDevices];
  const int dev = current_device();
  if (smem > 65536 && allowed[dev].load() < smem) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(stage1_qt_kernel<T, kW, kU>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
    if (e != hipSuccess) return e;
    allowed[dev].store(smem);
  }
  hipLaunchKernelGGL((stage1_qt_kernel<T, kW, kU>), dim3(static_cast<unsigned>(a.nb)), dim3(kQtThreads), smem, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t qt_go2(const QtArgs& a, bool write_state, size_t smem, hipStream_t s) {
  if (a.upw == 1) return write_state ? qt_go<T, true, 1>(a, smem, s) : qt_go<T, false, 1>(a, smem, s);
  return write_state ? qt_go<T, true, 2>(a, smem, s) : qt_go<T, false, 2>(a, smem, s);
}

// LDS bytes a block may use on the current device (queried once per device)
int device_max_lds() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 65536;
  std::atomic<int>* slot = dev < kMaxDevices ? &cached[dev] : nullptr;
  int v = slot ? slot->load() : 0;
  if (v > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0) return 65536;
  if (slot) slot->store(v);
  return v;
}

}  // namespace

bool qt_fits(const QtArgs& a, int wdtype) {
  const int gmax = (a.ng + a.nb - 1) / a.nb;
  // a wave that only builds (it also writes in_count), every unit streamed,
  // the part sums of the epilogue within the A image (gmax x P x 1 KB)
  if (a.s_waves < 1 || a.s_waves > kQtWaves - 1 || a.parts < 1 || a.parts > kQtMaxParts || a.nt < 1 ||
      a.nt > kBatchMax || (a.upw != 1 && a.upw != 2) || a.s_waves * a.upw < gmax * a.parts || gmax > 16)
    return false;
  return qt_smem_bytes(a.parts, a.nt, a.d, wdtype == PROX_BF16 ? 2 : 4) <= static_cast<size_t>(device_max_lds());
}

hipError_t launch_stage1_qt(const QtArgs& a, int wdtype, bool write_state, hipStream_t s) {
  if (!qt_fits(a, wdtype)) return hipErrorInvalidValue;
  const size_t smem = qt_smem_bytes(a.parts, a.nt, a.d, wdtype == PROX_BF16 ? 2 : 4);
  return wdtype == PROX_BF16 ? qt_go2<Bf16Tag>(a, write_state, smem, s) : qt_go2<F32Tag>(a, write_state, smem, s);
}

hipError_t launch_pack_qt(const uint8_t* proxy_q, int qstride, int d, int f, uint8_t* proxy_qt, hipStream_t s) {
  const size_t total = proxy_qt_bytes(d, f) / 4;
  const unsigned blocks = static_cast<unsigned>((total + 255) / 256);
  hipLaunchKernelGGL(pack_qt_kernel, dim3(blocks), dim3(256), 0, s, proxy_q, qstride, d, f / 16, total,
                     reinterpret_cast<uint32_t*>(proxy_qt));
  return hipGetLastError();
}

}  // namespace prox
