// Stage 2 of the Prox decode step for a group of 2..8 tokens on gfx950 (bf16
// weights): exact up/gate projections of the union of the tokens' kept
// channels, and the down projection, on the matrix cores.
//
// Method ([blog] = deep-dive blog "Prox 完全拆解", section "Stage 2"), per
// token b: s_b,j = u_b,j * act(g_b,j) for j in the token's channel list J_b
// (dense x_b, original weights), y_b = sum_{j in J_b} s_b,j W_down[j, :].
// A group reads each channel of the union of the J_b once; s_b,j is set to 0
// for a token that does not keep j, so each y_b sums exactly its own J_b.
//
// gfx950 design:
//   * upgate_batch_kernel: every block turns the tokens' Stage-1 bitmaps into
//     the union channel list and the per-token index lists (block scans of
//     the popcounts) for its slice of 16 union ordinals; the slice is filled
//     by whole waves, 32 lanes on the bits of one word at a time (a single
//     lane walking a word's bits and tokens took longer than the weight
//     stream).  Two waves per 8 channels split d in halves.
//     v_mfma_f32_16x16x32_bf16: A rows are the tokens' x (rows 8..15 zero),
//     B columns are the up rows (0..7) and the gate rows (8..15) of the 8
//     channels, read from K-tiles of W^T staged in LDS (the contraction runs
//     along a row, so each lane's 8 k-values are 16 contiguous bytes).  A DPP
//     rotate by 8 lanes brings g next to u.
//   * down_batch_kernel: a block owns a 512-column slice and a group of union
//     ordinals; 32-row tiles of W_down (1 KB per row) are staged in LDS and
//     ds_read_b64_tr_b16 turns them into B operands (8 rows of one column per
//     lane).  A rows are (token, part): s split into a bf16 high and low part
//     (~16 significant bits; products exact, fp32 accumulation), stored per
//     union ordinal by the up/gate kernel and loaded as rows.  Each block
//     writes its partial y; down_reduce_kernel adds the groups in fixed order,
//     so y is reproducible bit for bit.
#include "prox_device.h"
#include "prox_internal.h"

namespace prox {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kUgbChannels = 16;    // union channels per up/gate block (32 staged rows)
constexpr int kUgbKt = 512;         // K elements per staged tile (1 KB per row)
constexpr int kUgbRowBytes = kUgbKt * 2 + 16;  // staged row stride
constexpr int kUgbRowsPerThread = 2 * kUgbChannels / 4;  // 32 rows over 4 waves
constexpr int kDnbThreads = 512;    // down: 8 waves x 64 columns
constexpr int kDnbCols = 512;       // down: columns per block
constexpr int kDnbTileRows = 32;    // down: rows per K-tile
constexpr int kDnbPrefetch = 2;     // down: tiles in flight per thread
constexpr int kDnbMaxGroups = 64;   // down: groups of union ordinals (a plan bound)
// Every MFMA starts from zero and its result is added to the fp32 accumulator
// with a VALU add: the matrix core aligns the products (and the accumulator
// operand) to the largest term, so feeding it a large running sum would cost
// the small products bits.
constexpr f32x4_t kZero4 = {0.f, 0.f, 0.f, 0.f};

// bf16 round-to-nearest-even of a finite fp32 value
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// ---------------------------------------------------------------------------
// up/gate
// ---------------------------------------------------------------------------
// The union of a group's channel masks, as every up/gate block needs it: the
// union ordinals [u0, u0 + kSlice) of this block go to s_ch (channel) and s_tb
// (bit t set when token t keeps the channel) and to ulist; each token's index
// list receives the entries of those channels; block 0 publishes U (at
// ulist[f]) and every token's k_s.  Returns U.  Every thread reads
// kUnionWords consecutive words of each token's bitmap per round (one round
// up to d_ff = 32768 for 256 threads, so one round trip); a block scan of the
// 1 + nt popcounts of each thread gives its words their union and per-token
// prefixes.  The slice is then filled with all lanes of a wave on the 32 bits
// of one overlapping word at a time (its data broadcast with readlane), not
// by the word's own thread.  The first round's words come preloaded
// (union_words), so that a caller can issue other loads behind them before
// the block's first barrier.
constexpr int kUnionWords = 4;
template <int kNT>
__device__ __forceinline__ void union_words(const UpGateBatchArgs& a, int round, u32x4_t (&tw)[kBatchMax]) {
  const int nw = a.f / 32;  // a multiple of 4 (d_ff % 128 == 0)
  const int w0 = (round * kNT + static_cast<int>(threadIdx.x)) * kUnionWords;
  const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int t = 0; t < kBatchMax; ++t) {
    const uint32_t* bm =
        reinterpret_cast<const uint32_t*>(a.ws + static_cast<size_t>(min(t, a.nt - 1)) * a.tok_bytes + a.off_bitmap);
    tw[t] = w0 < nw ? *reinterpret_cast<const u32x4_t*>(bm + w0) : z;
  }
}

template <int kNT, int kSlice>
__device__ __forceinline__ int union_slice(const UpGateBatchArgs& a, int u0, int (&s_scan)[2][kNT / 64][1 + kBatchMax],
                                           int* s_ch, uint32_t* s_tb, u32x4_t (&tw)[kBatchMax]) {
  constexpr int kW = kNT / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int f = a.f;
  const int nt = a.nt;
  const int nw = f / 32;
  const int nrounds = (nw + kNT * kUnionWords - 1) / (kNT * kUnionWords);
  int* ulist = reinterpret_cast<int*>(a.ws + a.off_ulist);
  int base[1 + kBatchMax];
#pragma unroll
  for (int q = 0; q <= kBatchMax; ++q) base[q] = 0;
  for (int r = 0; r < nrounds; ++r) {
    if (r > 0) union_words<kNT>(a, r, tw);
    uint32_t uw[kUnionWords];
    int cnt[1 + kBatchMax];
#pragma unroll
    for (int q = 0; q <= kBatchMax; ++q) cnt[q] = 0;
#pragma unroll
    for (int t = 0; t < kBatchMax; ++t) {
      if (t >= nt) tw[t] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < kUnionWords; ++i) cnt[1 + t] += __popc(tw[t][i]);
    }
#pragma unroll
    for (int i = 0; i < kUnionWords; ++i) {
      uw[i] = 0u;
#pragma unroll
      for (int t = 0; t < kBatchMax; ++t) uw[i] |= tw[t][i];
      cnt[0] += __popc(uw[i]);
    }
    int inc[1 + kBatchMax];
#pragma unroll
    for (int q = 0; q <= kBatchMax; ++q) inc[q] = wave_inclusive_scan_int(cnt[q]);
    if (lane == 63) {
#pragma unroll
      for (int q = 0; q <= kBatchMax; ++q) s_scan[r & 1][wave][q] = inc[q];
    }
    __syncthreads();
    int excl[1 + kBatchMax];  // prefixes at this thread's first word
#pragma unroll
    for (int q = 0; q <= kBatchMax; ++q) {
      int pre = 0, tot = 0;
#pragma unroll
      for (int v = 0; v < kW; ++v) {
        const int c = s_scan[r & 1][v][q];
        pre += v < wave ? c : 0;
        tot += c;
      }
      excl[q] = base[q] + pre + inc[q] - cnt[q];
      base[q] += tot;
    }
    // words of this wave that hold ordinals of the slice, one at a time
#pragma unroll
    for (int i = 0; i < kUnionWords; ++i) {
      const int cu = __popc(uw[i]);
      uint64_t ovm = __ballot(cu > 0 && excl[0] < u0 + kSlice && excl[0] + cu > u0);
      while (ovm) {  // wave-uniform
        const int src = static_cast<int>(__builtin_ctzll(ovm));
        ovm &= ovm - 1ull;
        const uint32_t su = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(uw[i]), src));
        const int se = __builtin_amdgcn_readlane(excl[0], src);
        uint32_t st[kBatchMax];
        int sx[kBatchMax];
#pragma unroll
        for (int t = 0; t < kBatchMax; ++t) {
          st[t] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(tw[t][i]), src));
          sx[t] = __builtin_amdgcn_readlane(excl[1 + t], src);
        }
        const int bit = lane & 31;
        const uint32_t below = (1u << bit) - 1u;
        const int o = se + __popc(su & below);
        if (lane < 32 && ((su >> bit) & 1u) && o >= u0 && o < u0 + kSlice) {
          const int j = ((r * kNT + wave * 64 + src) * kUnionWords + i) * 32 + bit;
          uint32_t tb = 0u;
#pragma unroll
          for (int t = 0; t < kBatchMax; ++t) {
            if ((st[t] >> bit) & 1u) {
              tb |= 1u << t;
              a.mask_idx[static_cast<size_t>(t) * f + sx[t] + __popc(st[t] & below)] = j;
            }
          }
          s_ch[o - u0] = j;
          s_tb[o - u0] = tb;
          ulist[o] = j;
        }
      }
      // prefixes at the next word
      excl[0] += cu;
#pragma unroll
      for (int t = 0; t < kBatchMax; ++t) excl[1 + t] += __popc(tw[t][i]);
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    ulist[f] = base[0];
    for (int t = 0; t < nt; ++t) a.mask_count[t] = base[1 + t];
  }
  return base[0];
}

__global__ __launch_bounds__(kThreads) void upgate_batch_kernel(UpGateBatchArgs a) {
  __shared__ int s_scan[2][kThreads / 64][1 + kBatchMax];
  __shared__ int s_ch[kUgbChannels];
  __shared__ uint32_t s_tb[kUgbChannels];
  __shared__ float s_red[2][64][4];
  __shared__ __align__(16) uint8_t s_w[2 * kUgbChannels * kUgbRowBytes];
  __shared__ __align__(16) uint8_t s_x[16 * kUgbRowBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int d = a.d;
  const int nt = a.nt;

  const int u0 = static_cast<int>(blockIdx.x) * kUgbChannels;
  u32x4_t tw[kBatchMax];
  union_words<kThreads>(a, 0, tw);
  const int U = union_slice<kThreads, kUgbChannels>(a, u0, s_scan, s_ch, s_tb, tw);
  if (u0 >= U) return;  // block-uniform
  const int u1 = min(U, u0 + kUgbChannels);
  const int nloc = u1 - u0;
  __syncthreads();

  // ---- MFMA: wave -> (channel half ch = wave & 1, K half kh = wave >> 1)
  const int chh = wave & 1;
  const int kh = wave >> 1;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int slot = chh * 8 + (n & 7);
  const int j = s_ch[min(slot, nloc - 1)];
  typedef uint16_t S;
  // K-tiles of 512 elements are staged in LDS: each wave load instruction
  // reads one contiguous 1 KB row segment (the DRAM-friendly pattern), and
  // the MFMA operands are read back from LDS.  Staged row r = 16 tt + n holds,
  // for n < 8, the up row of slot 8 tt + n and, for n >= 8, its gate row;
  // rows are padded by 16 B so the operand reads are conflict-free.  x of the
  // group sits in LDS rows 0..7 (rows 8..15 stay zero: the A rows past the
  // tokens).  The next tile's loads are in flight while a tile is computed.
  const S* W = static_cast<const S*>(a.w_upgate_t);
  const S* X = static_cast<const S*>(a.x);
  const int unit = tid & 63;
  const S* wsrc[kUgbRowsPerThread];
#pragma unroll
  for (int q = 0; q < kUgbRowsPerThread; ++q) {
    const int r = (tid >> 6) + 4 * q;
    const int sl = 8 * (r >> 4) + (r & 7);
    wsrc[q] = W + (static_cast<size_t>(s_ch[min(sl, nloc - 1)]) * 2 + ((r >> 3) & 1)) * d;
  }
  const int xt = tid >> 5;  // token row of this thread's x units
  const S* xsrc = X + static_cast<size_t>(min(xt, nt - 1)) * d;
  const bool xon = xt < nt;
  {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < 8 * kUgbRowBytes / 16; i += kThreads)
      *reinterpret_cast<u32x4_t*>(s_x + 8 * kUgbRowBytes + 16 * i) = z;
  }
  u32x4_t wv[kUgbRowsPerThread], xv[2];
  const int nkt = (d + kUgbKt - 1) / kUgbKt;
  auto load_tile = [&](int kt) {
    const int k0 = kt * kUgbKt;
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const bool won = k0 + unit * 8 < d;
#pragma unroll
    for (int q = 0; q < kUgbRowsPerThread; ++q)
      wv[q] = won ? ldg16v_nt(wsrc[q] + k0 + unit * 8) : z;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int xu = (tid & 31) + 32 * q;
      xv[q] = (xon && k0 + xu * 8 < d) ? *reinterpret_cast<const u32x4_t*>(xsrc + k0 + xu * 8) : z;
    }
  };
  load_tile(0);
  f32x4_t C = {0.f, 0.f, 0.f, 0.f};
  const int m = lane & 15;  // A row = token
  const int brow = 16 * chh + n;
  for (int kt = 0; kt < nkt; ++kt) {
#pragma unroll
    for (int q = 0; q < kUgbRowsPerThread; ++q)
      *reinterpret_cast<u32x4_t*>(s_w + ((tid >> 6) + 4 * q) * kUgbRowBytes + 16 * unit) = wv[q];
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<u32x4_t*>(s_x + xt * kUgbRowBytes + 16 * ((tid & 31) + 32 * q)) = xv[q];
    __syncthreads();
    if (kt + 1 < nkt) load_tile(kt + 1);
    const int kvalid = min(kUgbKt, d - kt * kUgbKt);
#pragma unroll
    for (int s2 = 0; s2 < kUgbKt / 64; ++s2) {
      const int st = kh * (kUgbKt / 64) + s2;  // this wave's half of the tile's K-steps
      if (32 * st < kvalid) {  // wave-uniform
        const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(s_w + brow * kUgbRowBytes + 64 * st + 16 * g);
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(s_x + m * kUgbRowBytes + 64 * st + 16 * g);
        C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, C, 0, 0, 0);
      }
    }
    __syncthreads();  // the staged tile is rewritten next
  }
  // ---- add the two K halves, then s = u * act(g) for the tokens that keep j
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s_red[chh][lane][i] = C[i];
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) C[i] += s_red[chh][lane][i];
  float gt[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)  // lane n < 8 receives lane n + 8 (gate of the same channel)
    gt[i] = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(C[i]), 0x128, 0xF, 0xF, false));
  // s of tokens 4g..4g+3 (0 where the token does not keep the channel, and
  // for token slots past nt), stored as the down kernel's A-row entries:
  // ordinal o holds (hi, lo) bf16 pairs of tokens 0..7, 32 bytes
  if (n < 8 && g < 2 && slot < nloc) {
    const uint32_t tb = s_tb[slot];
    uint32_t pk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g + i;
      const float sv = (t < nt && ((tb >> t) & 1u)) ? C[i] * gate_act(gt[i], a.act) : 0.f;
      const uint32_t hi = f32_to_bf16_rne(sv);
      const uint32_t lo = f32_to_bf16_rne(sv - __uint_as_float(hi << 16));
      pk[i] = hi | (lo << 16);
    }
    u32x4_t* ar = reinterpret_cast<u32x4_t*>(a.ws + a.off_arows) + static_cast<size_t>(u0 + slot) * 2 + g;
    *ar = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
  }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kDnbThreads) void down_batch_kernel(DownBatchArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int d = a.d;
  const int f = a.f;
  const int nt = a.nt;
  const int cs = static_cast<int>(blockIdx.x) % a.col_slices;
  const int gi = static_cast<int>(blockIdx.x) / a.col_slices;
  const int* ulist = reinterpret_cast<const int*>(a.ws + a.off_ulist);
  const int U = min(max(ulist[f], 0), f);
  const int o0 = static_cast<int>(static_cast<long long>(U) * gi / a.groups);
  const int o1 = static_cast<int>(static_cast<long long>(U) * (gi + 1) / a.groups);
  const int nr = o1 - o0;  // <= a.max_rows
  const int ntile = (nr + kDnbTileRows - 1) / kDnbTileRows;

  // LDS: staged W tiles [2][32][512] bf16, A tiles [max_rows/32][4][16][8] bf16, rows' channels
  uint16_t* wb = reinterpret_cast<uint16_t*>(smem);
  uint16_t* As = wb + 2 * kDnbTileRows * kDnbCols;
  int* ul = reinterpret_cast<int*>(As + static_cast<size_t>(a.max_rows) * 16);
  // the group's channels, and its A rows as the up/gate kernel stored them
  // (ordinal o: m = 2t + part, s_t split into bf16 hi and lo), both in one
  // round trip; rows past the group (the last tile's padding) are zero
  for (int r = tid; r < nr; r += kDnbThreads) ul[r] = min(max(ulist[o0 + r], 0), f - 1);
  {
    const u32x4_t* arow = reinterpret_cast<const u32x4_t*>(a.ws + a.off_arows);
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int r = tid; r < ntile * kDnbTileRows; r += kDnbThreads) {
      const u32x4_t v0 = r < nr ? arow[static_cast<size_t>(o0 + r) * 2] : z;
      const u32x4_t v1 = r < nr ? arow[static_cast<size_t>(o0 + r) * 2 + 1] : z;
      const int kt = r / kDnbTileRows;
      const int k = r % kDnbTileRows;
      uint16_t* at = As + static_cast<size_t>(kt) * 512 + ((k >> 3) * 16) * 8 + (k & 7);
      const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        at[(2 * q) * 8] = static_cast<uint16_t>(w[q] & 0xFFFFu);
        at[(2 * q + 1) * 8] = static_cast<uint16_t>(w[q] >> 16);
      }
    }
  }
  __syncthreads();

  // staging: thread -> (16-B unit u = tid % 64, rows tid / 64 + 8q); unit u of
  // row r sits at unit u ^ (2 * (r & 3)) (conflict-free transposed reads)
  const int unit = tid & 63;
  const int col0 = cs * kDnbCols;
  const bool col_ok = col0 + unit * 8 < d;
  u32x4_t ld[kDnbPrefetch][4];
  // W_down through a buffer resource with the non-temporal hint (each row
  // slice is read once per launch); the last tile's padding rows and columns
  // past d load from past the buffer's records: zeros, no memory access
  const __amdgpu_buffer_rsrc_t wr = weight_rsrc(a.w_down, f, d, 2);
  auto issue = [&](int kt, u32x4_t (&dst)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = kt * kDnbTileRows + (tid >> 6) + 8 * q;
      const int ch = ul[min(r, nr - 1)];
      const uint32_t off =
          (r < nr && col_ok) ? (static_cast<uint32_t>(ch) * static_cast<uint32_t>(d) + static_cast<uint32_t>(col0 + unit * 8)) * 2u
                             : kWeightOob;
      dst[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2 /* nt */));
    }
  };
#pragma unroll
  for (int p = 0; p < kDnbPrefetch; ++p)
    if (p < ntile) issue(p, ld[p]);
  __syncthreads();  // A complete

  const int g = lane >> 4;
  const int jq = lane & 15;
  const int ri = jq >> 2;  // row within the 4-row transposed read
  const int qq = jq & 3;   // 4-column group within the 16-column tile
  const int m = lane & 15;
  const bool wave_on = col0 + 64 * wave < d;  // d % 64 == 0
  f32x4_t C[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) C[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kt0 = 0; kt0 < ntile; kt0 += kDnbPrefetch) {
#pragma unroll
    for (int p = 0; p < kDnbPrefetch; ++p) {
      const int kt = kt0 + p;
      if (kt >= ntile) break;  // block-uniform
      uint16_t* buf = wb + (kt & 1) * kDnbTileRows * kDnbCols;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = (tid >> 6) + 8 * q;
        *reinterpret_cast<u32x4_t*>(buf + r * kDnbCols + 8 * (unit ^ (2 * (r & 3)))) = ld[p][q];
      }
      if (kt + kDnbPrefetch < ntile) issue(kt + kDnbPrefetch, ld[p]);
      __syncthreads();
      if (wave_on) {
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(As + static_cast<size_t>(kt) * 512 + (g * 16 + m) * 8);
#pragma unroll
        for (int nn = 0; nn < 4; ++nn) {
          const int ut = 2 * (4 * wave + nn) + (qq >> 1);  // 16-B unit of this lane's 4 columns
          const int r1 = 8 * g + ri;
          const int r2 = r1 + 4;
          const int o1 = r1 * kDnbCols + 8 * (ut ^ (2 * (r1 & 3))) + 4 * (qq & 1);
          const int o2 = r2 * kDnbCols + 8 * (ut ^ (2 * (r2 & 3))) + 4 * (qq & 1);
          const bf16x4_t b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4_t*)((__attribute__((address_space(3))) uint16_t*)(buf) + o1));
          const bf16x4_t b2 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4_t*)((__attribute__((address_space(3))) uint16_t*)(buf) + o2));
          const bf16x8_t bv = {b1[0], b1[1], b1[2], b1[3], b2[0], b2[1], b2[2], b2[3]};
          C[nn] += __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, kZero4, 0, 0, 0);
        }
      }
      // the buffer written two tiles later is the one just read: every wave
      // passes the next iteration's barrier before that write
    }
  }
  // ---- partial y of this group: lane (g, n) holds tokens 2g, 2g+1 of column n
  if (wave_on) {
    const int n = lane & 15;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int t = 2 * g + tt;
      if (t >= nt) continue;
      float* dp = reinterpret_cast<float*>(a.ws + static_cast<size_t>(t) * a.tok_bytes + a.off_dpart) +
                  static_cast<size_t>(gi) * d;
#pragma unroll
      for (int nn = 0; nn < 4; ++nn)
        dp[col0 + 64 * wave + 16 * nn + n] = C[nn][2 * tt] + C[nn][2 * tt + 1];
    }
  }
}

// 64 outputs per block; wave q adds groups [q kG/4, (q + 1) kG/4) of them
// (kG >= a.groups: every partial in the range is loaded unconditionally,
// indices past the last group re-read it and are not added, so all loads are
// in flight before the first use), then wave 0 adds the four sums as
// (q0 + q1) + (q2 + q3): a fixed order, so y is reproducible bit for bit.
template <int kG>
__global__ __launch_bounds__(kThreads) void down_reduce_kernel(DownBatchArgs a, float* y) {
  constexpr int kPer = kG / 4;
  __shared__ float s_part[4][64];
  const int lane = threadIdx.x & 63;
  const int q = threadIdx.x >> 6;
  const int idx = blockIdx.x * 64 + lane;
  const bool on = idx < a.nt * a.d;
  const int ii = on ? idx : 0;
  const int t = ii / a.d;
  const int c = ii - t * a.d;
  const float* dp = reinterpret_cast<const float*>(a.ws + static_cast<size_t>(t) * a.tok_bytes + a.off_dpart) + c;
  float v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) v[u] = dp[static_cast<size_t>(min(q * kPer + u, a.groups - 1)) * a.d];
  float sum = 0.f;
#pragma unroll
  for (int u = 0; u < kPer; ++u) sum += q * kPer + u < a.groups ? v[u] : 0.f;
  s_part[q][lane] = sum;
  __syncthreads();
  if (q == 0 && on) y[idx] = (s_part[0][lane] + s_part[1][lane]) + (s_part[2][lane] + s_part[3][lane]);
}

}  // namespace

size_t down_batch_smem(const DownBatchArgs& a) {
  return static_cast<size_t>(2) * kDnbTileRows * kDnbCols * 2 + static_cast<size_t>(a.max_rows) * 16 * 2 +
         static_cast<size_t>(a.max_rows) * 4;
}

hipError_t launch_upgate_batch(const UpGateBatchArgs& a, hipStream_t s) {
  const int blocks = (a.f + kUgbChannels - 1) / kUgbChannels;
  hipLaunchKernelGGL(upgate_batch_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_down_batch(const DownBatchArgs& a, float* y, hipStream_t s) {
  hipLaunchKernelGGL(down_batch_kernel, dim3(static_cast<unsigned>(a.col_slices * a.groups)), dim3(kDnbThreads),
                     down_batch_smem(a), s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = a.nt * a.d;
  const dim3 rgrid(static_cast<unsigned>((n + 63) / 64));
  if (a.groups <= 8)
    hipLaunchKernelGGL(down_reduce_kernel<8>, rgrid, dim3(kThreads), 0, s, a, y);
  else if (a.groups <= 16)
    hipLaunchKernelGGL(down_reduce_kernel<16>, rgrid, dim3(kThreads), 0, s, a, y);
  else if (a.groups <= 32)
    hipLaunchKernelGGL(down_reduce_kernel<32>, rgrid, dim3(kThreads), 0, s, a, y);
  else
    hipLaunchKernelGGL(down_reduce_kernel<kDnbMaxGroups>, rgrid, dim3(kThreads), 0, s, a, y);
  return hipGetLastError();
}

}  // namespace prox
