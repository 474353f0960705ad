// Internal declarations shared by the host library and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/prox.h"

namespace prox {

// ---------------------------------------------------------------------------
// Kernel geometry (compile-time)
// ---------------------------------------------------------------------------
constexpr int kThreads = 256;          // every kernel uses 4 waves of 64
constexpr int kStage1Unroll = 16;      // proxy rows loaded per lane per batch
constexpr int kUpGateUnroll = 8;       // 16-B steps per channel batch (x2 loads)
constexpr int kUgResidentBlocks = 1024;  // up/gate: blocks resident at once (4 per CU over 256 CUs)
constexpr int kUgThreads = 256;        // up/gate kernel: threads per block
constexpr int kDownUnroll = 8;         // W_down rows per wave per batch
constexpr int kDownTargetBlocks = 512;  // down kernel: at most this many blocks (two per CU)
constexpr int kDownThreads = 1024;     // down kernel: 16 waves share one column slice
constexpr int kFusedThreads = 1024;    // fused Stage-2 kernel: 16 waves per block, one block per CU
constexpr int kFusedItems = 256;       // fused Stage-2 kernel: down items planned (the CU count of MI355X)
constexpr int kMaxGridFlags = 1024;    // fused Stage-2 kernel: grid-barrier flags in the workspace
constexpr uint32_t kDefaultWaitTicks = 4000000u;  // bounded waits: 40 ms of the 100 MHz real-time clock
constexpr int kBatchMax = 8;           // tokens per group of the batched kernels
constexpr int kS1MaxRowsPerSplit = 896;  // Stage 1: input rows per K-split at most (one gather batch per wave)
constexpr int kGroupedMinTokens = 3;   // smaller groups run the per-token kernels (faster there)

// ---------------------------------------------------------------------------
// Per-launch plan (host-computed, passed by value to kernels)
// ---------------------------------------------------------------------------
struct Plan {
  int d, f, wdtype;
  // Stage 1
  int proxy_stride;  // bytes between proxy rows (odd multiple of 128)
  int proxy16_stride;  // bytes between 16-bit proxy rows (odd multiple of 128)
  int panel;         // Stage-1 output columns per block (256 or 128)
  int n_panels;      // f / panel
  int splits;        // K-splits over input rows
  int rows_per_split;
  // Stage 2 up/gate
  int ug_blocks;     // blocks per token
  // Stage 2 down
  int dn_col_slices; // ceil(d / column-slice width)
  int dn_row_groups;
  int dn_max_rows;   // max rows per group (list mode) / LDS rows
  int dn_chan_per_group;  // decode mode: channels per row group (multiple of 32, <= 1024)
  // (dn_row_groups, dn_max_rows and dn_chan_per_group are those of a
  // one-token launch; down_groups gives them for any token count)
  // batched down (groups of 2..8 tokens): 512-column slices x groups of union ordinals
  int dnb_col_slices;
  int dnb_groups;
  int dnb_max_rows;  // rows per group, multiple of 32
  // fused Stage 2 (batch 1): down items of (column slice, row group)
  int fz_col_slices, fz_row_groups, fz_chan_per_group, fz_max_rows, fz_red_bytes;
  // workspace layout, bytes per token and offsets inside a token's slice; the
  // error word, the fused kernel's completion ticket and the grid-barrier
  // flags sit at fixed offsets at the start of a slice (shape-independent)
  size_t tok_bytes;
  size_t off_err, off_done, off_flags;
  size_t off_tickets, off_kcount, off_partial, off_bitmap, off_ssp;
  size_t off_arows;  // grouped path: per union ordinal, the tokens' s as bf16 (hi, lo) pairs [f][16]
  size_t off_ulist;  // group's first token: union channel list [f] + count at [f]
  size_t off_dpart;  // batched down partials [dnb_groups][d] fp32
};

Plan make_plan(int d, int f, int wdtype);

// Down kernel row groups for a launch over `tokens` tokens
struct DownGroups {
  int row_groups, chan_per_group, max_rows;
};
DownGroups down_groups(const Plan& p, int tokens);

struct Stage1Args {
  int d, f, splits, rows_per_split, n_panels, panel, proxy_stride;
  const uint8_t* proxy_q;
  const float* proxy_scale;
  const void* x;          // [batch][d]
  float tau_x, tau_s;
  uint8_t* ws;            // base of token 0's slice
  size_t tok_bytes, off_tickets, off_kcount, off_partial, off_bitmap;
  float* s_tilde;         // [batch][f] or nullptr
  int* in_count;          // [batch] or nullptr
  int act;                // prox_activation
  int nt;                 // batched kernel: tokens in the group (2..8)
  int proxy_kind;         // prox_proxy_kind
  int proxy16_stride;     // PROX_PROXY_W16: bytes between proxy rows
  const void* proxy_w16;  // PROX_PROXY_W16: [d][proxy16_stride] bf16 rows
};

// Stage 1 of a group of nt <= kBatchMax tokens from the channel-major copy of
// the INT4 proxy (proxy_qt).  Grid: nb blocks, block b owning 16-channel
// groups [b ng / nb, (b + 1) ng / nb); each group's K range is cut into
// `parts` contiguous ranges of ncp 128-row chunks (the last may run past d).
struct QtArgs {
  int d, f, nt, act;
  int nck;        // 128-row chunks of the K range, ceil(d / 128)
  int parts;      // 1, 2 or 4
  int ncp;        // chunks per part, ceil(nck / parts)
  int ng, nb;     // 16-channel groups (f / 16) and blocks
  int s_waves;    // streaming waves per block (all 16 build operands, the rest only that)
  int upw;        // units (group, part) per streaming wave: 1 or 2
  const uint8_t* proxy_qt;
  const float* proxy_scale;
  const void* x;  // [nt][d]
  float tau_x, tau_s;
  uint8_t* ws;    // the group's first token slice
  size_t tok_bytes, off_bitmap;
  float* s_tilde; // [nt][f] or nullptr
  int* in_count;  // [nt] or nullptr
};

// Plan of the channel-major Stage-1 kernel for (d, f); `blocks` is the grid cap.
QtArgs qt_plan(int d, int f, int blocks);
size_t proxy_qt_bytes(int d, int f);

// Batched Stage 2 (bf16 weights), one group of nt <= kBatchMax tokens; ws is
// the group's first token slice, token t's slice is ws + t * tok_bytes.
struct UpGateBatchArgs {
  int d, f, nt, act;
  const void* w_upgate_t;  // [f][2][d] bf16
  const void* x;           // [nt][d] bf16
  uint8_t* ws;
  size_t tok_bytes, off_bitmap, off_ulist, off_arows;
  int* mask_idx;           // [nt][f]
  int* mask_count;         // [nt]
};

struct DownBatchArgs {
  int d, f, nt, col_slices, groups, max_rows;
  const void* w_down;      // [f][d] bf16
  uint8_t* ws;
  size_t tok_bytes, off_ulist, off_arows, off_dpart;
};

struct UpGateArgs {
  int d, f;
  int act;                // prox_activation
  const void* w_upgate_t; // [f][2][d]
  const void* x;          // [batch][d]
  const uint8_t* ws;      // bitmap source (decode mode)
  uint8_t* ws_mut;        // s_sp destination
  size_t tok_bytes, off_bitmap, off_ssp;
  int* mask_idx;          // decode mode: written; list mode: read (const)
  int* mask_count;        // decode mode: written; list mode: read
  float* y;               // zeroed here
};

struct DownArgs {
  int d, f, col_slices, row_groups, max_rows, chan_per_group;
  const void* w_down;     // [f][d]
  const uint8_t* ws;      // s (by channel in decode mode, by list position otherwise), bitmap
  size_t tok_bytes, off_ssp, off_bitmap;
  const int* mask_idx;
  const int* mask_count;
  float* y;
};

// Fused Stage 2 of one token (batch 1): up/gate then down in one launch.
struct FusedArgs {
  UpGateArgs ug;          // decode mode; ug.ws_mut is token 0's workspace slice
  const void* w_down;     // [f][d]
  int col_slices, row_groups, chan_per_group, max_rows;
  int red_bytes;          // LDS bytes before the row list: max(x, down reduction buffer)
  size_t off_flags, off_err, off_done;
  uint32_t wait_ticks;    // bounded wait of the grid barrier (100 MHz clock ticks)
};

// Launchers (return hipSuccess or the launch error).
hipError_t launch_stage1(const Stage1Args& a, int wdtype, int batch, bool write_state,
                         hipStream_t s);
hipError_t launch_upgate(const UpGateArgs& a, int wdtype, int batch, int blocks,
                         bool from_bitmap, hipStream_t s);
hipError_t launch_down(const DownArgs& a, int wdtype, int batch, bool from_bitmap, hipStream_t s);
hipError_t launch_stage2_fused(const FusedArgs& a, int wdtype, int grid, hipStream_t s);
hipError_t fused_occupancy(int wdtype, size_t smem, int* blocks_per_cu);
size_t fused_smem(const FusedArgs& a);
hipError_t launch_stage1_batch(const Stage1Args& a, int wdtype, bool write_state, hipStream_t s);
hipError_t launch_stage1_qt(const QtArgs& a, int wdtype, bool write_state, hipStream_t s);
// whether the channel-major Stage 1 of this plan fits the kernel's waves and
// the device's LDS (x of the group's tokens and the scales are staged there);
// if not, the union-of-rows Stage 1 runs instead
bool qt_fits(const QtArgs& a, int wdtype);
hipError_t launch_pack_qt(const uint8_t* proxy_q, int qstride, int d, int f, uint8_t* proxy_qt, hipStream_t s);
hipError_t launch_stage1_w16(const Stage1Args& a, int batch, bool write_state, hipStream_t s);
int proxy16_row_stride(int f);
hipError_t launch_pack16(const void* w_up, const void* w_gate, int d, int f, int stride, void* proxy_w16,
                         hipStream_t s);
hipError_t launch_upgate_batch(const UpGateBatchArgs& a, hipStream_t s);
hipError_t launch_down_batch(const DownBatchArgs& a, float* y, hipStream_t s);
size_t down_batch_smem(const DownBatchArgs& a);
int proxy_row_stride(int f);
hipError_t launch_pack(const void* w_up, const void* w_gate, int d, int f, int qstride, int wdtype,
                       uint8_t* proxy_q, float* proxy_scale, void* w_upgate_t, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// Histogram calibration: |v| at n evenly strided positions (m of n values)
// into out, with the maximum's fp32 bits atomically maxed into *maxbits; and
// a linear nb-bin histogram of m non-negative values with bin width w.
hipError_t launch_sample_abs(const void* v, uint64_t n, int vdtype, uint32_t m, float* out, uint32_t* maxbits,
                             hipStream_t s);
hipError_t launch_bin_hist(const float* v, uint32_t m, float w, int nb, uint32_t* hist, hipStream_t s);
// Calibration helpers: histogram of 8-bit digits of |v| keys that match a
// prefix; keys are fp32 bit patterns of |value| (values in wdtype or fp32).
hipError_t launch_digit_histogram(const void* v, size_t n, int vdtype, uint32_t prefix,
                                  uint32_t prefix_mask, int shift, uint32_t* hist,
                                  hipStream_t s);

}  // namespace prox
