// Host side of the C ABI declared in include/prox.h: argument validation,
// launch planning, workspace layout and calibration orchestration.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "prox_internal.h"

#define PROX_API extern "C" __attribute__((visibility("default")))

namespace prox {
namespace {

thread_local std::string g_err;

prox_status fail(prox_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

prox_status hip_fail(hipError_t e, const char* what) {
  return fail(PROX_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(int wdtype) { return wdtype == PROX_BF16 ? 2 : 4; }

prox_status check_shape(int32_t d, int32_t f, int32_t wdtype) {
  if (wdtype != PROX_F32 && wdtype != PROX_BF16)
    return fail(PROX_ERR_INVALID_ARG, "wdtype %d is neither PROX_F32 nor PROX_BF16", wdtype);
  if (d < 64 || f < 128)
    return fail(PROX_ERR_INVALID_ARG, "shape d_model=%d d_ff=%d below the minimum 64 x 128", d, f);
  if (d % 64 != 0 || f % 128 != 0)
    return fail(PROX_ERR_UNSUPPORTED, "shape d_model=%d d_ff=%d: need d_model %% 64 == 0 and "
                "d_ff %% 128 == 0", d, f);
  if (d > 12288 || f > 65536)
    return fail(PROX_ERR_UNSUPPORTED, "shape d_model=%d d_ff=%d above 12288 x 65536", d, f);
  return PROX_OK;
}

prox_status check_layer(const prox_layer* L) {
  if (L == nullptr) return fail(PROX_ERR_INVALID_ARG, "layer descriptor is NULL");
  prox_status st = check_shape(L->d_model, L->d_ff, L->wdtype);
  if (st != PROX_OK) return st;
  if (L->activation != PROX_ACT_SILU && L->activation != PROX_ACT_GELU_TANH)
    return fail(PROX_ERR_INVALID_ARG, "layer->activation %d is neither PROX_ACT_SILU nor PROX_ACT_GELU_TANH",
                L->activation);
  if (L->reserved != 0) return fail(PROX_ERR_INVALID_ARG, "layer->reserved must be 0");
  if (L->proxy_kind == PROX_PROXY_INT4) {
    if (!L->proxy_q || !L->proxy_scale)
      return fail(PROX_ERR_INVALID_ARG, "layer proxy_q / proxy_scale is NULL (PROX_PROXY_INT4)");
    if (!aligned(L->proxy_q, 16) || !aligned(L->proxy_scale, 16))
      return fail(PROX_ERR_INVALID_ARG, "layer buffers must be 16-byte aligned");
  } else if (L->proxy_kind == PROX_PROXY_W16) {
    if (L->wdtype != PROX_BF16)
      return fail(PROX_ERR_UNSUPPORTED, "the 16-bit proxy is for bf16 layers (wdtype %d)", L->wdtype);
    if (!L->proxy_w16) return fail(PROX_ERR_INVALID_ARG, "layer proxy_w16 is NULL (PROX_PROXY_W16)");
    if (!aligned(L->proxy_w16, 16)) return fail(PROX_ERR_INVALID_ARG, "layer buffers must be 16-byte aligned");
  } else {
    return fail(PROX_ERR_INVALID_ARG, "layer->proxy_kind %d is neither PROX_PROXY_INT4 nor PROX_PROXY_W16",
                L->proxy_kind);
  }
  if (L->proxy_qt && (L->proxy_kind != PROX_PROXY_INT4 || !aligned(L->proxy_qt, 16)))
    return fail(PROX_ERR_INVALID_ARG, "layer proxy_qt must be 16-byte aligned and belongs to PROX_PROXY_INT4 layers");
  if (!L->w_upgate_t || !L->w_down) return fail(PROX_ERR_INVALID_ARG, "layer buffer pointer is NULL");
  if (!aligned(L->w_upgate_t, 16) || !aligned(L->w_down, 16))
    return fail(PROX_ERR_INVALID_ARG, "layer buffers must be 16-byte aligned");
  return PROX_OK;
}

prox_status check_tau(float t, const char* name) {
  if (std::isnan(t) || t < 0.f)
    return fail(PROX_ERR_INVALID_ARG, "%s = %g: thresholds must be >= 0 or +inf", name,
                static_cast<double>(t));
  return PROX_OK;
}

prox_status check_batch(int32_t batch) {
  if (batch < 1 || batch > 256) return fail(PROX_ERR_INVALID_ARG, "batch %d outside [1, 256]", batch);
  return PROX_OK;
}

prox_status check_ws(const Plan& p, int32_t batch, const void* ws, size_t ws_bytes) {
  if (ws == nullptr) return fail(PROX_ERR_INVALID_ARG, "workspace is NULL");
  if (!aligned(ws, 256)) return fail(PROX_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t need = p.tok_bytes * static_cast<size_t>(batch);
  if (ws_bytes < need)
    return fail(PROX_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  return PROX_OK;
}

Stage1Args stage1_args(const Plan& p, const prox_layer* L, const void* x, float tau_x, float tau_s,
                       void* ws, float* s_tilde, int* in_count) {
  Stage1Args a;
  a.d = p.d;
  a.f = p.f;
  a.splits = p.splits;
  a.rows_per_split = p.rows_per_split;
  a.n_panels = p.n_panels;
  a.panel = p.panel;
  a.proxy_stride = p.proxy_stride;
  a.proxy_q = static_cast<const uint8_t*>(L->proxy_q);
  a.proxy_scale = L->proxy_scale;
  a.x = x;
  a.tau_x = tau_x;
  a.tau_s = tau_s;
  a.ws = static_cast<uint8_t*>(ws);
  a.tok_bytes = p.tok_bytes;
  a.off_tickets = p.off_tickets;
  a.off_kcount = p.off_kcount;
  a.off_partial = p.off_partial;
  a.off_bitmap = p.off_bitmap;
  a.s_tilde = s_tilde;
  a.in_count = in_count;
  a.act = L->activation;
  a.nt = 1;
  a.proxy_kind = L->proxy_kind;
  a.proxy16_stride = p.proxy16_stride;
  a.proxy_w16 = L->proxy_w16;
  return a;
}

UpGateArgs upgate_args(const Plan& p, const prox_layer* L, const void* x, void* ws, int* mask_idx,
                       int* mask_count, float* y) {
  UpGateArgs a;
  a.d = p.d;
  a.f = p.f;
  a.act = L->activation;
  a.w_upgate_t = L->w_upgate_t;
  a.x = x;
  a.ws = static_cast<const uint8_t*>(ws);
  a.ws_mut = static_cast<uint8_t*>(ws);
  a.tok_bytes = p.tok_bytes;
  a.off_bitmap = p.off_bitmap;
  a.off_ssp = p.off_ssp;
  a.mask_idx = mask_idx;
  a.mask_count = mask_count;
  a.y = y;
  return a;
}

DownArgs down_args(const Plan& p, const prox_layer* L, void* ws, const int* mask_idx,
                   const int* mask_count, float* y, int tokens) {
  DownArgs a;
  a.d = p.d;
  a.f = p.f;
  const DownGroups g = down_groups(p, tokens);
  a.col_slices = p.dn_col_slices;
  a.row_groups = g.row_groups;
  a.max_rows = g.max_rows;
  a.chan_per_group = g.chan_per_group;
  a.w_down = L->w_down;
  a.ws = static_cast<const uint8_t*>(ws);
  a.tok_bytes = p.tok_bytes;
  a.off_ssp = p.off_ssp;
  a.off_bitmap = p.off_bitmap;
  a.mask_idx = mask_idx;
  a.mask_count = mask_count;
  a.y = y;
  return a;
}

UpGateBatchArgs upgate_batch_args(const Plan& p, const prox_layer* L, const void* x, void* ws, int nt,
                                  int* mask_idx, int* mask_count) {
  UpGateBatchArgs a;
  a.d = p.d;
  a.f = p.f;
  a.nt = nt;
  a.act = L->activation;
  a.w_upgate_t = L->w_upgate_t;
  a.x = x;
  a.ws = static_cast<uint8_t*>(ws);
  a.tok_bytes = p.tok_bytes;
  a.off_bitmap = p.off_bitmap;
  a.off_ulist = p.off_ulist;
  a.off_arows = p.off_arows;
  a.mask_idx = mask_idx;
  a.mask_count = mask_count;
  return a;
}

DownBatchArgs down_batch_args(const Plan& p, const prox_layer* L, void* ws, int nt) {
  DownBatchArgs a;
  a.d = p.d;
  a.f = p.f;
  a.nt = nt;
  a.col_slices = p.dnb_col_slices;
  a.groups = p.dnb_groups;
  a.max_rows = p.dnb_max_rows;
  a.w_down = L->w_down;
  a.ws = static_cast<uint8_t*>(ws);
  a.tok_bytes = p.tok_bytes;
  a.off_ulist = p.off_ulist;
  a.off_arows = p.off_arows;
  a.off_dpart = p.off_dpart;
  return a;
}

// Token groups of the batched kernels: [g0, g0 + nt) with nt <= kBatchMax.
template <typename Fn>
hipError_t for_each_group(int32_t batch, Fn fn) {
  for (int g0 = 0; g0 < batch; g0 += kBatchMax) {
    const hipError_t e = fn(g0, std::min<int>(kBatchMax, batch - g0));
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// CUs of the current device (the channel-major Stage-1 grid: one block per
// CU), cached per device; 256 if the query fails.
int device_cus();

// Channel-major Stage 1 of one group of nt tokens (ws: the group's first slice).
QtArgs qt_args(const Plan& p, const prox_layer* L, const void* x, float tau_x, float tau_s, void* ws,
               float* s_tilde, int* in_count, int nt) {
  QtArgs a = qt_plan(p.d, p.f, device_cus());
  a.nt = nt;
  a.act = L->activation;
  a.proxy_qt = static_cast<const uint8_t*>(L->proxy_qt);
  a.proxy_scale = L->proxy_scale;
  a.x = x;
  a.tau_x = tau_x;
  a.tau_s = tau_s;
  a.ws = static_cast<uint8_t*>(ws);
  a.tok_bytes = p.tok_bytes;
  a.off_bitmap = p.off_bitmap;
  a.s_tilde = s_tilde;
  a.in_count = in_count;
  return a;
}

// The channel-major Stage 1 for a group of nt tokens: when the layer has the
// copy and the group's x and scales fit the device's LDS.
bool qt_usable(const Plan& p, const prox_layer* L, int nt) {
  QtArgs a = qt_plan(p.d, p.f, device_cus());
  a.nt = nt;
  return qt_fits(a, L->wdtype);
}

FusedArgs fused_args(const Plan& p, const prox_layer* L, const void* x, void* ws, int* mask_idx, int* mask_count,
                     float* y, uint32_t wait_ticks) {
  FusedArgs a;
  a.ug = upgate_args(p, L, x, ws, mask_idx, mask_count, y);
  a.w_down = L->w_down;
  a.col_slices = p.fz_col_slices;
  a.row_groups = p.fz_row_groups;
  a.chan_per_group = p.fz_chan_per_group;
  a.max_rows = p.fz_max_rows;
  a.red_bytes = p.fz_red_bytes;
  a.off_flags = p.off_flags;
  a.off_err = p.off_err;
  a.off_done = p.off_done;
  a.wait_ticks = wait_ticks;
  return a;
}

std::atomic<uint32_t> g_wait_ticks{kDefaultWaitTicks};

// Per device: the CU count and the fused Stage-2 kernel's resident blocks per
// CU for each (weight dtype, LDS bytes) seen.
struct DevInfo {
  int cus = 0;
  int coop = -1;  // hipDeviceAttributeCooperativeLaunch
  std::vector<std::pair<std::pair<int, size_t>, int>> occ;
};
std::mutex g_dev_mu;
std::vector<DevInfo> g_dev;

// Grid of the fused Stage-2 kernel on the current device (one block per CU),
// or 0 when it cannot run there: no cooperative launches, fewer than one
// resident block per CU, more CUs than the workspace holds barrier flags for,
// or a failed query (the two Stage-2 kernels run instead).
int fused_grid(int wdtype, size_t smem) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (g_dev.size() <= static_cast<size_t>(dev)) g_dev.resize(static_cast<size_t>(dev) + 1);
  DevInfo& di = g_dev[static_cast<size_t>(dev)];
  if (di.cus == 0 && hipDeviceGetAttribute(&di.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    di.cus = 0;
    return 0;
  }
  if (di.coop < 0 && hipDeviceGetAttribute(&di.coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess) {
    di.coop = -1;
    return 0;
  }
  if (di.coop != 1) return 0;
  int occ = -1;
  for (const auto& e : di.occ)
    if (e.first.first == wdtype && e.first.second == smem) occ = e.second;
  if (occ < 0) {
    if (fused_occupancy(wdtype, smem, &occ) != hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    di.occ.push_back({{wdtype, smem}, occ});
  }
  if (occ < 1 || di.cus < 1 || di.cus > kMaxGridFlags) return 0;
  return di.cus;
}

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  std::lock_guard<std::mutex> lock(g_dev_mu);
  if (g_dev.size() <= static_cast<size_t>(dev)) g_dev.resize(static_cast<size_t>(dev) + 1);
  DevInfo& di = g_dev[static_cast<size_t>(dev)];
  if (di.cus == 0 && hipDeviceGetAttribute(&di.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    di.cus = 0;
  return di.cus > 0 ? di.cus : 256;
}

// Checks of prox_ffn_decode's arguments other than the workspace.
prox_status check_decode_args(const prox_layer* layer, const void* x, int32_t batch, float tau_x, float tau_s,
                              const float* y, const int32_t* mask_idx, const int32_t* mask_count,
                              const int32_t* in_count) {
  prox_status st = check_layer(layer);
  if (st != PROX_OK) return st;
  if ((st = check_batch(batch)) != PROX_OK) return st;
  if ((st = check_tau(tau_x, "tau_x")) != PROX_OK) return st;
  if ((st = check_tau(tau_s, "tau_s")) != PROX_OK) return st;
  if (!x || !y || !mask_idx || !mask_count)
    return fail(PROX_ERR_INVALID_ARG, "x, y, mask_idx and mask_count must be non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(mask_idx, 4) || !aligned(mask_count, 4) ||
      (in_count && !aligned(in_count, 4)))
    return fail(PROX_ERR_INVALID_ARG, "x and y must be 16-byte aligned, index buffers 4-byte aligned");
  return PROX_OK;
}

prox_status decode_impl(const prox_layer* layer, const void* x, int32_t batch, float tau_x,
                        float tau_s, float* y, int32_t* mask_idx, int32_t* mask_count,
                        int32_t* in_count, void* ws, size_t ws_bytes, void* stream,
                        void* const* events, int32_t stages = 7) {
  prox_status st = check_decode_args(layer, x, batch, tau_x, tau_s, y, mask_idx, mask_count, in_count);
  if (st != PROX_OK) return st;
  const Plan p = make_plan(layer->d_model, layer->d_ff, layer->wdtype);
  if ((st = check_ws(p, batch, ws, ws_bytes)) != PROX_OK) return st;
  if (events) {
    for (int i = 0; i < 4; ++i)
      if (!events[i]) return fail(PROX_ERR_INVALID_ARG, "events[%d] is NULL", i);
  }
  if ((stages & 7) == 0 || stages < 0 || stages > 63 ||
      ((stages & PROX_STAGE_PER_TOKEN) && (stages & PROX_STAGE_GROUPED)))
    return fail(PROX_ERR_INVALID_ARG, "stages %d: a non-empty subset of 1|2|4, plus at most one of 8 and 16, "
                "and optionally 32", stages);
  // Kernels per group of nt <= kBatchMax tokens: the grouped ones (each proxy
  // row and channel of the group's unions read once; Stage 2 grouped for bf16
  // weights, INT4 proxy only) from kGroupedMinTokens tokens up, where they are
  // faster, the per-token ones below; PROX_STAGE_PER_TOKEN / PROX_STAGE_GROUPED
  // force either for every group.
  auto grouped1 = [&](int nt) {
    if (batch < 2 || layer->proxy_kind != PROX_PROXY_INT4 || (stages & PROX_STAGE_PER_TOKEN)) return false;
    return (stages & PROX_STAGE_GROUPED) != 0 || nt >= kGroupedMinTokens;
  };
  auto grouped2 = [&](int nt) { return grouped1(nt) && layer->wdtype == PROX_BF16; };
  // Stage 1 from the channel-major proxy copy, when the layer has one: for
  // the groups that take the grouped kernels (faster than the union-of-rows
  // Stage 1 there; for two tokens the per-token Stage 1 is faster still)
  auto qt1 = [&](int nt) {
    return layer->proxy_qt != nullptr && layer->proxy_kind == PROX_PROXY_INT4 && nt >= 2 &&
           !(stages & PROX_STAGE_PER_TOKEN) &&
           ((stages & PROX_STAGE_GROUPED) != 0 || nt >= kGroupedMinTokens) && qt_usable(p, layer, nt);
  };
  bool any1 = false, any2 = false;
  for (int g0 = 0; g0 < batch; g0 += kBatchMax) {
    const int nt = std::min<int>(kBatchMax, batch - g0);
    any1 = any1 || grouped1(nt) || qt1(nt);
    any2 = any2 || grouped2(nt);
  }
  const size_t es = elem_size(layer->wdtype);
  auto x_at = [&](int g0) { return static_cast<const uint8_t*>(x) + static_cast<size_t>(g0) * p.d * es; };
  auto ws_at = [&](int g0) { return static_cast<uint8_t*>(ws) + static_cast<size_t>(g0) * p.tok_bytes; };
  auto mi_at = [&](int g0) { return mask_idx + static_cast<size_t>(g0) * p.f; };
  auto y_at = [&](int g0) { return y + static_cast<size_t>(g0) * p.d; };
  auto ic_at = [&](int g0) { return in_count ? in_count + g0 : nullptr; };
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (events && (e = hipEventRecord(static_cast<hipEvent_t>(events[0]), s)) != hipSuccess)
    return hip_fail(e, "hipEventRecord");
  if (stages & PROX_STAGE_PROXY) {
    if (!any1) {
      e = launch_stage1(stage1_args(p, layer, x, tau_x, tau_s, ws, nullptr, in_count), layer->wdtype, batch,
                        false, s);
    } else {
      e = for_each_group(batch, [&](int g0, int nt) {
        if (qt1(nt))
          return launch_stage1_qt(qt_args(p, layer, x_at(g0), tau_x, tau_s, ws_at(g0), nullptr, ic_at(g0), nt),
                                  layer->wdtype, false, s);
        Stage1Args a1 = stage1_args(p, layer, x_at(g0), tau_x, tau_s, ws_at(g0), nullptr, ic_at(g0));
        if (!grouped1(nt)) return launch_stage1(a1, layer->wdtype, nt, false, s);
        a1.nt = nt;
        return launch_stage1_batch(a1, layer->wdtype, false, s);
      });
    }
    if (e != hipSuccess) return hip_fail(e, "stage-1 launch");
  }
  if (events && (e = hipEventRecord(static_cast<hipEvent_t>(events[1]), s)) != hipSuccess)
    return hip_fail(e, "hipEventRecord");
  // batch 1, both Stage-2 kernels and PROX_STAGE_FUSED_STAGE2: one fused
  // launch where the device can hold its grid
  int fgrid = 0;
  FusedArgs fa;
  if (batch == 1 && (stages & PROX_STAGE_UPGATE) && (stages & PROX_STAGE_DOWN) &&
      (stages & PROX_STAGE_FUSED_STAGE2)) {
    fa = fused_args(p, layer, x, ws, mask_idx, mask_count, y, g_wait_ticks.load());
    fgrid = fused_grid(layer->wdtype, fused_smem(fa));
  }
  if (fgrid > 0) {
    e = launch_stage2_fused(fa, layer->wdtype, fgrid, s);
    if (e == hipErrorCooperativeLaunchTooLarge) {  // the runtime cannot hold the grid now: two kernels
      (void)hipGetLastError();
      fgrid = 0;
    } else if (e != hipSuccess) {
      return hip_fail(e, "fused stage-2 launch");
    }
  }
  if (fgrid == 0 && (stages & PROX_STAGE_UPGATE)) {
    if (!any2) {
      e = launch_upgate(upgate_args(p, layer, x, ws, mask_idx, mask_count, y), layer->wdtype, batch,
                        p.ug_blocks, true, s);
    } else {
      e = for_each_group(batch, [&](int g0, int nt) {
        if (!grouped2(nt))
          return launch_upgate(upgate_args(p, layer, x_at(g0), ws_at(g0), mi_at(g0), mask_count + g0, y_at(g0)),
                               layer->wdtype, nt, p.ug_blocks, true, s);
        return launch_upgate_batch(upgate_batch_args(p, layer, x_at(g0), ws_at(g0), nt, mi_at(g0), mask_count + g0),
                                   s);
      });
    }
    if (e != hipSuccess) return hip_fail(e, "stage-2 up/gate launch");
  }
  if (events && (e = hipEventRecord(static_cast<hipEvent_t>(events[2]), s)) != hipSuccess)
    return hip_fail(e, "hipEventRecord");
  if ((stages & PROX_STAGE_DOWN) && fgrid == 0) {
    if (!any2) {
      e = launch_down(down_args(p, layer, ws, mask_idx, mask_count, y, batch), layer->wdtype, batch, true, s);
    } else {
      e = for_each_group(batch, [&](int g0, int nt) {
        if (!grouped2(nt))
          return launch_down(down_args(p, layer, ws_at(g0), mi_at(g0), mask_count + g0, y_at(g0), nt), layer->wdtype, nt,
                             true, s);
        return launch_down_batch(down_batch_args(p, layer, ws_at(g0), nt), y_at(g0), s);
      });
    }
    if (e != hipSuccess) return hip_fail(e, "stage-2 down launch");
  }
  if (events && (e = hipEventRecord(static_cast<hipEvent_t>(events[3]), s)) != hipSuccess)
    return hip_fail(e, "hipEventRecord");
  return PROX_OK;
}

// keep-th largest |v| over n values by an MSB-first radix select on the fp32
// bit patterns of |v| (order-preserving for non-negative floats).  Counting
// runs on the GPU; the host walks the 256-bin histograms.  Blocks.
prox_status select_kth_largest(const void* v, size_t n, int vdtype, uint64_t keep,
                               uint32_t* hist_dev, hipStream_t s, float* out) {
  if (keep == 0) {
    *out = INFINITY;
    return PROX_OK;
  }
  uint32_t prefix = 0, pmask = 0;
  uint64_t remaining = keep;
  std::vector<uint32_t> hist(256);
  for (int shift = 24; shift >= 0; shift -= 8) {
    hipError_t e = launch_fill_zero(hist_dev, 256 * sizeof(uint32_t), s);
    if (e != hipSuccess) return hip_fail(e, "histogram clear");
    e = launch_digit_histogram(v, n, vdtype, prefix, pmask, shift, hist_dev, s);
    if (e != hipSuccess) return hip_fail(e, "histogram launch");
    e = hipMemcpyAsync(hist.data(), hist_dev, 256 * sizeof(uint32_t), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "histogram copy");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "calibration synchronisation");
    uint64_t cum = 0;
    int digit = -1;
    for (int dg = 255; dg >= 0; --dg) {
      if (cum + hist[dg] >= remaining) {
        digit = dg;
        break;
      }
      cum += hist[dg];
    }
    if (digit < 0) return fail(PROX_ERR_INTERNAL, "radix select lost its rank (count %llu)",
                               static_cast<unsigned long long>(cum));
    remaining -= cum;
    prefix |= static_cast<uint32_t>(digit) << shift;
    pmask |= 255u << shift;
  }
  uint32_t bits = prefix;
  float r;
  std::memcpy(&r, &bits, 4);
  *out = r;
  return PROX_OK;
}

uint64_t keep_count(double keep, uint64_t n) {
  const double k = std::ceil(keep * static_cast<double>(n));
  if (!(k > 0.0)) return 0;
  if (k >= static_cast<double>(n)) return n;
  return static_cast<uint64_t>(k);
}

constexpr int kCalChunk = 16;  // calibration tokens per Stage-1 launch

size_t calib_bytes(const Plan& p, int32_t n_tokens) {
  return align256(static_cast<size_t>(n_tokens) * p.f * sizeof(float)) +
         p.tok_bytes * std::min<int32_t>(n_tokens, kCalChunk) + 1024;
}

constexpr uint32_t kMaxHistSamples = 1u << 24;  // keeps i * N below 2^64
constexpr int kMaxHistBins = 8192;              // the LDS histogram of one block

size_t calib_hist_bytes(const Plan& p, int32_t n_tokens, uint32_t max_samples, int n_bins) {
  return calib_bytes(p, n_tokens) + align256(static_cast<size_t>(max_samples) * sizeof(float)) +
         align256(static_cast<size_t>(n_bins) * sizeof(uint32_t)) + 256;
}

// Threshold from an evenly strided sample of at most max_samples of the n
// values |v| and a linear nb-bin histogram over [0, max]: the lower edge of
// the bin where the count from the top first reaches ceil(keep * m).  Bin
// decisions use IEEE fp32 divisions; the edge is fp32(b * w).  Blocks.
prox_status hist_threshold(const void* v, uint64_t n, int vdtype, double keep, uint32_t max_samples, int nb,
                           float* samples, uint32_t* hist_dev, uint32_t* max_dev, hipStream_t s, float* out) {
  const uint32_t m = static_cast<uint32_t>(std::min<uint64_t>(n, max_samples));
  const uint64_t keep_n = keep_count(keep, m);
  if (keep_n == 0) {
    *out = INFINITY;
    return PROX_OK;
  }
  hipError_t e = launch_fill_zero(max_dev, sizeof(uint32_t), s);
  if (e != hipSuccess) return hip_fail(e, "sample maximum clear");
  e = launch_sample_abs(v, n, vdtype, m, samples, max_dev, s);
  if (e != hipSuccess) return hip_fail(e, "sample launch");
  uint32_t maxbits = 0;
  e = hipMemcpyAsync(&maxbits, max_dev, sizeof(uint32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "sample maximum copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "calibration synchronisation");
  float vmax;
  std::memcpy(&vmax, &maxbits, 4);
  if (!std::isfinite(vmax)) return fail(PROX_ERR_INVALID_ARG, "calibration values are not all finite");
  const float w = vmax / static_cast<float>(nb);
  if (!(w > 0.f)) {
    *out = 0.f;
    return PROX_OK;
  }
  e = launch_fill_zero(hist_dev, static_cast<size_t>(nb) * sizeof(uint32_t), s);
  if (e != hipSuccess) return hip_fail(e, "histogram clear");
  e = launch_bin_hist(samples, m, w, nb, hist_dev, s);
  if (e != hipSuccess) return hip_fail(e, "histogram launch");
  std::vector<uint32_t> hist(static_cast<size_t>(nb));
  e = hipMemcpyAsync(hist.data(), hist_dev, static_cast<size_t>(nb) * sizeof(uint32_t), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return hip_fail(e, "histogram copy");
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "calibration synchronisation");
  uint64_t cum = 0;
  for (int b = nb - 1; b >= 0; --b) {
    cum += hist[b];
    if (cum >= keep_n) {
      *out = static_cast<float>(b) * w;
      return PROX_OK;
    }
  }
  *out = 0.f;
  return PROX_OK;
}

// s~ of every calibration token under tau_x into s_all ([n_tokens][f] fp32),
// in chunks of kCalChunk tokens on the workspace slice tws.
prox_status proxy_state_all(const Plan& p, const prox_layer* layer, const void* X_cal, int32_t n_tokens,
                            float tau_x, float* s_all, uint8_t* tws, hipStream_t s) {
  const int chunk = std::min<int32_t>(n_tokens, kCalChunk);
  const size_t es = elem_size(layer->wdtype);
  for (int t0 = 0; t0 < n_tokens; t0 += chunk) {
    const int nb = std::min(chunk, n_tokens - t0);
    const void* xt = static_cast<const uint8_t*>(X_cal) + static_cast<size_t>(t0) * p.d * es;
    const hipError_t e = launch_stage1(stage1_args(p, layer, xt, tau_x, INFINITY, tws,
                                                   s_all + static_cast<size_t>(t0) * p.f, nullptr),
                                       layer->wdtype, nb, true, s);
    if (e != hipSuccess) return hip_fail(e, "stage-1 launch (calibration)");
  }
  return PROX_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
int proxy_row_stride(int f) { return ((f / 128) % 2 == 1) ? f : f + 128; }
int proxy16_row_stride(int f) { return ((4 * f / 128) % 2 == 1) ? 4 * f : 4 * f + 128; }

// Row groups of the down kernel for a launch over `tokens` tokens (the grid
// is column slices x row groups x tokens).  One token: at most
// kDownTargetBlocks blocks of 16 waves, two per CU (the kernel needs ~55
// VGPRs, so two 1024-thread blocks are resident at once); measured on the
// Qwen3-32B-shaped layer: ~256 blocks 19.6 us, ~384 18.2 us, ~512 16.7 us, the
// Qwen3-8B-shaped layer unchanged (8.2 us).  Two or more tokens: half that per
// token (two tokens then fill the same two blocks per CU; with the one-token
// target they ran in two rounds, 36.8 against 34.9 us for Stage 2 of two 8B
// tokens).
DownGroups down_groups(const Plan& p, int tokens) {
  const int f = p.f;
  const int cw = 64 * (16 / static_cast<int>(elem_size(p.wdtype)));
  const int target = tokens <= 1 ? kDownTargetBlocks : kDownTargetBlocks / 2;
  int rg = std::max(1, target / p.dn_col_slices);
  rg = std::max(1, std::min(f / 16, rg));
  // LDS per block: the 16 waves' partial rows plus (index, s) per row of the group
  const int red_bytes = (kDownThreads / 64) * cw * 4;
  const int max_rows_cap = (61440 - red_bytes) / 8;
  rg = std::max(rg, (f + max_rows_cap - 1) / max_rows_cap);
  // decode mode: a row group is a channel range of at most one channel per thread
  rg = std::max(rg, (f + kDownThreads - 1) / kDownThreads);
  DownGroups g;
  g.chan_per_group = ((f + rg - 1) / rg + 31) / 32 * 32;
  g.row_groups = (f + g.chan_per_group - 1) / g.chan_per_group;
  g.max_rows = std::max((f + g.row_groups - 1) / g.row_groups, g.chan_per_group);
  return g;
}

Plan make_plan(int d, int f, int wdtype) {
  Plan p;
  p.d = d;
  p.f = f;
  p.wdtype = wdtype;
  p.proxy_stride = proxy_row_stride(f);
  p.proxy16_stride = proxy16_row_stride(f);
  // 128-column panels: wider panels gather faster but double the split
  // partials and the last block's reduction, which costs more than it saves
  p.panel = 128;
  p.n_panels = f / p.panel;
  // Stage 1: at least about three 256-thread blocks per CU over 256 CUs, and
  // at most kS1MaxRowsPerSplit input rows per split, so that at keep 1/2 a
  // wave's share of the kept rows (a quarter of the split) fits one 128-row
  // gather batch: a second batch is a second round trip (measured on the
  // Qwen3-32B-shaped layer: 4 splits 20.4 us, 6 splits 18.6 us)
  const int target = 768;
  int splits = std::max((target + p.n_panels - 1) / p.n_panels, (d + kS1MaxRowsPerSplit - 1) / kS1MaxRowsPerSplit);
  splits = std::max(1, std::min(64, splits));
  int rps = (d + splits - 1) / splits;
  rps = (rps + 63) / 64 * 64;
  rps = std::min(rps, 2048);  // bounds the LDS list of kept rows (20 B per row)
  p.rows_per_split = rps;
  p.splits = (d + rps - 1) / rps;
  {  // up/gate: about one wave per 3 channels (at least 256 waves), in whole
     // rounds of kUgResidentBlocks (the blocks resident at once: the kernel
     // needs ~126 VGPRs, so four 4-wave blocks per CU): a partial last round
     // pays the prologue again for a few blocks (Qwen3-32B-shaped layer: 2133
     // blocks 32.1 us, 2048 31.7 us)
    const int wpb = kUgThreads / 64;
    p.ug_blocks = std::max(256 / wpb, f / (3 * wpb));
    if (p.ug_blocks > kUgResidentBlocks) p.ug_blocks = p.ug_blocks / kUgResidentBlocks * kUgResidentBlocks;
  }
  // down: column slices of one wave-load; row groups per launch (down_groups)
  const int cw = 64 * (16 / static_cast<int>(elem_size(wdtype)));
  p.dn_col_slices = (d + cw - 1) / cw;
  {
    const DownGroups g = down_groups(p, 1);
    p.dn_row_groups = g.row_groups;
    p.dn_chan_per_group = g.chan_per_group;
    p.dn_max_rows = g.max_rows;
  }
  // batched down: 512-column slices, about 256 blocks; a group holds at most
  // 2048 union ordinals (LDS)
  p.dnb_col_slices = (d + 511) / 512;
  int gb = (256 + p.dnb_col_slices - 1) / p.dnb_col_slices;
  gb = std::max(gb, (f + 2047) / 2048);
  gb = std::max(1, std::min({gb, f / 32, 64}));  // at most 64 groups: the reduction holds one value per group
  p.dnb_groups = gb;
  p.dnb_max_rows = ((f + gb - 1) / gb + 31) / 32 * 32;
  // fused Stage 2 (batch 1): the same column slices, about kFusedItems items
  // (one per block of the grid), a row group at most one channel per thread;
  // LDS: max(x, the 16 waves' partial rows) + (index, s) per row
  p.fz_col_slices = p.dn_col_slices;
  {
    int frg = std::max(1, kFusedItems / p.fz_col_slices);
    frg = std::max(frg, (f + kFusedThreads - 1) / kFusedThreads);
    p.fz_chan_per_group = ((f + frg - 1) / frg + 31) / 32 * 32;
    p.fz_row_groups = (f + p.fz_chan_per_group - 1) / p.fz_chan_per_group;
    p.fz_max_rows = p.fz_chan_per_group;
    const int fz_red = (kFusedThreads / 64) * cw * 4;
    const int x_bytes = d * static_cast<int>(elem_size(wdtype));
    p.fz_red_bytes = (std::max(fz_red, x_bytes) + 15) / 16 * 16;
  }
  // per-token workspace slice
  size_t off = 0;
  p.off_err = off;       // error word of the bounded waits
  p.off_done = off + 4;  // completion ticket of the fused Stage-2 kernel
  off = align256(off + 8);
  p.off_flags = off;  // grid-barrier flags of the fused Stage-2 kernel
  off = align256(off + static_cast<size_t>(kMaxGridFlags) * 4);
  p.off_tickets = off;
  off = align256(off + static_cast<size_t>(p.n_panels) * 4);
  p.off_kcount = off;
  off = align256(off + static_cast<size_t>(p.splits) * 4);
  p.off_partial = off;
  off = align256(off + static_cast<size_t>(p.splits) * 2 * f * 4);
  p.off_bitmap = off;
  off = align256(off + static_cast<size_t>(f / 32) * 4);
  p.off_ssp = off;
  off = align256(off + static_cast<size_t>(f) * 4);
  p.off_ulist = off;
  off = align256(off + static_cast<size_t>(f + 64) * 4);
  p.off_arows = off;
  off = align256(off + static_cast<size_t>(f) * 16 * 2);
  p.off_dpart = off;
  off = align256(off + static_cast<size_t>(p.dnb_groups) * d * 4);
  p.tok_bytes = off;
  return p;
}

}  // namespace prox

using namespace prox;

PROX_API int32_t prox_abi_version(void) { return PROX_ABI_VERSION; }

PROX_API const char* prox_last_error(void) { return g_err.c_str(); }

PROX_API prox_status prox_layer_sizes(int32_t d, int32_t f, int32_t wdtype, size_t* bytes_out) {
  try {
    g_err.clear();
    if (!bytes_out) return fail(PROX_ERR_INVALID_ARG, "bytes_out is NULL");
    prox_status st = check_shape(d, f, wdtype);
    if (st != PROX_OK) return st;
    const size_t es = elem_size(wdtype);
    bytes_out[0] = static_cast<size_t>(d) * proxy_row_stride(f);
    bytes_out[1] = static_cast<size_t>(2) * d * sizeof(float);
    bytes_out[2] = static_cast<size_t>(2) * f * d * es;
    bytes_out[3] = static_cast<size_t>(f) * d * es;
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_workspace_size(int32_t d, int32_t f, int32_t batch, size_t* bytes) {
  try {
    g_err.clear();
    if (!bytes) return fail(PROX_ERR_INVALID_ARG, "bytes is NULL");
    prox_status st = check_shape(d, f, PROX_BF16);
    if (st != PROX_OK) return st;
    if ((st = check_batch(batch)) != PROX_OK) return st;
    // the layout does not depend on the weight dtype
    *bytes = make_plan(d, f, PROX_BF16).tok_bytes * static_cast<size_t>(batch);
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_calibrate_workspace_size(int32_t d, int32_t f, int32_t n_tokens,
                                                   size_t* bytes) {
  try {
    g_err.clear();
    if (!bytes) return fail(PROX_ERR_INVALID_ARG, "bytes is NULL");
    prox_status st = check_shape(d, f, PROX_BF16);
    if (st != PROX_OK) return st;
    if (n_tokens < 1 || n_tokens > 65536)
      return fail(PROX_ERR_INVALID_ARG, "n_tokens %d outside [1, 65536]", n_tokens);
    *bytes = calib_bytes(make_plan(d, f, PROX_BF16), n_tokens);
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

namespace {
prox_status check_budget_args(float a, float b, float alpha) {
  if (!(a >= 0.f && a <= 1.f) || !(b >= 0.f && b <= 1.f))
    return fail(PROX_ERR_INVALID_ARG, "sparsities must lie in [0, 1]");
  if (!(alpha > 0.f) || std::isinf(alpha))
    return fail(PROX_ERR_INVALID_ARG, "alpha = %g must be finite and > 0", static_cast<double>(alpha));
  return PROX_OK;
}
}  // namespace

PROX_API prox_status prox_budget_effective(float s1, float s2, float alpha, float* e_out) {
  g_err.clear();
  if (!e_out) return fail(PROX_ERR_INVALID_ARG, "e_out is NULL");
  const prox_status st = check_budget_args(s1, s2, alpha);
  if (st != PROX_OK) return st;
  const double cost = 2.0 * alpha * (1.0 - static_cast<double>(s1)) + 3.0 * (1.0 - static_cast<double>(s2));
  *e_out = static_cast<float>(1.0 - cost / 3.0);
  return PROX_OK;
}

PROX_API prox_status prox_budget_s2(float e_target, float s1, float alpha, float* s2_out) {
  g_err.clear();
  if (!s2_out) return fail(PROX_ERR_INVALID_ARG, "s2_out is NULL");
  const prox_status st = check_budget_args(e_target, s1, alpha);
  if (st != PROX_OK) return st;
  const double s2 = static_cast<double>(e_target) + 2.0 * alpha * (1.0 - static_cast<double>(s1)) / 3.0;
  if (s2 > 1.0)
    return fail(PROX_ERR_UNSUPPORTED, "effective sparsity %g is out of reach at s1 = %g, alpha = %g (needs s2 = %g)",
                static_cast<double>(e_target), static_cast<double>(s1), static_cast<double>(alpha), s2);
  *s2_out = static_cast<float>(s2);
  return PROX_OK;
}

PROX_API prox_status prox_calibrate_hist_workspace_size(int32_t d, int32_t f, int32_t n_tokens,
                                                        int32_t max_samples, int32_t n_bins, size_t* bytes) {
  try {
    g_err.clear();
    if (!bytes) return fail(PROX_ERR_INVALID_ARG, "bytes is NULL");
    prox_status st = check_shape(d, f, PROX_BF16);
    if (st != PROX_OK) return st;
    if (n_tokens < 1 || n_tokens > 65536)
      return fail(PROX_ERR_INVALID_ARG, "n_tokens %d outside [1, 65536]", n_tokens);
    if (max_samples < 1 || static_cast<uint32_t>(max_samples) > kMaxHistSamples || n_bins < 2 ||
        n_bins > kMaxHistBins)
      return fail(PROX_ERR_INVALID_ARG, "max_samples %d outside [1, %u] or n_bins %d outside [2, %d]", max_samples,
                  kMaxHistSamples, n_bins, kMaxHistBins);
    *bytes = calib_hist_bytes(make_plan(d, f, PROX_BF16), n_tokens, static_cast<uint32_t>(max_samples), n_bins);
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_calibrate_hist(const prox_layer* layer, const void* X_cal, int32_t n_tokens,
                                         float keep_x, float sparsity_s, int32_t max_samples, int32_t n_bins,
                                         float* tau_x, float* tau_s, void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    prox_status st = check_layer(layer);
    if (st != PROX_OK) return st;
    if (!X_cal || !tau_x || !tau_s) return fail(PROX_ERR_INVALID_ARG, "X_cal, tau_x, tau_s must be non-NULL");
    if (!aligned(X_cal, 16)) return fail(PROX_ERR_INVALID_ARG, "X_cal must be 16-byte aligned");
    if (n_tokens < 1 || n_tokens > 65536)
      return fail(PROX_ERR_INVALID_ARG, "n_tokens %d outside [1, 65536]", n_tokens);
    if (!(keep_x >= 0.f && keep_x <= 1.f) || !(sparsity_s >= 0.f && sparsity_s <= 1.f))
      return fail(PROX_ERR_INVALID_ARG, "keep_x and sparsity_s must lie in [0, 1]");
    if (max_samples < 1 || static_cast<uint32_t>(max_samples) > kMaxHistSamples || n_bins < 2 ||
        n_bins > kMaxHistBins)
      return fail(PROX_ERR_INVALID_ARG, "max_samples %d outside [1, %u] or n_bins %d outside [2, %d]", max_samples,
                  kMaxHistSamples, n_bins, kMaxHistBins);
    const Plan p = make_plan(layer->d_model, layer->d_ff, layer->wdtype);
    if (!ws || !aligned(ws, 256)) return fail(PROX_ERR_INVALID_ARG, "workspace NULL or not 256-byte aligned");
    const size_t need = calib_hist_bytes(p, n_tokens, static_cast<uint32_t>(max_samples), n_bins);
    if (ws_bytes < need)
      return fail(PROX_ERR_INVALID_ARG, "calibration workspace of %zu bytes is smaller than the %zu needed",
                  ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* base = static_cast<uint8_t*>(ws);
    float* s_all = reinterpret_cast<float*>(base);
    uint8_t* tws = base + align256(static_cast<size_t>(n_tokens) * p.f * sizeof(float));
    const int chunk = std::min<int32_t>(n_tokens, kCalChunk);
    float* samples = reinterpret_cast<float*>(base + calib_bytes(p, n_tokens));
    uint32_t* hist = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(samples) +
                                                 align256(static_cast<size_t>(max_samples) * sizeof(float)));
    uint32_t* maxw = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(hist) +
                                                 align256(static_cast<size_t>(n_bins) * sizeof(uint32_t)));
    hipError_t e = launch_fill_zero(tws, p.tok_bytes * chunk, s);
    if (e != hipSuccess) return hip_fail(e, "workspace fill");
    float tx = 0.f;
    st = hist_threshold(X_cal, static_cast<uint64_t>(n_tokens) * p.d, layer->wdtype, static_cast<double>(keep_x),
                        static_cast<uint32_t>(max_samples), n_bins, samples, hist, maxw, s, &tx);
    if (st != PROX_OK) return st;
    if ((st = proxy_state_all(p, layer, X_cal, n_tokens, tx, s_all, tws, s)) != PROX_OK) return st;
    float ts = 0.f;
    st = hist_threshold(s_all, static_cast<uint64_t>(n_tokens) * p.f, PROX_F32, 1.0 - static_cast<double>(sparsity_s),
                        static_cast<uint32_t>(max_samples), n_bins, samples, hist, maxw, s, &ts);
    if (st != PROX_OK) return st;
    *tau_x = tx;
    *tau_s = ts;
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    if (!ws) return fail(PROX_ERR_INVALID_ARG, "workspace is NULL");
    if (!aligned(ws, 4)) return fail(PROX_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
    hipError_t e = launch_fill_zero(ws, ws_bytes, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "workspace fill");
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_proxy_qt_size(int32_t d, int32_t f, size_t* bytes) {
  try {
    g_err.clear();
    if (!bytes) return fail(PROX_ERR_INVALID_ARG, "bytes is NULL");
    prox_status st = check_shape(d, f, PROX_BF16);
    if (st != PROX_OK) return st;
    *bytes = proxy_qt_bytes(d, f);
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_pack_proxy_qt(const prox_layer* layer, void* stream) {
  try {
    g_err.clear();
    prox_status st = check_layer(layer);
    if (st != PROX_OK) return st;
    if (layer->proxy_kind != PROX_PROXY_INT4)
      return fail(PROX_ERR_UNSUPPORTED, "the channel-major copy is of the INT4 proxy (PROX_PROXY_INT4 layers)");
    if (!layer->proxy_qt) return fail(PROX_ERR_INVALID_ARG, "layer->proxy_qt is NULL");
    const hipError_t e = launch_pack_qt(static_cast<const uint8_t*>(layer->proxy_q), proxy_row_stride(layer->d_ff),
                                        layer->d_model, layer->d_ff, static_cast<uint8_t*>(layer->proxy_qt),
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pack_qt launch");
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_proxy16_size(int32_t d, int32_t f, int32_t wdtype, size_t* bytes) {
  try {
    g_err.clear();
    if (!bytes) return fail(PROX_ERR_INVALID_ARG, "bytes is NULL");
    prox_status st = check_shape(d, f, wdtype);
    if (st != PROX_OK) return st;
    if (wdtype != PROX_BF16) return fail(PROX_ERR_UNSUPPORTED, "the 16-bit proxy is for bf16 layers");
    *bytes = static_cast<size_t>(d) * proxy16_row_stride(f);
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_pack_proxy16(const void* W_up, const void* W_gate, const prox_layer* out, void* stream) {
  try {
    g_err.clear();
    if (out == nullptr) return fail(PROX_ERR_INVALID_ARG, "layer descriptor is NULL");
    prox_status st = check_shape(out->d_model, out->d_ff, out->wdtype);
    if (st != PROX_OK) return st;
    if (out->wdtype != PROX_BF16) return fail(PROX_ERR_UNSUPPORTED, "the 16-bit proxy is for bf16 layers");
    if (!out->proxy_w16 || !aligned(out->proxy_w16, 16))
      return fail(PROX_ERR_INVALID_ARG, "out->proxy_w16 must be non-NULL and 16-byte aligned");
    if (!W_up || !W_gate) return fail(PROX_ERR_INVALID_ARG, "input weight pointer is NULL");
    if (!aligned(W_up, 16) || !aligned(W_gate, 16))
      return fail(PROX_ERR_INVALID_ARG, "input weights must be 16-byte aligned");
    const hipError_t e = launch_pack16(W_up, W_gate, out->d_model, out->d_ff, proxy16_row_stride(out->d_ff),
                                       out->proxy_w16, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "pack16 launch");
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_pack_proxy(const void* W_up, const void* W_gate, const void* W_down,
                                     const prox_layer* out, void* stream) {
  try {
    g_err.clear();
    prox_status st = check_layer(out);
    if (st != PROX_OK) return st;
    if (!out->proxy_q || !out->proxy_scale)
      return fail(PROX_ERR_INVALID_ARG, "out->proxy_q and out->proxy_scale receive the INT4 proxy: non-NULL");
    if (!W_up || !W_gate || !W_down) return fail(PROX_ERR_INVALID_ARG, "input weight pointer is NULL");
    if (!aligned(W_up, 16) || !aligned(W_gate, 16) || !aligned(W_down, 16))
      return fail(PROX_ERR_INVALID_ARG, "input weights must be 16-byte aligned");
    const int d = out->d_model, f = out->d_ff;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_pack(W_up, W_gate, d, f, proxy_row_stride(f), out->wdtype,
                               static_cast<uint8_t*>(out->proxy_q),
                               out->proxy_scale, out->w_upgate_t, s);
    if (e != hipSuccess) return hip_fail(e, "pack launch");
    if (out->w_down != W_down) {
      e = hipMemcpyAsync(out->w_down, W_down, static_cast<size_t>(f) * d * elem_size(out->wdtype),
                         hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "W_down copy");
    }
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_calibrate(const prox_layer* layer, const void* X_cal, int32_t n_tokens,
                                    float keep_x, float sparsity_s, float* tau_x, float* tau_s,
                                    void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    prox_status st = check_layer(layer);
    if (st != PROX_OK) return st;
    if (!X_cal || !tau_x || !tau_s) return fail(PROX_ERR_INVALID_ARG, "X_cal, tau_x, tau_s must be non-NULL");
    if (!aligned(X_cal, 16)) return fail(PROX_ERR_INVALID_ARG, "X_cal must be 16-byte aligned");
    if (n_tokens < 1 || n_tokens > 65536)
      return fail(PROX_ERR_INVALID_ARG, "n_tokens %d outside [1, 65536]", n_tokens);
    if (!(keep_x >= 0.f && keep_x <= 1.f) || !(sparsity_s >= 0.f && sparsity_s <= 1.f))
      return fail(PROX_ERR_INVALID_ARG, "keep_x and sparsity_s must lie in [0, 1]");
    const Plan p = make_plan(layer->d_model, layer->d_ff, layer->wdtype);
    if (!ws || !aligned(ws, 256)) return fail(PROX_ERR_INVALID_ARG, "workspace NULL or not 256-byte aligned");
    const size_t need = calib_bytes(p, n_tokens);
    if (ws_bytes < need)
      return fail(PROX_ERR_INVALID_ARG, "calibration workspace of %zu bytes is smaller than the %zu needed",
                  ws_bytes, need);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* base = static_cast<uint8_t*>(ws);
    float* s_all = reinterpret_cast<float*>(base);
    uint8_t* tws = base + align256(static_cast<size_t>(n_tokens) * p.f * sizeof(float));
    const int chunk = std::min<int32_t>(n_tokens, kCalChunk);
    uint32_t* hist = reinterpret_cast<uint32_t*>(tws + p.tok_bytes * chunk);
    hipError_t e = launch_fill_zero(tws, p.tok_bytes * chunk, s);
    if (e != hipSuccess) return hip_fail(e, "workspace fill");

    const uint64_t nx = static_cast<uint64_t>(n_tokens) * p.d;
    float tx = 0.f;
    st = select_kth_largest(X_cal, nx, layer->wdtype, keep_count(static_cast<double>(keep_x), nx), hist,
                            s, &tx);
    if (st != PROX_OK) return st;

    const size_t es = elem_size(layer->wdtype);
    for (int t0 = 0; t0 < n_tokens; t0 += chunk) {
      const int nb = std::min(chunk, n_tokens - t0);
      const void* xt = static_cast<const uint8_t*>(X_cal) + static_cast<size_t>(t0) * p.d * es;
      e = launch_stage1(stage1_args(p, layer, xt, tx, INFINITY, tws, s_all + static_cast<size_t>(t0) * p.f,
                                    nullptr),
                        layer->wdtype, nb, true, s);
      if (e != hipSuccess) return hip_fail(e, "stage-1 launch (calibration)");
    }
    const uint64_t ns = static_cast<uint64_t>(n_tokens) * p.f;
    const double keep_s = 1.0 - static_cast<double>(sparsity_s);
    float ts = 0.f;
    st = select_kth_largest(s_all, ns, PROX_F32, keep_count(keep_s, ns), hist, s, &ts);
    if (st != PROX_OK) return st;
    *tau_x = tx;
    *tau_s = ts;
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_ffn_decode(const prox_layer* layer, const void* x, int32_t batch, float tau_x,
                                     float tau_s, float* y, int32_t* mask_idx, int32_t* mask_count,
                                     int32_t* in_count, void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    return decode_impl(layer, x, batch, tau_x, tau_s, y, mask_idx, mask_count, in_count, ws, ws_bytes,
                       stream, nullptr);
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_ffn_decode_events(const prox_layer* layer, const void* x, int32_t batch,
                                            float tau_x, float tau_s, float* y, int32_t* mask_idx,
                                            int32_t* mask_count, int32_t* in_count, void* ws,
                                            size_t ws_bytes, void* stream, void* const* events) {
  try {
    g_err.clear();
    if (!events) return fail(PROX_ERR_INVALID_ARG, "events is NULL");
    return decode_impl(layer, x, batch, tau_x, tau_s, y, mask_idx, mask_count, in_count, ws, ws_bytes,
                       stream, events);
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_ffn_decode_stages(const prox_layer* layer, const void* x, int32_t batch,
                                            float tau_x, float tau_s, float* y, int32_t* mask_idx,
                                            int32_t* mask_count, int32_t* in_count, void* ws,
                                            size_t ws_bytes, void* stream, int32_t stages) {
  try {
    g_err.clear();
    return decode_impl(layer, x, batch, tau_x, tau_s, y, mask_idx, mask_count, in_count, ws, ws_bytes,
                       stream, nullptr, stages);
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_ffn_stage2(const prox_layer* layer, const void* x, int32_t batch,
                                     const int32_t* mask_idx, const int32_t* mask_count, float* y,
                                     void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    prox_status st = check_layer(layer);
    if (st != PROX_OK) return st;
    if ((st = check_batch(batch)) != PROX_OK) return st;
    if (!x || !y || !mask_idx || !mask_count)
      return fail(PROX_ERR_INVALID_ARG, "x, y, mask_idx and mask_count must be non-NULL");
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(mask_idx, 4) || !aligned(mask_count, 4))
      return fail(PROX_ERR_INVALID_ARG, "x and y must be 16-byte aligned, index buffers 4-byte aligned");
    const Plan p = make_plan(layer->d_model, layer->d_ff, layer->wdtype);
    if ((st = check_ws(p, batch, ws, ws_bytes)) != PROX_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int* mi = const_cast<int*>(mask_idx);   // read only in list mode
    int* mc = const_cast<int*>(mask_count);
    hipError_t e = launch_upgate(upgate_args(p, layer, x, ws, mi, mc, y), layer->wdtype, batch,
                                 p.ug_blocks, false, s);
    if (e != hipSuccess) return hip_fail(e, "stage-2 up/gate launch");
    e = launch_down(down_args(p, layer, ws, mask_idx, mask_count, y, batch), layer->wdtype, batch, false, s);
    if (e != hipSuccess) return hip_fail(e, "stage-2 down launch");
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_proxy_state(const prox_layer* layer, const void* x, int32_t batch, float tau_x,
                                      float* s_tilde, int32_t* in_count, void* ws, size_t ws_bytes,
                                      void* stream) {
  try {
    g_err.clear();
    prox_status st = check_layer(layer);
    if (st != PROX_OK) return st;
    if ((st = check_batch(batch)) != PROX_OK) return st;
    if ((st = check_tau(tau_x, "tau_x")) != PROX_OK) return st;
    if (!x || !s_tilde) return fail(PROX_ERR_INVALID_ARG, "x and s_tilde must be non-NULL");
    if (!aligned(x, 16) || !aligned(s_tilde, 4) || (in_count && !aligned(in_count, 4)))
      return fail(PROX_ERR_INVALID_ARG, "x must be 16-byte aligned, outputs 4-byte aligned");
    const Plan p = make_plan(layer->d_model, layer->d_ff, layer->wdtype);
    if ((st = check_ws(p, batch, ws, ws_bytes)) != PROX_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (batch >= 2 && layer->proxy_kind == PROX_PROXY_INT4) {  // per group, as prox_ffn_decode runs it
      const size_t es = elem_size(layer->wdtype);
      e = for_each_group(batch, [&](int g0, int nt) {
        Stage1Args a1 = stage1_args(p, layer, static_cast<const uint8_t*>(x) + static_cast<size_t>(g0) * p.d * es,
                                    tau_x, INFINITY, static_cast<uint8_t*>(ws) + static_cast<size_t>(g0) * p.tok_bytes,
                                    s_tilde + static_cast<size_t>(g0) * p.f, in_count ? in_count + g0 : nullptr);
        if (layer->proxy_qt != nullptr && nt >= kGroupedMinTokens && qt_usable(p, layer, nt))
          return launch_stage1_qt(qt_args(p, layer, a1.x, tau_x, INFINITY, a1.ws, a1.s_tilde, a1.in_count, nt),
                                  layer->wdtype, true, s);
        if (nt < kGroupedMinTokens) return launch_stage1(a1, layer->wdtype, nt, true, s);
        a1.nt = nt;
        return launch_stage1_batch(a1, layer->wdtype, true, s);
      });
    } else {
      e = launch_stage1(stage1_args(p, layer, x, tau_x, INFINITY, ws, s_tilde, in_count), layer->wdtype, batch,
                        true, s);
    }
    if (e != hipSuccess) return hip_fail(e, "stage-1 launch");
    return PROX_OK;
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

// ---------------------------------------------------------------------------
// Allocation-free decode.  The workspace is the file-scope device array
// `scratch` (one copy per GPU, held until the process ends).  In host code the
// array's name is only a handle for hipGetSymbolAddress: the device address
// of each GPU's copy is looked up once per device, with that device current,
// and only that address is passed to kernels and fills.
namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(32) << 20;  // PROX_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == PROX_NOALLOC_SCRATCH_BYTES, "scratch size and header disagree");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

// Per device: the address of its scratch copy and the layout (shape, tokens)
// whose must-be-zero words (the Stage-1 tickets) are known to be zero.
struct ScratchState {
  uint8_t* ptr = nullptr;
  int d = 0, f = 0, batch = 0;
};
std::mutex g_scratch_mu;
std::vector<ScratchState> g_scratch;

}  // namespace

PROX_API prox_status prox_ffn_decode_noalloc(const prox_layer* layer, const void* x, int32_t batch, float tau_x,
                                             float tau_s, float* y, int32_t* mask_idx, int32_t* mask_count,
                                             int32_t* in_count, void* stream) {
  try {
    g_err.clear();
    prox_status st = check_decode_args(layer, x, batch, tau_x, tau_s, y, mask_idx, mask_count, in_count);
    if (st != PROX_OK) return st;
    const Plan p = make_plan(layer->d_model, layer->d_ff, layer->wdtype);
    const size_t need = p.tok_bytes * static_cast<size_t>(batch);
    if (need > kScratchBytes)
      return fail(PROX_ERR_UNSUPPORTED,
                  "d_model=%d d_ff=%d batch=%d needs %zu bytes of scratch, above the %zu bytes the allocation-free "
                  "entry point holds per GPU (use prox_ffn_decode with a workspace)",
                  layer->d_model, layer->d_ff, batch, need, kScratchBytes);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0) return fail(PROX_ERR_INTERNAL, "hipGetDevice returned %d", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch.size() <= static_cast<size_t>(dev)) g_scratch.resize(static_cast<size_t>(dev) + 1);
    ScratchState& sc = g_scratch[static_cast<size_t>(dev)];
    if (sc.ptr == nullptr) {  // once per device, with that device current
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (addr == nullptr) return fail(PROX_ERR_INTERNAL, "hipGetSymbolAddress(scratch) gave NULL");
      sc.ptr = static_cast<uint8_t*>(addr);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Every completed call leaves its tickets at zero; another shape moves the
    // token slices (and their tickets) onto bytes that held other data, and a
    // larger batch reaches slices not used before: clear the region then.  The
    // slice size and offsets make_plan computes depend on d_model and d_ff
    // only (no term in the weight type or proxy kind), so those and the batch
    // are the key.
    // (A fill kernel, not a memset, so a captured call replays correctly.)
    if (sc.d != layer->d_model || sc.f != layer->d_ff || batch > sc.batch) {
      e = launch_fill_zero(sc.ptr, need, s);
      if (e != hipSuccess) return hip_fail(e, "scratch fill");
      sc.d = layer->d_model;
      sc.f = layer->d_ff;
      sc.batch = batch;
    }
    return decode_impl(layer, x, batch, tau_x, tau_s, y, mask_idx, mask_count, in_count, sc.ptr, kScratchBytes,
                       stream, nullptr);
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_workspace_check(const void* ws, size_t ws_bytes, void* stream) {
  try {
    g_err.clear();
    if (!ws || !aligned(ws, 256)) return fail(PROX_ERR_INVALID_ARG, "workspace NULL or not 256-byte aligned");
    if (ws_bytes < 4) return fail(PROX_ERR_INVALID_ARG, "workspace of %zu bytes holds no error word", ws_bytes);
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t word = 0;
    hipError_t e = hipMemcpyAsync(&word, ws, sizeof(word), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "error word copy");
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "workspace check synchronisation");
    if (word == 0u) return PROX_OK;
    e = launch_fill_zero(const_cast<void*>(ws), sizeof(word), s);
    if (e != hipSuccess) return hip_fail(e, "error word clear");
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "workspace check synchronisation");
    return fail(PROX_ERR_INTERNAL,
                "a decode on this workspace gave up waiting at the fused Stage-2 grid barrier (error word 0x%x): "
                "its blocks were not all resident within the wait limit; its y was not computed", word);
  } catch (...) {
    return fail(PROX_ERR_INTERNAL, "unexpected exception");
  }
}

PROX_API prox_status prox_set_wait_limit(uint32_t ticks, uint32_t* previous) {
  g_err.clear();
  const uint32_t old = g_wait_ticks.exchange(ticks);
  if (previous) *previous = old;
  return PROX_OK;
}
