// Device-side helpers for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prox {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
// 16 bytes as a native vector: whole-value copies stay in registers (copies of
// the HIP uint4 struct can be left in private memory)
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

// Weight / activation element types.  bf16 values travel as raw 16-bit
// patterns; fp32 as float.
struct Bf16Tag { typedef uint16_t storage; };
struct F32Tag { typedef float storage; };

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <typename T> __device__ __forceinline__ float load_elem(const void* p, size_t i);
template <> __device__ __forceinline__ float load_elem<Bf16Tag>(const void* p, size_t i) {
  return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float load_elem<F32Tag>(const void* p, size_t i) {
  return static_cast<const float*>(p)[i];
}

// 16-byte global load.
__device__ __forceinline__ uint4 ldg16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// 16-byte global load with the non-temporal hint (global_load_dwordx4 ... nt),
// for weight streams that one launch reads exactly once per address: the
// lines are not kept as recently used in L2 and the Infinity Cache.  Measured
// on MI355X (graph-replayed, one token per launch): the up/gate kernel 13.43
// -> 12.15 us on the Qwen3-8B-shaped layer and 31.7 -> 28.9 us on the
// Qwen3-32B-shaped one, Stage 1 10.45 -> 10.22 us.  Loads that re-read an
// address within the launch stay on ldg16: with the hint each re-read went
// to memory again (the down kernel's batch slots past the list end, when they
// re-read its last row: 8.16 -> 9.32 us; per-token kernels over 8 tokens,
// whose kept rows and channels overlap: 144.5 -> 155.9 us per step).  The
// down kernels instead point such slots past their buffer's records.
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ u32x4_t ldg16v_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
// A weight matrix of rows x cols elements of es bytes (below 4 GiB for every
// supported shape) as a raw buffer resource.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t weight_rsrc(const void* w, int rows, int cols, int es) {
  const uint32_t bytes = static_cast<uint32_t>(rows) * static_cast<uint32_t>(cols) * static_cast<uint32_t>(es);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(w), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000 /* raw buffer, 32-bit data */);
}
// An offset past the records of every weight_rsrc buffer: a load from it
// returns zeros without a memory access.
constexpr uint32_t kWeightOob = 0xFFFFFF00u;

// ldg16_nt for a launch over one token (kNt), ldg16 otherwise
template <bool kNt>
__device__ __forceinline__ uint4 ldg16_w(const void* p) {
  if constexpr (kNt) return ldg16_nt(p);
  else return ldg16(p);
}

// Two bf16 pairs multiplied and added into an fp32 accumulator
// (v_dot2c_f32_bf16: products exact, fp32 sum).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Dot product of 16 bytes of weights with 16 bytes of x (same element type).
template <typename T> __device__ __forceinline__ float dot16(uint4 w, uint4 x, float acc);
template <> __device__ __forceinline__ float dot16<Bf16Tag>(uint4 w, uint4 x, float acc) {
  acc = dot2_bf16(w.x, x.x, acc);
  acc = dot2_bf16(w.y, x.y, acc);
  acc = dot2_bf16(w.z, x.z, acc);
  acc = dot2_bf16(w.w, x.w, acc);
  return acc;
}
template <> __device__ __forceinline__ float dot16<F32Tag>(uint4 w, uint4 x, float acc) {
  acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
  acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
  acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
  acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
  return acc;
}

// Inclusive prefix sums over the 64 lanes of a wave with DPP (VALU only, no
// LDS round trips): row shifts by 1, 2, 4, 8 give prefix sums within each row
// of 16 lanes (a source lane outside the row reads 0), then row broadcasts of
// lane 15 and lane 31 carry the earlier rows' totals forward.
__device__ __forceinline__ float wave_inclusive_scan(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));  // row_shr:1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false));  // row_shr:2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false));  // row_shr:4
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false));  // row_shr:8
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan_int(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Sum over the 64 lanes of a wave; every lane receives the total (lane 63 of
// the inclusive scan).
__device__ __forceinline__ float wave_sum(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_inclusive_scan(v)), 63));
}

// Maximum over the 64 lanes of a wave of non-negative floats, returned to
// every lane: DPP row shifts give each row's maximum in its lane 15, two row
// broadcasts carry it to lane 63 (VALU only, no LDS round trips).  Lanes whose
// DPP source is outside the row read 0, the identity for non-negative values.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  int x = __float_as_int(v);  // non-negative floats order like their bits
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false));  // row_shr:1
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false));  // row_shr:2
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false));  // row_shr:4
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false));  // row_shr:8
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(x, 63));
}

__device__ __forceinline__ int wave_sum_int(int v) {
  return __builtin_amdgcn_readlane(wave_inclusive_scan_int(v), 63);
}

// SiLU(z) = z / (1 + e^{-z}); e^{-z} overflowing to +inf gives -0 as required.
__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// GELU in its tanh form, 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
__device__ __forceinline__ float gelu_tanh_f32(float z) {
  const float k = 0.7978845608028654f;  // sqrt(2 / pi)
  return 0.5f * z * (1.0f + tanhf(k * (z + 0.044715f * z * z * z)));
}

// The layer's gate non-linearity (prox_activation); `act` is uniform.
__device__ __forceinline__ float gate_act(float z, int act) {
  return act == 1 ? gelu_tanh_f32(z) : silu_f32(z);
}

}  // namespace prox
