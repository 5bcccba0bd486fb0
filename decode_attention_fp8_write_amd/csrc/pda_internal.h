// pda_internal.h — helpers shared by the gfx950 kernels and their host
// launchers inside libpda.so. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pda.h"

namespace pda {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Host: compute units of the current device (cached per device id).
int device_cu_count();

// Host: map the runtime's error state after a launch onto a status code.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? PDA_OK : PDA_ERR_LAUNCH;
}

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ---- device helpers ---------------------------------------------------------

__device__ __forceinline__ uint32_t as_u32(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float as_f32(uint32_t x) { return __builtin_bit_cast(float, x); }

// DPP move with a compile-time control word; lanes whose row is masked off
// keep `old`.
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF, bool BOUND_CTRL = false>
__device__ __forceinline__ float dpp_f32(float old, float src) {
  return as_f32(__builtin_amdgcn_update_dpp((int)as_u32(old), (int)as_u32(src), CTRL,
                                            ROW_MASK, BANK_MASK, BOUND_CTRL));
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)src, CTRL, 0xF, 0xF, false);
}

// DPP control words (GCN/CDNA encoding).
constexpr int DPP_QUAD_1032 = 0xB1;   // quad_perm:[1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;   // quad_perm:[2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;
constexpr int DPP_ROW_NEWBCAST0 = 0x150;  // + lane (0..15): broadcast within row

// Full-wave maximum, returned as a wave-uniform value.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<DPP_QUAD_1032>(x, x));
  x = fmaxf(x, dpp_f32<DPP_QUAD_2301>(x, x));
  x = fmaxf(x, dpp_f32<DPP_ROW_HALF_MIRROR>(x, x));
  x = fmaxf(x, dpp_f32<DPP_ROW_MIRROR>(x, x));
  x = fmaxf(x, dpp_f32<DPP_ROW_BCAST15, 0xA>(x, x));
  x = fmaxf(x, dpp_f32<DPP_ROW_BCAST31, 0xC>(x, x));
  return as_f32(__builtin_amdgcn_readlane((int)as_u32(x), 63));
}

// Full-wave sum, returned as a wave-uniform value.
__device__ __forceinline__ float wave_sum(float x) {
  x = x + dpp_f32<DPP_QUAD_1032>(0.0f, x);
  x = x + dpp_f32<DPP_QUAD_2301>(0.0f, x);
  x = x + dpp_f32<DPP_ROW_HALF_MIRROR>(0.0f, x);
  x = x + dpp_f32<DPP_ROW_MIRROR>(0.0f, x);
  x = x + dpp_f32<DPP_ROW_BCAST15, 0xA>(0.0f, x);
  x = x + dpp_f32<DPP_ROW_BCAST31, 0xC>(0.0f, x);
  return as_f32(__builtin_amdgcn_readlane((int)as_u32(x), 63));
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
  int lane = __lane_id();
  return as_f32((uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, (int)as_u32(x)));
}

}  // namespace pda
