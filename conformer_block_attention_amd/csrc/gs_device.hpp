// gs_device.hpp -- gfx950 (CDNA4) device helpers shared by the libgsattn kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gs {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define GS_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float f) { return (bf16)f; }

__device__ __forceinline__ float to_f32(bf16 b) { return (float)b; }

// 16-byte asynchronous copy global -> LDS.  Every lane of the wave provides
// its own global address; lane i's 16 bytes land at lds_wave_base + 16*i.
// lds_wave_base must be wave-uniform.
__device__ __forceinline__ void copy16_to_lds(const void* gsrc, GS_LDS void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_wave_base, 16, 0, 0);
}

// Wait until all of this wave's outstanding vector-memory loads (including
// the LDS-direct copies above) have completed.
// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8.  0x0F70 = vmcnt(0) with the other two counters at max.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// lgkmcnt(0) with vmcnt and expcnt at max: this wave's LDS reads have landed.
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Raw buffer resource over [base, base + bytes) (stride 0; gfx9 word 3).
// Accesses through it are range-checked by the hardware: a load past the end
// returns zero and a store past the end is dropped, while the instruction
// still issues for the whole wave (so it counts in vmcnt like any other).
// base and bytes must be wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

}  // namespace gs
