// Shared device-side definitions of the HIP path (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (gfx950 converts in
// hardware: v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <typename T>
struct ElemSize;
template <>
struct ElemSize<uint16_t> {
  static constexpr int value = 2;
};
template <>
struct ElemSize<float> {
  static constexpr int value = 4;
};

__host__ __device__ constexpr int ceil_div(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// s_waitcnt with vmcnt = n (other counters left at their maximum): gfx9
// encoding, vmcnt split over bits 3:0 and 15:14.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// One 16-byte global -> LDS transfer per lane (global_load_lds_dwordx4):
// lane i writes lds_wave + 16 i, where lds_wave is the same for the wave.
// STREAM marks the load non-temporal (data read once: weights that no other
// tile of the launch reads again).
template <bool STREAM = false>
__device__ __forceinline__ void lds_dma16(const unsigned char* src, unsigned char* lds_run) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_run, 16, 0, STREAM ? 2 : 0);
}

}  // namespace moe
