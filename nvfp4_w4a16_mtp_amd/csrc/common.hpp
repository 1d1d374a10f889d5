// Shared device/host helpers of the NVFP4 W4A16 MTP library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_mtp.h"

namespace nvfp4 {

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// ---------------------------------------------------------------- errors --
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int ok();
// After a launch: NVFP4_OK or NVFP4_ERR_HIP with hipGetErrorString.
int check_launch(const char *what);

inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int validate_weight(const nvfp4_weight *w, const char *what);

// Number of compute units of the current device (cached per device).
int num_cus();
// Resident workgroups per CU for a kernel at a block size and dynamic LDS
// (hipOccupancyMaxActiveBlocksPerMultiprocessor, cached; at least 1).
int blocks_per_cu(const void *kernel, int block, size_t lds);
int allow_lds(const void *kernel, size_t bytes, const char *who);

// ----------------------------------------------------------- bf16 / fp32 --
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// E4M3FN byte -> fp32 (exact).  e == 0: m * 2^-9; else (1 + m/8) * 2^(e-7).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
    return (b & 0x80u) ? -mag : mag;
}

// Two E2M1 codes (the byte `sel` of `word`, low nibble first) -> two exact
// bf16 values.  The hardware conversion applies only the exponent of its
// scale operand, so the scale here is 1 and the E4M3 block scale is applied
// by the caller.
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_to_bf16(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

// acc + a.x * b.x + a.y * b.y with fp32 accumulation.
__device__ __forceinline__ float dot2(bf16x2 a, bf16x2 b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
// The butterfly order is the same for every row, so identical inputs give
// bit-identical sums wherever they run.
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)); // xor 1
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)); // xor 2
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)); // half mirror
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)); // mirror
    return v;
}

// Cross-workgroup hand-off without cache-wide fences.  Values one workgroup
// publishes for another are written with device-scope stores (they write
// through the XCD-local L2), the writer waits for its memory operations to
// complete before taking a ticket with a device-scope atomic, and the
// workgroup that draws the last ticket reads with device-scope loads (they
// do not hit stale L2 lines).  A release/acquire fence would also work but
// writes back or invalidates the whole L2 of the XCD, once per workgroup.
template <class T>
__device__ __forceinline__ void st_dev(T *p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_dev(const T *p) {
    return __hip_atomic_load(const_cast<T *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until every memory operation this thread issued has completed.
__device__ __forceinline__ void wait_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Argmax combine: (v, i) beats (bv, bi) when v > bv, or v == bv with a lower
// index.  NaN never wins (both comparisons are false).
__device__ __forceinline__ bool beats(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

}  // namespace nvfp4
