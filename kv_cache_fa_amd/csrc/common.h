// Device-side building blocks for the gfx950 (CDNA4) attention kernels:
// vector types, bf16 conversion, buffer-resource loads, MFMA wrappers and
// cross-lane helpers. Everything here is written for wave64 and gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- buffer resources -------------------------------------------------------------
// A raw buffer descriptor: loads past num_bytes return zero instead of faulting, which
// is how tile loads handle ragged tails without per-lane branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, num_bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// The same with the nontemporal hint (the `nt` bit; cache-policy argument 2 on gfx950),
// for data that is streamed once.
__device__ __forceinline__ u32x4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2);
}

// 8 bytes per lane, nontemporal.
__device__ __forceinline__ u32x2 buf_load8_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 2);
}

// ---- fp8 (OCP e4m3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
// infinities, 0x7f / 0xff are NaN) ----------------------------------------------------
// Every e4m3 value is exactly representable in bf16 and fp32, so these conversions are
// exact (hardware conversion with a scale of 1).
// Four e4m3 bytes (byte i = element i) -> four bf16 in two dwords.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t w) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// 16 bytes per lane from a buffer straight into LDS: lane L writes lds_base + 16 L
// (buffer_load_dwordx4 ... lds). lds_base must be the same in all lanes; loads past the
// descriptor's size write zeros. The builtin only exists for the device, and naming it
// in a kernel template's host-side instantiation drops the kernel's launch stub, so it
// lives behind this device-only wrapper.
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                               uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 0);
#endif
}

// The same with the nontemporal hint, for data read once per call.
__device__ __forceinline__ void buf_load16_lds_nt(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                                  uint32_t voff, uint32_t soff) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 2);
#endif
}

// ---- bf16 <-> fp32 --------------------------------------------------------------
// Low / high bf16 of a packed dword, widened exactly.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> one dword of two bf16 (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// ---- MFMA -------------------------------------------------------------------------
// 32x32x16 bf16 -> fp32. Lane l supplies A[m = l%32][k = 8*(l/32) + u] and
// B[k = 8*(l/32) + u][n = l%32] for u = 0..7, and holds
// D[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32] in element i of the accumulator.
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16x32 bf16 -> fp32. Lane l supplies A[m = l%16][k = 8*(l/16) + u] and
// B[k = 8*(l/16) + u][n = l%16], and holds D[m = 4*(l/16) + i][n = l%16] in element i.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- cross-lane ------------------------------------------------------------------
// Value of the same register in lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float xor32(float x) {
    uint32_t u = __float_as_uint(x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // r[0]: lanes 0-31 keep their value, lanes 32-63 receive lanes 0-31;
    // r[1]: lanes 0-31 receive lanes 32-63, lanes 32-63 keep theirs.
    const bool hi = (__lane_id() >= 32);
    return __uint_as_float(hi ? r[0] : r[1]);
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
    return __shfl_xor(x, mask, 64);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Orders LDS accesses of one wave (no work-group barrier): the compiler may not move
// memory operations across it, and the hardware completes a wave's LDS operations in
// issue order.
__device__ __forceinline__ void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace kvfa
