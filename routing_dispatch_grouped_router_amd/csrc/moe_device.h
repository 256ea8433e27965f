// Device-side helpers shared by the gfx950 kernels: bfloat16 and E4M3 encodes,
// orderable routing keys, vector types.  Internal to the library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
// Native 16-byte vector for register-held tiles (HIP's uint4 wrapper can defeat
// scalar replacement and end up in scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// float32 -> bfloat16, round to nearest even.  The conversion is the
// hardware's (v_cvt_pk_bf16_f32), checked equal to the integer rounding
// (u + 0x7FFF + bit 16) >> 16 over every finite float32 input on gfx950.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// x rounded to the nearest bfloat16 (ties to even), as a float32.
__device__ __forceinline__ float bf16_round(float x) { return __uint_as_float((uint32_t)f32_to_bf16(x) << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- MXFP8 (OCP MX v1.0)

// Shared block exponent floor(log2(amax)) - 8 clamped to [-127, 127], from the
// float32 exponent field (amax is finite and >= 0; zero or float32-subnormal
// amax gives the floor -127 because floor(log2) <= -127 there).
__device__ __forceinline__ int mx_shared_exp(float amax) {
    int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
    if (ef == 0) return -127;
    int se = ef - 127 - 8;
    return se < -127 ? -127 : se;
}

// 2^-se as a float32 (se in [-127, 119] -> exponent field 127 - se in [8, 254]).
__device__ __forceinline__ float mx_inv_scale(int se) {
    return __uint_as_float((uint32_t)(127 - se) << 23);
}

// E4M3 "FN" code of v: round to nearest even, saturate to +-448, keep sign on zero.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    float a = __uint_as_float(u & 0x7FFFFFFFu);
    uint32_t code;
    if (a >= 448.0f) {
        code = 0x7Eu;
    } else if (a < 0.015625f) {                       // below 2^-6: subnormal step 2^-9
        code = (uint32_t)rintf(a * 512.0f);           // 0..8; 8 is the smallest normal
    } else {
        int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;      // -6..8
        float m = __uint_as_float((__float_as_uint(a) & 0x007FFFFFu) | 0x3F800000u);  // [1,2)
        uint32_t q = (uint32_t)rintf((m - 1.0f) * 8.0f);   // 0..8
        if (q == 8u) { q = 0u; e += 1; }
        code = ((uint32_t)(e + 7) << 3) | q;
        if (code > 0x7Eu) code = 0x7Eu;
    }
    return sign | code;
}

// Four E4M3 codes (a in byte 0 .. d in byte 3) by the hardware conversion
// (round to nearest even) after clamping to +-448, which makes it the
// saturating encode above; checked equal to e4m3_encode over every finite
// float32 input on gfx950.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    int pk = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, -448.f), 448.f), fminf(fmaxf(b, -448.f), 448.f), 0, false);
    pk = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(c, -448.f), 448.f), fminf(fmaxf(d, -448.f), 448.f), pk, true);
    return (uint32_t)pk;
}

}  // namespace moe
