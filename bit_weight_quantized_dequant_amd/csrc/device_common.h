// device_common.h -- small device helpers shared by the libqmv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QMV_DEV static __device__ __forceinline__

typedef _Float16 qmv_h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 128-bit streaming load of read-once weight bytes (nontemporal: do not keep in cache).
QMV_DEV uint4 ld_stream16(const void *p) {
    u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// IEEE binary16 bits -> float (exact; subnormals kept).
QMV_DEV float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// bfloat16 bits -> float (exact).
QMV_DEV float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// The two binary16 halves of a dword, as floats.  Used on dwords whose halves hold
// small integers q as binary16 subnormals (bit pattern q, value q * 2^-24): the
// conversion is exact, and the compiler folds it into v_fma_mix_f32.
QMV_DEV float lo_h(uint32_t v) { return (float)__builtin_bit_cast(qmv_h2, v).x; }
QMV_DEV float hi_h(uint32_t v) { return (float)__builtin_bit_cast(qmv_h2, v).y; }

// Sum over the 64 lanes of a wavefront; every lane receives the total.
QMV_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Load one activation element of type XT (0 = fp32, 1 = bf16 bits) as float.
template <int XT>
QMV_DEV float ld_act(const void *x, int64_t i) {
    if (XT == 0) return ((const float *)x)[i];
    return bf2f(((const uint16_t *)x)[i]);
}

// Eight consecutive activations starting at element i (i % 8 == 0, 16-byte aligned
// for bf16, 32-byte for fp32) as floats.
template <int XT>
QMV_DEV void ld_act8(const void *x, int64_t i, float *o) {
    if (XT == 0) {
        const float4 *p = (const float4 *)((const float *)x + i);
        float4 a = p[0], b = p[1];
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    } else {
        uint4 v = *(const uint4 *)((const uint16_t *)x + i);
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xFFFF0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xFFFF0000u);
        o[4] = __uint_as_float(v.z << 16); o[5] = __uint_as_float(v.z & 0xFFFF0000u);
        o[6] = __uint_as_float(v.w << 16); o[7] = __uint_as_float(v.w & 0xFFFF0000u);
    }
}
