// device_common.h -- small device helpers shared by the libqmv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QMV_DEV static __device__ __forceinline__

typedef _Float16 qmv_h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 128-bit streaming load of read-once weight bytes (nontemporal: do not keep in cache).
QMV_DEV uint4 ld_stream16(const void *p) {
    u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16 bytes from LDS at byte address a (16-byte aligned).
QMV_DEV uint4 lds_ld16(uint32_t a) {
    const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)(uintptr_t)a;
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Workgroup barrier that orders LDS only: this wave's LDS operations complete, then
// s_barrier.  __syncthreads() also waits for every outstanding global load of the wave
// (its workgroup-scope fence covers global memory), so loads issued ahead for a later step
// would be waited for at every barrier; here they stay in flight across it.  Only for
// kernels whose waves exchange data through LDS alone.
QMV_DEV void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// IEEE binary16 bits -> float (exact; subnormals kept).
QMV_DEV float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// bfloat16 bits -> float (exact).
QMV_DEV float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// The two binary16 halves of a dword, as floats.  Used on dwords whose halves hold
// small integers q as binary16 subnormals (bit pattern q, value q * 2^-24): the
// conversion is exact, and the compiler folds it into v_fma_mix_f32.
QMV_DEV qmv_h2 as_h2(uint32_t v) { return __builtin_bit_cast(qmv_h2, v); }

// (a & mask) | bits in one v_and_or_b32.  gfx950 VOP3 encodings take no literal and at
// most one scalar operand, so the compiler otherwise splits this into v_and + v_or with
// literals; here mask and bits live in (loop-invariant) VGPRs.
QMV_DEV uint32_t and_or(uint32_t a, uint32_t mask, uint32_t bits) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(mask), "v"(bits));
    return r;
}
QMV_DEV float lo_h(uint32_t v) { return (float)__builtin_bit_cast(qmv_h2, v).x; }
QMV_DEV float hi_h(uint32_t v) { return (float)__builtin_bit_cast(qmv_h2, v).y; }

// DPP move of a float within a row of 16 lanes (or row broadcast); rows masked off by
// RM, or lanes whose source is out of range, contribute 0.
template <int CTRL, int RM = 0xF>
QMV_DEV float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, RM, 0xF, false));
}

// Sum over the 64 lanes of a wavefront with DPP (xor-1, xor-2, half-row mirror, row mirror,
// then row broadcasts 15 and 31); the total is read from lane 63 and returned uniformly.
QMV_DEV float wave_sum(float v) {
    v += dpp_f<0xB1>(v);         // quad_perm [1,0,3,2]
    v += dpp_f<0x4E>(v);         // quad_perm [2,3,0,1]
    v += dpp_f<0x141>(v);        // row_half_mirror
    v += dpp_f<0x140>(v);        // row_mirror: every lane holds its row-of-16 sum
    v += dpp_f<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp_f<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Sum over aligned groups of 8 lanes; every lane of the group receives the group total.
QMV_DEV float sum8(float v) {
    v += dpp_f<0xB1>(v);
    v += dpp_f<0x4E>(v);
    v += dpp_f<0x141>(v);
    return v;
}

// Sum over aligned groups of G lanes (G = 2, 4, ..., 64) with xor shuffles.
QMV_DEV float group_sum(float v, int G) {
    for (int o = G >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Four consecutive activations starting at element i (16-byte aligned) as floats.
template <int XT>
QMV_DEV float4 ld_act4(const void *x, int64_t i) {
    if (XT == 0) return *(const float4 *)((const float *)x + i);
    const uint2 v = *(const uint2 *)((const uint16_t *)x + i);
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
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
