// kda_common.h -- small device helpers shared by the libkda kernels
// (dtype conversion and vector loads).  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// bf16 is carried as its 16-bit pattern; widening to fp32 is exact.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 with round-to-nearest-even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <typename T> struct io;

template <> struct io<float> {
    // load N consecutive values (N*4 bytes, 16-byte aligned when N % 4 == 0)
    template <int N>
    __device__ __forceinline__ static void load(const float* __restrict__ p, float (&x)[N]) {
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int i = 0; i < N; i += 4) {
                float4 t = *reinterpret_cast<const float4*>(p + i);
                x[i] = t.x; x[i + 1] = t.y; x[i + 2] = t.z; x[i + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) x[i] = p[i];
        }
    }
    __device__ __forceinline__ static void store4(float* __restrict__ p, float a, float b,
                                                  float c, float d) {
        *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
    }
};

template <> struct io<bf16_t> {
    template <int N>
    __device__ __forceinline__ static void load(const bf16_t* __restrict__ p, float (&x)[N]) {
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int i = 0; i < N; i += 8) {
                uint4 t = *reinterpret_cast<const uint4*>(p + i);
                uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[i + 2 * j] = bf16_bits_to_f32(w[j] & 0xffffu);
                    x[i + 2 * j + 1] = bf16_bits_to_f32(w[j] >> 16);
                }
            }
        } else if constexpr (N % 4 == 0) {
#pragma unroll
            for (int i = 0; i < N; i += 4) {
                uint2 t = *reinterpret_cast<const uint2*>(p + i);
                x[i] = bf16_bits_to_f32(t.x & 0xffffu);
                x[i + 1] = bf16_bits_to_f32(t.x >> 16);
                x[i + 2] = bf16_bits_to_f32(t.y & 0xffffu);
                x[i + 3] = bf16_bits_to_f32(t.y >> 16);
            }
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) x[i] = bf16_bits_to_f32(p[i].bits);
        }
    }
    __device__ __forceinline__ static void store4(bf16_t* __restrict__ p, float a, float b,
                                                  float c, float d) {
        uint2 t;
        t.x = (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
        t.y = (uint32_t)f32_to_bf16_bits(c) | ((uint32_t)f32_to_bf16_bits(d) << 16);
        *reinterpret_cast<uint2*>(p) = t;
    }
};

// 16-byte loads and stores that bypass cache retention: for data touched
// once per kernel (the decode state streams through HBM in place).
typedef float f32v4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream4(const float* p) {
    const f32v4 x = __builtin_nontemporal_load(reinterpret_cast<const f32v4*>(p));
    return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store_stream4(float* p, const float4& v) {
    const f32v4 x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<f32v4*>(p));
}

// alpha = exp(g) through the hardware base-2 exponential.
__device__ __forceinline__ float exp_gate(float g) {
    return __builtin_amdgcn_exp2f(g * 1.4426950408889634f);
}
__device__ __forceinline__ float4 exp4(const float4& g) {
    return make_float4(exp_gate(g.x), exp_gate(g.y), exp_gate(g.z), exp_gate(g.w));
}

// 8 consecutive input values as fp32 (one 16-byte load for bf16, two for fp32)
__device__ __forceinline__ void load8f(const bf16_t* p, float4& lo, float4& hi) {
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    lo = make_float4(bf16_bits_to_f32(t.x & 0xffffu), bf16_bits_to_f32(t.x >> 16),
                     bf16_bits_to_f32(t.y & 0xffffu), bf16_bits_to_f32(t.y >> 16));
    hi = make_float4(bf16_bits_to_f32(t.z & 0xffffu), bf16_bits_to_f32(t.z >> 16),
                     bf16_bits_to_f32(t.w & 0xffffu), bf16_bits_to_f32(t.w >> 16));
}
__device__ __forceinline__ void load8f(const float* p, float4& lo, float4& hi) {
    lo = reinterpret_cast<const float4*>(p)[0];
    hi = reinterpret_cast<const float4*>(p)[1];
}

// v from another lane of the same 16-lane row (DPP: no LDS round trip)
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// sum over aligned groups of N consecutive lanes (N = 8 or 16), left in
// every lane of the group: quad permutations for lane ^ 1 and lane ^ 2, the
// half-row mirror for the other quad of 8, a row rotation by 8 for 16
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 8 || N == 16, "lane groups of 8 or 16");
    v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);  // row_half_mirror
    if constexpr (N == 16) v += dpp<0x128>(v);  // row_ror 8
    return v;
}

// sum over the 64 lanes of a wave, left in every lane: DPP inside each
// 16-lane row, then the rows by lane permutes
__device__ __forceinline__ float wave_sum(float v) {
    v = group_sum<16>(v);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
}

}  // namespace kda
