// Shared device helpers for the gfx950 kernels of the GPT-2 training step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define GPT_DEV __device__ __forceinline__

// ---------------------------------------------------------------- conversions

GPT_DEV float to_f32(float x) { return x; }
GPT_DEV float to_f32(bf16 x) { return (float)x; }

template <typename T> GPT_DEV T from_f32(float x);
template <> GPT_DEV float from_f32<float>(float x) { return x; }
template <> GPT_DEV bf16 from_f32<bf16>(float x) { return (bf16)x; }   // round to nearest even

// Four consecutive elements as fp32 (address must be aligned to 4 elements).
GPT_DEV float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
GPT_DEV float4 load4(const bf16* p) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}
GPT_DEV void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
GPT_DEV void store4(bf16* p, float4 v) {
    bf16x4 o;
    o[0] = (bf16)v.x; o[1] = (bf16)v.y; o[2] = (bf16)v.z; o[3] = (bf16)v.w;
    *reinterpret_cast<bf16x4*>(p) = o;
}

// ---------------------------------------------------------------- reductions

GPT_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
GPT_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
GPT_DEV double wave_sum_d(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// ---------------------------------------------------------------- activations

// tanh(u) = 1 - 2 / (1 + e^(2u)) with the hardware exp2 and reciprocal (one
// v_exp_f32, one v_rcp_f32, about 1 ulp each); saturates to +-1 without
// overflow issues (e^(2u) = inf gives 1, e^(2u) = 0 gives -1). Absolute error
// ~1e-7.
GPT_DEV float tanh_exp2(float u) {
    return fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(2.8853900817779268f * u)), 1.0f);
}

// GELU, tanh approximation: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3),
// evaluated as x * sigma(2u) with sigma(2u) = 1 / (1 + 2^(-2 log2(e) u)), which
// equals 0.5 (1 + tanh(u)). One exp2 and one reciprocal; saturates cleanly
// (2^+inf gives sigma = 0, 2^-inf gives sigma = 1).
GPT_DEV float gelu_sigma(float x) {
    const float k1 = -2.0f * 1.4426950408889634f * 0.7978845608028654f;   // -2 log2(e) sqrt(2/pi)
    const float k3 = k1 * 0.044715f;
    const float a = x * fmaf(k3, x * x, k1);
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a));
}
GPT_DEV float gelu_tanh_f(float x) { return x * gelu_sigma(x); }
// d/dx [x sigma(2u)] = sigma + x sigma (1 - sigma) 2 u'(x), u' = sqrt(2/pi) (1 + 3 * 0.044715 x^2)
GPT_DEV float gelu_tanh_grad_f(float x) {
    const float c2 = 2.0f * 0.7978845608028654f;
    const float s = gelu_sigma(x);
    return fmaf(x * s * (1.0f - s), fmaf(c2 * 3.0f * 0.044715f, x * x, c2), s);
}
GPT_DEV float relu2_f(float x) { float r = fmaxf(x, 0.0f); return r * r; }
GPT_DEV float relu2_grad_f(float x) { return 2.0f * fmaxf(x, 0.0f); }

enum ActKind { ACT_GELU = 0, ACT_RELU2 = 1 };

template <int ACT> GPT_DEV float act_f(float x) { return ACT == ACT_RELU2 ? relu2_f(x) : gelu_tanh_f(x); }
template <int ACT> GPT_DEV float act_grad_f(float x) { return ACT == ACT_RELU2 ? relu2_grad_f(x) : gelu_tanh_grad_f(x); }
// the activation and its derivative at x together (GELU shares one sigma)
template <int ACT> GPT_DEV void act_and_grad(float x, float& a, float& da) {
    if constexpr (ACT == ACT_RELU2) {
        const float r = fmaxf(x, 0.0f);
        a = r * r;
        da = 2.0f * r;
    } else {
        const float c2 = 2.0f * 0.7978845608028654f;
        const float s = gelu_sigma(x);
        a = x * s;
        da = fmaf(x * s * (1.0f - s), fmaf(c2 * 3.0f * 0.044715f, x * x, c2), s);
    }
}
GPT_DEV void act_and_grad_rt(int act, float x, float& a, float& da) {
    if (act == ACT_RELU2) act_and_grad<ACT_RELU2>(x, a, da);
    else act_and_grad<ACT_GELU>(x, a, da);
}

__host__ __device__ inline int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
