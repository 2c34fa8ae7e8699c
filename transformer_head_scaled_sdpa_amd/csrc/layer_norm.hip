// Row-wise layer normalisation, the "norm" of the pre-norm residual sublayer
// x + attention(norm(x)) (The Annotated Transformer, sublayer connection).
// The pages print two forms, both supported:
//   kind 0 (The Annotated Transformer, LayerNorm class): a * (x - mean) /
//          (std + eps) + b with std using Bessel's correction (n - 1);
//   kind 1 (the "Transformer" study notes' torch layer): a * (x - mean) /
//          sqrt(var + eps) + b with the biased variance (n).
// One wave64 per row of D features (D a multiple of 4): the mean, then the
// sum of squared deviations (two passes over the row, the second from
// cache), in fp32.
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4(const bf16_t* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xffff0000u));
}
__device__ __forceinline__ void st4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
__device__ __forceinline__ void st4(bf16_t* p, float4 v) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <typename T>
__global__ __launch_bounds__(256) void layer_norm_rows(const T* x, const T* gain, const T* bias, T* y, int M, int D,
                                                       int kind, float eps) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= M) return;
    const T* xr = x + (long long)row * D;
    float s = 0.0f;
    for (int c = lane * 4; c < D; c += 256) {
        const float4 v = ld4(xr + c);
        s += (v.x + v.y) + (v.z + v.w);
    }
    const float mean = wave_sum(s) / D;
    float ss = 0.0f;
    for (int c = lane * 4; c < D; c += 256) {
        const float4 v = ld4(xr + c);
        const float a = v.x - mean, b = v.y - mean, cc = v.z - mean, d = v.w - mean;
        ss += (a * a + b * b) + (cc * cc + d * d);
    }
    ss = wave_sum(ss);
    const float den = kind == 0 ? sqrtf(ss / (D - 1)) + eps : sqrtf(ss / D + eps);
    const float inv = 1.0f / den;
    T* yr = y + (long long)row * D;
    for (int c = lane * 4; c < D; c += 256) {
        const float4 v = ld4(xr + c);
        const float4 g = gain ? ld4(gain + c) : make_float4(1.f, 1.f, 1.f, 1.f);
        const float4 b = bias ? ld4(bias + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        st4(yr + c, make_float4(g.x * (v.x - mean) * inv + b.x, g.y * (v.y - mean) * inv + b.y,
                                g.z * (v.z - mean) * inv + b.z, g.w * (v.w - mean) * inv + b.w));
    }
}

}  // namespace

hipError_t launch_layer_norm(const void* x, const void* gain, const void* bias, void* y, int M, int D, int kind,
                             float eps, bool f32, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (D % 4 != 0 || D < 2) return hipErrorInvalidValue;
    const dim3 grid((M + 3) / 4);
    if (f32)
        hipLaunchKernelGGL(layer_norm_rows<float>, grid, dim3(256), 0, s, static_cast<const float*>(x),
                           static_cast<const float*>(gain), static_cast<const float*>(bias), static_cast<float*>(y), M,
                           D, kind, eps);
    else
        hipLaunchKernelGGL(layer_norm_rows<bf16_t>, grid, dim3(256), 0, s, static_cast<const bf16_t*>(x),
                           static_cast<const bf16_t*>(gain), static_cast<const bf16_t*>(bias),
                           static_cast<bf16_t*>(y), M, D, kind, eps);
    return hipGetLastError();
}

}  // namespace mha
