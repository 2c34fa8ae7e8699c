// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace mha {

// Scaled dot-product attention on split heads, d_k = d_v = 64.
// Element strides are {batch, head, position}; the feature axis is contiguous.
struct SdpaArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    // bf16 only: low parts of a hi + lo split of Q and K (same strides as q
    // and k), or nullptr.  With them the scores are formed as
    // Kh Qh^T + Kl Qh^T + Kh Ql^T, which keeps ~16 significant bits per operand.
    const void* q_lo;
    const void* k_lo;
    long long sq[3], sk[3], sv[3], so[3];
    int B, H, Lq, Lk;
    const int* valid_lens;  // device int32 [B] or nullptr
    int causal;
};

// C[m, n] = sum_k A[m, k] * W[n, k] + bias[n] for up to three problems that
// share N and K (the fused Q/K/V projection is three problems in one launch).
struct GemmProblem {
    const void* a;     // [M, K] row-major
    const void* w;     // [N, K] row-major (a linear layer's [out, in])
    const void* bias;  // [N] or nullptr
    void* c;           // [M, N] row-major
    int M;
    void* c_lo;        // bf16 output only: [M, N] plane of c's rounding residue
                       // (x - bf16(x), rounded to bf16), or nullptr
};

struct GemmArgs {
    GemmProblem p[3];
    int nprob;
    int N;
    int K;
};

hipError_t launch_sdpa_bf16(const SdpaArgs& a, bool out_f32, hipStream_t s);
// Single-operand bf16 attention, software-pipelined, 32 queries per wave.
hipError_t launch_sdpa_bf16_pipe(const SdpaArgs& a, bool out_f32, hipStream_t s);
hipError_t launch_sdpa_f32(const SdpaArgs& a, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmArgs& a, bool out_f32, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s);

}  // namespace mha
