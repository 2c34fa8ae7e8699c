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
    long long sq[3], sk[3], sv[3], so[3];
    int B, H, Lq, Lk;
    const int* valid_lens;  // device int32 [B] or nullptr
    int causal;
    // Optional second bf16 planes of Q and K (same strides): when set, q and
    // q_lo hold q * log2(e) / sqrt(d_k) as hi + lo and k, k_lo hold k as
    // hi + lo; scores are formed from three products (hi.hi + lo.hi + hi.lo)
    // and come out in log2 units.  Bf16 output only.
    const void* q_lo = nullptr;
    const void* k_lo = nullptr;
    // Optional output: each query's log-sum-exp of its scaled scores
    // (natural log, contiguous [B, H, Lq]; ln(Lk) for a row with no allowed
    // key, whose weights are uniform).
    float* lse = nullptr;
};

// C[m, n] = sum_k A[m, k] * W[n, k] + bias[n] for up to three problems that
// share N and K (the fp32 Q/K/V projection is three problems in one launch).
struct GemmProblem {
    const void* a;     // [M, K] row-major
    const void* w;     // [N, K] row-major (a linear layer's [out, in])
    const void* bias;  // [N] or nullptr
    void* c;           // [M, N] row-major
    int M;
    const void* res = nullptr;  // [M, N] in the input dtype, added to c (a residual), or nullptr
    // bf16 output only: when c_lo is set, y = (A W^T + bias) * scale is
    // written as two bf16 planes, c = bf16(y) and c_lo = bf16(y - c), which
    // together carry about 16 significant bits.
    void* c_lo = nullptr;
    float scale = 1.0f;
};

struct GemmArgs {
    GemmProblem p[3];
    int nprob;
    int N;
    int K;
};

// Multi-head attention with the Q/K/V projections fused in (bf16, d_k = 64):
// writes the merged-head attention output; the output projection follows.
struct FusedArgs {
    const void* x_q;   // [B, Lq, D] bf16
    const void* x_kv;  // [B, Lk, D] bf16 (may equal x_q)
    const void* w_q;   // [D, D] bf16, [out, in]
    const void* w_k;
    const void* w_v;
    const void* b_q;   // [D] bf16 or nullptr
    const void* b_k;
    const void* b_v;
    void* o;           // [B, Lq, D] bf16: head h in columns h*64 .. h*64+63
    int B, H, Lq, Lk, D;
    const int* valid_lens;  // device int32 [B] or nullptr
    int causal;
};

// One decoding step: a single query per (batch, head) against cached keys
// and values [B, H, L, 64] (bf16), keys j < lens[b] attended.
struct DecodeArgs {
    const void* q;     // [B, H, 64]: element strides sq[0] (batch), sq[1] (head)
    const void* k;     // [B, H, L, 64]: strides {batch, head, position}
    const void* v;
    void* o;           // [B, H, 64]: strides so[0], so[1]
    long long sq[2], sk[3], sv[3], so[2];
    int B, H, L;
    const int* lens;   // device int32 [B]
};

// The inspection path: lengths per sequence or per query, optional fp32
// attention weights [B, H, Lq, Lk] (unit stride over keys), fp32 arithmetic.
struct WeightsArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    long long sq[3], sk[3], sv[3], so[3];   // element strides (batch, head, position)
    int B, H, Lq, Lk;
    const int* valid_lens;                  // device int32 [B] or [B, Lq] (vl_rank 1, 2), or nullptr
    int vl_rank;                            // 0 (no lengths), 1, 2
    int causal;
    bool in_f32, out_f32;
    float* p;                               // weights or nullptr
    long long sp[3];
};

// Attention backward: dq, dk, dv for the output gradient dout (fp32
// arithmetic).  `rows` is the workspace: (log-sum-exp in log2 units, D) per
// query, [B, H, Lq, 2] floats.
struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    long long sq[3], sk[3], sv[3], so[3], sdo[3], sdq[3], sdk[3], sdv[3];
    int B, H, Lq, Lk;
    const int* valid_lens;
    int vl_rank;                            // 0 (no lengths), 1 ([B]), 2 ([B, Lq])
    int causal;
    bool in_f32, out_f32;
    float* rows;
    // Optional log-sum-exp of each query's scaled scores (natural log,
    // contiguous [B, H, Lq]) from the forward; bf16 inputs use it in place
    // of their own pass over the keys.
    const float* lse_in = nullptr;
};

hipError_t launch_sdpa_bf16(const SdpaArgs& a, bool out_f32, hipStream_t s);
int decode_splits(int L);
size_t decode_workspace_bytes(int B, int H, int L);
hipError_t launch_sdpa_decode(const DecodeArgs& a, bool out_f32, void* workspace, hipStream_t s);
hipError_t launch_mha_attn_fused(const FusedArgs& a, hipStream_t s);
// Self-attention with L <= 128 (x_q == x_kv, Lq == Lk): one projection pass
// and the attention split over two key halves.  launch_mha_attn_fused picks
// it by itself when it fits.
bool mha_attn_fused_small_fits(const FusedArgs& a);
hipError_t launch_mha_attn_fused_small(const FusedArgs& a, hipStream_t s);
hipError_t launch_sdpa_f32(const SdpaArgs& a, hipStream_t s);
hipError_t launch_sdpa_weights(const WeightsArgs& a, hipStream_t s);
// bf16 inputs, d = 64, on MFMA (launch_sdpa_weights dispatches to it).
hipError_t launch_sdpa_weights_bf16(const WeightsArgs& a, hipStream_t s);
size_t backward_workspace_bytes(int B, int H, int Lq);
hipError_t launch_sdpa_backward(const BackwardArgs& a, hipStream_t s);
// bf16 inputs, d = 64, on MFMA (launch_sdpa_backward dispatches to it).
hipError_t launch_sdpa_backward_bf16(const BackwardArgs& a, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmArgs& a, bool out_f32, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s);
// Row-wise layer normalisation y = norm(x) of [M, D], bf16 or fp32 in and
// out: kind 0 = std with Bessel's correction, eps added to the std; kind 1 =
// biased variance, eps inside the root.  Gain and bias [D] or nullptr.
hipError_t launch_layer_norm(const void* x, const void* gain, const void* bias, void* y, int M, int D, int kind,
                             float eps, bool f32, hipStream_t s);

// Weight and bias gradients of linear layers, dW = dy^T x and db = the column
// sums of dy (bf16 in, fp32 out), for up to three problems in one launch
// pair (slice partials, then their sum in a fixed order).
struct TnProblem {
    const uint16_t* y;          // dy [M, N1] bf16, row stride ldy (elements)
    const uint16_t* x;          // x [M, N2] bf16, row stride ldx
    long long ldy, ldx;
    int M, N1, N2;              // N1, N2 multiples of 64
    float* dw;                  // [N1, N2] fp32, contiguous
    float* db;                  // [N1] fp32, or nullptr
    float* dw2 = nullptr;       // when set, rows N1/2 .. of dW (and db) go to dw2 (db2): two stacked layers
    float* db2 = nullptr;
    // Set by launch_gemm_tn.
    int slices = 0, rows_per_slice = 0, tiles1 = 0, tiles2 = 0, blocks = 0, reduce_blocks = 0;
    float* w_part = nullptr;
    float* db_part = nullptr;
};
struct TnArgs {
    TnProblem p[3];
    int nprob;
};
// Row slices of each problem (the launch's workgroups shared by work).
void gemm_tn_slices(const int* M, const int* N1, const int* N2, int nprob, int* slices);
size_t gemm_tn_workspace_bytes(const int* M, const int* N1, const int* N2, int nprob);
hipError_t launch_gemm_tn(TnArgs g, void* workspace, hipStream_t s);
// Transposes of square bf16 weights: dst[q] = w[q]^T, [n, n] each, written
// at column offset col0[q] of a row-major destination with row stride ld.
struct TransposeArgs {
    const uint16_t* w[4];
    uint16_t* dst[4];
    int col0[4];
    long long ld[4];
    int n, count;
};
hipError_t launch_transpose_bf16(const TransposeArgs& a, hipStream_t s);

// Zeros written into a [B, H, L, 64] view (element strides {batch, head,
// position}, 16-byte aligned rows) of 2- or 4-byte elements, and into n
// contiguous floats.
hipError_t launch_zero_view(void* p, const long long s[3], int B, int H, int L, int elem, hipStream_t st);
hipError_t launch_zero_f32(float* p, long long n, hipStream_t st);

}  // namespace mha
