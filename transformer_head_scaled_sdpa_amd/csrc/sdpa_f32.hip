// Scaled dot-product attention forward in fp32 (FMA only, no reduced
// precision anywhere), d_k = d_v = 64.  Same mathematics and mask rules as
// the bf16 kernel (The Annotated Transformer, "Attention" section):
// o_i = sum_j softmax_j(q_i . k_j / sqrt(d_k)) v_j over allowed keys, with a
// row that has no allowed key weighting all Lk keys uniformly.
//
// One wave64 per 64 queries of one (batch, head); each lane owns one query,
// its 64 query features and 64 output accumulators in registers.  The keys
// are walked one at a time in a loop (not unrolled over keys), with every
// lane reading the same key and value row, so the row loads are uniform
// (scalar loads) and the code stays small: the fp32 path serves short
// sequences, where a few waves run cold and instruction fetch, not
// arithmetic, sets the time of a long unrolled body.  Two passes over the
// keys: the row max, then the weights, their sum and the output.
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kD = 64;
constexpr int kBQ = 64;   // queries per workgroup (one per lane)

__device__ __forceinline__ float row_dot(const float (&q)[kD], const float* kr) {
    float acc = 0.0f;
#pragma unroll
    for (int t4 = 0; t4 < kD / 4; ++t4) {
        const float4 kx = *reinterpret_cast<const float4*>(kr + t4 * 4);
        acc = fmaf(q[t4 * 4], kx.x, acc);
        acc = fmaf(q[t4 * 4 + 1], kx.y, acc);
        acc = fmaf(q[t4 * 4 + 2], kx.z, acc);
        acc = fmaf(q[t4 * 4 + 3], kx.w, acc);
    }
    return acc;
}

template <bool kCausal, bool kHasVl>
__global__ __launch_bounds__(64) void sdpa_fwd_f32_d64(SdpaArgs a, int n_qtiles, float c_log2) {
    const int lane = threadIdx.x;
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    int qt = blockIdx.x / BH;
    if (kCausal) qt = n_qtiles - 1 - qt;
    const int b = bh / a.H, hd = bh % a.H;
    const int q_wg = qt * kBQ;
    const int i = q_wg + lane;

    const int Lk = a.Lk;
    const int vlen = kHasVl ? a.valid_lens[b] : Lk;
    const bool none = vlen <= 0;                  // every key masked -> uniform weights
    const int kv_lim = none ? Lk : min(vlen, Lk);
    int kv_end = kv_lim;                          // keys the wave visits (uniform)
    if (kCausal && !none) kv_end = min(kv_end, q_wg + kBQ);
    const int key_lim = none ? Lk : (kCausal ? min(kv_lim, i + 1) : kv_lim);   // this lane's keys [0, key_lim)

    const float* qb = static_cast<const float*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const float* kb = static_cast<const float*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const float* vb = static_cast<const float*>(a.v) + b * a.sv[0] + hd * a.sv[1];

    float q[kD], o[kD];
#pragma unroll
    for (int t = 0; t < kD; t += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < a.Lq) x = *reinterpret_cast<const float4*>(qb + i * a.sq[2] + t);
        q[t] = x.x; q[t + 1] = x.y; q[t + 2] = x.z; q[t + 3] = x.w;
        o[t] = o[t + 1] = o[t + 2] = o[t + 3] = 0.0f;
    }

    // ---- pass 1: row max over the allowed keys (scores in raw units) ----
    float m = -INFINITY;
    for (int j = 0; j < kv_end; ++j) {
        const float sj = none ? 0.0f : row_dot(q, kb + (long long)j * a.sk[2]);
        if (j < key_lim) m = fmaxf(m, sj);
    }
    // ---- pass 2: weights, their sum and the output ----
    const float mc = m * c_log2;
    float l = 0.0f;
    for (int j = 0; j < kv_end; ++j) {
        const float sj = none ? 0.0f : row_dot(q, kb + (long long)j * a.sk[2]);
        const float p = j < key_lim ? __builtin_amdgcn_exp2f(fmaf(sj, c_log2, -mc)) : 0.0f;
        l += p;
        const float* vr = vb + (long long)j * a.sv[2];
#pragma unroll
        for (int t4 = 0; t4 < kD / 4; ++t4) {
            const float4 vx = *reinterpret_cast<const float4*>(vr + t4 * 4);
            o[t4 * 4] = fmaf(p, vx.x, o[t4 * 4]);
            o[t4 * 4 + 1] = fmaf(p, vx.y, o[t4 * 4 + 1]);
            o[t4 * 4 + 2] = fmaf(p, vx.z, o[t4 * 4 + 2]);
            o[t4 * 4 + 3] = fmaf(p, vx.w, o[t4 * 4 + 3]);
        }
    }

    if (i >= a.Lq) return;
    const float inv = 1.0f / l;
    // The log-sum-exp of the scaled scores (natural log) when asked for.
    if (a.lse) a.lse[(long long)bh * a.Lq + i] = (mc + __builtin_amdgcn_logf(l)) * kLn2;
    float* ob = static_cast<float*>(a.o) + b * a.so[0] + hd * a.so[1] + i * a.so[2];
#pragma unroll
    for (int t = 0; t < kD; t += 4)
        *reinterpret_cast<float4*>(ob + t) = make_float4(o[t] * inv, o[t + 1] * inv, o[t + 2] * inv, o[t + 3] * inv);
}

template <bool kCausal, bool kHasVl>
hipError_t launch_variant(const SdpaArgs& a, hipStream_t s) {
    const int n_qtiles = (a.Lq + kBQ - 1) / kBQ;
    const long long grid = (long long)n_qtiles * a.B * a.H;
    const float c_log2 = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    hipLaunchKernelGGL((sdpa_fwd_f32_d64<kCausal, kHasVl>), dim3((unsigned)grid), dim3(64), 0, s, a,
                       n_qtiles, c_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sdpa_f32(const SdpaArgs& a, hipStream_t s) {
    const bool c = a.causal != 0, v = a.valid_lens != nullptr;
    if (c) return v ? launch_variant<true, true>(a, s) : launch_variant<true, false>(a, s);
    return v ? launch_variant<false, true>(a, s) : launch_variant<false, false>(a, s);
}

}  // namespace mha
