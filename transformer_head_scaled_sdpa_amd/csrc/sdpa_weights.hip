// Attention with the inspection extras for fp32 inputs, in fp32 arithmetic
// (FMA only), d_k = d_v = 64: key-padding lengths per sequence [B] or per
// query [B, Lq], the causal rule, and optionally the attention weights
// themselves.  bf16 inputs take the MFMA kernel in sdpa_weights_mfma.hip.
//
// What it computes (The Annotated Transformer, "Attention" section: the
// attention function returns the weights p_attn beside the output, which the
// multi-head layer keeps for visualisation; d2l Transformer digest: the masked
// softmax takes valid lengths per sequence or per query, and the decoder's
// training pass gives query i the length i + 1):
//   p_ij = softmax_j(s_ij),  s_ij = q_i . k_j / sqrt(d_k), masked s_ij := -1e9
//   o_i  = sum_j p_ij v_j
// A key j is allowed for query i when j < len(b, i) and, if causal, j <= i;
// a row with no allowed key weights all Lk keys uniformly (every score is the
// fill).  The weights of masked keys are written as exact zeros.
//
// One wave64 per 64 queries of one (batch, head); each lane owns one query,
// its 64 features and 64 output accumulators.  K/V tiles of 32 rows are
// staged in LDS (converted to fp32) and read as broadcasts.  Two passes over
// the keys: the first finds every row's max and weight sum (online), the
// second recomputes the scores, writes the normalised weights and
// accumulates the output, so the weights written are final values.
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kD = 64;
constexpr int kBQ = 64;   // queries per workgroup (one per lane)
constexpr int kBK = 32;   // keys per tile

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }

template <typename T, bool kCausal>
__global__ __launch_bounds__(64) void sdpa_weights_d64(WeightsArgs a, int n_qtiles, float c_log2) {
    __shared__ float4 ks[kBK * kD / 4];
    __shared__ float4 vs[kBK * kD / 4];

    const int lane = threadIdx.x;
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int qt = blockIdx.x / BH;
    const int b = bh / a.H, hd = bh % a.H;
    const int i = qt * kBQ + lane;
    const int Lq = a.Lq, Lk = a.Lk;

    // This row's key rule.
    int len = Lk;
    if (a.vl_rank == 1) len = a.valid_lens[b];
    else if (a.vl_rank == 2 && i < Lq) len = a.valid_lens[(long long)b * Lq + i];
    const bool none = a.vl_rank != 0 && len <= 0;   // every key masked -> uniform weights
    const int lim = none ? Lk : min(len, Lk);
    auto allowed = [&](int key) { return none ? key < Lk : (key < lim && (!kCausal || key <= i)); };

    const T* qb = static_cast<const T*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const T* kb = static_cast<const T*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const T* vb = static_cast<const T*>(a.v) + b * a.sv[0] + hd * a.sv[1];

    float q[kD], o[kD];
#pragma unroll
    for (int t = 0; t < kD; t += 4) {
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i < Lq) x = load4(qb + (long long)i * a.sq[2] + t);
        q[t] = x.x; q[t + 1] = x.y; q[t + 2] = x.z; q[t + 3] = x.w;
        o[t] = o[t + 1] = o[t + 2] = o[t + 3] = 0.0f;
    }

    auto stage = [&](int kv0, bool with_v) {
        __syncthreads();
        // 32 rows x 16 float4 per tensor: 8 float4 per lane each.
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int c = lane + n * 64;
            const int r = c >> 4, col = (c & 15) * 4;
            const int key = kv0 + r;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (key < Lk) {
                kx = load4(kb + (long long)key * a.sk[2] + col);
                if (with_v) vx = load4(vb + (long long)key * a.sv[2] + col);
            }
            ks[c] = kx;
            if (with_v) vs[c] = vx;
        }
        __syncthreads();
    };
    // Scores of one tile; disallowed keys (and keys past Lk) are -inf, the
    // keys of a fully masked row score 0.
    auto scores = [&](int kv0, float (&s)[kBK]) {
#pragma unroll
        for (int j = 0; j < kBK; ++j) {
            float acc = 0.0f;
#pragma unroll
            for (int t4 = 0; t4 < kD / 4; ++t4) {
                const float4 kx = ks[j * (kD / 4) + t4];
                acc = fmaf(q[t4 * 4], kx.x, acc);
                acc = fmaf(q[t4 * 4 + 1], kx.y, acc);
                acc = fmaf(q[t4 * 4 + 2], kx.z, acc);
                acc = fmaf(q[t4 * 4 + 3], kx.w, acc);
            }
            s[j] = allowed(kv0 + j) ? (none ? 0.0f : acc) : -INFINITY;
        }
    };

    // ---- pass 1: row max and weight sum ----
    float m_run = -INFINITY, l_run = 0.0f;
    for (int kv0 = 0; kv0 < Lk; kv0 += kBK) {
        stage(kv0, false);
        float s[kBK];
        scores(kv0, s);
        float mt = s[0];
#pragma unroll
        for (int j = 1; j < kBK; ++j) mt = fmaxf(mt, s[j]);
        const float m_new = fmaxf(m_run, mt);
        if (m_new == -INFINITY) continue;        // nothing allowed yet
        float rs = 0.0f;
#pragma unroll
        for (int j = 0; j < kBK; ++j) rs += __builtin_amdgcn_exp2f((s[j] - m_new) * c_log2);
        l_run = l_run * __builtin_amdgcn_exp2f((m_run - m_new) * c_log2) + rs;
        m_run = m_new;
    }
    // Every row has an allowed key (a fully masked row allows all), so m_run
    // is finite and l_run >= 1 for rows below Lq.
    const float m_use = m_run == -INFINITY ? 0.0f : m_run;
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;

    // ---- pass 2: weights, output ----
    float* prow = (a.p && i < Lq) ? a.p + b * a.sp[0] + hd * a.sp[1] + (long long)i * a.sp[2] : nullptr;
    // 16-byte stores when every weight row starts 16-byte aligned.
    const bool vec4 = ((reinterpret_cast<uintptr_t>(a.p) | (uintptr_t)(a.sp[0] | a.sp[1] | a.sp[2]) * 4) & 15u) == 0;
    for (int kv0 = 0; kv0 < Lk; kv0 += kBK) {
        stage(kv0, true);
        float s[kBK];
        scores(kv0, s);
#pragma unroll
        for (int j = 0; j < kBK; ++j) s[j] = __builtin_amdgcn_exp2f((s[j] - m_use) * c_log2) * inv;
        if (prow) {
            if (vec4 && kv0 + kBK <= Lk) {
#pragma unroll
                for (int j = 0; j < kBK; j += 4)
                    *reinterpret_cast<float4*>(prow + kv0 + j) = make_float4(s[j], s[j + 1], s[j + 2], s[j + 3]);
            } else {
#pragma unroll
                for (int j = 0; j < kBK; ++j)
                    if (kv0 + j < Lk) prow[kv0 + j] = s[j];
            }
        }
#pragma unroll
        for (int j = 0; j < kBK; ++j) {
#pragma unroll
            for (int t4 = 0; t4 < kD / 4; ++t4) {
                const float4 vx = vs[j * (kD / 4) + t4];
                o[t4 * 4] = fmaf(s[j], vx.x, o[t4 * 4]);
                o[t4 * 4 + 1] = fmaf(s[j], vx.y, o[t4 * 4 + 1]);
                o[t4 * 4 + 2] = fmaf(s[j], vx.z, o[t4 * 4 + 2]);
                o[t4 * 4 + 3] = fmaf(s[j], vx.w, o[t4 * 4 + 3]);
            }
        }
    }

    if (i >= Lq) return;
    const long long ob = b * a.so[0] + hd * a.so[1] + (long long)i * a.so[2];
    if (a.out_f32) {
        float* op = static_cast<float*>(a.o) + ob;
#pragma unroll
        for (int t = 0; t < kD; t += 4) *reinterpret_cast<float4*>(op + t) = make_float4(o[t], o[t + 1], o[t + 2], o[t + 3]);
    } else {
        bf16_t* op = static_cast<bf16_t*>(a.o) + ob;
#pragma unroll
        for (int t = 0; t < kD; t += 4)
            *reinterpret_cast<uint2*>(op + t) = make_uint2(pack_bf16x2(o[t], o[t + 1]), pack_bf16x2(o[t + 2], o[t + 3]));
    }
}

template <typename T, bool kCausal>
hipError_t launch_variant(const WeightsArgs& a, hipStream_t s) {
    const int n_qtiles = (a.Lq + kBQ - 1) / kBQ;
    const long long grid = (long long)n_qtiles * a.B * a.H;
    if (grid == 0) return hipSuccess;
    const float c_log2 = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    hipLaunchKernelGGL((sdpa_weights_d64<T, kCausal>), dim3((unsigned)grid), dim3(64), 0, s, a, n_qtiles, c_log2);
    return hipGetLastError();
}

}  // namespace

// fp32 inputs run here; bf16 inputs take the MFMA kernel.
hipError_t launch_sdpa_weights(const WeightsArgs& a, hipStream_t s) {
    if (a.in_f32) return a.causal ? launch_variant<float, true>(a, s) : launch_variant<float, false>(a, s);
    return launch_sdpa_weights_bf16(a, s);
}

}  // namespace mha
