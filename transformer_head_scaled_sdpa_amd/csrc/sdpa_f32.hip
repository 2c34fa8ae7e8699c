// Scaled dot-product attention forward in fp32 (FMA only, no reduced
// precision anywhere), d_k = d_v = 64.  Same mathematics and mask rules as
// the bf16 kernel (The Annotated Transformer, "Attention" section):
// o_i = sum_j softmax_j(q_i . k_j / sqrt(d_k)) v_j over allowed keys, with a
// row that has no allowed key weighting all Lk keys uniformly.
//
// One wave64 per 64 queries of one (batch, head); each lane owns one query,
// its 64 query features and 64 output accumulators in registers.  Key/value
// tiles of 16 rows are staged in LDS and read as broadcasts (every lane reads
// the same address), so there are no bank conflicts.  Online softmax in fp32.
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kD = 64;
constexpr int kBQ = 64;   // queries per workgroup (one per lane)
constexpr int kBK = 16;   // keys per tile (short sequences waste at most 15 masked keys)

template <bool kCausal, bool kHasVl>
__global__ __launch_bounds__(64) void sdpa_fwd_f32_d64(SdpaArgs a, int n_qtiles, float c_log2) {
    __shared__ float4 ks[kBK * kD / 4];
    __shared__ float4 vs[kBK * kD / 4];

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
    const bool none = vlen <= 0;
    const int kv_lim = none ? Lk : min(vlen, Lk);
    int kv_end = kv_lim;
    if (kCausal && !none) kv_end = min(kv_end, q_wg + kBQ);

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
    float m_run = -INFINITY, l_run = 0.0f;

    for (int kv0 = 0; kv0 < kv_end; kv0 += kBK) {
        __syncthreads();
        // kBK rows x 16 float4 per tensor: kBK / 4 float4 per lane each.
#pragma unroll
        for (int n = 0; n < kBK / 4; ++n) {
            const int c = lane + n * 64;
            const int r = c >> 4, col = (c & 15) * 4;
            const int key = kv0 + r;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (key < Lk) {
                kx = *reinterpret_cast<const float4*>(kb + key * a.sk[2] + col);
                vx = *reinterpret_cast<const float4*>(vb + key * a.sv[2] + col);
            }
            ks[c] = kx;
            vs[c] = vx;
        }
        __syncthreads();

        float s[kBK];
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
            const int key = kv0 + j;
            bool ok;
            if (none) {
                ok = key < Lk;
                acc = 0.0f;
            } else {
                ok = key < kv_lim && (!kCausal || key <= i);
            }
            s[j] = ok ? acc : -INFINITY;
        }
        float mt = s[0];
#pragma unroll
        for (int j = 1; j < kBK; ++j) mt = fmaxf(mt, s[j]);
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c_log2);
        const float mc = m_use * c_log2;
        float rs = 0.0f;
#pragma unroll
        for (int j = 0; j < kBK; ++j) {
            s[j] = __builtin_amdgcn_exp2f(fmaf(s[j], c_log2, -mc));
            rs += s[j];
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int t = 0; t < kD; ++t) o[t] *= alpha;
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

    if (i >= a.Lq) return;
    const float inv = 1.0f / l_run;
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
