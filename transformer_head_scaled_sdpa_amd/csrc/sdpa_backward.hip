// Backward pass of scaled dot-product attention in fp32 arithmetic (FMA),
// d_k = d_v = 64: the gradients dq, dk, dv for an output gradient do.
//
// What it computes (the pages train these models end to end; the forward is
// The Annotated Transformer's attention function): with tau = 1/sqrt(d_k),
// p_ij = softmax_j(tau q_i . k_j) over the allowed keys (a row with none
// weights all Lk keys uniformly) and the forward output o,
//   dv_j  = sum_i p_ij do_i
//   dp_ij = do_i . v_j,   D_i = do_i . o_i  (= sum_j p_ij dp_ij)
//   ds_ij = p_ij (dp_ij - D_i)
//   dq_i  = tau sum_j ds_ij k_j,   dk_j = tau sum_i ds_ij q_i
// over allowed pairs only (a masked score is the constant fill and passes no
// gradient to q or k).  Masks: key-padding lengths per sequence or per query
// and the causal rule, as in the forward.
//
// Two kernels; a lane pair owns one row (32 features per lane, dot products
// summed over the pair) and keeps it in registers:
//  * rows (64 queries per workgroup): a first pass over the keys finds each row's
//    max and weight sum (its log-sum-exp), then a second pass recomputes the
//    weights and accumulates dq.  The row's log-sum-exp and D_i go to the
//    workspace.
//  * keys (64 keys per workgroup): walks the queries in tiles of 32 staged in LDS
//    (q, do, log-sum-exp, D, length), recomputes the weights and accumulates
//    dk and dv.
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kD = 64;
constexpr int kH = kD / 2;  // features per lane: a lane pair shares one row
constexpr int kRows = 64;   // rows (queries or keys) per workgroup
constexpr int kThreads = 2 * kRows;
constexpr int kTile = 32;   // keys / queries per LDS tile

__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16_t* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xffff0000u));
}

// This lane's half (32 features) of a row.
template <typename T>
__device__ __forceinline__ void load_half(const T* p, bool ok, float (&r)[kH]) {
#pragma unroll
    for (int t = 0; t < kH; t += 4) {
        const float4 x = ok ? load4(p + t) : make_float4(0.f, 0.f, 0.f, 0.f);
        r[t] = x.x; r[t + 1] = x.y; r[t + 2] = x.z; r[t + 3] = x.w;
    }
}

__device__ __forceinline__ void store_half(void* base, long long off, bool out_f32, const float (&r)[kH]) {
    if (out_f32) {
        float* p = static_cast<float*>(base) + off;
#pragma unroll
        for (int t = 0; t < kH; t += 4) *reinterpret_cast<float4*>(p + t) = make_float4(r[t], r[t + 1], r[t + 2], r[t + 3]);
    } else {
        bf16_t* p = static_cast<bf16_t*>(base) + off;
#pragma unroll
        for (int t = 0; t < kH; t += 4)
            *reinterpret_cast<uint2*>(p + t) = make_uint2(pack_bf16x2(r[t], r[t + 1]), pack_bf16x2(r[t + 2], r[t + 3]));
    }
}

// Dot product of this lane's half with the same half of an LDS row (16
// float4 per row), summed over the lane pair.
__device__ __forceinline__ float pair_dot(const float (&x)[kH], const float4* row, int half) {
    float acc = 0.0f;
#pragma unroll
    for (int t4 = 0; t4 < kH / 4; ++t4) {
        const float4 y = row[half * (kH / 4) + t4];
        acc = fmaf(x[t4 * 4], y.x, acc);
        acc = fmaf(x[t4 * 4 + 1], y.y, acc);
        acc = fmaf(x[t4 * 4 + 2], y.z, acc);
        acc = fmaf(x[t4 * 4 + 3], y.w, acc);
    }
    return acc + __shfl_xor(acc, 1);
}

__device__ __forceinline__ void axpy_half(float (&y)[kH], float a, const float4* row, int half) {
#pragma unroll
    for (int t4 = 0; t4 < kH / 4; ++t4) {
        const float4 x = row[half * (kH / 4) + t4];
        y[t4 * 4] = fmaf(a, x.x, y[t4 * 4]);
        y[t4 * 4 + 1] = fmaf(a, x.y, y[t4 * 4 + 1]);
        y[t4 * 4 + 2] = fmaf(a, x.z, y[t4 * 4 + 2]);
        y[t4 * 4 + 3] = fmaf(a, x.w, y[t4 * 4 + 3]);
    }
}

// The key length of query i of batch b (Lk when there are no lengths).
__device__ __forceinline__ int row_len(const BackwardArgs& a, int b, int i) {
    if (a.vl_rank == 1) return a.valid_lens[b];
    if (a.vl_rank == 2) return a.valid_lens[(long long)b * a.Lq + i];
    return a.Lk;
}

// Stage rows r0 .. r0+31 of one or two [L, 64] operands into LDS as fp32
// (rows at or past L read as zero): 512 float4 each, 4 per thread.
template <typename T>
__device__ __forceinline__ void stage_tile(float4* xs, const T* x, long long sx, float4* ys, const T* y,
                                           long long sy, int r0, int L, int tid) {
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int c = tid + n * kThreads;
        const int r = c >> 4, col = (c & 15) * 4;
        const int row = r0 + r;
        float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
        if (row < L) {
            a = load4(x + (long long)row * sx + col);
            if (ys) b = load4(y + (long long)row * sy + col);
        }
        xs[c] = a;
        if (ys) ys[c] = b;
    }
    __syncthreads();
}

// ---------------------------------------------------------------------------
// rows: log-sum-exp, D and dq.  Lane pair (2r, 2r+1) owns query r of the
// block; lane half `half` owns features 32*half .. +31.
// ---------------------------------------------------------------------------
template <typename T, bool kCausal>
__global__ __launch_bounds__(kThreads) void bwd_rows(BackwardArgs a, float c_log2, float tau) {
    __shared__ float4 ks[kTile * kD / 4];
    __shared__ float4 vs[kTile * kD / 4];

    const int tid = threadIdx.x, half = tid & 1;
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int b = bh / a.H, hd = bh % a.H;
    const int i = (blockIdx.x / BH) * kRows + (tid >> 1);
    const int Lq = a.Lq, Lk = a.Lk;
    const bool live = i < Lq;

    const int len = live ? row_len(a, b, i) : Lk;
    const bool none = a.vl_rank != 0 && len <= 0;     // every key masked -> uniform weights
    const int lim = none ? Lk : min(len, Lk);
    auto allowed = [&](int key) { return none ? key < Lk : (key < lim && (!kCausal || key <= i)); };

    const T* kb = static_cast<const T*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const T* vb = static_cast<const T*>(a.v) + b * a.sv[0] + hd * a.sv[1];
    float q[kH], g[kH];
    load_half(static_cast<const T*>(a.q) + b * a.sq[0] + hd * a.sq[1] + (long long)i * a.sq[2] + half * kH, live, q);
    load_half(static_cast<const T*>(a.dout) + b * a.sdo[0] + hd * a.sdo[1] + (long long)i * a.sdo[2] + half * kH,
              live, g);
    float dsum;                                       // D_i = do_i . o_i
    {
        float o[kH];
        load_half(static_cast<const T*>(a.o) + b * a.so[0] + hd * a.so[1] + (long long)i * a.so[2] + half * kH, live,
                  o);
        float acc = 0.0f;
#pragma unroll
        for (int t = 0; t < kH; ++t) acc = fmaf(g[t], o[t], acc);
        dsum = acc + __shfl_xor(acc, 1);
    }

    // ---- pass 1: the row's log-sum-exp (log2 units: tau * log2(e) folded
    // into the scores; a fully masked row scores 0 everywhere) ----
    float m_run = -INFINITY, l_run = 0.0f;
    for (int kv0 = 0; kv0 < Lk; kv0 += kTile) {
        stage_tile<T>(ks, kb, a.sk[2], nullptr, nullptr, 0, kv0, Lk, tid);
        float s[kTile];
#pragma unroll
        for (int j = 0; j < kTile; ++j) {
            const float d = pair_dot(q, ks + j * (kD / 4), half);
            s[j] = allowed(kv0 + j) ? (none ? 0.0f : d * c_log2) : -INFINITY;
        }
        float mt = s[0];
#pragma unroll
        for (int j = 1; j < kTile; ++j) mt = fmaxf(mt, s[j]);
        const float m_new = fmaxf(m_run, mt);
        if (m_new == -INFINITY) continue;
        float rs = 0.0f;
#pragma unroll
        for (int j = 0; j < kTile; ++j) rs += __builtin_amdgcn_exp2f(s[j] - m_new);
        l_run = l_run * __builtin_amdgcn_exp2f(m_run - m_new) + rs;
        m_run = m_new;
    }
    // Every row below Lq has an allowed key (a fully masked row allows all).
    // v_log_f32 is the base-2 logarithm, matching the log2-unit scores.
    const float lse = live ? m_run + __builtin_amdgcn_logf(l_run) : 0.0f;

    // ---- pass 2: dq ----
    float dq[kH];
#pragma unroll
    for (int t = 0; t < kH; ++t) dq[t] = 0.0f;
    for (int kv0 = 0; kv0 < Lk; kv0 += kTile) {
        stage_tile<T>(ks, kb, a.sk[2], vs, vb, a.sv[2], kv0, Lk, tid);
#pragma unroll 4
        for (int j = 0; j < kTile; ++j) {
            const float d = pair_dot(q, ks + j * (kD / 4), half);
            const float sj = allowed(kv0 + j) ? (none ? 0.0f : d * c_log2) : -INFINITY;
            const float p = __builtin_amdgcn_exp2f(sj - lse);
            const float dp = pair_dot(g, vs + j * (kD / 4), half);
            // A fully masked row's scores are constants: no gradient to q.
            const float ds = none ? 0.0f : p * (dp - dsum) * tau;
            axpy_half(dq, ds, ks + j * (kD / 4), half);
        }
    }
    if (!live) return;
    if (half == 0) {
        a.rows[((long long)bh * Lq + i) * 2] = lse;
        a.rows[((long long)bh * Lq + i) * 2 + 1] = dsum;
    }
    store_half(a.dq, b * a.sdq[0] + hd * a.sdq[1] + (long long)i * a.sdq[2] + half * kH, a.out_f32, dq);
}

// ---------------------------------------------------------------------------
// keys: dk and dv.  Lane pair (2r, 2r+1) owns key r of the block.
// ---------------------------------------------------------------------------
template <typename T, bool kCausal>
__global__ __launch_bounds__(kThreads) void bwd_keys(BackwardArgs a, float c_log2, float tau) {
    __shared__ float4 qs[kTile * kD / 4];
    __shared__ float4 gs[kTile * kD / 4];
    __shared__ float lse_s[kTile], dsum_s[kTile];
    __shared__ int len_s[kTile];

    const int tid = threadIdx.x, half = tid & 1;
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int b = bh / a.H, hd = bh % a.H;
    const int k0 = (blockIdx.x / BH) * kRows;
    const int j = k0 + (tid >> 1);
    const int Lq = a.Lq, Lk = a.Lk;
    const bool live = j < Lk;

    float kr[kH], vr[kH], dk[kH], dv[kH];
    load_half(static_cast<const T*>(a.k) + b * a.sk[0] + hd * a.sk[1] + (long long)j * a.sk[2] + half * kH, live, kr);
    load_half(static_cast<const T*>(a.v) + b * a.sv[0] + hd * a.sv[1] + (long long)j * a.sv[2] + half * kH, live, vr);
#pragma unroll
    for (int t = 0; t < kH; ++t) dk[t] = dv[t] = 0.0f;

    const T* qb = static_cast<const T*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const T* gb = static_cast<const T*>(a.dout) + b * a.sdo[0] + hd * a.sdo[1];
    // Causal without lengths: queries below the block's first key weight
    // none of its keys (with lengths a fully masked row weights all keys).
    const int i_start = (kCausal && a.vl_rank == 0) ? k0 : 0;
    for (int i0 = i_start; i0 < Lq; i0 += kTile) {
        stage_tile<T>(qs, qb, a.sq[2], gs, gb, a.sdo[2], i0, Lq, tid);
        if (tid < kTile) {
            const int qi = i0 + tid;
            const bool ok = qi < Lq;
            lse_s[tid] = ok ? a.rows[((long long)bh * Lq + qi) * 2] : 0.0f;
            dsum_s[tid] = ok ? a.rows[((long long)bh * Lq + qi) * 2 + 1] : 0.0f;
            len_s[tid] = ok ? row_len(a, b, qi) : 0;
        }
        __syncthreads();
        const int n_q = min(kTile, Lq - i0);
        for (int r = 0; r < n_q; ++r) {
            const int i = i0 + r;
            const int len = len_s[r];
            const bool none = a.vl_rank != 0 && len <= 0;
            const bool ok = live && (none || (j < min(len, Lk) && (!kCausal || j <= i)));
            const float s = pair_dot(kr, qs + r * (kD / 4), half);
            const float dp = pair_dot(vr, gs + r * (kD / 4), half);
            const float p = ok ? __builtin_amdgcn_exp2f((none ? 0.0f : s * c_log2) - lse_s[r]) : 0.0f;
            const float ds = none ? 0.0f : p * (dp - dsum_s[r]) * tau;
            axpy_half(dv, p, gs + r * (kD / 4), half);
            axpy_half(dk, ds, qs + r * (kD / 4), half);
        }
    }
    if (!live) return;
    store_half(a.dk, b * a.sdk[0] + hd * a.sdk[1] + (long long)j * a.sdk[2] + half * kH, a.out_f32, dk);
    store_half(a.dv, b * a.sdv[0] + hd * a.sdv[1] + (long long)j * a.sdv[2] + half * kH, a.out_f32, dv);
}

template <typename T, bool kCausal>
hipError_t launch_variant(const BackwardArgs& a, hipStream_t s) {
    const float c_log2 = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    const float tau = 0.125f;             // 1 / sqrt(64)
    const long long BH = (long long)a.B * a.H;
    const long long gq = BH * ((a.Lq + kRows - 1) / kRows), gk = BH * ((a.Lk + kRows - 1) / kRows);
    if (gq == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_rows<T, kCausal>), dim3((unsigned)gq), dim3(kThreads), 0, s, a, c_log2, tau);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_keys<T, kCausal>), dim3((unsigned)gk), dim3(kThreads), 0, s, a, c_log2, tau);
    return hipGetLastError();
}

}  // namespace

size_t backward_workspace_bytes(int B, int H, int Lq) { return (size_t)B * H * Lq * 2 * sizeof(float); }

// fp32 inputs run here; bf16 inputs take the MFMA kernels.
hipError_t launch_sdpa_backward(const BackwardArgs& a, hipStream_t s) {
    if (a.in_f32) return a.causal ? launch_variant<float, true>(a, s) : launch_variant<float, false>(a, s);
    return launch_sdpa_backward_bf16(a, s);
}

}  // namespace mha
