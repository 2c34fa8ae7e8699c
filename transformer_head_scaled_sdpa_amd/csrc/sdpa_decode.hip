// One decoding step of attention: a single new query per (batch, head)
// against its cache of keys and values, d_k = d_v = 64, bf16 in, fp32
// arithmetic.  The pages' decoder, when predicting, concatenates the keys and
// values of every earlier step with the current one and attends from the
// current position only (d2l Transformer digest, decoder block: the state
// keeps the per-layer key/value history at prediction time); the mask is the
// key-padding rule with the cache length as valid length, so this is exactly
//   o = sum_j softmax_j(q . k_j / sqrt(d_k)) v_j,  j < len[b]
// (len[b] <= 0: every score is the -1e9 fill, uniform weights over all L
// cached positions, as for a fully masked row).
//
// The step reads every cached key and value once and does 4*d_k flops per
// key, so it is HBM-bound.  One workgroup (4 wave64s) per (batch, head, key
// slice); every K and V load of the slice is issued at the start, so the
// whole slice is in flight at once and the step costs one memory round trip:
//  * scores: a thread pair shares a key (features [0,32) and [32,64) from
//    16-byte loads), fp32 dot products, summed over the pair;
//  * the slice's max and weight sum are block reductions;
//  * P.V: thread t accumulates features (t % 8) * 8 .. +7 over keys
//    t / 8 + 32 i from its 16-byte V loads; the 32 key groups are reduced by
//    shuffles and LDS.
// A cache that fits one slice (512 keys, or 256 when the grid would be too
// small to fill the GPU) is finished in place: the normalised output is
// written directly.  Longer caches are split over many workgroups (split-K,
// "flash decoding"); each slice's (max, sum, unnormalised output) goes to the
// workspace and a second kernel merges the slices by rescaling each to the
// common max (the online-softmax merge).
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kD = 64;
constexpr int kThreads = 256;
constexpr int kSplitMin = 256;         // smallest slice: the workspace is sized for it
constexpr int kPart = kD + 2;          // floats per partial: max, sum, 64 outputs

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// 8 bf16 -> fp32
__device__ __forceinline__ void unpack8(const uint4& r, float (&f)[8]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
}

template <int kKeys, bool kDirect, bool kOutF32>
__global__ __launch_bounds__(kThreads) void decode_split(DecodeArgs a, int n_split, float c, float* part) {
    constexpr int kKPass = kKeys / (kThreads / 2);   // keys per thread pair
    constexpr int kVKeys = kKeys / (kThreads / 8);   // V rows per thread
    __shared__ float sc[kKeys];
    __shared__ float red[kThreads / 64];
    __shared__ float ored[kThreads / 64][kD];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x % n_split;
    const int bh = blockIdx.x / n_split;
    const int b = bh / a.H, hd = bh % a.H;
    const int len = a.lens[b];
    const bool none = len <= 0;                 // every position masked -> uniform weights
    const int n = none ? a.L : min(len, a.L);   // positions that carry weight
    const int j0 = split * kKeys;
    float* out = part + ((long long)bh * n_split + split) * kPart;
    if (!kDirect && j0 >= n) {                  // empty slice: contributes nothing
        if (tid == 0) {
            out[0] = -INFINITY;
            out[1] = 0.0f;
        }
        return;
    }
    const int cnt = min(kKeys, n - j0);         // >= 1

    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1];

    // ---- every load of the slice, issued up front: the query first, then
    // K in the order the score passes use it, then V, all unconditional (a
    // buffer range ending with the slice's last key: rows past it read as
    // zeros), so each pass waits only for its own keys and the V loads are
    // still landing while the scores and the softmax run.
    const int half = tid & 1;
    const int f8 = (tid & 7) * 8, jg = tid >> 3;
    uint4 qr[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) qr[x] = *reinterpret_cast<const uint4*>(qp + half * 32 + x * 8);
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    constexpr int kBufWord3 = 0x00020000;       // raw buffer, 32-bit data format
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(kp + (long long)j0 * a.sk[2]), (short)0,
        (int)((long long)(cnt - 1) * a.sk[2] * 2 + kD * 2), kBufWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(vp + (long long)j0 * a.sv[2]), (short)0,
        (int)((long long)(cnt - 1) * a.sv[2] * 2 + kD * 2), kBufWord3);
    auto ld = [](__amdgpu_buffer_rsrc_t r, uint32_t off) {
        const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        return make_uint4(v[0], v[1], v[2], v[3]);
    };
    uint4 kr[kKPass][4], vr[kVKeys];
#pragma unroll
    for (int p = 0; p < kKPass; ++p) {
        const int jl = p * (kThreads / 2) + (tid >> 1);
        const uint32_t row = (uint32_t)(jl * a.sk[2] * 2) + half * 64;
#pragma unroll
        for (int x = 0; x < 4; ++x) kr[p][x] = ld(krs, row + x * 16);
    }
#pragma unroll
    for (int i = 0; i < kVKeys; ++i) {
        const int jl = jg + i * (kThreads / 8);
        vr[i] = ld(vrs, (uint32_t)(jl * a.sv[2] * 2) + f8 * 2);
    }
    __builtin_amdgcn_sched_barrier(0);   // every load out before the first wait
    float qf[32];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        float f[8];
        unpack8(qr[x], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[x * 8 + e] = f[e];
    }

    // ---- scores ----
#pragma unroll
    for (int p = 0; p < kKPass; ++p) {
        const int jl = p * (kThreads / 2) + (tid >> 1);   // key within the slice
        float acc = 0.0f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            float f[8];
            unpack8(kr[p][x], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = fmaf(qf[x * 8 + e], f[e], acc);
        }
        acc += __shfl_xor(acc, 1);
        if (half == 0) sc[jl] = jl < cnt ? (none ? 0.0f : acc * c) : -INFINITY;
    }
    __syncthreads();

    // ---- slice max and weights ----
    float m = -INFINITY;
#pragma unroll
    for (int j = tid; j < kKeys; j += kThreads) m = fmaxf(m, sc[j]);
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float s = 0.0f;
#pragma unroll
    for (int j = tid; j < kKeys; j += kThreads) {
        const float p = __builtin_amdgcn_exp2f(sc[j] - m);   // exp2(-inf) = 0 past cnt
        sc[j] = p;
        s += p;
    }
    s = wave_sum(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    s = (red[0] + red[1]) + (red[2] + red[3]);

    // ---- unnormalised output ----
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < kVKeys; ++i) {
        const float p = sc[jg + i * (kThreads / 8)];          // 0 past cnt
        float f[8];
        unpack8(vr[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(p, f[e], o[e]);
    }
    // groups jg and jg ^ 16, ^ 8, ^ 4 share a wave (jg = 8 * wave + lane / 8);
    // reduce those with shuffles, then the 4 waves' partials in LDS.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        o[e] += __shfl_xor(o[e], 32);
        o[e] += __shfl_xor(o[e], 16);
        o[e] += __shfl_xor(o[e], 8);
    }
    if (lane < 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ored[wave][f8 + e] = o[e];
    }
    __syncthreads();
    if (tid < kD) {
        const float y = (ored[0][tid] + ored[1][tid]) + (ored[2][tid] + ored[3][tid]);
        if (kDirect) {
            const long long off = b * a.so[0] + hd * a.so[1] + tid;
            if (kOutF32) static_cast<float*>(a.o)[off] = y / s;
            else static_cast<bf16_t*>(a.o)[off] = __builtin_bit_cast(bf16_t, static_cast<__bf16>(y / s));
        } else {
            out[2 + tid] = y;
            if (tid == 0) {
                out[0] = m;
                out[1] = s;
            }
        }
    }
}

template <bool kOutF32>
__global__ __launch_bounds__(kD) void decode_merge(DecodeArgs a, int n_split, const float* part) {
    const int bh = blockIdx.x, t = threadIdx.x;
    const int b = bh / a.H, hd = bh % a.H;
    const float* pp = part + (long long)bh * n_split * kPart;
    float M = -INFINITY;
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, pp[s * kPart]);
    float l = 0.0f, acc = 0.0f;
    for (int s = 0; s < n_split; ++s) {
        const float ms = pp[s * kPart];
        if (ms == -INFINITY) continue;          // empty split
        const float w = __builtin_amdgcn_exp2f(ms - M);
        l = fmaf(pp[s * kPart + 1], w, l);
        acc = fmaf(pp[s * kPart + 2 + t], w, acc);
    }
    const float y = acc / l;
    const long long off = b * a.so[0] + hd * a.so[1] + t;
    if (kOutF32) static_cast<float*>(a.o)[off] = y;
    else static_cast<bf16_t*>(a.o)[off] = __builtin_bit_cast(bf16_t, static_cast<__bf16>(y));
}

// Keys per slice: 512 when that still gives at least 512 workgroups, else 256.
int decode_slice(int B, int H, int L) {
    const long long wg512 = (long long)B * H * ((L + 511) / 512);
    return wg512 >= 512 ? 512 : 256;
}

template <int kKeys>
hipError_t launch_slices(const DecodeArgs& a, bool out_f32, float* part, hipStream_t s) {
    const int n_split = (a.L + kKeys - 1) / kKeys;
    const long long grid = (long long)a.B * a.H * n_split;
    const float c = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    if (n_split == 1) {
        if (out_f32) hipLaunchKernelGGL((decode_split<kKeys, true, true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, 1, c, part);
        else hipLaunchKernelGGL((decode_split<kKeys, true, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, 1, c, part);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((decode_split<kKeys, false, false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, n_split, c, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (out_f32) hipLaunchKernelGGL(decode_merge<true>, dim3(a.B * a.H), dim3(kD), 0, s, a, n_split, part);
    else hipLaunchKernelGGL(decode_merge<false>, dim3(a.B * a.H), dim3(kD), 0, s, a, n_split, part);
    return hipGetLastError();
}

}  // namespace

// The workspace holds one partial per 256-key slice, the most any launch uses.
int decode_splits(int L) { return (L + kSplitMin - 1) / kSplitMin; }

size_t decode_workspace_bytes(int B, int H, int L) {
    return (size_t)B * H * decode_splits(L) * kPart * sizeof(float);
}

hipError_t launch_sdpa_decode(const DecodeArgs& a, bool out_f32, void* workspace, hipStream_t s) {
    if ((long long)a.B * a.H == 0) return hipSuccess;
    float* part = static_cast<float*>(workspace);
    return decode_slice(a.B, a.H, a.L) == 512 ? launch_slices<512>(a, out_f32, part, s)
                                              : launch_slices<256>(a, out_f32, part, s);
}

}  // namespace mha
