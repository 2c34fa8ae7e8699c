// The inspection path for bf16 inputs on MFMA, d_k = d_v = 64, gfx950: the
// attention output and, optionally, the attention weights themselves as fp32
// [B, H, Lq, Lk], with key-padding lengths per sequence [B] or per query
// [B, Lq] and the causal rule (what sdpa_weights.hip computes in fp32 FMA).
//
// What it computes (The Annotated Transformer, "Attention" section: the
// attention function returns p_attn beside the output; d2l Transformer
// digest: valid lengths per sequence or per query):
//   p_ij = softmax_j(q_i . k_j / sqrt(d_k)) over the allowed keys (masked
//   keys weigh exactly 0; a row with none allowed weighs all Lk keys 1/Lk),
//   o_i = sum_j p_ij v_j.
//
// Layout of mfma_rows.h with 8 waves: 64 queries per workgroup, keys
// streamed in steps of 128 (four phases of 32; measured faster here than 4
// waves with two workgroups per CU: 16.0 against 18.4 us on B4 h8 L512).
// Two passes over the keys:
//  * pass 1: S^T = K Q^T on the MFMA (exact bf16 products, fp32 sums), an
//    online (max, sum) per lane half and phase, merged into each query's
//    log-sum-exp;
//  * pass 2: the scores again, p = exp2(s - lse) in fp32 written as the final
//    weights, and O^T += V^T P^T with P split into two bf16 terms (hi + lo,
//    about 16 significant bits), so the output keeps fp32-level accuracy.
// The phases' partial outputs are summed through LDS.  Causal launches
// without lengths stream only the keys the triangle allows and fill the rest
// of the weight rows with zeros.
// Rows of at most 512 keys (other than causal without lengths) take
// weights_mfma_short, which loads everything at once and keeps the scores
// in registers between the two passes instead of streaming K twice (the
// same arithmetic, bit for bit).  The weights are written with streaming
// stores.
#include "common.h"
#include "kernels.h"
#define MFMA_ROWS_WAVES 8
#include "mfma_rows.h"

namespace mha {

namespace {

using namespace rows64;

constexpr int kKR = 0;                    // K, 144-byte rows (score fragments)
constexpr int kVT = kTileRB;              // V, 192-byte rows (transposed reads)
constexpr int kPhaseB = kTileRB + kTileTB;
constexpr int kRedB = kGroups * (kPhases - 1) * 32 * 64 * 4;   // reduction slots (reuse the tiles)
constexpr int kSmemB = kPhases * kPhaseB > kRedB ? kPhases * kPhaseB : kRedB;
constexpr int kWstPitch = kTile + 4;      // fp32 per staged weight row (144 bytes)

// Write this lane's four weights of keys t .. t+3 (row prow), as one 16-byte
// store when aligned and whole, else element by element inside the row.  The
// weights are written once and not read back here, so the stores stream
// (non-temporal): they do not fill the L2 with lines that would be written
// back at the end of the kernel.
__device__ __forceinline__ void put4(float* prow, int t, int Lk, bool vec4, float p0, float p1, float p2, float p3) {
    if (vec4 && t + 3 < Lk) {
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        const f32x4v w = {p0, p1, p2, p3};
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4v*>(prow + t));
        return;
    }
    if (t < Lk) __builtin_nontemporal_store(p0, prow + t);
    if (t + 1 < Lk) __builtin_nontemporal_store(p1, prow + t + 1);
    if (t + 2 < Lk) __builtin_nontemporal_store(p2, prow + t + 2);
    if (t + 3 < Lk) __builtin_nontemporal_store(p3, prow + t + 3);
}

template <bool kCausal>
__global__ __launch_bounds__(kThreads, 1) void weights_mfma(WeightsArgs a, float c, bool vec4) {
    __shared__ __attribute__((aligned(16))) char smem[kSmemB];
    __shared__ float2 stat_s[kGroups][kPhases][2][32];
    __shared__ __attribute__((aligned(16))) float wst_s[kWaves][kTile * kWstPitch];   // per-wave weight tile

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave % kGroups, ph = wave / kGroups;
    const int hb = lane >> 5, l32 = lane & 31;
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int b = bh / a.H, hd = bh % a.H;
    const int n_wg = (a.Lq + kRowsWg - 1) / kRowsWg;
    const int blk = blockIdx.x / BH;
    const int q_wg = (kCausal ? n_wg - 1 - blk : blk) * kRowsWg;   // causal: longest rows first
    const int i = q_wg + grp * 32 + l32;
    const int Lq = a.Lq, Lk = a.Lk;
    const bool live = i < Lq;

    bool none = false;
    const int klim = live ? key_limit<kCausal>(a, b, i, none) : Lk;
    const float cs = none ? 0.0f : c;       // score scale (log2 units); 0: equal scores
    int kmin = klim;                        // smallest key limit in the wave
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmin = min(kmin, __shfl_xor(kmin, o));
    kmin = __builtin_amdgcn_readfirstlane(kmin);
    const int kv_end = (kCausal && a.vl_rank == 0) ? min(Lk, q_wg + kRowsWg) : Lk;
    const int n_steps = (kv_end + kStep - 1) / kStep;

    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1];

    const StepSrc ksrc = step_src(kp, a.sk[2], Lk, tid), vsrc = step_src(vp, a.sv[2], Lk, tid);
    Chunks nk = load_step(ksrc, 0);
    bf16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 rq = make_uint4(0, 0, 0, 0);
        if (live) rq = *reinterpret_cast<const uint4*>(qp + (long long)i * a.sq[2] + kk * 16 + hb * 8);
        qf[kk] = __builtin_bit_cast(bf16x8, rq);
    }

    // Scores of this wave's tile in log2 units, masked keys -inf.
    auto scores = [&](int t0) {
        f32x16 s = tile_dot(reinterpret_cast<const bf16_t*>(smem + ph * kPhaseB + kKR), qf, l32, hb);
        if (t0 + kTile <= kmin) {
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] *= cs;
        } else {
            const int rel = klim - (t0 + hb * 4);
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] = acc_row(v) < rel ? s[v] * cs : -INFINITY;
        }
        return s;
    };

    // ---- pass 1: log-sum-exp ----
    float m_run = -INFINITY, l_run = 0.0f;
    for (int st = 0; st < n_steps; ++st) {
        __syncthreads();
        store_step(nk, smem, kPhaseB, kKR, -1, tid);
        if (st + 1 < n_steps) nk = load_step(ksrc, (st + 1) * kStep);
        __syncthreads();
        const f32x16 s = scores(st * kStep + ph * kTile);
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        float rs = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) rs += __builtin_amdgcn_exp2f(s[v] - m_use);
        l_run = l_run * __builtin_amdgcn_exp2f(m_run - m_use) + rs;
        m_run = m_new;
    }
    stat_s[grp][ph][hb][l32] = make_float2(m_run, l_run);
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int p = 0; p < kPhases; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) M = fmaxf(M, stat_s[grp][p][h][l32].x);
    float L = 0.0f;
#pragma unroll
    for (int p = 0; p < kPhases; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float2 x = stat_s[grp][p][h][l32];
            L += x.x == -INFINITY ? 0.0f : x.y * __builtin_amdgcn_exp2f(x.x - M);
        }
    // v_log_f32 is the base-2 logarithm, matching the log2-unit scores.
    const float lse = L > 0.0f ? M + __builtin_amdgcn_logf(L) : 0.0f;

    // ---- pass 2: weights and output ----
    // The wave's 32 x 32 weight tile goes through its own LDS slice so that
    // each store instruction writes whole 128-byte runs of 8 weight rows.
    float* const pq = a.p ? a.p + b * a.sp[0] + hd * a.sp[1] : nullptr;
    const int q_w = q_wg + grp * 32;           // first query of this wave's tile
    float* const wst = wst_s[wave];
    f32x16 o[2] = {};
    nk = load_step(ksrc, 0);
    Chunks nv = load_step(vsrc, 0);
    for (int st = 0; st < n_steps; ++st) {
        __syncthreads();
        store_step(nk, smem, kPhaseB, kKR, -1, tid);
        store_step(nv, smem, kPhaseB, -1, kVT, tid);
        if (st + 1 < n_steps) {
            nk = load_step(ksrc, (st + 1) * kStep);
            nv = load_step(vsrc, (st + 1) * kStep);
        }
        __syncthreads();
        const int t0 = st * kStep + ph * kTile;
        f32x16 p = scores(t0);
#pragma unroll
        for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(p[v] - lse);   // masked: exp2(-inf) = 0
        if (pq) {
            // Lane (query l32, half hb) holds keys t0 + g4*8 + hb*4 + 0..3.
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                *reinterpret_cast<float4*>(wst + l32 * kWstPitch + g4 * 8 + hb * 4) =
                    make_float4(p[g4 * 4], p[g4 * 4 + 1], p[g4 * 4 + 2], p[g4 * 4 + 3]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // 8 lanes per row, keys t0 + c4 .. c4+3; rows past Lq are not stored.
#pragma unroll
            for (int pass = 0; pass < kTile / 8; ++pass) {
                const int r = pass * 8 + (lane >> 3), c4 = (lane & 7) * 4;
                if (q_w + r < Lq) {
                    const float4 w4 = *reinterpret_cast<const float4*>(wst + r * kWstPitch + c4);
                    put4(pq + (long long)(q_w + r) * a.sp[2], t0 + c4, Lk, vec4, w4.x, w4.y, w4.z, w4.w);
                }
            }
        }
        // P = hi + lo in bf16; O^T += V^T (hi + lo)^T.
        u32x4 ph_w[2], pl_w[2];
        pack_b(p, ph_w);
        f32x16 r;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = ph_w[kb][e];
                r[kb * 8 + 2 * e] = p[kb * 8 + 2 * e] - __uint_as_float(w << 16);
                r[kb * 8 + 2 * e + 1] = p[kb * 8 + 2 * e + 1] - __uint_as_float(w & 0xffff0000u);
            }
        pack_b(r, pl_w);
        const bf16_t* vt = reinterpret_cast<const bf16_t*>(smem + ph * kPhaseB + kVT);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 hi = __builtin_bit_cast(bf16x8, ph_w[kb]), lo = __builtin_bit_cast(bf16x8, pl_w[kb]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const bf16x8 vf = tr_frag(vt, kb, tb, hb, lane);
                o[tb] = mfma32x32x16(vf, hi, o[tb]);
                o[tb] = mfma32x32x16(vf, lo, o[tb]);
            }
        }
    }
    // Causal without lengths: keys past the streamed range weigh 0 for every
    // row of this workgroup; the whole workgroup writes those zeros.
    if (a.p && kv_end < Lk) {
        const int width = Lk - kv_end;
        const int rows = min(kRowsWg, Lq - q_wg);
        for (int e = tid; e < rows * width; e += kThreads) {
            const int r = e / width, col = kv_end + e % width;
            a.p[b * a.sp[0] + hd * a.sp[1] + (long long)(q_wg + r) * a.sp[2] + col] = 0.0f;
        }
    }
    __syncthreads();
    reduce_write(reinterpret_cast<float*>(smem), o, grp, ph, lane);
    __syncthreads();
    reduce_read(reinterpret_cast<const float*>(smem), o, grp, ph, lane);
    if (ph != 0 || !live) return;
    store_rowT(a.o, b * a.so[0] + hd * a.so[1] + (long long)i * a.so[2], a.out_f32, o, 1.0f, hb);
}


// Rows of at most kShortSteps steps (Lk <= 512; not the causal rule without
// lengths, whose short rows the two-pass kernel cuts to the triangle): every
// K and V load and the Q fragments are issued at the start, so the workgroup
// pays one memory round trip; K is stored to LDS once, each wave keeps its
// scores in registers from the log-sum-exp pass to the weights pass, and V
// is then stored once in the space K used.  Three barriers before the output
// reduction instead of two per step and pass.  The products, the online
// (max, sum) update and its order, and the weights are those of
// weights_mfma, so every result is bit for bit the same.
constexpr int kShortSteps = 4;
constexpr int kKvB = kShortSteps * kPhases * kTileTB;   // V in 192-byte rows (96 KiB); K takes 72
static_assert(kKvB >= kShortSteps * kPhases * kTileRB && kKvB >= kRedB, "K tiles and reduction slots fit");

template <bool kCausal>
__global__ __launch_bounds__(kThreads, 1) void weights_mfma_short(WeightsArgs a, float c, bool vec4) {
    __shared__ __attribute__((aligned(16))) char kv[kKvB];
    __shared__ float2 stat_s[kGroups][kPhases][2][32];
    __shared__ __attribute__((aligned(16))) float wst_s[kWaves][kTile * kWstPitch];   // per-wave weight tile

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave % kGroups, ph = wave / kGroups;
    const int hb = lane >> 5, l32 = lane & 31;
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int b = bh / a.H, hd = bh % a.H;
    const int n_wg = (a.Lq + kRowsWg - 1) / kRowsWg;
    const int blk = blockIdx.x / BH;
    const int q_wg = (kCausal ? n_wg - 1 - blk : blk) * kRowsWg;   // causal: longest rows first
    const int i = q_wg + grp * 32 + l32;
    const int Lq = a.Lq, Lk = a.Lk;
    const bool live = i < Lq;

    bool none = false;
    const int klim = live ? key_limit<kCausal>(a, b, i, none) : Lk;
    const float cs = none ? 0.0f : c;
    int kmin = klim;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmin = min(kmin, __shfl_xor(kmin, o));
    kmin = __builtin_amdgcn_readfirstlane(kmin);
    const int n_steps = (Lk + kStep - 1) / kStep;   // at most kShortSteps (the launcher's rule)

    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1];

    const StepSrc ksrc = step_src(kp, a.sk[2], Lk, tid), vsrc = step_src(vp, a.sv[2], Lk, tid);
    // Steps past Lk hold zeros: every step then runs the same straight-line
    // code (their scores are masked, their weights are 0), so the steps'
    // products and exponentials interleave.
    Chunks nk[kShortSteps] = {}, nv[kShortSteps] = {};
#pragma unroll
    for (int st = 0; st < kShortSteps; ++st)
        if (st < n_steps) nk[st] = load_step(ksrc, st * kStep);
#pragma unroll
    for (int st = 0; st < kShortSteps; ++st)
        if (st < n_steps) nv[st] = load_step(vsrc, st * kStep);
    bf16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 rq = make_uint4(0, 0, 0, 0);
        if (live) rq = *reinterpret_cast<const uint4*>(qp + (long long)i * a.sq[2] + kk * 16 + hb * 8);
        qf[kk] = __builtin_bit_cast(bf16x8, rq);
    }
    // Step st, phase p: K rows st*kStep + p*kTile .. +31 at tile st*kPhases + p.
#pragma unroll
    for (int st = 0; st < kShortSteps; ++st) store_step(nk[st], kv + st * kPhases * kTileRB, kTileRB, 0, -1, tid);
    __syncthreads();

    // ---- log-sum-exp, keeping the scores ----
    // A step past Lk is wholly masked: it leaves the running (max, sum)
    // exactly as it was.
    f32x16 sk[kShortSteps];
#pragma unroll
    for (int st = 0; st < kShortSteps; ++st) {
        const int t0 = st * kStep + ph * kTile;
        f32x16 s = tile_dot(reinterpret_cast<const bf16_t*>(kv + (st * kPhases + ph) * kTileRB), qf, l32, hb);
        if (t0 + kTile <= kmin) {
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] *= cs;
        } else {
            const int rel = klim - (t0 + hb * 4);
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] = acc_row(v) < rel ? s[v] * cs : -INFINITY;
        }
        sk[st] = s;
    }
    float m_run = -INFINITY, l_run = 0.0f;
#pragma unroll
    for (int st = 0; st < kShortSteps; ++st) {
        const f32x16& s = sk[st];
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.0f : m_new;
        float rs = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) rs += __builtin_amdgcn_exp2f(s[v] - m_use);
        l_run = l_run * __builtin_amdgcn_exp2f(m_run - m_use) + rs;
        m_run = m_new;
    }
    stat_s[grp][ph][hb][l32] = make_float2(m_run, l_run);
    __syncthreads();   // every wave is past its K reads and has written its statistics
    // Step st, phase p: V rows at tile st*kPhases + p, 192-byte rows.
#pragma unroll
    for (int st = 0; st < kShortSteps; ++st) store_step(nv[st], kv + st * kPhases * kTileTB, kTileTB, -1, 0, tid);
    float M = -INFINITY;
#pragma unroll
    for (int p = 0; p < kPhases; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) M = fmaxf(M, stat_s[grp][p][h][l32].x);
    float L = 0.0f;
#pragma unroll
    for (int p = 0; p < kPhases; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float2 x = stat_s[grp][p][h][l32];
            L += x.x == -INFINITY ? 0.0f : x.y * __builtin_amdgcn_exp2f(x.x - M);
        }
    const float lse = L > 0.0f ? M + __builtin_amdgcn_logf(L) : 0.0f;
    __syncthreads();   // V is in LDS

    // ---- weights and output, from the kept scores ----
    float* const pq = a.p ? a.p + b * a.sp[0] + hd * a.sp[1] : nullptr;
    const int q_w = q_wg + grp * 32;
    float* const wst = wst_s[wave];
    f32x16 o[2] = {};
#pragma unroll
    for (int st = 0; st < kShortSteps; ++st) {
        const int t0 = st * kStep + ph * kTile;
        f32x16 p = sk[st];
#pragma unroll
        for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(p[v] - lse);   // masked: exp2(-inf) = 0
        if (pq && st < n_steps) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                *reinterpret_cast<float4*>(wst + l32 * kWstPitch + g4 * 8 + hb * 4) =
                    make_float4(p[g4 * 4], p[g4 * 4 + 1], p[g4 * 4 + 2], p[g4 * 4 + 3]);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int pass = 0; pass < kTile / 8; ++pass) {
                const int r = pass * 8 + (lane >> 3), c4 = (lane & 7) * 4;
                if (q_w + r < Lq) {
                    const float4 w4 = *reinterpret_cast<const float4*>(wst + r * kWstPitch + c4);
                    put4(pq + (long long)(q_w + r) * a.sp[2], t0 + c4, Lk, vec4, w4.x, w4.y, w4.z, w4.w);
                }
            }
            // The next step's tile overwrites the slice.
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
        u32x4 ph_w[2], pl_w[2];
        pack_b(p, ph_w);
        f32x16 r;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = ph_w[kb][e];
                r[kb * 8 + 2 * e] = p[kb * 8 + 2 * e] - __uint_as_float(w << 16);
                r[kb * 8 + 2 * e + 1] = p[kb * 8 + 2 * e + 1] - __uint_as_float(w & 0xffff0000u);
            }
        pack_b(r, pl_w);
        const bf16_t* vt = reinterpret_cast<const bf16_t*>(kv + (st * kPhases + ph) * kTileTB);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 hi = __builtin_bit_cast(bf16x8, ph_w[kb]), lo = __builtin_bit_cast(bf16x8, pl_w[kb]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const bf16x8 vf = tr_frag(vt, kb, tb, hb, lane);
                o[tb] = mfma32x32x16(vf, hi, o[tb]);
                o[tb] = mfma32x32x16(vf, lo, o[tb]);
            }
        }
    }
    __syncthreads();   // every wave is past its V reads: the reduction slots reuse the space
    reduce_write(reinterpret_cast<float*>(kv), o, grp, ph, lane);
    __syncthreads();
    reduce_read(reinterpret_cast<const float*>(kv), o, grp, ph, lane);
    if (ph != 0 || !live) return;
    store_rowT(a.o, b * a.so[0] + hd * a.so[1] + (long long)i * a.so[2], a.out_f32, o, 1.0f, hb);
}


}  // namespace

hipError_t launch_sdpa_weights_bf16(const WeightsArgs& a, hipStream_t s) {
    if (!fits_buffer(a.sk[2], a.Lk) || !fits_buffer(a.sv[2], a.Lk)) return hipErrorInvalidValue;
    const long long grid = (long long)a.B * a.H * ((a.Lq + kRowsWg - 1) / kRowsWg);
    if (grid == 0) return hipSuccess;
    const float c = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    // 16-byte weight stores when every weight row starts 16-byte aligned.
    const bool vec4 = ((reinterpret_cast<uintptr_t>(a.p) | (uintptr_t)(a.sp[0] | a.sp[1] | a.sp[2]) * 4) & 15u) == 0;
    if (a.Lk <= kShortSteps * kStep && !(a.causal && a.vl_rank == 0)) {   // every key step fits the registers
        if (a.causal)
            hipLaunchKernelGGL((weights_mfma_short<true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, c, vec4);
        else
            hipLaunchKernelGGL((weights_mfma_short<false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, c, vec4);
    } else if (a.causal) {
        hipLaunchKernelGGL((weights_mfma<true>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, c, vec4);
    } else {
        hipLaunchKernelGGL((weights_mfma<false>), dim3((unsigned)grid), dim3(kThreads), 0, s, a, c, vec4);
    }
    return hipGetLastError();
}

}  // namespace mha
