// Backward pass of scaled dot-product attention on bf16 MFMA (fp32
// accumulate), d_k = d_v = 64, gfx950: the same gradients as the fp32 kernels
// (dq, dk, dv for an output gradient do; see sdpa_backward.hip), for bf16
// inputs.  With tau = 1/sqrt(d_k), p the weights, D_i = do_i . o_i:
//   dv_j = sum_i p_ij do_i,  ds_ij = p_ij (do_i . v_j - D_i),
//   dq_i = tau sum_j ds_ij k_j,  dk_j = tau sum_i ds_ij q_i   (allowed pairs;
// a row with no allowed key weights all keys uniformly and passes no
// gradient to q or k).
//
// Two kernels of 8 wave64s per workgroup.  A workgroup owns 64 rows (two
// groups of 32, one row per lane column of the 32x32 MFMA tile) and streams
// the other side in steps of 128 rows: four phases of 32, one per wave of a
// group, so every wave works on its own tile and the four partial sums of a
// row are added through LDS at the end.  Products run on
// v_mfma_f32_32x32x16_bf16 in the operand layouts of the forward kernel: an
// accumulator packed to bf16 feeds the next MFMA as its B operand, and
// transposed tiles are read from LDS with ds_read_b64_tr_b16 (each tile is
// stored twice: 144-byte rows for 16-byte fragment reads, 192-byte rows for
// the transposed reads).
//  * rows (queries; q and do fragments in registers): one pass over the
//    keys: S^T = K Q^T and dP^T = V dO^T, unnormalised weights exp2(S - m)
//    with a lazy per-query offset m (the online softmax), dS^T = P^T (dP^T -
//    D), and dQ^T += K^T dS^T; the phases' (m, weight sum, dq) are merged at
//    the end and dq divided by the weight sum.  D_i comes from the supplied
//    output.  The log-sum-exp and D go to the workspace.
//  * keys (k and v fragments in registers): S = Q K^T and dP = dO V^T, P and
//    dS from the stored log-sum-exp and D, then dV^T += dO^T P and
//    dK^T += Q^T dS.
// dS (and P for dV) is rounded to bf16 for its products, as P is in the
// forward.  Tiles where every pair is allowed skip the mask arithmetic.
#include "common.h"
#include "kernels.h"
#include "mfma_rows.h"

namespace mha {

namespace {

using namespace rows64;

// ---------------------------------------------------------------------------
// rows: log-sum-exp, D, dq
// ---------------------------------------------------------------------------
constexpr int kRowsKR = 0;                        // K, 144-byte rows
constexpr int kRowsKT = kTileRB;                  // K, 192-byte rows
constexpr int kRowsVR = kTileRB + kTileTB;        // V, 144-byte rows
constexpr int kRowsPhase = 2 * kTileRB + kTileTB;

template <bool kCausal>
__global__ __launch_bounds__(kThreads, 1) void bwd_rows_mfma(BackwardArgs a, float c) {
    __shared__ __attribute__((aligned(16))) char smem[kPhases * kRowsPhase];
    __shared__ float2 stat_s[kGroups][kPhases][2][32];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave % kGroups, ph = wave / kGroups;
    const int hb = lane >> 5, l32 = lane & 31;
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int b = bh / a.H, hd = bh % a.H;
    // Causal rows late in the sequence see the most keys: they go first.
    const int n_wg = (a.Lq + kRowsWg - 1) / kRowsWg;
    const int blk = blockIdx.x / BH;
    const int q_wg = (kCausal ? n_wg - 1 - blk : blk) * kRowsWg;
    const int i = q_wg + grp * 32 + l32;
    const int Lq = a.Lq, Lk = a.Lk;
    const bool live = i < Lq;

    bool none = false;
    const int klim = live ? key_limit<kCausal>(a, b, i, none) : Lk;
    const float cs = none ? 0.0f : c;      // score scale (log2 units); 0: equal scores
    const float dm = none ? 0.0f : 1.0f;   // 0: no gradient through the scores
    int kmin = klim;                        // smallest key limit in the wave
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmin = min(kmin, __shfl_xor(kmin, o));
    kmin = __builtin_amdgcn_readfirstlane(kmin);
    // Keys this workgroup must visit: up to the causal bound unless lengths
    // are given (a fully masked row then spans all keys).
    const int kv_end = (kCausal && a.vl_rank == 0) ? min(Lk, q_wg + kRowsWg) : Lk;
    const int n_steps = (kv_end + kStep - 1) / kStep;

    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const bf16_t* gp = static_cast<const bf16_t*>(a.dout) + b * a.sdo[0] + hd * a.sdo[1];
    const bf16_t* op = static_cast<const bf16_t*>(a.o) + b * a.so[0] + hd * a.so[1];
    const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1];

    const StepSrc ksrc = step_src(kp, a.sk[2], Lk, tid), vsrc = step_src(vp, a.sv[2], Lk, tid);
    Chunks nk = load_step(ksrc, 0);

    // Q and dO fragments (B operands: query lane%32, features kk*16 + hb*8 ..).
    bf16x8 qf[4], gf[4];
    float dsum = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 rq = make_uint4(0, 0, 0, 0), rg = rq, ro = rq;
        if (live) {
            rq = *reinterpret_cast<const uint4*>(qp + (long long)i * a.sq[2] + kk * 16 + hb * 8);
            rg = *reinterpret_cast<const uint4*>(gp + (long long)i * a.sdo[2] + kk * 16 + hb * 8);
            ro = *reinterpret_cast<const uint4*>(op + (long long)i * a.so[2] + kk * 16 + hb * 8);
        }
        qf[kk] = __builtin_bit_cast(bf16x8, rq);
        gf[kk] = __builtin_bit_cast(bf16x8, rg);
        const uint32_t ug[4] = {rg.x, rg.y, rg.z, rg.w}, uo[4] = {ro.x, ro.y, ro.z, ro.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dsum += __uint_as_float(ug[e] << 16) * __uint_as_float(uo[e] << 16) +
                    __uint_as_float(ug[e] & 0xffff0000u) * __uint_as_float(uo[e] & 0xffff0000u);
    }
    dsum = pair_sum(dsum);                  // D_i over both lane halves

    // ---- one pass: online softmax with a lazy offset ----
    // dq accumulates exp2(s - m) (dp - D) k with the offset m of this lane's
    // query (equal on both lane halves); m moves only when a tile's max
    // exceeds it by more than kLazy, and then dq and the weight sum l (this
    // lane half's keys) are rescaled.  The phases merge at the end.
    constexpr float kLazy = 10.0f;
    const float ddm = dsum * dm;
    float m = -INFINITY, l = 0.0f;
    f32x16 dq[2] = {};
    Chunks nv = load_step(vsrc, 0);
    for (int st = 0; st < n_steps; ++st) {
        __syncthreads();
        store_step(nk, smem, kRowsPhase, kRowsKR, kRowsKT, tid);
        store_step(nv, smem, kRowsPhase, kRowsVR, -1, tid);
        if (st + 1 < n_steps) {
            nk = load_step(ksrc, (st + 1) * kStep);
            nv = load_step(vsrc, (st + 1) * kStep);
        }
        __syncthreads();
        const int t0 = st * kStep + ph * kTile;   // this wave's keys t0 .. t0+31
        const char* area = smem + ph * kRowsPhase;
        const f32x16 s = tile_dot(reinterpret_cast<const bf16_t*>(area + kRowsKR), qf, l32, hb);
        f32x16 ds = tile_dot(reinterpret_cast<const bf16_t*>(area + kRowsVR), gf, l32, hb);
        // The tile's row max in log2 units (raw scores times cs >= 0; masked
        // keys excluded), then the weights exp2(s * cs - m) (masked: 0).
        const bool full = t0 + kTile <= kmin;
        const int rel = klim - (t0 + hb * 4);
        float mx = -INFINITY;
        if (full) {
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, acc_row(v) < rel ? s[v] : -INFINITY);
        }
        float mt = mx == -INFINITY ? -INFINITY : mx * cs;
        mt = pair_max(mt);
        if (__any(mt > m + kLazy)) {
            const float m_new = mt > m + kLazy ? mt : m;
            const float alpha = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
            l *= alpha;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                dq[0][v] *= alpha;
                dq[1][v] *= alpha;
            }
            m = m_new;
        }
        const float m_use = m == -INFINITY ? 0.0f : m;   // no allowed key yet: every weight is 0
        float rs = 0.0f;
        if (full) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = __builtin_amdgcn_exp2f(fmaf(s[v], cs, -m_use));
                rs += p;
                ds[v] = p * fmaf(ds[v], dm, -ddm);
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float e = __builtin_amdgcn_exp2f(fmaf(s[v], cs, -m_use));
                const float p = acc_row(v) < rel ? e : 0.0f;
                rs += p;
                ds[v] = p * fmaf(ds[v], dm, -ddm);
            }
        }
        l += rs;
        u32x4 w[2];
        pack_b(ds, w);
        const bf16_t* kt = reinterpret_cast<const bf16_t*>(area + kRowsKT);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 d8 = __builtin_bit_cast(bf16x8, w[kb]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) dq[tb] = mfma32x32x16(tr_frag(kt, kb, tb, hb, lane), d8, dq[tb]);
        }
    }
    // Merge the phases: common offset M, total weight L, rescaled dq.
    stat_s[grp][ph][hb][l32] = make_float2(m, l);
    __syncthreads();
    float M = -INFINITY;
#pragma unroll
    for (int p = 0; p < kPhases; ++p) M = fmaxf(M, stat_s[grp][p][0][l32].x);
    float L = 0.0f;
#pragma unroll
    for (int p = 0; p < kPhases; ++p)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float2 x = stat_s[grp][p][h][l32];
            L += x.x == -INFINITY ? 0.0f : x.y * __builtin_amdgcn_exp2f(x.x - M);
        }
    const float own = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        dq[0][v] *= own;
        dq[1][v] *= own;
    }
    // v_log_f32 is the base-2 logarithm, matching the log2-unit scores.
    const float lse = L > 0.0f ? M + __builtin_amdgcn_logf(L) : 0.0f;
    __syncthreads();
    reduce_write(reinterpret_cast<float*>(smem), dq, grp, ph, lane);
    __syncthreads();
    reduce_read(reinterpret_cast<const float*>(smem), dq, grp, ph, lane);
    if (ph != 0 || !live) return;
    if (hb == 0) {
        a.rows[((long long)bh * Lq + i) * 2] = lse;
        a.rows[((long long)bh * Lq + i) * 2 + 1] = dsum;
    }
    store_rowT(a.dq, b * a.sdq[0] + hd * a.sdq[1] + (long long)i * a.sdq[2], a.out_f32, dq,
               L > 0.0f ? 0.125f / L : 0.0f, hb);
}

// ---------------------------------------------------------------------------
// keys: dk, dv
// ---------------------------------------------------------------------------
constexpr int kKeysQR = 0;                        // Q, 144-byte rows
constexpr int kKeysQT = kTileRB;                  // Q, 192-byte rows
constexpr int kKeysGR = kTileRB + kTileTB;        // dO, 144-byte rows
constexpr int kKeysGT = 2 * kTileRB + kTileTB;    // dO, 192-byte rows
constexpr int kKeysPhase = 2 * kTileRB + 2 * kTileTB;

template <bool kCausal>
__global__ __launch_bounds__(kThreads, 1) void bwd_keys_mfma(BackwardArgs a, float c) {
    __shared__ __attribute__((aligned(16))) char smem[kPhases * kKeysPhase];
    __shared__ float4 rowf_s[kStep];   // per streamed query: log-sum-exp, D, score scale, gradient factor
    __shared__ int klim_s[kStep];      // per streamed query: key limit
    __shared__ int tmin_s[kPhases];    // per phase tile: smallest key limit (-1 if a row has none allowed)

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave % kGroups, ph = wave / kGroups;
    const int hb = lane >> 5, l32 = lane & 31;
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    const int b = bh / a.H, hd = bh % a.H;
    const int k_wg = (blockIdx.x / BH) * kRowsWg;   // causal: early keys see the most queries and go first
    const int j = k_wg + grp * 32 + l32;            // this lane's key
    const int j_last = k_wg + grp * 32 + 31;
    const int Lq = a.Lq, Lk = a.Lk;

    const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1];
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const bf16_t* gp = static_cast<const bf16_t*>(a.dout) + b * a.sdo[0] + hd * a.sdo[1];

    // Causal without lengths: queries before the workgroup's first key
    // weight none of its keys.
    const int i_begin = (kCausal && a.vl_rank == 0) ? k_wg : 0;
    const int n_steps = (Lq - i_begin + kStep - 1) / kStep;
    const StepSrc qsrc = step_src(qp, a.sq[2], Lq, tid), gsrc = step_src(gp, a.sdo[2], Lq, tid);
    Chunks nq = load_step(qsrc, i_begin);
    Chunks ng = load_step(gsrc, i_begin);

    // K and V fragments (B operands: key lane%32, features kk*16 + hb*8 ..).
    bf16x8 kf[4], vf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 rk = make_uint4(0, 0, 0, 0), rv = rk;
        if (j < Lk) {
            rk = *reinterpret_cast<const uint4*>(kp + (long long)j * a.sk[2] + kk * 16 + hb * 8);
            rv = *reinterpret_cast<const uint4*>(vp + (long long)j * a.sv[2] + kk * 16 + hb * 8);
        }
        kf[kk] = __builtin_bit_cast(bf16x8, rk);
        vf[kk] = __builtin_bit_cast(bf16x8, rv);
    }

    // Per streamed query (threads below kStep): log-sum-exp, D and key limit,
    // fetched one step ahead like the tiles.
    struct RowData {
        float lse, dsum;
        int kl;
        bool none;
    };
    auto fetch_rows = [&](int i0) {
        RowData r = {0.0f, 0.0f, 0, false};
        const int qi = i0 + tid;
        if (tid < kStep && qi < Lq) {
            r.lse = a.rows[((long long)bh * Lq + qi) * 2];
            r.dsum = a.rows[((long long)bh * Lq + qi) * 2 + 1];
            r.kl = key_limit<kCausal>(a, b, qi, r.none);
        }
        return r;
    };
    RowData nr = fetch_rows(i_begin);

    f32x16 dk[2] = {}, dv[2] = {};
    for (int st = 0; st < n_steps; ++st) {
        const int i0 = i_begin + st * kStep;
        __syncthreads();
        store_step(nq, smem, kKeysPhase, kKeysQR, kKeysQT, tid);
        store_step(ng, smem, kKeysPhase, kKeysGR, kKeysGT, tid);
        if (tid < kStep) {
            rowf_s[tid] = make_float4(nr.lse, nr.dsum, nr.none ? 0.0f : c, nr.none ? 0.0f : 1.0f);
            klim_s[tid] = nr.kl;
            int mn = nr.none ? -1 : nr.kl;
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) mn = min(mn, __shfl_xor(mn, o));
            if ((tid & 31) == 0) tmin_s[tid >> 5] = mn;
        }
        if (st + 1 < n_steps) {
            nq = load_step(qsrc, i0 + kStep);
            ng = load_step(gsrc, i0 + kStep);
            nr = fetch_rows(i0 + kStep);
        }
        __syncthreads();
        // S = Q K^T and dP = dO V^T: element v is query ph*32 + acc_row(v) +
        // hb*4 of this step, key j.
        const char* area = smem + ph * kKeysPhase;
        f32x16 p = tile_dot(reinterpret_cast<const bf16_t*>(area + kKeysQR), kf, l32, hb);
        f32x16 ds = tile_dot(reinterpret_cast<const bf16_t*>(area + kKeysGR), vf, l32, hb);
        const int rb = ph * kTile + hb * 4;
        if (j_last < __builtin_amdgcn_readfirstlane(tmin_s[ph])) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float4 rf = rowf_s[rb + acc_row(v)];
                const float e = __builtin_amdgcn_exp2f(fmaf(p[v], c, -rf.x));
                p[v] = e;
                ds[v] = e * (ds[v] - rf.y);
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float4 rf = rowf_s[rb + acc_row(v)];
                const int kl = klim_s[rb + acc_row(v)];
                const float e = j < kl ? __builtin_amdgcn_exp2f(fmaf(p[v], rf.z, -rf.x)) : 0.0f;
                p[v] = e;
                ds[v] = e * (ds[v] - rf.y) * rf.w;
            }
        }
        u32x4 pw[2], dw[2];
        pack_b(p, pw);
        pack_b(ds, dw);
        const bf16_t* qt = reinterpret_cast<const bf16_t*>(area + kKeysQT);
        const bf16_t* gt = reinterpret_cast<const bf16_t*>(area + kKeysGT);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 p8 = __builtin_bit_cast(bf16x8, pw[kb]), d8 = __builtin_bit_cast(bf16x8, dw[kb]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                dv[tb] = mfma32x32x16(tr_frag(gt, kb, tb, hb, lane), p8, dv[tb]);
                dk[tb] = mfma32x32x16(tr_frag(qt, kb, tb, hb, lane), d8, dk[tb]);
            }
        }
    }
    float* red = reinterpret_cast<float*>(smem);
    __syncthreads();
    reduce_write(red, dv, grp, ph, lane);
    __syncthreads();
    reduce_read(red, dv, grp, ph, lane);
    __syncthreads();
    reduce_write(red, dk, grp, ph, lane);
    __syncthreads();
    reduce_read(red, dk, grp, ph, lane);
    if (ph != 0 || j >= Lk) return;
    store_rowT(a.dk, b * a.sdk[0] + hd * a.sdk[1] + (long long)j * a.sdk[2], a.out_f32, dk, 1.0f / 8.0f, hb);
    store_rowT(a.dv, b * a.sdv[0] + hd * a.sdv[1] + (long long)j * a.sdv[2], a.out_f32, dv, 1.0f, hb);
}

static_assert(kGroups * (kPhases - 1) * 32 * 64 * 4 <= kPhases * kRowsPhase, "reduction slots fit the rows tiles");
static_assert(kGroups * (kPhases - 1) * 32 * 64 * 4 <= kPhases * kKeysPhase, "reduction slots fit the keys tiles");

template <bool kCausal>
hipError_t launch_variant(const BackwardArgs& a, hipStream_t s) {
    const float c = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    const long long BH = (long long)a.B * a.H;
    const long long gq = BH * ((a.Lq + kRowsWg - 1) / kRowsWg), gk = BH * ((a.Lk + kRowsWg - 1) / kRowsWg);
    if (gq == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_rows_mfma<kCausal>), dim3((unsigned)gq), dim3(kThreads), 0, s, a, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_keys_mfma<kCausal>), dim3((unsigned)gk), dim3(kThreads), 0, s, a, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sdpa_backward_bf16(const BackwardArgs& a, hipStream_t s) {
    if (!fits_buffer(a.sq[2], a.Lq) || !fits_buffer(a.sdo[2], a.Lq) || !fits_buffer(a.sk[2], a.Lk) ||
        !fits_buffer(a.sv[2], a.Lk))
        return hipErrorInvalidValue;
    return a.causal ? launch_variant<true>(a, s) : launch_variant<false>(a, s);
}

}  // namespace mha
