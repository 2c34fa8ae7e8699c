// Multi-head attention with the Q/K/V projections fused into the attention
// kernel (bf16 in, fp32 accumulate, d_k = d_v = 64), gfx950.
//
// What it computes ("Transformer" study notes, multi-head attention section;
// The Annotated Transformer, "Attention" section): for head h,
//   Q = X_q W_Q[h]^T + b_Q[h],  K = X_kv W_K[h]^T + b_K[h],  V = X_kv W_V[h]^T + b_V[h]
// (W[h] = rows h*64 .. h*64+63 of the d_model x d_model weight), then
//   o_i = sum_j softmax_j(q_i . k_j / sqrt(d_k)) v_j
// over the keys allowed by the key-padding length and the causal rule, stored
// at columns h*64 .. h*64+63 of the merged-head output [B, Lq, d_model].
// Masked scores are replaced by -1e9 in the pages' code: weight exactly zero
// whenever a row has an allowed key, uniform weights over all Lk keys when it
// has none.  The output projection runs afterwards as a GEMM.
//
// Design.
//  * One workgroup = 8 wave64s for one (batch, head) and a block of 256
//    queries; each wave owns 32 queries.  Q, K and V never go to HBM: the
//    workgroup projects its own queries once, then walks the keys in chunks
//    of 128, projecting each chunk's K and V into LDS and attending to it.
//  * Projections are MFMA GEMMs over d_model in 64-wide slices whose operand
//    tiles are copied straight into LDS (global_load_lds_dwordx4, two
//    stages).  They compute the transposed product W X^T, so each lane holds
//    one query or key and 4-feature runs of its 32-feature block.
//  * Q is scaled by log2(e)/sqrt(d_k) and K kept as well, each as a bf16
//    pair hi + lo (~16 significant bits), and scores are formed from three
//    products Kh Qh^T + Kl Qh^T + Kh Ql^T: large logits (embeddings scaled by
//    sqrt(d_model)) then do not flip near-tied softmax rows.  The feature
//    order inside each 16-feature MFMA step is the order in which a lane's Q
//    projection result arrives; K is written to LDS in that same order, so Q
//    fragments come straight from the projection accumulators.
//  * The score accumulator starts from -m (the row's exponent offset) instead
//    of zero, so the weights are exp2 of the accumulator with no per-score
//    VALU scaling.  m is the row max of the first key tile; a later tile whose
//    weights sum past 2^20 in a lane folds its max into m, rescales the
//    accumulators and is recomputed.  Masks are evaluated only on tiles that
//    cross the valid length or the diagonal; K/V rows past the valid length
//    (or above the workgroup's diagonal) are never projected.
#include "common.h"
#include "kernels.h"
#include "lds_tile.h"

namespace mha {

namespace {

constexpr int kW = 8;                    // waves per workgroup
constexpr int kThreads = 64 * kW;
constexpr int kBQ = 32 * kW;             // queries per workgroup
constexpr int kKC = 128;                 // keys per chunk
constexpr int kHd = 64;                  // d_k = d_v
constexpr int kLdsV = kHd + 32;          // V rows in LDS (192 B: conflict-free transpose reads)
constexpr float kSumLimit = 1048576.0f;  // 2^20

// LDS: two projection stages (the larger of X_q 256 rows + W_Q 64 rows and
// X_kv 128 rows + W_K, W_V 128 rows, 144 B each), then the chunk's K hi, K lo
// ([128][72] bf16 each) and V ([128][96] bf16).
constexpr int kStageBytes = (kBQ + kHd) * kTileRowBytes;          // 46080
constexpr int kKhOff = 2 * kStageBytes;
constexpr int kKlOff = kKhOff + kKC * kTileRowBytes;
constexpr int kVOff = kKlOff + kKC * kTileRowBytes;
constexpr int kLdsBytes = kVOff + kKC * kLdsV * 2;                // 153600

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 frag(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// 4 consecutive bf16 of a bias vector (or zeros).
__device__ __forceinline__ void bias4(const bf16_t* b, int f, float (&r)[4]) {
    if (!b) {
        r[0] = r[1] = r[2] = r[3] = 0.0f;
        return;
    }
    const uint2 w = *reinterpret_cast<const uint2*>(b + f);
    r[0] = __uint_as_float(w.x << 16);
    r[1] = __uint_as_float(w.x & 0xffff0000u);
    r[2] = __uint_as_float(w.y << 16);
    r[3] = __uint_as_float(w.y & 0xffff0000u);
}

// V^T fragment for key slice kb (16 keys) and features tb*32 + (lane % 32),
// read from V rows [key][feature] with the LDS transpose read: in each
// 16-lane group, lane r points at key row base + r/4, features T + (r%4)*4;
// lane j of the group receives features T + j of keys base .. base+3.
__device__ __forceinline__ bf16x8 v_frag(const bf16_t* vs, int kb, int tb, int hb, int lane) {
    const int g = lane >> 4, r = lane & 15;
    const int row = kb * 16 + hb * 4 + (r >> 2);
    const int col = tb * 32 + (g & 1) * 16 + (r & 3) * 4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vs + row * kLdsV + col));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vs + (row + 8) * kLdsV + col));
    const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, both);
}

// Row max over a 64-key tile (both lane halves).
__device__ __forceinline__ float tile_max(const f32x16 (&s)[2]) {
    float mr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) mr[r] = fmaxf(s[0][r], s[1][r]);
#pragma unroll
    for (int v = 4; v < 16; v += 4)
#pragma unroll
        for (int r = 0; r < 4; ++r) mr[r] = fmaxf(mr[r], fmaxf(s[0][v + r], s[1][v + r]));
    return pair_max(fmaxf(fmaxf(mr[0], mr[1]), fmaxf(mr[2], mr[3])));
}

// Weights exp2(s) packed as the B operand of O^T += V^T P^T (slice kb covers
// keys kb*16 + (e/4)*8 + hb*4 + e%4); returns this lane's sum of the rounded
// weights.
__device__ __forceinline__ float weights(const f32x16 (&s)[2], u32x4 (&w)[4]) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int v = (kb & 1) * 8 + e;
            const float p0 = __builtin_amdgcn_exp2f(s[kb >> 1][v]);
            const float p1 = __builtin_amdgcn_exp2f(s[kb >> 1][v + 1]);
            const bf16x2 pp = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
            w[kb][e >> 1] = __builtin_bit_cast(uint32_t, pp);
            acc[kb & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc[kb & 1], false);
        }
    }
    return acc[0] + acc[1];
}

__device__ __forceinline__ void sub_all(f32x16 (&s)[2], float d) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        s[0][v] -= d;
        s[1][v] -= d;
    }
}

template <bool kCausal, bool kHasVl>
__global__ __launch_bounds__(kThreads, 1) void mha_attn_fused_bf16(FusedArgs a, int n_qtiles, float c) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hb = lane >> 5, l32 = lane & 31;

    // Workgroup -> (query block, batch, head).  Causal launches issue the
    // longest query blocks first.  The hardware deals workgroup ids to the
    // eight XCDs round-robin; when B is a multiple of 8, XCD x gets the
    // batches b = x (mod 8) with all their heads, so every head's workgroup
    // re-reads that batch's inputs from the same L2.
    int qt, b, hd;
    if (a.B % 8 == 0) {
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
        const int per_q = (a.B >> 3) * a.H;
        qt = j / per_q;
        const int rem = j % per_q;
        b = x + 8 * (rem / a.H);
        hd = rem % a.H;
    } else {
        const int BH = a.B * a.H;
        const int bh = blockIdx.x % BH;
        qt = blockIdx.x / BH;
        b = bh / a.H;
        hd = bh % a.H;
    }
    if (kCausal) qt = n_qtiles - 1 - qt;
    const int D = a.D, Lq = a.Lq, Lk = a.Lk;
    const int nd = D / 64;

    const int q_wg = qt * kBQ;
    const int q0 = q_wg + wave * 32;          // this wave's first query
    const int i = q0 + l32;                   // this lane's query
    const bool active = q0 < Lq;              // wave-uniform: the wave has queries

    const int vlen = kHasVl ? a.valid_lens[b] : Lk;
    const bool none = vlen <= 0;              // every key masked -> uniform weights
    const int kv_lim = none ? Lk : min(vlen, Lk);
    int kv_end = kv_lim;
    if (kCausal && !none) kv_end = min(kv_end, q_wg + kBQ);
    // This wave's keys lie below w_end; keys below key_lim are allowed for this lane.
    const int w_end = (kCausal && !none) ? min(kv_end, q0 + 32) : kv_end;
    const int key_lim = none ? Lk : (kCausal ? min(kv_lim, i + 1) : kv_lim);

    const bf16_t* xq = static_cast<const bf16_t*>(a.x_q) + (long long)b * Lq * D;
    const bf16_t* xkv = static_cast<const bf16_t*>(a.x_kv) + (long long)b * Lk * D;
    const bf16_t* wq = static_cast<const bf16_t*>(a.w_q) + (long long)hd * kHd * D;
    const bf16_t* wk = static_cast<const bf16_t*>(a.w_k) + (long long)hd * kHd * D;
    const bf16_t* wv = static_cast<const bf16_t*>(a.w_v) + (long long)hd * kHd * D;
    const bf16_t* bq = a.b_q ? static_cast<const bf16_t*>(a.b_q) + hd * kHd : nullptr;
    const bf16_t* bk = a.b_k ? static_cast<const bf16_t*>(a.b_k) + hd * kHd : nullptr;
    const bf16_t* bv = a.b_v ? static_cast<const bf16_t*>(a.b_v) + hd * kHd : nullptr;

    // Projection loads go to stage gstep & 1, gstep counting 64-wide slices
    // over both phases; the last slice of one phase prefetches the first slice
    // of the next, so no phase starts on a cold load.
    int gstep = 0;
    LdsTileLoader<kKC, kW> lkx;       // X_kv rows of the current key chunk
    LdsTileLoader<kHd, kW> lkw;       // W_K[h] and W_V[h] rows 0..63 each
    LdsTileLoader<kHd, kW> lvw;
    lkw.init(wave, lane, wk, 0, kHd, D);
    lvw.init(wave, lane, wv, 0, kHd, D);
    lkx.init(wave, lane, xkv, 0, Lk, D);
    auto kv_issue = [&](int stage, int d0) {
        unsigned char* base = smem + stage * kStageBytes;
        lkx.issue(d0, base, wave);
        lkw.issue(d0, base + kKC * kTileRowBytes, wave);
        lvw.issue(d0, base + (kKC + kHd) * kTileRowBytes, wave);
    };

    // ---------------- Q projection: Q^T (64 x 256) = W_Q[h] X_q^T -------------
    bf16x8 qh[4], ql[4];
    {
        LdsTileLoader<kBQ, kW> lx;
        LdsTileLoader<kHd, kW> lw;
        // Query rows past Lq only feed their own (never stored) outputs.
        lx.init(wave, lane, xq, q_wg, Lq, D, true);
        lw.init(wave, lane, wq, 0, kHd, D);
        auto issue = [&](int stage, int d0) {
            unsigned char* base = smem + stage * kStageBytes;
            lx.issue(d0, base, wave);
            lw.issue(d0, base + kBQ * kTileRowBytes, wave);
        };
        f32x16 acc[2] = {};
        issue(0, 0);
        for (int dt = 0; dt < nd; ++dt, ++gstep) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (dt + 1 < nd) issue((gstep + 1) & 1, (dt + 1) * 64);
            else kv_issue((gstep + 1) & 1, 0);
            const bf16_t* xs = reinterpret_cast<const bf16_t*>(smem + (gstep & 1) * kStageBytes);
            const bf16_t* ws = xs + kBQ * kTileLdsRow;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 xf = frag(xs + (wave * 32 + l32) * kTileLdsRow + kk * 16 + hb * 8);
#pragma unroll
                for (int fb = 0; fb < 2; ++fb)
                    acc[fb] = mfma32x32x16(frag(ws + (fb * 32 + l32) * kTileLdsRow + kk * 16 + hb * 8), xf, acc[fb]);
            }
        }
        // acc[fb][v]: query i, feature fb*32 + (v/4)*8 + hb*4 + v%4.  It becomes
        // element v%8 of MFMA step kk = 2*fb + v/8 (the step's feature order).
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float bb[4];
                bias4(bq, fb * 32 + g * 8 + hb * 4, bb);
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int v = g * 4 + e4;
                    const float x = (acc[fb][v] + bb[e4]) * c;
                    const __bf16 h = static_cast<__bf16>(x);
                    qh[2 * fb + (v >> 3)][v & 7] = h;
                    ql[2 * fb + (v >> 3)][v & 7] = static_cast<__bf16>(x - static_cast<float>(h));
                }
            }
        }
    }

    // ---------------- key chunks: project K, V into LDS, attend --------------
    bf16_t* kh_s = reinterpret_cast<bf16_t*>(smem + kKhOff);
    bf16_t* kl_s = reinterpret_cast<bf16_t*>(smem + kKlOff);
    bf16_t* v_s = reinterpret_cast<bf16_t*>(smem + kVOff);
    // Projection work split: wave -> tensor t (K or V), feature block fb, key
    // blocks kbp and kbp + 1 of the chunk (32 keys each).
    const int pt = wave >> 2, pfb = (wave >> 1) & 1, pkb = (wave & 1) * 2;

    f32x16 o[2] = {};                 // O^T accumulators: features [0,32) and [32,64)
    f32x16 bias = {};                 // -m in every element (score accumulator start)
    bool have_m = false;              // wave-uniform: the offset has been set
    float l = 0.0f;                   // this lane's share of the weight sum
    for (int k0 = 0; k0 < kv_end; k0 += kKC) {
        f32x16 acc[2] = {};
        for (int dt = 0; dt < nd; ++dt, ++gstep) {
            // Also orders the previous chunk's attention (LDS reads of K, V)
            // before this chunk's K, V are written below.
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (dt + 1 < nd) {
                kv_issue((gstep + 1) & 1, (dt + 1) * 64);
            } else if (k0 + kKC < kv_end) {
                lkx.init(wave, lane, xkv, k0 + kKC, Lk, D);
                kv_issue((gstep + 1) & 1, 0);
            }
            const bf16_t* xs = reinterpret_cast<const bf16_t*>(smem + (gstep & 1) * kStageBytes);
            const bf16_t* ws = xs + kKC * kTileLdsRow;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 wf = frag(ws + (pt * kHd + pfb * 32 + l32) * kTileLdsRow + kk * 16 + hb * 8);
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[j] = mfma32x32x16(wf, frag(xs + ((pkb + j) * 32 + l32) * kTileLdsRow + kk * 16 + hb * 8),
                                          acc[j]);
            }
        }
        // acc[j][v]: key k0 + (pkb+j)*32 + l32, feature pfb*32 + (v/4)*8 + hb*4 + v%4.
        // K goes to LDS in the MFMA step order (step kk = 2*pfb + v/8 holds
        // it at element v%8 of lane half hb, i.e. column kk*16 + hb*8 + v%8);
        // V in natural [key][feature] order.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = (pkb + j) * 32 + l32;
            float bb[4][4];
#pragma unroll
            for (int g = 0; g < 4; ++g) bias4(pt == 0 ? bk : bv, pfb * 32 + g * 8 + hb * 4, bb[g]);
            if (pt == 0) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    uint32_t hw[4], lw4[4];
#pragma unroll
                    for (int e = 0; e < 8; e += 2) {
                        const int v = half * 8 + e;
                        const float x0 = acc[j][v] + bb[v >> 2][v & 3];
                        const float x1 = acc[j][v + 1] + bb[(v + 1) >> 2][(v + 1) & 3];
                        hw[e >> 1] = pack_bf16x2(x0, x1);
                        lw4[e >> 1] = pack_bf16x2(x0 - __uint_as_float(hw[e >> 1] << 16),
                                                  x1 - __uint_as_float(hw[e >> 1] & 0xffff0000u));
                    }
                    const int col = (2 * pfb + half) * 16 + hb * 8;
                    *reinterpret_cast<uint4*>(kh_s + row * kTileLdsRow + col) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                    *reinterpret_cast<uint4*>(kl_s + row * kTileLdsRow + col) =
                        make_uint4(lw4[0], lw4[1], lw4[2], lw4[3]);
                }
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int v = g * 4;
                    *reinterpret_cast<uint2*>(v_s + row * kLdsV + pfb * 32 + g * 8 + hb * 4) =
                        make_uint2(pack_bf16x2(acc[j][v] + bb[g][0], acc[j][v + 1] + bb[g][1]),
                                   pack_bf16x2(acc[j][v + 2] + bb[g][2], acc[j][v + 3] + bb[g][3]));
                }
            }
        }
        __syncthreads();

        if (active) {
#pragma unroll 1
            for (int st = 0; st < 2; ++st) {
                const int kv0 = k0 + st * 64;
                if (kv0 >= w_end) break;
                // ---- scores (log2 units, offset by -m) ----
                f32x16 s[2];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) {
                        const int r = (st * 64 + jb * 32 + l32) * kTileLdsRow + kk * 16 + hb * 8;
                        const bf16x8 kfh = frag(kh_s + r), kfl = frag(kl_s + r);
                        s[jb] = mfma32x32x16(kfh, qh[kk], kk == 0 ? bias : s[jb]);
                        s[jb] = mfma32x32x16(kfl, qh[kk], s[jb]);
                        s[jb] = mfma32x32x16(kfh, ql[kk], s[jb]);
                    }
                }
                // ---- masks: only tiles crossing the valid length or diagonal ----
                if (none || kv0 + 64 > kv_lim || (kCausal && kv0 + 63 > q0)) {
                    const int rel = key_lim - (kv0 + hb * 4);
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int jr = (v >> 2) * 8 + (v & 3);
                        s[0][v] = jr < rel ? (none ? 0.0f : s[0][v]) : -INFINITY;
                        s[1][v] = jr + 32 < rel ? (none ? 0.0f : s[1][v]) : -INFINITY;
                    }
                }
                if (!have_m) {
                    // First tile: the offset becomes its row max (every row has
                    // an allowed key in tile 0).
                    const float m = tile_max(s);
                    sub_all(s, m);
#pragma unroll
                    for (int v = 0; v < 16; ++v) bias[v] = -m;
                    have_m = true;
                }
                u32x4 p[4];
                float r = weights(s, p);
                if (__any(r > kSumLimit)) {
                    // Weights outgrew the offset: fold the tile max into it.
                    const float d = fmaxf(tile_max(s), 0.0f);
                    const float alpha = __builtin_amdgcn_exp2f(-d);
                    l *= alpha;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        o[0][v] *= alpha;
                        o[1][v] *= alpha;
                        bias[v] -= d;
                    }
                    sub_all(s, d);
                    r = weights(s, p);
                }
                l += r;
                // ---- O^T += V^T P^T ----
                const bf16_t* vs = v_s + st * 64 * kLdsV;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    const bf16x8 pk = __builtin_bit_cast(bf16x8, p[kb]);
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) o[tb] = mfma32x32x16(v_frag(vs, kb, tb, hb, lane), pk, o[tb]);
                }
            }
        }
    }

    if (!active) return;
    const float inv = 1.0f / pair_sum(l);
    // O^T element v of block tb: feature tb*32 + (v/4)*8 + hb*4 + v%4, query i.
    // The wave stages its 32 x 64 bf16 result in its own slice of the
    // projection stages (no wave reads them once the last chunk is
    // projected) and stores whole 128-byte head rows.
    bf16_t* o_s = reinterpret_cast<bf16_t*>(smem + wave * 32 * kTileRowBytes);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int tt = tb * 32 + g4 * 8 + hb * 4;
            *reinterpret_cast<uint2*>(o_s + l32 * kTileLdsRow + tt) =
                make_uint2(pack_bf16x2(o[tb][g4 * 4] * inv, o[tb][g4 * 4 + 1] * inv),
                           pack_bf16x2(o[tb][g4 * 4 + 2] * inv, o[tb][g4 * 4 + 3] * inv));
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // 8 lanes per row, 16 bytes each; rows past Lq are not stored.
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
        const int r = pass * 8 + (lane >> 3), c8 = (lane & 7) * 8;
        if (q0 + r < Lq)
            *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.o) + ((long long)b * Lq + q0 + r) * D + hd * kHd + c8) =
                *reinterpret_cast<const uint4*>(o_s + r * kTileLdsRow + c8);
    }
}

template <bool kCausal, bool kHasVl>
hipError_t launch_variant(const FusedArgs& a, hipStream_t s) {
    const int n_qtiles = (a.Lq + kBQ - 1) / kBQ;
    const long long grid = (long long)n_qtiles * a.B * a.H;
    const float c = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    hipLaunchKernelGGL((mha_attn_fused_bf16<kCausal, kHasVl>), dim3((unsigned)grid), dim3(kThreads), 0, s, a,
                       n_qtiles, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mha_attn_fused(const FusedArgs& a, hipStream_t s) {
    if (a.D % 64 != 0) return hipErrorInvalidValue;
    if (mha_attn_fused_small_fits(a)) return launch_mha_attn_fused_small(a, s);
    const bool c = a.causal != 0, v = a.valid_lens != nullptr;
    if (c) return v ? launch_variant<true, true>(a, s) : launch_variant<true, false>(a, s);
    return v ? launch_variant<false, true>(a, s) : launch_variant<false, false>(a, s);
}

}  // namespace mha
