// Multi-head self-attention for sequences of at most 128 positions with the
// Q/K/V projections fused in (bf16 in, fp32 accumulate, d_k = d_v = 64),
// gfx950.
//
// What it computes is the same as the general fused kernel ("Transformer"
// study notes, multi-head attention section; The Annotated Transformer,
// "Attention" section): for head h of batch b,
//   Q = X W_Q[h]^T + b_Q[h],  K = X W_K[h]^T + b_K[h],  V = X W_V[h]^T + b_V[h]
//   o_i = sum_j softmax_j(q_i . k_j / sqrt(d_k)) v_j
// over the keys the key-padding length and the causal rule allow (masked
// scores are the pages' -1e9 fill: weight exactly zero when a row has an
// allowed key, uniform weights over all L keys when it has none), stored at
// columns h*64 .. h*64+63 of the merged-head output [B, L, d_model].
//
// Design for L <= 128 (one workgroup of 8 wave64s per (batch, head)):
//  * Queries and keys are the same 128 rows of X, so Q, K and V come out of
//    one pass over d_model: each 64-wide slice stages X (128 rows) and the
//    three weight slices (64 rows each) in LDS (global_load_lds_dwordx4,
//    three stages so two slices are in flight, 144-byte rows).  The 24
//    output blocks (32 rows x 32 features of Q, K, V) are dealt 3 per wave:
//    wave w takes rows 32*(w%4) .. +31 and feature blocks Q0, Q1, K0 (w < 4)
//    or K1, V0, V1 (w >= 4), so per MFMA step it reads one X fragment and
//    three weight fragments for three MFMAs.
//  * Q is scaled by log2(e)/sqrt(d_k) and kept, like K, as a bf16 pair
//    hi + lo; scores are formed from three products Kh Qh^T + Kl Qh^T +
//    Kh Ql^T, so large logits (embeddings scaled by sqrt(d_model)) keep
//    near-fp32 accuracy.  Waves 0-3 hand their Q fragments to waves 4-7
//    through LDS.
//  * Attention is split over the keys: wave w takes queries 32*(w%4) .. +31
//    against keys 64*(w/4) .. +63.  Each half is a single 64-key tile, so
//    its weights are exp2 of the scores minus the exact row max of the tile.
//    Waves 4-7 then pass (max, weight sum, unnormalised output) through LDS
//    and waves 0-3 merge the halves by rescaling to the common max (the
//    online-softmax merge) and store the normalised result.
#include "common.h"
#include "kernels.h"
#include "lds_tile.h"

namespace mha {

namespace {

constexpr int kW = 8;                    // waves per workgroup
constexpr int kThreads = 64 * kW;
constexpr int kL = 128;                  // positions per workgroup (queries = keys)
constexpr int kHd = 64;                  // d_k = d_v
constexpr int kLdsV = kHd + 32;          // V rows in LDS (192 B: conflict-free transpose reads)
constexpr int kPart = 2 * 16 + 2;        // floats a key-half wave hands over per lane: O^T, max, sum

// LDS: three projection stages (X rows 0..127, then W_Q, W_K, W_V rows,
// 144 B each).  Once the projection is done the same bytes hold K hi, K lo
// ([128][72] bf16 each), V ([128][96] bf16) and after them the Q hand-over
// (32 KB), later reused for the partial results of the second key half
// (4 x 34 x 64 floats).
constexpr int kStages = 3;
constexpr int kStageBytes = (kL + 3 * kHd) * kTileRowBytes;      // 46080
constexpr int kLdsBytes = kStages * kStageBytes;                 // 138240
constexpr int kKhOff = 0;
constexpr int kKlOff = kKhOff + kL * kTileRowBytes;
constexpr int kVOff = kKlOff + kL * kTileRowBytes;
constexpr int kXOff = kVOff + kL * kLdsV * 2;                    // 61440
static_assert(kXOff + 4 * 4 * 2 * 1024 <= kLdsBytes, "Q hand-over fits");
static_assert(kXOff + 4 * kPart * 64 * 4 <= kLdsBytes, "partials fit");

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

// V^T fragment for key slice kb (16 keys) and features tb*32 + (lane % 32)
// from V rows [key][feature] with the LDS transpose read: in each 16-lane
// group, lane r points at key row base + r/4, features T + (r%4)*4; lane j of
// the group receives features T + j of keys base .. base+3.
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

// Weights exp2(s - m) packed as the B operand of O^T += V^T P^T (slice kb
// covers keys kb*16 + (e/4)*8 + hb*4 + e%4); returns this lane's sum of the
// rounded weights.
__device__ __forceinline__ float weights(const f32x16 (&s)[2], float m, u32x4 (&w)[4]) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    float acc[2] = {0.0f, 0.0f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int v = (kb & 1) * 8 + e;
            const float p0 = __builtin_amdgcn_exp2f(s[kb >> 1][v] - m);
            const float p1 = __builtin_amdgcn_exp2f(s[kb >> 1][v + 1] - m);
            const bf16x2 pp = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
            w[kb][e >> 1] = __builtin_bit_cast(uint32_t, pp);
            acc[kb & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc[kb & 1], false);
        }
    }
    return acc[0] + acc[1];
}

template <bool kCausal, bool kHasVl>
__global__ __launch_bounds__(kThreads, 1) void mha_attn_fused_small_bf16(FusedArgs a, float c) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[kLdsBytes];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hb = lane >> 5, l32 = lane & 31;

    // Workgroup -> (batch, head).  Workgroup ids are dealt to the eight XCDs
    // round-robin; when B is a multiple of 8, XCD x gets the batches
    // b = x (mod 8) with all their heads, so the heads of one batch read X
    // through the same L2.
    int b, hd;
    if (a.B % 8 == 0) {
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
        b = x + 8 * (j / a.H);
        hd = j % a.H;
    } else {
        b = blockIdx.x / a.H;
        hd = blockIdx.x % a.H;
    }
    const int D = a.D, L = a.Lq;
    const int nd = D / 64;

    const bf16_t* x = static_cast<const bf16_t*>(a.x_q) + (long long)b * L * D;
    const bf16_t* wq = static_cast<const bf16_t*>(a.w_q) + (long long)hd * kHd * D;
    const bf16_t* wk = static_cast<const bf16_t*>(a.w_k) + (long long)hd * kHd * D;
    const bf16_t* wv = static_cast<const bf16_t*>(a.w_v) + (long long)hd * kHd * D;
    const bf16_t* bq = a.b_q ? static_cast<const bf16_t*>(a.b_q) + hd * kHd : nullptr;
    const bf16_t* bk = a.b_k ? static_cast<const bf16_t*>(a.b_k) + hd * kHd : nullptr;
    const bf16_t* bv = a.b_v ? static_cast<const bf16_t*>(a.b_v) + hd * kHd : nullptr;

    // ---------------- Q, K, V projections: one pass over d_model ------------
    LdsTileLoader<kL, kW> lx;         // X rows 0..127 (rows past L re-read row L-1)
    LdsTileLoader<kHd, kW> lwq, lwk, lwv;   // 64 rows of one weight slice each
    lx.init(wave, lane, x, 0, L, D);
    lwq.init(wave, lane, wq, 0, kHd, D);
    lwk.init(wave, lane, wk, 0, kHd, D);
    lwv.init(wave, lane, wv, 0, kHd, D);
    auto issue = [&](int stage, int d0) {
        unsigned char* base = smem + stage * kStageBytes;
        lx.issue(d0, base, wave);
        lwq.issue(d0, base + kL * kTileRowBytes, wave);
        lwk.issue(d0, base + (kL + kHd) * kTileRowBytes, wave);
        lwv.issue(d0, base + (kL + 2 * kHd) * kTileRowBytes, wave);
    };
    // Feature blocks 0..5 are Q0, Q1, K0, K1, V0, V1 (weight rows 32*f ..);
    // wave w owns rows rb = w % 4 and feature blocks 3*(w/4) + j in acc[j].
    const bool qwave = wave < 4;
    const int rb = wave & 3, f0 = qwave ? 0 : 3;
    // Loads this wave issues per slice (rows dealt round-robin to the waves).
    const int per_slice = (wave < 2 ? 3 : 2) + (wave == 0 ? 6 : 3);
    f32x16 acc[3] = {};
    issue(0, 0);
    if (nd > 1) issue(1, 64);
    for (int dt = 0; dt < nd; ++dt) {
        // This wave's loads of slice dt have landed (those of slice dt + 1
        // may still be in flight); after the barrier every wave's have, and
        // every wave is done reading the stage refilled next (read at dt - 1).
        if (dt + 1 < nd) {
            if (per_slice == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
            else if (per_slice == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
            else asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        if (dt + 2 < nd) issue((dt + 2) % kStages, (dt + 2) * 64);
        const bf16_t* xs = reinterpret_cast<const bf16_t*>(smem + (dt % kStages) * kStageBytes);
        const bf16_t* ws = xs + kL * kTileLdsRow;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int col = kk * 16 + hb * 8;
            const bf16x8 xf = frag(xs + (rb * 32 + l32) * kTileLdsRow + col);
#pragma unroll
            for (int j = 0; j < 3; ++j)
                acc[j] = mfma32x32x16(frag(ws + ((f0 + j) * 32 + l32) * kTileLdsRow + col), xf, acc[j]);
        }
    }
    // Every wave is done with the stages: K, V and the Q hand-over reuse them.
    __syncthreads();

    // K/V epilogue.  acc element v of block (tensor t, feature block fb): key rb*32 + l32,
    // feature fb*32 + (v/4)*8 + hb*4 + v%4.  K goes to LDS in the MFMA step
    // order of the Q fragments (step kk = 2*fb + v/8 holds it at element v%8
    // of lane half hb, i.e. column kk*16 + hb*8 + v%8), as hi + lo; V in
    // natural [key][feature] order.
    bf16_t* kh_s = reinterpret_cast<bf16_t*>(smem + kKhOff);
    bf16_t* kl_s = reinterpret_cast<bf16_t*>(smem + kKlOff);
    bf16_t* v_s = reinterpret_cast<bf16_t*>(smem + kVOff);
    auto store_kv = [&](const f32x16& y, int t, int fb) {
        const int row = rb * 32 + l32;
        float bb[4][4];
#pragma unroll
        for (int g = 0; g < 4; ++g) bias4(t == 0 ? bk : bv, fb * 32 + g * 8 + hb * 4, bb[g]);
        if (t == 0) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                uint32_t hw[4], lw4[4];
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const int v = half * 8 + e;
                    const float x0 = y[v] + bb[v >> 2][v & 3];
                    const float x1 = y[v + 1] + bb[(v + 1) >> 2][(v + 1) & 3];
                    hw[e >> 1] = pack_bf16x2(x0, x1);
                    lw4[e >> 1] = pack_bf16x2(x0 - __uint_as_float(hw[e >> 1] << 16),
                                              x1 - __uint_as_float(hw[e >> 1] & 0xffff0000u));
                }
                const int col = (2 * fb + half) * 16 + hb * 8;
                *reinterpret_cast<uint4*>(kh_s + row * kTileLdsRow + col) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                *reinterpret_cast<uint4*>(kl_s + row * kTileLdsRow + col) = make_uint4(lw4[0], lw4[1], lw4[2], lw4[3]);
            }
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int v = g * 4;
                *reinterpret_cast<uint2*>(v_s + row * kLdsV + fb * 32 + g * 8 + hb * 4) =
                    make_uint2(pack_bf16x2(y[v] + bb[g][0], y[v + 1] + bb[g][1]),
                               pack_bf16x2(y[v + 2] + bb[g][2], y[v + 3] + bb[g][3]));
            }
        }
    };
    // Q epilogue (waves 0-3).  acc[fb][v]: query wave*32 + l32, feature
    // fb*32 + (v/4)*8 + hb*4 + v%4; it becomes element v%8 of MFMA step
    // kk = 2*fb + v/8.
    bf16x8 qh[4], ql[4];
    if (qwave) {
        store_kv(acc[2], 0, 0);
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float bb[4];
                bias4(bq, fb * 32 + g * 8 + hb * 4, bb);
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int v = g * 4 + e4;
                    const float xq = (acc[fb][v] + bb[e4]) * c;
                    const __bf16 h = static_cast<__bf16>(xq);
                    qh[2 * fb + (v >> 3)][v & 7] = h;
                    ql[2 * fb + (v >> 3)][v & 7] = static_cast<__bf16>(xq - static_cast<float>(h));
                }
            }
        }
    } else {
        store_kv(acc[0], 0, 1);
        store_kv(acc[1], 1, 0);
        store_kv(acc[2], 1, 1);
    }
    // Hand the Q fragments of query block q to the wave that takes its
    // second key half.  Layout: ((q*4 + kk)*2 + {hi, lo}) KB after K and V,
    // lane at 16*lane.
    unsigned char* xch = smem + kXOff;
    if (qwave) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            *reinterpret_cast<bf16x8*>(xch + ((wave * 4 + kk) * 2) * 1024 + lane * 16) = qh[kk];
            *reinterpret_cast<bf16x8*>(xch + ((wave * 4 + kk) * 2 + 1) * 1024 + lane * 16) = ql[kk];
        }
    }
    __syncthreads();
    if (!qwave) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            qh[kk] = *reinterpret_cast<const bf16x8*>(xch + ((rb * 4 + kk) * 2) * 1024 + lane * 16);
            ql[kk] = *reinterpret_cast<const bf16x8*>(xch + ((rb * 4 + kk) * 2 + 1) * 1024 + lane * 16);
        }
    }

    // ---------------- attention: queries 32*(wave%4).., keys 64*(wave/4).. ---
    const int qb = wave & 3, kv0 = (wave >> 2) * 64;
    const int q0 = qb * 32, i = q0 + l32;
    const int vlen = kHasVl ? a.valid_lens[b] : L;
    const bool none = vlen <= 0;              // every key masked -> uniform weights
    const int kv_lim = none ? L : min(vlen, L);
    // This wave's keys lie below w_end; keys below key_lim are allowed for this lane.
    const int w_end = (kCausal && !none) ? min(kv_lim, q0 + 32) : kv_lim;
    const int key_lim = none ? L : (kCausal ? min(kv_lim, i + 1) : kv_lim);
    const bool active = q0 < L && kv0 < w_end;   // wave-uniform

    f32x16 o[2] = {};
    float m = -INFINITY, l = 0.0f;
    if (active) {
        f32x16 s[2] = {};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                const int r = (kv0 + jb * 32 + l32) * kTileLdsRow + kk * 16 + hb * 8;
                const bf16x8 kfh = frag(kh_s + r), kfl = frag(kl_s + r);
                s[jb] = mfma32x32x16(kfh, qh[kk], s[jb]);
                s[jb] = mfma32x32x16(kfl, qh[kk], s[jb]);
                s[jb] = mfma32x32x16(kfh, ql[kk], s[jb]);
            }
        }
        // Masks only when the tile crosses the valid length or the diagonal.
        if (none || kv0 + 64 > kv_lim || (kCausal && kv0 + 63 > q0)) {
            const int rel = key_lim - (kv0 + hb * 4);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int jr = (v >> 2) * 8 + (v & 3);
                s[0][v] = jr < rel ? (none ? 0.0f : s[0][v]) : -INFINITY;
                s[1][v] = jr + 32 < rel ? (none ? 0.0f : s[1][v]) : -INFINITY;
            }
        }
        // The tile is the whole key half: its row max is the exact offset.  A
        // row with no allowed key in this half (second half only) keeps
        // m = -inf and contributes nothing.
        m = tile_max(s);
        u32x4 p[4];
        l = weights(s, m == -INFINITY ? 0.0f : m, p);
        const bf16_t* vs = v_s + kv0 * kLdsV;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const bf16x8 pk = __builtin_bit_cast(bf16x8, p[kb]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) o[tb] = mfma32x32x16(v_frag(vs, kb, tb, hb, lane), pk, o[tb]);
        }
    }

    // ---------------- merge the key halves ---------------------------------
    // Every wave is done with the Q hand-over area; waves 4-7 leave (O^T,
    // max, sum) of each lane at float ((q*34 + f)*64 + lane).
    __syncthreads();
    float* part = reinterpret_cast<float*>(xch);
    if (!qwave) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            part[(qb * kPart + v) * 64 + lane] = o[0][v];
            part[(qb * kPart + 16 + v) * 64 + lane] = o[1][v];
        }
        part[(qb * kPart + 32) * 64 + lane] = m;
        part[(qb * kPart + 33) * 64 + lane] = l;
    }
    __syncthreads();
    // Waves 0-3 merge and normalise; the bf16 result goes to LDS (K's bytes,
    // free since the attention) and then out as whole 128-byte head rows.
    bf16_t* o_s = reinterpret_cast<bf16_t*>(smem + kKhOff);
    if (qwave) {
        const float m1 = part[(qb * kPart + 32) * 64 + lane];
        const float l1 = part[(qb * kPart + 33) * 64 + lane];
        // The first half always holds an allowed key of every row (key 0).
        const float mx = fmaxf(m, m1);
        const float a0 = __builtin_amdgcn_exp2f(m - mx);
        const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mx);
        const float inv = 1.0f / pair_sum(a0 * l + a1 * l1);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = g4 * 4 + e;
                    y[e] = (a0 * o[tb][v] + a1 * part[(qb * kPart + tb * 16 + v) * 64 + lane]) * inv;
                }
                *reinterpret_cast<uint2*>(o_s + i * kTileLdsRow + tb * 32 + g4 * 8 + hb * 4) =
                    make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
            }
        }
    }
    __syncthreads();
    // 8 lanes per row, 16 bytes each; rows past L are not stored.
#pragma unroll
    for (int pass = 0; pass < kL * 8 / kThreads; ++pass) {
        const int r = pass * (kThreads / 8) + (tid >> 3), c8 = (tid & 7) * 8;
        if (r < L)
            *reinterpret_cast<uint4*>(static_cast<bf16_t*>(a.o) + ((long long)b * L + r) * D + hd * kHd + c8) =
                *reinterpret_cast<const uint4*>(o_s + r * kTileLdsRow + c8);
    }
}

template <bool kCausal, bool kHasVl>
hipError_t launch_variant(const FusedArgs& a, hipStream_t s) {
    const long long grid = (long long)a.B * a.H;
    const float c = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    hipLaunchKernelGGL((mha_attn_fused_small_bf16<kCausal, kHasVl>), dim3((unsigned)grid), dim3(kThreads), 0, s, a,
                       c);
    return hipGetLastError();
}

}  // namespace

bool mha_attn_fused_small_fits(const FusedArgs& a) {
    return a.x_q == a.x_kv && a.Lq == a.Lk && a.Lq <= kL && a.D % 64 == 0;
}

hipError_t launch_mha_attn_fused_small(const FusedArgs& a, hipStream_t s) {
    if (!mha_attn_fused_small_fits(a)) return hipErrorInvalidValue;
    const bool c = a.causal != 0, v = a.valid_lens != nullptr;
    if (c) return v ? launch_variant<true, true>(a, s) : launch_variant<true, false>(a, s);
    return v ? launch_variant<false, true>(a, s) : launch_variant<false, false>(a, s);
}

}  // namespace mha
