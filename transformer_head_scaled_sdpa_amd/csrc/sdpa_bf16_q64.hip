// Fused scaled dot-product attention forward for single bf16 operands (the
// split-head entry point): bf16 in, fp32 accumulate, d_k = d_v = 64, gfx950.
//
// What it computes (The Annotated Transformer, "Attention" section):
//   o_i = sum_j softmax_j(q_i . k_j / sqrt(d_k)) v_j
// over the keys j allowed by the key-padding length and the causal rule.
// Masked scores are replaced by -1e9 in the pages' code, which gives them a
// weight of exactly zero whenever a row has an allowed key, so masked keys
// are skipped.  A row with no allowed key (valid length <= 0) has all its
// scores equal to -1e9, hence uniform weights over all Lk keys.
//
// Design.
//  * One workgroup = 4 wave64s covering 256 consecutive queries of one
//    (batch, head); each wave owns 64 queries as two blocks of 32 and keeps
//    their Q fragments in registers.  Every K or V fragment read from LDS
//    feeds two MFMAs (one per query block), which halves LDS bytes per flop
//    against 32-query waves.  At <= 256 registers per lane two workgroups
//    share a CU, so each SIMD runs one wave of each; their tiles are not
//    synchronised, and one wave's softmax overlaps the other's MFMAs.
//  * Keys/values stream through LDS in tiles of 64 in their natural
//    [key][feature] layout, copied with 16-byte coalesced loads staged in
//    registers; two LDS buffers, one barrier per tile, and the next tile's
//    global loads are in flight during the current tile's math.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//    each lane owns ONE query (lane % 32) and 32 of the tile's keys, so row
//    reductions are in-lane plus one v_permlane32_swap.  O^T += V^T P^T takes
//    P straight from the score accumulator (the key order inside each 16-key
//    slice is permuted identically on both operands); V^T is read with the
//    LDS transpose read ds_read_b64_tr_b16.
//  * Weights are exp2(s * c - m) with c = log2(e)/sqrt(d_k) applied by one
//    FMA per score on the fp32 product (folding c into bf16 Q would round the
//    logits by 2^-9 of their size, too coarse for sharp rows).  The offset m
//    is the row max of the first tile.  Later tiles keep it unless the
//    tile's weights (which are summed anyway) exceed 2^20 for some lane:
//    then the tile is recomputed with the row max folded into m and the
//    accumulators rescaled.  Weights stay below 2^20 * 64 per tile, far from
//    fp32 and bf16 limits, and no per-tile max reduction is needed.  The row
//    sum adds the bf16-rounded weights the P.V product uses
//    (v_dot2c_f32_bf16 with (1, 1)).
//  * Causal: tiles above the diagonal are never loaded or multiplied; masks
//    are evaluated only on tiles that cross the diagonal or the valid length.
//    Workgroups are issued heaviest-first, and consecutive workgroup ids take
//    different (batch, head) pairs (so with B*h a multiple of 8 each pair's
//    workgroups share one XCD's L2).
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kD = 64;                 // d_k = d_v
constexpr int kBN = 64;                // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = kWaves * 64;       // queries per workgroup
// LDS row strides (bf16 elements), conflict-free on gfx950: K rows read as
// 16-byte fragments at 144 B, V rows read with the transpose read at 192 B.
constexpr int kLdsK = kD + 8;
constexpr int kLdsV = kD + 32;
constexpr int kTileK = kBN * kLdsK;
constexpr int kTileV = kBN * kLdsV;
constexpr float kSumLimit = 1048576.0f;   // 2^20

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// A 64 x 64 bf16 tile is 512 16-byte chunks: two per thread.  Chunk c holds
// row c / 8, features (c % 8) * 8 .. +7.
__device__ __forceinline__ void load_rows(uint4 (&r)[2], const bf16_t* base, long long stride, int kv0, int Lk,
                                          int tid) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int c = tid + n * kThreads;
        const int key = kv0 + (c >> 3);
        r[n] = key < Lk ? *reinterpret_cast<const uint4*>(base + key * stride + (c & 7) * 8) : make_uint4(0, 0, 0, 0);
    }
}

template <int kLds>
__device__ __forceinline__ void store_rows(const uint4 (&r)[2], bf16_t* tile, int tid) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int c = tid + n * kThreads;
        *reinterpret_cast<uint4*>(tile + (c >> 3) * kLds + (c & 7) * 8) = r[n];
    }
}

__device__ __forceinline__ bf16x8 frag(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// V^T fragment for key slice kb (16 keys) and features tb*32 + (lane % 32):
// in each 16-lane group, lane r points at key row base + r/4, features
// T + (r%4)*4; the transpose read then hands lane j of the group features
// T + j of keys base .. base+3.  Two reads cover keys base..+3 and base+8..+11.
__device__ __forceinline__ bf16x8 v_frag(const bf16_t* vs, int kb, int tb, int hb, int lane) {
    const int g = lane >> 4, r = lane & 15;
    const int row = kb * 16 + hb * 4 + (r >> 2);
    const int col = tb * 32 + (g & 1) * 16 + (r & 3) * 4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vs + row * kLdsV + col));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vs + (row + 8) * kLdsV + col));
    // Join as whole vectors: inserting the 16-bit elements one by one is
    // lowered incorrectly by the compiler.
    const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, both);
}

// Raw scores q.k of one 64-key tile for both query blocks: s[qb][jb]
// element v holds key kv0 + jb*32 + (v/4)*8 + hb*4 + v%4 of query block qb's
// query lane % 32.
__device__ __forceinline__ void tile_scores(f32x16 (&s)[2][2], const bf16_t* ks, const bf16x8 (&qf)[2][4],
                                            int l32, int hb) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const bf16x8 kf = frag(ks + (jb * 32 + l32) * kLdsK + kk * 16 + hb * 8);
            s[0][jb] = mfma32x32x16(kf, qf[0][kk], kk == 0 ? f32x16{} : s[0][jb]);
            s[1][jb] = mfma32x32x16(kf, qf[1][kk], kk == 0 ? f32x16{} : s[1][jb]);
        }
    }
}

// Mask rule on a tile: keys [0, key_lim[qb]) may carry weight for the row;
// a row with no allowed key at all scores every key equally (score 0).
__device__ __forceinline__ void apply_mask(f32x16 (&s)[2][2], const int (&key_lim)[2], bool none, int kv0, int hb) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int rel = key_lim[qb] - (kv0 + hb * 4);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int jr = (v >> 2) * 8 + (v & 3);
            s[qb][0][v] = jr < rel ? (none ? 0.0f : s[qb][0][v]) : -INFINITY;
            s[qb][1][v] = jr + 32 < rel ? (none ? 0.0f : s[qb][1][v]) : -INFINITY;
        }
    }
}

// Row max of block qb over the tile (both lane halves).
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

// Weights exp2(s * c - m) packed as the B operand of O^T += V^T P^T: slice
// kb covers keys kb*16 + (e/4)*8 + hb*4 + e%4 as bf16 pairs.  rs gets this
// lane's sum of the rounded weights.
__device__ __forceinline__ void weights(const f32x16 (&s)[2][2], const float (&m)[2], float c, u32x4 (&w)[2][4],
                                        float (&rs)[2]) {
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float acc[2] = {0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const int v = (kb & 1) * 8 + e;
                const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb >> 1][v], c, -m[qb]));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qb][kb >> 1][v + 1], c, -m[qb]));
                const bf16x2 pp = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
                w[qb][kb][e >> 1] = __builtin_bit_cast(uint32_t, pp);
                acc[kb & 1] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, acc[kb & 1], false);
            }
        }
        rs[qb] = acc[0] + acc[1];
    }
}

template <bool kCausal, bool kHasVl, bool kOutF32>
__global__ __launch_bounds__(kThreads, 2)
void sdpa_fwd_bf16_q64(SdpaArgs a, int n_qtiles, float c_log2) {
    __shared__ __attribute__((aligned(16))) bf16_t kbuf[2 * kTileK];
    __shared__ __attribute__((aligned(16))) bf16_t vbuf[2 * kTileV];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // The wave index as a scalar: tile-range and mask decisions derived from
    // it are then wave-uniform branches, not per-lane selects.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hb = lane >> 5, l32 = lane & 31;

    // Workgroup -> (query tile, batch, head): (batch, head) varies fastest;
    // causal issues the longest tiles first.
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    int qt = blockIdx.x / BH;
    if (kCausal) qt = n_qtiles - 1 - qt;
    const int b = bh / a.H, hd = bh % a.H;

    const int q_wg = qt * kBM;
    const int q0 = q_wg + wave * 64;              // this wave's first query
    const int iq[2] = {q0 + l32, q0 + 32 + l32};  // this lane's query in each block

    const int Lk = a.Lk;
    const int vlen = kHasVl ? a.valid_lens[b] : Lk;
    const bool none = vlen <= 0;                  // every key masked -> uniform weights
    const int kv_lim = none ? Lk : min(vlen, Lk); // keys [0, kv_lim) can carry weight
    int kv_end = kv_lim;
    if (kCausal && !none) kv_end = min(kv_end, q_wg + kBM);
    const int n_tiles = (kv_end + kBN - 1) / kBN;
    // Tiles from index n_wave on lie wholly above this wave's queries.
    const int n_wave = (kCausal && !none) ? min(n_tiles, (q0 + 63) / kBN + 1) : n_tiles;
    // Tiles from index t_mask on need the key-padding, causal or fully-masked rule.
    int t_mask = none ? 0 : kv_lim / kBN;
    if (kCausal && !none) t_mask = min(t_mask, q0 / kBN);
    int key_lim[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) key_lim[qb] = none ? Lk : (kCausal ? min(kv_lim, iq[qb] + 1) : kv_lim);

    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1];

    // Prologue: tiles 0 and 1 into the two LDS buffers, tile 2 into registers.
    uint4 rk[2], rv[2], rk1[2], rv1[2];
    load_rows(rk, kp, a.sk[2], 0, Lk, tid);
    load_rows(rv, vp, a.sv[2], 0, Lk, tid);
    if (n_tiles > 1) {
        load_rows(rk1, kp, a.sk[2], kBN, Lk, tid);
        load_rows(rv1, vp, a.sv[2], kBN, Lk, tid);
    }
    bf16x8 qf[2][4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (iq[qb] < a.Lq) raw = *reinterpret_cast<const uint4*>(qp + iq[qb] * a.sq[2] + kk * 16 + hb * 8);
            qf[qb][kk] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    store_rows<kLdsK>(rk, kbuf, tid);
    store_rows<kLdsV>(rv, vbuf, tid);
    if (n_tiles > 1) {
        store_rows<kLdsK>(rk1, kbuf + kTileK, tid);
        store_rows<kLdsV>(rv1, vbuf + kTileV, tid);
    }
    if (n_tiles > 2) {
        load_rows(rk, kp, a.sk[2], 2 * kBN, Lk, tid);
        load_rows(rv, vp, a.sv[2], 2 * kBN, Lk, tid);
    }
    __syncthreads();

    f32x16 o[2][2] = {};           // O^T accumulators [query block][feature half]
    float m[2] = {0.0f, 0.0f};     // exponent offsets (log2 units of the scaled scores)
    float l[2] = {0.0f, 0.0f};     // this lane's share of the weight sums

    for (int t = 0; t < n_tiles; ++t) {
        const int kv0 = t * kBN;
        const bf16_t* ks = kbuf + (t & 1) * kTileK;
        const bf16_t* vs = vbuf + (t & 1) * kTileV;
        if (t < n_wave) {
            f32x16 s[2][2];
            tile_scores(s, ks, qf, l32, hb);
            if (t >= t_mask) [[unlikely]] {
                // Keep this a real branch: speculated, it would cost ~200 VALU
                // operations on every tile instead of only on edge tiles.
                asm volatile("" ::: "memory");
                apply_mask(s, key_lim, none, kv0, hb);
            }
            if (t == 0) {
                // First tile: the offset becomes the row max (every row has
                // an allowed key in tile 0).
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) m[qb] = tile_max(s[qb]) * c_log2;
            }
            u32x4 w[2][4];
            float rs[2];
            weights(s, m, c_log2, w, rs);
            if (t > 0 && __any(rs[0] > kSumLimit || rs[1] > kSumLimit)) [[unlikely]] {
                // Some weight outgrew the offset: fold this tile's row max in
                // (never lowering the offset), rescale and recompute.
                asm volatile("" ::: "memory");
                tile_scores(s, ks, qf, l32, hb);
                if (t >= t_mask) apply_mask(s, key_lim, none, kv0, hb);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const float d = fmaxf(fmaf(tile_max(s[qb]), c_log2, -m[qb]), 0.0f);
                    m[qb] += d;
                    const float alpha = __builtin_amdgcn_exp2f(-d);
                    l[qb] *= alpha;
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        o[qb][0][v] *= alpha;
                        o[qb][1][v] *= alpha;
                    }
                }
                weights(s, m, c_log2, w, rs);
            }
            l[0] += rs[0];
            l[1] += rs[1];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const bf16x8 p0 = __builtin_bit_cast(bf16x8, w[0][kb]);
                const bf16x8 p1 = __builtin_bit_cast(bf16x8, w[1][kb]);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb) {
                    const bf16x8 vf = v_frag(vs, kb, tb, hb, lane);
                    o[0][tb] = mfma32x32x16(vf, p0, o[0][tb]);
                    o[1][tb] = mfma32x32x16(vf, p1, o[1][tb]);
                }
            }
        }

        // Tile t+2 goes into the buffers tile t used; every wave is done
        // with them after this barrier.
        __syncthreads();
        if (t + 2 < n_tiles) {
            store_rows<kLdsK>(rk, kbuf + (t & 1) * kTileK, tid);
            store_rows<kLdsV>(rv, vbuf + (t & 1) * kTileV, tid);
            if (t + 3 < n_tiles) {
                load_rows(rk, kp, a.sk[2], (t + 3) * kBN, Lk, tid);
                load_rows(rv, vp, a.sv[2], (t + 3) * kBN, Lk, tid);
            }
        }
    }

    // O^T element v of block tb: feature tb*32 + (v/4)*8 + hb*4 + v%4.
    char* ob = static_cast<char*>(a.o);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float inv = 1.0f / pair_sum(l[qb]);
        if (iq[qb] >= a.Lq) continue;
        const long long orow = b * a.so[0] + hd * a.so[1] + (long long)iq[qb] * a.so[2];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int tt = tb * 32 + g4 * 8 + hb * 4;
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = o[qb][tb][g4 * 4 + e] * inv;
                if (kOutF32) {
                    *reinterpret_cast<float4*>(ob + (orow + tt) * 4) = make_float4(y[0], y[1], y[2], y[3]);
                } else {
                    *reinterpret_cast<uint2*>(ob + (orow + tt) * 2) =
                        make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
                }
            }
        }
    }
}

template <bool kCausal, bool kHasVl, bool kOutF32>
hipError_t launch_variant(const SdpaArgs& a, hipStream_t s) {
    const int n_qtiles = (a.Lq + kBM - 1) / kBM;
    const long long grid = (long long)n_qtiles * a.B * a.H;
    const float c_log2 = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    hipLaunchKernelGGL((sdpa_fwd_bf16_q64<kCausal, kHasVl, kOutF32>), dim3((unsigned)grid), dim3(kThreads), 0, s,
                       a, n_qtiles, c_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sdpa_bf16_q64(const SdpaArgs& a, bool out_f32, hipStream_t s) {
    const bool c = a.causal != 0, v = a.valid_lens != nullptr;
    if (out_f32) {
        if (c) return v ? launch_variant<true, true, true>(a, s) : launch_variant<true, false, true>(a, s);
        return v ? launch_variant<false, true, true>(a, s) : launch_variant<false, false, true>(a, s);
    }
    if (c) return v ? launch_variant<true, true, false>(a, s) : launch_variant<true, false, false>(a, s);
    return v ? launch_variant<false, true, false>(a, s) : launch_variant<false, false, false>(a, s);
}

}  // namespace mha
