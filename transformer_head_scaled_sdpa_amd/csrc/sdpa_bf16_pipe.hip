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
//  * One workgroup = 8 wave64s (two per SIMD) covering 256 consecutive
//    queries of one (batch, head); each wave owns 32 queries and keeps their
//    Q fragments in registers.  Keys/values stream through LDS in tiles of
//    64 keys, copied with one 16-byte coalesced load per thread per tensor,
//    loaded into registers two stages before they are stored to LDS (two
//    register sets, one for even and one for odd stages) through buffer
//    loads that zero-fill rows past Lk, so the copy is branch-free.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16
//    so every lane owns ONE query (lane % 32) and 32 keys of a tile; row sums
//    are in-lane plus one v_permlane32_swap.  O^T += V^T P^T takes P straight
//    from the score accumulator (the key order inside each 16-key slice is
//    permuted identically on both operands) and reads V^T from LDS with the
//    transpose read ds_read_b64_tr_b16.
//  * Software pipeline inside each wave.  Stage s computes the softmax of
//    tile s while the matrix cores run the scores of tile s+1 and the
//    P.V product of tile s-1; the three are independent, so the scheduler
//    interleaves the exponentials (which overlap MFMA execution) with the
//    MFMAs instead of letting a wave alternate between MFMA-only and
//    VALU-only phases.  K tiles are read one stage ahead of their softmax
//    and V tiles one stage behind it, from two LDS buffers each, with one
//    barrier per stage.
//  * Weights are exp2(s * c - m) with c = log2(e)/sqrt(d_k) applied by one
//    FMA on the fp32 score.  The offset m is the row max of the first tile;
//    later tiles keep it unless a query's sum of weights for the tile
//    exceeds 2^22, in which case the tile's row max is folded into m, the
//    accumulators are rescaled and the tile's weights recomputed.  Weights
//    stay below 2^22, far from fp32 and bf16 limits, and no per-tile max
//    reduction runs in the common case.  Row sums of
//    the bf16 weights run on the matrix core (a 16x16x32 MFMA with a 0/1
//    selector per 16-key slice), which idles half the time, instead of the
//    VALU, which bounds the loop.
//  * Causal: tiles above the diagonal are never loaded or multiplied; masks
//    are evaluated only on the tiles that cross the diagonal or the valid
//    length.  Workgroups are issued heaviest-first, and consecutive
//    workgroup ids take different (batch, head) pairs.
//  * The normalised output goes through LDS once the keys are done, so each
//    row of 64 features leaves as whole 128-byte runs instead of 8- or
//    16-byte pieces per lane.
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kD = 64;                 // d_k = d_v
constexpr int kBN = 64;                // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = kWaves * 32;       // queries per workgroup
// LDS row strides (bf16 elements), conflict-free on gfx950: K rows read as
// 16-byte fragments at 144 B, V rows read with the transpose read at 192 B.
constexpr int kLdsK = kD + 8;
constexpr int kLdsV = kD + 32;
constexpr int kTileK = kBN * kLdsK;
constexpr int kTileV = kBN * kLdsV;
constexpr float kSumLimit = 4194304.0f;   // 2^22: a tile's weight sum per query that triggers a rescale

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// A 64 x 64 bf16 tile is 512 16-byte chunks, one per thread: chunk c holds
// row c / 8, features (c % 8) * 8 .. +7.  Tiles are read through a buffer
// resource based at the tile's first row whose range ends with row Lk - 1,
// so rows at or past Lk read as zero in hardware and the copy needs no
// branch; straight-line loads and stores let the compiler wait for exactly
// the loads a store needs.  Each lane adds a fixed byte offset.
struct TileSrc {
    const char* base;    // row 0 of the (batch, head)
    uint32_t range;      // bytes from row 0 to the end of row Lk - 1
    uint32_t tile_bytes; // bytes per tile of rows
    uint32_t lane_off;   // this thread's chunk within a tile
};
constexpr int kBufWord3 = 0x00020000;   // raw buffer, 32-bit data format (gfx9 descriptor word 3)

__device__ __forceinline__ uint4 load_tile(const TileSrc& src, int t) {
    const unsigned long long skip = (unsigned long long)(uint32_t)t * src.tile_bytes;
    const bool any = skip < src.range;
    const uint32_t left = any ? src.range - (uint32_t)skip : 0u;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(src.base + (any ? skip : 0ull)), (short)0, (int)left, kBufWord3);
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, src.lane_off, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int kLds>
__device__ __forceinline__ void store_chunk(const uint4& r, bf16_t* tile, int tid) {
    *reinterpret_cast<uint4*>(tile + (tid >> 3) * kLds + (tid & 7) * 8) = r;
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

// Raw scores q.k of one 64-key tile: s[jb] element v holds key
// kv0 + jb*32 + (v/4)*8 + hb*4 + v%4 for query lane % 32.
__device__ __forceinline__ void tile_scores(f32x16 (&s)[2], const bf16_t* ks, const bf16x8 (&qf)[4], int l32,
                                            int hb) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const bf16x8 kf = frag(ks + (jb * 32 + l32) * kLdsK + kk * 16 + hb * 8);
            s[jb] = mfma32x32x16(kf, qf[kk], kk == 0 ? f32x16{} : s[jb]);
        }
    }
}

// Scores of one 64-key tile from hi + lo operands (q * log2(e)/sqrt(d_k)
// and k each split as hi + lo): hi.hi + lo.hi + hi.lo, in log2 units.
__device__ __forceinline__ void tile_scores_hilo(f32x16 (&s)[2], const bf16_t* ks, const bf16_t* ksl,
                                                 const bf16x8 (&qf)[4], const bf16x8 (&qfl)[4], int l32, int hb) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int off = (jb * 32 + l32) * kLdsK + kk * 16 + hb * 8;
            const bf16x8 kf = frag(ks + off), kfl = frag(ksl + off);
            s[jb] = mfma32x32x16(kf, qf[kk], kk == 0 ? f32x16{} : s[jb]);
            s[jb] = mfma32x32x16(kfl, qf[kk], s[jb]);
            s[jb] = mfma32x32x16(kf, qfl[kk], s[jb]);
        }
    }
}

// O^T += V^T P^T over one 64-key tile.
__device__ __forceinline__ void tile_pv(f32x16 (&o)[2], const bf16_t* vs, const u32x4 (&p)[4], int hb, int lane) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 pk = __builtin_bit_cast(bf16x8, p[kb]);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) o[tb] = mfma32x32x16(v_frag(vs, kb, tb, hb, lane), pk, o[tb]);
    }
}

// Mask rule on a tile: keys [0, key_lim) may carry weight for the row; a
// row with no allowed key at all scores every key equally (score 0).
__device__ __forceinline__ void apply_mask(f32x16 (&s)[2], int key_lim, bool none, int kv0, int hb) {
    const int rel = key_lim - (kv0 + hb * 4);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int jr = (v >> 2) * 8 + (v & 3);
        s[0][v] = jr < rel ? (none ? 0.0f : s[0][v]) : -INFINITY;
        s[1][v] = jr + 32 < rel ? (none ? 0.0f : s[1][v]) : -INFINITY;
    }
}

// Row max over the tile (both lane halves).
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
// kb covers keys kb*16 + (e/4)*8 + hb*4 + e%4 as bf16 pairs.
__device__ __forceinline__ void weights(const f32x16 (&s)[2], float m, float c, u32x4 (&w)[4]) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int v = (kb & 1) * 8 + e;
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb >> 1][v], c, -m));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb >> 1][v + 1], c, -m));
            const bf16x2 pp = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
            w[kb][e >> 1] = __builtin_bit_cast(uint32_t, pp);
        }
    }
}

// Row sums of the packed weights on the matrix core.  Read as the B operand
// of v_mfma_f32_16x16x32_bf16, lane l holds 8 weights of query l % 32 (keys
// of lane half l / 32), which the MFMA files under column l % 16 and k-group
// l / 16.  The selector A has row 0 = 1 over k-groups 0 and 2 (lanes l and
// l + 32: query l) and row 1 = 1 over k-groups 1 and 3 (query l + 16), and
// 2^-126 elsewhere, so lanes 0..15 receive the sums over the tile's 64 keys:
// element 0 for query l, element 1 for query l + 16.  These are sums of the same bf16 weights
// the P.V product uses, formed where the VALU (which bounds the loop) is not
// involved.
__device__ __forceinline__ f32x4 tile_sums(const bf16x8& sel, const u32x4 (&w)[4]) {
    f32x4 t = {};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
        t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, __builtin_bit_cast(bf16x8, w[kb]), t, 0, 0, 0);
    return t;
}

// The sum of query lane % 32 from tile_sums' layout (lane l < 16: element 0,
// lane l + 16: element 1 of lane l).
__device__ __forceinline__ float query_sum(const float (&t)[2], int l32) {
    const int src = (l32 & 15) * 4;
    const float lo = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, t[0])));
    const float hi = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, t[1])));
    return l32 < 16 ? lo : hi;
}

// A tile's weights outgrew the offset m: fold the tile's row max into m
// (never lowering it), rescale the output accumulators and the running sums
// (lanes 0..15 hold queries l and l + 16) and recompute the tile's weights.
__device__ __forceinline__ void rescale(const f32x16 (&s)[2], float& m, float c, float (&l)[2], f32x16 (&o)[2],
                                        u32x4 (&w)[4], int l32) {
    const float d = fmaxf(fmaf(tile_max(s), c, -m), 0.0f);
    m += d;
    const float alpha = __builtin_amdgcn_exp2f(-d);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        o[0][v] *= alpha;
        o[1][v] *= alpha;
    }
    const int src = ((l32 & 15) + 16) * 4;
    const float alpha_hi = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, alpha)));
    l[0] *= alpha;
    l[1] *= alpha_hi;
    weights(s, m, c, w);
}

template <bool kCausal, bool kHasVl, bool kOutF32, bool kHiLo>
__global__ __launch_bounds__(kThreads, 1)
void sdpa_fwd_bf16_pipe(SdpaArgs a, int n_qtiles, float c) {
    // K tiles (two buffers), then with hi + lo operands the two K lo tiles.
    __shared__ __attribute__((aligned(16))) bf16_t kbuf[(kHiLo ? 4 : 2) * kTileK];
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
    const int q0 = q_wg + wave * 32;              // this wave's first query
    const int i = q0 + l32;                       // this lane's query

    const int Lk = a.Lk;
    const int vlen = kHasVl ? a.valid_lens[b] : Lk;
    const bool none = vlen <= 0;                  // every key masked -> uniform weights
    const int kv_lim = none ? Lk : min(vlen, Lk); // keys [0, kv_lim) can carry weight
    int kv_end = kv_lim;
    if (kCausal && !none) kv_end = min(kv_end, q_wg + kBM);
    const int n_tiles = (kv_end + kBN - 1) / kBN; // tiles the workgroup streams
    // This wave's tiles are [0, n_w): later ones lie wholly above its queries.
    const int n_w = (kCausal && !none) ? min(n_tiles, (q0 + 31) / kBN + 1) : n_tiles;
    // Tiles from index t_mask on need the key-padding, causal or fully-masked rule.
    int t_mask = none ? 0 : kv_lim / kBN;
    if (kCausal && !none) t_mask = min(t_mask, q0 / kBN);
    // Keys below key_lim are allowed for this lane's row.
    const int key_lim = none ? Lk : (kCausal ? min(kv_lim, i + 1) : kv_lim);

    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const TileSrc ksrc{reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1]),
                       (uint32_t)((long long)(Lk - 1) * a.sk[2] * 2 + kD * 2), (uint32_t)(a.sk[2] * 2 * kBN),
                       (uint32_t)((tid >> 3) * a.sk[2] * 2) + (tid & 7) * 16};
    const TileSrc vsrc{reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1]),
                       (uint32_t)((long long)(Lk - 1) * a.sv[2] * 2 + kD * 2), (uint32_t)(a.sv[2] * 2 * kBN),
                       (uint32_t)((tid >> 3) * a.sv[2] * 2) + (tid & 7) * 16};
    auto load_k = [&](int t) { return load_tile(ksrc, t); };
    // K lo plane (hi + lo operands only; same strides as K).
    const TileSrc klsrc{kHiLo ? reinterpret_cast<const char*>(static_cast<const bf16_t*>(a.k_lo) + b * a.sk[0] + hd * a.sk[1])
                              : ksrc.base,
                        ksrc.range, ksrc.tile_bytes, ksrc.lane_off};
    auto load_kl = [&](int t) { return load_tile(klsrc, t); };
    bf16_t* const klbuf = kbuf + 2 * kTileK;
    auto load_v = [&](int t) { return load_tile(vsrc, t); };

    // Prologue: K tiles 0 and 1 into LDS, scores of tile 0; K(2), K(3), V(0)
    // and V(1) wait in registers for stages 0 and 1.
    uint4 nk_e = load_k(0);
    uint4 nk_o = load_k(1);
    bf16x8 qf[4], qfl[4];
    const bf16_t* qlp = kHiLo ? static_cast<const bf16_t*>(a.q_lo) + b * a.sq[0] + hd * a.sq[1] : qp;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 raw = make_uint4(0, 0, 0, 0), rawl = make_uint4(0, 0, 0, 0);
        if (i < a.Lq) {
            raw = *reinterpret_cast<const uint4*>(qp + (long long)i * a.sq[2] + kk * 16 + hb * 8);
            if (kHiLo) rawl = *reinterpret_cast<const uint4*>(qlp + (long long)i * a.sq[2] + kk * 16 + hb * 8);
        }
        qf[kk] = __builtin_bit_cast(bf16x8, raw);
        qfl[kk] = __builtin_bit_cast(bf16x8, rawl);
    }
    store_chunk<kLdsK>(nk_e, kbuf, tid);
    store_chunk<kLdsK>(nk_o, kbuf + kTileK, tid);
    // With hi + lo operands the K tiles run one stage ahead (hi in nk_e, lo
    // in nk_o, both for the same tile) to keep the register count; plain
    // operands run two stages ahead (even and odd tiles in nk_e, nk_o).
    if constexpr (kHiLo) {
        store_chunk<kLdsK>(load_kl(0), klbuf, tid);
        store_chunk<kLdsK>(load_kl(1), klbuf + kTileK, tid);
        nk_e = load_k(2);
        nk_o = load_kl(2);
    } else {
        nk_e = load_k(2);
        nk_o = load_k(3);
    }
    uint4 nv_e = load_v(0);
    uint4 nv_o = load_v(1);
    __syncthreads();
    f32x16 sc[2];                 // scores of the tile whose softmax runs next
    if constexpr (kHiLo) tile_scores_hilo(sc, kbuf, klbuf, qf, qfl, l32, hb);
    else tile_scores(sc, kbuf, qf, l32, hb);
    __syncthreads();              // K(0)'s buffer is refilled in stage 0

    f32x16 o[2] = {};             // O^T accumulators: features [0,32) and [32,64)
    f32x16 sn[2];                 // scores being formed for the next stage
    u32x4 pa[4], pb[4];           // weights of two consecutive tiles (B operand)
    float m = 0.0f;               // exponent offset (log2 units of the scaled scores)
    float l[2] = {0.0f, 0.0f};    // running weight sums (elements 0, 1 of tile_sums' layout)
    // Row selector of tile_sums: 1 in lanes 0, 32 and 17, 49; elsewhere the
    // smallest normal bf16, 2^-126, rather than 0, so that a weight that
    // overflowed to infinity (a tile far above the offset) makes the sums
    // infinite, which triggers the rescale, instead of 0 * inf = NaN.  The
    // stray terms are below 2^-100 of any sum.
    bf16x8 sel;
    {
        const uint16_t bits = (lane == 0 || lane == 32 || lane == 17 || lane == 49) ? 0x3f80u : 0x0080u;
        const __bf16 v = __builtin_bit_cast(__bf16, bits);
#pragma unroll
        for (int e = 0; e < 8; ++e) sel[e] = v;
    }
    auto over = [&](const f32x4& t) { return __any(fmaxf(t[0], t[1]) > kSumLimit); };

    // Stage s reads K(s+1) and V(s-1) and fills the other buffers with K(s+2)
    // and V(s), loaded two stages earlier (every wave finished with those
    // buffers at the last barrier); it loads K(s+4) and V(s+2).  Even and odd
    // stages use their own register sets.  Tiles past the last one load as
    // zeros and land in buffers no stage reads again, so the copy is the same
    // straight-line code every stage.
    auto copy_tiles = [&](int s, uint4& nk, uint4& nv) {
        if constexpr (kHiLo) {
            store_chunk<kLdsK>(nk_e, kbuf + (s & 1) * kTileK, tid);
            store_chunk<kLdsK>(nk_o, klbuf + (s & 1) * kTileK, tid);
            nk_e = load_k(s + 3);
            nk_o = load_kl(s + 3);
        } else {
            store_chunk<kLdsK>(nk, kbuf + (s & 1) * kTileK, tid);
            nk = load_k(s + 4);
        }
        store_chunk<kLdsV>(nv, vbuf + (s & 1) * kTileV, tid);
        nv = load_v(s + 2);
    };
    auto scores = [&](f32x16 (&nxt)[2], int s) {
        const bf16_t* ks = kbuf + ((s + 1) & 1) * kTileK;
        if constexpr (kHiLo) tile_scores_hilo(nxt, ks, klbuf + ((s + 1) & 1) * kTileK, qf, qfl, l32, hb);
        else tile_scores(nxt, ks, qf, l32, hb);
    };
    // Unmasked steady state: softmax(s), scores(s+1) and P.V(s-1), independent.
    // Everything up to the barrier is one branch-free block, so the scheduler
    // can spread the softmax over all the stage's MFMAs; the rare offset
    // check runs after the barrier, while S(s) is still held (the next
    // stage's scores overwrite it only after the check) and before P(s)
    // enters a product.
    auto fast_stage = [&](int s, f32x16 (&cur)[2], f32x16 (&nxt)[2], const u32x4 (&prev)[4], u32x4 (&pcur)[4], uint4& nk, uint4& nv) {
        copy_tiles(s, nk, nv);
        const bf16_t* vs = vbuf + ((s + 1) & 1) * kTileV;
        weights(cur, m, c, pcur);
        f32x4 t = tile_sums(sel, pcur);
        scores(nxt, s);
        tile_pv(o, vs, prev, hb, lane);
        __syncthreads();
        if (over(t)) [[unlikely]] {
            asm volatile("" ::: "memory");
            rescale(cur, m, c, l, o, pcur, l32);
            t = tile_sums(sel, pcur);
        }
        l[0] += t[0];
        l[1] += t[1];
    };
    // Pipeline edges, masked tiles and fully masked rows.
    auto slow_stage = [&](int s, f32x16 (&cur)[2], f32x16 (&nxt)[2], const u32x4 (&prev)[4], u32x4 (&pcur)[4], uint4& nk, uint4& nv) {
        copy_tiles(s, nk, nv);
        const bf16_t* vs = vbuf + ((s + 1) & 1) * kTileV;
        if (s >= 1 && s - 1 < n_w) tile_pv(o, vs, prev, hb, lane);
        if (s < n_w) {
            if (s >= t_mask) apply_mask(cur, key_lim, none, s * kBN, hb);
            // The first tile sets the offset (every row has an allowed key in
            // tile 0).
            if (s == 0) m = tile_max(cur) * c;
            weights(cur, m, c, pcur);
            f32x4 t = tile_sums(sel, pcur);
            if (s > 0 && over(t)) {
                rescale(cur, m, c, l, o, pcur, l32);
                t = tile_sums(sel, pcur);
            }
            l[0] += t[0];
            l[1] += t[1];
        }
        if (s + 1 < n_w) scores(nxt, s);
        __syncthreads();
    };

    // Stage 0, then unmasked stages in pairs from stage 1, then the rest.
    // Even stages keep the current scores in sc and their weights in pa, odd
    // stages in sn and pb, so no registers are copied between stages.
    slow_stage(0, sc, sn, pb, pa, nk_e, nv_e);
    const int fast_last = 1 + 2 * max(0, (min(n_w - 1, t_mask) - 1) / 2);   // fast stages [1, fast_last)
    int s = 1;
    for (; s < fast_last; s += 2) {
        fast_stage(s, sn, sc, pa, pb, nk_o, nv_o);
        fast_stage(s + 1, sc, sn, pb, pa, nk_e, nv_e);
    }
    for (; s <= n_tiles; s += 2) {
        slow_stage(s, sn, sc, pa, pb, nk_o, nv_o);
        if (s + 1 > n_tiles) break;
        slow_stage(s + 1, sc, sn, pb, pa, nk_e, nv_e);
    }

    const float lsum = query_sum(l, l32);
    const float inv = 1.0f / lsum;
    // The log-sum-exp of the scaled scores (natural log) when asked for: the
    // offset m and the weight sum are in log2 units (v_log_f32 is log2).
    if (a.lse && hb == 0 && i < a.Lq) a.lse[(long long)bh * a.Lq + i] = (m + __builtin_amdgcn_logf(lsum)) * kLn2;
    // O^T element v of block tb: feature tb*32 + (v/4)*8 + hb*4 + v%4, query
    // i.  Every wave is past the last barrier, so the K/V buffers are idle:
    // each wave stages 32 rows x 128 bytes of its output in its own slice
    // (144-byte rows) and stores each row's 128 bytes as one run, 8 lanes per
    // row; fp32 rows take two such rounds.  Output rows start 16-byte aligned
    // (the entry points reject other pointers and strides).
    constexpr int kEl = kOutF32 ? 4 : 2;           // bytes per output element
    constexpr int kRounds = kOutF32 ? 2 : 1;
    char* const o_s = reinterpret_cast<char*>(wave < 4 ? vbuf + wave * 32 * kLdsK : kbuf + (wave - 4) * 32 * kLdsK);
    char* const orow0 = static_cast<char*>(a.o) + (b * a.so[0] + hd * a.so[1] + (long long)q0 * a.so[2]) * kEl;
#pragma unroll
    for (int rd = 0; rd < kRounds; ++rd) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
            if (kOutF32 && tb != rd) continue;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] = o[tb][g4 * 4 + e] * inv;
                char* dst = o_s + l32 * kLdsK * 2 + (tb * 32 + g4 * 8 + hb * 4) * kEl - rd * 128;
                if (kOutF32)
                    *reinterpret_cast<float4*>(dst) = make_float4(y[0], y[1], y[2], y[3]);
                else
                    *reinterpret_cast<uint2*>(dst) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int r = pass * 8 + (lane >> 3), cb = (lane & 7) * 16;
            if (q0 + r < a.Lq)
                *reinterpret_cast<uint4*>(orow0 + (long long)r * a.so[2] * kEl + rd * 128 + cb) =
                    *reinterpret_cast<const uint4*>(o_s + r * kLdsK * 2 + cb);
        }
        if (rd + 1 < kRounds) {   // the next round overwrites the slice
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
}

template <bool kCausal, bool kHasVl, bool kOutF32, bool kHiLo>
hipError_t launch_variant(const SdpaArgs& a, hipStream_t s) {
    const int n_qtiles = (a.Lq + kBM - 1) / kBM;
    const long long grid = (long long)n_qtiles * a.B * a.H;
    // Exponent scale: log2(e) / sqrt(64), or 1 when q arrives pre-scaled.
    const float c = kHiLo ? 1.0f : kLog2e / 8.0f;
    hipLaunchKernelGGL((sdpa_fwd_bf16_pipe<kCausal, kHasVl, kOutF32, kHiLo>), dim3((unsigned)grid), dim3(kThreads), 0,
                       s, a, n_qtiles, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sdpa_bf16(const SdpaArgs& a, bool out_f32, hipStream_t s) {
    const bool c = a.causal != 0, v = a.valid_lens != nullptr;
    if (a.q_lo) {   // hi + lo operands: bf16 output
        if (out_f32 || !a.k_lo) return hipErrorInvalidValue;
        if (c) return v ? launch_variant<true, true, false, true>(a, s) : launch_variant<true, false, false, true>(a, s);
        return v ? launch_variant<false, true, false, true>(a, s) : launch_variant<false, false, false, true>(a, s);
    }
    if (out_f32) {
        if (c) return v ? launch_variant<true, true, true, false>(a, s) : launch_variant<true, false, true, false>(a, s);
        return v ? launch_variant<false, true, true, false>(a, s) : launch_variant<false, false, true, false>(a, s);
    }
    if (c) return v ? launch_variant<true, true, false, false>(a, s) : launch_variant<true, false, false, false>(a, s);
    return v ? launch_variant<false, true, false, false>(a, s) : launch_variant<false, false, false, false>(a, s);
}

}  // namespace mha
