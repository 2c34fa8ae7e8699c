// Fused scaled dot-product attention forward, bf16 in / fp32 accumulate,
// d_k = d_v = 64, for gfx950 (CDNA4).
//
// What it computes (The Annotated Transformer, "Attention" section):
//   o_i = sum_j softmax_j(q_i . k_j / sqrt(d_k)) v_j
// over the keys j allowed by the key-padding length and the causal rule;
// masked scores are replaced by -1e9 in the pages' code, which gives them a
// weight of exactly zero whenever a row has an allowed key, so masked keys
// are skipped here.  A row with no allowed key (valid length <= 0) has all
// its scores equal to -1e9, hence uniform weights over all Lk keys.
//
// Design.
//  * One workgroup = W wave64s (W = 8, or 4 on the multi-head path) covering
//    32*W consecutive queries of one (batch, head); each wave owns 32
//    queries and keeps their Q fragments in registers.  Registers are kept
//    at <= 128 per lane so that four waves share each SIMD: a single wave
//    spends most of a tile waiting on its own dependency chains (MFMA
//    results, LDS reads, transcendentals), and the other waves fill it.
//  * Keys/values stream through LDS in tiles of 64 in their natural
//    [key][feature] layout, copied with 16-byte coalesced loads staged in
//    registers; two LDS buffers, one barrier per tile, and the next tile's
//    global loads are in flight during the current tile's math.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//    the accumulator then gives every lane ONE query (lane % 32) and 32 of the
//    tile's keys, so the row max and row sum are in-lane reductions plus one
//    v_permlane32_swap between the two 32-lane halves.
//  * The output is accumulated transposed too, O^T += V^T P^T: P leaves the
//    score accumulator already in the B-operand layout (the key order inside
//    each 16-key slice is permuted identically on both operands), and V^T is
//    read with ds_read_b64_tr_b16, the LDS transpose read.
//  * Online softmax with lazy rescaling: the max used in the exponent only
//    moves when a row's max grows by more than a factor 2^8 in probability
//    (8 in log2 units), so the output accumulators are rarely rescaled;
//    weights are then at most 2^8, harmless in fp32 and bf16.  The row sum
//    adds the bf16-rounded weights the P.V product uses (v_dot2c_f32_bf16
//    with (1, 1)).  exp2 of log2(e)/sqrt(d_k)-scaled scores; the Lq x Lk
//    score matrix never leaves registers.
//  * Multi-head path: Q and K arrive as bf16 hi + lo pairs (the projection
//    keeps the rounding residue), and S^T = Kh Qh^T + Kl Qh^T + Kh Ql^T on
//    three MFMAs, so scores keep ~16 significant bits per operand; large
//    logits (embeddings scaled by sqrt(d_model)) then do not flip near-tied
//    softmax rows the way single bf16 operands would.
//  * Causal: tiles above the diagonal are never loaded or multiplied; masks
//    are evaluated only on tiles that cross the diagonal or the valid length.
//    Workgroups are issued heaviest-first, and consecutive workgroup ids take
//    different (batch, head) pairs so that each pair stays on one XCD's L2.
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kD = 64;                 // d_k = d_v
constexpr int kBN = 64;                // keys per tile
template <bool kSplit> constexpr int waves_per_wg() { return kSplit ? 4 : 8; }
// LDS row strides (bf16 elements), measured conflict-free on gfx950: K rows
// read as 16-byte MFMA fragments at 144 B; V rows read with the transpose
// read at 192 B (a 144 B stride costs ~2 conflict cycles per read).
constexpr int kLdsK = kD + 8;
constexpr int kLdsV = kD + 32;
constexpr int kTileK = kBN * kLdsK;    // bf16 elements per K tile
constexpr int kTileV = kBN * kLdsV;    // bf16 elements per V tile
constexpr float kRescaleLog2 = 8.0f;   // lazy-rescale threshold (log2 units)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Per-thread staging registers for one 64 x 64 tile of K and V (and K's low
// parts): 512 16-byte chunks per tensor, spread over the workgroup.
template <bool kSplit, int kThreads>
struct Stage {
    static constexpr int kN = 512 / kThreads;
    uint4 k[kN];
    uint4 v[kN];
    uint4 kl[kSplit ? kN : 1];
};

template <bool kSplit, int kThreads>
__device__ __forceinline__ void load_tile(Stage<kSplit, kThreads>& t, const bf16_t* kb, const bf16_t* klb,
                                          const bf16_t* vb, long long skl, long long svl, int kv0, int Lk,
                                          int tid) {
#pragma unroll
    for (int n = 0; n < Stage<kSplit, kThreads>::kN; ++n) {
        const int c = tid + n * kThreads;
        const int r = c >> 3, col = (c & 7) * 8;
        const int key = kv0 + r;
        if (key < Lk) {
            t.k[n] = *reinterpret_cast<const uint4*>(kb + key * skl + col);
            t.v[n] = *reinterpret_cast<const uint4*>(vb + key * svl + col);
            if (kSplit) t.kl[n] = *reinterpret_cast<const uint4*>(klb + key * skl + col);
        } else {
            t.k[n] = make_uint4(0, 0, 0, 0);
            t.v[n] = make_uint4(0, 0, 0, 0);
            if (kSplit) t.kl[n] = make_uint4(0, 0, 0, 0);
        }
    }
}

// Buffer layout: K [64][kLdsK] | V [64][kLdsV] | (split) K low parts [64][kLdsK].
template <bool kSplit, int kThreads>
__device__ __forceinline__ void store_tile(const Stage<kSplit, kThreads>& t, bf16_t* buf, int tid) {
#pragma unroll
    for (int n = 0; n < Stage<kSplit, kThreads>::kN; ++n) {
        const int c = tid + n * kThreads;
        const int r = c >> 3, col = (c & 7) * 8;
        *reinterpret_cast<uint4*>(buf + r * kLdsK + col) = t.k[n];
        *reinterpret_cast<uint4*>(buf + kTileK + r * kLdsV + col) = t.v[n];
        if (kSplit) *reinterpret_cast<uint4*>(buf + kTileK + kTileV + r * kLdsK + col) = t.kl[n];
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

// Scores S^T (keys x 32 queries) of one 64-key tile: element v of block jb
// holds key kv0 + jb*32 + (v/4)*8 + hb*4 + v%4 for query lane % 32.
template <bool kSplit>
__device__ __forceinline__ void tile_scores(f32x16 (&s)[2], const bf16_t* ks, const bf16_t* kls,
                                            const bf16x8 (&qf)[4], const bf16x8 (&qfl)[4], int l32, int hb) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const bf16x8 kf = frag(ks + (jb * 32 + l32) * kLdsK + kk * 16 + hb * 8);
            s[jb] = mfma32x32x16(kf, qf[kk], kk == 0 ? f32x16{} : s[jb]);
            if (kSplit) {
                const bf16x8 klf = frag(kls + (jb * 32 + l32) * kLdsK + kk * 16 + hb * 8);
                s[jb] = mfma32x32x16(klf, qf[kk], s[jb]);
                s[jb] = mfma32x32x16(kf, qfl[kk], s[jb]);
            }
        }
    }
}

template <bool kCausal, bool kHasVl, bool kOutF32, bool kSplit>
__global__ __launch_bounds__(64 * waves_per_wg<kSplit>(), 2)
void sdpa_fwd_bf16_d64(SdpaArgs a, int n_qtiles, float c_log2) {
    constexpr int kWaves = waves_per_wg<kSplit>();
    constexpr int kThreads = 64 * kWaves;
    constexpr int kBM = kWaves * 32;                           // queries per workgroup
    constexpr int kBuf = (kSplit ? 2 : 1) * kTileK + kTileV;   // bf16 elements per buffer
    __shared__ __attribute__((aligned(16))) bf16_t smem[2 * kBuf];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // The wave index as a scalar: tile-range and mask decisions derived from
    // it are then wave-uniform branches, not per-lane selects.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hb = lane >> 5, l32 = lane & 31;

    // Workgroup -> (query tile, batch, head): (batch, head) varies fastest so
    // one pair's tiles share an XCD; causal issues the longest tiles first.
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
    const int n_tiles = (kv_end + kBN - 1) / kBN;
    // Tiles from index n_wave on lie wholly above this wave's queries.
    const int n_wave = (kCausal && !none) ? min(n_tiles, (q0 + 31) / kBN + 1) : n_tiles;
    // Tiles from index t_mask on need the key-padding, causal or fully-masked rule.
    int t_mask = none ? 0 : kv_lim / kBN;
    if (kCausal && !none) t_mask = min(t_mask, (q0 + 1) / kBN);
    // Per row: keys below key_lim are allowed (a row with no allowed key
    // scores all Lk keys equally, as the -1e9 fill does).
    const int key_lim = none ? Lk : (kCausal ? min(kv_lim, i + 1) : kv_lim);

    const bf16_t* qb = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const bf16_t* kb = static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const bf16_t* vb = static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1];
    const bf16_t* qlb = kSplit ? static_cast<const bf16_t*>(a.q_lo) + b * a.sq[0] + hd * a.sq[1] : nullptr;
    const bf16_t* klb = kSplit ? static_cast<const bf16_t*>(a.k_lo) + b * a.sk[0] + hd * a.sk[1] : nullptr;

    // Prologue: tile 0 into buffer 0, tile 1 into registers.
    Stage<kSplit, kThreads> pre;
    load_tile<kSplit, kThreads>(pre, kb, klb, vb, a.sk[2], a.sv[2], 0, Lk, tid);
    bf16x8 qf[4], qfl[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        if (i < a.Lq) {
            qf[kk] = frag(qb + i * a.sq[2] + kk * 16 + hb * 8);
            if (kSplit) qfl[kk] = frag(qlb + i * a.sq[2] + kk * 16 + hb * 8);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) qf[kk][e] = qfl[kk][e] = static_cast<__bf16>(0.0f);
        }
    }
    store_tile<kSplit, kThreads>(pre, smem, tid);
    if (n_tiles > 1) load_tile<kSplit, kThreads>(pre, kb, klb, vb, a.sk[2], a.sv[2], kBN, Lk, tid);
    __syncthreads();

    f32x16 o0 = {}, o1 = {};          // O^T accumulators: features [0,32) and [32,64)
    float m_used = -INFINITY;          // exponent offset (raw score units)
    float l_run = 0.0f;                // this half's sum of weights
    const float rescale_gap = kRescaleLog2 / c_log2;
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

    int buf = 0;
    for (int t = 0; t < n_tiles; ++t) {
        const int kv0 = t * kBN;
        if (t < n_wave) {
            const bf16_t* ks = smem + buf * kBuf;
            f32x16 s[2];
            tile_scores<kSplit>(s, ks, ks + kTileK + kTileV, qf, qfl, l32, hb);
            // ---- masks (only on tiles that cross the valid length or the
            // diagonal, or when every key of the row is masked) -------------
            if (t >= t_mask) [[unlikely]] {
                // Keep this a real branch: speculated, it would cost ~96 VALU
                // operations on every tile instead of only on edge tiles.
                asm volatile("" ::: "memory");
                // Keys [0, key_lim) of this tile may carry weight for this row.
                const int rel = key_lim - (kv0 + hb * 4);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int jr = (v >> 2) * 8 + (v & 3);
                    s[0][v] = jr < rel ? (none ? 0.0f : s[0][v]) : -INFINITY;
                    s[1][v] = jr + 32 < rel ? (none ? 0.0f : s[1][v]) : -INFINITY;
                }
            }
            // ---- row max (tree of v_max3), lazy rescale ---------------------
            float mr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) mr[r] = fmaxf(s[0][r], s[1][r]);
#pragma unroll
            for (int v = 4; v < 16; v += 4)
#pragma unroll
                for (int r = 0; r < 4; ++r) mr[r] = fmaxf(mr[r], fmaxf(s[0][v + r], s[1][v + r]));
            const float mt = pair_max(fmaxf(fmaxf(mr[0], mr[1]), fmaxf(mr[2], mr[3])));
            // The exponent offset moves only when the max outgrows it by 2^8.
            const bool grow = mt > m_used + rescale_gap;
            if (__any(grow)) {
                const float m_new = grow ? mt : m_used;
                const float alpha = __builtin_amdgcn_exp2f((m_used - m_new) * c_log2);
                m_used = m_new;
                l_run *= alpha;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    o0[v] *= alpha;
                    o1[v] *= alpha;
                }
            }
            // ---- weights, packed as the B operand of O^T += V^T P^T ------------
            // Slice kb covers keys kb*16 + (e/4)*8 + hb*4 + e%4, as bf16 pairs;
            // the row sum adds the rounded pairs.
            const float mc = (m_used == -INFINITY) ? 0.0f : m_used * c_log2;
            float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            u32x4 w[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
#pragma unroll
                for (int qq = 0; qq < 4; ++qq) {
                    const int v = (qq & 1) * 8 + e;
                    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[qq >> 1][v], c_log2, -mc));
                    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[qq >> 1][v + 1], c_log2, -mc));
                    const bf16x2 pp = {static_cast<__bf16>(p0), static_cast<__bf16>(p1)};
                    w[qq][e >> 1] = __builtin_bit_cast(uint32_t, pp);
                    rs[qq] = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, rs[qq], false);
                }
            }
            l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
            const bf16_t* vs = ks + kTileK;
#pragma unroll
            for (int kb2 = 0; kb2 < 4; ++kb2) {
                const bf16x8 pk = __builtin_bit_cast(bf16x8, w[kb2]);
                o0 = mfma32x32x16(v_frag(vs, kb2, 0, hb, lane), pk, o0);
                o1 = mfma32x32x16(v_frag(vs, kb2, 1, hb, lane), pk, o1);
            }
        }

        // Next tile: its registers arrived during this tile's math; the other
        // buffer was last read before the previous barrier.
        if (t + 1 < n_tiles) {
            store_tile<kSplit, kThreads>(pre, smem + (buf ^ 1) * kBuf, tid);
            if (t + 2 < n_tiles) load_tile<kSplit, kThreads>(pre, kb, klb, vb, a.sk[2], a.sv[2], (t + 2) * kBN, Lk, tid);
        }
        __syncthreads();
        buf ^= 1;
    }

    if (i >= a.Lq) return;
    const float inv = 1.0f / pair_sum(l_run);
    // O^T element v of block tb: feature tb*32 + (v/4)*8 + hb*4 + v%4, query i.
    char* ob = static_cast<char*>(a.o);
    const long long orow = b * a.so[0] + hd * a.so[1] + (long long)i * a.so[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int tt = tb * 32 + g4 * 8 + hb * 4;
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (tb == 0 ? o0[g4 * 4 + e] : o1[g4 * 4 + e]) * inv;
            if (kOutF32) {
                *reinterpret_cast<float4*>(ob + (orow + tt) * 4) = make_float4(y[0], y[1], y[2], y[3]);
            } else {
                *reinterpret_cast<uint2*>(ob + (orow + tt) * 2) =
                    make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
            }
        }
    }
}

template <bool kCausal, bool kHasVl, bool kOutF32, bool kSplit>
hipError_t launch_variant(const SdpaArgs& a, hipStream_t s) {
    constexpr int kWaves = waves_per_wg<kSplit>();
    constexpr int kBM = kWaves * 32;
    const int n_qtiles = (a.Lq + kBM - 1) / kBM;
    const long long grid = (long long)n_qtiles * a.B * a.H;
    const float c_log2 = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    hipLaunchKernelGGL((sdpa_fwd_bf16_d64<kCausal, kHasVl, kOutF32, kSplit>), dim3((unsigned)grid),
                       dim3(64 * kWaves), 0, s, a, n_qtiles, c_log2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sdpa_bf16(const SdpaArgs& a, bool out_f32, hipStream_t s) {
    const bool c = a.causal != 0, v = a.valid_lens != nullptr;
    if (a.q_lo != nullptr && a.k_lo != nullptr) {
        // hi + lo operands (the multi-head path); output is the bf16 merged-head buffer
        if (out_f32) return hipErrorInvalidValue;
        if (c) return v ? launch_variant<true, true, false, true>(a, s) : launch_variant<true, false, false, true>(a, s);
        return v ? launch_variant<false, true, false, true>(a, s) : launch_variant<false, false, false, true>(a, s);
    }
    return launch_sdpa_bf16_pipe(a, out_f32, s);
}

}  // namespace mha
