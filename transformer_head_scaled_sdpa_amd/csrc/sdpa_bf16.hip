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
//  * One workgroup = 4 wave64s = 128 consecutive queries of one (batch, head);
//    each wave owns 32 queries and keeps their Q fragment in registers.
//  * Keys/values stream through LDS in tiles of 64, in their natural
//    [key][feature] layout, copied with 16-byte coalesced loads; the next
//    tile is fetched into registers while the current one is used.
//  * Scores are computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//    the accumulator then gives every lane ONE query (lane % 32) and 32 of the
//    tile's keys, so the row max and row sum are in-lane reductions plus one
//    v_permlane32_swap between the two 32-lane halves.
//  * The output is accumulated transposed too, O^T += V^T P^T: P leaves the
//    score accumulator already in the B-operand layout (the key order inside
//    each 16-key slice is permuted identically on both operands), and V^T is
//    read with ds_read_b64_tr_b16, the LDS transpose read.
//  * Online softmax with running max m and running sum l per query; exp2 of
//    log2(e)/sqrt(d_k)-scaled scores; the Lq x Lk score matrix never leaves
//    registers.
//  * Multi-head path: Q and K arrive as bf16 hi + lo pairs (the projection
//    keeps the rounding residue), and S^T = Kh Qh^T + Kl Qh^T + Kh Ql^T on
//    three MFMAs, so scores keep ~16 significant bits per operand; large
//    logits (embeddings scaled by sqrt(d_model)) then do not flip near-tied
//    softmax rows the way single bf16 operands would.
//  * Causal: tiles above the diagonal are never loaded; masks are evaluated
//    only on tiles that cross the diagonal or the valid length.  Workgroups
//    are issued heaviest-first, and consecutive workgroup ids take different
//    (batch, head) pairs so that each pair stays on one XCD's L2.
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kD = 64;                 // d_k = d_v
constexpr int kWaves = 4;
constexpr int kBM = 32 * kWaves;       // queries per workgroup
constexpr int kBN = 64;                // keys per tile
constexpr int kLds = kD + 8;           // LDS row stride (bf16): 144 B, staggers banks

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

struct Tile {
    uint4 k[2];
    uint4 v[2];
    uint4 kl[2];   // low parts of K (split variant only)
};

template <bool kSplit>
__device__ __forceinline__ void load_tile(Tile& t, const bf16_t* kb, const bf16_t* klb, const bf16_t* vb,
                                          long long skl, long long svl, int kv0, int Lk, int tid) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int c = tid + n * 256;          // 512 16-byte chunks per 64 x 64 tile
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

template <bool kSplit>
__device__ __forceinline__ void store_tile(const Tile& t, bf16_t* ks, bf16_t* kls, bf16_t* vs, int tid) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int c = tid + n * 256;
        const int r = c >> 3, col = (c & 7) * 8;
        *reinterpret_cast<uint4*>(ks + r * kLds + col) = t.k[n];
        *reinterpret_cast<uint4*>(vs + r * kLds + col) = t.v[n];
        if (kSplit) *reinterpret_cast<uint4*>(kls + r * kLds + col) = t.kl[n];
    }
}

template <bool kCausal, bool kHasVl, bool kOutF32, bool kSplit>
__global__ __launch_bounds__(256) void sdpa_fwd_bf16_d64(SdpaArgs a, int n_qtiles, float c_log2) {
    __shared__ __attribute__((aligned(16))) bf16_t smem[(kSplit ? 3 : 2) * kBN * kLds];
    bf16_t* const ks = smem;
    bf16_t* const vs = smem + kBN * kLds;
    bf16_t* const kls = smem + 2 * kBN * kLds;   // split variant only

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hb = lane >> 5, l32 = lane & 31;

    // Workgroup -> (query tile, batch, head): (batch, head) varies fastest so
    // one pair's tiles share an XCD; causal issues the longest tiles first.
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH;
    int qt = blockIdx.x / BH;
    if (kCausal) qt = n_qtiles - 1 - qt;
    const int b = bh / a.H, hd = bh % a.H;

    const int q_wg = qt * kBM;
    const int q0 = q_wg + wave * 32;
    const int i = q0 + l32;                       // this lane's query

    const int Lk = a.Lk;
    int vlen = kHasVl ? a.valid_lens[b] : Lk;
    const bool none = vlen <= 0;                  // every key masked -> uniform weights
    const int kv_lim = none ? Lk : min(vlen, Lk); // keys [0, kv_lim) can carry weight
    int kv_end = kv_lim;
    if (kCausal && !none) kv_end = min(kv_end, q_wg + kBM);

    const bf16_t* qb = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const bf16_t* kb = static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const bf16_t* vb = static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1];
    const bf16_t* qlb = kSplit ? static_cast<const bf16_t*>(a.q_lo) + b * a.sq[0] + hd * a.sq[1] : nullptr;
    const bf16_t* klb = kSplit ? static_cast<const bf16_t*>(a.k_lo) + b * a.sk[0] + hd * a.sk[1] : nullptr;

    // Q fragment (B operand of S^T = K Q^T): lane holds q_i[kk*16 + hb*8 .. +8).
    bf16x8 qf[4], qfl[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        if (i < a.Lq) {
            qf[kk] = *reinterpret_cast<const bf16x8*>(qb + i * a.sq[2] + kk * 16 + hb * 8);
            if (kSplit) qfl[kk] = *reinterpret_cast<const bf16x8*>(qlb + i * a.sq[2] + kk * 16 + hb * 8);
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) qf[kk][s] = qfl[kk][s] = static_cast<__bf16>(0.0f);
        }
    }

    f32x16 o0 = {}, o1 = {};        // O^T accumulators: features [0,32) and [32,64)
    float m_run = -INFINITY;        // running max of raw scores (both halves agree)
    float l_run = 0.0f;             // running sum over this half's keys

    Tile pre;
    if (kv_end > 0) load_tile<kSplit>(pre, kb, klb, vb, a.sk[2], a.sv[2], 0, Lk, tid);

    for (int kv0 = 0; kv0 < kv_end; kv0 += kBN) {
        __syncthreads();                          // previous tile fully consumed
        store_tile<kSplit>(pre, ks, kls, vs, tid);
        __syncthreads();
        if (kv0 + kBN < kv_end) load_tile<kSplit>(pre, kb, klb, vb, a.sk[2], a.sv[2], kv0 + kBN, Lk, tid);

        // Whole tile above this wave's queries: nothing to add.
        if (kCausal && !none && kv0 > q0 + 31) continue;

        // ---- S^T = K Q^T for 64 keys (two 32-key blocks) -------------------
        f32x16 s0 = {}, s1 = {};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(ks + l32 * kLds + kk * 16 + hb * 8);
            const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(ks + (32 + l32) * kLds + kk * 16 + hb * 8);
            s0 = mfma32x32x16(k0, qf[kk], s0);
            s1 = mfma32x32x16(k1, qf[kk], s1);
            if (kSplit) {
                const bf16x8 kl0 = *reinterpret_cast<const bf16x8*>(kls + l32 * kLds + kk * 16 + hb * 8);
                const bf16x8 kl1 = *reinterpret_cast<const bf16x8*>(kls + (32 + l32) * kLds + kk * 16 + hb * 8);
                s0 = mfma32x32x16(kl0, qf[kk], s0);
                s1 = mfma32x32x16(kl1, qf[kk], s1);
                s0 = mfma32x32x16(k0, qfl[kk], s0);
                s1 = mfma32x32x16(k1, qfl[kk], s1);
            }
        }
        // Element v of block jb holds key kv0 + jb*32 + (v/4)*8 + hb*4 + v%4.
        const int jl = kv0 + hb * 4;
        if (none) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = jl + (v >> 2) * 8 + (v & 3);
                s0[v] = (j < Lk) ? 0.0f : -INFINITY;
                s1[v] = (j + 32 < Lk) ? 0.0f : -INFINITY;
            }
        } else if (kv0 + kBN > kv_lim || (kCausal && kv0 + kBN - 1 > q0)) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int j = jl + (v >> 2) * 8 + (v & 3);
                bool ok0 = j < kv_lim, ok1 = j + 32 < kv_lim;
                if (kCausal) {
                    ok0 = ok0 && (j <= i);
                    ok1 = ok1 && (j + 32 <= i);
                }
                s0[v] = ok0 ? s0[v] : -INFINITY;
                s1[v] = ok1 ? s1[v] : -INFINITY;
            }
        }

        // ---- online softmax --------------------------------------------------
        float mt = fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int v = 1; v < 16; ++v) mt = fmaxf(mt, fmaxf(s0[v], s1[v]));
        mt = pair_max(mt);
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * c_log2);
        const float mc = m_use * c_log2;
        float rs = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            s0[v] = __builtin_amdgcn_exp2f(fmaf(s0[v], c_log2, -mc));
            s1[v] = __builtin_amdgcn_exp2f(fmaf(s1[v], c_log2, -mc));
            rs += s0[v] + s1[v];
        }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            o0[v] *= alpha;
            o1[v] *= alpha;
        }

        // P^T as B operand: slice kb covers keys kb*16 + (s/4)*8 + hb*4 + s%4.
        bf16x8 pb[4];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            pb[0][s] = static_cast<__bf16>(s0[s]);
            pb[1][s] = static_cast<__bf16>(s0[8 + s]);
            pb[2][s] = static_cast<__bf16>(s1[s]);
            pb[3][s] = static_cast<__bf16>(s1[8 + s]);
        }

        // ---- O^T += V^T P^T ------------------------------------------------
        // Transpose read: in each 16-lane group, lane r points at key row
        // base + r/4, features T + (r%4)*4; lane j of the group then receives
        // features T + j of keys base .. base+3.
        const int g = lane >> 4, r = lane & 15;
        const int th = g & 1;
#pragma unroll
        for (int kb2 = 0; kb2 < 4; ++kb2) {
            const int row = kb2 * 16 + hb * 4 + (r >> 2);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const int col = tb * 32 + th * 16 + (r & 3) * 4;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vs + row * kLds + col));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vs + (row + 8) * kLds + col));
                // Join the two halves as whole vectors: inserting the 16-bit
                // elements one by one is lowered incorrectly by the compiler.
                const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                const bf16x8 va = __builtin_bit_cast(bf16x8, both);
                if (tb == 0) o0 = mfma32x32x16(va, pb[kb2], o0);
                else o1 = mfma32x32x16(va, pb[kb2], o1);
            }
        }
    }

    if (i >= a.Lq) return;
    const float l_tot = pair_sum(l_run);
    const float inv = 1.0f / l_tot;
    // O^T element v of block tb: feature tb*32 + (v/4)*8 + hb*4 + v%4, query i.
    char* ob = static_cast<char*>(a.o);
    const long long orow = b * a.so[0] + hd * a.so[1] + (long long)i * a.so[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int t = tb * 32 + g4 * 8 + hb * 4;
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) x[e] = (tb == 0 ? o0[g4 * 4 + e] : o1[g4 * 4 + e]) * inv;
            if (kOutF32) {
                *reinterpret_cast<float4*>(ob + (orow + t) * 4) = make_float4(x[0], x[1], x[2], x[3]);
            } else {
                *reinterpret_cast<uint2*>(ob + (orow + t) * 2) =
                    make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
            }
        }
    }
}

template <bool kCausal, bool kHasVl, bool kOutF32, bool kSplit>
hipError_t launch_variant(const SdpaArgs& a, hipStream_t s) {
    const int n_qtiles = (a.Lq + kBM - 1) / kBM;
    const long long grid = (long long)n_qtiles * a.B * a.H;
    const float c_log2 = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    hipLaunchKernelGGL((sdpa_fwd_bf16_d64<kCausal, kHasVl, kOutF32, kSplit>), dim3((unsigned)grid), dim3(256),
                       0, s, a, n_qtiles, c_log2);
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
    if (out_f32) {
        if (c) return v ? launch_variant<true, true, true, false>(a, s) : launch_variant<true, false, true, false>(a, s);
        return v ? launch_variant<false, true, true, false>(a, s) : launch_variant<false, false, true, false>(a, s);
    }
    if (c) return v ? launch_variant<true, true, false, false>(a, s) : launch_variant<true, false, false, false>(a, s);
    return v ? launch_variant<false, true, false, false>(a, s) : launch_variant<false, false, false, false>(a, s);
}

}  // namespace mha
