// Backward pass of scaled dot-product attention on bf16 MFMA (fp32
// accumulate), d_k = d_v = 64, gfx950: the same gradients as the fp32 kernels
// (dq, dk, dv for an output gradient do; see sdpa_backward.hip), for bf16
// inputs.  With tau = 1/sqrt(d_k), p the weights, D_i = do_i . o_i:
//   dv_j = sum_i p_ij do_i,  ds_ij = p_ij (do_i . v_j - D_i),
//   dq_i = tau sum_j ds_ij k_j,  dk_j = tau sum_i ds_ij q_i   (allowed pairs;
// a row with no allowed key weights all keys uniformly and passes no
// gradient to q or k).
//
// Workgroups of 4 wave64s in two roles, two workgroups per CU.  A workgroup
// owns 64 rows (two groups of 32, one row per lane column of the 32x32 MFMA
// tile) and streams the other side in steps of 64 rows: two phases of 32,
// one per wave of a group, so every wave works on its own tile and the two
// partial sums of a row are added through LDS at the end.  Products run on
// v_mfma_f32_32x32x16_bf16 in the operand layouts of the forward kernel: an
// accumulator packed to bf16 feeds the next MFMA as its B operand, and
// transposed tiles are read from LDS with ds_read_b64_tr_b16 (tiles read both
// ways are stored twice: 144-byte rows for 16-byte fragment reads, 192-byte
// rows for the transposed reads).
//  * rows (queries; q and do fragments in registers): S^T = K Q^T and
//    dP^T - D = V dO^T - D, the weights P^T, dS^T = P^T (dP^T - D) and
//    dQ^T += K^T dS^T over the keys.  Without the forward's log-sum-exp the
//    weights are exp2(S - m) with a lazy per-query offset m (the online
//    softmax); the phases' (m, weight sum, dq) are merged at the end, dq is
//    divided by the weight sum, and the log-sum-exp and D_i (from the
//    supplied output) go to the workspace.  With it they are
//    exp2(S - lse) directly.
//  * keys (k and v fragments in registers): S = Q K^T and dP - D = dO V^T - D,
//    P and dS from the log-sum-exp and D in the workspace, then
//    dV^T += dO^T P and dK^T += Q^T dS.
// Without a log-sum-exp the rows kernel runs first and the keys kernel reads
// its results.  With one, a small kernel writes D_i and the log-sum-exp in
// log2 units to the workspace, and a single launch holds both roles (they no
// longer depend on each other): the key side first, each side heaviest
// blocks first.
// dS (and P for dV) is rounded to bf16 for its products, as P is in the
// forward.  Tiles where every pair is allowed skip the mask arithmetic.
#include "common.h"
#include "kernels.h"
#define MFMA_ROWS_WAVES 4
#include "mfma_rows.h"

namespace mha {

namespace {

using namespace rows64;

// ---------------------------------------------------------------------------
// rows: dq (and without a log-sum-exp: the log-sum-exp and D)
// ---------------------------------------------------------------------------
// LDS: the K and V tiles in 144-byte rows (score products) in two slots,
// the K tiles in 192-byte rows (transposed reads for dq) in three: step st
// goes to K/V slot st % 2 and K^T slot st % 3.  The scores of step st + 1 are
// computed during step st, so at step st the K/V slot of st + 1 and the K^T
// slot of st are read while step st + 2 is written to the slots of st (K/V,
// last read during step st - 1) and st - 1 (K^T).  The staged Q, dO and O
// sit at the start until every wave has read its fragments (then the first
// two steps are stored), the dq partials at the start after the last step,
// and the per-phase (m, weight sum) after everything.  75 KB in all, so two
// workgroups fit a CU.
constexpr int kRowsSlotR = kPhases * kTileRB;     // one step in 144-byte rows
constexpr int kRowsSlotT = kPhases * kTileTB;     // one step in 192-byte rows
constexpr int kRowsKR = 0;
constexpr int kRowsVR = 2 * kRowsSlotR;
constexpr int kRowsKT = 4 * kRowsSlotR;
constexpr int kRowsStat = kRowsKT + 3 * kRowsSlotT;
static_assert(3 * kStageB <= kRowsStat, "staging fits");
constexpr int kRowsLds = kRowsStat + kGroups * kPhases * 2 * 32 * 8;
static_assert(kRowsKT + 3 * kRowsSlotT <= kRowsStat && kRedAllB <= kRowsStat, "tiles and partials fit");

// ---------------------------------------------------------------------------
// keys: dk, dv
// ---------------------------------------------------------------------------
constexpr int kKeysQR = 0;                        // Q, 144-byte rows
constexpr int kKeysQT = kTileRB;                  // Q, 192-byte rows
constexpr int kKeysGR = kTileRB + kTileTB;        // dO, 144-byte rows
constexpr int kKeysGT = 2 * kTileRB + kTileTB;    // dO, 192-byte rows
constexpr int kKeysPhase = 2 * kTileRB + 2 * kTileTB;
// The step tiles, reused first for the staged K and V and last for the dv
// and dk partials; then per streamed query the log-sum-exp, -D, score scale
// and gradient factor (0 for a row with no allowed key), key limit, and per
// phase tile the smallest key limit (-1 if a row has none allowed).
constexpr int kKeysTiles = kPhases * kKeysPhase > 2 * kRedAllB ? kPhases * kKeysPhase : 2 * kRedAllB;
constexpr int kKeysRowData = kKeysTiles;
constexpr int kKeysLds = kKeysRowData + 5 * kStep * 4 + kPhases * 4;
static_assert(2 * kStageB <= kKeysTiles, "staging fits");

constexpr int kFusedLds = kRowsLds > kKeysLds ? kRowsLds : kKeysLds;

template <bool kCausal, bool kLse>
__device__ __forceinline__ void rows_body(const BackwardArgs& a, float c, int blk, int bh, char* smem) {
    float2* const stat = reinterpret_cast<float2*>(smem + kRowsStat);   // [grp][phase][half][32]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave % kGroups, ph = wave / kGroups;
    const int hb = lane >> 5, l32 = lane & 31;
    const int b = bh / a.H, hd = bh % a.H;
    // Causal rows late in the sequence see the most keys: they go first.
    const int n_wg = (a.Lq + kRowsWg - 1) / kRowsWg;
    const int q_wg = (kCausal ? n_wg - 1 - blk : blk) * kRowsWg;
    const int i = q_wg + grp * 32 + l32;
    const int Lq = a.Lq, Lk = a.Lk;
    const bool live = i < Lq;

    // One length per sequence is read once as a scalar: a per-lane read of it
    // (under the lane's `live` test) would be a vector load whose wait comes
    // before the prologue's loads are issued.
    const int len_b = a.vl_rank == 1 ? a.valid_lens[b] : 0;
    bool none = false;
    const int klim = !live ? Lk
                           : (a.vl_rank == 2 ? key_limit<kCausal>(a, b, i, none)
                                             : limit_from_len<kCausal>(a, a.vl_rank == 1 ? len_b : Lk, i, none));
    // Score scale (log2 units).  A row with no allowed key weights its keys
    // equally: its scale 2^-100 makes every finite score's exponent round to
    // the same value while masked keys (-inf) still weigh 0.
    const float cs = none ? 0x1p-100f : c;
    int kmin = klim;                        // smallest key limit in the wave
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) kmin = min(kmin, __shfl_xor(kmin, o));
    kmin = __builtin_amdgcn_readfirstlane(kmin);
    // Keys this workgroup must visit.  With one length per sequence, a
    // positive length bounds every row's keys (and the causal bound still
    // holds), while a length <= 0 spreads each row over all Lk keys; lengths
    // per query keep every key.
    const bool len_bound = a.vl_rank == 1 && len_b > 0;
    int kv_end = len_bound ? min(Lk, len_b) : Lk;
    if (kCausal && (a.vl_rank == 0 || len_bound)) kv_end = min(kv_end, q_wg + kRowsWg);
    const int n_steps = (kv_end + kStep - 1) / kStep;

    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const bf16_t* gp = static_cast<const bf16_t*>(a.dout) + b * a.sdo[0] + hd * a.sdo[1];
    const bf16_t* op = static_cast<const bf16_t*>(a.o) + b * a.so[0] + hd * a.so[1];
    const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1];

    // This workgroup's 64 rows of Q and dO (and O when D is formed here):
    // one range-checked 16-byte chunk per thread each (zeros past the
    // queries), issued first and staged through LDS, so the phase waves
    // of a group read their fragments from there instead of each loading
    // them.  With a log-sum-exp, that and D come from the workspace.
    const StepSrc qsrc = step_src(qp, a.sq[2], Lq, tid), gsrc = step_src(gp, a.sdo[2], Lq, tid);
    const StageChunks cq = load_chunks(qsrc, q_wg), cg = load_chunks(gsrc, q_wg);
    StageChunks co;
    float2 given = make_float2(0.0f, 0.0f);   // (log-sum-exp in log2 units, D) with kLse
    if constexpr (kLse) {
        // Range-checked: rows past the queries read zeros.
        typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
        const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
            a.rows + (long long)bh * Lq * 2, (short)0, Lq * 8, kBufWord3);
        const u32x2v x = __builtin_amdgcn_raw_buffer_load_b64(rr, (uint32_t)i * 8u, 0, 0);
        given = make_float2(__uint_as_float(x[0]), __uint_as_float(x[1]));
    } else {
        co = load_chunks(step_src(op, a.so[2], Lq, tid), q_wg);
    }
    __builtin_amdgcn_sched_barrier(0);

    // K and V steps go to LDS two steps before their scores are computed
    // (see the slots above), from registers loaded two steps before that
    // (even and odd steps in their own registers).  The range ends at the
    // last key the workgroup visits, so loads past it read zeros without a
    // memory access and every load and store is unconditional: each store
    // waits only for its own loads.  The prologue issues them in the loop's
    // order, so the waits the compiler derives hold on every iteration.
    const StepSrc ksrc = step_src(kp, a.sk[2], kv_end, tid), vsrc = step_src(vp, a.sv[2], kv_end, tid);
    Chunks nk_e = load_step(ksrc, 0), nv_e = load_step(vsrc, 0);
    __builtin_amdgcn_sched_barrier(0);
    Chunks nk_o = load_step(ksrc, kStep), nv_o = load_step(vsrc, kStep);
    __builtin_amdgcn_sched_barrier(0);
    auto put = [&](const Chunks& nk, const Chunks& nv, int slot2, int slot3) {
        store_step(nk, smem + kRowsKR + slot2 * kRowsSlotR, kTileRB, 0, -1, tid);
        store_step(nv, smem + kRowsVR + slot2 * kRowsSlotR, kTileRB, 0, -1, tid);
        store_step(nk, smem + kRowsKT + slot3 * kRowsSlotT, kTileTB, -1, 0, tid);
    };
    char* const stage = smem;   // overlaps the tile slots: read out before the first steps go in
    stage_chunks(stage, 0, cq, tid);
    stage_chunks(stage, 1, cg, tid);
    if constexpr (!kLse) stage_chunks(stage, 2, co, tid);
    __syncthreads();

    // Q and dO fragments (B operands: query lane%32, features kk*16 + hb*8 ..);
    // a row with no allowed key passes no gradient through its scores, so
    // its dO fragment is zero (with D below, dp - D is then 0).
    bf16x8 qf[4], gf[4];
    float dsum = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const uint4 rq = staged_frag(stage, 0, grp * 32 + l32, kk, hb);
        const uint4 rg = staged_frag(stage, 1, grp * 32 + l32, kk, hb);
        qf[kk] = __builtin_bit_cast(bf16x8, rq);
        gf[kk] = __builtin_bit_cast(bf16x8, none ? make_uint4(0, 0, 0, 0) : rg);
        if constexpr (!kLse) {
            const uint4 ro = staged_frag(stage, 2, grp * 32 + l32, kk, hb);
            const uint32_t ug[4] = {rg.x, rg.y, rg.z, rg.w}, uo[4] = {ro.x, ro.y, ro.z, ro.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dsum += __uint_as_float(ug[e] << 16) * __uint_as_float(uo[e] << 16) +
                        __uint_as_float(ug[e] & 0xffff0000u) * __uint_as_float(uo[e] & 0xffff0000u);
        }
    }
    if constexpr (kLse) dsum = given.y;
    else dsum = pair_sum(dsum);             // D_i over both lane halves
    __syncthreads();                        // every wave's fragments read: the steps may overwrite the staging
    put(nk_e, nv_e, 0, 0);
    nk_e = load_step(ksrc, 2 * kStep);
    nv_e = load_step(vsrc, 2 * kStep);
    put(nk_o, nv_o, 1, 1);
    nk_o = load_step(ksrc, 3 * kStep);
    nv_o = load_step(vsrc, 3 * kStep);
    __syncthreads();
    // dP^T - D starts from -D in the accumulator (element v of a lane is the
    // lane's query).
    f32x16 neg_d;
#pragma unroll
    for (int v = 0; v < 16; ++v) neg_d[v] = none ? 0.0f : -dsum;

    // ---- the pass over the keys ----
    // Without a log-sum-exp: online softmax with a lazy offset.  dq
    // accumulates exp2(s - m) (dp - D) k with the offset m of this lane's
    // query (equal on both lane halves); m moves only when a tile's max
    // exceeds it by more than kLazy, and then dq and the weight sum l (this
    // lane half's keys) are rescaled.  The phases merge at the end.  With
    // one, m is the log-sum-exp and never moves.
    constexpr float kLazy = 10.0f;
    float m = kLse ? given.x : -INFINITY, l = 0.0f;
    f32x16 dq[2] = {};
    // S^T = K Q^T and dP^T - D = V dO^T - D of step st from its K/V slot.
    auto scores = [&](int st, f32x16& s, f32x16& dp) {
        const char* kr = smem + kRowsKR + (st & 1) * kRowsSlotR + ph * kTileRB;
        const char* vr = smem + kRowsVR + (st & 1) * kRowsSlotR + ph * kTileRB;
        s = tile_dot(reinterpret_cast<const bf16_t*>(kr), qf, l32, hb);
        dp = tile_dot_from(reinterpret_cast<const bf16_t*>(vr), gf, neg_d, l32, hb);
    };
    f32x16 s_e, dp_e, s_o, dp_o;
    scores(0, s_e, dp_e);
    // Step st (K^T slot t3 = st % 3): its scores (s, dp) were computed during
    // step st - 1; compute step st + 1's into (s_n, dp_n), then the weights
    // and dq; store step st + 2 from (nk, nv) and load step st + 4 there.
    auto step = [&](int st, int t3, Chunks& nk, Chunks& nv, f32x16& s, f32x16& dp, f32x16& s_n, f32x16& dp_n) {
        __syncthreads();   // step st + 1 stored; the slots of st (K/V) and st - 1 (K^T) free
        put(nk, nv, st & 1, t3 == 0 ? 2 : t3 - 1);
        nk = load_step(ksrc, (st + 4) * kStep);
        nv = load_step(vsrc, (st + 4) * kStep);
        scores(st + 1, s_n, dp_n);
        const int t0 = st * kStep + ph * kTile;   // this wave's keys t0 .. t0+31
        // Masked keys score -inf (weight 0).
        if (t0 + kTile > kmin) {
            const int rel = klim - (t0 + hb * 4);
#pragma unroll
            for (int v = 0; v < 16; ++v) s[v] = acc_row(v) < rel ? s[v] : -INFINITY;
        }
        if constexpr (!kLse) {
            // The tile's row max in log2 units; raise the offset if needed.
            float mx = s[0];
#pragma unroll
            for (int v = 1; v < 16; ++v) mx = fmaxf(mx, s[v]);
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
        }
        // The weights exp2(s * cs - m): without a log-sum-exp, m is 0 until a
        // row has an allowed key (its weights are 0 until then).
        const float m_use = (kLse || m != -INFINITY) ? m : 0.0f;
        f32x16 ds;
        [[maybe_unused]] float q4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            float pr[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int v = g * 4 + e;
                pr[e] = __builtin_amdgcn_exp2f(fmaf(s[v], cs, -m_use));
                ds[v] = pr[e] * dp[v];
            }
            if constexpr (!kLse) q4[g] = (pr[0] + pr[1]) + (pr[2] + pr[3]);
        }
        if constexpr (!kLse) l += (q4[0] + q4[1]) + (q4[2] + q4[3]);
        u32x4 w[2];
        pack_b(ds, w);
        const bf16_t* kt = reinterpret_cast<const bf16_t*>(smem + kRowsKT + t3 * kRowsSlotT + ph * kTileTB);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 d8 = __builtin_bit_cast(bf16x8, w[kb]);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) dq[tb] = mfma32x32x16(tr_frag(kt, kb, tb, hb, lane), d8, dq[tb]);
        }
    };
    // Pairs of steps, then a lone last step: no path through the loop skips
    // a load, so every wait covers exactly the step it stores.  (The scores
    // computed during the last step are past the keys and unused.)
    int st = 0, t3 = 0;
    for (; st + 1 < n_steps; st += 2) {
        step(st, t3, nk_e, nv_e, s_e, dp_e, s_o, dp_o);
        t3 = t3 == 2 ? 0 : t3 + 1;
        step(st + 1, t3, nk_o, nv_o, s_o, dp_o, s_e, dp_e);
        t3 = t3 == 2 ? 0 : t3 + 1;
    }
    if (st < n_steps) step(st, t3, nk_e, nv_e, s_e, dp_e, s_o, dp_o);

    float own = 1.0f, dq_scale = 0.125f, lse = 0.0f;
    if constexpr (!kLse) {
        // Merge the phases: common offset M, total weight L, rescaled dq.
        stat[((grp * kPhases + ph) * 2 + hb) * 32 + l32] = make_float2(m, l);
        __syncthreads();
        float M = -INFINITY;
#pragma unroll
        for (int p = 0; p < kPhases; ++p) M = fmaxf(M, stat[((grp * kPhases + p) * 2) * 32 + l32].x);
        float L = 0.0f;
#pragma unroll
        for (int p = 0; p < kPhases; ++p)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float2 x = stat[((grp * kPhases + p) * 2 + h) * 32 + l32];
                L += x.x == -INFINITY ? 0.0f : x.y * __builtin_amdgcn_exp2f(x.x - M);
            }
        own = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - M);
        dq_scale = L > 0.0f ? 0.125f / L : 0.0f;
        // v_log_f32 is the base-2 logarithm, matching the log2-unit scores.
        lse = L > 0.0f ? M + __builtin_amdgcn_logf(L) : 0.0f;
    } else {
        __syncthreads();
    }
    // The barrier above also ends every wave's reads of the last step's
    // tiles, so the partials may overwrite them.
    float* red = reinterpret_cast<float*>(smem);
    part_write(red, dq, own, grp, ph, lane);
    __syncthreads();
    float4 r[kPartQ];
    part_sum(red, r, grp, ph, lane);
    if (!live) return;
    if constexpr (!kLse) {
        if (ph == 0 && hb == 0)
            reinterpret_cast<float2*>(a.rows)[(long long)bh * Lq + i] = make_float2(lse, dsum);
    }
    store_part(a.dq, b * a.sdq[0] + hd * a.sdq[1] + (long long)i * a.sdq[2], a.out_f32, r, dq_scale, ph, hb);
}

template <bool kCausal>
__device__ __forceinline__ void keys_body(const BackwardArgs& a, float c, int blk, int bh, char* smem) {
    float* const lse_s = reinterpret_cast<float*>(smem + kKeysRowData);
    float* const nd_s = lse_s + kStep;
    float* const sc_s = nd_s + kStep;
    float* const gw_s = sc_s + kStep;
    int* const klim_s = reinterpret_cast<int*>(gw_s + kStep);
    int* const tmin_s = klim_s + kStep;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = wave % kGroups, ph = wave / kGroups;
    const int hb = lane >> 5, l32 = lane & 31;
    const int b = bh / a.H, hd = bh % a.H;
    const int k_wg = blk * kRowsWg;                 // causal: early keys see the most queries and go first
    const int j = k_wg + grp * 32 + l32;            // this lane's key
    const int j_last = k_wg + grp * 32 + 31;
    const int Lq = a.Lq, Lk = a.Lk;

    const bf16_t* kp = static_cast<const bf16_t*>(a.k) + b * a.sk[0] + hd * a.sk[1];
    const bf16_t* vp = static_cast<const bf16_t*>(a.v) + b * a.sv[0] + hd * a.sv[1];
    const bf16_t* qp = static_cast<const bf16_t*>(a.q) + b * a.sq[0] + hd * a.sq[1];
    const bf16_t* gp = static_cast<const bf16_t*>(a.dout) + b * a.sdo[0] + hd * a.sdo[1];

    // Under the causal rule queries before the workgroup's first key weigh
    // none of its keys, unless a length <= 0 (or lengths per query) may
    // spread a query over all keys.  With one positive length per sequence,
    // keys at or past it are weighed by no query: their gradients are zero.
    const int len_all = a.vl_rank == 1 ? a.valid_lens[b] : Lk;
    const bool len_bound = a.vl_rank == 1 && len_all > 0;
    const int i_begin = (kCausal && (a.vl_rank == 0 || len_bound)) ? k_wg : 0;
    const int n_steps = (len_bound && k_wg >= len_all) ? 0 : (Lq - i_begin + kStep - 1) / kStep;
    // This workgroup's 64 rows of K and V: one range-checked 16-byte chunk
    // per thread each (zeros past the keys), staged through LDS like the
    // rows' Q and dO.
    const StepSrc ksrc = step_src(kp, a.sk[2], Lk, tid), vsrc = step_src(vp, a.sv[2], Lk, tid);
    const StageChunks ck = load_chunks(ksrc, k_wg), cv = load_chunks(vsrc, k_wg);
    __builtin_amdgcn_sched_barrier(0);

    // Per streamed query (threads below kStep keep them): log-sum-exp and D
    // from the workspace and the query's length, read one step ahead by
    // range-checked loads (zeros past the queries; the length load has an
    // empty range unless lengths vary by query).
    const __amdgpu_buffer_rsrc_t rows_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        a.rows + (long long)bh * Lq * 2, (short)0, Lq * 8, kBufWord3);
    const __amdgpu_buffer_rsrc_t len_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int*>(a.vl_rank == 2 ? a.valid_lens + (long long)b * Lq : a.valid_lens), (short)0,
        a.vl_rank == 2 ? Lq * 4 : 0, kBufWord3);
    struct RowRaw {
        float lse, dsum;
        int len;
    };
    auto fetch_rows = [&](int i0) {
        typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
        const uint32_t qi = (uint32_t)(i0 + (tid & (kStep - 1)));
        const u32x2v v = __builtin_amdgcn_raw_buffer_load_b64(rows_rsrc, qi * 8u, 0, 0);
        const int len = (int)__builtin_amdgcn_raw_buffer_load_b32(len_rsrc, qi * 4u, 0, 0);
        return RowRaw{__uint_as_float(v[0]), __uint_as_float(v[1]), a.vl_rank == 2 ? len : len_all};
    };

    // Q and dO steps are loaded two steps before they are stored (even and
    // odd steps in their own registers) and the query data one step before,
    // all unconditionally: steps past the queries read as zeros.  The
    // prologue issues them in the loop's order, so the waits the compiler
    // derives hold on every iteration.
    const StepSrc qsrc = step_src(qp, a.sq[2], Lq, tid), gsrc = step_src(gp, a.sdo[2], Lq, tid);
    __builtin_amdgcn_sched_barrier(0);
    Chunks nq_e = load_step(qsrc, i_begin), ng_e = load_step(gsrc, i_begin);
    __builtin_amdgcn_sched_barrier(0);
    RowRaw nr = fetch_rows(i_begin);
    __builtin_amdgcn_sched_barrier(0);
    Chunks nq_o = load_step(qsrc, i_begin + kStep), ng_o = load_step(gsrc, i_begin + kStep);
    __builtin_amdgcn_sched_barrier(0);
    stage_chunks(smem, 0, ck, tid);
    stage_chunks(smem, 1, cv, tid);
    __syncthreads();
    // K and V fragments (B operands: key lane%32, features kk*16 + hb*8 ..).
    bf16x8 kf[4], vf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        kf[kk] = __builtin_bit_cast(bf16x8, staged_frag(smem, 0, grp * 32 + l32, kk, hb));
        vf[kk] = __builtin_bit_cast(bf16x8, staged_frag(smem, 1, grp * 32 + l32, kk, hb));
    }

    f32x16 dk[2] = {}, dv[2] = {};
    auto step = [&](int st, Chunks& nq, Chunks& ng) {
        const int i0 = i_begin + st * kStep;
        __syncthreads();
        store_step(nq, smem, kKeysPhase, kKeysQR, kKeysQT, tid);
        store_step(ng, smem, kKeysPhase, kKeysGR, kKeysGT, tid);
        if (tid < kStep) {
            const int qi = i0 + tid;
            bool none = false;
            const int kl = qi < Lq ? limit_from_len<kCausal>(a, nr.len, qi, none) : 0;
            lse_s[tid] = nr.lse;
            nd_s[tid] = -nr.dsum;
            sc_s[tid] = none ? 0.0f : c;
            gw_s[tid] = none ? 0.0f : 1.0f;
            klim_s[tid] = kl;
            int mn = none ? -1 : kl;
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) mn = min(mn, __shfl_xor(mn, o));
            if ((tid & 31) == 0) tmin_s[tid >> 5] = mn;
        }
        __builtin_amdgcn_sched_barrier(0);
        nr = fetch_rows(i0 + kStep);
        __builtin_amdgcn_sched_barrier(0);
        nq = load_step(qsrc, i0 + 2 * kStep);
        ng = load_step(gsrc, i0 + 2 * kStep);
        __syncthreads();
        // S = Q K^T and dP - D = dO V^T - D: element v is query ph*32 +
        // acc_row(v) + hb*4 of this step, key j; the dP accumulator starts
        // from -D of its query (four consecutive queries per 16-byte read).
        const char* area = smem + ph * kKeysPhase;
        const int rb = ph * kTile + hb * 4;
        f32x16 nd;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 x = *reinterpret_cast<const float4*>(nd_s + rb + g * 8);
            nd[g * 4] = x.x;
            nd[g * 4 + 1] = x.y;
            nd[g * 4 + 2] = x.z;
            nd[g * 4 + 3] = x.w;
        }
        f32x16 p = tile_dot(reinterpret_cast<const bf16_t*>(area + kKeysQR), kf, l32, hb);
        f32x16 ds = tile_dot_from(reinterpret_cast<const bf16_t*>(area + kKeysGR), vf, nd, l32, hb);
        if (j_last < __builtin_amdgcn_readfirstlane(tmin_s[ph])) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const float4 x = *reinterpret_cast<const float4*>(lse_s + rb + g * 8);
                const float lse4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int v = g * 4 + e;
                    p[v] = __builtin_amdgcn_exp2f(fmaf(p[v], c, -lse4[e]));
                    ds[v] *= p[v];
                }
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int r = rb + acc_row(v);
                const float e = __builtin_amdgcn_exp2f(fmaf(p[v], sc_s[r], -lse_s[r]));
                p[v] = j < klim_s[r] ? e : 0.0f;
                ds[v] *= p[v] * gw_s[r];
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
    };
    // Pairs of steps, then a lone last step.  The loads past the last step
    // read past the end of Q and dO (the stream runs to the last query), so
    // they return zeros without a memory access and cost the end nothing.
    int st = 0;
    for (; st + 1 < n_steps; st += 2) {
        step(st, nq_e, ng_e);
        step(st + 1, nq_o, ng_o);
    }
    if (st < n_steps) step(st, nq_e, ng_e);
    // Both sums in one round: dv's slots, then dk's.
    float* red = reinterpret_cast<float*>(smem);
    __syncthreads();
    part_write(red, dv, 1.0f, grp, ph, lane);
    part_write(red + kRedAllB / 4, dk, 1.0f / 8.0f, grp, ph, lane);
    __syncthreads();
    float4 rv[kPartQ], rk[kPartQ];
    part_sum(red, rv, grp, ph, lane);
    part_sum(red + kRedAllB / 4, rk, grp, ph, lane);
    if (j >= Lk) return;
    store_part(a.dk, b * a.sdk[0] + hd * a.sdk[1] + (long long)j * a.sdk[2], a.out_f32, rk, 1.0f, ph, hb);
    store_part(a.dv, b * a.sdv[0] + hd * a.sdv[1] + (long long)j * a.sdv[2], a.out_f32, rv, 1.0f, ph, hb);
}

template <bool kCausal>
__global__ __launch_bounds__(kThreads, 2) void bwd_rows_mfma(BackwardArgs a, float c) {
    __shared__ __attribute__((aligned(16))) char smem[kRowsLds];
    const int BH = a.B * a.H;
    rows_body<kCausal, false>(a, c, blockIdx.x / BH, blockIdx.x % BH, smem);
}

template <bool kCausal>
__global__ __launch_bounds__(kThreads, 2) void bwd_keys_mfma(BackwardArgs a, float c) {
    __shared__ __attribute__((aligned(16))) char smem[kKeysLds];
    const int BH = a.B * a.H;
    keys_body<kCausal>(a, c, blockIdx.x / BH, blockIdx.x % BH, smem);
}

// With the forward's log-sum-exp: per query row, D = do . o (fp32 sum of the
// bf16 products) and the log-sum-exp in log2 units, as the rows kernel
// leaves them.  Eight lanes per row, 16 bytes of do and o each.
constexpr int kPrepRows = 32;   // rows per 256-thread workgroup
__global__ __launch_bounds__(256) void bwd_prep(BackwardArgs a) {
    // B*h*Lq < 2^31 (the launcher checks), so rows index in 32 bits.
    const int n = a.B * a.H * a.Lq;
    const int row = blockIdx.x * kPrepRows + (threadIdx.x >> 3);
    const int part = threadIdx.x & 7;
    float d = 0.0f;
    if (row < n) {
        const int bhh = row / a.Lq;
        const int i = row - bhh * a.Lq, b = bhh / a.H, hd = bhh - b * a.H;
        const uint4 g = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.dout) + b * a.sdo[0] +
                                                         hd * a.sdo[1] + (long long)i * a.sdo[2] + part * 8);
        const uint4 o = *reinterpret_cast<const uint4*>(static_cast<const bf16_t*>(a.o) + b * a.so[0] +
                                                         hd * a.so[1] + (long long)i * a.so[2] + part * 8);
        const uint32_t ug[4] = {g.x, g.y, g.z, g.w}, uo[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
            d += __uint_as_float(ug[e] << 16) * __uint_as_float(uo[e] << 16) +
                 __uint_as_float(ug[e] & 0xffff0000u) * __uint_as_float(uo[e] & 0xffff0000u);
    }
    d += __shfl_xor(d, 1);
    d += __shfl_xor(d, 2);
    d += __shfl_xor(d, 4);
    if (row < n && part == 0) reinterpret_cast<float2*>(a.rows)[row] = make_float2(a.lse_in[row] * kLog2e, d);
}

// Both roles in one grid: block index u = blockIdx / (B*h) takes keys block
// u while u < n_kb, then rows block u - n_kb; each kind's blocks go heaviest
// first, so the lightest query blocks fill the end.  (Measured: alternating
// the kinds block by block ran the key side about 15% slower per step.)
template <bool kCausal>
__global__ __launch_bounds__(kThreads, 2) void bwd_fused_mfma(BackwardArgs a, float c, int n_kb) {
    __shared__ __attribute__((aligned(16))) char smem[kFusedLds];
    const int BH = a.B * a.H;
    const int bh = blockIdx.x % BH, u = blockIdx.x / BH;
    if (u < n_kb) keys_body<kCausal>(a, c, u, bh, smem);
    else rows_body<kCausal, true>(a, c, u - n_kb, bh, smem);
}

template <bool kCausal>
hipError_t launch_variant(const BackwardArgs& a, hipStream_t s) {
    const float c = kLog2e / 8.0f;   // log2(e) / sqrt(64)
    const long long BH = (long long)a.B * a.H;
    const int n_qb = (a.Lq + kRowsWg - 1) / kRowsWg, n_kb = (a.Lk + kRowsWg - 1) / kRowsWg;
    if (BH == 0 || a.Lq == 0) return hipSuccess;
    if (a.lse_in) {
        const long long n = BH * a.Lq;
        if (n >= (1ll << 31)) return hipErrorInvalidValue;
        hipLaunchKernelGGL(bwd_prep, dim3((unsigned)((n + kPrepRows - 1) / kPrepRows)), dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_fused_mfma<kCausal>), dim3((unsigned)(BH * (n_qb + n_kb))), dim3(kThreads), 0, s,
                           a, c, n_kb);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((bwd_rows_mfma<kCausal>), dim3((unsigned)(BH * n_qb)), dim3(kThreads), 0, s, a, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_keys_mfma<kCausal>), dim3((unsigned)(BH * n_kb)), dim3(kThreads), 0, s, a, c);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sdpa_backward_bf16(const BackwardArgs& a, hipStream_t s) {
    if (!fits_buffer(a.sq[2], a.Lq) || !fits_buffer(a.sdo[2], a.Lq) || !fits_buffer(a.so[2], a.Lq) ||
        !fits_buffer(a.sk[2], a.Lk) || !fits_buffer(a.sv[2], a.Lk))
        return hipErrorInvalidValue;
    return a.causal ? launch_variant<true>(a, s) : launch_variant<false>(a, s);
}

}  // namespace mha
