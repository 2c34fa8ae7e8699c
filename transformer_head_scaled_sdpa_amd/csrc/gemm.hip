// Projection GEMMs of multi-head attention: C = A W^T + bias, with W stored
// [out, in] as a torch linear layer stores it ("Transformer" study notes,
// multi-head attention class: four d_model x d_model linear layers).  The
// per-head split and merge need no kernel: [B*L, h*d_k] row-major already is
// [B, L, h, d_k], which the attention kernel addresses through strides.
//
// Up to three problems sharing N and K run in one launch; the fused Q/K/V
// projection of self-attention is three problems over the same A.
//
// bf16 kernel: 128 x BN output tile per workgroup (BN = 128, or 64 when
// 128-wide tiles would leave CUs without a tile), eight wave64s in a 4 x 2
// grid each owning 32 x BN/2 through v_mfma_f32_32x32x16_bf16 with fp32
// accumulators; K in steps of 64.
//  * Operand tiles go from global memory straight into LDS
//    (global_load_lds_dwordx4: each wave instruction fills 1 KB of LDS, lane
//    i at byte 16*i, so the per-lane source address decides the layout) in
//    144-byte rows, the stride at which the 16-byte fragment reads are
//    conflict-free; two LDS stages, one barrier per K step, the next step's
//    loads in flight during the current step's MFMAs; two workgroups per CU
//    when the grid has more tiles than CUs, and two waves per SIMD even when
//    it has fewer.
//  * The MFMA computes the transposed block C^T = W A^T, so each lane ends up
//    owning one output row and runs of four consecutive columns; the
//    epilogue stages the fp32 tile in LDS with 16-byte writes and stores
//    whole output rows with 16-byte coalesced stores.
//  * Every wave keeps four independent accumulators (its output blocks
//    times a split of the K steps, summed at the end); with two or more
//    waves per SIMD that re-use distance costs little.
//  * Bias (and, for a residual sublayer, the residual input) is added in the
//    epilogue.
//
// Workgroups are mapped XCD-aware: the hardware deals workgroup ids to the
// eight XCDs round-robin, so consecutive logical tiles (those sharing rows
// of A) are given to ids on the same XCD and share its L2.
#include "common.h"
#include "kernels.h"
#include "lds_tile.h"

namespace mha {

namespace {

constexpr int kTM = 128, kTK = 64;
constexpr int kGemmWaves = 8;                  // waves per workgroup of the bf16 GEMM
constexpr int kLds = kTileLdsRow;              // bf16 per LDS row (144 B)
constexpr int kRowBytes = kTileRowBytes;

struct TileMap {
    int prob, tm, tn;
};

// Logical tile t -> (problem, row tile, column tile).  When every problem
// reads the same A (the self-attention Q/K/V projection), tiles of one row
// block are consecutive across problems; otherwise problems are consecutive.
__device__ __forceinline__ TileMap map_tile(const GemmArgs& g, int t, int tiles_n, bool shared_a) {
    TileMap r{-1, 0, 0};
    if (shared_a) {
        const int per_row = g.nprob * tiles_n;
        r.tm = t / per_row;
        const int rem = t % per_row;
        r.prob = rem / tiles_n;
        r.tn = rem % tiles_n;
        if (r.tm * kTM >= g.p[0].M) r.prob = -1;
        return r;
    }
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        if (p >= g.nprob) break;
        const int tiles = ((g.p[p].M + kTM - 1) / kTM) * tiles_n;
        if (t < tiles) {
            r.prob = p;
            r.tm = t / tiles_n;
            r.tn = t % tiles_n;
            return r;
        }
        t -= tiles;
    }
    return r;
}

// y[e] += x[e] for kW (4 or 8) consecutive bf16 values x.
template <int kW>
__device__ __forceinline__ void add_bf16_row(float* y, const bf16_t* x) {
    uint32_t w[kW / 2];
    if constexpr (kW == 8) {
        const uint4 raw = *reinterpret_cast<const uint4*>(x);
        w[0] = raw.x, w[1] = raw.y, w[2] = raw.z, w[3] = raw.w;
    } else {
        const uint2 raw = *reinterpret_cast<const uint2*>(x);
        w[0] = raw.x, w[1] = raw.y;
    }
#pragma unroll
    for (int e = 0; e < kW / 2; ++e) {
        y[2 * e] += __uint_as_float(w[e] << 16);
        y[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
    }
}

// 8 waves per workgroup in a 4 x 2 grid over the tile: at most ~110 VGPRs,
// so two workgroups (four waves per SIMD) share a CU when the grid has more
// tiles than CUs, and a single workgroup still keeps two waves per SIMD.
template <int kTN, bool kOutF32>
__global__ __launch_bounds__(64 * kGemmWaves, 2) void gemm_bf16_nt(GemmArgs g, int tiles_n, int tiles_total,
                                                                   int per_xcd, int shared_a) {
    constexpr int kWv = kGemmWaves, kThr = 64 * kWv;
    constexpr int kRowsW = kTM / (kWv / 2);        // A rows per wave
    constexpr int kMI = kRowsW / 32;               // 32-row blocks per wave
    constexpr int kABytes = kTM * kRowBytes, kWBytes = kTN * kRowBytes;
    constexpr int kStage = kABytes + kWBytes;
    constexpr int kNB = kTN / 64;                  // 32-wide column blocks per wave (2 or 1)
    constexpr int kSplit = 4 / kNB;                // K-step split of the accumulators
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kStage];

    // XCD-aware order: ids x, x+8, x+16, ... run on XCD x; give them a
    // contiguous range of logical tiles.
    const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (t >= tiles_total) return;
    const TileMap tmap = map_tile(g, t, tiles_n, shared_a != 0);
    if (tmap.prob < 0) return;
    const GemmProblem& P = g.p[tmap.prob];
    const int M = P.M, N = g.N, K = g.K;
    const int m0 = tmap.tm * kTM, n0 = tmap.tn * kTN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hb = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;

    const bf16_t* A = static_cast<const bf16_t*>(P.a);
    const bf16_t* W = static_cast<const bf16_t*>(P.w);
    LdsTileLoader<kTM, kWv> la;
    LdsTileLoader<kTN, kWv> lw;
    la.init(wave, lane, A, m0, M, K);
    lw.init(wave, lane, W, n0, N, K);
    auto issue = [&](int stage, int k0) {
        unsigned char* base = smem + stage * kStage;
        la.issue(k0, base, wave);
        lw.issue(k0, base + kABytes, wave);
    };

    // acc[mi][ni][p]: A rows wm*kRowsW + mi*32 .., W rows wn*kTN/2 + ni*32 .., K split p.
    f32x16 acc[kMI][kNB][kSplit] = {};
    const int nk = K / kTK;
    issue(0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        // This wave's loads of step kt have landed; after the barrier every
        // wave's have, and every wave is done reading the other stage.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (kt + 1 < nk) issue((kt + 1) & 1, (kt + 1) * kTK);
        const bf16_t* as = reinterpret_cast<const bf16_t*>(smem + (kt & 1) * kStage);
        const bf16_t* ws = reinterpret_cast<const bf16_t*>(smem + (kt & 1) * kStage + kABytes);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 fa[kMI], fw[kNB];
#pragma unroll
            for (int x = 0; x < kMI; ++x)
                fa[x] = *reinterpret_cast<const bf16x8*>(as + (wm * kRowsW + x * 32 + l32) * kLds + kk * 16 + hb * 8);
#pragma unroll
            for (int x = 0; x < kNB; ++x)
                fw[x] = *reinterpret_cast<const bf16x8*>(ws + (wn * (kTN / 2) + x * 32 + l32) * kLds + kk * 16 + hb * 8);
            const int p = kk % kSplit;
#pragma unroll
            for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
                for (int ni = 0; ni < kNB; ++ni) acc[mi][ni][p] = mfma32x32x16(fw[ni], fa[mi], acc[mi][ni][p]);
        }
    }

    // Epilogue.  Block (mi, ni) element v is output row wm*kRowsW + mi*32 + l32,
    // column wn*kTN/2 + ni*32 + (v/4)*8 + hb*4 + v%4 of the tile: stage the
    // fp32 tile in LDS four columns at a time, then write whole rows with
    // 16-byte stores.
    constexpr int kPitch = kTN + 4;                // fp32 per staged row
    __syncthreads();
    float* st = reinterpret_cast<float*>(smem);
#pragma unroll
    for (int mi = 0; mi < kMI; ++mi)
#pragma unroll
        for (int ni = 0; ni < kNB; ++ni) {
            f32x16 y = acc[mi][ni][0];
#pragma unroll
            for (int p = 1; p < kSplit; ++p) y += acc[mi][ni][p];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                *reinterpret_cast<float4*>(st + (wm * kRowsW + mi * 32 + l32) * kPitch + wn * (kTN / 2) + ni * 32 +
                                           g4 * 8 + hb * 4) =
                    make_float4(y[g4 * 4], y[g4 * 4 + 1], y[g4 * 4 + 2], y[g4 * 4 + 3]);
        }
    __syncthreads();
    // Each lane stores 16 bytes: 4 fp32 or 8 bf16 columns; consecutive lanes
    // cover a tile row left to right, so a row's output is one contiguous run.
    const bf16_t* bias = static_cast<const bf16_t*>(P.bias);
    const bf16_t* res = static_cast<const bf16_t*>(P.res);   // residual (pre-norm sublayer: x + attention(norm(x)))
    constexpr int kW = kOutF32 ? 4 : 8;            // columns per lane
    constexpr int kChunks = kTN / kW;              // lanes per tile row
#pragma unroll
    for (int j = 0; j < kTM * kChunks / kThr; ++j) {
        const int q = tid + kThr * j;
        const int r = q / kChunks, c = (q % kChunks) * kW;
        const int m = m0 + r, n = n0 + c;
        if (m >= M || n >= N) continue;
        const long long o = (long long)m * N + n;
        float y[kW];
#pragma unroll
        for (int e = 0; e < kW; e += 4) {
            const float4 v4 = *reinterpret_cast<const float4*>(st + r * kPitch + c + e);
            y[e] = v4.x, y[e + 1] = v4.y, y[e + 2] = v4.z, y[e + 3] = v4.w;
        }
        if (bias) add_bf16_row<kW>(y, bias + n);
        if (res) add_bf16_row<kW>(y, res + o);
        if constexpr (kOutF32) {
            *reinterpret_cast<float4*>(static_cast<float*>(P.c) + o) = make_float4(y[0], y[1], y[2], y[3]);
        } else {
            if (P.c_lo) {
                // y * scale as a bf16 pair: hi, then the rounding remainder.
                float lo[kW];
#pragma unroll
                for (int e = 0; e < kW; ++e) {
                    const float x = y[e] * P.scale;
                    y[e] = bf16_to_f32(static_cast<bf16_t>(pack_bf16x2(x, 0.0f) & 0xffffu));
                    lo[e] = x - y[e];
                }
                *reinterpret_cast<uint4*>(static_cast<bf16_t*>(P.c_lo) + o) =
                    make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]), pack_bf16x2(lo[4], lo[5]),
                               pack_bf16x2(lo[6], lo[7]));
            }
            *reinterpret_cast<uint4*>(static_cast<bf16_t*>(P.c) + o) =
                make_uint4(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                           pack_bf16x2(y[6], y[7]));
        }
    }
}

template <int kTN>
hipError_t launch_bf16(const GemmArgs& g, bool out_f32, hipStream_t s, bool shared_a) {
    const int tiles_n = (g.N + kTN - 1) / kTN;
    long long tiles = 0;
    for (int p = 0; p < g.nprob; ++p) tiles += (long long)((g.p[p].M + kTM - 1) / kTM) * tiles_n;
    if (tiles == 0) return hipSuccess;
    const int per_xcd = (int)((tiles + 7) / 8);
    const dim3 grid(8u * per_xcd), block(64 * kGemmWaves);
    if (out_f32)
        hipLaunchKernelGGL((gemm_bf16_nt<kTN, true>), grid, block, 0, s, g, tiles_n, (int)tiles, per_xcd,
                           (int)shared_a);
    else
        hipLaunchKernelGGL((gemm_bf16_nt<kTN, false>), grid, block, 0, s, g, tiles_n, (int)tiles, per_xcd,
                           (int)shared_a);
    return hipGetLastError();
}

// fp32: 64 x 64 tile, each of 256 threads owns 4 x 4 outputs.  K in steps of
// 64: every thread loads four 16-byte pieces of each operand per step, and
// the next step's pieces are loaded while the current step computes (the
// small-M projections of short sequences are latency-bound: few workgroups,
// so each step's load latency is the cost).
constexpr int kFT = 64, kFK = 64;

struct F32Step {
    float4 a[4], w[4];
};

__global__ __launch_bounds__(256) void gemm_f32_nt(GemmArgs g, int tiles_n) {
    __shared__ float as[kFK][kFT + 4];
    __shared__ float ws[kFK][kFT + 4];

    int id = blockIdx.x, prob = -1, tm = 0, tn = 0;
    for (int p = 0; p < g.nprob; ++p) {
        const int tiles = ((g.p[p].M + kFT - 1) / kFT) * tiles_n;
        if (id < tiles) { prob = p; tm = id / tiles_n; tn = id % tiles_n; break; }
        id -= tiles;
    }
    if (prob < 0) return;
    // Constant indices only: a runtime index into the argument array would
    // copy it to scratch memory.
    const GemmProblem P = prob == 0 ? g.p[0] : (prob == 1 ? g.p[1] : g.p[2]);
    const int M = P.M, N = g.N, K = g.K;
    const int m0 = tm * kFT, n0 = tn * kFT;
    const float* A = static_cast<const float*>(P.a);
    const float* W = static_cast<const float*>(P.w);

    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;     // outputs rows ty*4.., cols tx*4..
    // Piece n of a step: row (tid + 256 n) / 16, k (tid % 16) * 4 .. +3 (K is
    // a multiple of 64, so a piece is whole or past K).
    auto load = [&](int k0) {
        F32Step st;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int c = tid + n * 256;
            const int r = c >> 4, k = k0 + (c & 15) * 4;
            st.a[n] = make_float4(0.f, 0.f, 0.f, 0.f);
            st.w[n] = st.a[n];
            if (m0 + r < M && k < K) st.a[n] = *reinterpret_cast<const float4*>(A + (long long)(m0 + r) * K + k);
            if (n0 + r < N && k < K) st.w[n] = *reinterpret_cast<const float4*>(W + (long long)(n0 + r) * K + k);
        }
        return st;
    };
    float acc[4][4] = {};
    F32Step nxt = load(0);
    for (int k0 = 0; k0 < K; k0 += kFK) {
        __syncthreads();
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int c = tid + n * 256;
            const int r = c >> 4, kq = (c & 15) * 4;
            as[kq][r] = nxt.a[n].x; as[kq + 1][r] = nxt.a[n].y; as[kq + 2][r] = nxt.a[n].z; as[kq + 3][r] = nxt.a[n].w;
            ws[kq][r] = nxt.w[n].x; ws[kq + 1][r] = nxt.w[n].y; ws[kq + 2][r] = nxt.w[n].z; ws[kq + 3][r] = nxt.w[n].w;
        }
        if (k0 + kFK < K) nxt = load(k0 + kFK);
        __syncthreads();
#pragma unroll
        for (int kq = 0; kq < kFK; ++kq) {
            float ar[4], wr[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                ar[x] = as[kq][ty * 4 + x];
                wr[x] = ws[kq][tx * 4 + x];
            }
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[x][y] = fmaf(ar[x], wr[y], acc[x][y]);
        }
    }
    const float* bias = static_cast<const float*>(P.bias);
    float* C = static_cast<float*>(P.c);
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int m = m0 + ty * 4 + x;
        if (m >= M) continue;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            const int n = n0 + tx * 4 + y;
            if (n >= N) continue;
            const float r = P.res ? static_cast<const float*>(P.res)[(long long)m * N + n] : 0.0f;
            C[(long long)m * N + n] = acc[x][y] + (bias ? bias[n] : 0.0f) + r;
        }
    }
}

// fp32 with few rows (M <= 64, the projections of short sequences): a tile is
// 8 rows x 64 columns, one column per lane, and the four waves of a
// workgroup split K; the 8 A rows (all of K) sit in LDS and are read as
// broadcasts, each lane streams its own W row.  The four partial sums are
// added through LDS.  Small tiles give more workgroups and short loops (few
// waves run cold here, so instruction fetch matters as much as arithmetic).
constexpr int kSM = 8, kSN = 64, kSW = 4;

__global__ __launch_bounds__(64 * kSW) void gemm_f32_smallm(GemmArgs g, int tiles_n) {
    extern __shared__ float sm[];                       // A tile [kSM][K], then partials [kSW][kSM][kSN]
    int id = blockIdx.x, prob = -1, tm = 0, tn = 0;
    for (int p = 0; p < g.nprob; ++p) {
        const int tiles = ((g.p[p].M + kSM - 1) / kSM) * tiles_n;
        if (id < tiles) { prob = p; tm = id / tiles_n; tn = id % tiles_n; break; }
        id -= tiles;
    }
    if (prob < 0) return;
    // Constant indices only: a runtime index into the argument array would
    // copy it to scratch memory.
    const GemmProblem P = prob == 0 ? g.p[0] : (prob == 1 ? g.p[1] : g.p[2]);
    const int M = P.M, N = g.N, K = g.K;
    const int m0 = tm * kSM, n0 = tn * kSN;
    const float* A = static_cast<const float*>(P.a);
    const float* W = static_cast<const float*>(P.w);
    float* as = sm;
    float* red = sm + kSM * K;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // A rows m0 .. m0+7, all of K (rows past M read as zero), 16 bytes a piece.
    for (int c = tid; c < kSM * K / 4; c += 64 * kSW) {
        const int r = (c * 4) / K, k = (c * 4) % K;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m0 + r < M) x = *reinterpret_cast<const float4*>(A + (long long)(m0 + r) * K + k);
        *reinterpret_cast<float4*>(as + r * K + k) = x;
    }
    __syncthreads();
    const int n = n0 + lane;
    const int kq = K / kSW, k0 = wave * kq;
    const float* wr = W + (long long)min(n, N - 1) * K;   // rows past N compute a discarded copy
    float acc[kSM] = {};
    for (int k = k0; k < k0 + kq; k += 4) {
        const float4 wv = *reinterpret_cast<const float4*>(wr + k);
#pragma unroll
        for (int r = 0; r < kSM; ++r) {
            const float4 av = *reinterpret_cast<const float4*>(as + r * K + k);
            acc[r] = fmaf(av.x, wv.x, acc[r]);
            acc[r] = fmaf(av.y, wv.y, acc[r]);
            acc[r] = fmaf(av.z, wv.z, acc[r]);
            acc[r] = fmaf(av.w, wv.w, acc[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < kSM; ++r) red[(wave * kSM + r) * kSN + lane] = acc[r];
    __syncthreads();
    // Wave w adds the partials of rows 2w and 2w + 1 and stores them.
    const float* bias = static_cast<const float*>(P.bias);
    float* C = static_cast<float*>(P.c);
#pragma unroll
    for (int rr = 0; rr < kSM / kSW; ++rr) {
        const int r = wave * (kSM / kSW) + rr;
        const int m = m0 + r;
        if (m >= M || n >= N) continue;
        float y = 0.0f;
#pragma unroll
        for (int w = 0; w < kSW; ++w) y += red[(w * kSM + r) * kSN + lane];
        const float res = P.res ? static_cast<const float*>(P.res)[(long long)m * N + n] : 0.0f;
        C[(long long)m * N + n] = y + (bias ? bias[n] : 0.0f) + res;
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, bool out_f32, hipStream_t s) {
    // K must be a multiple of the 64-wide K step and N of the 64-wide column
    // block (both hold for d_model = h * 64).
    if (g.K % kTK != 0 || g.N % 64 != 0) return hipErrorInvalidValue;
    bool shared_a = true;
    for (int p = 1; p < g.nprob; ++p) shared_a = shared_a && g.p[p].a == g.p[0].a && g.p[p].M == g.p[0].M;
    // 128-wide column tiles unless that leaves CUs without a tile.
    long long tiles128 = 0;
    for (int p = 0; p < g.nprob; ++p) tiles128 += (long long)((g.p[p].M + kTM - 1) / kTM) * ((g.N + 127) / 128);
    if (g.N % 128 == 0 && tiles128 >= 256) return launch_bf16<128>(g, out_f32, s, shared_a);
    return launch_bf16<64>(g, out_f32, s, shared_a);
}

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
    if (g.K % 4 != 0) return hipErrorInvalidValue;   // 16-byte operand pieces along K
    int max_m = 0;
    for (int p = 0; p < g.nprob; ++p) max_m = max(max_m, g.p[p].M);
    const size_t small_lds = (size_t)(kSM * g.K + kSW * kSM * kSN) * sizeof(float);
    if (max_m <= 64 && g.K % (4 * kSW) == 0 && small_lds <= 64 * 1024) {
        const int tiles_n = (g.N + kSN - 1) / kSN;
        long long tiles = 0;
        for (int p = 0; p < g.nprob; ++p) tiles += (long long)((g.p[p].M + kSM - 1) / kSM) * tiles_n;
        if (tiles == 0) return hipSuccess;
        hipLaunchKernelGGL(gemm_f32_smallm, dim3((unsigned)tiles), dim3(64 * kSW), small_lds, s, g, tiles_n);
        return hipGetLastError();
    }
    const int tiles_n = (g.N + kFT - 1) / kFT;
    long long tiles = 0;
    for (int p = 0; p < g.nprob; ++p) tiles += (long long)((g.p[p].M + kFT - 1) / kFT) * tiles_n;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_f32_nt, dim3((unsigned)tiles), dim3(256), 0, s, g, tiles_n);
    return hipGetLastError();
}

}  // namespace mha
