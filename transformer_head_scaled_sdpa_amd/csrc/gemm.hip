// Projection GEMMs of multi-head attention: C = A W^T + bias, with W stored
// [out, in] as a torch linear layer stores it ("Transformer" study notes,
// multi-head attention class: four d_model x d_model linear layers).  The
// per-head split and merge need no kernel: [B*L, h*d_k] row-major already is
// [B, L, h, d_k], which the attention kernel addresses through strides.
//
// Up to three problems sharing N and K run in one launch; the fused Q/K/V
// projection of self-attention is three problems over the same A.
//
// bf16 kernel: 128 x 128 output tile per workgroup, K in steps of 64, four
// wave64s in a 2 x 2 grid each owning 64 x 64 = 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16 with fp32 accumulators.  Both operands are
// K-contiguous in memory, so they are copied to LDS with 16-byte coalesced
// loads and read back as 16-byte MFMA fragments; the next K step is fetched
// into registers while the current one is multiplied.
#include "common.h"
#include "kernels.h"

namespace mha {

namespace {

constexpr int kTM = 128, kTN = 128, kTK = 64;
constexpr int kLds = kTK + 8;     // bf16 per LDS row (144 B)

struct TileMap {
    int prob, tm, tn;
};

__device__ __forceinline__ TileMap map_tile(const GemmArgs& g, int id, int tiles_n) {
    TileMap t{0, 0, 0};
#pragma unroll
    for (int p = 0; p < 3; ++p) {
        if (p >= g.nprob) break;
        const int tiles = ((g.p[p].M + kTM - 1) / kTM) * tiles_n;
        if (id < tiles) {
            t.prob = p;
            t.tm = id / tiles_n;
            t.tn = id % tiles_n;
            return t;
        }
        id -= tiles;
    }
    t.prob = -1;
    return t;
}

template <bool kOutF32>
__global__ __launch_bounds__(256) void gemm_bf16_nt(GemmArgs g, int tiles_n) {
    __shared__ __attribute__((aligned(16))) bf16_t as[kTM * kLds];
    __shared__ __attribute__((aligned(16))) bf16_t ws[kTN * kLds];

    const TileMap tmap = map_tile(g, blockIdx.x, tiles_n);
    if (tmap.prob < 0) return;
    const GemmProblem& P = g.p[tmap.prob];
    const int M = P.M, N = g.N, K = g.K;
    const int m0 = tmap.tm * kTM, n0 = tmap.tn * kTN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hb = lane >> 5, l32 = lane & 31;
    const int wm = wave >> 1, wn = wave & 1;

    const bf16_t* A = static_cast<const bf16_t*>(P.a);
    const bf16_t* W = static_cast<const bf16_t*>(P.w);

    // 128 rows x 64 columns = 1024 16-byte chunks per operand: 4 per thread.
    uint4 pa[4], pw[4];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int c = tid + n * 256;
            const int r = c >> 3, col = (c & 7) * 8;
            pa[n] = (m0 + r < M) ? *reinterpret_cast<const uint4*>(A + (long long)(m0 + r) * K + k0 + col)
                                 : make_uint4(0, 0, 0, 0);
            pw[n] = (n0 + r < N) ? *reinterpret_cast<const uint4*>(W + (long long)(n0 + r) * K + k0 + col)
                                 : make_uint4(0, 0, 0, 0);
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int c = tid + n * 256;
            const int r = c >> 3, col = (c & 7) * 8;
            *reinterpret_cast<uint4*>(as + r * kLds + col) = pa[n];
            *reinterpret_cast<uint4*>(ws + r * kLds + col) = pw[n];
        }
    };

    f32x16 acc[2][2] = {};
    fetch(0);
    for (int k0 = 0; k0 < K; k0 += kTK) {
        __syncthreads();
        stash();
        __syncthreads();
        if (k0 + kTK < K) fetch(k0 + kTK);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 fa[2], fw[2];
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                fa[x] = *reinterpret_cast<const bf16x8*>(as + (wm * 64 + x * 32 + l32) * kLds + kk * 16 + hb * 8);
                fw[x] = *reinterpret_cast<const bf16x8*>(ws + (wn * 64 + x * 32 + l32) * kLds + kk * 16 + hb * 8);
            }
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < 2; ++ni) acc[mi][ni] = mfma32x32x16(fa[mi], fw[ni], acc[mi][ni]);
        }
    }

    // Epilogue: element v of block (mi, ni) is row (v/4)*8 + hb*4 + v%4, column l32.
    const bf16_t* bias = static_cast<const bf16_t*>(P.bias);
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int n = n0 + wn * 64 + ni * 32 + l32;
        if (n >= N) continue;
        const float bn = bias ? bf16_to_f32(bias[n]) : 0.0f;
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + wm * 64 + mi * 32 + (v >> 2) * 8 + hb * 4 + (v & 3);
                if (m >= M) continue;
                const float x = acc[mi][ni][v] + bn;
                if (kOutF32) {
                    static_cast<float*>(P.c)[(long long)m * N + n] = x;
                } else {
                    const __bf16 hi = static_cast<__bf16>(x);
                    static_cast<bf16_t*>(P.c)[(long long)m * N + n] = __builtin_bit_cast(bf16_t, hi);
                    if (P.c_lo) {
                        // x - hi is exact in fp32; its bf16 rounding keeps 8 more bits.
                        const __bf16 lo = static_cast<__bf16>(x - static_cast<float>(hi));
                        static_cast<bf16_t*>(P.c_lo)[(long long)m * N + n] = __builtin_bit_cast(bf16_t, lo);
                    }
                }
            }
        }
    }
}

// fp32: 64 x 64 tile, K in steps of 16, each of 256 threads owns 4 x 4 outputs.
constexpr int kFT = 64, kFK = 16;

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
    const GemmProblem& P = g.p[prob];
    const int M = P.M, N = g.N, K = g.K;
    const int m0 = tm * kFT, n0 = tn * kFT;
    const float* A = static_cast<const float*>(P.a);
    const float* W = static_cast<const float*>(P.w);

    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;     // outputs rows ty*4.., cols tx*4..
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += kFK) {
        __syncthreads();
        // 64 rows x 16 k per operand = 1024 floats: 4 per thread, stored k-major.
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            const int c = tid + n * 256;
            const int r = c >> 4, kq = c & 15;
            const int k = k0 + kq;
            as[kq][r] = (m0 + r < M && k < K) ? A[(long long)(m0 + r) * K + k] : 0.0f;
            ws[kq][r] = (n0 + r < N && k < K) ? W[(long long)(n0 + r) * K + k] : 0.0f;
        }
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
            C[(long long)m * N + n] = acc[x][y] + (bias ? bias[n] : 0.0f);
        }
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, bool out_f32, hipStream_t s) {
    const int tiles_n = (g.N + kTN - 1) / kTN;
    long long tiles = 0;
    for (int p = 0; p < g.nprob; ++p) tiles += (long long)((g.p[p].M + kTM - 1) / kTM) * tiles_n;
    if (tiles == 0) return hipSuccess;
    if (out_f32) hipLaunchKernelGGL(gemm_bf16_nt<true>, dim3((unsigned)tiles), dim3(256), 0, s, g, tiles_n);
    else hipLaunchKernelGGL(gemm_bf16_nt<false>, dim3((unsigned)tiles), dim3(256), 0, s, g, tiles_n);
    return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
    const int tiles_n = (g.N + kFT - 1) / kFT;
    long long tiles = 0;
    for (int p = 0; p < g.nprob; ++p) tiles += (long long)((g.p[p].M + kFT - 1) / kFT) * tiles_n;
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_f32_nt, dim3((unsigned)tiles), dim3(256), 0, s, g, tiles_n);
    return hipGetLastError();
}

}  // namespace mha
