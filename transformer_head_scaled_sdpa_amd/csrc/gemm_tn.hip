// Weight and bias gradients of linear layers, for the backward pass of the
// multi-head layer: a linear layer y = x W^T + b ("Transformer" study notes,
// multi-head attention class: four d_model x d_model linear layers stored
// [out, in]) has
//   dW = dy^T x   (dW[o, i] = sum_m dy[m, o] x[m, i])  and  db = sum_m dy[m, :]
// over the rows m of a batch.  bf16 operands, fp32 accumulation and output.
//
// The reduction runs over the M rows (B * L, thousands) while the output is
// small (d_model x d_model), so the rows are split into S slices: each
// workgroup forms one 128 x 128 output tile over one slice into an fp32
// partial in the workspace, and a second kernel adds the S partials in a
// fixed order (no atomics: the result does not depend on scheduling).
//
// Partial kernel: 8 wave64s per workgroup in a 4 x 2 grid, each owning 32
// output rows (features of dy) x 64 output columns (features of x) through
// v_mfma_f32_32x32x16_bf16.  Steps of 32 rows: dy and x tiles [32 rows][128
// features] go to LDS (two 64-feature sub-tiles in 192-byte rows, two
// stages, loaded two steps ahead into registers through range-checked buffer
// loads, so rows past M read zeros), and both MFMA operands are transposed
// reads (ds_read_b64_tr_b16): the reduction index m is the tile's row.  The
// bias gradient rides along as one more MFMA against an all-ones operand in
// the workgroups of the first column tile.
#include "common.h"
#include "kernels.h"

#define MFMA_ROWS_WAVES 8
#include "mfma_rows.h"

namespace mha {

namespace {

using rows64::tr_frag;
using rows64::kLdsT;

constexpr int kTnWaves = 8;
constexpr int kTnThreads = 64 * kTnWaves;
constexpr int kTnRows = 32;                        // rows of the reduction per step
constexpr int kTnTile = 128;                       // output tile edge
constexpr int kSubB = kTnRows * kLdsT * 2;         // one [32][64] sub-tile, 192-byte rows
constexpr int kStageTnB = 4 * kSubB;               // dy: 2 sub-tiles, x: 2 sub-tiles
constexpr int kBufTnWord3 = 0x00020000;            // raw buffer, 32-bit data format
constexpr int kTnWgs = 512;                        // workgroups per launch to aim for (two per CU)

// Buffer resource over rows r0 .. M-1 of a row-major [M, cols] bf16 operand
// with row stride ld: the range ends with row M - 1's last column, so rows at
// or past M read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tn_rows(const bf16_t* p, long long ld, int cols, int r0, int M) {
    const long long left = r0 < M ? (long long)(M - 1 - r0) * ld * 2 + (long long)cols * 2 : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p + (r0 < M ? (long long)r0 * ld : 0)), (short)0,
                                             (int)left, kBufTnWord3);
}

__global__ __launch_bounds__(kTnThreads, 1) void gemm_tn_partial(TnArgs g, int blocks, int per_xcd) {
    __shared__ __attribute__((aligned(16))) char smem[2 * kStageTnB];

    // XCD-aware order: the hardware deals workgroup ids to the eight XCDs
    // round-robin, so ids x, x+8, ... (one XCD) take a contiguous range of
    // logical blocks: the tiles of one slice, which read the same rows of
    // both operands, then share that XCD's L2.
    int blk = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3), pi = 0;
    if (blk >= blocks) return;
    // Block -> (problem, row tile, column tile, slice).
    while (pi + 1 < g.nprob && blk >= g.p[pi].blocks) {
        blk -= g.p[pi].blocks;
        ++pi;
    }
    const TnProblem& p = g.p[pi];
    const int t1 = p.tiles1, t2 = p.tiles2;
    const int sl = blk / (t1 * t2), rem = blk % (t1 * t2);
    const int n1_0 = (rem / t2) * kTnTile, n2_0 = (rem % t2) * kTnTile;
    const int m_begin = sl * p.rows_per_slice;
    const int m_end = min(p.M, m_begin + p.rows_per_slice);
    const int n_steps = max(0, (m_end - m_begin + kTnRows - 1) / kTnRows);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wy = wave & 3, wx = wave >> 2;
    const int hb = lane >> 5;

    // This thread's chunk of each [32][128] tile: row tid / 16, features
    // (tid % 16) * 8 .. +7 (sub-tile (tid % 16) / 8).  Chunks at or past
    // the operand's columns are zeroed after the load (the load itself stays
    // inside the rows, which are at least that long).
    const int cr = tid >> 4, cc = (tid & 15) * 8;
    const bool y_in = n1_0 + cc < p.N1, x_in = n2_0 + cc < p.N2;
    const uint32_t y_off = (uint32_t)((long long)cr * p.ldy * 2 + (long long)(n1_0 + cc) * 2);
    const uint32_t x_off = (uint32_t)((long long)cr * p.ldx * 2 + (long long)(n2_0 + cc) * 2);
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    struct Pair {
        uint4 y, x;
    };
    auto load = [&](int st) {
        const int r0 = m_begin + st * kTnRows;
        // Rows of the next slice read as zero too: clip to this slice's end.
        const u32x4v vy = __builtin_amdgcn_raw_buffer_load_b128(tn_rows(p.y, p.ldy, p.N1, r0, m_end), y_off, 0, 0);
        const u32x4v vx = __builtin_amdgcn_raw_buffer_load_b128(tn_rows(p.x, p.ldx, p.N2, r0, m_end), x_off, 0, 0);
        Pair r;
        r.y = y_in ? make_uint4(vy[0], vy[1], vy[2], vy[3]) : make_uint4(0, 0, 0, 0);
        r.x = x_in ? make_uint4(vx[0], vx[1], vx[2], vx[3]) : make_uint4(0, 0, 0, 0);
        return r;
    };
    auto store = [&](const Pair& r, int stage) {
        char* base = smem + stage * kStageTnB;
        const int sub = cc >> 6, col = cc & 63;
        *reinterpret_cast<uint4*>(base + sub * kSubB + (cr * kLdsT + col) * 2) = r.y;
        *reinterpret_cast<uint4*>(base + (2 + sub) * kSubB + (cr * kLdsT + col) * 2) = r.x;
    };

    f32x16 acc[2] = {}, accb = {};
    const bool bias = p.db_part != nullptr && n2_0 == 0 && wx == 0;
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = static_cast<__bf16>(1.0f);

    // Two steps in flight in registers (even and odd), one stage in LDS
    // being read while the other is written.
    Pair ne = load(0), no = load(1);
    auto step = [&](int st, Pair& nr) {
        store(nr, st & 1);
        nr = load(st + 2);
        __syncthreads();
        const char* base = smem + (st & 1) * kStageTnB;
        const bf16_t* ys = reinterpret_cast<const bf16_t*>(base + (wy >> 1) * kSubB);
        const bf16_t* xs = reinterpret_cast<const bf16_t*>(base + (2 + wx) * kSubB);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const bf16x8 a = tr_frag(ys, kb, wy & 1, hb, lane);
#pragma unroll
            for (int t = 0; t < 2; ++t) acc[t] = mfma32x32x16(a, tr_frag(xs, kb, t, hb, lane), acc[t]);
            if (bias) accb = mfma32x32x16(a, ones, accb);
        }
    };
    int st = 0;
    for (; st + 1 < n_steps; st += 2) {
        step(st, ne);
        step(st + 1, no);
    }
    if (st < n_steps) step(st, ne);

    // Partial tile: element v of block t is row n1_0 + wy*32 + (v/4)*8 +
    // hb*4 + v%4, column n2_0 + wx*64 + t*32 + lane%32.
    float* part = p.w_part + (long long)sl * p.N1 * p.N2;
    const int col0 = n2_0 + wx * 64 + (lane & 31);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const int row = n1_0 + wy * 32 + (v >> 2) * 8 + hb * 4 + (v & 3);
        if (row >= p.N1) continue;
#pragma unroll
        for (int t = 0; t < 2; ++t)
            if (col0 + t * 32 < p.N2) part[(long long)row * p.N2 + col0 + t * 32] = acc[t][v];
        if (bias && (lane & 31) == 0) p.db_part[(long long)sl * p.N1 + row] = accb[v];
    }
}

// dW = the sum of the S partials, in slice order; db likewise.
__global__ __launch_bounds__(256) void gemm_tn_reduce(TnArgs g) {
    int blk = blockIdx.x, pi = 0;
    while (pi + 1 < g.nprob && blk >= g.p[pi].reduce_blocks) {
        blk -= g.p[pi].reduce_blocks;
        ++pi;
    }
    const TnProblem& p = g.p[pi];
    const long long n4 = (long long)p.N1 * p.N2 / 4;
    const long long i = (long long)blk * 256 + threadIdx.x;
    if (i < n4) {
        float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        for (int k = 0; k < p.slices; ++k) {
            const float4 x = reinterpret_cast<const float4*>(p.w_part + (long long)k * p.N1 * p.N2)[i];
            s.x += x.x;
            s.y += x.y;
            s.z += x.z;
            s.w += x.w;
        }
        // Row r = 4i / N2 of dW goes to dw (or dw2 for the second half of a
        // stacked pair of layers).
        const long long e = 4 * i, r = e / p.N2, c = e % p.N2;
        float* dst = (p.dw2 && r >= p.N1 / 2) ? p.dw2 + (r - p.N1 / 2) * p.N2 + c : p.dw + r * p.N2 + c;
        *reinterpret_cast<float4*>(dst) = s;
    }
    if (p.db_part && i < p.N1) {
        float s = 0.0f;
        for (int k = 0; k < p.slices; ++k) s += p.db_part[(long long)k * p.N1 + i];
        if (p.db2 && i >= p.N1 / 2) p.db2[i - p.N1 / 2] = s;
        else p.db[i] = s;
    }
}

// dst[q][i][col0 + o] = w[q][o][i] for [n, n] bf16 weights, 64 x 64 tiles
// through LDS so both sides move as whole rows.
__global__ __launch_bounds__(256) void transpose_bf16(TransposeArgs a) {
    __shared__ uint16_t t[64][66];
    const int q = blockIdx.y;
    const int tiles = a.n / 64;
    const int o0 = (blockIdx.x / tiles) * 64, i0 = (blockIdx.x % tiles) * 64;
    const uint16_t* w = a.w[q];
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int r = e >> 6, c = e & 63;
        t[r][c] = w[(long long)(o0 + r) * a.n + i0 + c];
    }
    __syncthreads();
    uint16_t* d = a.dst[q];
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
        const int r = e >> 6, c = e & 63;
        d[(long long)(i0 + r) * a.ld[q] + a.col0[q] + o0 + c] = t[c][r];
    }
}

}  // namespace

hipError_t launch_transpose_bf16(const TransposeArgs& a, hipStream_t s) {
    if (a.n % 64 || a.count < 1 || a.count > 4) return hipErrorInvalidValue;
    const int tiles = (a.n / 64) * (a.n / 64);
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(transpose_bf16, dim3((unsigned)tiles, (unsigned)a.count), dim3(256), 0, s, a);
    return hipGetLastError();
}

size_t gemm_tn_workspace_bytes(const int* M, const int* N1, const int* N2, int nprob) {
    int slices[3];
    gemm_tn_slices(M, N1, N2, nprob, slices);
    size_t bytes = 0;
    for (int q = 0; q < nprob; ++q) {
        bytes += (size_t)slices[q] * ((size_t)N1[q] * N2[q] + N1[q]) * 4;
        bytes = (bytes + 255) / 256 * 256;
    }
    return bytes;
}

void gemm_tn_slices(const int* M, const int* N1, const int* N2, int nprob, int* slices) {
    // The launch's workgroups (about kTnWgs in all) are shared among the
    // problems in proportion to their work; each slice is at least 4 steps
    // long.  Fewer, longer slices mean fewer partials to write and add.
    double work[3], total = 0.0;
    int tiles[3];
    for (int q = 0; q < nprob; ++q) {
        tiles[q] = ((N1[q] + kTnTile - 1) / kTnTile) * ((N2[q] + kTnTile - 1) / kTnTile);
        work[q] = (double)M[q] * tiles[q];
        total += work[q];
    }
    for (int q = 0; q < nprob; ++q) {
        const int want = total > 0.0 ? (int)(kTnWgs * work[q] / total / tiles[q] + 0.5) : 1;
        const int most = max(1, (M[q] + 4 * kTnRows - 1) / (4 * kTnRows));
        slices[q] = max(1, min(want, most));
    }
}

hipError_t launch_gemm_tn(TnArgs g, void* workspace, hipStream_t s) {
    char* ws = static_cast<char*>(workspace);
    long long blocks = 0, rblocks = 0;
    if (g.nprob < 1 || g.nprob > 3) return hipErrorInvalidValue;
    int M[3], N1[3], N2[3], slices[3];
    for (int q = 0; q < g.nprob; ++q) {
        M[q] = g.p[q].M;
        N1[q] = g.p[q].N1;
        N2[q] = g.p[q].N2;
    }
    gemm_tn_slices(M, N1, N2, g.nprob, slices);
    for (int q = 0; q < g.nprob; ++q) {
        TnProblem& p = g.p[q];
        if (p.N1 % 64 || p.N2 % 64 || p.M < 0) return hipErrorInvalidValue;
        // The operands' buffer ranges count bytes in 31 bits.
        if ((long long)p.M * (p.ldy > p.ldx ? p.ldy : p.ldx) * 2 >= (1ll << 31)) return hipErrorInvalidValue;
        p.slices = slices[q];
        p.rows_per_slice = ((p.M + p.slices - 1) / p.slices + kTnRows - 1) / kTnRows * kTnRows;
        p.tiles1 = (p.N1 + kTnTile - 1) / kTnTile;
        p.tiles2 = (p.N2 + kTnTile - 1) / kTnTile;
        p.blocks = p.tiles1 * p.tiles2 * p.slices;
        p.w_part = reinterpret_cast<float*>(ws);
        ws += (size_t)p.slices * p.N1 * p.N2 * 4;
        p.db_part = p.db ? reinterpret_cast<float*>(ws) : nullptr;
        ws += (size_t)p.slices * p.N1 * 4;
        ws = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(ws) + 255) / 256 * 256);
        const long long n = (long long)p.N1 * p.N2 / 4;
        p.reduce_blocks = (int)((max(n, (long long)p.N1) + 255) / 256);
        blocks += p.blocks;
        rblocks += p.reduce_blocks;
    }
    if (blocks == 0) return hipSuccess;
    const int per_xcd = (int)((blocks + 7) / 8);
    hipLaunchKernelGGL(gemm_tn_partial, dim3(8u * per_xcd), dim3(kTnThreads), 0, s, g, (int)blocks, per_xcd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gemm_tn_reduce, dim3((unsigned)rblocks), dim3(256), 0, s, g);
    return hipGetLastError();
}

}  // namespace mha
