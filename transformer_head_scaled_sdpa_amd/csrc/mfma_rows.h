// Tile layout shared by the bf16 MFMA kernels that own 64 rows per
// workgroup and stream the other side (the attention backward and the
// weights-export kernel), d = 64, gfx950.
//
// A workgroup is MFMA_ROWS_WAVES wave64s (the including file defines it: 4
// or 8): two groups of 32 rows (one row per lane column of the 32x32 MFMA
// tile) times kPhases = waves / 2 phases; a step streams 32 rows per phase,
// so each wave works on its own 32x32 tile.  With 4 waves two workgroups
// share a CU (one wave of each per SIMD), so one workgroup's prologue,
// barriers and epilogue overlap the other's steps; with 8, one workgroup
// fills a CU with twice the rows per step.  Products run on
// v_mfma_f32_32x32x16_bf16: an accumulator packed to bf16 feeds the next MFMA
// as its B operand, and transposed tiles are read from LDS with
// ds_read_b64_tr_b16.  Streamed tiles are stored in 144-byte rows for 16-byte
// fragment reads (conflict-free) and, where a transposed read is needed, in
// 192-byte rows.  Row masks are key limits: keys [0, limit) are allowed.
#pragma once

#include "common.h"

#if !defined(MFMA_ROWS_WAVES) || (MFMA_ROWS_WAVES != 4 && MFMA_ROWS_WAVES != 8)
#error "define MFMA_ROWS_WAVES (4 or 8) before including mfma_rows.h"
#endif

namespace mha {
namespace rows64 {
// The geometry names the inner namespace, so files built with different
// geometries never share a symbol.
#if MFMA_ROWS_WAVES == 4
inline namespace waves4 {
#else
inline namespace waves8 {
#endif

constexpr int kD = 64;
constexpr int kWaves = MFMA_ROWS_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroups = 2;                   // row groups of 32 per workgroup
constexpr int kPhases = kWaves / kGroups;    // streamed tiles per step
constexpr int kRowsWg = 32 * kGroups;
constexpr int kTile = 32;                    // streamed rows per phase
constexpr int kStep = kTile * kPhases;       // streamed rows per step
constexpr int kLdsR = kD + 8;                // 144-byte rows
constexpr int kLdsT = kD + 32;               // 192-byte rows
constexpr int kTileRB = kTile * kLdsR * 2;   // bytes
constexpr int kTileTB = kTile * kLdsT * 2;
constexpr int kChunks = kStep * 8 / kThreads;  // 16-byte chunks per thread per streamed operand

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 frag(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// A 32-row tile (144-byte rows) times 32 register rows: element v of the
// result is tile row (v/4)*8 + hb*4 + v%4 against register row lane % 32.
__device__ __forceinline__ f32x16 tile_dot(const bf16_t* t, const bf16x8 (&f)[4], int l32, int hb) {
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mfma32x32x16(frag(t + l32 * kLdsR + kk * 16 + hb * 8), f[kk], acc);
    return acc;
}

// The same product added to a given accumulator.
__device__ __forceinline__ f32x16 tile_dot_from(const bf16_t* t, const bf16x8 (&f)[4], const f32x16& init, int l32,
                                                int hb) {
    f32x16 acc = mfma32x32x16(frag(t + l32 * kLdsR + hb * 8), f[0], init);
#pragma unroll
    for (int kk = 1; kk < 4; ++kk) acc = mfma32x32x16(frag(t + l32 * kLdsR + kk * 16 + hb * 8), f[kk], acc);
    return acc;
}

// Transposed fragment of a row-major [32 rows][64 features] LDS tile (192 B
// rows): the A operand [32 features x 16 rows] for features tb*32 + lane%32
// and the tile rows of slice kb in the order the packed B operands use
// (kb*16 + hb*4 + 0..3, then + 8..11).
__device__ __forceinline__ bf16x8 tr_frag(const bf16_t* ts, int kb, int tb, int hb, int lane) {
    const int g = lane >> 4, r = lane & 15;
    const int row = kb * 16 + hb * 4 + (r >> 2);
    const int col = tb * 32 + (g & 1) * 16 + (r & 3) * 4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(ts + row * kLdsT + col));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(ts + (row + 8) * kLdsT + col));
    const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, both);
}

// Pack a 32-row accumulator (element v: row (v/4)*8 + hb*4 + v%4) as two B
// operands: slice kb holds rows kb*16 + {hb*4 + 0..3, hb*4 + 8..11}.
__device__ __forceinline__ void pack_b(const f32x16& x, u32x4 (&w)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const bf16x2 pp = {static_cast<__bf16>(x[kb * 8 + e]), static_cast<__bf16>(x[kb * 8 + e + 1])};
            w[kb][e >> 1] = __builtin_bit_cast(uint32_t, pp);
        }
}

// Row offset of accumulator element v within its 32-row tile, less hb*4.
__device__ __forceinline__ constexpr int acc_row(int v) { return (v >> 2) * 8 + (v & 3); }

// One step of a [L, 64] bf16 operand: rows r0 .. r0+127 as 1024 chunks of 16
// bytes (chunk n: row n / 8, features (n % 8) * 8 ..), kChunks per thread.
// Each step reads through a buffer resource based at row r0 whose range ends
// with row L - 1, so rows at or past L read as zero in hardware (the range
// check covers the per-lane offset only, which is why the step's row offset
// goes into the resource's base and range rather than into soffset).  Each
// thread's chunk offsets within a step are fixed; the per-step resource is
// scalar arithmetic.
struct Chunks {
    uint4 c[kChunks];
};
struct StepSrc {
    const char* base;         // row 0 of the operand
    uint32_t range;           // bytes from row 0 to the end of row L - 1
    uint32_t voff[kChunks];   // byte offsets of this thread's chunks within a step
    uint32_t row_bytes;       // row stride in bytes
};
// Raw buffer (stride 0, range in bytes) with 32-bit data format: the gfx9
// descriptor word 3.
constexpr int kBufWord3 = 0x00020000;
// Whether an [L, 64] view with row stride ld fits one buffer range (32-bit
// byte offsets); launchers refuse views that do not.
// The per-lane offsets of a step (up to kStep rows) must not wrap either.
inline bool fits_buffer(long long ld, int L) {
    return ld * 2 * kStep < (1ll << 31) && (L <= 0 || (long long)(L - 1) * ld * 2 + kD * 2 < (1ll << 31));
}

__device__ __forceinline__ StepSrc step_src(const bf16_t* x, long long ld, int L, int tid) {
    StepSrc s;
    s.base = reinterpret_cast<const char*>(x);
    s.row_bytes = (uint32_t)(ld * 2);
    s.range = L > 0 ? (uint32_t)((long long)(L - 1) * ld * 2 + kD * 2) : 0u;
#pragma unroll
    for (int n = 0; n < kChunks; ++n) {
        const int ch = tid + n * kThreads;
        s.voff[n] = (uint32_t)(ch >> 3) * s.row_bytes + (uint32_t)(ch & 7) * 16u;
    }
    return s;
}
__device__ __forceinline__ Chunks load_step(const StepSrc& s, int r0) {
    Chunks t;
    // A step wholly past row L - 1 gets an empty range (every load reads zero).
    const unsigned long long skip = (unsigned long long)(uint32_t)r0 * s.row_bytes;
    const bool any = skip < s.range;
    const uint32_t left = any ? s.range - (uint32_t)skip : 0u;   // bytes of rows r0 .. L-1
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(s.base + (any ? skip : 0ull)), (short)0, (int)left, kBufWord3);
#pragma unroll
    for (int n = 0; n < kChunks; ++n) {
        typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
        const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, s.voff[n], 0, 0);
        t.c[n] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    return t;
}
// Store a step into the per-phase tiles: row r goes to phase r / 32, in
// 144-byte rows at byte offset offR of the phase area (if offR >= 0) and in
// 192-byte rows at offT (if offT >= 0).
// The 64 rows r0 .. r0+63 as 512 chunks (chunk c: row c / 8, features
// (c % 8) * 8 ..), kStageChunks per thread (chunk tid + n * kThreads), zero
// past row L - 1: the first chunks of a step.
constexpr int kStageChunks = kRowsWg * 8 / kThreads;
struct StageChunks {
    uint4 c[kStageChunks];
};
__device__ __forceinline__ StageChunks load_chunks(const StepSrc& s, int r0) {
    const unsigned long long skip = (unsigned long long)(uint32_t)r0 * s.row_bytes;
    const bool any = skip < s.range;
    const uint32_t left = any ? s.range - (uint32_t)skip : 0u;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(s.base + (any ? skip : 0ull)), (short)0, (int)left, kBufWord3);
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    StageChunks t;
#pragma unroll
    for (int n = 0; n < kStageChunks; ++n) {
        const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, s.voff[n], 0, 0);
        t.c[n] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    return t;
}
// 64-row staging tiles of 144-byte rows in LDS: store the chunks of tile t,
// read the fragment of row r, features kk*16 + hb*8 .. +7.
constexpr int kStageB = kRowsWg * kLdsR * 2;
__device__ __forceinline__ void stage_chunks(char* smem, int t, const StageChunks& c, int tid) {
#pragma unroll
    for (int n = 0; n < kStageChunks; ++n) {
        const int ch = tid + n * kThreads;
        *reinterpret_cast<uint4*>(smem + t * kStageB + (ch >> 3) * (kLdsR * 2) + (ch & 7) * 16) = c.c[n];
    }
}
__device__ __forceinline__ uint4 staged_frag(const char* smem, int t, int r, int kk, int hb) {
    return *reinterpret_cast<const uint4*>(smem + t * kStageB + r * (kLdsR * 2) + kk * 32 + hb * 16);
}

__device__ __forceinline__ void store_step(const Chunks& t, char* smem, int phase_bytes, int offR, int offT, int tid) {
#pragma unroll
    for (int n = 0; n < kChunks; ++n) {
        const int ch = tid + n * kThreads, r = ch >> 3, col = (ch & 7) * 8;
        char* base = smem + (r >> 5) * phase_bytes;
        const int lr = r & 31;
        if (offR >= 0) *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(base + offR) + lr * kLdsR + col) = t.c[n];
        if (offT >= 0) *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(base + offT) + lr * kLdsT + col) = t.c[n];
    }
}

template <typename Args>
__device__ __forceinline__ int row_len(const Args& a, int b, int i) {
    if (a.vl_rank == 1) return a.valid_lens[b];
    if (a.vl_rank == 2) return a.valid_lens[(long long)b * a.Lq + i];
    return a.Lk;
}

// Keys [0, klim) are allowed for query i; a row with no allowed key (lengths
// given, length <= 0) allows all Lk keys with equal scores (`none`).
template <bool kCausal, typename Args>
__device__ __forceinline__ int limit_from_len(const Args& a, int len, int i, bool& none) {
    none = a.vl_rank != 0 && len <= 0;
    if (none) return a.Lk;
    const int lim = min(len, a.Lk);
    return kCausal ? min(lim, i + 1) : lim;
}
template <bool kCausal, typename Args>
__device__ __forceinline__ int key_limit(const Args& a, int b, int i, bool& none) {
    return limit_from_len<kCausal>(a, row_len(a, b, i), i, none);
}

// Sum the per-phase partials of a 32-row accumulator pair through LDS: the
// waves of phases 1.. write theirs, the phase-0 wave of the group adds them.
// Leaves the result in `acc` of the phase-0 waves.  `red` holds
// kGroups * (kPhases - 1) slots of 8 KiB; the caller brackets the calls with
// barriers.
__device__ __forceinline__ void reduce_write(float* red, const f32x16 (&acc)[2], int grp, int ph, int lane) {
    if (ph == 0) return;
    float* slot = red + (grp * (kPhases - 1) + ph - 1) * 32 * 64;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) slot[(tb * 16 + v) * 64 + lane] = acc[tb][v];
}
__device__ __forceinline__ void reduce_read(const float* red, f32x16 (&acc)[2], int grp, int ph, int lane) {
    if (ph != 0) return;
#pragma unroll
    for (int p = 1; p < kPhases; ++p) {
        const float* slot = red + (grp * (kPhases - 1) + p - 1) * 32 * 64;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[tb][v] += slot[(tb * 16 + v) * 64 + lane];
    }
}

// The same sum spread over all the phase waves, an equal share of the 64
// features each.  part_write: every wave writes its partial times `scale` to
// its own 8 KiB slot (values 4q .. 4q+3 of lane l, q = tb*4 + g4, at float
// (q*64 + l)*4, 16-byte accesses).  After a barrier (the caller's),
// part_sum: wave ph adds its groups q over the kPhases slots of its group.
// The slots take kRedAllB bytes.
constexpr int kRedSlotF = 32 * 64;
constexpr int kRedAllB = kGroups * kPhases * kRedSlotF * 4;
__device__ __forceinline__ void part_write(float* red, const f32x16 (&acc)[2], float scale, int grp, int ph,
                                           int lane) {
    float* slot = red + (grp * kPhases + ph) * kRedSlotF;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
            *reinterpret_cast<float4*>(slot + ((tb * 4 + g4) * 64 + lane) * 4) =
                make_float4(acc[tb][g4 * 4] * scale, acc[tb][g4 * 4 + 1] * scale, acc[tb][g4 * 4 + 2] * scale,
                            acc[tb][g4 * 4 + 3] * scale);
}
// Wave ph sums and stores kPartQ of the 8 groups q = tb*4 + g4 of four
// features (features tb*32 + g4*8 + hb*4 .. +3): q = ph * kPartQ + n.
constexpr int kPartQ = 8 / kPhases;
__device__ __forceinline__ void part_sum(const float* red, float4 (&r)[kPartQ], int grp, int ph, int lane) {
#pragma unroll
    for (int n = 0; n < kPartQ; ++n) {
        const int q = ph * kPartQ + n;
        float4 t = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
        for (int p = 0; p < kPhases; ++p) {
            const float4 x = *reinterpret_cast<const float4*>(red + (grp * kPhases + p) * kRedSlotF + (q * 64 + lane) * 4);
            t.x += x.x;
            t.y += x.y;
            t.z += x.z;
            t.w += x.w;
        }
        r[n] = t;
    }
}
__device__ __forceinline__ void store_part(void* base, long long off, bool out_f32, const float4 (&r)[kPartQ],
                                              float scale, int ph, int hb) {
#pragma unroll
    for (int n = 0; n < kPartQ; ++n) {
        const int q = ph * kPartQ + n;
        const int t = (q >> 2) * 32 + (q & 3) * 8 + hb * 4;
        const float y0 = r[n].x * scale, y1 = r[n].y * scale, y2 = r[n].z * scale, y3 = r[n].w * scale;
        if (out_f32)
            *reinterpret_cast<float4*>(static_cast<float*>(base) + off + t) = make_float4(y0, y1, y2, y3);
        else
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(base) + off + t) =
                make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
    }
}

// Store a transposed accumulator pair (element v of block tb: feature
// tb*32 + (v/4)*8 + hb*4 + v%4, row = the lane's row) times `scale`.
__device__ __forceinline__ void store_rowT(void* base, long long off, bool out_f32, const f32x16 (&acc)[2], float scale,
                                           int hb) {
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int t = tb * 32 + g4 * 8 + hb * 4;
            const float y0 = acc[tb][g4 * 4] * scale, y1 = acc[tb][g4 * 4 + 1] * scale,
                        y2 = acc[tb][g4 * 4 + 2] * scale, y3 = acc[tb][g4 * 4 + 3] * scale;
            if (out_f32)
                *reinterpret_cast<float4*>(static_cast<float*>(base) + off + t) = make_float4(y0, y1, y2, y3);
            else
                *reinterpret_cast<uint2*>(static_cast<bf16_t*>(base) + off + t) =
                    make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
        }
}


}  // inline namespace
}  // namespace rows64
}  // namespace mha
