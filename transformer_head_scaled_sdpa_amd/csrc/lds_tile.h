// Direct-to-LDS copies of bf16 operand tiles (gfx950 global_load_lds_dwordx4).
#pragma once

#include "common.h"

namespace mha {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void global_cvoid;

// An operand tile is kRows rows x 64 bf16 (one 64-wide slice of the
// reduction dimension).  In LDS each row takes 144 bytes, the stride at which
// 16-byte MFMA fragment reads (32 rows x 2 halves per wave) are free of bank
// conflicts.
constexpr int kTileLdsRow = 72;                   // bf16 per LDS row
constexpr int kTileRowBytes = kTileLdsRow * 2;

// global_load_lds_dwordx4 writes lane i's 16 bytes to LDS byte 16*i after the
// wave-uniform base, so one wave instruction fills 1 KB of LDS and the
// per-lane source address decides the layout.  Wave load i (i = wave +
// kWaves*j) fills LDS bytes [1024 i, 1024 i + 1024): lane -> row x / 144,
// 16-byte chunk (x % 144) / 16 of that row.  Chunk 8 is row padding: its
// lanes are switched off, so those LDS bytes keep stale data and must never
// be read; rows at or past `limit` re-read row limit - 1 (their
// products are never stored).  With skip_dead, a wave load whose rows all lie
// at or past `limit` is not issued at all: those LDS rows keep stale data of
// any value, so only callers whose rows never mix with other rows' results
// (each output row depends on its own input row only) may ask for it.
// Per-lane offsets are relative to the tile's first row (held as a 64-bit,
// wave-uniform pointer), so they stay below kRows * ld whatever the size of
// the whole matrix.  kRows must be a multiple of 64.
template <int kRows, int kWaves>
struct LdsTileLoader {
    static constexpr int kLoads = kRows * kTileRowBytes / 1024;
    static constexpr int kPerWave = (kLoads + kWaves - 1) / kWaves;
    static_assert(kRows % 64 == 0, "tile rows must be a multiple of 64");
    const bf16_t* rows = nullptr;   // row r0 of the matrix
    uint32_t off[kPerWave];   // element offsets from row r0, before the slice offset
    uint32_t live = 0;        // bit j: wave load j has a row below the limit (wave-uniform)
    uint32_t pad = 0;         // bit j: this lane's chunk of wave load j is row padding

    // Rows r0 .. r0 + kRows - 1 of the row-major matrix `m` with `ld`
    // elements per row.
    __device__ __forceinline__ void init(int wave, int lane, const bf16_t* m, int r0, int limit, int ld,
                                         bool skip_dead = false) {
        rows = m + (long long)r0 * ld;
        live = 0;
        pad = 0;
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            const int x = (wave + kWaves * j) * 1024 + lane * 16;
            const int r = x / kTileRowBytes;
            int c = (x % kTileRowBytes) / 16;
            if (c == 8) {
                c = 0;
                pad |= 1u << j;
            }
            // A tile that starts at or past the limit has no row to read.
            const int rr = min(r0 + r, limit - 1) - r0;
            off[j] = rr >= 0 ? (uint32_t)(rr * ld + c * 8) : 0u;
            const int first = (wave + kWaves * j) * 1024 / kTileRowBytes;   // first row of the load
            if (r0 < limit && (!skip_dead || r0 + first < limit)) live |= 1u << j;
        }
    }

    // Copy the 64-wide slice starting at element column d0.
    __device__ __forceinline__ void issue(int d0, unsigned char* lds, int wave) const {
        const bf16_t* src = rows + d0;
#pragma unroll
        for (int j = 0; j < kPerWave; ++j) {
            const int i = wave + kWaves * j;
            if (i < kLoads && (live >> j & 1u) && !(pad >> j & 1u))
                __builtin_amdgcn_global_load_lds((global_cvoid*)(src + off[j]), (lds_void*)(lds + i * 1024), 16, 0, 0);
        }
    }
};

}  // namespace mha
