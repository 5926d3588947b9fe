// plan.h - host-side launch planning shared by the C ABI (validation and the
// workspace query) and the kernel launchers. Pure C++: no HIP calls, so the
// same code runs in the CPU-only test build.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace rmsn {

// How one row is spread over threads. A "row group" of tpr threads (a power of
// two, 16..1024) owns one row at a time; thread t of the group owns the vector
// chunks t, t + tpr, ..., t + (k - 1) * tpr, each vec elements wide. A block of
// `block` threads holds rpb = block / tpr row groups. Rows of up to 64 threads
// live inside one wavefront (several short rows per wavefront when tpr < 64);
// longer rows span tpr / 64 wavefronts and combine through LDS.
struct RowPlan {
    int vec;    // elements per load: 16 bytes' worth on the vector path, 1 on the element path
    int tpr;    // threads per row
    int k;      // chunks per thread
    int block;  // threads per block
    int rpb;    // rows per block per step
};

inline int pow2_ceil(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Build-time tuning knobs (defaults measured on MI355X):
//   RMSN_BWD_MAX_BLOCKS  cap of the backward's persistent grid
//   RMSN_BLOCK_MIN       threads per block when a row needs fewer
//   RMSN_K_TARGET        16-byte chunks per thread on the vector path
//   RMSN_DEPTH           row windows in flight per row group (blocks <= 512)
#ifndef RMSN_BWD_MAX_BLOCKS
#define RMSN_BWD_MAX_BLOCKS 256
#endif
#ifndef RMSN_BLOCK_MIN
#define RMSN_BLOCK_MIN 256
#endif
#ifndef RMSN_K_TARGET
#define RMSN_K_TARGET 4
#endif
#ifndef RMSN_DEPTH
#define RMSN_DEPTH 3
#endif

// Largest supported row length.
constexpr int64_t MAX_N = 16384;

// Choose the row plan for N elements of esize bytes. vector_ok says every
// row-tensor pointer and gamma are 16-byte aligned; the vector path also needs
// N to be a multiple of the vector width so that every row start stays aligned.
// A thread holds at most 32 elements of a row (16 in 1024-thread blocks,
// whose waves get at most 128 VGPRs). Returns false when N is out of range.
inline bool plan_rows(int64_t N, int esize, bool vector_ok, RowPlan *p) {
    if (N < 1 || N > MAX_N) return false;
    const int vw = 16 / esize;
    if (vector_ok && N % vw == 0) {
        const int64_t C = N / vw;  // vector chunks per row
        p->vec = vw;
        if (C <= 64) {
            p->tpr = 16;
            p->k = C <= 16 ? 1 : (C <= 32 ? 2 : 4);
        } else {
            p->k = RMSN_K_TARGET;
            p->tpr = pow2_ceil((C + p->k - 1) / p->k);
            if (p->tpr > 1024) {  // long fp32 rows: 4 chunks of 1024 threads (16 elements)
                p->tpr = 1024;
                p->k = 4;
            }
        }
    } else {
        p->vec = 1;
        if (N <= 1024) {
            p->tpr = 64;
            p->k = N <= 256 ? 4 : (N <= 512 ? 8 : 16);
        } else if (N <= 4096) {
            p->tpr = 256;
            p->k = 16;
        } else {
            p->tpr = 1024;
            p->k = 16;
        }
    }
    p->block = p->tpr > RMSN_BLOCK_MIN ? p->tpr : RMSN_BLOCK_MIN;
    p->rpb = p->block / p->tpr;
    return true;
}

// Upper bound on the backward's persistent grid: the number of per-block
// fp32 dgamma partials the workspace must hold.
constexpr int BWD_MAX_BLOCKS = RMSN_BWD_MAX_BLOCKS;
constexpr size_t WS_HEADER = 256;

// Blocks the backward launches for M rows: one block per rpb rows at small M,
// capped so each block folds many rows into one dgamma partial.
inline int64_t bwd_blocks(int64_t M, const RowPlan &p) {
    int64_t steps = (M + p.rpb - 1) / p.rpb;
    if (steps < 1) steps = 1;
    return steps < BWD_MAX_BLOCKS ? steps : BWD_MAX_BLOCKS;
}

// dgamma combining modes actually run.
enum : int { DG_DIRECT = 0, DG_PARTIAL = 1, DG_ATOMIC = 2 };

// Block partials of dgamma are stored in tiles of FIN_TILE columns: tile t
// holds, for every block g, the block's partials of columns
// [FIN_TILE t, FIN_TILE (t + 1)) contiguously, so one tile is a [G][FIN_TILE]
// array and the finalize reads it in one contiguous run.
constexpr int FIN_TILE = 16;

constexpr int64_t partial_index(int64_t col, int64_t block, int64_t G) {
    return (col / FIN_TILE) * G * FIN_TILE + block * FIN_TILE + col % FIN_TILE;
}

// Bytes of workspace for a backward call: a header, then the tiled fp32 block
// partials when they are combined by the fixed-order kernel.
inline size_t bwd_workspace(int64_t M, int64_t N, const RowPlan &p, int mode) {
    size_t ws = WS_HEADER;
    if (mode == DG_PARTIAL) {
        const int64_t tiles = (N + FIN_TILE - 1) / FIN_TILE;
        ws += (size_t)bwd_blocks(M, p) * (size_t)(tiles * FIN_TILE) * sizeof(float);
    }
    return ws;
}

}  // namespace rmsn
