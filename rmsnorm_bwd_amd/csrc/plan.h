// plan.h - host-side launch planning shared by the C ABI (validation and the
// workspace query) and the kernel launchers. Pure C++: no HIP calls, so the
// same code runs in the CPU-only test build.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace rmsn {

// How one row is spread over threads. A "row group" of tpr threads (a power of
// two, 16..512) owns one row at a time; thread t of the group owns the vector
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
    bool long_row;  // a row of more than LONG_N elements: the kernels of long_rows.hip
};

inline int pow2_ceil(int64_t v) {
    int p = 1;
    while (p < v) p <<= 1;
    return p;
}

// Build-time tuning knobs (defaults measured on MI355X):
//   RMSN_BWD_MAX_BLOCKS  cap of the backward's persistent grid
//   RMSN_BLOCK_MIN       threads per block when a row spans 2..4 wavefronts
//   RMSN_BLOCK_WAVE      threads per block when a row fits in one wavefront
//   RMSN_TPR_MAX         most threads one row is spread over on the vector path
//   RMSN_K_MIN           fewest 16-byte chunks per thread on the vector path
//   RMSN_DEPTH           most row windows in flight per row group
//   RMSN_RING_VGPRS      registers per thread the window ring may take
//   RMSN_FIN_TILE        columns per tile of the dgamma partials (16, 32 or 64)
#ifndef RMSN_BWD_MAX_BLOCKS
#define RMSN_BWD_MAX_BLOCKS 256
#endif
#ifndef RMSN_BLOCK_MIN
#define RMSN_BLOCK_MIN 512
#endif
#ifndef RMSN_BLOCK_WAVE
#define RMSN_BLOCK_WAVE 256
#endif
#ifndef RMSN_TPR_MAX
#define RMSN_TPR_MAX 512
#endif
#ifndef RMSN_K_MIN
#define RMSN_K_MIN 1
#endif
#ifndef RMSN_DEPTH
#define RMSN_DEPTH 3
#endif
#ifndef RMSN_RING_VGPRS
#define RMSN_RING_VGPRS 144
#endif

// Threads per block for rows of tpr threads. Rows inside one wavefront
// (several per wavefront when tpr < 64) run in 256-thread blocks: larger
// blocks would leave each block too few row windows for its load ring to
// hide latency. Wider rows run in blocks of 512 threads, or of tpr when it
// is larger.
constexpr int block_threads(int tpr) {
    return tpr <= 64 ? RMSN_BLOCK_WAVE : (tpr > RMSN_BLOCK_MIN ? tpr : RMSN_BLOCK_MIN);
}

// Largest supported row length, and the longest row the register-resident
// window ring takes (longer rows: 512 threads a row, 64 elements a thread).
constexpr int64_t MAX_N = 32768;
constexpr int64_t LONG_N = 16384;

// Choose the row plan for N elements of esize bytes. vector_ok says every
// row-tensor pointer and gamma are 16-byte aligned; the vector path also needs
// N to be a multiple of the vector width so that every row start stays aligned.
// Longer rows take more chunks per thread rather than more threads: a row
// spreads over at most 512 threads, so a thread holds up to 32 elements of a
// 16384-element row, and every block has at most 512 threads (whose waves
// may use 256 VGPRs). Rows of more than LONG_N elements take the long-row
// kernels: 512 threads a row, 64 elements a thread (vector chunks or single
// elements), or, for 16-bit rows on 16-byte chunks of at most LONG6_N
// elements, 48 (six chunks): the backward then does no arithmetic and no
// accumulator traffic for a quarter of the slots that would stay past the
// row end (measured on MI355X against eight chunks, bf16: fused 4096 x 16400
// 128.8 -> 116.2 us, 4096 x 24576 164.4 -> 153.1 us, 8192 x 24576 298.6 ->
// 280.4 us; LayerNorm 4096 x 20000 137.6 -> 128.9 us; plain 4096 x 16400
// 88.6 -> 85.3 us, 4096 x 20000 and 4096 x 24576 unchanged). The forward
// keeps 64 elements a thread. Returns false when N is out of range.
constexpr int64_t LONG6_N = 24576;
inline bool plan_rows(int64_t N, int esize, bool vector_ok, RowPlan *p) {
    if (N < 1 || N > MAX_N) return false;
    const int vw = 16 / esize;
    p->long_row = N > LONG_N;
    if (p->long_row) {
        p->vec = vector_ok && N % vw == 0 ? vw : 1;
        p->k = p->vec == 8 && N <= LONG6_N ? 6 : 64 / p->vec;
        p->tpr = 512;
        p->block = 512;
        p->rpb = 1;
        return true;
    }
    if (vector_ok && N % vw == 0) {
        const int64_t C = N / vw;  // vector chunks per row
        p->vec = vw;
        if (C <= 64) {
            p->tpr = 16;
            p->k = C <= 16 ? 1 : (C <= 32 ? 2 : 4);
        } else {
            // the fewest chunks (a power of two, at least RMSN_K_MIN) that fit
            // the row in RMSN_TPR_MAX threads
            int k = RMSN_K_MIN;
            while ((int64_t)k * RMSN_TPR_MAX < C) k <<= 1;
            p->k = k;
            p->tpr = pow2_ceil((C + k - 1) / k);
        }
    } else {
        p->vec = 1;
        if (N <= 1024) {
            p->tpr = 64;
            p->k = N <= 256 ? 4 : (N <= 512 ? 8 : 16);
        } else if (N <= 4096) {
            p->tpr = 256;
            p->k = N <= 2048 ? 8 : 16;
        } else {
            p->tpr = 512;
            p->k = N <= 8192 ? 16 : 32;
        }
    }
    p->block = block_threads(p->tpr);
    p->rpb = p->block / p->tpr;
    return true;
}

// Upper bound on the backward's persistent grid: the number of per-block
// fp32 dgamma partials the workspace must hold.
constexpr int BWD_MAX_BLOCKS = RMSN_BWD_MAX_BLOCKS;
#ifndef RMSN_FUSED_MAX_BLOCKS
#define RMSN_FUSED_MAX_BLOCKS 192
#endif
#ifndef RMSN_FUSED_CAP_MIN_M
#define RMSN_FUSED_CAP_MIN_M 4096
#endif
static_assert(RMSN_FUSED_MAX_BLOCKS <= RMSN_BWD_MAX_BLOCKS, "the workspace query assumes the larger grid");
constexpr size_t WS_HEADER = 256;

// The dgamma mode a caller asks for (the low two flag bits of the C ABI):
// the measured default, the two-stage fixed-order sum, fp32 atomics, or one
// block writing the gradients itself.
enum : unsigned { DM_AUTO = 0, DM_DETERMINISTIC = 1, DM_ATOMIC = 2, DM_ONE_BLOCK = 3 };

// Blocks the backward launches for M rows: one block per rpb rows at small M,
// capped so each block folds many rows into one dgamma partial. In the
// default mode a problem of short rows (N <= 1024) and at most 8192 elements,
// or of at most two rows of up to 8192 elements, runs in one block that
// writes the gradients itself, saving the finalize launch; DM_ONE_BLOCK asks
// for that at any size, and the two explicit cross-block modes never take it.
// Measured on MI355X (GPU time per call from HIP-graph replay, median of
// three, one block against the two-stage sum at the same shape), bf16:
// 32 x 256 4.8 vs 6.6 us, 8 x 1024 4.8 vs 6.3, 2 x 4096 4.0 vs 5.6,
// 2 x 8192 4.8 vs 6.3 (fp32 2 x 8192 6.4 vs 6.8); but 128 x 256 8.1 vs 6.6,
// 16 x 1024 6.6 vs 6.4, 8 x 4096 7.8 vs 5.7 and 2 x 16384 8.2 vs 7.9, where
// one CU holding the rows is latency-bound (4 x 4096: 5.7 either way). The
// fp32-atomic mode never beats the two-stage sum.
//
// A fused-add backward with a dresidual_out reads three row tensors; from
// 4096 rows on it runs at most 192 blocks (RMSN_FUSED_MAX_BLOCKS,
// RMSN_FUSED_CAP_MIN_M). Measured on MI355X, bf16, against 256 blocks:
// 32768 x 8192 354-359 -> 344.5 us, 32768 x 4096 179.3 -> 171.4 us,
// 8192 x 4096 48.6 -> 46.8 us, 4096 x 4096 27.6 -> 27.0 us; the plain and
// LayerNorm backwards (two row reads) lose with fewer blocks, and so do
// fused calls of fewer rows (1024 x 8192: 18.1 -> 19.4 us).
inline bool one_block_rule(int64_t M, int64_t N) { return (N <= 1024 && M * N <= 8192) || (M <= 2 && N <= 8192); }

inline int64_t bwd_blocks(int64_t M, int64_t N, const RowPlan &p, bool three_reads = false,
                          unsigned dmode = DM_AUTO) {
    if (M <= 0 || dmode == DM_ONE_BLOCK || (dmode == DM_AUTO && one_block_rule(M, N))) return 1;
    int64_t steps = (M + p.rpb - 1) / p.rpb;
    if (steps < 1) steps = 1;
    const int64_t cap = three_reads && M >= RMSN_FUSED_CAP_MIN_M ? RMSN_FUSED_MAX_BLOCKS : BWD_MAX_BLOCKS;
    return steps < cap ? steps : cap;
}

// How the long-row RMSNorm backward on 16-byte chunks (long_rows.hip) runs
// through a block's rows:
//   LM_RELOAD    one row in flight; gamma re-read from the caches for each
//                group of chunks.
//   LM_RESIDENT  gamma held in registers for the whole kernel. Loads and
//                stores retire through one in-order counter, so a gamma load
//                issued after a group's dx stores cannot be waited on without
//                waiting for those stores; with gamma resident nothing is
//                waited on between a row's arrival and its last store.
//   LM_PREFETCH  LM_RESIDENT, and the block's next row (x, dy, rstd) is
//                loaded while the current one is computed; 16-bit types only,
//                where two rows fit the registers beside gamma.
// Measured on MI355X against LM_RELOAD (GPU time per call, rotated buffers,
// 1024-8192 rows of 16400-32768 elements): fused bf16 with dresidual_out
// 2.5-17% faster with LM_PREFETCH (fused f16 4096 x 24576: 18%); plain bf16
// 3.6-18.7% faster up to 24576 elements and at 1024-4096 rows of 28672-32768
// (1.7-8.1%), but slower at 8192 rows of 28672 (+1.8%) and 32768 (+8.2%);
// plain fp32 2.8-7.8% faster with LM_RESIDENT; fused fp32 does not fit
// gamma beside its row.
enum : int { LM_RELOAD = 0, LM_RESIDENT = 1, LM_PREFETCH = 2 };
inline int long_mode(int esize, bool fused, int64_t M, int64_t N) {
    if (esize == 2) return fused || N <= 24576 || M <= 4096 ? LM_PREFETCH : LM_RELOAD;
    return fused ? LM_RELOAD : LM_RESIDENT;
}

// The backward kernel a row of four 16-byte chunks a thread on a 512-thread
// group (1025-2048 chunks) runs on, by variant (`fused`: the fused backward
// with a dresidual_out; the measurements are at dispatch_bwd in
// kernels.hip):
//   BR_THREE_CHUNKS  three chunks a thread, for rows of at most 1536 chunks
//                    of the fused backward and the 16-bit LayerNorm one: two
//                    windows in flight where four chunks leave them one;
//   BR_NEXT_ROW      the long-row kernel that loads a block's next row during
//                    the current one (long_rows.hip), for 16-bit rows of
//                    1537-2048 chunks of the fused backward and of LayerNorm
//                    (full rows of 16384 elements up to 2^26 elements a call);
//   BR_PLAN          the row plan as planned (everything else, the plain
//                    backward always).
// The grid and the workspace do not depend on the route.
enum : int { BR_PLAN = 0, BR_THREE_CHUNKS = 1, BR_NEXT_ROW = 2 };
inline int bwd_route(int esize, bool fused, bool layer, const RowPlan &p, int64_t M, int64_t N) {
    const int vw = 16 / esize;
    if (p.long_row || p.vec != vw || p.tpr != RMSN_TPR_MAX || p.k != 4) return BR_PLAN;
    const bool b16 = esize == 2;
    if (N <= (int64_t)3 * RMSN_TPR_MAX * vw) return fused || (b16 && layer) ? BR_THREE_CHUNKS : BR_PLAN;
    const bool full = N == (int64_t)4 * RMSN_TPR_MAX * vw;
    if (b16 && (fused || (layer && (!full || M * N <= (int64_t(1) << 26))))) return BR_NEXT_ROW;
    return BR_PLAN;
}

// The forward kernel a 16-bit row whose plan leaves chunk slots empty runs
// on:
//   FR_THREE_CHUNKS  three 16-byte chunks a thread on 512 threads for rows of
//                    1025-1536 chunks (8200-12288 elements; the plan has four
//                    a thread): LayerNorm's (two row passes) at every size,
//                    the plain and fused forwards' up to 2^26 elements a call;
//   FR_HALF_ROWS     three chunks a thread on 256-thread groups, two rows a
//                    block, for the plain forward's rows of 513-768 chunks
//                    (4104-6144 elements; the plan has two a thread on 512
//                    threads) from 4096 rows;
//   FR_QUARTER_ROWS  three chunks a thread on 128-thread groups, four rows a
//                    block, for rows of 257-384 chunks (2056-3072 elements;
//                    the plan has one a thread on 512 threads) of every
//                    forward from 3072 rows;
//   FR_WAVE_ROWS     three chunks a thread on one wavefront a row, four rows
//                    a block, for rows of 129-192 chunks (1032-1536
//                    elements; the plan has one a thread on 256 threads) of
//                    the plain and LayerNorm forwards, and of the fused
//                    forward from 2048 rows;
//   FR_NARROW_ROWS   three chunks a thread on 32-thread groups, eight rows a
//                    block, for rows of 65-96 chunks (520-768 elements; the
//                    plan has one a thread on 128 threads) of the LayerNorm
//                    forward at any size, the plain one from 256 rows and
//                    the fused one from 4096 rows;
//   FR_SHORT_ROWS    three chunks a thread on the plan's 16-thread groups
//                    (sixteen rows a block) instead of four, for 16-bit rows
//                    of 33-48 chunks (264-384 elements) of every forward;
//   FR_PLAN          the row plan as planned (everything else).
// The row lengths above are 16-bit elements; the fp32 LayerNorm forward takes
// the wave, quarter and narrow routes too at the same chunk counts (516-768,
// 1028-1536 and 260-384 fp32 elements), with LayerNorm's limits.
// Measured on MI355X, GPU time per call, bf16 unless stated:
//   three chunks: LayerNorm 4096 x 12288 42.8-43.1 -> 39.6-40.0 us, 1024 x
//   12288 14.4-14.5 -> 13.1-13.2, 4096 x 10240 39.4 -> 36.2-36.4, 16384 x
//   12288 142.3-142.7 -> 136.4-136.8, 32768 x 12288 277-278 -> 267-268, f16
//   4096 x 12288 43.5-44.1 -> 39.8-40.2; plain 1024 x 8200 10.5-10.6 ->
//   8.4-8.5, 2048 x 12288 20.3-20.5 -> 18.1-18.3, 4096 x 10240 32.0-32.6 ->
//   30.0-30.2, fused 1024 x 12288 18.7-18.9 -> 17.0-17.2, 2048 x 10240
//   30.5-30.8 -> 28.6-28.7, 4096 x 12288 68.8-69.1 -> 66.3-66.5; but from
//   8192 x 12288 on the plain and fused forwards lose with it (plain 8192 x
//   12288 67.5-68.5 -> 68.1-68.5, 16384 x 12288 133.3-133.6 -> 135.6-137.5;
//   fused 8192 x 12288 135.5-138.5 -> 137.4-140.1, 16384 x 10240
//   224.5-225.5 -> 235.5-238.8). fp32 LayerNorm rows lose too (16384 x 6144
//   137-140 -> 147-150 us, 8192 x 4100 53.4 -> 58.0 us).
//   half rows, plain: 4096 x 5120 16.9-17.0 -> 15.9-16.0 us, 16384 x 5120
//   59.7-59.9 -> 56.6-56.9, 32768 x 5120 118.0-120.4 -> 112.7-114.0, 4096 x
//   6144 19.2-19.4 -> 18.2-18.4, 8192 x 4160 26.4-27.0 -> 25.0-25.1, 16384
//   x 4608 55.0-55.6 -> 51.6-52.3, 4096 x 4104 15.1-15.4 -> 14.5, f16 4096
//   x 5120 16.8-17.1 -> 15.8-16.0, 8192 x 6144 35.6-35.8 -> 34.6-35.2; below
//   4096 rows mixed (3072 x 5120 13.8 -> 12.1 but 2048 x 6144 10.1-10.3 ->
//   10.4-10.7, 1024 x 5120 5.8 -> 6.8-7.0). The fused forward (4096 x 5120
//   30.4-30.9 -> 28.7-29.1 but 16384 x 6144 131.4-132.3 -> 135.0-135.3) and
//   LayerNorm's (4096 x 5120 19.6-19.8 -> 20.4-20.8, 1024 x 6144 7.6 -> 8.9)
//   keep the plan.
//   quarter rows: plain 4096 x 2560 10.7-10.8 -> 9.0-9.1 us, 16384 x 2560
//   34.4-34.5 -> 29.6-29.7, 32768 x 2560 65.5-65.7 -> 56.4-56.5, 16384 x
//   3072 37.0-37.2 -> 34.7-34.9, 3072 x 3072 9.7 -> 7.7-7.8, 8192 x 2056
//   18.5-19.0 -> 14.2-14.3, f16 4096 x 2816 11.2-11.4 -> 9.8-9.9; fused
//   16384 x 2560 64.5-64.8 -> 56.4-56.5, 4096 x 3072 20.6-20.8 -> 17.1-17.2,
//   3072 x 2560 14.2-14.3 -> 13.3-13.4, 8192 x 2304 33.1-33.6 -> 26.7-26.9,
//   16384 x 3072 70.8-71.1 -> 67.2-67.5; LayerNorm 16384 x 2560 43.5-45.0 ->
//   35.5-35.7, 4096 x 3072 13.7-13.8 -> 12.9-13.0, 3072 x 2560 11.2-11.5 ->
//   10.1-10.2, f16 16384 x 3072 48.1-49.6 -> 39.2-39.7. With fewer rows the
//   blocks hold fewer windows: 2048 rows even to slower (fused 2048 x 2560
//   10.0-10.1 -> 10.4-10.5, 2048 x 3072 11.0-11.1 -> 11.4), 1024 rows
//   slower (fused 1024 x 2560 5.7 -> 7.3, LayerNorm 1024 x 3072 5.7-5.9 ->
//   6.3-6.4). The backward on the same groups loses (plain 16384 x 2560
//   44.4-44.7 -> 48.8-49.0 us, 4096 x 2560 15.7-16.0 -> 20.3-20.6).
//   wave rows: plain 4096 x 1536 7.6 -> 6.0 us, 16384 x 1536 21.0-21.1 ->
//   19.3-19.4, 65536 x 1536 74.3-75.3 -> 70.2-70.6, 32768 x 1280 34.3-35.3
//   -> 30.6-30.8, 8192 x 1032 11.3-11.4 -> 8.1-8.2, 1024 x 1536 3.9 -> 3.5,
//   one row of 1536 2.3 -> 2.1, f16 16384 x 1280 19.8-20.1 -> 16.4-16.5;
//   LayerNorm 4096 x 1280 9.0-9.4 -> 5.6-5.7, 16384 x 1536 25.2-25.3 ->
//   19.8-20.1, 65536 x 1536 86.5-89.4 -> 72.2-72.3, 1024 x 1536 4.3-4.4 ->
//   3.8, 128 x 1536 3.2 -> 3.1; fused 4096 x 1280 10.1-10.3 -> 8.7-8.8,
//   2048 x 1536 5.9-6.0 -> 5.7-5.8, 65536 x 1280 117.7-118.0 -> 115.8-116.7,
//   but 512 x 1536 3.54-3.57 -> 3.72-3.75 and 128 x 1280 3.21-3.23 ->
//   3.29-3.32.
//   narrow rows: LayerNorm 16384 x 768 14.6-14.7 -> 10.7-10.8 us, 65536 x
//   768 47.1-47.4 -> 36.7-36.8, 4096 x 640 5.6 -> 4.3, 1024 x 768 3.5 ->
//   3.3, one row of 768 2.7 -> 2.4; plain 16384 x 768 11.8-12.0 ->
//   9.9-10.0, 65536 x 768 38.0-38.4 -> 35.5-35.7, 4096 x 768 4.8 -> 4.1,
//   2048 x 520 3.8-3.9 -> 3.3, f16 16384 x 768 11.9 -> 9.8-10.0, but 128 x
//   768 2.7-2.8 -> 2.8-2.9; fused 16384 x 768 20.2-20.5 -> 19.0-19.1, 65536
//   x 640 63.2-63.3 -> 58.1-58.2, 8192 x 768 10.6-10.8 -> 9.2-9.3, 4096 x
//   768 5.9-6.0 -> 5.7-5.8, but 3072 x 640 4.7-4.8 -> 5.0, 2048 x 768
//   4.2-4.3 -> 4.6.
//   fp32 LayerNorm: 4096 x 768 8.3-8.4 -> 6.7-7.0 us, 16384 x 768 23.1-23.3
//   -> 19.7-19.8, 65536 x 768 80.9-82.0 -> 73.0-73.4, 128 x 768 2.9-3.1 ->
//   2.7-2.9, one row of 640 2.5 -> 2.3 (wave rows); 16384 x 1536 42.7-43.0
//   -> 37.2-37.3, 8192 x 1028 22.4-22.7 -> 17.4-17.5, 3072 x 1536 10.4-10.5
//   -> 8.5 (quarter rows); 16384 x 384 13.1 -> 11.0, 1024 x 384 3.4 -> 3.35
//   (narrow rows). The fp32 plain and fused forwards measured within 3%
//   either way (plain 4096 x 1536 10.8-10.9 -> 11.0-11.2, fused 16384 x
//   1536 67.9-68.2 -> 68.1-68.3) and keep the plan.
//   short rows: plain 16384 x 384 6.2 -> 5.9 us, 65536 x 384 19.0-19.2 ->
//   18.8-19.0, 131072 x 320 30.9-31.1 -> 30.4-30.5, 1024 x 384 3.2 -> 3.0;
//   LayerNorm 16384 x 384 6.2-6.3 -> 5.8, 65536 x 384 20.6-20.7 ->
//   19.5-19.7, 1024 x 384 3.4-3.5 -> 3.2; fused 16384 x 320 8.9-9.0 ->
//   8.5-8.6, 65536 x 384 35.6-35.7 -> 35.7.
enum : int { FR_PLAN = 0, FR_THREE_CHUNKS = 1, FR_HALF_ROWS = 2, FR_QUARTER_ROWS = 3, FR_WAVE_ROWS = 4,
             FR_NARROW_ROWS = 5, FR_SHORT_ROWS = 6 };
inline int fwd_route(int esize, bool fused, bool layer, const RowPlan &p, int64_t M, int64_t N) {
    const int vw = 16 / esize;
    if (p.long_row || p.vec != vw || (esize != 2 && !layer)) return FR_PLAN;
    if (p.tpr == RMSN_TPR_MAX / 2 && p.k == 1 && N > (int64_t)(RMSN_TPR_MAX / 4) * vw &&
        N <= (int64_t)3 * 64 * vw && (!fused || M >= 2048))
        return FR_WAVE_ROWS;
    if (p.tpr == RMSN_TPR_MAX / 4 && p.k == 1 && N > (int64_t)(RMSN_TPR_MAX / 8) * vw &&
        N <= (int64_t)3 * 32 * vw && (layer || M >= (fused ? 4096 : 256)))
        return FR_NARROW_ROWS;
    if (esize == 2 && p.tpr == 16 && p.k == 4 && N <= (int64_t)3 * 16 * vw) return FR_SHORT_ROWS;
    if (p.tpr != RMSN_TPR_MAX) return FR_PLAN;
    if (esize == 2 && p.k == 4 && N <= (int64_t)3 * RMSN_TPR_MAX * vw && (layer || M * N <= (int64_t(1) << 26)))
        return FR_THREE_CHUNKS;
    if (p.k == 2 && N <= (int64_t)3 * (RMSN_TPR_MAX / 2) * vw && !fused && !layer && M >= 4096)
        return FR_HALF_ROWS;
    if (p.k == 1 && N > (int64_t)(RMSN_TPR_MAX / 2) * vw && N <= (int64_t)3 * (RMSN_TPR_MAX / 4) * vw && M >= 3072)
        return FR_QUARTER_ROWS;
    return FR_PLAN;
}

// Blocks for the forward: at most 512, each walking rows with a stride of
// the grid, so any M is covered and a block holds several windows in its
// ring. Measured on MI355X against the earlier cap of 2048 (one or two rows
// a block): fused-add 1024 x 8192 bf16 15.5 -> 12.4 us, 32768 x 8192
// 415 -> 373 us, LayerNorm 4096 x 4096 16.1 -> 14.9 us, the plain forward
// unchanged; 384 and 768 lose where rows do not split evenly. The fused-add
// forward (two row reads, two row writes) on the window ring runs at most
// 256 from 1024 row windows and 2^23 elements on: bf16 1024 x 8192
// 12.2-12.3 -> 11.8-11.9 us, 4096 x 4096 25.0-25.2 -> 24.0-24.3 us,
// 16384 x 1024 25.3-25.5 -> 24.4-24.5 us, 16384 x 2048 49.0-49.5 ->
// 45.5-45.9 us, 32768 x 8192 368-376 -> 363-375 us. Smaller calls are
// faster with more blocks (4096 x 1024 7.4-7.6 against 7.9 us with 256,
// 512 x 4096 4.8 against 5.2 us), and the plain forward loses with 256
// (4096 x 4096 13.9 -> 15.6 us), LayerNorm more (15.0 -> 19.2 us).
inline int64_t fwd_blocks(int64_t M, int64_t N, const RowPlan &p, bool fused) {
    int64_t steps = (M + p.rpb - 1) / p.rpb;
    const bool narrow = fused && !p.long_row && steps >= 1024 && M * N >= (int64_t(1) << 23);
    const int64_t cap = narrow ? 256 : 512;
    if (steps < 1) steps = 1;
    return steps < cap ? steps : cap;
}

// dgamma combining modes actually run.
enum : int { DG_DIRECT = 0, DG_PARTIAL = 1, DG_ATOMIC = 2 };

// What a call in mode dmode runs on `grid` blocks: one block writes dgamma
// itself in the default and one-block modes; otherwise the requested
// cross-block sum, the default resolving to the deterministic two-stage sum.
inline int resolve_mode(unsigned dmode, int64_t grid) {
    if (dmode == DM_ONE_BLOCK || (dmode == DM_AUTO && grid <= 1)) return DG_DIRECT;
    if (dmode == DM_ATOMIC) return DG_ATOMIC;
    return DG_PARTIAL;
}

// Block partials of dgamma are stored in tiles of FIN_TILE columns: tile t
// holds, for every block g, the block's partials of columns
// [FIN_TILE t, FIN_TILE (t + 1)) contiguously, so one tile is a [G][FIN_TILE]
// array and the finalize reads it in one contiguous run.
#ifndef RMSN_FIN_TILE
#define RMSN_FIN_TILE 16
#endif
constexpr int FIN_TILE = RMSN_FIN_TILE;
static_assert(FIN_TILE == 16 || FIN_TILE == 32 || FIN_TILE == 64, "partial tile of 16, 32 or 64 columns");

constexpr int64_t partial_index(int64_t col, int64_t block, int64_t G) {
    return (col / FIN_TILE) * G * FIN_TILE + block * FIN_TILE + col % FIN_TILE;
}

// Bytes of workspace for a backward call in mode dmode: a header, then the
// tiled fp32 block partials, one array per weight gradient (narrays: 1 for
// RMSNorm's dgamma, 2 for LayerNorm's dgamma and dbeta), when they are
// combined by the fixed-order kernel. Sized for the larger (two-read) grid.
inline size_t bwd_workspace(int64_t M, int64_t N, const RowPlan &p, unsigned dmode, int narrays = 1) {
    size_t ws = WS_HEADER;
    const int64_t G = bwd_blocks(M, N, p, false, dmode);
    if (resolve_mode(dmode, G) == DG_PARTIAL) {
        const int64_t tiles = (N + FIN_TILE - 1) / FIN_TILE;
        ws += (size_t)narrays * (size_t)G * (size_t)(tiles * FIN_TILE) * sizeof(float);
    }
    return ws;
}

}  // namespace rmsn
