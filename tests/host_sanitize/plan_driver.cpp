// Exercises the host-side launch planning (rmsnorm_bwd_amd/csrc/plan.h) over
// every row length the library accepts, both element sizes and both load
// paths, and a range of row counts up to the largest M, checking the
// invariants the kernels rely on. Built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py, so signed
// overflow in the size arithmetic is reported too. Exit status 0 when every
// invariant holds.
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "plan.h"

using namespace rmsn;

static int failures = 0;
#define CHECK(c, ...)                                   \
    do {                                                \
        if (!(c)) {                                     \
            if (failures++ < 20) {                      \
                std::fprintf(stderr, "%s: ", #c);       \
                std::fprintf(stderr, __VA_ARGS__);      \
                std::fprintf(stderr, "\n");             \
            }                                           \
        }                                               \
    } while (0)

static bool pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

int main() {
    RowPlan p;
    CHECK(!plan_rows(0, 2, true, &p), "N = 0 accepted");
    CHECK(!plan_rows(MAX_N + 1, 2, true, &p), "N = MAX_N + 1 accepted");
    const int64_t Ms[] = {0, 1, 2, 15, 16, 17, 255, 256, 257, 4095, 4096, 32768, 1000003, (int64_t(1) << 31) - 1};
    for (int esize : {2, 4}) {
        for (int vok = 0; vok < 2; ++vok) {
            for (int64_t N = 1; N <= MAX_N; ++N) {
                if (!plan_rows(N, esize, vok != 0, &p)) {
                    CHECK(false, "N = %lld refused", (long long)N);
                    continue;
                }
                const bool vec = p.vec != 1;
                CHECK(!vec || (vok && p.vec * esize == 16 && N % p.vec == 0), "vector plan for N = %lld", (long long)N);
                CHECK((int64_t)p.vec * p.k * p.tpr >= N, "plan does not cover N = %lld", (long long)N);
                CHECK(pow2(p.tpr) && p.tpr >= 16 && p.tpr <= 512, "tpr %d", p.tpr);
                // long rows: 64 elements a thread, or six 16-byte chunks of a
                // 16-bit row of at most LONG6_N elements
                const bool six = p.long_row && p.vec == 8 && N <= LONG6_N;
                CHECK(p.long_row ? p.k * p.vec == (six ? 48 : 64) : pow2(p.k) && p.k * p.vec <= 32,
                      "k %d vec %d at N = %lld", p.k, p.vec, (long long)N);
                CHECK(p.long_row == (N > LONG_N), "long-row plan at N = %lld", (long long)N);
                CHECK(!p.long_row || (p.tpr == 512 && p.block == 512 && p.rpb == 1),
                      "long-row plan shape at N = %lld", (long long)N);
                CHECK(p.block <= 512 && p.block % p.tpr == 0 && p.rpb == p.block / p.tpr, "block %d", p.block);
                CHECK(p.block % 64 == 0, "block %d not whole wavefronts", p.block);
                if (N % 97 != 1 && N > 64) continue;  // the row-count sweep on a sample of N
                for (int64_t M : Ms) {
                    const int64_t G = bwd_blocks(M, N, p);
                    CHECK(G >= 1 && G <= BWD_MAX_BLOCKS, "G %lld at M %lld N %lld", (long long)G, (long long)M,
                          (long long)N);
                    if (M > 0 && G > 1)
                        CHECK(G <= (M + p.rpb - 1) / p.rpb, "idle blocks at M %lld", (long long)M);
                    // a three-read (fused) call never runs more blocks than the
                    // workspace query sizes for
                    const int64_t G3 = bwd_blocks(M, N, p, true);
                    CHECK(G3 >= 1 && G3 <= G, "fused grid %lld above %lld", (long long)G3, (long long)G);
                    for (unsigned dm : {DM_AUTO, DM_DETERMINISTIC, DM_ATOMIC, DM_ONE_BLOCK})
                        for (int na : {1, 2}) {
                            const size_t ws = bwd_workspace(M, N, p, dm, na);
                            CHECK(ws >= WS_HEADER, "workspace below its header");
                            const int64_t Gm = bwd_blocks(M, N, p, false, dm);
                            CHECK(dm != DM_ONE_BLOCK || Gm == 1, "one-block mode on %lld blocks", (long long)Gm);
                            CHECK(dm != DM_AUTO || Gm == G, "default grid differs");
                            CHECK(bwd_blocks(M, N, p, true, dm) <= Gm, "fused grid above the sized one");
                            if (resolve_mode(dm, Gm) != DG_PARTIAL) continue;
                            // the last partial of every array lies inside the workspace
                            const int64_t tiles = (N + FIN_TILE - 1) / FIN_TILE;
                            const int64_t pstride = tiles * FIN_TILE * Gm;
                            const int64_t last = (na - 1) * pstride + partial_index(N - 1, Gm - 1, Gm);
                            CHECK((size_t)(last + 1) * sizeof(float) + WS_HEADER <= ws,
                                  "partial index %lld past a workspace of %zu bytes", (long long)last, ws);
                            // the header bound the C header states for the default tile
                            CHECK(ws <= WS_HEADER + (size_t)na * BWD_MAX_BLOCKS * (size_t)(tiles * FIN_TILE) * 4,
                                  "workspace above its bound");
                        }
                }
            }
        }
    }
    // partial_index is a bijection from (column, block) onto [0, tiles * FIN_TILE * G)
    for (int64_t G : {int64_t(1), int64_t(2), int64_t(255), int64_t(256)}) {
        const int64_t N = 100, tiles = (N + FIN_TILE - 1) / FIN_TILE;
        static unsigned char seen[256 * 112];
        for (int64_t i = 0; i < tiles * FIN_TILE * G; ++i) seen[i] = 0;
        for (int64_t b = 0; b < G; ++b)
            for (int64_t c = 0; c < tiles * FIN_TILE; ++c) {
                const int64_t k = partial_index(c, b, G);
                CHECK(k >= 0 && k < tiles * FIN_TILE * G && !seen[k], "partial_index collision");
                if (k >= 0 && k < tiles * FIN_TILE * G) seen[k] = 1;
            }
    }
    // the long-row backward's mode: the measured rule, and the prefetching
    // mode only for 16-bit types (two rows fit the registers beside gamma)
    for (int64_t M : {int64_t(1), int64_t(1024), int64_t(4096), int64_t(4097), int64_t(8192), int64_t(1) << 20})
        for (int64_t N : {LONG_N + 1, int64_t(24576), int64_t(24577), int64_t(28672), MAX_N}) {
            CHECK(long_mode(2, true, M, N) == LM_PREFETCH, "fused 16-bit long rows not prefetched");
            CHECK(long_mode(2, false, M, N) == (N <= 24576 || M <= 4096 ? LM_PREFETCH : LM_RELOAD),
                  "plain 16-bit long-row mode at M %lld N %lld", (long long)M, (long long)N);
            CHECK(long_mode(4, false, M, N) == LM_RESIDENT, "plain fp32 long rows: gamma not resident");
            CHECK(long_mode(4, true, M, N) == LM_RELOAD, "fused fp32 long rows: gamma does not fit");
        }
    // The backward's route for four-chunk rows: never for the plain backward;
    // three chunks a thread cover the row; the next-row kernel (four chunks
    // of 512 threads) only for 16-bit rows it covers and the three-chunk
    // plan does not.
    for (int esize : {2, 4})
        for (int64_t N = 1; N <= MAX_N; ++N) {
            if (!plan_rows(N, esize, true, &p)) continue;
            for (int64_t M : {int64_t(1), int64_t(300), int64_t(4096), int64_t(4100), int64_t(1) << 20})
                for (int v = 0; v < 3; ++v) {
                    const bool fused = v == 1, layer = v == 2;
                    const int r = bwd_route(esize, fused, layer, p, M, N);
                    CHECK(v != 0 || r == BR_PLAN, "plain backward routed at N = %lld", (long long)N);
                    if (r == BR_THREE_CHUNKS)
                        CHECK(p.k == 4 && p.tpr == 512 && (int64_t)3 * p.tpr * p.vec >= N && p.vec * esize == 16 &&
                                  (fused || esize == 2),
                              "three-chunk route at N = %lld esize %d", (long long)N, esize);
                    if (r == BR_NEXT_ROW)
                        CHECK(esize == 2 && p.vec == 8 && p.k == 4 && N > 12288 && N <= 16384 && !p.long_row,
                              "next-row route at N = %lld", (long long)N);
                    // the rows the measurements chose for each route take it
                    if (esize == 2 && p.vec == 8 && N > 8192 && N <= 12288 && (fused || layer))
                        CHECK(r == BR_THREE_CHUNKS, "16-bit N = %lld not on three chunks", (long long)N);
                    if (esize == 2 && p.vec == 8 && N > 12288 && N < 16384 && (fused || layer))
                        CHECK(r == BR_NEXT_ROW, "16-bit N = %lld not on the next-row kernel", (long long)N);
                }
            // the forward's route: three chunks of 512 threads for 16-bit rows
            // of 8200-12288 elements exactly (LayerNorm's at every M, the
            // others' up to 2^26 elements a call); three chunks of 256-thread
            // groups for the plain forward's 16-bit rows of 4104-6144
            // elements from 4096 rows; three chunks of 128-thread groups for
            // every forward's 16-bit rows of 2056-3072 elements from 3072
            // rows; three chunks of one wavefront for 16-bit rows of
            // 1032-1536 elements (the fused forward's from 2048 rows); three
            // chunks of 32-thread groups for 16-bit rows of 520-768 elements
            // (LayerNorm's at every M, the plain forward's from 256 rows, the
            // fused one's from 4096); three chunks instead of four on
            // 16-thread groups for 16-bit rows of 264-384 elements; in each
            // case the chunks cover the row
            for (int64_t M : {int64_t(1), int64_t(255), int64_t(256), int64_t(300), int64_t(2047), int64_t(2048),
                              int64_t(3071), int64_t(3072),
                              int64_t(4095), int64_t(4096), int64_t(5461), int64_t(5462), int64_t(8192),
                              int64_t(1) << 20})
                for (int v = 0; v < 3; ++v) {
                    const bool fused = v == 1, layer = v == 2;
                    const int r = fwd_route(esize, fused, layer, p, M, N);
                    const bool b16v = esize == 2 && p.vec == 8;
                    CHECK((r == FR_THREE_CHUNKS) ==
                              (b16v && N > 8192 && N <= 12288 && (layer || M * N <= (int64_t(1) << 26))),
                          "forward three-chunk route at M %lld N %lld esize %d variant %d", (long long)M,
                          (long long)N, esize, v);
                    CHECK((r == FR_HALF_ROWS) == (b16v && N > 4096 && N <= 6144 && v == 0 && M >= 4096),
                          "forward half-row route at M %lld N %lld esize %d variant %d", (long long)M, (long long)N,
                          esize, v);
                    if (r == FR_THREE_CHUNKS)
                        CHECK((int64_t)3 * 512 * p.vec >= N && p.tpr == 512, "three chunks do not cover N = %lld",
                              (long long)N);
                    if (r == FR_HALF_ROWS)
                        CHECK((int64_t)3 * 256 * p.vec >= N && p.tpr == 512 && p.k == 2,
                              "half-row chunks do not cover N = %lld", (long long)N);
                    CHECK((r == FR_QUARTER_ROWS) ==
                              (p.vec == 16 / esize && (esize == 2 || layer) && N > 256 * (16 / esize) &&
                               N <= 384 * (16 / esize) && M >= 3072),
                          "forward quarter-row route at M %lld N %lld esize %d variant %d", (long long)M,
                          (long long)N, esize, v);
                    if (r == FR_QUARTER_ROWS)
                        CHECK((int64_t)3 * 128 * p.vec >= N && p.tpr == 512 && p.k == 1,
                              "quarter-row chunks do not cover N = %lld", (long long)N);
                    // the fp32 LayerNorm forward takes the wave, quarter and
                    // narrow routes at the same chunk counts
                    const int vwd = 16 / esize;
                    const bool elig = p.vec == vwd && (esize == 2 || layer);
                    CHECK((r == FR_WAVE_ROWS) ==
                              (elig && N > 128 * vwd && N <= 192 * vwd && (!fused || M >= 2048)),
                          "forward wave-row route at M %lld N %lld esize %d variant %d", (long long)M,
                          (long long)N, esize, v);
                    if (r == FR_WAVE_ROWS)
                        CHECK((int64_t)3 * 64 * p.vec >= N && p.tpr == 256 && p.k == 1,
                              "wave-row chunks do not cover N = %lld", (long long)N);
                    CHECK((r == FR_NARROW_ROWS) ==
                              (elig && N > 64 * vwd && N <= 96 * vwd && (layer || M >= (fused ? 4096 : 256))),
                          "forward narrow-row route at M %lld N %lld esize %d variant %d", (long long)M,
                          (long long)N, esize, v);
                    CHECK((r == FR_SHORT_ROWS) == (b16v && N > 256 && N <= 384),
                          "forward short-row route at M %lld N %lld esize %d variant %d", (long long)M,
                          (long long)N, esize, v);
                    if (r == FR_SHORT_ROWS)
                        CHECK((int64_t)3 * 16 * p.vec >= N && p.tpr == 16 && p.k == 4,
                              "short-row chunks do not cover N = %lld", (long long)N);
                    if (r == FR_NARROW_ROWS)
                        CHECK((int64_t)3 * 32 * p.vec >= N && p.tpr == 128 && p.k == 1,
                              "narrow-row chunks do not cover N = %lld", (long long)N);
                }
            // the forward's grid: at least one block, at most one per row
            // window and 512, the fused forward's smaller cap only on the
            // window ring
            for (int64_t M : {int64_t(0), int64_t(1), int64_t(511), int64_t(4096), int64_t(1) << 20})
                for (bool fused : {false, true}) {
                    const int64_t G = fwd_blocks(M, N, p, fused);
                    const int64_t steps = (M + p.rpb - 1) / p.rpb;
                    CHECK(G >= 1 && G <= 512 && (steps < 1 || G <= steps), "forward grid %lld at M %lld N %lld",
                          (long long)G, (long long)M, (long long)N);
                    if (!fused || p.long_row) CHECK(G == (steps < 1 ? 1 : (steps < 512 ? steps : 512)),
                                                    "forward grid %lld off the 512 cap", (long long)G);
                }
        }
    std::printf("plan driver: %d failed checks\n", failures);
    return failures ? 1 : 0;
}
