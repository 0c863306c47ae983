// Host check of the fused op's launch geometry (csrc/fused_geometry.h) for
// every row width of 1..8192 packs, both layouts (few rows or many), both
// element sizes and every rank count (16-bit types take the 512-lane register
// path for every row of 2049..4096 packs, fp32 only where its instance keeps
// everything in registers). For each shape it checks what the
// kernels assume: whole waves, no more lanes than the instance's launch
// bound, lanes x packs covering the row, no lane slot that is empty for every
// lane, a (packs per lane, launch bound, slot walk) combination that the
// library compiles, and the preconditions of the pipelined slot walks.
// Prints "ok <shapes checked>" or the first failures, and exits non-zero on
// any failure.
#include <cstddef>
#include <cstdio>
#include <initializer_list>

#include "fused_geometry.h"

using namespace ar_geometry;

static int failures = 0;
static const FusedGeometry none{0, 0, 0};

static void fail(const char *what, int ppr, bool few, bool wide, const FusedGeometry &g)
{
    if (++failures <= 20)
        std::printf("FAIL %s: ppr=%d few_rows=%d wide=%d -> ppt=%d threads=%d bound=%d rows=%d waves=%d\n", what, ppr,
                    few, wide, g.ppt, g.threads, g.bound, g.rows, g.waves);
}

// The instances ar.hip compiles for the one-row-per-workgroup kernel, for an
// element size and rank count.
static bool instance_exists(int ppt, int bound, int mode, int elem_size, int ranks)
{
    if (bound == kFusedMaxThreads)
        return (ppt == 1 || ppt == 2) && mode == kPlain;
    if (bound == 512 && (ppt == 1 || ppt == 2))
        return mode == kPlain;
    if (bound == kWideRowLanes && ppt >= 5 && ppt <= kMaxPPT)
        return (mode == kFull || mode == kRagged) && wide_rows_fit(elem_size, ranks, ppt, mode == kRagged);
    if (bound == 256)
        return ppt >= 3 && ppt <= kMaxPPT && (mode == kFull || (mode == kRagged && ppt >= 5));
    return false;
}

int main()
{
    long checked = 0;
    for (int ppr = 1; ppr <= 8192; ++ppr) {
        for (int few = 0; few < 2; ++few) {
            for (int cls = 0; cls < 16; ++cls) {
                const int elem_size = cls < 8 ? 2 : 4, ranks = cls % 8 + 1;
                const bool wide = wide_rows_in_registers(elem_size, ranks, ppr);
                const FusedGeometry g = fused_geometry(ppr, few, wide);
                ++checked;
                const bool in_registers = ppr <= kMaxPPT * 256 || (wide && ppr <= kMaxPPT * kWideRowLanes);
                if (g.ppt == 0) {
                    if (in_registers)
                        fail("wide kernel for a row the register path takes", ppr, few, wide, g);
                    if (g.threads != kWideThreads || g.bound != kWideThreads)
                        fail("wide kernel shape", ppr, few, wide, g);
                    continue;
                }
                if (!in_registers)
                    fail("register path for a row it cannot hold", ppr, few, wide, g);
                if (g.threads < kWave || g.threads % kWave != 0 || g.threads > g.bound)
                    fail("workgroup not whole waves within the launch bound", ppr, few, wide, g);
                if (g.waves > 0) {
                    const bool known = (g.ppt == 2 && g.waves == 8) || (g.ppt == 4 && g.waves == 4);
                    if (few || !known || g.threads != g.waves * kWave || ppr != g.ppt * kWave || g.bound != 512)
                        fail("wave-per-row shape", ppr, few, wide, g);
                    continue;
                }
                if (g.rows > 1) {
                    if (few || g.rows != 2 || g.ppt != 1 || g.threads < ppr || g.threads > kRowsMaxPacks ||
                        g.bound != kRowsMaxPacks)
                        fail("multi-row shape", ppr, few, wide, g);
                    continue;
                }
                if (g.ppt > kMaxPPT || g.ppt * g.threads < ppr)
                    fail("lanes x packs do not cover the row", ppr, few, wide, g);
                if ((g.ppt - 1) * g.threads >= ppr)
                    fail("a slot empty for every lane", ppr, few, wide, g);
                const int mode = pipeline_mode(g.ppt, g.threads, ppr);
                if (!instance_exists(g.ppt, g.bound, mode, elem_size, ranks))
                    fail("no compiled instance for this shape", ppr, few, wide, g);
                if (mode == kFull && ppr != g.ppt * g.threads)
                    fail("full pipeline on a row that does not fill every slot", ppr, few, wide, g);
                if (mode == kRagged && !((g.ppt - 1) * g.threads < ppr && ppr < g.ppt * g.threads))
                    fail("ragged pipeline with a slot other than the last one partial", ppr, few, wide, g);
            }
        }
    }
    // The layout switch: the latency layout only when rows do not outnumber
    // the CUs, and then at most 1 or 2 packs per lane on up to 1024 lanes, or
    // rows the register path does not hold, or the 512-lane register path.
    for (int cus : {80, 104, 256, 304}) {
        for (int ppr = 1; ppr <= 8192; ppr += (ppr < 2100 ? 1 : 7)) {
            for (size_t rows : {size_t(1), size_t(cus / 2), size_t(cus * 3 / 4), size_t(cus * 3 / 4 + 1),
                                size_t(cus), size_t(cus + 1), size_t(1) << 20}) {
                const bool lat = latency_layout(ppr, rows, cus);
                if (lat && rows > size_t(cus))
                    fail("latency layout with more rows than CUs", ppr, true, false, none);
                for (int wide = 0; wide < 2; ++wide) {
                    const FusedGeometry g = fused_geometry(ppr, lat, wide);
                    ++checked;
                    if (lat && g.ppt > 0 && g.bound != kFusedMaxThreads && g.bound != kWideRowLanes &&
                        ppr > kRowsMaxPacks)
                        fail("latency layout on a throughput instance", ppr, lat, wide, g);
                }
            }
        }
    }
    // The slot walk on its own, for every packs-per-lane count, workgroup size
    // and row it could be asked about: a pipelined walk never leaves a slot
    // other than the last one partial.
    for (int ppt = 1; ppt <= kMaxPPT; ++ppt)
        for (int threads = kWave; threads <= kFusedMaxThreads; threads += kWave)
            for (int ppr = 1; ppr <= ppt * threads; ++ppr) {
                const int mode = pipeline_mode(ppt, threads, ppr);
                if (mode == kFull && ppr != ppt * threads)
                    fail("pipeline_mode: full walk on a partial row", ppr, false, false, none);
                if (mode == kRagged && !((ppt - 1) * threads < ppr && ppr < ppt * threads))
                    fail("pipeline_mode: ragged walk with an earlier slot partial", ppr, false, false, none);
                if (mode != kPlain && (ppt < 3 || (threads > kFullLanes && threads != kWideRowLanes)))
                    fail("pipeline_mode: pipelined walk outside the compiled shapes", ppr, false, false, none);
            }
    // Rows of more than 4096 packs take the chunked path - rows that no
    // register path holds in any type; a chunk is whole lanes x whole packs.
    if (kChunkPacks % kChunkLanes != 0 || kChunkLanes % kWave != 0)
        fail("chunk shape", kChunkPacks, false, false, none);
    for (int ppr = 1; ppr <= 16384; ++ppr)
        if (wide_rows_chunked(ppr) != (ppr > kMaxPPT * kWideRowLanes) ||
            (wide_rows_chunked(ppr) && (fused_geometry(ppr, true, true).ppt != 0 ||
                                        fused_geometry(ppr, false, true).ppt != 0)))
            fail("chunked-path rule", ppr, false, true, none);
    // Which rows take the 512-lane register path: every 16-bit row of
    // 2049..4096 packs; fp32 rows up to 2 ranks, and from 3 ranks only rows of
    // 2049..2560 packs (5 per lane), at 8 ranks only the full ones.
    for (int ranks = 1; ranks <= 8; ++ranks)
        for (int ppr = 2049; ppr <= 4096; ++ppr) {
            if (!wide_rows_in_registers(2, ranks, ppr))
                fail("16-bit row kept off the 512-lane register path", ppr, false, false, none);
            const bool fp32 = ranks <= kFp32WideRowMaxRanks || (ppr <= 2560 && (ranks <= 7 || ppr == 2560));
            if (wide_rows_in_registers(4, ranks, ppr) != fp32)
                fail("fp32 rule of the 512-lane register path", ppr, false, true, none);
        }
    if (failures) {
        std::printf("%d failures\n", failures);
        return 1;
    }
    std::printf("ok %ld\n", checked);
    return 0;
}
