// fused_geometry.h - launch shape of the fused op's register-row kernels
// (host code only). For a row of `ppr` 16-byte packs it picks the kernel, the
// packs per lane, the workgroup size and the kernel instance's launch bound,
// and for the one-row-per-workgroup kernel whether its slots run pipelined.
// Included by ar.hip; a host test checks every row width against the kernel
// instances ar.hip compiles.
#ifndef AR_FUSED_GEOMETRY_H
#define AR_FUSED_GEOMETRY_H

#include <stddef.h>

namespace ar_geometry {

constexpr int kWave = 64;
// Register-row fused kernel, two layouts. Throughput layout (more rows than
// CUs): a row of up to 1024 packs takes 1 or 2 packs per lane on up to 512
// lanes; wider rows (up to 2048 packs) take 3..8 packs per lane on up to 256
// lanes, which keeps every variant within the VGPR budget of its launch bound
// (those on 256 lanes run pipelined, the last slot possibly partial, and so
// do rows of exactly 1024 packs, as 4 x 256); rows of 2049..4096 packs in
// 16-bit types, and in fp32 with one or two ranks, take 5..8 pipelined packs
// per lane on 512 lanes;
// rows of 320, 384 and 640 packs take 64 or 128 lanes (see fused_geometry).
// Latency layout (no more rows than CUs - for rows of 1024..2048 packs, no
// more than three quarters of them - and rows of 513..2048 packs): up to 1024
// lanes, so each lane's packs - and so the memory round trips of a row - are
// halved when the chip is not full anyway.
constexpr int kMaxPPT = 8;
constexpr int kFusedMaxThreads = 1024;
constexpr int kLatencyMaxPPT = 2;
constexpr int kFullMaxPPT = 8;      // pipelined variant: slots per lane, at most
constexpr int kFullLanes = 256;     // pipelined variant: workgroup size, at most (but see kWideRowLanes)
constexpr int kRowsMaxPacks = 512;  // multi-row kernel: widest row, and workgroup size bound
constexpr int kWideRowLanes = 512;  // register path for rows of 2049..4096 packs (16-bit types)
constexpr int kWideThreads = 1024;  // workgroup size of the two-pass kernel for rows wider than that

// Whether the 512-lane register path has an instance for rows of 2049..4096
// packs at `ppt` packs per lane (ragged: the last slot partly covered): every
// one in 16-bit types, and in fp32 those that keep every value in registers -
// all of them up to 2 ranks (101-230 VGPRs), and at 5 packs per lane every
// rank count (152-253 VGPRs) except the 8-rank ragged walk, which spills.
// Most other fp32 ones spill too (every one at 7-8 packs from 4 ranks, at 6
// packs from 7 ranks and in the 6-rank ragged walk, the 3-rank ragged walk
// at 8); the few that do not are left out to keep this rule short, and those
// rows take the two-pass wide kernel.
constexpr int kFp32WideRowMaxRanks = 2;
constexpr bool wide_rows_fit(int elem_size, int ranks, int ppt, bool ragged)
{
    return elem_size == 2 || ranks <= kFp32WideRowMaxRanks || (ppt == 5 && (ranks <= 7 || !ragged));
}

// Whether a row of `ppr` packs (2049..4096) takes the 512-lane register path.
constexpr bool wide_rows_in_registers(int elem_size, int ranks, int ppr)
{
    return wide_rows_fit(elem_size, ranks, (ppr + kWideRowLanes - 1) / kWideRowLanes, ppr % kWideRowLanes != 0);
}

// Rows of more than 4096 packs: each row is cut into chunks of kChunkPacks
// packs (kChunkLanes lanes x 2), one workgroup per chunk, over three launches
// (sums, row scale, norm), so the work spreads over the whole chip whatever
// the row count. Against the two-pass kernel (one workgroup per row):
// 11-74 % faster at 1-128 rows of hidden 40960..131072 in 16-bit types and
// 16388..65536 in fp32, 4-9 % at 192-819 rows, within 2 % at 512-2048 8-rank
// rows; 4-6 % slower only at 256 two-rank and 768 one-rank rows of 65536.
// Narrower rows that take the two-pass kernel (fp32 rows of 2049..4096 packs
// from 3 ranks) keep it: there the chunked path was 24 % slower on small
// calls (100 3-rank rows of 10240) and 28 % faster on others, no better on
// the whole.
constexpr int kChunkLanes = 512;
constexpr int kChunkPacks = 2 * kChunkLanes;
inline bool wide_rows_chunked(int ppr)
{
    return ppr > kMaxPPT * kWideRowLanes;
}

// How the one-row-per-workgroup kernel walks a lane's slots.
enum PipelineMode {
    kPlain = 0,   // one bounds-tested slot at a time
    kFull = 1,    // every slot of every lane holds a pack; pipelined two deep
    kRagged = 2,  // pipelined; every slot but the last is full
};

// Launch shape of the register-row kernel for a row of `ppr` packs.
struct FusedGeometry {
    int ppt;      // packs per lane; 0 = the row is too wide, the wide kernel takes it
    int threads;  // workgroup size: the fewest whole waves that cover the row
    int bound;    // launch bound of the kernel instance (512, 256 or 1024)
    int rows = 1; // rows per workgroup iteration: > 1 selects the multi-row kernel
    int waves = 0; // > 0 selects the wave-per-row kernel, with this many waves (rows) per workgroup
};

// Throughput layout: rows of 128 and 256 packs take the wave-per-row kernel
// (2 or 4 packs per lane, 8 or 4 rows per workgroup, no barrier): measured
// 5-7 % faster than one workgroup per row on hidden 1024 and 2048 in 16-bit
// types. Rows of 512 packs take the multi-row kernel (one pack per lane, 2
// adjacent rows per iteration, one barrier): 1.5-4 % faster on hidden 4096
// in 16-bit types, where the wave-per-row kernel (8 packs per lane) was
// slower. Other rows up to 512 packs keep one row per workgroup, 1 pack per
// lane (4 rows per iteration measured 3-5 % slower at 448 packs). Wider
// rows: 2 packs per lane up to 1024, then ceil(ppr / 256) up to kMaxPPT;
// rows of exactly 1024 packs (hidden 8192 in 16-bit types, 4096 in fp32)
// take 256 lanes x 4 packs in the pipelined full-row variant instead, 1.5-2 %
// faster than 512 x 2 (and 8 x 128 was 1-5 % slower). Three row
// widths would get workgroups of 5 or 6 waves, which a CU's four SIMDs share
// unequally; they take 64 or 128 lanes with 3 or 5 packs each instead (the
// pipelined full-row variant): rows of 320, 384 and 640 packs (hidden 2560,
// 3072 and 5120 in 16-bit types) measured 3-9 % faster so. Rows of 768 packs
// (6 waves of 2 packs) gained at most 2 % and rows of 896 (7 waves) lost on
// 128 lanes, so they keep the default. Rows of 1025..2048 packs fill 5..8
// slots on 256 lanes, all full or all but the last, and so run pipelined too.
// Rows of 2049..4096 packs where `wide_rows_in_registers` holds (16-bit
// types; fp32 with one or two ranks) take 512 lanes x ceil(ppr / 512) packs,
// pipelined, at any row count (replayed from a HIP graph, 5-36 % faster than
// the two-pass kernel at 16..256 rows of hidden 20480 and 32768 in 16-bit
// types; 5-30 % on fp32 one- and two-rank rows of hidden 9216..16384); wider
// rows, and the other fp32 rows past 2048 packs, take the two-pass wide
// kernel.
// Latency layout (`few_rows`, rows of more than 512 packs): ceil(ppr / 1024)
// packs per lane, up to kLatencyMaxPPT.
inline FusedGeometry fused_geometry(int ppr, bool few_rows, bool wide_rows_in_registers)
{
    int k, bound;
    if (wide_rows_in_registers && ppr > kMaxPPT * 256 && ppr <= kMaxPPT * kWideRowLanes)
        return FusedGeometry{(ppr + kWideRowLanes - 1) / kWideRowLanes, kWideRowLanes, kWideRowLanes};
    if (!few_rows) {
        switch (ppr) {
        case 320: return FusedGeometry{5, 64, 256};
        case 384: return FusedGeometry{3, 128, 256};
        case 640: return FusedGeometry{5, 128, 256};
        default: break;
        }
        if (ppr == 128 || ppr == 256) {
            FusedGeometry g{ppr / kWave, ppr == 128 ? 8 * kWave : 4 * kWave, 512};
            g.waves = g.threads / kWave;
            return g;
        }
        if (ppr == kRowsMaxPacks)
            return FusedGeometry{1, ppr, kRowsMaxPacks, 2};
        if (ppr == 1024)
            return FusedGeometry{4, 256, 256};
    }
    if (few_rows && ppr > 512 && ppr <= kLatencyMaxPPT * kFusedMaxThreads) {
        k = (ppr + kFusedMaxThreads - 1) / kFusedMaxThreads;
        bound = kFusedMaxThreads;
    } else if (ppr <= 512) {
        k = 1;
        bound = 512;
    } else if (ppr <= 1024) {
        k = 2;
        bound = 512;
    } else {
        k = (ppr + 255) / 256;
        bound = 256;
    }
    if (k > kMaxPPT)
        return FusedGeometry{0, kWideThreads, kWideThreads};
    int t = (ppr + k - 1) / k;
    t = (t + kWave - 1) / kWave * kWave;
    return FusedGeometry{k, t < kWave ? kWave : t, bound};
}

// Whether a call of `rows` rows of `ppr` packs on `cus` compute units takes
// the latency layout: no more rows than CUs, except that rows of 1024..2048
// packs take the throughput layout once they exceed three quarters of the
// CUs (replayed from a HIP graph at 256 CUs: 2-8 % faster at 224 and 256
// rows of hidden 8192..16384 in 16-bit types and 4096 in fp32, within 2 % at
// 160 and 192 rows, 4-6 % slower at 16 and 64).
inline bool latency_layout(int ppr, size_t rows, int cus)
{
    if (rows > static_cast<size_t>(cus))
        return false;
    if (ppr >= 1024 && ppr <= kMaxPPT * 256 && rows * 4 > static_cast<size_t>(cus) * 3)
        return false;
    return true;
}

// Slot walk of the one-row-per-workgroup kernel for `ppt` packs per lane on
// `threads` lanes. Pipelined where it was measured faster: 3..8 slots on up
// to 256 lanes when every slot is full; 256 lanes when every slot but the
// last is full; 512 lanes with 5..8 slots (rows of 2049..4096 packs), full or
// ragged. Everything else walks one slot at a time.
inline int pipeline_mode(int ppt, int threads, int ppr)
{
    if (ppt < 3 || ppt > kFullMaxPPT || ppr > ppt * threads)
        return kPlain;
    const bool wide = threads == kWideRowLanes && ppt >= 5;
    if (ppr == ppt * threads && (threads <= kFullLanes || wide))
        return kFull;
    if ((threads == kFullLanes || wide) && ppr > (ppt - 1) * threads)
        return kRagged;
    return kPlain;
}

}  // namespace ar_geometry

#endif  // AR_FUSED_GEOMETRY_H
