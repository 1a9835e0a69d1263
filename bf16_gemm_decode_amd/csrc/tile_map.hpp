// tile_map.hpp -- workgroup id -> output tile, shared by the GEMM kernel and
// the host-side helper that tests evaluate without a GPU.
//
// Two steps:
//  1. XCD renumbering.  The dispatcher hands workgroup ids to the 8 XCDs of an
//     MI355X round-robin (id % 8), and each XCD has its own L2.  Renumber so
//     that the ids one XCD receives form one contiguous range of the
//     ordering below; tiles that share A or B panels then meet in one L2.
//  2. Grouped ordering (FlagGems "Hygon 优化" page, section "分组调度"):
//     the tile rows are cut into bands of group_m rows (the last band may be
//     shorter); the ordering visits the bands in turn and, inside a band,
//     every tile column in turn, taking the band's rows of that column one
//     after another.  A band's consecutive ids therefore share one B panel
//     and the band's A panels.
#pragma once

#include <stdint.h>

namespace migemm {

template <typename I>
__host__ __device__ inline void tile_coord(I wg, I num_pid_m, I num_pid_n, I group_m,
                                           I num_xcd, I &pid_m, I &pid_n)
{
    I id = wg;
    if (num_xcd > 1) {
        // XCD x receives ids x, x + num_xcd, ...: q + 1 of them when x < r.
        const I total = num_pid_m * num_pid_n;
        const I q = total / num_xcd, r = total % num_xcd;
        const I x = wg % num_xcd, slot = wg / num_xcd;
        id = (x < r) ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
    }
    // Ids of the full bands are the mixed-radix numbers (band, column, row)
    // with digit bases (-, num_pid_n, group_m), row least significant.
    const I full_bands = num_pid_m / group_m;
    const I full_ids = full_bands * group_m * num_pid_n;
    if (id < full_ids) {
        const I row = id % group_m, rest = id / group_m;
        pid_n = rest % num_pid_n;
        pid_m = (rest / num_pid_n) * group_m + row;
    } else {
        // the short band: its rows_left rows, again row least significant
        const I rows_left = num_pid_m - full_bands * group_m;
        const I local = id - full_ids;
        pid_m = full_bands * group_m + local % rows_left;
        pid_n = local / rows_left;
    }
}

}  // namespace migemm
