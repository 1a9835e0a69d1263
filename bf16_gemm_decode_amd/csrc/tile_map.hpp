// tile_map.hpp -- workgroup id -> output tile, shared by the GEMM kernel and
// the host-side helper that tests evaluate without a GPU.
//
// Two steps:
//  1. XCD renumbering.  The dispatcher hands workgroup ids to the 8 XCDs of an
//     MI355X round-robin (id % 8), and each XCD has its own L2.  Renumber so
//     that the ids one XCD receives form one contiguous range of the
//     ordering below; tiles that share A or B panels then meet in one L2.
//  2. Grouped ordering (FlagGems "Hygon 优化" page, section "分组调度"):
//     consecutive ids walk down a group of group_m tile rows, then move to
//     the next tile column, so a group shares one B panel (and group_m A
//     panels); the last group may hold fewer rows.
#pragma once

#include <stdint.h>

namespace migemm {

template <typename I>
__host__ __device__ inline void tile_coord(I wg, I num_pid_m, I num_pid_n, I group_m,
                                           I num_xcd, I &pid_m, I &pid_n)
{
    I total = num_pid_m * num_pid_n;
    I id = wg;
    if (num_xcd > 1) {
        // XCD x receives ids x, x + num_xcd, ...: q + 1 of them when x < r.
        I q = total / num_xcd, r = total % num_xcd;
        I x = wg % num_xcd, slot = wg / num_xcd;
        id = (x < r) ? x * (q + 1) + slot : r * (q + 1) + (x - r) * q + slot;
    }
    I per_group = group_m * num_pid_n;
    I group = id / per_group;
    I first_m = group * group_m;
    I rows = num_pid_m - first_m;
    if (rows > group_m) rows = group_m;
    I local = id - group * per_group;
    pid_m = first_m + local % rows;
    pid_n = local / rows;
}

}  // namespace migemm
