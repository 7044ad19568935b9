// Workgroup id -> output tile, shared by the MFMA tile kernels.
//
// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs of
// MI355X, each with its own L2. The id is remapped so that every XCD receives
// one compact range of tiles (its A row-blocks and B column-blocks stay in its
// own L2), and that range is walked in groups of kGroupM tile rows so that
// workgroups running together share operands.
#pragma once

namespace libgemm {

constexpr int kXcds = 8;
constexpr int kGroupM = 4;

__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int full = total - total % kXcds;
    int id = bid;
    if (bid < full) id = (bid % kXcds) * (full / kXcds) + bid / kXcds;  // XCD x owns ids [x*per, (x+1)*per)
    const int group_span = kGroupM * tiles_n;
    const int group = id / group_span;
    const int first_m = group * kGroupM;
    const int rows = min(tiles_m - first_m, kGroupM);
    const int in_group = id - group * group_span;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

}  // namespace libgemm
