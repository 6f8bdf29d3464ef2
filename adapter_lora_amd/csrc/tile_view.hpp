// What a workgroup needs to know about one tile of the schedule
// ("vLLM-Ascend dynamic LoRA operator" walkthrough, section 2.4: which block
// covers which segment and rank is settled before the product kernels run):
// the tile's segment, adapter, first sorted position and row count, the
// token index of each of its 64 rows (one per lane), and the adapter's padded
// rank and weight offset.  Everything comes from independent loads issued
// together (for tables of up to 256 slots every slot's rank and offset,
// picked by lane shuffle), so it costs one memory round trip.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace mlora {

constexpr int kRowTile = kRowTileRows;
static_assert(kRowTile == 64, "tile functions assume 64-row tiles");

struct TileView {
    int seg;       // -1 when the tile does not exist
    int id;
    int pbeg;
    int n;
    int rp;
    int64_t off;
    int row;       // lane i: token index of row i (-1 past n)
};

__device__ __forceinline__ TileView tile_view(const LinearArgs& a, int t, bool a_side) {
    const int lane = lane_id();
    const int64_t* offs = a_side ? a.a_off : a.b_off;
    TileView v;
    const int nt = a.num_tiles[0];
    const int tt = t < a.max_tiles ? t : 0;
    v.seg = a.tile_info[tt * 4 + 0];
    v.id = a.tile_info[tt * 4 + 1];
    v.pbeg = a.tile_info[tt * 4 + 2];
    v.n = a.tile_info[tt * 4 + 3];
    v.row = a.tile_rows[(int64_t)tt * kRowTile + lane];
    if (a.L <= 4 * kWave) {
        int rk[4];
        int64_t of[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = q * kWave + lane;
            rk[q] = j < a.L ? a.rank[j] : 0;
            of[q] = j < a.L ? offs[j] : 0;
        }
        const int id = (t < nt && v.id >= 0 && v.id < a.L) ? v.id : 0;
        const int q = id / kWave, src = id % kWave;
        const int r_sel = q == 0 ? rk[0] : q == 1 ? rk[1] : q == 2 ? rk[2] : rk[3];
        const int64_t o_sel = q == 0 ? of[0] : q == 1 ? of[1] : q == 2 ? of[2] : of[3];
        v.rp = __shfl(r_sel, src, kWave);
        v.off = __shfl(o_sel, src, kWave);
    } else {
        const int id = (t < nt && v.id >= 0 && v.id < a.L) ? v.id : 0;
        v.rp = a.rank[id];
        v.off = offs[id];
    }
    if (t >= nt) v.seg = -1;
    if (kTableChecks && t < nt) {
        // the tile must lie inside the batch and name a slot of the table;
        // rows past its count are -1
        const bool head_ok = v.seg >= 0 && v.id >= 0 && v.id < a.L && v.n >= 1 &&
                             v.n <= kRowTile && v.pbeg >= 0 && v.pbeg <= a.M - v.n;
        const bool row_ok = lane < v.n ? (v.row >= 0 && v.row < a.M) : v.row == -1;
        if (table_fault(a.err, !(head_ok && row_ok))) v.seg = -1;
    }
    return v;
}

}  // namespace mlora
