// instances.hpp -- the launch table for one storage type S: every supported
// (VEC, T, W, mode) instance of scan_tiles / scan_one.  Included once per
// storage type by kernels_<type>.hip.
#pragma once

#include "launch.hpp"

namespace linrec_host {

template <typename S, int VEC, int T, int W>
void run_tiles(dim3 grid, dim3 block, const void* a, const void* b, void* h, const linrec::Geometry& g,
               linrec::WorkspaceHeader* hdr, uint64_t* stat, hipStream_t stream) {
    hipLaunchKernelGGL((linrec::scan_tiles<S, VEC, T, W>), grid, block, 0, stream, static_cast<const S*>(a),
                       static_cast<const S*>(b), static_cast<S*>(h), g, hdr, stat);
}

template <typename S, int VEC, int T, int W>
hipError_t occupancy_tiles(int* groups_per_cu, int threads) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(groups_per_cu, linrec::scan_tiles<S, VEC, T, W>, threads, 0);
}

template <typename S, int VEC, int T, int W>
void run_one(dim3 grid, dim3 block, const void* a, const void* b, void* h, const linrec::Geometry& g,
             linrec::WorkspaceHeader* hdr, uint64_t* stat, hipStream_t stream) {
    hipLaunchKernelGGL((linrec::scan_one<S, VEC, T, W>), grid, block, 0, stream, static_cast<const S*>(a),
                       static_cast<const S*>(b), static_cast<S*>(h), g, hdr, stat);
}

template <typename S, int VEC, int T, int W>
hipError_t occupancy_one(int* groups_per_cu, int threads) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(groups_per_cu, linrec::scan_one<S, VEC, T, W>, threads, 0);
}

template <typename S, int VEC, int T, int W>
const Launch* launch_entry(int mode) {
    // register bytes a lane spends on one buffer of T positions (see tile_supported)
    constexpr int lane_bytes = VEC * T * (VEC == 4 && linrec::storage_bytes<S>() == 2 ? 2 : 4);
    if constexpr (W == 15 && lane_bytes > 64) {
        return nullptr;
    } else {
        if (mode == 1) {
            static const Launch one{reinterpret_cast<const void*>(&linrec::scan_one<S, VEC, T, W>),
                                    &run_one<S, VEC, T, W>, &occupancy_one<S, VEC, T, W>};
            return &one;
        }
        if constexpr (lane_bytes > 128) {
            return nullptr;
        } else {
            static const Launch persistent{reinterpret_cast<const void*>(&linrec::scan_tiles<S, VEC, T, W>),
                                           &run_tiles<S, VEC, T, W>, &occupancy_tiles<S, VEC, T, W>};
            return &persistent;
        }
    }
}

template <typename S, int VEC, int T>
const Launch* pick_w(int w, int m) {
    switch (w) {
        case 1: return launch_entry<S, VEC, T, 1>(m);
        case 2: return launch_entry<S, VEC, T, 2>(m);
        case 4: return launch_entry<S, VEC, T, 4>(m);
        case 7: return launch_entry<S, VEC, T, 7>(m);
        case 8: return launch_entry<S, VEC, T, 8>(m);
        case 15: return launch_entry<S, VEC, T, 15>(m);
        default: return nullptr;
    }
}

template <typename S, int VEC>
const Launch* pick_t(int t, int w, int m) {
    switch (t) {
        case 4: return pick_w<S, VEC, 4>(w, m);
        case 8: return pick_w<S, VEC, 8>(w, m);
        case 16: return pick_w<S, VEC, 16>(w, m);
        default: return nullptr;
    }
}

template <typename S>
const Launch* pick_launch(const TileShape& s) {
    if (!tile_supported(s, linrec::storage_bytes<S>())) return nullptr;
    return s.vec == 4 ? pick_t<S, 4>(s.t, s.w, s.m) : pick_t<S, 1>(s.t, s.w, s.m);
}

}  // namespace linrec_host
