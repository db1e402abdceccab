// instances.hpp -- the launch table for one storage type S: every supported
// (VEC, T, W, mode) instance of scan_tiles / scan_one / scan_relay, each in the plain form
// and in the reverse form whose decays are one time step ahead (AHEAD), which
// has kernels of its own so that the plain ones are not changed by it.
// Included once per storage type by kernels_<type>.hip.
#pragma once

#include "launch.hpp"

namespace linrec_host {

template <typename S, int VEC, int T, int W, bool AHEAD>
void run_tiles(dim3 grid, dim3 block, const void* a, const void* b, void* h, const linrec::Geometry& g,
               linrec::WorkspaceHeader* hdr, uint64_t* stat, hipStream_t stream) {
    hipLaunchKernelGGL((linrec::scan_tiles<S, VEC, T, W, AHEAD>), grid, block, 0, stream, static_cast<const S*>(a),
                       static_cast<const S*>(b), static_cast<S*>(h), g, hdr, stat);
}

template <typename S, int VEC, int T, int W, bool AHEAD>
hipError_t occupancy_tiles(int* groups_per_cu, int threads) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(groups_per_cu, linrec::scan_tiles<S, VEC, T, W, AHEAD>, threads,
                                                        0);
}

template <typename S, int VEC, int T, int W, bool AHEAD>
void run_one(dim3 grid, dim3 block, const void* a, const void* b, void* h, const linrec::Geometry& g,
             linrec::WorkspaceHeader* hdr, uint64_t* stat, hipStream_t stream) {
    hipLaunchKernelGGL((linrec::scan_one<S, VEC, T, W, AHEAD>), grid, block, 0, stream, static_cast<const S*>(a),
                       static_cast<const S*>(b), static_cast<S*>(h), g, hdr, stat);
}

template <typename S, int VEC, int T, int W, bool AHEAD>
hipError_t occupancy_one(int* groups_per_cu, int threads) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(groups_per_cu, linrec::scan_one<S, VEC, T, W, AHEAD>, threads,
                                                        0);
}

template <typename S, int VEC, int T, int W, bool AHEAD>
void run_relay(dim3 grid, dim3 block, const void* a, const void* b, void* h, const linrec::Geometry& g,
               linrec::WorkspaceHeader*, uint64_t*, hipStream_t stream) {
    hipLaunchKernelGGL((linrec::scan_relay<S, VEC, T, W, AHEAD>), grid, block, 0, stream, static_cast<const S*>(a),
                       static_cast<const S*>(b), static_cast<S*>(h), g);
}

template <typename S, int VEC, int T, int W, bool AHEAD>
hipError_t occupancy_relay(int* groups_per_cu, int threads) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(groups_per_cu, linrec::scan_relay<S, VEC, T, W, AHEAD>,
                                                        threads, 0);
}

template <typename S, int VEC, int T, int W, bool AHEAD>
const Launch* launch_entry(int mode) {
    // register bytes a lane spends on one buffer of T positions (see tile_supported)
    constexpr int lane_bytes = VEC * T * (VEC == 4 && linrec::storage_bytes<S>() == 2 ? 2 : 4);
    if constexpr (W == 15 && lane_bytes > 64) {
        return nullptr;
    } else {
        if (mode == 1) {
            static const Launch one{reinterpret_cast<const void*>(&linrec::scan_one<S, VEC, T, W, AHEAD>),
                                    &run_one<S, VEC, T, W, AHEAD>, &occupancy_one<S, VEC, T, W, AHEAD>};
            return &one;
        }
        if constexpr (lane_bytes > 128) {
            return nullptr;
        } else {
            if (mode == 2) {
                if constexpr (W > 2) {
                    return nullptr;
                } else {
                    static const Launch relay{reinterpret_cast<const void*>(&linrec::scan_relay<S, VEC, T, W, AHEAD>),
                                              &run_relay<S, VEC, T, W, AHEAD>, &occupancy_relay<S, VEC, T, W, AHEAD>};
                    return &relay;
                }
            }
            static const Launch persistent{reinterpret_cast<const void*>(&linrec::scan_tiles<S, VEC, T, W, AHEAD>),
                                           &run_tiles<S, VEC, T, W, AHEAD>, &occupancy_tiles<S, VEC, T, W, AHEAD>};
            return &persistent;
        }
    }
}

template <typename S, int VEC, int T, bool AHEAD>
const Launch* pick_w(int w, int m) {
    switch (w) {
        case 1: return launch_entry<S, VEC, T, 1, AHEAD>(m);
        case 2: return launch_entry<S, VEC, T, 2, AHEAD>(m);
        case 4: return launch_entry<S, VEC, T, 4, AHEAD>(m);
        case 7: return launch_entry<S, VEC, T, 7, AHEAD>(m);
        case 8: return launch_entry<S, VEC, T, 8, AHEAD>(m);
        case 15: return launch_entry<S, VEC, T, 15, AHEAD>(m);
        default: return nullptr;
    }
}

template <typename S, int VEC, bool AHEAD>
const Launch* pick_t(int t, int w, int m) {
    switch (t) {
        case 4: return pick_w<S, VEC, 4, AHEAD>(w, m);
        case 8: return pick_w<S, VEC, 8, AHEAD>(w, m);
        case 16: return pick_w<S, VEC, 16, AHEAD>(w, m);
        default: return nullptr;
    }
}

template <typename S>
const Launch* pick_launch(const TileShape& s, bool ahead) {
    if (!tile_supported(s, linrec::storage_bytes<S>())) return nullptr;
    if (ahead) return s.vec == 4 ? pick_t<S, 4, true>(s.t, s.w, s.m) : pick_t<S, 1, true>(s.t, s.w, s.m);
    return s.vec == 4 ? pick_t<S, 4, false>(s.t, s.w, s.m) : pick_t<S, 1, false>(s.t, s.w, s.m);
}

}  // namespace linrec_host
