// launch.hpp -- host-side description of one kernel instantiation: the tile
// shape a call asks for and the table entry that launches the matching
// template instance.  The instances for each storage type live in their own
// translation unit (kernels_f32.hip, kernels_bf16.hip, kernels_f16.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "scan_kernel.hpp"

namespace linrec_host {

struct TileShape {
    int vec;  // channels per lane
    int t;    // positions per lane
    int w;    // data waves per workgroup
    int p;    // most lanes that share one position of a channel slab (power of two <= 64)
    int q;    // persistent workgroups per CU (0: as many as fit)
    int m;    // 0: persistent workgroups with carry waves; 1: one tile per workgroup;
              // 2: as 0, but where the carry stays local the relay kernel runs it (the
              // carry wave does the group scan, one tile behind); with w > 2 or slabs
              // wider than 64 channels the plan runs as 0
    int l;    // 1: persistent workgroups keep the carry local when their grid can divide
              // the sequences among them; 0: always look back
    int x = 1;  // 1: slabs that share a cache line are scanned on one XCD (when rows are
                // narrower than a line); 0: sequences in dispatch order
};

// Register bytes a lane spends per channel and position: 4 (fp32 values, or
// 16-bit values widened on load with VEC = 1), 2 (16-bit values kept packed,
// VEC = 4).
inline int register_bytes(int vec, int storage_bytes) { return vec == 4 && storage_bytes == 2 ? 2 : 4; }

// Instantiated tile shapes, for a storage type of storage_bytes per element.
// Persistent workgroups keep two register buffers of T positions x VEC
// channels, which spill beyond 128 bytes a lane each (the relay keeps three);
// 15 data waves leave at most 128 registers a lane, which spill beyond 64
// bytes of positions.
inline bool tile_supported(const TileShape& s, int storage_bytes = 4) {
    const bool vec_ok = s.vec == 1 || s.vec == 4;
    const bool t_ok = s.t == 4 || s.t == 8 || s.t == 16;
    const bool w_ok = s.w == 1 || s.w == 2 || s.w == 4 || s.w == 7 || s.w == 8 || s.w == 15;
    const bool m_ok = s.m == 0 || s.m == 1 || s.m == 2;
    const int lane_bytes = s.vec * s.t * register_bytes(s.vec, storage_bytes);
    const bool fits = !(s.m != 1 && lane_bytes > 128) && !(s.w == 15 && lane_bytes > 64);
    const bool p_ok = s.p >= 1 && s.p <= 64 && (s.p & (s.p - 1)) == 0;
    const bool q_ok = s.q >= 0 && s.q <= 64;
    const bool l_ok = s.l == 0 || s.l == 1;
    const bool x_ok = s.x == 0 || s.x == 1;
    return vec_ok && t_ok && w_ok && m_ok && fits && p_ok && q_ok && l_ok && x_ok;
}

struct Launch {
    const void* kernel;   // identifies the instantiation (occupancy cache key)
    void (*run)(dim3 grid, dim3 block, const void* a, const void* b, void* h, const linrec::Geometry&,
                linrec::WorkspaceHeader*, uint64_t*, hipStream_t);
    hipError_t (*occupancy)(int* groups_per_cu, int threads);
};

// Table lookups, one per storage type; nullptr when the shape has no instance.
// `ahead`: the reverse form with the decays one time step ahead.
const Launch* pick_launch_f32(const TileShape& s, bool ahead);
const Launch* pick_launch_bf16(const TileShape& s, bool ahead);
const Launch* pick_launch_f16(const TileShape& s, bool ahead);

}  // namespace linrec_host
