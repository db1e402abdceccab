// linrec.hip -- host side of the C ABI in include/linrec.h: argument checks,
// tile choice, the per-device lookback workspace and the kernel launch.
//
// The operation and its evaluation order are described in scan_kernel.hpp and
// in the header; this file holds no arithmetic of the recurrence.
#include "linrec.h"
#include "scan_kernel.hpp"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

namespace {

using linrec::Geometry;
using linrec::WorkspaceHeader;

thread_local std::string t_last_error;

linrec_status fail(linrec_status s, const std::string& msg) {
    t_last_error = msg;
    return s;
}

std::string hip_text(hipError_t e) { return std::string(hipGetErrorName(e)) + ": " + hipGetErrorString(e); }

// ----------------------------------------------------------------------------- tile shapes

struct TileShape {
    int vec;  // channels per lane
    int t;    // steps per lane
    int w;    // waves per workgroup
    int p;    // most lanes that share one time step of a channel slab (power of two <= 64)
    int q;    // persistent workgroups per CU (0: as many as fit)
    int m;    // 0: persistent workgroups with carry waves; 1: one tile per workgroup
};

bool tile_supported(const TileShape& s) {
    const bool vec_ok = s.vec == 1 || s.vec == 4;
    const bool t_ok = s.t == 4 || s.t == 8 || s.t == 16;
    // w data waves plus the carry wave make up a workgroup
    const bool w_ok = s.w == 1 || s.w == 2 || s.w == 4 || s.w == 6 || s.w == 7 || s.w == 8 || s.w == 14 || s.w == 15;
    const bool m_ok = s.m == 0 || s.m == 1;
    // two register buffers of 16 steps x 4 channels do not fit the registers a
    // lane gets once the workgroup may hold up to 4 carry waves (they spill)
    const bool fits = !(s.m == 0 && s.vec == 4 && s.t == 16) &&
                      // 14 or 15 data waves leave at most 128 registers a lane
                      !(s.w >= 14 && s.vec * s.t > 16);
    const bool p_ok = s.p >= 1 && s.p <= 64 && (s.p & (s.p - 1)) == 0;
    const bool q_ok = s.q >= 0 && s.q <= 64;
    return vec_ok && t_ok && w_ok && m_ok && fits && p_ok && q_ok;
}

// Tile choice, from sweeps on MI355X over the five workloads: persistent
// workgroups of 8 data waves, 4 steps per lane and 32 lanes (512 bytes) per
// row segment stream best when there are many (batch row, channel slab)
// sequences.  With few sequences each carry chain is long: one workgroup per
// tile, 15 data waves and a single carry wave (64-channel slabs) then keep
// more tiles in flight along each chain.
TileShape default_tile(int64_t B, int64_t L, int64_t D, bool vec4) {
    const int vec = vec4 ? 4 : 1;
    const double n = static_cast<double>(B) * static_cast<double>(L) * static_cast<double>(D);
    if (n <= 65536.0) return TileShape{vec, 4, 1, 64, 0, 0};
    TileShape s{vec, 4, 8, 32, 0, 0};
    const int64_t lanes = std::min<int64_t>(32, (D + vec - 1) / vec);
    const int64_t sequences = B * ((D + vec * lanes - 1) / (vec * lanes));
    if (sequences < 32) {
        s.m = 1;
        s.w = 15;
        s.p = 64 / vec;
    }
    return s;
}

// LINREC_TILE="t=16,w=4,vec=4,p=64,q=2,m=0" (any subset of the keys).
bool apply_tile_env(TileShape& s, std::string& err) {
    const char* env = std::getenv("LINREC_TILE");
    if (env == nullptr || *env == '\0') return true;
    std::string spec(env);
    size_t pos = 0;
    while (pos <= spec.size()) {
        size_t end = spec.find(',', pos);
        if (end == std::string::npos) end = spec.size();
        const std::string item = spec.substr(pos, end - pos);
        const size_t eq = item.find('=');
        if (eq == std::string::npos) {
            err = "LINREC_TILE item '" + item + "' is not key=value";
            return false;
        }
        const std::string key = item.substr(0, eq);
        char* stop = nullptr;
        const long val = std::strtol(item.c_str() + eq + 1, &stop, 10);
        if (stop == item.c_str() + eq + 1 || *stop != '\0') {
            err = "LINREC_TILE value in '" + item + "' is not an integer";
            return false;
        }
        if (key == "t") s.t = static_cast<int>(val);
        else if (key == "w") s.w = static_cast<int>(val);
        else if (key == "vec") s.vec = static_cast<int>(val);
        else if (key == "p") s.p = static_cast<int>(val);
        else if (key == "q") s.q = static_cast<int>(val);
        else if (key == "m") s.m = static_cast<int>(val);
        else {
            err = "LINREC_TILE key '" + key + "' is not one of t, w, vec, p, q, m";
            return false;
        }
        pos = end + 1;
    }
    if (!tile_supported(s)) {
        err = "LINREC_TILE asks for an unsupported tile (t in {4,8,16}, w in {1,2,4,6,7,8,14,15}, vec in {1,4}, "
              "p a power of two <= 64, q in [0, 64], m in {0,1}; not vec=4 with t=16 and m=0, "
              "not w >= 14 with vec*t > 16)";
        return false;
    }
    return true;
}

uint32_t spin_limit() {
    const char* env = std::getenv("LINREC_SPIN_LIMIT");
    if (env != nullptr && *env != '\0') {
        char* stop = nullptr;
        const unsigned long v = std::strtoul(env, &stop, 10);
        if (stop != env && *stop == '\0') return static_cast<uint32_t>(v > 0xffffffffUL ? 0xffffffffUL : v);
    }
    // polls of one predecessor (each a memory round trip plus a short sleep,
    // about a microsecond) before its pair is recomputed from the inputs
    return 512u;
}

// ----------------------------------------------------------------------------- geometry

struct Plan {
    TileShape tile;
    Geometry geom;
    int64_t tiles;
    size_t workspace_bytes;
};

bool checked_mul(int64_t x, int64_t y, int64_t& out) {
    if (x == 0 || y == 0) { out = 0; return true; }
    if (x > INT64_MAX / y) return false;
    out = x * y;
    return true;
}

linrec_status make_plan(int64_t B, int64_t L, int64_t D, bool aligned16, Plan& p) {
    if (B < 0 || L < 0 || D < 0) return fail(LINREC_ERR_INVALID_ARGUMENT, "B, L and D must be >= 0");
    int64_t bl = 0, n = 0;
    if (!checked_mul(B, L, bl) || !checked_mul(bl, D, n) || n > INT64_MAX / 8)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "B*L*D*4 bytes overflows");

    TileShape s = default_tile(B, L, D, aligned16 && D % 4 == 0);
    if (!tile_supported(s)) return fail(LINREC_ERR_INVALID_ARGUMENT, "internal: default tile not supported");
    std::string err;
    if (!apply_tile_env(s, err)) return fail(LINREC_ERR_INVALID_ARGUMENT, err);
    if (s.vec == 4 && !(aligned16 && D % 4 == 0))
        return fail(LINREC_ERR_INVALID_ARGUMENT, "vec=4 needs D % 4 == 0 and 16-byte aligned buffers");

    p = Plan{};
    p.tile = s;
    Geometry& g = p.geom;
    g.L = L;
    g.D = D;
    g.spin_limit = spin_limit();
    if (n == 0) {
        p.tiles = 0;
        p.workspace_bytes = 0;
        return LINREC_OK;
    }
    const int64_t quads = (D + s.vec - 1) / s.vec;
    int lanes = 1, log2_lanes = 0;
    while (lanes < s.p && lanes < quads) { lanes <<= 1; ++log2_lanes; }
    g.lanes_d = lanes;
    g.log2_lanes_d = log2_lanes;
    g.groups = linrec::kWave / lanes;
    g.slab_channels = lanes * s.vec;
    g.carry_waves = (g.slab_channels + linrec::kWave - 1) / linrec::kWave;
    if ((s.w + g.carry_waves) * linrec::kWave > 1024)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "the tile needs more than 1024 threads per workgroup (data waves w "
                                                 "plus one carry wave per 64 slab channels); pick a smaller w or p");
    g.nslab = static_cast<int32_t>((quads + lanes - 1) / lanes);
    g.nseq = B * g.nslab;
    g.steps_per_tile = static_cast<int64_t>(s.w) * g.groups * s.t;
    g.nchunks = (L + g.steps_per_tile - 1) / g.steps_per_tile;
    int64_t tiles = 0;
    if (!checked_mul(g.nseq, g.nchunks, tiles) || tiles > 0x7fffffffLL)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "problem needs more than 2^31 - 1 tiles; pick a larger tile (LINREC_TILE)");
    // a lane addresses its tile through a buffer descriptor with a 31-bit range
    if (g.steps_per_tile * D * 4 > linrec::kMaxRange)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "one tile's rows span more than 2 GiB; pick a smaller tile (LINREC_TILE)");
    p.tiles = tiles;
    g.ntiles = tiles;
    if (g.nchunks > 1) {
        g.nstatus = tiles * g.slab_channels;
        p.workspace_bytes = sizeof(WorkspaceHeader) + linrec::kDoneBytes +
                            3 * static_cast<size_t>(g.nstatus) * sizeof(uint64_t);
    } else {
        g.nstatus = 0;
        p.workspace_bytes = 0;
    }
    return LINREC_OK;
}

// ----------------------------------------------------------------------------- launch table

struct Launch {
    const void* kernel;   // identifies the instantiation (occupancy cache key)
    void (*run)(dim3 grid, dim3 block, const float*, const float*, float*, const Geometry&, WorkspaceHeader*,
                uint64_t*, hipStream_t);
    hipError_t (*occupancy)(int* groups_per_cu, int threads);
};

template <int VEC, int T, int W>
void run_tiles(dim3 grid, dim3 block, const float* a, const float* b, float* h, const Geometry& g,
               WorkspaceHeader* hdr, uint64_t* stat, hipStream_t stream) {
    hipLaunchKernelGGL((linrec::scan_tiles<VEC, T, W>), grid, block, 0, stream, a, b, h, g, hdr, stat);
}

template <int VEC, int T, int W>
hipError_t occupancy_of(int* groups_per_cu, int threads) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(groups_per_cu, linrec::scan_tiles<VEC, T, W>, threads, 0);
}

template <int VEC, int T, int W>
void run_one(dim3 grid, dim3 block, const float* a, const float* b, float* h, const Geometry& g,
             WorkspaceHeader* hdr, uint64_t* stat, hipStream_t stream) {
    hipLaunchKernelGGL((linrec::scan_one<VEC, T, W>), grid, block, 0, stream, a, b, h, g, hdr, stat);
}

template <int VEC, int T, int W>
hipError_t occupancy_one(int* groups_per_cu, int threads) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(groups_per_cu, linrec::scan_one<VEC, T, W>, threads, 0);
}

template <int VEC, int T, int W>
const Launch* launch_entry(int mode) {
    if (mode == 1) {
        static const Launch one{reinterpret_cast<const void*>(&linrec::scan_one<VEC, T, W>), &run_one<VEC, T, W>,
                                &occupancy_one<VEC, T, W>};
        return &one;
    }
    if constexpr (VEC == 4 && T == 16) {
        return nullptr;   // two such register buffers spill
    } else {
        static const Launch persistent{reinterpret_cast<const void*>(&linrec::scan_tiles<VEC, T, W>),
                                       &run_tiles<VEC, T, W>, &occupancy_of<VEC, T, W>};
        return &persistent;
    }
}

using LaunchFn = const Launch*;

template <int VEC, int T>
LaunchFn pick_w(int w, int m) {
    switch (w) {
        case 1: return launch_entry<VEC, T, 1>(m);
        case 2: return launch_entry<VEC, T, 2>(m);
        case 4: return launch_entry<VEC, T, 4>(m);
        case 6: return launch_entry<VEC, T, 6>(m);
        case 7: return launch_entry<VEC, T, 7>(m);
        case 8: return launch_entry<VEC, T, 8>(m);
        case 14: return launch_entry<VEC, T, 14>(m);
        case 15: return launch_entry<VEC, T, 15>(m);
        default: return nullptr;
    }
}

template <int VEC>
LaunchFn pick_t(int t, int w, int m) {
    switch (t) {
        case 4: return pick_w<VEC, 4>(w, m);
        case 8: return pick_w<VEC, 8>(w, m);
        case 16: return pick_w<VEC, 16>(w, m);
        default: return nullptr;
    }
}

LaunchFn pick_launch(const TileShape& s) {
    return s.vec == 4 ? pick_t<4>(s.t, s.w, s.m) : pick_t<1>(s.t, s.w, s.m);
}

// ----------------------------------------------------------------------------- persistent grid

// Workgroups of one kernel instantiation that fit on the device at once
// (occupancy per CU x CUs), cached per (device, instantiation).
std::mutex g_grid_mutex;
std::map<std::tuple<int, const void*, int>, int64_t> g_resident;

linrec_status resident_groups(int device, const Launch* l, int threads, int64_t& out) {
    std::lock_guard<std::mutex> lock(g_grid_mutex);
    const auto key = std::make_tuple(device, l->kernel, threads);
    auto it = g_resident.find(key);
    if (it != g_resident.end()) {
        out = it->second;
        return LINREC_OK;
    }
    int per_cu = 0, cus = 0;
    hipError_t e = l->occupancy(&per_cu, threads);
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipOccupancyMaxActiveBlocksPerMultiprocessor: " + hip_text(e));
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipDeviceGetAttribute(CU count): " + hip_text(e));
    // The occupancy query counts waves per CU; measured on gfx950, workgroups
    // whose wave count is not a multiple of the 4 SIMDs do not all fit that
    // way (a 5-wave workgroup puts 2 waves on one SIMD).  Count per SIMD
    // instead: each workgroup needs ceil(waves / 4) slots on some SIMD.
    hipFuncAttributes attr;
    e = hipFuncGetAttributes(&attr, l->kernel);
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipFuncGetAttributes: " + hip_text(e));
    const int vgprs = attr.numRegs > 0 ? (attr.numRegs + 7) / 8 * 8 : 512;
    const int waves_per_simd = std::min(8, 512 / vgprs);
    const int waves = threads / linrec::kWave;
    const int per_simd_need = (waves + 3) / 4;
    const int by_simd = std::max(1, waves_per_simd / per_simd_need);
    per_cu = std::max(1, std::min(per_cu, by_simd));
    out = static_cast<int64_t>(per_cu) * (cus < 1 ? 1 : cus);
    g_resident[key] = out;
    return LINREC_OK;
}

// ----------------------------------------------------------------------------- workspace

// The epoch in the status tags has 30 bits; clearing the workspace every 2^29
// calls keeps a stale word from ever carrying the current epoch.
constexpr uint64_t kClearPeriod = 1ull << 29;

struct DeviceWorkspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    uint64_t calls = 0;
};

std::mutex g_mutex;
std::map<int, DeviceWorkspace> g_workspaces;

linrec_status zero_fill(void* p, size_t bytes, hipStream_t stream) {
    const int64_t words = static_cast<int64_t>(bytes / sizeof(uint32_t));
    const int64_t blocks64 = (words + 255) / 256;
    const unsigned blocks = static_cast<unsigned>(blocks64 < 4096 ? (blocks64 < 1 ? 1 : blocks64) : 4096);
    hipLaunchKernelGGL(linrec::fill_zero_u32, dim3(blocks), dim3(256), 0, stream, static_cast<uint32_t*>(p), words);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "workspace clear failed: " + hip_text(e));
    return LINREC_OK;
}

// Returns the device workspace of at least `need` bytes, allocating or growing it.
linrec_status acquire_workspace(int device, size_t need, hipStream_t stream, void*& out) {
    std::lock_guard<std::mutex> lock(g_mutex);
    DeviceWorkspace& ws = g_workspaces[device];
    if (ws.bytes < need) {
        if (ws.ptr != nullptr) {
            // the old workspace may still be in use by enqueued work
            hipError_t e = hipDeviceSynchronize();
            if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipDeviceSynchronize before growing the workspace: " + hip_text(e));
            e = hipFree(ws.ptr);
            ws = DeviceWorkspace{};
            if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipFree of the old workspace: " + hip_text(e));
        }
        const size_t mib = size_t(1) << 20;
        const size_t bytes = (need + need / 4 + mib - 1) / mib * mib;
        void* p = nullptr;
        hipError_t e = hipMalloc(&p, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(LINREC_ERR_OUT_OF_MEMORY, "hipMalloc of " + std::to_string(bytes) + " workspace bytes: " + hip_text(e));
        }
        e = hipMemset(p, 0, bytes);
        if (e != hipSuccess) {
            (void)hipFree(p);
            return fail(LINREC_ERR_HIP, "clearing the new workspace: " + hip_text(e));
        }
        ws.ptr = p;
        ws.bytes = bytes;
        ws.calls = 0;
    }
    ws.calls += 1;
    if (ws.calls % kClearPeriod == 0) {
        const linrec_status s = zero_fill(ws.ptr, ws.bytes, stream);
        if (s != LINREC_OK) return s;
    }
    out = ws.ptr;
    return LINREC_OK;
}

// ----------------------------------------------------------------------------- argument checks

linrec_status check_buffer(const void* p, size_t bytes, int device, const char* name) {
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(LINREC_ERR_INVALID_ARGUMENT, std::string(name) + " is not memory known to HIP (" + hip_text(e) + ")");
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return fail(LINREC_ERR_INVALID_ARGUMENT, std::string(name) + " is not device memory");
    if (attr.type == hipMemoryTypeDevice && attr.device != device)
        return fail(LINREC_ERR_INVALID_ARGUMENT, std::string(name) + " lives on device " + std::to_string(attr.device) +
                                                     ", the current device is " + std::to_string(device));
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(LINREC_ERR_INVALID_ARGUMENT, std::string(name) + ": allocation range unknown (" + hip_text(e) + ")");
    }
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base);
    const uintptr_t at = reinterpret_cast<uintptr_t>(p);
    if (at < lo || at - lo > size || size - (at - lo) < bytes)
        return fail(LINREC_ERR_INVALID_ARGUMENT, std::string(name) + " holds fewer than B*L*D floats");
    return LINREC_OK;
}

bool overlaps(const void* x, const void* y, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return a < b + bytes && b < a + bytes;
}

}  // namespace

// ============================================================================= C ABI

extern "C" {

linrec_status linrec_scan_plan(int64_t B, int64_t L, int64_t D, int aligned16, linrec_plan* plan) {
    if (plan == nullptr) return fail(LINREC_ERR_INVALID_ARGUMENT, "plan is null");
    Plan p;
    const linrec_status s = make_plan(B, L, D, aligned16 != 0, p);
    if (s != LINREC_OK) return s;
    plan->vec = p.tile.vec;
    plan->steps_per_lane = p.tile.t;
    plan->waves = p.tile.w;
    plan->lanes_per_row = p.tiles ? p.geom.lanes_d : 0;
    plan->steps_per_tile = p.tiles ? p.geom.steps_per_tile : 0;
    plan->chunks = p.tiles ? p.geom.nchunks : 0;
    plan->tiles = p.tiles;
    plan->workspace_bytes = p.workspace_bytes;
    plan->mode = p.tile.m;
    return LINREC_OK;
}

linrec_status linrec_scan(const float* a, const float* b, float* h, int64_t B, int64_t L, int64_t D, void* stream) {
    t_last_error.clear();
    if (B < 0 || L < 0 || D < 0) return fail(LINREC_ERR_INVALID_ARGUMENT, "B, L and D must be >= 0");
    if (B == 0 || L == 0 || D == 0) return LINREC_OK;
    if (a == nullptr || b == nullptr || h == nullptr)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "a, b and h must be non-null when B*L*D > 0");

    const bool aligned16 = ((reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                             reinterpret_cast<uintptr_t>(h)) & 15u) == 0;
    Plan p;
    linrec_status s = make_plan(B, L, D, aligned16, p);
    if (s != LINREC_OK) return s;
    const size_t bytes = static_cast<size_t>(B * L * D) * sizeof(float);
    if (overlaps(h, a, bytes) || overlaps(h, b, bytes))
        return fail(LINREC_ERR_OVERLAP, "h overlaps a or b");

    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipGetDevice: " + hip_text(e));
    if ((s = check_buffer(a, bytes, device, "a")) != LINREC_OK) return s;
    if ((s = check_buffer(b, bytes, device, "b")) != LINREC_OK) return s;
    if ((s = check_buffer(h, bytes, device, "h")) != LINREC_OK) return s;

    const hipStream_t hs = static_cast<hipStream_t>(stream);
    void* ws = nullptr;
    if (p.workspace_bytes > 0) {
        s = acquire_workspace(device, p.workspace_bytes, hs, ws);
        if (s != LINREC_OK) return s;
    }
    WorkspaceHeader* hdr = static_cast<WorkspaceHeader*>(ws);
    uint64_t* stat = ws ? reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + sizeof(WorkspaceHeader) +
                                                      linrec::kDoneBytes)
                        : nullptr;

    const LaunchFn fn = pick_launch(p.tile);
    if (fn == nullptr) return fail(LINREC_ERR_INVALID_ARGUMENT, "no kernel for the chosen tile");
    if (p.tile.m == 1) {
        // one tile per workgroup; the hardware keeps as many resident as fit
        (void)hipGetLastError();
        fn->run(dim3(static_cast<uint32_t>(p.tiles)), dim3((p.tile.w + p.geom.carry_waves) * linrec::kWave), a, b, h,
                p.geom, hdr, stat, hs);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(LINREC_ERR_HIP, "kernel launch: " + hip_text(e));
        return LINREC_OK;
    }
    const int threads = (p.tile.w + p.geom.carry_waves) * linrec::kWave;
    int64_t resident = 0;
    if ((s = resident_groups(device, fn, threads, resident)) != LINREC_OK) return s;
    // persistent workgroups: as many as fit at once (or fewer, per LINREC_TILE's
    // q = workgroups per CU), never more than there are tiles
    int64_t groups = resident;
    if (p.tile.q > 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) == hipSuccess && cus > 0)
            groups = std::min<int64_t>(resident, static_cast<int64_t>(p.tile.q) * cus);
    }
    groups = std::min<int64_t>(groups, p.tiles);
    (void)hipGetLastError();
    fn->run(dim3(static_cast<uint32_t>(groups)), dim3(threads), a, b, h, p.geom, hdr, stat, hs);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "kernel launch: " + hip_text(e));
    return LINREC_OK;
}

const char* linrec_status_string(int status) {
    switch (status) {
        case LINREC_OK: return "success";
        case LINREC_ERR_INVALID_ARGUMENT: return "invalid argument";
        case LINREC_ERR_OVERLAP: return "output overlaps an input";
        case LINREC_ERR_HIP: return "HIP runtime error";
        case LINREC_ERR_OUT_OF_MEMORY: return "out of device memory";
        default: return "unknown status";
    }
}

const char* linrec_last_error_message(void) { return t_last_error.c_str(); }

linrec_status linrec_device_timeouts(uint64_t* count) {
    if (count == nullptr) return fail(LINREC_ERR_INVALID_ARGUMENT, "count is null");
    *count = 0;
    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipGetDevice: " + hip_text(e));
    void* ptr = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        auto it = g_workspaces.find(device);
        if (it != g_workspaces.end()) ptr = it->second.ptr;
    }
    if (ptr == nullptr) return LINREC_OK;
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipDeviceSynchronize: " + hip_text(e));
    WorkspaceHeader hdr;
    e = hipMemcpy(&hdr, ptr, sizeof(hdr), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "reading the workspace header: " + hip_text(e));
    *count = hdr.timeouts;
    return LINREC_OK;
}

void linrec_release(void) {
    std::lock_guard<std::mutex> lock(g_mutex);
    int current = 0;
    const bool have_current = hipGetDevice(&current) == hipSuccess;
    for (auto& kv : g_workspaces) {
        if (kv.second.ptr == nullptr) continue;
        if (hipSetDevice(kv.first) == hipSuccess) {
            (void)hipDeviceSynchronize();
            (void)hipFree(kv.second.ptr);
        }
    }
    g_workspaces.clear();
    if (have_current) (void)hipSetDevice(current);
    (void)hipGetLastError();
}

}  // extern "C"
