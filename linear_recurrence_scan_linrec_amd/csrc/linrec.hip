// linrec.hip -- host side of the C ABI in include/linrec.h: argument checks,
// tile choice, the per-device lookback workspace and the kernel launch.
//
// The operation and its evaluation order are described in scan_kernel.hpp and
// in the header; this file holds no arithmetic of the recurrence.  The kernel
// instances live in kernels_f32.hip, kernels_bf16.hip and kernels_f16.hip.
#include "linrec.h"
#include "launch.hpp"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <utility>
#include <vector>

// Zero-fill used to (re)initialise a workspace; a kernel rather than a memset
// so that it can sit inside captured graphs.
__global__ void linrec_fill_zero_u32(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t k = i; k < n; k += step) p[k] = 0u;
}

// A scan over zero positions leaves the state unchanged: h_final = h_init (or 0).
__global__ void linrec_pass_state(const float* __restrict__ h_init, float* __restrict__ h_final, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t k = i; k < n; k += step) h_final[k] = h_init != nullptr ? h_init[k] : 0.0f;
}

namespace {

using linrec::Geometry;
using linrec::WorkspaceHeader;
using linrec_host::Launch;
using linrec_host::TileShape;
using linrec_host::tile_supported;

thread_local std::string t_last_error;

linrec_status fail(linrec_status s, const std::string& msg) {
    t_last_error = msg;
    return s;
}

std::string hip_text(hipError_t e) { return std::string(hipGetErrorName(e)) + ": " + hipGetErrorString(e); }

// ----------------------------------------------------------------------------- tile shapes

// CUs assumed by the plan entry points, which make no HIP call (MI355X).
constexpr int kPlanCus = 256;

// Lanes per row segment that make_plan derives from a requested p: the
// smallest power of two that is >= min(p, channel groups per row).
int64_t lanes_for(int p, int64_t quads) {
    int64_t lanes = 1;
    while (lanes < p && lanes < quads) lanes <<= 1;
    return lanes;
}

// Tile choice, from sweeps on MI355X over the five workloads.
//  - When some slab width gives every CU a (batch row, channel slab) sequence
//    of its own (1..kMaxLocalSeqs per workgroup), persistent workgroups keep
//    the carry local: no status words and no cross-workgroup wait.  The widest
//    such slab up to 32 lanes is taken (wider row segments stream better, but
//    64-lane slabs need four carry waves and measured slower); 8 positions per
//    lane.  Slabs of at most 64 channels go to the relay (m=2) over tiles of
//    64 positions: the carry wave does the group scan one tile behind, and
//    these short tiles walk memory faster than the 128-position tiles the
//    group scan needs to stay hidden (B=32 L=4096 D=256: 72-74 us against
//    74.5-76.5 us for 2 data waves x 128 positions with the group scan in the
//    data waves; B=8 L=16384 D=1024: 270 against 296 us, medians).  Wider
//    slabs keep 2 data waves when a wave covers 8 or more row segments, else
//    4 (B=16 L=512 D=8192: 32-lane slabs, 131-134 us against 146 us with 64
//    lanes; the relay with its 2 carry waves took 161 us there).  Looking
//    back instead took 82.5 us at B=32 L=4096 D=256.
//  - Otherwise the tiles look back: persistent workgroups of 8 data waves, 4
//    positions per lane and 32 lanes (512 bytes of fp32) per row segment; with
//    fewer than 32 sequences each chain is long, and one workgroup per tile
//    keeps more tiles in flight along each chain: 7 data waves and a carry
//    wave, 8 positions per lane, 8-lane slabs (B=2 L=262144 D=64: 79 us).
//    Two such 8-wave workgroups share a CU within the register file (about
//    100 VGPRs each), so one tile's loads run while another waits for its
//    carry; 16-wave workgroups of 15 data waves took 102 us once the carry's
//    products of decays became fp64 (70 VGPRs: one workgroup per CU).
//  With 16-bit storage and 4 channels per lane, a lane's loads are 8 bytes,
//  so narrow slabs give short row segments and the pipeline does not shorten
//  with the bytes; these plans stream more per tile instead: 8 positions per
//  lane and 8 data waves with a local carry over 64- or 32-lane slabs when
//  possible; else one workgroup per tile of 7 data waves x 16 positions over
//  16-lane slabs (the values stay packed in registers, so 16 positions cost
//  what 8 cost in fp32) while that makes at most 16 tiles per CU; else 32-lane
//  slabs looking back.  (bf16: B=32 L=4096 D=256 44 us, B=2 L=262144 D=64 51 us,
//  B=8 L=16384 D=1024 177 us, B=16 L=512 D=8192 73 us.)
TileShape default_tile(int64_t B, int64_t L, int64_t D, bool vec4, int cus, int es) {
    const int vec = vec4 ? 4 : 1;
    const double n = static_cast<double>(B) * static_cast<double>(L) * static_cast<double>(D);
    if (n <= 65536.0) return TileShape{vec, 4, 1, 64, 0, 0, 1};
    const int64_t quads = (D + vec - 1) / vec;
    if (es == 2 && vec == 4) {
        auto seqs = [&](int p) { return B * ((quads + lanes_for(p, quads) - 1) / lanes_for(p, quads)); };
        auto local = [&](int p) {
            for (int m = 1; m <= linrec::kMaxLocalSeqs; ++m)
                if (seqs(p) % m == 0 && seqs(p) / m >= cus) return true;
            return false;
        };
        for (int p = 64; p >= 32; p >>= 1)
            if (local(p)) return TileShape{vec, 8, 8, p, 0, 0, 1};
        // one tile per workgroup (7 waves x 16 steps over 16-lane slabs, packed 16-bit
        // registers) while that makes at most 16 tiles per CU, or when there are too few
        // sequences for persistent lookback; beyond that its one lookback per workgroup
        // costs more than the persistent plan's
        const int64_t lanes16 = lanes_for(16, quads);
        const int64_t steps16 = int64_t{16} * (64 / lanes16) * 7;
        const int64_t tiles16 = seqs(16) * ((L + steps16 - 1) / steps16);
        if (tiles16 <= int64_t{16} * cus || seqs(32) < 32) return TileShape{vec, 16, 7, 16, 0, 1, 1};
        return TileShape{vec, 8, 8, 32, 0, 0, 1};
    }
    for (int p = 32; p >= 8; p >>= 1) {
        const int64_t lanes = lanes_for(p, quads);
        const int64_t nseq = B * ((quads + lanes - 1) / lanes);
        bool local = false;
        for (int m = 1; m <= linrec::kMaxLocalSeqs && !local; ++m) local = nseq % m == 0 && nseq / m >= cus;
        // the relay when the sequences come to 1 to 4 per CU, so that its
        // grid is one workgroup per CU, the grid it was measured with: tiles
        // of 64 positions, 1 data wave for 8-lane slabs, 2 for 16-lane ones
        if (local && lanes * vec <= 64 && nseq % cus == 0 && nseq / cus <= linrec::kMaxLocalSeqs) {
            const int64_t groups = 64 / lanes;
            const int w = groups >= 8 ? 1 : 2;
            if (L > w * groups * 8) return TileShape{vec, 8, w, p, 0, 2, 1};
        }
        const int w = 64 / lanes >= 8 ? 2 : 4;
        const int64_t steps = static_cast<int64_t>(w) * (64 / lanes) * 8;
        if (local && L > steps) return TileShape{vec, 8, w, p, 0, 0, 1};
    }
    TileShape s{vec, 4, 8, 32, 0, 0, 1};
    const int64_t lanes = std::min<int64_t>(32, quads);
    const int64_t sequences = B * ((D + vec * lanes - 1) / (vec * lanes));
    if (sequences < 32) {
        s.m = 1;
        s.t = 8;
        s.w = 7;
        s.p = 32 / vec;
    }
    return s;
}

// LINREC_TILE="t=16,w=4,vec=4,p=64,q=2,m=0,l=1,x=1" (any subset of the keys).
bool apply_tile_env(TileShape& s, int es, std::string& err) {
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
        else if (key == "l") s.l = static_cast<int>(val);
        else if (key == "x") s.x = static_cast<int>(val);
        else {
            err = "LINREC_TILE key '" + key + "' is not one of t, w, vec, p, q, m, l, x";
            return false;
        }
        pos = end + 1;
    }
    if (!tile_supported(s, es)) {
        err = "LINREC_TILE asks for an unsupported tile (t in {4,8,16}, w in {1,2,4,7,8,15}, vec in {1,4}, "
              "p a power of two <= 64, q in [0, 64], m in {0,1,2}, l in {0,1}, x in {0,1}; with r register bytes "
              "per channel and position (2 for 16-bit storage with vec=4, else 4): vec*t*r <= 128 for m=0 and m=2 "
              "and <= 64 for w=15)";
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

// ----------------------------------------------------------------------------- the problem

bool checked_mul(int64_t x, int64_t y, int64_t& out) {
    if (x == 0 || y == 0) { out = 0; return true; }
    if (x < 0 || y < 0 || x > INT64_MAX / y) return false;
    out = x * y;
    return true;
}

bool checked_add(int64_t x, int64_t y, int64_t& out) {
    if (x < 0 || y < 0 || x > INT64_MAX - y) return false;
    out = x + y;
    return true;
}

int element_bytes(int32_t dtype) { return dtype == LINREC_F32 ? 4 : 2; }

// Bytes from an operand's first element to one past the last element its
// strides reach (0 for an empty problem); false on overflow.
bool operand_extent(const linrec_operand& o, int64_t B, int64_t L, int64_t D, int es, int64_t& bytes) {
    if (B == 0 || L == 0 || D == 0) { bytes = 0; return true; }
    int64_t rb = 0, rl = 0, last = 0, n = 0;
    return checked_mul(B - 1, o.stride_b, rb) && checked_mul(L - 1, o.stride_l, rl) && checked_add(rb, rl, last) &&
           checked_add(last, D, n) && checked_mul(n, es, bytes);
}

// h's rows (i, t) of D elements are pairwise disjoint: taking the batch and
// time dimensions in increasing stride, each stride must clear everything the
// smaller ones span.
bool rows_disjoint(const linrec_operand& h, int64_t B, int64_t L, int64_t D) {
    struct Dim { int64_t stride, count; };
    Dim dims[2] = {{h.stride_b, B}, {h.stride_l, L}};
    if (dims[1].stride < dims[0].stride) std::swap(dims[0], dims[1]);
    int64_t span = D;   // elements spanned by one row and the smaller dimensions so far
    for (const Dim& d : dims) {
        if (d.count <= 1) continue;
        if (d.stride < span) return false;
        int64_t reach = 0;
        if (!checked_mul(d.count - 1, d.stride, reach) || !checked_add(reach, span, span)) return false;
    }
    return true;
}

struct Problem {
    linrec_scan_desc desc;   // strides normalised: unused ones set to harmless values
    int es;                  // bytes per element
    int64_t extent_a, extent_b, extent_h;
    bool vec4;               // 4-channel accesses possible
};

linrec_status make_problem(const linrec_scan_desc* d, Problem& p) {
    if (d == nullptr) return fail(LINREC_ERR_INVALID_ARGUMENT, "desc is null");
    p.desc = *d;
    linrec_scan_desc& q = p.desc;
    if (q.B < 0 || q.L < 0 || q.D < 0) return fail(LINREC_ERR_INVALID_ARGUMENT, "B, L and D must be >= 0");
    if (q.dtype != LINREC_F32 && q.dtype != LINREC_BF16 && q.dtype != LINREC_F16)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "dtype must be LINREC_F32, LINREC_BF16 or LINREC_F16");
    if (q.reverse < 0 || q.reverse > 2) return fail(LINREC_ERR_INVALID_ARGUMENT, "reverse must be 0, 1 or 2");
    linrec_operand* ops[3] = {&q.a, &q.b, &q.h};
    for (linrec_operand* o : ops)
        if (o->stride_b < 0 || o->stride_l < 0) return fail(LINREC_ERR_INVALID_ARGUMENT, "strides must be >= 0");
    // a stride along a dimension of extent 1 is never used; normalise it so
    // that the kernels' range arithmetic holds (time strides of h >= D)
    for (linrec_operand* o : ops) {
        if (q.B <= 1) o->stride_b = 0;
        if (q.L <= 1) o->stride_l = q.D;
    }
    p.es = element_bytes(q.dtype);
    int64_t n = 0, bl = 0;
    if (!checked_mul(q.B, q.L, bl) || !checked_mul(bl, q.D, n) || n > INT64_MAX / 8)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "B*L*D elements overflow (B*L*D*8 must fit in 63 bits)");
    if (!operand_extent(q.a, q.B, q.L, q.D, p.es, p.extent_a) || !operand_extent(q.b, q.B, q.L, q.D, p.es, p.extent_b) ||
        !operand_extent(q.h, q.B, q.L, q.D, p.es, p.extent_h))
        return fail(LINREC_ERR_INVALID_ARGUMENT, "an operand's strides reach beyond 2^63 bytes");
    if (n > 0 && !rows_disjoint(q.h, q.B, q.L, q.D))
        return fail(LINREC_ERR_INVALID_ARGUMENT, "the strides of h make rows (i, t) overlap one another");
    for (linrec_operand* o : ops)
        if (reinterpret_cast<uintptr_t>(o->ptr) % static_cast<uintptr_t>(p.es) != 0)
            return fail(LINREC_ERR_INVALID_ARGUMENT, "a, b and h must be aligned to their element size");
    if (reinterpret_cast<uintptr_t>(q.h_init) % alignof(float) != 0 ||
        reinterpret_cast<uintptr_t>(q.h_final) % alignof(float) != 0)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "h_init and h_final must be aligned to 4 bytes");
    const uintptr_t align = static_cast<uintptr_t>(4 * p.es) - 1;
    bool vec4 = q.D % 4 == 0;
    for (linrec_operand* o : ops)
        vec4 = vec4 && (reinterpret_cast<uintptr_t>(o->ptr) & align) == 0 && o->stride_b % 4 == 0 &&
               o->stride_l % 4 == 0;
    p.vec4 = vec4;
    return LINREC_OK;
}

struct Plan {
    TileShape tile;
    Geometry geom;
    int64_t tiles;
    size_t workspace_bytes;
};

linrec_status make_plan(const Problem& pr, Plan& p, int cus) {
    const linrec_scan_desc& q = pr.desc;
    TileShape s = default_tile(q.B, q.L, q.D, pr.vec4, cus, pr.es);
    if (!tile_supported(s, pr.es)) return fail(LINREC_ERR_INVALID_ARGUMENT, "internal: default tile not supported");
    std::string err;
    if (!apply_tile_env(s, pr.es, err)) return fail(LINREC_ERR_INVALID_ARGUMENT, err);
    if (s.vec == 4 && !pr.vec4)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "vec=4 needs D % 4 == 0, strides that are multiples of 4 and "
                                                 "operands aligned to 4 elements");

    p = Plan{};
    p.tile = s;
    Geometry& g = p.geom;
    g.L = q.L;
    g.D = q.D;
    g.a_sb = q.a.stride_b; g.a_sl = q.a.stride_l;
    g.b_sb = q.b.stride_b; g.b_sl = q.b.stride_l;
    g.h_sb = q.h.stride_b; g.h_sl = q.h.stride_l;
    g.h_init = q.h_init;
    g.h_final = q.h_final;
    g.reverse = q.reverse != 0 ? 1 : 0;   // 2: reverse, with the decays one time step ahead
    g.spin_limit = spin_limit();
    if (q.B == 0 || q.L == 0 || q.D == 0) {
        p.tiles = 0;
        p.workspace_bytes = 0;
        return LINREC_OK;
    }
    const int64_t quads = (q.D + s.vec - 1) / s.vec;
    const int lanes = static_cast<int>(lanes_for(s.p, quads));
    int log2_lanes = 0;
    while ((1 << log2_lanes) < lanes) ++log2_lanes;
    g.lanes_d = lanes;
    g.log2_lanes_d = log2_lanes;
    g.groups = linrec::kWave / lanes;
    g.slab_channels = lanes * s.vec;
    g.carry_waves = (g.slab_channels + linrec::kWave - 1) / linrec::kWave;
    // the relay has one carry wave and at most 2 data waves; other shapes of
    // m=2 run as m=0
    if (s.m == 2 && (s.w > 2 || g.carry_waves > 1)) s.m = p.tile.m = 0;
    if ((s.w + g.carry_waves) * linrec::kWave > 1024)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "the tile needs more than 1024 threads per workgroup (data waves w "
                                                 "plus one carry wave per 64 slab channels); pick a smaller w or p");
    g.nslab = static_cast<int32_t>((quads + lanes - 1) / lanes);
    g.nseq = q.B * g.nslab;
    // slab rows narrower than a 128-byte line: the slabs of one line go to one
    // XCD (see sequence_of) when whole lines of slabs fit in each batch row
    // and the sequences fill whole blocks of 8 lines' slabs
    g.line_shift = 0;
    const int64_t row_bytes = static_cast<int64_t>(g.slab_channels) * pr.es;
    if (s.x == 1 && row_bytes < 128 && 128 % row_bytes == 0) {
        const int64_t per_line = 128 / row_bytes;
        if (g.nslab % per_line == 0 && g.nseq % (8 * per_line) == 0)
            while ((int64_t{1} << g.line_shift) < per_line) ++g.line_shift;
    }
    g.steps_per_tile = static_cast<int64_t>(s.w) * g.groups * s.t;
    g.nchunks = (q.L + g.steps_per_tile - 1) / g.steps_per_tile;
    int64_t tiles = 0;
    if (!checked_mul(g.nseq, g.nchunks, tiles) || tiles > 0x7fffffffLL)
        return fail(LINREC_ERR_INVALID_ARGUMENT, "problem needs more than 2^31 - 1 tiles; pick a larger tile (LINREC_TILE)");
    // a lane addresses its tile of each operand through a buffer descriptor
    // with 32-bit offsets; out-of-range offsets stay out of range only while a
    // tile spans less than kMaxTileBytes
    for (const linrec_operand* o : {&q.a, &q.b, &q.h}) {
        int64_t reach = 0, bytes = 0;
        if (!checked_mul(g.steps_per_tile, o->stride_l, reach) || !checked_add(reach, q.D, reach) ||
            !checked_mul(reach, pr.es, bytes) || bytes >= linrec::kMaxTileBytes)
            return fail(LINREC_ERR_INVALID_ARGUMENT, "one tile of an operand spans 1 GiB or more; pick a smaller "
                                                     "tile (LINREC_TILE)");
    }
    p.tiles = tiles;
    g.ntiles = tiles;
    // lookback window: the wider long-chain window (3 predecessors per round
    // trip in fp32, 4 in 16 bits) only for one tile per workgroup over long
    // chains, else 2 (see lookback_channel)
    g.lookback_window = (s.m == 1 && g.nchunks > 64) ? 4 : 2;
    if (g.nchunks > 1) {
        g.nstatus = tiles * g.slab_channels;
        p.workspace_bytes = sizeof(WorkspaceHeader) + linrec::kDoneBytes +
                            linrec::kStatusArrays * static_cast<size_t>(g.nstatus) * sizeof(uint64_t);
    } else {
        g.nstatus = 0;
        p.workspace_bytes = 0;
    }
    return LINREC_OK;
}

void fill_plan(const Plan& p, linrec_plan* plan) {
    plan->vec = p.tile.vec;
    plan->steps_per_lane = p.tile.t;
    plan->waves = p.tile.w;
    plan->lanes_per_row = p.tiles ? p.geom.lanes_d : 0;
    plan->steps_per_tile = p.tiles ? p.geom.steps_per_tile : 0;
    plan->chunks = p.tiles ? p.geom.nchunks : 0;
    plan->tiles = p.tiles;
    plan->workspace_bytes = p.workspace_bytes;
    plan->mode = p.tile.m;
}

// Grid of persistent workgroups that keeps the carry local, filling in
// p.geom.local_seqs, or 0 (local_seqs = 0: the tiles look back).  The grid
// must divide the (batch row, channel slab) sequences into at most
// kMaxLocalSeqs per workgroup: workgroup k then takes tiles k, k + grid, ...,
// which are chunks 0, 1, ... of its own sequences in order, so the state
// entering each tile is the one its previous tile of that sequence left.  Of
// the grids with at least one workgroup per CU that fit at once, the smallest
// is taken (exactly q per CU when LINREC_TILE sets q).  Not with l=0, nor
// with one chunk per sequence (nothing to carry).
int64_t local_grid(Plan& p, int64_t resident, int cus) {
    Geometry& g = p.geom;
    g.local_seqs = 0;
    if (p.tile.l == 0 || g.nchunks <= 1) return 0;
    const int64_t want = p.tile.q > 0 ? static_cast<int64_t>(p.tile.q) * cus : 0;
    for (int m = linrec::kMaxLocalSeqs; m >= 1; --m) {
        if (g.nseq % m != 0) continue;
        const int64_t grid = g.nseq / m;
        if (grid < cus || grid > resident || (want > 0 && grid != want)) continue;
        g.local_seqs = m;
        return grid;
    }
    return 0;
}

const Launch* pick_launch(int32_t dtype, const TileShape& s, bool ahead) {
    switch (dtype) {
        case LINREC_F32: return linrec_host::pick_launch_f32(s, ahead);
        case LINREC_BF16: return linrec_host::pick_launch_bf16(s, ahead);
        case LINREC_F16: return linrec_host::pick_launch_f16(s, ahead);
        default: return nullptr;
    }
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

// The epoch in the status tags has 30 bits; clearing a workspace every 2^29
// calls keeps a stale word from ever carrying the current epoch.
constexpr uint64_t kClearPeriod = 1ull << 29;
// Alignment asked of a caller's workspace (its header and slot lines are
// 128-byte lines; the status words are 64-bit atomics).
constexpr uintptr_t kWorkspaceAlign = 256;

struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    uint64_t calls = 0;
};

// Library-owned workspaces, one per (device, stream): calls on one stream are
// ordered, which the in-kernel epoch advance relies on, and calls on
// different streams never share status words.  A workspace that a larger
// shape outgrows is retired, not freed: graphs captured with it may still be
// replayed, and work enqueued with it may still be running.  linrec_release
// frees both kinds.
std::mutex g_mutex;
std::map<std::pair<int, void*>, Workspace> g_workspaces;
std::vector<std::pair<int, void*>> g_retired;   // (device, pointer)
// calls per caller-provided workspace, for the periodic clear
std::map<std::pair<int, void*>, uint64_t> g_caller_calls;

unsigned grid_for(int64_t n) {
    const int64_t blocks = (n + 255) / 256;
    return static_cast<unsigned>(blocks < 1 ? 1 : (blocks > 4096 ? 4096 : blocks));
}

linrec_status zero_fill(void* p, size_t bytes, hipStream_t stream) {
    const int64_t words = static_cast<int64_t>(bytes / sizeof(uint32_t));
    hipLaunchKernelGGL(linrec_fill_zero_u32, dim3(grid_for(words)), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                       words);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "workspace clear failed: " + hip_text(e));
    return LINREC_OK;
}

// True when `stream` is being captured into a graph (then nothing may be allocated).
bool capturing(hipStream_t stream) {
    hipStreamCaptureStatus status = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &status) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return status != hipStreamCaptureStatusNone;
}

// The library's workspace of `stream` on `device`, at least `need` bytes:
// allocated (and cleared) on first need, replaced by a larger one when a shape
// needs more.
linrec_status acquire_workspace(int device, size_t need, hipStream_t stream, void*& out) {
    std::lock_guard<std::mutex> lock(g_mutex);
    Workspace& ws = g_workspaces[std::make_pair(device, static_cast<void*>(stream))];
    if (ws.bytes < need) {
        if (capturing(stream))
            return fail(LINREC_ERR_INVALID_ARGUMENT,
                        "the call needs a lookback workspace of " + std::to_string(need) +
                            " bytes on this stream and the stream is being captured, where nothing may be "
                            "allocated: make one call of this or a larger shape on the stream before capturing, "
                            "or pass a workspace (linrec_scan_ws / linrec_scan_ex_ws)");
        const size_t mib = size_t(1) << 20;
        const size_t bytes = (need + need / 4 + mib - 1) / mib * mib;
        void* p = nullptr;
        hipError_t e = hipMalloc(&p, bytes);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(LINREC_ERR_OUT_OF_MEMORY, "hipMalloc of " + std::to_string(bytes) + " workspace bytes: " + hip_text(e));
        }
        // cleared on the call's stream, so the clear is ordered before the
        // scan: a hipMemset would run on the null stream, which work on a
        // non-blocking stream (torch's side streams) does not wait for, and
        // the first scan could then read uncleared slot lines
        const linrec_status cleared = zero_fill(p, bytes, stream);
        if (cleared != LINREC_OK) {
            (void)hipFree(p);
            return cleared;
        }
        if (ws.ptr != nullptr) g_retired.emplace_back(device, ws.ptr);
        ws = Workspace{p, bytes, 0};
    }
    ws.calls += 1;
    if (ws.calls % kClearPeriod == 0) {
        const linrec_status s = zero_fill(ws.ptr, ws.bytes, stream);
        if (s != LINREC_OK) return s;
    }
    out = ws.ptr;
    return LINREC_OK;
}

// ----------------------------------------------------------------------------- static scratch

// The lookback workspace of linrec_scan_ex_noalloc: a file-scope device array,
// so that entry point never allocates.  Each device the library runs on holds
// its own copy from module load to process end.  In host code `scratch` only
// names the symbol: its device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is used.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct ScratchState {
    void* ptr = nullptr;   // device address of `scratch` on this device
    bool cleared = false;  // an eager clear has been enqueued
    uint64_t calls = 0;
};
std::map<int, ScratchState> g_scratch;   // per device, under g_mutex

// The device address of this device's scratch, cleared before its first use:
// the clear is a fill kernel on the call's stream.  When that call is being
// captured the clear is recorded in the graph (each replay then starts from a
// clean scratch) and the next eager call clears it again.
linrec_status scratch_for(int device, hipStream_t stream, void*& out) {
    std::lock_guard<std::mutex> lock(g_mutex);
    ScratchState& st = g_scratch[device];
    if (st.ptr == nullptr) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return fail(LINREC_ERR_HIP, "hipGetSymbolAddress(scratch): " + hip_text(e));
        }
        st.ptr = p;
    }
    st.calls += 1;
    const bool eager = !capturing(stream);
    if (!st.cleared || st.calls % kClearPeriod == 0) {
        const linrec_status s = zero_fill(st.ptr, kScratchBytes, stream);
        if (s != LINREC_OK) return s;
        if (eager) st.cleared = true;
    }
    out = st.ptr;
    return LINREC_OK;
}

// A caller's workspace: counted for the periodic clear, which this call then
// enqueues on `stream` (never allocated or freed here).
linrec_status use_caller_workspace(int device, void* ptr, size_t bytes, hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_mutex);
    uint64_t& calls = g_caller_calls[std::make_pair(device, ptr)];
    calls += 1;
    if (calls % kClearPeriod == 0) return zero_fill(ptr, bytes, stream);
    return LINREC_OK;
}

// ----------------------------------------------------------------------------- argument checks

linrec_status check_buffer(const void* p, int64_t bytes, int device, const char* name) {
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
    if (at < lo || at - lo > size || size - (at - lo) < static_cast<size_t>(bytes))
        return fail(LINREC_ERR_INVALID_ARGUMENT, std::string(name) + " reaches beyond its allocation");
    return LINREC_OK;
}

bool overlaps(const void* x, int64_t xbytes, const void* y, int64_t ybytes) {
    if (x == nullptr || y == nullptr || xbytes == 0 || ybytes == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(x), b = reinterpret_cast<uintptr_t>(y);
    return a < b + static_cast<uintptr_t>(ybytes) && b < a + static_cast<uintptr_t>(xbytes);
}

// Where a call's lookback workspace comes from.
struct WorkspaceSource {
    bool caller = false;   // true: the caller's (ptr, bytes), possibly null; false: the library's own
    void* ptr = nullptr;
    size_t bytes = 0;
    bool scratch = false;  // true: the device's static scratch (linrec_scan_ex_noalloc)
};

linrec_status run_scan(const Problem& pr, void* stream, const WorkspaceSource& src = WorkspaceSource{}) {
    const linrec_scan_desc& q = pr.desc;
    const int64_t states = q.B * q.D;
    const int64_t state_bytes = states * static_cast<int64_t>(sizeof(float));
    const bool empty = q.B == 0 || q.L == 0 || q.D == 0;
    if (empty && (states == 0 || q.h_final == nullptr)) return LINREC_OK;
    if (!empty && (q.a.ptr == nullptr || q.b.ptr == nullptr || q.h.ptr == nullptr))
        return fail(LINREC_ERR_INVALID_ARGUMENT, "a, b and h must be non-null when B*L*D > 0");
    // written buffers overlap nothing else; a, b and h_init may overlap each other
    if (overlaps(q.h.ptr, pr.extent_h, q.a.ptr, pr.extent_a) || overlaps(q.h.ptr, pr.extent_h, q.b.ptr, pr.extent_b))
        return fail(LINREC_ERR_OVERLAP, "h overlaps a or b");
    if (overlaps(q.h_init, state_bytes, q.h.ptr, pr.extent_h))
        return fail(LINREC_ERR_OVERLAP, "h_init overlaps h");
    if (overlaps(q.h_final, state_bytes, q.a.ptr, pr.extent_a) || overlaps(q.h_final, state_bytes, q.b.ptr, pr.extent_b) ||
        overlaps(q.h_final, state_bytes, q.h.ptr, pr.extent_h) || overlaps(q.h_final, state_bytes, q.h_init, state_bytes))
        return fail(LINREC_ERR_OVERLAP, "h_final overlaps another buffer");

    int device = 0;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipGetDevice: " + hip_text(e));
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess || cus < 1) return fail(LINREC_ERR_HIP, "hipDeviceGetAttribute(CU count): " + hip_text(e));
    Plan p;
    linrec_status s = make_plan(pr, p, cus);
    if (s != LINREC_OK) return s;
    if (!empty) {
        if ((s = check_buffer(q.a.ptr, pr.extent_a, device, "a")) != LINREC_OK) return s;
        if ((s = check_buffer(q.b.ptr, pr.extent_b, device, "b")) != LINREC_OK) return s;
        if ((s = check_buffer(q.h.ptr, pr.extent_h, device, "h")) != LINREC_OK) return s;
    }
    if (q.h_init != nullptr && (s = check_buffer(q.h_init, state_bytes, device, "h_init")) != LINREC_OK) return s;
    if (q.h_final != nullptr && (s = check_buffer(q.h_final, state_bytes, device, "h_final")) != LINREC_OK) return s;

    const hipStream_t hs = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (empty) {
        // only L == 0 with B*D > 0 and an h_final reaches here: the state passes through
        hipLaunchKernelGGL(linrec_pass_state, dim3(grid_for(states)), dim3(256), 0, hs, q.h_init, q.h_final, states);
        e = hipGetLastError();
        if (e != hipSuccess) return fail(LINREC_ERR_HIP, "kernel launch: " + hip_text(e));
        return LINREC_OK;
    }

    const bool ahead = q.reverse == 2;   // the reverse form with the decays one time step ahead
    const Launch* fn = pick_launch(q.dtype, p.tile, ahead);
    if (fn == nullptr) return fail(LINREC_ERR_INVALID_ARGUMENT, "no kernel for the chosen tile");
    const int threads = (p.tile.w + p.geom.carry_waves) * linrec::kWave;
    int64_t groups = p.tiles;   // one tile per workgroup
    if (p.tile.m != 1) {
        // persistent workgroups: a grid that gives each of them whole
        // sequences when there is one (the carry then stays local), else as
        // many as fit at once (or q per CU), never more than there are tiles
        int64_t resident = 0;
        if ((s = resident_groups(device, fn, threads, resident)) != LINREC_OK) return s;
        groups = local_grid(p, resident, cus);
        if (groups == 0 && p.tile.m == 2) {
            // no local carry: the relay needs one, so the tiles look back
            // through the m=0 kernel of the same shape
            TileShape looked = p.tile;
            looked.m = 0;
            fn = pick_launch(q.dtype, looked, ahead);
            if (fn == nullptr) return fail(LINREC_ERR_INVALID_ARGUMENT, "no kernel for the chosen tile");
            if ((s = resident_groups(device, fn, threads, resident)) != LINREC_OK) return s;
        }
        if (groups == 0) {
            groups = resident;
            if (p.tile.q > 0) groups = std::min<int64_t>(resident, static_cast<int64_t>(p.tile.q) * cus);
            groups = std::min<int64_t>(groups, p.tiles);
        }
    }
    void* ws = nullptr;
    if (p.workspace_bytes > 0 && p.geom.local_seqs == 0) {
        if (src.scratch) {
            if (p.workspace_bytes > kScratchBytes)
                return fail(LINREC_ERR_INVALID_ARGUMENT,
                            "this call needs " + std::to_string(p.workspace_bytes) +
                                " bytes of lookback workspace and the static scratch of linrec_scan_ex_noalloc "
                                "holds " + std::to_string(kScratchBytes) + "; pass a workspace to linrec_scan_ex_ws");
            if ((s = scratch_for(device, hs, ws)) != LINREC_OK) return s;
        } else if (src.caller) {
            if (src.ptr == nullptr || src.bytes < p.workspace_bytes)
                return fail(LINREC_ERR_INVALID_ARGUMENT,
                            "this call needs a workspace of " + std::to_string(p.workspace_bytes) + " bytes, got " +
                                std::to_string(src.ptr == nullptr ? 0 : src.bytes));
            if (reinterpret_cast<uintptr_t>(src.ptr) % kWorkspaceAlign != 0)
                return fail(LINREC_ERR_INVALID_ARGUMENT, "the workspace must be aligned to 256 bytes");
            const int64_t wb = static_cast<int64_t>(src.bytes);
            if (overlaps(src.ptr, wb, q.a.ptr, pr.extent_a) || overlaps(src.ptr, wb, q.b.ptr, pr.extent_b) ||
                overlaps(src.ptr, wb, q.h.ptr, pr.extent_h) || overlaps(src.ptr, wb, q.h_init, state_bytes) ||
                overlaps(src.ptr, wb, q.h_final, state_bytes))
                return fail(LINREC_ERR_OVERLAP, "the workspace overlaps another buffer");
            if ((s = check_buffer(src.ptr, wb, device, "workspace")) != LINREC_OK) return s;
            if ((s = use_caller_workspace(device, src.ptr, src.bytes, hs)) != LINREC_OK) return s;
            ws = src.ptr;
        } else {
            s = acquire_workspace(device, p.workspace_bytes, hs, ws);
            if (s != LINREC_OK) return s;
        }
    }
    WorkspaceHeader* hdr = static_cast<WorkspaceHeader*>(ws);
    uint64_t* stat = ws ? reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + sizeof(WorkspaceHeader) +
                                                      linrec::kDoneBytes)
                        : nullptr;
    // decays one time step ahead: the kernel reads a through a pointer
    // advanced by one time step, and never reads that pointer's row L-1,
    // which would be a's row L (load_tile)
    const void* a_arg =
        ahead ? static_cast<const void*>(static_cast<const char*>(q.a.ptr) + q.a.stride_l * pr.es) : q.a.ptr;
    (void)hipGetLastError();
    fn->run(dim3(static_cast<uint32_t>(groups)), dim3(threads), a_arg, q.b.ptr, const_cast<void*>(q.h.ptr), p.geom,
            hdr, stat, hs);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "kernel launch: " + hip_text(e));
    return LINREC_OK;
}

// linrec_scan's operands as a descriptor: contiguous fp32 (B, L, D), forward.
linrec_scan_desc contiguous_f32(const float* a, const float* b, float* h, int64_t B, int64_t L, int64_t D) {
    linrec_scan_desc d;
    std::memset(&d, 0, sizeof(d));
    d.B = B;
    d.L = L;
    d.D = D;
    d.dtype = LINREC_F32;
    d.reverse = 0;
    const int64_t sl = D, sb = L * D;   // callers have checked that B*L*D does not overflow
    d.a = linrec_operand{a, sb, sl};
    d.b = linrec_operand{b, sb, sl};
    d.h = linrec_operand{h, sb, sl};
    return d;
}

bool size_ok(int64_t B, int64_t L, int64_t D) {
    int64_t bl = 0, n = 0;
    return B >= 0 && L >= 0 && D >= 0 && checked_mul(B, L, bl) && checked_mul(bl, D, n) && n <= INT64_MAX / 8;
}

// CUs of the current device, or the plan entry points' assumption when there is none.
int current_cus() {
    int device = 0, cus = 0;
    if (hipGetDevice(&device) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus < 1) {
        (void)hipGetLastError();
        return kPlanCus;
    }
    return cus;
}

// Lookback workspace bytes a call of this problem may need on the current device (0: none).
linrec_status workspace_need(const linrec_scan_desc* desc, size_t& bytes) {
    bytes = 0;
    Problem pr;
    linrec_status s = make_problem(desc, pr);
    if (s != LINREC_OK) return s;
    Plan p;
    if ((s = make_plan(pr, p, current_cus())) != LINREC_OK) return s;
    bytes = p.workspace_bytes;
    return LINREC_OK;
}

}  // namespace

// ============================================================================= C ABI

extern "C" {

linrec_status linrec_scan_plan(int64_t B, int64_t L, int64_t D, int aligned16, linrec_plan* plan) {
    if (plan == nullptr) return fail(LINREC_ERR_INVALID_ARGUMENT, "plan is null");
    if (!size_ok(B, L, D)) return fail(LINREC_ERR_INVALID_ARGUMENT, "B, L and D must be >= 0 and B*L*D*8 must fit in 63 bits");
    // stand-in addresses with the alignment asked about; nothing is dereferenced
    const float* base = reinterpret_cast<const float*>(aligned16 ? uintptr_t(256) : uintptr_t(260));
    const linrec_scan_desc d = contiguous_f32(base, base, const_cast<float*>(base), B, L, D);
    Problem pr;
    linrec_status s = make_problem(&d, pr);
    if (s != LINREC_OK) return s;
    Plan p;
    if ((s = make_plan(pr, p, kPlanCus)) != LINREC_OK) return s;
    fill_plan(p, plan);
    return LINREC_OK;
}

linrec_status linrec_scan_ex_plan(const linrec_scan_desc* desc, linrec_plan* plan) {
    if (plan == nullptr) return fail(LINREC_ERR_INVALID_ARGUMENT, "plan is null");
    Problem pr;
    linrec_status s = make_problem(desc, pr);
    if (s != LINREC_OK) return s;
    Plan p;
    if ((s = make_plan(pr, p, kPlanCus)) != LINREC_OK) return s;
    fill_plan(p, plan);
    return LINREC_OK;
}

linrec_status linrec_scan_ex(const linrec_scan_desc* desc, void* stream) {
    t_last_error.clear();
    Problem pr;
    const linrec_status s = make_problem(desc, pr);
    if (s != LINREC_OK) return s;
    return run_scan(pr, stream);
}

size_t linrec_scan_workspace_bytes(int64_t B, int64_t L, int64_t D) {
    if (!size_ok(B, L, D)) return 0;
    size_t most = 0;
    // the plan follows the buffers' alignment: take the larger of the two
    for (uintptr_t base : {uintptr_t(256), uintptr_t(260)}) {
        const float* f = reinterpret_cast<const float*>(base);
        const linrec_scan_desc d = contiguous_f32(f, f, const_cast<float*>(f), B, L, D);
        size_t bytes = 0;
        if (workspace_need(&d, bytes) == LINREC_OK) most = std::max(most, bytes);
    }
    return most;
}

linrec_status linrec_scan_ex_workspace_bytes(const linrec_scan_desc* desc, size_t* bytes) {
    if (bytes == nullptr) return fail(LINREC_ERR_INVALID_ARGUMENT, "bytes is null");
    return workspace_need(desc, *bytes);
}

linrec_status linrec_scan_ws(const float* a, const float* b, float* h, int64_t B, int64_t L, int64_t D,
                             void* workspace, size_t workspace_bytes, void* stream) {
    t_last_error.clear();
    if (B < 0 || L < 0 || D < 0) return fail(LINREC_ERR_INVALID_ARGUMENT, "B, L and D must be >= 0");
    if (B == 0 || L == 0 || D == 0) return LINREC_OK;
    if (!size_ok(B, L, D)) return fail(LINREC_ERR_INVALID_ARGUMENT, "B*L*D elements overflow (B*L*D*8 must fit in 63 bits)");
    const linrec_scan_desc d = contiguous_f32(a, b, h, B, L, D);
    Problem pr;
    const linrec_status s = make_problem(&d, pr);
    if (s != LINREC_OK) return s;
    return run_scan(pr, stream, WorkspaceSource{true, workspace, workspace_bytes});
}

linrec_status linrec_scan_ex_ws(const linrec_scan_desc* desc, void* workspace, size_t workspace_bytes, void* stream) {
    t_last_error.clear();
    Problem pr;
    const linrec_status s = make_problem(desc, pr);
    if (s != LINREC_OK) return s;
    return run_scan(pr, stream, WorkspaceSource{true, workspace, workspace_bytes});
}

linrec_status linrec_scan_ex_noalloc(const linrec_scan_desc* desc, void* stream) {
    t_last_error.clear();
    Problem pr;
    const linrec_status s = make_problem(desc, pr);
    if (s != LINREC_OK) return s;
    WorkspaceSource src;
    src.scratch = true;
    return run_scan(pr, stream, src);
}

linrec_status linrec_scan(const float* a, const float* b, float* h, int64_t B, int64_t L, int64_t D, void* stream) {
    t_last_error.clear();
    if (B < 0 || L < 0 || D < 0) return fail(LINREC_ERR_INVALID_ARGUMENT, "B, L and D must be >= 0");
    if (B == 0 || L == 0 || D == 0) return LINREC_OK;
    if (!size_ok(B, L, D)) return fail(LINREC_ERR_INVALID_ARGUMENT, "B*L*D elements overflow (B*L*D*8 must fit in 63 bits)");
    const linrec_scan_desc d = contiguous_f32(a, b, h, B, L, D);
    Problem pr;
    const linrec_status s = make_problem(&d, pr);
    if (s != LINREC_OK) return s;
    return run_scan(pr, stream);
}

const char* linrec_status_string(int status) {
    switch (status) {
        case LINREC_OK: return "success";
        case LINREC_ERR_INVALID_ARGUMENT: return "invalid argument";
        case LINREC_ERR_OVERLAP: return "output overlaps another buffer";
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
    std::vector<void*> ptrs;
    {
        std::lock_guard<std::mutex> lock(g_mutex);
        for (const auto& kv : g_workspaces)
            if (kv.first.first == device && kv.second.ptr != nullptr) ptrs.push_back(kv.second.ptr);
        for (const auto& r : g_retired)
            if (r.first == device) ptrs.push_back(r.second);
    }
    if (ptrs.empty()) return LINREC_OK;
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return fail(LINREC_ERR_HIP, "hipDeviceSynchronize: " + hip_text(e));
    for (void* ptr : ptrs) {
        WorkspaceHeader hdr;
        e = hipMemcpy(&hdr, ptr, sizeof(hdr), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return fail(LINREC_ERR_HIP, "reading a workspace header: " + hip_text(e));
        *count += hdr.timeouts;
    }
    return LINREC_OK;
}

void linrec_release(void) {
    std::lock_guard<std::mutex> lock(g_mutex);
    int current = 0;
    const bool have_current = hipGetDevice(&current) == hipSuccess;
    std::vector<std::pair<int, void*>> all(g_retired);
    for (const auto& kv : g_workspaces)
        if (kv.second.ptr != nullptr) all.emplace_back(kv.first.first, kv.second.ptr);
    std::map<int, bool> synced;
    for (const auto& w : all) {
        if (hipSetDevice(w.first) != hipSuccess) continue;
        if (!synced[w.first]) {
            (void)hipDeviceSynchronize();
            synced[w.first] = true;
        }
        (void)hipFree(w.second);
    }
    g_workspaces.clear();
    g_retired.clear();
    if (have_current) (void)hipSetDevice(current);
    (void)hipGetLastError();
}

}  // extern "C"
