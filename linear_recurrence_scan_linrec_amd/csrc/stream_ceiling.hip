// stream_ceiling.hip -- libstream_ceiling.so: z = x + y over fp32 arrays with
// the scan kernel's memory instructions, the read-two-write-one stream that
// bounds what the scan (read a and b, write h) can reach on a part.  The C ABI
// is include/linrec_stream.h.
//
// Persistent workgroups of 4 waves.  Each wave takes segments of 64 lanes x
// UNROLL 128-bit accesses of each array (1, 2 or 4 KiB), the next segment's
// loads in flight while the current one is added and stored, as the scan's
// data waves keep the next tile's loads in flight.  Segment s of a walk over
// R rows is chunk s / R of row s % R, so R > 1 reproduces the scan's order of
// one chunk of every batch row before the next chunk; R = 1 is contiguous.
//
// column_walk is the same stream in the walk of the scan's local-carry plans:
// one workgroup per (batch row, channel slab) sequence of a (B, L, D) array,
// W waves, each lane 4 channels and T consecutive rows, the slab's P lanes
// side by side along D; the workgroup takes tiles of W * (64 / P) * T rows in
// order along L, the next tile's loads in flight while the current one is
// added and stored, and two barriers per tile as the scan has.  It isolates
// what that walk costs from what the scan computes.
#include "linrec_stream.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <string>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufferConfig = 0x00020000;   // descriptor word 3 for gfx9-family raw buffers
constexpr int kNontemporal = 2;
constexpr int kWave = 64;
constexpr int kWavesPerGroup = 4;

struct Walk {
    int64_t n;             // elements
    int64_t nseg;          // segments
    int64_t rows;          // R
    int64_t row_elems;     // n / R
};

template <int UNROLL>
__device__ __forceinline__ int64_t segment_start(const Walk& w, int64_t s) {
    constexpr int64_t seg = int64_t{kWave} * 4 * UNROLL;
    const int64_t row = s % w.rows;
    return row * w.row_elems + (s / w.rows) * seg;
}

template <int UNROLL>
__device__ __forceinline__ void load_segment(const float* p, int64_t start, int lane, u32x4 (&v)[UNROLL]) {
    constexpr int bytes = kWave * 16 * UNROLL;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p + start), 0, bytes, kBufferConfig);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (u * kWave + lane) * 16, 0, kNontemporal);
}

template <int UNROLL>
__device__ __forceinline__ void add_store(float* z, int64_t start, int lane, const u32x4 (&x)[UNROLL],
                                          const u32x4 (&y)[UNROLL]) {
    constexpr int bytes = kWave * 16 * UNROLL;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(z + start, 0, bytes, kBufferConfig);
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        u32x4 o;
        o.x = __float_as_uint(__uint_as_float(x[u].x) + __uint_as_float(y[u].x));
        o.y = __float_as_uint(__uint_as_float(x[u].y) + __uint_as_float(y[u].y));
        o.z = __float_as_uint(__uint_as_float(x[u].z) + __uint_as_float(y[u].z));
        o.w = __float_as_uint(__uint_as_float(x[u].w) + __uint_as_float(y[u].w));
        __builtin_amdgcn_raw_buffer_store_b128(o, r, (u * kWave + lane) * 16, 0, kNontemporal);
    }
}

template <int UNROLL>
__global__ void __launch_bounds__(kWave * kWavesPerGroup)
stream_r2w1(const float* __restrict__ x, const float* __restrict__ y, float* __restrict__ z, Walk w) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t waves = static_cast<int64_t>(gridDim.x) * kWavesPerGroup;
    int64_t s = static_cast<int64_t>(blockIdx.x) * kWavesPerGroup + threadIdx.x / kWave;
    if (s >= w.nseg) return;
    u32x4 xa[UNROLL], ya[UNROLL], xb[UNROLL], yb[UNROLL];
    int64_t cur = segment_start<UNROLL>(w, s);
    load_segment<UNROLL>(x, cur, lane, xa);
    load_segment<UNROLL>(y, cur, lane, ya);
    for (;;) {
        const int64_t s1 = s + waves;
        const int64_t nxt = s1 < w.nseg ? segment_start<UNROLL>(w, s1) : cur;
        if (s1 < w.nseg) {
            load_segment<UNROLL>(x, nxt, lane, xb);
            load_segment<UNROLL>(y, nxt, lane, yb);
        }
        add_store<UNROLL>(z, cur, lane, xa, ya);
        if (s1 >= w.nseg) return;
        const int64_t s2 = s1 + waves;
        const int64_t nn = s2 < w.nseg ? segment_start<UNROLL>(w, s2) : nxt;
        if (s2 < w.nseg) {
            load_segment<UNROLL>(x, nn, lane, xa);
            load_segment<UNROLL>(y, nn, lane, ya);
        }
        add_store<UNROLL>(z, nxt, lane, xb, yb);
        if (s2 >= w.nseg) return;
        s = s2;
        cur = nn;
    }
}

// One (batch row, slab) sequence per workgroup: rows of D floats, the slab's
// P lanes x 4 channels, W waves of G = 64 / P lane groups x T rows per tile.
struct Columns {
    int64_t L, D;
    int32_t nslab;        // D / (4 P)
    int32_t lanes;        // P
    int32_t log2_lanes;
};

template <int W, int T>
__device__ __forceinline__ void column_load(__amdgpu_buffer_rsrc_t r, uint32_t off0, uint32_t row_bytes, u32x4 (&v)[T]) {
#pragma unroll
    for (int j = 0; j < T; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, off0 + j * row_bytes, 0, kNontemporal);
}

template <int W, int T>
__global__ void __launch_bounds__(W * kWave)
column_walk(const float* __restrict__ x, const float* __restrict__ y, float* __restrict__ z, Columns c) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int quad = lane & (c.lanes - 1), grp = lane >> c.log2_lanes;
    const int groups = kWave / c.lanes;
    const int64_t row = blockIdx.x / c.nslab, slab = blockIdx.x % c.nslab;
    const int64_t steps = static_cast<int64_t>(W) * groups * T;   // rows per tile
    const int64_t ntile = (c.L + steps - 1) / steps;
    // one descriptor per array and batch row: rows past L fall outside it
    // (loads read 0, stores are dropped)
    const int64_t bytes = c.L * c.D * 4;
    const int nrec = static_cast<int>(bytes < 0x7fffffff ? bytes : 0x7fffffff);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(x + row * c.L * c.D), 0, nrec, kBufferConfig);
    const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(y + row * c.L * c.D), 0, nrec, kBufferConfig);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(z + row * c.L * c.D, 0, nrec, kBufferConfig);
    const uint32_t row_bytes = static_cast<uint32_t>(c.D * 4);
    const uint32_t col = static_cast<uint32_t>((slab * 4 * c.lanes + quad * 4) * 4);
    const int64_t lane_row = static_cast<int64_t>(wave) * groups * T + static_cast<int64_t>(grp) * T;
    auto first = [&](int64_t tile) -> uint32_t {
        return tile < ntile ? static_cast<uint32_t>((tile * steps + lane_row) * c.D * 4) + col : 0x80000000u;
    };
    u32x4 xa[T], ya[T], xb[T], yb[T];
    column_load<W, T>(rx, first(0), row_bytes, xa);
    column_load<W, T>(ry, first(0), row_bytes, ya);
    auto add_store = [&](int64_t tile, const u32x4 (&p)[T], const u32x4 (&q)[T]) {
        const uint32_t off = first(tile);
#pragma unroll
        for (int j = 0; j < T; ++j) {
            u32x4 o;
            o.x = __float_as_uint(__uint_as_float(p[j].x) + __uint_as_float(q[j].x));
            o.y = __float_as_uint(__uint_as_float(p[j].y) + __uint_as_float(q[j].y));
            o.z = __float_as_uint(__uint_as_float(p[j].z) + __uint_as_float(q[j].z));
            o.w = __float_as_uint(__uint_as_float(p[j].w) + __uint_as_float(q[j].w));
            __builtin_amdgcn_raw_buffer_store_b128(o, rz, off + j * row_bytes, 0, kNontemporal);
        }
    };
    for (int64_t tile = 0; tile < ntile; tile += 2) {
        column_load<W, T>(rx, first(tile + 1), row_bytes, xb);
        column_load<W, T>(ry, first(tile + 1), row_bytes, yb);
        __syncthreads();
        __syncthreads();
        add_store(tile, xa, ya);
        if (tile + 1 >= ntile) break;
        column_load<W, T>(rx, first(tile + 2), row_bytes, xa);
        column_load<W, T>(ry, first(tile + 2), row_bytes, ya);
        __syncthreads();
        __syncthreads();
        add_store(tile + 1, xb, yb);
    }
}

thread_local std::string t_error;

int fail(int code, const std::string& msg) {
    t_error = msg;
    return code;
}

}  // namespace

extern "C" {

int linrec_stream_r2w1(const float* x, const float* y, float* z, int64_t n, int64_t rows, int32_t unroll,
                       int32_t groups_per_cu, void* stream) {
    t_error.clear();
    if (unroll != 1 && unroll != 2 && unroll != 4) return fail(1, "unroll must be 1, 2 or 4");
    if (groups_per_cu < 1 || groups_per_cu > 16) return fail(1, "groups_per_cu must be in 1..16");
    if (n < 0 || rows < 1) return fail(1, "n must be >= 0 and rows >= 1");
    if (n == 0) return 0;
    const int64_t seg = int64_t{kWave} * 4 * unroll;
    if (n % (rows * seg) != 0) return fail(1, "n must be a multiple of rows * 256 * unroll");
    if (x == nullptr || y == nullptr || z == nullptr) return fail(1, "null buffer");
    for (const void* p : {static_cast<const void*>(x), static_cast<const void*>(y), static_cast<const void*>(z)})
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(1, "buffers must be 16-byte aligned");
    const uintptr_t zb = reinterpret_cast<uintptr_t>(z), ze = zb + static_cast<uintptr_t>(n) * 4;
    for (const float* p : {x, y}) {
        const uintptr_t b = reinterpret_cast<uintptr_t>(p), e = b + static_cast<uintptr_t>(n) * 4;
        if (b < ze && zb < e) return fail(1, "z overlaps x or y");
    }
    int device = 0, cus = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return fail(2, std::string("HIP: ") + hipGetErrorString(e));
    Walk w{n, n / seg, rows, n / rows};
    const int64_t groups = std::min<int64_t>(static_cast<int64_t>(cus) * groups_per_cu,
                                             (w.nseg + kWavesPerGroup - 1) / kWavesPerGroup);
    const dim3 grid(static_cast<uint32_t>(groups)), block(kWave * kWavesPerGroup);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    switch (unroll) {
        case 1: hipLaunchKernelGGL(stream_r2w1<1>, grid, block, 0, s, x, y, z, w); break;
        case 2: hipLaunchKernelGGL(stream_r2w1<2>, grid, block, 0, s, x, y, z, w); break;
        default: hipLaunchKernelGGL(stream_r2w1<4>, grid, block, 0, s, x, y, z, w); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess) return fail(2, std::string("kernel launch: ") + hipGetErrorString(e));
    return 0;
}

int linrec_stream_column_walk(const float* x, const float* y, float* z, int64_t B, int64_t L, int64_t D,
                              int32_t lanes, int32_t waves, int32_t steps_per_lane, void* stream) {
    t_error.clear();
    if (B < 0 || L < 0 || D < 0) return fail(1, "B, L and D must be >= 0");
    if (lanes != 8 && lanes != 16 && lanes != 32 && lanes != 64) return fail(1, "lanes must be 8, 16, 32 or 64");
    if (waves != 1 && waves != 2 && waves != 4 && waves != 8) return fail(1, "waves must be 1, 2, 4 or 8");
    if (steps_per_lane != 4 && steps_per_lane != 8) return fail(1, "steps_per_lane must be 4 or 8");
    if (B == 0 || L == 0 || D == 0) return 0;
    if (D % (4 * lanes) != 0) return fail(1, "D must be a multiple of 4 * lanes");
    // every row a tile reaches (up to 512 past L) has a 32-bit offset, and
    // those past L lie outside the batch row's range
    if ((L + 512) > ((int64_t{1} << 31) - 1) / 4 / D) return fail(1, "one batch row of an array must span less than 2 GiB");
    if (x == nullptr || y == nullptr || z == nullptr) return fail(1, "null buffer");
    for (const void* p : {static_cast<const void*>(x), static_cast<const void*>(y), static_cast<const void*>(z)})
        if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(1, "buffers must be 16-byte aligned");
    const int64_t n = B * L * D;
    const uintptr_t zb = reinterpret_cast<uintptr_t>(z), ze = zb + static_cast<uintptr_t>(n) * 4;
    for (const float* p : {x, y}) {
        const uintptr_t b = reinterpret_cast<uintptr_t>(p), e = b + static_cast<uintptr_t>(n) * 4;
        if (b < ze && zb < e) return fail(1, "z overlaps x or y");
    }
    int log2 = 0;
    while ((1 << log2) < lanes) ++log2;
    const int32_t nslab = static_cast<int32_t>(D / (4 * lanes));
    if (B * nslab > 0x7fffffff) return fail(1, "too many (batch row, slab) sequences");
    const Columns c{L, D, nslab, lanes, log2};
    const dim3 grid(static_cast<uint32_t>(B * nslab)), block(waves * kWave);
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
#define LINREC_COLUMN_CASE(W_, T_) \
    if (waves == W_ && steps_per_lane == T_) hipLaunchKernelGGL((column_walk<W_, T_>), grid, block, 0, s, x, y, z, c);
    LINREC_COLUMN_CASE(1, 4) LINREC_COLUMN_CASE(1, 8) LINREC_COLUMN_CASE(2, 4) LINREC_COLUMN_CASE(2, 8)
    LINREC_COLUMN_CASE(4, 4) LINREC_COLUMN_CASE(4, 8) LINREC_COLUMN_CASE(8, 4) LINREC_COLUMN_CASE(8, 8)
#undef LINREC_COLUMN_CASE
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(2, std::string("kernel launch: ") + hipGetErrorString(e));
    return 0;
}

const char* linrec_stream_last_error(void) { return t_error.c_str(); }

}  // extern "C"
