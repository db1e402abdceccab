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

const char* linrec_stream_last_error(void) { return t_error.c_str(); }

}  // extern "C"
