// scan_kernel.hpp -- gfx950 kernels of the channel-wise linear-recurrence scan.
//
// The recurrence h_t = a_t * h_{t-1} + b_t (h_0 = b_0) runs independently in
// every (batch row, channel) pair of a (B, L, D) fp32 tensor with D contiguous
// (problem statement of the POPCORNBENCH "Kimi-K2.6 l1_p9" transcript).  Each
// step is the affine map x -> a_t*x + b_t; applying (a1,b1) and then (a2,b2)
// is the pair (a2*a1, a2*b1 + b2), identity (1,0) (operator derivation in that
// transcript's first reasoning block), so any stretch of time steps reduces to
// one pair and only the running h has to cross a stretch boundary (its
// running-carry passage).  The kernel is built on that:
//
//   tile     one workgroup = one (batch row, channel slab, time chunk).
//   lane     owns VEC consecutive channels (VEC = 4: 128-bit loads along D) and
//            T consecutive time steps, all held in registers.
//   wave     64 lanes = G groups of P lanes along t; the P lanes of a group
//            cover the slab's SC = P*VEC channels (a full 1 KiB row span when
//            D >= 256, or G whole consecutive rows when D < 256).
//   steps    (1) load a, b for the lane's T steps (identity pairs past L or D);
//            (2) per-lane sequential composition -> the lane's pair;
//            (3) exclusive scan of the G group pairs across the wave;
//            (4) wave pairs -> LDS -> per-wave exclusive prefix and the tile pair;
//            (5) cross-workgroup carry by decoupled lookback: publish the tile
//                pair, walk back over predecessors' pairs until one publishes
//                its inclusive state, publish this tile's inclusive state;
//            (6) replay h = fma(a_t, h, b_t) from the carried-in state, store.
//
// Status words for the lookback are self-validating 64-bit values: the high
// half is a tag (call epoch << 2 | kind), the low half the fp32 payload, stored
// and loaded with agent-scope relaxed atomics.  A single 64-bit access is
// atomic, so no fence orders payload against flag and no per-call clearing is
// needed: words from earlier calls carry an older epoch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linrec {

constexpr int kWave = 64;
constexpr uint32_t kKindAggregate = 1u;   // payload: one component of the tile pair
constexpr uint32_t kKindInclusive = 2u;   // payload: state h at the tile's last step

// Per-device workspace header; sits in front of the status arrays.
struct WorkspaceHeader {
    uint32_t ticket;     // next tile index to hand out (reset by the last tile)
    uint32_t done;       // tiles finished in the current call
    uint32_t epoch;      // call counter used in status tags
    uint32_t timeouts;   // tiles that gave up waiting (sticky)
    uint32_t pad[60];
};
static_assert(sizeof(WorkspaceHeader) == 256, "header must keep the status arrays 256-byte aligned");

// Launch geometry, computed on the host.
struct Geometry {
    int64_t L, D;
    int64_t nseq;          // B * nslab
    int64_t nchunks;       // time chunks per sequence
    int64_t steps_per_tile;
    int64_t ntiles;        // nseq * nchunks
    int64_t nstatus;       // entries per status array (ntiles * SC)
    int32_t nslab;         // channel slabs per batch row
    int32_t lanes_d;       // P, power of two <= 64
    int32_t log2_lanes_d;
    int32_t groups;        // G = 64 / P
    int32_t slab_channels; // SC = P * VEC
    uint32_t spin_limit;
};

template <int VEC> struct Vec { float v[VEC]; };

template <int VEC> __device__ __forceinline__ Vec<VEC> splat(float x) {
    Vec<VEC> r;
#pragma unroll
    for (int i = 0; i < VEC; ++i) r.v[i] = x;
    return r;
}

template <int VEC> __device__ __forceinline__ Vec<VEC> load_vec(const float* p) {
    Vec<VEC> r;
    if constexpr (VEC == 4) {
        const float4 t = *reinterpret_cast<const float4*>(p);
        r.v[0] = t.x; r.v[1] = t.y; r.v[2] = t.z; r.v[3] = t.w;
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) r.v[i] = p[i];
    }
    return r;
}

template <int VEC> __device__ __forceinline__ void store_vec(float* p, const Vec<VEC>& x) {
    if constexpr (VEC == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(x.v[0], x.v[1], x.v[2], x.v[3]);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) p[i] = x.v[i];
    }
}

// Two ways to grow a pair (A, Bv) that stands for a stretch of consecutive steps.
// then_apply: append the later pair (La, Lb)   -> (La*A, La*Bv + Lb)
// after:      prepend the earlier pair (Ea, Eb) -> (A*Ea, A*Eb + Bv)
template <int VEC>
__device__ __forceinline__ void then_apply(Vec<VEC>& A, Vec<VEC>& Bv, const Vec<VEC>& La, const Vec<VEC>& Lb) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        Bv.v[i] = __builtin_fmaf(La.v[i], Bv.v[i], Lb.v[i]);
        A.v[i] = La.v[i] * A.v[i];
    }
}

template <int VEC>
__device__ __forceinline__ void after(Vec<VEC>& A, Vec<VEC>& Bv, const Vec<VEC>& Ea, const Vec<VEC>& Eb) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        Bv.v[i] = __builtin_fmaf(A.v[i], Eb.v[i], Bv.v[i]);
        A.v[i] = A.v[i] * Ea.v[i];
    }
}

// Value of `x` held by lane `src` of this wave (ds_bpermute).
__device__ __forceinline__ float lane_value(float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

template <int VEC> __device__ __forceinline__ Vec<VEC> lane_value(const Vec<VEC>& x, int src) {
    Vec<VEC> r;
#pragma unroll
    for (int i = 0; i < VEC; ++i) r.v[i] = lane_value(x.v[i], src);
    return r;
}

__device__ __forceinline__ void publish(uint64_t* p, uint32_t tag, float payload) {
    const uint64_t w = (static_cast<uint64_t>(tag) << 32) | static_cast<uint64_t>(__float_as_uint(payload));
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t observe(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return static_cast<uint32_t>(w >> 32); }
__device__ __forceinline__ float payload_of(uint64_t w) { return __uint_as_float(static_cast<uint32_t>(w)); }

// Decoupled lookback for the VEC channels of one lane, starting at predecessor
// chunk-1.  Returns the state entering this tile; sets `timed_out` (and returns
// NaN) when a predecessor publishes nothing within the spin limit.
template <int VEC>
__device__ Vec<VEC> lookback(const uint64_t* __restrict__ stat_a, const uint64_t* __restrict__ stat_b,
                             const uint64_t* __restrict__ stat_p, int64_t first_idx, int64_t stride,
                             int64_t chunk, uint32_t tag_agg, uint32_t tag_inc, uint32_t spin_limit,
                             bool& timed_out) {
    Vec<VEC> acc_a = splat<VEC>(1.0f), acc_b = splat<VEC>(0.0f), h_in = splat<VEC>(0.0f);
    bool done[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) done[i] = false;

    int64_t j = chunk - 1;
    int64_t idx = first_idx - stride;   // status index of predecessor j for channel 0 of this lane
    uint32_t spins = 0;
    timed_out = false;
    while (true) {
        if (j < 0) {   // cannot happen: chunk 0 always publishes its inclusive state
            timed_out = true;
            return splat<VEC>(__builtin_nanf(""));
        }
        uint64_t wp[VEC], wa[VEC], wb[VEC];
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            if (!done[i]) {
                wp[i] = observe(stat_p + idx + i);
                wa[i] = observe(stat_a + idx + i);
                wb[i] = observe(stat_b + idx + i);
            }
        }
        bool waiting = false, all_done = true;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            if (done[i]) continue;
            if (tag_of(wp[i]) == tag_inc) {
                h_in.v[i] = __builtin_fmaf(acc_a.v[i], payload_of(wp[i]), acc_b.v[i]);
                done[i] = true;
            } else {
                all_done = false;
                if (tag_of(wa[i]) != tag_agg || tag_of(wb[i]) != tag_agg) waiting = true;
            }
        }
        if (all_done) break;
        if (waiting) {
            if (++spins > spin_limit) {
                timed_out = true;
                return splat<VEC>(__builtin_nanf(""));
            }
            __builtin_amdgcn_s_sleep(1);
            continue;
        }
        // every open channel has predecessor j's pair: prepend it (it is earlier
        // than everything folded so far) and step back
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
            if (done[i]) continue;
            acc_b.v[i] = __builtin_fmaf(acc_a.v[i], payload_of(wb[i]), acc_b.v[i]);
            acc_a.v[i] = acc_a.v[i] * payload_of(wa[i]);
        }
        --j;
        idx -= stride;
        spins = 0;
    }
    return h_in;
}

template <int VEC, int T, int W>
__global__ void __launch_bounds__(W * kWave)
scan_tiles(const float* __restrict__ a, const float* __restrict__ b, float* __restrict__ h,
           Geometry g, WorkspaceHeader* __restrict__ hdr, uint64_t* __restrict__ stat) {
    __shared__ Vec<VEC> s_agg_a[W][kWave];
    __shared__ Vec<VEC> s_agg_b[W][kWave];
    __shared__ Vec<VEC> s_h_in[kWave];
    __shared__ int64_t s_tile;
    __shared__ uint32_t s_epoch;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const bool chained = g.nchunks > 1;

    if (threadIdx.x == 0) {
        if (chained) {
            // Tiles are handed out in the order workgroups start, so every
            // predecessor of a tile is already running when the tile waits on it.
            s_tile = __hip_atomic_fetch_add(&hdr->ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            s_epoch = __hip_atomic_load(&hdr->epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            s_tile = blockIdx.x;
            s_epoch = 0;
        }
    }
    __syncthreads();
    // a tile index outside the grid can only come from a header corrupted by an
    // overlapping call; such a workgroup touches no memory
    const bool tile_ok = s_tile < g.ntiles;
    const int64_t tile = tile_ok ? s_tile : 0;
    const uint32_t epoch = s_epoch;

    // time chunk is the slow index, so the tiles in flight at once spread over every sequence
    const int64_t chunk = tile / g.nseq;
    const int64_t seq = tile - chunk * g.nseq;
    const int64_t row = seq / g.nslab;
    const int64_t slab = seq - row * g.nslab;

    const int quad = lane & (g.lanes_d - 1);
    const int grp = lane >> g.log2_lanes_d;
    const int64_t d0 = slab * g.slab_channels + static_cast<int64_t>(quad) * VEC;
    const bool d_ok = tile_ok && d0 < g.D;
    const int64_t t0 = chunk * g.steps_per_tile + static_cast<int64_t>(wave * g.groups + grp) * T;
    const int64_t base = (row * g.L + t0) * g.D + d0;

    // (1) loads: identity pairs (1, 0) past the end of the sequence or the channels
    Vec<VEC> av[T], bv[T];
    if (d_ok && t0 + T <= g.L) {
#pragma unroll
        for (int j = 0; j < T; ++j) {
            av[j] = load_vec<VEC>(a + base + j * g.D);
            bv[j] = load_vec<VEC>(b + base + j * g.D);
        }
    } else {
#pragma unroll
        for (int j = 0; j < T; ++j) {
            if (d_ok && t0 + j < g.L) {
                av[j] = load_vec<VEC>(a + base + j * g.D);
                bv[j] = load_vec<VEC>(b + base + j * g.D);
            } else {
                av[j] = splat<VEC>(1.0f);
                bv[j] = splat<VEC>(0.0f);
            }
        }
    }
    // the state before t = 0 is zero, so a_0 never contributes: use 0 for it
    if (t0 == 0) av[0] = splat<VEC>(0.0f);

    // (2) per-lane sequential composition over the T steps
    Vec<VEC> la = av[0], lb = bv[0];
#pragma unroll
    for (int j = 1; j < T; ++j) then_apply<VEC>(la, lb, av[j], bv[j]);

    // (3) groups along t inside the wave: inclusive scan, then shift to exclusive
    Vec<VEC> ex_a = splat<VEC>(1.0f), ex_b = splat<VEC>(0.0f);
    Vec<VEC> wave_a = la, wave_b = lb;
    if (g.groups > 1) {
        Vec<VEC> in_a = la, in_b = lb;
        for (int off = g.lanes_d; off < kWave; off <<= 1) {
            const int src = (lane - off) & (kWave - 1);
            const Vec<VEC> pa = lane_value<VEC>(in_a, src);
            const Vec<VEC> pb = lane_value<VEC>(in_b, src);
            if (lane >= off) after<VEC>(in_a, in_b, pa, pb);
        }
        const int prev = (lane - g.lanes_d) & (kWave - 1);
        const Vec<VEC> pa = lane_value<VEC>(in_a, prev);
        const Vec<VEC> pb = lane_value<VEC>(in_b, prev);
        if (grp > 0) { ex_a = pa; ex_b = pb; }
        const int last = (g.groups - 1) * g.lanes_d + quad;
        wave_a = lane_value<VEC>(in_a, last);
        wave_b = lane_value<VEC>(in_b, last);
    }

    // (4) wave pairs through LDS
    if (grp == 0) {
        s_agg_a[wave][quad] = wave_a;
        s_agg_b[wave][quad] = wave_b;
    }
    __syncthreads();
    Vec<VEC> pw_a = splat<VEC>(1.0f), pw_b = splat<VEC>(0.0f);
    for (int v = 0; v < wave; ++v) then_apply<VEC>(pw_a, pw_b, s_agg_a[v][quad], s_agg_b[v][quad]);

    // (5) carry into the tile, computed by wave 0
    if (wave == 0) {
        Vec<VEC> h_in = splat<VEC>(0.0f);
        bool timed_out = false;
        if (grp == 0 && d_ok && chained) {
            Vec<VEC> ta = s_agg_a[0][quad], tb = s_agg_b[0][quad];
#pragma unroll
            for (int v = 1; v < W; ++v) then_apply<VEC>(ta, tb, s_agg_a[v][quad], s_agg_b[v][quad]);
            const uint32_t tag_agg = (epoch << 2) | kKindAggregate;
            const uint32_t tag_inc = (epoch << 2) | kKindInclusive;
            const int64_t stride = g.slab_channels;
            const int64_t idx = (seq * g.nchunks + chunk) * stride + static_cast<int64_t>(quad) * VEC;
            uint64_t* stat_a = stat;
            uint64_t* stat_b = stat + g.nstatus;
            uint64_t* stat_p = stat + 2 * g.nstatus;
            const bool has_successor = chunk + 1 < g.nchunks;
            if (chunk > 0) {
                if (has_successor) {
#pragma unroll
                    for (int i = 0; i < VEC; ++i) {
                        publish(stat_a + idx + i, tag_agg, ta.v[i]);
                        publish(stat_b + idx + i, tag_agg, tb.v[i]);
                    }
                }
                h_in = lookback<VEC>(stat_a, stat_b, stat_p, idx, stride, chunk,
                                     tag_agg, tag_inc, g.spin_limit, timed_out);
            }
            if (has_successor) {
#pragma unroll
                for (int i = 0; i < VEC; ++i)
                    publish(stat_p + idx + i, tag_inc, __builtin_fmaf(ta.v[i], h_in.v[i], tb.v[i]));
            }
        }
        if (grp == 0) s_h_in[quad] = h_in;
        const uint64_t late = __ballot(timed_out);
        if (late != 0 && lane == 0)
            __hip_atomic_fetch_add(&hdr->timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();

    // (6) state entering this lane's steps, then replay and store
    Vec<VEC> hs = s_h_in[quad];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
        hs.v[i] = __builtin_fmaf(pw_a.v[i], hs.v[i], pw_b.v[i]);
        hs.v[i] = __builtin_fmaf(ex_a.v[i], hs.v[i], ex_b.v[i]);
    }
    if (d_ok) {
        if (t0 + T <= g.L) {
#pragma unroll
            for (int j = 0; j < T; ++j) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) hs.v[i] = __builtin_fmaf(av[j].v[i], hs.v[i], bv[j].v[i]);
                store_vec<VEC>(h + base + j * g.D, hs);
            }
        } else {
#pragma unroll
            for (int j = 0; j < T; ++j) {
#pragma unroll
                for (int i = 0; i < VEC; ++i) hs.v[i] = __builtin_fmaf(av[j].v[i], hs.v[i], bv[j].v[i]);
                if (t0 + j < g.L) store_vec<VEC>(h + base + j * g.D, hs);
            }
        }
    }

    // the last tile to finish rearms the header for the next call
    if (chained && threadIdx.x == 0) {
        const uint32_t ntiles = static_cast<uint32_t>(g.ntiles);
        const uint32_t prev = __hip_atomic_fetch_add(&hdr->done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (prev + 1 == ntiles) {
            __hip_atomic_store(&hdr->ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&hdr->done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&hdr->epoch, (epoch + 1u) & 0x3fffffffu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Zero-fill used to (re)initialise a workspace; a kernel rather than a memset
// so that it can sit inside captured graphs.
__global__ void fill_zero_u32(uint32_t* __restrict__ p, int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t step = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t k = i; k < n; k += step) p[k] = 0u;
}

}  // namespace linrec
