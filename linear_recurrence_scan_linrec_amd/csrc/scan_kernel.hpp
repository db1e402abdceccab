// scan_kernel.hpp -- gfx950 kernels of the channel-wise linear-recurrence scan.
//
// The recurrence h_t = a_t * h_{t-1} + b_t (h_0 = b_0) runs independently in
// every (batch row, channel) pair of a (B, L, D) tensor with D contiguous
// (problem statement of the POPCORNBENCH "Kimi-K2.6 l1_p9" transcript).  Each
// step is the affine map x -> a_t*x + b_t; applying (a1,b1) and then (a2,b2)
// is the pair (a2*a1, a2*b1 + b2), identity (1,0) (operator derivation in that
// transcript's first reasoning block), so any stretch of time steps reduces to
// one pair and only the running h has to cross a stretch boundary (its
// running-carry passage).  The kernels are built on that:
//
//   order    the scan runs over positions tau = 0 .. L-1; forward, tau is the
//            time step t; in reverse (h_t = a_t * h_{t+1} + b_t), t = L-1-tau.
//            The state before tau = 0 is zero, or h_init when given (then the
//            first step uses its a); h_final receives the state after tau = L-1.
//   tile     (batch row, channel slab, chunk of positions): SC channels x
//            W*G*T positions.  Tile index = chunk * nseq + slot; the slot maps
//            to a (batch row, slab) sequence, permuted when slabs narrower than
//            a cache line would otherwise split their lines across XCDs.
//   lane     owns VEC consecutive channels (VEC = 4: 128-bit fp32 or 64-bit
//            16-bit accesses along D) and T consecutive positions, in registers.
//   wave     64 lanes = G groups of P lanes along tau; the P lanes of a group
//            cover the slab's SC = P*VEC channels.
//   workgroup either persistent (scan_tiles: W data waves and ceil(SC/64)
//            carry waves take tiles blockIdx, blockIdx + grid, ... in order,
//            the next tile's loads in flight while the current one waits for
//            its carry) or one per tile (scan_one, which always looks back).
//   steps    (1) load a, b for the lane's T positions;
//            (2) per-lane sequential composition -> the lane's pair;
//            (3) exclusive scan of the G group pairs across the wave;
//            (4) wave pairs -> LDS -> per channel, the tile pair;
//            (5) the state entering the tile, in the carry wave, one channel
//                per lane: kept in LDS when the workgroup's previous tile was
//                the sequence's previous chunk (a persistent grid that divides
//                the sequences: local carry), else by decoupled lookback:
//                publish the tile pair, read the status of the next K
//                predecessors in one round trip, fold their pairs until one
//                has published its inclusive state, publish ours;
//            (6) the carry wave turns the wave pairs into the state entering
//                each wave; replay h = fma(a, h, b) from it, store.
//
// Memory: a, b and h each have their own element strides between batch rows
// and between time steps (the channel stride is 1) and one storage type S
// (fp32, bf16 or fp16).  Values are fp32 in registers; outputs are replayed in
// fp32, and the pairs that carry the state into each lane are fp64 (see
// "Precision of the carry path" below).
//
// Status words are self-validating 64-bit values: the high half is a tag
// (call epoch << 2 | kind), the low half an fp32 payload, stored and loaded
// with agent-scope relaxed atomics.  A single 64-bit access is atomic, so no
// fence orders payload against flag and no per-call clearing is needed: words
// from earlier calls carry an older epoch.  A predecessor that publishes
// nothing for a while has its pair recomputed from the inputs, so every wait
// ends whatever order the workgroups run in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "call_epoch.hpp"

namespace linrec {

constexpr int kWave = 64;
constexpr uint32_t kKindAggregate = 1u;   // payload: one component of the tile pair
constexpr uint32_t kKindInclusive = 2u;   // payload: state after the tile's last position

// Workspace: a header, the kDoneSlots slot lines of the call epoch
// (call_epoch.hpp), then kStatusArrays status arrays of nstatus words (see
// StatusArrays).
constexpr int kMaxLocalSeqs = 4;  // sequences one workgroup may carry locally
constexpr int kStatusArrays = 4;

struct WorkspaceHeader {
    uint32_t reserved;
    uint32_t pad0[kLineWords - 1];
    uint32_t timeouts;                 // waits resolved by recomputation (sticky)
    uint32_t pad1[kLineWords - 1];
    uint32_t finished;                 // slot lines filled in the current call
    uint32_t pad2[kLineWords - 1];
    uint32_t pad3[kLineWords];
};
static_assert(sizeof(WorkspaceHeader) == 512, "header layout");
constexpr size_t kDoneBytes = size_t(kDoneSlots) * kLineWords * sizeof(uint32_t);

// Launch geometry, computed on the host.
struct Geometry {
    int64_t L, D;
    int64_t nseq;          // B * nslab
    int64_t nchunks;       // chunks of positions per sequence
    int64_t steps_per_tile;
    int64_t ntiles;        // nseq * nchunks
    int64_t nstatus;       // entries per status array (ntiles * SC)
    int64_t a_sb, a_sl;    // element strides of a between batch rows and time steps
    int64_t b_sb, b_sl;
    int64_t h_sb, h_sl;    // h_sl >= D whenever L > 1 (h rows never overlap)
    const float* h_init;   // (B, D) fp32, the state before position 0; null: zero
    float* h_final;        // (B, D) fp32, receives the state after position L-1; may be null
    int32_t nslab;         // channel slabs per batch row
    int32_t lanes_d;       // P, power of two <= 64
    int32_t log2_lanes_d;
    int32_t groups;        // G = 64 / P
    int32_t slab_channels; // SC = P * VEC
    int32_t carry_waves;   // ceil(SC / 64): one slab channel per carry-wave lane
    uint32_t spin_limit;   // polls of one predecessor before recomputing its pair
    int32_t reverse;       // 0: position tau is time step tau; 1: time step L-1-tau
    int32_t local_seqs;    // > 0: the persistent grid divides nseq into local_seqs (<= kMaxLocalSeqs)
                           // sequences per workgroup, so every tile's predecessor was this
                           // workgroup's own tile local_seqs tiles earlier and the carry stays in
                           // LDS (no status words, no workspace); 0: decoupled lookback
    int32_t line_shift;    // log2 of the slabs that share one 128-byte line (0: slots are sequences)
    int32_t lookback_window;  // 2: read 2 predecessors per round trip; above 2: the long-chain window
};

template <int VEC> struct Vec { float v[VEC]; };

template <int VEC> __device__ __forceinline__ Vec<VEC> splat(float x) {
    Vec<VEC> r;
#pragma unroll
    for (int i = 0; i < VEC; ++i) r.v[i] = x;
    return r;
}

// ---------------------------------------------------------------------------
// Storage types.  a, b and h are fp32, bf16 or fp16 in memory; values widen to
// fp32 on load and round to nearest even on store.
struct Bf16 { uint16_t bits; };
struct F16 { uint16_t bits; };

template <typename S> constexpr int storage_bytes() { return sizeof(S) == 4 ? 4 : 2; }

__device__ __forceinline__ float widen_bits(Bf16, uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float widen_bits(F16, uint32_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}
__device__ __forceinline__ uint32_t narrow_bits(Bf16, float x) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}
__device__ __forceinline__ uint32_t narrow_bits(F16, float x) {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
}

// Value of element p (plain load; used off the streaming path).
__device__ __forceinline__ float load_one(const float* p) { return *p; }
__device__ __forceinline__ float load_one(const Bf16* p) { return widen_bits(Bf16{}, p->bits); }
__device__ __forceinline__ float load_one(const F16* p) { return widen_bits(F16{}, p->bits); }

// Streaming accesses of a, b and h go through buffer resources: each tile
// gets a descriptor per operand whose range ends with the tile's last valid
// element, so a load outside it returns 0 and a store outside it is dropped by
// the hardware.  The loops therefore have no branches, which lets the compiler
// wait only for the loads a step needs instead of everything in flight.  The
// accesses are nontemporal (every byte is touched once); on gfx950 that
// measured 10-20% faster than plain accesses for this pattern.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufferConfig = 0x00020000;   // descriptor word 3 for gfx9-family raw buffers
constexpr int kNontemporal = 2;             // cache-policy bit: no temporal reuse expected
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset beyond every tile's range
constexpr int64_t kMaxRange = 0x7fffffff;      // largest range one descriptor is given
// Largest byte span the host lets one tile of an operand cover.  Below 2^30,
// every offset a lane forms stays outside its tile's range whenever it should:
// kOutOfRange moved by up to a tile's span either way (reverse scans step
// backwards, as wrapping 32-bit offsets), and a negative offset before the
// range start, both land at or above 2^30, beyond any range.
constexpr int64_t kMaxTileBytes = int64_t(1) << 30;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_range(const void* base, int64_t bytes) {
    const int64_t n = bytes < kMaxRange ? bytes : kMaxRange;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n), kBufferConfig);
}

template <typename S, int VEC>
__device__ __forceinline__ Vec<VEC> load_vec(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Vec<VEC> x;
    if constexpr (storage_bytes<S>() == 4) {
        if constexpr (VEC == 4) {
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kNontemporal);
            x.v[0] = __uint_as_float(t.x); x.v[1] = __uint_as_float(t.y);
            x.v[2] = __uint_as_float(t.z); x.v[3] = __uint_as_float(t.w);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                x.v[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off + 4 * i, 0, kNontemporal));
        }
    } else {
        if constexpr (VEC == 4) {
            const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNontemporal);
            x.v[0] = widen_bits(S{}, t.x & 0xffffu); x.v[1] = widen_bits(S{}, t.x >> 16);
            x.v[2] = widen_bits(S{}, t.y & 0xffffu); x.v[3] = widen_bits(S{}, t.y >> 16);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                x.v[i] = widen_bits(S{}, __builtin_amdgcn_raw_buffer_load_b16(r, off + 2 * i, 0, kNontemporal));
        }
    }
    return x;
}

template <typename S, int VEC>
__device__ __forceinline__ void store_vec(__amdgpu_buffer_rsrc_t r, uint32_t off, const Vec<VEC>& x) {
    if constexpr (storage_bytes<S>() == 4) {
        if constexpr (VEC == 4) {
            const u32x4 t = {__float_as_uint(x.v[0]), __float_as_uint(x.v[1]), __float_as_uint(x.v[2]),
                             __float_as_uint(x.v[3])};
            __builtin_amdgcn_raw_buffer_store_b128(t, r, off, 0, kNontemporal);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x.v[i]), r, off + 4 * i, 0, kNontemporal);
        }
    } else {
        if constexpr (VEC == 4) {
            const u32x2 t = {narrow_bits(S{}, x.v[0]) | (narrow_bits(S{}, x.v[1]) << 16),
                             narrow_bits(S{}, x.v[2]) | (narrow_bits(S{}, x.v[3]) << 16)};
            __builtin_amdgcn_raw_buffer_store_b64(t, r, off, 0, kNontemporal);
        } else {
#pragma unroll
            for (int i = 0; i < VEC; ++i)
                __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(narrow_bits(S{}, x.v[i])), r,
                                                      off + 2 * i, 0, kNontemporal);
        }
    }
}

// Register form of one position's VEC channels.  fp32 keeps the floats.  With
// 16-bit storage and VEC = 4 a lane keeps the two loaded 32-bit words (four
// packed values, half the registers) and widens them where they are used, so
// it can hold twice the positions in the same registers.
struct Packed4 {
    uint32_t w[2];
};
template <typename S, int VEC> struct RegOf { using type = Vec<VEC>; };
template <> struct RegOf<Bf16, 4> { using type = Packed4; };
template <> struct RegOf<F16, 4> { using type = Packed4; };
template <typename S, int VEC> using Reg = typename RegOf<S, VEC>::type;

template <typename S, int VEC>
__device__ __forceinline__ Reg<S, VEC> load_reg(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (storage_bytes<S>() == 2 && VEC == 4) {
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kNontemporal);
        return Packed4{{t.x, t.y}};
    } else {
        return load_vec<S, VEC>(r, off);
    }
}

template <typename S, int VEC>
__device__ __forceinline__ Vec<VEC> widen(const Reg<S, VEC>& x) {
    if constexpr (storage_bytes<S>() == 2 && VEC == 4) {
        Vec<VEC> v;
        v.v[0] = widen_bits(S{}, x.w[0] & 0xffffu); v.v[1] = widen_bits(S{}, x.w[0] >> 16);
        v.v[2] = widen_bits(S{}, x.w[1] & 0xffffu); v.v[3] = widen_bits(S{}, x.w[1] >> 16);
        return v;
    } else {
        return x;
    }
}

// The replay widens the packed words again rather than keep the widened values
// of the scan alive across the hand-over: an empty asm statement that may
// "change" the words stops the compiler from reusing the scan's conversions,
// so only the packed words stay live (no instruction is emitted).
template <typename S, int VEC>
__device__ __forceinline__ Reg<S, VEC> rewiden_source(const Reg<S, VEC>& x) {
    Reg<S, VEC> y = x;
    if constexpr (storage_bytes<S>() == 2 && VEC == 4) asm volatile("" : "+v"(y.w[0]), "+v"(y.w[1]));
    return y;
}

// Every channel of x set to c (0 or 1: exact in every storage type).
template <typename S, int VEC>
__device__ __forceinline__ void set_reg(Reg<S, VEC>& x, float c) {
    if constexpr (storage_bytes<S>() == 2 && VEC == 4) {
        const uint32_t bits = narrow_bits(S{}, c);
        x.w[0] = x.w[1] = bits | (bits << 16);
    } else {
        x = splat<VEC>(c);
    }
}

// Precision of the carry path.  Outputs are replayed in fp32 (h = fma(a, h, b))
// from the state entering each lane's positions, like a sequential fp32 loop.
// What carries the state from tile to tile is the product of each stretch's
// decays, and those products are kept in fp64 from the lane upwards (a lane's
// product starts from exact products of two fp32 values).  The reason: with a
// decay that is the same at every step, every lane, wave and tile would round
// an fp32 product of decays the same way, and the carry multiplies the running
// state by those products stretch after stretch, so their equal errors would
// add up along the sequence instead of averaging out (with a decay near 1 and
// |h| near 100 that exceeds the 1e-4 * (1 + |h|) bar where h crosses zero).
// The B half of a pair is fp32: its rounding errors follow the b values, so
// they do not line up.  Values that only seed one lane's or one wave's replay
// (its prefix pair, the state entering it) are rounded to fp32 once.
template <int VEC> struct VecD { double v[VEC]; };

// Product of the decays of positions [lo, hi) of a lane, as a tree: the
// leaves multiply two fp32 values (exact in fp64), the tree is shallow.
template <int LO, int HI, typename R>
__device__ __forceinline__ double decay_product(const R& a, int i) {
    if constexpr (HI - LO == 1) {
        return static_cast<double>(a[LO].v[i]);
    } else {
        constexpr int MID = (LO + HI) / 2;
        return decay_product<LO, MID>(a, i) * decay_product<MID, HI>(a, i);
    }
}

// Value of `x` held by lane `src` of this wave (ds_bpermute, one per 32-bit half).
__device__ __forceinline__ double lane_value(double x, int src) {
    const uint64_t bits = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(bits)));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute(src << 2, static_cast<int>(bits >> 32)));
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ float lane_value(float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}

template <typename V> __device__ __forceinline__ V lane_values(const V& x, int src) {
    V r;
#pragma unroll
    for (int i = 0; i < static_cast<int>(sizeof(x.v) / sizeof(x.v[0])); ++i) r.v[i] = lane_value(x.v[i], src);
    return r;
}

__device__ __forceinline__ void publish(uint64_t* p, uint32_t tag, float payload) {
    const uint64_t w = (static_cast<uint64_t>(tag) << 32) | static_cast<uint64_t>(__float_as_uint(payload));
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t observe(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t observe32(const uint32_t* p) {
    return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return static_cast<uint32_t>(w >> 32); }
__device__ __forceinline__ float payload_of(uint64_t w) { return __uint_as_float(static_cast<uint32_t>(w)); }

// Time step of scan position tau.
__device__ __forceinline__ int64_t time_of(const Geometry& g, int64_t tau) { return g.reverse ? g.L - 1 - tau : tau; }

// State before position 0 for channel d of batch row `row`.
__device__ __forceinline__ float initial_state(const Geometry& g, int64_t row, int64_t d) {
    return g.h_init != nullptr ? g.h_init[row * g.D + d] : 0.0f;
}

// One operand's view of a tile: descriptor, this lane's first offset and the
// offset step between consecutive positions (negative, as a wrapping 32-bit
// value, when the scan runs backwards in memory).
struct OperandSpot {
    __amdgpu_buffer_rsrc_t r;
    uint32_t off;
    uint32_t step;
};

// Where one tile sits and what this lane covers of it.
struct TileSpot {
    int64_t chunk, seq, row, slab;
    int64_t tau0;   // first position of this lane
    bool d_ok;      // this lane's channels exist
    OperandSpot a, b, h;
};

// The tile covers positions [first, end) of its sequence, end <= L, i.e. time
// steps [t_lo, t_lo + span) with span = end - first.  The descriptor starts at
// time step t_lo of the batch row and its range ends with the element
// (t_lo + span - 1, D - 1).  A position past L is, forward, a time step past
// the range's end (time strides of h are >= D), and in reverse a step before
// t_lo, whose negative offset wraps beyond 2^31 > any range; channels past D
// get kOutOfRange.  So such loads read 0 and such stores are dropped.
template <typename S>
__device__ __forceinline__ OperandSpot operand_spot(const S* base, int64_t sb, int64_t sl, const Geometry& g,
                                                    int64_t row, int64_t t_lo, int64_t span, int64_t lane_rel,
                                                    int64_t d0, bool d_ok) {
    constexpr int64_t es = storage_bytes<S>();
    OperandSpot o;
    const int64_t bytes = ((span - 1) * sl + g.D) * es;
    o.r = make_range(base + row * sb + t_lo * sl, bytes);
    o.off = d_ok ? static_cast<uint32_t>((lane_rel * sl + d0) * es) : kOutOfRange;
    o.step = static_cast<uint32_t>((g.reverse ? -sl : sl) * es);
    return o;
}

// Dispatch slot (tile modulo nseq) -> sequence.  A slab row narrower than a
// 128-byte cache line shares each line with the neighbouring slabs of its
// batch row: n = 2^line_shift slabs per line.  Within each block of 8n slots,
// slot x + 8i (x < 8, i < n) takes sequence n*x + i, so the n slabs of one
// line sit on slots that are equal modulo 8.  Workgroups are dispatched to the
// 8 XCDs in turn, so those slabs are scanned on one XCD and each line is
// fetched into one L2 once instead of into n.  The host sets line_shift only
// when nseq is a multiple of 8n; any value gives a bijection on the slots.
__device__ __forceinline__ int64_t sequence_of(const Geometry& g, int64_t slot) {
    if (g.line_shift == 0) return slot;
    const int64_t block = int64_t{8} << g.line_shift;
    const int64_t r = slot & (block - 1);
    return (slot - r) + ((r & 7) << g.line_shift) + (r >> 3);
}

// Tile index -> (chunk, sequence, batch row, slab).  The operands are
// wave-uniform, so each division is a long scalar instruction sequence (the
// carry waves therefore run it before the barrier that starts their part of
// a tile).  Tiles number fewer than 2^31 (the host refuses more),
// so the 32-bit form is exact.  Measured on MI355X, same-run A/B: with 16-bit
// storage, whose tiles move half the bytes, the 32-bit form is 2-10% faster;
// with fp32 storage the 64-bit form is 3-10% faster on the local-carry plans
// (the workgroups that share a batch row stay closer in step) and no slower
// on the others.
struct TileIndex {
    int64_t chunk, seq, row, slab;
};

template <typename S>
__device__ __forceinline__ TileIndex tile_index(const Geometry& g, int64_t tile) {
    if constexpr (storage_bytes<S>() == 2) {
        const uint32_t t = static_cast<uint32_t>(tile);
        const uint32_t nseq = static_cast<uint32_t>(g.nseq);
        const uint32_t chunk = t / nseq;
        const uint32_t seq = static_cast<uint32_t>(sequence_of(g, t - chunk * nseq));
        const uint32_t nslab = static_cast<uint32_t>(g.nslab);
        const uint32_t row = seq / nslab;
        return TileIndex{chunk, seq, row, seq - row * nslab};
    } else {
        const int64_t chunk = tile / g.nseq;
        const int64_t seq = sequence_of(g, tile - chunk * g.nseq);
        const int64_t row = seq / g.nslab;
        return TileIndex{chunk, seq, row, seq - row * g.nslab};
    }
}

template <typename S>
__device__ __forceinline__ TileSpot locate_at(const S* a, const S* b, S* h, const Geometry& g, const TileIndex& ix,
                                              int wave, int quad, int grp, int vec, int T) {
    TileSpot s;
    s.chunk = ix.chunk;
    s.seq = ix.seq;
    s.row = ix.row;
    s.slab = ix.slab;
    const int64_t d0 = s.slab * g.slab_channels + static_cast<int64_t>(quad) * vec;
    s.d_ok = d0 < g.D;
    const int64_t first = s.chunk * g.steps_per_tile;
    const int64_t end = first + g.steps_per_tile < g.L ? first + g.steps_per_tile : g.L;
    const int64_t local = static_cast<int64_t>(wave * g.groups + grp) * T;
    s.tau0 = first + local;
    const int64_t span = end - first;
    // time step of the range start, and this lane's first time step relative to it
    const int64_t t_lo = g.reverse ? g.L - end : first;
    const int64_t rel = g.reverse ? span - 1 - local : local;
    s.a = operand_spot<S>(a, g.a_sb, g.a_sl, g, s.row, t_lo, span, rel, d0, s.d_ok);
    s.b = operand_spot<S>(b, g.b_sb, g.b_sl, g, s.row, t_lo, span, rel, d0, s.d_ok);
    s.h = operand_spot<S>(h, g.h_sb, g.h_sl, g, s.row, t_lo, span, rel, d0, s.d_ok);
    return s;
}

template <typename S>
__device__ __forceinline__ TileSpot locate(const S* a, const S* b, S* h, const Geometry& g, int64_t tile,
                                           int wave, int quad, int grp, int vec, int T) {
    // the chunk is the slow index: a tile's predecessors come before it in
    // every workgroup's order, and the tiles in flight spread over all sequences
    return locate_at<S>(a, b, h, g, tile_index<S>(g, tile), wave, quad, grp, vec, T);
}

// (1) loads of one tile into a register buffer.  Positions past L and channels
// past D read as (a, b) = (0, 0) (or, for a or b whose time stride is below D,
// other in-bounds elements): such positions come after every real position of
// their lane, group and wave, and their channels are never stored, so no
// stored output depends on them.
//
// All of a is requested before any of b: a lane's requests then walk one
// array at a time, which measured 2% faster than alternating a and b rows.
//
// AHEAD (decays one time step ahead, reverse only): a arrives advanced by one
// time step, so the first position's read would be a's row L, past the batch
// row's last.  That read is not made; the value is replaced anyway (see
// scan_registers).
template <typename S, int VEC, int T, bool AHEAD = false>
__device__ __forceinline__ void load_tile(Reg<S, VEC> (&av)[T], Reg<S, VEC> (&bv)[T], const TileSpot& s) {
#pragma unroll
    for (int j = 0; j < T; ++j)
        av[j] = load_reg<S, VEC>(s.a.r, AHEAD && j == 0 && s.tau0 == 0 ? kOutOfRange : s.a.off + j * s.a.step);
#pragma unroll
    for (int j = 0; j < T; ++j) bv[j] = load_reg<S, VEC>(s.b.r, s.b.off + j * s.b.step);
}

// The pair of chunk j for one channel, composed directly from a and b: the
// fallback when chunk j's tile has published nothing for a while.  It only
// reads inputs, so it always finishes.
template <typename S, bool AHEAD>
__device__ inline void chunk_pair_from_inputs(const S* __restrict__ a, const S* __restrict__ b, const Geometry& g,
                                              int64_t row, int64_t d, int64_t j, double& A, double& Bv) {
    A = 1.0;
    float bl = 0.0f;
    const int64_t tau_begin = j * g.steps_per_tile;
    const int64_t tau_end = tau_begin + g.steps_per_tile < g.L ? tau_begin + g.steps_per_tile : g.L;
    for (int64_t tau = tau_begin; tau < tau_end; ++tau) {
        const int64_t t = time_of(g, tau);
        // (with AHEAD, a is advanced by one time step: this read gives a at
        // t+1, and position 0, whose decay would be a at L, takes 1 with h_init)
        float at;
        if constexpr (AHEAD)
            at = tau == 0 ? (g.h_init == nullptr ? 0.0f : 1.0f) : load_one(a + row * g.a_sb + t * g.a_sl + d);
        else
            at = (tau == 0 && g.h_init == nullptr) ? 0.0f : load_one(a + row * g.a_sb + t * g.a_sl + d);
        const float bt = load_one(b + row * g.b_sb + t * g.b_sl + d);
        bl = __builtin_fmaf(at, bl, bt);
        A = static_cast<double>(at) * A;
    }
    Bv = bl;
}

// Status arrays of a lookback workspace, nstatus words each: the tile pair
// (its product of decays as the fp32 pair hi + lo, which keeps about 48 bits
// of it, or hi alone for 16-bit storage; and B), and the inclusive state
// after the tile.
struct StatusArrays {
    uint64_t *a_hi, *a_lo, *b, *p;
};

__device__ __forceinline__ StatusArrays status_arrays(uint64_t* stat, int64_t nstatus) {
    return StatusArrays{stat, stat + nstatus, stat + 2 * nstatus, stat + 3 * nstatus};
}

// With 16-bit storage the published product of decays is the single fp32 word
// hi (a_lo is neither written nor read).  Rounding it once per tile costs at
// most 2^-24 of the product; with a constant decay those errors repeat, and
// they add up over the chain's memory of about 1 / (1 - tile product) tiles,
// which at a decay of 0.99999 and 448 positions per tile is 224 tiles: about
// 1.3e-5 of the state, against outputs rounded at 2^-8 (bf16) or 2^-11 (fp16).
// fp32 outputs keep the hi + lo pair.
template <typename S>
constexpr bool product_in_one_word() {
    return sizeof(S) == 2;
}

// The long-chain lookback window (see lookback_channel): predecessors read per
// round trip, and on the first round trip.
template <typename S>
__device__ constexpr int long_window() {
    return product_in_one_word<S>() ? 4 : 3;
}
template <typename S>
__device__ constexpr int first_window() {
    return product_in_one_word<S>() ? 2 : 3;
}

// Decoupled lookback for one channel of a tile in chunk `chunk` (> 0): reads
// the status of up to WIN predecessors per round trip and folds their pairs,
// nearest first, until one of them has published its inclusive state.  A
// predecessor that shows nothing within spin_limit polls has its pair
// recomputed from the inputs (`recomputed` is set).  Returns the state that
// enters the tile.
//
// The window trades status reads against round trips, and status reads are
// not free (one more inclusive-state word per round trip made 586-chunk
// chains 1-4% slower).  Measured on MI355X (same-run A/B): where
// the tiles of a chunk-major round look back at each other (persistent
// workgroups), reading 2 predecessors instead of 4 was 4-15% faster; one tile
// per workgroup over very long chains (over 64 chunks per sequence, most
// predecessors still pending) wants a wider window: 3 with fp32 storage (1.5%
// faster than 4), 4 with 16-bit storage, whose tiles publish the product of
// decays in one word (3 was no faster).  The host picks the long-chain form
// through Geometry::lookback_window.  FIRST (at most WIN) is the window of the
// first round trip only: with 16-bit storage a tile's life is short enough
// that its nearest predecessor has mostly published by the time it looks
// back, and reading 2 there, 4 after, was 1.5-2% faster on 586-chunk chains;
// with fp32, 2 then 4 was 0.7% slower than 4 throughout.
template <typename S, int WIN, bool AHEAD, int FIRST = WIN>
__device__ inline double lookback_channel(const S* __restrict__ a, const S* __restrict__ b, const Geometry& g,
                                          int64_t row, int64_t d, const StatusArrays& st, int64_t idx, int64_t chunk,
                                          uint32_t tag_agg, uint32_t tag_inc, bool& recomputed) {
    const int64_t stride = g.slab_channels;   // status distance between consecutive chunks
    double acc_a = 1.0, acc_b = 0.0;
    int64_t j = chunk - 1;                    // nearest predecessor not folded yet
    uint32_t spins = 0;
    int reach = FIRST;                        // predecessors read this round trip
    while (j >= 0) {
        uint64_t wp[WIN], wh[WIN], wl[WIN], wb[WIN];
#pragma unroll
        for (int m = 0; m < WIN; ++m) {
            wp[m] = wh[m] = wl[m] = wb[m] = 0;
            if (j - m >= 0 && m < reach) {
                const int64_t k = idx - (chunk - (j - m)) * stride;
                wp[m] = observe(st.p + k);
                wh[m] = observe(st.a_hi + k);
                if constexpr (!product_in_one_word<S>()) wl[m] = observe(st.a_lo + k);
                wb[m] = observe(st.b + k);
            }
        }
        int folded = 0;
        bool found = false;
        double h_prev = 0.0;
#pragma unroll
        for (int m = 0; m < WIN; ++m) {
            if (found || folded != m || j - m < 0 || m >= reach) continue;   // stopped earlier in this window
            if (tag_of(wp[m]) == tag_inc) {
                h_prev = payload_of(wp[m]);
                found = true;
            } else if (tag_of(wh[m]) == tag_agg && (product_in_one_word<S>() || tag_of(wl[m]) == tag_agg) &&
                       tag_of(wb[m]) == tag_agg) {
                const double pa = product_in_one_word<S>()
                                      ? static_cast<double>(payload_of(wh[m]))
                                      : static_cast<double>(payload_of(wh[m])) + static_cast<double>(payload_of(wl[m]));
                acc_b = __builtin_fma(acc_a, static_cast<double>(payload_of(wb[m])), acc_b);
                acc_a = acc_a * pa;
                folded = m + 1;
            }
        }
        if (found) return __builtin_fma(acc_a, h_prev, acc_b);
        reach = WIN;
        if (folded > 0) {
            j -= folded;
            spins = 0;
            continue;
        }
        if (spins < g.spin_limit) {
            ++spins;
            __builtin_amdgcn_s_sleep(2);
            continue;
        }
        // predecessor j shows nothing: compose its pair from the inputs
        double pa, pb;
        chunk_pair_from_inputs<S, AHEAD>(a, b, g, row, d, j, pa, pb);
        acc_b = __builtin_fma(acc_a, pb, acc_b);
        acc_a = acc_a * pa;
        recomputed = true;
        --j;
        spins = 0;
    }
    // walked past chunk 0 through recomputed pairs: apply them to the state before position 0
    return __builtin_fma(acc_a, static_cast<double>(initial_state(g, row, d)), acc_b);
}

// ---------------------------------------------------------------------------
// Call epochs (call_epoch.hpp) over agent-scope atomics.  The slot lines
// follow the header; every wave of a workgroup that publishes or reads status
// words reads the epoch before the workgroup's count_done (behind a barrier).

struct AgentAtomics {
    __device__ static uint32_t load(uint32_t* p) { return observe32(p); }
    __device__ static uint32_t add(uint32_t* p, uint32_t v) {
        return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ static void store(uint32_t* p, uint32_t v) {
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
};

__device__ __forceinline__ EpochWords epoch_words(WorkspaceHeader* hdr) {
    return EpochWords{reinterpret_cast<uint32_t*>(hdr + 1), &hdr->finished};
}

__device__ __forceinline__ uint32_t call_epoch(WorkspaceHeader* hdr) {
    return epoch_of_call<AgentAtomics>(epoch_words(hdr), blockIdx.x, gridDim.x);
}

// Lane 0 counts the workgroup in its slot line; returns the count before the
// addition on lane 0, 0 elsewhere.
__device__ __forceinline__ uint32_t count_in(WorkspaceHeader* hdr, uint32_t epoch, int lane) {
    if (lane != 0) return 0u;
    return epoch_count_in<AgentAtomics>(epoch_words(hdr), blockIdx.x, gridDim.x, epoch);
}

// Whole wave, after a barrier that every wave reading the epoch has passed:
// given count_in's result, rearm the slot line if this workgroup filled it,
// and advance the epoch if it filled the last line.
__device__ inline void count_done(WorkspaceHeader* hdr, uint32_t epoch, uint32_t before, int lane) {
    const EpochWords w = epoch_words(hdr);
    const int last = lane == 0 && epoch_count_done<AgentAtomics>(w, blockIdx.x, gridDim.x, before) ? 1 : 0;
    if (__shfl(last, 0) != 0) epoch_advance<AgentAtomics>(w, epoch, lane, kWave);
}

// LDS shared by the waves of one workgroup.  Between the two barriers of a
// tile, (pair_a, pair_b)[w] hold data wave w's pair; after the second barrier
// pair_b[w] holds the state entering wave w's positions (the carry wave
// rewrites it in place).  Each data wave reads and writes only its own slot.
template <int VEC, int W>
struct TileShared {
    VecD<VEC> pair_a[W][kWave];   // per data wave and lane channel group: the wave's product of decays
    Vec<VEC> pair_b[W][kWave];    // its B; after the second barrier, the state entering the wave
};

// What a lane keeps of its tile between the scan in registers and the store.
template <int VEC>
struct LanePrefix {
    Vec<VEC> ex_a, ex_b;   // pair of the positions before this lane's in its wave (group scan)
};

// Steps (2)-(4) up to the hand-over: per-lane composition, the group scan
// along tau inside the wave, and the wave's pair into LDS.  Without h_init the
// state before position 0 is zero, so that position's a never contributes: use
// 0 for it.
template <typename S, int VEC, int T, int W, bool AHEAD = false>
__device__ __forceinline__ LanePrefix<VEC> scan_registers(const Geometry& g, TileShared<VEC, W>& sh, const TileSpot& s,
                                                          int lane, int wave, int quad, int grp,
                                                          Reg<S, VEC> (&av)[T], Reg<S, VEC> (&bv)[T]) {
    if (s.tau0 == 0 && g.h_init == nullptr) set_reg<S, VEC>(av[0], 0.0f);
    else if (AHEAD && s.tau0 == 0) set_reg<S, VEC>(av[0], 1.0f);   // h_init enters with decay 1
    if (g.h_final != nullptr && (s.chunk + 1) * g.steps_per_tile > g.L) {
        // positions past L (only the last chunk of a ragged length has them;
        // the test is uniform, so other tiles skip the per-lane checks)
        // become identity steps (1, 0): they then leave the state of position
        // L-1 unchanged to the end of its lane (no stored output depends on
        // them either way)
#pragma unroll
        for (int j = 0; j < T; ++j) {
            if (s.tau0 + j >= g.L) {
                set_reg<S, VEC>(av[j], 1.0f);
                set_reg<S, VEC>(bv[j], 0.0f);
            }
        }
    }

    // (2) per-lane sequential composition over the T positions
    Vec<VEC> in_b = widen<S, VEC>(bv[0]);
#pragma unroll
    for (int j = 1; j < T; ++j) {
        const Vec<VEC> aj = widen<S, VEC>(av[j]), bj = widen<S, VEC>(bv[j]);
#pragma unroll
        for (int i = 0; i < VEC; ++i) in_b.v[i] = __builtin_fmaf(aj.v[i], in_b.v[i], bj.v[i]);
    }
    VecD<VEC> in_a;
    {
        Vec<VEC> aw[T];
#pragma unroll
        for (int j = 0; j < T; ++j) aw[j] = widen<S, VEC>(av[j]);
#pragma unroll
        for (int i = 0; i < VEC; ++i) in_a.v[i] = decay_product<0, T>(aw, i);
    }

    // (3) groups along tau inside the wave: inclusive scan, then shift to exclusive
    LanePrefix<VEC> pre;
    pre.ex_a = splat<VEC>(1.0f);
    pre.ex_b = splat<VEC>(0.0f);
    if (g.groups > 1) {
        for (int off = g.lanes_d; off < kWave; off <<= 1) {
            const int src = (lane - off) & (kWave - 1);
            const VecD<VEC> pa = lane_values(in_a, src);
            const Vec<VEC> pb = lane_values(in_b, src);
            if (lane >= off) {
                // prepend the earlier pair (pa, pb)
#pragma unroll
                for (int i = 0; i < VEC; ++i) {
                    in_b.v[i] = __builtin_fmaf(static_cast<float>(in_a.v[i]), pb.v[i], in_b.v[i]);
                    in_a.v[i] = in_a.v[i] * pa.v[i];
                }
            }
        }
        const int prev = (lane - g.lanes_d) & (kWave - 1);
        const VecD<VEC> pa = lane_values(in_a, prev);
        const Vec<VEC> pb = lane_values(in_b, prev);
        if (grp > 0) {
#pragma unroll
            for (int i = 0; i < VEC; ++i) pre.ex_a.v[i] = static_cast<float>(pa.v[i]);
            pre.ex_b = pb;
        }
    }

    // (4) the wave's pair into LDS, from the last group's lanes, which hold it
    if (grp == g.groups - 1) {
        sh.pair_a[wave][quad] = in_a;
        sh.pair_b[wave][quad] = in_b;
    }
    return pre;
}

// (6) once the state entering the tile is in LDS: the state entering this
// lane's positions, then replay and store.  Stores past L or D are dropped.
// When h_final is wanted, positions past L were made identity steps (see
// scan_registers), so the lane holding position L-1 ends its replay on the
// state there and writes it out.
template <typename S, int VEC, int T>
__device__ __forceinline__ void replay_from(const Geometry& g, Vec<VEC> hs, const TileSpot& s, int quad,
                                            const LanePrefix<VEC>& pre, const Reg<S, VEC> (&av)[T],
                                            const Reg<S, VEC> (&bv)[T]) {
    // hs: the state entering this wave's positions
#pragma unroll
    for (int i = 0; i < VEC; ++i) hs.v[i] = __builtin_fmaf(pre.ex_a.v[i], hs.v[i], pre.ex_b.v[i]);
#pragma unroll
    for (int j = 0; j < T; ++j) {
        const Vec<VEC> aj = widen<S, VEC>(rewiden_source<S, VEC>(av[j]));
        const Vec<VEC> bj = widen<S, VEC>(rewiden_source<S, VEC>(bv[j]));
#pragma unroll
        for (int i = 0; i < VEC; ++i) hs.v[i] = __builtin_fmaf(aj.v[i], hs.v[i], bj.v[i]);
        store_vec<S, VEC>(s.h.r, s.h.off + j * s.h.step, hs);
    }
    // the state after position L-1, written by the lane that holds it: an
    // unconditional store whose offset is out of range for every other lane
    // (and whose range is empty without h_final), so that every replay issues
    // the same number of memory operations
    const bool holds_last = g.h_final != nullptr && s.d_ok && s.tau0 <= g.L - 1 && g.L - 1 < s.tau0 + T;
    const __amdgpu_buffer_rsrc_t fr =
        make_range(g.h_final != nullptr ? g.h_final + s.row * g.D : nullptr, g.h_final != nullptr ? g.D * 4 : 0);
    const uint32_t foff = holds_last ? static_cast<uint32_t>((s.slab * g.slab_channels + quad * VEC) * 4) : kOutOfRange;
    store_vec<float, VEC>(fr, foff, hs);
}

template <typename S, int VEC, int T, int W>
__device__ __forceinline__ void replay_store(const Geometry& g, const TileShared<VEC, W>& sh, const TileSpot& s,
                                             int wave, int quad, const LanePrefix<VEC>& pre,
                                             const Reg<S, VEC> (&av)[T], const Reg<S, VEC> (&bv)[T]) {
    replay_from<S, VEC, T>(g, sh.pair_b[wave][quad], s, quad, pre, av, bv);
}

// (5) for slab channel c of the tile (one per lane; the caller has passed the
// hand-over barrier): fold the data waves' pairs into the tile pair, publish
// it, look back for the state entering the tile, publish the state leaving
// it, and replace each data wave's pair in LDS by the state entering that
// wave's positions.
//
// With a local carry (g.local_seqs > 0), `local` is this channel's LDS cell
// for the tile's sequence: it holds the state after the workgroup's previous
// tile of that sequence, which is the state entering this one, and receives
// the state after this tile.  `early`, when given, is the tile's
// decomposition, computed by the caller before the barrier.
template <typename S, int VEC, int W, bool AHEAD>
__device__ __forceinline__ void carry_channel(const S* __restrict__ a, const S* __restrict__ b, const Geometry& g,
                                              uint64_t* __restrict__ stat, TileShared<VEC, W>& sh, int c,
                                              uint32_t epoch, bool& recomputed, int64_t tile, const TileIndex* early,
                                              double* local) {
    if (c >= g.slab_channels) return;
    const TileIndex ix = early != nullptr ? *early : tile_index<S>(g, tile);
    const int64_t chunk = ix.chunk, seq = ix.seq, row = ix.row, slab = ix.slab;
    const int64_t d = slab * g.slab_channels + c;
    const double* pair_a = &sh.pair_a[0][0].v[0];
    float* pair_b = &sh.pair_b[0][0].v[0];
    double h_in = 0.0;
    if (d < g.D) {
        // the initial state is read only where it enters: chunk 0 here, or a
        // lookback that walks back past chunk 0 (a global load on every
        // tile would put its latency on each hand-over)
        if (chunk == 0) h_in = initial_state(g, row, d);
        if (g.local_seqs > 0) {
            if (chunk > 0) h_in = *local;
        } else if (g.nchunks > 1) {
            const bool has_successor = chunk + 1 < g.nchunks;
            const uint32_t tag_agg = (epoch << 2) | kKindAggregate;
            const uint32_t tag_inc = (epoch << 2) | kKindInclusive;
            const StatusArrays st = status_arrays(stat, g.nstatus);
            double ta = pair_a[c], tb = pair_b[c];
#pragma unroll
            for (int v = 1; v < W; ++v) {
                const double na = pair_a[v * kWave * VEC + c], nb = pair_b[v * kWave * VEC + c];
                tb = __builtin_fma(na, tb, nb);
                ta = na * ta;
            }
            // status entries are sequence-major: chunk j-1 of a sequence sits
            // slab_channels entries before chunk j
            const int64_t idx = (seq * g.nchunks + chunk) * g.slab_channels + c;
            if (chunk > 0) {
                if (has_successor) {
                    const float hi = static_cast<float>(ta);
                    publish(st.a_hi + idx, tag_agg, hi);
                    if constexpr (!product_in_one_word<S>())
                        publish(st.a_lo + idx, tag_agg, static_cast<float>(ta - static_cast<double>(hi)));
                    publish(st.b + idx, tag_agg, static_cast<float>(tb));
                }
                h_in = g.lookback_window > 2
                           ? lookback_channel<S, long_window<S>(), AHEAD, first_window<S>()>(
                                 a, b, g, row, d, st, idx, chunk, tag_agg, tag_inc, recomputed)
                           : lookback_channel<S, 2, AHEAD>(a, b, g, row, d, st, idx, chunk, tag_agg, tag_inc, recomputed);
            }
            if (has_successor) publish(st.p + idx, tag_inc, static_cast<float>(__builtin_fma(ta, h_in, tb)));
        }
    }
    double hv = h_in;
#pragma unroll
    for (int v = 0; v < W; ++v) {
        const int k = v * kWave * VEC + c;
        const double na = pair_a[k], nb = pair_b[k];
        pair_b[k] = static_cast<float>(hv);
        hv = __builtin_fma(na, hv, nb);
    }
    if (g.local_seqs > 0) *local = hv;
}

// LDS cells of the local carry: [sequence slot][slab channel].
template <int VEC>
struct LocalCarry {
    double h[kMaxLocalSeqs][kWave * VEC];
};

// ---------------------------------------------------------------------------
// Relay: persistent workgroups whose carry stays local, with the group scan
// moved from the data waves to the carry wave and the carry one tile behind.
//
// A workgroup whose tiles are chunks 0, 1, ... of its own local_seqs = m
// sequences (tile k of the workgroup: chunk k / m of its sequence k mod m)
// needs no status words.  Each data-wave lane composes its own T positions
// into one pair and puts it into LDS; the carry wave folds the W * G pairs of
// each slab channel in the order of their positions, in fp64, from the state
// entering the tile, and writes back, in place of each lane's B, the state
// entering that lane's positions (rounded to fp32 once).  In step k the data
// waves put tile k's pairs into LDS slot k & 1, pass one barrier, then replay
// tile k-1 from the states that the carry wave wrote into slot (k-1) & 1
// during step k-1; after the same barrier the carry wave turns tile k's pairs
// into its entering states.  One barrier per tile, and neither a group scan
// nor the carry sits on the data waves' path.  Their register buffers rotate
// through three tiles: the one whose pairs are formed, the one replayed, and
// the next, whose loads are in flight.  The tiles' positions advance by counting, so
// no division by the sequence count sits in the loop.
struct LocalPos {
    int64_t chunk;
    int j;   // which of the workgroup's sequences
};

__device__ __forceinline__ LocalPos advance(LocalPos p, int m) {
    return p.j + 1 == m ? LocalPos{p.chunk + 1, 0} : LocalPos{p.chunk, p.j + 1};
}

// The decomposition of the workgroup's tile at position p: with one sequence
// per workgroup it never changes (s0); otherwise the slot's sequence, batch
// row and slab are recomputed (32-bit: there are fewer than 2^31 tiles).
struct LocalSeqs {
    TileIndex s0;
};

template <typename S>
__device__ __forceinline__ TileIndex local_index(const Geometry& g, const LocalSeqs& ls, LocalPos p) {
    if (g.local_seqs == 1) {
        TileIndex r = ls.s0;
        r.chunk = p.chunk;
        return r;
    }
    const uint32_t slot = static_cast<uint32_t>(blockIdx.x) + static_cast<uint32_t>(p.j) * gridDim.x;
    const uint32_t seq = static_cast<uint32_t>(sequence_of(g, slot));
    const uint32_t nslab = static_cast<uint32_t>(g.nslab);
    const uint32_t row = seq / nslab;
    return TileIndex{p.chunk, seq, row, seq - row * nslab};
}

template <typename S>
__device__ __forceinline__ LocalSeqs local_sequences(const Geometry& g) {
    return LocalSeqs{tile_index<S>(g, blockIdx.x)};
}

// The spots of one local-carry sequence's full tiles differ only in where
// each operand's descriptor starts: chunk c's start lies c * delta bytes after
// chunk 0's (before it, in reverse: delta < 0); offsets, steps and ranges are
// the same.  A ragged last chunk is located in full.  With one sequence per
// workgroup this replaces each tile's 64-bit offset arithmetic by one scalar
// multiply-add per operand.
struct SeqWalk {
    TileSpot s0;                        // chunk 0
    const char *a0, *b0, *h0;           // chunk 0's descriptor bases
    int64_t da, db, dh;                 // their advance per chunk, in bytes
    int nrec_a, nrec_b, nrec_h;         // range of a full tile
    int64_t ragged;                     // chunk located in full (nchunks when none)
};

template <typename S>
__device__ __forceinline__ SeqWalk seq_walk(const S* a, const S* b, S* h, const Geometry& g, const TileIndex& ix0,
                                            int wave, int quad, int grp, int vec, int T) {
    SeqWalk w;
    TileIndex i0 = ix0;
    i0.chunk = 0;
    w.s0 = locate_at<S>(a, b, h, g, i0, wave, quad, grp, vec, T);
    constexpr int64_t es = storage_bytes<S>();
    const int64_t steps = g.steps_per_tile;
    const int64_t dir = g.reverse ? -1 : 1;
    // chunk 0's range starts at time step 0 (forward) or L - steps (reverse) of the batch row
    const int64_t t0 = g.reverse ? g.L - steps : 0;
    w.a0 = reinterpret_cast<const char*>(a + w.s0.row * g.a_sb + t0 * g.a_sl);
    w.b0 = reinterpret_cast<const char*>(b + w.s0.row * g.b_sb + t0 * g.b_sl);
    w.h0 = reinterpret_cast<const char*>(h + w.s0.row * g.h_sb + t0 * g.h_sl);
    w.da = dir * steps * g.a_sl * es;
    w.db = dir * steps * g.b_sl * es;
    w.dh = dir * steps * g.h_sl * es;
    auto nrec = [&](int64_t sl) {
        const int64_t bytes = ((steps - 1) * sl + g.D) * es;
        return static_cast<int>(bytes < kMaxRange ? bytes : kMaxRange);
    };
    w.nrec_a = nrec(g.a_sl);
    w.nrec_b = nrec(g.b_sl);
    w.nrec_h = nrec(g.h_sl);
    w.ragged = g.L % steps != 0 ? g.nchunks - 1 : g.nchunks;
    return w;
}

template <typename S>
__device__ __forceinline__ TileSpot walk_spot(const S* a, const S* b, S* h, const Geometry& g, const SeqWalk& w,
                                              const TileIndex& ix0, int64_t chunk, int wave, int quad, int grp,
                                              int vec, int T) {
    if (chunk == w.ragged) {
        TileIndex i = ix0;
        i.chunk = chunk;
        return locate_at<S>(a, b, h, g, i, wave, quad, grp, vec, T);
    }
    TileSpot s = w.s0;
    s.chunk = chunk;
    s.tau0 = w.s0.tau0 + chunk * g.steps_per_tile;
    s.a.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(w.a0 + chunk * w.da), 0, w.nrec_a, kBufferConfig);
    s.b.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(w.b0 + chunk * w.db), 0, w.nrec_b, kBufferConfig);
    s.h.r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(w.h0 + chunk * w.dh), 0, w.nrec_h, kBufferConfig);
    return s;
}

// The spot of the workgroup's tile at position p.
template <typename S>
__device__ __forceinline__ TileSpot local_spot(const S* a, const S* b, S* h, const Geometry& g, const LocalSeqs& ix,
                                               const SeqWalk& w, LocalPos p, int wave, int quad, int grp, int vec,
                                               int T) {
    if (g.local_seqs == 1) return walk_spot<S>(a, b, h, g, w, ix.s0, p.chunk, wave, quad, grp, vec, T);
    return locate_at<S>(a, b, h, g, local_index<S>(g, ix, p), wave, quad, grp, vec, T);
}

// (2) of the relay: a lane's pair of its T positions, into LDS at
// [wave][lane] (lane = group * P + quad).  Without h_init the state before
// position 0 is zero, so that position's a never contributes: use 0 for it
// (1 in the form with the decays ahead, where h_init enters with decay 1).
// With h_final, positions past L become identity steps (see scan_registers).
template <typename S, int VEC, int T, int W, bool AHEAD>
__device__ __forceinline__ void lane_pair(const Geometry& g, TileShared<VEC, W>& sh, const TileSpot& s, int lane,
                                          int wave, Reg<S, VEC> (&av)[T], Reg<S, VEC> (&bv)[T]) {
    if (s.tau0 == 0 && g.h_init == nullptr) set_reg<S, VEC>(av[0], 0.0f);
    else if (AHEAD && s.tau0 == 0) set_reg<S, VEC>(av[0], 1.0f);
    if (g.h_final != nullptr && (s.chunk + 1) * g.steps_per_tile > g.L) {
#pragma unroll
        for (int j = 0; j < T; ++j) {
            if (s.tau0 + j >= g.L) {
                set_reg<S, VEC>(av[j], 1.0f);
                set_reg<S, VEC>(bv[j], 0.0f);
            }
        }
    }
    Vec<VEC> in_b = widen<S, VEC>(bv[0]);
#pragma unroll
    for (int j = 1; j < T; ++j) {
        const Vec<VEC> aj = widen<S, VEC>(av[j]), bj = widen<S, VEC>(bv[j]);
#pragma unroll
        for (int i = 0; i < VEC; ++i) in_b.v[i] = __builtin_fmaf(aj.v[i], in_b.v[i], bj.v[i]);
    }
    VecD<VEC> in_a;
    {
        Vec<VEC> aw[T];
#pragma unroll
        for (int j = 0; j < T; ++j) aw[j] = widen<S, VEC>(av[j]);
#pragma unroll
        for (int i = 0; i < VEC; ++i) in_a.v[i] = decay_product<0, T>(aw, i);
    }
    sh.pair_a[wave][lane] = in_a;
    sh.pair_b[wave][lane] = in_b;
}

// (6) of the relay: replay from the state entering the lane's positions,
// which the carry wave left at [wave][lane].  Stores past L or D are dropped.
template <typename S, int VEC, int T, int W>
__device__ __forceinline__ void replay_lane(const Geometry& g, const TileShared<VEC, W>& sh, const TileSpot& s,
                                            int wave, int lane, int quad, const Reg<S, VEC> (&av)[T],
                                            const Reg<S, VEC> (&bv)[T]) {
    LanePrefix<VEC> none;
    none.ex_a = splat<VEC>(1.0f);
    none.ex_b = splat<VEC>(0.0f);
    replay_from<S, VEC, T>(g, sh.pair_b[wave][lane], s, quad, none, av, bv);
}

// One step of the relay's data waves: loads of tile k+1 into (la, lb) (past
// the workgroup's last tile every offset is out of range), the pairs of tile
// k (loaded one step earlier, in (sa, sb)) into LDS slot k & 1, the barrier,
// the replay of tile k-1 (in (ra, rb)).  In step 0 the replay runs with every
// store out of range, so that every step issues the same memory operations
// and the compiler's waits for each tile's loads stay exact.
template <typename S, int VEC, int T, int W, bool AHEAD>
__device__ __forceinline__ void relay_step(const S* __restrict__ a, const S* __restrict__ b, S* __restrict__ h,
                                           const Geometry& g, TileShared<VEC, W> (&sh)[2], const LocalSeqs& ix,
                                           const SeqWalk& sw, int lane, int wave, int quad, int grp, int64_t k,
                                           int64_t n, LocalPos pk, Reg<S, VEC> (&sa)[T], Reg<S, VEC> (&sb)[T],
                                           const Reg<S, VEC> (&ra)[T], const Reg<S, VEC> (&rb)[T],
                                           Reg<S, VEC> (&la)[T], Reg<S, VEC> (&lb)[T]) {
    const int m = g.local_seqs;
    {
        const LocalPos p1 = advance(pk, m);
        TileSpot ns = local_spot<S>(a, b, h, g, ix, sw, k + 1 < n ? p1 : pk, wave, quad, grp, VEC, T);
        if (k + 1 >= n) ns.a.off = ns.b.off = kOutOfRange;
        load_tile<S, VEC, T, AHEAD>(la, lb, ns);
    }
    const TileSpot s = local_spot<S>(a, b, h, g, ix, sw, pk, wave, quad, grp, VEC, T);
    lane_pair<S, VEC, T, W, AHEAD>(g, sh[k & 1], s, lane, wave, sa, sb);
    __syncthreads();   // tile k's pairs are in slot k & 1; tile k-1's entering states in the other
    const bool have_prev = k >= 1;
    const LocalPos pp = LocalPos{pk.j == 0 ? pk.chunk - 1 : pk.chunk, pk.j == 0 ? m - 1 : pk.j - 1};
    TileSpot rs = local_spot<S>(a, b, h, g, ix, sw, have_prev ? pp : pk, wave, quad, grp, VEC, T);
    if (!have_prev) {
        rs.h.off = kOutOfRange;
        rs.d_ok = false;   // no final-state store either
    }
    replay_lane<S, VEC, T, W>(g, sh[(k - 1) & 1], rs, wave, lane, quad, ra, rb);
}

// A replay whose stores are all out of range (nothing is written): issues the
// memory operations of one replay.
template <typename S, int VEC, int T, int W>
__device__ __forceinline__ void idle_replay(const Geometry& g, const TileShared<VEC, W>& sh, TileSpot s, int wave,
                                            int lane, int quad, const Reg<S, VEC> (&ra)[T],
                                            const Reg<S, VEC> (&rb)[T]) {
    s.h.off = kOutOfRange;
    s.d_ok = false;
    replay_lane<S, VEC, T, W>(g, sh, s, wave, lane, quad, ra, rb);
}

// The relay's data waves.  Three register buffers rotate: step k forms the
// pairs of buffer k % 3, replays buffer (k-1) % 3 and loads tile k+1 into
// buffer (k+1) % 3 (which held tile k-2).  (Four buffers with the loads two
// tiles ahead measured 1-2% slower at B=32 L=4096 D=256 and fill the VGPRs
// at 8 positions x 4 channels.)  A local carry has at least two chunks per
// sequence, so every workgroup has n >= 2 tiles.
template <typename S, int VEC, int T, int W, bool AHEAD>
__device__ __forceinline__ void relay_data_waves(const S* __restrict__ a, const S* __restrict__ b,
                                                 S* __restrict__ h, const Geometry& g, TileShared<VEC, W> (&sh)[2],
                                                 int lane, int wave, int quad, int grp) {
    const int m = g.local_seqs;
    const int64_t n = g.nchunks * m;
    const LocalSeqs ix = local_sequences<S>(g);
    const SeqWalk sw = seq_walk<S>(a, b, h, g, ix.s0, wave, quad, grp, VEC, T);
    Reg<S, VEC> a0[T], b0[T], a1[T], b1[T], a2[T], b2[T];
    // the replays before the first tile's (preamble and step 0) read buffer 2
    // and store nothing; give them defined values
#pragma unroll
    for (int j = 0; j < T; ++j) {
        set_reg<S, VEC>(a2[j], 0.0f);
        set_reg<S, VEC>(b2[j], 0.0f);
    }
    LocalPos pk{0, 0};
    {
        // the loop is entered with what every step leaves in flight: a tile's
        // loads, then a replay's stores
        const TileSpot s0 = local_spot<S>(a, b, h, g, ix, sw, pk, wave, quad, grp, VEC, T);
        load_tile<S, VEC, T, AHEAD>(a0, b0, s0);
        idle_replay<S, VEC, T, W>(g, sh[1], s0, wave, lane, quad, a2, b2);
    }
    int64_t k = 0;
    for (;;) {
        relay_step<S, VEC, T, W, AHEAD>(a, b, h, g, sh, ix, sw, lane, wave, quad, grp, k, n, pk, a0, b0, a2, b2, a1, b1);
        pk = advance(pk, m);
        if (++k >= n) break;
        relay_step<S, VEC, T, W, AHEAD>(a, b, h, g, sh, ix, sw, lane, wave, quad, grp, k, n, pk, a1, b1, a0, b0, a2, b2);
        pk = advance(pk, m);
        if (++k >= n) break;
        relay_step<S, VEC, T, W, AHEAD>(a, b, h, g, sh, ix, sw, lane, wave, quad, grp, k, n, pk, a2, b2, a1, b1, a0, b0);
        pk = advance(pk, m);
        if (++k >= n) break;
    }
    __syncthreads();   // the last tile's entering states are in slot (n-1) & 1
    // replay of tile n-1, whose buffer is the one the last step formed
    const LocalPos pl = LocalPos{pk.j == 0 ? pk.chunk - 1 : pk.chunk, pk.j == 0 ? m - 1 : pk.j - 1};
    const TileSpot rs = local_spot<S>(a, b, h, g, ix, sw, pl, wave, quad, grp, VEC, T);
    TileShared<VEC, W>& last_slot = sh[(n - 1) & 1];
    const int last = static_cast<int>((n - 1) % 3);
    if (last == 0) replay_lane<S, VEC, T, W>(g, last_slot, rs, wave, lane, quad, a0, b0);
    else if (last == 1) replay_lane<S, VEC, T, W>(g, last_slot, rs, wave, lane, quad, a1, b1);
    else replay_lane<S, VEC, T, W>(g, last_slot, rs, wave, lane, quad, a2, b2);
}

// (5) of the relay, for slab channel c (c < slab_channels <= 64: one carry
// wave): fold the tile's lane pairs in the order of their positions, from the
// state entering the tile (h_init or zero for chunk 0, else this channel's
// local cell), replacing each lane's B by the state entering that lane's
// positions; the state after the tile goes back into the local cell.  The
// pairs are read in batches of 8 so that their LDS latency is paid once per
// batch, not once per pair.
template <int VEC, int W>
__device__ __forceinline__ void relay_carry(const Geometry& g, TileShared<VEC, W>& sh, int c, const TileIndex& ix,
                                            double* local) {
    if (c >= g.slab_channels) return;
    const int64_t d = ix.slab * g.slab_channels + c;
    double hv = 0.0;
    if (d < g.D) hv = ix.chunk == 0 ? initial_state(g, ix.row, d) : *local;
    const double* pa = &sh.pair_a[0][0].v[0];
    float* pb = &sh.pair_b[0][0].v[0];
    const int G = g.groups, P = g.lanes_d;
    constexpr int kBatch = 8;
#pragma unroll
    for (int v = 0; v < W; ++v) {
        for (int g0 = 0; g0 < G; g0 += kBatch) {
            double ra[kBatch];
            float rb[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                const int gr = g0 + j < G ? g0 + j : G - 1;
                const int k = (v * kWave + gr * P) * VEC + c;
                ra[j] = pa[k];
                rb[j] = pb[k];
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (g0 + j < G) {
                    const int k = (v * kWave + (g0 + j) * P) * VEC + c;
                    pb[k] = static_cast<float>(hv);
                    hv = __builtin_fma(ra[j], hv, static_cast<double>(rb[j]));
                }
            }
        }
    }
    *local = hv;
}

template <typename S, int VEC, int W>
__device__ __forceinline__ void relay_carry_wave(const Geometry& g, TileShared<VEC, W> (&sh)[2],
                                                 LocalCarry<VEC>& local, int c) {
    const int m = g.local_seqs;
    const int64_t n = g.nchunks * m;
    const LocalSeqs ix = local_sequences<S>(g);
    LocalPos pk{0, 0};
    for (int64_t k = 0; k < n; ++k) {
        const TileIndex t = local_index<S>(g, ix, pk);
        __syncthreads();   // tile k's pairs are in slot k & 1
        relay_carry<VEC, W>(g, sh[k & 1], c, t, &local.h[pk.j][c]);
        pk = advance(pk, m);
    }
    __syncthreads();   // pairs with the data waves' last barrier
}

// Data wave, one tile of the persistent loop: start the loads of the
// workgroup's next tile into (nav, nbv), scan the tile whose inputs are in
// (av, bv), hand the wave's pair to the carry wave, and once the carry is in,
// replay and store.
template <typename S, int VEC, int T, int W, bool AHEAD>
__device__ __forceinline__ void data_tile(const S* __restrict__ a, const S* __restrict__ b, S* __restrict__ h,
                                          const Geometry& g, TileShared<VEC, W>& sh, int lane, int wave, int quad,
                                          int grp, int64_t tile, Reg<S, VEC> (&av)[T], Reg<S, VEC> (&bv)[T],
                                          int64_t next, Reg<S, VEC> (&nav)[T], Reg<S, VEC> (&nbv)[T]) {
    // (1) the next tile's loads stay in flight while this tile is scanned,
    // waits for its carry and is stored.  They are issued even when there is
    // no next tile (then every lane's offset is out of range and nothing is
    // read), so that every step issues the same memory operations and the
    // compiler can count exactly which loads a step has to wait for.
    {
        TileSpot ns = locate<S>(a, b, h, g, next < g.ntiles ? next : tile, wave, quad, grp, VEC, T);
        if (next >= g.ntiles) ns.a.off = ns.b.off = kOutOfRange;
        load_tile<S, VEC, T, AHEAD>(nav, nbv, ns);
    }
    const TileSpot s = locate<S>(a, b, h, g, tile, wave, quad, grp, VEC, T);
    const LanePrefix<VEC> pre = scan_registers<S, VEC, T, W, AHEAD>(g, sh, s, lane, wave, quad, grp, av, bv);
    __syncthreads();   // wave pairs are in LDS
    __syncthreads();   // the carry wave has written the states entering the waves
    replay_store<S, VEC, T, W>(g, sh, s, wave, quad, pre, av, bv);
}

// Most threads a workgroup of W data waves and up to VEC carry waves may have
// (the host never launches more than 1024).
constexpr int group_limit(int w, int vec) { return (w + vec) * kWave < 1024 ? (w + vec) * kWave : 1024; }

// Persistent workgroup of W data waves and carry_waves (<= VEC) carry waves.
// Tiles blockIdx, blockIdx + grid, ... are taken in order; every wave runs the
// same number of tiles and meets the same two barriers per tile.  Carry waves
// issue no data loads or stores, so their status polls never queue behind the
// data traffic (loads and stores retire in order per wave).
template <typename S, int VEC, int T, int W, bool AHEAD>
__global__ void __launch_bounds__(group_limit(W, VEC))
scan_tiles(const S* __restrict__ a, const S* __restrict__ b, S* __restrict__ h,
           Geometry g, WorkspaceHeader* __restrict__ hdr, uint64_t* __restrict__ stat) {
    __shared__ TileShared<VEC, W> sh;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const bool chained = g.nchunks > 1 && g.local_seqs == 0;
    const int64_t stride = gridDim.x;

    if (wave >= W) {
        __shared__ LocalCarry<VEC> local;
        const int carry = wave - W;
        const int c = carry * kWave + lane;
        uint32_t epoch = 0, before = 0;
        if (chained) {
            epoch = call_epoch(hdr);
            if (carry == 0) before = count_in(hdr, epoch, lane);
        }
        bool recomputed = false;
        int slot = 0;   // sequence slot of the local carry: tiles cycle through local_seqs sequences
        for (int64_t tile = blockIdx.x; tile < g.ntiles; tile += stride) {
            // The tile's decomposition is a long instruction sequence.  With at
            // most 2 data waves every wave of the workgroup has a SIMD of its
            // own, so it runs while the data waves scan instead of between the
            // barriers, where they wait for it (measured: 2-3% off the B=32
            // L=4096 D=256 and B=8 L=16384 D=1024 fp32 scans).  With more data
            // waves the carry waves share their SIMDs, and there it cost the
            // data waves about 1% (B=16 L=512 D=8192).
            double* cell = &local.h[slot][c % (kWave * VEC)];
            if constexpr (W <= 2) {
                const TileIndex ix = tile_index<S>(g, tile);
                __syncthreads();   // wave pairs are in LDS
                carry_channel<S, VEC, W, AHEAD>(a, b, g, stat, sh, c, epoch, recomputed, tile, &ix, cell);
            } else {
                __syncthreads();   // wave pairs are in LDS
                carry_channel<S, VEC, W, AHEAD>(a, b, g, stat, sh, c, epoch, recomputed, tile, nullptr, cell);
            }
            if (g.local_seqs > 0 && ++slot == g.local_seqs) slot = 0;
            __syncthreads();   // the states entering the waves are in LDS
        }
        if (!chained) return;
        if (__ballot(recomputed) != 0 && lane == 0)
            __hip_atomic_fetch_add(&hdr->timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // after the tile loop's barriers, which every carry wave (each reads
        // the epoch) has passed; a workgroup without tiles passes none, but
        // then its carry waves touch no status word
        if (carry == 0) count_done(hdr, epoch, before, lane);
        return;
    }

    const int quad = lane & (g.lanes_d - 1);
    const int grp = lane >> g.log2_lanes_d;
    // two register buffers: one tile being scanned, the next one loading.  The
    // first step is peeled so that both ways into the loop start right after
    // the same step, with the same loads and stores in flight.  (The compiler
    // folds the exit between the two steps into the loop header, whose wait
    // then lets the current tile's loads land before the next tile's are
    // issued on every other step; a loop that checks its exit once per two
    // tiles avoids that wait and measured no faster, so this form stays.)
    Reg<S, VEC> a0[T], b0[T], a1[T], b1[T];
    int64_t tile = blockIdx.x;
    if (tile >= g.ntiles) return;
    load_tile<S, VEC, T, AHEAD>(a0, b0, locate<S>(a, b, h, g, tile, wave, quad, grp, VEC, T));
    data_tile<S, VEC, T, W, AHEAD>(a, b, h, g, sh, lane, wave, quad, grp, tile, a0, b0, tile + stride, a1, b1);
    tile += stride;
    while (tile < g.ntiles) {
        data_tile<S, VEC, T, W, AHEAD>(a, b, h, g, sh, lane, wave, quad, grp, tile, a1, b1, tile + stride, a0, b0);
        tile += stride;
        if (tile >= g.ntiles) break;
        data_tile<S, VEC, T, W, AHEAD>(a, b, h, g, sh, lane, wave, quad, grp, tile, a0, b0, tile + stride, a1, b1);
        tile += stride;
    }
}

// Relay workgroup: W data waves and one carry wave (slabs of at most 64
// channels), launched only with a grid that keeps the carry local
// (g.local_seqs > 0, g.nchunks > 1): workgroup k takes sequences k, k + grid,
// ... (through sequence_of), chunk by chunk.
template <typename S, int VEC, int T, int W, bool AHEAD>
__global__ void __launch_bounds__((W + 1) * kWave)
scan_relay(const S* __restrict__ a, const S* __restrict__ b, S* __restrict__ h, Geometry g) {
    __shared__ TileShared<VEC, W> sh[2];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (wave >= W) {
        __shared__ LocalCarry<VEC> local;
        relay_carry_wave<S, VEC, W>(g, sh, local, lane);
        return;
    }
    relay_data_waves<S, VEC, T, W, AHEAD>(a, b, h, g, sh, lane, wave, lane & (g.lanes_d - 1),
                                          lane >> g.log2_lanes_d);
}

// One tile per workgroup (grid = number of tiles) of W data waves and
// carry_waves carry waves: the data waves load, scan in registers and hand
// over through LDS; the carry waves look back for the tile's channels, one
// per lane; the data waves replay and store.  Keeping the lookback out of the
// data waves keeps their register count down.  While a workgroup looks back
// its CU has no loads of its own in flight; other CUs load meanwhile (measured
// on gfx950: one 16-wave workgroup per CU at a time, tiles starting in the
// order their lookbacks end).
template <typename S, int VEC, int T, int W, bool AHEAD>
__global__ void __launch_bounds__(group_limit(W, VEC))
scan_one(const S* __restrict__ a, const S* __restrict__ b, S* __restrict__ h,
         Geometry g, WorkspaceHeader* __restrict__ hdr, uint64_t* __restrict__ stat) {
    __shared__ TileShared<VEC, W> sh;

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int64_t tile = blockIdx.x;
    const bool chained = g.nchunks > 1;

    if (wave >= W) {
        const int carry = wave - W;
        uint32_t epoch = 0, before = 0;
        if (chained) {
            epoch = call_epoch(hdr);
            if (carry == 0) before = count_in(hdr, epoch, lane);
        }
        bool recomputed = false;
        const TileIndex ix = tile_index<S>(g, tile);   // while the data waves wait for their loads
        __syncthreads();   // wave pairs are in LDS
        carry_channel<S, VEC, W, AHEAD>(a, b, g, stat, sh, carry * kWave + lane, epoch, recomputed, tile, &ix, nullptr);
        __syncthreads();   // the states entering the waves are in LDS
        if (!chained) return;
        if (__ballot(recomputed) != 0 && lane == 0)
            __hip_atomic_fetch_add(&hdr->timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (carry == 0) count_done(hdr, epoch, before, lane);
        return;
    }

    const int quad = lane & (g.lanes_d - 1);
    const int grp = lane >> g.log2_lanes_d;
    const TileSpot s = locate<S>(a, b, h, g, tile, wave, quad, grp, VEC, T);
    Reg<S, VEC> av[T], bv[T];
    load_tile<S, VEC, T, AHEAD>(av, bv, s);
    const LanePrefix<VEC> pre = scan_registers<S, VEC, T, W, AHEAD>(g, sh, s, lane, wave, quad, grp, av, bv);
    __syncthreads();   // wave pairs are in LDS
    __syncthreads();   // the states entering the waves are in LDS
    replay_store<S, VEC, T, W>(g, sh, s, wave, quad, pre, av, bv);
}


}  // namespace linrec
