// call_epoch.hpp -- call epochs of a lookback workspace.
//
// A lookback workspace is reused from call to call without being cleared:
// every status word carries the epoch of the call that wrote it, and a call
// accepts only words of its own epoch.  This header keeps the epoch of the
// current call and advances it once per call.  It is written once, over an
// `Atomics` policy: the kernels use agent-scope atomics, and a host model
// (tests/epoch_model.hip) runs the same functions under random interleavings
// of their atomic steps.
//
// Layout: kDoneSlots slot lines of 128 bytes.  Word 0 of a line counts the
// workgroups of the current call that hold the epoch; word 1 is the epoch.
// One more word, `finished`, counts the lines filled in the current call.
//
// Protocol, for workgroup k of a grid of G:
//   1. every wave that needs the epoch reads it from k's slot line
//      (epoch_of_call); the waves of one workgroup may read it at any time
//      before step 3;
//   2. one wave counts the workgroup into the line (epoch_count_in), with an
//      addend computed from the epoch it read, so the count cannot be
//      performed before that read has returned;
//   3. after every wave of the workgroup has read the epoch (a barrier), the
//      counting wave calls epoch_count_done with step 2's result.  The
//      workgroup that fills a line clears its count and counts the line into
//      `finished`; the one that fills `finished` clears it and gets `true`,
//      and then writes the next epoch into every line (epoch_advance).
// Every workgroup of the call has read its epoch before the last one reaches
// step 3, so none can see the next one; the next call on the stream cannot
// start before this one has ended, so the order of the workgroups does not
// matter.  Workgroup k belongs to line k * kDoneSlots / G: contiguous ranges,
// so lines fill one after another during the call instead of all at its end,
// and same-address traffic stays rare.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linrec {

constexpr int kLineWords = 32;                // uint32 words per 128-byte line
constexpr int kDoneSlots = 256;               // slot lines
constexpr uint32_t kEpochMask = 0x3fffffffu;  // epochs stay below 2^30

// Slot line of workgroup `group` of a grid of `groups`.
__host__ __device__ constexpr int64_t slot_of(int64_t group, int64_t groups) { return group * kDoneSlots / groups; }

// First workgroup of line `slot`: ceil(slot * groups / kDoneSlots).
__host__ __device__ constexpr int64_t slot_begin(int64_t slot, int64_t groups) {
    return (slot * groups + kDoneSlots - 1) / kDoneSlots;
}

// Workgroups that count into line `slot`.
__host__ __device__ constexpr uint32_t slot_members(int64_t slot, int64_t groups) {
    return static_cast<uint32_t>(slot_begin(slot + 1, groups) - slot_begin(slot, groups));
}

// Lines that a grid of `groups` fills (every one of them has a member).
__host__ __device__ constexpr uint32_t slot_lines(int64_t groups) {
    return static_cast<uint32_t>(groups < kDoneSlots ? groups : kDoneSlots);
}

__host__ __device__ constexpr uint32_t next_epoch(uint32_t epoch) { return (epoch + 1u) & kEpochMask; }

struct EpochWords {
    uint32_t* lines;      // kDoneSlots lines of kLineWords words
    uint32_t* finished;   // lines filled in the current call
};

// Step 1: the epoch of the current call, read from the workgroup's line.
template <class Atomics>
__host__ __device__ inline uint32_t epoch_of_call(const EpochWords& w, int64_t group, int64_t groups) {
    return Atomics::load(w.lines + slot_of(group, groups) * kLineWords + 1);
}

// Step 2: count the workgroup into its line (the addend is 1, since epochs
// stay below 2^30).  Returns the count before the addition.
template <class Atomics>
__host__ __device__ inline uint32_t epoch_count_in(const EpochWords& w, int64_t group, int64_t groups,
                                                   uint32_t epoch) {
    return Atomics::add(w.lines + slot_of(group, groups) * kLineWords, 1u + (epoch >> 30));
}

// Step 3: `before` is epoch_count_in's result.  True for the one workgroup of
// the call that must then call epoch_advance.
template <class Atomics>
__host__ __device__ inline bool epoch_count_done(const EpochWords& w, int64_t group, int64_t groups,
                                                 uint32_t before) {
    const int64_t slot = slot_of(group, groups);
    if (before + 1 != slot_members(slot, groups)) return false;
    Atomics::store(w.lines + slot * kLineWords, 0u);
    const uint32_t filled = Atomics::add(w.finished, 1u);
    if (filled + 1 != slot_lines(groups)) return false;
    Atomics::store(w.finished, 0u);
    return true;
}

// Write the next epoch into lines first, first + step, ... (a wave passes its
// lane and its width; one thread passes 0 and 1).
template <class Atomics>
__host__ __device__ inline void epoch_advance(const EpochWords& w, uint32_t epoch, int first, int step) {
    for (int k = first; k < kDoneSlots; k += step) Atomics::store(w.lines + k * kLineWords + 1, next_epoch(epoch));
}

}  // namespace linrec
