// scratch_state.hpp -- which chained-carry state of a scratch buffer a call
// may trust, and what it must clear first.  Plain C++ (no HIP): the C ABI
// turns a plan into fill kernels, and a host-only test drives the same code.
//
// Tickets (the scratch header) and tile descriptors (the front of the body)
// stay valid from launch to launch because every word carries the epoch of
// the launch that wrote it.  Three things break that:
//   * data of another layout written over a descriptor range (the
//     three-pass block sums, the radix rows);
//   * a buffer whose contents the library has never seen;
//   * a call recorded into a HIP graph.  The host decides what to clear when
//     the call is enqueued, but a graph replays its calls later, any number
//     of times, after whatever ran on the buffer in between -- and the eager
//     calls around it cannot see the replays either.  So a buffer that has
//     been used under capture is never trusted again: every later call on it,
//     captured or not, clears the header and all the state it reads (which
//     also restarts the epochs, so no stale descriptor can carry a live tag).
//
// Kinds of what a call leaves in the body:
//   ZERO  -- libscan_scratch_init zeroed the header; no body byte is trusted.
//   DESC  -- descriptors of the look-back scans, segmented scans, compaction
//            or runs in the first `state` body bytes: valid for any of those,
//            a larger call clears only the extra range.
//   RADIX -- the radix layout for one (n, bits per pass): valid only for the
//            same pair.
//   DATA  -- block sums or other data over the body: nothing valid.
// After 2^29 launches on one buffer the state is cleared too, long before
// the 30-bit epoch in the descriptors could repeat.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <mutex>
#include <unordered_map>
#include <unordered_set>

namespace libscan {

enum StateKind { kKindNone = 0, kKindZero = 1, kKindDesc = 2, kKindRadix = 3, kKindData = 4 };

struct StateRecord {
    int kind;              // StateKind of the last call (kKindNone: unknown buffer)
    uint64_t sig;          // RADIX: (n << 3) | bits per pass
    size_t state;          // body bytes of valid state from the front
    uint64_t launches;     // launches since the last full clear
};

// What to clear before the call's kernels run.  header: the 256-byte header
// and body bytes [0, state); else body bytes [from, from + bytes), nothing
// when bytes is 0.
struct ClearPlan {
    bool header;
    size_t from, bytes;
};

constexpr uint64_t kMaxLaunchesBetweenClears = 1ull << 29;

// The decision for one call of `kind` that reads `state` body bytes of
// state and makes `launches` chained-carry launches, on a buffer whose last
// call left `prev`.  `never_trust`: the buffer has been used under capture.
// Returns the plan; *next is the record to keep once the plan's clears and
// the call's launches are enqueued.
inline ClearPlan plan_call(const StateRecord &prev, bool never_trust, int kind, uint64_t sig,
                           size_t state, uint64_t launches, StateRecord *next)
{
    if (kind == kKindData) {
        *next = StateRecord{kKindData, 0, 0, prev.launches};
        return ClearPlan{false, 0, 0};
    }
    const bool fresh_epochs =
        prev.kind != kKindNone && prev.launches + launches < kMaxLaunchesBetweenClears;
    size_t valid = 0;          // body bytes this call may trust as they are
    bool header_ok = false;
    if (!never_trust && fresh_epochs) {
        if (prev.kind == kKindZero || (prev.kind == kKindDesc && kind == kKindDesc)) {
            header_ok = true;
            valid = prev.state;
        } else if (prev.kind == kKindRadix && kind == kKindRadix && prev.sig == sig) {
            header_ok = true;
            valid = state;
        }
    }
    *next = StateRecord{kind, sig, state, prev.launches + launches};
    if (!header_ok) {
        next->launches = launches;
        return ClearPlan{true, 0, state};
    }
    if (valid < state)
        return ClearPlan{false, valid, state - valid};
    if (kind == kKindDesc)
        next->state = valid;   // the larger valid range stays valid
    return ClearPlan{false, 0, 0};
}

// The records of every scratch buffer a caller has passed, by address.
// Forgetting a record is safe (the next call on that buffer clears), so the
// table is emptied when it grows large; the set of buffers used under
// capture is kept, since forgetting one of those would let an eager call
// trust state that a later replay overwrites.
class StateTable {
public:
    static constexpr size_t kMaxTracked = 4096;

    ClearPlan prepare(uintptr_t key, int kind, uint64_t sig, size_t state, uint64_t launches,
                      bool capturing)
    {
        std::lock_guard<std::mutex> lock(mu_);
        if (records_.size() > kMaxTracked)
            records_.clear();
        if (capturing)
            captured_.insert(key);
        StateRecord prev{kKindNone, 0, 0, 0};
        auto it = records_.find(key);
        if (it != records_.end())
            prev = it->second;
        StateRecord next;
        const ClearPlan p = plan_call(prev, captured_.count(key) != 0, kind, sig, state, launches,
                                      &next);
        records_[key] = next;
        return p;
    }

    // The plan's clears could not be enqueued: nothing is known any more.
    void forget(uintptr_t key)
    {
        std::lock_guard<std::mutex> lock(mu_);
        records_.erase(key);
    }

    // libscan_scratch_init: header zeroed, no body byte trusted.
    void zeroed(uintptr_t key)
    {
        std::lock_guard<std::mutex> lock(mu_);
        records_[key] = StateRecord{kKindZero, 0, 0, 0};
    }

private:
    std::mutex mu_;
    std::unordered_map<uintptr_t, StateRecord> records_;
    std::unordered_set<uintptr_t> captured_;
};

}  // namespace libscan
