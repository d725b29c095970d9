// Host mirror of every slot's live-log length, and the rule that keeps it
// equal to the device counters when a call is split into several launches.
//
// [DL] "DeltaLog: Deferred Materialization of Recurrent States for Linear
// Attention Decoding", design section (append-merge cycle): a decoded slot
// whose log holds C = L - 1 entries merges and its log empties; any other
// slot appends one entry.  A merge without a token, a fresh assignment and a
// resident-state window all leave the log empty.
//
// Plain C++ with no HIP dependency, so the host tests compile it on its own.
#pragma once

#include <stdint.h>

namespace dl {

// One decode of these slots.
inline void mirror_decode(int32_t *n, const int32_t *ids, int32_t cnt, int32_t C) {
    for (int32_t j = 0; j < cnt; ++j) {
        int32_t &x = n[ids[j]];
        x = (x == C) ? 0 : x + 1;
    }
}

// These slots' logs are empty afterwards (merge, assignment, window).
inline void mirror_clear(int32_t *n, const int32_t *ids, int32_t cnt) {
    for (int32_t j = 0; j < cnt; ++j) n[ids[j]] = 0;
}

// Issue launch(lo, cnt) over [0, total) in chunks of at most `chunk` entries,
// and apply commit(lo, cnt) to the mirror right after each launch that was
// enqueued.  A launch that fails stops the call: the chunks before it have run
// (or will run) on the device and are committed, the failed chunk and the
// ones after it were never enqueued and are not.  Returns 0 or the failing
// launch's code.
template <class Launch, class Commit>
int launch_chunks(int32_t total, int32_t chunk, Launch &&launch, Commit &&commit) {
    for (int32_t lo = 0; lo < total; lo += chunk) {
        const int32_t cnt = total - lo < chunk ? total - lo : chunk;
        const int e = launch(lo, cnt);
        if (e != 0) return e;
        commit(lo, cnt);
    }
    return 0;
}

}  // namespace dl
