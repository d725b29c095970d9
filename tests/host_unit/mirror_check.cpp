// Host check of the live-length mirror rule (dl_mirror.hpp), no GPU: a call
// split into launches of at most `chunk` slots, whose launch number `fail_at`
// fails, must leave the mirror advanced for the launches before it and
// unchanged for that launch and the ones after.  The device side is modelled
// by applying each launch that succeeds to a second array, as the kernels
// would.  Prints "ok" or the first mismatch; the exit code says the same.
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "dl_mirror.hpp"

static int check(int P, int B, int chunk, int C, int fail_at, int kind) {
    std::vector<int32_t> host(P), dev(P), ids(B);
    for (int s = 0; s < P; ++s) host[s] = dev[s] = (s * 7) % (C + 1);
    for (int j = 0; j < B; ++j) ids[j] = (j * 13 + 5) % P;       // distinct while gcd(13, P) == 1
    int launches = 0;
    auto launch = [&](int32_t lo, int32_t cnt) -> int {
        if (launches++ == fail_at) return -6;
        if (kind == 0) dl::mirror_decode(dev.data(), ids.data() + lo, cnt, C);
        else dl::mirror_clear(dev.data(), ids.data() + lo, cnt);
        return 0;
    };
    auto commit = [&](int32_t lo, int32_t cnt) {
        if (kind == 0) dl::mirror_decode(host.data(), ids.data() + lo, cnt, C);
        else dl::mirror_clear(host.data(), ids.data() + lo, cnt);
    };
    const int rc = dl::launch_chunks(B, chunk, launch, commit);
    const int nchunks = (B + chunk - 1) / chunk;
    if ((fail_at < nchunks) != (rc != 0)) {
        printf("P=%d B=%d chunk=%d fail_at=%d: rc %d\n", P, B, chunk, fail_at, rc);
        return 1;
    }
    // the slots of launches before the failure moved one step, the rest not at all
    std::vector<int32_t> want(P);
    for (int s = 0; s < P; ++s) want[s] = (s * 7) % (C + 1);
    const int done = fail_at < nchunks ? fail_at * chunk : B;
    for (int j = 0; j < done; ++j) {
        int32_t &x = want[ids[j]];
        x = kind == 0 ? (x == C ? 0 : x + 1) : 0;
    }
    for (int s = 0; s < P; ++s) {
        if (host[s] != dev[s] || host[s] != want[s]) {
            printf("P=%d B=%d chunk=%d fail_at=%d kind=%d: slot %d host %d device %d want %d\n", P, B, chunk,
                   fail_at, kind, s, host[s], dev[s], want[s]);
            return 1;
        }
    }
    return 0;
}

int main() {
    int bad = 0;
    for (int kind = 0; kind < 2; ++kind)
        for (int fail_at = 0; fail_at <= 4; ++fail_at) {
            bad += check(1024, 1000, 512, 15, fail_at, kind);
            bad += check(1024, 1024, 256, 7, fail_at, kind);
            bad += check(64, 1, 512, 31, fail_at, kind);
            bad += check(2048, 1537, 512, 0, fail_at, kind);
        }
    puts(bad ? "mismatch" : "ok");
    return bad ? 1 : 0;
}
