// Host-only check of the scratch state table (prefix_scan_amd/csrc/
// scratch_state.hpp), built with g++ by tests/test_state_table.py.
//
// A model of one scratch buffer follows what the calls actually leave in it,
// in the order they execute on the GPU: eager calls run when they are
// enqueued, calls recorded into a graph run at each replay, with the clear
// plan chosen when they were recorded.  Whenever a call runs, the state it
// reads must be trustworthy: a header left by the library, and a state range
// that is either freshly zeroed or was last written by a call of a kind that
// can reuse it.  The check runs the scenario of a captured scan followed by
// a captured one-bit radix sort replayed twice (whose second replay reads the
// radix rows as descriptors if the plan ignores capture), fixed mixes of
// eager and captured calls, and many random ones; and it shows that the same
// model does catch the failure when the table is not told about capture.
#include "scratch_state.hpp"

#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <string>
#include <vector>

using namespace libscan;

namespace {

struct Call {
    int kind;          // kKindDesc, kKindRadix or kKindData
    uint64_t sig;      // radix signature
    size_t state;      // body bytes of state the call reads
    uint64_t launches;
};

// What is really in the buffer.
struct Truth {
    bool header_ok = false;   // tickets left by the library (or zeroed)
    int kind = kKindNone;     // kKindZero: zeroed range, usable by any kind
    uint64_t sig = 0;
    size_t valid = 0;         // body bytes of usable state from the front
};

struct Recorded {
    Call c;
    ClearPlan p;
};

int g_failures = 0;
bool g_quiet = false;

void fail(const std::string &what)
{
    ++g_failures;
    if (!g_quiet)
        fprintf(stderr, "FAIL: %s\n", what.c_str());
}

// Executes one call with its plan on the buffer's true contents.
void execute(Truth &t, const Call &c, const ClearPlan &p, const char *ctx)
{
    if (c.kind == kKindData) {          // writes data over the body; no state read
        t.kind = kKindNone;
        t.valid = 0;
        return;
    }
    if (p.header) {
        t.header_ok = true;
        t.kind = kKindZero;
        t.sig = 0;
        t.valid = c.state;
    } else if (p.bytes) {
        // Zeroes body bytes [from, from + bytes).  From the front, the range
        // is usable by any kind; further on, only if it extends a usable
        // range (whose kind then still decides who may use it).
        if (p.from == 0) {
            t.kind = kKindZero;
            t.sig = 0;
            t.valid = p.bytes;
        } else if (p.from <= t.valid && t.kind != kKindNone) {
            t.valid = p.from + p.bytes > t.valid ? p.from + p.bytes : t.valid;
        }
    }
    const bool kind_ok = t.kind == kKindZero || (t.kind == c.kind && (c.kind != kKindRadix ||
                                                                      t.sig == c.sig));
    if (!t.header_ok || !kind_ok || t.valid < c.state) {
        char buf[256];
        snprintf(buf, sizeof buf,
                 "%s: call kind %d sig %llu reads %zu state bytes, buffer holds kind %d sig %llu "
                 "valid %zu header %d",
                 ctx, c.kind, (unsigned long long)c.sig, c.state, t.kind,
                 (unsigned long long)t.sig, t.valid, (int)t.header_ok);
        fail(buf);
    }
    t.header_ok = true;
    if (c.kind == kKindDesc)
        t.valid = t.valid > c.state && (t.kind == kKindDesc || t.kind == kKindZero) ? t.valid
                                                                                   : c.state;
    else
        t.valid = c.state;
    t.kind = c.kind;
    t.sig = c.sig;
}

struct Harness {
    StateTable table;
    Truth truth;
    bool tell_capture = true;    // false: the table is not told about capture
    uintptr_t key = 0x1000;

    void eager(const Call &c, const char *ctx)
    {
        const ClearPlan p = table.prepare(key, c.kind, c.sig, c.state, c.launches, false);
        execute(truth, c, p, ctx);
    }
    Recorded record(const Call &c)
    {
        return Recorded{c, table.prepare(key, c.kind, c.sig, c.state, c.launches, tell_capture)};
    }
    void replay(const std::vector<Recorded> &g, const char *ctx)
    {
        for (const Recorded &r : g)
            execute(truth, r.c, r.p, ctx);
    }
};

const Call kScanBig{kKindDesc, 0, 8192 * 8, 1};
const Call kScanSmall{kKindDesc, 0, 512 * 8, 1};
const Call kRadix1{kKindRadix, (1000000ull << 3) | 1, 4096 * 8, 32};
const Call kRadix4{kKindRadix, (1000000ull << 3) | 4, 4096 * 8 + 2048, 8};
const Call kThreePass{kKindData, 0, 0, 0};

// The failing order: capture [scan, one-bit radix], replay twice.
int scenario_scan_then_radix(bool tell_capture)
{
    g_failures = 0;
    Harness h;
    h.tell_capture = tell_capture;
    h.eager(kScanBig, "warm-up scan");
    std::vector<Recorded> g = {h.record(kScanBig), h.record(kRadix1)};
    h.replay(g, "replay 1");
    h.replay(g, "replay 2");
    h.eager(kScanBig, "eager scan after replays");
    h.replay(g, "replay 3");
    h.eager(kRadix1, "eager radix after replay");
    h.replay(g, "replay 4");
    return g_failures;
}

int scenario_mixed()
{
    g_failures = 0;
    Harness h;
    h.eager(kScanSmall, "first call on an unknown buffer");
    h.eager(kScanBig, "larger scan");
    h.eager(kScanSmall, "smaller scan");
    h.eager(kRadix4, "four-bit radix");
    h.eager(kRadix4, "four-bit radix again");
    h.eager(kRadix1, "one-bit radix");
    h.eager(kThreePass, "three-pass");
    h.eager(kScanBig, "scan after data");
    std::vector<Recorded> g1 = {h.record(kRadix4), h.record(kScanSmall), h.record(kThreePass),
                                h.record(kScanBig)};
    std::vector<Recorded> g2 = {h.record(kScanBig), h.record(kScanSmall)};
    h.eager(kRadix1, "eager between captures");
    h.replay(g2, "g2");
    h.replay(g1, "g1");
    h.replay(g1, "g1 again");
    h.eager(kScanSmall, "eager scan");
    h.replay(g2, "g2 again");
    h.eager(kRadix4, "eager radix");
    h.eager(kRadix4, "eager radix again");
    h.replay(g1, "g1 third");
    return g_failures;
}

int scenario_random(uint64_t seed, int steps)
{
    g_failures = 0;
    std::mt19937_64 rng(seed);
    Harness h;
    const Call menu[] = {kScanBig, kScanSmall, kRadix1, kRadix4, kThreePass,
                         Call{kKindDesc, 0, 100 * 8, 1}, Call{kKindRadix, 77 << 3 | 1, 1024, 32}};
    std::vector<std::vector<Recorded>> graphs;
    for (int i = 0; i < steps; ++i) {
        // The first half is eager only: once a buffer has been captured,
        // every call on it clears, so the trust logic is tested before that.
        const int what = i < steps / 2 ? 0 : (int)(rng() % 10);
        if (what < 6) {
            h.eager(menu[rng() % 7], "random eager");
        } else if (what < 8 || graphs.empty()) {
            std::vector<Recorded> g;
            const int len = 1 + (int)(rng() % 4);
            for (int j = 0; j < len; ++j)
                g.push_back(h.record(menu[rng() % 7]));
            graphs.push_back(g);
        } else {
            h.replay(graphs[rng() % graphs.size()], "random replay");
        }
        if (rng() % 50 == 0) {         // libscan_scratch_init: header zeroed
            h.table.zeroed(h.key);
            h.truth.header_ok = true;
            h.truth.kind = kKindZero;
            h.truth.sig = 0;
            h.truth.valid = 0;
        }
    }
    return g_failures;
}

}  // namespace

int main()
{
    int bad = 0;
    if (scenario_scan_then_radix(true)) {
        fprintf(stderr, "capture scenario failed\n");
        ++bad;
    }
    g_quiet = true;
    if (scenario_scan_then_radix(false) == 0) {
        fprintf(stderr, "the model did not catch the capture-blind table\n");
        ++bad;
    }
    g_quiet = false;
    if (scenario_mixed()) {
        fprintf(stderr, "mixed scenario failed\n");
        ++bad;
    }
    for (uint64_t seed = 1; seed <= 300; ++seed) {
        if (scenario_random(seed, 200)) {
            fprintf(stderr, "random scenario %llu failed\n", (unsigned long long)seed);
            ++bad;
            break;
        }
    }
    if (bad)
        return 1;
    printf("state table: all scenarios ok\n");
    return 0;
}
