// Host check of the top-k kernel's candidate buffer (vl_topk.hip), run on
// the CPU before the kernel runs on a GPU.  One wave's pass over a row is
// replayed at sub-tile granularity with the kernel's rules and its buffer
// sizes (topk_cap and topk_sel_limit from vl_launch.hpp, the header the
// kernel uses):
//  - a sub-tile holds 64 lanes x N values (N = 4 float32, 8 bf16, 1 on the
//    element path); its candidates are the valid values above the
//    threshold, every valid value before the first compaction.  bf16 values
//    in the high half of a 32-bit word are compared as the whole word, so
//    a value equal to a positive threshold is admitted when its word's low
//    half is nonzero (the kernel's compare; such a value cannot win).
//  - a sub-tile that could overflow the buffer (cnt + 64 N > cap) compacts
//    it first: mid-row by a radix select that stops at the first bin edge
//    keeping at most the limit, at the end exactly to k.  The select's
//    histogram, digit walk and in-place rewrite follow the kernel's.
//  - candidates are appended at cnt + (candidates in lower lanes) + (their
//    index within the lane), in id order.
// Checked: every buffer write lands below cap; a compaction reads at most
// cap entries and its in-place rewrite of chunk e (64 entries) writes only
// below 64 (e + 1); the histogram index stays below 256; the final buffer
// holds exactly k entries, equal to a brute-force top-k in the order (value
// descending, id ascending).  Exits non-zero on the first violation.
#include "vl_launch.hpp"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

namespace {

uint32_t bits_of(float f)
{
    uint32_t u;
    std::memcpy(&u, &f, 4);
    return u;
}

float float_of(uint32_t u)
{
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

// The kernel's order-preserving key: sign-flipped, -0 folded onto +0.
uint32_t order_key(float f)
{
    uint32_t u = bits_of(f);
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

float key_value(uint32_t k)
{
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return float_of(u);
}

[[noreturn]] void fail(const char *what, long a, long b, long c)
{
    std::printf("FAIL %s (%ld %ld %ld)\n", what, a, b, c);
    std::exit(1);
}

struct Wave {
    int cap, k, sub, limit;
    std::vector<uint32_t> keys, ids;
    int cnt = 0;
    long compactions = 0;
};

// The kernel's select_compact: returns the kept count and kstar.
int select_compact(Wave &w, int limit, uint32_t &kstar_out)
{
    const int cnt = w.cnt, k = w.k, E = w.cap / 64;
    if (cnt > 64 * E)
        fail("compaction reads past the buffer", cnt, w.cap, 0);
    if (cnt < k)
        fail("compaction with fewer than k entries", cnt, k, 0);
    uint32_t lo = 0xFFFFFFFFu, hi = 0u, vary = 0u;
    for (int i = 0; i < cnt; ++i) {
        lo = std::min(lo, w.keys[i]);
        hi = std::max(hi, w.keys[i]);
    }
    for (int i = 0; i < cnt; ++i)
        vary |= w.keys[i] - lo;
    const uint32_t span = hi - lo;
    const int low = vary ? __builtin_ctz(vary) : 0;
    uint32_t prefix = 0u;
    int rem = k;
    bool keep_ge = false;
    if (span != 0u) {
        for (int hb = 32 - __builtin_clz(span); hb > low; hb -= 8) {
            const int sh = hb - 8 > low ? hb - 8 : low;
            const uint32_t dmask = (1u << (hb - sh)) - 1u;
            const uint32_t above_mask = hb >= 32 ? 0u : ~((1u << hb) - 1u);
            uint32_t hist[256] = {0};
            for (int i = 0; i < cnt; ++i) {
                const uint32_t rel = w.keys[i] - lo;
                if ((rel & above_mask) == prefix) {
                    const uint32_t b = (rel >> sh) & dmask;
                    if (b >= 256u)
                        fail("histogram bin out of range", (long)b, hb, sh);
                    ++hist[b];
                }
            }
            // bins scanned from 255 down: the bin holding the rem-th key
            uint32_t above = 0u;
            int found = -1;
            uint32_t fa = 0u;
            for (int b = 255; b >= 0; --b) {
                if (above < (uint32_t)rem && (uint32_t)rem <= above + hist[b]) {
                    found = b;
                    fa = above;
                    break;
                }
                above += hist[b];
            }
            if (found < 0)
                fail("radix pass found no bin", rem, cnt, hb);
            prefix |= ((uint32_t)found & dmask) << sh;
            if (limit > 0 && (k - rem) + (int)fa + (int)hist[found] <= limit) {
                keep_ge = true;
                break;
            }
            rem -= (int)fa;
        }
    }
    const uint32_t kstar = lo + prefix;
    // in-place rewrite, chunk by chunk of 64 entries
    int out = 0, eq_seen = 0;
    for (int e = 0; e < E; ++e) {
        int eq_below = 0, kept_below = 0;
        std::vector<std::pair<uint32_t, uint32_t>> wr;
        for (int lane = 0; lane < 64; ++lane) {
            const int i = lane + 64 * e;
            const bool valid = i < cnt;
            const uint32_t key = valid ? w.keys[i] : 0u, id = valid ? w.ids[i] : 0u;
            const bool gt = valid && key > kstar;
            const bool eq = valid && key == kstar;
            const bool keep = gt || (eq && (keep_ge || eq_seen + eq_below < rem));
            if (eq)
                ++eq_below;
            if (keep) {
                const int pos = out + kept_below;
                if (pos >= 64 * (e + 1))
                    fail("compaction writes past the chunk it reads", pos, e, cnt);
                wr.push_back({key, id});
                ++kept_below;
            }
        }
        // every lane of the chunk read its entry before any lane writes
        for (size_t j = 0; j < wr.size(); ++j) {
            w.keys[out + j] = wr[j].first;
            w.ids[out + j] = wr[j].second;
        }
        out += kept_below;
        eq_seen += eq_below;
    }
    kstar_out = kstar;
    return out;
}

// One row through the filter.  vals[id] are the row's values; `bf` marks
// bf16 rows (values already bf16 numbers) read 8 per 16-byte vector; n is
// the values per vector (1, 4 or 8).
void run_row(const std::vector<float> &vals, int n, bool bf, int k, long &writes, long &comps)
{
    const int V = (int)vals.size();
    const int sub = 64 * n;
    Wave w;
    w.cap = vl::topk_cap(k, sub);
    w.k = k;
    w.sub = sub;
    w.limit = vl::topk_sel_limit(k, w.cap, sub);
    w.keys.assign(w.cap, 0xDEADBEEFu);
    w.ids.assign(w.cap, 0xDEADBEEFu);
    if (k > w.cap - sub)
        fail("k does not fit beside one sub-tile", k, w.cap, sub);
    bool thr_set = false;
    float thr = -INFINITY;
    const int nvec = V / n;
    for (int vbase = 0; vbase < nvec; vbase += 64) {
        auto candidates = [&](std::vector<int> &out) {
            out.clear();
            for (int lane = 0; lane < 64; ++lane) {
                const int v = vbase + lane;
                if (v >= nvec)
                    break;
                for (int c = 0; c < n; ++c) {
                    const int id = v * n + c;
                    bool pass;
                    if (!thr_set) {
                        pass = true;
                    } else if (bf && (c & 1)) {
                        // whole-word compare: high half = this value, low
                        // half = the previous element's bits
                        const uint32_t word = (bits_of(vals[id]) & 0xFFFF0000u) |
                                              (bits_of(vals[id - 1]) >> 16);
                        pass = float_of(word) > thr;
                    } else {
                        pass = vals[id] > thr;
                    }
                    if (pass)
                        out.push_back(id);
                }
            }
        };
        std::vector<int> cand;
        candidates(cand);
        if (cand.empty())
            continue;
        if (w.cnt + sub > w.cap) {
            uint32_t ks;
            w.cnt = select_compact(w, w.limit, ks);
            ++comps;
            if (w.cnt > w.limit && w.cnt != k)
                fail("mid-row compaction kept more than the limit", w.cnt, w.limit, k);
            thr = key_value(ks);
            thr_set = true;
            candidates(cand);
            if (cand.empty())
                continue;
        }
        for (size_t j = 0; j < cand.size(); ++j) {
            const int pos = w.cnt + (int)j;
            if (pos >= w.cap)
                fail("append past the buffer", pos, w.cap, (long)cand.size());
            w.keys[pos] = order_key(vals[cand[j]]);
            w.ids[pos] = (uint32_t)cand[j];
            ++writes;
        }
        w.cnt += (int)cand.size();
    }
    uint32_t ks;
    w.cnt = select_compact(w, 0, ks);
    if (w.cnt != k)
        fail("final selection does not hold k entries", w.cnt, k, V);
    // brute force: (key desc, id asc)
    std::vector<int> ord(V);
    for (int i = 0; i < V; ++i)
        ord[i] = i;
    std::stable_sort(ord.begin(), ord.end(), [&](int a, int b) {
        return order_key(vals[a]) > order_key(vals[b]);
    });
    std::vector<uint32_t> want(ord.begin(), ord.begin() + k), got(w.ids.begin(), w.ids.begin() + k);
    std::sort(want.begin(), want.end());
    std::sort(got.begin(), got.end());
    if (want != got)
        fail("selection differs from the brute-force top-k", V, k, n);
}

float to_bf16(float f)
{
    uint32_t u = bits_of(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return float_of(u & 0xFFFF0000u);
}

}  // namespace

int main()
{
    std::mt19937 rng(12345);
    std::normal_distribution<float> nd(0.f, 2.f);
    long rows = 0, writes = 0, comps = 0;
    const int kinds = 8;
    for (int n : {1, 4, 8})
        for (int V : {7, 100, 1000, 4104, 32000, 151936})
            for (int k : {1, 7, 64, 256, 1000, 2048}) {
                if (k > V || V % n)
                    continue;
                for (int kind = 0; kind < kinds; ++kind) {
                    // large rows: a few kinds only (runtime)
                    if (V > 40000 && kind % 3 != 0)
                        continue;
                    std::vector<float> vals(V);
                    for (int i = 0; i < V; ++i) {
                        float x;
                        switch (kind) {
                        case 0: x = nd(rng); break;                        // normal
                        case 1: x = (float)i * 1e-3f; break;               // ascending: worst case
                        case 2: x = -(float)i * 1e-3f; break;              // descending
                        case 3: x = 1.5f; break;                           // all tied
                        case 4: x = (float)(rng() % 5); break;             // few distinct
                        case 5: x = 2.f * std::log((float)(1 + rng() % 1000)) + 0.5f * nd(rng); break;
                        case 6: x = (rng() & 1) ? 0.f : -0.f; break;       // +0 / -0
                        default: x = (i % 97 == 0) ? 100.f + nd(rng) : nd(rng); break;
                        }
                        vals[i] = x;
                    }
                    if (n == 8)
                        for (float &x : vals)
                            x = to_bf16(x);
                    run_row(vals, n, n == 8, k, writes, comps);
                    ++rows;
                }
            }
    std::printf("ok: %ld rows, %ld buffer writes, %ld compactions in bounds; selections exact\n",
                rows, writes, comps);
    return 0;
}
