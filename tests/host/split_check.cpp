// Host check of the split-row kernels' schedule and mailbox, built from the
// library's own header (vl_launch.hpp) and run on the CPU before the kernels
// run on a GPU.
//
// 1. Index bounds, over many (V, dtype, S) and grid shapes: every part is
//    non-empty and inside the row, a thread's clamped vector index stays in
//    its part, every marked column's bit lies inside the part bitmap, a
//    16-byte vector's bits never straddle two bitmap words, the members of a
//    group are distinct workgroups of the grid, and every mailbox slot lies
//    inside the words the launch clears and inside the workspace.
// 2. The handshake, with real threads: the workgroups of a few groups each
//    walk their rows (the kernel's row walk), publish a record per row with
//    relaxed atomic stores and take every partner's with relaxed atomic
//    exchanges against 0, under random delays.  Every record taken must be
//    the partner's record of that same row, no wait may reach its bound, and
//    the mailbox must be all zero at the end (every record was taken).
// Exits non-zero on the first violation; prints "ok" and counts.
#include "vl_launch.hpp"

#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <thread>
#include <vector>

namespace {

int fail(const char *what, long a, long b, long c)
{
    std::printf("FAIL %s (%ld %ld %ld)\n", what, a, b, c);
    std::exit(1);
}

// Bounds of one launch shape.
long check_shape(int64_t V, int N, const vl::SplitShape &shape, int per_cu, int cus, size_t ws)
{
    const int S = vl::split_parts_n(V, N, shape);
    if (S == 0)
        return 0;
    const bool kl = true;
    const vl::SplitShape fit{shape.block, shape.nv, shape.pf, per_cu};
    const vl::SplitPlan p = vl::split_plan(V, N, S, kl, fit, cus, ws);
    if (p.groups == 0)
        return 0;  // the launcher refuses
    const int64_t nvec = V / N;
    const int64_t cap = (int64_t)shape.block * shape.nv;
    if (S < 2 || S > vl::kMaxSplit)
        fail("part count out of range", V, N, S);
    if ((int64_t)p.part_vecs > cap)
        fail("part exceeds a workgroup's registers", V, N, S);
    if ((int64_t)p.part_vecs * (S - 1) >= nvec)
        fail("empty last part", V, N, S);
    if ((size_t)p.mbox_words * sizeof(uint64_t) > ws)
        fail("mailbox past the workspace", V, (long)p.mbox_words, (long)ws);
    if (p.lds * (size_t)per_cu > 160 * 1024)
        fail("LDS of the workgroups on a CU exceeds 160 KB", V, N, (long)p.lds);
    const int64_t grid = p.groups * S;
    if (grid > (int64_t)per_cu * cus)
        fail("grid larger than the resident workgroups", V, (long)grid, per_cu * cus);
    std::vector<int> seen(grid, 0);
    for (int64_t b = 0; b < grid; ++b) {
        int me;
        int64_t g;
        vl::split_member(b, S, me, g);
        if (me < 0 || me >= S || g < 0 || g >= p.groups)
            fail("member or group out of range", b, me, (long)g);
        // workgroups of one group share an XCD (b mod 8)
        if (g % 8 != b % 8)
            fail("group spans XCDs", b, (long)g, S);
        ++seen[g * S + me];
        const int64_t vbeg = (int64_t)me * p.part_vecs;
        const int64_t vend = vbeg + p.part_vecs < nvec ? vbeg + p.part_vecs : nvec;
        const int64_t np = vend - vbeg;
        if (np < 1 || vend > nvec)
            fail("part outside the row", V, me, (long)np);
        // clamped loads (and PF slots) of every thread slot
        for (int64_t lv = 0; lv < cap; lv += 97) {
            const int64_t c = lv < np ? lv : np - 1;
            if (vbeg + c < 0 || vbeg + c >= nvec)
                fail("clamped load outside the row", V, me, (long)lv);
        }
        // every column of the part, as a marked id: bit inside the bitmap;
        // the vector's N bits inside one 32-bit word
        const int64_t c0 = vbeg * N, c1 = vend * N;
        for (int64_t id = c0; id < c1; id += (id % 257 == 0 ? 1 : 61)) {
            const int64_t j = id - c0;
            if ((size_t)(j >> 5) >= p.words)
                fail("bitmap bit outside the bitmap", V, me, (long)id);
            const int64_t j0 = (id / N) * N - c0;
            if ((j0 & 31) + N > 32)
                fail("vector bits straddle two words", V, me, (long)id);
        }
        for (int r = 0; r < S; ++r)
            for (int par = 0; par < 2; ++par) {
                const int64_t i = vl::mbox_index(g, S, me, r, par);
                if (i < 0 || i + 1 >= p.mbox_words)
                    fail("mailbox slot outside the cleared words", (long)g, me, r);
            }
    }
    for (int64_t i = 0; i < grid; ++i)
        if (seen[i] != 1)
            fail("a (group, member) pair not taken exactly once", i, seen[i], S);
    return grid;
}

uint64_t pack(uint32_t lo, uint32_t hi) { return ~(((uint64_t)hi << 32) | lo); }

// The record a member publishes for a row (any injective function will do).
void record(int64_t row, int me, uint32_t &a, uint32_t &b, uint32_t &c, uint32_t &d)
{
    a = (uint32_t)(row * 8 + me);
    b = (uint32_t)(row ^ 0x5a5a5a5a) + (uint32_t)me;
    c = 0;  // an all-zero half must still read as published
    d = (uint32_t)me * 7919u;
}

// The handshake of `groups` groups of S members over the rows of `walk`.
long run_handshake(int S, int64_t groups, const vl::RowWalk &walk, unsigned seed)
{
    const int64_t words = groups * S * S * 4;
    std::vector<std::atomic<uint64_t>> mb(words);
    for (auto &w : mb)
        w.store(0);
    std::atomic<long> taken{0};
    std::atomic<int> bad{0};
    auto member = [&](int64_t b) {
        int me;
        int64_t g;
        vl::split_member(b, S, me, g);
        std::mt19937 rng(seed * 131u + (unsigned)b);
        vl::RowCursor c;
        c.init(g, groups, walk.len_in);
        int par = 0;
        for (; c.j < walk.n_in; c.advance(), par ^= 1) {
            const int64_t row = c.in_row(walk);
            if (rng() % 4 == 0)
                std::this_thread::sleep_for(std::chrono::microseconds(rng() % 50));
            uint32_t a0, a1, a2, a3;
            record(row, me, a0, a1, a2, a3);
            for (int r = 0; r < S; ++r) {
                if (r == me)
                    continue;
                const int64_t o = vl::mbox_index(g, S, me, r, par);
                mb[o].store(pack(a0, a1), std::memory_order_relaxed);
                mb[o + 1].store(pack(a2, a3), std::memory_order_relaxed);
            }
            for (int r = 0; r < S; ++r) {
                if (r == me)
                    continue;
                const int64_t in = vl::mbox_index(g, S, r, me, par);
                uint64_t u0 = 0, u1 = 0;
                long it = 0;
                for (;; ++it) {
                    if (u0 == 0)
                        u0 = mb[in].exchange(0, std::memory_order_relaxed);
                    if (u1 == 0)
                        u1 = mb[in + 1].exchange(0, std::memory_order_relaxed);
                    if ((u0 != 0 && u1 != 0) || it > 50000000)
                        break;
                    std::this_thread::yield();
                }
                uint32_t e0, e1, e2, e3;
                record(row, r, e0, e1, e2, e3);
                if (u0 != pack(e0, e1) || u1 != pack(e2, e3)) {
                    std::printf("FAIL record of member %d for row %ld at member %d (group %ld)%s\n",
                                r, (long)row, me, (long)g, (u0 == 0 || u1 == 0) ? ": timed out" : "");
                    bad = 1;
                    return;
                }
                ++taken;
            }
        }
    };
    std::vector<std::thread> th;
    for (int64_t b = 0; b < groups * S; ++b)
        th.emplace_back(member, b);
    for (auto &t : th)
        t.join();
    if (bad)
        std::exit(1);
    for (int64_t i = 0; i < words; ++i)
        if (mb[i].load() != 0)
            fail("record left in the mailbox", (long)i, S, (long)groups);
    return taken;
}

}  // namespace

int main()
{
    long shapes = 0, grids = 0;
    for (int N : {4, 8})
        for (int64_t V : {32772, 40000, 65536, 65540, 100000, 128256, 131072, 131076, 151936,
                          155648, 155656, 200000, 262144, 262148, 311296, 524288, 622592})
            for (int per_cu = 1; per_cu <= (N == 4 ? vl::kSplitF32 : vl::kSplitBf16).per_cu;
                 ++per_cu)
                for (int cus : {8, 80, 256, 304})
                    for (size_t ws : {size_t(4096), size_t(65536), vl::kSplitWorkspaceBytes}) {
                        const long g = check_shape(V, N, N == 4 ? vl::kSplitF32 : vl::kSplitBf16,
                                                   per_cu, cus, ws);
                        shapes += g > 0;
                        grids += g;
                    }
    long records = 0;
    unsigned seed = 1;
    for (int S : {2, 3, 5, 8, 16})
        for (int64_t groups : {8, 16})
            for (auto rng : {std::vector<int64_t>{0, 0, 0}, {7, 1, 6}, {16, 0, 16}, {5, 2, 2}}) {
                const int64_t ntok = groups * 5 + 3;
                const vl::RowWalk w = vl::make_walk(ntok, rng[0], rng[1], rng[2]);
                records += run_handshake(S, groups, w, seed++);
            }
    std::printf("ok: %ld launch shapes (%ld workgroups) in bounds; %ld records exchanged\n",
                shapes, grids, records);
    return 0;
}
