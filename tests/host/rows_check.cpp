// Host check of the fused row kernels' launch shapes and LDS layout
// (vl_rows.hip), built from the header the launcher uses (row_shape,
// row_lds in vl_launch.hpp) and run on the CPU before the kernels run on a
// GPU.  For float32 and bf16 rows, whole-vector and element paths, CE and
// KL, over V from 1 to 2^19:
//  - a staged shape holds the whole row: block x nv vectors >= the row's
//    vectors; only the shapes the launcher instantiates occur;
//  - the dynamic LDS stays within the 159 KB a block may take, and its
//    regions are in order and disjoint: the next-row slots (pf), the two
//    V-bit bitmaps (KL), the online variant's row slots, which come in
//    whole units of block vectors and hold no more of the row than remains
//    after the chunks held in registers;
//  - every teacher id below V marks a bit inside its row's bitmap, and the
//    bits of the 16-byte vector holding it lie in one 32-bit word (the
//    hand-off reads them with one load).
// Exits non-zero on the first violation.
#include "vl_launch.hpp"

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

[[noreturn]] void fail(const char *what, long a, long b, long c)
{
    std::printf("FAIL %s (%ld %ld %ld)\n", what, a, b, c);
    std::exit(1);
}

bool known(const vl::RowShape &s, bool f32, bool vec)
{
    struct K {
        int block, nv;
        bool pf, rl;
        int hk;
    };
    static const K common[] = {{64, 1, false, false, 0}, {64, 2, false, false, 0},
                               {64, 4, false, false, 0}, {256, 4, false, false, 0},
                               {512, 8, true, false, 0}};
    static const K f32only[] = {{64, 8, false, false, 0}, {256, 8, false, false, 0},
                                {1024, 8, true, false, 0}, {1024, 0, false, false, 4}};
    static const K bf16only[] = {{1024, 19, false, true, 0}, {1024, 0, false, false, 0}};
    auto eq = [&](const K &k) {
        return s.block == k.block && s.nv == k.nv && s.pf == k.pf && s.rl == k.rl && s.hk == k.hk;
    };
    if (!vec)
        return eq({256, 0, false, false, 0});
    for (const K &k : common)
        if (eq(k))
            return true;
    for (const K &k : (f32 ? std::vector<K>(f32only, f32only + 4) : std::vector<K>(bf16only, bf16only + 2)))
        if (eq(k))
            return true;
    return false;
}

long check(int64_t V, bool f32, bool vec, bool kl)
{
    const int n = vec ? (f32 ? 4 : 8) : 1;
    if (V % n)
        return 0;
    const vl::RowShape s = vl::row_shape(f32, vec, V);
    if (!known(s, f32, vec))
        fail("launch shape the launcher does not instantiate", (long)V, s.block, s.nv);
    const int64_t nvec = V / n;
    if (s.nv > 0 && (int64_t)s.block * s.nv < nvec)
        fail("staged shape smaller than the row", (long)V, s.block, s.nv);
    if (s.block % 64 || s.block > 1024)
        fail("block not a whole number of waves", (long)V, s.block, 0);
    const size_t raw = vec ? 16 : 4;
    const vl::RowLds L = vl::row_lds(s, kl, V, n, raw, vl::kMaxDynLds);
    if (L.bytes > vl::kMaxDynLds)
        fail("dynamic LDS above the block's share", (long)V, (long)L.bytes, kl);
    const size_t pf_end = s.pf ? (size_t)s.block * (s.nv > 0 ? s.nv : 1) * 16 : 0;
    const int64_t words = (V + 31) >> 5;
    if (L.bitmap_off != pf_end)
        fail("bitmaps overlap the next-row slots", (long)V, (long)L.bitmap_off, (long)pf_end);
    if (kl && L.lrow_off < L.bitmap_off + 2 * (size_t)words * 4)
        fail("row slots overlap the bitmaps", (long)V, (long)L.lrow_off, (long)words);
    if (L.lrow_off + (size_t)L.lds_vecs * raw != L.bytes)
        fail("row slots and LDS size disagree", (long)V, (long)L.lds_vecs, (long)L.bytes);
    if (s.nv > 0 && L.lds_vecs != 0)
        fail("staged kernel with online row slots", (long)V, (long)L.lds_vecs, 0);
    if (s.nv == 0) {
        if (L.lds_vecs % s.block)
            fail("row slots not whole units of the block", (long)V, (long)L.lds_vecs, s.block);
        const int64_t held = (int64_t)s.hk * s.block * vl::online_unroll_n(n, s.hk);
        const int64_t rest = nvec > held ? nvec - held : 0;
        if (L.lds_vecs > (rest + s.block - 1) / s.block * s.block)
            fail("more row slots than the row has vectors left", (long)V, (long)L.lds_vecs,
                 (long)rest);
    }
    if (kl) {
        // a sample of ids, every vector boundary near the row's end included
        for (int64_t id = 0; id < V; id += (id < 4096 || V - id < 4096) ? 1 : 997) {
            if ((id >> 5) >= words)
                fail("bit outside the bitmap", (long)V, (long)id, (long)words);
            const int64_t j0 = id / n * n;
            if ((j0 & 31) + n > 32)
                fail("vector bits straddle two words", (long)V, (long)id, n);
        }
    }
    return 1;
}

}  // namespace

int main()
{
    long cases = 0;
    std::vector<int64_t> vs;
    for (int64_t v = 1; v <= 4096; ++v)
        vs.push_back(v);
    for (int64_t v = 4096; v <= vl::kMaxKlVocab; v += 4093)
        vs.push_back(v);
    for (int64_t b : {256, 512, 1024, 2048, 4096, 8192, 16384, 19456, 32768, 65536, 131072})
        for (int64_t d : {-8, -4, -1, 0, 1, 4, 8})
            for (int64_t n : {4, 8}) {
                const int64_t v = b * n + d;
                if (v >= 1 && v <= vl::kMaxKlVocab)
                    vs.push_back(v);
            }
    for (int64_t v : {32000, 128256, 151936, 155648, 155656, 200000, 262144, 524288})
        vs.push_back(v);
    for (int64_t V : vs)
        for (bool f32 : {true, false})
            for (bool vec : {true, false})
                for (bool kl : {false, true})
                    cases += check(V, f32, vec, kl);
    std::printf("ok: %ld row-kernel launch plans in bounds\n", cases);
    return 0;
}
