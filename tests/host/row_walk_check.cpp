// Host check of the row walk of the CE/KL kernel: over every block of a
// persistent grid, the in-range list and the out-of-range list together
// visit each row exactly once, in-range rows only in the first and the
// others only in the second.  Exits non-zero on the first violation.
#include "vl_launch.hpp"

#include <cstdio>
#include <vector>

int main()
{
    long configs = 0;
    for (int64_t ntok : {0, 1, 5, 7, 64, 100, 513, 1000, 4096})
        for (int64_t seq : {0, 1, 3, 7, 16, 512})
            for (int64_t st = 0; st <= (seq > 0 ? seq : 0); st += (seq > 4 ? seq / 4 : 1))
                for (int64_t en = st; en <= (seq > 0 ? seq : 0); en += (seq > 4 ? seq / 3 : 1))
                    for (int64_t G : {1, 2, 3, 7, 256, 5000}) {
                        const vl::RowWalk w = vl::make_walk(ntok, seq, st, en);
                        std::vector<int> seen(ntok, 0);
                        auto in_range = [&](int64_t r) {
                            return seq <= 0 || (st <= r % seq && r % seq < en);
                        };
                        for (int64_t b = 0; b < G; ++b) {
                            vl::RowCursor c;
                            for (c.init(b, G, w.len_in); c.j < w.n_in; c.advance()) {
                                const int64_t r = c.in_row(w);
                                if (r < 0 || r >= ntok || !in_range(r)) {
                                    std::printf("in-range list: ntok=%ld seq=%ld [%ld,%ld) grid=%ld row=%ld\n",
                                                (long)ntok, (long)seq, (long)st, (long)en, (long)G, (long)r);
                                    return 1;
                                }
                                ++seen[r];
                            }
                            vl::RowCursor o;
                            for (o.init(b, G, w.len_out); o.j < w.n_out; o.advance()) {
                                const int64_t r = o.out_row(w);
                                if (r < 0 || r >= ntok || in_range(r)) {
                                    std::printf("out-of-range list: ntok=%ld seq=%ld [%ld,%ld) grid=%ld row=%ld\n",
                                                (long)ntok, (long)seq, (long)st, (long)en, (long)G, (long)r);
                                    return 1;
                                }
                                ++seen[r];
                            }
                        }
                        for (int64_t r = 0; r < ntok; ++r)
                            if (seen[r] != 1) {
                                std::printf("row %ld visited %d times: ntok=%ld seq=%ld [%ld,%ld) grid=%ld\n",
                                            (long)r, seen[r], (long)ntok, (long)seq, (long)st, (long)en,
                                            (long)G);
                                return 1;
                            }
                        ++configs;
                    }
    std::printf("ok %ld configurations\n", configs);
    return 0;
}
