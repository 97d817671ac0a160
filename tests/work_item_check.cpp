// Host check of the workgroup -> (head, tile) order of the attention kernels
// (work_item in fa_common.hpp): for grids of every size up to a few thousand items,
// with and without the weight-sorted causal list, every item is visited exactly
// once; with the sorted list on whole heads and at most kSortedMax items per XCD,
// the items of each XCD reach it heaviest (lowest rank) first in each group of
// four dispatches.  Prints "ok" and exits 0 when all hold.
#include <cstdio>
#include <vector>

#include "fa_common.hpp"

int main()
{
    int checked = 0;
    for (int heads = 1; heads <= 40; ++heads)
        for (int n_tiles : {1, 2, 3, 4, 5, 7, 8, 16, 31, 32, 33, 64, 128}) {
            const int n = heads * n_tiles;
            for (int heavy = 0; heavy < 2; ++heavy) {
                std::vector<int> seen(n, 0);
                for (int wg = 0; wg < n; ++wg) {
                    const fa::WorkItem w = fa::work_item(wg, n, n_tiles, heavy != 0);
                    if (w.head < 0 || w.head >= heads || w.rank < 0 || w.rank >= n_tiles) {
                        std::printf("out of range: heads %d tiles %d wg %d -> (%d, %d)\n", heads,
                                    n_tiles, wg, w.head, w.rank);
                        return 1;
                    }
                    ++seen[w.head * n_tiles + w.rank];
                }
                for (int i = 0; i < n; ++i)
                    if (seen[i] != 1) {
                        std::printf("item %d seen %d times: heads %d tiles %d heavy %d\n", i,
                                    seen[i], heads, n_tiles, heavy);
                        return 1;
                    }
                ++checked;
                // sorted list: on an XCD holding whole heads and at most kSortedMax
                // items, the ranks of its workgroups, taken in dispatch order four at a
                // time, never decrease from one group to the next
                if (heavy && n % fa::kXcds == 0 && (n / fa::kXcds) % n_tiles == 0 &&
                    n / fa::kXcds <= fa::kSortedMax)
                    for (int x = 0; x < fa::kXcds; ++x) {
                        int prev_max = -1;
                        const int cnt = n / fa::kXcds;
                        for (int g = 0; g * fa::kSesPerXcd < cnt; ++g) {
                            int lo = 1 << 30, hi = -1;
                            for (int e = 0; e < fa::kSesPerXcd && g * fa::kSesPerXcd + e < cnt; ++e) {
                                const int wg = x + fa::kXcds * (g * fa::kSesPerXcd + e);
                                const int r = fa::work_item(wg, n, n_tiles, true).rank;
                                lo = r < lo ? r : lo;
                                hi = r > hi ? r : hi;
                            }
                            if (lo < prev_max) {
                                std::printf("order: heads %d tiles %d xcd %d group %d\n", heads,
                                            n_tiles, x, g);
                                return 1;
                            }
                            prev_max = hi;
                        }
                    }
            }
        }
    std::printf("ok %d grids\n", checked);
    return 0;
}
