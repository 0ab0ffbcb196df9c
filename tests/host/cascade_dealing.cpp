// Host check of the single-launch cascade's dealing of block roles. The test
// extracts cascade_role from the kernel source into cascade_role_extracted.inc
// (the same text, with the device qualifiers dropped) and builds this file
// around it.
//  1. For every pair of prefix and suffix block counts in a range (every count
//     up to 600, then strides up to 1100), the blocks 0 .. NP + NS - 1 receive
//     each prefix index 0 .. NP - 1 and each suffix index 0 .. NS - 1 exactly once.
//  2. Under the dispatch order the dealing is built for (block b to XCD b % 8,
//     compute unit (b / 8) % 32 of it, one block per unit before any unit gets
//     a second), 256 + 256 blocks give every compute unit one block of each role.
#include <algorithm>
#include <cstdio>
#include <vector>
using std::min;
namespace fdec {
#include "cascade_role_extracted.inc"
}

int main() {
    long bad = 0, cases = 0;
    for (int NP = 0; NP <= 1100; NP += (NP < 600 ? 1 : 37))
        for (int NS = 0; NS <= 1100; NS += (NS < 600 ? 1 : 41)) {
            std::vector<int> seen_p(NP, 0), seen_s(NS, 0);
            for (int b = 0; b < NP + NS; ++b) {
                bool prefix = false;
                int v = -1;
                fdec::cascade_role(b, NP, NS, prefix, v);
                std::vector<int> &seen = prefix ? seen_p : seen_s;
                if (v < 0 || v >= (int)seen.size()) {
                    if (bad++ < 5) std::printf("NP %d NS %d block %d: index %d out of range\n", NP, NS, b, v);
                    continue;
                }
                seen[v]++;
            }
            for (int c : seen_p) bad += c != 1;
            for (int c : seen_s) bad += c != 1;
            ++cases;
        }
    int mixed = 0;
    for (int x = 0; x < 8; ++x)
        for (int cu = 0; cu < 32; ++cu) {
            int np = 0, ns = 0;
            for (int b = 0; b < 512; ++b)
                if (b % 8 == x && (b / 8) % 32 == cu) {
                    bool prefix = false;
                    int v = -1;
                    fdec::cascade_role(b, 256, 256, prefix, v);
                    (prefix ? np : ns)++;
                }
            mixed += np == 1 && ns == 1;
        }
    std::printf("pairs of counts %ld, mismatches %ld, units with one block of each role %d of 256\n", cases, bad,
                mixed);
    if (bad == 0 && mixed == 256) std::printf("dealing ok\n");
    return bad == 0 && mixed == 256 ? 0 : 1;
}
