// Host harness: the decode automaton functions of rosa_sam.hip (compiled for
// the host) over one symbol stream.  The first T0 positions are appended
// without last-end walks and the last ends are then set in one pass, as
// rosa_build does; the remaining positions are stepped one by one with the
// walk, as rosa_step does.  Prints E and L of every stepped position, one
// "t E L" line each, for the CPU test to compare with the oracle.
//   usage: sam_build_check K T0 < symbols (T bytes on stdin)
#include "rosa_sam_core.h"

#include <cstdio>
#include <cstdlib>
#include <vector>

int main(int argc, char **argv)
{
    if (argc != 3)
        return 2;
    const int K = std::atoi(argv[1]);
    const long T0 = std::atol(argv[2]);
    std::vector<unsigned char> x;
    for (int c; (c = std::getchar()) != EOF;)
        x.push_back((unsigned char)c);
    const long T = (long)x.size();
    if (K < 1 || K > 256 || T0 < 0 || T0 > T)
        return 2;
    const long ncap = T <= 1 ? 2 : 2 * T - 1;
    // records as in the decode state: node, then the transition row, the
    // record rounded up to 64 bytes
    const long rsi = ((16 + 4 * K + 63) / 64 * 64) / 4;
    std::vector<int4> recs((size_t)(ncap * rsi / 4));
    rosa::SamStream a;
    a.nd = recs.data();
    a.nds = rsi / 4;
    a.nx = reinterpret_cast<int32_t *>(recs.data()) + 4;
    a.nxs = rsi;
    a.K = K;
    a.tail = 0;
    a.nst = 0;
    a.tail_len = 0;
    a.tail_link = -1;
    rosa::sam_new_state(a, 0);
    for (long t = 0; t < T0; ++t)
        rosa::sam_extend(a, x[(size_t)t]);
    rosa::sam_fill_last(a);
    for (long t = T0; t < T; ++t) {
        const int cur = rosa::sam_extend(a, x[(size_t)t]);
        int e, l;
        rosa::sam_match(a, cur, (int)t, e, l);
        std::printf("%ld %d %d\n", t, e, l);
    }
    return 0;
}
