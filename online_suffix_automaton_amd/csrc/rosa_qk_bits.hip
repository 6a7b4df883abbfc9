// rosa_qk_bits.hip -- query/key retrieval, bit-parallel over the key units.
//
// Method: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix Matching"
// (arXiv 2602.02499), Sec. 3.3 with separate query and key streams (the
// match is the longest suffix of the query units that occurs among the
// earlier key units, its end the most recent such unit; run folding as in
// the run-length paragraph), App. C.5 (counterfactual branches: one more
// matching update with one query bit forced).
//
// The same results as the automaton kernels of rosa_sam.hip, computed as
// sets instead of states.  For unit u and length l let B_l(u) be the set of
// key units e < u at which the last l query units end as well:
//   B_1(u) = { e < u : k_e = q_u },
//   B_l(u) = { e < u : k_e = q_u and e-1 in B_{l-1}(u-1) },
// so B_l(u) = (B_{l-1}(u-1) shifted up by one) & EQ(q_u), with EQ(c) the set
// of key units so far with symbol c.  L(u) is the largest l with B_l(u)
// nonempty and E(u) its largest member; L(u) <= L(u-1) + 1.  A stream of at
// most 4096 units is one wave: every set is a 4096-bit vector, lane w holding
// bits 64w..64w+63, so one update of a set is a few instructions for all
// candidate ends at once, and the levels 1..L live in registers.  A
// counterfactual branch is the same update with the flipped symbol's EQ,
// computed from the sets before the unit's own update.
//
// Matches longer than kQbLevels units are not followed: such a stream is
// marked in redo[] and answered by the automaton kernel instead.
#include "rosa_internal.h"

namespace rosa {

constexpr int kQbLevels = 32;    // levels kept in registers
constexpr int kQbMaxT = 4096;    // one 64-bit word per lane
constexpr int kQbMaxK = 64;

// The 4096-bit vector shifted up by one: bit e of the result is bit e-1 of v
// (the carry into each word is the top bit of the lane below, by a
// wave_shr:1 DPP move; lane 0 receives 0).
__device__ __forceinline__ uint64_t qb_shl1(uint64_t v)
{
    const int top = (int)(uint32_t)(v >> 63);
    const int c = __builtin_amdgcn_update_dpp(0, top, 0x138, 0xF, 0xF, false);
    return (v << 1) | (uint64_t)(uint32_t)c;
}

// The chains of one unit: the unit's own update (chain 0) and its
// counterfactual branches (chains 1..NCH-1), each with its symbol's EQ word,
// its number of nonempty levels and the set at the last of them.
template <int NCH>
struct QbChains {
    uint64_t eq[NCH], top[NCH];
    int L[NCH];
    bool over;   // a chain is still nonempty past kQbLevels
};

// Level l of every chain: all of them shift the same set, B_{l-1} of the
// previous unit (`prev`, read before chain 0 overwrites it), and AND it with
// their EQ; chain 0 stores its new level in B.  A set that is empty at one
// level is empty at every higher one (B_l is contained in B_{l-1}), so the
// chains need no liveness of their own: the levels stop once all of them are
// empty or the previous unit's depth is passed.  Unrolled by template
// recursion so that B stays in registers.
template <int l, int NCH>
__device__ __forceinline__ void qb_levels(uint64_t (&B)[kQbLevels], uint64_t prev,
                                          int lim, QbChains<NCH> &c)
{
    if constexpr (l <= kQbLevels) {
        if (l > lim)
            return;
        const uint64_t old = B[l - 1];
        const uint64_t sh = l == 1 ? ~0ull : qb_shl1(prev);
        bool any = false;
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const uint64_t nw = sh & c.eq[i];
            const bool ne = __builtin_amdgcn_ballot_w64(nw != 0) != 0;
            c.top[i] = ne ? nw : c.top[i];
            c.L[i] = ne ? l : c.L[i];
            any = any || ne;
            if (i == 0)
                B[l - 1] = nw;
        }
        if (!any)
            return;
        qb_levels<l + 1, NCH>(B, old, lim, c);
    } else {
        // past the kept levels: a chain that would still grow is not followed
        if (l <= lim) {
            const uint64_t sh = qb_shl1(prev);
#pragma unroll
            for (int i = 0; i < NCH; ++i)
                if (__builtin_amdgcn_ballot_w64((sh & c.eq[i]) != 0))
                    c.over = true;
        }
    }
}

// Largest member of a nonempty set (wave-uniform).
__device__ __forceinline__ int qb_top(uint64_t v)
{
    const uint64_t lanes = __builtin_amdgcn_ballot_w64(v != 0);
    const int h = 63 - __clzll((long long)lanes);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, h);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), h);
    const uint64_t w = ((uint64_t)hi << 32) | lo;
    return 64 * h + 63 - __clzll((long long)w);
}

// Symbol of chain i for query symbol q: q itself, then q with bit i-1 flipped.
template <int i>
__device__ __forceinline__ int qb_sym(int q)
{
    return (i == 0 ? q : (q ^ (1 << ((i - 1) & 7)))) & (kQbMaxK - 1);
}

// Reads the EQ words of every chain's symbol for query symbol q.
template <int i, int NCH>
__device__ __forceinline__ void qb_read_next(uint64_t (&eqn)[NCH],
                                             const uint64_t (&eq)[kQbMaxK][64],
                                             int q, int lane)
{
    if constexpr (i < NCH) {
        eqn[i] = eq[qb_sym<i>(q)][lane];
        qb_read_next<i + 1, NCH>(eqn, eq, q, lane);
    }
}

// One wave per stream.  NCH chains per unit (1, or 1 + M with the
// counterfactual tables); RLE: key runs folded into units.
//
// Per position the wave does wave-uniform work only: a new unit appends its
// key symbol to EQ and issues the LDS reads of the next position's EQ words
// (so their latency hides behind this unit's levels), then runs the levels.
// The unit's answer (end, length, unit index, query symbol, branch ends) is
// staged in lane j of the 64-position chunk by writelane; the outputs that
// need the start time of a unit are formed after the chunk, one position per
// lane, with the unit starts read from LDS in one gather.
template <int NCH, bool RLE>
__global__ __launch_bounds__(64) void qk_bits_kernel(QkParams p)
{
    __shared__ uint64_t eq[kQbMaxK][64];
    __shared__ uint16_t st[RLE ? kQbMaxT : 1];
    constexpr int M = NCH - 1;
    const int lane = threadIdx.x;
    const int64_t s = blockIdx.x;
    const int T = (int)p.T;
    for (int c = 0; c < p.K; ++c)
        eq[c][lane] = 0;
    __syncthreads();
    const uint8_t *qr = p.q + s * p.Tp + kPadFront;
    const uint8_t *kr = p.k + s * p.Tp + kPadFront;
    const int64_t base = s * (int64_t)T;
    uint64_t B[kQbLevels];
#pragma unroll
    for (int l = 0; l < kQbLevels; ++l)
        B[l] = 0;
    int Lc = 0;               // levels 1..Lc of the previous unit are nonempty
    bool over = false;
    int u = -1, kprev = -1, qc = 0, ue = -1, ul = 0;
    int cfe[M > 0 ? M : 1];
#pragma unroll
    for (int b = 0; b < M; ++b)
        cfe[b] = -1;
    // EQ words of the next position's query symbol (nothing appended yet)
    uint64_t eqn[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i)
        eqn[i] = 0;
    // the next key unit's bit: unit u is bit u%64 of lane u/64
    uint64_t wbit = lane == 0 ? 1ull : 0ull;
    // the rows carry 64 bytes of padding after T: chunk loads stay in the row
    int kn = kr[lane], qn = qr[lane];
    for (int t0 = 0; t0 < T && !over; t0 += 64) {
        const int kch = kn, qch = qn;
        if (t0 + 64 < T) {
            kn = kr[t0 + 64 + lane];
            qn = qr[t0 + 64 + lane];
        }
        int o_end = -1, o_len = 0, o_run = -1, o_q = 0;
        int o_ce[M > 0 ? M : 1];
#pragma unroll
        for (int b = 0; b < M; ++b)
            o_ce[b] = -1;
        const int n = T - t0 < 64 ? T - t0 : 64;
        for (int j = 0; j < n; ++j) {
            const int kc = __builtin_amdgcn_readlane(kch, j);
            // query symbol of the next position (the padding past T reads 0)
            const int qx = j < 63 ? __builtin_amdgcn_readlane(qch, j + 1)
                                  : __builtin_amdgcn_readlane(qn, 0);
            if (!RLE || kc != kprev) {
                ++u;
                qc = __builtin_amdgcn_readlane(qch, j);
                if (RLE && lane == 0)
                    st[u] = (uint16_t)(t0 + j);
                QbChains<NCH> c;
#pragma unroll
                for (int i = 0; i < NCH; ++i) {
                    c.eq[i] = eqn[i];
                    c.top[i] = 0;
                    c.L[i] = 0;
                }
                c.over = false;
                // append key unit u (this unit's chains use the words read
                // before it), then read the next position's words
                atomicOr(reinterpret_cast<unsigned long long *>(&eq[kc & (kQbMaxK - 1)][lane]),
                         (unsigned long long)wbit);
                wbit = qb_shl1(wbit);
                qb_read_next<0, NCH>(eqn, eq, qx, lane);
                qb_levels<1, NCH>(B, 0ull, Lc + 1, c);
                over = over || c.over;
                Lc = c.L[0];
                ul = c.L[0];
                ue = ul > 0 ? qb_top(c.top[0]) : -1;
#pragma unroll
                for (int b = 0; b < M; ++b)
                    cfe[b] = c.L[b + 1] > 0 ? qb_top(c.top[b + 1]) : -1;
                kprev = kc;
            } else {
                qb_read_next<0, NCH>(eqn, eq, qx, lane);
            }
            // this position's answer, staged in lane j
            const bool mine = lane == j;
            o_end = mine ? ue : o_end;
            o_len = mine ? ul : o_len;
            o_run = mine ? u : o_run;
            if (M > 0)
                o_q = mine ? qc : o_q;
#pragma unroll
            for (int b = 0; b < M; ++b)
                o_ce[b] = mine ? cfe[b] : o_ce[b];
        }
        if (lane < n && !over) {
            const int t = t0 + lane;
            const int64_t o = base + t;
            // a match ending at unit e is usable once unit e+1 has started
            const int ds = o_end >= 0 ? (RLE ? (int)st[o_end + 1] : o_end + 1) : -1;
            const int tt = (o_end >= 0 && ds < t) ? ds : -1;
            const int rt = tt >= 0 ? o_end + 1 : -1;
            p.tau[o] = tt;
            if (p.end)
                p.end[o] = o_end;
            if (p.len)
                p.len[o] = o_len;
            if (p.run_of)
                p.run_of[o] = o_run;
            if (p.ridx)
                p.ridx[o] = rt;
#pragma unroll
            for (int b = 0; b < M; ++b) {
                const int ce = o_ce[b];
                const int cd = ce >= 0 ? (RLE ? (int)st[ce + 1] : ce + 1) : -1;
                const int tb = (ce >= 0 && cd < t) ? cd : -1;
                const int rb = tb >= 0 ? ce + 1 : -1;
                const bool bit = (o_q >> b) & 1;
                const int64_t c0 = (o * M + b) * 2;
                if (p.cf_tau)
                    *reinterpret_cast<int2 *>(p.cf_tau + c0) =
                        bit ? make_int2(tb, tt) : make_int2(tt, tb);
                if (p.cf_ridx)
                    *reinterpret_cast<int2 *>(p.cf_ridx + c0) =
                        bit ? make_int2(rb, rt) : make_int2(rt, rb);
            }
        }
    }
    if (!over && p.run_start)
        for (int v = lane; v < T; v += 64)
            p.run_start[base + v] = v <= u ? (RLE ? (int32_t)st[v] : v) : -1;
    if (lane == 0)
        p.redo[s] = over ? 1 : 0;
}

bool qk_bits_fits(const QkParams &p)
{
    // with the tables, K = 2^M <= 64: at most 7 chains
    return p.T <= kQbMaxT && p.K <= kQbMaxK &&
           (!(p.cf_tau || p.cf_ridx) || p.M <= 6);
}

template <bool RLE>
static hipError_t launch_qk_bits_r(const QkParams &p, int nch, hipStream_t st)
{
    const dim3 g((unsigned)p.S), b(64);
    switch (nch) {
    case 1: hipLaunchKernelGGL((qk_bits_kernel<1, RLE>), g, b, 0, st, p); break;
    case 2: hipLaunchKernelGGL((qk_bits_kernel<2, RLE>), g, b, 0, st, p); break;
    case 3: hipLaunchKernelGGL((qk_bits_kernel<3, RLE>), g, b, 0, st, p); break;
    case 4: hipLaunchKernelGGL((qk_bits_kernel<4, RLE>), g, b, 0, st, p); break;
    case 5: hipLaunchKernelGGL((qk_bits_kernel<5, RLE>), g, b, 0, st, p); break;
    case 6: hipLaunchKernelGGL((qk_bits_kernel<6, RLE>), g, b, 0, st, p); break;
    case 7: hipLaunchKernelGGL((qk_bits_kernel<7, RLE>), g, b, 0, st, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_qk_bits(const QkParams &p, hipStream_t st)
{
    const int nch = (p.cf_tau || p.cf_ridx) ? 1 + p.M : 1;
    return p.rle ? launch_qk_bits_r<true>(p, nch, st)
                 : launch_qk_bits_r<false>(p, nch, st);
}

}  // namespace rosa
