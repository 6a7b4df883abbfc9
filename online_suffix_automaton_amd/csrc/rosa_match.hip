// rosa_match.hip -- batch retrieval for all positions of all streams.
//
// Method: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix Matching"
// (arXiv 2602.02499).  Sec. 3.3 with App. B.3: at position t the retrieval
// hits the longest suffix of x[0..t] that occurred before, and the
// destination is the end position of that earlier occurrence plus one
// (the most recent one).  Sec. 4.1: streams are independent.  The pages run
// this with one suffix automaton per stream on CPU cores; that design is a
// chain of dependent pointer loads per stream and does not map onto a GPU.
// Here the same result is computed data-parallel over the time axis.
//
// Formulation.  With lcs(t,e) the length of the common suffix of x[0..t]
// and x[0..e], the pair (L(t), E(t)) is the lexicographic maximum of
// (lcs(t,e), e) over e < t (L = 0, E = -1 when every lcs is 0).  Group the
// positions of a stream by their reversed l-gram (x[t], x[t-1], ..,
// x[t-l+1]); in time order, the predecessor of t inside its l-group is the
// most recent earlier occurrence of that l-gram.  Refining groups level by
// level (MSD order on the reversed prefixes), an element's answer is fixed
// at the level where it stops having an earlier group member:
//   L(t) = that level l, E(t) = its predecessor in the level-l group.
//
// Kernels.
//   stream_kernel (one 1024-thread workgroup per stream):
//     0  the stream's symbols are staged in LDS (T <= 65536);
//     A  histogram of d-gram keys in LDS, first occurrence of every l-gram
//        (l <= d) by LDS atomicMin;
//     B  scan -> bucket offsets; buckets packed into <=64-element tasks;
//        buckets larger than 64 go to a global list;
//     D  positions whose d-gram is new (L < d) and the first d-1 positions
//        are answered from the first-occurrence tables plus a time-ordered
//        scan per segment (ballot match inside 64-position chunks, LDS
//        last-end tables across chunks and segments);
//     E  positions scattered into buckets (LDS atomics), each bucket put in
//        time order (insertion sort, one bucket per thread); each wave then
//        takes tasks: a group is the lane range of one bucket, refined with
//        lane masks (solve_wave).
//   big_kernel (one wave per bucket of more than 64 positions): rebuilds the
//     bucket in time order, then refines it with stable partitions by the
//     next symbol until groups fit a wave, then solve_wave.
#include "rosa_internal.h"

namespace rosa {

constexpr uint32_t kFirstFlag = 0x80000000u;
// level steps only for groups larger than this (the direct comparison runs
// as many rounds as the wave's largest group has earlier members, so a
// split is cheaper past two: measured 2 against 3, long workload 1% faster,
// repeat workload 1% slower)
constexpr int kWordThresh = 2;
constexpr int kMiscPass = 26;        // misc[26..31]: tasks per slot range
constexpr int kMiscNext = 20;        // misc[20]: next task of the pass (phase E)
constexpr int kMiscLastQ = 21;       // misc[21]: last position with L < d (phase D)
constexpr int kMiscBig = 22;         // misc[22]: the stream's large buckets (LDS kernel)
constexpr int kWordThreshDeep = 32;  // ... and past the first levels, larger than this

// ----------------------------------------------------------- wave helpers

// The stream's own list of buckets of more than 64 members (LDS kernel):
// {s, key, start, n} entries, at most T/65 + 1 per stream (the global list's
// capacity is S times that).
__device__ __forceinline__ int32_t *big_own(const MatchParams &p, int s)
{
    return p.big + 64 + 4 * (int64_t)s * (p.T / 65 + 1);
}

__device__ __forceinline__ uint64_t ballot(bool p)
{
    return __builtin_amdgcn_ballot_w64(p);
}

__device__ __forceinline__ int wave_incl_scan(int v)
{
    const int lane = __lane_id();
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(v, o);
        if (lane >= o)
            v += u;
    }
    return v;
}

// Symbols x[p .. p+15] as two little-endian 64-bit halves: byte i of
// (lo, hi) is x[p+i].  `row` is 4-byte aligned and zero padded, so p may be
// slightly negative or run past the end.  Five aligned dword reads and a
// byte funnel shift (pointer arithmetic keeps the row's address space, so
// an LDS row is read with ds_read).
__device__ __forceinline__ void load_window(const uint8_t *row, int p,
                                            uint64_t &lo, uint64_t &hi)
{
    const uint32_t *q = reinterpret_cast<const uint32_t *>(row) + (p >> 2);
    const uint32_t sh = (uint32_t)(p & 3);
    const uint32_t d0 = q[0], d1 = q[1], d2 = q[2], d3 = q[3], d4 = q[4];
    const uint32_t w0 = __builtin_amdgcn_alignbyte(d1, d0, sh);
    const uint32_t w1 = __builtin_amdgcn_alignbyte(d2, d1, sh);
    const uint32_t w2 = __builtin_amdgcn_alignbyte(d3, d2, sh);
    const uint32_t w3 = __builtin_amdgcn_alignbyte(d4, d3, sh);
    lo = (uint64_t)w0 | ((uint64_t)w1 << 32);
    hi = (uint64_t)w2 | ((uint64_t)w3 << 32);
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src)
{
    const uint32_t a = __shfl((uint32_t)v, src);
    const uint32_t b = __shfl((uint32_t)(v >> 32), src);
    return (uint64_t)a | ((uint64_t)b << 32);
}

// Where results go.  Direct mode writes E / SYM / L of the stream at t.
// Record mode (streams of <= 65536 positions) writes one 32-bit record
// (t << 16 | E+1) per bucket slot, coalesced; a later kernel scatters the
// records into time order in LDS and writes E and SYM.  L, if requested,
// is always written directly.
struct StreamOut {
    const uint8_t *x;  // padded symbol row of the stream (LDS or HBM)
    int32_t *E;
    int16_t *SYM;
    int32_t *L;
    uint32_t *rec;     // record row (record mode) or null
};

__device__ __forceinline__ void emit(const StreamOut &o, int t, int e, int l)
{
    o.E[t] = e;
    if (o.L)
        o.L[t] = l;
    if (o.SYM)
        o.SYM[t] = e >= 0 ? (int16_t)o.x[e + 1] : (int16_t)-1;
}

__device__ __forceinline__ void emit_record(const StreamOut &o, int slot,
                                            int t, int e, int l)
{
    o.rec[slot] = ((uint32_t)t << 16) | (uint32_t)(e + 1);
    if (o.L)
        o.L[t] = l;
}

struct Found {
    int e, l;       // deep: e = 1 when the record overflowed (more than seven members)
    bool ok;
    bool deep;      // CAP mode: answer deferred, its record written (solve_wave)
};

// Lanes of the wave with `sel` set whose symbol `dig` (< 16) equals mine, by
// one LDS OR and one LDS read on the wave's 16-word table `tab` (cleared
// first).  A wave's LDS operations are performed in issue order, so the
// clear, the ORs and the reads need no wait between them; the wave
// barriers only keep the compiler from moving them past each other.  The
// result is 0 for lanes without `sel`.
__device__ __forceinline__ uint64_t wave_symbol_mask(uint64_t *tab, bool sel,
                                                     uint32_t dig, uint64_t self)
{
    const int lane = __lane_id();
    if (lane < 16)
        tab[lane] = 0;
    __builtin_amdgcn_wave_barrier();
    if (sel)
        __hip_atomic_fetch_or(tab + dig, self, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
    __builtin_amdgcn_wave_barrier();
    const uint64_t r = sel ? tab[dig] : 0ull;
    __builtin_amdgcn_wave_barrier();
    return r;
}

// ------------------------------------------------------------ solve_wave
//
// Each lane holds one element t (or none).  g is the lane mask of its group:
// all members share the reversed `ell`-gram ending at their position, lane
// order is time order inside every group, and every member except the first
// already has L >= ell.  Returns (E, L) for every member that has an earlier
// member (ok); the first member of each group gets nothing.
//
//  level steps (while groups are large and still splitting: the first
//    levels after bucketing, or very large groups): split by the symbol
//    x[t-ell]; an element that is first in its new group but was not first
//    before gets L = ell and E = its previous group member.
//  direct resolution (then): each element compares its history with each
//    earlier member's, 16 symbols per step, up to the first mismatch or the
//    start of that member's history; the longest common extension c (the
//    latest member among equals) gives L = ell + c and E = that member.
//  CAP: the comparison stops after the first 16 symbols.  An element with
//    a member that matches all 16 and has a longer history (a recurrence of
//    more than ell + 16 symbols, inside long repeats) is answered later, in
//    time order (unpermute_kernel): its answer follows from the previous
//    position's by the extension rule, and otherwise from these members (the
//    only ones that can reach ell + 16).  The deferred record of element t
//    is drec[t]: sixteen-bit fields 0..6 hold up to seven such members,
//    field 7 their count (3 bits; 0: more than seven) and ell + 16 above it
//    (a lower bound of their common suffix with t).
template <bool CAP>
__device__ Found solve_wave(const uint8_t *x, int nbits, int t, uint64_t g,
                            int ell, bool has, uint4 *drec = nullptr,
                            uint64_t *eqw = nullptr)
{
    const int lane = __lane_id();
    const uint64_t self = 1ull << lane;
    const uint64_t below = self - 1;
    Found r = {-1, 0, false, false};
    if (!has)
        g = self;
    const int ell0 = ell;
    for (;;) {
        // the lane's group size, 0 without an element (the predicates below
        // are compares of it, so each ballot is one vector compare)
        const int pc = has ? __popcll(g) : 0;
        const bool live = pc >= 2;
        const uint64_t liveb = ballot(pc >= 2);
        if (liveb == 0)
            return r;
        // level steps while some group is larger than kWordThresh during the
        // first two levels after bucketing (groups still split fast there),
        // later only while some group is larger than kWordThreshDeep
        const int th = ell <= ell0 + 1 ? kWordThresh : kWordThreshDeep;
        if (ballot(pc > th) == 0)
            break;
        // ---------------------------------------------------- level step
        // split every group by the symbol x[t-ell]: lanes agree on it iff
        // they agree on each of its nbits bits (one ballot per bit)
        const bool valid = pc >= 2 && (t - ell >= 0);
        const uint32_t dig = valid ? (uint32_t)x[t - ell] : 0u;
        uint64_t eq;
        if (eqw) {
            // alphabets of at most 16 symbols: every valid lane ORs its bit
            // into its symbol's word of the wave's LDS table and reads the
            // word back (one wave's LDS operations complete in issue order,
            // so the clear, the ORs and the reads need no wait between them)
            eq = wave_symbol_mask(eqw, valid, dig, self);
        } else {
            // (a compare straight to a lane mask: the compiler would rebuild
            // the ballot of the compare it already made for `valid`)
            const uint64_t vmask = liveb & __builtin_amdgcn_sicmp(t - ell, 0, 39 /* >= */);
            // eq = lanes of vmask whose symbol equals mine; per bit b, with
            // m = all ones where my bit is set, each 32-bit half is
            // e & (B == m), one 3-input bit op (table 0x90 over (e, B, m));
            // vmask is applied last, so that no bit op takes two scalar
            // operands
            uint32_t eql = ~0u, eqh = ~0u;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)dig, b, 1);
                const uint64_t B = ballot(m != 0);
                eql = __builtin_amdgcn_bitop3_b32(eql, (uint32_t)B, m, 0x90);
                eqh = __builtin_amdgcn_bitop3_b32(eqh, (uint32_t)(B >> 32), m, 0x90);
                if (b + 1 >= nbits)
                    break;
            }
            eq = vmask & (((uint64_t)eqh << 32) | eql);
        }
        const uint64_t ng = valid ? (g & eq) : self;
        const uint64_t prev = g & below;
        const int p = prev ? 63 - __clzll((long long)prev) : lane;
        const int e_prev = __shfl(t, p);
        if (live && prev && !(ng & below)) {
            r.e = e_prev;
            r.l = ell;
            r.ok = true;
        }
        if (live)
            g = ng;
        ++ell;
    }
    // ------------------------------------------------- direct resolution
    uint64_t rem = (has && __popcll(g) >= 2) ? (g & below) : 0;
    int best_c = -1, best_e = -1;
    int ntr = 0;            // CAP: members deferred (full 16-symbol match)
    uint16_t *dr = CAP && has ? reinterpret_cast<uint16_t *>(drec + t) : nullptr;
    // every element's first 16 symbols past level ell, shared by shuffle
    uint64_t w0lo = 0, w0hi = 0;
    if (has && t - ell >= 0)
        load_window(x, t - ell - 15, w0lo, w0hi);
    while (ballot(rem != 0)) {
        const bool have = rem != 0;
        const int j = have ? __ffsll((long long)rem) - 1 : lane;
        rem &= rem - 1;
        const int tj = __shfl(t, j);
        const uint64_t jlo = shfl64(w0lo, j), jhi = shfl64(w0hi, j);
        if (have) {
            const int aj = tj - ell + 1;   // history of member j from x[tj-ell]
            // first 16 symbols from the shared windows, further ones from
            // memory while they keep matching
            const uint64_t fh = w0hi ^ jhi, fl = w0lo ^ jlo;
            // leading equal bytes of (fh, fl), at most 16 (both counts
            // computed and one selected: no divergent branch)
            const int zh = __clzll((long long)fh), zl = __clzll((long long)fl);
            int c = (fh != 0 ? zh : 64 + zl) >> 3;
            if (CAP && !(fh | fl) && c < aj) {
                if (ntr < 7)
                    dr[ntr] = (uint16_t)tj;
                ++ntr;
                c = -2;   // never wins below
            } else if (!CAP && !(fh | fl)) {
                // 64 symbols per step (long recurrences); every read stays
                // at or after position -63 because c < aj <= t - ell and
                // tj - ell - c >= 0, inside the rows' front padding
                while (c < aj) {
                    uint64_t xs[8];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        uint64_t alo, ahi, blo, bhi;
                        load_window(x, t - ell - c - 15 - 16 * q, alo, ahi);
                        load_window(x, tj - ell - c - 15 - 16 * q, blo, bhi);
                        xs[2 * q] = ahi ^ bhi;
                        xs[2 * q + 1] = alo ^ blo;
                    }
                    int k = 0;
                    while (k < 8 && !xs[k])
                        ++k;
                    if (k < 8) {
                        c += 8 * k + (__clzll((long long)xs[k]) >> 3);
                        break;
                    }
                    c += 64;
                }
            }
            c = min(c, aj);
            if (c >= best_c) {
                best_c = c;
                best_e = tj;
            }
        }
    }
    if (CAP && ntr > 0) {
        // an exact 16 among the others ties with a deferred member that
        // stops at 16: it joins them
        if (best_c == 16) {
            if (ntr < 7)
                dr[ntr] = (uint16_t)best_e;
            ++ntr;
        }
        dr[7] = (uint16_t)((ntr > 7 ? 0 : ntr) | (min(ell + 16, 8191) << 3));
        r.e = ntr > 7 ? 1 : 0;   // more members than the record holds
        r.ok = true;
        r.deep = true;
        return r;
    }
    if (best_c >= 0) {
        r.e = best_e;
        r.l = ell + best_c;
        r.ok = true;
    }
    return r;
}

// ------------------------------------------------------------ block scan

// Exclusive scan over the block of one int per thread; returns the prefix,
// writes the total to *total.  ws: >= 16 ints of LDS.
__device__ int block_excl_scan(int v, int *ws, int *total)
{
    const int lane = __lane_id();
    const int wid = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63)
        ws[wid] = incl;
    __syncthreads();
    if (wid == 0) {
        int s = lane < nw ? ws[lane] : 0;
        const int si = wave_incl_scan(s);
        if (lane < nw)
            ws[lane] = si - s;
        if (lane == nw - 1)
            ws[16] = si;
    }
    __syncthreads();
    const int r = ws[wid] + incl - v;
    *total = ws[16];
    __syncthreads();
    return r;
}

// ---------------------------------------------------------- shared phases

constexpr int kSegTabInts = 8192;

// The four symbols x[t-3..t] as one word, x[t] in the top byte (one LDS or
// cache round trip instead of one per symbol; rows carry zero padding in
// front, so t-3 >= -3 stays inside).
__device__ __forceinline__ uint32_t load4_end(const uint8_t *row, int t)
{
    const int p = t - 3;
    const uint32_t *q = reinterpret_cast<const uint32_t *>(row) + (p >> 2);
    return __builtin_amdgcn_alignbyte(q[1], q[0], (uint32_t)(p & 3));
}

// The eight symbols x[t-7..t] (x[t] in the top byte); t-7 >= -7 stays in
// the front padding.
__device__ __forceinline__ uint64_t load8_end(const uint8_t *row, int t)
{
    const int p = t - 7;
    const uint32_t *q = reinterpret_cast<const uint32_t *>(row) + (p >> 2);
    const uint32_t sh = (uint32_t)(p & 3);
    const uint32_t d0 = q[0], d1 = q[1], d2 = q[2];
    return (uint64_t)__builtin_amdgcn_alignbyte(d1, d0, sh) |
           ((uint64_t)__builtin_amdgcn_alignbyte(d2, d1, sh) << 32);
}

// Key of the d-gram (d <= 4) whose last symbol is the top byte of w.
__device__ __forceinline__ int key_of_word(uint32_t w, int d, int K)
{
    int k = (int)(w >> 24);
    if (d > 1)
        k = (int)__umul24((uint32_t)k, (uint32_t)K) + (int)((w >> 16) & 0xFFu);
    if (d > 2)
        k = (int)__umul24((uint32_t)k, (uint32_t)K) + (int)((w >> 8) & 0xFFu);
    if (d > 3)
        k = (int)__umul24((uint32_t)k, (uint32_t)K) + (int)(w & 0xFFu);
    return k;
}

// Symbol x[t-i] (i < 4) out of load4_end's word.
__device__ __forceinline__ int sym_of(uint32_t w, int i)
{
    return (int)((w >> (24 - 8 * i)) & 0xFFu);
}

// Key of the reversed d-gram ending at t (t >= d-1): x[t] is the most
// significant digit.  Its top l digits form the key of the l-gram.
__device__ __forceinline__ int dgram_key(const uint8_t *x, int t, int d, int K)
{
    if (d <= 4)
        return key_of_word(load4_end(x, t), d, K);
    int k = 0;
    for (int i = 0; i < d; ++i)
        k = (int)__umul24((uint32_t)k, (uint32_t)K) + x[t - i];
    return k;
}

// Phase A: d-gram histogram and first occurrence of every l-gram, l <= d.
// Positions are counted four per thread (one 8-symbol read covers their
// d-grams when d <= 4).  The first occurrence of a shorter l-gram is the
// minimum over its K one-symbol-longer extensions (the l-gram ending at t
// is the top l digits of the d-gram ending at t), taken level by level
// down from d-1; the few positions t < d-1 that end l-grams but no d-gram
// enter the l-gram tables directly.
template <int DC>
__device__ void phase_hist(const MatchParams &p, const uint8_t *x, int32_t *cnt,
                           int32_t *firstd, int32_t *firstl)
{
    const int tid = threadIdx.x, nt = blockDim.x;
    const int T = p.T, K = p.K, d = DC > 0 ? DC : p.d;
    for (int i = tid; i < p.NB; i += nt) {
        cnt[i] = 0;
        firstd[i] = 0x7FFFFFFF;
    }
    for (int i = tid; i < p.fl_total; i += nt)
        firstl[i] = 0x7FFFFFFF;
    __syncthreads();
    for (int t0 = d - 1 + 4 * tid; t0 < T; t0 += 4 * nt) {
        const uint64_t v8 = d <= 4 ? load8_end(x, t0 + 3) : 0ull;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = t0 + u;
            if (t < T) {
                const int k = d <= 4 ? key_of_word((uint32_t)(v8 >> (8 * (u + 1))), d, K)
                                     : dgram_key(x, t, d, K);
                atomicAdd(&cnt[k], 1);
                if (t < firstd[k])
                    atomicMin(&firstd[k], t);
            }
        }
    }
    if (tid < d - 1 && tid < T) {
        const int t = tid;
        int k = 0;
        for (int i = 0; i <= t; ++i) {
            k = (int)__umul24((uint32_t)k, (uint32_t)K) + x[t - i];
            atomicMin(&firstl[p.fl_off[i + 1] + k], t);
        }
    }
    __syncthreads();
    for (int l = d - 1; l >= 1; --l) {
        const int n = p.pw[l];
        const int32_t *up = l + 1 == d ? firstd : firstl + p.fl_off[l + 1];
        for (int g = tid; g < n; g += nt) {
            int m = firstl[p.fl_off[l] + g];
            for (int c = 0; c < K; ++c)
                m = min(m, up[g * K + c]);
            firstl[p.fl_off[l] + g] = m;
        }
        __syncthreads();
    }
}

// Phase B: bucket offsets, then buckets of 2..64 members are packed into
// tasks of at most 64 positions (a task never spans a singleton or large
// bucket, nor a boundary between position ranges of `pcap` slots) and
// lists buckets of more than 64 members for the large-group kernel.
// Returns the number of tasks in misc[24] and the number of tasks of each
// slot range in misc[kMiscPass + range] (tasks are in slot order, so the
// tasks of one range are consecutive).
template <class OffT>
__device__ void phase_tasks(const MatchParams &p, int s, const int32_t *cnt,
                            OffT *off, uint32_t *tasks, int32_t *misc,
                            int pcap, bool own_big = false, int run_pos = 256)
{
    const int tid = threadIdx.x, nt = blockDim.x;
    const int NB = p.NB;
    {
        const int per = (NB + nt - 1) / nt;
        const int b0 = tid * per;
        int local = 0;
        for (int q = 0; q < per; ++q)
            if (b0 + q < NB)
                local += cnt[b0 + q];
        int total;
        int ex = block_excl_scan(local, misc, &total);
        for (int q = 0; q < per; ++q)
            if (b0 + q < NB) {
                off[b0 + q] = (OffT)ex;
                ex += cnt[b0 + q];
            }
        if (tid == 0)
            off[NB] = (OffT)total;
    }
    __syncthreads();
    // Each thread packs a run of `bpl` consecutive buckets (about run_pos
    // positions' worth, at least NB/nt so every bucket is covered); tasks
    // do not span runs, so longer runs pack tasks fuller, while shorter ones
    // spread the packing over more threads (the better trade on short
    // streams, whose packing is a larger share of the kernel).
    const int avg = max(1, (int)off[NB] / NB);
    const int bpl = max((NB + nt - 1) / nt, min(64, max(1, run_pos / avg)));
    const int b0 = min(NB, tid * bpl), b1 = min(NB, b0 + bpl);
    int ntask = 0, cur = 0, crange = -1;
    for (int b = b0; b < b1; ++b) {
        const int c = cnt[b];
        if (c == 0)
            continue;
        if (c == 1 || c > 64) {
            if (cur) {
                ++ntask;
                cur = 0;
            }
            continue;
        }
        const int rg = (int)off[b] / pcap;
        if (cur + c > 64 || (cur && rg != crange)) {
            ++ntask;
            cur = 0;
        }
        crange = rg;
        cur += c;
    }
    if (cur)
        ++ntask;
    int total;
    int k = block_excl_scan(ntask, misc, &total);
    auto put_task = [&](int i, int st, int n) {
        tasks[i] = ((uint32_t)st << 6) | (uint32_t)(n - 1);
        atomicAdd(&misc[kMiscPass + st / pcap], 1);
    };
    int start = 0;
    cur = 0;
    crange = -1;
    for (int b = b0; b < b1; ++b) {
        const int c = cnt[b];
        if (c == 0)
            continue;
        if (c == 1 || c > 64) {
            if (cur) {
                put_task(k++, start, cur);
                cur = 0;
            }
            if (c > 64) {
                // own_big: the stream's own list (misc[kMiscBig] entries from
                // big_own(p, s)), solved by the stream's workgroup; else the
                // global list of big_kernel
                int32_t *ent = nullptr;
                if (own_big) {
                    const int idx = atomicAdd(&misc[kMiscBig], 1);
                    ent = big_own(p, s) + 4 * (int64_t)idx;   // < T/65 + 1 entries
                } else {
                    const int idx = atomicAdd(&p.big[0], 1);
                    if (idx < p.big_cap)
                        ent = p.big + 64 + 4 * (int64_t)idx;
                }
                if (ent) {
                    ent[0] = s;
                    ent[1] = b;
                    ent[2] = (int32_t)off[b];
                    ent[3] = c;
                }
            }
            continue;
        }
        const int rg = (int)off[b] / pcap;
        if (cur + c > 64 || (cur && rg != crange)) {
            put_task(k++, start, cur);
            cur = 0;
        }
        crange = rg;
        if (cur == 0)
            start = (int)off[b];
        cur += c;
    }
    if (cur)
        put_task(k++, start, cur);
    if (tid == 0)
        misc[24] = total;
    __syncthreads();
}

// Phase D: positions with L < d: the first d-1 positions and the first
// occurrence of every d-gram.  L is the longest l < d whose l-gram occurred
// before t (first-occurrence tables); E is the latest earlier end of that
// l-gram.  Wave w scans time segment w in chunks of 64 in order, keeping the
// last end of every l-gram seen so far in segment w (segtab[w]); inside a
// chunk, the latest earlier lane with the same l-gram comes from a ballot
// match.  Queries with no earlier end inside their segment are resolved
// after the scan from the tables of earlier segments.  `put(t, e, l, k)`
// receives every answer, with k the d-gram key of t when t >= d-1.
template <int DC, class Put, class PendT>
__device__ void phase_short(const MatchParams &p, const uint8_t *x,
                            const int32_t *firstd, const int32_t *firstl,
                            int32_t *segtab, int segcap, PendT *pend,
                            int32_t *misc, Put put, uint64_t *eqw = nullptr)
{
    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63, wid = tid >> 6, nw = nt >> 6;
    const uint64_t self = 1ull << lane;
    const uint64_t below = self - 1;
    const uint64_t above = ~(below | self);
    const int T = p.T, K = p.K, d = DC > 0 ? DC : p.d, FL = p.fl_total;
    const int nseg = FL > 0 ? max(1, min(nw, segcap / FL)) : nw;
    for (int i = tid; i < nseg * FL; i += nt)
        segtab[i] = -1;
    if (tid == 0)
        misc[25] = 0;
    // The last query: the latest first occurrence of a d-gram (or d-2).  The
    // tables are read only by queries, for their own or earlier segments, so
    // the scan stops after it (misc[kMiscLastQ] starts at zero).
    {
        int m = 0;
        for (int i = tid; i < p.NB; i += nt) {
            const int f = firstd[i];
            if (f < T)
                m = max(m, f);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            m = max(m, __shfl_xor(m, o));
        if (lane == 0)
            atomicMax(&misc[kMiscLastQ], m);
    }
    __syncthreads();
    const int tend = min(T, max(misc[kMiscLastQ], d - 2) + 1);
    // segments of whole chunks over [0, tend)
    const int Ts = (((tend + nseg - 1) / nseg) + 63) & ~63;
    // lanes with the same digit as mine among those of m0: per bit, with
    // mb = all ones where my bit is set, each 32-bit half is e & (B == mb),
    // one 3-input bit op (table 0x90); m0 (two compares straight to lane
    // masks) is applied at the end
    auto same_digit = [&](int dig, uint64_t m0) {
        uint32_t ml = ~0u, mh = ~0u;
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint32_t mb = (uint32_t)__builtin_amdgcn_sbfe(dig, b, 1);
            const uint64_t B = ballot(mb != 0);
            ml = __builtin_amdgcn_bitop3_b32(ml, (uint32_t)B, mb, 0x90);
            mh = __builtin_amdgcn_bitop3_b32(mh, (uint32_t)(B >> 32), mb, 0x90);
            if (b + 1 >= p.nbits)
                break;
        }
        return m0 & (((uint64_t)mh << 32) | ml);
    };
    if constexpr (DC >= 1 && DC <= 4) {
        // d <= 4: a chunk's symbols x[t-3..t] are one word per lane, so every
        // table read of the chunk is issued at once, right after that word
        // (the next chunk's word is fetched with them).  The last-end reads
        // see the tables left by the earlier chunks, as in time order: this
        // chunk's writes come after them.
        if (wid < nseg) {
            int32_t *tab = segtab + wid * FL;
            const int lo = wid * Ts, hi = min(tend, lo + Ts);
            uint32_t wn = lo < hi ? load4_end(x, lo + lane) : 0u;
            for (int c0 = lo; c0 < hi; c0 += 64) {
                const int t = c0 + lane;
                const bool inr = t < hi;
                const uint32_t w = wn;
                const int kq = key_of_word(w, DC, K);
                const int fd = firstd[kq];
                int slot[DC], fl[DC], tb[DC];
                int gk = 0;
#pragma unroll
                for (int l = 1; l < DC; ++l) {
                    const bool v = inr && t >= l - 1;
                    gk = (int)__umul24((uint32_t)gk, (uint32_t)K) + (v ? sym_of(w, l - 1) : 0);
                    slot[l] = p.fl_off[l] + gk;
                    fl[l] = firstl[slot[l]];
                    tb[l] = tab[slot[l]];
                }
                if (c0 + 64 < hi)
                    wn = load4_end(x, t + 64);
                const bool q = inr && (t < DC - 1 || fd == t);
                int Lq = 0, Eq = -1;
                bool miss = false;
                uint64_t eq = ~0ull;
#pragma unroll
                for (int l = 1; l < DC; ++l) {
                    const bool v = inr && t >= l - 1;
                    const int dig = v ? sym_of(w, l - 1) : 0;
                    // lanes with t < hi and t >= l-1 (= v) and my digit
                    if (eqw)
                        eq &= wave_symbol_mask(eqw, v, (uint32_t)dig, self);
                    else
                        eq &= same_digit(dig, __builtin_amdgcn_sicmp(t, hi, 40 /* < */) &
                                                  __builtin_amdgcn_sicmp(t, l - 1, 39 /* >= */));
                    if (q && v && fl[l] < t) {
                        Lq = l;
                        const uint64_t pm = eq & below;
                        Eq = pm ? c0 + 63 - __clzll((long long)pm) : tb[l];
                        miss = !pm && tb[l] < 0;
                    }
                    if (v && !(eq & above))
                        tab[slot[l]] = t;
                }
                if (q) {
                    if (miss)
                        pend[atomicAdd(&misc[25], 1)] = (PendT)t;
                    else
                        put(t, Lq > 0 ? Eq : -1, Lq, kq);
                }
            }
        }
    } else if (wid < nseg) {
        int32_t *tab = segtab + wid * FL;
        const int lo = wid * Ts, hi = min(tend, lo + Ts);
        for (int c0 = lo; c0 < hi; c0 += 64) {
            const int t = c0 + lane;
            const bool inr = t < hi;
            const int kq = inr && t >= d - 1 ? dgram_key(x, t, d, K) : 0;
            const bool q = inr && (t < d - 1 || firstd[kq] == t);
            int Lq = 0, Eq = -1;
            bool miss = false;
            int gk = 0;
            uint64_t eq = ~0ull;
            for (int l = 1; l < d; ++l) {
                const bool v = inr && t >= l - 1;
                const int dig = v ? (int)x[t - l + 1] : 0;
                gk = (int)__umul24((uint32_t)gk, (uint32_t)K) + dig;
                eq &= same_digit(dig, __builtin_amdgcn_sicmp(t, hi, 40 /* < */) &
                                          __builtin_amdgcn_sicmp(t, l - 1, 39 /* >= */));
                const int slot = p.fl_off[l] + gk;
                if (q && v && firstl[slot] < t) {
                    Lq = l;
                    const uint64_t pm = eq & below;
                    if (pm) {
                        Eq = c0 + 63 - __clzll((long long)pm);
                        miss = false;
                    } else {
                        Eq = tab[slot];
                        miss = Eq < 0;
                    }
                }
                if (v && !(eq & above))
                    tab[slot] = t;
            }
            if (q) {
                if (miss)
                    pend[atomicAdd(&misc[25], 1)] = (PendT)t;
                else
                    put(t, Lq > 0 ? Eq : -1, Lq, kq);
            }
        }
    }
    __syncthreads();
    const int npend = misc[25];
    for (int i = tid; i < npend; i += nt) {
        const int t = (int)pend[i];
        int Lq = 0, gq = 0, gk = 0;
        for (int l = 1; l < d && l <= t + 1; ++l) {
            gk = gk * K + x[t - l + 1];
            if (firstl[p.fl_off[l] + gk] < t) {
                Lq = l;
                gq = gk;
            }
        }
        int e = -1;
        for (int w = t / Ts - 1; w >= 0 && e < 0; --w)
            e = segtab[w * FL + p.fl_off[Lq] + gq];
        put(t, e, Lq, t >= d - 1 ? dgram_key(x, t, d, K) : 0);
    }
    __syncthreads();
}

// Puts every selected bucket's positions in time order, one bucket per
// thread (insertion sort in place).  The scatter that filled the buckets
// appends in nearly increasing time, so each insertion moves an element a
// few places at most.  `list` + off[k] - base holds bucket k's positions.
template <class Ptr, class OffT, class Sel>
__device__ void sort_buckets(Ptr list, const OffT *off, int NB, int base,
                             Sel selected)
{
    for (int k = threadIdx.x; k < NB; k += blockDim.x) {
        if (!selected(k))
            continue;
        const int b0 = (int)off[k] - base, c = (int)off[k + 1] - (int)off[k];
        for (int i = 1; i < c; ++i) {
            const auto v = list[b0 + i];
            int j = i - 1;
            while (j >= 0) {
                const auto u = list[b0 + j];
                if (u <= v)
                    break;
                list[b0 + j + 1] = u;
                --j;
            }
            list[b0 + j + 1] = v;
        }
    }
}

// One task: `n` positions of consecutive buckets read from `src` (SORT:
// put each bucket in time order here; otherwise the buckets come sorted).
// Bucket boundaries are where the d-gram key changes; a group is the lane
// range of one bucket, so inside a group lane order is time order.  Returns solve_wave's answer for the lane (not ok for
// the first member of each bucket: its answer has L < d) and the lane's
// position in t_out.
template <int DC, bool SORT, bool CAP, class Src>
__device__ Found run_task(const MatchParams &p, const uint8_t *x, Src src,
                          int n, int &t_out, int &key_out, uint4 *drec = nullptr,
                          uint64_t *eqw = nullptr)
{
    const int lane = __lane_id();
    const uint64_t self = 1ull << lane;
    const bool has = lane < n;
    const int t0 = has ? src(lane) : 0;
    const int d = DC > 0 ? DC : p.d;
    const int k0 = has ? dgram_key(x, t0, d, p.K) : -1;
    key_out = k0;   // the lane's bucket (sorting stays inside buckets)
    const int kprev = __shfl_up(k0, 1);
    // bucket starts: lane 0 and key changes, among the task's lanes (compares
    // straight to lane masks)
    const uint64_t B = __builtin_amdgcn_sicmp(lane, n, 40 /* < */) &
                       (1ull | __builtin_amdgcn_sicmp(kprev, k0, 33 /* != */));
    const uint64_t upto = (self << 1) - 1;   // lanes 0..lane (lane 63: all)
    const uint64_t nxt = B & ~upto;          // bucket starts above this lane
    const int ss = 63 - __clzll((long long)(B & upto | 1ull));
    const int se = nxt ? __ffsll((long long)nxt) - 1 : n;   // exclusive
    const uint64_t hi = se >= 64 ? ~0ull : ((1ull << se) - 1);
    const uint64_t g = has ? (hi & ~((1ull << ss) - 1)) : self;
    // time order inside each bucket: odd-even transposition over the wave
    // on (bucket, t); buckets are already in lane order, so no element
    // crosses a bucket boundary.  The scatter leaves each bucket nearly in
    // time order, so the sort usually stops after a few rounds (64 rounds
    // always suffice).
    if (!SORT) {
        t_out = t0;
        return solve_wave<CAP>(x, p.nbits, t0, g, d, has, drec, eqw);
    }
    uint32_t key = has ? (((uint32_t)__popcll(B & upto) << 16) | (uint32_t)t0)
                       : 0xFFFFFFFFu;
    for (int r = 0; r < 64; r += 2) {
        uint64_t swapped = 0;   // lanes whose key changed (direct compares)
#pragma unroll
        for (int par = 0; par < 2; ++par) {
            // wave_shl:1 / wave_shr:1: the keys of lanes i+1 and i-1
            const uint32_t nx = (uint32_t)__builtin_amdgcn_update_dpp(
                (int)0xFFFFFFFF, (int)key, 0x130, 0xF, 0xF, false);
            const uint32_t pv = (uint32_t)__builtin_amdgcn_update_dpp(
                0, (int)key, 0x138, 0xF, 0xF, false);
            const bool left = (lane & 1) == par;
            const uint32_t nk = left ? min(key, nx) : max(key, pv);
            swapped |= ballot(nk != key);
            key = nk;
        }
        if (swapped == 0)
            break;
    }
    const int t1 = has ? (int)(key & 0xFFFFu) : 0;
    t_out = t1;
    return solve_wave<CAP>(x, p.nbits, t1, g, d, has, drec, eqw);
}

// ------------------------------------------------------- large buckets
//
struct GroupRef {
    int start, n, ell, buf;
};

// Every LDS access below is made by one wave, whose LDS operations are
// performed in issue order; the wave barriers only keep the compiler from
// moving accesses across them.
__device__ __forceinline__ void wave_sync() { __builtin_amdgcn_wave_barrier(); }

// One wave solves the bucket of stream s with d-gram key `key`, n0 > 64
// members from bucket slot `start` on (x: the stream's padded symbol row;
// bcnt, bbase, bbase0: the wave's own LDS arrays of at least K + 2 ints).
//
// DEFER (record mode): a group of more than 64 members whose members all
// agree on the next kBigDeferLevels symbols (one pass comparing each
// member's window of that many symbols with the last member's) -- constant
// or periodic stretches, where refining level by level would cost O(T)
// levels of O(n) work -- is not refined further.  Its members other than
// the first are deferred to the time-ordered pass of unpermute_kernel, like
// the long repeats of solve_wave's CAP mode: each gets a placeholder
// record, its bit in the deferred bitmap and a record pointing at the
// group's position list (slot a, n members, buffer), which holds every
// earlier position sharing its reversed level-gram, so the list is
// complete for the fallback of the extension rule there.  (A group that
// is uniform for fewer levels, e.g. a periodic stream with a disturbance,
// is refined level by level: the fallback would compare with every member
// once per period.)
constexpr int kBigDeferLevels = 8;

// Whether the n members (positions X[0 .. n), in time order) of a group at
// level ell agree for the next kBigDeferLevels (= 8) levels: member t's
// symbols x[t-ell-7 .. t-ell] against the last member's (the longest
// history), one 8-byte window per member, 1024 members per round (16 position loads
// of a lane in flight: the check is bound by their latency).  Symbols
// before position 0 do not exist: a member compares only the symbols of its
// own history, as a level step treats a member whose history has ended as
// agreeing (such members are the group's first ones, which the level steps
// would drop one by one).  Every member has t >= ell - 1, so the window
// reads stay inside the row's zero padding.
__device__ bool big_group_uniform(const int32_t *X, int n, const uint8_t *x, int ell)
{
    static_assert(kBigDeferLevels == 8, "one 8-symbol window per member");
    const int lane = __lane_id();
    const uint64_t ref = load8_end(x, X[n - 1] - ell);
    for (int i0 = 0; i0 < n; i0 += 64 * 16) {
        int tt[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int i = i0 + 64 * u + lane;
            tt[u] = i < n ? X[i] : -1;
        }
        bool bad = false;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int v = tt[u] - ell + 1;   // symbols of the member's history in the window
            if (tt[u] >= 0 && v > 0) {
                const uint64_t m = v >= 8 ? ~0ull : ~0ull << (8 * (8 - v));
                bad = bad || ((load8_end(x, tt[u] - ell) ^ ref) & m) != 0;
            }
        }
        if (ballot(bad))
            return false;
    }
    return true;
}

template <bool DEFER>
__device__ void solve_big_bucket(const MatchParams &p, const uint8_t *x, int s,
                                 int key, int start, int n0, int32_t *bcnt,
                                 int32_t *bbase, int32_t *bbase0)
{
    const int K = p.K;
    const int lane = __lane_id();
    const uint64_t self = 1ull << lane;
    const uint64_t below = self - 1;
    const int T = p.T, d = p.d;
    int32_t *buf0 = p.pos + (int64_t)s * T;
    int32_t *buf1 = p.pos2 + (int64_t)s * T;
    StreamOut o;
    o.x = x;
    o.E = p.E ? p.E + (int64_t)s * T : nullptr;
    o.SYM = p.SYM ? p.SYM + (int64_t)s * T : nullptr;
    o.L = p.L ? p.L + (int64_t)s * T : nullptr;
    o.rec = p.rec ? p.rec + (int64_t)s * T : nullptr;
    int4 *stk = p.stack + (int64_t)s * (T / 16 + 4) + start / 16;
    const int stack_cap = n0 / 16;
    int nrec = 0;   // records written so far (uniform)
    // emits the answers of the lanes with `want`, compacting record slots
    auto put = [&](bool want, int t, int e, int l) {
        if (o.rec) {
            const uint64_t m = ballot(want);
            if (want)
                emit_record(o, start + 1 + nrec + __popcll(m & below), t, e, l);
            nrec += __popcll(m);
        } else if (want) {
            emit(o, t, e, l);
        }
    };

    // the bucket's positions in time order, 256 per round (the four key
    // reads of a lane issued together)
    {
        int w = 0;
        for (int t0 = d - 1; t0 < T; t0 += 256) {
            bool m[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = t0 + 64 * u + lane;
                m[u] = t < T && dgram_key(x, t, d, K) == key;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint64_t bm = ballot(m[u]);
                if (m[u])
                    buf0[start + w + __popcll(bm & below)] = t0 + 64 * u + lane;
                w += __popcll(bm);
            }
        }
    }
    int sp = 0;
    GroupRef cur = {start, n0, d, 0};
    // after a failed window check, the next one waits kBigDeferLevels
    // levels (groups that split at every few levels pay it once per 8)
    int next_wcheck = 0;
    bool have = true;
    while (have) {
        const int32_t *X = cur.buf ? buf1 : buf0;
        int32_t *Y = cur.buf ? buf0 : buf1;
        bool defer_now = false;
        if (DEFER && cur.n > 64 && cur.ell >= next_wcheck) {
            defer_now = big_group_uniform(X + cur.start, cur.n, x, cur.ell);
            if (!defer_now)
                next_wcheck = cur.ell + kBigDeferLevels;
        }
        if (cur.n <= 64) {
            const bool hs = lane < cur.n;
            const int t = hs ? X[cur.start + lane] : 0;
            const uint64_t g = cur.n >= 64 ? ~0ull : ((1ull << cur.n) - 1);
            const Found f = solve_wave<false>(x, p.nbits, t, hs ? g : self, cur.ell, hs);
            put(hs && f.ok, t, f.e, f.l);
        } else if (defer_now) {
            // members 1 .. n-1 deferred (see above): whatever answers the
            // level steps would give the first members as they drop, the
            // group's list holds every candidate of every member
            const int ga = cur.start, gn = cur.n;
            uint32_t *deepbits = p.deep + (int64_t)s * deep_words(T);
            uint4 *dinfo = p.dinfo + (int64_t)s * T;
            const uint32_t lb = (uint32_t)min(cur.ell + kBigDeferLevels, 8191);
            const uint4 drec = make_uint4((uint32_t)ga,
                                          (uint32_t)gn | ((uint32_t)cur.buf << 31),
                                          0u, (lb << 3) << 16);
            // 512 members per round, a lane's eight position loads in flight
            for (int i0 = 1; i0 < gn; i0 += 64 * 8) {
                int tt[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int i = i0 + 64 * u + lane;
                    tt[u] = i < gn ? X[ga + i] : -1;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const bool hs = tt[u] >= 0;
                    const uint64_t m = ballot(hs);
                    const int t = tt[u];
                    if (hs) {
                        o.rec[start + 1 + nrec + __popcll(m & below)] = (uint32_t)t << 16;
                        dinfo[t] = drec;
                    }
                    nrec += __popcll(m);
                    // the bitmap bits, one atomic per word: members are in
                    // time order, so the lanes of one word are adjacent (the
                    // lanes without a member, at the end, each stand alone);
                    // a segmented OR gathers each word's bits in its first
                    // lane.  Per-lane atomics on one word are serialised at
                    // the cache and made this loop the most expensive part
                    // of a constant stream.
                    const int wd = hs ? (t >> 5) : -1 - lane;
                    uint32_t bits = hs ? 1u << (t & 31) : 0u;
#pragma unroll
                    for (int sh = 1; sh < 64; sh <<= 1) {
                        const uint32_t ob = (uint32_t)__shfl_down((int)bits, sh);
                        const int ow = __shfl_down(wd, sh);
                        if (lane + sh < 64 && ow == wd)
                            bits |= ob;
                    }
                    const int pw = __shfl_up(wd, 1);
                    if (hs && (lane == 0 || pw != wd))
                        atomicOr(&deepbits[wd], bits);
                }
            }
        } else {
            const int a = cur.start, n = cur.n, ell = cur.ell;
            // uniform level?  reference symbol from the last member
            const int tl = X[a + n - 1];
            const int dref = x[tl - ell];
            // 256 members per round, a lane's four loads in flight together
            bool uni = true;
            for (int i0 = 0; i0 < n; i0 += 256) {
                int tt[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = i0 + 64 * u + lane;
                    tt[u] = i < n ? X[a + i] : -1;
                }
                bool bad = false;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    bad = bad || (tt[u] - ell >= 0 && x[tt[u] - ell] != dref);
                if (ballot(bad)) {
                    uni = false;
                    break;
                }
            }
            if (uni) {
                const int t0 = X[a];
                if (t0 - ell < 0) {
                    // the first member's history ends: the next member
                    // loses its only predecessor at this level
                    put(lane == 0, X[a + 1], t0, ell);
                    cur.start = a + 1;
                    cur.n = n - 1;
                }
                cur.ell = ell + 1;
                if (cur.n >= 2)
                    continue;
            } else {
                // stable partition by x[t-ell] into Y[a .. a+n)
                for (int q = lane; q <= K; q += 64)
                    bcnt[q] = 0;
                wave_sync();
                for (int i0 = 0; i0 < n; i0 += 64) {
                    const int i = i0 + lane;
                    if (i < n) {
                        const int t = X[a + i];
                        const int dg = (t - ell >= 0) ? x[t - ell] : K;
                        atomicAdd(&bcnt[dg], 1);
                    }
                }
                wave_sync();
                if (lane == 0) {
                    int acc = 0;
                    for (int q = 0; q <= K; ++q) {
                        bbase[q] = acc;
                        bbase0[q] = acc;
                        acc += bcnt[q];
                    }
                }
                wave_sync();
                for (int i0 = 0; i0 < n; i0 += 64) {
                    const int i = i0 + lane;
                    const bool hs = i < n;
                    const int t = hs ? X[a + i] : 0;
                    const int dg = hs ? ((t - ell >= 0) ? x[t - ell] : K) : K + 1;
                    uint64_t eq = ballot(hs);
                    for (int b = 0; b < 9; ++b) {
                        const bool bit = (dg >> b) & 1;
                        const uint64_t Bb = ballot(hs && bit);
                        eq &= bit ? Bb : ~Bb;
                    }
                    const int rank = __popcll(eq & below);
                    int dest = 0;
                    if (hs)
                        dest = bbase[dg] + rank;
                    wave_sync();
                    if (hs && !(eq & ~(below | self)))   // last of its class
                        bbase[dg] = dest + 1;
                    wave_sync();
                    const bool moved = hs && dg < K;
                    if (moved)
                        Y[a + dest] = t;
                    const bool fin = moved && dest == bbase0[dg] && i > 0;
                    put(fin, t, fin ? X[a + i - 1] : 0, ell);
                }
                wave_sync();
                // children: small ones solved now, large ones stacked;
                // continue with the smallest large child
                int best = -1, bestn = 0x7FFFFFFF;
                for (int q = 0; q < K; ++q) {
                    const int c = bcnt[q];
                    if (c < 2)
                        continue;
                    const int cs = a + bbase0[q];
                    if (c <= 64) {
                        const bool hs = lane < c;
                        const int t = hs ? Y[cs + lane] : 0;
                        const uint64_t g = c >= 64 ? ~0ull : ((1ull << c) - 1);
                        const Found f = solve_wave<false>(x, p.nbits, t, hs ? g : self,
                                                          ell + 1, hs);
                        put(hs && f.ok, t, f.e, f.l);
                    } else if (c < bestn) {
                        if (best >= 0 && sp < stack_cap && lane == 0)
                            stk[sp] = make_int4(a + bbase0[best], bcnt[best],
                                                ell + 1, cur.buf ^ 1);
                        if (best >= 0 && sp < stack_cap)
                            ++sp;
                        best = q;
                        bestn = c;
                    } else if (sp < stack_cap) {
                        if (lane == 0)
                            stk[sp] = make_int4(cs, c, ell + 1, cur.buf ^ 1);
                        ++sp;
                    }
                }
                if (best >= 0) {
                    cur = GroupRef{a + bbase0[best], bcnt[best], ell + 1,
                                   cur.buf ^ 1};
                    continue;
                }
            }
        }
        if (sp > 0) {
            // the stack entry was written by lane 0 in an earlier iteration;
            // global stores and loads of one wave to the same address are
            // ordered once the store has completed
            __builtin_amdgcn_s_waitcnt(0);
            wave_sync();
            const int4 e = stk[--sp];
            cur = GroupRef{e.x, e.y, e.z, e.w};
        } else {
            have = false;
        }
    }
}

template <bool Vec, bool Nib>
__device__ void unpermute_stream(const MatchParams &p, int s, uint16_t *tau,
                                 uint8_t *nib, const uint8_t *x);

// The stream a workgroup of the stream kernel takes.  Workgroup i runs on
// XCD i % 8; with S a multiple of 128, the 16 consecutive streams of a
// route group (the routes whose channels share a 128-byte line of a hidden
// row) go to workgroups of one XCD, so when they read their symbols from
// the rows themselves each line is fetched into one L2.
__device__ __forceinline__ int stream_of_block(int b, int S)
{
    if (S % 128 != 0)
        return b;
    const int x = b & 7, j = b >> 3;
    return ((j >> 4) * 8 + x) * 16 + (j & 15);
}

// ------------------------------------------------- stream kernel (LDS)
//
// Streams of up to 65536 positions: one workgroup per stream with the
// padded symbol row, 16-bit bucket offsets, the answers of the buckets'
// first members and a union reused across phases in LDS (plan below).
// The task list lives in the workspace (written once in phase B, read once
// per task).  Phase E runs in passes over ranges of bucket slots that fit
// the position buffer: each pass scatters the range's positions into LDS
// (LDS atomics on the cursors), then the waves solve the range's tasks
// from LDS, each task putting its buckets in time order first.  All
// results are staged as records, written by whole tasks so that the stores
// are coalesced, and put into time order by unpermute_kernel.
// LDS plan for streams of up to TMAX positions and THREADS threads per
// workgroup (all sizes in bytes; B buckets, F first-occurrence entries):
//   A-B  cnt [0, 4B) | firstd [4B, 8B) | firstl [8B, 8B+4F)
//   D    pending u16 [0, 4B) | firstd | firstl | segment tables [8B+4F, U)
//   E    cursors [0, 2B+16) | pass id [2B+16, 3B+32) | positions u16
// d-gram buckets: K^d <= max(min(4096, T/8), K), so B = that bound for
// TMAX (K <= 256); first-occurrence tables: sum_{l<d} K^l < K^d, or at
// most 11 entries when K = 1.
template <int TMAX, int THREADS, int UNION, int MINBLOCKS = 1>
struct LdsCfg {
    static constexpr int kThreads = THREADS;
    static constexpr int kMinBlocks = MINBLOCKS;   // workgroups per CU
    static constexpr int kTMax = TMAX;
    static constexpr int kSymBytes = (TMAX + kPadFront + kPadBack + 255) / 256 * 256;
    static constexpr int kBuckets =
        TMAX / 8 >= kMaxBuckets ? kMaxBuckets : (TMAX / 8 > 256 ? TMAX / 8 : 256);
    static constexpr int kFirst = (kBuckets < kMaxFirstTab ? kBuckets : kMaxFirstTab) + 16;
    static constexpr int kUnion = UNION;
    static constexpr int kUFirstd = 4 * kBuckets;
    static constexpr int kUFirstl = 8 * kBuckets;
    static constexpr int kUSegTab = 8 * kBuckets + 4 * kFirst;
    static constexpr int kSegTab = (kUnion - kUSegTab) / 4;
    static constexpr int kUPassId = 2 * kBuckets + 16;
    static constexpr int kULpos = 3 * kBuckets + 32;
    static constexpr int kLposCap = (kUnion - kULpos) / 2;
    static constexpr int kPassCap = kLposCap - 64;
    static_assert(kSegTab > 0 && kLposCap > 64, "LDS plan");
    // the workgroup's LDS, one buffer: padded symbol row | bucket offsets
    // u16 [B+16] | first members' answers u16 [B] | misc int [32] | symbol
    // split words u64 [waves][16] | union (every part 16-byte aligned)
    static constexpr int kOffOff = kSymBytes;
    static constexpr int kOffQres = kOffOff + (kBuckets + 16) * 2;
    static constexpr int kOffMisc = kOffQres + kBuckets * 2;
    static constexpr int kOffEq = kOffMisc + 128;
    static constexpr int kOffU = kOffEq + (THREADS / 64) * 16 * 8;
    static constexpr int kLdsBytes = kOffU + kUnion;
    static_assert(kOffOff % 16 == 0 && kOffQres % 16 == 0 && kOffU % 16 == 0,
                  "LDS plan alignment");
    static_assert(kLdsBytes <= 163840, "LDS plan size");
    // after the tasks the whole buffer can hold the time-ordered pass of a
    // stream of TMAX positions over at most 16 symbols: the symbols as
    // nibbles [TMAX/2] and the u16 destinations [TMAX]
    static constexpr bool kNibPass = TMAX / 2 + 2 * TMAX <= kLdsBytes;
};

// Streams of up to 65536 positions, one 1024-thread workgroup per CU (the
// whole LDS: two scatter passes for a 65536-position stream).
using CfgLarge = LdsCfg<65536, 1024,
                        163840 - 65792 - (kMaxBuckets + 16) * 2 - kMaxBuckets * 2 - 128 -
                            16 * 16 * 8>;
// Streams of up to 8192 positions: 42 KiB per 512-thread workgroup; two
// workgroups per CU run 512 streams in one round, with the register budget
// of four waves per SIMD (the large-bucket and time-ordered passes at the
// end of the kernel need it).
using CfgSmall = LdsCfg<8192, 512, 28672, 2>;

// DC: the bucketing depth d as a compile-time constant (1..4), or 0 to read
// it from p.
template <class Cfg, int DC>
__global__ __launch_bounds__(Cfg::kThreads)
__attribute__((amdgpu_waves_per_eu(Cfg::kThreads / 256 * Cfg::kMinBlocks)))
void stream_kernel_lds(MatchParams p)
{
    constexpr int kPassCap = Cfg::kPassCap;
    __shared__ __align__(16) unsigned char lds[Cfg::kLdsBytes];
    unsigned char *symrow = lds;
    // bucket offsets fit 16 bits: off[NB] = T - d + 1 <= 65535
    uint16_t *off = reinterpret_cast<uint16_t *>(lds + Cfg::kOffOff);
    // E+1 of each bucket's first member (L < d, from phase D), written
    // with the bucket's task so all record stores stay coalesced
    uint16_t *qres = reinterpret_cast<uint16_t *>(lds + Cfg::kOffQres);
    int32_t *misc = reinterpret_cast<int32_t *>(lds + Cfg::kOffMisc);
    // per wave: 16 words for the symbol splits of alphabets of at most 16
    // symbols (wave_symbol_mask)
    uint64_t(*eqtab)[16] = reinterpret_cast<uint64_t(*)[16]>(lds + Cfg::kOffEq);
    unsigned char *U = lds + Cfg::kOffU;
    int32_t *cnt = reinterpret_cast<int32_t *>(U);
    int32_t *firstd = reinterpret_cast<int32_t *>(U + Cfg::kUFirstd);
    int32_t *firstl = reinterpret_cast<int32_t *>(U + Cfg::kUFirstl);
    uint16_t *pend = reinterpret_cast<uint16_t *>(U);
    int32_t *segtab = reinterpret_cast<int32_t *>(U + Cfg::kUSegTab);
    // bucket k's cursor is half k & 1 of word k >> 1 (slot relative to the
    // pass, < 65536, so an increment never carries into the other half)
    uint32_t *cur2 = reinterpret_cast<uint32_t *>(U);
    uint8_t *passid = U + Cfg::kUPassId;
    uint16_t *lpos = reinterpret_cast<uint16_t *>(U + Cfg::kULpos);
    const int s = stream_of_block(blockIdx.x, gridDim.x);
    uint32_t *tasks = p.tasks + (int64_t)s * kTaskCap;
    // positions whose answers are deferred (long repeats): one bit each,
    // and their candidates
    uint32_t *deepbits = p.deep + (int64_t)s * deep_words(p.T);
    uint4 *dinfo = p.dinfo + (int64_t)s * p.T;
    int32_t *posrow = p.pos + (int64_t)s * p.T;

    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63, wid = tid >> 6, nw = nt >> 6;
    const int T = p.T, K = p.K, d = DC > 0 ? DC : p.d, NB = p.NB;
    uint64_t *eqw = p.nbits <= 4 ? eqtab[wid] : nullptr;
    if (p.stage == 1) {
        // the padding, then the symbols straight from the bf16 rows: route
        // r packs channels 4r .. 4r+3 (one 8-byte load per position), bit j
        // = I[h > 0] of channel 4r+j (Sec. 3.2, Eq. (10)-(15)); eight loads
        // of a thread in flight at once
        if (s == 0 && tid < 64)
            p.flags[tid] = 0;
        for (int i = tid; i < kPadFront; i += nt)
            symrow[i] = 0;
        for (int i = kPadFront + T + tid; i < Cfg::kSymBytes; i += nt)
            symrow[i] = 0;
        const int64_t b = s / p.R, r = s % p.R;
        const uint16_t *h = p.H + b * (int64_t)T * p.Hld + r * 4;
        for (int t0 = tid; t0 < T; t0 += 8 * nt) {
            uint2 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + u * nt;
                v[u] = t < T ? *reinterpret_cast<const uint2 *>(h + (int64_t)t * p.Hld)
                             : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = t0 + u * nt;
                if (t < T) {
                    const uint8_t c = (uint8_t)(bf16_is_pos(v[u].x & 0xFFFFu) |
                                                (bf16_is_pos(v[u].x >> 16) << 1) |
                                                (bf16_is_pos(v[u].y & 0xFFFFu) << 2) |
                                                (bf16_is_pos(v[u].y >> 16) << 3));
                    symrow[kPadFront + t] = c;
                    if (p.sym_copy)
                        p.sym_copy[(int64_t)s * T + t] = c;
                }
            }
        }
    } else if (p.stage == 2) {
        // the caller's row (16-byte aligned), 16 symbols per thread and
        // step, with the zero padding around it; symbols >= K are clamped
        // (as the copy into the workspace rows does) and reported in the
        // stream's status slot (no launch clears a flag before this one).
        // The padded row also goes to the workspace for the later kernel
        // that reads it, unless this kernel runs the time-ordered pass
        // itself.
        const uint8_t *src = p.symin + (int64_t)s * p.symld;
        uint4 *dst = reinterpret_cast<uint4 *>(symrow);
        uint4 *wdst = p.fuse == 1 ? nullptr
                                  : reinterpret_cast<uint4 *>(p.sym_w + (int64_t)s * p.Tp);
        const bool pow2 = (K & (K - 1)) == 0;
        const uint32_t hm = (uint32_t)(~(K - 1) & 0xFF) * 0x01010101u;
        int anybad = 0;
        for (int i = tid; i < (int)(p.Tp >> 4); i += nt) {
            const int t0 = 16 * i - kPadFront;
            uint4 v;
            if (t0 >= 0 && t0 + 16 <= T) {
                v = *reinterpret_cast<const uint4 *>(src + t0);
            } else {
                uint32_t wv[4] = {0u, 0u, 0u, 0u};
                for (int q = 0; q < 16; ++q)
                    if (t0 + q >= 0 && t0 + q < T)
                        wv[q >> 2] |= (uint32_t)src[t0 + q] << (8 * (q & 3));
                v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            }
            bool bad;
            if (pow2) {
                bad = ((v.x | v.y | v.z | v.w) & hm) != 0;
            } else {
                bad = false;
                const uint32_t wq[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    bad |= ((wq[q >> 2] >> (8 * (q & 3))) & 0xFFu) >= (uint32_t)K;
            }
            if (bad) {
                anybad = 1;
                uint8_t *b = reinterpret_cast<uint8_t *>(&v);
                for (int q = 0; q < 16; ++q)
                    if (b[q] >= K)
                        b[q] = (uint8_t)(K - 1);
            }
            dst[i] = v;
            if (wdst)
                wdst[i] = v;
        }
        // OR over the workgroup through the per-wave split words (unused
        // until the tasks, which clear them before use)
        const uint64_t wb = ballot(anybad != 0);
        if (lane == 0)
            eqtab[wid][0] = wb;
        __syncthreads();
        if (tid == 0) {
            for (int w = 0; w < nw; ++w)
                anybad |= eqtab[w][0] != 0 ? 1 : 0;
            p.sflag[s] = anybad;
            if (s == 0) {
                p.flags[kFlagSymbol] = 0;
                p.flags[kFlagSlots] = (int32_t)gridDim.x;   // one workgroup per stream
                p.flags[kFlagSlotMark] = kSlotMark;
            }
        }
    } else {
        const uint4 *src = reinterpret_cast<const uint4 *>(p.sym + (int64_t)s * p.Tp);
        uint4 *dst = reinterpret_cast<uint4 *>(symrow);
        for (int i = tid; i < (int)(p.Tp >> 4); i += nt)
            dst[i] = src[i];
    }
    if (tid < 32)
        misc[tid] = 0;
    for (int i = tid; i < deep_words(T); i += nt)
        deepbits[i] = 0;
    const uint8_t *x = symrow + kPadFront;
    StreamOut o;
    o.x = x;
    o.E = nullptr;
    o.SYM = nullptr;
    o.L = p.L ? p.L + (int64_t)s * T : nullptr;
    o.rec = p.rec + (int64_t)s * T;

    phase_hist<DC>(p, x, cnt, firstd, firstl);
    phase_tasks(p, s, cnt, off, tasks, misc, kPassCap, true, Cfg::kTMax <= 8192 ? 96 : 256);

    // D: records of the first d-1 positions go to the slots T-d+1.. (no
    // bucket holds them); the first occurrence of a d-gram in a singleton
    // or large bucket takes the bucket's first slot; for buckets of 2..64
    // members the answer waits in qres until the bucket's task writes it.
    phase_short<DC>(p, x, firstd, firstl, segtab, Cfg::kSegTab, pend, misc,
                [&](int t, int e, int l, int k) {
                    if (t < d - 1) {
                        emit_record(o, T - d + 1 + t, t, e, l);
                        return;
                    }
                    const int c = (int)off[k + 1] - (int)off[k];
                    if (c == 1 || c > 64) {
                        emit_record(o, off[k], t, e, l);
                    } else {
                        qres[k] = (uint16_t)(e + 1);
                        if (o.L)
                            o.L[t] = l;
                    }
                }, eqw);

    // E: passes over slot ranges.  passid[k] is the pass that scatters
    // bucket k (255: not scattered, a singleton or large bucket).
    for (int i = tid; i < NB; i += nt) {
        const int c = (int)off[i + 1] - (int)off[i];
        passid[i] = (c >= 2 && c <= 64) ? (uint8_t)((int)off[i] / kPassCap) : (uint8_t)255;
    }
    const int nslots = (int)off[NB];
    int tfirst = 0;
    __syncthreads();
    for (int base = 0; base < nslots; base += kPassCap) {
        const int rg = base / kPassCap;
        if (tid == 0)
            misc[kMiscNext] = tfirst + nw;
        for (int i = tid; i < (NB + 1) / 2; i += nt) {
            const int k0 = 2 * i, k1 = 2 * i + 1;
            const uint32_t c0 = passid[k0] == rg ? (uint32_t)((int)off[k0] - base) : 0u;
            const uint32_t c1 = (k1 < NB && passid[k1] == rg) ? (uint32_t)((int)off[k1] - base) : 0u;
            cur2[i] = c0 | (c1 << 16);
        }
        __syncthreads();
        // four positions per thread per iteration, independent chains
        for (int t0 = d - 1 + 4 * tid; t0 < T; t0 += 4 * nt) {
            int kk[4];
            bool in[4];
            // one 8-symbol read covers the four d-grams when d <= 4
            const uint64_t v8 = d <= 4 ? load8_end(x, t0 + 3) : 0ull;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int t = t0 + u;
                kk[u] = t >= T ? 0
                        : d <= 4 ? key_of_word((uint32_t)(v8 >> (8 * (u + 1))), d, K)
                                 : dgram_key(x, t, d, K);
                in[u] = t < T && passid[kk[u]] == rg;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (in[u]) {
                    const uint32_t sh = 16u * (uint32_t)(kk[u] & 1);
                    const uint32_t old = atomicAdd(&cur2[kk[u] >> 1], 1u << sh);
                    lpos[(old >> sh) & 0xFFFFu] = (uint16_t)(t0 + u);
                }
        }
        __syncthreads();
        // this range's tasks: [tlo, thi).  Wave w starts with task tlo + w,
        // then takes the next one from a counter (tasks inside long
        // recurrences cost many times the others); the next task's
        // descriptor is loaded while this one is solved.  A task's records
        // are stored at the start of the wave's next task, after the load of
        // the descriptor after it.  (Loads and stores complete under one
        // counter, so the wait for a descriptor also covers the stores
        // issued before it.  Loading descriptors two ahead, or by scalar
        // loads, which wait on the LDS counter instead, measured the same,
        // also with the gather and the discretisation running beside.)
        const int tlo = tfirst, thi = tfirst + misc[kMiscPass + rg];
        tfirst = thi;
        int ti = tlo + wid;
        uint32_t tk_next = ti < thi ? __builtin_nontemporal_load(&tasks[ti]) : 0u;
        Found pf = {-1, 0, false, false};   // the previous task's answers
        int pt = 0, pk = 0, pstart = 0, pn = 0;
        auto store_prev = [&]() {
            if (ballot(pf.deep)) {
                // answers deferred to the time-ordered pass (unpermute_kernel),
                // their records written by solve_wave; with more candidates
                // than a record holds, the task's positions go to the
                // workspace and the record points there
                const bool ovf = pf.deep && pf.e != 0;
                if (ballot(ovf) && lane < pn)
                    posrow[pstart + lane] = pt;
                if (ovf) {
                    dinfo[pt].x = (uint32_t)pstart;
                    dinfo[pt].y = (uint32_t)pn;
                }
                if (lane < pn && pf.deep) {
                    o.rec[pstart + lane] = (uint32_t)pt << 16;
                    atomicOr(&deepbits[pt >> 5], 1u << (pt & 31));
                } else if (lane < pn && pf.ok) {
                    emit_record(o, pstart + lane, pt, pf.e, pf.l);
                } else if (lane < pn) {
                    o.rec[pstart + lane] = ((uint32_t)pt << 16) | (uint32_t)qres[pk];
                }
            } else if (lane < pn) {
                if (pf.ok)
                    emit_record(o, pstart + lane, pt, pf.e, pf.l);
                else   // a bucket's first member: its answer from phase D
                    o.rec[pstart + lane] = ((uint32_t)pt << 16) | (uint32_t)qres[pk];
            }
        };
        while (ti < thi) {
            const uint32_t tk = __builtin_amdgcn_readfirstlane(tk_next);
            const int start = (int)(tk >> 6);
            const int n = (int)(tk & 63u) + 1;
            int tn = 0;
            if (lane == 0)
                tn = atomicAdd(&misc[kMiscNext], 1);
            tn = __builtin_amdgcn_readfirstlane(tn);
            if (tn < thi)
                tk_next = __builtin_nontemporal_load(&tasks[tn]);
            store_prev();
            int t, k;
            pf = run_task<DC, true, true>(
                p, x, [&](int i) { return (int)lpos[start - base + i]; }, n, t, k,
                dinfo, eqw);
            pt = t;
            pk = k;
            pstart = start;
            pn = n;
            ti = tn;
        }
        store_prev();
        __syncthreads();
    }
    // buckets of more than 64 members (low-entropy streams), listed by
    // phase B: one wave each, with its partition counters in the union
    const int nbig = misc[kMiscBig];
    if (nbig > 0) {
        constexpr int kBigInts = 3 * 264;
        const int nbw = min(nw, Cfg::kUnion / (kBigInts * 4));
        if (wid < nbw) {
            int32_t *bl = reinterpret_cast<int32_t *>(U) + wid * kBigInts;
            const int32_t *list = big_own(p, s);
            for (int i = wid; i < nbig; i += nbw) {
                const int32_t *ent = list + 4 * (int64_t)i;
                solve_big_bucket<true>(p, x, s, ent[1], ent[2], ent[3], bl, bl + 264,
                                       bl + 528);
                wave_sync();
            }
        }
    }
    // streams whose u16 destinations fit the union (fuse, set by the
    // launcher): the time-ordered pass here, on this workgroup's records
    // (still in cache) and its LDS copy of the symbols, instead of a launch
    // of unpermute_kernel
    if (p.fuse == 1) {
        // the records were stored by this workgroup's waves; the barrier
        // (a workgroup-scope fence) makes them visible to all of them
        __syncthreads();
        uint16_t *tau = reinterpret_cast<uint16_t *>(U);
        const bool vec = (T & 3) == 0 && ((uintptr_t)p.E & 15) == 0 &&
                         ((uintptr_t)p.SYM & 7) == 0;
        if (vec)
            unpermute_stream<true, false>(p, s, tau, nullptr, x);
        else
            unpermute_stream<false, false>(p, s, tau, nullptr, x);
    }
    if constexpr (Cfg::kNibPass && Cfg::kTMax > 8192) {
        // longer streams over at most 16 symbols (fuse = 2, set by the
        // launcher when the outputs allow 16-byte stores): once every wave
        // is done with it, the whole LDS holds the time-ordered pass -- the
        // symbols as nibbles, read back from the padded workspace row, then
        // the u16 destinations -- as in a launch of unpermute_kernel, but
        // with each workgroup's tail overlapping the other workgroups' tasks
        if (p.fuse == 2) {
            __syncthreads();
            uint16_t *tau = reinterpret_cast<uint16_t *>(lds + Cfg::kTMax / 2);
            unpermute_stream<true, true>(p, s, tau, lds,
                                         p.sym + (int64_t)s * p.Tp + kPadFront);
        }
    }
}

// ---------------------------------------------- stream kernel (HBM rows)
//
// Streams of more than 65536 positions: the same phases with symbols and
// bucket positions in HBM and results written directly.
constexpr int kArenaBytes = 90368;

__global__ __launch_bounds__(kStreamThreads) void stream_kernel_hbm(MatchParams p)
{
    __shared__ __align__(16) unsigned char arena[kArenaBytes];
    int32_t *cnt = reinterpret_cast<int32_t *>(arena);
    int32_t *off = reinterpret_cast<int32_t *>(arena + 16384);
    int32_t *segtab = reinterpret_cast<int32_t *>(arena);
    int32_t *firstd = reinterpret_cast<int32_t *>(arena + 32832);
    int32_t *firstl = reinterpret_cast<int32_t *>(arena + 49216);
    int32_t *pend = reinterpret_cast<int32_t *>(arena + 57408);
    uint32_t *tasks = reinterpret_cast<uint32_t *>(arena + 73856);
    int32_t *misc = reinterpret_cast<int32_t *>(arena + 90240);

    const int s = blockIdx.x;
    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63, wid = tid >> 6, nw = nt >> 6;
    const int T = p.T, K = p.K, d = p.d;
    const uint8_t *x = p.sym + (int64_t)s * p.Tp + kPadFront;
    int32_t *pos = p.pos + (int64_t)s * T;
    if (tid < 32)
        misc[tid] = 0;
    StreamOut o;
    o.x = x;
    o.E = p.E + (int64_t)s * T;
    o.SYM = p.SYM ? p.SYM + (int64_t)s * T : nullptr;
    o.L = p.L ? p.L + (int64_t)s * T : nullptr;
    o.rec = nullptr;

    phase_hist<0>(p, x, cnt, firstd, firstl);
    phase_tasks(p, s, cnt, off, tasks, misc, 0x7FFFFFFF);
    for (int i = tid; i < p.NB; i += nt)
        cnt[i] = off[i];   // cursors
    __syncthreads();
    // scatter positions of buckets with 2..64 members
    for (int t = d - 1 + tid; t < T; t += nt) {
        const int k = dgram_key(x, t, d, K);
        const int c = off[k + 1] - off[k];
        if (c >= 2 && c <= 64)
            pos[atomicAdd(&cnt[k], 1)] = t;
    }
    __syncthreads();
    sort_buckets(pos, off, p.NB, 0, [&](int k) {
        const int c = off[k + 1] - off[k];
        return c >= 2 && c <= 64;
    });
    __syncthreads();
    phase_short<0>(p, x, firstd, firstl, segtab, kSegTabInts, pend, misc,
                [&](int t, int e, int l, int) { emit(o, t, e, l); });
    const int ntasks = misc[24];
    for (int ti = wid; ti < ntasks; ti += nw) {
        const uint32_t tk = tasks[ti];
        const int start = (int)(tk >> 6);
        const int n = (int)(tk & 63u) + 1;
        int t, k;
        const Found f = run_task<0, false, false>(p, x, [&](int i) { return pos[start + i]; }, n, t, k);
        if (lane < n && f.ok)
            emit(o, t, f.e, f.l);
    }
}

// ------------------------------------------------------------- big kernel
//
// Streams of more than 65536 positions (direct mode): one wave per bucket
// with more than 64 members, from the global list.  Stack entries
// {start, n, level, buffer} describe groups (contiguous, time-ordered,
// sharing the level-gram).  Only groups of more than 64 members are
// stacked (smaller ones are solved at once) and stacked groups are
// disjoint, so a bucket of n members never has more than n/65 entries; the
// bucket starting at offset `start` of its stream keeps its stack in the
// stream's stack region from entry start/16 on (n/16 >= n/65 + 2 entries
// for n >= 65, and ranges of different buckets do not overlap).  A level
// where every member has the same next symbol only drops the first member
// if its history ends (t = level-1).  In record mode (streams of at most
// 65536 positions, solved by the stream kernel itself) the bucket's members
// other than the first (answered in slot `start`) fill slots start+1 ..
// start+n-1 in completion order.
__global__ __launch_bounds__(kBigThreads) void big_kernel(MatchParams p)
{
    __shared__ int32_t bcnt[264];     // K+1 counts (digit K = drop)
    __shared__ int32_t bbase[264];    // running bases
    __shared__ int32_t bbase0[264];   // initial bases
    const int count = min((int64_t)p.big[0], p.big_cap);
    for (int item = blockIdx.x; item < count; item += gridDim.x) {
        const int32_t *ent = p.big + 64 + 4 * (int64_t)item;
        const int s = ent[0], key = ent[1], start = ent[2], n0 = ent[3];
        const uint8_t *x = p.sym + (int64_t)s * p.Tp + kPadFront;
        solve_big_bucket<false>(p, x, s, key, start, n0, bcnt, bbase, bbase0);
        wave_sync();
    }
}

// ------------------------------------------------------ unpermute kernel
//
// Record mode: one workgroup per stream.  The stream's records are read
// once (coalesced) and scattered into tau[t] = E+1 in LDS (u16 for all of
// the up to 65536 positions, 128 KiB); then E and SYM = x[E+1] are written
// in time order with coalesced stores, the symbol read from the stream's
// padded row (64 KiB per stream, served from cache).  Vec: T % 4 == 0 and
// 16-byte aligned E / 8-byte aligned SYM rows, four positions per thread.
// Nib (alphabets of at most 16 symbols, with Vec): the row is first staged
// in the rest of the LDS as 4-bit symbols (32 KiB), so the SYM reads are
// LDS reads instead of scattered byte loads.
// TMAX: the longest stream the LDS arrays hold (65536, or 8192 for short
// streams, whose workgroups then share a CU).
// The time-ordered pass of stream s, by one workgroup: `tau` holds T u16
// in LDS, `nib` (Nib) T/2 bytes of LDS for the 4-bit copy of the symbols,
// `x` the stream's padded symbol row (device memory, or the stream
// kernel's LDS copy when it runs this pass itself).
template <bool Vec, bool Nib>
__device__ void unpermute_stream(const MatchParams &p, int s, uint16_t *tau,
                                 uint8_t *nib, const uint8_t *x)
{
    const int tid = threadIdx.x, nt = blockDim.x;
    const int T = p.T;
    const uint32_t *rec = p.rec + (int64_t)s * T;
    int32_t *E = p.E + (int64_t)s * T;
    int16_t *SYM = p.SYM ? p.SYM + (int64_t)s * T : nullptr;
    // every record names a position t < T <= 65536 (16-bit field), so the
    // scatter stays inside tau; tau <= T-1 for every record, the clamp
    // below only keeps the symbol read inside the row
    if (Vec) {
        // four 16-byte loads in flight per thread before the LDS scatter
        const uint4 *r4 = reinterpret_cast<const uint4 *>(rec);
        const int n4 = T >> 2;
        for (int i0 = tid; i0 < n4; i0 += 4 * nt) {
            uint4 r[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (i0 + u * nt < n4)
                    r[u] = r4[i0 + u * nt];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (i0 + u * nt < n4) {
                    tau[r[u].x >> 16] = (uint16_t)r[u].x;
                    tau[r[u].y >> 16] = (uint16_t)r[u].y;
                    tau[r[u].z >> 16] = (uint16_t)r[u].z;
                    tau[r[u].w >> 16] = (uint16_t)r[u].w;
                }
        }
    } else {
        for (int i = tid; i < T; i += nt) {
            const uint32_t r = rec[i];
            tau[r >> 16] = (uint16_t)r;
        }
    }
    if (Nib) {
        // 16 symbols -> 8 bytes per thread-step (low nibble = even position)
        const uint4 *x4 = reinterpret_cast<const uint4 *>(x);
        uint2 *n8 = reinterpret_cast<uint2 *>(nib);
        for (int i = tid; i < (T + 15) / 16; i += nt) {
            const uint4 v = x4[i];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t a = w[2 * h], b = w[2 * h + 1];
                const uint32_t pa = (a & 0xFu) | ((a >> 4) & 0xF0u) |
                                    ((a >> 8) & 0xF00u) | ((a >> 12) & 0xF000u);
                const uint32_t pb = (b & 0xFu) | ((b >> 4) & 0xF0u) |
                                    ((b >> 8) & 0xF00u) | ((b >> 12) & 0xF000u);
                o[h] = pa | (pb << 16);
            }
            n8[i] = make_uint2(o[0], o[1]);
        }
    }
    __syncthreads();
    // Deferred positions (inside long repeats, solve_wave's CAP mode): each
    // run of consecutive ones is answered in time order by one wave.  When
    // x[E(t-1)+1] = x[t], the longest earlier suffix grows by one and its
    // latest occurrence moves by one: L(t) = L(t-1)+1, E(t) = E(t-1)+1 (an
    // occurrence of the longer suffix ending at e makes e-1 an occurrence of
    // the shorter one, so e <= E(t-1)+1).  The wave checks this along the
    // run 64 positions at a time; where it fails, the answer is the maximum
    // of (common suffix length, e) over the members the position's task
    // recorded, each length found 64 symbols at a time.
    {
        const int W = deep_words(T);
        const uint32_t *db = p.deep + (int64_t)s * W;
        const uint4 *dinfo = p.dinfo + (int64_t)s * T;
        int32_t *Lrow = p.L ? p.L + (int64_t)s * T : nullptr;
        const int lane = tid & 63, wid = tid >> 6, nw = nt >> 6;
        auto sym = [&](int i) -> int {
            return Nib ? (int)(nib[i >> 1] >> (4 * (i & 1))) & 0xF : (int)x[i];
        };
        // common suffix length of x[0..t] and x[0..e] (e < t), at least c
        auto lcs_wave = [&](int t, int e, int c) -> int {
            for (;;) {
                const int pi = c + lane;
                const bool eq = pi <= e && sym(t - pi) == sym(e - pi);
                const uint64_t em = ballot(eq);
                if (em != ~0ull)
                    return c + __ffsll((long long)~em) - 1;
                c += 64;
            }
        };
        // the same for one lane: eight symbols per step from the 4-bit copy
        auto lcs_from = [&](int t, int e, int c) -> int {
            if (Nib) {
                const uint32_t *n32 = reinterpret_cast<const uint32_t *>(nib);
                // symbols pe-7..pe, pe in the top nibble (pe >= 7; the second
                // word is read only when the window straddles two)
                auto win8 = [&](int pe) -> uint32_t {
                    const int q = pe - 7, wi = q >> 3, sh = 4 * (q & 7);
                    const uint32_t lo = n32[wi];
                    const uint32_t hi = sh ? n32[wi + 1] : 0u;
                    return __builtin_amdgcn_alignbit(hi, lo, (uint32_t)sh);
                };
                while (e - c >= 7) {
                    const uint32_t df = win8(t - c) ^ win8(e - c);
                    if (df)
                        return c + (__clz((int)df) >> 2);
                    c += 8;
                }
            }
            while (c <= e && sym(t - c) == sym(e - c))
                ++c;
            return c;
        };
        auto run = [&](int t) {
            // the run's end: the first position after t whose bit is clear
            int tend = T;
            for (int wb = t >> 5;; wb += 64) {
                const int wi = wb + lane;
                uint32_t m = wi < W ? db[wi] : 0u;
                if (wi == (t >> 5))
                    m |= (1u << (t & 31)) - 1;   // bits before t count as set
                const uint64_t zm = ballot(m != ~0u);
                if (zm) {
                    const int l = __ffsll((long long)zm) - 1;
                    const uint32_t ml = (uint32_t)__shfl((int)m, l);
                    tend = min(T, (wb + l) * 32 + __ffs((int)~ml) - 1);
                    break;
                }
                if (wb + 64 >= W)
                    break;
            }
            int e1 = tau[t - 1];                 // final: t-1 is not deferred
            int L = Lrow ? Lrow[t - 1] : 0;
            while (t < tend) {
                const int ti = t + lane;
                const bool ok = ti < tend && sym(e1 + lane) == sym(ti);
                const uint64_t okm = ballot(ok);
                const int k = okm == ~0ull ? 64 : __ffsll((long long)~okm) - 1;
                if (lane < k) {
                    tau[ti] = (uint16_t)(e1 + lane + 1);
                    if (Lrow)
                        Lrow[ti] = L + lane + 1;
                }
                t += k;
                e1 += k;
                L += k;
                if (k == 64 || t >= tend)
                    continue;
                const uint4 in = dinfo[t];
                const int nc = (int)((in.w >> 16) & 7u);
                const int lb = (int)(in.w >> 19);
                int bc = -1, be = -1;
                for (int j = 0; j < nc; ++j) {
                    const uint32_t wj = j < 2 ? in.x : j < 4 ? in.y : j < 6 ? in.z : in.w;
                    const int e = (int)((wj >> (16 * (j & 1))) & 0xFFFFu);
                    const int c = lcs_wave(t, e, min(lb, e + 1));
                    if (c > bc || (c == bc && e > be)) {
                        bc = c;
                        be = e;
                    }
                }
                if (nc == 0) {
                    // more candidates than a record holds: a list of positions
                    // (in.x: first slot, in.y: size, top bit: the second
                    // buffer) that holds every earlier position that can be
                    // the answer -- the position's task (at most 64), or its
                    // group of a large bucket; every earlier one is compared
                    // in full, one per lane
                    const int nl = (int)(in.y & 0x7FFFFFFFu);
                    const int32_t *tp = (in.y >> 31 ? p.pos2 : p.pos) + (int64_t)s * T + in.x;
                    for (int i0 = 0; i0 < nl; i0 += 64) {
                        const int e = i0 + lane < nl ? tp[i0 + lane] : T;
                        if (e < t) {
                            const int c = lcs_from(t, e, 0);
                            if (c > bc || (c == bc && e > be)) {
                                bc = c;
                                be = e;
                            }
                        }
                    }
                    // the lexicographic maximum of (c, e) over the lanes
                    for (int o = 32; o >= 1; o >>= 1) {
                        const int oc = __shfl_xor(bc, o), oe = __shfl_xor(be, o);
                        if (oc > bc || (oc == bc && oe > be)) {
                            bc = oc;
                            be = oe;
                        }
                    }
                }
                if (lane == 0) {
                    tau[t] = (uint16_t)(be + 1);
                    if (Lrow)
                        Lrow[t] = bc;
                }
                e1 = be + 1;   // E(t) + 1 for the next position
                L = bc;
                ++t;
            }
        };
        // wave w takes the runs that start in its share of the bitmap
        const int per = (W + nw - 1) / nw;
        const int w0 = wid * per, w1 = min(W, w0 + per);
        for (int wb = w0; wb < w1; wb += 64) {
            const int wi = wb + lane;
            uint32_t st = 0;
            if (wi < w1) {
                const uint32_t m = db[wi];
                const uint32_t before = wi > 0 ? db[wi - 1] >> 31 : 0u;
                st = m & ~((m << 1) | before);
            }
            uint64_t has = ballot(st != 0);
            while (has) {
                const int l = __ffsll((long long)has) - 1;
                has &= has - 1;
                uint32_t sw = (uint32_t)__shfl((int)st, l);
                while (sw) {
                    const int bit = __ffs((int)sw) - 1;
                    sw &= sw - 1;
                    run((wb + l) * 32 + bit);
                }
            }
        }
    }
    __syncthreads();
    if (Vec) {
        const uint2 *t4 = reinterpret_cast<const uint2 *>(tau);
        int4 *E4 = reinterpret_cast<int4 *>(E);
        uint2 *S4 = reinterpret_cast<uint2 *>(SYM);
        // two groups of four positions per thread: eight symbol reads in
        // flight
        const int n4 = T >> 2;
        for (int i0 = tid; i0 < n4; i0 += 2 * nt) {
            uint32_t sv[2][4];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int i = i0 + u * nt;
                if (i < n4) {
                    const uint2 w = t4[i];
                    const int a = (int)(w.x & 0xFFFFu), b = (int)(w.x >> 16);
                    const int c = (int)(w.y & 0xFFFFu), d = (int)(w.y >> 16);
                    E4[i] = make_int4(a - 1, b - 1, c - 1, d - 1);
                    if (SYM && Nib) {
                        const int v4[4] = {a, b, c, d};
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int e = min(v4[q], T - 1);
                            sv[u][q] = v4[q] ? (uint32_t)(nib[e >> 1] >> (4 * (e & 1))) & 0xFu
                                             : 0xFFFFu;
                        }
                    } else if (SYM) {
                        sv[u][0] = a ? x[min(a, T - 1)] : 0xFFFFu;
                        sv[u][1] = b ? x[min(b, T - 1)] : 0xFFFFu;
                        sv[u][2] = c ? x[min(c, T - 1)] : 0xFFFFu;
                        sv[u][3] = d ? x[min(d, T - 1)] : 0xFFFFu;
                    }
                }
            }
            if (SYM) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int i = i0 + u * nt;
                    if (i < n4)
                        S4[i] = make_uint2(sv[u][0] | (sv[u][1] << 16),
                                           sv[u][2] | (sv[u][3] << 16));
                }
            }
        }
    } else {
        for (int t = tid; t < T; t += nt) {
            const int e1 = tau[t];
            E[t] = e1 - 1;
            if (SYM)
                SYM[t] = e1 ? (int16_t)x[min(e1, T - 1)] : (int16_t)-1;
        }
    }
}

template <bool Vec, bool Nib, int TMAX>
__global__ __launch_bounds__(kStreamThreads) void unpermute_kernel(MatchParams p)
{
    __shared__ __align__(16) uint16_t tau[TMAX];
    __shared__ __align__(16) uint8_t nib[Nib ? TMAX / 2 : 16];
    const int s = blockIdx.x;
    unpermute_stream<Vec, Nib>(p, s, tau, nib, p.sym + (int64_t)s * p.Tp + kPadFront);
}

// --------------------------------------------------------------- launchers

bool stream_uses_records(int64_t T) { return T <= 65536; }

// Whether the stream kernel runs the time-ordered pass itself: its u16
// destinations must fit the union of the LDS plan that takes the stream.
bool stream_fuses_unpermute(int64_t T)
{
    if (!stream_uses_records(T))
        return false;
    const int64_t uni = T <= CfgSmall::kTMax ? CfgSmall::kUnion : CfgLarge::kUnion;
    return 2 * T <= uni;
}

// Whether the stream kernel runs the time-ordered pass itself over its whole
// LDS (streams of the large plan too long for the union, at most 16
// symbols, outputs that take 16-byte stores).
bool stream_nib_pass(const MatchParams &p)
{
    return stream_uses_records(p.T) && !stream_fuses_unpermute(p.T) &&
           p.T > CfgSmall::kTMax && CfgLarge::kNibPass && p.K <= 16 &&
           (p.T & 3) == 0 && ((uintptr_t)p.E & 15) == 0 &&
           ((uintptr_t)p.SYM & 7) == 0;
}

// Whether the stream kernel can read bf16 symbols itself (stage): streams
// of the small LDS plan, which also runs the time-ordered pass itself (no
// later kernel reads the padded symbol rows).
bool stream_can_stage(int64_t T)
{
    return T <= CfgSmall::kTMax && stream_fuses_unpermute(T);
}

hipError_t launch_stream(const MatchParams &p_in, int64_t S, hipStream_t st)
{
    MatchParams p = p_in;
    p.fuse = stream_fuses_unpermute(p.T) ? 1 : stream_nib_pass(p) ? 2 : 0;
    if (stream_uses_records(p.T)) {
        const bool small = p.T <= CfgSmall::kTMax;
        const dim3 grid((unsigned)S);
#define ROSA_LAUNCH_LDS(D)                                                          \
    do {                                                                            \
        if (small)                                                                  \
            hipLaunchKernelGGL((stream_kernel_lds<CfgSmall, D>), grid,              \
                               dim3(CfgSmall::kThreads), 0, st, p);                 \
        else                                                                        \
            hipLaunchKernelGGL((stream_kernel_lds<CfgLarge, D>), grid,              \
                               dim3(CfgLarge::kThreads), 0, st, p);                 \
    } while (0)
        switch (p.d) {
        case 1: ROSA_LAUNCH_LDS(1); break;
        case 2: ROSA_LAUNCH_LDS(2); break;
        case 3: ROSA_LAUNCH_LDS(3); break;
        case 4: ROSA_LAUNCH_LDS(4); break;
        default: ROSA_LAUNCH_LDS(0); break;
        }
#undef ROSA_LAUNCH_LDS
    } else
        hipLaunchKernelGGL(stream_kernel_hbm, dim3((unsigned)S),
                           dim3(kStreamThreads), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_big(const MatchParams &p, int grid, hipStream_t st)
{
    // streams of up to 65536 positions: the stream kernel solved its own
    if (stream_uses_records(p.T))
        return hipSuccess;
    hipLaunchKernelGGL(big_kernel, dim3((unsigned)grid), dim3(kBigThreads), 0,
                       st, p);
    return hipGetLastError();
}

hipError_t launch_unpermute(const MatchParams &p, int64_t S, hipStream_t st)
{
    if (!stream_uses_records(p.T) || stream_fuses_unpermute(p.T) || stream_nib_pass(p))
        return hipSuccess;
    const bool vec = (p.T & 3) == 0 && ((uintptr_t)p.E & 15) == 0 &&
                     ((uintptr_t)p.SYM & 7) == 0;
    const dim3 grid((unsigned)S), block(kStreamThreads);
#define ROSA_LAUNCH_UNPERMUTE(TM)                                                   \
    do {                                                                            \
        if (vec && p.K <= 16)                                                       \
            hipLaunchKernelGGL((unpermute_kernel<true, true, TM>), grid, block, 0,  \
                               st, p);                                              \
        else if (vec)                                                               \
            hipLaunchKernelGGL((unpermute_kernel<true, false, TM>), grid, block, 0, \
                               st, p);                                              \
        else                                                                        \
            hipLaunchKernelGGL((unpermute_kernel<false, false, TM>), grid, block,   \
                               0, st, p);                                           \
    } while (0)
    if (p.T <= 8192)
        ROSA_LAUNCH_UNPERMUTE(8192);
    else
        ROSA_LAUNCH_UNPERMUTE(65536);
#undef ROSA_LAUNCH_UNPERMUTE
    return hipGetLastError();
}

}  // namespace rosa
