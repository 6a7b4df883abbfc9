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
//     C  positions scattered into buckets (LDS atomics);
//     D  positions whose d-gram is new (L < d) and the first d-1 positions
//        are answered from the first-occurrence tables plus a time-ordered
//        scan per segment (ballot match inside 64-position chunks, LDS
//        last-end tables across chunks and segments);
//     E  each wave takes tasks: sorts the task's positions by time
//        (bitonic over the 64 lanes), then refines groups with lane masks
//        (solve_wave).
//   big_kernel (one wave per bucket of more than 64 positions): rebuilds the
//     bucket in time order, then refines it with stable partitions by the
//     next symbol until groups fit a wave, then solve_wave.
#include "rosa_internal.h"

namespace rosa {

constexpr uint32_t kFirstFlag = 0x80000000u;
constexpr int kWordThresh = 4;

// ----------------------------------------------------------- wave helpers

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ int wave_max(int v)
{
    for (int o = 32; o > 0; o >>= 1)
        v = max(v, __shfl_xor(v, o));
    return v;
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

struct StreamOut {
    const uint8_t *x;  // padded symbol row of the stream
    int32_t *E;
    int16_t *SYM;
    int32_t *L;
};

__device__ __forceinline__ void emit(const StreamOut &o, int t, int e, int l)
{
    o.E[t] = e;
    if (o.L)
        o.L[t] = l;
    if (o.SYM)
        o.SYM[t] = e >= 0 ? (int16_t)o.x[e + 1] : (int16_t)-1;
}

// ------------------------------------------------------------ solve_wave
//
// Each lane holds one element t (or none).  g is the lane mask of its group:
// all members share the reversed `ell`-gram ending at their position, lanes
// of a group are contiguous and in increasing time order, and every member
// except the first already has L >= ell.  Refines until every group is a
// singleton, emitting (L, E) for each element when it leaves its last
// group with an earlier member.
//
// Two step kinds, chosen per iteration for the whole wave:
//  level step (large groups): split by the symbol x[t-ell]; an element that
//    is first in its new group but was not first before gets L = ell and
//    E = its previous group member.
//  word step (groups of <= kWordThresh): compare the next 16 symbols with
//    every group member at once; the common run c with the latest earlier
//    member that maximises it gives L = ell + c (c < 16); members equal on
//    all 16 symbols stay grouped at level ell + 16.
__device__ void solve_wave(const StreamOut &o, int nbits, int t, uint64_t g,
                           int ell, bool has)
{
    const int lane = __lane_id();
    const uint64_t self = 1ull << lane;
    const uint64_t below = self - 1;
    if (!has)
        g = self;
    uint64_t lo = 0, hi = 0;
    int wl = -(1 << 30);
    for (;;) {
        const bool live = has && __popcll(g) >= 2;
        if (ballot(live) == 0)
            break;
        const int gmax = wave_max(live ? __popcll(g) : 0);
        if (gmax > kWordThresh) {
            // ---------------------------------------------- level step
            if (ell - wl >= 16) {
                if (live && t - ell >= 0)
                    load_window(o.x, t - ell - 15, lo, hi);
                wl = ell;
            }
            const int bi = 15 - (ell - wl);
            const uint32_t dig =
                (uint32_t)((bi >= 8 ? (hi >> (8 * (bi - 8))) : (lo >> (8 * bi))) &
                           0xFFu);
            const bool valid = live && (t - ell >= 0);
            uint64_t eq = ballot(valid);
            for (int b = 0; b < nbits; ++b) {
                const bool bit = (dig >> b) & 1u;
                const uint64_t B = ballot(valid && bit);
                eq &= bit ? B : ~B;
            }
            const uint64_t ng = valid ? (g & eq) : self;
            const uint64_t prev = g & below;
            const int p = prev ? 63 - __clzll((long long)prev) : lane;
            const int e_prev = __shfl(t, p);
            if (live && prev && !(ng & below))
                emit(o, t, e_prev, ell);
            if (live)
                g = ng;
            ++ell;
        } else {
            // ----------------------------------------------- word step
            const bool valid = live && (t - ell >= 0);
            if (valid)
                load_window(o.x, t - ell - 15, lo, hi);
            wl = ell;
            const int avail = valid ? (t - ell + 1) : 0;
            int best_c = -1, best_e = -1;
            uint64_t gnew = self;
            uint64_t rem = valid ? g : 0;
            while (ballot(rem != 0)) {
                const bool have = rem != 0;
                const int j = have ? __ffsll((long long)rem) - 1 : lane;
                rem &= rem - 1;
                const uint64_t lo_j = shfl64(lo, j);
                const uint64_t hi_j = shfl64(hi, j);
                const int t_j = __shfl(t, j);
                const int a_j = __shfl(avail, j);
                if (have && j != lane) {
                    const uint64_t xh = hi ^ hi_j, xl = lo ^ lo_j;
                    const int c = xh ? (__clzll((long long)xh) >> 3)
                                     : (xl ? 8 + (__clzll((long long)xl) >> 3) : 16);
                    if (j < lane) {
                        const int cc = min(c, a_j);
                        if (cc >= best_c) {
                            best_c = cc;
                            best_e = t_j;
                        }
                    }
                    if (c == 16 && avail >= 16 && a_j >= 16)
                        gnew |= 1ull << j;
                }
            }
            if (valid && best_c >= 0 && best_c < 16)
                emit(o, t, best_e, ell + best_c);
            if (live)
                g = avail >= 16 ? gnew : self;
            ell += 16;
        }
    }
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

// ---------------------------------------------------------- stream kernel
//
// LDS: the stream's padded symbol row (when T <= 65536; otherwise symbols
// are read from the workspace row in HBM), plus an arena reused across
// phases (byte offsets):
//   [0, 32832)       A-C: cnt[4096] + off[4112]     D: segment tables
//   [32832, 49216)   A-D: firstd[4096]
//   [49216, 57408)   A-D: firstl[2048]
//   [57408, 73856)   D:   pending queries[4112]
//   [73856, 90240)   B-E: tasks[4096]
//   [90240, 90368)   misc
constexpr int kArenaBytes = 90368;
constexpr int kSegTabInts = 8192;
constexpr int kSymLds = 65792;     // padded row bytes for T <= 65536

// Key of the reversed d-gram ending at t (t >= d-1): x[t] is the most
// significant digit.  Its top l digits form the key of the l-gram.
__device__ __forceinline__ int dgram_key(const uint8_t *x, int t, int d, int K)
{
    int k = 0;
    for (int i = 0; i < d; ++i)
        k = k * K + x[t - i];
    return k;
}

template <bool kLds>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(MatchParams p)
{
    __shared__ __align__(16) unsigned char arena[kArenaBytes];
    __shared__ __align__(16) unsigned char symrow[kLds ? kSymLds : 16];
    int32_t *cnt = reinterpret_cast<int32_t *>(arena);
    int32_t *off = reinterpret_cast<int32_t *>(arena + 16384);
    int32_t *segtab = reinterpret_cast<int32_t *>(arena);
    int32_t *firstd = reinterpret_cast<int32_t *>(arena + 32832);
    int32_t *firstl = reinterpret_cast<int32_t *>(arena + 49216);
    int32_t *pend = reinterpret_cast<int32_t *>(arena + 57408);
    uint32_t *tasks = reinterpret_cast<uint32_t *>(arena + 73856);
    int32_t *misc = reinterpret_cast<int32_t *>(arena + 90240);

    const int s = blockIdx.x;
    const int tid = threadIdx.x;
    const int nt = blockDim.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int nw = nt >> 6;
    const uint64_t self = 1ull << lane;
    const uint64_t below = self - 1;
    const uint64_t above = ~(below | self);
    const int T = p.T, K = p.K, d = p.d, NB = p.NB, FL = p.fl_total;
    const uint8_t *xg = p.sym + (int64_t)s * p.Tp + kPadFront;
    int32_t *pos = p.pos + (int64_t)s * T;

    if (kLds) {
        const uint4 *src = reinterpret_cast<const uint4 *>(p.sym + (int64_t)s * p.Tp);
        uint4 *dst = reinterpret_cast<uint4 *>(symrow);
        for (int i = tid; i < (int)(p.Tp >> 4); i += nt)
            dst[i] = src[i];
    }
    const uint8_t *x = kLds ? symrow + kPadFront : xg;
    StreamOut o;
    o.x = x;
    o.E = p.E + (int64_t)s * T;
    o.SYM = p.SYM ? p.SYM + (int64_t)s * T : nullptr;
    o.L = p.L ? p.L + (int64_t)s * T : nullptr;

    // ---- A: histogram, first occurrences
    for (int i = tid; i < NB; i += nt) {
        cnt[i] = 0;
        firstd[i] = 0x7FFFFFFF;
    }
    for (int i = tid; i < FL; i += nt)
        firstl[i] = 0x7FFFFFFF;
    if (tid < 32)
        misc[tid] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += nt) {
        int k = 0;
        const int dm = min(d, t + 1);
        for (int i = 0; i < dm; ++i) {
            k = k * K + x[t - i];
            if (i + 1 < d) {
                int32_t *f = &firstl[p.fl_off[i + 1] + k];
                if (t < *f)
                    atomicMin(f, t);
            }
        }
        if (t >= d - 1) {
            atomicAdd(&cnt[k], 1);
            if (t < firstd[k])
                atomicMin(&firstd[k], t);
        }
    }
    __syncthreads();

    // ---- B: bucket offsets, task packing, large buckets
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
                off[b0 + q] = ex;
                ex += cnt[b0 + q];
            }
        if (tid == 0)
            off[NB] = total;
    }
    __syncthreads();
    if (wid == 0) {
        const int b0 = (int)((int64_t)lane * NB / 64);
        const int b1 = (int)((int64_t)(lane + 1) * NB / 64);
        int ntask = 0, cur = 0;
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
            if (cur + c > 64) {
                ++ntask;
                cur = 0;
            }
            cur += c;
        }
        if (cur)
            ++ntask;
        const int incl = wave_incl_scan(ntask);
        int k = incl - ntask;
        int start = 0;
        cur = 0;
        for (int b = b0; b < b1; ++b) {
            const int c = cnt[b];
            if (c == 0)
                continue;
            if (c == 1 || c > 64) {
                if (cur) {
                    tasks[k++] = ((uint32_t)start << 6) | (uint32_t)(cur - 1);
                    cur = 0;
                }
                if (c > 64) {
                    const int idx = atomicAdd(&p.big[0], 1);
                    if (idx < p.big_cap) {
                        int32_t *ent = p.big + 64 + 4 * (int64_t)idx;
                        ent[0] = s;
                        ent[1] = b;
                        ent[2] = off[b];
                        ent[3] = c;
                    }
                }
                continue;
            }
            if (cur + c > 64) {
                tasks[k++] = ((uint32_t)start << 6) | (uint32_t)(cur - 1);
                cur = 0;
            }
            if (cur == 0)
                start = off[b];
            cur += c;
        }
        if (cur)
            tasks[k++] = ((uint32_t)start << 6) | (uint32_t)(cur - 1);
        if (lane == 63)
            misc[24] = incl;
    }
    __syncthreads();
    for (int i = tid; i < NB; i += nt)
        cnt[i] = off[i];   // cursors
    __syncthreads();

    // ---- C: scatter positions of buckets with 2..64 members
    for (int t = tid; t < T; t += nt) {
        if (t < d - 1)
            continue;
        const int k = dgram_key(x, t, d, K);
        const int c = off[k + 1] - off[k];
        if (c >= 2 && c <= 64) {
            const int slot = atomicAdd(&cnt[k], 1);
            pos[slot] = t | (slot == off[k] ? (int)kFirstFlag : 0);
        }
    }
    __syncthreads();

    // ---- D: positions with L < d: the first d-1 positions and the first
    // occurrence of every d-gram.  L is the longest l < d whose l-gram
    // occurred before t (first-occurrence tables); E is the latest earlier
    // end of that l-gram.  Wave w scans time segment w in chunks of 64 in
    // order, keeping the last end of every l-gram seen so far in segment w
    // (segtab[w]); inside a chunk, the latest earlier lane with the same
    // l-gram comes from a ballot match.  Queries with no earlier end inside
    // their segment are resolved after the scan from the tables of earlier
    // segments.
    const int nseg = FL > 0 ? min(nw, kSegTabInts / FL) : nw;
    const int Ts = (((T + nseg - 1) / nseg) + 63) & ~63;
    for (int i = tid; i < nseg * FL; i += nt)
        segtab[i] = -1;
    __syncthreads();
    if (wid < nseg) {
        int32_t *tab = segtab + wid * FL;
        const int lo = wid * Ts, hi = min(T, lo + Ts);
        for (int c0 = lo; c0 < hi; c0 += 64) {
            const int t = c0 + lane;
            const bool inr = t < hi;
            const bool q = inr && (t < d - 1 || firstd[dgram_key(x, t, d, K)] == t);
            int Lq = 0, Eq = -1;
            bool miss = false;
            int gk = 0;
            uint64_t eq = ~0ull;
            for (int l = 1; l < d; ++l) {
                const bool v = inr && t >= l - 1;
                const int dig = v ? x[t - l + 1] : 0;
                gk = gk * K + dig;
                uint64_t m = ballot(v);
                for (int b = 0; b < p.nbits; ++b) {
                    const bool bit = (dig >> b) & 1;
                    const uint64_t B = ballot(v && bit);
                    m &= bit ? B : ~B;
                }
                eq &= m;
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
                    pend[atomicAdd(&misc[25], 1)] = t;
                else
                    emit(o, t, Lq > 0 ? Eq : -1, Lq);
            }
        }
    }
    __syncthreads();
    {
        const int npend = misc[25];
        for (int i = tid; i < npend; i += nt) {
            const int t = pend[i];
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
            emit(o, t, e, Lq);
        }
    }

    // ---- E: tasks of buckets with 2..64 members, one wave per task.  The
    // task's members are sorted by time across the whole wave (bitonic on
    // t<<6 | bucket); a group is the set of lanes with the same bucket
    // index, so lane order is time order inside every group.
    const int ntasks = misc[24];
    for (int ti = wid; ti < ntasks; ti += nw) {
        const uint32_t tk = tasks[ti];
        const int start = (int)(tk >> 6);
        const int n = (int)(tk & 63u) + 1;
        const bool has = lane < n;
        const uint32_t v = has ? (uint32_t)pos[start + lane] : 0u;
        const uint64_t F = ballot(has && (v & kFirstFlag));
        const uint64_t upto = (self << 1) - 1;   // lanes 0..lane (lane 63: all)
        const uint32_t seg = (uint32_t)__popcll(F & upto) - 1u;
        uint32_t key = has ? (((v & ~kFirstFlag) << 6) | seg) : 0xFFFFFFFFu;
        for (int kk = 2; kk <= 64; kk <<= 1)
            for (int j = kk >> 1; j > 0; j >>= 1) {
                const uint32_t other = (uint32_t)__shfl_xor((int)key, j);
                const bool up = (lane & kk) == 0;
                const bool lower = (lane & j) == 0;
                key = (lower == up) ? min(key, other) : max(key, other);
            }
        const int nbk = 64 - __clzll((long long)__popcll(F));   // bits for bucket ids
        const uint32_t sg = key & 63u;
        uint64_t g = ballot(has);
        for (int b = 0; b < nbk; ++b) {
            const bool bit = (sg >> b) & 1u;
            const uint64_t B = ballot(has && bit);
            g &= bit ? B : ~B;
        }
        if (!has)
            g = self;
        solve_wave(o, p.nbits, (int)(key >> 6), g, d, has);
    }
}

// ------------------------------------------------------------- big kernel
//
// One wave per bucket with more than 64 members.  Stack entries
// {start, n, level, buffer} describe groups (contiguous, time-ordered,
// sharing the level-gram).  Only groups of more than 64 members are
// stacked (smaller ones are solved at once) and stacked groups are disjoint,
// so a bucket of n members never has more than n/65 entries; the bucket
// starting at offset `start` of its stream keeps its stack in the stream's
// stack region from entry start/16 on (n/16 >= n/65 + 2 entries for
// n >= 65, and ranges of different buckets do not overlap).  A level where
// every member has the same next symbol only drops the first member if its
// history ends (t = level-1).

struct GroupRef {
    int start, n, ell, buf;
};

__global__ __launch_bounds__(kBigThreads) void big_kernel(MatchParams p)
{
    __shared__ int32_t bcnt[264];     // K+1 counts (digit K = drop)
    __shared__ int32_t bbase[264];    // running bases
    __shared__ int32_t bbase0[264];   // initial bases
    const int K = p.K;
    const int lane = threadIdx.x;
    const uint64_t self = 1ull << lane;
    const uint64_t below = self - 1;
    const int T = p.T, d = p.d;
    const int count = min((int64_t)p.big[0], p.big_cap);

    for (int item = blockIdx.x; item < count; item += gridDim.x) {
        const int32_t *ent = p.big + 64 + 4 * (int64_t)item;
        const int s = ent[0], key = ent[1], start = ent[2], n0 = ent[3];
        const uint8_t *x = p.sym + (int64_t)s * p.Tp + kPadFront;
        int32_t *buf[2] = {p.pos + (int64_t)s * T, p.pos2 + (int64_t)s * T};
        StreamOut o;
        o.x = x;
        o.E = p.E + (int64_t)s * T;
        o.SYM = p.SYM ? p.SYM + (int64_t)s * T : nullptr;
        o.L = p.L ? p.L + (int64_t)s * T : nullptr;
        int4 *stk = p.stack + (int64_t)s * (T / 16 + 4) + start / 16;
        const int stack_cap = n0 / 16;

        // the bucket's positions in time order
        {
            int w = 0;
            for (int t0 = d - 1; t0 < T; t0 += 64) {
                const int t = t0 + lane;
                const bool m = t < T && dgram_key(x, t, d, K) == key;
                const uint64_t bm = ballot(m);
                if (m)
                    buf[0][start + w + __popcll(bm & below)] = t;
                w += __popcll(bm);
            }
        }
        int sp = 0;
        GroupRef cur = {start, n0, d, 0};
        bool have = true;
        while (have) {
            if (cur.n <= 64) {
                const bool hs = lane < cur.n;
                const int t = hs ? buf[cur.buf][cur.start + lane] : 0;
                const uint64_t g = cur.n >= 64 ? ~0ull : ((1ull << cur.n) - 1);
                solve_wave(o, p.nbits, t, hs ? g : self, cur.ell, hs);
            } else {
                const int32_t *X = buf[cur.buf];
                int32_t *Y = buf[cur.buf ^ 1];
                const int a = cur.start, n = cur.n, ell = cur.ell;
                // uniform level?  reference symbol from the last member
                const int tl = X[a + n - 1];
                const int dref = x[tl - ell];
                bool uni = true;
                for (int i0 = 0; i0 < n; i0 += 64) {
                    const int i = i0 + lane;
                    bool bad = false;
                    if (i < n) {
                        const int t = X[a + i];
                        bad = (t - ell >= 0) && x[t - ell] != dref;
                    }
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
                        if (lane == 0)
                            emit(o, X[a + 1], t0, ell);
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
                    __syncthreads();
                    for (int i0 = 0; i0 < n; i0 += 64) {
                        const int i = i0 + lane;
                        if (i < n) {
                            const int t = X[a + i];
                            const int dg = (t - ell >= 0) ? x[t - ell] : K;
                            atomicAdd(&bcnt[dg], 1);
                        }
                    }
                    __syncthreads();
                    if (lane == 0) {
                        int acc = 0;
                        for (int q = 0; q <= K; ++q) {
                            bbase[q] = acc;
                            bbase0[q] = acc;
                            acc += bcnt[q];
                        }
                    }
                    __syncthreads();
                    for (int i0 = 0; i0 < n; i0 += 64) {
                        const int i = i0 + lane;
                        const bool hs = i < n;
                        const int t = hs ? X[a + i] : 0;
                        const int dg = hs ? ((t - ell >= 0) ? x[t - ell] : K) : K + 1;
                        uint64_t eq = ballot(hs);
                        for (int b = 0; b < 9; ++b) {
                            const bool bit = (dg >> b) & 1;
                            const uint64_t B = ballot(hs && bit);
                            eq &= bit ? B : ~B;
                        }
                        const int rank = __popcll(eq & below);
                        int dest = 0;
                        if (hs)
                            dest = bbase[dg] + rank;
                        __syncthreads();
                        if (hs && !(eq & ~(below | self)))   // last of its class
                            bbase[dg] = dest + 1;
                        __syncthreads();
                        if (hs && dg < K) {
                            Y[a + dest] = t;
                            if (dest == bbase0[dg] && i > 0)
                                emit(o, t, X[a + i - 1], ell);
                        }
                    }
                    __syncthreads();
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
                            solve_wave(o, p.nbits, t, hs ? g : self, ell + 1, hs);
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
                __syncthreads();
                const int4 e = stk[--sp];
                cur = GroupRef{e.x, e.y, e.z, e.w};
            } else {
                have = false;
            }
        }
    }
}

// --------------------------------------------------------------- launchers

hipError_t launch_stream(const MatchParams &p, int64_t S, hipStream_t st)
{
    if (p.Tp <= kSymLds)
        hipLaunchKernelGGL(stream_kernel<true>, dim3((unsigned)S),
                           dim3(kStreamThreads), 0, st, p);
    else
        hipLaunchKernelGGL(stream_kernel<false>, dim3((unsigned)S),
                           dim3(kStreamThreads), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_big(const MatchParams &p, int grid, hipStream_t st)
{
    hipLaunchKernelGGL(big_kernel, dim3((unsigned)grid), dim3(kBigThreads), 0,
                       st, p);
    return hipGetLastError();
}

}  // namespace rosa
