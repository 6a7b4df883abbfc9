// rosa_qk_batch.hip -- query/key retrieval for long streams: keys grouped by
// their last d symbols, one thread per query unit.
//
// Method: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix Matching"
// (arXiv 2602.02499), Sec. 3.3 with separate query and key streams and its
// run-length paragraph (key runs folded into units), App. C.5
// (counterfactual branches: the unit's query symbol with one bit flipped).
//
// For unit u and query symbol c (the unit's own, or a counterfactual one)
// the match length L is the largest l such that the query units
// u-l+1 .. u-1 followed by c equal the key units e-l+1 .. e for some
// e <= u-1, and E is the latest such e.  The automaton kernels reach the
// same by matching statistics (a suffix found among key units 0..u-1 lost
// its last symbol is found among units 0..u-2, so the growing automaton
// never misses a longer match).  Read backwards, L is the longest common
// prefix of (c, Q[u-1], Q[u-2], ...) and (C[e], C[e-1], ..., C[0]) over
// e < u, and E the latest e reaching it.
//
//   key groups: keys e >= d-1 sorted by their reversed d-gram
//     (C[e], ..., C[e-d+1]) with a counting sort (per-segment histograms,
//     offsets, scatter); an entry holds e and the next P symbols of its
//     history, C[e-d] .. C[e-d-P+1], packed into one word.
//   short tables: for l < d, the latest key up to the end of each 64-unit
//     chunk that ends each l-gram (per-chunk last keys, then prefix maxima
//     over the chunks).
//   queries: one thread per unit, for each query symbol in turn.  With an
//     earlier key in its group, L = d + the longest common extension over
//     those keys (packed words, then the rows), E the latest key reaching
//     it.  Otherwise L < d: for each l < d the latest earlier key ending the
//     same l-gram comes from the keys of the unit's own chunk (lane masks
//     from ballots of the key symbols) or from the short table of the chunk
//     before; L is the largest l with one.
//
// A query symbol whose key group holds more than kcap keys, or whose match
// runs more than kQtLcap units past d (low-entropy streams, long repeats),
// is left to a time-ordered pass per stream (qt_defer_kernel) that answers
// it by the extension rule from the previous unit's answer, else directly.
#include "rosa_internal.h"

namespace rosa {

namespace {

constexpr int kQtThreads = 1024;   // segment kernels: kQbtSeg units, 4 per thread
constexpr int kQtQThreads = 256;   // query kernel: 4 chunks of 64 units
constexpr int kQtLcap = 1024;      // extension past d followed before giving up

// Everything the kernels need besides QkParams: group depth, alphabet
// powers, short-table offsets, packing.
struct QtShape {
    int d, nb, fl, P, nbits, kcap;
    int rnb;                  // ceil(65536 / nbits): n / nbits = (n * rnb) >> 16 for n <= 32
    int64_t nseg, nch;
    int pw[kQbtMaxD + 1];     // K^l
    int floff[kQbtMaxD + 1];  // first short-table slot of level l (l >= 1)
};

__device__ __forceinline__ uint64_t qt_ballot(bool b)
{
    return __builtin_amdgcn_ballot_w64(b);
}

// Symbols row[p-7 .. p] as one word, row[p] in the top byte.  Rows are
// 4-byte aligned with kPadFront bytes in front, so p >= -54 stays inside.
__device__ __forceinline__ uint64_t qt_load8_end(const uint8_t *row, int p)
{
    const int a = p - 7;
    const uint32_t *q = reinterpret_cast<const uint32_t *>(row) + (a >> 2);
    const uint32_t sh = (uint32_t)(a & 3);
    const uint32_t d0 = q[0], d1 = q[1], d2 = q[2];
    return (uint64_t)__builtin_amdgcn_alignbyte(d1, d0, sh) |
           ((uint64_t)__builtin_amdgcn_alignbyte(d2, d1, sh) << 32);
}

// row[p], row[p-1], ..., row[p-P+1], each masked to nb bits, packed into
// one word with row[p] in the top bits (P * nb <= 32; p - P >= -40).
__device__ __forceinline__ uint32_t qt_pack(const uint8_t *row, int p, int nb, int P)
{
    const uint32_t m = (1u << nb) - 1u;
    uint32_t w = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (8 * k < P) {
            const uint64_t x = qt_load8_end(row, p - 8 * k);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = 8 * k + j;
                if (i < P)
                    w |= ((uint32_t)(x >> (56 - 8 * j)) & m) << (32 - nb * (i + 1));
            }
        }
    }
    return w;
}

// Exclusive scan over the workgroup of one int per thread (ws: 64 ints of
// LDS); *total receives the sum.
__device__ int qt_block_scan(int v, int *ws, int *total)
{
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nw = (int)(blockDim.x >> 6);
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o)
            x += y;
    }
    if (lane == 63)
        ws[wid] = x;
    __syncthreads();
    if (wid == 0) {
        int t = lane < nw ? ws[lane] : 0;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int y = __shfl_up(t, o);
            if (lane >= o)
                t += y;
        }
        if (lane < nw)
            ws[32 + lane] = t;
    }
    __syncthreads();
    const int before = wid > 0 ? ws[32 + wid - 1] : 0;
    *total = ws[32 + nw - 1];
    __syncthreads();
    return before + x - v;
}

// Key lanes whose digit kd equals my qd, among the lanes with vk set: the
// nb bits of the key digits by ballot, each compared with my bit.
__device__ __forceinline__ uint64_t qt_match(int kd, bool vk, int qd, int nb)
{
    uint64_t m = qt_ballot(vk);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        if (b < nb) {
            const uint64_t B = qt_ballot((kd >> b) & 1);
            m &= ((qd >> b) & 1) ? B : ~B;
        }
    }
    return m;
}

__device__ __forceinline__ int qt_units(const QkParams &p, int64_t s)
{
    return p.rle ? p.nunit[s] : (int)p.T;
}

__device__ __forceinline__ const uint8_t *qt_qrow(const QkParams &p, int64_t s)
{
    return (p.rle ? p.qu : p.q) + s * p.Tp + kPadFront;
}

__device__ __forceinline__ const uint8_t *qt_krow(const QkParams &p, int64_t s)
{
    return (p.rle ? p.ku : p.k) + s * p.Tp + kPadFront;
}

// ---------------------------------------------------------------- units
//
// With run folding, unit u is the u-th maximal run of equal key symbols;
// start[u] is its first time, and its query / key symbols are those at that
// time.  Segment g of kQbtSeg time steps per workgroup, four per thread.

__device__ __forceinline__ int qt_run_flags(const QkParams &p, int64_t s, int t0)
{
    if (t0 >= p.T)
        return 0;
    const uint8_t *kr = p.k + s * p.Tp + kPadFront;
    const uint64_t w = qt_load8_end(kr, t0 + 3);   // k[t0-4 .. t0+3], inside the row
    int f = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + i;
        const uint32_t cur = (uint32_t)(w >> (32 + 8 * i)) & 0xFFu;
        const uint32_t prv = (uint32_t)(w >> (24 + 8 * i)) & 0xFFu;
        if (t < p.T && (t == 0 || cur != prv))
            f |= 1 << i;
    }
    return f;
}

__global__ __launch_bounds__(kQtThreads) void qt_runs_count_kernel(QkParams p, QtShape sh)
{
    __shared__ int ws[64];
    const int64_t s = blockIdx.y;
    const int g = blockIdx.x;
    const int t0 = g * kQbtSeg + 4 * (int)threadIdx.x;
    const int f = qt_run_flags(p, s, t0);
    int tot;
    qt_block_scan(__popc(f), ws, &tot);
    if (threadIdx.x == 0)
        p.ucnt[s * sh.nseg + g] = tot;
}

__global__ __launch_bounds__(kQtThreads) void qt_runs_write_kernel(QkParams p, QtShape sh)
{
    __shared__ int ws[64];
    const int64_t s = blockIdx.y;
    const int g = blockIdx.x;
    int before = 0;
    for (int i = threadIdx.x; i < g; i += kQtThreads)
        before += p.ucnt[s * sh.nseg + i];
    int base;
    qt_block_scan(before, ws, &base);
    const int t0 = g * kQbtSeg + 4 * (int)threadIdx.x;
    const int f = qt_run_flags(p, s, t0);
    int tot;
    int u = base + qt_block_scan(__popc(f), ws, &tot);
    const uint8_t *qr = p.q + s * p.Tp + kPadFront;
    const uint8_t *kr = p.k + s * p.Tp + kPadFront;
    uint8_t *qu = p.qu + s * p.Tp + kPadFront;
    uint8_t *ku = p.ku + s * p.Tp + kPadFront;
    int32_t *st = p.start + s * p.T;
    int32_t *uo = p.uof + s * p.T;
    int cur = u - 1;   // the unit t0 - 1 belongs to
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + i;
        if (f & (1 << i)) {
            qu[u] = qr[t];
            ku[u] = kr[t];
            st[u] = t;
            cur = u;
            ++u;
        }
        if (t < p.T)
            uo[t] = cur;
    }
    if (g == sh.nseg - 1 && threadIdx.x == 0)
        p.nunit[s] = base + tot;
}

// ---------------------------------------------------------- key groups
//
// Segment g of kQbtSeg units per workgroup, 16 chunks of 64 units per
// round: the d-gram histogram of the segment's keys (LDS), and each chunk's
// latest key per short l-gram (wave tables in LDS, written out as rows of
// 16 chunks), and the run_start outputs of the segment's time steps.
// Segment 0 clears the stream's flags and counters.

__global__ __launch_bounds__(kQtThreads) void qt_keys_count_kernel(QkParams p, QtShape sh)
{
    extern __shared__ int qt_smem[];
    int *hist = qt_smem;                  // [nb]
    int *tabs = qt_smem + sh.nb;          // [16][fl]
    const int64_t s = blockIdx.y;
    const int g = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint64_t above = lane == 63 ? 0ull : (~0ull << (lane + 1));
    const int N = qt_units(p, s);
    const int K = p.K, d = sh.d, nb = sh.nbits;
    const uint8_t *C = qt_krow(p, s);
    if (g == 0 && tid == 0) {
        p.redo[s] = 0;
        p.dstream[s] = 0;
        p.xn[s] = 0;
    }
    for (int i = tid; i < sh.nb; i += kQtThreads)
        hist[i] = 0;
    int *tab = tabs + w * sh.fl;
    for (int r = 0; r < kQbtSeg / 1024; ++r) {
        for (int i = lane; i < sh.fl; i += 64)
            tab[i] = -1;
        __syncthreads();   // the zeroed histogram; the last round's rows written
        const int c = g * (kQbtSeg / 64) + r * 16 + w;   // chunk of this wave
        const int e = c * 64 + lane;
        const bool act = e < N;
        int gram = 0;
        uint64_t mk = ~0ull;
        for (int l = 1; l <= d; ++l) {
            const int j = l - 1;
            const bool v = act && e - j >= 0;
            const int dig = v ? min((int)C[e - j], K - 1) : 0;
            gram = gram * K + dig;
            if (l < d) {
                // keys of this chunk ending the same l-gram; the latest of
                // them enters the chunk's table
                mk &= qt_match(dig, v, dig, nb);
                if (v && !(mk & above))
                    tab[sh.floff[l] + gram] = e;
            } else if (v) {
                atomicAdd(&hist[gram], 1);
            }
        }
        __syncthreads();
        // rows of 16 consecutive chunks: thread -> (slot, chunk)
        const int c0 = g * (kQbtSeg / 64) + r * 16;
        int32_t *pt = p.ptab + s * sh.fl * sh.nch;
        for (int i = tid; i < sh.fl * 16; i += kQtThreads) {
            const int slot = i >> 4, ci = i & 15;
            if (c0 + ci < sh.nch)
                pt[(int64_t)slot * sh.nch + c0 + ci] = tabs[ci * sh.fl + slot];
        }
        __syncthreads();   // every table read before the next round clears it
    }
    int32_t *hc = p.hcnt + (s * sh.nseg + g) * sh.nb;
    for (int i = tid; i < sh.nb; i += kQtThreads)
        hc[i] = hist[i];
    if (p.run_start) {
        const int64_t T = p.T;
        for (int i = tid; i < kQbtSeg; i += kQtThreads) {
            const int t = g * kQbtSeg + i;
            if (t < T)
                p.run_start[s * T + t] = p.rle ? (t < N ? p.start[s * T + t] : -1) : t;
        }
    }
}

// Workgroup 0 of a stream: group offsets (a running sum over the segments
// per group, sixteen segments' counts in flight at a time, then a scan over
// the groups, in rounds of 1024 groups).  Workgroups 1..: one wave per
// short-table row, prefix maxima over its chunks: each lane takes 16
// consecutive chunks, a wave scan joins the lanes, 1024 chunks per pass.
__global__ __launch_bounds__(kQtThreads) void qt_keys_scan_kernel(QkParams p, QtShape sh)
{
    __shared__ int ws[64];
    const int64_t s = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int N = qt_units(p, s);
    if (blockIdx.x == 0) {
        // rounds of kQtThreads consecutive groups, thread tid taking group
        // r * kQtThreads + tid (so a segment's counts are read and written
        // coalesced): each group's counts become exclusive running sums
        // over the segments, and the groups' totals are scanned in group
        // order, one block scan per round with the carry between rounds
        const int R = (sh.nb + kQtThreads - 1) / kQtThreads;   // <= 16
        const int nsegN = (N + kQbtSeg - 1) / kQbtSeg;
        int32_t *hc = p.hcnt + s * sh.nseg * sh.nb;
        int32_t *ko = p.koff + s * (sh.nb + 1);
        int carry = 0;
        for (int r = 0; r < R; ++r) {
            const int b = r * kQtThreads + tid;
            int acc = 0;
            if (b < sh.nb) {
                // sixteen segments' counts in flight at a time (all of a
                // stream of 65536 units)
                int32_t *col = hc + b;
                for (int g0 = 0; g0 < nsegN; g0 += 16) {
                    int h[16];
#pragma unroll
                    for (int k = 0; k < 16; ++k)
                        h[k] = g0 + k < nsegN ? col[(int64_t)(g0 + k) * sh.nb] : 0;
#pragma unroll
                    for (int k = 0; k < 16; ++k)
                        if (g0 + k < nsegN) {
                            col[(int64_t)(g0 + k) * sh.nb] = acc;
                            acc += h[k];
                        }
                }
            }
            int total;
            const int base = qt_block_scan(acc, ws, &total);
            if (b < sh.nb)
                ko[b] = carry + base;
            carry += total;
        }
        if (tid == 0)
            ko[sh.nb] = carry;
        return;
    }
    const int slot = ((int)blockIdx.x - 1) * 16 + w;
    if (slot >= sh.fl)
        return;
    const int nchN = (N + 63) / 64;
    int32_t *row = p.ptab + (s * sh.fl + slot) * sh.nch;
    int carry = -1;
    for (int c0 = 0; c0 < nchN; c0 += 1024) {
        const int cl = c0 + 16 * lane;
        // a lane's 16 chunks are 64 aligned bytes of the row (pitch x16)
        int x[16];
        if (cl < nchN) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int4 v4 = reinterpret_cast<const int4 *>(row + cl)[k];
                x[4 * k] = v4.x;
                x[4 * k + 1] = v4.y;
                x[4 * k + 2] = v4.z;
                x[4 * k + 3] = v4.w;
            }
        }
#pragma unroll
        for (int k = 0; k < 16; ++k)
            x[k] = cl + k < nchN ? x[k] : -1;
#pragma unroll
        for (int k = 1; k < 16; ++k)
            x[k] = max(x[k], x[k - 1]);
        // lanes below: inclusive max scan of the lanes' last values
        int v = x[15];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(v, o);
            if (lane >= o)
                v = max(v, y);
        }
        int before = __shfl_up(v, 1);
        before = lane == 0 ? carry : max(before, carry);
        if (cl < nchN) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                reinterpret_cast<int4 *>(row + cl)[k] =
                    make_int4(max(x[4 * k], before), max(x[4 * k + 1], before),
                              max(x[4 * k + 2], before), max(x[4 * k + 3], before));
        }
        carry = max(carry, __shfl(v, 63));
    }
}

// Keys into their groups: LDS cursors from the offsets, then one entry
// {e, packed history} per key e >= d-1 of the segment.
__global__ __launch_bounds__(kQtThreads) void qt_keys_scatter_kernel(QkParams p, QtShape sh)
{
    extern __shared__ int qt_smem[];
    int *cur = qt_smem;   // [nb]
    const int64_t s = blockIdx.y;
    const int g = blockIdx.x;
    const int N = qt_units(p, s);
    if (g * kQbtSeg >= N)
        return;
    const int32_t *hc = p.hcnt + (s * sh.nseg + g) * sh.nb;
    const int32_t *ko = p.koff + s * (sh.nb + 1);
    for (int i = threadIdx.x; i < sh.nb; i += kQtThreads)
        cur[i] = ko[i] + hc[i];
    __syncthreads();
    const int K = p.K, d = sh.d;
    const uint8_t *C = qt_krow(p, s);
    int2 *kl = p.klist + s * qbt_kpitch(p.T);
#pragma unroll
    for (int r = 0; r < kQbtSeg / kQtThreads; ++r) {
        const int e = g * kQbtSeg + r * kQtThreads + (int)threadIdx.x;
        if (e < N && e >= d - 1) {
            int b = 0;
            for (int j = 0; j < d; ++j)
                b = b * K + min((int)C[e - j], K - 1);
            const uint32_t kh = qt_pack(C, e - d, sh.nbits, sh.P);
            const int slot = atomicAdd(&cur[b], 1);
            kl[slot] = make_int2(e, (int)kh);
        }
    }
}

// ------------------------------------------------------------- queries
//
// One thread per unit; the waves cover chunks of 64 units (the lane masks
// of the short path need a chunk's keys in one wave).  Workgroups go to the
// XCDs so that all of a stream's run on one of them (its groups and tables
// in one L2).  DC: the group depth when it is at most 4 (register arrays
// sized to it), 0 for any depth.  VB query symbols (the unit's own first,
// then the counterfactual ones) are taken together, so that their memory
// reads overlap: the group ranges, each round of group entries, each level
// of the short path and the destination times are one round trip for all
// VB of them.
//
// A group lists its keys segment by segment (the scatter runs one
// workgroup per segment of kQbtSeg units), so the scan of a group stops at
// the first key past the query unit's segment; keys of that segment at or
// after the unit are skipped.  Two entries per symbol are read per round.
template <int DC, int VB>
__global__ __launch_bounds__(kQtQThreads) void qt_query_kernel(QkParams p, QtShape sh, int W)
{
    constexpr int DM = DC > 0 ? DC : kQbtMaxD;
    const int bid = blockIdx.x;
    int64_t s;
    int wg;
    if (p.S >= 8) {
        const int x = bid & 7, i = bid >> 3;
        s = x + 8 * (int64_t)(i / W);
        wg = i % W;
    } else {
        s = bid / W;
        wg = bid % W;
    }
    if (s >= p.S || p.redo[s])
        return;
    const int N = qt_units(p, s);
    if (wg * kQtQThreads >= N)
        return;
    const int tid = threadIdx.x, lane = tid & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    const int u = wg * kQtQThreads + tid;
    const bool act = u < N;
    const int chunk = u >> 6, cbase = chunk << 6;
    const int K = p.K, d = DC > 0 ? DC : sh.d, nb = sh.nbits;
    const int64_t T = p.T;
    const uint8_t *Q = qt_qrow(p, s);
    const uint8_t *C = qt_krow(p, s);
    const int32_t *st = p.start + s * T;
    auto start_of = [&](int x) { return p.rle ? st[x] : x; };

    // ---- symbols of this unit as a query and as a key
    const int qu = act ? min((int)Q[u], K - 1) : 0;
    int qg[DM + 1];            // qg[l]: query digits 1..l-1 as the low part of an l-gram
    uint64_t eqk[DM];          // eqk[j]: chunk keys e with C[e-j] == Q[u-j] (j >= 1)
    qg[1] = 0;
    eqk[0] = ~0ull;
    int qrest = 0;             // qg[d]: the d-gram without its first symbol
    // depth 0: ballots of the key symbols C[e] of the chunk
    uint64_t B0[8];
    const int kd0 = act ? min((int)C[u], K - 1) : 0;
    const uint64_t vk0 = qt_ballot(act);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
        const uint64_t bb = qt_ballot((kd0 >> b) & 1);
        B0[b] = b < nb ? bb : 0ull;
    }
#pragma unroll
    for (int j = 1; j < DM; ++j) {
        if (j < d) {
            // as a key (lane's own unit) and as a query the same validity
            const bool v = act && u - j >= 0;
            const int qd = v ? min((int)Q[u - j], K - 1) : 0;
            const int kd = v ? min((int)C[u - j], K - 1) : 0;
            qg[j + 1] = qg[j] * K + qd;
            qrest = qg[j + 1];
            const uint64_t mm = qt_match(kd, v, qd, nb);
            eqk[j] = v ? mm : 0ull;
        }
    }
    const uint32_t qh = act && u >= d ? qt_pack(Q, u - d, nb, sh.P) : 0u;
    const int32_t *ko = p.koff + s * (sh.nb + 1);
    const int2 *kl = p.klist + s * qbt_kpitch(T);
    const int32_t *pt = p.ptab + s * sh.fl * sh.nch;
    const int segend = (u / kQbtSeg + 1) * kQbtSeg;
    const bool grp = act && u >= d - 1;
    // ---- run of time steps of this unit
    const int ts = act ? start_of(u) : 0;
    const int te = act ? (u + 1 < N ? start_of(u + 1) : (int)T) : 0;

    const bool want_cf = p.cf_tau || p.cf_ridx;
    const int V = want_cf ? 1 + p.M : 1;
    int D0 = -1, E0 = -1;
    uint32_t dmask = 0;   // query symbols left to the time-ordered pass
    for (int v0 = 0; v0 < V; v0 += VB) {
        int cv[VB], lo[VB], hi[VB], bc[VB], be[VB], E[VB], L[VB];
        bool dk[VB];   // left to the time-ordered pass
        // -- group ranges; a group of more than kcap keys leaves the symbol
        //    to the time-ordered pass
#pragma unroll
        for (int k = 0; k < VB; ++k) {
            const int v = v0 + k;
            cv[k] = v == 0 ? qu : (qu ^ (1 << ((v - 1) & 7)));
            lo[k] = hi[k] = 0;
            dk[k] = false;
            if (grp && v < V) {
                const int bk = cv[k] * sh.pw[d - 1] + qrest;
                lo[k] = ko[bk];
                hi[k] = ko[bk + 1];
                if (hi[k] - lo[k] > sh.kcap) {
                    dk[k] = true;
                    lo[k] = hi[k] = 0;
                }
            }
            bc[k] = be[k] = -1;
        }
        // -- groups: keys with the same d-gram, compared past it by their
        //    packed words; two entries of every symbol's group per round.
        //    best[k] = (c << 26) | (e + 1) of the best key so far (longest
        //    extension c <= P, then latest e; 0: none); lng[k]: some key
        //    matched all P packed symbols and has more history, so the
        //    longest extension may be longer (resolved below, from the rows)
        uint32_t best[VB];
        bool lng[VB];
#pragma unroll
        for (int k = 0; k < VB; ++k) {
            best[k] = 0u;
            lng[k] = false;
        }
        // entry pairs from the even index at or below the group's start
        // (16-byte loads; the entries outside [lo, hi) are masked)
        int base[VB];
#pragma unroll
        for (int k = 0; k < VB; ++k)
            base[k] = lo[k] & ~1;
        for (int i = 0;; i += 2) {
            bool more = false;
            int4 en[VB];
#pragma unroll
            for (int k = 0; k < VB; ++k)
                en[k] = base[k] + i < hi[k]
                            ? *reinterpret_cast<const int4 *>(kl + base[k] + i)
                            : make_int4(0x7FFFFFFF, 0, 0x7FFFFFFF, 0);
#pragma unroll
            for (int k = 0; k < VB; ++k) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int idx = base[k] + i + j;
                    const int ej = j ? en[k].z : en[k].x;
                    const uint32_t kh = (uint32_t)(j ? en[k].w : en[k].y);
                    const bool valid = idx >= lo[k] && idx < hi[k];
                    const int e = valid ? ej : 0x7FFFFFFF;
                    if (valid && e >= segend)
                        hi[k] = 0;   // the rest of the group lies past u
                    const uint32_t x = qh ^ kh;
                    const int avail = e - d + 1;   // key symbols past the d-gram
                    const int c = min(x ? (int)((__clz(x) * sh.rnb) >> 16) : sh.P, avail);
                    lng[k] |= e < u && x == 0u && avail > sh.P;
                    const uint32_t key = e < u ? ((uint32_t)c << 26) | (uint32_t)(e + 1) : 0u;
                    best[k] = max(best[k], key);
                }
                more |= base[k] + i + 2 < hi[k];
            }
            if (!more)
                break;
        }
#pragma unroll
        for (int k = 0; k < VB; ++k) {
            bc[k] = best[k] ? (int)(best[k] >> 26) : -1;
            be[k] = (int)(best[k] & 0x3FFFFFFu) - 1;
            if (lng[k]) {
                // long extensions: the group again, extending the keys that
                // matched all packed symbols 8 symbols per step from the rows
                const int bk = cv[k] * sh.pw[d - 1] + qrest;
                const int gl = ko[bk], gh = ko[bk + 1];
                int lc = -1, le = -1;
                for (int i = gl; i < gh && !dk[k]; ++i) {
                    const int2 en = kl[i];
                    const int e = en.x;
                    if (e >= segend)
                        break;
                    if (e >= u)
                        continue;
                    const uint32_t x = qh ^ (uint32_t)en.y;
                    const int avail = e - d + 1;
                    int c = x ? (int)((__clz(x) * sh.rnb) >> 16) : sh.P;
                    if (x == 0u && avail > sh.P) {
                        while (c < avail && c < kQtLcap) {
                            const uint64_t a = qt_load8_end(Q, u - d - c);
                            const uint64_t y = qt_load8_end(C, e - d - c);
                            if (a != y) {
                                c += __clzll((long long)(a ^ y)) >> 3;
                                break;
                            }
                            c += 8;
                        }
                        if (c >= kQtLcap && avail > kQtLcap)
                            dk[k] = true;   // a long repeat: the time-ordered pass
                    }
                    c = min(c, avail);
                    if (c > lc || (c == lc && e > le)) {
                        lc = c;
                        le = e;
                    }
                }
                bc[k] = lc;
                be[k] = le;
            }
        }
        // -- short grams for the symbols without a group answer: this
        //    chunk's keys by lane mask, earlier chunks from the table
        //    (wave-uniform masks, for every lane); one level at a time, the
        //    table reads of all VB symbols together
        uint64_t m[VB];
        bool alive[VB];
#pragma unroll
        for (int k = 0; k < VB; ++k) {
            m[k] = vk0;
#pragma unroll
            for (int b = 0; b < 8; ++b)
                if (b < nb)
                    m[k] &= ((cv[k] >> b) & 1) ? B0[b] : ~B0[b];
            E[k] = be[k];
            L[k] = be[k] >= 0 ? d + bc[k] : 0;
            alive[k] = act && be[k] < 0 && v0 + k < V && !dk[k];
        }
#pragma unroll
        for (int l = 1; l < DM; ++l) {
            if (l < d) {
                int el[VB];
#pragma unroll
                for (int k = 0; k < VB; ++k) {
                    if (l >= 2)
                        m[k] &= eqk[l - 1];
                    el[k] = -1;
                    alive[k] = alive[k] && u >= l - 1;
                    if (alive[k]) {
                        const uint64_t cand = m[k] & below;
                        if (cand)
                            el[k] = cbase + 63 - __clzll((long long)cand);
                        else if (chunk > 0)
                            el[k] = pt[(int64_t)(sh.floff[l] + cv[k] * sh.pw[l - 1] + qg[l]) *
                                           sh.nch + chunk - 1];
                    }
                }
#pragma unroll
                for (int k = 0; k < VB; ++k) {
                    if (alive[k] && el[k] >= 0) {
                        E[k] = el[k];
                        L[k] = l;
                    } else {
                        alive[k] = false;
                    }
                }
            }
        }
        // -- destinations: the start of unit E+1, for all VB symbols at once
        int D[VB];
#pragma unroll
        for (int k = 0; k < VB; ++k)
            D[k] = (act && E[k] >= 0 && E[k] + 1 < N) ? start_of(E[k] + 1) : -1;
#pragma unroll
        for (int k = 0; k < VB; ++k)
            if (act && v0 + k < V && dk[k])
                dmask |= 1u << (v0 + k);
        // the unit's answers are kept for the pieces qt_expand_kernel writes
        // (symbols left to the time-ordered pass; steps past the first 64)
        const bool keep = dmask != 0u || te - ts > 64 || V > VB;
        const int tw = min(te, ts + 64);
        // -- outputs of the unit's first 64 time steps (rewritten from the
        //    kept answers where a symbol was left)
#pragma unroll
        for (int k = 0; k < VB; ++k) {
            const int v = v0 + k;
            if (v >= V || !act)
                break;
            if (v == 0) {
                D0 = D[k];
                E0 = E[k];
                p.eo[s * T + u] = make_int4(E0, L[k], D0, 0);
                for (int t = ts; t < tw; ++t) {
                    const int64_t o = s * T + t;
                    const int tt = (D0 >= 0 && D0 < t) ? D0 : -1;
                    p.tau[o] = tt;
                    if (p.end)
                        p.end[o] = E0;
                    if (p.len)
                        p.len[o] = L[k];
                    if (p.run_of)
                        p.run_of[o] = u;
                    if (p.ridx)
                        p.ridx[o] = tt >= 0 ? E0 + 1 : -1;
                }
            } else {
                const int j = v - 1;
                if (keep && !dk[k])
                    p.cfe[(s * T + u) * p.M + j] = make_int2(E[k], D[k]);
                const bool bit = (qu >> j) & 1;
                for (int t = ts; t < tw; ++t) {
                    const int64_t c0 = ((s * T + t) * p.M + j) * 2;
                    const int t0 = (D0 >= 0 && D0 < t) ? D0 : -1;
                    const int tj = (D[k] >= 0 && D[k] < t) ? D[k] : -1;
                    const int r0 = t0 >= 0 ? E0 + 1 : -1;
                    const int rj = tj >= 0 ? E[k] + 1 : -1;
                    if (p.cf_tau)
                        *reinterpret_cast<int2 *>(p.cf_tau + c0) =
                            bit ? make_int2(tj, t0) : make_int2(t0, tj);
                    if (p.cf_ridx)
                        *reinterpret_cast<int2 *>(p.cf_ridx + c0) =
                            bit ? make_int2(rj, r0) : make_int2(r0, rj);
                }
            }
        }
    }
    if (act) {
        p.dfl[s * T + u] = dmask;
        if (dmask)
            p.dstream[s] = 1;
        // pieces of 64 steps left to qt_expand_kernel: the whole run when a
        // symbol was left, else the steps past the first 64
        const int first = dmask ? ts : ts + 64;
        if (first < te) {
            const int np = (te - first + 63) / 64;
            const int at = atomicAdd(&p.xn[s], np);
            int2 *xl = p.xl + s * qbt_xcap(T);
            for (int i = 0; i < np; ++i)
                xl[at + i] = make_int2(u, first + 64 * i);
        }
    }
}

// ------------------------------------------------------ time-ordered pass
//
// Query symbols the groups left (a group of more than kcap keys, or a match
// running more than kQtLcap units past d: low-entropy and repetitive
// streams) are answered here, one wave per stream, in time order.  The
// extension rule: if unit u-1's own answer (E, L) has L >= 1 and key unit
// E+1 carries the query symbol c, then c's answer at u is (E+1, L+1) -- a
// match at u without its last unit is a match at u-1, so none is longer,
// and E+1 is the latest end of that length.  A run of units whose own
// symbols were left is checked 64 units at a time (key units after E
// against the run's query symbols); where the rule fails, qt_direct
// computes the answer.

// The answer (E, L) of unit u for query symbol c from the definition, by
// the whole wave (u and c uniform): with u >= d-1, the keys of c's group
// before u, compared past the d-gram in full (packed words, then the rows),
// one per lane, scanning the group from its last segment back and stopping
// once no earlier segment can reach the best length; with no key before u
// in the group, the latest key ending each shorter gram (this chunk's keys
// directly, earlier chunks from the short table), longest gram first.
__device__ int2 qt_direct(const QkParams &p, const QtShape &sh, int64_t s, int u, int c,
                          const uint8_t *Q, const uint8_t *C)
{
    const int lane = __lane_id();
    const int d = sh.d, K = p.K, nb = sh.nbits;
    if (u >= d - 1) {
        int qrest = 0;
        for (int j = 1; j < d; ++j)
            qrest = qrest * K + min((int)Q[u - j], K - 1);
        const uint32_t qh = u >= d ? qt_pack(Q, u - d, nb, sh.P) : 0u;
        const int32_t *ko = p.koff + s * (sh.nb + 1);
        const int2 *kl = p.klist + s * qbt_kpitch(p.T);
        const int bk = c * sh.pw[d - 1] + qrest;
        const int lo = ko[bk], hi = ko[bk + 1];
        int bc = -1, be = -1;
        for (int i1 = hi; i1 > lo; i1 -= 64) {
            const int i = i1 - 64 + lane;
            int e = -1;
            uint32_t kh = 0;
            if (i >= lo) {
                const int2 en = kl[i];
                e = en.x;
                kh = (uint32_t)en.y;
            }
            if (e >= 0 && e < u) {
                const int avail = e - d + 1;
                const uint32_t x = qh ^ kh;
                int cc = x ? (int)((__clz(x) * sh.rnb) >> 16) : sh.P;
                if (x == 0u && avail > sh.P) {
                    while (cc < avail) {
                        const uint64_t a = qt_load8_end(Q, u - d - cc);
                        const uint64_t y = qt_load8_end(C, e - d - cc);
                        if (a != y) {
                            cc += __clzll((long long)(a ^ y)) >> 3;
                            break;
                        }
                        cc += 8;
                    }
                }
                cc = min(cc, avail);
                if (cc > bc || (cc == bc && e > be)) {
                    bc = cc;
                    be = e;
                }
            }
            // the lexicographic maximum of (c, e) over the lanes
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const int oc = __shfl_xor(bc, o), oe = __shfl_xor(be, o);
                if (oc > bc || (oc == bc && oe > be)) {
                    bc = oc;
                    be = oe;
                }
            }
            // entries below this round lie in segments up to lane 0's
            if (i1 - 64 > lo) {
                const int e0 = __shfl(e, 0);
                const int emax = (e0 / kQbtSeg + 1) * kQbtSeg - 1;
                if (emax - d + 1 < bc)
                    break;
            }
        }
        if (be >= 0)
            return make_int2(be, d + bc);
    }
    const int chunk = u >> 6, cb = chunk << 6;
    const int32_t *pt = p.ptab + s * sh.fl * sh.nch;
    for (int l = min(d - 1, u + 1); l >= 1; --l) {
        const int e = cb + lane;
        bool m = e < u && e >= l - 1 && min((int)C[e], K - 1) == c;
        for (int i = 1; i < l && m; ++i)
            m = min((int)C[e - i], K - 1) == min((int)Q[u - i], K - 1);
        const uint64_t bm = qt_ballot(m);
        if (bm)
            return make_int2(cb + 63 - __clzll((long long)bm), l);
        if (chunk > 0) {
            int g = c;
            for (int i = 1; i < l; ++i)
                g = g * K + min((int)Q[u - i], K - 1);
            const int ee = pt[(int64_t)(sh.floff[l] + g) * sh.nch + chunk - 1];
            if (ee >= 0)
                return make_int2(ee, l);
        }
    }
    return make_int2(-1, 0);
}

__global__ __launch_bounds__(64) void qt_defer_kernel(QkParams p, QtShape sh)
{
    const int64_t s = blockIdx.x;
    if (s >= p.S || !p.dstream[s])
        return;
    const int lane = threadIdx.x;
    const int N = qt_units(p, s);
    const int64_t T = p.T;
    const int K = p.K;
    const uint8_t *Q = qt_qrow(p, s);
    const uint8_t *C = qt_krow(p, s);
    const int32_t *st = p.start + s * T;
    auto dest = [&](int E) {
        return (E >= 0 && E + 1 < N) ? (p.rle ? st[E + 1] : E + 1) : -1;
    };
    const bool want_cf = p.cf_tau || p.cf_ridx;
    const int V = want_cf ? 1 + p.M : 1;
    int Ep = -1, Lp = 0;   // own answer of the unit before the chunk
    // a chunk's flags, kept answers and query symbols are loaded while the
    // chunk before it is answered (one wave per stream: the walk is bound by
    // memory latency, and a load issued after the chunk's stores would wait
    // for them too)
    uint32_t dfn = lane < N ? p.dfl[s * T + lane] : 0u;
    int4 eon = lane < N ? p.eo[s * T + lane] : make_int4(-1, 0, -1, 0);
    int qn = lane < N ? (int)Q[lane] : 0;
    for (int c0 = 0; c0 < N; c0 += 64) {
        const int u = c0 + lane;
        const bool act = u < N;
        const int n = min(64, N - c0);
        const uint32_t df = dfn;
        const int4 eoa = eon;
        const int qraw = qn;
        {
            const int un = u + 64;
            dfn = un < N ? p.dfl[s * T + un] : 0u;
            eon = un < N ? p.eo[s * T + un] : make_int4(-1, 0, -1, 0);
            qn = un < N ? (int)Q[un] : 0;
        }
        if (!qt_ballot(df != 0u)) {
            Ep = __shfl(eoa.x, n - 1);
            Lp = __shfl(eoa.y, n - 1);
            continue;
        }
        const int Ein = Ep, Lin = Lp;
        const int qs = act ? min(qraw, K - 1) : 0;
        int myE = eoa.x, myL = eoa.y;
        const uint64_t dm0 = qt_ballot(df & 1u);
        // own symbols in time order: runs by the extension rule
        int j = 0;
        while (j < n) {
            const uint64_t rest = dm0 & (~0ull << j);
            const int a = rest ? (int)__builtin_ctzll(rest) : n;
            if (a > j) {
                Ep = __shfl(myE, a - 1);
                Lp = __shfl(myL, a - 1);
            }
            if (a >= n)
                break;
            int k = 0;
            if (Lp >= 1) {
                const int i = lane - a;
                // key unit Ep+1+i <= u-1 since Ep <= c0 + a - 2
                const bool ok = lane >= a && lane < n && ((dm0 >> lane) & 1ull) &&
                                min((int)C[Ep + 1 + i], K - 1) == qs;
                const uint64_t okm = qt_ballot(ok) >> a;
                k = okm == ~0ull >> a ? 64 - a : (int)__builtin_ctzll(~okm);
                if (lane >= a && lane < a + k) {
                    myE = Ep + 1 + i;
                    myL = Lp + 1 + i;
                }
                Ep += k;
                Lp += k;
            }
            j = a + k;
            if (j < n && ((dm0 >> j) & 1ull)) {
                const int uj = c0 + j;
                const int2 r = qt_direct(p, sh, s, uj, __shfl(qs, j), Q, C);
                if (lane == j) {
                    myE = r.x;
                    myL = r.y;
                }
                Ep = r.x;
                Lp = r.y;
                ++j;
            }
        }
        Ep = __shfl(myE, n - 1);
        Lp = __shfl(myL, n - 1);
        if (df & 1u)
            p.eo[s * T + u] = make_int4(myE, myL, dest(myE), 0);
        // counterfactual symbols left to this pass: the rule from the
        // previous unit's own answer, else qt_direct one lane at a time
        int pE = __shfl_up(myE, 1), pL = __shfl_up(myL, 1);
        if (lane == 0) {
            pE = Ein;
            pL = Lin;
        }
        for (int v = 1; v < V; ++v) {
            const bool dv = (df >> v) & 1u;
            const int cvv = qs ^ (1 << (v - 1));
            int Ev = -1;
            bool need = false;
            if (dv) {
                if (pL >= 1 && min((int)C[pE + 1], K - 1) == cvv)
                    Ev = pE + 1;
                else
                    need = true;
            }
            uint64_t nm = qt_ballot(need);
            while (nm) {
                const int l = (int)__builtin_ctzll(nm);
                nm &= nm - 1;
                const int2 r = qt_direct(p, sh, s, c0 + l, __shfl(cvv, l), Q, C);
                if (lane == l)
                    Ev = r.x;
            }
            if (dv)
                p.cfe[(s * T + u) * p.M + v - 1] = make_int2(Ev, dest(Ev));
        }
    }
}

// ------------------------------------------------------------- outputs
//
// The pieces the query kernel left: 64 time steps of one unit per thread,
// written from the unit's kept answers.  The destination of an answer E is
// the start of unit E+1 when that start is before t (Eq. (16)'s range:
// strictly from the past); the counterfactual table pairs the unit's own
// destination with the branch's, in the order of the query symbol's bit.
__global__ __launch_bounds__(256) void qt_expand_kernel(QkParams p)
{
    const int64_t s = blockIdx.y;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (p.redo[s] || i >= p.xn[s])
        return;
    const int64_t T = p.T;
    const int N = qt_units(p, s);
    const int2 pc = p.xl[s * qbt_xcap(T) + i];
    const int u = pc.x;
    const int te0 = u + 1 < N ? (p.rle ? p.start[s * T + u + 1] : u + 1) : (int)T;
    const int te = min(te0, pc.y + 64);
    const int4 r = p.eo[s * T + u];
    const bool cf = p.cf_tau || p.cf_ridx;
    const int qs = cf ? min((int)qt_qrow(p, s)[u], p.K - 1) : 0;
    int2 cv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        cv[j] = cf && j < p.M ? p.cfe[(s * T + u) * p.M + j] : make_int2(-1, -1);
    for (int t = pc.y; t < te; ++t) {
        const int64_t o = s * T + t;
        const int t0 = (r.z >= 0 && r.z < t) ? r.z : -1;
        const int r0 = t0 >= 0 ? r.x + 1 : -1;
        p.tau[o] = t0;
        if (p.end)
            p.end[o] = r.x;
        if (p.len)
            p.len[o] = r.y;
        if (p.run_of)
            p.run_of[o] = u;
        if (p.ridx)
            p.ridx[o] = r0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (!cf || j >= p.M)
                break;
            const int2 c = cv[j];
            const int tj = (c.y >= 0 && c.y < t) ? c.y : -1;
            const int rj = tj >= 0 ? c.x + 1 : -1;
            const bool bit = (qs >> j) & 1;
            const int64_t c0 = (o * p.M + j) * 2;
            if (p.cf_tau)
                *reinterpret_cast<int2 *>(p.cf_tau + c0) = bit ? make_int2(tj, t0) : make_int2(t0, tj);
            if (p.cf_ridx)
                *reinterpret_cast<int2 *>(p.cf_ridx + c0) = bit ? make_int2(rj, r0) : make_int2(r0, rj);
        }
    }
}

template <int VB>
static void launch_query(const QkParams &p, const QtShape &sh, int W, int64_t blocks,
                         hipStream_t st)
{
    const dim3 g((unsigned)blocks), b(kQtQThreads);
    switch (sh.d) {
    case 1: hipLaunchKernelGGL((qt_query_kernel<1, VB>), g, b, 0, st, p, sh, W); break;
    case 2: hipLaunchKernelGGL((qt_query_kernel<2, VB>), g, b, 0, st, p, sh, W); break;
    case 3: hipLaunchKernelGGL((qt_query_kernel<3, VB>), g, b, 0, st, p, sh, W); break;
    case 4: hipLaunchKernelGGL((qt_query_kernel<4, VB>), g, b, 0, st, p, sh, W); break;
    default: hipLaunchKernelGGL((qt_query_kernel<0, 1>), g, b, 0, st, p, sh, W); break;
    }
}

bool raise_lds(const void *fn, size_t bytes)
{
    if (bytes <= 65536)
        return true;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) ==
           hipSuccess;
}

}  // namespace

// Launches the grouped-key kernels, which answer every stream (redo[] is
// cleared and stays clear).  hipErrorNotSupported: this path does not apply
// to the shape (one symbol; grids past their limits), nothing launched.
hipError_t launch_qk_batch(const QkParams &p, hipStream_t st)
{
    if (p.K < 2 || p.T < 1 || p.M > 8)
        return hipErrorNotSupported;
    const QbtShape q = qbt_shape(p.T, p.K);
    QtShape sh;
    sh.d = q.d;
    sh.nb = (int)q.nb;
    sh.fl = (int)q.fl;
    sh.nseg = q.nseg;
    sh.nch = q.nch;
    int nbits = 0;
    while ((1 << nbits) < p.K)
        ++nbits;
    sh.nbits = nbits;
    sh.P = 32 / nbits;
    sh.rnb = (65536 + nbits - 1) / nbits;
    if (sh.P > 32)
        sh.P = 32;
    // keys per group at most: a few times the mean, never below 256
    const int64_t mean = (p.T + q.nb - 1) / q.nb;
    sh.kcap = (int)(8 * mean > 256 ? 8 * mean : 256);
    // pw[l] = K^l (l <= d); level l's short-table slots follow those of
    // levels 1..l-1: floff[l] = K^1 + ... + K^(l-1)
    int pw = 1, fo = 0;
    for (int l = 0; l <= kQbtMaxD; ++l) {
        sh.pw[l] = l <= q.d ? pw : 0;
        sh.floff[l] = fo;
        if (l >= 1 && l < q.d)
            fo += pw;
        if (l < q.d)
            pw *= p.K;
    }
    const int W = (int)((p.T + kQtQThreads - 1) / kQtQThreads);
    const int64_t sgroups = p.S >= 8 ? (p.S + 7) / 8 * 8 : p.S;
    const int64_t qblocks = sgroups * W;
    if (qblocks >= ((int64_t)1 << 31) || q.nseg >= 65536 || p.S >= 65536)
        return hipErrorNotSupported;
    const size_t lds_count = (size_t)(sh.nb + 16 * sh.fl) * 4;
    const size_t lds_scatter = (size_t)sh.nb * 4;
    static bool raised = false;
    if (!raised) {
        if (!raise_lds(reinterpret_cast<const void *>(&qt_keys_count_kernel),
                       (size_t)(kQbtMaxNB + 16 * kQbtMaxFL) * 4) ||
            !raise_lds(reinterpret_cast<const void *>(&qt_keys_scatter_kernel),
                       (size_t)kQbtMaxNB * 4)) {
            (void)hipGetLastError();
            return hipErrorNotSupported;
        }
        raised = true;
    }
    const dim3 seg((unsigned)q.nseg, (unsigned)p.S);
    if (p.rle) {
        hipLaunchKernelGGL(qt_runs_count_kernel, seg, dim3(kQtThreads), 0, st, p, sh);
        hipLaunchKernelGGL(qt_runs_write_kernel, seg, dim3(kQtThreads), 0, st, p, sh);
    }
    hipLaunchKernelGGL(qt_keys_count_kernel, seg, dim3(kQtThreads), lds_count, st, p, sh);
    hipLaunchKernelGGL(qt_keys_scan_kernel, dim3((unsigned)(1 + (sh.fl + 15) / 16), (unsigned)p.S),
                       dim3(kQtThreads), 0, st, p, sh);
    hipLaunchKernelGGL(qt_keys_scatter_kernel, seg, dim3(kQtThreads), lds_scatter, st, p, sh);
    // the counterfactual symbols in rounds of up to five (M <= 4: one round)
    if (p.cf_tau || p.cf_ridx)
        launch_query<5>(p, sh, W, qblocks, st);
    else
        launch_query<1>(p, sh, W, qblocks, st);
    hipLaunchKernelGGL(qt_defer_kernel, dim3((unsigned)p.S), dim3(64), 0, st, p, sh);
    hipLaunchKernelGGL(qt_expand_kernel, dim3((unsigned)((qbt_xcap(p.T) + 255) / 256), (unsigned)p.S),
                       dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace rosa
