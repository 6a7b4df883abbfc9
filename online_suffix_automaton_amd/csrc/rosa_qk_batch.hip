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
// A stream with a key group of more than kcap keys, or a match that runs
// more than kQtLcap symbols past d, is marked in redo[] and answered by the
// automaton kernel afterwards (long repeats; low-entropy streams).
#include "rosa_internal.h"

namespace rosa {

namespace {

constexpr int kQtThreads = 1024;   // segment kernels: kQbtSeg units, 4 per thread
constexpr int kQtQThreads = 256;   // query kernel: 4 chunks of 64 units
constexpr int kQtLcap = 1024;      // extension past d followed before giving up
constexpr int kQtMaxV = 9;         // the unit's own query symbol + M <= 8 branches

// Everything the kernels need besides QkParams: group depth, alphabet
// powers, short-table offsets, packing.
struct QtShape {
    int d, nb, fl, P, nbits, kcap;
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
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (f & (1 << i)) {
            const int t = t0 + i;
            qu[u] = qr[t];
            ku[u] = kr[t];
            st[u] = t;
            ++u;
        }
    }
    if (g == sh.nseg - 1 && threadIdx.x == 0)
        p.nunit[s] = base + tot;
}

// ---------------------------------------------------------- key groups
//
// Segment g of kQbtSeg units per workgroup, 16 chunks of 64 units per
// round: the d-gram histogram of the segment's keys (LDS), and each chunk's
// latest key per short l-gram (wave tables in LDS, written out as rows of
// 16 chunks).  Also the run_start outputs of the segment's time steps and,
// from segment 0, the stream's redo flag cleared.

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
    if (g == 0 && tid == 0)
        p.redo[s] = 0;
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
// per group, then a scan over the groups) and the group-size cap.
// Workgroups 1..: prefix maxima over the chunks of 64 short-table rows.
__global__ __launch_bounds__(kQtThreads) void qt_keys_scan_kernel(QkParams p, QtShape sh)
{
    __shared__ int ws[64];
    const int64_t s = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int N = qt_units(p, s);
    if (blockIdx.x == 0) {
        const int R = (sh.nb + kQtThreads - 1) / kQtThreads;   // <= 16
        const int nsegN = (N + kQbtSeg - 1) / kQbtSeg;
        int32_t *hc = p.hcnt + s * sh.nseg * sh.nb;
        int tot[16];
        int sum = 0, big = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            tot[r] = 0;
            const int b = tid * R + r;
            if (r < R && b < sh.nb) {
                int run = 0;
                for (int gg = 0; gg < nsegN; ++gg) {
                    const int h = hc[(int64_t)gg * sh.nb + b];
                    hc[(int64_t)gg * sh.nb + b] = run;
                    run += h;
                }
                tot[r] = run;
                sum += run;
                big = max(big, run);
            }
        }
        int total;
        int base = qt_block_scan(sum, ws, &total);
        int32_t *ko = p.koff + s * (sh.nb + 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int b = tid * R + r;
            if (r < R && b < sh.nb) {
                ko[b] = base;
                base += tot[r];
            }
        }
        if (tid == 0)
            ko[sh.nb] = total;
        if (big > sh.kcap)
            p.redo[s] = 1;
        return;
    }
    const int nchN = (N + 63) / 64;
    int32_t *pt = p.ptab + s * sh.fl * sh.nch;
    for (int k = 0; k < 4; ++k) {
        const int slot = ((int)blockIdx.x - 1) * 64 + k * 16 + w;
        if (slot >= sh.fl)
            break;
        int32_t *row = pt + (int64_t)slot * sh.nch;
        int carry = -1;
        for (int c0 = 0; c0 < nchN; c0 += 64) {
            const int c = c0 + lane;
            int v = c < nchN ? row[c] : -1;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(v, o);
                if (lane >= o)
                    v = max(v, y);
            }
            v = max(v, carry);
            if (c < nchN)
                row[c] = v;
            carry = __shfl(v, 63);
        }
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
    int2 *kl = p.klist + s * p.T;
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
// in one L2).
__global__ __launch_bounds__(kQtQThreads) void qt_query_kernel(QkParams p, QtShape sh, int W)
{
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
    const int K = p.K, d = sh.d, nb = sh.nbits;
    const int64_t T = p.T;
    const uint8_t *Q = qt_qrow(p, s);
    const uint8_t *C = qt_krow(p, s);
    const int32_t *st = p.start + s * T;
    auto start_of = [&](int x) { return p.rle ? st[x] : x; };

    // ---- symbols of this unit as a query and as a key
    const int qu = act ? min((int)Q[u], K - 1) : 0;
    int qg[kQbtMaxD + 1];      // qg[l]: query digits 1..l-1 as the low part of an l-gram
    uint64_t eqk[kQbtMaxD];    // eqk[j]: chunk keys e with C[e-j] == Q[u-j] (j >= 1)
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
    for (int j = 1; j < kQbtMaxD; ++j) {
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
    const int2 *kl = p.klist + s * T;
    const int32_t *pt = p.ptab + s * sh.fl * sh.nch;

    // ---- run of time steps of this unit
    const int ts = act ? start_of(u) : 0;
    const int te = act ? (u + 1 < N ? start_of(u + 1) : (int)T) : 0;

    const bool want_cf = p.cf_tau || p.cf_ridx;
    const int V = want_cf ? 1 + p.M : 1;
    int D0 = -1, E0 = -1;
    bool over = false;
    for (int v = 0; v < V; ++v) {
        const int cv = v == 0 ? qu : (qu ^ (1 << (v - 1)));
        int E = -1, L = 0;
        bool found = false;
        // -- groups: keys with the same d-gram, compared past it
        if (act && u >= d - 1) {
            const int bk = cv * sh.pw[d - 1] + qrest;
            const int lo = ko[bk], hi = ko[bk + 1];
            int bc = -1, be = -1;
            for (int i = lo; i < hi; ++i) {
                const int2 en = kl[i];
                const int e = en.x;
                if (e >= u)
                    continue;
                const int avail = e - d + 1;   // key symbols past the d-gram
                const uint32_t x = qh ^ (uint32_t)en.y;
                int c = x ? (int)(__clz(x) / nb) : sh.P;
                if (c >= sh.P && avail > sh.P) {
                    // past the packed words: 8 symbols per step from the rows
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
                        over = true;
                }
                c = min(c, avail);
                if (c > bc || (c == bc && e > be)) {
                    bc = c;
                    be = e;
                }
            }
            if (be >= 0) {
                E = be;
                L = d + bc;
                found = true;
            }
        }
        // -- short grams: this chunk's keys by lane mask, earlier chunks
        //    from the table (wave-uniform masks, for every lane)
        uint64_t m = vk0;
#pragma unroll
        for (int b = 0; b < 8; ++b)
            if (b < nb)
                m &= ((cv >> b) & 1) ? B0[b] : ~B0[b];
        bool alive = act && !found;
#pragma unroll
        for (int l = 1; l < kQbtMaxD; ++l) {
            if (l < d) {
                if (l >= 2)
                    m &= eqk[l - 1];
                if (alive && u >= l - 1) {
                    const uint64_t cand = m & below;
                    int e = -1;
                    if (cand)
                        e = cbase + 63 - __clzll((long long)cand);
                    else if (chunk > 0)
                        e = pt[(int64_t)(sh.floff[l] + cv * sh.pw[l - 1] + qg[l]) * sh.nch +
                               chunk - 1];
                    if (e >= 0) {
                        E = e;
                        L = l;
                    } else {
                        alive = false;
                    }
                } else {
                    alive = false;
                }
            }
        }
        // -- outputs for every time step of the unit
        const int D = (E >= 0 && E + 1 < N) ? start_of(E + 1) : -1;
        if (v == 0) {
            D0 = D;
            E0 = E;
            for (int t = ts; t < te; ++t) {
                const int64_t o = s * T + t;
                const int tt = (D >= 0 && D < t) ? D : -1;
                p.tau[o] = tt;
                if (p.end)
                    p.end[o] = E;
                if (p.len)
                    p.len[o] = L;
                if (p.run_of)
                    p.run_of[o] = u;
                if (p.ridx)
                    p.ridx[o] = tt >= 0 ? E + 1 : -1;
            }
        } else {
            const int j = v - 1;
            const bool bit = (qu >> j) & 1;
            for (int t = ts; t < te; ++t) {
                const int64_t c0 = ((s * T + t) * p.M + j) * 2;
                const int t0 = (D0 >= 0 && D0 < t) ? D0 : -1;
                const int tj = (D >= 0 && D < t) ? D : -1;
                if (p.cf_tau)
                    *reinterpret_cast<int2 *>(p.cf_tau + c0) =
                        bit ? make_int2(tj, t0) : make_int2(t0, tj);
                if (p.cf_ridx) {
                    const int r0 = t0 >= 0 ? E0 + 1 : -1;
                    const int rj = tj >= 0 ? E + 1 : -1;
                    *reinterpret_cast<int2 *>(p.cf_ridx + c0) =
                        bit ? make_int2(rj, r0) : make_int2(r0, rj);
                }
            }
        }
    }
    if (over)
        p.redo[s] = 1;
}

bool raise_lds(const void *fn, size_t bytes)
{
    if (bytes <= 65536)
        return true;
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) ==
           hipSuccess;
}

}  // namespace

// Launches the grouped-key kernels for every stream; streams they give up
// on are marked in redo[] (zeroed here first).  hipErrorNotSupported: this
// path does not apply to the shape, nothing launched.
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
    hipLaunchKernelGGL(qt_keys_scan_kernel, dim3((unsigned)(1 + (sh.fl + 63) / 64), (unsigned)p.S),
                       dim3(kQtThreads), 0, st, p, sh);
    hipLaunchKernelGGL(qt_keys_scatter_kernel, seg, dim3(kQtThreads), lds_scatter, st, p, sh);
    hipLaunchKernelGGL(qt_query_kernel, dim3((unsigned)qblocks), dim3(kQtQThreads), 0, st, p, sh,
                       W);
    return hipGetLastError();
}

}  // namespace rosa
