// rosa_sam.hip -- online suffix automaton per stream, for incremental
// decoding: rosa_build over a prefix, then one rosa_step per new position.
//
// Method: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix Matching"
// (arXiv 2602.02499), Sec. 2.2 (suffix automaton: at most 2n-1 states,
// amortised O(1) transitions and suffix-link jumps, Blumer et al. 1985) and
// Sec. 3.3 / App. B.3 (retrieval destination = end position of the longest
// suffix seen before, plus one); Sec. 4.1: one automaton per (b, r) stream.
//
// Per step and stream: append the symbol (new state, missing transitions
// set up the suffix-link path, attach to the target or split it with a clone
// that inherits the target's transitions, link and last end position); the
// new state's suffix link is the longest suffix that occurred before: its
// length is L and its last end position (read before the update) is E; then
// every state on the new state's suffix path gets last = t.
//
// Layout in the caller's state buffer (all per stream, stream-major):
//   flags    [64]   int32 (flags[0]: symbol >= K seen)
//   meta     [S]    int2 {tail state, number of states}
//   nodes    [S][Ncap] int4 {len, link, last, 0}, Ncap = max(2, 2*Tcap-1)
//   next     [S][Ncap][K] int32 dense transition rows (-1 = none)
//   hist     [S][Hs] uint8 symbol history (SYM = hist[E+1])
// One lane owns one stream, so every access to a stream's tables is ordered
// by program order; lanes of a wave work on different streams.
#include "rosa_internal.h"

namespace rosa {

struct SamLayout {
    size_t flags, meta, nodes, next, hist, total;
    int64_t Ncap, Hs;
};

SamLayout sam_layout(int64_t S, int64_t K, int64_t Tcap)
{
    SamLayout l;
    l.Ncap = Tcap <= 1 ? 2 : 2 * Tcap - 1;
    l.Hs = (int64_t)align_up((size_t)Tcap + 16, 16);
    size_t o = 0;
    l.flags = o;  o += 256;
    l.meta = o;   o = align_up(o + (size_t)S * 8, 256);
    l.nodes = o;  o = align_up(o + (size_t)S * l.Ncap * 16, 256);
    l.next = o;   o = align_up(o + (size_t)S * l.Ncap * K * 4, 256);
    l.hist = o;   o = align_up(o + (size_t)S * l.Hs, 256);
    l.total = o;
    return l;
}

struct SamView {
    int32_t *flags;
    int2 *meta;
    int4 *nodes;
    int32_t *next;
    uint8_t *hist;
    int64_t Ncap, Hs;
    int32_t K;
};

struct SamStream {
    int4 *nd;
    int32_t *nx;
    int K;
    int tail, nst;
};

__device__ __forceinline__ int sam_new_state(SamStream &a, int len)
{
    const int v = a.nst++;
    a.nd[v] = make_int4(len, -1, -1, 0);
    int32_t *row = a.nx + (int64_t)v * a.K;
    if ((a.K & 3) == 0) {
        int4 *r4 = reinterpret_cast<int4 *>(row);
        for (int c = 0; c < (a.K >> 2); ++c)
            r4[c] = make_int4(-1, -1, -1, -1);
    } else {
        for (int c = 0; c < a.K; ++c)
            row[c] = -1;
    }
    return v;
}

// Append symbol c; returns the new state.
__device__ int sam_extend(SamStream &a, int c)
{
    const int K = a.K;
    const int cur = sam_new_state(a, a.nd[a.tail].x + 1);
    int p = a.tail;
    while (p != -1 && a.nx[(int64_t)p * K + c] == -1) {
        a.nx[(int64_t)p * K + c] = cur;
        p = a.nd[p].y;
    }
    if (p == -1) {
        a.nd[cur].y = 0;
    } else {
        const int q = a.nx[(int64_t)p * K + c];
        const int4 nq = a.nd[q];
        const int lp = a.nd[p].x;
        if (lp + 1 == nq.x) {
            a.nd[cur].y = q;
        } else {
            const int clone = a.nst++;
            a.nd[clone] = make_int4(lp + 1, nq.y, nq.z, 0);
            const int32_t *src = a.nx + (int64_t)q * K;
            int32_t *dst = a.nx + (int64_t)clone * K;
            if ((K & 3) == 0) {
                const int4 *s4 = reinterpret_cast<const int4 *>(src);
                int4 *d4 = reinterpret_cast<int4 *>(dst);
                for (int k = 0; k < (K >> 2); ++k)
                    d4[k] = s4[k];
            } else {
                for (int k = 0; k < K; ++k)
                    dst[k] = src[k];
            }
            while (p != -1 && a.nx[(int64_t)p * K + c] == q) {
                a.nx[(int64_t)p * K + c] = clone;
                p = a.nd[p].y;
            }
            a.nd[q].y = clone;
            a.nd[cur].y = clone;
        }
    }
    a.tail = cur;
    return cur;
}

// Match for position t after the extension, then the last-end update.
__device__ __forceinline__ void sam_match(SamStream &a, int cur, int t,
                                          int &E, int &L)
{
    const int v = a.nd[cur].y;
    E = -1;
    L = 0;
    if (v > 0) {
        const int4 nv = a.nd[v];
        L = nv.x;
        E = nv.z;
    }
    for (int u = cur; u != -1; u = a.nd[u].y)
        a.nd[u].z = t;
}

__device__ __forceinline__ SamStream sam_open(const SamView &v, int64_t s)
{
    SamStream a;
    a.nd = v.nodes + s * v.Ncap;
    a.nx = v.next + s * v.Ncap * v.K;
    a.K = v.K;
    const int2 m = v.meta[s];
    a.tail = m.x;
    a.nst = m.y;
    return a;
}

// Build over hist[s][0..T): one lane per stream, `spw` streams per wave.
__global__ __launch_bounds__(64) void sam_build_kernel(
    SamView v, int64_t S, int64_t T, int spw, int32_t *__restrict__ E,
    int16_t *__restrict__ SYM, int32_t *__restrict__ L)
{
    const int lane = threadIdx.x;
    if (lane >= spw)
        return;
    const int64_t s = (int64_t)blockIdx.x * spw + lane;
    if (s >= S)
        return;
    SamStream a;
    a.nd = v.nodes + s * v.Ncap;
    a.nx = v.next + s * v.Ncap * v.K;
    a.K = v.K;
    a.tail = 0;
    a.nst = 0;
    sam_new_state(a, 0);   // root: len 0, no link
    const uint8_t *h = v.hist + s * v.Hs;
    for (int64_t t = 0; t < T; ++t) {
        const int c = h[t];
        const int cur = sam_extend(a, c);
        int e, l;
        sam_match(a, cur, (int)t, e, l);
        if (E) {
            E[s * T + t] = e;
            if (L)
                L[s * T + t] = l;
            if (SYM)
                SYM[s * T + t] = e >= 0 ? (int16_t)h[e + 1] : (int16_t)-1;
        }
    }
    v.meta[s] = make_int2(a.tail, a.nst);
}

// Validate/clamp symbols of a SYMBOLS prefix into the history rows.
__global__ void sam_hist_kernel(const uint8_t *__restrict__ in, int64_t ld,
                                int64_t T, int32_t K, uint8_t *__restrict__ hist,
                                int64_t Hs, uint8_t *__restrict__ copy_out,
                                int32_t *__restrict__ flags)
{
    const int64_t s = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= T)
        return;
    uint8_t c = in[s * ld + t];
    if (c >= K) {
        atomicOr(&flags[0], 1);
        c = (uint8_t)(K - 1);
    }
    hist[s * Hs + t] = c;
    if (copy_out)
        copy_out[s * T + t] = c;
}

__device__ __forceinline__ uint32_t bf16_pos_s(uint32_t h)
{
    return (h - 1u) < 0x7F80u ? 1u : 0u;
}

// One position for every stream.  kind 0: symbols row[s*ld]; kind 1: bf16
// row [B][ld], stream s = b*R + r reads channels r*M .. r*M+M-1.
__global__ __launch_bounds__(64) void sam_step_kernel(
    SamView v, int64_t S, int64_t t, int spw, int kind, const void *row,
    int64_t ld, int64_t R, int M, const uint16_t *__restrict__ V, int64_t ldv,
    int64_t ldv_b, int32_t *__restrict__ end, int16_t *__restrict__ sym,
    uint16_t *__restrict__ out_row, int64_t ldo_b)
{
    const int lane = threadIdx.x;
    if (lane >= spw)
        return;
    const int64_t s = (int64_t)blockIdx.x * spw + lane;
    if (s >= S)
        return;
    int c;
    const int64_t b = s / R, r = s % R;
    if (kind == 0) {
        c = reinterpret_cast<const uint8_t *>(row)[s * ld];
        if (c >= v.K) {
            atomicOr(&v.flags[0], 1);
            c = v.K - 1;
        }
    } else {
        const uint16_t *hrow = reinterpret_cast<const uint16_t *>(row) + b * ld + r * M;
        c = 0;
        for (int j = 0; j < M; ++j)
            c |= (int)bf16_pos_s(hrow[j]) << j;
    }
    uint8_t *h = v.hist + s * v.Hs;
    h[t] = (uint8_t)c;
    SamStream a = sam_open(v, s);
    const int cur = sam_extend(a, c);
    int e, l;
    sam_match(a, cur, (int)t, e, l);
    v.meta[s] = make_int2(a.tail, a.nst);
    end[s] = e;
    if (sym)
        sym[s] = e >= 0 ? (int16_t)h[e + 1] : (int16_t)-1;
    if (out_row) {
        uint16_t *o = out_row + b * ldo_b + r * M;
        const uint16_t *src = V + b * ldv_b + (int64_t)(e + 1) * ldv + r * M;
        for (int m = 0; m < M; ++m)
            o[m] = e >= 0 ? src[m] : (uint16_t)0;
    }
}

// ------------------------------------------------- query / key retrieval
//
// Sec. 3.3 with separate streams: one automaton per stream over the key
// units, one matching state (state, length) advanced by the query units.
// Units are time steps, or with run folding the maximal runs of equal key
// symbols (Sec. 3.3 RLE paragraph): the automaton and the matching state
// move once per run, at its first time step, with the run's key symbol and
// the query symbol at that time.  At unit u the automaton holds the key
// units 0..u-1 (the query is matched before the key symbol of u is
// appended), so the match is strictly earlier; its end unit e is the
// matched state's last end position and the destination is the start time
// of unit e+1, kept when it is before t (the range of Eq. (16)).  App. C.5:
// for each query bit the branch with the bit flipped is one more matching
// update from the same state (the branch with the bit as it is equals the
// forward pass).
//
// The matching state is not re-normalised after an append that splits the
// state it sits in: until the next append the split state and its clone
// have identical transition rows, and the next query update leaves the
// state through a transition or a suffix link, so both give the same
// result.

// One matching update by symbol c: follow suffix links until a transition
// on c exists, take it (length + 1), or fall to the root (length 0).
__device__ __forceinline__ void qk_advance(const SamStream &a, int &s, int &l,
                                           int c)
{
    const int K = a.K;
    for (;;) {
        const int nx = a.nx[(int64_t)s * K + c];
        if (nx != -1) {
            s = nx;
            ++l;
            return;
        }
        if (s == 0) {
            l = 0;
            return;
        }
        s = a.nd[s].y;
        l = a.nd[s].x;
    }
}

// One wave per stream: lane 0 advances the matching state and appends the
// key units; lanes 1..M make the counterfactual updates (bit lane-1 of the
// query symbol flipped) from the same state at the same time.  Only lane 0
// writes the automaton; a workgroup barrier (the workgroup is this one
// wave) orders its writes before the next unit's reads by the other lanes.
__global__ __launch_bounds__(64) void qk_kernel(QkParams p)
{
    const int lane = threadIdx.x;
    const int64_t s = blockIdx.x;
    if (s >= p.S || (p.only && p.only[s] == 0))
        return;
    const bool want_cf = p.cf_tau || p.cf_ridx;
    const int nl = want_cf ? 1 + p.M : 1;   // active lanes
    const bool act = lane < nl;
    const int64_t T = p.T;
    SamStream a;
    a.nd = p.nodes + s * p.Ncap;
    a.nx = p.next + s * p.Ncap * p.K;
    a.K = p.K;
    a.tail = 0;
    a.nst = 0;
    if (lane == 0)
        sam_new_state(a, 0);
    a.nst = 1;
    __syncthreads();
    const uint8_t *qr = p.q + s * p.Tp + kPadFront;
    const uint8_t *kr = p.k + s * p.Tp + kPadFront;
    int32_t *st = p.start + s * T;
    // lane 0: the forward pass; lane j+1: bit j forced to the other value
    int u = -1, ms = 0, ml = 0, ue = -1, ul = 0, dstart = -1, kprev = -1, qc = 0;
    for (int64_t t = 0; t < T; ++t) {
        const int kc = kr[t];
        if (!p.rle || kc != kprev) {
            ++u;
            if (lane == 0)
                st[u] = (int32_t)t;
            qc = qr[t];
            __syncthreads();   // start of unit u visible to every lane
            if (act) {
                int s2 = ms, l2 = ml;
                qk_advance(a, s2, l2, lane == 0 ? qc : (qc ^ (1 << (lane - 1))));
                ue = l2 > 0 ? a.nd[s2].z : -1;
                ul = l2;
                dstart = ue >= 0 ? st[ue + 1] : -1;
                if (lane == 0) {
                    ms = s2;
                    ml = l2;
                }
            }
            __syncthreads();   // every read of this unit before the append
            if (lane == 0) {
                const int cur = sam_extend(a, kc);
                for (int w = cur; w != -1; w = a.nd[w].y)
                    a.nd[w].z = u;
            }
            // every lane follows lane 0's matching state
            ms = __shfl(ms, 0);
            ml = __shfl(ml, 0);
            __syncthreads();   // this unit's appends before the next reads
            kprev = kc;
        }
        const int64_t o = s * T + t;
        // lane v's destination for this time step
        const int tv = (ue >= 0 && dstart < t) ? dstart : -1;
        const int rv = tv >= 0 ? ue + 1 : -1;
        const int tt = __shfl(tv, 0), rt = __shfl(rv, 0);
        if (lane == 0) {
            p.tau[o] = tt;
            if (p.end)
                p.end[o] = ue;
            if (p.len)
                p.len[o] = ul;
            if (p.run_of)
                p.run_of[o] = u;
            if (p.ridx)
                p.ridx[o] = rt;
        }
        if (want_cf && lane >= 1 && lane <= p.M) {
            const int j = lane - 1;
            const int b = (qc >> j) & 1;
            const int64_t c0 = (o * p.M + j) * 2;
            if (p.cf_tau) {
                p.cf_tau[c0 + b] = tt;
                p.cf_tau[c0 + 1 - b] = tv;
            }
            if (p.cf_ridx) {
                p.cf_ridx[c0 + b] = rt;
                p.cf_ridx[c0 + 1 - b] = rv;
            }
        }
    }
    if (p.run_start)
        for (int64_t v = lane; v < T; v += 64)
            p.run_start[s * T + v] = v <= u ? st[v] : -1;
}

// ---------------------------------- query / key retrieval, tables in LDS
//
// The same automaton and matching state as qk_kernel for streams of at most
// MT time steps over at most 64 symbols, with every table in the
// workgroup's LDS instead of HBM:
//   ll[v]     len(v) | (link(v) + 1) << 16        (2T - 1 states at most)
//   lastu[v]  last end unit of v (0xFFFF: none)
//   st[u]     start time of unit u
//   ht        transitions as an open-addressing hash table: entry
//             (v*K + c) << 13 | target, linear probing; the automaton has at
//             most 3T - 4 transitions (Blumer et al.), so the table (6 MT
//             slots) is at most half full and every probe ends at a free slot.
// 152 KiB at MT = 4096 (one stream per CU), 76 KiB at 2048 (two), 38 KiB at
// 1024 (four).  One wave per stream.  The append is computed by every lane
// on the same values (LDS reads of one address are broadcasts) and written
// by lane 0; the transitions of a split state are copied by lanes 0..K-1,
// one symbol each.  The wave's LDS instructions complete in issue order, so
// the lanes see each other's writes in program order with no barrier (the
// workgroup is this one wave), and no global store is waited for inside
// the loop.  Outputs are staged in registers, lane i holding time step
// t0 + i, and written 64 steps at a time.
constexpr int kQlTgtBits = 13;
constexpr uint32_t kQlEmpty = 0xFFFFFFFFu;
constexpr int kQlMaxK = 64;   // (states * K) << 13 must fit 32 bits

template <int MT>
struct QlCfg {
    static constexpr int kStates = 2 * MT;
    static constexpr int kSlots = 6 * MT;
    static constexpr size_t kLds = (size_t)kSlots * 4 + (size_t)kStates * 6 + (size_t)MT * 2;
};

struct QlHit {
    int tgt;    // target state, or -1
    int slot;   // slot holding the key, else the free slot that ends the probe
};

template <int NS>
__device__ __forceinline__ QlHit ql_find(const uint32_t *ht, uint32_t key)
{
    uint32_t slot = __umulhi(key * 0x9E3779B1u, (uint32_t)NS);
    for (;;) {
        const uint32_t e = ht[slot];
        if (e == kQlEmpty)
            return {-1, (int)slot};
        if ((e >> kQlTgtBits) == key)
            return {(int)(e & ((1u << kQlTgtBits) - 1)), (int)slot};
        slot = slot + 1 == (uint32_t)NS ? 0u : slot + 1;
    }
}

__device__ __forceinline__ int ql_link(uint32_t w) { return (int)(w >> 16) - 1; }
__device__ __forceinline__ int ql_len(uint32_t w) { return (int)(w & 0xFFFFu); }
__device__ __forceinline__ int ql_uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int MT>
__global__ __launch_bounds__(64) void qk_lds_kernel(QkParams p)
{
    using C = QlCfg<MT>;
    constexpr int NS = C::kSlots;
    __shared__ __align__(16) uint32_t ht[NS];
    __shared__ uint32_t ll[C::kStates];
    __shared__ uint16_t lastu[C::kStates];
    __shared__ uint16_t st[MT];
    const int lane = threadIdx.x;
    const int64_t s = blockIdx.x;
    if (p.only && p.only[s] == 0)
        return;
    const int T = (int)p.T, K = p.K, M = p.M;
    const bool want_cf = p.cf_tau || p.cf_ridx;
    const int nl = want_cf ? 1 + M : 1;
    {
        uint4 *h4 = reinterpret_cast<uint4 *>(ht);
        for (int i = lane; i < NS / 4; i += 64)
            h4[i] = make_uint4(kQlEmpty, kQlEmpty, kQlEmpty, kQlEmpty);
        if (lane == 0) {
            ll[0] = 0;          // root: len 0, no link
            lastu[0] = 0xFFFF;
        }
    }
    __syncthreads();
    const uint8_t *qr = p.q + s * p.Tp + kPadFront;
    const uint8_t *kr = p.k + s * p.Tp + kPadFront;
    const int64_t base = s * (int64_t)T;
    int u = -1, ms = 0, ml = 0, kprev = -1, qc = 0;
    int tail = 0, tlen = 0, nst = 1;
    int ue = -1, ul = 0, dstart = -1;   // this lane's chain (lane j+1: bit j flipped)
    // the rows carry 64 bytes of padding after T: chunk loads stay in the row
    int kn = kr[lane], qn = qr[lane];
    for (int t0 = 0; t0 < T; t0 += 64) {
        const int kch = kn, qch = qn;
        if (t0 + 64 < T) {
            kn = kr[t0 + 64 + lane];
            qn = qr[t0 + 64 + lane];
        }
        int o_tau = -1, o_end = -1, o_len = 0, o_run = -1, o_ridx = -1;
        int o_ct[16], o_cr[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            o_ct[i] = -1;
            o_cr[i] = -1;
        }
        const int n = T - t0 < 64 ? T - t0 : 64;
        for (int j = 0; j < n; ++j) {
            const int t = t0 + j;
            const int kc = __builtin_amdgcn_readlane(kch, j);
            if (!p.rle || kc != kprev) {
                ++u;
                qc = __builtin_amdgcn_readlane(qch, j);
                if (lane == 0)
                    st[u] = (uint16_t)t;
                // matching updates: lane 0 by q, lane j+1 by q with bit j flipped
                int s2 = ms, l2 = ml;
                if (lane < nl) {
                    const int c = lane == 0 ? qc : (qc ^ (1 << ((lane - 1) & 7)));
                    for (;;) {
                        const QlHit h = ql_find<NS>(ht, (uint32_t)(s2 * K + c));
                        if (h.tgt >= 0) {
                            s2 = h.tgt;
                            ++l2;
                            break;
                        }
                        if (s2 == 0) {
                            l2 = 0;
                            break;
                        }
                        s2 = ql_link(ll[s2]);
                        l2 = ql_len(ll[s2]);
                    }
                    const int lu = lastu[s2];
                    ue = l2 > 0 ? lu : -1;
                    ul = l2;
                    dstart = ue >= 0 ? (int)st[ue + 1] : -1;
                }
                ms = __builtin_amdgcn_readlane(s2, 0);
                ml = __builtin_amdgcn_readlane(l2, 0);
                // append key symbol kc
                const int cur = nst++;
                int pp = tail, q = -1, lp = 0;
                while (pp >= 0) {
                    const uint32_t key = (uint32_t)(pp * K + kc);
                    const uint32_t wp = ll[pp];
                    const QlHit h = ql_find<NS>(ht, key);
                    const int tg = ql_uni(h.tgt);
                    if (tg >= 0) {
                        q = tg;
                        lp = ql_len(wp);
                        break;
                    }
                    if (lane == 0)
                        ht[h.slot] = key << kQlTgtBits | (uint32_t)cur;
                    pp = ql_uni(ql_link(wp));
                }
                int lk = 0;
                if (pp >= 0) {
                    const uint32_t wq = (uint32_t)ql_uni((int)ll[q]);
                    if (lp + 1 == ql_len(wq)) {
                        lk = q;
                    } else {
                        const int cl = nst++;
                        if (lane == 0) {
                            ll[cl] = (uint32_t)(lp + 1) | (wq & 0xFFFF0000u);
                            lastu[cl] = lastu[q];
                        }
                        if (lane < K) {
                            const QlHit h = ql_find<NS>(ht, (uint32_t)(q * K + lane));
                            if (h.tgt >= 0) {
                                const uint32_t key = (uint32_t)(cl * K + lane);
                                const uint32_t e = key << kQlTgtBits | (uint32_t)h.tgt;
                                uint32_t slot = __umulhi(key * 0x9E3779B1u, (uint32_t)NS);
                                while (atomicCAS(&ht[slot], kQlEmpty, e) != kQlEmpty)
                                    slot = slot + 1 == (uint32_t)NS ? 0u : slot + 1;
                            }
                        }
                        // redirect (v, kc) -> q to the clone up the suffix path
                        while (pp >= 0) {
                            const uint32_t key = (uint32_t)(pp * K + kc);
                            const uint32_t wp = ll[pp];
                            const QlHit h = ql_find<NS>(ht, key);
                            if (ql_uni(h.tgt) != q)
                                break;
                            if (lane == 0)
                                ht[h.slot] = key << kQlTgtBits | (uint32_t)cl;
                            pp = ql_uni(ql_link(wp));
                        }
                        if (lane == 0)
                            ll[q] = (wq & 0xFFFFu) | (uint32_t)(cl + 1) << 16;
                        lk = cl;
                    }
                }
                if (lane == 0)
                    ll[cur] = (uint32_t)(tlen + 1) | (uint32_t)(lk + 1) << 16;
                // every state on the new state's suffix path ends at unit u
                for (int w = cur; w >= 0; w = ql_uni(ql_link(ll[w])))
                    if (lane == 0)
                        lastu[w] = (uint16_t)u;
                tail = cur;
                ++tlen;
                kprev = kc;
            }
            // this step's outputs, staged in lane j
            const int tv = (ue >= 0 && dstart < t) ? dstart : -1;
            const int rv = tv >= 0 ? ue + 1 : -1;
            const int tt = __builtin_amdgcn_readlane(tv, 0);
            const int rt = __builtin_amdgcn_readlane(rv, 0);
            const int e0 = __builtin_amdgcn_readlane(ue, 0);
            const int l0 = __builtin_amdgcn_readlane(ul, 0);
            if (lane == j) {
                o_tau = tt;
                o_end = e0;
                o_len = l0;
                o_run = u;
                o_ridx = rt;
            }
            if (want_cf) {
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    if (b < M) {
                        const int tb = __builtin_amdgcn_readlane(tv, b + 1);
                        const int rb = __builtin_amdgcn_readlane(rv, b + 1);
                        const int bit = (qc >> b) & 1;
                        if (lane == j) {
                            o_ct[2 * b] = bit ? tb : tt;
                            o_ct[2 * b + 1] = bit ? tt : tb;
                            o_cr[2 * b] = bit ? rb : rt;
                            o_cr[2 * b + 1] = bit ? rt : rb;
                        }
                    }
                }
            }
        }
        if (lane < n) {
            const int64_t o = base + t0 + lane;
            p.tau[o] = o_tau;
            if (p.end)
                p.end[o] = o_end;
            if (p.len)
                p.len[o] = o_len;
            if (p.run_of)
                p.run_of[o] = o_run;
            if (p.ridx)
                p.ridx[o] = o_ridx;
            if (want_cf) {
#pragma unroll
                for (int b = 0; b < 8; ++b) {
                    if (b < M) {
                        const int64_t c0 = (o * M + b) * 2;
                        if (p.cf_tau)
                            *reinterpret_cast<int2 *>(p.cf_tau + c0) =
                                make_int2(o_ct[2 * b], o_ct[2 * b + 1]);
                        if (p.cf_ridx)
                            *reinterpret_cast<int2 *>(p.cf_ridx + c0) =
                                make_int2(o_cr[2 * b], o_cr[2 * b + 1]);
                    }
                }
            }
        }
    }
    if (p.run_start)
        for (int v = lane; v < T; v += 64)
            p.run_start[base + v] = v <= u ? (int32_t)st[v] : -1;
}

// --------------------------------------------------------------- launchers

SamView sam_view(void *buf, int64_t S, int64_t K, int64_t Tcap)
{
    const SamLayout l = sam_layout(S, K, Tcap);
    char *base = reinterpret_cast<char *>(buf);
    SamView v;
    v.flags = reinterpret_cast<int32_t *>(base + l.flags);
    v.meta = reinterpret_cast<int2 *>(base + l.meta);
    v.nodes = reinterpret_cast<int4 *>(base + l.nodes);
    v.next = reinterpret_cast<int32_t *>(base + l.next);
    v.hist = base ? reinterpret_cast<uint8_t *>(base + l.hist) : nullptr;
    v.Ncap = l.Ncap;
    v.Hs = l.Hs;
    v.K = (int32_t)K;
    return v;
}

size_t sam_total_bytes(int64_t S, int64_t K, int64_t Tcap)
{
    return sam_layout(S, K, Tcap).total;
}

uint8_t *sam_hist_base(void *buf, int64_t S, int64_t K, int64_t Tcap,
                       int64_t *Hs)
{
    const SamLayout l = sam_layout(S, K, Tcap);
    *Hs = l.Hs;
    return reinterpret_cast<uint8_t *>(buf) + l.hist;
}

int32_t *sam_flags(void *buf) { return reinterpret_cast<int32_t *>(buf); }

// One stream per wave: the per-stream work is a chain of dependent memory
// accesses with data-dependent loop counts; lanes of one wave would wait for
// the slowest stream at every loop, so each stream gets its own wave (the
// prefix build of 512 x 65536 positions takes 231 ms this way against 374 ms
// with eight streams per wave).
constexpr int kSamStreamsPerWave = 1;

hipError_t launch_sam_hist(const uint8_t *in, int64_t ld, int64_t S, int64_t T,
                           int32_t K, void *buf, int64_t Tcap,
                           uint8_t *copy_out, hipStream_t st)
{
    if (T == 0)
        return hipSuccess;
    SamView v = sam_view(buf, S, K, Tcap);
    dim3 grid((unsigned)((T + 255) / 256), (unsigned)S);
    hipLaunchKernelGGL(sam_hist_kernel, grid, dim3(256), 0, st, in, ld, T, K,
                       v.hist, v.Hs, copy_out, v.flags);
    return hipGetLastError();
}

hipError_t launch_clear_flags(int32_t *flags, hipStream_t st,
                              int32_t *flags2 = nullptr);

hipError_t launch_sam_build(void *buf, int64_t S, int64_t K, int64_t Tcap,
                            int64_t T, int32_t *E, int16_t *SYM, int32_t *L,
                            hipStream_t st)
{
    SamView v = sam_view(buf, S, K, Tcap);
    const int spw = kSamStreamsPerWave;
    dim3 grid((unsigned)((S + spw - 1) / spw));
    hipLaunchKernelGGL(sam_build_kernel, grid, dim3(64), 0, st, v, S, T, spw,
                       E, SYM, L);
    return hipGetLastError();
}

hipError_t launch_sam_step(void *buf, int64_t S, int64_t K, int64_t Tcap,
                           int64_t t, int kind, const void *row, int64_t ld,
                           int64_t R, int M, const uint16_t *V, int64_t ldv,
                           int64_t ldv_b, int32_t *end, int16_t *sym,
                           uint16_t *out_row, int64_t ldo_b, hipStream_t st)
{
    SamView v = sam_view(buf, S, K, Tcap);
    const int spw = kSamStreamsPerWave;
    dim3 grid((unsigned)((S + spw - 1) / spw));
    hipLaunchKernelGGL(sam_step_kernel, grid, dim3(64), 0, st, v, S, t, spw,
                       kind, row, ld, R, M, V, ldv, ldv_b, end, sym, out_row,
                       ldo_b);
    return hipGetLastError();
}

// LDS tables when the stream fits a configuration and the streams fit the
// device in one round (one workgroup per stream resident at once), or when
// only a few streams are expected (`any`: the leftovers of the bit-parallel
// kernel); otherwise the HBM tables, whose many waves per CU hide their
// latency better than a second round of LDS workgroups.
template <int MT>
static bool qk_lds_try(const QkParams &p, hipStream_t st, bool any)
{
    if (p.T > MT)
        return false;
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return false;
    if (cus[dev] == 0 &&
        hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return false;
    const int64_t per_cu = 163840 / (int64_t)QlCfg<MT>::kLds;
    if (!any && p.S > per_cu * cus[dev])
        return false;
    hipLaunchKernelGGL(qk_lds_kernel<MT>, dim3((unsigned)p.S), dim3(64), 0, st, p);
    return true;
}

bool qk_bits_fits(const QkParams &p);
hipError_t launch_qk_bits(const QkParams &p, hipStream_t st);

// The bit-parallel kernel when the streams fit it, then an automaton kernel
// for the streams it left (matches longer than its levels); otherwise an
// automaton kernel for every stream.
hipError_t launch_qk(QkParams p, hipStream_t st)
{
    p.spw = 1;
    p.only = nullptr;
    bool bits = qk_bits_fits(p);
    if (bits) {
        // hipErrorNotSupported: not launched, the automaton takes every stream
        const hipError_t e = launch_qk_bits(p, st);
        if (e == hipErrorNotSupported)
            bits = false;
        else if (e != hipSuccess)
            return e;
        else
            p.only = p.redo;
    }
    const bool lds_ok = p.K <= kQlMaxK && p.M <= 8;
    if (!(lds_ok && (qk_lds_try<1024>(p, st, bits) || qk_lds_try<2048>(p, st, bits) ||
                     qk_lds_try<4096>(p, st, bits))))
        hipLaunchKernelGGL(qk_kernel, dim3((unsigned)p.S), dim3(64), 0, st, p);
    return hipGetLastError();
}

}  // namespace rosa
