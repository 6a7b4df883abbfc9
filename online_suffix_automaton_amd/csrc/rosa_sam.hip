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
// every state on the new state's suffix path gets last = t.  A step costs
// the length of that suffix path, which is short on varied streams but
// grows with t on a constant or short-period stream (t+1 states).
//
// The prefix build (rosa_build) takes the prefix's outputs from the batch
// retrieval kernels and appends the prefix without the last-end walks; the
// last end of every state is then set in one pass: the last end of a state
// is the largest end position in its suffix-link subtree, i.e. the latest
// position whose prefix state (a non-clone state, created at that position
// with length position + 1) lies in the subtree.  Visiting the non-clone
// states from the latest position down, each walks up its suffix path
// until it meets a state already set, so every state is written once: O(T)
// per stream on any input.
//
// Layout in the caller's state buffer (all per stream, stream-major):
//   flags    [64]   int32 (flags[0]: symbol >= K seen)
//   meta     [S]    int4 {tail state, number of states, tail length,
//                         tail suffix link}
//   states   [S][Ncap] records of RS bytes: node int4 {len, link, last,
//            clone ? 1 : 0}, then the dense transition row int32 [K]
//            (-1 = none); RS = 16 + 4K rounded up to 64 bytes (one 128-byte
//            line at K = 16), Ncap = max(2, 2*Tcap-1)
//   hist     [S][Hs] uint8 symbol history (SYM = hist[E+1])
// A state's node and row share a record, so each state the append's chain
// visits costs one cache line.  The states region (padded if needed) first
// serves as the batch retrieval's workspace during rosa_build; the
// automaton overwrites it after that (same stream, so in order).
// One lane owns one stream, so every access to a stream's tables is ordered
// by program order; lanes of a wave work on different streams.
#include "rosa_internal.h"
#include "rosa_qk_decode.h"
#include "rosa_sam_core.h"

namespace rosa {

struct SamLayout {
    size_t flags, meta, states, hist, total;
    size_t ws_bytes;   // workspace of the prefix retrieval, from `states` on
    int64_t Ncap, Hs, RS;
};

SamLayout sam_layout(int64_t S, int64_t K, int64_t Tcap)
{
    SamLayout l;
    l.Ncap = Tcap <= 1 ? 2 : 2 * Tcap - 1;
    l.Hs = (int64_t)align_up((size_t)Tcap + 16, 16);
    size_t o = 0;
    l.flags = o;  o += 256;
    l.meta = o;   o = align_up(o + (size_t)S * 16, 256);
    l.RS = (int64_t)align_up((size_t)(16 + 4 * K), 64);
    l.states = o; o = align_up(o + (size_t)S * l.Ncap * l.RS, 256);
    // the batch retrieval's workspace for any prefix length up to Tcap
    // (record mode ends at 65536 positions, so its size can drop past it)
    const int64_t Tr = Tcap < 65536 ? Tcap : 65536;
    size_t ws = ws_layout(S, Tcap).total;
    if (ws_layout(S, Tr).total > ws)
        ws = ws_layout(S, Tr).total;
    if (l.states + ws > o)
        o = align_up(l.states + ws, 256);
    l.ws_bytes = o - l.states;
    l.hist = o;   o = align_up(o + (size_t)S * l.Hs, 256);
    l.total = o;
    return l;
}

struct SamView {
    int32_t *flags;
    int4 *meta;
    int32_t *states;   // records of RSi ints
    uint8_t *hist;
    int64_t Ncap, Hs, RSi;
    int32_t K;
};

// Stream s's automaton in the decode state (tail and size not set).
__device__ __forceinline__ SamStream sam_stream(const SamView &v, int64_t s)
{
    SamStream a;
    int32_t *rec = v.states + s * v.Ncap * v.RSi;
    a.nd = reinterpret_cast<int4 *>(rec);
    a.nds = v.RSi / 4;
    a.nx = rec + 4;
    a.nxs = v.RSi;
    a.K = v.K;
    a.tail = 0;
    a.nst = 0;
    a.tail_len = 0;
    a.tail_link = -1;
    return a;
}

__device__ __forceinline__ SamStream sam_open(const SamView &v, int64_t s)
{
    SamStream a = sam_stream(v, s);
    const int4 m = v.meta[s];
    a.tail = m.x;
    a.nst = m.y;
    a.tail_len = m.z;
    a.tail_link = m.w;
    return a;
}

// Build over hist[s][0..T): one lane per stream, `spw` streams per wave.
// The appends run without last-end walks; then the last ends are set in one
// pass over the states (see the top of this file).
// Last ends after appends made without the last-end walks, by the 64 lanes
// of the stream's wave (the result of sam_fill_last): a state's last end is
// the latest position among the non-clone states of its link subtree (a
// non-clone state of length n was created at position n-1).  Rounds of 64
// states from the newest down; each lane with a non-clone state raises its
// last end and its ancestors' to the state's position by atomic max, and
// stops at a node that already holds a later or equal one: whatever walk
// put that value there raises every ancestor above it as well.  Taking the
// states from the newest down makes most walks stop within a few links.
__device__ void sam_fill_last_wave(const SamStream &a, int nst)
{
    const int lane = __lane_id();
    for (int top = nst - 1; top >= 1; top -= 64) {
        const int w = top - lane;
        int u = -1, pos = 0;
        if (w >= 1) {
            const int4 nw = a.node(w);
            if (nw.w == 0) {
                u = w;
                pos = nw.x - 1;
            }
        }
        while (u != -1) {
            int *lastp = &a.node(u).z;
            const int up = a.node(u).y;   // links do not change here
            const int old = atomicMax(lastp, pos);
            if (old >= pos)
                break;
            u = up;
        }
    }
}

// Appends by the whole wave, for K <= 60: a state's record (node ints 0..3,
// transition c at int 4+c) is one 4-byte load per lane, lane i holding int i,
// so a record is one coalesced round trip and any field is a lane read.
// Every int of a record is stored by the lane that loads it (lane i for int
// i), so each lane reads its own earlier stores in program order and no
// fence is needed between appends.  The record of the tail's suffix link
// (the state the next append's walk starts from: the matched state, its
// clone, or the root) is kept in the lanes between appends, with every
// store this wave makes to it mirrored, so most appends need one or two
// round trips (the record of the transition's target) instead of one per
// field.  Same steps and results as sam_extend.
struct WaveSam {
    int cid;    // state whose record the lanes hold (-2: none)
    int cval;   // this lane's int of that record
};

__device__ __forceinline__ int32_t *sam_rec(const SamStream &a, int v)
{
    return reinterpret_cast<int32_t *>(&a.node(v));
}

__device__ __forceinline__ int wave_rec_load(const SamStream &a, int v, int nint)
{
    const int lane = __lane_id();
    return lane < nint ? sam_rec(a, v)[lane] : -1;
}

__device__ void sam_extend_wave(SamStream &a, WaveSam &ws, int c)
{
    const int lane = __lane_id();
    const int nint = 4 + a.K;
    const int cur = a.nst++;
    if (lane == 4 + c)
        sam_rec(a, a.tail)[4 + c] = cur;   // the tail has no transitions
    int p = a.tail_link;
    int val = -1, pc = -1;
    while (p != -1) {
        val = p == ws.cid ? ws.cval : wave_rec_load(a, p, nint);
        pc = __builtin_amdgcn_readlane(val, 4 + c);
        if (pc != -1)
            break;
        if (lane == 4 + c)
            sam_rec(a, p)[4 + c] = cur;
        val = lane == 4 + c ? cur : val;
        if (p == ws.cid)
            ws.cval = val;
        if (p == 0) {   // the root: keep its record for the next walk
            ws.cid = 0;
            ws.cval = val;
        }
        p = __builtin_amdgcn_readlane(val, 1);
    }
    int lk = 0;
    if (p != -1) {
        const int q = pc;
        const int lp = __builtin_amdgcn_readlane(val, 0);
        const int qval = q == ws.cid ? ws.cval : wave_rec_load(a, q, nint);
        if (lp + 1 == __builtin_amdgcn_readlane(qval, 0)) {
            lk = q;
            ws.cid = q;
            ws.cval = qval;
        } else {
            // clone of q with length lp + 1: q's link, last end and
            // transitions, the clone flag set
            const int clone = a.nst++;
            const int cv = lane == 0 ? lp + 1 : lane == 3 ? 1 : qval;
            if (lane < nint)
                sam_rec(a, clone)[lane] = cv;
            // transitions on c into q from p and its ancestors go to the clone
            int rv = val;
            while (p != -1) {
                if (__builtin_amdgcn_readlane(rv, 4 + c) != q)
                    break;
                if (lane == 4 + c)
                    sam_rec(a, p)[4 + c] = clone;
                if (p == ws.cid)
                    ws.cval = lane == 4 + c ? clone : ws.cval;
                p = __builtin_amdgcn_readlane(rv, 1);
                if (p != -1)
                    rv = p == ws.cid ? ws.cval : wave_rec_load(a, p, nint);
            }
            if (lane == 1)
                sam_rec(a, q)[1] = clone;
            lk = clone;
            ws.cid = clone;
            ws.cval = cv;
        }
    }
    // the new state's record: length, link, no last end, not a clone, no
    // transitions
    if (lane < nint)
        sam_rec(a, cur)[lane] = lane == 0 ? a.tail_len + 1 : lane == 1 ? lk : lane == 3 ? 0 : -1;
    a.tail = cur;
    a.tail_len += 1;
    a.tail_link = lk;
}

// One stream per wave: the wave appends the prefix (lane 0 alone for
// alphabets over 60 symbols), then fills the last ends.
__global__ __launch_bounds__(64) void sam_build_kernel(SamView v, int64_t S,
                                                       int64_t T)
{
    const int lane = threadIdx.x;
    const int64_t s = blockIdx.x;
    if (s >= S)
        return;
    SamStream a = sam_stream(v, s);
    int nst = 0;
    const uint8_t *h = v.hist + s * v.Hs;
    if (a.K <= 60) {
        // root: len 0, no link, no last end, no transitions (each int by its lane)
        if (lane < 4 + a.K)
            sam_rec(a, 0)[lane] = lane == 0 ? 0 : lane == 3 ? 0 : -1;
        a.nst = 1;
        WaveSam ws = {-2, -1};
        for (int64_t t = 0; t < T; ++t)
            sam_extend_wave(a, ws, h[t]);
        if (lane == 0)
            v.meta[s] = make_int4(a.tail, a.nst, a.tail_len, a.tail_link);
        nst = a.nst;
    } else {
        if (lane == 0) {
            sam_new_state(a, 0);
            for (int64_t t = 0; t < T; ++t)
                sam_extend(a, h[t]);
            v.meta[s] = make_int4(a.tail, a.nst, a.tail_len, a.tail_link);
            nst = a.nst;
        }
        nst = __shfl(nst, 0);
    }
    // the records visible to every lane (the workgroup is this wave)
    __syncthreads();
    sam_fill_last_wave(a, nst);
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
    v.meta[s] = make_int4(a.tail, a.nst, a.tail_len, a.tail_link);
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
        const int nx = a.row(s)[c];
        if (nx != -1) {
            s = nx;
            ++l;
            return;
        }
        if (s == 0) {
            l = 0;
            return;
        }
        s = a.node(s).y;
        l = a.node(s).x;
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
    a.nds = 1;
    a.nx = p.next + s * p.Ncap * p.K;
    a.nxs = p.K;
    a.K = p.K;
    a.tail = 0;
    a.nst = 0;
    a.tail_len = 0;
    a.tail_link = -1;
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
                ue = l2 > 0 ? a.node(s2).z : -1;
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
                for (int w = cur; w != -1; w = a.node(w).y)
                    a.node(w).z = u;
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

// ------------------------------------------ query / key retrieval, decode
//
// The same automaton and matching state as qk_kernel, kept in a caller's
// state buffer between calls: qkd_kernel loads a stream's state, runs time
// steps t0 .. t0+n-1 and stores the state back.  rosa_build_qk runs it over
// the prefix (init: empty automaton, no unit yet) and rosa_step_qk for one
// time step, so build + steps give the batch call's outputs by
// construction.  With run folding a step that continues the current key
// run moves neither the automaton nor the matching state; its outputs come
// from the unit's kept answers (E, L, destination, and each flipped query
// bit's E and destination), with the destination kept only when it is
// before t.  The flipped branches are computed at every unit whenever the
// alphabet has query bits (K = 2^M), whether or not the call asks for them,
// so a later step that asks finds them current.

__device__ __forceinline__ int qkd_symbol(const QkdParams &p, const void *in,
                                          int64_t ld, int64_t s, int64_t i)
{
    if (p.kind == 0) {
        int c = reinterpret_cast<const uint8_t *>(in)[s * ld + i];
        if (c >= p.K) {
            atomicOr(&p.flags[0], 1);
            c = p.K - 1;
        }
        return c;
    }
    const int64_t b = s / p.R, r = s % p.R;
    const uint16_t *h = reinterpret_cast<const uint16_t *>(in) +
                        (b * p.Tin + i) * ld + r * p.Min;
    int c = 0;
    for (int j = 0; j < p.Min; ++j)
        c |= (int)bf16_pos_s(h[j]) << j;
    return c;
}

// A stream's decode registers between time steps: the current unit, the
// matching state, the previous key symbol, the unit's query symbol and its
// answers (lane 0: E, L, destination; lane j+1: E and destination with
// query bit j flipped).
struct QkdRegs {
    int u, ms, ml, kprev, qc, ue, ul, dstart;
};

__device__ __forceinline__ SamStream qkd_stream(const QkdParams &p, int64_t s)
{
    SamStream a;
    int32_t *rec = p.states + s * p.Ncap * p.RSi;
    a.nd = reinterpret_cast<int4 *>(rec);
    a.nds = p.RSi / 4;
    a.nx = rec + 4;
    a.nxs = p.RSi;
    a.K = p.K;
    a.tail = 0;
    a.nst = 0;
    a.tail_len = 0;
    a.tail_link = -1;
    return a;
}

__device__ __forceinline__ QkdRegs qkd_fresh()
{
    QkdRegs r;
    r.u = -1; r.ms = 0; r.ml = 0; r.kprev = -1; r.qc = 0;
    r.ue = -1; r.ul = 0; r.dstart = -1;
    return r;
}

__device__ __forceinline__ void qkd_save(const QkdParams &p, const SamStream &a, int64_t s,
                         const QkdRegs &r)
{
    const int lane = threadIdx.x;
    if (lane == 0) {
        p.meta[s] = make_int4(a.tail, a.nst, a.tail_len, a.tail_link);
        p.mst[2 * s] = make_int4(r.u, r.ms, r.ml, r.kprev);
        p.mst[2 * s + 1] = make_int4(r.qc, r.ue, r.ul, r.dstart);
    } else if (lane <= p.M) {
        p.cfst[s * kQkdMaxBits + lane - 1] = make_int2(r.ue, r.dstart);
    }
}

// Time steps tb .. te-1 of stream s, in order, from the registers `r` (the
// input and output index of time t is t - p.t0).  One wave: lane 0
// advances the matching state and appends the key units, lanes 1..M make
// the flipped-bit updates from the same state; a workgroup barrier (the
// workgroup is this one wave) orders lane 0's writes before the next
// unit's reads by the other lanes.  The symbols of 64 steps are loaded at
// once, one step per lane, and broadcast.
__device__ __forceinline__ void qkd_steps(const QkdParams &p, SamStream &a, int64_t s,
                          int64_t tb, int64_t te, QkdRegs &r)
{
    const int lane = threadIdx.x;
    const bool act = lane <= p.M;   // lane 0, and a lane per query bit
    int32_t *st = p.start + s * p.Ucap;
    // the registers as locals (kept out of memory), written back at the end
    int u = r.u, ms = r.ms, ml = r.ml, kprev = r.kprev, qc = r.qc;
    int ue = r.ue, ul = r.ul, dstart = r.dstart;
    int kbuf = 0, qbuf = 0;
    for (int64_t t = tb; t < te; ++t) {
        const int64_t j = t - tb;
        if ((j & 63) == 0 && t + lane < te) {
            kbuf = qkd_symbol(p, p.k, p.ldk, s, t + lane - p.t0);
            qbuf = qkd_symbol(p, p.q, p.ldq, s, t + lane - p.t0);
        }
        const int kc = __shfl(kbuf, (int)(j & 63));
        const int qcur = __shfl(qbuf, (int)(j & 63));
        if (!p.rle || kc != kprev) {
            ++u;
            if (lane == 0)
                st[u] = (int32_t)t;
            qc = qcur;
            __syncthreads();   // start of unit u visible to every lane
            if (act) {
                int s2 = ms, l2 = ml;
                qk_advance(a, s2, l2, lane == 0 ? qc : (qc ^ (1 << (lane - 1))));
                ue = l2 > 0 ? a.node(s2).z : -1;
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
                for (int w = cur; w != -1; w = a.node(w).y)
                    a.node(w).z = u;
            }
            ms = __shfl(ms, 0);
            ml = __shfl(ml, 0);
            __syncthreads();   // this unit's appends before the next reads
            kprev = kc;
        }
        const int64_t o = s * p.ostride + (t - p.t0);
        const int tv = (ue >= 0 && dstart < t) ? dstart : -1;
        const int rv = tv >= 0 ? ue + 1 : -1;
        const int tt = __shfl(tv, 0), rt = __shfl(rv, 0);
        if (lane == 0) {
            if (p.tau)
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
        if (lane >= 1 && act) {
            const int jb = lane - 1;
            const int b = (qc >> jb) & 1;
            const int64_t c0 = (o * p.M + jb) * 2;
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
    r.u = u; r.ms = ms; r.ml = ml; r.kprev = kprev; r.qc = qc;
    r.ue = ue; r.ul = ul; r.dstart = dstart;
}

// Time steps t0 .. t0+n-1 for every stream, one wave each: from an empty
// automaton (init) or the saved state, then the state saved back.
__global__ __launch_bounds__(64) void qkd_kernel(QkdParams p)
{
    const int lane = threadIdx.x;
    const int64_t s = blockIdx.x;
    if (s >= p.S)
        return;
    SamStream a = qkd_stream(p, s);
    QkdRegs r = qkd_fresh();
    if (p.init) {
        if (lane == 0)
            sam_new_state(a, 0);
        a.nst = 1;
    } else {
        const int4 m = p.meta[s];
        a.tail = m.x;
        a.nst = m.y;
        a.tail_len = m.z;
        a.tail_link = m.w;
        const int4 m1 = p.mst[2 * s], m2 = p.mst[2 * s + 1];
        r.u = m1.x; r.ms = m1.y; r.ml = m1.z; r.kprev = m1.w; r.qc = m2.x;
        if (lane == 0) {
            r.ue = m2.y; r.ul = m2.z; r.dstart = m2.w;
        } else if (lane <= p.M) {
            const int2 c = p.cfst[s * kQkdMaxBits + lane - 1];
            r.ue = c.x; r.dstart = c.y;
        }
    }
    __syncthreads();   // the root record before any lane reads it
    qkd_steps(p, a, s, p.t0, p.t0 + p.n, r);
    qkd_save(p, a, s, r);
    if (p.run_start) {
        const int32_t *st = p.start + s * p.Ucap;
        for (int64_t v = lane; v < p.n; v += 64)
            p.run_start[s * p.ostride + v] = v <= r.u ? st[v] : -1;
    }
}

// Build over a prefix of p.n steps (p.t0 = 0) whose E and L per time step
// the batch retrieval has already written (bend, blen: [S][bld]).  With U
// units in the prefix, the key units 0..U-2 are appended by the whole wave
// without the last-unit walks and the last units filled afterwards (the
// self-match build's method: a state's last unit is the newest unit among
// the non-clone states of its link subtree, which is what the walks
// compute).  The matching state after unit U-2 is the state of the string
// of length L ending at unit E (unit U-2's answer): the state created at
// unit E, up its suffix links while the link's length is at least L (the
// suffix path of a string's state holds every suffix of it).  The steps of
// the last unit then run through qkd_steps, which computes that unit's
// answers and its flipped-bit branches and leaves the registers a later
// step continues from.  The walk-free appends need K <= 60 (one int per
// lane); qkd_kernel serves larger alphabets.
__global__ __launch_bounds__(64) void qkd_prefix_kernel(QkdParams p,
                                                        const int32_t *__restrict__ bend,
                                                        const int32_t *__restrict__ blen,
                                                        int64_t bld)
{
    const int lane = threadIdx.x;
    const int64_t s = blockIdx.x;
    if (s >= p.S)
        return;
    SamStream a = qkd_stream(p, s);
    int32_t *st = p.start + s * p.Ucap;
    const int64_t T = p.n;
    // units: start times into st, 64 steps at a time
    int U = 0, kp = -1;
    for (int64_t t0 = 0; t0 < T; t0 += 64) {
        const int64_t t = t0 + lane;
        const int kc = t < T ? qkd_symbol(p, p.k, p.ldk, s, t) : -1;
        const int prev = __shfl_up(kc, 1);
        const int before = lane == 0 ? kp : prev;
        const bool nu = t < T && (!p.rle || kc != before);
        const uint64_t m = __ballot(nu);
        if (nu)
            st[U + __popcll(m & ((1ull << lane) - 1))] = (int32_t)t;
        U += __popcll(m);
        kp = __shfl(kc, 63);
    }
    __syncthreads();   // unit starts visible to every lane
    QkdRegs r = qkd_fresh();
    int64_t tl = 0;
    if (lane < 4 + a.K)
        sam_rec(a, 0)[lane] = lane == 0 ? 0 : lane == 3 ? 0 : -1;
    a.nst = 1;
    if (U >= 2) {
        tl = st[U - 1];
        const int e = bend[s * bld + tl - 1];
        const int ml = blen[s * bld + tl - 1];
        WaveSam ws = {-2, -1};
        int se = 0;
        int kc = 0;
        for (int v0 = 0; v0 < U - 1; v0 += 64) {
            // the key symbols of units v0 .. v0+63, one per lane
            const int v = v0 + lane;
            const int kv = v < U - 1 ? qkd_symbol(p, p.k, p.ldk, s, st[v]) : 0;
            const int nv = min(64, U - 1 - v0);
            for (int i = 0; i < nv; ++i) {
                kc = __shfl(kv, i);
                sam_extend_wave(a, ws, kc);
                if (v0 + i == e)
                    se = a.tail;
            }
        }
        __syncthreads();   // the records visible to every lane
        sam_fill_last_wave(a, a.nst);
        // the fill's atomics are made in L2; invalidate this CU's L1 so that
        // the plain loads below and in qkd_steps see them
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "agent");
        __syncthreads();   // the last units before any read
        int ms = 0;
        if (ml > 0) {
            ms = se;
            for (;;) {
                const int lk = a.node(ms).y;
                if (lk < 0 || a.node(lk).x < ml)
                    break;
                ms = lk;
            }
        }
        r.u = U - 2;
        r.ms = ms;
        r.ml = ml;
        r.kprev = kc;
    }
    __syncthreads();   // the root record before any lane reads it
    qkd_steps(p, a, s, tl, T, r);
    qkd_save(p, a, s, r);
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
    v.meta = reinterpret_cast<int4 *>(base + l.meta);
    v.states = reinterpret_cast<int32_t *>(base + l.states);
    v.hist = base ? reinterpret_cast<uint8_t *>(base + l.hist) : nullptr;
    v.Ncap = l.Ncap;
    v.Hs = l.Hs;
    v.RSi = l.RS / 4;
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
                            int64_t T, hipStream_t st)
{
    SamView v = sam_view(buf, S, K, Tcap);
    hipLaunchKernelGGL(sam_build_kernel, dim3((unsigned)S), dim3(64), 0, st, v, S, T);
    return hipGetLastError();
}

// The batch retrieval's workspace inside a state buffer (valid until the
// automaton is built over it).
void *sam_match_ws(void *buf, int64_t S, int64_t K, int64_t Tcap,
                   size_t *bytes)
{
    const SamLayout l = sam_layout(S, K, Tcap);
    *bytes = l.ws_bytes;
    return reinterpret_cast<char *>(buf) + l.states;
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

QkdLayout qkd_layout(int64_t S, int64_t K, int64_t Tcap)
{
    QkdLayout l;
    l.Ncap = Tcap <= 1 ? 2 : 2 * Tcap - 1;
    l.RS = (int64_t)align_up((size_t)(16 + 4 * K), 64);
    size_t o = 0;
    l.flags = o;  o += 256;
    l.meta = o;   o = align_up(o + (size_t)S * 16, 256);
    l.mst = o;    o = align_up(o + (size_t)S * 32, 256);
    l.cfst = o;   o = align_up(o + (size_t)S * kQkdMaxBits * 8, 256);
    size_t rec = (size_t)S * l.Ncap * l.RS;
    const size_t ws = qk_layout(S, Tcap, K).total;
    l.ws_bytes = rec > ws ? rec : ws;
    l.states = o; o = align_up(o + l.ws_bytes, 256);
    l.start = o;  o = align_up(o + (size_t)S * Tcap * 4, 256);
    l.bscr = o;   o = align_up(o + (size_t)S * Tcap * 8, 256);
    l.total = o;
    return l;
}

hipError_t launch_qkd(const QkdParams &p, hipStream_t st)
{
    hipLaunchKernelGGL(qkd_kernel, dim3((unsigned)p.S), dim3(64), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_qkd_prefix(const QkdParams &p, const int32_t *bend,
                             const int32_t *blen, int64_t bld, hipStream_t st)
{
    hipLaunchKernelGGL(qkd_prefix_kernel, dim3((unsigned)p.S), dim3(64), 0, st, p,
                       bend, blen, bld);
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
hipError_t launch_qk_batch(const QkParams &p, hipStream_t st);

// The grouped-key kernels for every shape they take (alphabets of two
// symbols or more; they answer every stream themselves).  Otherwise the
// bit-parallel kernel when the streams fit it, then an automaton kernel for
// the streams it left (matches longer than its levels), or an automaton
// kernel for every stream.
hipError_t launch_qk(QkParams p, hipStream_t st)
{
    p.spw = 1;
    p.only = nullptr;
    {
        const hipError_t e = launch_qk_batch(p, st);
        if (e != hipErrorNotSupported)
            return e;
    }
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
