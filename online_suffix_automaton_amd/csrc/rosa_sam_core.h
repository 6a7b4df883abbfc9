// rosa_sam_core.h -- the online suffix automaton of one stream (append,
// match with the last-end walk, and the one-pass last ends after appends
// without walks).  Used by the kernels of rosa_sam.hip; the functions are
// also compiled for the host, where a CPU test runs them against the
// oracle.  Method: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix
// Matching" (arXiv 2602.02499), Sec. 2.2 (Blumer et al. 1985) and App. B.3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rosa {

// One stream's automaton: state v's node {len, link, last, clone flag} at
// nd[v * nds] and its K-wide transition row (-1 = none) at nx + v * nxs.
// The decode state interleaves them (node and row of a state in one
// record, so the append's chain touches one cache line per state); the
// query/key workspace keeps two arrays (nds = 1, nxs = K).
struct SamStream {
    int4 *nd;
    int32_t *nx;
    int64_t nds, nxs;
    int K;
    int tail, nst;
    int tail_len, tail_link;   // the tail state's length and suffix link
    __host__ __device__ int4 &node(int v) const { return nd[(int64_t)v * nds]; }
    __host__ __device__ int32_t *row(int v) const { return nx + (int64_t)v * nxs; }
};

__host__ __device__ inline int sam_new_state(SamStream &a, int len)
{
    const int v = a.nst++;
    a.node(v) = make_int4(len, -1, -1, 0);
    int32_t *row = a.row(v);
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

// Append symbol c; returns the new state.  The tail (the newest state) has
// no transition yet, so its row needs no read; its length and link are
// kept in the stream's registers rather than read back.
__host__ __device__ inline int sam_extend(SamStream &a, int c)
{
    const int cur = sam_new_state(a, a.tail_len + 1);
    a.row(a.tail)[c] = cur;
    int p = a.tail_link;
    while (p != -1 && a.row(p)[c] == -1) {
        a.row(p)[c] = cur;
        p = a.node(p).y;
    }
    int lk = 0;
    if (p != -1) {
        const int q = a.row(p)[c];
        const int4 nq = a.node(q);
        const int lp = a.node(p).x;
        if (lp + 1 == nq.x) {
            lk = q;
        } else {
            const int clone = a.nst++;
            a.node(clone) = make_int4(lp + 1, nq.y, nq.z, 1);
            const int32_t *src = a.row(q);
            int32_t *dst = a.row(clone);
            if ((a.K & 3) == 0) {
                const int4 *s4 = reinterpret_cast<const int4 *>(src);
                int4 *d4 = reinterpret_cast<int4 *>(dst);
                for (int k = 0; k < (a.K >> 2); ++k)
                    d4[k] = s4[k];
            } else {
                for (int k = 0; k < a.K; ++k)
                    dst[k] = src[k];
            }
            while (p != -1 && a.row(p)[c] == q) {
                a.row(p)[c] = clone;
                p = a.node(p).y;
            }
            a.node(q).y = clone;
            lk = clone;
        }
    }
    a.node(cur).y = lk;
    a.tail = cur;
    a.tail_len += 1;
    a.tail_link = lk;
    return cur;
}

// Match for position t after the extension, then the last-end update.
__host__ __device__ inline void sam_match(SamStream &a, int cur, int t,
                                          int &E, int &L)
{
    const int v = a.node(cur).y;
    E = -1;
    L = 0;
    if (v > 0) {
        const int4 nv = a.node(v);
        L = nv.x;
        E = nv.z;
    }
    for (int u = cur; u != -1; u = a.node(u).y)
        a.node(u).z = t;
}

// Last ends after appends made without the last-end walks (every last end
// still -1): non-clone states from the latest position down (a non-clone
// state of length n was created at position n-1); each sets its unset
// ancestors and stops at the first one already set, whose ancestors are
// all set (by a later position).
__host__ __device__ inline void sam_fill_last(SamStream &a)
{
    for (int w = a.nst - 1; w >= 1; --w) {
        const int4 nw = a.node(w);
        if (nw.w != 0 || nw.z != -1)
            continue;
        const int tw = nw.x - 1;
        a.node(w).z = tw;
        for (int u = nw.y; u != -1;) {
            const int4 nu = a.node(u);
            if (nu.z != -1)
                break;
            a.node(u).z = tw;
            u = nu.y;
        }
    }
}

}  // namespace rosa
