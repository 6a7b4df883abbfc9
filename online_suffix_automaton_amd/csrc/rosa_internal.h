// rosa_internal.h -- layouts and launch parameters shared by librosa's HIP
// sources.  Not part of the public ABI (that is include/rosa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rosa {

// Symbol rows in the match workspace carry zero padding on both sides so
// that 16-byte windows ending near position 0 or T-1 never leave the row.
constexpr int kPadFront = 64;
constexpr int kPadBack = 64;

// d-gram bucketing limits (per stream, held in LDS by the stream kernel).
constexpr int kMaxBuckets = 4096;    // K^d
constexpr int kMaxFirstTab = 2048;   // sum_{l=1}^{d-1} K^l
constexpr int kMaxD = 12;

constexpr int kStreamThreads = 1024; // one workgroup per stream
constexpr int kTaskCap = 4128;       // tasks per stream (<= kMaxBuckets)
constexpr int kBigThreads = 64;      // one wave per large group

// Flags word layout in the match workspace (first 256 bytes).
constexpr int kFlagSymbol = 0;       // int32: nonzero if a symbol >= K was seen

// Words of the per-stream bitmap of deferred positions (record mode).
inline __host__ __device__ int deep_words(int64_t T) { return (int)((T + 31) / 32); }

struct WsLayout {
    size_t flags, sym, pos, pos2, rec, big, stack, tasks, deep, dinfo, total;
    int64_t Tp;          // bytes per padded symbol row
    int64_t big_cap;     // entries in the large-group list
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline WsLayout ws_layout(int64_t S, int64_t T)
{
    WsLayout w;
    w.Tp = (int64_t)align_up((size_t)T + kPadFront + kPadBack, 256);
    w.big_cap = S * (T / 65 + 1);
    size_t o = 0;
    w.flags = o;  o += 256;
    w.sym = o;    o = align_up(o + (size_t)S * w.Tp, 256);
    w.pos = o;    o = align_up(o + (size_t)S * T * 4, 256);
    w.pos2 = o;   o = align_up(o + (size_t)S * T * 4, 256);
    w.rec = o;    o = align_up(o + (size_t)S * T * 4, 256);
    w.big = o;    o = align_up(o + 256 + (size_t)w.big_cap * 16, 256);
    w.stack = o;  o = align_up(o + (size_t)S * (T / 16 + 4) * 16, 256);
    w.tasks = o;  o = align_up(o + (size_t)S * kTaskCap * 4, 256);
    // deferred positions exist only in record mode (T <= 65536)
    const bool rec_mode = T <= 65536;
    w.deep = o;   o = align_up(o + (rec_mode ? (size_t)S * deep_words(T) * 4 : 0), 256);
    w.dinfo = o;  o = align_up(o + (rec_mode ? (size_t)S * T * 16 : 0), 256);
    w.total = o;
    return w;
}

// Parameters of the bucketing/solve kernels (passed by value).
struct MatchParams {
    const uint8_t *sym;  // padded rows: stream s at sym + s*Tp + kPadFront
    int64_t Tp;
    int32_t T, K, d, NB, nbits, fl_total;
    int32_t pw[kMaxD + 1];      // K^i
    int32_t fl_off[kMaxD + 1];  // first-occurrence table offset of level l
    int32_t *pos;               // [S][T] bucket-ordered positions
    int32_t *pos2;              // [S][T] second buffer for large groups
    int32_t *big;               // [0]: count; entries from +64: {s, key, start, n}
    int64_t big_cap;
    int4 *stack;                // [S][T/16+4] group stacks of the large-group pass
    uint32_t *rec;              // [S][T] result records (streams of <= 65536)
    uint32_t *tasks;            // [S][kTaskCap] task lists (LDS kernel)
    uint32_t *deep;             // [S][deep_words(T)] deferred positions (LDS kernel)
    uint4 *dinfo;               // [S][T] their candidates (LDS kernel)
    int32_t *E;                 // [S][T]
    int16_t *SYM;               // [S][T] or null
    int32_t *L;                 // [S][T] or null
};

// Choice of the bucketing depth d for alphabet K and stream length T: the
// largest d with K^d <= min(4096, T/8) (about 8+ positions per bucket on
// i.i.d. streams, so buckets fit a 64-lane wave) and first-occurrence tables
// for levels below d within kMaxFirstTab entries.
inline int choose_d(int64_t K, int64_t T)
{
    int64_t cap = T / 8;
    if (cap > kMaxBuckets) cap = kMaxBuckets;
    if (cap < K) cap = K;
    int d = 1;
    int64_t pw = K, fl = 0;
    while (d < kMaxD && d + 1 <= T) {
        int64_t nb_next = pw * K;
        int64_t fl_next = fl + pw;  // tables for levels 1..d
        if (nb_next > cap || fl_next > kMaxFirstTab) break;
        fl = fl_next;
        pw = nb_next;
        ++d;
    }
    return d;
}

// Parameters of the query/key automaton kernel (rosa_sam.hip).
struct QkParams {
    const uint8_t *q, *k;   // padded rows: stream s at + s*Tp + kPadFront
    int64_t Tp, S, T, Ncap;
    int32_t K, M, rle, spw;
    int4 *nodes;            // [S][Ncap] {len, link, last unit, 0}
    int32_t *next;          // [S][Ncap][K]
    int32_t *start;         // [S][T] start time of each unit
    int32_t *tau, *end, *len, *run_of, *run_start, *ridx, *cf_tau, *cf_ridx;
    int32_t *redo;          // [S] streams the bit-parallel kernel left to the automaton
    const int32_t *only;    // automaton kernels: when set, only streams with only[s] != 0
};


// Workspace of rosa_match_qk: flags, padded query and key rows, unit starts,
// the automaton nodes and dense transition rows.
struct QkLayout {
    size_t flags, qrows, krows, start, nodes, next, redo, total;
    int64_t Tp, Ncap;
};

inline QkLayout qk_layout(int64_t S, int64_t T, int64_t K)
{
    QkLayout l;
    l.Tp = (int64_t)align_up((size_t)T + kPadFront + kPadBack, 256);
    l.Ncap = T <= 1 ? 2 : 2 * T - 1;
    size_t o = 0;
    l.flags = o;  o += 256;
    l.qrows = o;  o = align_up(o + (size_t)S * l.Tp, 256);
    l.krows = o;  o = align_up(o + (size_t)S * l.Tp, 256);
    l.start = o;  o = align_up(o + (size_t)S * T * 4, 256);
    l.nodes = o;  o = align_up(o + (size_t)S * l.Ncap * 16, 256);
    l.next = o;   o = align_up(o + (size_t)S * l.Ncap * K * 4, 256);
    l.redo = o;   o = align_up(o + (size_t)S * 4, 256);
    l.total = o;
    return l;
}

// Parameters of the destination-scatter kernels (rosa_scatter.hip).
struct ScatterParams {
    const float *theta;     // [B][T][ldt]
    float *G;               // [B][T][ldg]
    const int32_t *end;     // [S][T], destination E+1 where E >= 0
    int64_t ldt, ldg, B, T, D, R, Tq, big_cap;
    int32_t M;
    int32_t *cnt;           // [S][T] counts, then fill cursors
    int32_t *off;           // [S][Tq] exclusive prefix, Tq = T + 1
    int32_t *list;          // [S][T] time steps grouped by destination
    int32_t *big;           // [0]: count; entries from +64: {s, tau}
};

struct ScatterLayout {
    size_t cnt, off, list, big, total;
    int64_t Tq, big_cap;
};

inline ScatterLayout scatter_layout(int64_t S, int64_t T)
{
    ScatterLayout l;
    l.Tq = T + 1;
    l.big_cap = S * (T / 65 + 1);
    size_t o = 0;
    l.cnt = o;   o = align_up(o + (size_t)S * T * 4, 256);
    l.off = o;   o = align_up(o + (size_t)S * l.Tq * 4, 256);
    l.list = o;  o = align_up(o + (size_t)S * T * 4, 256);
    l.big = o;   o = align_up(o + 256 + (size_t)l.big_cap * 8, 256);
    l.total = o;
    return l;
}

}  // namespace rosa
