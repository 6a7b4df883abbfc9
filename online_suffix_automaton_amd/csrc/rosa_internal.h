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

// Size of the fixed device array behind rosa_match_noalloc (the match
// workspace of 512 streams x 4096 positions, 69 MiB, fits).
constexpr size_t kNoAllocScratchBytes = (size_t)96 << 20;

// Flags word layout in the match workspace (first 256 bytes).
constexpr int kFlagSymbol = 0;       // int32: nonzero if a symbol >= K was seen
// When the stream kernel reads the caller's symbol rows itself, each of its
// workgroups stores its stream's symbol check into a slot (the int32 array
// right after the 256 header bytes) and workgroup 0 stores the slot count
// and kSlotMark into the header, so that no launch has to clear a flag
// first; every other path clears the whole header before it runs.
constexpr int kFlagSlots = 1;        // int32: number of per-stream slots
constexpr int kFlagSlotMark = 2;     // int32: kSlotMark when the slots are valid
constexpr int32_t kSlotMark = 0x534c4f54;

// Words of the per-stream bitmap of deferred positions (record mode).
inline __host__ __device__ int deep_words(int64_t T) { return (int)((T + 31) / 32); }

struct WsLayout {
    size_t flags, sflag, sym, pos, pos2, rec, big, stack, tasks, deep, dinfo, total;
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
    w.sflag = o;  o = align_up(o + (size_t)S * 4, 256);   // right after the header
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
    int32_t fuse;               // the stream kernel runs the time-ordered pass itself
                                // (1: in its union, 2: over its whole LDS)
    // stage 1: the stream kernel reads its symbols straight from bf16 hidden
    // states H [B][T][Hld] (M = 4, route r of batch row b = stream b*R + r),
    // writes the optional symbol copy and clears the flags itself.
    // stage 2: it reads the caller's symbol rows symin [S][symld] (16-byte
    // aligned), checks them against K and, unless it runs the time-ordered
    // pass itself, writes its padded row to sym_w for the later kernel.
    int32_t stage, R;
    const uint16_t *H;
    int64_t Hld;
    const uint8_t *symin;
    int64_t symld;
    uint8_t *sym_w;
    uint8_t *sym_copy;          // [S][T] or null
    int32_t *flags;
    int32_t *sflag;             // [S] per-stream symbol check slots, or null
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

// I[h > 0] on a bf16 bit pattern, as an integer range test: the positive
// non-NaN patterns are exactly 0x0001 (smallest subnormal) .. 0x7F80 (+inf).
__device__ __forceinline__ uint32_t bf16_is_pos(uint32_t h)
{
    return (h - 1u) < 0x7F80u ? 1u : 0u;
}

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
    // grouped-key kernels (rosa_qk_batch.hip); sizes in QkLayout
    uint8_t *qu, *ku;       // [S][Tp] unit query / key symbols (run folding), padded
    int32_t *nunit;         // [S] units of each stream (run folding)
    int32_t *ucnt;          // [S][G] run starts per segment
    int32_t *hcnt;          // [S][G][NB] keys per group and segment, then prefixes
    int32_t *koff;          // [S][NB + 1] first slot of each key group
    int2 *klist;            // [S][T] keys by group: {unit, packed history}
    int32_t *ptab;          // [S][FL][nch] latest key per short gram up to each chunk
    uint32_t *dfl;          // [S][T] query symbols of each unit left to the time-ordered pass
    int4 *eo;               // [S][T] (E, L, destination, 0) of each unit's own query symbol
    int2 *cfe;              // [S][T][M] (E, destination) of each unit's counterfactual symbols
    int32_t *uof;           // [S][T] unit of each time step (run folding)
    int32_t *dstream;       // [S] nonzero: the stream has units in dfl
    int2 *xl;               // [S][qbt_xcap(T)] (unit, first step) of output pieces left
    int32_t *xn;            // [S] entries in xl
};

// Output pieces per stream the grouped-key kernels may leave to their
// expansion kernel: 64 time steps each, one per unit at most beyond the
// pieces of the steps themselves.
inline __host__ __device__ int64_t qbt_xcap(int64_t T) { return T + T / 64 + 64; }

// Grouped-key q/k kernels: units per segment workgroup, key groups (K^d)
// and short-gram tables (sum of K^l over l < d) at most, deepest d.
constexpr int kQbtSeg = 4096;
constexpr int kQbtMaxNB = 16384;
constexpr int kQbtMaxFL = 1024;
constexpr int kQbtMaxD = 10;

// Group depth d for alphabet K and T units: the largest d with
// K^d <= min(16384, max(K, T/4)) (a few keys per group at least) whose short
// tables keep within kQbtMaxFL entries.
inline int qbt_choose_d(int64_t K, int64_t T)
{
    int64_t cap = T / 4;
    if (cap > kQbtMaxNB) cap = kQbtMaxNB;
    if (cap < K) cap = K;
    int d = 1;
    int64_t pw = K, fl = 0;
    while (d < kQbtMaxD) {
        const int64_t nb_next = pw * K, fl_next = fl + pw;
        if (nb_next > cap || fl_next > kQbtMaxFL) break;
        pw = nb_next;
        fl = fl_next;
        ++d;
    }
    return d;
}

// Entries per stream of the grouped-key list: T rounded up to even, so
// that entry pairs are 16-byte aligned.
inline __host__ __device__ int64_t qbt_kpitch(int64_t T) { return (T + 1) & ~(int64_t)1; }

struct QbtShape {
    int d;
    int64_t nb, fl, nseg, nch;  // K^d, sum_{l<d} K^l, ceil(T/kQbtSeg), ceil(T/64) -> x16
};

inline QbtShape qbt_shape(int64_t T, int64_t K)
{
    QbtShape q;
    q.d = qbt_choose_d(K, T);
    q.nb = 1;
    q.fl = 0;
    for (int l = 0; l < q.d; ++l) {
        if (l > 0) q.fl += q.nb;
        q.nb *= K;
    }
    q.nseg = (T + kQbtSeg - 1) / kQbtSeg;
    q.nch = ((T + 63) / 64 + 15) / 16 * 16;   // short-table row pitch, 64-byte rows
    return q;
}


// Workspace of rosa_match_qk: flags, padded query and key rows, unit starts,
// the automaton nodes and dense transition rows.
struct QkLayout {
    size_t flags, qrows, krows, start, nodes, next, redo, total;
    size_t qu, ku, nunit, ucnt, hcnt, koff, klist, ptab, dfl, eo, cfe, uof, dstream, xl, xn;
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
    const QbtShape q = qbt_shape(T, K);
    l.qu = o;     o = align_up(o + (size_t)S * l.Tp, 256);
    l.ku = o;     o = align_up(o + (size_t)S * l.Tp, 256);
    l.nunit = o;  o = align_up(o + (size_t)S * 4, 256);
    l.ucnt = o;   o = align_up(o + (size_t)S * q.nseg * 4, 256);
    l.hcnt = o;   o = align_up(o + (size_t)S * q.nseg * q.nb * 4, 256);
    l.koff = o;   o = align_up(o + (size_t)S * (q.nb + 1) * 4, 256);
    l.klist = o;  o = align_up(o + (size_t)S * qbt_kpitch(T) * 8, 256);
    l.ptab = o;   o = align_up(o + (size_t)S * q.fl * q.nch * 4, 256);
    l.dfl = o;    o = align_up(o + (size_t)S * T * 4, 256);
    l.eo = o;     o = align_up(o + (size_t)S * T * 16, 256);
    l.cfe = o;    o = align_up(o + (size_t)S * T * 8 * 8, 256);   // M <= 8
    l.uof = o;    o = align_up(o + (size_t)S * T * 4, 256);
    l.dstream = o; o = align_up(o + (size_t)S * 4, 256);
    l.xl = o;     o = align_up(o + (size_t)S * qbt_xcap(T) * 8, 256);
    l.xn = o;     o = align_up(o + (size_t)S * 4, 256);
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
    int32_t skip0;          // lists leave out t = 0 (the sum adds its term first)
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
