// rosa_api.hip -- the C-ABI of librosa (declared in include/rosa.h):
// argument validation, workspace/state layout and kernel launches on the
// caller's stream.  No device allocation, no implicit synchronisation.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>
#include <unordered_set>

#include "rosa.h"
#include "rosa_internal.h"
#include "rosa_qk_decode.h"

namespace rosa {
// rosa_stream_io.hip
hipError_t launch_prep_symbols(const uint8_t *in, int64_t ld, int64_t S,
                               int64_t T, int32_t K, uint8_t *rows, int64_t Tp,
                               uint8_t *copy_out, int32_t *flags,
                               hipStream_t st);
hipError_t launch_clear_flags(int32_t *flags, hipStream_t st,
                              int32_t *flags2 = nullptr);
hipError_t launch_discretize(const uint16_t *H, int64_t B, int64_t T,
                             int64_t D, int64_t ld, int M, uint8_t *rows,
                             int64_t row_stride, int64_t row_off,
                             uint8_t *copy_out, hipStream_t st,
                             int64_t pad_end = 0, int32_t *zero_a = nullptr,
                             int32_t *zero_b = nullptr);
hipError_t launch_gather(const uint16_t *V, int64_t B, int64_t T, int64_t D,
                         int64_t ldv, int M, const int32_t *E, uint16_t *out,
                         int64_t ldo, hipStream_t st);
// rosa_match.hip
hipError_t launch_stream(const MatchParams &p, int64_t S, hipStream_t st);
hipError_t launch_big(const MatchParams &p, int grid, hipStream_t st);
hipError_t launch_unpermute(const MatchParams &p, int64_t S, hipStream_t st);
bool stream_can_stage(int64_t T);
bool stream_uses_records(int64_t T);
// rosa_sam.hip
size_t sam_total_bytes(int64_t S, int64_t K, int64_t Tcap);
uint8_t *sam_hist_base(void *buf, int64_t S, int64_t K, int64_t Tcap,
                       int64_t *Hs);
int32_t *sam_flags(void *buf);
hipError_t launch_sam_hist(const uint8_t *in, int64_t ld, int64_t S, int64_t T,
                           int32_t K, void *buf, int64_t Tcap,
                           uint8_t *copy_out, hipStream_t st);
hipError_t launch_sam_build(void *buf, int64_t S, int64_t K, int64_t Tcap,
                            int64_t T, hipStream_t st);
void *sam_match_ws(void *buf, int64_t S, int64_t K, int64_t Tcap,
                   size_t *bytes);
hipError_t launch_sam_step(void *buf, int64_t S, int64_t K, int64_t Tcap,
                           int64_t t, int kind, const void *row, int64_t ld,
                           int64_t R, int M, const uint16_t *V, int64_t ldv,
                           int64_t ldv_b, int32_t *end, int16_t *sym,
                           uint16_t *out_row, int64_t ldo_b, hipStream_t st);
hipError_t launch_qk(QkParams p, hipStream_t st);
// rosa_scatter.hip
hipError_t launch_scatter(const ScatterParams &p, hipStream_t st);
}  // namespace rosa

using namespace rosa;

struct rosa_state {
    uint64_t magic;
    void *buf;
    size_t bytes;
    int64_t S, K, Tcap, len;
    int32_t kind, M;
    int64_t B, D, R;
    int32_t qk;      // 0: self-match (rosa_build), 1: query/key (rosa_build_qk)
    int32_t rle;     // query/key: ROSA_QK_RLE given at build
    int32_t cfbits;  // query/key: query bits of the counterfactual branches (0: none)
};

static const uint64_t kStateMagic = 0x524f53415354ull;  // "ROSAST"

// Live handles.  A handle is looked up here before it is dereferenced, so a
// freed, foreign or null pointer is rejected (ROSA_ERR_STATE; rosa_free
// ignores it) without reading its memory.
static std::mutex g_handles_mu;
static std::unordered_set<const rosa_state *> *g_handles = nullptr;

static bool handle_live(const rosa_state *h)
{
    if (!h)
        return false;
    std::lock_guard<std::mutex> lk(g_handles_mu);
    return g_handles && g_handles->count(h) != 0;
}

static bool handle_add(const rosa_state *h)
{
    std::lock_guard<std::mutex> lk(g_handles_mu);
    if (!g_handles) {
        g_handles = new (std::nothrow) std::unordered_set<const rosa_state *>();
        if (!g_handles)
            return false;
    }
    try {
        g_handles->insert(h);
    } catch (...) {
        return false;
    }
    return true;
}

static bool handle_remove(const rosa_state *h)
{
    std::lock_guard<std::mutex> lk(g_handles_mu);
    return g_handles && g_handles->erase(h) != 0;
}

static const int64_t kMaxT = (int64_t)1 << 26;
static const int64_t kMaxST = (int64_t)1 << 40;

namespace {

// Resolved shape of a rosa_input.
struct Shape {
    int kind;
    int64_t S, T, B, D, R, ld;
    int32_t M, K;
};

rosa_status resolve(const rosa_input *in, Shape *sh, bool allow_empty_T)
{
    if (!in)
        return ROSA_ERR_ARG;
    Shape s;
    memset(&s, 0, sizeof s);
    s.kind = in->kind;
    s.T = in->T;
    s.ld = in->ld;
    if (s.T < 0 || s.T >= kMaxT || (s.T == 0 && !allow_empty_T))
        return ROSA_ERR_ARG;
    if (in->kind == ROSA_IN_SYMBOLS) {
        if (in->K < 1 || in->K > 256 || in->S < 1)
            return ROSA_ERR_ARG;
        s.K = in->K;
        s.S = in->S;
        s.B = 1;
        s.R = s.S;
        s.M = 0;
        if (s.ld < s.T)
            return ROSA_ERR_ARG;
    } else if (in->kind == ROSA_IN_BF16) {
        if (in->M < 1 || in->M > 8 || in->B < 1 || in->D < in->M ||
            in->D % in->M != 0)
            return ROSA_ERR_ARG;
        s.M = in->M;
        s.K = 1 << in->M;
        s.B = in->B;
        s.D = in->D;
        s.R = in->D / in->M;
        s.S = s.B * s.R;
        if (s.ld < s.D)
            return ROSA_ERR_ARG;
    } else {
        return ROSA_ERR_ARG;
    }
    if (s.T > 0 && !in->data)
        return ROSA_ERR_ARG;
    if (s.S * (s.T > 0 ? s.T : 1) >= kMaxST)
        return ROSA_ERR_ARG;
    *sh = s;
    return ROSA_OK;
}

rosa_status hip_ok(hipError_t e) { return e == hipSuccess ? ROSA_OK : ROSA_ERR_HIP; }

#define ROSA_TRY(expr)                      \
    do {                                    \
        rosa_status _st = hip_ok(expr);     \
        if (_st != ROSA_OK)                 \
            return _st;                     \
    } while (0)

MatchParams match_params(const Shape &sh, char *ws, const WsLayout &w,
                         const rosa_out *out)
{
    MatchParams p;
    memset(&p, 0, sizeof p);
    p.sym = reinterpret_cast<const uint8_t *>(ws + w.sym);
    p.Tp = w.Tp;
    p.T = (int32_t)sh.T;
    p.K = sh.K;
    p.d = choose_d(sh.K, sh.T);
    int64_t pw = 1;
    for (int i = 0; i <= kMaxD; ++i) {
        p.pw[i] = (int32_t)(i <= p.d ? pw : 0);
        if (i < p.d)
            pw *= sh.K;
    }
    p.NB = p.pw[p.d];
    int nb = 0;
    while ((1 << nb) < sh.K)
        ++nb;
    p.nbits = nb;
    int fl = 0;
    for (int l = 0; l <= kMaxD; ++l) {
        p.fl_off[l] = fl;
        if (l >= 1 && l < p.d)
            fl += p.pw[l];
    }
    p.fl_total = fl;
    p.pos = reinterpret_cast<int32_t *>(ws + w.pos);
    p.pos2 = reinterpret_cast<int32_t *>(ws + w.pos2);
    p.big = reinterpret_cast<int32_t *>(ws + w.big);
    p.big_cap = w.big_cap;
    p.stack = reinterpret_cast<int4 *>(ws + w.stack);
    p.rec = sh.T <= 65536 ? reinterpret_cast<uint32_t *>(ws + w.rec) : nullptr;
    p.tasks = reinterpret_cast<uint32_t *>(ws + w.tasks);
    p.deep = reinterpret_cast<uint32_t *>(ws + w.deep);
    p.dinfo = reinterpret_cast<uint4 *>(ws + w.dinfo);
    p.E = out->end;
    p.SYM = out->sym;
    p.L = out->len;
    return p;
}

}  // namespace

extern "C" {

const char *rosa_error_string(rosa_status st)
{
    switch (st) {
    case ROSA_OK: return "ok";
    case ROSA_ERR_ARG: return "invalid argument";
    case ROSA_ERR_CAPACITY: return "insufficient workspace, state buffer or capacity";
    case ROSA_ERR_SYMBOL: return "input symbol outside [0, K)";
    case ROSA_ERR_HIP: return "HIP runtime error";
    case ROSA_ERR_STATE: return "invalid state handle";
    case ROSA_ERR_NOMEM: return "host memory allocation failed";
    }
    return "unknown status";
}

rosa_status rosa_discretize(const rosa_input *in, uint8_t *symbols,
                            int64_t ld, hipStream_t stream)
{
    Shape sh;
    rosa_status st = resolve(in, &sh, true);
    if (st != ROSA_OK)
        return st;
    if (sh.kind != ROSA_IN_BF16 || (sh.T > 0 && (!symbols || ld < sh.T)))
        return ROSA_ERR_ARG;
    if (sh.T == 0)
        return ROSA_OK;
    ROSA_TRY(launch_discretize(reinterpret_cast<const uint16_t *>(in->data), sh.B,
                               sh.T, sh.D, sh.ld, sh.M, symbols, ld, 0, nullptr,
                               stream));
    return ROSA_OK;
}

size_t rosa_match_workspace_bytes(int64_t S, int64_t T, int32_t K)
{
    if (S < 1 || T < 0 || T >= kMaxT || K < 1 || K > 256 ||
        S * (T > 0 ? T : 1) >= kMaxST)
        return 0;
    return ws_layout(S, T).total;
}

static rosa_status match_impl(const rosa_input *in, const rosa_out *out,
                              void *ws, size_t ws_bytes, hipStream_t stream,
                              hipEvent_t ev_begin, hipEvent_t ev_end)
{
    Shape sh;
    rosa_status st = resolve(in, &sh, true);
    if (st != ROSA_OK)
        return st;
    if (!out || (!out->end && sh.T > 0) || !ws ||
        (reinterpret_cast<uintptr_t>(ws) & 255) != 0)
        return ROSA_ERR_ARG;
    const WsLayout w = ws_layout(sh.S, sh.T);
    if (ws_bytes < w.total)
        return ROSA_ERR_CAPACITY;
    char *base = reinterpret_cast<char *>(ws);
    int32_t *flags = reinterpret_cast<int32_t *>(base + w.flags);
    if (sh.T == 0) {
        ROSA_TRY(launch_clear_flags(flags, stream));
        return ROSA_OK;
    }
    uint8_t *rows = reinterpret_cast<uint8_t *>(base + w.sym);
    MatchParams p = match_params(sh, base, w, out);
    // the flags and the large-group counter start at zero: cleared by a
    // launch of their own before a copy of the symbol rows, inside the
    // discretisation launch (bf16), or -- when the stream kernel reads the
    // caller's rows itself -- replaced by per-stream status slots that the
    // stream kernel always writes (no clear needed)
    if (sh.kind == ROSA_IN_SYMBOLS && !out->symbols && stream_uses_records(sh.T) &&
        sh.ld % 16 == 0 && (reinterpret_cast<uintptr_t>(in->data) & 15) == 0) {
        // 16-byte aligned rows of a stream of the LDS plans: the stream
        // kernel reads them itself (no copy into the workspace rows first)
        // and reports bad symbols in per-stream slots, so nothing is
        // cleared before it (the large-group counter is unused there)
        p.stage = 2;
        p.symin = reinterpret_cast<const uint8_t *>(in->data);
        p.symld = sh.ld;
        p.sym_w = rows;
        p.flags = flags;
        p.sflag = reinterpret_cast<int32_t *>(base + w.sflag);
    } else if (sh.kind == ROSA_IN_SYMBOLS) {
        ROSA_TRY(launch_clear_flags(flags, stream, p.big));
        ROSA_TRY(launch_prep_symbols(reinterpret_cast<const uint8_t *>(in->data),
                                     sh.ld, sh.S, sh.T, sh.K, rows, w.Tp,
                                     out->symbols, flags, stream));
    } else if (sh.M == 4 && sh.ld % 4 == 0 &&
               (reinterpret_cast<uintptr_t>(in->data) & 7) == 0 &&
               stream_can_stage(sh.T)) {
        // short streams: the stream kernel reads its symbols from the rows
        // itself (and clears the flags); no discretisation launch
        p.stage = 1;
        p.R = (int32_t)sh.R;
        p.H = reinterpret_cast<const uint16_t *>(in->data);
        p.Hld = sh.ld;
        p.sym_copy = out->symbols;
        p.flags = flags;
    } else {
        ROSA_TRY(launch_discretize(reinterpret_cast<const uint16_t *>(in->data),
                                   sh.B, sh.T, sh.D, sh.ld, sh.M, rows, w.Tp,
                                   kPadFront, out->symbols, stream, w.Tp, flags,
                                   p.big));
    }
    if (ev_begin)
        ROSA_TRY(hipEventRecord(ev_begin, stream));
    ROSA_TRY(launch_stream(p, sh.S, stream));
    if (ev_end)
        ROSA_TRY(hipEventRecord(ev_end, stream));
    int grid = (int)(w.big_cap < 1024 ? w.big_cap : 1024);
    if (grid < 1)
        grid = 1;
    ROSA_TRY(launch_big(p, grid, stream));
    ROSA_TRY(launch_unpermute(p, sh.S, stream));
    return ROSA_OK;
}

rosa_status rosa_match(const rosa_input *in, const rosa_out *out, void *ws,
                       size_t ws_bytes, hipStream_t stream)
{
    return match_impl(in, out, ws, ws_bytes, stream, nullptr, nullptr);
}

rosa_status rosa_match_timed(const rosa_input *in, const rosa_out *out,
                             void *ws, size_t ws_bytes, hipStream_t stream,
                             hipEvent_t ev_begin, hipEvent_t ev_end)
{
    if (!ev_begin || !ev_end)
        return ROSA_ERR_ARG;
    return match_impl(in, out, ws, ws_bytes, stream, ev_begin, ev_end);
}

// ------------------------------------------------- allocation-free match
//
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops, harnesses that forbid it): rosa_match with its
// workspace in a fixed device array of this library.  The array's name is a
// host-side stand-in in host code; its device address is looked up once per
// device with hipGetSymbolAddress and only that address is used.  Every call
// on a device shares the device's one array, which keeps the last call's
// contents (the launches clear what must start at zero): calls that overlap
// on one device, e.g. on two streams, race.

static_assert(kNoAllocScratchBytes == ROSA_NOALLOC_MAX_WORKSPACE_BYTES,
              "the header states the array's size");
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
constexpr int kScratchDevices = 64;
static void *g_scratch_ptr[kScratchDevices];

// Device address of `scratch` on the current device (null on a HIP error).
static void *scratch_ptr()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices)
        return nullptr;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

rosa_status rosa_match_noalloc(const rosa_input *in, const rosa_out *out,
                               hipStream_t stream)
{
    Shape sh;
    rosa_status st = resolve(in, &sh, true);
    if (st != ROSA_OK)
        return st;
    if (!out || (!out->end && sh.T > 0))
        return ROSA_ERR_ARG;
    if (ws_layout(sh.S, sh.T).total > kNoAllocScratchBytes)
        return ROSA_ERR_CAPACITY;
    void *ws = scratch_ptr();
    if (!ws)
        return ROSA_ERR_HIP;
    return match_impl(in, out, ws, kNoAllocScratchBytes, stream, nullptr, nullptr);
}

}  // extern "C"

namespace {

// Symbols of one input into padded rows (stride Tp, data at kPadFront).
rosa_status prep_rows(const Shape &sh, const rosa_input *in, uint8_t *rows,
                      int64_t Tp, int32_t *flags, hipStream_t stream)
{
    if (sh.kind == ROSA_IN_SYMBOLS) {
        ROSA_TRY(launch_prep_symbols(reinterpret_cast<const uint8_t *>(in->data),
                                     sh.ld, sh.S, sh.T, sh.K, rows, Tp, nullptr,
                                     flags, stream));
    } else {
        ROSA_TRY(launch_discretize(reinterpret_cast<const uint16_t *>(in->data),
                                   sh.B, sh.T, sh.D, sh.ld, sh.M, rows, Tp,
                                   kPadFront, nullptr, stream, Tp));
    }
    return ROSA_OK;
}

}  // namespace

namespace {

// Query bits of the counterfactual branches: M for bf16 inputs, log2 K for
// symbols when K is a power of two >= 2, else 0.
int qk_cf_bits(const Shape &sh)
{
    if (sh.kind != ROSA_IN_SYMBOLS)
        return sh.M;
    int M = 0;
    while ((1 << M) < sh.K)
        ++M;
    return (1 << M) == sh.K ? M : 0;
}

// The query/key retrieval over shapes already checked (T > 0): symbol rows
// into the workspace `ws` (layout qk_layout(S, T, K); a symbol >= K sets
// *fl), then the kernels.  M: query bits of the counterfactual tables.
rosa_status qk_impl(const Shape &sq, const Shape &sk, const rosa_input *q,
                    const rosa_input *k, int rle, int M, const rosa_qk_out *out,
                    void *ws, int32_t *fl, hipStream_t stream)
{
    const QkLayout l = qk_layout(sq.S, sq.T, sq.K);
    char *base = reinterpret_cast<char *>(ws);
    uint8_t *qrows = reinterpret_cast<uint8_t *>(base + l.qrows);
    uint8_t *krows = reinterpret_cast<uint8_t *>(base + l.krows);
    rosa_status st = prep_rows(sq, q, qrows, l.Tp, fl, stream);
    if (st != ROSA_OK)
        return st;
    st = prep_rows(sk, k, krows, l.Tp, fl, stream);
    if (st != ROSA_OK)
        return st;
    QkParams p;
    memset(&p, 0, sizeof p);
    p.q = qrows;
    p.k = krows;
    p.Tp = l.Tp;
    p.S = sq.S;
    p.T = sq.T;
    p.Ncap = l.Ncap;
    p.K = sq.K;
    p.M = M;
    p.rle = rle;
    p.nodes = reinterpret_cast<int4 *>(base + l.nodes);
    p.next = reinterpret_cast<int32_t *>(base + l.next);
    p.start = reinterpret_cast<int32_t *>(base + l.start);
    p.redo = reinterpret_cast<int32_t *>(base + l.redo);
    p.qu = reinterpret_cast<uint8_t *>(base + l.qu);
    p.ku = reinterpret_cast<uint8_t *>(base + l.ku);
    p.nunit = reinterpret_cast<int32_t *>(base + l.nunit);
    p.ucnt = reinterpret_cast<int32_t *>(base + l.ucnt);
    p.hcnt = reinterpret_cast<int32_t *>(base + l.hcnt);
    p.koff = reinterpret_cast<int32_t *>(base + l.koff);
    p.klist = reinterpret_cast<int2 *>(base + l.klist);
    p.ptab = reinterpret_cast<int32_t *>(base + l.ptab);
    p.dfl = reinterpret_cast<uint32_t *>(base + l.dfl);
    p.eo = reinterpret_cast<int4 *>(base + l.eo);
    p.cfe = reinterpret_cast<int2 *>(base + l.cfe);
    p.uof = reinterpret_cast<int32_t *>(base + l.uof);
    p.dstream = reinterpret_cast<int32_t *>(base + l.dstream);
    p.xl = reinterpret_cast<int2 *>(base + l.xl);
    p.xn = reinterpret_cast<int32_t *>(base + l.xn);
    p.tau = out->tau;
    p.end = out->end;
    p.len = out->len;
    p.run_of = out->run_of;
    p.run_start = out->run_start;
    p.ridx = out->ridx;
    p.cf_tau = out->cf_tau;
    p.cf_ridx = out->cf_ridx;
    ROSA_TRY(launch_qk(p, stream));
    return ROSA_OK;
}

// Pointers of a query/key decode state and the launch's input geometry.
QkdParams qkd_params(void *buf, int64_t S, int64_t K, int64_t Tcap,
                     const Shape &sh, const rosa_input *q, const rosa_input *k,
                     int rle, int cfbits)
{
    const QkdLayout l = qkd_layout(S, K, Tcap);
    char *base = reinterpret_cast<char *>(buf);
    QkdParams p;
    memset(&p, 0, sizeof p);
    p.flags = reinterpret_cast<int32_t *>(base + l.flags);
    p.meta = reinterpret_cast<int4 *>(base + l.meta);
    p.mst = reinterpret_cast<int4 *>(base + l.mst);
    p.cfst = reinterpret_cast<int2 *>(base + l.cfst);
    p.states = reinterpret_cast<int32_t *>(base + l.states);
    p.start = reinterpret_cast<int32_t *>(base + l.start);
    p.S = S;
    p.Ncap = l.Ncap;
    p.RSi = l.RS / 4;
    p.Ucap = Tcap;
    p.K = (int32_t)K;
    p.M = cfbits;
    p.rle = rle;
    p.kind = sh.kind;
    p.Min = sh.M;
    p.q = q->data;
    p.k = k->data;
    p.ldq = q->ld;
    p.ldk = k->ld;
    p.R = sh.R;
    p.Tin = sh.T;
    return p;
}

void qkd_outputs(QkdParams &p, const rosa_qk_out *out)
{
    if (!out)
        return;
    p.tau = out->tau;
    p.end = out->end;
    p.len = out->len;
    p.run_of = out->run_of;
    p.run_start = out->run_start;
    p.ridx = out->ridx;
    p.cf_tau = out->cf_tau;
    p.cf_ridx = out->cf_ridx;
}

}  // namespace

extern "C" {

size_t rosa_match_qk_workspace_bytes(int64_t S, int64_t T, int32_t K)
{
    if (S < 1 || T < 0 || T >= kMaxT || K < 1 || K > 256 ||
        S * (T > 0 ? T : 1) >= kMaxST)
        return 0;
    return qk_layout(S, T, K).total;
}

rosa_status rosa_match_qk(const rosa_input *q, const rosa_input *k,
                          int32_t flags, const rosa_qk_out *out, void *ws,
                          size_t ws_bytes, hipStream_t stream)
{
    Shape sq, sk;
    rosa_status st = resolve(q, &sq, true);
    if (st != ROSA_OK)
        return st;
    st = resolve(k, &sk, true);
    if (st != ROSA_OK)
        return st;
    if (sq.kind != sk.kind || sq.S != sk.S || sq.T != sk.T || sq.K != sk.K ||
        sq.B != sk.B || sq.D != sk.D || sq.M != sk.M)
        return ROSA_ERR_ARG;
    if ((flags & ~ROSA_QK_RLE) != 0 || !out || (!out->tau && sq.T > 0) || !ws ||
        (reinterpret_cast<uintptr_t>(ws) & 255) != 0)
        return ROSA_ERR_ARG;
    const int M = qk_cf_bits(sq);
    if ((out->cf_tau || out->cf_ridx) && M < 1)
        return ROSA_ERR_ARG;
    const QkLayout l = qk_layout(sq.S, sq.T, sq.K);
    if (ws_bytes < l.total)
        return ROSA_ERR_CAPACITY;
    int32_t *fl = reinterpret_cast<int32_t *>(reinterpret_cast<char *>(ws) + l.flags);
    ROSA_TRY(launch_clear_flags(fl, stream));
    if (sq.T == 0)
        return ROSA_OK;
    return qk_impl(sq, sk, q, k, (flags & ROSA_QK_RLE) ? 1 : 0, M, out, ws, fl,
                   stream);
}

size_t rosa_scatter_grad_workspace_bytes(int64_t S, int64_t T)
{
    if (S < 1 || T < 0 || T >= kMaxT || S * (T > 0 ? T : 1) >= kMaxST)
        return 0;
    return scatter_layout(S, T).total;
}

rosa_status rosa_scatter_grad(const float *theta, int64_t B, int64_t T,
                              int64_t D, int64_t ldt, int32_t M,
                              const int32_t *end, float *G, int64_t ldg,
                              void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (B < 1 || T < 0 || T >= kMaxT || M < 1 || M > 8 || D < M || D % M != 0 ||
        ldt < D || ldg < D || B * (D / M) * (T > 0 ? T : 1) >= kMaxST)
        return ROSA_ERR_ARG;
    if (T == 0)
        return ROSA_OK;
    if (!theta || !end || !G || !ws || (reinterpret_cast<uintptr_t>(ws) & 255) != 0)
        return ROSA_ERR_ARG;
    const int64_t S = B * (D / M);
    const ScatterLayout l = scatter_layout(S, T);
    if (ws_bytes < l.total)
        return ROSA_ERR_CAPACITY;
    char *base = reinterpret_cast<char *>(ws);
    ScatterParams p;
    memset(&p, 0, sizeof p);
    p.theta = theta;
    p.G = G;
    p.end = end;
    p.ldt = ldt;
    p.ldg = ldg;
    p.B = B;
    p.T = T;
    p.D = D;
    p.R = D / M;
    p.Tq = l.Tq;
    p.big_cap = l.big_cap;
    p.M = M;
    p.cnt = reinterpret_cast<int32_t *>(base + l.cnt);
    p.off = reinterpret_cast<int32_t *>(base + l.off);
    p.list = reinterpret_cast<int32_t *>(base + l.list);
    p.big = reinterpret_cast<int32_t *>(base + l.big);
    ROSA_TRY(launch_scatter(p, stream));
    return ROSA_OK;
}

rosa_status rosa_match_status(const void *ws, hipStream_t stream)
{
    if (!ws)
        return ROSA_ERR_ARG;
    if (hipStreamSynchronize(stream) != hipSuccess)
        return ROSA_ERR_HIP;
    // the header's symbol flag, and the per-stream slots right after the
    // header when the last call's stream kernel marked them valid
    int32_t h[3] = {0, 0, 0};
    if (hipMemcpy(h, ws, sizeof h, hipMemcpyDeviceToHost) != hipSuccess)
        return ROSA_ERR_HIP;
    if (h[kFlagSymbol])
        return ROSA_ERR_SYMBOL;
    if (h[kFlagSlotMark] == kSlotMark && h[kFlagSlots] > 0 && h[kFlagSlots] <= (1 << 24)) {
        const int32_t n = h[kFlagSlots];
        int32_t *slots = static_cast<int32_t *>(malloc((size_t)n * sizeof(int32_t)));
        if (!slots)
            return ROSA_ERR_NOMEM;
        const hipError_t e = hipMemcpy(slots, static_cast<const char *>(ws) + 256,
                                       (size_t)n * sizeof(int32_t),
                                       hipMemcpyDeviceToHost);
        bool bad = false;
        for (int32_t i = 0; i < n && e == hipSuccess; ++i)
            bad = bad || slots[i] != 0;
        free(slots);
        if (e != hipSuccess)
            return ROSA_ERR_HIP;
        if (bad)
            return ROSA_ERR_SYMBOL;
    }
    return ROSA_OK;
}

rosa_status rosa_gather(const uint16_t *V, int64_t B, int64_t T, int64_t D,
                        int64_t ldv, int32_t M, const int32_t *end,
                        uint16_t *out, int64_t ldo, hipStream_t stream)
{
    if (B < 1 || T < 0 || T >= kMaxT || M < 1 || M > 8 || D < M ||
        D % M != 0 || ldv < D || ldo < D)
        return ROSA_ERR_ARG;
    if (T == 0)
        return ROSA_OK;
    if (!V || !end || !out)
        return ROSA_ERR_ARG;
    ROSA_TRY(launch_gather(V, B, T, D, ldv, M, end, out, ldo, stream));
    return ROSA_OK;
}

size_t rosa_state_bytes(int64_t S, int32_t K, int64_t t_capacity)
{
    if (S < 1 || K < 1 || K > 256 || t_capacity < 1 || t_capacity >= kMaxT ||
        S * t_capacity >= kMaxST)
        return 0;
    return sam_total_bytes(S, K, t_capacity);
}

rosa_status rosa_build(const rosa_input *in, int64_t t_capacity,
                       void *state_buf, size_t state_bytes,
                       rosa_state **handle, const rosa_out *out,
                       hipStream_t stream)
{
    Shape sh;
    rosa_status st = resolve(in, &sh, true);
    if (st != ROSA_OK)
        return st;
    if (!handle || !state_buf || t_capacity < 1 || t_capacity < sh.T ||
        t_capacity >= kMaxT || (reinterpret_cast<uintptr_t>(state_buf) & 255))
        return ROSA_ERR_ARG;
    if (out && sh.T > 0 && !out->end)
        return ROSA_ERR_ARG;
    const size_t need = rosa_state_bytes(sh.S, sh.K, t_capacity);
    if (need == 0)
        return ROSA_ERR_ARG;
    if (state_bytes < need)
        return ROSA_ERR_CAPACITY;
    rosa_state *h = (rosa_state *)calloc(1, sizeof(rosa_state));
    if (!h)
        return ROSA_ERR_NOMEM;
    if (!handle_add(h)) {
        free(h);
        return ROSA_ERR_NOMEM;
    }
    int32_t *flags = sam_flags(state_buf);
    hipError_t e = launch_clear_flags(flags, stream);
    int64_t Hs = 0;
    uint8_t *hist = sam_hist_base(state_buf, sh.S, sh.K, t_capacity, &Hs);
    if (e == hipSuccess && sh.T > 0) {
        if (sh.kind == ROSA_IN_SYMBOLS)
            e = launch_sam_hist(reinterpret_cast<const uint8_t *>(in->data),
                                sh.ld, sh.S, sh.T, sh.K, state_buf, t_capacity,
                                out ? out->symbols : nullptr, stream);
        else
            e = launch_discretize(reinterpret_cast<const uint16_t *>(in->data),
                                  sh.B, sh.T, sh.D, sh.ld, sh.M, hist, Hs, 0,
                                  out ? out->symbols : nullptr, stream);
    }
    // the prefix's outputs come from the batch retrieval over the history
    // rows (already clamped to [0, K)), with its workspace in the region
    // the automaton is built in next
    rosa_status ms = ROSA_OK;
    if (e == hipSuccess && sh.T > 0 && out) {
        size_t wsb = 0;
        void *ws = sam_match_ws(state_buf, sh.S, sh.K, t_capacity, &wsb);
        rosa_input hin;
        memset(&hin, 0, sizeof hin);
        hin.kind = ROSA_IN_SYMBOLS;
        hin.K = (int32_t)sh.K;
        hin.S = sh.S;
        hin.T = sh.T;
        hin.ld = Hs;
        hin.data = hist;
        rosa_out o2 = *out;
        o2.symbols = nullptr;   // written with the history rows
        ms = match_impl(&hin, &o2, ws, wsb, stream, nullptr, nullptr);
    }
    if (e == hipSuccess && ms == ROSA_OK)
        e = launch_sam_build(state_buf, sh.S, sh.K, t_capacity, sh.T, stream);
    if (e != hipSuccess || ms != ROSA_OK) {
        handle_remove(h);
        free(h);
        return ms != ROSA_OK ? ms : ROSA_ERR_HIP;
    }
    h->magic = kStateMagic;
    h->buf = state_buf;
    h->bytes = state_bytes;
    h->S = sh.S;
    h->K = sh.K;
    h->Tcap = t_capacity;
    h->len = sh.T;
    h->kind = sh.kind;
    h->M = sh.M;
    h->B = sh.B;
    h->D = sh.D;
    h->R = sh.R;
    *handle = h;
    return ROSA_OK;
}

rosa_status rosa_step(rosa_state *h, const rosa_input *row, const uint16_t *V,
                      int64_t ldv, int64_t ldv_b, int32_t *end, int16_t *sym,
                      uint16_t *out_row, int64_t ldo_b, hipStream_t stream)
{
    if (!handle_live(h))
        return ROSA_ERR_STATE;
    if (h->qk)
        return ROSA_ERR_ARG;
    Shape sh;
    rosa_status st = resolve(row, &sh, false);
    if (st != ROSA_OK)
        return st;
    if (sh.T != 1 || sh.kind != h->kind || sh.S != h->S || sh.K != h->K ||
        (sh.kind == ROSA_IN_BF16 && (sh.B != h->B || sh.D != h->D || sh.M != h->M)))
        return ROSA_ERR_ARG;
    if (!end)
        return ROSA_ERR_ARG;
    if (out_row) {
        const int64_t D = sh.kind == ROSA_IN_BF16 ? sh.D : 0;
        if (sh.kind != ROSA_IN_BF16 || !V || ldv < D || ldo_b < D ||
            (h->B > 1 && ldv_b < ldv * (h->len + 1)))
            return ROSA_ERR_ARG;
    }
    if (h->len >= h->Tcap)
        return ROSA_ERR_CAPACITY;
    const int64_t ld = sh.kind == ROSA_IN_SYMBOLS ? sh.ld : sh.ld;
    hipError_t e = launch_sam_step(h->buf, h->S, h->K, h->Tcap, h->len, sh.kind,
                                   row->data, ld, h->R, h->M, V, ldv, ldv_b, end,
                                   sym, out_row, ldo_b, stream);
    if (e != hipSuccess)
        return ROSA_ERR_HIP;
    h->len += 1;
    return ROSA_OK;
}

size_t rosa_qk_state_bytes(int64_t S, int32_t K, int64_t t_capacity)
{
    if (S < 1 || K < 1 || K > 256 || t_capacity < 1 || t_capacity >= kMaxT ||
        S * t_capacity >= kMaxST)
        return 0;
    return qkd_layout(S, K, t_capacity).total;
}

rosa_status rosa_build_qk(const rosa_input *q, const rosa_input *k,
                          int32_t flags, int64_t t_capacity, void *state_buf,
                          size_t state_bytes, rosa_state **handle,
                          const rosa_qk_out *out, hipStream_t stream)
{
    Shape sq, sk;
    rosa_status st = resolve(q, &sq, true);
    if (st != ROSA_OK)
        return st;
    st = resolve(k, &sk, true);
    if (st != ROSA_OK)
        return st;
    if (sq.kind != sk.kind || sq.S != sk.S || sq.T != sk.T || sq.K != sk.K ||
        sq.B != sk.B || sq.D != sk.D || sq.M != sk.M)
        return ROSA_ERR_ARG;
    if ((flags & ~ROSA_QK_RLE) != 0 || !handle || !state_buf ||
        t_capacity < 1 || t_capacity < sq.T || t_capacity >= kMaxT ||
        (reinterpret_cast<uintptr_t>(state_buf) & 255))
        return ROSA_ERR_ARG;
    const int cfbits = qk_cf_bits(sq);
    if (out && ((sq.T > 0 && !out->tau) ||
                ((out->cf_tau || out->cf_ridx) && cfbits < 1)))
        return ROSA_ERR_ARG;
    const size_t need = rosa_qk_state_bytes(sq.S, sq.K, t_capacity);
    if (need == 0)
        return ROSA_ERR_ARG;
    if (state_bytes < need)
        return ROSA_ERR_CAPACITY;
    rosa_state *h = (rosa_state *)calloc(1, sizeof(rosa_state));
    if (!h)
        return ROSA_ERR_NOMEM;
    if (!handle_add(h)) {
        free(h);
        return ROSA_ERR_NOMEM;
    }
    const int rle = (flags & ROSA_QK_RLE) ? 1 : 0;
    QkdParams p = qkd_params(state_buf, sq.S, sq.K, t_capacity, sq, q, k, rle,
                             cfbits);
    p.init = 1;
    p.t0 = 0;
    p.n = sq.T;
    p.ostride = sq.T;
    qkd_outputs(p, out);
    hipError_t e = launch_clear_flags(p.flags, stream);
    rosa_status bs = ROSA_OK;
    // Prefixes of two steps or more: the batch retrieval gives every time
    // step's E and L (and the caller's outputs), the automaton is built by
    // whole-wave appends, and only the last key run is walked in time order
    // (qkd_prefix_kernel).  Otherwise, or for alphabets over 60 symbols, the
    // whole prefix is walked in time order.
    const QkdLayout l = qkd_layout(sq.S, sq.K, t_capacity);
    const bool fast = sq.T >= 2 && sq.K <= 60 &&
                      qk_layout(sq.S, sq.T, sq.K).total <= l.ws_bytes;
    if (e == hipSuccess && fast) {
        char *base = reinterpret_cast<char *>(state_buf);
        int32_t *bscr = reinterpret_cast<int32_t *>(base + l.bscr);
        rosa_qk_out o2;
        memset(&o2, 0, sizeof o2);
        if (out)
            o2 = *out;
        if (!o2.tau)
            o2.tau = p.start;   // not read; the unit starts overwrite it
        if (!o2.end)
            o2.end = bscr;
        if (!o2.len)
            o2.len = bscr + sq.S * sq.T;
        bs = qk_impl(sq, sk, q, k, rle, cfbits, &o2, base + l.states, p.flags,
                     stream);
        if (bs == ROSA_OK)
            e = launch_qkd_prefix(p, o2.end, o2.len, sq.T, stream);
    } else if (e == hipSuccess) {
        e = launch_qkd(p, stream);
    }
    if (e != hipSuccess || bs != ROSA_OK) {
        handle_remove(h);
        free(h);
        return bs != ROSA_OK ? bs : ROSA_ERR_HIP;
    }
    h->magic = kStateMagic;
    h->buf = state_buf;
    h->bytes = state_bytes;
    h->S = sq.S;
    h->K = sq.K;
    h->Tcap = t_capacity;
    h->len = sq.T;
    h->kind = sq.kind;
    h->M = sq.M;
    h->B = sq.B;
    h->D = sq.D;
    h->R = sq.R;
    h->qk = 1;
    h->rle = rle;
    h->cfbits = cfbits;
    *handle = h;
    return ROSA_OK;
}

rosa_status rosa_step_qk(rosa_state *h, const rosa_input *q_row,
                         const rosa_input *k_row, const rosa_qk_out *out,
                         hipStream_t stream)
{
    if (!handle_live(h))
        return ROSA_ERR_STATE;
    if (!h->qk)
        return ROSA_ERR_ARG;
    Shape sq, sk;
    rosa_status st = resolve(q_row, &sq, false);
    if (st != ROSA_OK)
        return st;
    st = resolve(k_row, &sk, false);
    if (st != ROSA_OK)
        return st;
    for (const Shape *sh : {&sq, &sk})
        if (sh->T != 1 || sh->kind != h->kind || sh->S != h->S || sh->K != h->K ||
            (sh->kind == ROSA_IN_BF16 &&
             (sh->B != h->B || sh->D != h->D || sh->M != h->M)))
            return ROSA_ERR_ARG;
    if (!out || !out->tau || out->run_start ||
        ((out->cf_tau || out->cf_ridx) && h->cfbits < 1))
        return ROSA_ERR_ARG;
    if (h->len >= h->Tcap)
        return ROSA_ERR_CAPACITY;
    QkdParams p = qkd_params(h->buf, h->S, h->K, h->Tcap, sq, q_row, k_row,
                             h->rle, h->cfbits);
    p.init = 0;
    p.t0 = h->len;
    p.n = 1;
    p.ostride = 1;
    qkd_outputs(p, out);
    if (launch_qkd(p, stream) != hipSuccess)
        return ROSA_ERR_HIP;
    h->len += 1;
    return ROSA_OK;
}

int64_t rosa_state_length(const rosa_state *h)
{
    if (!handle_live(h))
        return -1;
    return h->len;
}

rosa_status rosa_state_status(rosa_state *h, hipStream_t stream)
{
    if (!handle_live(h))
        return ROSA_ERR_STATE;
    if (hipStreamSynchronize(stream) != hipSuccess)
        return ROSA_ERR_HIP;
    int32_t f = 0;
    if (hipMemcpy(&f, sam_flags(h->buf), sizeof f, hipMemcpyDeviceToHost) !=
        hipSuccess)
        return ROSA_ERR_HIP;
    return f ? ROSA_ERR_SYMBOL : ROSA_OK;
}

void rosa_free(rosa_state *h)
{
    // the registry decides, so a double free never reads the freed handle
    if (!handle_remove(h))
        return;
    h->magic = 0;
    free(h);
}

}  // extern "C"
