/*
 * rosa.h -- C-ABI of librosa: ROSA retrieval (online suffix-automaton
 * longest-suffix matching over many independent symbol streams) on AMD
 * Instinct MI355X (gfx950).
 *
 * Method: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix Matching"
 * (Zheng, Wang, Ren, Chen; arXiv 2602.02499).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates device memory; scratch comes from a caller
 *    workspace (rosa_match, rosa_match_qk, rosa_scatter_grad) or a caller
 *    state buffer (rosa_build/rosa_step, rosa_build_qk/rosa_step_qk).
 *    The one exception is the fixed device array behind rosa_match_noalloc,
 *    which the HIP runtime places on each device the library runs on.
 *  - Every call only enqueues work on the caller's `stream` and returns; no
 *    implicit device synchronisation, no internal streams.  The exceptions,
 *    which synchronise `stream`, are rosa_match_status and rosa_state_status.
 *  - Errors found on the host (ROSA_ERR_ARG, ROSA_ERR_CAPACITY,
 *    ROSA_ERR_STATE, ROSA_ERR_NOMEM) are returned before anything is
 *    enqueued, so no output has been written.  ROSA_ERR_HIP means a HIP call
 *    failed (a launch or an event record): work of the same call enqueued
 *    before it may still run, and the outputs of that call are unspecified.
 *  - Streams: stream s = b*R + r with R = D/M routes per batch row (Sec. 4.1:
 *    one symbol stream per (b, r) pair).  Time is 0-based.  Per-stream outputs
 *    are laid out [S][T], contiguous in t.
 *  - Outputs per position t of stream x (Sec. 3.3 and App. B.3; the body of
 *    Eq. (16) is lost from the page text and is read as follows):
 *        L(t)   length of the longest suffix of x[0..t] that also ends at
 *               some earlier position e < t (0 if none);
 *        E(t)   the largest such e, i.e. the most recent earlier occurrence
 *               ("endpos" of the hit), or -1;
 *        SYM(t) x[E+1], the symbol that followed that occurrence, or -1;
 *        tau(t) = E+1, the retrieval destination read by the value gather
 *               (App. C.4), or -1.
 *    These values are unique, so results are bit-exact and independent of
 *    launch geometry.
 *  - Causality of the destination.  The self-match (rosa_match, rosa_build,
 *    rosa_step) gives tau = E+1 <= t: tau = t happens when the previous
 *    position is the latest occurrence (E = t-1), and row t of the values
 *    is then read at position t.  The page states the range of Eq. (16) as
 *    tau <= t-1, which its run-length folding guarantees (adjacent runs
 *    differ); without folding that range does not hold.  rosa_match_qk
 *    applies the strict-past rule as a mask (tau = -1 unless tau < t); a
 *    self-match caller that needs it sets tau = -1 where E = t-1.
 */
#ifndef ROSA_H
#define ROSA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rosa_status {
    ROSA_OK = 0,
    ROSA_ERR_ARG = 1,      /* null pointer, bad size, shape or range        */
    ROSA_ERR_CAPACITY = 2, /* workspace/state buffer too small, or a step
                              past the capacity given to rosa_build         */
    ROSA_ERR_SYMBOL = 3,   /* an input symbol >= K was seen (reported by
                              rosa_match_status / rosa_state_status)        */
    ROSA_ERR_HIP = 4,      /* a HIP runtime call failed                     */
    ROSA_ERR_STATE = 5,    /* null, freed or foreign state handle           */
    ROSA_ERR_NOMEM = 6     /* a host memory allocation failed               */
} rosa_status;

/* Input kinds. */
enum {
    /* uint8 symbols [S][ld] (ld >= T, in bytes), values in [0, K). */
    ROSA_IN_SYMBOLS = 0,
    /* bf16 hidden states [B][T][ld] as raw 16-bit patterns (ld >= D, in
     * elements).  Sec. 3.2, Eq. (10)-(15): channel c = r*M + j gives the
     * bit I[h > 0] (+0, -0 and NaN give 0; +inf and positive subnormals
     * give 1), route r packs its M bits with weight 2^j, K = 2^M. */
    ROSA_IN_BF16 = 1
};

typedef struct rosa_input {
    int32_t kind;      /* ROSA_IN_SYMBOLS or ROSA_IN_BF16                    */
    int32_t M;         /* BF16: bits per symbol, 1..8, D % M == 0            */
    int32_t K;         /* SYMBOLS: alphabet size 1..256; BF16: ignored (2^M) */
    int32_t reserved;
    const void *data;  /* device pointer                                      */
    int64_t S;         /* SYMBOLS: number of streams; BF16: ignored (B*D/M)  */
    int64_t T;         /* positions per stream                                */
    int64_t B, D;      /* BF16 only: batch rows and channels                  */
    int64_t ld;        /* row stride: bytes per stream (SYMBOLS) or elements
                          per position (BF16)                                 */
} rosa_input;

typedef struct rosa_out {
    int32_t *end;      /* [S][T] E, required                                  */
    int16_t *sym;      /* [S][T] SYM, may be NULL                             */
    int32_t *len;      /* [S][T] L, may be NULL                               */
    uint8_t *symbols;  /* [S][T] the packed input symbols, may be NULL        */
} rosa_out;

/* --------------------------------------------------------------- symbols */

/* Sec. 3.2, Eq. (10)-(15): the symbols of a bf16 input alone, the first
 * step of rosa_match (bit j = I[h > 0] of channel r*M + j, packed with
 * weight 2^j): symbols[s*ld + t] for stream s = b*R + r and t < T.  `in`:
 * kind ROSA_IN_BF16.  `symbols`: device bytes, rows of ld >= T.  Every
 * symbol is < 2^M, so rosa_match over these rows (ROSA_IN_SYMBOLS, K = 2^M)
 * gives the same outputs as over the bf16 input.  A caller that pipelines
 * the path over parts of the streams (for instance one part's retrieval
 * beside another part's gather, on two streams) can run this step apart
 * from the retrieval.  With M = 4, rows whose pitch is a multiple of 16
 * bytes at a 16-byte aligned address take a kernel that uses no LDS, so it
 * can run on the same CUs as a retrieval kernel (which holds their LDS). */
rosa_status rosa_discretize(const rosa_input *in, uint8_t *symbols,
                            int64_t ld, hipStream_t stream);

/* ------------------------------------------------------------ batch match */

/* Bytes of device workspace rosa_match needs for S streams of T positions
 * over an alphabet of K symbols.  0 on bad arguments. */
size_t rosa_match_workspace_bytes(int64_t S, int64_t T, int32_t K);

/* Sec. 3.3 / Sec. 4.1: for every stream and every position t, L, E and SYM
 * as defined above, for all S*T positions at once.  `in` gives the symbols
 * (or the bf16 hidden states, discretised on the device first); `out->end`
 * is required, the other outputs are optional.  `ws` is a device workspace
 * of at least rosa_match_workspace_bytes(S, T, K) bytes, 256-byte aligned;
 * it must not be shared by calls in flight at the same time.  Limits:
 * 1 <= T < 2^26, S*T < 2^40.  A symbol >= K sets a sticky flag in `ws`
 * (read it with rosa_match_status); the outputs of that call are then
 * unspecified.  No device memory is read outside the given buffers.
 * Symbol rows with T <= 65536, a pitch that is a multiple of 16 bytes and a
 * 16-byte aligned address (and no packed-symbol copy requested) are read by
 * the retrieval kernel itself; other symbol rows are first copied into the
 * workspace by a kernel of their own. */
rosa_status rosa_match(const rosa_input *in, const rosa_out *out, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/* Same as rosa_match, and also records `ev_begin` on `stream` just before
 * the retrieval kernel (per-stream bucketing and group refinement) and
 * `ev_end` just after it, so a caller can time that kernel alone with
 * hipEventElapsedTime.  Both events must be valid (ROSA_ERR_ARG otherwise). */
rosa_status rosa_match_timed(const rosa_input *in, const rosa_out *out,
                             void *ws, size_t ws_bytes, hipStream_t stream,
                             hipEvent_t ev_begin, hipEvent_t ev_end);

/* Synchronises `stream`, then returns ROSA_ERR_SYMBOL if the last rosa_match
 * that used `ws` saw a symbol >= K, else ROSA_OK (or ROSA_ERR_HIP, or
 * ROSA_ERR_NOMEM if the host buffer for the per-stream status words cannot
 * be allocated).  It reads the workspace's 256-byte header and, when the
 * last call's retrieval kernel checked the symbols itself (16-byte aligned
 * symbol rows), one status word per stream after it. */
rosa_status rosa_match_status(const void *ws, hipStream_t stream);

/* Size of the fixed device array rosa_match_noalloc works in. */
#define ROSA_NOALLOC_MAX_WORKSPACE_BYTES ((size_t)96 << 20)

/* For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): rosa_match with no
 * workspace argument.  The workspace is a fixed array of
 * ROSA_NOALLOC_MAX_WORKSPACE_BYTES in the library, one per device, held
 * until the process ends; inputs and outputs are the caller's, as for
 * rosa_match.  Shapes whose rosa_match_workspace_bytes(S, T, K) exceeds
 * that size give ROSA_ERR_CAPACITY (512 streams of 4096 positions fit).
 * The call makes no allocation of any kind.  Every call on a device shares
 * that device's array: calls that overlap on one device (e.g. on two
 * streams) race, and rosa_match_status does not apply (a symbol >= K still
 * leaves the outputs unspecified). */
rosa_status rosa_match_noalloc(const rosa_input *in, const rosa_out *out,
                               hipStream_t stream);

/* --------------------------------------------------- query / key retrieval */

/* Flags of rosa_match_qk. */
enum {
    /* Fold the key stream into runs of equal adjacent symbols (Sec. 3.3, the
     * run-length paragraph; App. C.6): the automaton and the matching state
     * move once per run, at its first time step. */
    ROSA_QK_RLE = 1
};

typedef struct rosa_qk_out {
    int32_t *tau;       /* [S][T] destination time, -1 if none; required      */
    int32_t *end;       /* [S][T] end unit e of the match, -1; may be NULL      */
    int32_t *len;       /* [S][T] match length in units; may be NULL            */
    int32_t *run_of;    /* [S][T] unit of each time step; may be NULL           */
    int32_t *run_start; /* [S][T] first time of unit u (u < number of units),
                           -1 for the remaining entries; may be NULL            */
    int32_t *ridx;      /* [S][T] destination unit e+1 where tau >= 0, else -1;
                           may be NULL                                          */
    int32_t *cf_tau;    /* [S][T][M][2] counterfactual destinations; may be NULL */
    int32_t *cf_ridx;   /* [S][T][M][2] their destination units; may be NULL    */
} rosa_qk_out;

/* Bytes of device workspace rosa_match_qk needs (0 on bad arguments). */
size_t rosa_match_qk_workspace_bytes(int64_t S, int64_t T, int32_t K);

/* Sec. 3.3 with a query stream q and a key stream k (k_{1:t} = a^(k),
 * q_{1:t} = a^(q)), one suffix automaton per stream over the key units and
 * one matching state advanced by the query units.
 *   Units: time steps; with ROSA_QK_RLE the maximal runs of equal adjacent
 *   key symbols, whose key symbol is the run's symbol and whose query
 *   symbol is q at the run's first time step.
 *   At unit u the match is the longest suffix of the query units 0..u that
 *   occurs in the key units 0..u-1 (strictly earlier); e is the most recent
 *   unit at which it ends.  For every time t of unit u,
 *     tau(t) = first time of unit e+1  if a match exists and that time is
 *              < t (the read position is strictly from the past, Eq. (16)),
 *     tau(t) = -1 otherwise.
 *   With q = k and no folding, end/len equal rosa_match's E/L.
 *   Counterfactual tables (App. C.5, C.6; Sec. 4.2 step 3): entry [t][j][v]
 *   is tau (or the destination unit) when bit j of the unit's query symbol
 *   is forced to v and one matching update is made from the same state;
 *   they need K = 2^M (bf16 inputs: M; symbols: K a power of two >= 2),
 *   else ROSA_ERR_ARG.
 * q and k: same kind and shape (S, T, K; B, D, M for bf16), each laid out
 * as for rosa_match.  `ws`: at least rosa_match_qk_workspace_bytes(S, T, K)
 * bytes, 256-byte aligned, not shared by calls in flight; its first 256
 * bytes hold the symbol flag, so rosa_match_status(ws, stream) reports a
 * symbol >= K in q or k.
 * Kernels (the same results whichever runs): for K >= 2, the key units
 * sorted by their last d symbols into groups, one thread per query unit
 * comparing the packed histories of its group's earlier keys (and, below d
 * symbols, tables of the latest key per shorter gram), for the unit's own
 * and every counterfactual symbol; symbols whose group is very large or
 * whose match runs more than 1024 units past d are answered in time order
 * by the extension rule.  For K = 1, a bit-parallel kernel (at most 4096
 * units) or one wave per stream walking the pages' automaton. */
rosa_status rosa_match_qk(const rosa_input *q, const rosa_input *k,
                          int32_t flags, const rosa_qk_out *out, void *ws,
                          size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ value gather */

/* App. C.4 read-out with the validity mask of Eq. (17):
 *   out[b][t][r*M+m] = V[b][E[s][t]+1][r*M+m]  if E[s][t] >= 0, else 0x0000,
 * for s = b*R + r, m < M.  A bit copy of bf16 patterns (NaN payloads and -0
 * kept).  V: [B][T][ldv], out: [B][T][ldo] (elements), E: [S][T] with every
 * value in [-1, T-2] (as rosa_match produces; other values give ROSA-
 * unspecified output but no out-of-bounds access: E is clamped on device). */
rosa_status rosa_gather(const uint16_t *V, int64_t B, int64_t T, int64_t D,
                        int64_t ldv, int32_t M, const int32_t *end,
                        uint16_t *out, int64_t ldo, hipStream_t stream);

/* ---------------------------------------- destination scatter (gradient) */

/* Bytes of device workspace rosa_scatter_grad needs for S = B*D/M streams of
 * T positions (0 on bad arguments). */
size_t rosa_scatter_grad_workspace_bytes(int64_t S, int64_t T);

/* App. C.4 (destination-scatter aggregation), the transpose of rosa_gather:
 *   G[b][tau][r*M+m] = sum over t of theta[b][t][r*M+m] * I[E[s][t]+1 == tau]
 * for s = b*R + r, m < M; rows no time step points at get 0.  Entries with
 * E < 0 or E+1 >= T add nothing.  theta, G: float [B][T][ldt] / [B][T][ldg]
 * (ld >= D, in elements); E: int32 [S][T] (rosa_match's `end`; for
 * rosa_match_qk pass tau - 1).  The sum over t runs in increasing t in
 * double precision and is rounded to float once: the result is
 * deterministic and independent of launch geometry.  Cost: a counting sort
 * of the time steps by destination per stream, then one thread per
 * (row, route) walking its few time steps in order; a destination with more
 * than 64 time steps is summed by one wave scanning the stream's E row.
 * `ws`: rosa_scatter_grad_workspace_bytes(B*D/M, T) bytes, 256-byte aligned,
 * not shared by calls in flight.  G must not overlap theta. */
rosa_status rosa_scatter_grad(const float *theta, int64_t B, int64_t T,
                              int64_t D, int64_t ldt, int32_t M,
                              const int32_t *end, float *G, int64_t ldg,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------ online automaton (decode) */

typedef struct rosa_state rosa_state;   /* opaque host handle */

/* Bytes of device state for S streams, alphabet K, up to t_capacity
 * positions per stream: one suffix automaton per stream with at most
 * max(2, 2*t_capacity - 1) states (Sec. 2.2 bound), dense K-wide transition
 * rows, and the symbol history.  0 on bad arguments. */
size_t rosa_state_bytes(int64_t S, int32_t K, int64_t t_capacity);

/* Sec. 2.2 / Sec. 4.1: builds, in the caller's device buffer `state_buf`,
 * one online suffix automaton per stream over the prefix `in` (T may be 0),
 * and returns a host handle in *handle.  If `out` is not NULL it receives
 * L/E/SYM for the prefix positions, identical to rosa_match.  in->K (or
 * 2^M) fixes the alphabet; t_capacity >= T bounds the total length.
 * The handle must be released with rosa_free (which does not free
 * state_buf).  A handle must not be used on two streams concurrently.
 * rosa_step_qk does not take it (ROSA_ERR_ARG). */
rosa_status rosa_build(const rosa_input *in, int64_t t_capacity,
                       void *state_buf, size_t state_bytes,
                       rosa_state **handle, const rosa_out *out,
                       hipStream_t stream);

/* Sec. 4.1 (per position, the stream's symbol extends its structure and the
 * retrieval emits the destination), Sec. 2.2 (the automaton's online
 * extension) and App. B.3 (destination = end of the latest earlier
 * occurrence, plus one).  One online step for every stream at position
 * t = current length: extend each automaton by the new symbol (`row`:
 * T == 1, same kind, S, B, D, M/K as at build), read E(t) from the new
 * state's suffix link, then set the last end of every state on the new
 * state's suffix path to t.  Writes end[S] = E(t), sym[S] = SYM(t) (may be
 * NULL) and, if out_row is not NULL, the gathered values
 *   out_row[b*ldo_b + r*M + m] = V[b*ldv_b + (E+1)*ldv + r*M + m]  (0 if E<0)
 * V must already hold position t (tau = E+1 can equal t).  Returns
 * ROSA_ERR_CAPACITY (checked on the host) once t_capacity positions exist;
 * ROSA_ERR_ARG for a query/key handle (rosa_build_qk).
 * Cost per stream: the append is O(1) amortised (Sec. 2.2); the last-end
 * walk visits the new state's suffix path, a few states on typical streams
 * but up to t on a constant or short-period stream, where a step is then t
 * dependent memory accesses. */
rosa_status rosa_step(rosa_state *h, const rosa_input *row, const uint16_t *V,
                      int64_t ldv, int64_t ldv_b, int32_t *end, int16_t *sym,
                      uint16_t *out_row, int64_t ldo_b, hipStream_t stream);

/* Bytes of device state for the query/key decode of S streams, alphabet K,
 * up to t_capacity time steps per stream: one suffix automaton per stream
 * over the key units (at most max(2, 2*t_capacity - 1) states, Sec. 2.2
 * bound), the matching state and the current unit's answers, and the start
 * time of every unit.  0 on bad arguments. */
size_t rosa_qk_state_bytes(int64_t S, int32_t K, int64_t t_capacity);

/* Sec. 3.3 and Sec. 4.1 for separate query and key streams, online: the
 * pages update each stream's automaton and matching state once per time
 * step (with ROSA_QK_RLE, once per key run, App. C.6), which is what a
 * decoder needs.  Builds, in the caller's buffer `state_buf` (256-byte
 * aligned, at least rosa_qk_state_bytes(S, K, t_capacity) bytes), the state
 * after the prefix q, k (same kind and shape as for rosa_match_qk; T may be
 * 0) and returns a host handle in *handle.  If `out` is not NULL it
 * receives the prefix's outputs exactly as rosa_match_qk would write them
 * ([S][T] arrays; tau required when T > 0; the counterfactual tables need
 * K = 2^M).  `flags`: 0 or ROSA_QK_RLE, fixed for the handle.  The handle
 * works with rosa_state_length, rosa_state_status and rosa_free, not with
 * rosa_step.  Cost: for prefixes of two steps or more and K <= 60, the
 * batch query/key retrieval gives every step's answers, the automaton is
 * built by appends without the last-unit walks (the last units filled in
 * one pass afterwards), and only the last key run is walked in time order;
 * otherwise the whole prefix is walked in time order, one wave per stream.
 * During the build, the state buffer also holds the batch retrieval's
 * workspace, which rosa_qk_state_bytes includes. */
rosa_status rosa_build_qk(const rosa_input *q, const rosa_input *k,
                          int32_t flags, int64_t t_capacity, void *state_buf,
                          size_t state_bytes, rosa_state **handle,
                          const rosa_qk_out *out, hipStream_t stream);

/* One online query/key time step t = current length for every stream (Sec.
 * 3.3; Eq. (16): the destination is strictly before t; App. C.5: the
 * counterfactual branches are one more matching update from the same
 * state).  q_row, k_row: T == 1, same kind, S, B, D, M/K as at build.  With
 * ROSA_QK_RLE, a key symbol equal to the previous one continues the current
 * run: the automaton and the matching state do not move and the outputs
 * are the run's (its destination now kept if it is before t).  Writes the
 * step's outputs into `out` as [S] arrays (cf_tau, cf_ridx: [S][M][2]):
 * tau required, end, len, run_of, ridx, cf_tau, cf_ridx optional,
 * run_start must be NULL.  The values equal rosa_match_qk's at time t over
 * the concatenated streams.  ROSA_ERR_CAPACITY (checked on the host) once
 * t_capacity steps exist; ROSA_ERR_ARG for a self-match handle.  A symbol
 * >= K sets the handle's sticky flag (rosa_state_status).  Cost per stream:
 * the append is O(1) amortised and the matching update follows suffix
 * links; the last-unit walk after an append visits the new state's suffix
 * path (up to the number of units on a periodic key stream without run
 * folding). */
rosa_status rosa_step_qk(rosa_state *h, const rosa_input *q_row,
                         const rosa_input *k_row, const rosa_qk_out *out,
                         hipStream_t stream);

/* Positions processed so far by the handle (host value, no sync). */
int64_t rosa_state_length(const rosa_state *h);

/* Synchronises `stream`; ROSA_ERR_SYMBOL if any build/step of this handle
 * saw a symbol >= K, else ROSA_OK. */
rosa_status rosa_state_status(rosa_state *h, hipStream_t stream);

/* Frees the host handle only (the caller owns and frees state_buf).
 * NULL is ignored. */
void rosa_free(rosa_state *h);

const char *rosa_error_string(rosa_status status);

#ifdef __cplusplus
}
#endif

#endif /* ROSA_H */
