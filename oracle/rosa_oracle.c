/*
 * rosa_oracle.c -- plain, slow, single-threaded CPU oracle for ROSA retrieval.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  The product path never
 * calls it and shares no code, header, table or helper with it.
 *
 * Source: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix Matching"
 * (Zheng, Wang, Ren, Chen; arXiv 2602.02499).
 *
 *   - oracle_discretize_bf16: Sec. 3.2, Eq. (10)-(15).  Each channel becomes
 *     the bit I[x > 0]; route r packs its M channels (r, j) with weight 2^j.
 *     Written as the definition: convert the bf16 to float and compare with 0.
 *   - oracle_match: Sec. 2.2 (suffix automaton, Blumer et al. 1985) and
 *     Sec. 3.3 / App. B.3 (retrieval destination = endpos of the matched
 *     suffix, plus one).  The body of Eq. (16) is lost in the page text; the
 *     reading implemented here: at position t, L is the length of the longest
 *     suffix of x[0..t] that also ends at some e < t, E is the largest such e
 *     (the most recent occurrence), SYM = x[E+1], tau = E+1; with no such
 *     suffix L = 0, E = -1, SYM = -1.  Computed with the textbook online
 *     automaton: extend by x[t], then the suffix link of the new state is the
 *     longest suffix seen before; its stored last end position (read before
 *     this step's update) is E; then every state on the suffix path of the
 *     new state gets last = t.  A clone inherits last from the state it splits.
 *   - oracle_brute: the same definition as an O(T^2) common-suffix table,
 *     lcs(t,e) = x[t]==x[e] ? 1 + lcs(t-1,e-1) : 0.  Used to pin oracle_match.
 *   - oracle_gather: App. C.4 read-out at the destination (value slice of row
 *     tau = E+1 for the route's M channels), masked to zero when tau < 0
 *     (App. C.1, Eq. (17)).  A byte copy.
 *   - oracle_sam_stats: state and transition counts of the automaton, and the
 *     number of distinct substrings it represents (Sec. 2.2: at most 2n-1
 *     states), for invariant tests.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- discretize */

static float bf16_to_float(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* H: [B][T][D] bf16 bit patterns, contiguous.  sym: [S][T], S = B*D/M,
 * stream s = b*R + r with R = D/M.  Returns 0, or -1 on bad arguments. */
int oracle_discretize_bf16(const uint16_t *H, int64_t B, int64_t T, int64_t D,
                           int M, uint8_t *sym)
{
    if (M < 1 || M > 8 || D % M != 0)
        return -1;
    int64_t R = D / M;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t r = 0; r < R; ++r) {
                int a = 0;
                for (int j = 0; j < M; ++j) {
                    float v = bf16_to_float(H[(b * T + t) * D + r * M + j]);
                    int bit = (v > 0.0f) ? 1 : 0;
                    a += bit << j;
                }
                sym[(b * R + r) * T + t] = (uint8_t)a;
            }
    return 0;
}

/* ---------------------------------------------------------- suffix automaton */

typedef struct {
    int64_t n_states;
    int K;
    int32_t *len;
    int32_t *link;
    int32_t *last;   /* largest end position seen so far, -1 if none */
    int32_t *next;   /* [n_states][K], -1 = no transition */
    int32_t tail;    /* state of the whole prefix */
} sam_t;

static int sam_init(sam_t *a, int64_t T, int K)
{
    int64_t cap = 2 * T + 2;
    a->K = K;
    a->len = (int32_t *)malloc(sizeof(int32_t) * cap);
    a->link = (int32_t *)malloc(sizeof(int32_t) * cap);
    a->last = (int32_t *)malloc(sizeof(int32_t) * cap);
    a->next = (int32_t *)malloc(sizeof(int32_t) * cap * K);
    if (!a->len || !a->link || !a->last || !a->next)
        return -1;
    a->n_states = 1;
    a->len[0] = 0;
    a->link[0] = -1;
    a->last[0] = -1;
    for (int c = 0; c < K; ++c)
        a->next[c] = -1;
    a->tail = 0;
    return 0;
}

static void sam_free(sam_t *a)
{
    free(a->len);
    free(a->link);
    free(a->last);
    free(a->next);
}

static int32_t sam_new_state(sam_t *a, int32_t len)
{
    int32_t v = (int32_t)a->n_states++;
    a->len[v] = len;
    a->link[v] = -1;
    a->last[v] = -1;
    for (int c = 0; c < a->K; ++c)
        a->next[(int64_t)v * a->K + c] = -1;
    return v;
}

/* Append symbol c (the symbol at position t); returns the new state. */
static int32_t sam_extend(sam_t *a, int c)
{
    int K = a->K;
    int32_t cur = sam_new_state(a, a->len[a->tail] + 1);
    int32_t p = a->tail;
    while (p != -1 && a->next[(int64_t)p * K + c] == -1) {
        a->next[(int64_t)p * K + c] = cur;
        p = a->link[p];
    }
    if (p == -1) {
        a->link[cur] = 0;
    } else {
        int32_t q = a->next[(int64_t)p * K + c];
        if (a->len[p] + 1 == a->len[q]) {
            a->link[cur] = q;
        } else {
            int32_t clone = sam_new_state(a, a->len[p] + 1);
            memcpy(&a->next[(int64_t)clone * K], &a->next[(int64_t)q * K],
                   sizeof(int32_t) * K);
            a->link[clone] = a->link[q];
            a->last[clone] = a->last[q];
            while (p != -1 && a->next[(int64_t)p * K + c] == q) {
                a->next[(int64_t)p * K + c] = clone;
                p = a->link[p];
            }
            a->link[q] = clone;
            a->link[cur] = clone;
        }
    }
    a->tail = cur;
    return cur;
}

/* One stream.  x: [T] symbols in [0, K).  E, SYM, L: [T] outputs (SYM and L
 * may be NULL).  Returns 0, -1 on bad arguments, -2 on a symbol >= K,
 * -3 on allocation failure. */
int oracle_match(const uint8_t *x, int64_t T, int K, int32_t *E, int16_t *SYM,
                 int32_t *L)
{
    if (T < 0 || K < 1 || K > 256)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        if (x[t] >= K)
            return -2;
    if (T == 0)
        return 0;
    sam_t a;
    if (sam_init(&a, T, K) != 0) {
        sam_free(&a);
        return -3;
    }
    for (int64_t t = 0; t < T; ++t) {
        int32_t cur = sam_extend(&a, x[t]);
        int32_t v = a.link[cur];
        int32_t e = -1, l = 0;
        if (v > 0) {            /* a non-root state: some suffix recurred */
            l = a.len[v];
            e = a.last[v];      /* read before this step's update */
        }
        E[t] = e;
        if (L)
            L[t] = l;
        if (SYM)
            SYM[t] = (int16_t)(e >= 0 ? x[e + 1] : -1);
        for (int32_t u = cur; u != -1; u = a.link[u])
            a.last[u] = (int32_t)t;
    }
    sam_free(&a);
    return 0;
}

/* Same outputs for S streams: x is [S][ld], outputs are [S][T]. */
int oracle_match_streams(const uint8_t *x, int64_t S, int64_t T, int64_t ld,
                         int K, int32_t *E, int16_t *SYM, int32_t *L)
{
    for (int64_t s = 0; s < S; ++s) {
        int rc = oracle_match(x + s * ld, T, K, E + s * T,
                              SYM ? SYM + s * T : NULL, L ? L + s * T : NULL);
        if (rc != 0)
            return rc;
    }
    return 0;
}

/* Automaton statistics for x[0..T): number of states, of transitions, of
 * clones, and the number of distinct non-empty substrings,
 * sum over non-root states of len(v) - len(link(v)). */
int oracle_sam_stats(const uint8_t *x, int64_t T, int K, int64_t *out4)
{
    if (T < 0 || K < 1 || K > 256)
        return -1;
    sam_t a;
    if (sam_init(&a, T, K) != 0) {
        sam_free(&a);
        return -3;
    }
    int64_t clones_before = 0, created = 0;
    for (int64_t t = 0; t < T; ++t) {
        if (x[t] >= K) {
            sam_free(&a);
            return -2;
        }
        int64_t before = a.n_states;
        sam_extend(&a, x[t]);
        created += a.n_states - before;
        clones_before += (a.n_states - before) - 1;
    }
    int64_t trans = 0, distinct = 0;
    for (int64_t v = 0; v < a.n_states; ++v) {
        for (int c = 0; c < K; ++c)
            trans += a.next[v * K + c] != -1;
        if (v > 0)
            distinct += a.len[v] - a.len[a.link[v]];
    }
    out4[0] = a.n_states;
    out4[1] = trans;
    out4[2] = clones_before;
    out4[3] = distinct;
    (void)created;
    sam_free(&a);
    return 0;
}

/* ------------------------------------------------------------- brute force */

/* O(T^2) time, O(T) memory.  E and L as in oracle_match. */
int oracle_brute(const uint8_t *x, int64_t T, int32_t *E, int32_t *L)
{
    if (T < 0)
        return -1;
    int32_t *prev = (int32_t *)calloc((size_t)(T + 1), sizeof(int32_t));
    int32_t *row = (int32_t *)calloc((size_t)(T + 1), sizeof(int32_t));
    if (!prev || !row) {
        free(prev);
        free(row);
        return -3;
    }
    /* row[e] = lcs(t, e) for e < t; prev[e] = lcs(t-1, e) */
    for (int64_t t = 0; t < T; ++t) {
        int32_t best = 0, arg = -1;
        for (int64_t e = 0; e < t; ++e) {
            int32_t v = 0;
            if (x[t] == x[e])
                v = 1 + (e >= 1 ? prev[e - 1] : 0);
            row[e] = v;
            if (v > 0 && v >= best) { /* ties: the later e wins */
                best = v;
                arg = (int32_t)e;
            }
        }
        E[t] = arg;
        L[t] = best;
        int32_t *tmp = prev;
        prev = row;
        row = tmp;
    }
    free(prev);
    free(row);
    return 0;
}

/* ------------------------------------------------------------------ gather */

/* V, out: [B][T][D] bf16 bit patterns.  E: [S][T] with S = B*D/M.
 * out[b][t][r*M+m] = V[b][E+1][r*M+m] when E >= 0, else 0. */
int oracle_gather(const uint16_t *V, int64_t B, int64_t T, int64_t D, int M,
                  const int32_t *E, uint16_t *out)
{
    if (M < 1 || M > 8 || D % M != 0)
        return -1;
    int64_t R = D / M;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t t = 0; t < T; ++t)
            for (int64_t r = 0; r < R; ++r) {
                int64_t e = E[(b * R + r) * T + t];
                for (int m = 0; m < M; ++m) {
                    uint16_t v = 0;
                    if (e >= 0)
                        v = V[(b * T + (e + 1)) * D + r * M + m];
                    out[(b * T + t) * D + r * M + m] = v;
                }
            }
    return 0;
}

/* ---------------------------------------------- query / key retrieval */

/*
 * oracle_match_qk -- Sec. 3.3 with a query stream q and a key stream k
 * (k_{1:t} = a^(k), q_{1:t} = a^(q)), optionally with run-length folding of
 * the key stream (Sec. 3.3, RLE paragraph; App. C.6) and with per-bit
 * counterfactual destinations (App. C.5 and C.6; Sec. 4.2 step 3).
 *
 * Units.  Without folding, unit u is time u.  With folding, unit u is the
 * u-th maximal run of equal adjacent key symbols; start[u] is its first
 * time, its key symbol C[u] is the run's symbol and its query symbol Q[u]
 * is q[start[u]] (the automaton and the matching state move only at run
 * boundaries).  N = number of units.
 *
 * Retrieval at unit u.  The automaton holds C[0..u-1] (strictly earlier
 * units); the matching state is advanced by Q[u].  The match is the longest
 * suffix of Q[0..u] that occurs in C[0..u-1] (length L, in units, 0 if
 * none) and e is the last unit at which it ends (the state's last end
 * position).  Destination unit d = e + 1.  For every time t of unit u:
 *   tau(t) = start[d]  if L >= 1, d < N and start[d] < t  (strictly from
 *            the past, the range of Eq. (16)), else -1.
 * Computed the textbook way (matching statistics on a suffix automaton):
 * from (state s, length l), follow suffix links until a transition on the
 * symbol exists, take it and add one, or fall to the root with l = 0; after
 * the key symbol of unit u is appended, move s up the suffix links while
 * the link's length is still >= l (a clone may have taken the matched
 * string).  That last move keeps (s, l) a valid pair but changes no output:
 * until the next append a split state and its clone have the same
 * transitions, and the next update leaves s through a transition (reaching
 * the same state from either) or up the suffix links (from the split state
 * the first link is the clone itself).
 *
 * Counterfactual (bit j < M, value v): the query symbol of unit u with bit j
 * forced to v, one matching update from the same state; tau^(v) as above.
 *
 * Outputs, all [T] (per time step) unless noted, NULL to skip:
 *   tau, end (e, in units; -1), len (L, in units);
 *   run_of (unit of t), run_start ([T]: start[u] for u < N, then -1),
 *   ridx (d where tau(t) >= 0, else -1);
 *   cf_tau, cf_ridx ([T][M][2]: entry [t][j][v]).
 * K must be 2^M when counterfactual outputs are asked for.
 * Returns 0, -1 on bad arguments, -2 on a symbol >= K, -3 on allocation
 * failure.
 */
static void qk_advance(const sam_t *a, int32_t *s, int32_t *l, int c)
{
    int K = a->K;
    while (*s != 0 && a->next[(int64_t)*s * K + c] == -1) {
        *s = a->link[*s];
        *l = a->len[*s];
    }
    int32_t nx = a->next[(int64_t)*s * K + c];
    if (nx != -1) {
        *s = nx;
        *l += 1;
    } else {
        *s = 0;
        *l = 0;
    }
}

static int32_t qk_dest_time(int32_t e, int64_t t, int64_t N,
                            const int32_t *start)
{
    if (e < 0 || e + 1 >= N)
        return -1;
    return start[e + 1] < t ? start[e + 1] : -1;
}

int oracle_match_qk(const uint8_t *q, const uint8_t *k, int64_t T, int K,
                    int M, int rle, int32_t *tau, int32_t *end, int32_t *len,
                    int32_t *run_of, int32_t *run_start, int32_t *ridx,
                    int32_t *cf_tau, int32_t *cf_ridx)
{
    if (T < 0 || K < 1 || K > 256 || M < 0 || M > 8)
        return -1;
    if ((cf_tau || cf_ridx) && (M < 1 || K != (1 << M)))
        return -1;
    for (int64_t t = 0; t < T; ++t)
        if (q[t] >= K || k[t] >= K)
            return -2;
    if (T == 0)
        return 0;
    int32_t *start = (int32_t *)malloc(sizeof(int32_t) * T);
    int32_t *unit = (int32_t *)malloc(sizeof(int32_t) * T);
    int32_t *ue = (int32_t *)malloc(sizeof(int32_t) * T);
    int32_t *ul = (int32_t *)malloc(sizeof(int32_t) * T);
    int32_t *ucf = (int32_t *)malloc(sizeof(int32_t) * T * (M > 0 ? 2 * M : 1));
    sam_t a;
    if (!start || !unit || !ue || !ul || !ucf || sam_init(&a, T, K) != 0) {
        free(start); free(unit); free(ue); free(ul); free(ucf);
        return -3;
    }
    /* units */
    int64_t N = 0;
    for (int64_t t = 0; t < T; ++t) {
        if (!rle || t == 0 || k[t] != k[t - 1])
            start[N++] = (int32_t)t;
        unit[t] = (int32_t)(N - 1);
    }
    int want_cf = (cf_tau || cf_ridx) ? 1 : 0;
    int32_t s = 0, l = 0;
    for (int64_t u = 0; u < N; ++u) {
        int Qu = q[start[u]];
        if (want_cf)
            for (int j = 0; j < M; ++j)
                for (int v = 0; v < 2; ++v) {
                    int c = (Qu & ~(1 << j)) | (v << j);
                    int32_t s2 = s, l2 = l;
                    qk_advance(&a, &s2, &l2, c);
                    ucf[(u * M + j) * 2 + v] = l2 > 0 ? a.last[s2] : -1;
                }
        qk_advance(&a, &s, &l, Qu);
        ul[u] = l;
        ue[u] = l > 0 ? a.last[s] : -1;
        int32_t cur = sam_extend(&a, k[start[u]]);
        for (int32_t w = cur; w != -1; w = a.link[w])
            a.last[w] = (int32_t)u;
        while (s != 0 && a.len[a.link[s]] >= l)
            s = a.link[s];
    }
    for (int64_t t = 0; t < T; ++t) {
        int32_t u = unit[t];
        int32_t tt = qk_dest_time(ue[u], t, N, start);
        if (tau)
            tau[t] = tt;
        if (end)
            end[t] = ue[u];
        if (len)
            len[t] = ul[u];
        if (run_of)
            run_of[t] = u;
        if (run_start)
            run_start[t] = t < N ? start[t] : -1;
        if (ridx)
            ridx[t] = tt >= 0 ? ue[u] + 1 : -1;
        if (want_cf)
            for (int j = 0; j < M; ++j)
                for (int v = 0; v < 2; ++v) {
                    int32_t e = ucf[(u * M + j) * 2 + v];
                    int32_t ct = qk_dest_time(e, t, N, start);
                    int64_t o = (t * M + j) * 2 + v;
                    if (cf_tau)
                        cf_tau[o] = ct;
                    if (cf_ridx)
                        cf_ridx[o] = ct >= 0 ? e + 1 : -1;
                }
    }
    sam_free(&a);
    free(start); free(unit); free(ue); free(ul); free(ucf);
    return 0;
}

/* ---------------------------------------------- destination scatter (grad) */

/* App. C.4 (destination-scatter aggregation) and the gradient of the values
 * in Sec. 3: the value read at destination tau collects the upstream
 * gradient of every time step that read it,
 *   G[b][tau][c] = sum over t = 0..T-1 of theta[b][t][c] * I[tau(b,r(c),t) = tau],
 * the transpose of oracle_gather.  Here tau(s,t) = E[s][t] + 1 for
 * E[s][t] >= 0 (and E+1 < T); other entries read nothing and add nothing.
 * theta, G: float [B][T][D]; E: [S][T], S = B*D/M, s = b*R + r, channel
 * c = r*M + m.  The sum runs over t in increasing order in double precision
 * and is rounded to float once. */
int oracle_scatter_grad(const float *theta, int64_t B, int64_t T, int64_t D,
                        int M, const int32_t *E, float *G)
{
    if (M < 1 || M > 8 || D % M != 0 || B < 0 || T < 0)
        return -1;
    int64_t R = D / M;
    double *acc = (double *)calloc((size_t)(B * T * D > 0 ? B * T * D : 1),
                                   sizeof(double));
    if (!acc)
        return -3;
    for (int64_t b = 0; b < B; ++b)
        for (int64_t r = 0; r < R; ++r)
            for (int64_t t = 0; t < T; ++t) {
                int64_t e = E[(b * R + r) * T + t];
                if (e < 0 || e + 1 >= T)
                    continue;
                for (int m = 0; m < M; ++m)
                    acc[(b * T + (e + 1)) * D + r * M + m] +=
                        (double)theta[(b * T + t) * D + r * M + m];
            }
    for (int64_t i = 0; i < B * T * D; ++i)
        G[i] = (float)acc[i];
    free(acc);
    return 0;
}
