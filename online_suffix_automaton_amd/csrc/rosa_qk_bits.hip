// rosa_qk_bits.hip -- query/key retrieval, bit-parallel over the key units.
//
// Method: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix Matching"
// (arXiv 2602.02499), Sec. 3.3 with separate query and key streams (the
// match is the longest suffix of the query units that occurs among the
// earlier key units, its end the most recent such unit; run folding as in
// the run-length paragraph), App. C.5 (counterfactual branches: one more
// matching update with one query bit forced).
//
// The same results as the automaton kernels of rosa_sam.hip, computed as
// sets instead of states.  For unit u and length l let B_l(u) be the set of
// key units e < u at which the last l query units end as well:
//   B_1(u) = { e < u : k_e = q_u },
//   B_l(u) = { e < u : k_e = q_u and e-1 in B_{l-1}(u-1) },
// so B_l(u) = (B_{l-1}(u-1) shifted up by one) & EQ(q_u), with EQ(c) the set
// of key units so far with symbol c.  L(u) is the largest l with B_l(u)
// nonempty and E(u) its largest member; L(u) <= L(u-1) + 1, and B_l(u) is
// contained in B_{l-1}(u), so the nonempty levels are 1..L(u).  A stream of
// at most 4096 units is one wave: every set is a 4096-bit vector, lane w
// holding bits 64w..64w+63, so one update of a set is a few instructions for
// all candidate ends at once, and the levels 1..L live in registers.  A
// counterfactual branch is the same update with the flipped symbol's EQ,
// computed from the sets before the unit's own update.
//
// Matches longer than kQbLevels units are not followed: such a stream is
// marked in redo[] and answered by the automaton kernel instead.
#include "rosa_internal.h"

namespace rosa {

constexpr int kQbLevels = 32;    // levels kept in registers
constexpr int kQbMaxT = 4096;    // one 64-bit word per lane
constexpr int kQbMaxK = 64;
constexpr int kQbMaxChains = 7;  // the unit's own update + M <= 6 branches

// The 4096-bit vector shifted up by one: bit e of the result is bit e-1 of v
// (the carry into each word is the top bit of the lane below, by a
// wave_shr:1 DPP move; lane 0 receives 0).
__device__ __forceinline__ uint64_t qb_shl1(uint64_t v)
{
    const int top = (int)(uint32_t)(v >> 63);
    const int c = __builtin_amdgcn_update_dpp(0, top, 0x138, 0xF, 0xF, false);
    return (v << 1) | (uint64_t)(uint32_t)c;
}

// What the levels of one unit leave per chain: the set at the highest
// nonempty level, and for chain 0 that level, L(u).
template <int NCH>
struct QbAcc {
    uint64_t top[NCH];
    int L0;
};

// Levels l..lim of every chain, from the bottom up: level l of a chain is
// the previous unit's B_{l-1} (`prev`, read before chain 0 overwrites it)
// shifted up by one and masked with the chain's EQ; chain 0 stores its new
// level in B[l-1].  A set that is empty at one level is empty at every
// higher one, so the last nonempty level visited is the top one.  Levels
// above lim = L(u-1) + 1 are empty and not visited; B keeps stale values
// there, which no later unit reads (it visits at most L(u) + 1 levels).
// Unrolled by template recursion so that B stays in registers.
template <int l, int NCH>
__device__ __forceinline__ void qb_levels(uint64_t (&B)[kQbLevels], uint64_t prev, int lim,
                                          const uint64_t (&e)[NCH], QbAcc<NCH> &a)
{
    if constexpr (l <= kQbLevels) {
        const uint64_t old = B[l - 1];
        const uint64_t sh = l == 1 ? ~0ull : qb_shl1(prev);
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            const uint64_t nw = sh & e[i];
            const bool ne = __builtin_amdgcn_ballot_w64(nw != 0) != 0;
            a.top[i] = ne ? nw : a.top[i];
            if (i == 0) {
                a.L0 = ne ? l : a.L0;
                B[l - 1] = nw;
            }
        }
        if (l < lim)
            qb_levels<l + 1, NCH>(B, old, lim, e, a);
    }
}

// Symbol of chain i for query symbol q: q itself, then q with one bit
// flipped, flip[i] = 1 << (its query bit).
template <int i, int NCH>
__device__ __forceinline__ int qb_sym(int q, const int (&flip)[NCH])
{
    return i == 0 ? q : (q ^ flip[i]);
}

// Reads the EQ words of every chain's symbol for query symbol q.
template <int i, int NCH>
__device__ __forceinline__ void qb_read_eq(uint64_t (&dst)[NCH], const uint64_t *eq,
                                           int q, int kmask, int lane, const int (&flip)[NCH])
{
    if constexpr (i < NCH) {
        dst[i] = eq[(qb_sym<i, NCH>(q, flip) & kmask) * 64 + lane];
        qb_read_eq<i + 1, NCH>(dst, eq, q, kmask, lane, flip);
    }
}

// Largest member of this lane's part of a set, or -1.
__device__ __forceinline__ int qb_lane_top(uint64_t w, int lane)
{
    return w ? 64 * lane + 63 - __clzll((long long)w) : -1;
}

// Largest value of one 64-entry row of lane tops (int16).  The lanes of a
// wave read different rows; each starts at another 16-byte piece of its row
// so that they spread over the banks.
__device__ __forceinline__ int qb_row_max(const int16_t *row, int r)
{
    typedef short v2s __attribute__((ext_vector_type(2)));
    v2s m = {-1, -1};
#pragma unroll
    for (int pc = 0; pc < 8; ++pc) {
        const uint4 w = *reinterpret_cast<const uint4 *>(row + 8 * ((pc ^ r) & 7));
        const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v2s x;
            __builtin_memcpy(&x, &d[k], 4);
            m = __builtin_elementwise_max(m, x);
        }
    }
    return m.x > m.y ? m.x : m.y;
}

// Shared memory of one stream: EQ words [KB][64] u64 (KB = K rounded up to a
// power of two), lane-top rows [NCH][64 positions][64 lanes] int16, and with
// run folding the start time of every unit [4096] u16.
inline size_t qb_lds_bytes(int kb, int nch, bool rle)
{
    return (size_t)kb * 512 + (size_t)nch * 8192 + (rle ? (size_t)kQbMaxT * 2 : 0);
}

// One wave per stream, or per half of a stream's counterfactual branches
// (halves = 2: workgroup 2s + h does the unit's own update, which drives
// the sets, and the branches of query bits h*(NCH-1) .. h*(NCH-1) + NCH-2;
// the first half also writes the stream's own outputs).  NCH chains per
// unit (1, or 1 + the branches); RLE: key runs folded into units;
// kmask = KB - 1.
//
// Per position the wave does wave-uniform work only: a new unit appends its
// key symbol to EQ and issues the LDS reads of the next position's EQ words
// (their latency hides behind this unit's levels), runs the levels, and
// writes every chain's lane tops into the position's row.  After each
// 64-position chunk every lane forms one position's outputs: the largest
// member of each chain's top set is the maximum of its row, and the start
// time of a unit comes from LDS.
template <int NCH, bool RLE>
__global__ __launch_bounds__(64) void qk_bits_kernel(QkParams p, int kmask, int halves)
{
    extern __shared__ __align__(16) uint64_t qb_smem[];
    constexpr int NB = NCH - 1;   // branches of this workgroup
    uint64_t *eq = qb_smem;
    int16_t *rows = reinterpret_cast<int16_t *>(qb_smem + (kmask + 1) * 64);
    uint16_t *st = reinterpret_cast<uint16_t *>(rows + NCH * 4096);
    const int lane = threadIdx.x;
    const int64_t s = blockIdx.x / halves;
    const int half = (int)(blockIdx.x % halves);
    const int bit0 = half * NB;   // query bit of branch 1
    const bool own = half == 0;   // writes the stream's own outputs
    // flip[i]: the query bit branch i forces (a branch past the last bit
    // repeats the last one and writes nothing)
    int flip[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int bq = bit0 + i - 1;
        flip[i] = i == 0 ? 0 : 1 << (bq < p.M ? bq : p.M - 1);
    }
    const int T = (int)p.T;
    for (int c = 0; c <= kmask; ++c)
        eq[c * 64 + lane] = 0;
    __syncthreads();
    const uint8_t *qr = p.q + s * p.Tp + kPadFront;
    const uint8_t *kr = p.k + s * p.Tp + kPadFront;
    const int64_t base = s * (int64_t)T;
    uint64_t B[kQbLevels];
#pragma unroll
    for (int l = 0; l < kQbLevels; ++l)
        B[l] = 0;
    int Lc = 0;               // levels 1..Lc of the previous unit are nonempty
    bool over = false;
    int u = -1, kprev = -1, qc = 0, ul = 0;
    int eqn_q = -1;           // query symbol the words in eqn were read for
    int carry[NCH];           // largest members of the unit a chunk begins in
#pragma unroll
    for (int i = 0; i < NCH; ++i)
        carry[i] = -1;
    // EQ words of the next position's query symbol (nothing appended yet)
    uint64_t eqn[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i)
        eqn[i] = 0;
    // the next key unit's bit: unit u is bit u%64 of lane u/64
    uint64_t wbit = lane == 0 ? 1ull : 0ull;
    // chunk loads, one chunk ahead: key and query symbols of each lane's
    // position and the query symbol of the position after it (the rows carry
    // 64 bytes of padding after T, so these loads stay in the row).  The
    // last goes through its own pointer, opaque to the compiler: merged with
    // the query load into one 2-byte load, its bytes would be split, and
    // waited for, right after the load.
    typedef const __attribute__((address_space(1))) uint8_t *qb_gbytes;
    const uint8_t *xp = qr + 1;
    asm volatile("" : "+s"(xp));
    const qb_gbytes xr = (qb_gbytes)xp;   // global memory, not flat
    int kn = kr[lane], qn = qr[lane], xn = xr[lane];
    for (int t0 = 0; t0 < T && !over; t0 += 64) {
        const int kch = kn, qch = qn, qnext = xn;
        if (t0 + 64 < T) {
            kn = kr[t0 + 64 + lane];
            qn = qr[t0 + 64 + lane];
            xn = xr[t0 + 64 + lane];
        }
        int o_len = 0, o_run = -1, o_q = 0, o_row = -1;
        const int n = T - t0 < 64 ? T - t0 : 64;
        // One unit, starting at chunk position j with key symbol kc and
        // query symbol qcu; qx is the query symbol of the next unit's start,
        // whose EQ words are read ahead.
        auto unit = [&](int j, int kc, int qcu, int qx) {
            ++u;
            qc = qcu;
            if (RLE && lane == 0)
                st[u] = (uint16_t)(t0 + j);
            uint64_t e[NCH];
#pragma unroll
            for (int i = 0; i < NCH; ++i)
                e[i] = eqn[i];
            if (RLE && qcu != eqn_q)   // the read-ahead was for another symbol
                qb_read_eq<0, NCH>(e, eq, qcu, kmask, lane, flip);
            // append key unit u (this unit's chains use the words read
            // before it), then read the next unit's words
            atomicOr(reinterpret_cast<unsigned long long *>(&eq[(kc & kmask) * 64 + lane]),
                     (unsigned long long)wbit);
            wbit = qb_shl1(wbit);
            qb_read_eq<0, NCH>(eqn, eq, qx, kmask, lane, flip);
            eqn_q = qx;
            int lim = Lc + 1;
            if (lim > kQbLevels) {
                // a chain that would still grow past the kept levels
                const uint64_t sh = qb_shl1(B[kQbLevels - 1]);
#pragma unroll
                for (int i = 0; i < NCH; ++i)
                    if (__builtin_amdgcn_ballot_w64((sh & e[i]) != 0))
                        over = true;
                lim = kQbLevels;
            }
            QbAcc<NCH> a;
#pragma unroll
            for (int i = 0; i < NCH; ++i)
                a.top[i] = 0;
            // L(u) starts at 0; through an opaque register, so that level 1
            // sets it with a scalar select, not a vector select read back
            int zero = 0;
            asm volatile("" : "+s"(zero));
            a.L0 = zero;
            qb_levels<1, NCH>(B, 0ull, lim, e, a);
            Lc = a.L0;
            ul = a.L0;
#pragma unroll
            for (int i = 0; i < NCH; ++i)
                rows[(i * 64 + j) * 64 + lane] = (int16_t)qb_lane_top(a.top[i], lane);
        };
        if constexpr (!RLE) {
            // every position is a unit
            for (int j = 0; j < n; ++j) {
                unit(j, __builtin_amdgcn_readlane(kch, j), __builtin_amdgcn_readlane(qch, j),
                     __builtin_amdgcn_readlane(qnext, j));
                o_len = lane == j ? ul : o_len;   // staged in lane j
            }
            o_row = lane;
            o_run = t0 + lane;
            o_q = qch;
        } else {
            // units start where the key symbol changes; the loop visits the
            // starts only, and each staged its unit in the start's lane
            const int kup = __builtin_amdgcn_update_dpp(0, kch, 0x138, 0xF, 0xF, false);
            const uint64_t S0 = __builtin_amdgcn_ballot_w64(
                lane < n && kch != (lane == 0 ? kprev : kup));
            const int ul_c = ul, u_c = u, qc_c = qc;   // the unit the chunk begins in
            uint64_t S = S0;
            while (S) {
                const int j = __builtin_ctzll(S);
                S &= S - 1;
                // the next unit's query symbol: its start in this chunk, else
                // a guess, the next chunk's first position (checked there)
                const int qx = S ? __builtin_amdgcn_readlane(qch, __builtin_ctzll(S))
                                 : __builtin_amdgcn_readlane(qn, 0);
                unit(j, __builtin_amdgcn_readlane(kch, j), __builtin_amdgcn_readlane(qch, j), qx);
                const bool mine = lane == j;
                o_len = mine ? ul : o_len;
                o_run = mine ? u : o_run;
                o_q = mine ? qc : o_q;
            }
            kprev = __builtin_amdgcn_readlane(kch, n - 1);
            // each position's unit: the last start at or before it in this
            // chunk (values from that lane), else the unit the chunk began in
            const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1);
            const uint64_t m = S0 & upto;
            const int js = m ? 63 - __clzll((long long)m) : -1;
            const int src = (js < 0 ? 0 : js) * 4;
            const int bl = __builtin_amdgcn_ds_bpermute(src, o_len);
            const int br = __builtin_amdgcn_ds_bpermute(src, o_run);
            const int bq = __builtin_amdgcn_ds_bpermute(src, o_q);
            o_len = js >= 0 ? bl : ul_c;
            o_run = js >= 0 ? br : u_c;
            o_q = js >= 0 ? bq : qc_c;
            o_row = js;
        }
        // the rows and unit starts were written by other lanes of this wave
        __builtin_amdgcn_wave_barrier();
        // every chain's largest member at this lane's position: the maximum
        // of the unit's row, or the unit the chunk began in
        int E[NCH];
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
            E[i] = o_row >= 0 ? qb_row_max(rows + (i * 64 + (o_row & 63)) * 64, o_row)
                              : carry[i];
            if (RLE)
                carry[i] = __builtin_amdgcn_readlane(E[i], n - 1);
        }
        if (lane < n && !over) {
            const int t = t0 + lane;
            const int64_t o = base + t;
            // a match ending at unit e is usable once unit e+1 has started
            const int ue = E[0];
            const int ds = ue >= 0 ? (RLE ? (int)st[ue + 1] : ue + 1) : -1;
            const int tt = (ue >= 0 && ds < t) ? ds : -1;
            const int rt = tt >= 0 ? ue + 1 : -1;
            if (own) {
                p.tau[o] = tt;
                if (p.end)
                    p.end[o] = ue;
                if (p.len)
                    p.len[o] = o_len;
                if (p.run_of)
                    p.run_of[o] = o_run;
                if (p.ridx)
                    p.ridx[o] = rt;
            }
#pragma unroll
            for (int i = 1; i < NCH; ++i) {
                const int b = bit0 + i - 1;   // query bit of branch i
                if (b >= p.M)
                    break;
                const int ce = E[i];
                const int cd = ce >= 0 ? (RLE ? (int)st[ce + 1] : ce + 1) : -1;
                const int tb = (ce >= 0 && cd < t) ? cd : -1;
                const int rb = tb >= 0 ? ce + 1 : -1;
                const bool bit = (o_q >> b) & 1;
                const int64_t c0 = (o * p.M + b) * 2;
                if (p.cf_tau)
                    *reinterpret_cast<int2 *>(p.cf_tau + c0) =
                        bit ? make_int2(tb, tt) : make_int2(tt, tb);
                if (p.cf_ridx)
                    *reinterpret_cast<int2 *>(p.cf_ridx + c0) =
                        bit ? make_int2(rb, rt) : make_int2(rt, rb);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
    if (own && !over && p.run_start)
        for (int v = lane; v < T; v += 64)
            p.run_start[base + v] = v <= u ? (RLE ? (int32_t)st[v] : v) : -1;
    // with two halves redo[] starts at zero and either half may set it
    if (lane == 0 && (halves == 1 || over))
        p.redo[s] = over ? 1 : 0;
}

// Zeroes n int32 values.
__global__ void qb_zero_kernel(int32_t *a, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        a[i] = 0;
}

static int qb_kb(int K)
{
    int kb = 1;
    while (kb < K)
        kb <<= 1;
    return kb;
}

static int qb_chains(const QkParams &p)
{
    return (p.cf_tau || p.cf_ridx) ? 1 + p.M : 1;
}

bool qk_bits_fits(const QkParams &p)
{
    // with the tables, K = 2^M <= 64: at most 7 chains
    return p.T <= kQbMaxT && p.K <= kQbMaxK && qb_chains(p) <= kQbMaxChains;
}

// Compute units of the current device (cached per device), 0 if unknown.
static int qb_cus()
{
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 0;
    if (cus[dev] == 0 &&
        hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus[dev] = -1;
    return cus[dev] > 0 ? cus[dev] : 0;
}

template <int NCH, bool RLE>
static hipError_t launch_qk_bits_n(const QkParams &p, int halves, hipStream_t st)
{
    const int kb = qb_kb(p.K);
    const size_t lds = qb_lds_bytes(kb, NCH, RLE);
    if (lds > 65536) {
        // more dynamic shared memory than the default limit: raise it once
        // per process (the chip has 160 KiB per workgroup)
        static bool raised = false;
        if (!raised) {
            const hipError_t e = hipFuncSetAttribute(
                reinterpret_cast<const void *>(&qk_bits_kernel<NCH, RLE>),
                hipFuncAttributeMaxDynamicSharedMemorySize,
                (int)qb_lds_bytes(kQbMaxK, NCH, RLE));
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return hipErrorNotSupported;   // not launched
            }
            raised = true;
        }
    }
    if (halves > 1)
        hipLaunchKernelGGL(qb_zero_kernel, dim3((unsigned)((p.S + 255) / 256)), dim3(256), 0,
                           st, p.redo, p.S);
    hipLaunchKernelGGL((qk_bits_kernel<NCH, RLE>), dim3((unsigned)(p.S * halves)), dim3(64),
                       lds, st, p, kb - 1, halves);
    return hipGetLastError();
}

template <bool RLE>
static hipError_t launch_qk_bits_r(const QkParams &p, int nch, int halves, hipStream_t st)
{
    switch (nch) {
    case 1: return launch_qk_bits_n<1, RLE>(p, halves, st);
    case 2: return launch_qk_bits_n<2, RLE>(p, halves, st);
    case 3: return launch_qk_bits_n<3, RLE>(p, halves, st);
    case 4: return launch_qk_bits_n<4, RLE>(p, halves, st);
    case 5: return launch_qk_bits_n<5, RLE>(p, halves, st);
    case 6: return launch_qk_bits_n<6, RLE>(p, halves, st);
    case 7: return launch_qk_bits_n<7, RLE>(p, halves, st);
    default: return hipErrorInvalidValue;
    }
}

// One wave per stream, or two per stream with the counterfactual branches
// split between them when the doubled grid still gives every wave a SIMD of
// its own and fits the LDS at once (each wave is bound by its own
// instruction issue, so the second wave uses otherwise idle SIMDs).
hipError_t launch_qk_bits(const QkParams &p, hipStream_t st)
{
    int nch = qb_chains(p), halves = 1;
    if (nch >= 3) {
        const int nh = 1 + (p.M + 1) / 2;
        const int64_t cus = qb_cus();
        const int64_t per_cu = 163840 / (int64_t)qb_lds_bytes(qb_kb(p.K), nh, p.rle != 0);
        if (cus > 0 && 2 * p.S <= 4 * cus && 2 * p.S <= per_cu * cus) {
            nch = nh;
            halves = 2;
        }
    }
    return p.rle ? launch_qk_bits_r<true>(p, nch, halves, st)
                 : launch_qk_bits_r<false>(p, nch, halves, st);
}

}  // namespace rosa
