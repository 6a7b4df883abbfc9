// rosa_scatter.hip -- destination-scatter gradient: the transpose of the
// value gather.
//
// Method: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix Matching"
// (arXiv 2602.02499), App. C.4 (destination-scatter aggregation) and the
// value gradient of Sec. 3: the value read at destination tau receives the
// sum of the upstream gradient theta of every time step t whose destination
// is tau, channel by channel within the route:
//   G[b][tau][r*M+m] = sum_t theta[b][t][r*M+m] * I[E[s][t] + 1 == tau],
// s = b*R + r.  The sum runs over t in increasing order in double precision
// and is rounded to float once, so the result is deterministic and does not
// depend on the launch geometry.
//
// Per stream, a counting sort groups the time steps by destination:
//   count   cnt[s][tau]        (integer atomics: order-free)
//   scan    off[s][tau]        (exclusive prefix, one workgroup per stream)
//   fill    list[s][off + i]   (unordered inside a destination)
// (for streams of up to 65536 positions all three run in one workgroup per
// stream with the counters in LDS)
//   sum     one thread per (b, tau, route): walks its time steps in
//           increasing order (selection over the few entries a destination
//           has) and writes the route's M values of row tau; rows are
//           written route-contiguous, so the stores are coalesced.
// A destination with more than kSelectMax time steps is handed to a wave
// that visits the stream's time steps in order (ballot over 64 at a time).
#include "rosa_internal.h"

namespace rosa {

constexpr int kSelectMax = 64;

__global__ void scatter_zero_kernel(int32_t *__restrict__ p, int64_t n)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

__global__ void scatter_count_kernel(ScatterParams p)
{
    const int64_t s = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= p.T)
        return;
    const int64_t e = p.end[s * p.T + t];
    if (e >= 0 && e + 1 < p.T)
        atomicAdd(&p.cnt[s * p.T + e + 1], 1);
}

__device__ __forceinline__ int sc_wave_incl_scan(int v)
{
    const int lane = __lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int o = __shfl_up(v, d);
        if (lane >= d)
            v += o;
    }
    return v;
}

// Exclusive prefix of cnt[s][0..T) into off[s][0..T]; cnt is cleared for
// its second use as the fill cursor.
__global__ __launch_bounds__(1024) void scatter_scan_kernel(ScatterParams p)
{
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int64_t s = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    int32_t *cnt = p.cnt + s * p.T;
    int32_t *off = p.off + s * p.Tq;
    if (tid == 0)
        carry_s = 0;
    __syncthreads();
    for (int64_t c0 = 0; c0 < p.T; c0 += 4096) {
        int v[4], sum = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = c0 + 4 * tid + u;
            v[u] = i < p.T ? cnt[i] : 0;
            sum += v[u];
        }
        const int incl = sc_wave_incl_scan(sum);
        if (lane == 63)
            wsum[wid] = incl;
        __syncthreads();
        if (wid == 0) {
            const int w = lane < 16 ? wsum[lane] : 0;
            const int wi = sc_wave_incl_scan(w);
            if (lane < 16)
                wsum[lane] = wi - w;
        }
        __syncthreads();
        int run = carry_s + wsum[wid] + incl - sum;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t i = c0 + 4 * tid + u;
            if (i < p.T) {
                off[i] = run;
                cnt[i] = 0;
            }
            run += v[u];
        }
        __syncthreads();
        if (tid == 1023)
            carry_s = run;
        __syncthreads();
    }
    if (tid == 0)
        off[p.T] = carry_s;
}

__global__ void scatter_fill_kernel(ScatterParams p)
{
    const int64_t s = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= p.T)
        return;
    const int64_t e = p.end[s * p.T + t];
    if (e >= 0 && e + 1 < p.T) {
        const int slot = p.off[s * p.Tq + e + 1] + atomicAdd(&p.cnt[s * p.T + e + 1], 1);
        p.list[s * p.T + slot] = (int32_t)t;
    }
}

// XCDs of the chip: consecutive workgroups of a launch go to consecutive
// XCDs, round robin.
constexpr int kScXcds = 8;
constexpr int kSumTP = 64;          // destination rows per tile
constexpr int64_t kSumW = 128;      // workgroups per XCD

// One destination row tau of route r: its time steps in increasing order.
template <int MC>
__device__ __forceinline__ void scatter_sum_one(const ScatterParams &p, int64_t b, int64_t r,
                                                int64_t tau)
{
    const int64_t s = b * p.R + r;
    const int o0 = p.off[s * p.Tq + tau], o1 = p.off[s * p.Tq + tau + 1];
    const int n = o1 - o0;
    float *g = p.G + (b * p.T + tau) * p.ldg + r * MC;
    if (n > kSelectMax) {
        const int idx = atomicAdd(&p.big[0], 1);
        if (idx < p.big_cap) {
            p.big[64 + 2 * (int64_t)idx] = (int32_t)s;
            p.big[64 + 2 * (int64_t)idx + 1] = (int32_t)tau;
        }
        return;
    }
    double acc[MC];
#pragma unroll
    for (int m = 0; m < MC; ++m)
        acc[m] = 0.0;
    if (p.skip0) {
        // the lists leave out t = 0, the first term of the sum in t order
        const int32_t e0 = p.end[s * p.T];
        if (e0 >= 0 && (int64_t)e0 + 1 == tau) {
            const float *th = p.theta + b * p.T * p.ldt + r * MC;
#pragma unroll
            for (int m = 0; m < MC; ++m)
                acc[m] += (double)th[m];
        }
    }
    const int32_t *lst = p.list + s * p.T;
    int prev = -1;
    for (int k = 0; k < n; ++k) {
        int tmin = 0x7FFFFFFF;
        for (int i = o0; i < o1; ++i) {
            const int t = lst[i];
            if (t > prev && t < tmin)
                tmin = t;
        }
        prev = tmin;
        const float *th = p.theta + (b * p.T + tmin) * p.ldt + r * MC;
#pragma unroll
        for (int m = 0; m < MC; ++m)
            acc[m] += (double)th[m];
    }
#pragma unroll
    for (int m = 0; m < MC; ++m)
        g[m] = (float)acc[m];
}

// Tile: kSumTP destination rows x RG routes of one batch row, 256 threads
// (RG consecutive threads = the routes of one row, so the rows of G are
// written RG routes at a time).  The theta rows a destination reads lie a
// few thousand rows after it, at random, each read MC floats wide; as in the
// value gather, the route groups are dealt to the XCDs in passes and each
// XCD walks its group's destinations in order with W workgroups, so the
// theta lines of a group stay in that XCD's L2 between the reads of the
// group's routes.  RG = 8 (one 128-byte line of theta per row at MC = 4)
// unless the row pitch is a multiple of 2 KiB, where rows alias into few L2
// sets and RG = 16 does better (chosen by timing on the long workload).
template <int MC, int RG>
__global__ __launch_bounds__(256) void scatter_sum_kernel(ScatterParams p, int W)
{
    constexpr int PSTEP = 256 / RG;
    const int64_t ng = (p.R + RG - 1) / RG, ntt = (p.T + kSumTP - 1) / kSumTP;
    const int x = (int)(blockIdx.x % kScXcds), jw = (int)(blockIdx.x / kScXcds);
    const int64_t b = blockIdx.y;
    const int tid = threadIdx.x;
    for (int64_t k = jw;; k += W) {
        const int64_t pass = k / ntt, tt = k - pass * ntt;
        const int64_t g = pass * kScXcds + x;
        if (g >= ng)
            break;
        const int64_t r = g * RG + tid % RG;
        if (r >= p.R)
            continue;
        for (int i = 0; i < kSumTP / PSTEP; ++i) {
            const int64_t tau = tt * kSumTP + tid / RG + (int64_t)PSTEP * i;
            if (tau < p.T)
                scatter_sum_one<MC>(p, b, r, tau);
        }
    }
}

// Streams of up to 65536 positions: count, prefix and fill of one stream in
// one workgroup, with the per-destination counters in LDS (two 16-bit
// halves per word).  The time step t = 0 is left out of the lists (the sum
// kernel adds its term first), so at most T-1 <= 65535 steps are counted:
// no count, prefix or list slot leaves 16 bits, whatever the destinations
// (a prefix plus its count never exceeds the number of counted steps).
constexpr int kScatterLdsT = 65536;

__global__ __launch_bounds__(1024) void scatter_group_lds_kernel(ScatterParams p)
{
    __shared__ uint32_t c2[kScatterLdsT / 2];   // 128 KiB
    __shared__ int wsum[16];
    __shared__ int carry_s;
    const int64_t s = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int T = (int)p.T;
    const int32_t *E = p.end + s * p.T;
    const int nwords = (T + 1) / 2;
    // visits (t, E[t]) for every t of the stream; with 16-byte aligned rows
    // of a multiple of 4 positions, 4 per load and all of a thread's loads
    // (16 at T = 65536) in flight before the first is used, so the pass
    // waits for memory once rather than once per position
    constexpr int kEIt = kScatterLdsT / (4 * 1024);
    const bool vec = (T & 3) == 0 && (((uintptr_t)E) & 15) == 0;
    auto each = [&](auto fn) {
        if (vec) {
            const int4 *E4 = reinterpret_cast<const int4 *>(E);
            const int n4 = T >> 2;
            int4 ev[kEIt];
#pragma unroll
            for (int j = 0; j < kEIt; ++j) {
                const int i = tid + j * 1024;
                ev[j] = i < n4 ? E4[i] : make_int4(-1, -1, -1, -1);
            }
#pragma unroll
            for (int j = 0; j < kEIt; ++j) {
                const int t0 = 4 * (tid + j * 1024);
                fn(t0, ev[j].x);
                fn(t0 + 1, ev[j].y);
                fn(t0 + 2, ev[j].z);
                fn(t0 + 3, ev[j].w);
            }
        } else {
            for (int t = tid; t < T; t += 1024)
                fn(t, E[t]);
        }
    };
    for (int i = tid; i < nwords; i += 1024)
        c2[i] = 0u;
    if (tid == 0)
        carry_s = 0;
    __syncthreads();
    each([&](int t, int e) {
        if (t > 0 && e >= 0 && e + 1 < T) {
            const int tau = e + 1;
            atomicAdd(&c2[tau >> 1], 1u << (16 * (tau & 1)));
        }
    });
    __syncthreads();
    // exclusive prefix, 4096 destinations per round (4 per thread); the
    // prefix goes to off[] for the sum kernel and back into c2 as cursors
    int32_t *off = p.off + s * p.Tq;
    for (int c0 = 0; c0 < T; c0 += 4096) {
        const int w0 = (c0 >> 1) + 2 * tid;
        const uint32_t a = w0 < nwords ? c2[w0] : 0u;
        const uint32_t b = w0 + 1 < nwords ? c2[w0 + 1] : 0u;
        const int v0 = (int)(a & 0xFFFFu), v1 = (int)(a >> 16);
        const int v2 = (int)(b & 0xFFFFu), v3 = (int)(b >> 16);
        const int sum = v0 + v1 + v2 + v3;
        const int incl = sc_wave_incl_scan(sum);
        if (lane == 63)
            wsum[wid] = incl;
        __syncthreads();
        if (wid == 0) {
            const int w = lane < 16 ? wsum[lane] : 0;
            const int wi = sc_wave_incl_scan(w);
            if (lane < 16)
                wsum[lane] = wi - w;
        }
        __syncthreads();
        const int r0 = carry_s + wsum[wid] + incl - sum;
        const int r1 = r0 + v0, r2 = r1 + v1, r3 = r2 + v2;
        const int tau0 = c0 + 4 * tid;
        if (tau0 < T)
            off[tau0] = r0;
        if (tau0 + 1 < T)
            off[tau0 + 1] = r1;
        if (tau0 + 2 < T)
            off[tau0 + 2] = r2;
        if (tau0 + 3 < T)
            off[tau0 + 3] = r3;
        if (w0 < nwords)
            c2[w0] = (uint32_t)r0 | ((uint32_t)r1 << 16);
        if (w0 + 1 < nwords)
            c2[w0 + 1] = (uint32_t)r2 | ((uint32_t)r3 << 16);
        __syncthreads();
        if (tid == 1023)
            carry_s = r3 + v3;
        __syncthreads();
    }
    if (tid == 0)
        off[T] = carry_s;
    __syncthreads();
    int32_t *list = p.list + s * p.T;
    each([&](int t, int e) {
        if (t > 0 && e >= 0 && e + 1 < T) {
            const int tau = e + 1;
            const uint32_t sh = 16u * (uint32_t)(tau & 1);
            const uint32_t old = atomicAdd(&c2[tau >> 1], 1u << sh);
            list[(old >> sh) & 0xFFFFu] = t;
        }
    });
}

// One wave per destination with many time steps: the stream's time steps
// are visited in order, 64 at a time; lanes m < M hold channel m's sum.
template <int MC>
__global__ __launch_bounds__(64) void scatter_big_kernel(ScatterParams p)
{
    const int lane = threadIdx.x;
    const int64_t nbig = min((int64_t)p.big[0], p.big_cap);
    for (int64_t w = blockIdx.x; w < nbig; w += gridDim.x) {
        const int64_t s = p.big[64 + 2 * w], tau = p.big[64 + 2 * w + 1];
        const int64_t b = s / p.R, r = s % p.R;
        const int32_t *E = p.end + s * p.T;
        double acc = 0.0;
        for (int64_t c0 = 0; c0 < p.T; c0 += 64) {
            const int64_t t = c0 + lane;
            const bool hit = t < p.T && (int64_t)E[t] + 1 == tau;
            uint64_t mask = __ballot(hit);
            while (mask) {
                const int j = __ffsll((long long)mask) - 1;
                mask &= mask - 1;
                if (lane < MC)
                    acc += (double)p.theta[(b * p.T + c0 + j) * p.ldt + r * MC + lane];
            }
        }
        if (lane < MC)
            p.G[(b * p.T + tau) * p.ldg + r * MC + lane] = (float)acc;
    }
}

hipError_t launch_scatter(const ScatterParams &p_in, hipStream_t st)
{
    ScatterParams p = p_in;
    p.skip0 = p.T <= kScatterLdsT ? 1 : 0;
    const int64_t S = p.B * p.R;
    hipLaunchKernelGGL(scatter_zero_kernel, dim3(1), dim3(64), 0, st, p.big,
                       (int64_t)64);
    if (p.T <= kScatterLdsT) {
        hipLaunchKernelGGL(scatter_group_lds_kernel, dim3((unsigned)S), dim3(1024),
                           0, st, p);
    } else {
        hipLaunchKernelGGL(scatter_zero_kernel, dim3(1024), dim3(256), 0, st,
                           p.cnt, S * p.T);
        const dim3 gt((unsigned)((p.T + 255) / 256), (unsigned)S);
        hipLaunchKernelGGL(scatter_count_kernel, gt, dim3(256), 0, st, p);
        hipLaunchKernelGGL(scatter_scan_kernel, dim3((unsigned)S), dim3(1024), 0,
                           st, p);
        hipLaunchKernelGGL(scatter_fill_kernel, gt, dim3(256), 0, st, p);
    }
    const bool aliased = ((p.ldt * 4) % 2048) == 0;
    const int rg = aliased ? 16 : 8;
    const int64_t per_xcd = ((p.R + rg - 1) / rg + kScXcds - 1) / kScXcds *
                            ((p.T + kSumTP - 1) / kSumTP);
    const int W = (int)(per_xcd < kSumW ? per_xcd : kSumW);
    const dim3 gs((unsigned)(kScXcds * W), (unsigned)p.B);
    const unsigned gb = 1024;
    switch (p.M) {
#define ROSA_SCATTER_M(MM)                                                             \
    case MM:                                                                           \
        if (aliased)                                                                   \
            hipLaunchKernelGGL((scatter_sum_kernel<MM, 16>), gs, dim3(256), 0, st, p, W); \
        else                                                                           \
            hipLaunchKernelGGL((scatter_sum_kernel<MM, 8>), gs, dim3(256), 0, st, p, W);  \
        hipLaunchKernelGGL(scatter_big_kernel<MM>, dim3(gb), dim3(64), 0, st, p);      \
        break;
        ROSA_SCATTER_M(1)
        ROSA_SCATTER_M(2)
        ROSA_SCATTER_M(3)
        ROSA_SCATTER_M(4)
        ROSA_SCATTER_M(5)
        ROSA_SCATTER_M(6)
        ROSA_SCATTER_M(7)
        ROSA_SCATTER_M(8)
#undef ROSA_SCATTER_M
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rosa
