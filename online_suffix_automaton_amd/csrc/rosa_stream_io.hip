// rosa_stream_io.hip -- streaming kernels of librosa: symbol preparation,
// bf16 discretisation and value gather.  All HBM-bound; each is laid out so
// that global reads and writes are coalesced and the [B][T][D] <-> [S][T]
// transposes happen in LDS.
//
// Method: "ROSA-Tuning: Enhancing Long-Context Modeling via Suffix Matching"
// (arXiv 2602.02499), Sec. 3.2 (Eq. 10-15: sign bits packed M per route) and
// App. C.4 with Eq. (17) (read-out at tau = E+1, zero without a hit).
#include "rosa_internal.h"

namespace rosa {

// I[h > 0] on a bf16 bit pattern, as an integer range test: the positive
// non-NaN patterns are exactly 0x0001 (smallest subnormal) .. 0x7F80 (+inf).
__device__ __forceinline__ uint32_t bf16_pos(uint32_t h)
{
    return (h - 1u) < 0x7F80u ? 1u : 0u;
}

// ------------------------------------------------------------ symbol prep

// Copies caller symbols [S][ld] into padded workspace rows (zero padding on
// both sides), clamps values >= K to K-1 and raises the sticky flag for them.
__global__ void prep_symbols_kernel(const uint8_t *__restrict__ in, int64_t ld,
                                    int64_t T, int32_t K,
                                    uint8_t *__restrict__ rows, int64_t Tp,
                                    uint8_t *__restrict__ copy_out,
                                    int32_t *__restrict__ flags)
{
    const int64_t s = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 0..Tp-1
    if (i >= Tp)
        return;
    const int64_t t = i - kPadFront;
    uint8_t v = 0;
    if (t >= 0 && t < T) {
        v = in[s * ld + t];
        if (v >= K) {
            atomicOr(&flags[kFlagSymbol], 1);
            v = (uint8_t)(K - 1);
        }
        if (copy_out)
            copy_out[s * T + t] = v;
    }
    rows[s * Tp + i] = v;
}

// Zeroes the 64-word headers at a and b (b may be null).
__global__ void clear_flags_kernel(int32_t *a, int32_t *b)
{
    if (threadIdx.x < 64) {
        a[threadIdx.x] = 0;
        if (b)
            b[threadIdx.x] = 0;
    }
}

// --------------------------------------------------------- discretisation

// Tile: 64 positions x 64 routes of one batch row.  256 threads = 4 waves;
// wave w discretises positions t0+16w .. t0+16w+15, lane = route, reading the
// route's M channels (coalesced along the row), into an LDS tile [route][t];
// then the tile is written out as 64-byte runs of each stream's row.  Tiles
// are numbered route tile fastest, so consecutive workgroups read the
// consecutive 512-byte pieces of the same rows of H (whole rows at a time:
// 18% faster than position tiles fastest); a workgroup loops over tiles
// with the grid's stride, so any T fits the grid.
// With pad_end > 0 the first and last position tiles also zero the row
// bytes before row_off and from row_off + T to pad_end, and the first block
// zeroes the 64-word headers zero_a and zero_b (each may be null): the
// launches that would do this separately are folded in here.
template <int MC>
__global__ __launch_bounds__(256) void discretize_kernel(
    const uint16_t *__restrict__ H, int64_t T, int64_t D, int64_t ld, int M,
    uint8_t *__restrict__ rows, int64_t row_stride, int64_t row_off,
    uint8_t *__restrict__ copy_out, int64_t pad_end, int32_t *zero_a,
    int32_t *zero_b)
{
    if ((blockIdx.x | blockIdx.y) == 0 && threadIdx.x < 64) {
        if (zero_a)
            zero_a[threadIdx.x] = 0;
        if (zero_b)
            zero_b[threadIdx.x] = 0;
    }
    __shared__ uint8_t tile[64][64 + 4];
    const int64_t R = D / M;
    const int64_t b = blockIdx.y;
    const int64_t nrt = (R + 63) / 64, ntt = (T + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    for (int64_t tile_i = blockIdx.x; tile_i < nrt * ntt; tile_i += gridDim.x) {
        const int64_t tt = tile_i / nrt;
        const int64_t t0 = tt * 64;
        const int64_t r0 = (tile_i - tt * nrt) * 64;
        const int64_t r = r0 + lane;
        if (MC == 4) {
            // four channels in one 8-byte load (alignment checked on host); all
            // 16 loads of the thread in flight before they are used
            uint2 v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int64_t t = t0 + w * 16 + k;
                v[k] = make_uint2(0u, 0u);
                if (t < T && r < R)
                    v[k] = *reinterpret_cast<const uint2 *>(H + (b * T + t) * ld + r * M);
            }
#pragma unroll
            for (int k = 0; k < 16; ++k)
                tile[lane][w * 16 + k] =
                    (uint8_t)(bf16_pos(v[k].x & 0xFFFFu) | (bf16_pos(v[k].x >> 16) << 1) |
                              (bf16_pos(v[k].y & 0xFFFFu) << 2) |
                              (bf16_pos(v[k].y >> 16) << 3));
        } else {
            for (int k = 0; k < 16; ++k) {
                const int tl = w * 16 + k;
                const int64_t t = t0 + tl;
                uint32_t a = 0;
                if (t < T && r < R) {
                    const uint16_t *h = H + (b * T + t) * ld + r * M;
                    for (int j = 0; j < M; ++j)
                        a |= bf16_pos(h[j]) << j;
                }
                tile[lane][tl] = (uint8_t)a;
            }
        }
        __syncthreads();
        // write: thread i -> route i/4, 16 positions starting at (i%4)*16
        const int rr = threadIdx.x >> 2;
        const int tc = (threadIdx.x & 3) * 16;
        const int64_t rg = r0 + rr;
        if (rg < R) {
            const int64_t s = b * R + rg;
            if (pad_end > 0) {
                uint8_t *row = rows + s * row_stride;
                const int q4 = threadIdx.x & 3;
                if (tt == 0)
                    for (int64_t i = q4; i < row_off; i += 4)
                        row[i] = 0;
                if (tt == ntt - 1)
                    for (int64_t i = row_off + T + q4; i < pad_end; i += 4)
                        row[i] = 0;
            }
            uint8_t *dst = rows + s * row_stride + row_off + t0 + tc;
            if (t0 + tc + 16 <= T && (((uintptr_t)dst) & 15) == 0) {
                uint4 v;
                uint32_t *vv = reinterpret_cast<uint32_t *>(&v);
                for (int q = 0; q < 4; ++q)
                    vv[q] = (uint32_t)tile[rr][tc + 4 * q] |
                            ((uint32_t)tile[rr][tc + 4 * q + 1] << 8) |
                            ((uint32_t)tile[rr][tc + 4 * q + 2] << 16) |
                            ((uint32_t)tile[rr][tc + 4 * q + 3] << 24);
                *reinterpret_cast<uint4 *>(dst) = v;
            } else {
                for (int q = 0; q < 16; ++q)
                    if (t0 + tc + q < T)
                        dst[q] = tile[rr][tc + q];
            }
            if (copy_out) {
                uint8_t *c = copy_out + s * T + t0 + tc;
                for (int q = 0; q < 16; ++q)
                    if (t0 + tc + q < T)
                        c[q] = tile[rr][tc + q];
            }
        }
        __syncthreads();   // the tile is rewritten by the next iteration
    }
}

// ----------------------------------------------------------------- gather

// XCDs of the chip (consecutive workgroups of a launch go to consecutive
// XCDs, round robin); the gather's positions per tile and workgroups per XCD.
constexpr int kXcds = 8;
constexpr int kGatherTP = 128;
constexpr int64_t kGatherW = 128;

// Tile: kGatherTP positions x RG routes of one batch row, 256 threads.  The reads of a route go to random earlier rows (tau = E+1,
// inherent to the method; half of them within about 4K rows, nine in ten
// within 27K on i.i.d. streams), and with M = 4 each 128-byte line of a V
// row holds the values of 16 routes, read by them at different positions.
// So the kernel keeps those lines in L2 between the reads: the route groups
// are dealt to the 8 XCDs (group g to XCD g % 8; workgroup i runs on XCD
// i % 8), an XCD does its groups one after another, and inside a group its
// W workgroups walk the positions in order, side by side.  The lines of the
// recent rows of one group then mostly fit the XCD's 4 MiB L2.  E and the
// output are streamed with non-temporal accesses so that they do not push
// those lines out.  With a row pitch that is a multiple of 2 KiB every row's
// line of a group falls into the same few L2 sets, which holds far fewer
// rows: there two lines per row and group (RG = 32) do best, otherwise one
// (RG = 16).  Tile length and W were chosen by timing on the long workload
// (fewer workgroups in flight lose memory parallelism).
template <int MC, int RG>
__global__ __launch_bounds__(256) void gather_kernel(
    const uint16_t *__restrict__ V, int64_t T, int64_t D, int64_t ldv, int M,
    const int32_t *__restrict__ E, uint16_t *__restrict__ out, int64_t ldo, int W)
{
    constexpr int TP = kGatherTP;
    constexpr int PSTEP = 256 / RG;          // positions per round of values
    constexpr int NV = TP / PSTEP;           // value loads per thread
    __shared__ int32_t et[RG][TP + 1];
    const int64_t R = D / M;
    const int64_t b = blockIdx.y;
    const int64_t ng = (R + RG - 1) / RG, ntt = (T + TP - 1) / TP;
    const int x = (int)(blockIdx.x % kXcds), jw = (int)(blockIdx.x / kXcds);
    const int tid = threadIdx.x;
    for (int64_t k = jw;; k += W) {
        const int64_t pass = k / ntt, tt = k - pass * ntt;
        const int64_t g = pass * kXcds + x;
        if (g >= ng)
            break;
        const int64_t t0 = tt * TP, r0 = g * RG;
        // E tile: consecutive threads read consecutive positions of a route
        for (int idx = tid; idx < RG * TP; idx += 256) {
            const int rl = idx / TP, tl = idx % TP;
            const int64_t r = r0 + rl;
            int32_t e = -1;
            if (r < R && t0 + tl < T) {
                e = __builtin_nontemporal_load(E + (b * R + r) * T + t0 + tl);
                if (e < -1) e = -1;
                if (e > T - 2) e = (int32_t)(T - 2);
            }
            et[rl][tl] = e;
        }
        __syncthreads();
        // values: RG consecutive threads = the routes of one position
        const int rl = tid % RG;
        const int64_t r = r0 + rl;
        if (r < R && MC == 4) {
            uint64_t v[NV];
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int tl = tid / RG + PSTEP * i;
                const int32_t e = et[rl][tl];
                v[i] = 0;
                if (t0 + tl < T && e >= 0)
                    v[i] = *reinterpret_cast<const uint64_t *>(
                        V + (b * T + (e + 1)) * ldv + r * M);
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int64_t t = t0 + tid / RG + PSTEP * i;
                if (t < T)
                    __builtin_nontemporal_store(
                        v[i], reinterpret_cast<uint64_t *>(out + (b * T + t) * ldo + r * M));
            }
        } else if (r < R) {
            for (int i = 0; i < NV; ++i) {
                const int tl = tid / RG + PSTEP * i;
                const int64_t t = t0 + tl;
                if (t >= T)
                    break;
                const int32_t e = et[rl][tl];
                uint16_t *o = out + (b * T + t) * ldo + r * M;
                const uint16_t *src = V + (b * T + (e + 1)) * ldv + r * M;
                for (int m = 0; m < M; ++m)
                    o[m] = e >= 0 ? src[m] : (uint16_t)0;
            }
        }
        __syncthreads();   // the E tile is rewritten by the next iteration
    }
}

// --------------------------------------------------------------- launchers

// Workgroups of the tiled kernels (beyond this, each loops over tiles).
constexpr int64_t kTileGrid = 1 << 20;

hipError_t launch_prep_symbols(const uint8_t *in, int64_t ld, int64_t S,
                               int64_t T, int32_t K, uint8_t *rows, int64_t Tp,
                               uint8_t *copy_out, int32_t *flags,
                               hipStream_t st)
{
    dim3 grid((unsigned)((Tp + 255) / 256), (unsigned)S);
    hipLaunchKernelGGL(prep_symbols_kernel, grid, dim3(256), 0, st, in, ld, T,
                       K, rows, Tp, copy_out, flags);
    return hipGetLastError();
}

hipError_t launch_clear_flags(int32_t *flags, hipStream_t st, int32_t *flags2)
{
    hipLaunchKernelGGL(clear_flags_kernel, dim3(1), dim3(64), 0, st, flags, flags2);
    return hipGetLastError();
}

hipError_t launch_discretize(const uint16_t *H, int64_t B, int64_t T,
                             int64_t D, int64_t ld, int M, uint8_t *rows,
                             int64_t row_stride, int64_t row_off,
                             uint8_t *copy_out, hipStream_t st, int64_t pad_end,
                             int32_t *zero_a, int32_t *zero_b)
{
    const int64_t R = D / M;
    const int64_t ntiles = ((R + 63) / 64) * ((T + 63) / 64);
    dim3 grid((unsigned)(ntiles < kTileGrid ? ntiles : kTileGrid), (unsigned)B);
    const bool vec4 = M == 4 && (ld % 4) == 0 &&
                      (((uintptr_t)H) & 7) == 0;
    if (vec4)
        hipLaunchKernelGGL(discretize_kernel<4>, grid, dim3(256), 0, st, H, T,
                           D, ld, M, rows, row_stride, row_off, copy_out,
                           pad_end, zero_a, zero_b);
    else
        hipLaunchKernelGGL(discretize_kernel<0>, grid, dim3(256), 0, st, H, T,
                           D, ld, M, rows, row_stride, row_off, copy_out,
                           pad_end, zero_a, zero_b);
    return hipGetLastError();
}

hipError_t launch_gather(const uint16_t *V, int64_t B, int64_t T, int64_t D,
                         int64_t ldv, int M, const int32_t *E, uint16_t *out,
                         int64_t ldo, hipStream_t st)
{
    // W workgroups per XCD (four per CU), fewer when an XCD has fewer tiles;
    // route groups of one 128-byte line per row unless the row pitch aliases
    const int64_t R = D / M;
    const bool aliased = ((ldv * 2) % 2048) == 0;
    const int rg = aliased ? 32 : 16;
    const int64_t per_xcd = ((R + rg - 1) / rg + kXcds - 1) / kXcds *
                            ((T + kGatherTP - 1) / kGatherTP);
    const int W = (int)(per_xcd < kGatherW ? per_xcd : kGatherW);
    dim3 grid((unsigned)(kXcds * W), (unsigned)B);
    const bool vec4 = M == 4 && (ldv % 4) == 0 && (ldo % 4) == 0 &&
                      (((uintptr_t)V) & 7) == 0 && (((uintptr_t)out) & 7) == 0;
    if (vec4 && aliased)
        hipLaunchKernelGGL((gather_kernel<4, 32>), grid, dim3(256), 0, st, V, T, D,
                           ldv, M, E, out, ldo, W);
    else if (vec4)
        hipLaunchKernelGGL((gather_kernel<4, 16>), grid, dim3(256), 0, st, V, T, D,
                           ldv, M, E, out, ldo, W);
    else if (aliased)
        hipLaunchKernelGGL((gather_kernel<0, 32>), grid, dim3(256), 0, st, V, T, D,
                           ldv, M, E, out, ldo, W);
    else
        hipLaunchKernelGGL((gather_kernel<0, 16>), grid, dim3(256), 0, st, V, T, D,
                           ldv, M, E, out, ldo, W);
    return hipGetLastError();
}

}  // namespace rosa
