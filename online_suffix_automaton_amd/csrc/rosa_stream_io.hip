// rosa_stream_io.hip -- streaming kernels of librosa: symbol preparation,
// bf16 discretisation and value gather.  All HBM-bound; each is laid out so
// that global reads are coalesced and writes go in 16-byte or larger pieces.
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
// A thread moves 16 bytes of a padded row; with 16-byte aligned caller rows
// (vec) a chunk inside [0, T) is one vector load and store, its symbols
// checked on whole words (for K a power of two: no bit at or above K's), and
// only a chunk that holds a symbol >= K is clamped byte by byte.  Chunks at
// the row's ends, and unaligned rows, go byte by byte.
__global__ void prep_symbols_kernel(const uint8_t *__restrict__ in, int64_t ld,
                                    int64_t T, int32_t K,
                                    uint8_t *__restrict__ rows, int64_t Tp,
                                    uint8_t *__restrict__ copy_out,
                                    int32_t *__restrict__ flags, int vec)
{
    const int64_t s = blockIdx.y;
    const int64_t i0 = 16 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    if (i0 >= Tp)
        return;
    const int64_t t0 = i0 - kPadFront;
    uint8_t *dst = rows + s * Tp + i0;
    if (vec && t0 >= 0 && t0 + 16 <= T) {
        uint4 v = *reinterpret_cast<const uint4 *>(in + s * ld + t0);
        bool bad;
        if ((K & (K - 1)) == 0) {
            const uint32_t m = (uint32_t)(~(K - 1) & 0xFF) * 0x01010101u;
            bad = ((v.x | v.y | v.z | v.w) & m) != 0;
        } else {
            bad = false;
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 16; ++q)
                bad |= ((w[q >> 2] >> (8 * (q & 3))) & 0xFFu) >= (uint32_t)K;
        }
        if (bad) {
            atomicOr(&flags[kFlagSymbol], 1);
            uint8_t *b = reinterpret_cast<uint8_t *>(&v);
            for (int q = 0; q < 16; ++q)
                if (b[q] >= K)
                    b[q] = (uint8_t)(K - 1);
        }
        *reinterpret_cast<uint4 *>(dst) = v;
        if (copy_out) {
            uint8_t *c = copy_out + s * T + t0;
            if ((((uintptr_t)c) & 15) == 0) {
                *reinterpret_cast<uint4 *>(c) = v;
            } else {
                const uint8_t *b = reinterpret_cast<const uint8_t *>(&v);
                for (int q = 0; q < 16; ++q)
                    c[q] = b[q];
            }
        }
        return;
    }
    for (int q = 0; q < 16 && i0 + q < Tp; ++q) {
        const int64_t t = t0 + q;
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
        dst[q] = v;
    }
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

// The same 64-position x 64-route tiles with M = 4 and 16-byte aligned
// rows (row stride and first symbol), without LDS: lane = route, wave w =
// positions t0+16w .. t0+16w+15 (the same coalesced 512-byte row reads as
// above), and the lane packs its 16 symbols into one 16-byte store of its
// route's row.  The writes are the same 16-byte pieces the LDS kernel
// stores (a workgroup covers 64 bytes of each of 64 rows), so memory sees
// the same pattern; with no LDS and no barrier the kernel can run on a CU
// beside a workgroup that holds all of that CU's LDS (the retrieval
// kernel).  Padding, headers and copy_out as in discretize_kernel.
__global__ __launch_bounds__(256) void discretize4_kernel(
    const uint16_t *__restrict__ H, int64_t T, int64_t D, int64_t ld,
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
    const int64_t R = D / 4;
    const int64_t b = blockIdx.y;
    const int64_t nrt = (R + 63) / 64, ntt = (T + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    for (int64_t tile_i = blockIdx.x; tile_i < nrt * ntt; tile_i += gridDim.x) {
        const int64_t tt = tile_i / nrt;
        const int64_t tc = tt * 64 + w * 16;   // this wave's first position
        const int64_t r = (tile_i - tt * nrt) * 64 + lane;
        // one pointer stepped by a row per load (the per-load 64-bit index
        // products were most of this kernel's vector instructions, which
        // take issue slots from a retrieval kernel on the same CU)
        const int nk = (int)min<int64_t>(16, T - tc);
        const uint16_t *hp = H + (b * T + tc) * ld + r * 4;
        uint2 v[16];
        if (nk == 16 && r < R) {
#pragma unroll
            for (int k = 0; k < 16; ++k)
                v[k] = *reinterpret_cast<const uint2 *>(hp + k * ld);
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                v[k] = make_uint2(0u, 0u);
                if (k < nk && r < R)
                    v[k] = *reinterpret_cast<const uint2 *>(hp);
                hp += ld;
            }
        }
        if (r >= R)
            continue;
        uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int k = 0; k < 16; ++k)
            wv[k >> 2] |= (bf16_pos(v[k].x & 0xFFFFu) | (bf16_pos(v[k].x >> 16) << 1) |
                           (bf16_pos(v[k].y & 0xFFFFu) << 2) |
                           (bf16_pos(v[k].y >> 16) << 3))
                          << (8 * (k & 3));
        const int64_t s = b * R + r;
        uint8_t *row = rows + s * row_stride;
        if (pad_end > 0) {
            if (tt == 0 && w == 0)
                for (int64_t i = 0; i < row_off; ++i)
                    row[i] = 0;
            if (tt == ntt - 1 && w == 3)
                for (int64_t i = row_off + T; i < pad_end; ++i)
                    row[i] = 0;
        }
        if (tc >= T)
            continue;
        const uint4 pk = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        uint8_t *dst = row + row_off + tc;
        if (tc + 16 <= T) {
            *reinterpret_cast<uint4 *>(dst) = pk;
        } else {
            for (int q = 0; q < T - tc; ++q)
                dst[q] = (uint8_t)(wv[q >> 2] >> (8 * (q & 3)));
        }
        if (copy_out) {
            uint8_t *c = copy_out + s * T + tc;
            if (tc + 16 <= T && (((uintptr_t)c) & 15) == 0) {
                *reinterpret_cast<uint4 *>(c) = pk;
            } else {
                for (int q = 0; q < 16 && tc + q < T; ++q)
                    c[q] = (uint8_t)(wv[q >> 2] >> (8 * (q & 3)));
            }
        }
    }
}

// ----------------------------------------------------------------- gather

// XCDs of the chip (consecutive workgroups of a launch go to consecutive
// XCDs, round robin).
constexpr int kXcds = 8;

// The reads of a route go to random earlier rows (tau = E+1, inherent to
// the method; half of them within about 4K rows, nine in ten within 27K on
// i.i.d. streams), and with M = 4 each 128-byte line of a V row holds the
// values of 16 routes (a route group), read by them at different positions.
// The 8-byte path keeps those lines in L2 between the reads: route groups
// are dealt to the XCDs (workgroup i runs on XCD i % 8), an XCD does its
// groups one after another, and its waves walk a group's positions in order,
// side by side, so the lines of the recent rows of that group sit in the
// XCD's 4 MiB L2.  E and the output are streamed with non-temporal accesses
// so that they do not push those lines out.
//
// Wave layout: a wave covers the 16 routes of a group (lane & 15) and
// kGatherU chunks of 16 positions; lane quad q = lane >> 4 holds positions
// 4q .. 4q+3 of each chunk (one 16-byte E load), so its i-th store writes
// positions i, i+4, i+8, i+12 of the chunk: four whole 128-byte output lines.
// No LDS and no barrier, so each wave keeps its 32 value loads in flight
// independently.  The positions an XCD has in flight (waves x 128) trade
// memory parallelism against the span of rows its L2 must hold; one
// workgroup of 4 waves per CU did best on the long workload.  With a row
// pitch that is a multiple of 2 KiB every row's line of one group falls into
// the same few L2 sets; there an XCD walks two adjacent groups at once
// (GPX = 2: chunks alternate between them), which spreads the lines over
// twice the sets.
constexpr int kGatherU = 8;
constexpr int kGatherChunk = 16 * kGatherU;
constexpr int kGatherWG = 32;   // workgroups of 4 waves per XCD

typedef int32_t gather_v4i __attribute__((ext_vector_type(4)));

// O32 (T, the row pitches in bytes below 2^24, one batch row of V and of
// the output below 4 GiB): each row's byte offset is one 24-bit multiply-add
// on a uniform base, and a lane without a hit reads row 0 and keeps zero by
// a select, so a value load costs a few vector instructions instead of a
// 64-bit index product and a branch (vector instructions here take issue
// slots from a retrieval kernel on the same CU).
template <int GPX, bool O32>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void gather_wave_kernel(
    const uint16_t *__restrict__ V, int64_t T, int64_t R, int64_t ldv,
    const int32_t *__restrict__ E, uint16_t *__restrict__ out, int64_t ldo,
    int vec_e)
{
    constexpr int U = kGatherU, CH = kGatherChunk;
    const int64_t b = blockIdx.y;
    const int64_t ng = (R + 15) / 16, nch = (T + CH - 1) / CH;
    const int x = (int)(blockIdx.x % kXcds);
    const int lane = threadIdx.x & 63;
    // the chunk index is the wave's (scalar arithmetic)
    const int64_t wv = __builtin_amdgcn_readfirstlane(
        (int)(blockIdx.x / kXcds) * 4 + (int)(threadIdx.x >> 6));
    const int64_t Wv = (int64_t)(gridDim.x / kXcds) * 4;
    const int rl = lane & 15, q = lane >> 4;
    for (int64_t c = wv;; c += Wv) {
        // chunk c of this XCD: pass, then GPX groups side by side, chunks
        // alternating between them
        const int64_t pass = c / (nch * GPX), cw = c - pass * (nch * GPX);
        const int64_t first = (pass * kXcds + x) * GPX;
        if (first >= ng)
            break;
        const int64_t g = first + cw % GPX, t0 = (cw / GPX) * CH;
        const int64_t r = g * 16 + rl;
        if (g >= ng || r >= R)
            continue;
        const int32_t *er = E + (b * R + r) * T;
        int32_t e[U][4];
        if (vec_e && t0 + CH <= T) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const gather_v4i w = __builtin_nontemporal_load(
                    reinterpret_cast<const gather_v4i *>(er + t0 + 16 * u + 4 * q));
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    e[u][i] = w[i];
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t t = t0 + 16 * u + 4 * q + i;
                    e[u][i] = t < T ? __builtin_nontemporal_load(er + t) : -1;
                }
        }
        uint64_t v[U][4];
        if constexpr (O32) {
            const unsigned char *vb = reinterpret_cast<const unsigned char *>(V + b * T * ldv);
            const uint32_t lv = (uint32_t)ldv * 2u, col = (uint32_t)r * 8u;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int32_t ee = min(e[u][i], (int32_t)T - 2);
                    const uint32_t row = ee >= 0 ? (uint32_t)(ee + 1) : 0u;
                    const uint64_t w = *reinterpret_cast<const uint64_t *>(
                        vb + (__umul24(row, lv) + col));
                    v[u][i] = ee >= 0 ? w : 0ull;
                }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int32_t ee = e[u][i] > T - 2 ? (int32_t)(T - 2) : e[u][i];
                    v[u][i] = 0;
                    if (ee >= 0)
                        v[u][i] = *reinterpret_cast<const uint64_t *>(
                            V + (b * T + (ee + 1)) * ldv + r * 4);
                }
        }
        if (O32 && t0 + CH <= T) {
            unsigned char *ob = reinterpret_cast<unsigned char *>(out + b * T * ldo);
            const uint32_t lo = (uint32_t)ldo * 2u;
            const uint32_t o0 = (__umul24((uint32_t)(t0 + 4 * q), lo) + (uint32_t)r * 8u);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_nontemporal_store(
                        v[u][i], reinterpret_cast<uint64_t *>(
                                     ob + (o0 + (uint32_t)(16 * u + i) * lo)));
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t t = t0 + 16 * u + 4 * q + i;
                    if (t < T)
                        __builtin_nontemporal_store(
                            v[u][i], reinterpret_cast<uint64_t *>(out + (b * T + t) * ldo + r * 4));
                }
        }
    }
}

// Any M, pitch and alignment: tiles of 128 positions x RG routes of one
// batch row, 256 threads, the E tile staged through LDS so that its loads
// coalesce; route groups dealt to the XCDs as in the 8-byte path.
constexpr int kGatherTP = 128;
constexpr int64_t kGatherW = 128;

template <int RG>
__global__ __launch_bounds__(256) void gather_kernel(
    const uint16_t *__restrict__ V, int64_t T, int64_t D, int64_t ldv, int M,
    const int32_t *__restrict__ E, uint16_t *__restrict__ out, int64_t ldo, int W)
{
    constexpr int TP = kGatherTP;
    constexpr int PSTEP = 256 / RG;          // positions per round of values
    constexpr int NV = TP / PSTEP;           // positions per thread
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
        if (r < R) {
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
    const int vec = (ld % 16) == 0 && (((uintptr_t)in) & 15) == 0;
    const int64_t chunks = (Tp + 15) / 16;
    dim3 grid((unsigned)((chunks + 255) / 256), (unsigned)S);
    hipLaunchKernelGGL(prep_symbols_kernel, grid, dim3(256), 0, st, in, ld, T,
                       K, rows, Tp, copy_out, flags, vec);
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
    const bool rows16 = (row_stride % 16) == 0 &&
                        (((uintptr_t)(rows + row_off)) & 15) == 0;
    if (vec4 && rows16)
        hipLaunchKernelGGL(discretize4_kernel, grid, dim3(256), 0, st, H, T, D, ld,
                           rows, row_stride, row_off, copy_out, pad_end, zero_a,
                           zero_b);
    else if (vec4)
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
    const int64_t R = D / M;
    // a pitch that is a multiple of 2 KiB puts every row's line of a group
    // into the same few L2 sets
    const bool aliased = ((ldv * 2) % 2048) == 0;
    const bool vec8 = M == 4 && (ldv % 4) == 0 && (ldo % 4) == 0 &&
                      (((uintptr_t)V) & 7) == 0 && (((uintptr_t)out) & 7) == 0;
    if (vec8) {
        const int gpx = aliased ? 2 : 1;
        const int64_t ng = (R + 15) / 16;
        const int64_t chunks = (ng + kXcds * gpx - 1) / (kXcds * gpx) * gpx *
                               ((T + kGatherChunk - 1) / kGatherChunk);
        const int64_t wgs = (chunks + 3) / 4;   // 4 waves per workgroup
        const int W = (int)(wgs < kGatherWG ? wgs : kGatherWG);
        const int vec_e = (T % 4) == 0 && (((uintptr_t)E) & 15) == 0;
        dim3 grid((unsigned)(kXcds * W), (unsigned)B);
        const int64_t k24 = (int64_t)1 << 24, k32 = (int64_t)1 << 32;
        const bool o32 = T < k24 && ldv * 2 < k24 && ldo * 2 < k24 && T * ldv * 2 < k32 &&
                         T * ldo * 2 < k32;
        if (aliased && o32)
            hipLaunchKernelGGL((gather_wave_kernel<2, true>), grid, dim3(256), 0, st, V, T,
                               R, ldv, E, out, ldo, vec_e);
        else if (aliased)
            hipLaunchKernelGGL((gather_wave_kernel<2, false>), grid, dim3(256), 0, st, V, T,
                               R, ldv, E, out, ldo, vec_e);
        else if (o32)
            hipLaunchKernelGGL((gather_wave_kernel<1, true>), grid, dim3(256), 0, st, V, T,
                               R, ldv, E, out, ldo, vec_e);
        else
            hipLaunchKernelGGL((gather_wave_kernel<1, false>), grid, dim3(256), 0, st, V, T,
                               R, ldv, E, out, ldo, vec_e);
        return hipGetLastError();
    }
    // other widths: one 128-byte line per row and group unless the pitch
    // aliases; W workgroups per XCD (four per CU), fewer for small inputs
    const int rg = aliased ? 32 : 16;
    const int64_t per_xcd = ((R + rg - 1) / rg + kXcds - 1) / kXcds *
                            ((T + kGatherTP - 1) / kGatherTP);
    const int W = (int)(per_xcd < kGatherW ? per_xcd : kGatherW);
    dim3 grid((unsigned)(kXcds * W), (unsigned)B);
    if (aliased)
        hipLaunchKernelGGL(gather_kernel<32>, grid, dim3(256), 0, st, V, T, D,
                           ldv, M, E, out, ldo, W);
    else
        hipLaunchKernelGGL(gather_kernel<16>, grid, dim3(256), 0, st, V, T, D,
                           ldv, M, E, out, ldo, W);
    return hipGetLastError();
}

}  // namespace rosa
