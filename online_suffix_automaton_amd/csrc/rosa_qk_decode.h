// rosa_qk_decode.h -- the query/key decode state shared by rosa_sam.hip
// (kernels) and rosa_api.hip (rosa_build_qk / rosa_step_qk).
#pragma once

#include "rosa_internal.h"

namespace rosa {

// Query/key decode state (rosa_build_qk / rosa_step_qk): per stream the
// automaton over the key units (records of RS bytes: node {len, link, last
// unit, clone flag}, then the K-wide transition row), its registers, the
// matching state and the current unit's answers, and the start time of
// every unit.  Regions in QkdLayout, sizes for Ucap = t_capacity units.
// During rosa_build_qk the records' region first holds the batch query/key
// workspace (ws_bytes: room for t_capacity steps), and bscr the batch's E
// and L per time step ([S][T] each) when the caller does not ask for them.
constexpr int kQkdMaxBits = 8;   // counterfactual branches kept per stream

struct QkdLayout {
    size_t flags, meta, mst, cfst, states, start, bscr, total;
    size_t ws_bytes;
    int64_t Ncap, RS;
};
QkdLayout qkd_layout(int64_t S, int64_t K, int64_t Tcap);

struct QkdParams {
    int32_t *flags;         // [0]: a symbol >= K was seen (sticky)
    int4 *meta;             // [S] automaton {tail, states, tail length, tail link}
    int4 *mst;              // [S][2] {unit, match state, match length, previous key},
                            //        {query symbol of the unit, E, L, destination}
    int2 *cfst;             // [S][kQkdMaxBits] {E, destination} of each flipped query bit
    int32_t *states;        // [S][Ncap] records of RS / 4 ints
    int32_t *start;         // [S][Ucap] first time of each unit
    int64_t S, Ncap, RSi, Ucap;
    int32_t K, M, rle, init;
    // input: kind 0 symbols [S][ld] bytes, kind 1 bf16 [B][Tin][ld] elements
    // (route r of row b reads channels r*Min .. r*Min+Min-1); input index i
    // is time t0 + i; ldq and ldk are the two inputs' row strides
    int32_t kind, Min;
    const void *q, *k;
    int64_t ldq, ldk, R, Tin, t0, n;
    // outputs at index s*ostride + i (counterfactual: ((s*ostride + i)*M + j)*2 + v)
    int64_t ostride;
    int32_t *tau, *end, *len, *run_of, *run_start, *ridx, *cf_tau, *cf_ridx;
};
hipError_t launch_qkd(const QkdParams &p, hipStream_t st);
hipError_t launch_qkd_prefix(const QkdParams &p, const int32_t *bend,
                             const int32_t *blen, int64_t bld, hipStream_t st);

}  // namespace rosa
