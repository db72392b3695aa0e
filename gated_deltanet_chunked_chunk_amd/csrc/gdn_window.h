// The warm-up window of gate-decay context parallelism (agentlenshq.com
// FlashQLA blog, "gate-driven automatic intra-card context parallelism": the
// influence of past state decays with the gates, so a segment can start from
// a state rebuilt over the chunks before it instead of the exact one).  Shared
// by the forward (the window precedes a segment) and the backward's reverse
// pass (the window follows it: the state gradient decays with the same gates).
//
// Two states run from different starts over the same tokens differ by a
// matrix that each token multiplies by exp(g_t) (I - beta_t k_t k_t^T), whose
// norm is at most exp(g_t) for unit keys and beta in [0, 2].  A window whose
// summed log-gates reach ln 2^-24 therefore leaves an error below fp32
// resolution relative to the state at the window's far end; the window grows
// chunk by chunk until that holds or the sequence edge is reached (where the
// walk starts from the exact boundary state).
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float window_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}

// Inclusive prefix sum over the 64 lanes (DPP row shifts, then row broadcasts).
__device__ __forceinline__ float window_prefix64(float x) {
    x += window_dpp<0x111, 0xf>(x);  // row_shr:1
    x += window_dpp<0x112, 0xf>(x);  // row_shr:2
    x += window_dpp<0x114, 0xf>(x);  // row_shr:4
    x += window_dpp<0x118, 0xf>(x);  // row_shr:8
    x += window_dpp<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += window_dpp<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Length in chunks of the warm-up window that starts at chunk c0 and walks in
// direction dir (-1: towards the sequence start, +1: towards its end) over at
// most `avail` chunks (and at most `cap` when cap > 0): the smallest w whose
// chunks c0, c0 + dir, ..., c0 + dir (w - 1) sum their log-gates to ln 2^-24
// or below, else the limit.  g points at the sequence's first token row of
// log-gates ([rows][Hv], head j); tokens past seq_len count as zero.  Every lane
// returns the same value.  The gates are read 16 chunks per round first (four
// lanes per chunk), then 64 (one lane per chunk), with every load of a round
// independent of the others, so even a window over a whole long sequence costs
// a few dependent memory round trips.
__device__ __forceinline__ int gate_window(const float *g, const int Hv, const int j, const int seq_len, const int c0,
                                           const int dir, const int avail, const int cap, const int lane) {
    const int lim = (cap > 0 && cap < avail) ? cap : avail;
    float acc = 0.f;
    int base = 0;
    bool first = true;
    while (base < lim) {
        float part = 0.f;
        int i;
        if (first) {
            i = base + (lane >> 2);
            if (i < lim) {
                const int64_t tok0 = (int64_t)(c0 + dir * i) * kChunk + 16 * (lane & 3);
#pragma unroll
                for (int t = 0; t < 16; ++t)
                    if (tok0 + t < seq_len) part += g[(tok0 + t) * Hv + j];
            }
        } else {
            i = base + lane;
            if (i < lim) {
                const int64_t tok0 = (int64_t)(c0 + dir * i) * kChunk;
#pragma unroll 16
                for (int t = 0; t < kChunk; ++t)
                    if (tok0 + t < seq_len) part += g[(tok0 + t) * Hv + j];
            }
        }
        const float run = acc + window_prefix64(part);  // through this lane's tokens of the round
        const bool chunk_end = first ? ((lane & 3) == 3) : true;
        const uint64_t hit = __ballot(chunk_end && i < lim && run <= kLnNoiseFloor);
        if (hit) {
            const int l = __ffsll((long long)hit) - 1;
            return (first ? base + (l >> 2) : base + l) + 1;
        }
        acc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(run), 63));
        base += first ? 16 : 64;
        first = false;
    }
    return lim;
}

}  // namespace gdn
