// Internal declarations shared by the host planner (gdn_plan.cpp) and the
// kernels (gdn_fwd.hip, gdn_bwd.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/gdn.h"

// Functions the planner and the kernels share; host-only when the planner is
// built by the host compiler alone (the sanitizer tests).
#if defined(__HIPCC__)
#define GDN_HD __host__ __device__
#else
#define GDN_HD
#endif

namespace gdn {

constexpr int kChunk = 64;     // chunk length C
constexpr int kDimK = 128;     // key/query head dim K
constexpr int kDimV = 128;     // value head dim V
constexpr int kNumCUs = 256;   // MI355X compute units (occupancy model of the AUTO planner)
// ln(2^-24): once the summed log-gates of a warm-up window fall to this, the
// zero-start state differs from the true one by less than fp32 resolution
// (relative to the state at the window's far end).
constexpr float kLnNoiseFloor = -16.635532333438686f;

// One context-parallel segment of one sequence: chunks [c_begin, c_begin + c_count).
struct SegEntry {
    int32_t n;         // sequence index (-1: no such segment)
    int32_t c_begin;   // first chunk of the segment, counted from the sequence start
    int32_t c_count;   // chunks in the segment (0 only for an empty sequence)
    int32_t seq_len;   // tokens in the sequence
    int64_t row0;      // row of the sequence's first token in the flattened [B*T] axis
    int32_t last;      // 1 if this segment ends its sequence (writes final_state)
    int32_t pad;
};

// Integer segment rule, identical on host and device: a sequence of `len`
// tokens has ceil(len / C) chunks and max(1, ceil(chunks / L)) segments.
GDN_HD inline int32_t seq_chunks(int64_t len) {
    return (int32_t)((len + kChunk - 1) / kChunk);
}
GDN_HD inline int32_t seq_segments(int64_t len, int32_t L) {
    const int32_t nt = seq_chunks(len);
    const int32_t s = (nt + L - 1) / L;
    return s > 0 ? s : 1;
}

struct FwdParams {
    const uint16_t *q, *k, *v;   // bf16 bits
    const float *g, *beta, *h0;
    const int32_t *cu;           // device offsets or nullptr
    void *o;
    float *ht;
    int64_t T;                   // tokens per batch row
    int64_t rows;                // B * T
    int32_t B, N, Hqk, Hv, group;
    int32_t num_segments;
    int32_t L;                   // segment length in chunks
    int32_t cp_mode;             // resolved gdn_cp_mode
    int32_t warmup_cap;          // WARMUP window cap in chunks; 0: none (gate-driven)
    int32_t o_f32;
    float scale;
    // exact context parallelism (workspace, each [num_segments][Hv][K][V] fp32):
    // per-segment zero-start state S, transition map M, and segment-start state H
    float *ws_s, *ws_m, *ws_h;
    // optional low-level outputs: per-chunk start states, per-chunk WY matrices,
    // per-chunk v' = U - W h ([total_chunks][Hv][64][V], chunk-padded; for the backward)
    float *h_out, *a_out, *vn_out;
};

// Backward (gdn_bwd.hip): reverse pass over segments, then chunk-local gradients
// (which also sum dq and dk over each key head's v-heads).
struct BwdParams {
    const uint16_t *q, *k, *v, *dO;  // bf16 bits
    const float *g, *beta;
    const int32_t *cu;               // device offsets or nullptr
    const float *h;                  // [total_chunks][Hv][K][V] chunk-start states (forward's low-level h)
    const float *A;                  // [rows][Hv][64] WY matrices (forward's low-level A)
    const float *vn;                 // [total_chunks][Hv][64][V] v' of every chunk (forward's v_new)
    const float *dht;                // [N][Hv][K][V] or nullptr
    float *dh_ws;                    // [total_chunks][Hv][2][K][V] bf16 (hi, lo): gradient wrt the state after each chunk
    float *dvp_ws;                   // [total_chunks][Hv][2][64][V] bf16 (hi, lo): dv' (all 64 rows of every chunk)
    float *dq_ws, *dk_ws;            // [rows][H_qk][K] fp32 running sums of dq, dk over a key head's v-heads
    void *dq, *dk, *dv;              // bf16 or fp32 per grad_f32
    float *dg, *dbeta;               // [rows][Hv]
    float *dh0;                      // [N][Hv][K][V] or nullptr
    int64_t T, rows;
    int32_t N, Hqk, Hv, group;
    int32_t num_segments, L, cp_mode, warmup_cap;  // reverse pass
    // exact context parallelism of the reverse pass (workspace, each
    // [num_segments][Hv][K][V] fp32): per-segment zero-start result S, transition
    // map M (K x K), and the segment-end gradient each segment starts from
    float *ws_s, *ws_m, *ws_h;
    int32_t pass;                    // reverse-pass kernel: 0 main, 1 exact-CP pre-pass (S and M)
    int32_t num_chunk_entries;       // chunk-local grid: chunks of all sequences + one per empty sequence
    int32_t grad_f32;
    float scale;
};

// Launchers (gdn_fwd.hip, gdn_bwd.hip).  Each returns the hipError_t of its launch as int.
int launch_fwd_main(const FwdParams &p, void *stream);
int launch_cp_exact(const FwdParams &p, void *stream);  // pre-pass + combine
int launch_chunk_cumsum(const float *g, float *out, int64_t B, int64_t T, int32_t H, int32_t chunk,
                        const int32_t *cu, int32_t N, void *stream);
int launch_bwd(const BwdParams &p, void *stream);
const char *hip_error_text(int err);

// Planner helpers for the allocation-free entry point (gdn_api.hip): the
// thread's error message, and the workspace a forward call plans (validating it).
int set_error(int status, const char *msg);
int fwd_workspace_bytes(const gdn_fwd_desc *d, size_t *bytes);

}  // namespace gdn
