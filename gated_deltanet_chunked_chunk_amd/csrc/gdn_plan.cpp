// libgdn C ABI: argument validation, context-parallel planning, workspace
// layout, and the entry points that launch through the kernels' launchers
// (gdn_fwd.hip, gdn_bwd.hip).  Plain C++: this file makes no HIP call, so it
// also builds with the host compiler alone (the sanitizer tests do that).
#include <algorithm>
#include <queue>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

constexpr size_t kAlign = 256;

struct Plan {
    int64_t rows = 0;            // B * T
    int32_t N = 0;
    int32_t total_chunks = 0;
    int32_t max_chunks = 0;
    int32_t L = 1;
    int32_t num_segments = 0;
    int32_t cp_mode = GDN_CP_OFF;
    int32_t warmup = 0;
    size_t workspace = 0;
    size_t state_bytes = 0;
};

int32_t count_segments(const gdn_fwd_desc *d, int32_t L) {
    int64_t total = 0;
    if (d->cu_seqlens_host) {
        for (int32_t n = 0; n < d->num_seqs; ++n)
            total += gdn::seq_segments((int64_t)d->cu_seqlens_host[n + 1] - d->cu_seqlens_host[n], L);
    } else {
        total = (int64_t)d->B * gdn::seq_segments(d->T, L);
    }
    return total > INT32_MAX ? INT32_MAX : (int32_t)total;
}

// AUTO's cost of a segment length L: the makespan of the kernel's grid when
// workgroups start in grid order on the first free CU (one resident per CU),
// each taking its segment's chunks plus an expected warm-up (two chunks,
// fewer near a sequence edge) plus half a chunk of fixed cost, in chunk units.
// Varlen batches have segments of unequal length, which a count of workgroup
// waves misses.  Grids too large to simulate cheaply fall back to
// waves x (L + 2).  REVERSE: the warm-up lies after the segment (the backward's
// reverse pass); per_segment: workgroups per (segment, v-head).
double segment_cost(const gdn_fwd_desc *d, int32_t L, int32_t per_segment, bool reverse, double bound) {
    const int64_t wgs = (int64_t)count_segments(d, L) * d->H_v * per_segment;
    if (wgs > 16384) return std::ceil((double)wgs / gdn::kNumCUs) * (L + 2);
    const int32_t nseq = d->cu_seqlens_host ? d->num_seqs : (int32_t)d->B;
    auto seq_len = [&](int32_t n) {
        return d->cu_seqlens_host ? (int64_t)d->cu_seqlens_host[n + 1] - d->cu_seqlens_host[n] : (int64_t)d->T;
    };
    auto job = [&](int32_t nt, int32_t r) {
        const int32_t c0 = r * L, cnt = std::max(0, std::min(L, nt - c0));
        const int32_t warm = reverse ? std::min(2, std::max(0, nt - c0 - cnt)) : std::min(2, c0);
        return cnt + warm + 0.5;
    };
    // a lower bound first (all CUs busy to the end, and the longest job): a
    // candidate that cannot beat the best so far is not simulated
    double total = 0.0, longest = 0.0;
    for (int32_t n = 0; n < nseq; ++n) {
        const int64_t len = seq_len(n);
        const int32_t nt = gdn::seq_chunks(len), ns = gdn::seq_segments(len, L);
        for (int32_t r = 0; r < ns; ++r) {
            const double t = job(nt, r);
            total += t * d->H_v * per_segment;
            longest = std::max(longest, t);
        }
    }
    const double lb = std::max(total / gdn::kNumCUs, longest);
    if (lb >= bound) return lb;
    std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
    for (int i = 0; i < gdn::kNumCUs; ++i) free_at.push(0.0);
    double end = 0.0;
    for (int32_t n = 0; n < nseq; ++n) {
        const int64_t len = seq_len(n);
        const int32_t nt = gdn::seq_chunks(len), ns = gdn::seq_segments(len, L);
        for (int32_t r = 0; r < ns; ++r) {
            const double t = job(nt, r);
            for (int64_t w = 0; w < (int64_t)d->H_v * per_segment; ++w) {
                const double s0 = free_at.top();
                free_at.pop();
                free_at.push(s0 + t);
                end = std::max(end, s0 + t);
            }
        }
    }
    return end;
}

// AUTO: the candidate segment length with the smallest cost.
int32_t auto_segment_chunks(const gdn_fwd_desc *d, int32_t max_chunks, int32_t per_segment, bool reverse) {
    static const int32_t cands[] = {8, 12, 16, 24, 32, 48, 64, 96, 128, 192, 256};
    int32_t bestL = std::max(1, max_chunks);
    double best = segment_cost(d, bestL, per_segment, reverse, 1e300);
    for (int32_t L : cands) {
        if (L >= max_chunks) break;
        const double cost = segment_cost(d, L, per_segment, reverse, best);
        if (cost < best) {
            best = cost;
            bestL = L;
        }
    }
    return bestL;
}

int make_plan(const gdn_fwd_desc *d, Plan *P) {
    if (!d) return fail(GDN_EINVAL, "descriptor is NULL");
    if (d->B < 0 || d->T < 0) return fail(GDN_EINVAL, "B and T must be >= 0 (got B=%lld T=%lld)", (long long)d->B,
                                          (long long)d->T);
    if (d->H_qk <= 0 || d->H_v <= 0) return fail(GDN_EINVAL, "H_qk and H_v must be > 0");
    if (d->H_v % d->H_qk != 0)
        return fail(GDN_EINVAL, "H_v (%d) must be a multiple of H_qk (%d)", d->H_v, d->H_qk);
    if (d->K <= 0 || d->V <= 0) return fail(GDN_EINVAL, "K and V must be > 0");
    if (d->o_dtype != GDN_DTYPE_BF16 && d->o_dtype != GDN_DTYPE_F32) return fail(GDN_EINVAL, "unknown o_dtype %d",
                                                                                 d->o_dtype);
    if (d->cp_mode < GDN_CP_OFF || d->cp_mode > GDN_CP_AUTO) return fail(GDN_EINVAL, "unknown cp_mode %d", d->cp_mode);
    if (!(std::isfinite(d->scale))) return fail(GDN_EINVAL, "scale must be finite");
    if (!(d->cp_lambda >= 0.f) || !std::isfinite(d->cp_lambda)) return fail(GDN_EINVAL, "cp_lambda must be >= 0");
    if (d->cp_segment_chunks < 0) return fail(GDN_EINVAL, "cp_segment_chunks must be >= 0");
    if (d->K != gdn::kDimK || d->V != gdn::kDimV)
        return fail(GDN_EUNSUPPORTED, "only K = V = 128 is built (got K=%d V=%d)", d->K, d->V);
    if (d->chunk != gdn::kChunk) return fail(GDN_EUNSUPPORTED, "only chunk = 64 is built (got %d)", d->chunk);
    if (d->T > INT32_MAX || d->B > INT32_MAX) return fail(GDN_EINVAL, "B and T must fit in int32");

    int64_t max_len = 0, total_chunks = 0;
    if (d->cu_seqlens_host) {
        if (d->B != 1) return fail(GDN_EINVAL, "cu_seqlens requires B == 1 (got B=%lld)", (long long)d->B);
        if (d->num_seqs < 0) return fail(GDN_EINVAL, "num_seqs must be >= 0");
        const int32_t *cu = d->cu_seqlens_host;
        if (cu[0] != 0) return fail(GDN_EINVAL, "cu_seqlens[0] must be 0 (got %d)", cu[0]);
        for (int32_t n = 0; n < d->num_seqs; ++n) {
            if (cu[n + 1] < cu[n])
                return fail(GDN_EINVAL, "cu_seqlens must be non-decreasing (cu[%d]=%d > cu[%d]=%d)", n, cu[n], n + 1,
                            cu[n + 1]);
            const int64_t len = (int64_t)cu[n + 1] - cu[n];
            max_len = std::max(max_len, len);
            total_chunks += gdn::seq_chunks(len);
        }
        if (cu[d->num_seqs] != d->T)
            return fail(GDN_EINVAL, "cu_seqlens[-1] (%d) must equal T (%lld)", cu[d->num_seqs], (long long)d->T);
    } else {
        if (d->num_seqs != d->B)
            return fail(GDN_EINVAL, "num_seqs (%d) must equal B (%lld) without cu_seqlens", d->num_seqs,
                        (long long)d->B);
        max_len = d->T;
        total_chunks = d->B * (int64_t)gdn::seq_chunks(d->T);
    }
    if (total_chunks > INT32_MAX) return fail(GDN_EINVAL, "too many chunks");
    // every chunk of a sequence is read (and its outputs written) through
    // buffer resources over its 64 rows, whose byte range must stay below 2^31
    const int64_t osz = d->o_dtype == GDN_DTYPE_F32 ? 4 : 2;
    const int64_t row_bytes = std::max({(int64_t)d->H_qk * d->K * 2, (int64_t)d->H_v * d->V * osz,
                                        (int64_t)d->H_v * gdn::kChunk * 4});
    if ((int64_t)gdn::kChunk * row_bytes >= ((int64_t)1 << 31))
        return fail(GDN_EUNSUPPORTED, "%d heads exceed the 2 GiB per-chunk range", d->H_v);

    P->rows = d->B * d->T;
    P->N = d->num_seqs;
    P->total_chunks = (int32_t)total_chunks;
    P->max_chunks = gdn::seq_chunks(max_len);
    P->warmup = d->cp_warmup_chunks > 0 ? d->cp_warmup_chunks : 0;  // 0: no cap (gate-driven window)

    int32_t mode = d->cp_mode;
    int32_t L = std::max(1, P->max_chunks);
    if (mode == GDN_CP_OFF) {
        P->warmup = 0;
    } else {
        if (d->cp_segment_chunks > 0) {
            L = d->cp_segment_chunks;
        } else if (d->cp_lambda > 0.f) {
            L = (int32_t)std::lround(d->cp_lambda * std::sqrt((double)P->max_chunks));
        } else {
            L = auto_segment_chunks(d, P->max_chunks, 1, false);
        }
        L = std::max(1, std::min(L, std::max(1, P->max_chunks)));
        if (mode == GDN_CP_AUTO) mode = GDN_CP_WARMUP;
        if (L >= P->max_chunks) {
            mode = GDN_CP_OFF;
            P->warmup = 0;
        }
    }
    P->L = L;
    P->cp_mode = mode;
    P->num_segments = count_segments(d, L);
    if ((int64_t)P->num_segments * d->H_v > INT32_MAX) return fail(GDN_EINVAL, "grid too large");
    // OFF / WARMUP keep everything on chip; EXACT stores per-segment S, M and
    // start states (three [segments][H_v][K][V] fp32 arrays)
    P->workspace = 0;
    if (P->cp_mode == GDN_CP_EXACT) {
        P->state_bytes = (size_t)P->num_segments * d->H_v * d->K * d->V * sizeof(float);
        P->workspace = 3 * P->state_bytes;
    }
    return GDN_OK;
}

// Shape and plan fields of the forward's kernel parameters (pointers are the caller's).
gdn::FwdParams fwd_params(const gdn_fwd_desc *d, const Plan &P) {
    gdn::FwdParams fp{};
    fp.T = d->T;
    fp.rows = P.rows;
    fp.B = (int32_t)d->B;
    fp.N = d->num_seqs;
    fp.Hqk = d->H_qk;
    fp.Hv = d->H_v;
    fp.group = d->H_v / d->H_qk;
    fp.num_segments = P.num_segments;
    fp.L = P.L;
    fp.cp_mode = P.cp_mode;
    fp.warmup_cap = P.warmup;
    fp.o_f32 = d->o_dtype == GDN_DTYPE_F32;
    fp.scale = d->scale;
    return fp;
}

// ---- backward planning: the reverse pass runs one workgroup per (segment,
// v-head, half of V); AUTO picks L for that grid the same way as the forward.
struct BwdPlan {
    Plan fwd;                 // the differentiated forward (validation, recompute)
    int32_t L = 1, num_segments = 0, cp_mode = GDN_CP_OFF, warmup = 0;
    int32_t entries = 0;      // chunk-local grid entries (chunks + one per empty sequence)
    size_t off_o = 0, off_h = 0, off_a = 0, off_vn = 0, off_fws = 0;  // forward recompute (saved_fwd == 0 only)
    size_t off_dh = 0, off_dvp = 0, off_dq = 0, off_dk = 0;
    size_t off_cs = 0, off_cm = 0, off_ch = 0;  // exact CP: per-segment S, M, start gradient
    size_t workspace = 0;
};

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

int make_bwd_plan(const gdn_bwd_desc *bd, BwdPlan *B) {
    if (!bd) return fail(GDN_EINVAL, "descriptor is NULL");
    const gdn_fwd_desc *d = &bd->fwd;
    int rc = make_plan(d, &B->fwd);
    if (rc != GDN_OK) return rc;
    if (bd->grad_dtype != GDN_DTYPE_BF16 && bd->grad_dtype != GDN_DTYPE_F32)
        return fail(GDN_EINVAL, "unknown grad_dtype %d", bd->grad_dtype);
    const Plan &P = B->fwd;
    int32_t L = std::max(1, P.max_chunks);
    int32_t mode = d->cp_mode;
    int32_t warmup = d->cp_warmup_chunks > 0 ? d->cp_warmup_chunks : 0;  // 0: no cap
    if (mode != GDN_CP_OFF) {
        if (d->cp_segment_chunks > 0) {
            L = d->cp_segment_chunks;
        } else if (d->cp_lambda > 0.f) {
            L = (int32_t)std::lround(d->cp_lambda * std::sqrt((double)P.max_chunks));
        } else {
            L = auto_segment_chunks(d, P.max_chunks, 2, true);
        }
        L = std::max(1, std::min(L, std::max(1, P.max_chunks)));
        if (mode == GDN_CP_AUTO) mode = GDN_CP_WARMUP;
        if (L >= P.max_chunks) mode = GDN_CP_OFF;
    }
    if (mode == GDN_CP_OFF) warmup = 0;
    B->L = L;
    B->cp_mode = mode;
    B->warmup = warmup;
    B->num_segments = count_segments(d, L);
    B->entries = count_segments(d, 1);
    if ((int64_t)B->num_segments * d->H_v * 2 > INT32_MAX || (int64_t)B->entries * d->H_v > INT32_MAX)
        return fail(GDN_EINVAL, "grid too large");

    const size_t rows = (size_t)P.rows;
    const size_t n_h = (size_t)P.total_chunks * d->H_v * d->K * d->V;
    size_t off = 0;
    if (!bd->saved_fwd) {
        const size_t osz = d->o_dtype == GDN_DTYPE_F32 ? 4 : 2;
        B->off_o = off;
        off = align_up(off + rows * d->H_v * d->V * osz);
        B->off_h = off;
        off = align_up(off + n_h * 4);
        B->off_a = off;
        off = align_up(off + rows * d->H_v * gdn::kChunk * 4);
        B->off_vn = off;
        off = align_up(off + (size_t)P.total_chunks * d->H_v * gdn::kChunk * d->V * 4);
        B->off_fws = off;  // the forward's own workspace (exact CP: S, M, start states)
        off = align_up(off + P.workspace);
    }
    B->off_dh = off;
    off = align_up(off + n_h * 4);
    B->off_dvp = off;
    off = align_up(off + (size_t)P.total_chunks * d->H_v * gdn::kChunk * d->V * 4);
    B->off_dq = off;  // running key-head sums of dq and dk (fp32 [rows][H_qk][K])
    off = align_up(off + rows * d->H_qk * d->K * 4);
    B->off_dk = off;
    off = align_up(off + rows * d->H_qk * d->K * 4);
    if (mode == GDN_CP_EXACT) {
        const size_t st = (size_t)B->num_segments * d->H_v * d->K * d->V * 4;
        B->off_cs = off;
        off = align_up(off + st);
        B->off_cm = off;
        off = align_up(off + st);
        B->off_ch = off;
        off = align_up(off + st);
    }
    B->workspace = off;
    return GDN_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

}  // namespace

namespace gdn {

int set_error(int status, const char *msg) {
    g_last_error = msg;
    return status;
}

int fwd_workspace_bytes(const gdn_fwd_desc *d, size_t *bytes) {
    Plan P;
    const int rc = make_plan(d, &P);
    if (rc == GDN_OK) *bytes = P.workspace;
    return rc;
}

}  // namespace gdn

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char *gdn_status_str(int status) {
    switch (status) {
        case GDN_OK: return "GDN_OK";
        case GDN_EINVAL: return "GDN_EINVAL: invalid argument";
        case GDN_EUNSUPPORTED: return "GDN_EUNSUPPORTED: not supported by this library";
        case GDN_EWORKSPACE: return "GDN_EWORKSPACE: workspace too small or misaligned";
        case GDN_EHIP: return "GDN_EHIP: HIP runtime error";
        default: return "unknown gdn status";
    }
}

const char *gdn_last_error(void) { return g_last_error.c_str(); }

int gdn_fwd_plan(const gdn_fwd_desc *d, gdn_fwd_plan_info *out) {
    Plan P;
    const int rc = make_plan(d, &P);
    if (rc != GDN_OK) return rc;
    if (out) {
        out->workspace_bytes = P.workspace;
        out->total_chunks = P.total_chunks;
        out->segment_chunks = P.L;
        out->num_segments = P.num_segments;
        out->warmup_chunks = P.cp_mode == GDN_CP_WARMUP ? P.warmup : 0;
        out->cp_mode = P.cp_mode;
        out->workgroups = P.num_segments * d->H_v;
    }
    g_last_error.clear();
    return GDN_OK;
}

int gdn_fwd(const gdn_fwd_desc *d, const gdn_fwd_ptrs *p, void *workspace, size_t workspace_bytes, void *stream) {
    Plan P;
    int rc = make_plan(d, &P);
    if (rc != GDN_OK) return rc;
    if (!p) return fail(GDN_EINVAL, "pointer struct is NULL");
    const bool varlen = d->cu_seqlens_host != nullptr;
    if (varlen != (p->cu_seqlens != nullptr))
        return fail(GDN_EINVAL, "device cu_seqlens and host cu_seqlens_host must be given together");
    if ((d->has_h0 != 0) != (p->initial_state != nullptr))
        return fail(GDN_EINVAL, "initial_state pointer must be given iff has_h0");
    if ((d->want_ht != 0) != (p->final_state != nullptr))
        return fail(GDN_EINVAL, "final_state pointer must be given iff want_ht");

    const size_t rows = (size_t)P.rows;
    const size_t n_qk = rows * d->H_qk * d->K, n_v = rows * d->H_v * d->V, n_g = rows * d->H_v;
    const size_t n_state = (size_t)d->num_seqs * d->H_v * d->K * d->V;
    const size_t osz = d->o_dtype == GDN_DTYPE_F32 ? 4 : 2;
    if (rows > 0) {
        if (!p->q || !p->k || !p->v || !p->g || !p->beta || !p->o)
            return fail(GDN_EINVAL, "q, k, v, g, beta and o must be non-NULL");
        if (((uintptr_t)p->q | (uintptr_t)p->k | (uintptr_t)p->v) & 15)
            return fail(GDN_EINVAL, "q, k and v must be 16-byte aligned");
        if (((uintptr_t)p->g | (uintptr_t)p->beta) & 3) return fail(GDN_EINVAL, "g and beta must be 4-byte aligned");
        if ((uintptr_t)p->o & 15) return fail(GDN_EINVAL, "o must be 16-byte aligned");
    }
    const size_t n_h = (size_t)P.total_chunks * d->H_v * d->K * d->V, n_a = rows * d->H_v * gdn::kChunk;
    if (((uintptr_t)p->h | (uintptr_t)p->A | (uintptr_t)p->v_new) & 15)
        return fail(GDN_EINVAL, "h, A and v_new must be 16-byte aligned");
    struct Buf { const void *ptr; size_t bytes; const char *name; };
    const Buf in[] = {{p->q, n_qk * 2, "q"}, {p->k, n_qk * 2, "k"}, {p->v, n_v * 2, "v"},
                      {p->g, n_g * 4, "g"}, {p->beta, n_g * 4, "beta"},
                      {p->initial_state, n_state * 4, "initial_state"},
                      {p->cu_seqlens, varlen ? (size_t)(d->num_seqs + 1) * 4 : 0, "cu_seqlens"},
                      {workspace, P.workspace, "workspace"}};
    const size_t n_vn = (size_t)P.total_chunks * d->H_v * gdn::kChunk * d->V;
    const Buf outs[] = {{p->o, n_v * osz, "o"}, {p->final_state, n_state * 4, "final_state"},
                        {p->h, p->h ? n_h * 4 : 0, "h"}, {p->A, p->A ? n_a * 4 : 0, "A"},
                        {p->v_new, p->v_new ? n_vn * 4 : 0, "v_new"}};
    for (const Buf &ob : outs) {
        for (const Buf &b : in)
            if (overlaps(ob.ptr, ob.bytes, b.ptr, b.bytes)) return fail(GDN_EINVAL, "%s overlaps %s", ob.name, b.name);
        for (const Buf &b : outs)
            if (&b != &ob && overlaps(ob.ptr, ob.bytes, b.ptr, b.bytes))
                return fail(GDN_EINVAL, "%s overlaps %s", ob.name, b.name);
    }
    if ((P.workspace > 0 && !workspace) || workspace_bytes < P.workspace)
        return fail(GDN_EWORKSPACE, "workspace needs %zu bytes (got %zu at %p)", P.workspace, workspace_bytes,
                    workspace);
    if (P.workspace > 0 && ((uintptr_t)workspace & (kAlign - 1)))
        return fail(GDN_EWORKSPACE, "workspace must be 256-byte aligned");

    gdn::FwdParams fp = fwd_params(d, P);
    fp.q = (const uint16_t *)p->q;
    fp.k = (const uint16_t *)p->k;
    fp.v = (const uint16_t *)p->v;
    fp.g = p->g;
    fp.beta = p->beta;
    fp.h0 = p->initial_state;
    fp.cu = p->cu_seqlens;
    fp.o = p->o;
    fp.ht = p->final_state;
    fp.h_out = p->h;
    fp.a_out = p->A;
    fp.vn_out = p->v_new;
    if (P.cp_mode == GDN_CP_EXACT) {
        fp.ws_s = (float *)workspace;
        fp.ws_m = (float *)((char *)workspace + P.state_bytes);
        fp.ws_h = (float *)((char *)workspace + 2 * P.state_bytes);
    }

    if (P.num_segments == 0 || d->H_v == 0) {
        g_last_error.clear();
        return GDN_OK;
    }
    if (P.cp_mode == GDN_CP_EXACT) {
        const int err = gdn::launch_cp_exact(fp, stream);
        if (err) return fail(GDN_EHIP, "context-parallel pre-pass launch failed: %s", gdn::hip_error_text(err));
    }
    const int err = gdn::launch_fwd_main(fp, stream);
    if (err) return fail(GDN_EHIP, "forward launch failed: %s", gdn::hip_error_text(err));
    g_last_error.clear();
    return GDN_OK;
}

int gdn_bwd_plan(const gdn_bwd_desc *d, gdn_bwd_plan_info *out) {
    BwdPlan B;
    const int rc = make_bwd_plan(d, &B);
    if (rc != GDN_OK) return rc;
    if (out) {
        out->workspace_bytes = B.workspace;
        out->total_chunks = B.fwd.total_chunks;
        out->segment_chunks = B.L;
        out->num_segments = B.num_segments;
        out->warmup_chunks = B.cp_mode == GDN_CP_WARMUP ? B.warmup : 0;
        out->cp_mode = B.cp_mode;
        out->workgroups_reverse = B.num_segments * d->fwd.H_v * 2;
        out->workgroups_local = B.entries * d->fwd.H_qk;
    }
    g_last_error.clear();
    return GDN_OK;
}

int gdn_bwd(const gdn_bwd_desc *bd, const gdn_bwd_ptrs *p, void *workspace, size_t workspace_bytes, void *stream) {
    BwdPlan B;
    int rc = make_bwd_plan(bd, &B);
    if (rc != GDN_OK) return rc;
    if (!p) return fail(GDN_EINVAL, "pointer struct is NULL");
    const gdn_fwd_desc *d = &bd->fwd;
    const Plan &P = B.fwd;
    const bool varlen = d->cu_seqlens_host != nullptr;
    if (varlen != (p->cu_seqlens != nullptr))
        return fail(GDN_EINVAL, "device cu_seqlens and host cu_seqlens_host must be given together");
    if ((d->has_h0 != 0) != (p->initial_state != nullptr))
        return fail(GDN_EINVAL, "initial_state pointer must be given iff has_h0");
    if ((bd->has_dht != 0) != (p->d_final_state != nullptr))
        return fail(GDN_EINVAL, "d_final_state pointer must be given iff has_dht");
    if ((bd->saved_fwd != 0) != (p->h != nullptr) || (p->h != nullptr) != (p->A != nullptr) ||
        (p->h != nullptr) != (p->v_new != nullptr))
        return fail(GDN_EINVAL, "h, A and v_new must all be given iff saved_fwd");

    const size_t rows = (size_t)P.rows;
    const size_t n_qk = rows * d->H_qk * d->K, n_v = rows * d->H_v * d->V, n_g = rows * d->H_v;
    const size_t n_state = (size_t)d->num_seqs * d->H_v * d->K * d->V;
    const size_t n_h = (size_t)P.total_chunks * d->H_v * d->K * d->V, n_a = rows * d->H_v * gdn::kChunk;
    const size_t gsz = bd->grad_dtype == GDN_DTYPE_F32 ? 4 : 2;
    if (rows > 0) {
        if (!p->q || !p->k || !p->v || !p->g || !p->beta || !p->dO || !p->dq || !p->dk || !p->dv || !p->dg ||
            !p->dbeta)
            return fail(GDN_EINVAL, "q, k, v, g, beta, dO, dq, dk, dv, dg and dbeta must be non-NULL");
        if (((uintptr_t)p->q | (uintptr_t)p->k | (uintptr_t)p->v | (uintptr_t)p->dO | (uintptr_t)p->dq |
             (uintptr_t)p->dk | (uintptr_t)p->dv) & 15)
            return fail(GDN_EINVAL, "q, k, v, dO, dq, dk and dv must be 16-byte aligned");
        if (((uintptr_t)p->g | (uintptr_t)p->beta | (uintptr_t)p->dg | (uintptr_t)p->dbeta) & 3)
            return fail(GDN_EINVAL, "g, beta, dg and dbeta must be 4-byte aligned");
    }
    if (((uintptr_t)p->h | (uintptr_t)p->A | (uintptr_t)p->v_new | (uintptr_t)p->initial_state |
         (uintptr_t)p->d_final_state | (uintptr_t)p->d_initial_state) & 15)
        return fail(GDN_EINVAL, "h, A, v_new and the state tensors must be 16-byte aligned");
    const size_t n_vn = (size_t)P.total_chunks * d->H_v * gdn::kChunk * d->V;
    struct Buf { const void *ptr; size_t bytes; const char *name; };
    const Buf in[] = {{p->q, n_qk * 2, "q"}, {p->k, n_qk * 2, "k"}, {p->v, n_v * 2, "v"},
                      {p->g, n_g * 4, "g"}, {p->beta, n_g * 4, "beta"},
                      {p->initial_state, n_state * 4, "initial_state"},
                      {p->cu_seqlens, varlen ? (size_t)(d->num_seqs + 1) * 4 : 0, "cu_seqlens"},
                      {p->dO, n_v * 2, "dO"}, {p->d_final_state, n_state * 4, "d_final_state"},
                      {p->h, p->h ? n_h * 4 : 0, "h"}, {p->A, p->A ? n_a * 4 : 0, "A"},
                      {p->v_new, p->v_new ? n_vn * 4 : 0, "v_new"}, {workspace, B.workspace, "workspace"}};
    const Buf outs[] = {{p->dq, n_qk * gsz, "dq"}, {p->dk, n_qk * gsz, "dk"}, {p->dv, n_v * gsz, "dv"},
                        {p->dg, n_g * 4, "dg"}, {p->dbeta, n_g * 4, "dbeta"},
                        {p->d_initial_state, n_state * 4, "d_initial_state"}};
    for (const Buf &ob : outs) {
        for (const Buf &b : in)
            if (overlaps(ob.ptr, ob.bytes, b.ptr, b.bytes)) return fail(GDN_EINVAL, "%s overlaps %s", ob.name, b.name);
        for (const Buf &b : outs)
            if (&b != &ob && overlaps(ob.ptr, ob.bytes, b.ptr, b.bytes))
                return fail(GDN_EINVAL, "%s overlaps %s", ob.name, b.name);
    }
    if ((B.workspace > 0 && !workspace) || workspace_bytes < B.workspace)
        return fail(GDN_EWORKSPACE, "workspace needs %zu bytes (got %zu at %p)", B.workspace, workspace_bytes,
                    workspace);
    if (B.workspace > 0 && ((uintptr_t)workspace & (kAlign - 1)))
        return fail(GDN_EWORKSPACE, "workspace must be 256-byte aligned");
    char *ws = static_cast<char *>(workspace);

    const float *h = p->h, *A = p->A, *vn = p->v_new;
    if (!bd->saved_fwd && P.num_segments > 0 && rows > 0) {
        // recompute the forward's chunk-start states and WY matrices
        gdn::FwdParams fp = fwd_params(d, P);
        fp.q = (const uint16_t *)p->q;
        fp.k = (const uint16_t *)p->k;
        fp.v = (const uint16_t *)p->v;
        fp.g = p->g;
        fp.beta = p->beta;
        fp.h0 = p->initial_state;
        fp.cu = p->cu_seqlens;
        fp.o = ws + B.off_o;
        fp.ht = nullptr;
        fp.h_out = reinterpret_cast<float *>(ws + B.off_h);
        fp.a_out = reinterpret_cast<float *>(ws + B.off_a);
        fp.vn_out = reinterpret_cast<float *>(ws + B.off_vn);
        if (P.cp_mode == GDN_CP_EXACT) {
            fp.ws_s = reinterpret_cast<float *>(ws + B.off_fws);
            fp.ws_m = reinterpret_cast<float *>(ws + B.off_fws + P.state_bytes);
            fp.ws_h = reinterpret_cast<float *>(ws + B.off_fws + 2 * P.state_bytes);
            const int e1 = gdn::launch_cp_exact(fp, stream);
            if (e1) return fail(GDN_EHIP, "forward recompute pre-pass launch failed: %s", gdn::hip_error_text(e1));
        }
        const int err = gdn::launch_fwd_main(fp, stream);
        if (err) return fail(GDN_EHIP, "forward recompute launch failed: %s", gdn::hip_error_text(err));
        h = fp.h_out;
        A = fp.a_out;
        vn = fp.vn_out;
    }

    gdn::BwdParams bp{};
    bp.q = (const uint16_t *)p->q;
    bp.k = (const uint16_t *)p->k;
    bp.v = (const uint16_t *)p->v;
    bp.dO = (const uint16_t *)p->dO;
    bp.g = p->g;
    bp.beta = p->beta;
    bp.cu = p->cu_seqlens;
    bp.h = h;
    bp.A = A;
    bp.vn = vn;
    bp.dht = p->d_final_state;
    bp.dh_ws = reinterpret_cast<float *>(ws + B.off_dh);
    bp.dvp_ws = reinterpret_cast<float *>(ws + B.off_dvp);
    bp.dq_ws = reinterpret_cast<float *>(ws + B.off_dq);
    bp.dk_ws = reinterpret_cast<float *>(ws + B.off_dk);
    bp.dq = p->dq;
    bp.dk = p->dk;
    bp.dv = p->dv;
    bp.dg = p->dg;
    bp.dbeta = p->dbeta;
    bp.dh0 = p->d_initial_state;
    bp.T = d->T;
    bp.rows = P.rows;
    bp.N = d->num_seqs;
    bp.Hqk = d->H_qk;
    bp.Hv = d->H_v;
    bp.group = d->H_v / d->H_qk;
    bp.num_segments = B.num_segments;
    bp.L = B.L;
    bp.cp_mode = B.cp_mode;
    bp.warmup_cap = B.warmup;
    bp.num_chunk_entries = B.entries;
    if (B.cp_mode == GDN_CP_EXACT) {
        bp.ws_s = reinterpret_cast<float *>(ws + B.off_cs);
        bp.ws_m = reinterpret_cast<float *>(ws + B.off_cm);
        bp.ws_h = reinterpret_cast<float *>(ws + B.off_ch);
    }
    bp.grad_f32 = bd->grad_dtype == GDN_DTYPE_F32;
    bp.scale = d->scale;
    const int err = gdn::launch_bwd(bp, stream);
    if (err) return fail(GDN_EHIP, "backward launch failed: %s", gdn::hip_error_text(err));
    g_last_error.clear();
    return GDN_OK;
}

int gdn_chunk_cumsum(const float *g, float *out, int64_t B, int64_t T, int32_t H, int32_t chunk,
                     const int32_t *cu_seqlens, int32_t num_seqs, void *stream) {
    if (B < 0 || T < 0 || H <= 0) return fail(GDN_EINVAL, "bad shape B=%lld T=%lld H=%d", (long long)B,
                                              (long long)T, H);
    if (chunk <= 0) return fail(GDN_EINVAL, "chunk must be > 0");
    if (cu_seqlens && B != 1) return fail(GDN_EINVAL, "cu_seqlens requires B == 1");
    if (cu_seqlens && num_seqs < 1) return fail(GDN_EINVAL, "cu_seqlens needs num_seqs >= 1 (got %d)", num_seqs);
    if (!cu_seqlens && num_seqs != B) return fail(GDN_EINVAL, "num_seqs must equal B without cu_seqlens");
    if (B * T > 0 && (!g || !out)) return fail(GDN_EINVAL, "g and out must be non-NULL");
    const size_t bytes = (size_t)(B * T * H) * 4;
    if (out != g && overlaps(out, bytes, g, bytes)) return fail(GDN_EINVAL, "out partially overlaps g");
    const int err = gdn::launch_chunk_cumsum(g, out, B, T, H, chunk, cu_seqlens, num_seqs, stream);
    if (err) return fail(GDN_EHIP, "cumsum launch failed: %s", gdn::hip_error_text(err));
    g_last_error.clear();
    return GDN_OK;
}

}  // extern "C"
