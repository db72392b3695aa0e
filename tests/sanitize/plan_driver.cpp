// Drives libgdn's host-side planner and entry points (gdn_plan.cpp, built by
// the host compiler with AddressSanitizer and UndefinedBehaviorSanitizer) over
// seeded random descriptors: valid and invalid shapes, packed-sequence
// offsets (including empty sequences and broken offsets), every context-
// parallel mode, aliasing and alignment errors, workspaces that are too small.
// The kernel launchers are replaced by stubs that record what they were asked
// to launch, so every path runs without a GPU.  Besides the sanitizers'
// checks, the driver asserts the planner's contract: a failing call launches
// nothing and leaves a message; a valid call launches the planned grid, with
// segment counts that match an independent count, and never needs more
// workspace than gdn_fwd_plan / gdn_bwd_plan reported.  Exit status 0 means
// every check held.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "gdn.h"
#include "gdn_internal.h"

namespace {
int g_fwd_launches = 0, g_cp_launches = 0, g_bwd_launches = 0, g_cumsum_launches = 0;
gdn::FwdParams g_last_fwd;
gdn::BwdParams g_last_bwd;
int g_failures = 0;

void check(bool ok, const char *what, int line) {
    if (!ok) {
        std::fprintf(stderr, "check failed (line %d): %s\n", line, what);
        ++g_failures;
    }
}
#define CHECK(x) check((x), #x, __LINE__)
}  // namespace

// ---- launcher stubs (the real ones live with the kernels)
namespace gdn {
int launch_fwd_main(const FwdParams &p, void *) {
    ++g_fwd_launches;
    g_last_fwd = p;
    return 0;
}
int launch_cp_exact(const FwdParams &, void *) {
    ++g_cp_launches;
    return 0;
}
int launch_chunk_cumsum(const float *, float *, int64_t, int64_t, int32_t, int32_t, const int32_t *, int32_t,
                        void *) {
    ++g_cumsum_launches;
    return 0;
}
int launch_bwd(const BwdParams &p, void *) {
    ++g_bwd_launches;
    g_last_bwd = p;
    return 0;
}
const char *hip_error_text(int) { return "stub"; }
}  // namespace gdn

namespace {

std::mt19937_64 rng(20261202);
int uni(int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); }

// Fake, disjoint, 256-byte-aligned device addresses (never dereferenced).
struct Arena {
    uintptr_t next = 0x10000000;
    void *take(size_t bytes) {
        void *p = reinterpret_cast<void *>(next);
        next += (bytes + 4095) & ~size_t(4095);
        next += 4096;
        return p;
    }
};

int64_t count_segments(const std::vector<int32_t> &cu, int64_t B, int64_t T, int L) {
    if (cu.empty()) {
        const int64_t nt = (T + 63) / 64;
        return B * std::max<int64_t>(1, (nt + L - 1) / L);
    }
    int64_t total = 0;
    for (size_t n = 0; n + 1 < cu.size(); ++n) {
        const int64_t nt = (cu[n + 1] - cu[n] + 63) / 64;
        total += std::max<int64_t>(1, (nt + L - 1) / L);
    }
    return total;
}

void random_desc(gdn_fwd_desc &d, std::vector<int32_t> &cu, bool &expect_ok) {
    std::memset(&d, 0, sizeof(d));
    expect_ok = true;
    const int hqk = uni(1, 4);
    const int grp = uni(1, 4);
    d.H_qk = hqk;
    d.H_v = hqk * grp;
    d.K = d.V = 128;
    d.chunk = 64;
    d.scale = 0.0883883f;
    d.cp_mode = uni(0, 3);
    d.o_dtype = uni(0, 1);
    d.has_h0 = uni(0, 1);
    d.want_ht = uni(0, 1);
    if (uni(0, 3) == 0) d.cp_segment_chunks = uni(1, 9);
    if (uni(0, 5) == 0) d.cp_warmup_chunks = uni(1, 5);
    cu.clear();
    if (uni(0, 1)) {  // packed sequences
        const int n = uni(0, 7);
        cu.push_back(0);
        for (int i = 0; i < n; ++i) cu.push_back(cu.back() + (uni(0, 3) == 0 ? 0 : uni(1, 700)));
        d.B = 1;
        d.T = cu.back();
        d.num_seqs = n;
    } else {
        d.B = uni(0, 3);
        d.T = uni(0, 900);
        d.num_seqs = (int32_t)d.B;
    }
    // one deliberate defect in a quarter of the cases
    switch (uni(0, 15)) {
        case 0: d.H_v = d.H_qk * grp + 1; break;  // not a multiple of H_qk unless H_qk == 1
        case 1: d.K = 64; expect_ok = false; break;
        case 2: d.chunk = 32; expect_ok = false; break;
        case 3:
            if (!cu.empty() && cu.size() > 2) { std::swap(cu[1], cu[2]); expect_ok = cu[1] <= cu[2]; }
            break;
        case 4:
            if (!cu.empty()) { cu.back() += 1; expect_ok = false; }
            break;
        default: break;
    }
    if (d.H_v % d.H_qk != 0) expect_ok = false;
    d.cu_seqlens_host = cu.empty() ? nullptr : cu.data();
}

void test_forward(int iters) {
    for (int it = 0; it < iters; ++it) {
        gdn_fwd_desc d;
        std::vector<int32_t> cu;
        bool expect_ok;
        random_desc(d, cu, expect_ok);
        gdn_fwd_plan_info info;
        const int rc = gdn_fwd_plan(&d, &info);
        if (!expect_ok) {
            CHECK(rc != GDN_OK);
            CHECK(std::strlen(gdn_last_error()) > 0);
            continue;
        }
        CHECK(rc == GDN_OK);
        if (rc != GDN_OK) {
            std::fprintf(stderr, "  plan failed unexpectedly: %s\n", gdn_last_error());
            continue;
        }
        CHECK(info.num_segments == count_segments(cu, d.B, d.T, info.segment_chunks));
        CHECK(info.workgroups == info.num_segments * d.H_v);
        CHECK(info.cp_mode != GDN_CP_AUTO);
        CHECK(info.cp_mode == GDN_CP_EXACT ? info.workspace_bytes > 0 || info.num_segments == 0
                                           : info.workspace_bytes == 0);
        // a valid call with disjoint buffers launches the planned grid
        const size_t rows = (size_t)(d.B * d.T);
        const size_t n_state = (size_t)d.num_seqs * d.H_v * 128 * 128 * 4;
        Arena a;
        gdn_fwd_ptrs p;
        std::memset(&p, 0, sizeof(p));
        p.q = a.take(rows * d.H_qk * 128 * 2);
        p.k = a.take(rows * d.H_qk * 128 * 2);
        p.v = a.take(rows * d.H_v * 128 * 2);
        p.g = (const float *)a.take(rows * d.H_v * 4);
        p.beta = (const float *)a.take(rows * d.H_v * 4);
        p.initial_state = d.has_h0 ? (const float *)a.take(n_state) : nullptr;
        p.cu_seqlens = cu.empty() ? nullptr : (const int32_t *)a.take(cu.size() * 4);
        p.o = a.take(rows * d.H_v * 128 * (d.o_dtype ? 4 : 2));
        p.final_state = d.want_ht ? (float *)a.take(n_state) : nullptr;
        void *ws = a.take(info.workspace_bytes);
        const int before = g_fwd_launches, before_cp = g_cp_launches;
        const int rc2 = gdn_fwd(&d, &p, ws, info.workspace_bytes, nullptr);
        CHECK(rc2 == GDN_OK);
        if (rc2 != GDN_OK) std::fprintf(stderr, "  gdn_fwd failed unexpectedly: %s\n", gdn_last_error());
        if (rc2 == GDN_OK && info.num_segments > 0) {
            CHECK(g_fwd_launches == before + 1);
            CHECK(g_cp_launches == before_cp + (info.cp_mode == GDN_CP_EXACT ? 1 : 0));
            CHECK(g_last_fwd.num_segments == info.num_segments);
            CHECK(g_last_fwd.L == info.segment_chunks);
        }
        // the same call with one byte less workspace, an overlap, or a misaligned tensor fails and launches nothing
        const int launches = g_fwd_launches + g_cp_launches;
        if (info.workspace_bytes > 0) {
            CHECK(gdn_fwd(&d, &p, ws, info.workspace_bytes - 1, nullptr) == GDN_EWORKSPACE);
        }
        if (rows > 0) {
            gdn_fwd_ptrs bad = p;
            bad.o = const_cast<void *>(p.v);
            CHECK(gdn_fwd(&d, &bad, ws, info.workspace_bytes, nullptr) == GDN_EINVAL);
            bad = p;
            bad.q = (const char *)p.q + 2;
            CHECK(gdn_fwd(&d, &bad, ws, info.workspace_bytes, nullptr) == GDN_EINVAL);
        }
        CHECK(g_fwd_launches + g_cp_launches == launches);
    }
}

void test_backward(int iters) {
    for (int it = 0; it < iters; ++it) {
        gdn_bwd_desc d;
        std::memset(&d, 0, sizeof(d));
        std::vector<int32_t> cu;
        bool expect_ok;
        random_desc(d.fwd, cu, expect_ok);
        d.has_dht = uni(0, 1);
        d.grad_dtype = uni(0, 1);
        d.saved_fwd = uni(0, 1);
        gdn_bwd_plan_info info;
        const int rc = gdn_bwd_plan(&d, &info);
        if (!expect_ok) {
            CHECK(rc != GDN_OK);
            continue;
        }
        CHECK(rc == GDN_OK);
        if (rc != GDN_OK) continue;
        CHECK(info.num_segments == count_segments(cu, d.fwd.B, d.fwd.T, info.segment_chunks));
        const size_t rows = (size_t)(d.fwd.B * d.fwd.T);
        const int hv = d.fwd.H_v, hqk = d.fwd.H_qk;
        const size_t n_state = (size_t)d.fwd.num_seqs * hv * 128 * 128 * 4;
        Arena a;
        gdn_bwd_ptrs p;
        std::memset(&p, 0, sizeof(p));
        p.q = a.take(rows * hqk * 256);
        p.k = a.take(rows * hqk * 256);
        p.v = a.take(rows * hv * 256);
        p.g = (const float *)a.take(rows * hv * 4);
        p.beta = (const float *)a.take(rows * hv * 4);
        p.initial_state = d.fwd.has_h0 ? (const float *)a.take(n_state) : nullptr;
        p.cu_seqlens = cu.empty() ? nullptr : (const int32_t *)a.take(cu.size() * 4);
        p.dO = a.take(rows * hv * 256);
        p.d_final_state = d.has_dht ? (const float *)a.take(n_state) : nullptr;
        if (d.saved_fwd) {
            p.h = (const float *)a.take((size_t)info.total_chunks * hv * 128 * 128 * 4);
            p.A = (const float *)a.take(rows * hv * 64 * 4);
            p.v_new = (const float *)a.take((size_t)info.total_chunks * hv * 64 * 128 * 4);
        }
        const size_t gsz = d.grad_dtype ? 4 : 2;
        p.dq = a.take(rows * hqk * 128 * gsz);
        p.dk = a.take(rows * hqk * 128 * gsz);
        p.dv = a.take(rows * hv * 128 * gsz);
        p.dg = (float *)a.take(rows * hv * 4);
        p.dbeta = (float *)a.take(rows * hv * 4);
        p.d_initial_state = d.fwd.has_h0 ? (float *)a.take(n_state) : nullptr;
        void *ws = a.take(info.workspace_bytes);
        const int before = g_bwd_launches;
        const int rc2 = gdn_bwd(&d, &p, ws, info.workspace_bytes, nullptr);
        CHECK(rc2 == GDN_OK);
        if (rc2 != GDN_OK) std::fprintf(stderr, "  gdn_bwd failed unexpectedly: %s\n", gdn_last_error());
        CHECK(g_bwd_launches == before + 1);
        if (rc2 == GDN_OK) {
            CHECK(g_last_bwd.num_segments == info.num_segments);
            CHECK(g_last_bwd.num_chunk_entries * hqk == info.workgroups_local);
        }
        const int launches = g_bwd_launches;
        if (info.workspace_bytes > 0) CHECK(gdn_bwd(&d, &p, ws, info.workspace_bytes - 1, nullptr) == GDN_EWORKSPACE);
        if (rows > 0) {
            gdn_bwd_ptrs bad = p;
            bad.dv = const_cast<void *>(p.v);
            CHECK(gdn_bwd(&d, &bad, ws, info.workspace_bytes, nullptr) == GDN_EINVAL);
        }
        CHECK(g_bwd_launches == launches);
    }
}

void test_cumsum() {
    int32_t cu[3] = {0, 5, 10};
    const int before = g_cumsum_launches;
    CHECK(gdn_chunk_cumsum((const float *)0x1000, (float *)0x2000, 1, 10, 2, 64, cu, 0, nullptr) == GDN_EINVAL);
    CHECK(gdn_chunk_cumsum((const float *)0x1000, (float *)0x2000, 2, 10, 2, 64, cu, 2, nullptr) == GDN_EINVAL);
    CHECK(gdn_chunk_cumsum((const float *)0x1000, (float *)0x2000, -1, 10, 2, 64, nullptr, -1, nullptr) == GDN_EINVAL);
    CHECK(g_cumsum_launches == before);
    CHECK(gdn_chunk_cumsum((const float *)0x1000, (float *)0x3000, 1, 10, 2, 64, cu, 2, nullptr) == GDN_OK);
    CHECK(g_cumsum_launches == before + 1);
    CHECK(gdn_fwd_plan(nullptr, nullptr) == GDN_EINVAL);
    CHECK(gdn_bwd_plan(nullptr, nullptr) == GDN_EINVAL);
    for (int s = -5; s <= 1; ++s) CHECK(gdn_status_str(s) != nullptr);
}

}  // namespace

int main(int argc, char **argv) {
    const int iters = argc > 1 ? std::atoi(argv[1]) : 3000;
    test_forward(iters);
    test_backward(iters);
    test_cumsum();
    std::printf("plan driver: %d forward and %d backward cases, %d failed checks\n", iters, iters, g_failures);
    return g_failures == 0 ? 0 : 1;
}
