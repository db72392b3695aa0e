// Gated DeltaNet chunked-prefill forward: HIP kernels for gfx950 (MI355X).
//
// Chunked WY form of the gated delta rule (the pages' intermediates W, U, S,
// V', O: agentlenshq.com FlashQLA blog, "GDN chunked-prefill optimisation"
// and "TileLang warp-specialised kernels").  For one (sequence, v-head) and a
// chunk of C = 64 tokens with chunk-start state H (K x V = S^T), g-prefix sums
// G_i and gamma_i = e^{G_i}:
//
//   A    = strict-lower( beta_i e^{G_i - G_s} k_i.k_s )           64 x 64
//   T    = (I + A)^{-1}                                          unit lower
//   W    = (T diag(beta gamma)) K          U = (T diag(beta)) V
//   v'   = U - W H                                               64 x V
//   O    = scale [ diag(gamma) Q H + P v' ],   P_is = e^{G_i-G_s} q_i.k_s (s <= i)
//   H   <- gamma_last H + K^T diag(gamma_last / gamma) v'
//
// One workgroup (4 waves) owns one (segment, v-head): it walks the segment's
// chunks in order with H resident in MFMA accumulators, split by V columns
// across the waves (column j of H only ever mixes with column j of v, so the
// split is exact).  Everything chunk-local (cumsum, K K^T, inverse, W, U, P) is
// recomputed on chip; W, U and S never touch HBM.
//
// Precision (the pages' "restructure without losing precision", summarylog.com
// essay, "formula restructuring"): products of two exact bf16 inputs (K K^T,
// Q K^T, T K, Q H) use one bf16 MFMA; operands that carry fp32 values which
// feed the output with full weight are split into hi + lo bf16 pairs:
// T diag(beta), P, v', the decayed v', and H.  Decays and beta are applied as
// fp32 row/column scales; every exponent is a non-positive difference
// G_i - G_s (masked before the exp), so nothing overflows.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Lane l holds A row (l % 32) / B column
// (l % 32), 8 k-slots for lane half (l / 32); accumulator element 4i + j holds
// row 8i + 4(l/32) + j, column l % 32.  An accumulator tile read as a B operand
// therefore sees, in k-step s, the k indices 16s + {4h..4h+3, 8+4h..8+4h+3}
// (h = l/32); A operands that meet such a B are read from LDS with the same
// permutation (two 8-byte reads per lane).
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int CH = kChunk;   // 64
constexpr int DK = kDimK;    // 128
constexpr int DV = kDimV;    // 128
constexpr int NTHREADS = 256;
constexpr int KS = DK + 8;   // bf16 row stride of 128-wide tiles (272 B)
constexpr int CS = CH + 8;   // bf16 row stride of 64-wide tiles (144 B)
constexpr int AS = CH + 1;   // fp32 row stride of the 64 x 64 A / T tile

struct __attribute__((aligned(16))) Smem {
    bf16 k[CH * KS];       // K, row = token
    bf16 kt[DK * CS];      // K^T, row = key dim
    bf16 q[CH * KS];       // Q
    bf16 vt[DV * CS];      // V^T, row = value dim
    bf16 w[CH * KS];       // -W
    bf16 tt[CH * CS];      // T diag(beta gamma)
    bf16 th[2][CH * CS];   // T diag(beta), hi and lo
    bf16 p[2][CH * CS];    // P, hi and lo
    float a[CH * AS];      // A, inverted in place into T
    float scr[32 * 33];    // inverse scratch
    float graw[CH], beta[CH], gcum[CH], gam[CH], dec[CH];
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const bf16 *p) {   // 16-byte LDS read
    return *reinterpret_cast<const bf16x8 *>(p);
}

// A-operand read matching an accumulator-sourced B operand: k indices
// base + 4h .. base + 4h + 3 and base + 8 + 4h .. base + 8 + 4h + 3.
__device__ __forceinline__ bf16x8 lds8_perm(const bf16 *row, int base, int h) {
    bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row + base + 4 * h);
    bf16x4 hi = *reinterpret_cast<const bf16x4 *>(row + base + 8 + 4 * h);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Accumulator registers 8s .. 8s+7 of a tile as bf16 hi and lo B operands.
__device__ __forceinline__ void split8(const f32x16 &acc, int s, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = acc[8 * s + e];
        const bf16 h = (bf16)x;
        hi[e] = h;
        lo[e] = (bf16)(x - (float)h);
    }
}

__device__ __forceinline__ float bf2f(uint16_t u) {
    return __uint_as_float((uint32_t)u << 16);
}

// ---------------------------------------------------------------- chunk loads
// Thread t stages rows 4*(t % 16) .. +3, columns 8*(t / 16) .. +7 of each
// 64 x 128 tile (16-byte global loads; rows past the sequence end read as 0).
struct Stage {
    uint4 k[4], q[4], v[4];
    float g, b;
};

__device__ __forceinline__ void load_chunk(const FwdParams &p, Stage &st, int64_t row0, int c, int seq_len,
                                           int i_qk, int j, bool need_q, const int t) {
    const int rg = t & 15, cg = t >> 4;
    const int tok0 = c * CH;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tok = tok0 + 4 * rg + r;
        if (tok < seq_len) {
            const int64_t row = row0 + tok;
            st.k[r] = *reinterpret_cast<const uint4 *>(p.k + (row * p.Hqk + i_qk) * DK + 8 * cg);
            st.v[r] = *reinterpret_cast<const uint4 *>(p.v + (row * p.Hv + j) * DV + 8 * cg);
            st.q[r] = need_q ? *reinterpret_cast<const uint4 *>(p.q + (row * p.Hqk + i_qk) * DK + 8 * cg)
                             : make_uint4(0, 0, 0, 0);
        } else {
            st.k[r] = st.v[r] = st.q[r] = make_uint4(0, 0, 0, 0);
        }
    }
    if (t < CH) {
        const int tok = tok0 + t;
        if (tok < seq_len) {
            const int64_t row = row0 + tok;
            st.g = p.g[row * p.Hv + j];
            st.b = p.beta[row * p.Hv + j];
        } else {
            st.g = 0.f;
            st.b = 0.f;
        }
    }
}

__device__ __forceinline__ uint16_t half_of(const uint4 &x, int e) {
    const uint32_t w = (e < 2) ? x.x : (e < 4) ? x.y : (e < 6) ? x.z : x.w;
    return (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffff));
}

__device__ __forceinline__ void store_chunk(Smem &s, const Stage &st, bool need_q, const int t) {
    const int rg = t & 15, cg = t >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<uint4 *>(&s.k[(4 * rg + r) * KS + 8 * cg]) = st.k[r];
        if (need_q) *reinterpret_cast<uint4 *>(&s.q[(4 * rg + r) * KS + 8 * cg]) = st.q[r];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t k01 = (uint32_t)half_of(st.k[0], e) | ((uint32_t)half_of(st.k[1], e) << 16);
        const uint32_t k23 = (uint32_t)half_of(st.k[2], e) | ((uint32_t)half_of(st.k[3], e) << 16);
        *reinterpret_cast<uint2 *>(&s.kt[(8 * cg + e) * CS + 4 * rg]) = make_uint2(k01, k23);
        const uint32_t v01 = (uint32_t)half_of(st.v[0], e) | ((uint32_t)half_of(st.v[1], e) << 16);
        const uint32_t v23 = (uint32_t)half_of(st.v[2], e) | ((uint32_t)half_of(st.v[3], e) << 16);
        *reinterpret_cast<uint2 *>(&s.vt[(8 * cg + e) * CS + 4 * rg]) = make_uint2(v01, v23);
    }
    if (t < CH) {
        s.graw[t] = st.g;
        s.beta[t] = st.b;
    }
}

// ---------------------------------------------------------------- chunk prep
// Cumsum (wave 0) and masked, beta-weighted K K^T (waves 1..3) into s.a.
__device__ __forceinline__ void prep_cumsum_kkt(Smem &s, const int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    f32x16 acc = {};
    int rbi = 0, rbs = 0;
    if (wave == 0) {
        float x = s.graw[lane];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const float glast = __shfl(x, 63, 64);
        s.gcum[lane] = x;
        s.gam[lane] = __expf(x);
        s.dec[lane] = __expf(glast - x);
    } else {
        // blocks (row, col) of K K^T: (0,0), (1,0), (1,1)
        rbi = (wave >= 2) ? 1 : 0;
        rbs = (wave == 3) ? 1 : 0;
        const int m = lane & 31, h = lane >> 5;
        const bf16 *ra = &s.k[(32 * rbi + m) * KS + 8 * h];
        const bf16 *rb = &s.k[(32 * rbs + m) * KS + 8 * h];
#pragma unroll
        for (int kk = 0; kk < DK / 16; ++kk) acc = mfma(lds8(ra + 16 * kk), lds8(rb + 16 * kk), acc);
    }
    __syncthreads();
    if (wave != 0) {
        const int n = lane & 31, h = lane >> 5;
        const int col = 32 * rbs + n;
        const float gs = s.gcum[col];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = 32 * rbi + 8 * (e >> 2) + 4 * h + (e & 3);
            float val = 0.f;
            if (col < row) val = s.beta[row] * __expf(s.gcum[row] - gs) * acc[e];
            s.a[row * AS + col] = val;
        }
    }
    __syncthreads();
}

// In-place inverse of the unit lower-triangular (I + A) held as A in s.a:
// 16 x 16 diagonal blocks by forward substitution, then two levels of
// block merges  T_lo,hi = -T_lo,lo A_lo,hi T_hi,hi.  All fp32.
__device__ __forceinline__ void prep_inverse(Smem &s, const int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    // level 0: diagonal block `wave`, lane = column
    if (lane < 16) {
        const int b0 = 16 * wave;
        float t[16];
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
            float acc = (ii == lane) ? 1.f : 0.f;
#pragma unroll
            for (int ss = 0; ss < ii; ++ss) acc -= s.a[(b0 + ii) * AS + b0 + ss] * t[ss];
            t[ii] = acc;
        }
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) s.a[(b0 + ii) * AS + b0 + lane] = t[ii];
    }
    __syncthreads();
    // level 1: T_10 (wave 0) and T_32 (wave 1), 16 x 16 each
    float x[4];
    const int c = lane & 15, r0 = 4 * (lane >> 4);
    if (wave < 2) {
        const int hb = 32 * wave;  // block origin of the 32 x 32 diagonal block
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            float acc = 0.f;
            for (int ss = c; ss < 16; ++ss)  // T_00 is lower triangular
                acc += s.a[(hb + 16 + r0 + rr) * AS + hb + ss] * s.a[(hb + ss) * AS + hb + c];
            x[rr] = acc;
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) s.scr[wave * 256 + (r0 + rr) * 16 + c] = x[rr];
    }
    __syncthreads();
    if (wave < 2) {
        const int hb = 32 * wave;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int r = r0 + rr;
            float acc = 0.f;
            for (int ss = 0; ss <= r; ++ss)
                acc += s.a[(hb + 16 + r) * AS + hb + 16 + ss] * s.scr[wave * 256 + ss * 16 + c];
            s.a[(hb + 16 + r) * AS + hb + c] = -acc;
        }
    }
    __syncthreads();
    // level 2: rows 32..63, cols 0..31:  Y = A_lohi T_hi ; T_lohi = -T_lo Y
    const int t = tid;
    const int cc = t & 31, rq = 4 * (t >> 5);
    float y[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        float acc = 0.f;
        for (int ss = cc; ss < 32; ++ss) acc += s.a[(32 + rq + rr) * AS + ss] * s.a[ss * AS + cc];
        y[rr] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) s.scr[(rq + rr) * 33 + cc] = y[rr];
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        const int r = rq + rr;
        float acc = 0.f;
        for (int ss = 0; ss <= r; ++ss) acc += s.a[(32 + r) * AS + 32 + ss] * s.scr[ss * 33 + cc];
        s.a[(32 + r) * AS + cc] = -acc;
    }
    __syncthreads();
}

// T diag(beta gamma) (bf16) and T diag(beta) (hi, lo) from T in s.a.
__device__ __forceinline__ void prep_scaled_t(Smem &s, const int tid) {
    const int t = tid;
    const int i = t >> 2, s0 = 16 * (t & 3);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int col = s0 + e;
        const float tv = (col < i) ? s.a[i * AS + col] : (col == i ? 1.f : 0.f);
        const float tb = tv * s.beta[col];
        s.tt[i * CS + col] = (bf16)(tb * s.gam[col]);
        const bf16 hi = (bf16)tb;
        s.th[0][i * CS + col] = hi;
        s.th[1][i * CS + col] = (bf16)(tb - (float)hi);
    }
}

// P = causal e^{G_i - G_s} Q K^T, hi and lo (waves 0..2: blocks (0,0), (1,0), (1,1)).
__device__ __forceinline__ void prep_p(Smem &s, const int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    if (wave >= 3) return;
    const int rbi = (wave >= 1) ? 1 : 0;
    const int rbs = (wave == 2) ? 1 : 0;
    const int m = lane & 31, h = lane >> 5;
    const bf16 *ra = &s.q[(32 * rbi + m) * KS + 8 * h];
    const bf16 *rb = &s.k[(32 * rbs + m) * KS + 8 * h];
    f32x16 acc = {};
#pragma unroll
    for (int kk = 0; kk < DK / 16; ++kk) acc = mfma(lds8(ra + 16 * kk), lds8(rb + 16 * kk), acc);
    const int col = 32 * rbs + m;
    const float gs = s.gcum[col];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int row = 32 * rbi + 8 * (e >> 2) + 4 * h + (e & 3);
        float val = 0.f;
        if (col <= row) val = __expf(s.gcum[row] - gs) * acc[e];
        const bf16 hi = (bf16)val;
        s.p[0][row * CS + col] = hi;
        s.p[1][row * CS + col] = (bf16)(val - (float)hi);
    }
}

// ---------------------------------------------------------------- segment lookup
// Segment `seg` (counted over all sequences, L chunks each, an empty sequence
// keeping one empty segment so that its final state is written) -> its
// sequence and chunk range.  Varlen: a wave-wide scan over the offsets, 64
// sequences per step; the result is wave-uniform.
__device__ __forceinline__ SegEntry find_segment(const FwdParams &p, int seg, int lane) {
    SegEntry e;
    e.n = -1;
    int n = -1, r = 0;
    if (!p.cu) {
        const int per = seq_segments(p.T, p.L);
        n = seg / per;
        r = seg - n * per;
        if (n >= p.N) return e;
        e.row0 = (int64_t)n * p.T;
        e.seq_len = (int32_t)p.T;
    } else {
        int base = 0;
        for (int n0 = 0; n0 < p.N; n0 += 64) {
            const int nn = n0 + lane;
            int cnt = 0;
            if (nn < p.N) cnt = seq_segments((int64_t)p.cu[nn + 1] - p.cu[nn], p.L);
            int incl = cnt;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(incl, off, 64);
                if (lane >= off) incl += y;
            }
            const int total = __shfl(incl, 63, 64);
            if (seg < base + total) {
                const unsigned long long hit = __ballot(seg < base + incl && seg >= base + incl - cnt);
                const int src = __ffsll((long long)hit) - 1;
                n = n0 + src;
                r = seg - base - (__shfl(incl, src, 64) - __shfl(cnt, src, 64));
                break;
            }
            base += total;
        }
        n = __builtin_amdgcn_readfirstlane(n);
        r = __builtin_amdgcn_readfirstlane(r);
        if (n < 0) return e;
        e.row0 = p.cu[n];
        e.seq_len = p.cu[n + 1] - p.cu[n];
    }
    const int nt = seq_chunks(e.seq_len);
    const int cnt = seq_segments(e.seq_len, p.L);
    e.n = n;
    e.c_begin = r * p.L;
    e.c_count = min(p.L, max(0, nt - e.c_begin));
    e.last = (r == cnt - 1);
    e.pad = 0;
    return e;
}

// ---------------------------------------------------------------- main kernel
__global__ void __launch_bounds__(NTHREADS, 1) gdn_fwd_main_kernel(FwdParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    Smem &s = *reinterpret_cast<Smem *>(smem_raw);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int n32 = lane & 31, h = lane >> 5;
    const int seg = blockIdx.x / p.Hv;
    const int j = blockIdx.x % p.Hv;
    if (seg >= p.num_segments) return;
    const SegEntry e = find_segment(p, seg, lane);
    if (e.n < 0) return;  // beyond the planned segments: nothing to do
    const int i_qk = j / p.group;
    const int vcol = 32 * wave + n32;  // this lane's value column

    // ---- where this segment's state pass starts
    int c_first = e.c_begin;
    bool from_h0 = (e.c_begin == 0);
    if (!from_h0 && p.cp_mode == 2 /* WARMUP */) {
        // gate-driven window: walk back chunk by chunk until the summed
        // log-gates drop below the fp32 noise floor, the cap, or the start
        float acc = 0.f;
        int w = 0;
        while (w < p.warmup_cap && c_first > 0) {
            const int c = c_first - 1;
            const int tok = c * CH + lane;
            float gv = 0.f;
            if (tok < e.seq_len) gv = p.g[(e.row0 + tok) * p.Hv + j];
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) gv += __shfl_xor(gv, off, 64);
            // every lane holds the same sum; make that explicit so the loop
            // bounds below stay wave-uniform (scalar) values
            acc += __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gv)));
            c_first = c;
            ++w;
            if (acc <= kLnNoiseFloor) break;
        }
        // every wave computed the same window (same data, same order)
        from_h0 = (c_first == 0);
    }
    const int c_end = e.c_begin + e.c_count;

    // ---- state H[:, vcol] in four 32 x 32 accumulator tiles (rows = key dim)
    f32x16 hacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    if (from_h0 && p.h0) {
        const float *h0 = p.h0 + ((int64_t)e.n * p.Hv + j) * DK * DV + vcol;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                hacc[mb][r] = h0[(32 * mb + 8 * (r >> 2) + 4 * h + (r & 3)) * DV];
    }

    if (c_first < c_end) {
        Stage st;
        load_chunk(p, st, e.row0, c_first, e.seq_len, i_qk, j, c_first >= e.c_begin, threadIdx.x);
        for (int c = c_first; c < c_end; ++c) {
            // The thread index is made opaque once per chunk so that the
            // compiler recomputes lane-derived LDS addresses inside the loop
            // instead of hoisting hundreds of them into registers.
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int lane = tid & 63;
            const int n32 = lane & 31, h = lane >> 5;
            const bool out = (c >= e.c_begin);  // warm-up chunks only advance the state
            store_chunk(s, st, out, tid);
            __syncthreads();
            if (c + 1 < c_end) load_chunk(p, st, e.row0, c + 1, e.seq_len, i_qk, j, c + 1 >= e.c_begin, tid);

            prep_cumsum_kkt(s, tid);
            prep_inverse(s, tid);
            prep_scaled_t(s, tid);
            if (out) prep_p(s, tid);
            __syncthreads();

            // W (this wave's 32 key columns, all 64 rows) -> -W in LDS;  U (this wave's value columns)
            f32x16 u[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                f32x16 wacc = {};
                u[rb] = f32x16{};
                const bf16 *ta = &s.tt[(32 * rb + n32) * CS + 8 * h];
                const bf16 *ha = &s.th[0][(32 * rb + n32) * CS + 8 * h];
                const bf16 *la = &s.th[1][(32 * rb + n32) * CS + 8 * h];
                const bf16 *kb = &s.kt[(32 * wave + n32) * CS + 8 * h];
                const bf16 *vb = &s.vt[(32 * wave + n32) * CS + 8 * h];
                const int nk = (rb == 0) ? 2 : 4;  // T is lower triangular
                for (int kk = 0; kk < nk; ++kk) {
                    wacc = mfma(lds8(ta + 16 * kk), lds8(kb + 16 * kk), wacc);
                    const bf16x8 vv = lds8(vb + 16 * kk);
                    u[rb] = mfma(lds8(ha + 16 * kk), vv, u[rb]);
                    u[rb] = mfma(lds8(la + 16 * kk), vv, u[rb]);
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
                    s.w[row * KS + 32 * wave + n32] = (bf16)(-wacc[r]);
                }
            }
            __syncthreads();

            // ---- critical chain: v' = U - W H   (and Q H for the output)
            f32x16 vp[2] = {u[0], u[1]};
            f32x16 qh[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                bf16x8 hh, hl;
                split8(hacc[kk >> 1], kk & 1, hh, hl);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const bf16x8 a = lds8_perm(&s.w[(32 * rb + n32) * KS], 16 * kk, h);
                    vp[rb] = mfma(a, hh, vp[rb]);
                    vp[rb] = mfma(a, hl, vp[rb]);
                }
                if (out) {
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        const bf16x8 a = lds8_perm(&s.q[(32 * rb + n32) * KS], 16 * kk, h);
                        qh[rb] = mfma(a, hh, qh[rb]);
                        qh[rb] = mfma(a, hl, qh[rb]);
                    }
                }
            }
            if (out) {
                // O = scale (diag(gamma) Q H + P v')
                f32x16 pv[2] = {f32x16{}, f32x16{}};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    bf16x8 vh, vl;
                    split8(vp[kk >> 1], kk & 1, vh, vl);
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        if (rb == 0 && kk >= 2) continue;  // P is lower triangular
                        const bf16x8 ah = lds8_perm(&s.p[0][(32 * rb + n32) * CS], 16 * kk, h);
                        const bf16x8 al = lds8_perm(&s.p[1][(32 * rb + n32) * CS], 16 * kk, h);
                        pv[rb] = mfma(ah, vh, pv[rb]);
                        pv[rb] = mfma(ah, vl, pv[rb]);
                        pv[rb] = mfma(al, vh, pv[rb]);
                    }
                }
                const int valid = e.seq_len - c * CH;
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
                        if (row < valid) {
                            const float ov = p.scale * (s.gam[row] * qh[rb][r] + pv[rb][r]);
                            const int64_t off = ((e.row0 + (int64_t)c * CH + row) * p.Hv + j) * DV + 32 * wave + n32;
                            if (p.o_f32)
                                reinterpret_cast<float *>(p.o)[off] = ov;
                            else
                                reinterpret_cast<bf16 *>(p.o)[off] = (bf16)ov;
                        }
                    }
                }
            }
            // ---- H <- gamma_last H + K^T diag(gamma_last / gamma) v'
            const float glast = s.gam[CH - 1];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
                    vp[rb][r] *= s.dec[row];
                }
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) hacc[mb] *= glast;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 vh, vl;
                split8(vp[kk >> 1], kk & 1, vh, vl);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const bf16x8 a = lds8_perm(&s.kt[(32 * mb + n32) * CS], 16 * kk, h);
                    hacc[mb] = mfma(a, vh, hacc[mb]);
                    hacc[mb] = mfma(a, vl, hacc[mb]);
                }
            }
            __syncthreads();  // LDS is rewritten by the next chunk
        }
    }

    if (e.last && p.ht) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int krow = 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
                p.ht[(((int64_t)e.n * p.Hv + j) * DK + krow) * DV + vcol] = hacc[mb][r];
            }
    }
}

// ---------------------------------------------------------------- chunk cumsum
// One thread per (row, head); the thread whose row starts a chunk scans that
// chunk in order, reading each g before writing its sum, so out may equal g.
__global__ void __launch_bounds__(256) gdn_chunk_cumsum_kernel(const float *g, float *out, int64_t B, int64_t T,
                                                               int32_t H, int32_t chunk, const int32_t *cu,
                                                               int32_t N) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = B * T * H;
    if (idx >= total) return;
    const int64_t row = idx / H;
    const int hh = (int)(idx % H);
    int64_t seq0, seq1;
    if (cu) {
        int lo = 0, hi = N;  // sequence lo holds row: cu[lo] <= row < cu[lo + 1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (cu[mid] <= row) lo = mid; else hi = mid;
        }
        while (lo + 1 < N && cu[lo + 1] <= row) ++lo;  // skip empty sequences
        seq0 = cu[lo];
        seq1 = cu[lo + 1];
    } else {
        seq0 = (row / T) * T;
        seq1 = seq0 + T;
    }
    if ((row - seq0) % chunk != 0) return;
    const int64_t end = row + chunk < seq1 ? row + chunk : seq1;
    float acc = 0.f;
    for (int64_t r = row; r < end; ++r) {
        acc += g[r * H + hh];
        out[r * H + hh] = acc;
    }
}

// ---------------------------------------------------------------- launchers
int launch_fwd_main(const FwdParams &p, void *stream) {
    static const size_t smem = sizeof(Smem);
    static const int attr_rc =
        (int)hipFuncSetAttribute((const void *)gdn_fwd_main_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)smem);
    if (attr_rc != 0) return attr_rc;
    const unsigned grid = (unsigned)p.num_segments * (unsigned)p.Hv;
    hipLaunchKernelGGL(gdn_fwd_main_kernel, dim3(grid), dim3(NTHREADS), smem, (hipStream_t)stream, p);
    return (int)hipGetLastError();
}

int launch_chunk_cumsum(const float *g, float *out, int64_t B, int64_t T, int32_t H, int32_t chunk,
                        const int32_t *cu, int32_t N, void *stream) {
    const int64_t total = B * T * H;
    if (total == 0) return 0;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    hipLaunchKernelGGL(gdn_chunk_cumsum_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, g, out, B, T, H,
                       chunk, cu, N);
    return (int)hipGetLastError();
}

const char *hip_error_text(int err) { return hipGetErrorString((hipError_t)err); }


}  // namespace gdn
