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
// Q K^T, K^T T~^T, Q H) use one bf16 MFMA; operands that carry fp32 values
// which feed the output with full weight are split into hi + lo bf16 pairs:
// T diag(beta), P, v', the decayed v', and H.  Decays and beta are fp32
// row/column scales; every exponent is a non-positive difference G_i - G_s
// (masked before the exp), so nothing overflows.
//
// MFMA: v_mfma_f32_32x32x16_bf16.  Lane l holds A row (l % 32) / B column
// (l % 32), 8 k-slots for lane half h = l / 32; accumulator element 4i + j
// holds row 8i + 4h + j, column l % 32.  An accumulator tile read as a B
// operand therefore sees, in k-step s, the k indices 16s + {4h..4h+3,
// 8+4h..8+4h+3}; A operands that meet such a B are read with the same
// permutation.  W and P are produced transposed (W^T = K^T T~^T, P^T = K Q^T)
// so that each lane's accumulator already is its A fragment for W H and P v';
// those fragments go through LDS fragment-major (16 bytes per lane).
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = kChunk;   // 64
constexpr int DK = kDimK;    // 128
constexpr int DV = kDimV;    // 128
constexpr int NTHREADS = 256;
constexpr int KS = DK + 8;   // bf16 row stride of 128-wide tiles (272 B)
constexpr int CS = CH + 8;   // bf16 row stride of 64-wide tiles (144 B)
constexpr int AS = CH + 4;   // fp32 row stride of the 64 x 64 A / T tile (16-byte aligned rows)
constexpr int OS = 32 + 4;   // fp32 row stride of a wave's 64 x 32 output staging tile

struct __attribute__((aligned(16))) Smem {
    bf16 k[CH * KS];       // K, row = token
    bf16 q[CH * KS];       // Q
    bf16 kt[DK * CS];      // K^T, row = key dim
    bf16 vt[DV * CS];      // V^T, row = value dim
    union {
        float a[CH * AS];             // A, inverted in place into T
        float ostage[4][CH * OS];     // per-wave output tile on its way to HBM
    };
    bf16x8 wf[2][8][64];              // -W as A fragments [row block][k step][lane]
    bf16x8 pf[2][3][2][64];           // P as A fragments [hi, lo][tile][k step][lane]
    float scr[2][16 * 17];            // inverse scratch, one per merging wave
    float graw[CH], beta[CH], gcum[CH], gam[CH], dec[CH], bg[CH];
    // e^{G_i - G_s} = ep[i] * em[s] with ep = e^{G - G_ref}, em = e^{G_ref - G},
    // G_ref = G_31; rowa = beta * ep.  Used when every |G - G_ref| < 80 (no
    // overflow in either factor), flagged by fact_ok.
    float ep[CH], em[CH], rowa[CH];
    int fact_ok;
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

__device__ __forceinline__ void split8v(const float *x, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bf16 h = (bf16)x[e];
        hi[e] = h;
        lo[e] = (bf16)(x[e] - (float)h);
    }
}

// ---------------------------------------------------------------- chunk loads
// Buffer resources span exactly one sequence of one head, so rows past the
// sequence end come back as zeros (hardware range check): a partial last
// chunk behaves as if padded with g = beta = 0, k = q = v = 0.
struct Inputs {
    __amdgpu_buffer_rsrc_t k, q, v, g, b;
    unsigned kstride, vstride, gstride;  // bytes per token row
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Thread t stages rows 4*(t % 16) .. +3, columns 8*(t / 16) .. +7 of each
// 64 x 128 tile (16-byte loads).
struct Stage {
    u32x4 k[4], q[4], v[4];
    float g, b;
};

__device__ __forceinline__ void load_chunk(const Inputs &in, Stage &st, int c, bool need_q, int t) {
    const int rg = t & 15, cg = t >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        // offsets are unsigned: past the range they wrap to large values,
        // which the range check also turns into zeros
        const unsigned tok = (unsigned)(c * CH + 4 * rg + r);
        st.k[r] = __builtin_amdgcn_raw_buffer_load_b128(in.k, (int)(tok * in.kstride + 16u * cg), 0, 0);
        st.v[r] = __builtin_amdgcn_raw_buffer_load_b128(in.v, (int)(tok * in.vstride + 16u * cg), 0, 0);
        if (need_q) st.q[r] = __builtin_amdgcn_raw_buffer_load_b128(in.q, (int)(tok * in.kstride + 16u * cg), 0, 0);
    }
    if (t < CH) {
        const unsigned tok = (unsigned)(c * CH + t);
        // the b32 loads return raw bits
        st.g = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(in.g, (int)(tok * in.gstride), 0, 0));
        st.b = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(in.b, (int)(tok * in.gstride), 0, 0));
    }
}

__device__ __forceinline__ uint32_t half_of(const u32x4 &x, int e) {
    return (x[e >> 1] >> (16 * (e & 1))) & 0xffffu;
}

__device__ __forceinline__ void store_chunk(Smem &s, const Stage &st, bool need_q, const int t) {
    const int rg = t & 15, cg = t >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<u32x4 *>(&s.k[(4 * rg + r) * KS + 8 * cg]) = st.k[r];
        if (need_q) *reinterpret_cast<u32x4 *>(&s.q[(4 * rg + r) * KS + 8 * cg]) = st.q[r];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t k01 = half_of(st.k[0], e) | (half_of(st.k[1], e) << 16);
        const uint32_t k23 = half_of(st.k[2], e) | (half_of(st.k[3], e) << 16);
        *reinterpret_cast<uint2 *>(&s.kt[(8 * cg + e) * CS + 4 * rg]) = make_uint2(k01, k23);
        const uint32_t v01 = half_of(st.v[0], e) | (half_of(st.v[1], e) << 16);
        const uint32_t v23 = half_of(st.v[2], e) | (half_of(st.v[3], e) << 16);
        *reinterpret_cast<uint2 *>(&s.vt[(8 * cg + e) * CS + 4 * rg]) = make_uint2(v01, v23);
    }
    if (t < CH) {
        s.graw[t] = st.g;
        s.beta[t] = st.b;
    }
}

// ---------------------------------------------------------------- chunk prep
// Cumsum (wave 0), masked beta-weighted K K^T into s.a (waves 1..3), and the
// causal decayed P^T = K Q^T as hi/lo A fragments (waves 0..2, output chunks).
// P^T tile t covers (s block, i block) = (0,0), (0,1), (1,1).
__device__ __forceinline__ void prep_products(Smem &s, const int tid, const bool out) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, h = lane >> 5;
    f32x16 acck = {}, accp = {};
    const int rbi = (wave >= 2) ? 1 : 0, rbs = (wave == 3) ? 1 : 0;  // K K^T tile of waves 1..3
    const int psb = (wave == 2) ? 1 : 0, prb = (wave >= 1) ? 1 : 0;  // P^T tile of waves 0..2
    if (wave == 0) {
        float x = s.graw[lane];
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        const float glast = __shfl(x, 63, 64);
        const float gref = __shfl(x, 31, 64);
        const float gm = __expf(x);
        const float d = x - gref;
        const float bt = s.beta[lane];
        const float epv = __expf(d);
        s.gcum[lane] = x;
        s.gam[lane] = gm;
        s.dec[lane] = __expf(glast - x);
        s.bg[lane] = bt * gm;
        s.ep[lane] = epv;
        s.em[lane] = __expf(-d);
        s.rowa[lane] = bt * epv;
        const bool ok = __all(fabsf(d) < 80.f);
        if (lane == 0) s.fact_ok = ok ? 1 : 0;
    } else {
        const bf16 *ra = &s.k[(32 * rbi + m) * KS + 8 * h];
        const bf16 *rb = &s.k[(32 * rbs + m) * KS + 8 * h];
#pragma unroll
        for (int kk = 0; kk < DK / 16; ++kk) acck = mfma(lds8(ra + 16 * kk), lds8(rb + 16 * kk), acck);
    }
    if (out && wave <= 2) {
        const bf16 *ra = &s.k[(32 * psb + m) * KS + 8 * h];
        const bf16 *rb = &s.q[(32 * prb + m) * KS + 8 * h];
#pragma unroll
        for (int kk = 0; kk < DK / 16; ++kk) accp = mfma(lds8(ra + 16 * kk), lds8(rb + 16 * kk), accp);
    }
    __syncthreads();
    const bool fact = __builtin_amdgcn_readfirstlane(s.fact_ok) != 0;
    if (wave != 0) {
        // A_is = beta_i e^{G_i - G_s} k_i.k_s for s < i (rows of this lane: 4 runs of 4)
        const int col = 32 * rbs + m;
        float v[16];
        if (fact) {
            const float cf = s.em[col];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const f32x4 ra4 = *reinterpret_cast<const f32x4 *>(&s.rowa[32 * rbi + 8 * ii + 4 * h]);
#pragma unroll
                for (int j = 0; j < 4; ++j) v[4 * ii + j] = ra4[j] * cf * acck[4 * ii + j];
            }
        } else {
            const float gs = s.gcum[col];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&s.gcum[32 * rbi + 8 * ii + 4 * h]);
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&s.beta[32 * rbi + 8 * ii + 4 * h]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 32 * rbi + 8 * ii + 4 * h + j;
                    v[4 * ii + j] = (col < row) ? b4[j] * __expf(g4[j] - gs) * acck[4 * ii + j] : 0.f;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = 32 * rbi + 8 * (e >> 2) + 4 * h + (e & 3);
            s.a[row * AS + col] = (col < row) ? v[e] : 0.f;
        }
    }
    if (out && wave <= 2) {
        // P^T_si = e^{G_i - G_s} q_i.k_s for s <= i (i = this lane's column)
        const int i = 32 * prb + m;
        float pv[16];
        if (fact) {
            const float cf = s.ep[i];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const f32x4 e4 = *reinterpret_cast<const f32x4 *>(&s.em[32 * psb + 8 * ii + 4 * h]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int srow = 32 * psb + 8 * ii + 4 * h + j;
                    pv[4 * ii + j] = (srow <= i) ? cf * e4[j] * accp[4 * ii + j] : 0.f;
                }
            }
        } else {
            const float gi = s.gcum[i];
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&s.gcum[32 * psb + 8 * ii + 4 * h]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int srow = 32 * psb + 8 * ii + 4 * h + j;
                    pv[4 * ii + j] = (srow <= i) ? __expf(gi - g4[j]) * accp[4 * ii + j] : 0.f;
                }
            }
        }
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
            bf16x8 hi, lo;
            split8v(pv + 8 * kp, hi, lo);
            s.pf[0][wave][kp][lane] = hi;
            s.pf[1][wave][kp][lane] = lo;
        }
    }
    __syncthreads();
}

// In-place inverse of the unit lower-triangular (I + A) held as A in s.a.
// Level 0: the four 16 x 16 diagonal blocks by forward substitution (one lane
// per column).  Level 1: T_10 = -T_11 A_10 T_00 inside each 32 x 32 diagonal
// block.  Level 2 (MFMA, hi/lo bf16): T_lo,hi = -T_lo,lo A_lo,hi T_hi,hi.
// Entries above the diagonal of each diagonal block hold zeros throughout.
__device__ __forceinline__ void prep_inverse(Smem &s, const int tid) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    if (wave < 2 && lane < 32) {
        const int o = 32 * wave + 16 * (lane >> 4), c = lane & 15;
        float t[16];
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
            float ar[16];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                if (4 * q4 < ii) {
                    const f32x4 x = *reinterpret_cast<const f32x4 *>(&s.a[(o + ii) * AS + o + 4 * q4]);
#pragma unroll
                    for (int j = 0; j < 4; ++j) ar[4 * q4 + j] = x[j];
                }
            }
            float acc = (ii == c) ? 1.f : 0.f;
#pragma unroll
            for (int ss = 0; ss < ii; ++ss) acc -= ar[ss] * t[ss];
            t[ii] = acc;
        }
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) s.a[(o + ii) * AS + o + c] = t[ii];
    }
    __syncthreads();
    const int c = lane & 15, r4 = 4 * (lane >> 4);
    if (wave < 2) {
        const int b = 32 * wave;
        float tc[16];  // column c of T_00
#pragma unroll
        for (int ss = 0; ss < 16; ++ss) tc[ss] = s.a[(b + ss) * AS + b + c];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            float acc = 0.f;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(&s.a[(b + 16 + r4 + rr) * AS + b + 4 * q4]);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc += x[j] * tc[4 * q4 + j];
            }
            s.scr[wave][(r4 + rr) * 17 + c] = acc;
        }
    }
    __syncthreads();
    if (wave < 2) {
        const int b = 32 * wave;
        float xc[16];  // column c of X = A_10 T_00
#pragma unroll
        for (int ss = 0; ss < 16; ++ss) xc[ss] = s.scr[wave][ss * 17 + c];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            float acc = 0.f;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(&s.a[(b + 16 + r4 + rr) * AS + b + 16 + 4 * q4]);
#pragma unroll
                for (int j = 0; j < 4; ++j) acc += x[j] * xc[4 * q4 + j];
            }
            s.a[(b + 16 + r4 + rr) * AS + b + c] = -acc;
        }
    }
    __syncthreads();
    if (wave == 0) {
        const int m = lane & 31, h = lane >> 5;
        f32x16 y = {};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const float *ar = &s.a[(32 + m) * AS + 16 * kk + 8 * h];
            float av[8], bv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                av[e] = ar[e];
                bv[e] = s.a[(16 * kk + 8 * h + e) * AS + m];
            }
            bf16x8 ah, al, bh, bl;
            split8v(av, ah, al);
            split8v(bv, bh, bl);
            y = mfma(ah, bh, y);
            y = mfma(ah, bl, y);
            y = mfma(al, bh, y);
        }
        f32x16 z = {};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const float *tr = &s.a[(32 + m) * AS + 32 + 16 * kk + 4 * h];
            float av[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                av[e] = tr[e];
                av[4 + e] = tr[8 + e];
            }
            bf16x8 ah, al, bh, bl;
            split8v(av, ah, al);
            split8(y, kk, bh, bl);
            z = mfma(ah, bh, z);
            z = mfma(ah, bl, z);
            z = mfma(al, bh, z);
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) s.a[(32 + 8 * (e >> 2) + 4 * h + (e & 3)) * AS + m] = -z[e];
    }
    __syncthreads();
}

// W^T = K^T (T diag(beta gamma))^T for this wave's 32 key dims -> -W A
// fragments in LDS; U = (T diag(beta)) V for this wave's 32 value columns.
__device__ __forceinline__ void prep_wu(Smem &s, const int tid, f32x16 (&u)[2]) {
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int m = lane & 31, h = lane >> 5;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        f32x16 w = {};
        u[rb] = f32x16{};
        const int nk = (rb == 0) ? 2 : 4;  // T is lower triangular
#pragma unroll
        for (int kk = 0; kk < nk; ++kk) {
            const float *tr = &s.a[(32 * rb + m) * AS + 16 * kk + 8 * h];
            const float *bgp = &s.bg[16 * kk + 8 * h];
            const float *bp = &s.beta[16 * kk + 8 * h];
            bf16x8 tw, th, tl;
            float tb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float tv = tr[e];
                tw[e] = (bf16)(tv * bgp[e]);
                tb[e] = tv * bp[e];
            }
            split8v(tb, th, tl);
            w = mfma(lds8(&s.kt[(32 * wave + m) * CS + 16 * kk + 8 * h]), tw, w);
            const bf16x8 vv = lds8(&s.vt[(32 * wave + m) * CS + 16 * kk + 8 * h]);
            u[rb] = mfma(th, vv, u[rb]);
            u[rb] = mfma(tl, vv, u[rb]);
        }
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
            bf16x8 f;
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = (bf16)(-w[8 * kp + e]);
            s.wf[rb][2 * wave + kp][lane] = f;
        }
    }
    __syncthreads();
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

// ---------------------------------------------------------------- output store
// One chunk's output tile of this wave (64 rows x 32 value columns, in the
// accumulator layout) goes through a wave-private LDS staging tile so that
// every lane writes 16 contiguous bytes.
__device__ __forceinline__ void write_o(Smem &s, const FwdParams &p, const SegEntry &e, int j, int c,
                                        const f32x16 (&ov)[2], const int wave, const int ln) {
    const int m = ln & 31, h = ln >> 5;
    float *stg = s.ostage[wave];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) stg[(32 * rb + 8 * (r >> 2) + 4 * h + (r & 3)) * OS + m] = ov[rb][r];
    // the staging tile is private to this wave: LDS keeps the wave's own
    // write/read order; the fence keeps the compiler's
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    const int valid = e.seq_len - c * CH;
    const int64_t obase = ((e.row0 + (int64_t)c * CH) * p.Hv + j) * DV + 32 * wave;
    if (p.o_f32) {
#pragma unroll
        for (int pass = 0; pass < 8; ++pass) {
            const int row = 8 * pass + (ln >> 3), c4 = 4 * (ln & 7);
            if (row < valid)
                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.o) + obase + (int64_t)row * p.Hv * DV + c4) =
                    *reinterpret_cast<const f32x4 *>(&stg[row * OS + c4]);
        }
    } else {
#pragma unroll
        for (int pass = 0; pass < 4; ++pass) {
            const int row = 16 * pass + (ln >> 2), c8 = 8 * (ln & 3);
            const f32x4 x0 = *reinterpret_cast<const f32x4 *>(&stg[row * OS + c8]);
            const f32x4 x1 = *reinterpret_cast<const f32x4 *>(&stg[row * OS + c8 + 4]);
            const bf16x8 y = {(bf16)x0[0], (bf16)x0[1], (bf16)x0[2], (bf16)x0[3],
                              (bf16)x1[0], (bf16)x1[1], (bf16)x1[2], (bf16)x1[3]};
            if (row < valid)
                *reinterpret_cast<bf16x8 *>(reinterpret_cast<bf16 *>(p.o) + obase + (int64_t)row * p.Hv * DV + c8) = y;
        }
    }
}

// ---------------------------------------------------------------- state I/O
// A K x V fp32 state (row = key dim) <-> this wave's four accumulator tiles
// (value columns 32 wave .. 32 wave + 31); each access is one 128-byte row piece.
__device__ __forceinline__ void load_state(f32x16 (&t)[4], const float *src, const int wave, const int lane) {
    const int m = lane & 31, h = lane >> 5;
    const float *b = src + 32 * wave + m;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) t[mb][r] = b[(32 * mb + 8 * (r >> 2) + 4 * h + (r & 3)) * DV];
}

__device__ __forceinline__ void store_state(const f32x16 (&t)[4], float *dst, const int wave, const int lane) {
    const int m = lane & 31, h = lane >> 5;
    float *b = dst + 32 * wave + m;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) b[(32 * mb + 8 * (r >> 2) + 4 * h + (r & 3)) * DV] = t[mb][r];
}

// ---------------------------------------------------------------- main kernel
__global__ void __launch_bounds__(NTHREADS, 1) gdn_fwd_main_kernel(FwdParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    Smem &s = *reinterpret_cast<Smem *>(smem_raw);

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int seg = blockIdx.x / p.Hv;
    const int j = blockIdx.x % p.Hv;
    if (seg >= p.num_segments) return;
    const SegEntry e = find_segment(p, seg, lane);
    if (e.n < 0) return;  // beyond the planned segments: nothing to do
    const int i_qk = j / p.group;

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
        from_h0 = (c_first == 0);
    }
    const int c_end = e.c_begin + e.c_count;

    // ---- state H[:, this lane's value column] in four 32 x 32 accumulator tiles
    f32x16 hacc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    {
        const float *src = nullptr;
        if (from_h0 && p.h0) src = p.h0 + ((int64_t)e.n * p.Hv + j) * DK * DV;
        if (!from_h0 && p.cp_mode == 1 /* EXACT */) src = p.ws_h + ((int64_t)seg * p.Hv + j) * DK * DV;
        if (src) load_state(hacc, src, wave, lane);
    }

    if (c_first < c_end) {
        Inputs in;
        in.kstride = (unsigned)p.Hqk * DK * 2;
        in.vstride = (unsigned)p.Hv * DV * 2;
        in.gstride = (unsigned)p.Hv * 4;
        in.k = make_rsrc(p.k + (e.row0 * p.Hqk + i_qk) * DK, (int64_t)e.seq_len * in.kstride);
        in.q = make_rsrc(p.q + (e.row0 * p.Hqk + i_qk) * DK, (int64_t)e.seq_len * in.kstride);
        in.v = make_rsrc(p.v + (e.row0 * p.Hv + j) * DV, (int64_t)e.seq_len * in.vstride);
        in.g = make_rsrc(p.g + e.row0 * p.Hv + j, (int64_t)e.seq_len * in.gstride);
        in.b = make_rsrc(p.beta + e.row0 * p.Hv + j, (int64_t)e.seq_len * in.gstride);

        Stage st;
        load_chunk(in, st, c_first, c_first >= e.c_begin, threadIdx.x);
        // A chunk's output waits in registers and is stored at the top of the
        // next iteration, after that iteration's prefetched inputs have been
        // consumed: memory-counter waits for the prefetch then never have to
        // cover freshly issued output stores.
        f32x16 ov[2];
        int pend = -1;  // chunk whose output is held in ov, or -1
        for (int c = c_first; c < c_end; ++c) {
            // The thread index is made opaque once per chunk so that the
            // compiler recomputes lane-derived LDS addresses inside the loop
            // instead of hoisting hundreds of them into registers.
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int ln = tid & 63;
            const int m = ln & 31, h = ln >> 5;
            const bool out = (c >= e.c_begin);  // warm-up chunks only advance the state
            store_chunk(s, st, out, tid);
            __syncthreads();
            if (pend >= 0) write_o(s, p, e, j, pend, ov, wave, ln);  // staging aliases s.a, free until the masks
            pend = -1;
            if (c + 1 < c_end) load_chunk(in, st, c + 1, c + 1 >= e.c_begin, tid);

            prep_products(s, tid, out);
            prep_inverse(s, tid);
            f32x16 u[2];
            prep_wu(s, tid, u);

            // ---- critical chain: v' = U - W H   (and Q H for the output)
            f32x16 vp[2] = {u[0], u[1]};
            f32x16 qh[2] = {f32x16{}, f32x16{}};
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                bf16x8 hh, hl;
                split8(hacc[kk >> 1], kk & 1, hh, hl);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    const bf16x8 a = s.wf[rb][kk][ln];
                    vp[rb] = mfma(a, hh, vp[rb]);
                    vp[rb] = mfma(a, hl, vp[rb]);
                }
                if (out) {
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        const bf16x8 a = lds8_perm(&s.q[(32 * rb + m) * KS], 16 * kk, h);
                        qh[rb] = mfma(a, hh, qh[rb]);
                        qh[rb] = mfma(a, hl, qh[rb]);
                    }
                }
            }
            if (out) {
                // O = scale (diag(gamma) Q H + P v'), staged through LDS per wave
                f32x16 pv[2] = {f32x16{}, f32x16{}};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    bf16x8 vh, vl;
                    split8(vp[kk >> 1], kk & 1, vh, vl);
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        if (rb == 0 && kk >= 2) continue;  // P is lower triangular
                        const int t = (rb == 0) ? 0 : (kk < 2 ? 1 : 2);
                        const bf16x8 ah = s.pf[0][t][kk & 1][ln];
                        const bf16x8 al = s.pf[1][t][kk & 1][ln];
                        pv[rb] = mfma(ah, vh, pv[rb]);
                        pv[rb] = mfma(ah, vl, pv[rb]);
                        pv[rb] = mfma(al, vh, pv[rb]);
                    }
                }
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int row = 32 * rb + 8 * (r >> 2) + 4 * h + (r & 3);
                        ov[rb][r] = p.scale * (s.gam[row] * qh[rb][r] + pv[rb][r]);
                    }
                pend = c;
            }
            // ---- H <- gamma_last H + K^T diag(gamma_last / gamma) v'
            const float glast = s.gam[CH - 1];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int r = 0; r < 16; ++r) vp[rb][r] *= s.dec[32 * rb + 8 * (r >> 2) + 4 * h + (r & 3)];
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) hacc[mb] *= glast;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 vh, vl;
                split8(vp[kk >> 1], kk & 1, vh, vl);
#pragma unroll
                for (int mb = 0; mb < 4; ++mb) {
                    const bf16x8 a = lds8_perm(&s.kt[(32 * mb + m) * CS], 16 * kk, h);
                    hacc[mb] = mfma(a, vh, hacc[mb]);
                    hacc[mb] = mfma(a, vl, hacc[mb]);
                }
            }
            __syncthreads();  // LDS is rewritten by the next chunk
        }
        if (pend >= 0) write_o(s, p, e, j, pend, ov, wave, threadIdx.x & 63);
    }

    if (e.last && p.ht) store_state(hacc, p.ht + ((int64_t)e.n * p.Hv + j) * DK * DV, wave, lane);
}

// ---------------------------------------------------------------- exact context parallelism
// Pre-pass (blog, AutoCP: the per-segment M and S).  For every segment that is
// not the last of its sequence: S = the state pass over the segment from a
// zero state, and M = the same pass without inputs (U = 0) from the identity,
// i.e. the product of the chunk maps X -> gamma_last X - K^T diag(gamma_last /
// gamma) W X.  Then the segment's end state is M H_start + S.
__global__ void __launch_bounds__(NTHREADS, 1) gdn_cp_prepass_kernel(FwdParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    Smem &s = *reinterpret_cast<Smem *>(smem_raw);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int seg = blockIdx.x / p.Hv;
    const int j = blockIdx.x % p.Hv;
    if (seg >= p.num_segments) return;
    const SegEntry e = find_segment(p, seg, lane);
    if (e.n < 0 || e.last) return;  // a last segment's map is never used
    const int i_qk = j / p.group;

    f32x16 hs[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    f32x16 hm[4];
    {
        const int m = lane & 31, h = lane >> 5;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                hm[mb][r] = (32 * mb + 8 * (r >> 2) + 4 * h + (r & 3) == 32 * wave + m) ? 1.f : 0.f;
    }
    const int c_end = e.c_begin + e.c_count;
    Inputs in;
    in.kstride = (unsigned)p.Hqk * DK * 2;
    in.vstride = (unsigned)p.Hv * DV * 2;
    in.gstride = (unsigned)p.Hv * 4;
    in.k = make_rsrc(p.k + (e.row0 * p.Hqk + i_qk) * DK, (int64_t)e.seq_len * in.kstride);
    in.q = in.k;  // not read: no output here
    in.v = make_rsrc(p.v + (e.row0 * p.Hv + j) * DV, (int64_t)e.seq_len * in.vstride);
    in.g = make_rsrc(p.g + e.row0 * p.Hv + j, (int64_t)e.seq_len * in.gstride);
    in.b = make_rsrc(p.beta + e.row0 * p.Hv + j, (int64_t)e.seq_len * in.gstride);

    Stage st;
    load_chunk(in, st, e.c_begin, false, threadIdx.x);
    for (int c = e.c_begin; c < c_end; ++c) {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int ln = tid & 63;
        const int m = ln & 31, h = ln >> 5;
        store_chunk(s, st, false, tid);
        __syncthreads();
        if (c + 1 < c_end) load_chunk(in, st, c + 1, false, tid);
        prep_products(s, tid, false);
        prep_inverse(s, tid);
        f32x16 u[2];
        prep_wu(s, tid, u);

        f32x16 vs[2] = {u[0], u[1]};
        f32x16 vm[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            bf16x8 sh, sl, mh, ml;
            split8(hs[kk >> 1], kk & 1, sh, sl);
            split8(hm[kk >> 1], kk & 1, mh, ml);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const bf16x8 a = s.wf[rb][kk][ln];
                vs[rb] = mfma(a, sh, vs[rb]);
                vs[rb] = mfma(a, sl, vs[rb]);
                vm[rb] = mfma(a, mh, vm[rb]);
                vm[rb] = mfma(a, ml, vm[rb]);
            }
        }
        const float glast = s.gam[CH - 1];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float d = s.dec[32 * rb + 8 * (r >> 2) + 4 * h + (r & 3)];
                vs[rb][r] *= d;
                vm[rb][r] *= d;
            }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            hs[mb] *= glast;
            hm[mb] *= glast;
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 sh, sl, mh, ml;
            split8(vs[kk >> 1], kk & 1, sh, sl);
            split8(vm[kk >> 1], kk & 1, mh, ml);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const bf16x8 a = lds8_perm(&s.kt[(32 * mb + m) * CS], 16 * kk, h);
                hs[mb] = mfma(a, sh, hs[mb]);
                hs[mb] = mfma(a, sl, hs[mb]);
                hm[mb] = mfma(a, mh, hm[mb]);
                hm[mb] = mfma(a, ml, hm[mb]);
            }
        }
        __syncthreads();
    }
    const int64_t off = ((int64_t)seg * p.Hv + j) * DK * DV;
    store_state(hs, p.ws_s + off, wave, lane);
    store_state(hm, p.ws_m + off, wave, lane);
}

// Combine (sequential over a sequence's segments): H_start[0] = initial state,
// H_start[r+1] = M_r H_start[r] + S_r.  One workgroup per (sequence, v-head);
// wave w owns value columns 32w..32w+31, M_r H on MFMA with hi/lo operands.
__global__ void __launch_bounds__(NTHREADS, 1) gdn_cp_combine_kernel(FwdParams p) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int m = lane & 31, h = lane >> 5;
    const int n = blockIdx.x / p.Hv;
    const int j = blockIdx.x % p.Hv;
    if (n >= p.N) return;
    // first segment of sequence n and its segment count
    int seg0 = 0, R = 0;
    if (!p.cu) {
        R = seq_segments(p.T, p.L);
        seg0 = n * R;
    } else {
        int base = 0;
        for (int n0 = 0; n0 < n; n0 += 64) {
            const int nn = n0 + lane;
            int cnt = (nn < n) ? seq_segments((int64_t)p.cu[nn + 1] - p.cu[nn], p.L) : 0;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
            base += __builtin_amdgcn_readfirstlane(cnt);
        }
        seg0 = base;
        R = seq_segments((int64_t)p.cu[n + 1] - p.cu[n], p.L);
    }
    if (R <= 1) return;
    f32x16 H[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    if (p.h0) load_state(H, p.h0 + ((int64_t)n * p.Hv + j) * DK * DV, wave, lane);
    for (int r = 0; r + 1 < R; ++r) {
        const int64_t off = ((int64_t)(seg0 + r) * p.Hv + j) * DK * DV;
        const float *M = p.ws_m + off;
        f32x16 X[4];
        load_state(X, p.ws_s + off, wave, lane);  // start from S_r, accumulate M_r H
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            bf16x8 bh, bl;
            split8(H[kk >> 1], kk & 1, bh, bl);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const float *row = M + (int64_t)(32 * mb + m) * DK + 16 * kk + 4 * h;
                const f32x4 x0 = *reinterpret_cast<const f32x4 *>(row);
                const f32x4 x1 = *reinterpret_cast<const f32x4 *>(row + 8);
                const float av[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
                bf16x8 ah, al;
                split8v(av, ah, al);
                X[mb] = mfma(ah, bh, X[mb]);
                X[mb] = mfma(ah, bl, X[mb]);
                X[mb] = mfma(al, bh, X[mb]);
            }
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) H[mb] = X[mb];
        store_state(H, p.ws_h + ((int64_t)(seg0 + r + 1) * p.Hv + j) * DK * DV, wave, lane);
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

int launch_cp_exact(const FwdParams &p, void *stream) {
    static const size_t smem = sizeof(Smem);
    static const int attr_rc =
        (int)hipFuncSetAttribute((const void *)gdn_cp_prepass_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)smem);
    if (attr_rc != 0) return attr_rc;
    const unsigned grid = (unsigned)p.num_segments * (unsigned)p.Hv;
    hipLaunchKernelGGL(gdn_cp_prepass_kernel, dim3(grid), dim3(NTHREADS), smem, (hipStream_t)stream, p);
    int err = (int)hipGetLastError();
    if (err) return err;
    hipLaunchKernelGGL(gdn_cp_combine_kernel, dim3((unsigned)p.N * (unsigned)p.Hv), dim3(NTHREADS), 0,
                       (hipStream_t)stream, p);
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
