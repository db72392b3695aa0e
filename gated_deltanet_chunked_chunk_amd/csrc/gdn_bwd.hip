// Gated DeltaNet chunked backward: HIP kernels for gfx950 (MI355X).
//
// The chunked backward the FlashQLA pages announce (agentlenshq.com blog,
// title, "performance benchmarks": a fused backward; aisparkup.com wiki, "key
// features") is not printed there; it is the reverse-mode derivative of the
// chunked WY forward (gdn_fwd.hip).  Per (sequence, v-head) and chunk, with
// chunk-start state h, gradient dh' with respect to the state after the chunk,
// G the in-chunk prefix sums of g, gamma = e^G, Gamma_is = e^{G_i - G_s},
// rl_s = gamma_last / gamma_s, T the chunk's WY matrix (I + A~)^{-1}:
//
//   W   = T diag(beta gamma) K           v' = T diag(beta) V - W h
//   P   = (Q K^T) o Gamma (s <= i)       O  = scale [diag(gamma) Q h + P v']
//   h'  = gamma_last h + (diag(rl) K)^T v'
//
// reverse pass (sequential over chunks, the state-pass adjoint):
//   dv' = scale P^T dO + diag(rl) K dh'
//   dh  = gamma_last dh' + scale (diag(gamma) Q)^T dO - W^T dv'
// chunk-local gradients (every chunk independent):
//   dPm = scale (dO v'^T) o Gamma (s <= i)
//   dQ  = dPm K + scale diag(gamma) dO h^T
//   dW  = -dv' h^T,  dT = (dW K^T) diag(beta gamma) + (dv' V^T) diag(beta)
//   dA~ = -(T^T dT T^T) (strictly lower),  M = dA~ o beta_i Gamma_is
//   dK  = dPm^T Q + diag(rl) v' dh'^T + diag(beta gamma) T^T dW + M K + M^T K
//   dV  = diag(beta) T^T dv'
//   dbeta_s = gamma_s (T^T dW)_s.k_s + (T^T dv')_s.v_s + sum_c dA~_sc Gamma_sc k_s.k_c
//   dG_i: the gate terms of O (inter and intra), h', W and A~; dg = reverse
//         in-chunk cumsum of dG.
//
// Kernels: gdn_bwd_dh_kernel (reverse pass, one workgroup per (segment,
// v-head, half of V): the V columns of dh are independent), gdn_bwd_local_kernel
// (one workgroup per (chunk, v-head)), gdn_bwd_group_sum_kernel (dq, dk of a
// key head = sum over its v-heads).  h and T come from the forward (its
// low-level outputs); dh' and dv' of every chunk go through the workspace.
//
// Products: v_mfma_f32_16x16x32_bf16 on 16 x 16 output tiles.  Operands that
// hold exact bf16 inputs (K, Q, V, dO) enter as one bf16 term; fp32 operands
// (T, W, P, v', dv', h, dh, gate-scaled operands) are split hi + lo bf16 and
// enter as hi*hi + lo*hi + hi*lo.  Lane l holds A row / B column l % 16 with
// k-slots 8 (l / 16) .. +7; accumulator element j is row 4 (l / 16) + j,
// column l % 16.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "gdn_internal.h"

namespace gdn {
namespace bwdk {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int CH = kChunk;  // 64
constexpr int DK = kDimK;   // 128
constexpr int DV = kDimV;   // 128
constexpr int NT = 512;     // threads per workgroup (8 waves)
constexpr int HVC = 64;     // value columns per reverse-pass workgroup

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float ldf(const float *p) { return *p; }
__device__ __forceinline__ float ldf(const bf16 *p) { return (float)*p; }

// eight k-consecutive values of one operand row / column (k stride ks)
template <typename T, bool CONTIG>
__device__ __forceinline__ void load8(const T *p, int ks, float (&x)[8]) {
    if constexpr (CONTIG && sizeof(T) == 4) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[e] = a[e];
            x[4 + e] = b[e];
        }
    } else if constexpr (CONTIG) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)a[e];
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = ldf(p + e * ks);
    }
}

__device__ __forceinline__ void to_bf16(const float (&x)[8], bf16x8 &h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (bf16)x[e];
}

__device__ __forceinline__ void split(const float (&x)[8], bf16x8 &h, bf16x8 &l) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = (bf16)x[e];
        l[e] = (bf16)(x[e] - (float)h[e]);
    }
}

// acc += A (16 x kd) B (kd x 16) for one output tile, A(m, k) = a[m ams + k aks],
// B(k, n) = b[k bks + n bns]; AC / BC: unit k stride (vector loads).  SA: A is
// scaled by sa[k] along k (then split like an fp32 operand).
template <typename TA, bool AC, typename TB, bool BC, bool SA = false>
__device__ __forceinline__ f32x4 mm16(f32x4 acc, const TA *a, int ams, int aks, const TB *b, int bns, int bks,
                                      int kd, int lane, const float *sa = nullptr) {
    constexpr bool EA = sizeof(TA) == 2 && !SA;
    constexpr bool EB = sizeof(TB) == 2;
    const int r = lane & 15, kq = (lane >> 4) * 8;
    const TA *pa = a + r * ams + kq * aks;
    const TB *pb = b + r * bns + kq * bks;
    for (int k0 = 0; k0 < kd; k0 += 32) {
        float xa[8], xb[8];
        load8<TA, AC>(pa + k0 * aks, aks, xa);
        load8<TB, BC>(pb + k0 * bks, bks, xb);
        if constexpr (SA) {
#pragma unroll
            for (int e = 0; e < 8; ++e) xa[e] *= sa[k0 + kq + e];
        }
        bf16x8 ah, al, bh, bl;
        if constexpr (EA) to_bf16(xa, ah); else split(xa, ah, al);
        if constexpr (EB) to_bf16(xb, bh); else split(xb, bh, bl);
        acc = mfma(ah, bh, acc);
        if constexpr (!EA) acc = mfma(al, bh, acc);
        if constexpr (!EB) acc = mfma(ah, bl, acc);
    }
    return acc;
}

// sum over the 16 lanes that share l / 16 (one accumulator row group)
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}
// sum over the four lane groups l / 16 (lanes l % 16 equal)
__device__ __forceinline__ float sum4g(float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
}
__device__ __forceinline__ float sum64(float x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// ---------------------------------------------------------------- rows of a chunk
// Buffer resource over chunk c's rows of one sequence: rows past the sequence
// end read as zeros and stores to them are dropped (hardware range check), so
// a partial last chunk behaves as if padded with zero inputs.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void *base, unsigned stride, int c, int seq_len) {
    const int rows = min(max(seq_len - c * CH, 0), CH);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(static_cast<const char *>(base) + (int64_t)c * CH * stride), (short)0,
        (int)(rows * stride), 0x00020000);
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float ld4(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// 64 rows x (16-byte pieces per row) from HBM rows into a dense LDS tile
__device__ __forceinline__ void stage_rows(void *dst, const void *base, unsigned stride, int c, int seq_len,
                                           int pieces_per_row, int tid) {
    const __amdgpu_buffer_rsrc_t r = chunk_rsrc(base, stride, c, seq_len);
    u32x4 *d = static_cast<u32x4 *>(dst);
    const int total = CH * pieces_per_row;
    for (int pc = tid; pc < total; pc += NT) {
        const int row = pc / pieces_per_row, col = pc - row * pieces_per_row;
        d[pc] = ld16(r, (unsigned)row * stride + (unsigned)col * 16u);
    }
}

// ---------------------------------------------------------------- sequences
struct Where {
    int n;          // sequence (-1: none)
    int c_begin;    // first chunk (from the sequence start)
    int c_count;    // chunks
    int seq_len;
    int64_t row0;
    int last;       // segment ends its sequence
};

// Segment `seg` of L chunks, counted over all sequences (an empty sequence
// keeps one empty segment) -> sequence and chunk range.  Wave-uniform.
__device__ __forceinline__ Where find_segment(const int32_t *cu, int N, int64_t T, int L, int seg, int lane) {
    Where e;
    e.n = -1;
    int n = -1, r = 0;
    if (!cu) {
        const int per = seq_segments(T, L);
        n = seg / per;
        r = seg - n * per;
        if (n >= N) return e;
        e.row0 = (int64_t)n * T;
        e.seq_len = (int)T;
    } else {
        int base = 0;
        for (int n0 = 0; n0 < N; n0 += 64) {
            const int nn = n0 + lane;
            int cnt = 0;
            if (nn < N) cnt = seq_segments((int64_t)cu[nn + 1] - cu[nn], L);
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
        e.row0 = cu[n];
        e.seq_len = cu[n + 1] - cu[n];
    }
    const int nt = seq_chunks(e.seq_len);
    const int cnt = seq_segments(e.seq_len, L);
    e.n = n;
    e.c_begin = r * L;
    e.c_count = min(L, max(0, nt - e.c_begin));
    e.last = (r == cnt - 1);
    return e;
}

// index of sequence n's first chunk among the chunks of all sequences
__device__ __forceinline__ int seq_chunk_base(const int32_t *cu, int64_t T, int n, int lane) {
    if (!cu) return n * seq_chunks(T);
    int base = 0;
    for (int n0 = 0; n0 < n; n0 += 64) {
        const int nn = n0 + lane;
        int cnt = (nn < n) ? seq_chunks((int64_t)cu[nn + 1] - cu[nn]) : 0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
        base += __builtin_amdgcn_readfirstlane(cnt);
    }
    return base;
}

// in-chunk gate vectors from the staged raw g (lane i = token i; wave 0 only):
// G prefix sums, gamma, and the last-token ratios rl_i = e^{G_last - G_i}
__device__ __forceinline__ float prefix64(float x, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// ---------------------------------------------------------------- reverse pass
struct __attribute__((aligned(16))) SmemDh {
    bf16 k[CH * DK];     // K, row = token
    bf16 q[CH * DK];     // Q
    bf16 dO[CH * HVC];   // dO, this workgroup's 64 value columns
    float t[CH * CH];    // T, row = token
    float w[CH * DK];    // W
    float p[CH * CH];    // P (masked, decayed)
    float dvp[CH * HVC]; // dv'
    float dh[DK * HVC];  // dh (key rows x this workgroup's value columns)
    float G[CH], gam[CH], bg[CH], rl[CH];
};
static_assert(sizeof(SmemDh) <= 160 * 1024, "reverse-pass LDS over 160 KB");

__device__ __forceinline__ void stage_chunk_dh(SmemDh &s, const BwdParams &p, const Where &e, int j, int half, int c,
                                               int tid) {
    const int iq = j / p.group;
    const unsigned kstride = (unsigned)p.Hqk * DK * 2, vstride = (unsigned)p.Hv * DV * 2;
    const unsigned astride = (unsigned)p.Hv * CH * 4, gstride = (unsigned)p.Hv * 4;
    stage_rows(s.k, p.k + (e.row0 * p.Hqk + iq) * DK, kstride, c, e.seq_len, DK * 2 / 16, tid);
    stage_rows(s.q, p.q + (e.row0 * p.Hqk + iq) * DK, kstride, c, e.seq_len, DK * 2 / 16, tid);
    stage_rows(s.dO, p.dO + (e.row0 * p.Hv + j) * DV + half * HVC, vstride, c, e.seq_len, HVC * 2 / 16, tid);
    stage_rows(s.t, p.A + (e.row0 * p.Hv + j) * CH, astride, c, e.seq_len, CH * 4 / 16, tid);
    if (tid < 64) {
        const __amdgpu_buffer_rsrc_t rg = chunk_rsrc(p.g + e.row0 * p.Hv + j, gstride, c, e.seq_len);
        const __amdgpu_buffer_rsrc_t rb = chunk_rsrc(p.beta + e.row0 * p.Hv + j, gstride, c, e.seq_len);
        const float g = ld4(rg, (unsigned)tid * gstride), b = ld4(rb, (unsigned)tid * gstride);
        const float G = prefix64(g, tid);
        const float Gl = __shfl(G, 63, 64);
        const float gam = __expf(G);
        s.G[tid] = G;
        s.gam[tid] = gam;
        s.bg[tid] = b * gam;
        s.rl[tid] = __expf(Gl - G);
    }
}

// One workgroup per (segment, v-head, value half).  Walks the segment's chunks
// last to first, carrying dh (K x 64 fp32) in LDS; first runs a warm-up over
// the chunks after the segment when the segment does not end its sequence
// (gate-driven window, as in the forward).  Stores, for each own chunk c, dh'
// (the gradient with respect to the state after c) and dv'.
__global__ void __launch_bounds__(NT, 1) gdn_bwd_dh_kernel(BwdParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    SmemDh &s = *reinterpret_cast<SmemDh *>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int seg = blockIdx.x / (2 * p.Hv);
    const int rem = blockIdx.x - seg * 2 * p.Hv;
    const int j = rem >> 1, half = rem & 1;
    if (seg >= p.num_segments) return;
    const Where e = find_segment(p.cu, p.N, p.T, p.L, seg, lane);
    if (e.n < 0) return;
    const int nt = seq_chunks(e.seq_len);
    const int c_end = e.c_begin + e.c_count;

    // where the reverse walk starts: the sequence end (from d final_state) or
    // a warm-up window after the segment (from zero)
    int c_last = c_end;
    if (!e.last && p.cp_mode == 2 /* WARMUP */) {
        float acc = 0.f;
        int w = 0;
        while (w < p.warmup_cap && c_last < nt) {
            const int tok = c_last * CH + lane;
            float gv = 0.f;
            if (tok < e.seq_len) gv = p.g[(e.row0 + tok) * p.Hv + j];
            gv = sum64(gv);
            acc += __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gv)));
            ++c_last;
            ++w;
            if (acc <= kLnNoiseFloor) break;
        }
    } else {
        c_last = nt;
    }
    const bool from_end = (c_last == nt);

    // dh at the start of the walk
    const int64_t sbase = ((int64_t)e.n * p.Hv + j) * DK * DV + half * HVC;
    for (int x = tid; x < DK * HVC / 4; x += NT) {
        const int d = x / (HVC / 4), v4 = x - d * (HVC / 4);
        f32x4 val = f32x4{};
        if (from_end && p.dht) val = *reinterpret_cast<const f32x4 *>(p.dht + sbase + (int64_t)d * DV + 4 * v4);
        *reinterpret_cast<f32x4 *>(&s.dh[d * HVC + 4 * v4]) = val;
    }
    const int cbase = seq_chunk_base(p.cu, p.T, e.n, lane);
    const int g16 = lane >> 4, c16 = lane & 15;

    for (int c = c_last - 1; c >= e.c_begin; --c) {
        const bool own = c < c_end;
        __syncthreads();  // previous chunk's dh update done; tiles free
        stage_chunk_dh(s, p, e, j, half, c, tid);
        __syncthreads();
        const float gl = s.gam[CH - 1];

        // W = T diag(beta gamma) K: wave w -> value... key columns 16 w .. +15, all rows
        for (int rt = 0; rt < 4; ++rt) {
            f32x4 acc = mm16<float, true, bf16, false, true>(f32x4{}, s.t + 16 * rt * CH, CH, 1, s.k + 16 * wave, 1, DK,
                                                            CH, lane, s.bg);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) s.w[(16 * rt + 4 * g16 + jj) * DK + 16 * wave + c16] = acc[jj];
        }
        // P = (Q K^T) o Gamma, s <= i: wave w -> row tile w / 2, column tiles 2 (w % 2) + {0, 1}
        for (int ct2 = 0; ct2 < 2; ++ct2) {
            const int rt = wave >> 1, ct = 2 * (wave & 1) + ct2;
            f32x4 acc = mm16<bf16, true, bf16, true>(f32x4{}, s.q + 16 * rt * DK, DK, 1, s.k + 16 * ct * DK, DK, 1, DK,
                                                    lane);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i = 16 * rt + 4 * g16 + jj, sc = 16 * ct + c16;
                s.p[i * CH + sc] = sc <= i ? acc[jj] * __expf(s.G[i] - s.G[sc]) : 0.f;
            }
        }
        // dh' of chunk c (unchanged so far in this step) -> HBM
        if (own) {
            float *dst = p.dh_ws + ((int64_t)(cbase + c) * p.Hv + j) * DK * DV + half * HVC;
            for (int x = tid; x < DK * HVC / 4; x += NT) {
                const int d = x / (HVC / 4), v4 = x - d * (HVC / 4);
                *reinterpret_cast<f32x4 *>(dst + (int64_t)d * DV + 4 * v4) =
                    *reinterpret_cast<const f32x4 *>(&s.dh[d * HVC + 4 * v4]);
            }
        }
        __syncthreads();

        // dv' = scale P^T dO + diag(rl) K dh: wave w -> row tile w / 2, column tiles 2 (w % 2) + {0, 1}
        for (int ct2 = 0; ct2 < 2; ++ct2) {
            const int rt = wave >> 1, ct = 2 * (wave & 1) + ct2;
            f32x4 a1 = mm16<float, false, bf16, false>(f32x4{}, s.p + 16 * rt, 1, CH, s.dO + 16 * ct, 1, HVC, CH, lane);
            f32x4 a2 = mm16<bf16, true, float, false>(f32x4{}, s.k + 16 * rt * DK, DK, 1, s.dh + 16 * ct, 1, HVC, DK,
                                                     lane);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i = 16 * rt + 4 * g16 + jj, v = 16 * ct + c16;
                const float x = p.scale * a1[jj] + s.rl[i] * a2[jj];
                s.dvp[i * HVC + v] = x;
                if (own) p.dvp_ws[(((int64_t)(cbase + c) * p.Hv + j) * CH + i) * DV + half * HVC + v] = x;
            }
        }
        __syncthreads();

        // dh <- gamma_last dh + scale (diag(gamma) Q)^T dO - W^T dv': wave w -> key rows 16 w .. +15
        for (int ct = 0; ct < 4; ++ct) {
            f32x4 a1 = mm16<bf16, false, bf16, false, true>(f32x4{}, s.q + 16 * wave, 1, DK, s.dO + 16 * ct, 1, HVC, CH,
                                                           lane, s.gam);
            f32x4 a2 = mm16<float, false, float, false>(f32x4{}, s.w + 16 * wave, 1, DK, s.dvp + 16 * ct, 1, HVC, CH,
                                                       lane);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int d = 16 * wave + 4 * g16 + jj, v = 16 * ct + c16;
                s.dh[d * HVC + v] = gl * s.dh[d * HVC + v] + p.scale * a1[jj] - a2[jj];
            }
        }
    }
    __syncthreads();
    if (e.c_begin == 0 && p.dh0) {
        for (int x = tid; x < DK * HVC / 4; x += NT) {
            const int d = x / (HVC / 4), v4 = x - d * (HVC / 4);
            *reinterpret_cast<f32x4 *>(p.dh0 + sbase + (int64_t)d * DV + 4 * v4) =
                *reinterpret_cast<const f32x4 *>(&s.dh[d * HVC + 4 * v4]);
        }
    }
}

// ---------------------------------------------------------------- chunk-local gradients
struct __attribute__((aligned(16))) SmemLoc {
    bf16 k[CH * DK], q[CH * DK], v[CH * DV], dO[CH * DV];
    float t[CH * CH];
    float m1[CH * CH], m2[CH * CH];
    float x[CH * DK];                    // W, then v', then dW
    float G[CH], gam[CH], bt[CH], bg[CH], rl[CH];
    float dGp[8][CH], dbp[8][CH];        // per-wave partial sums of dG and dbeta
};
static_assert(sizeof(SmemLoc) <= 160 * 1024, "local-gradient LDS over 160 KB");

// One workgroup per (chunk, v-head).  Wave w owns, for 64 x 128 results, key
// (or value) columns 16 w .. 16 w + 15 of all 64 rows; for 64 x 64 results the
// row tile w / 2 and column tiles 2 (w % 2), 2 (w % 2) + 1.
__global__ void __launch_bounds__(NT, 1) gdn_bwd_local_kernel(BwdParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    SmemLoc &s = *reinterpret_cast<SmemLoc *>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ent = blockIdx.x / p.Hv;
    const int j = blockIdx.x - ent * p.Hv;
    if (ent >= p.num_chunk_entries) return;
    const Where e = find_segment(p.cu, p.N, p.T, 1, ent, lane);
    if (e.n < 0 || e.c_count == 0) return;
    const int c = e.c_begin;
    const int cg = seq_chunk_base(p.cu, p.T, e.n, lane) + c;
    const int iq = j / p.group;
    const int g16 = lane >> 4, c16 = lane & 15;

    {
        const unsigned kstride = (unsigned)p.Hqk * DK * 2, vstride = (unsigned)p.Hv * DV * 2;
        const unsigned astride = (unsigned)p.Hv * CH * 4, gstride = (unsigned)p.Hv * 4;
        stage_rows(s.k, p.k + (e.row0 * p.Hqk + iq) * DK, kstride, c, e.seq_len, DK * 2 / 16, tid);
        stage_rows(s.q, p.q + (e.row0 * p.Hqk + iq) * DK, kstride, c, e.seq_len, DK * 2 / 16, tid);
        stage_rows(s.v, p.v + (e.row0 * p.Hv + j) * DV, vstride, c, e.seq_len, DV * 2 / 16, tid);
        stage_rows(s.dO, p.dO + (e.row0 * p.Hv + j) * DV, vstride, c, e.seq_len, DV * 2 / 16, tid);
        stage_rows(s.t, p.A + (e.row0 * p.Hv + j) * CH, astride, c, e.seq_len, CH * 4 / 16, tid);
        if (tid < 64) {
            const __amdgpu_buffer_rsrc_t rg = chunk_rsrc(p.g + e.row0 * p.Hv + j, gstride, c, e.seq_len);
            const __amdgpu_buffer_rsrc_t rb = chunk_rsrc(p.beta + e.row0 * p.Hv + j, gstride, c, e.seq_len);
            const float g = ld4(rg, (unsigned)tid * gstride), b = ld4(rb, (unsigned)tid * gstride);
            const float G = prefix64(g, tid);
            const float Gl = __shfl(G, 63, 64);
            const float gam = __expf(G);
            s.G[tid] = G;
            s.gam[tid] = gam;
            s.bt[tid] = b;
            s.bg[tid] = b * gam;
            s.rl[tid] = __expf(Gl - G);
        }
        for (int x = tid; x < 8 * CH; x += NT) {
            (&s.dGp[0][0])[x] = 0.f;
            (&s.dbp[0][0])[x] = 0.f;
        }
    }
    __syncthreads();

    const float *hc = p.h + ((int64_t)cg * p.Hv + j) * DK * DV;       // chunk-start state
    const float *dhc = p.dh_ws + ((int64_t)cg * p.Hv + j) * DK * DV;  // gradient wrt the state after the chunk
    const float *dvc = p.dvp_ws + ((int64_t)cg * p.Hv + j) * CH * DV; // dv'
    float *dGw = s.dGp[wave];
    float *dbw = s.dbp[wave];
    const int rt64 = wave >> 1;  // 64 x 64 results: row tile
    const float gl = s.gam[CH - 1];

    // S1: W = T diag(beta gamma) K -> x;  Q K^T -> m1
    for (int rt = 0; rt < 4; ++rt) {
        f32x4 acc = mm16<float, true, bf16, false, true>(f32x4{}, s.t + 16 * rt * CH, CH, 1, s.k + 16 * wave, 1, DK, CH,
                                                        lane, s.bg);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s.x[(16 * rt + 4 * g16 + jj) * DK + 16 * wave + c16] = acc[jj];
    }
    for (int ct2 = 0; ct2 < 2; ++ct2) {
        const int ct = 2 * (wave & 1) + ct2;
        f32x4 acc = mm16<bf16, true, bf16, true>(f32x4{}, s.q + 16 * rt64 * DK, DK, 1, s.k + 16 * ct * DK, DK, 1, DK,
                                                lane);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s.m1[(16 * rt64 + 4 * g16 + jj) * CH + 16 * ct + c16] = acc[jj];
    }
    __syncthreads();

    // S2: v' = T diag(beta) V - W h (value columns 16 w ..), held, then -> x
    f32x4 vpt[4];
    for (int rt = 0; rt < 4; ++rt) {
        f32x4 a1 = mm16<float, true, bf16, false, true>(f32x4{}, s.t + 16 * rt * CH, CH, 1, s.v + 16 * wave, 1, DV, CH,
                                                       lane, s.bt);
        f32x4 a2 = mm16<float, true, float, false>(f32x4{}, s.x + 16 * rt * DK, DK, 1, hc + 16 * wave, 1, DV, DK, lane);
        vpt[rt] = a1 - a2;
    }
    __syncthreads();
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s.x[(16 * rt + 4 * g16 + jj) * DV + 16 * wave + c16] = vpt[rt][jj];
    __syncthreads();

    // S3: dPm = scale (dO v'^T) o Gamma (s <= i) -> m2; gate terms of P
    for (int ct2 = 0; ct2 < 2; ++ct2) {
        const int ct = 2 * (wave & 1) + ct2;
        f32x4 acc = mm16<bf16, true, float, true>(f32x4{}, s.dO + 16 * rt64 * DV, DV, 1, s.x + 16 * ct * DV, DV, 1, DV,
                                                 lane);
        float colsum = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = 16 * rt64 + 4 * g16 + jj, sc = 16 * ct + c16;
            const float dpm = sc <= i ? p.scale * acc[jj] * __expf(s.G[i] - s.G[sc]) : 0.f;
            s.m2[i * CH + sc] = dpm;
            const float d1 = dpm * s.m1[i * CH + sc];
            const float rs = sum16(d1);
            if (c16 == 0) dGw[i] += rs;
            colsum += d1;
        }
        colsum = sum4g(colsum);
        if (g16 == 0) dGw[16 * ct + c16] -= colsum;
    }
    __syncthreads();

    // S4: dQ, dK terms of P, h and h'; gate terms of O (inter) and h'
    f32x4 dq[4], dk[4];
    float lastacc = 0.f;
    for (int rt = 0; rt < 4; ++rt) {
        dq[rt] = mm16<float, true, bf16, false>(f32x4{}, s.m2 + 16 * rt * CH, CH, 1, s.k + 16 * wave, 1, DK, CH, lane);
        const f32x4 t1 = mm16<bf16, true, float, true>(f32x4{}, s.dO + 16 * rt * DV, DV, 1, hc + 16 * wave * DV, DV, 1,
                                                      DV, lane);
        dk[rt] = mm16<float, false, bf16, false>(f32x4{}, s.m2 + 16 * rt, 1, CH, s.q + 16 * wave, 1, DK, CH, lane);
        const f32x4 t2 = mm16<float, true, float, true>(f32x4{}, s.x + 16 * rt * DV, DV, 1, dhc + 16 * wave * DV, DV, 1,
                                                       DV, lane);
        const f32x4 t3 = mm16<bf16, true, float, false>(f32x4{}, s.k + 16 * rt * DK, DK, 1, dhc + 16 * wave, 1, DV, DK,
                                                       lane);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = 16 * rt + 4 * g16 + jj, col = 16 * wave + c16;
            const float sg = p.scale * s.gam[i];
            dq[rt][jj] += sg * t1[jj];
            const float qd = (float)s.q[i * DK + col] * t1[jj];
            const float rq = sum16(qd);
            if (c16 == 0) dGw[i] += sg * rq;
            dk[rt][jj] += s.rl[i] * t2[jj];
            // t3 is (K dh') over value columns 16 w ..: x_i = rl_i v'_i . (K dh')_i
            const float xv = s.x[i * DV + col] * s.rl[i] * t3[jj];
            const float rx = sum16(xv);
            if (c16 == 0) dGw[i] -= rx;
            lastacc += (c16 == 0) ? rx : 0.f;
        }
    }
    {
        // gamma_last <dh', h>: this wave's share of the 128 x 128 products
        float dot = 0.f;
        for (int x = lane; x < DK * DV / 8; x += 64) {
            const int idx = wave * (DK * DV / 8) + x;
            dot += dhc[idx] * hc[idx];
        }
        dot = sum64(dot);
        lastacc = sum64(lastacc);
        if (lane == 0) dGw[CH - 1] += lastacc + gl * dot;
    }
    __syncthreads();

    // S5: dW = -dv' h^T -> x
    for (int rt = 0; rt < 4; ++rt) {
        f32x4 acc = mm16<float, true, float, true>(f32x4{}, dvc + 16 * rt * DV, DV, 1, hc + 16 * wave * DV, DV, 1, DV,
                                                  lane);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s.x[(16 * rt + 4 * g16 + jj) * DK + 16 * wave + c16] = -acc[jj];
    }
    __syncthreads();

    // S6: dT -> m1;  dK and dbeta / dG terms of W;  dV and the dbeta term of U
    for (int ct2 = 0; ct2 < 2; ++ct2) {
        const int ct = 2 * (wave & 1) + ct2;
        f32x4 a1 = mm16<float, true, bf16, true>(f32x4{}, s.x + 16 * rt64 * DK, DK, 1, s.k + 16 * ct * DK, DK, 1, DK,
                                                lane);
        f32x4 a2 = mm16<float, true, bf16, true>(f32x4{}, dvc + 16 * rt64 * DV, DV, 1, s.v + 16 * ct * DV, DV, 1, DV,
                                                lane);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = 16 * rt64 + 4 * g16 + jj, sc = 16 * ct + c16;
            s.m1[i * CH + sc] = s.bg[sc] * a1[jj] + s.bt[sc] * a2[jj];
        }
    }
    const int rows_valid = min(CH, e.seq_len - c * CH);
    for (int rt = 0; rt < 4; ++rt) {
        const f32x4 kb = mm16<float, false, float, false>(f32x4{}, s.t + 16 * rt, 1, CH, s.x + 16 * wave, 1, DK, CH,
                                                         lane);
        const f32x4 vb = mm16<float, false, float, false>(f32x4{}, s.t + 16 * rt, 1, CH, dvc + 16 * wave, 1, DV, CH,
                                                         lane);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = 16 * rt + 4 * g16 + jj, col = 16 * wave + c16;
            dk[rt][jj] += s.bg[i] * kb[jj];
            const float rk = sum16(kb[jj] * (float)s.k[i * DK + col]);
            const float rv = sum16(vb[jj] * (float)s.v[i * DV + col]);
            if (c16 == 0) {
                dbw[i] += s.gam[i] * rk + rv;
                dGw[i] += s.bg[i] * rk;
            }
            const float dvv = s.bt[i] * vb[jj];
            if (i < rows_valid) {
                const int64_t off = ((e.row0 + (int64_t)c * CH + i) * p.Hv + j) * DV + col;
                if (p.grad_f32) static_cast<float *>(p.dv)[off] = dvv;
                else static_cast<bf16 *>(p.dv)[off] = (bf16)dvv;
            }
        }
    }
    __syncthreads();

    // S7: Y = T^T dT -> m2
    for (int ct2 = 0; ct2 < 2; ++ct2) {
        const int ct = 2 * (wave & 1) + ct2;
        f32x4 acc = mm16<float, false, float, false>(f32x4{}, s.t + 16 * rt64, 1, CH, s.m1 + 16 * ct, 1, CH, CH, lane);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) s.m2[(16 * rt64 + 4 * g16 + jj) * CH + 16 * ct + c16] = acc[jj];
    }
    __syncthreads();

    // S8: dA~ = -(Y T^T) strictly lower; M = dA~ o beta_i Gamma_is -> m1; gate / beta terms of A~
    for (int ct2 = 0; ct2 < 2; ++ct2) {
        const int ct = 2 * (wave & 1) + ct2;
        f32x4 ya = mm16<float, true, float, true>(f32x4{}, s.m2 + 16 * rt64 * CH, CH, 1, s.t + 16 * ct * CH, CH, 1, CH,
                                                 lane);
        f32x4 kk = mm16<bf16, true, bf16, true>(f32x4{}, s.k + 16 * rt64 * DK, DK, 1, s.k + 16 * ct * DK, DK, 1, DK,
                                               lane);
        float colsum = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = 16 * rt64 + 4 * g16 + jj, sc = 16 * ct + c16;
            float m = 0.f, d2 = 0.f, db = 0.f;
            if (sc < i) {
                const float da = -ya[jj];
                const float gm = __expf(s.G[i] - s.G[sc]);
                m = da * s.bt[i] * gm;
                d2 = m * kk[jj];
                db = da * gm * kk[jj];
            }
            s.m1[i * CH + sc] = m;
            const float rs = sum16(d2), rb = sum16(db);
            if (c16 == 0) {
                dGw[i] += rs;
                dbw[i] += rb;
            }
            colsum += d2;
        }
        colsum = sum4g(colsum);
        if (g16 == 0) dGw[16 * ct + c16] -= colsum;
    }
    __syncthreads();

    // S9: dK += M K + M^T K; store dq, dk of this v-head
    for (int rt = 0; rt < 4; ++rt) {
        dk[rt] = mm16<float, true, bf16, false>(dk[rt], s.m1 + 16 * rt * CH, CH, 1, s.k + 16 * wave, 1, DK, CH, lane);
        dk[rt] = mm16<float, false, bf16, false>(dk[rt], s.m1 + 16 * rt, 1, CH, s.k + 16 * wave, 1, DK, CH, lane);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = 16 * rt + 4 * g16 + jj, col = 16 * wave + c16;
            if (i < rows_valid) {
                const int64_t off = ((e.row0 + (int64_t)c * CH + i) * p.Hv + j) * DK + col;
                p.dq_ws[off] = dq[rt][jj];
                p.dk_ws[off] = dk[rt][jj];
            }
        }
    }
    __syncthreads();

    // dg = reverse in-chunk cumsum of dG; dbeta
    if (wave == 0) {
        float dG = 0.f, db = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            dG += s.dGp[w][lane];
            db += s.dbp[w][lane];
        }
        // suffix sum: sum over i >= lane
        float x = dG;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_down(x, off, 64);
            if (lane + off < 64) x += y;
        }
        if (lane < rows_valid) {
            const int64_t off = (e.row0 + (int64_t)c * CH + lane) * p.Hv + j;
            p.dg[off] = x;
            p.dbeta[off] = db;
        }
    }
}

// ---------------------------------------------------------------- key-head sums
// dq, dk of key head i = sum over its v-heads i G .. i G + G - 1 of the per-v-head
// partials; four elements per thread.
__global__ void __launch_bounds__(256) gdn_bwd_group_sum_kernel(BwdParams p) {
    const int64_t n4 = p.rows * p.Hqk * DK / 4;
    for (int64_t x = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; x < n4; x += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e0 = 4 * x;
        const int64_t row = e0 / ((int64_t)p.Hqk * DK);
        const int rem = (int)(e0 - row * p.Hqk * DK);
        const int iq = rem / DK, d = rem - iq * DK;
        f32x4 sq = f32x4{}, sk = f32x4{};
        for (int jj = 0; jj < p.group; ++jj) {
            const int64_t src = (row * p.Hv + iq * p.group + jj) * DK + d;
            sq += *reinterpret_cast<const f32x4 *>(p.dq_ws + src);
            sk += *reinterpret_cast<const f32x4 *>(p.dk_ws + src);
        }
        if (p.grad_f32) {
            *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dq) + e0) = sq;
            *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dk) + e0) = sk;
        } else {
            bf16 *oq = static_cast<bf16 *>(p.dq) + e0, *ok = static_cast<bf16 *>(p.dk) + e0;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                oq[t] = (bf16)sq[t];
                ok[t] = (bf16)sk[t];
            }
        }
    }
}

}  // namespace bwdk

int launch_bwd(const BwdParams &p, void *stream) {
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t err;
    err = hipFuncSetAttribute(reinterpret_cast<const void *>(bwdk::gdn_bwd_dh_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(bwdk::SmemDh));
    if (err != hipSuccess) return (int)err;
    err = hipFuncSetAttribute(reinterpret_cast<const void *>(bwdk::gdn_bwd_local_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(bwdk::SmemLoc));
    if (err != hipSuccess) return (int)err;
    if (p.num_segments > 0) {
        hipLaunchKernelGGL(bwdk::gdn_bwd_dh_kernel, dim3((unsigned)(p.num_segments * p.Hv * 2)), dim3(bwdk::NT),
                           sizeof(bwdk::SmemDh), st, p);
        err = hipGetLastError();
        if (err != hipSuccess) return (int)err;
    }
    if (p.num_chunk_entries > 0 && p.rows > 0) {
        hipLaunchKernelGGL(bwdk::gdn_bwd_local_kernel, dim3((unsigned)(p.num_chunk_entries * p.Hv)), dim3(bwdk::NT),
                           sizeof(bwdk::SmemLoc), st, p);
        err = hipGetLastError();
        if (err != hipSuccess) return (int)err;
        const int64_t n4 = p.rows * p.Hqk * kDimK / 4;
        const unsigned blocks = (unsigned)std::min<int64_t>((n4 + 255) / 256, 16384);
        hipLaunchKernelGGL(bwdk::gdn_bwd_group_sum_kernel, dim3(blocks), dim3(256), 0, st, p);
        err = hipGetLastError();
        if (err != hipSuccess) return (int)err;
    }
    return 0;
}

}  // namespace gdn
