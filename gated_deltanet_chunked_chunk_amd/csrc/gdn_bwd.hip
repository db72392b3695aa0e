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
// v-head, half of V): the V columns of dh are independent) and
// gdn_bwd_local_kernel (persistent workgroups, one per compute unit, taking
// (chunk, key head) items in turn and running each key head's v-heads one
// after another, so that dq and dk of the key head, the sums over its v-heads,
// add up in the workgroup).  h and T come from the forward (its
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
#include "gdn_window.h"

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

typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// k slot e of lane group g inside a 32-wide k step.  A step that reads any
// operand transposed uses the k order {4g..4g+3, 16+4g..16+4g+3} (what two
// transposed 16-row reads deliver) for both operands; otherwise 8g..8g+7.
__device__ __forceinline__ constexpr int kpos(int e, int g, bool perm) {
    return perm ? ((e & 3) + 4 * g + 16 * (e >> 2)) : (8 * g + e);
}

__device__ __forceinline__ bf16x4 tr4(const bf16 *p) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// hi + lo bf16 split of fp32 values, two at a time: hi = RNE(x) by a packed
// conversion, float(hi) by shifting / masking the packed word, lo = RNE(x - hi).
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &hi, bf16x8 &lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const bf16x2 hh = {(bf16)x[2 * i], (bf16)x[2 * i + 1]};
        h[i] = __builtin_bit_cast(uint32_t, hh);
        asm("" : "+v"(h[i]));
        const float h0 = __uint_as_float(h[i] << 16), h1 = __uint_as_float(h[i] & 0xffff0000u);
        const bf16x2 ll = {(bf16)(x[2 * i] - h0), (bf16)(x[2 * i + 1] - h1)};
        l[i] = __builtin_bit_cast(uint32_t, ll);
    }
    hi = __builtin_bit_cast(bf16x8, (u32x4{h[0], h[1], h[2], h[3]}));
    lo = __builtin_bit_cast(bf16x8, (u32x4{l[0], l[1], l[2], l[3]}));
}

// Cross-lane sums without the LDS crossbar.  A DPP row is 16 lanes: two quad
// permutations, then the half-row and row mirrors leave the row's sum in every
// lane of the row.  Across rows, v_permlane16_swap exchanges the odd rows of
// one operand with the even rows of the other (rows 0+1 and 2+3 after an
// add), v_permlane32_swap the upper half with the lower.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
// sum over the 16 lanes that share l / 16 (one accumulator row group)
__device__ __forceinline__ float sum16(float x) {
    x += dpp_row<0xb1>(x);   // quad_perm [1,0,3,2]
    x += dpp_row<0x4e>(x);   // quad_perm [2,3,0,1]
    x += dpp_row<0x141>(x);  // row_half_mirror
    x += dpp_row<0x140>(x);  // row_mirror
    return x;
}
// sum over the four lane groups l / 16 (lanes l % 16 equal)
__device__ __forceinline__ float sum4g(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(a[0]) + __int_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(b[0]) + __int_as_float(b[1]);
}
__device__ __forceinline__ float sum64(float x) { return sum4g(sum16(x)); }

// Workgroup barrier for LDS hand-offs only: the wave's own LDS operations
// complete first, its global loads and stores stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------- rows of a chunk
// Buffer resource over chunk c's rows of one sequence: rows past the sequence
// end read as zeros and stores to them are dropped (hardware range check), so
// a partial last chunk behaves as if padded with zero inputs.  Every caller
// passes values that are the same in all lanes of the wave; taking them
// through readfirstlane keeps the resource in scalar registers (otherwise
// the compiler cannot prove them uniform and wraps every load in a loop over
// the lanes' distinct resources).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void *base, unsigned stride, int c, int seq_len) {
    const int rows = min(max(seq_len - c * CH, 0), CH);
    const uint64_t a = reinterpret_cast<uint64_t>(static_cast<const char *>(base) + (int64_t)c * CH * stride);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)(rows * stride));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0, n,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float ld4(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// ---- direct HBM -> LDS loads (buffer_load ... lds: lane l of a wave writes
// LDS bytes 16 l .. 16 l + 15 past the wave-uniform base).
typedef __attribute__((address_space(3))) void lds_void;

// The LDS address of a generic pointer into this workgroup's LDS (its low 32
// bits), taken through integers rather than an address-space cast.
__device__ __forceinline__ lds_void *lds_ptr(const void *p) {
    return (lds_void *)(uintptr_t)(uint32_t)(uintptr_t)p;
}

// This wave's direct loads have landed in LDS (vmcnt(0); other counters untouched).
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// 64 rows x PPR 16-byte pieces of HBM rows, held in registers between their
// loads and their LDS stores (a dense tile), so that every load of a chunk is
// in flight before the first store.
template <int PPR>
struct Rows {
    static constexpr int PER = (CH * PPR + NT - 1) / NT;
    u32x4 x[PER];
};

template <int PPR>
__device__ __forceinline__ void load_rows(Rows<PPR> &R, const void *base, unsigned stride, int c, int seq_len,
                                          int tid) {
    const __amdgpu_buffer_rsrc_t r = chunk_rsrc(base, stride, c, seq_len);
#pragma unroll
    for (int i = 0; i < Rows<PPR>::PER; ++i) {
        const int pc = tid + i * NT;
        const int row = pc / PPR, col = pc - row * PPR;
        R.x[i] = (pc < CH * PPR) ? ld16(r, (unsigned)row * stride + (unsigned)col * 16u) : u32x4{};
    }
}

template <int PPR>
__device__ __forceinline__ void store_rows(void *dst, const Rows<PPR> &R, int tid) {
    u32x4 *d = static_cast<u32x4 *>(dst);
#pragma unroll
    for (int i = 0; i < Rows<PPR>::PER; ++i) {
        const int pc = tid + i * NT;
        if (pc < CH * PPR) d[pc] = R.x[i];
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
// Inclusive prefix sum over the 64 lanes with DPP: row shifts inside each
// 16-lane row, then the row broadcasts of lanes 15 and 31 into the rows after.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_scan(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float prefix64(float x) {
    x += dpp_scan<0x111, 0xf>(x);  // row_shr:1
    x += dpp_scan<0x112, 0xf>(x);  // row_shr:2
    x += dpp_scan<0x114, 0xf>(x);  // row_shr:4
    x += dpp_scan<0x118, 0xf>(x);  // row_shr:8
    x += dpp_scan<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_scan<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// Lane l takes lane 63 - l's value: the halves swap (v_permlane32_swap), then
// the rows of each half (v_permlane16_swap), then the lanes of each row
// (row_mirror).
__device__ __forceinline__ float reverse64(float x) {
    const int lane = threadIdx.x & 63;
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(lane < 32 ? a[1] : a[0]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(x), false, false);
    x = __int_as_float(((lane >> 4) & 1) ? b[0] : b[1]);
    return dpp_row<0x140>(x);  // row_mirror
}

// ---------------------------------------------------------------- chunk-local gradients
// Fragment readers.  A fragment is the 8 k-values lane l holds for row /
// column r = l % 16 in a 32-wide k step: k = 8 g .. 8 g + 7 (g = l / 16), or
// the permuted order {4g..4g+3, 16+4g..16+4g+3} when the step reads any
// operand transposed (PERM).
//   fr_row:  bf16, element (r, k) at p[r ld + k]           (16- or 8-byte reads)
//   fr_tr:   bf16 LDS, element (r, k) at p[k ld + r]      (ds_read_b64_tr_b16, PERM order)
//   fr_rowf: fp32, element (r, k) at p[r ld + k], split hi + lo
//   fr_colf: fp32, element (r, k) at p[k ks + r], split hi + lo
template <bool PERM>
__device__ __forceinline__ bf16x8 fr_row(const bf16 *p, int ld, int k0, int lane) {
    const int r = lane & 15, g = lane >> 4;
    const bf16 *q = p + r * ld + k0;
    if constexpr (!PERM) {
        return *reinterpret_cast<const bf16x8 *>(q + 8 * g);
    } else {
        const bf16x4 x0 = *reinterpret_cast<const bf16x4 *>(q + 4 * g);
        const bf16x4 x1 = *reinterpret_cast<const bf16x4 *>(q + 16 + 4 * g);
        return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    }
}

__device__ __forceinline__ bf16x8 fr_tr(const bf16 *p, int ld, int k0, int lane) {
    const bf16 *q = p + (k0 + (lane >> 2)) * ld + 4 * (lane & 3);
    const bf16x4 x0 = tr4(q), x1 = tr4(q + 16 * ld);
    return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

template <bool PERM>
__device__ __forceinline__ void fr_rowf(const float *p, int ld, int k0, int lane, bf16x8 &hi, bf16x8 &lo,
                                        float (&raw)[8]) {
    const int r = lane & 15, g = lane >> 4;
    const float *q = p + r * ld + k0;
    const f32x4 x0 = *reinterpret_cast<const f32x4 *>(q + (PERM ? 4 * g : 8 * g));
    const f32x4 x1 = *reinterpret_cast<const f32x4 *>(q + (PERM ? 16 + 4 * g : 8 * g + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        raw[e] = x0[e];
        raw[4 + e] = x1[e];
    }
    split8(raw, hi, lo);
}

template <bool PERM>
__device__ __forceinline__ void fr_colf(const float *p, int ks, int k0, int lane, bf16x8 &hi, bf16x8 &lo) {
    const int r = lane & 15, g = lane >> 4;
    float raw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) raw[e] = p[(k0 + kpos(e, g, PERM)) * ks + r];
    split8(raw, hi, lo);
}

// products of hi / lo pairs: exact x pair, pair x exact, pair x pair
__device__ __forceinline__ f32x4 mm_ep(f32x4 c, bf16x8 a, bf16x8 bh, bf16x8 bl) {
    return mfma(a, bl, mfma(a, bh, c));
}
__device__ __forceinline__ f32x4 mm_pe(f32x4 c, bf16x8 ah, bf16x8 al, bf16x8 b) {
    return mfma(al, b, mfma(ah, b, c));
}
__device__ __forceinline__ f32x4 mm_pp(f32x4 c, bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl) {
    return mfma(ah, bl, mfma(al, bh, mfma(ah, bh, c)));
}

// hi / lo bf16 of an accumulator tile (rows 4 (l / 16) + j, column l % 16) into
// row-major [row][col] arrays (st_split) or, transposed, into [col][row]
// arrays where the lane's four rows are contiguous (st_split_t).
__device__ __forceinline__ void split4(f32x4 v, bf16x4 &h, bf16x4 &l) {
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const bf16x2 hh = {(bf16)v[2 * i], (bf16)v[2 * i + 1]};
        hw[i] = __builtin_bit_cast(uint32_t, hh);
        asm("" : "+v"(hw[i]));
        const float h0 = __uint_as_float(hw[i] << 16), h1 = __uint_as_float(hw[i] & 0xffff0000u);
        const bf16x2 ll = {(bf16)(v[2 * i] - h0), (bf16)(v[2 * i + 1] - h1)};
        lw[i] = __builtin_bit_cast(uint32_t, ll);
    }
    h = __builtin_bit_cast(bf16x4, (u32x2{hw[0], hw[1]}));
    l = __builtin_bit_cast(bf16x4, (u32x2{lw[0], lw[1]}));
}
__device__ __forceinline__ void st_split(bf16 *hi, bf16 *lo, int ld, int r0, int c0, f32x4 v, int lane) {
    bf16x4 h, l;
    split4(v, h, l);
    const int c = c0 + (lane & 15), r = r0 + 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        hi[(r + j) * ld + c] = h[j];
        lo[(r + j) * ld + c] = l[j];
    }
}
__device__ __forceinline__ void st_split_t(bf16 *hi, bf16 *lo, int ld, int r0, int c0, f32x4 v, int lane) {
    bf16x4 h, l;
    split4(v, h, l);
    const int c = c0 + (lane & 15), r = r0 + 4 * (lane >> 4);
    *reinterpret_cast<bf16x4 *>(&hi[c * ld + r]) = h;
    *reinterpret_cast<bf16x4 *>(&lo[c * ld + r]) = l;
}

// The diagonal 16 x 16 tile (rows and columns from r0) of S = M + M^T for a
// strictly lower M given as an accumulator tile v: each element below the
// diagonal goes to its place and, mirrored, above it; the diagonal is zero.
__device__ __forceinline__ void st_sym_diag(bf16 *hi, bf16 *lo, int ld, int r0, f32x4 v, int lane) {
    bf16x4 h, l;
    split4(v, h, l);
    const int c = lane & 15, r = 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (c < r + j) {
            hi[(r0 + r + j) * ld + r0 + c] = h[j];
            lo[(r0 + r + j) * ld + r0 + c] = l[j];
            hi[(r0 + c) * ld + r0 + r + j] = h[j];
            lo[(r0 + c) * ld + r0 + r + j] = l[j];
        } else if (c == r + j) {
            hi[(r0 + c) * ld + r0 + c] = bf16(0.f);
            lo[(r0 + c) * ld + r0 + c] = bf16(0.f);
        }
    }
}

// LDS row strides (bf16 elements) of 128- and 64-wide tiles: 272 and 144
// bytes, so that the 16 rows one fragment read touches fall in distinct banks.
constexpr int LK = DK + 8;
constexpr int L64 = CH + 8;

// 64 rows of 256 bytes (bf16 x 128) through resource r (row stride `stride`
// bytes) into an LDS tile with rows of LK elements (272 bytes = 17 pieces of
// 16): 17 wave loads of 1 KB, spread over the 8 waves.  Lane l of load i
// fills piece 64 i + l of the tile, i.e. row (64 i + l) / 17 and piece
// (64 i + l) % 17; the pad piece reads past the resource and arrives as zeros,
// as do rows the resource does not cover.
constexpr int TSLOT = LK * 2 / 16;
constexpr int TLOADS = CH * TSLOT / 64;
static_assert(CH * TSLOT % 64 == 0, "a padded tile is a whole number of wave loads");
__device__ __forceinline__ void dma_tile(bf16 *tile, const __amdgpu_buffer_rsrc_t r, const unsigned stride,
                                         const int wave, const int lane) {
#pragma unroll
    for (int n = 0; n < (TLOADS + 7) / 8; ++n) {
        const int i = wave + 8 * n;
        if (i < TLOADS) {
            const int slot = 64 * i + lane;
            const int row = slot / TSLOT, piece = slot - TSLOT * row;
            const unsigned off = piece < 16 ? (unsigned)row * stride + 16u * (unsigned)piece : 0x80000000u;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(tile + 512 * i), 16, (int)off, 0, 0, 0);
        }
    }
}

struct __attribute__((aligned(16))) SmemLoc {
    bf16 k[CH * LK], q[CH * LK];
    bf16 ov[CH * LK];                 // dO, then V
    bf16 tH[CH * L64], tL[CH * L64];  // T
    bf16 nH[CH * LK], nL[CH * LK];    // v' [token][v], then dW [token][key dim], then Y [64][64] (stride L64)
    bf16 eH[CH * LK], eL[CH * LK];    // dv' [token][v]
    bf16 pH[CH * L64], pL[CH * L64];  // dPm, then dT, then S = M + M^T   [row][col]
    float G[CH], gam[CH], bt[CH];
    float dGp[8][CH], dbp[8][CH];     // per-wave partial sums of dG and dbeta
};
static_assert(sizeof(SmemLoc) <= 160 * 1024, "local-gradient LDS over 160 KB");

// bf16 16-byte pieces (eight values) of 64 rows into a tile of row stride ld
template <int PPR>
__device__ __forceinline__ void store_rows_ld(bf16 *dst, const Rows<PPR> &R, int ld, int tid) {
#pragma unroll
    for (int i = 0; i < Rows<PPR>::PER; ++i) {
        const int pc = tid + i * NT;
        const int row = pc / PPR, col = pc - row * PPR;
        if (pc < CH * PPR) *reinterpret_cast<u32x4 *>(&dst[row * ld + 8 * col]) = R.x[i];
    }
}

// fp32 16-byte pieces (four values) of 64 rows -> hi / lo bf16 tiles of row stride ld
template <int PPR>
__device__ __forceinline__ void store_rows_split(bf16 *hi, bf16 *lo, const Rows<PPR> &R, int ld, int tid) {
#pragma unroll
    for (int i = 0; i < Rows<PPR>::PER; ++i) {
        const int pc = tid + i * NT;
        const int row = pc / PPR, col = pc - row * PPR;
        if (pc < CH * PPR) {
            bf16x4 h, l;
            split4(__builtin_bit_cast(f32x4, R.x[i]), h, l);
            *reinterpret_cast<bf16x4 *>(&hi[row * ld + 4 * col]) = h;
            *reinterpret_cast<bf16x4 *>(&lo[row * ld + 4 * col]) = l;
        }
    }
}

// 64 x 128 fp32 rows (a dense per-chunk workspace tile) as 16-byte pieces
__device__ __forceinline__ void load_tile_f32(Rows<DV * 4 / 16> &R, const float *src, int tid) {
#pragma unroll
    for (int i = 0; i < Rows<DV * 4 / 16>::PER; ++i)
        R.x[i] = *reinterpret_cast<const u32x4 *>(src + 4 * (tid + i * NT));
}

// dq or dk of a key head = the sum over its v-heads: the workgroup runs them
// one after another and every lane adds its four values to what it stored for
// the previous v-head (fp32 workspace, the same lane and address: group_prev
// reads that sum ahead of the products it is added to); the last v-head writes
// the output in its dtype.
__device__ __forceinline__ f32x4 group_prev(const float *ws, int64_t idx, bool first, bool valid) {
    return (!first && valid) ? *reinterpret_cast<const f32x4 *>(ws + idx) : f32x4{};
}
__device__ __forceinline__ void group_put(const BwdParams &p, float *ws, void *out, int64_t idx, f32x4 v, bool last) {
    if (!last) {
        *reinterpret_cast<f32x4 *>(ws + idx) = v;
    } else if (p.grad_f32) {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(out) + idx) = v;
    } else {
        *reinterpret_cast<bf16x4 *>(static_cast<bf16 *>(out) + idx) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    }
}

// A work item of the chunk-local kernel: one (chunk, key head) pair.
struct LocItem {
    Where e;
    int c, cg, iq;   // chunk within its sequence, among all chunks, key head
    int64_t rowq_c;  // the chunk's first row of the key-head sums
    bool ok;         // false: an empty sequence's entry, or past the last item
};

__device__ __forceinline__ LocItem loc_item(const BwdParams &p, const int it, const int lane) {
    LocItem r;
    r.ok = false;
    const int ent = it / p.Hqk;
    r.iq = it - ent * p.Hqk;
    if (ent >= p.num_chunk_entries) return r;
    r.e = find_segment(p.cu, p.N, p.T, 1, ent, lane);
    if (r.e.n < 0 || r.e.c_count == 0) return r;
    r.c = r.e.c_begin;
    r.cg = seq_chunk_base(p.cu, p.T, r.e.n, lane) + r.c;
    r.rowq_c = (r.e.row0 + (int64_t)r.c * CH) * p.Hqk + r.iq;
    r.ok = true;
    return r;
}

// The first item at or after `it` in this workgroup's share (it, it + gridDim.x, ...)
// that has rows; `it` is left at that item.
__device__ __forceinline__ LocItem next_item(const BwdParams &p, int &it, const int lane) {
    const int n_items = p.num_chunk_entries * p.Hqk;
    for (; it < n_items; it += (int)gridDim.x) {
        const LocItem r = loc_item(p, it, lane);
        if (r.ok) return r;
    }
    LocItem r;
    r.ok = false;
    return r;
}

// Persistent workgroups (one per compute unit) take the (chunk, key head)
// items b, b + gridDim.x, ... and run each key head's v-heads in turn; the
// next item's K, Q and first-v-head loads go out during the current item's
// last v-head.  The key-dim results dq, dk and dW are
// computed transposed ((key dim, token) tiles): every product with h or dh'
// then contracts over the value dim, and wave w owns key dims 16 w .. +15, so
// it reads (and splits) its 16 rows of h and dh' once.  64 x 64 results: wave
// w has row tile w / 2 and column tiles 2 (w % 2), 2 (w % 2) + 1.  A v-head's
// HBM reads: V, T, v', g and beta at its start, through registers (T and v'
// split into hi / lo pairs on the way to LDS); dO and the dv' planes straight
// into LDS, and the wave's h rows into registers, during the previous v-head
// (at the start for the first); the dh' rows after the tiles, in flight during
// the first products; dk's running sum one phase before its products, ahead
// of the next v-head's direct loads.  Wave 0 reduces a v-head's dg and dbeta
// partial sums at the next v-head's start, while the loads are in flight (no
// phase of their own).  fp32 intermediates are stored once as hi / lo bf16
// pairs that every consumer reads without further arithmetic.  The barriers
// hand over LDS only: no data passes between waves through global memory, so
// loads issued for later phases stay in flight across them.
__global__ void __launch_bounds__(NT, 1) gdn_bwd_local_kernel(BwdParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    SmemLoc &s = *reinterpret_cast<SmemLoc *>(smem_raw);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane0 = threadIdx.x & 63;
    // persistent: workgroup b takes items b, b + gridDim.x, ... in turn, and the
    // next item's first loads go out during the current item's last v-head
    int it = blockIdx.x;
    LocItem cur = next_item(p, it, lane0);
    if (!cur.ok) return;
    const unsigned vstride = (unsigned)p.Hv * DV * 2;
    const unsigned tstride = (unsigned)p.Hv * DV;   // per-v-head outputs (dv): elements per token row
    const unsigned qstride = (unsigned)p.Hqk * DK;  // per-key-head sums (dq, dk): elements per token row
    const unsigned kstride = (unsigned)p.Hqk * DK * 2;

    // K and Q of item I straight into LDS, where they stay for all of its v-heads
    auto dma_k = [&](const LocItem &I, const int wv, const int l) {
        dma_tile(s.k, chunk_rsrc(p.k + (I.e.row0 * p.Hqk + I.iq) * DK, kstride, I.c, I.e.seq_len), kstride, wv, l);
    };
    auto dma_q = [&](const LocItem &I, const int wv, const int l) {
        dma_tile(s.q, chunk_rsrc(p.q + (I.e.row0 * p.Hqk + I.iq) * DK, kstride, I.c, I.e.seq_len), kstride, wv, l);
    };
    dma_k(cur, wave, lane0);
    dma_q(cur, wave, lane0);

    // this wave's 16 rows of h and dh' of v-head jn (A operands of the
    // transposed products), issued after the v-head's tiles; h of every v-head
    // but the first is issued already at the previous v-head's third phase and
    // waits in these registers (dh' as well would spill)
    f32x4 hr[4][2];
    bf16x8 dH[4], dL[4];  // dh' arrives already split
    auto load_h = [&](const LocItem &I, const int jn, const int wv, const int l) {
        const float *hn = p.h + ((int64_t)I.cg * p.Hv + jn) * DK * DV;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int off = (16 * wv + (l & 15)) * DV + 32 * kk + 8 * (l >> 4);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) hr[kk][hf] = *reinterpret_cast<const f32x4 *>(hn + off + 4 * hf);
        }
    };
    auto load_d = [&](const LocItem &I, const int jn, const int wv, const int l) {
        const bf16 *dn = reinterpret_cast<const bf16 *>(p.dh_ws) + ((int64_t)I.cg * p.Hv + jn) * 2 * DK * DV;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int off = (16 * wv + (l & 15)) * DV + 32 * kk + 8 * (l >> 4);
            dH[kk] = *reinterpret_cast<const bf16x8 *>(dn + off);
            dL[kk] = *reinterpret_cast<const bf16x8 *>(dn + DK * DV + off);
        }
    };

    // dO of v-head jn -> ov and its dv' (hi / lo planes) -> eH / eL, straight
    // into LDS: for the first v-head with its other loads, for each later one
    // during the previous v-head's fifth phase (its third phase is the last to
    // read those tiles; issued there, right after the h rows, the loads held
    // up the fourth phase)
    auto dma_do_dv = [&](const LocItem &I, const int jn, const int wv, const int l) {
        dma_tile(s.ov, chunk_rsrc(p.dO + (I.e.row0 * p.Hv + jn) * DV, vstride, I.c, I.e.seq_len), vstride, wv, l);
        const bf16 *dvn = reinterpret_cast<const bf16 *>(p.dvp_ws) + ((int64_t)I.cg * p.Hv + jn) * 2 * CH * DV;
        dma_tile(s.eH, chunk_rsrc(dvn, DV * 2, 0, CH), DV * 2, wv, l);
        dma_tile(s.eL, chunk_rsrc(dvn + CH * DV, DV * 2, 0, CH), DV * 2, wv, l);
    };

    // dg = reverse in-chunk cumsum of dG, and dbeta, of a finished v-head:
    // wave 0 sums the eight waves' partials and writes them at the next
    // v-head's start (its loads are in flight there), or after the last one
    int64_t dg_row = -1;  // first output row of the v-head whose dg is pending
    int dg_rows = 0;
    auto flush_dg = [&]() {
        float dG = 0.f, db = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            dG += s.dGp[w][lane0];
            db += s.dbp[w][lane0];
        }
        const float x = reverse64(prefix64(reverse64(dG)));  // sum over tokens >= lane
        if (lane0 < dg_rows) {
            const int64_t off = dg_row + (int64_t)lane0 * p.Hv;
            p.dg[off] = x;
            p.dbeta[off] = db;
        }
    };

    bool fresh = true;  // the workgroup's first item: nothing was loaded ahead for it
    while (true) {
    const Where e = cur.e;
    const int c = cur.c, cg = cur.cg, iq = cur.iq;
    const int64_t rowq_c = cur.rowq_c;
    int it_nx = it;  // the next item, found at the start of the last v-head
    LocItem nx;
    nx.ok = false;

    // the key head's v-heads one after another; dq and dk add up across them
    for (int jj = 0; jj < p.group; ++jj) {
    // an opaque thread index per v-head: lane-derived addresses are computed
    // inside the loop, not hoisted out of it and held live across all of it
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, g4 = lane >> 4, r16 = lane & 15;
    const int j = iq * p.group + jj;
    const bool first = jj == 0, last = jj == p.group - 1;
    if (last) {
        it_nx = it + (int)gridDim.x;
        nx = next_item(p, it_nx, lane0);
    }
    const int j_nx = nx.iq * p.group;  // the next item's first v-head
    const float *vnc = p.vn + ((int64_t)cg * p.Hv + j) * CH * DV;     // v'  [i][v]
    // this chunk's first row of the per-(token, v-head) outputs; a row of token t
    // lies t * Hv * 128 elements further (32-bit offsets inside a chunk)
    const int64_t row_c = (e.row0 + (int64_t)c * CH) * p.Hv + j;

    if (first && fresh) dma_do_dv(cur, j, wave, lane);
    Rows<DV * 2 / 16> rv;  // V, stored once dO is dead
    {
        const unsigned astride = (unsigned)p.Hv * CH * 4, gstride = (unsigned)p.Hv * 4;
        Rows<CH * 4 / 16> rtm;
        Rows<DV * 4 / 16> rn;
        load_rows(rv, p.v + (e.row0 * p.Hv + j) * DV, vstride, c, e.seq_len, tid);
        load_rows(rtm, p.A + (e.row0 * p.Hv + j) * CH, astride, c, e.seq_len, tid);
        load_tile_f32(rn, vnc, tid);
        float g = 0.f, b = 0.f;
        if (tid < 64) {
            const __amdgpu_buffer_rsrc_t rg = chunk_rsrc(p.g + e.row0 * p.Hv + j, gstride, c, e.seq_len);
            const __amdgpu_buffer_rsrc_t rb = chunk_rsrc(p.beta + e.row0 * p.Hv + j, gstride, c, e.seq_len);
            g = ld4(rg, (unsigned)tid * gstride);
            b = ld4(rb, (unsigned)tid * gstride);
        }
        store_rows_split(s.tH, s.tL, rtm, L64, tid);
        store_rows_split(s.nH, s.nL, rn, LK, tid);
        if (tid < 64) {
            const float G = prefix64(g);
            s.G[tid] = G;
            s.gam[tid] = __expf(G);
            s.bt[tid] = b;
        }
        if (wave == 0) {
            if (dg_row >= 0) flush_dg();
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                s.dGp[w][lane0] = 0.f;
                s.dbp[w][lane0] = 0.f;
            }
        }
    }
    dma_wait();  // this wave's direct loads (dO, dv', for a new item K and Q) have landed
    lds_barrier();
    if (first && fresh) load_h(cur, j, wave, lane);
    load_d(cur, j, wave, lane);

    float *dGw = s.dGp[wave];
    float *dbw = s.dbp[wave];
    const int rt64 = wave >> 1;
    const int rows_valid = min(CH, e.seq_len - c * CH);
    const float gl = s.gam[CH - 1];

    // ---- 1: dPm = scale (dO v'^T) o Gamma (s <= i) -> p;  gate terms of P
    // both column tiles per k step: the dO and Q rows of row tile rt64 are read once
    f32x4 acc1[2] = {f32x4{}, f32x4{}}, qk1[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 od = fr_row<false>(s.ov + 16 * rt64 * LK, LK, 32 * kk, lane);
        const bf16x8 qr = fr_row<false>(s.q + 16 * rt64 * LK, LK, 32 * kk, lane);
#pragma unroll
        for (int ct2 = 0; ct2 < 2; ++ct2) {
            const int ct = 2 * (wave & 1) + ct2;
            acc1[ct2] = mm_ep(acc1[ct2], od, fr_row<false>(s.nH + 16 * ct * LK, LK, 32 * kk, lane),
                              fr_row<false>(s.nL + 16 * ct * LK, LK, 32 * kk, lane));
            qk1[ct2] = mfma(qr, fr_row<false>(s.k + 16 * ct * LK, LK, 32 * kk, lane), qk1[ct2]);
        }
    }
    {
        float rsum[4] = {0.f, 0.f, 0.f, 0.f};  // row terms of both column tiles, reduced once
#pragma unroll
        for (int ct2 = 0; ct2 < 2; ++ct2) {
            const int ct = 2 * (wave & 1) + ct2;
            const f32x4 acc = acc1[ct2], qk = qk1[ct2];
            f32x4 dpm;
            float colsum = 0.f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int i = 16 * rt64 + 4 * g4 + jj, sc = 16 * ct + r16;
                dpm[jj] = sc <= i ? p.scale * acc[jj] * __expf(s.G[i] - s.G[sc]) : 0.f;
                const float d1 = dpm[jj] * qk[jj];
                rsum[jj] += d1;
                colsum += d1;
            }
            colsum = sum4g(colsum);
            if (g4 == 0) dGw[16 * ct + r16] -= colsum;
            st_split(s.pH, s.pL, L64, 16 * rt64, 16 * ct, dpm, lane);
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float rs = sum16(rsum[jj]);
            if (r16 == 0) dGw[16 * rt64 + 4 * g4 + jj] += rs;
        }
    }
    lds_barrier();

    // ---- 2: transposed dk, dq, dW over this wave's key dims 16 w ..
    f32x4 dkt[4];
    bf16x8 hH[4], hL[4];
    {
        float dot = 0.f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float rh[8];
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                rh[e2] = hr[kk][0][e2];
                rh[4 + e2] = hr[kk][1][e2];
            }
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) dot += rh[e2] * ((float)dH[kk][e2] + (float)dL[kk][e2]);
            split8(rh, hH[kk], hL[kk]);
        }
        // dk: rl_s (dh' v'^T) + Q^T dPm;  gate terms of h'
        float lastacc = 0.f;
        bf16x8 qa[2];  // this wave's rows of Q^T, read once for the four column tiles
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) qa[kk] = fr_tr(s.q + 16 * wave, LK, 32 * kk, lane);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            f32x4 t2 = f32x4{}, qp = f32x4{};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                t2 = mm_pp(t2, dH[kk], dL[kk], fr_row<false>(s.nH + 16 * ct * LK, LK, 32 * kk, lane),
                           fr_row<false>(s.nL + 16 * ct * LK, LK, 32 * kk, lane));
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                qp = mm_ep(qp, qa[kk], fr_tr(s.pH + 16 * ct, L64, 32 * kk, lane),
                           fr_tr(s.pL + 16 * ct, L64, 32 * kk, lane));
            const int col = 16 * ct + r16;  // key token s
            const float rl = __expf(s.G[CH - 1] - s.G[col]);
            float ksum = 0.f;
            {
                const bf16x4 k4 = *reinterpret_cast<const bf16x4 *>(&s.k[col * LK + 16 * wave + 4 * g4]);
                for (int jj = 0; jj < 4; ++jj) ksum += (float)k4[jj] * t2[jj];
            }
            ksum = sum4g(ksum);
            if (g4 == 0) {
                dGw[col] -= rl * ksum;
                lastacc += rl * ksum;
            }
            dkt[ct] = rl * t2 + qp;
        }
        lastacc = sum64(lastacc);
        dot = sum64(dot);
        if (lane == 0) dGw[CH - 1] += lastacc + gl * dot;
    }
    // dq: scale gamma_i (h dO^T) + K^T dPm^T;  gate term of O (inter); stored
    f32x4 qprev[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
        qprev[ct] = group_prev(p.dq_ws, rowq_c * DK + (unsigned)(16 * ct + r16) * qstride + 16 * wave + 4 * g4, first,
                               16 * ct + r16 < rows_valid);
    bf16x8 ka[2];  // this wave's rows of K^T, read once for the four column tiles
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) ka[kk] = fr_tr(s.k + 16 * wave, LK, 32 * kk, lane);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        f32x4 t1 = f32x4{}, kq = f32x4{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            t1 = mm_pe(t1, hH[kk], hL[kk], fr_row<false>(s.ov + 16 * ct * LK, LK, 32 * kk, lane));
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            kq = mm_ep(kq, ka[kk], fr_row<true>(s.pH + 16 * ct * L64, L64, 32 * kk, lane),
                       fr_row<true>(s.pL + 16 * ct * L64, L64, 32 * kk, lane));
        const int col = 16 * ct + r16;  // query token i
        const float sg = p.scale * s.gam[col];
        float qsum = 0.f;
        {
            const bf16x4 q4 = *reinterpret_cast<const bf16x4 *>(&s.q[col * LK + 16 * wave + 4 * g4]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) qsum += (float)q4[jj] * t1[jj];
        }
        qsum = sum4g(qsum);
        if (g4 == 0) dGw[col] += sg * qsum;
        if (col < rows_valid)
            group_put(p, p.dq_ws, p.dq, rowq_c * DK + (unsigned)col * qstride + 16 * wave + 4 * g4,
                      sg * t1 + kq + qprev[ct], last);
    }
    lds_barrier();  // v' and dO are dead: their tiles take dW and V

    // dW = -(h dv'^T)^T -> n [token][key dim];  V -> ov
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        f32x4 tw = f32x4{};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            tw = mm_pp(tw, hH[kk], hL[kk], fr_row<false>(s.eH + 16 * ct * LK, LK, 32 * kk, lane),
                       fr_row<false>(s.eL + 16 * ct * LK, LK, 32 * kk, lane));
        st_split_t(s.nH, s.nL, LK, 16 * wave, 16 * ct, -tw, lane);
    }
    store_rows_ld(s.ov, rv, LK, tid);
    lds_barrier();
    if (!last)
        load_h(cur, j + 1, wave, lane);
    else if (nx.ok)
        load_h(nx, j_nx, wave, lane);

    // ---- 3: dT -> p;  dK, dbeta, dG terms of W;  dV and the dbeta term of U
    // both column tiles per k step: the dW and dv' rows of row tile rt64 are read once
    f32x4 a1t[2] = {f32x4{}, f32x4{}}, a2t[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 nh = fr_row<false>(s.nH + 16 * rt64 * LK, LK, 32 * kk, lane);
        const bf16x8 nl = fr_row<false>(s.nL + 16 * rt64 * LK, LK, 32 * kk, lane);
        const bf16x8 eh = fr_row<false>(s.eH + 16 * rt64 * LK, LK, 32 * kk, lane);
        const bf16x8 el = fr_row<false>(s.eL + 16 * rt64 * LK, LK, 32 * kk, lane);
#pragma unroll
        for (int ct2 = 0; ct2 < 2; ++ct2) {
            const int ct = 2 * (wave & 1) + ct2;
            a1t[ct2] = mm_pe(a1t[ct2], nh, nl, fr_row<false>(s.k + 16 * ct * LK, LK, 32 * kk, lane));
            a2t[ct2] = mm_pe(a2t[ct2], eh, el, fr_row<false>(s.ov + 16 * ct * LK, LK, 32 * kk, lane));
        }
    }
#pragma unroll
    for (int ct2 = 0; ct2 < 2; ++ct2) {
        const int ct = 2 * (wave & 1) + ct2;
        const f32x4 a1 = a1t[ct2], a2 = a2t[ct2];
        const int sc = 16 * ct + r16;
        st_split(s.pH, s.pL, L64, 16 * rt64, 16 * ct, s.bt[sc] * (s.gam[sc] * a1 + a2), lane);
    }
    // T^T dW and (T^T dv')^T over the four token tiles x of T: both take the
    // transposed T fragments of tile x, read once for the two products
    //   T^T dW, transposed: (key dim, token s): this wave's key columns of dW;
    //   (T^T dv')^T = dv'^T T over value columns 16 w .., all token columns s:
    //   lane (m, g) holds value columns 16 w + 4 g .. +3 of token 16 x + m,
    //   so dv goes out as four contiguous values per lane and the dbeta term
    //   is a four-term dot product with V plus a sum over g.
    bf16x8 wH[2], wL[2], bh[2], bl[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        wH[kk] = fr_tr(s.nH + 16 * wave, LK, 32 * kk, lane);
        wL[kk] = fr_tr(s.nL + 16 * wave, LK, 32 * kk, lane);
        bh[kk] = fr_tr(s.eH + 16 * wave, LK, 32 * kk, lane);
        bl[kk] = fr_tr(s.eL + 16 * wave, LK, 32 * kk, lane);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        bf16x8 th[2], tl[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            th[kk] = fr_tr(s.tH + 16 * x, L64, 32 * kk, lane);
            tl[kk] = fr_tr(s.tL + 16 * x, L64, 32 * kk, lane);
        }
        const int sc = 16 * x + r16;  // token s of this lane's column
        {
            f32x4 acc = f32x4{};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) acc = mm_pp(acc, wH[kk], wL[kk], th[kk], tl[kk]);
            float rk = 0.f;
            {
                const bf16x4 k4 = *reinterpret_cast<const bf16x4 *>(&s.k[sc * LK + 16 * wave + 4 * g4]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) rk += acc[jj] * (float)k4[jj];
            }
            rk = sum4g(rk);
            const float bgs = s.bt[sc] * s.gam[sc];
            if (g4 == 0) {
                dbw[sc] += s.gam[sc] * rk;
                dGw[sc] += bgs * rk;
            }
            dkt[x] += bgs * acc;
        }
        {
            f32x4 acc = f32x4{};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) acc = mm_pp(acc, bh[kk], bl[kk], th[kk], tl[kk]);
            const int v0 = 16 * wave + 4 * g4;  // value columns v0 .. v0 + 3
            const bf16x4 vv4 = *reinterpret_cast<const bf16x4 *>(&s.ov[sc * LK + v0]);
            float rvv = 0.f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) rvv += acc[jj] * (float)vv4[jj];
            rvv = sum4g(rvv);
            if (g4 == 0) dbw[sc] += rvv;
            const f32x4 dvv = s.bt[sc] * acc;
            if (sc < rows_valid) {
                const int64_t off = row_c * DV + (int64_t)sc * tstride + v0;
                if (p.grad_f32)
                    *reinterpret_cast<f32x4 *>(static_cast<float *>(p.dv) + off) = dvv;
                else
                    *reinterpret_cast<bf16x4 *>(static_cast<bf16 *>(p.dv) + off) =
                        bf16x4{(bf16)dvv[0], (bf16)dvv[1], (bf16)dvv[2], (bf16)dvv[3]};
            }
        }
    }
    lds_barrier();

    // ---- 4: Y = T^T dT -> n (as [64][64])
    {
        // T^T rows of tile rt64, read once for both column tiles
        bf16x8 th[2], tl[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            th[kk] = fr_tr(s.tH + 16 * rt64, L64, 32 * kk, lane);
            tl[kk] = fr_tr(s.tL + 16 * rt64, L64, 32 * kk, lane);
        }
#pragma unroll
        for (int ct2 = 0; ct2 < 2; ++ct2) {
            const int ct = 2 * (wave & 1) + ct2;
            f32x4 acc = f32x4{};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                acc = mm_pp(acc, th[kk], tl[kk], fr_tr(s.pH + 16 * ct, L64, 32 * kk, lane),
                            fr_tr(s.pL + 16 * ct, L64, 32 * kk, lane));
            st_split(s.nH, s.nL, L64, 16 * rt64, 16 * ct, acc, lane);
        }
    }
    lds_barrier();

    // dk's running sum, read before the direct loads below: a wait for it then
    // leaves those loads in flight (the count of memory operations is in order)
    f32x4 kprev[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
        kprev[ct] = group_prev(p.dk_ws, rowq_c * DK + (unsigned)(16 * ct + r16) * qstride + 16 * wave + 4 * g4, first,
                              16 * ct + r16 < rows_valid);
    // ov, eH and eL are dead from here on, and q since the second phase
    if (!last) {
        dma_do_dv(cur, j + 1, wave, lane);
    } else if (nx.ok) {
        dma_do_dv(nx, j_nx, wave, lane);
        dma_q(nx, wave, lane);
    }

    // ---- 5: dA~ = -(Y T^T) strictly lower;  M = dA~ o beta_i Gamma_is;  S = M + M^T -> p;
    //      gate / beta terms of A~
    // both column tiles per k step: the Y and K rows of row tile rt64 are read once
    f32x4 yat[2] = {f32x4{}, f32x4{}}, kkt[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 yh = fr_row<false>(s.nH + 16 * rt64 * L64, L64, 32 * kk, lane);
        const bf16x8 yl = fr_row<false>(s.nL + 16 * rt64 * L64, L64, 32 * kk, lane);
#pragma unroll
        for (int ct2 = 0; ct2 < 2; ++ct2) {
            const int ct = 2 * (wave & 1) + ct2;
            yat[ct2] = mm_pp(yat[ct2], yh, yl, fr_row<false>(s.tH + 16 * ct * L64, L64, 32 * kk, lane),
                             fr_row<false>(s.tL + 16 * ct * L64, L64, 32 * kk, lane));
        }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const bf16x8 kr = fr_row<false>(s.k + 16 * rt64 * LK, LK, 32 * kk, lane);
#pragma unroll
        for (int ct2 = 0; ct2 < 2; ++ct2)
            kkt[ct2] = mfma(kr, fr_row<false>(s.k + 16 * (2 * (wave & 1) + ct2) * LK, LK, 32 * kk, lane), kkt[ct2]);
    }
    float rsum[4] = {0.f, 0.f, 0.f, 0.f}, bsum[4] = {0.f, 0.f, 0.f, 0.f};  // row terms of both column tiles
#pragma unroll
    for (int ct2 = 0; ct2 < 2; ++ct2) {
        const int ct = 2 * (wave & 1) + ct2;
        const f32x4 ya = yat[ct2], kk4 = kkt[ct2];
        f32x4 m;
        float colsum = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int i = 16 * rt64 + 4 * g4 + jj, sc = 16 * ct + r16;
            float d2 = 0.f, db = 0.f;
            m[jj] = 0.f;
            if (sc < i) {
                const float da = -ya[jj];
                const float gm = __expf(s.G[i] - s.G[sc]);
                m[jj] = da * s.bt[i] * gm;
                d2 = m[jj] * kk4[jj];
                db = da * gm * kk4[jj];
            }
            rsum[jj] += d2;
            bsum[jj] += db;
            colsum += d2;
        }
        colsum = sum4g(colsum);
        if (g4 == 0) dGw[16 * ct + r16] -= colsum;
        // S = M + M^T (the sixth phase needs only K^T S): a tile below the
        // diagonal goes to its place and, transposed, to the mirrored one; a
        // tile above it is zero in M and is written by its mirror's wave
        if (ct < rt64) {
            st_split(s.pH, s.pL, L64, 16 * rt64, 16 * ct, m, lane);
            st_split_t(s.pH, s.pL, L64, 16 * rt64, 16 * ct, m, lane);
        } else if (ct == rt64) {
            st_sym_diag(s.pH, s.pL, L64, 16 * ct, m, lane);
        }
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const float rs = sum16(rsum[jj]), rb = sum16(bsum[jj]);
        if (r16 == 0) {
            dGw[16 * rt64 + 4 * g4 + jj] += rs;
            dbw[16 * rt64 + 4 * g4 + jj] += rb;
        }
    }
    lds_barrier();

    // ---- 6: dK += M K + M^T K = S K (transposed: K^T S, S symmetric); store dk of this v-head
    bf16x8 ak6[2];  // this wave's rows of K^T, read once for the four token tiles
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) ak6[kk] = fr_tr(s.k + 16 * wave, LK, 32 * kk, lane);
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            dkt[ct] = mm_ep(dkt[ct], ak6[kk], fr_tr(s.pH + 16 * ct, L64, 32 * kk, lane),
                            fr_tr(s.pL + 16 * ct, L64, 32 * kk, lane));
        const int tok = 16 * ct + r16;
        if (tok < rows_valid)
            group_put(p, p.dk_ws, p.dk, rowq_c * DK + (unsigned)tok * qstride + 16 * wave + 4 * g4, dkt[ct] + kprev[ct],
                      last);
    }
    lds_barrier();
    if (last && nx.ok) dma_k(nx, wave, lane);  // k was last read in the sixth phase

    dg_row = row_c;
    dg_rows = rows_valid;
    }
    if (!nx.ok) break;
    cur = nx;
    it = it_nx;
    fresh = false;
    }
    if (wave == 0) flush_dg();  // the eight waves' partials are complete since the sixth phase's barrier
}

// ---------------------------------------------------------------- reverse pass
struct __attribute__((aligned(16))) SmemDh {
    bf16 k[CH * LK], q[CH * LK];      // K, Q   [token][key dim]
    bf16 dO[CH * L64];                // dO, this workgroup's 64 value columns
    bf16 aH[CH * L64], aL[CH * L64];  // dv'   [token][col]
    bf16 tH[CH * L64], tL[CH * L64];  // T diag(beta gamma), hi / lo
    bf16 pH[CH * L64], pL[CH * L64];  // P   [query token][key token]
    bf16 hH[DK * L64], hL[DK * L64];  // dh  [key dim][value column]
    float G[CH], gam[CH], bg[CH];
};
static_assert(sizeof(SmemDh) <= 160 * 1024, "reverse-pass LDS over 160 KB");

// One chunk's inputs of the reverse pass, in the registers of waves 0-3 (the
// waves that stage tiles) between load and store.
constexpr int NTD = NT / 2;  // threads of waves 0-3
template <int PPR>
struct RowsD {
    static_assert(CH * PPR % NTD == 0, "a tile is a whole number of pieces per staging thread");
    static constexpr int PER = CH * PPR / NTD;
    u32x4 x[PER];
};
struct ChunkDh {
    RowsD<DK * 2 / 16> k, q;
    RowsD<HVC * 2 / 16> dO;
    RowsD<CH * 4 / 16> t;
    float g, b;  // lane l: token l (every staging wave)
};

template <int PPR>
__device__ __forceinline__ void load_rows_d(RowsD<PPR> &R, const void *base, unsigned stride, int c, int seq_len,
                                            int td) {
    const __amdgpu_buffer_rsrc_t r = chunk_rsrc(base, stride, c, seq_len);
#pragma unroll
    for (int i = 0; i < RowsD<PPR>::PER; ++i) {
        const int pc = td + i * NTD;
        const int row = pc / PPR, col = pc - row * PPR;
        R.x[i] = ld16(r, (unsigned)row * stride + (unsigned)col * 16u);
    }
}

template <int PPR>
__device__ __forceinline__ void store_rows_d(bf16 *dst, const RowsD<PPR> &R, int ld, int td) {
#pragma unroll
    for (int i = 0; i < RowsD<PPR>::PER; ++i) {
        const int pc = td + i * NTD;
        const int row = pc / PPR, col = pc - row * PPR;
        *reinterpret_cast<u32x4 *>(&dst[row * ld + 8 * col]) = R.x[i];
    }
}

// td: thread index among waves 0-3
__device__ __forceinline__ void load_chunk_dh(ChunkDh &R, const BwdParams &p, const Where &e, int j, int half, int c,
                                              int td) {
    const int iq = j / p.group;
    const unsigned kstride = (unsigned)p.Hqk * DK * 2, vstride = (unsigned)p.Hv * DV * 2;
    const unsigned astride = (unsigned)p.Hv * CH * 4, gstride = (unsigned)p.Hv * 4;
    load_rows_d(R.k, p.k + (e.row0 * p.Hqk + iq) * DK, kstride, c, e.seq_len, td);
    load_rows_d(R.q, p.q + (e.row0 * p.Hqk + iq) * DK, kstride, c, e.seq_len, td);
    load_rows_d(R.dO, p.dO + (e.row0 * p.Hv + j) * DV + half * HVC, vstride, c, e.seq_len, td);
    load_rows_d(R.t, p.A + (e.row0 * p.Hv + j) * CH, astride, c, e.seq_len, td);
    const int lane = td & 63;
    const __amdgpu_buffer_rsrc_t rg = chunk_rsrc(p.g + e.row0 * p.Hv + j, gstride, c, e.seq_len);
    const __amdgpu_buffer_rsrc_t rb = chunk_rsrc(p.beta + e.row0 * p.Hv + j, gstride, c, e.seq_len);
    R.g = ld4(rg, (unsigned)lane * gstride);
    R.b = ld4(rb, (unsigned)lane * gstride);
}

// Tiles of one chunk into LDS (waves 0-3): K, Q, dO as bf16; T with its columns
// scaled by beta gamma as a hi / lo pair.  Every staging wave forms the gate
// prefix sums itself (lane = token) for the column scales.
__device__ __forceinline__ void store_chunk_dh(SmemDh &s, const ChunkDh &R, int td) {
    const int lane = td & 63;
    const float G = prefix64(R.g);
    const float gam = __expf(G);
    const float bg = R.b * gam;
    if (td < 64) s.G[lane] = G;
    // every staging wave writes the same scales and reads back only its own writes
    s.bg[lane] = bg;
    s.gam[lane] = gam;
    store_rows_d(s.k, R.k, LK, td);
    store_rows_d(s.q, R.q, LK, td);
    store_rows_d(s.dO, R.dO, L64, td);
    constexpr int PPR = CH * 4 / 16;
#pragma unroll
    for (int i = 0; i < RowsD<PPR>::PER; ++i) {
        const int pc = td + i * NTD;
        const int row = pc / PPR, col = 4 * (pc - row * PPR);
        f32x4 x = __builtin_bit_cast(f32x4, R.t.x[i]);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) x[e2] *= s.bg[col + e2];
        bf16x4 h, l;
        split4(x, h, l);
        *reinterpret_cast<bf16x4 *>(&s.tH[row * L64 + col]) = h;
        *reinterpret_cast<bf16x4 *>(&s.tL[row * L64 + col]) = l;
    }
}

// One workgroup per (segment, v-head, value half).  Walks the segment's chunks
// last to first.  The waves have two roles, so that each 64 x 64 product is
// tiled into 32 x 32 blocks and a shared operand is read by fewer waves:
// waves 0-3 form P and dv' (wave q: token row tiles 2 (q / 2) + {0, 1}, column
// tiles 2 (q % 2) + {0, 1}), copy dh' and dv' to HBM and stage the next chunk's
// tiles; waves 4-7 carry dh (K x 64 fp32) in registers -- wave 4 + q holds key
// dims 32 q .. 32 q + 31 -- and form W and Q^T diag(gamma) dO for those key
// dims and the dh update, with a hi / lo copy of dh in LDS for the K dh
// product.  Per chunk: (1) P | W; (2) dv' | Q^T diag(gamma) dO; (3) tile
// staging | dh update.
// Main pass (p.pass == 0): a segment that does not end its sequence starts
// after a warm-up over the chunks that follow it (WARMUP, gate-driven window as
// in the forward) or from its exact start gradient (EXACT, from the combine);
// stores, for each own chunk c, dh' (the gradient with respect to the state
// after c) and dv'.  Pre-pass (p.pass == 1, EXACT; two workgroups per
// (segment, v-head, half)): for every segment that is not the first of its
// sequence, the zero-start result S (which = 0) and the transition map M
// (which = 1: the walk applied to the identity with the dO terms left out).
__global__ void __launch_bounds__(NT, 1) gdn_bwd_dh_kernel(BwdParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    SmemDh &s = *reinterpret_cast<SmemDh *>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool pre = p.pass == 1;
    const int per = pre ? 4 * p.Hv : 2 * p.Hv;
    const int seg = blockIdx.x / per;
    const int rem = blockIdx.x - seg * per;
    const int j = rem / (pre ? 4 : 2), half = rem & 1;
    const bool mmap = pre && ((rem >> 1) & 1);  // pre-pass: transition map M
    if (seg >= p.num_segments) return;
    const Where e = find_segment(p.cu, p.N, p.T, p.L, seg, lane);
    if (e.n < 0) return;
    if (pre && e.c_begin == 0) return;  // the first segment needs no map
    const int nt = seq_chunks(e.seq_len);
    const int c_end = e.c_begin + e.c_count;
    const int g4 = lane >> 4, r16 = lane & 15;
    const bool exact_start = !pre && !e.last && p.cp_mode == 1 /* EXACT */;
    const bool prod = wave < 4;  // waves 0-3: P, dv', copies and staging; 4-7: dh
    const int q4 = wave & 3;
    const int td = tid & (NTD - 1);
    const int rt0 = 2 * (q4 >> 1), ct0 = 2 * (q4 & 1);  // a product wave's 32 x 32 block
    const int kt0 = 2 * q4;                              // a dh wave's first key tile

    // where the reverse walk starts: the sequence end (from d final_state), a
    // warm-up window after the segment (from zero), or the segment end (EXACT)
    int c_last = c_end;
    if (pre || exact_start) {
        c_last = c_end;
    } else if (!e.last && p.cp_mode == 2 /* WARMUP */) {
        // gate-driven window after the segment, until the summed log-gates
        // reach the fp32 noise floor, or to the sequence end (then the walk
        // begins from d final_state and is exact)
        const int w = gate_window(p.g + e.row0 * p.Hv, p.Hv, j, e.seq_len, c_end, 1, nt - c_end, p.warmup_cap, lane);
        c_last = __builtin_amdgcn_readfirstlane(c_end + w);
    } else {
        c_last = nt;
    }
    const bool from_end = !pre && !exact_start && (c_last == nt);

    const int cbase = seq_chunk_base(p.cu, p.T, e.n, lane);

    // The two roles run their own copies of the chunk loop, with the same three
    // barriers per chunk (a barrier counts arrivals, so the copies stay in step);
    // apart, each copy's registers are allocated for its role alone.
    if (prod) {
        // The tiles of the next chunk (walking backwards) go into LDS during the
        // dh update of the current one, which reads none of them; their inputs
        // are loaded into these waves' registers one chunk ahead of that.
        ChunkDh R;
        if (c_last - 1 >= e.c_begin) {
            load_chunk_dh(R, p, e, j, half, c_last - 1, td);
            store_chunk_dh(s, R, td);
        }
        if (c_last - 2 >= e.c_begin) load_chunk_dh(R, p, e, j, half, c_last - 2, td);
        for (int c = c_last - 1; c >= e.c_begin; --c) {
            const bool own = !pre && c < c_end;
            __syncthreads();  // chunk c's tiles in LDS; the previous dh update done
            // P = (Q K^T) o Gamma, s <= i: query row tiles rt0 + {0, 1}, key
            // column tiles ct0 + {0, 1} (each fragment read once for two products)
            f32x4 pacc[2][2] = {{f32x4{}, f32x4{}}, {f32x4{}, f32x4{}}};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 qr[2], kf[2];
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    qr[a] = fr_row<false>(s.q + 16 * (rt0 + a) * LK, LK, 32 * kk, lane);
                    kf[a] = fr_row<false>(s.k + 16 * (ct0 + a) * LK, LK, 32 * kk, lane);
                }
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) pacc[a][b] = mfma(qr[a], kf[b], pacc[a][b]);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int rt = rt0 + a, ct = ct0 + b;
                    const f32x4 acc = pacc[a][b];
                    f32x4 pv;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int i = 16 * rt + 4 * g4 + jj, sc = 16 * ct + r16;
                        pv[jj] = sc <= i ? acc[jj] * __expf(s.G[i] - s.G[sc]) : 0.f;
                    }
                    st_split(s.pH, s.pL, L64, 16 * rt, 16 * ct, pv, lane);
                }
            // dh' of chunk c (the hi / lo copy of dh in LDS, unchanged in this
            // step) -> HBM as two bf16 planes [d][v], 16 bytes per thread and plane piece
            if (own) {
                bf16 *dst = reinterpret_cast<bf16 *>(p.dh_ws) + ((int64_t)(cbase + c) * p.Hv + j) * 2 * DK * DV + half * HVC;
#pragma unroll
                for (int i = 0; i < DK * HVC / 8 / NTD; ++i) {
                    const int pc = td + i * NTD;
                    const int row = pc / (HVC / 8), col = 8 * (pc % (HVC / 8));
                    *reinterpret_cast<bf16x8 *>(dst + row * DV + col) = *reinterpret_cast<const bf16x8 *>(&s.hH[row * L64 + col]);
                    *reinterpret_cast<bf16x8 *>(dst + DK * DV + row * DV + col) =
                        *reinterpret_cast<const bf16x8 *>(&s.hL[row * L64 + col]);
                }
            }
            __syncthreads();

            // dv' = scale P^T dO + diag(rl) K dh: token row tiles rt0 + {0, 1},
            // value column tiles ct0 + {0, 1}
            f32x4 a1[2][2] = {{f32x4{}, f32x4{}}, {f32x4{}, f32x4{}}};
            f32x4 a2[2][2] = {{f32x4{}, f32x4{}}, {f32x4{}, f32x4{}}};
            if (!mmap) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    bf16x8 ph[2], pl[2], of[2];
#pragma unroll
                    for (int a = 0; a < 2; ++a) {
                        ph[a] = fr_tr(s.pH + 16 * (rt0 + a), L64, 32 * kk, lane);
                        pl[a] = fr_tr(s.pL + 16 * (rt0 + a), L64, 32 * kk, lane);
                        of[a] = fr_tr(s.dO + 16 * (ct0 + a), L64, 32 * kk, lane);
                    }
#pragma unroll
                    for (int a = 0; a < 2; ++a)
#pragma unroll
                        for (int b = 0; b < 2; ++b) a1[a][b] = mm_pe(a1[a][b], ph[a], pl[a], of[b]);
                }
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                bf16x8 kr[2], hf[2], hl[2];
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    kr[a] = fr_row<true>(s.k + 16 * (rt0 + a) * LK, LK, 32 * kk, lane);
                    hf[a] = fr_tr(s.hH + 16 * (ct0 + a), L64, 32 * kk, lane);
                    hl[a] = fr_tr(s.hL + 16 * (ct0 + a), L64, 32 * kk, lane);
                }
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int b = 0; b < 2; ++b) a2[a][b] = mm_ep(a2[a][b], kr[a], hf[b], hl[b]);
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int rt = rt0 + a, ct = ct0 + b;
                    f32x4 x;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int i = 16 * rt + 4 * g4 + jj;
                        x[jj] = p.scale * a1[a][b][jj] + __expf(s.G[CH - 1] - s.G[i]) * a2[a][b][jj];
                    }
                    st_split(s.aH, s.aL, L64, 16 * rt, 16 * ct, x, lane);
                }
            __syncthreads();

            if (own) {
                // dv' of chunk c -> HBM as two bf16 planes [token][v] (hi, lo): the
                // chunk-local kernel's split operands, 16 bytes per thread and plane
                bf16 *dst = reinterpret_cast<bf16 *>(p.dvp_ws) + ((int64_t)(cbase + c) * p.Hv + j) * 2 * CH * DV + half * HVC;
#pragma unroll
                for (int i = 0; i < CH * HVC / 8 / NTD; ++i) {
                    const int pc = td + i * NTD;
                    const int row = pc / (HVC / 8), col = 8 * (pc % (HVC / 8));
                    *reinterpret_cast<bf16x8 *>(dst + row * DV + col) = *reinterpret_cast<const bf16x8 *>(&s.aH[row * L64 + col]);
                    *reinterpret_cast<bf16x8 *>(dst + CH * DV + row * DV + col) =
                        *reinterpret_cast<const bf16x8 *>(&s.aL[row * L64 + col]);
                }
            }
            if (c - 1 >= e.c_begin) {
                store_chunk_dh(s, R, td);
                if (c - 2 >= e.c_begin) load_chunk_dh(R, p, e, j, half, c - 2, td);
            }
        }
        return;
    }

    // dh at the start of the walk (waves 4-7): rows 16 (kt0 + t) + 4 g + jj, value column 16 ct + r
    const int64_t sbase = ((int64_t)e.n * p.Hv + j) * DK * DV + half * HVC;
    const int64_t wbase = ((int64_t)seg * p.Hv + j) * DK * DV + half * HVC;  // exact-CP workspace
    f32x4 dh[2][4];
    {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int d = 16 * (kt0 + t) + 4 * g4 + jj, v = 16 * ct + r16;
                    float x = 0.f;
                    if (from_end && p.dht) x = p.dht[sbase + (int64_t)d * DV + v];
                    if (exact_start) x = p.ws_h[wbase + (int64_t)d * DV + v];
                    if (mmap) x = (d == half * HVC + v) ? 1.f : 0.f;  // identity columns of this half
                    dh[t][ct][jj] = x;
                }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) st_split(s.hH, s.hL, L64, 16 * (kt0 + t), 16 * ct, dh[t][ct], lane);
    }
    for (int c = c_last - 1; c >= e.c_begin; --c) {
        __syncthreads();  // chunk c's tiles in LDS; the previous dh update done
        const float gl = s.gam[CH - 1];
        // W^T operand fragments: [key tile t][token k step]
        bf16x8 wa[2][2], wl[2][2];
        {
            // W = T diag(beta gamma) K: key columns of tiles kt0 + {0, 1}, all token
            // rows.  Only this wave reads these columns back (as the A operand of
            // W^T dv'), and two stacked accumulator tiles are already that operand
            // at the transposed-read k order, so W stays in registers (hi / lo).
            bf16x8 bk[2][2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) bk[t][kk] = fr_tr(s.k + 16 * (kt0 + t), LK, 32 * kk, lane);
            f32x4 wt[2][4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                bf16x8 th[2], tl[2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    th[kk] = fr_row<true>(s.tH + 16 * rt * L64, L64, 32 * kk, lane);
                    tl[kk] = fr_row<true>(s.tL + 16 * rt * L64, L64, 32 * kk, lane);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    wt[t][rt] = f32x4{};
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) wt[t][rt] = mm_pe(wt[t][rt], th[kk], tl[kk], bk[t][kk]);
                }
            }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const float x[8] = {wt[t][2 * kk][0],     wt[t][2 * kk][1],     wt[t][2 * kk][2],
                                        wt[t][2 * kk][3],     wt[t][2 * kk + 1][0], wt[t][2 * kk + 1][1],
                                        wt[t][2 * kk + 1][2], wt[t][2 * kk + 1][3]};
                    split8(x, wa[t][kk], wl[t][kk]);
                }
        }
        __syncthreads();

        f32x4 u[2][4];
        {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) u[t][ct] = f32x4{};
            if (!mmap) {
                // (diag(gamma) Q)^T dO: this wave's key rows of Q^T (transposing
                // reads, k = tokens in the transposed-read order) scaled per token
                // by gamma and split hi / lo, against the exact dO tile
                bf16x8 aqh[2][2], aql[2][2];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const f32x4 ga = *reinterpret_cast<const f32x4 *>(&s.gam[32 * kk + 4 * g4]);
                    const f32x4 gb = *reinterpret_cast<const f32x4 *>(&s.gam[32 * kk + 16 + 4 * g4]);
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const bf16x8 qf = fr_tr(s.q + 16 * (kt0 + t), LK, 32 * kk, lane);
                        float f[8];
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2) {
                            f[e2] = (float)qf[e2] * ga[e2];
                            f[4 + e2] = (float)qf[4 + e2] * gb[e2];
                        }
                        split8(f, aqh[t][kk], aql[t][kk]);
                    }
                }
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) {
                        const bf16x8 of = fr_tr(s.dO + 16 * ct, L64, 32 * kk, lane);
#pragma unroll
                        for (int t = 0; t < 2; ++t) u[t][ct] = mm_pe(u[t][ct], aqh[t][kk], aql[t][kk], of);
                    }
            }
        }
        __syncthreads();

        {
            // dh <- gamma_last dh + scale Q^T diag(gamma) dO - W^T dv' (each dv'
            // fragment read once for both key tiles)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                f32x4 acc[2] = {f32x4{}, f32x4{}};
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bf16x8 af = fr_tr(s.aH + 16 * ct, L64, 32 * kk, lane);
                    const bf16x8 al = fr_tr(s.aL + 16 * ct, L64, 32 * kk, lane);
#pragma unroll
                    for (int t = 0; t < 2; ++t) acc[t] = mm_pp(acc[t], wa[t][kk], wl[t][kk], af, al);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    dh[t][ct] = gl * dh[t][ct] + p.scale * u[t][ct] - acc[t];
                    st_split(s.hH, s.hL, L64, 16 * (kt0 + t), 16 * ct, dh[t][ct], lane);
                }
            }
        }
    }
    if (pre) {
        float *dst = (mmap ? p.ws_m : p.ws_s) + wbase;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    dst[(int64_t)(16 * (kt0 + t) + 4 * g4 + jj) * DV + 16 * ct + r16] = dh[t][ct][jj];
    } else if (e.c_begin == 0 && p.dh0) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    p.dh0[sbase + (int64_t)(16 * (kt0 + t) + 4 * g4 + jj) * DV + 16 * ct + r16] = dh[t][ct][jj];
    }
}

// Exact context parallelism, combine: per (sequence, v-head), from the end of
// the sequence backwards, the gradient each segment starts from:
// G_in(R-1) = d final_state (or 0), G_in(r) = M_{r+1} G_in(r+1) + S_{r+1}.
// Wave w computes key rows 16 w .. +15 (eight value column tiles); M rows are
// split from HBM, G_in is read as a hi / lo pair from LDS.
struct __attribute__((aligned(16))) SmemComb {
    bf16 gH[DK * LK], gL[DK * LK];  // G_in [key dim][value]
};

__global__ void __launch_bounds__(NT, 1) gdn_bwd_cp_combine_kernel(BwdParams p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    SmemComb &s = *reinterpret_cast<SmemComb *>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, r16 = lane & 15;
    const int n = blockIdx.x / p.Hv;
    const int j = blockIdx.x - n * p.Hv;
    if (n >= p.N) return;
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
    f32x4 gin[8];
    const int64_t sbase = ((int64_t)n * p.Hv + j) * DK * DV;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            gin[ct][jj] = p.dht ? p.dht[sbase + (int64_t)(16 * wave + 4 * g4 + jj) * DV + 16 * ct + r16] : 0.f;
    for (int r = R - 2; r >= 0; --r) {
        __syncthreads();  // previous products done reading the pair
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) st_split(s.gH, s.gL, LK, 16 * wave, 16 * ct, gin[ct], lane);
        __syncthreads();
        const int64_t off = ((int64_t)(seg0 + r + 1) * p.Hv + j) * DK * DV;
        const float *M = p.ws_m + off, *S = p.ws_s + off;
        bf16x8 mh[4], ml[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float raw[8];
            fr_rowf<true>(M + 16 * wave * DK, DK, 32 * kk, lane, mh[kk], ml[kk], raw);
        }
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            f32x4 acc;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) acc[jj] = S[(int64_t)(16 * wave + 4 * g4 + jj) * DV + 16 * ct + r16];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = mm_pp(acc, mh[kk], ml[kk], fr_tr(s.gH + 16 * ct, LK, 32 * kk, lane),
                            fr_tr(s.gL + 16 * ct, LK, 32 * kk, lane));
            gin[ct] = acc;
        }
        float *dst = p.ws_h + ((int64_t)(seg0 + r) * p.Hv + j) * DK * DV;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dst[(int64_t)(16 * wave + 4 * g4 + jj) * DV + 16 * ct + r16] = gin[ct][jj];
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
    if (p.num_segments > 0 && p.cp_mode == 1 /* EXACT */ && p.rows > 0) {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(bwdk::gdn_bwd_cp_combine_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(bwdk::SmemComb));
        if (err != hipSuccess) return (int)err;
        BwdParams pre = p;
        pre.pass = 1;
        hipLaunchKernelGGL(bwdk::gdn_bwd_dh_kernel, dim3((unsigned)(p.num_segments * p.Hv * 4)), dim3(bwdk::NT),
                           sizeof(bwdk::SmemDh), st, pre);
        err = hipGetLastError();
        if (err != hipSuccess) return (int)err;
        hipLaunchKernelGGL(bwdk::gdn_bwd_cp_combine_kernel, dim3((unsigned)(p.N * p.Hv)), dim3(bwdk::NT),
                           sizeof(bwdk::SmemComb), st, p);
        err = hipGetLastError();
        if (err != hipSuccess) return (int)err;
    }
    if (p.num_segments > 0) {
        BwdParams mp = p;
        mp.pass = 0;
        hipLaunchKernelGGL(bwdk::gdn_bwd_dh_kernel, dim3((unsigned)(p.num_segments * p.Hv * 2)), dim3(bwdk::NT),
                           sizeof(bwdk::SmemDh), st, mp);
        err = hipGetLastError();
        if (err != hipSuccess) return (int)err;
    }
    if (p.num_chunk_entries > 0 && p.rows > 0) {
        // one persistent workgroup per compute unit (its LDS allows one), at most one per item
        int dev = 0, cus = 0;
        err = hipGetDevice(&dev);
        if (err != hipSuccess) return (int)err;
        err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess) return (int)err;
        const int64_t items = (int64_t)p.num_chunk_entries * p.Hqk;
        const unsigned grid = (unsigned)std::max<int64_t>(1, std::min<int64_t>(items, cus));
        hipLaunchKernelGGL(bwdk::gdn_bwd_local_kernel, dim3(grid), dim3(bwdk::NT),
                           sizeof(bwdk::SmemLoc), st, p);
        err = hipGetLastError();
        if (err != hipSuccess) return (int)err;
    }
    return 0;
}

}  // namespace gdn
