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
// One workgroup owns one (segment, v-head): it walks the segment's chunks in
// order with H resident in MFMA accumulators, split by V columns across its
// state waves (column j of H only ever mixes with column j of v, so the split
// is exact), while its preparation waves build the next chunk's operands
// (cumsum, K K^T, inverse, W, T diag(beta), P) on chip; W, U and S never touch
// HBM.  The exact context-parallel mode adds a pre-pass on the same chunk loop
// (per-segment S and transition map M) and a combine over segments.
//
// Precision (the pages' "restructure without losing precision", summarylog.com
// essay, "formula restructuring"): products of two exact bf16 inputs (K K^T,
// Q K^T) use one bf16 MFMA; operands that carry fp32 values which feed the
// output or the state with full weight are split into hi + lo bf16 pairs:
// T diag(beta), T diag(beta gamma), W, P, v', the decayed v', and H (in Q H
// only when o is fp32: a bf16 o takes Q times the bf16-rounded H, whose error
// stays below the output's own rounding and never reaches the state).  Decays and beta are fp32
// row/column scales; every exponent is a non-positive difference G_i - G_s
// (masked before the exp), so nothing overflows.
//
// MFMA shapes: v_mfma_f32_16x16x32_bf16 for the chunk loop's products
// (fragment layouts described with the kernel), v_mfma_f32_32x32x16_bf16 for
// K K^T and the combine (lane l holds A row / B column l % 32 with 8 k-slots
// for lane half l / 32; accumulator element 4i + j holds row 8i + 4(l / 32) + j,
// column l % 32).
#include <hip/hip_runtime.h>

#include <type_traits>

#include "gdn_internal.h"
#include "gdn_window.h"

namespace gdn {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int CH = kChunk;   // 64
constexpr int DK = kDimK;    // 128
constexpr int DV = kDimV;    // 128
constexpr int AS = CH + 4;   // fp32 row stride of the 64 x 64 A / T tile (16-byte aligned rows)

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const bf16 *p) {   // 16-byte LDS read
    return *reinterpret_cast<const bf16x8 *>(p);
}

// hi + lo bf16 split of fp32 values, two at a time: hi = RNE(x) for both in
// one packed conversion; float(hi) is the packed word shifted or masked (no
// unpacking conversion); lo = RNE(x - float(hi)) in a second packed conversion.
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2(float x0, float x1, uint32_t &hi, uint32_t &lo) {
    const bf16x2 h = {(bf16)x0, (bf16)x1};
    hi = __builtin_bit_cast(uint32_t, h);
    asm("" : "+v"(hi));  // keep the packed word: re-deriving each half costs an extra conversion
    const float h0 = __uint_as_float(hi << 16), h1 = __uint_as_float(hi & 0xffff0000u);
    const bf16x2 l = {(bf16)(x0 - h0), (bf16)(x1 - h1)};
    lo = __builtin_bit_cast(uint32_t, l);
}

__device__ __forceinline__ void split8v(const float *x, bf16x8 &hi, bf16x8 &lo) {
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) split2(x[2 * i], x[2 * i + 1], h[i], l[i]);
    hi = __builtin_bit_cast(bf16x8, (u32x4{h[0], h[1], h[2], h[3]}));
    lo = __builtin_bit_cast(bf16x8, (u32x4{l[0], l[1], l[2], l[3]}));
}

// ---------------------------------------------------------------- chunk loads
// Every chunk of a sequence is read (and its output written) through buffer
// resources that start at the chunk's first row and end at the chunk's last
// row inside the sequence, so rows past the sequence end come back as zeros
// and stores to them are dropped (hardware range check): a partial last chunk
// behaves as if padded with g = beta = 0, k = q = v = 0.  Offsets stay below
// 64 rows, whatever the sequence length.
struct Inputs {
    const char *k, *q, *v, *g, *b;       // this sequence's first row, this head
    unsigned kstride, vstride, gstride;  // bytes per token row
    int seq_len;
};

// A buffer resource over [base, base + bytes).  Every caller passes values that
// are the same in all lanes; taking them through readfirstlane lets the
// compiler keep the resource in scalar registers instead of looping over the
// distinct values of lanes it cannot prove equal.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int n = __builtin_amdgcn_readfirstlane((int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), (short)0, n,
                                             0x00020000);
}

// Resource over chunk c's rows of a per-sequence tensor (no rows past the end).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const void *base, unsigned stride, int c, int seq_len) {
    const int rows = min(max(seq_len - c * CH, 0), CH);
    return make_rsrc(static_cast<const char *>(base) + (int64_t)c * CH * stride, (int64_t)rows * stride);
}

// ---------------------------------------------------------------- XCD-aware work order
// The dispatcher hands workgroup b to XCD b % 8 (each XCD has its own L2).
// When the whole grid is resident at once (one workgroup per CU, at most one
// per CU), work item w = b % 8 * (n / 8) + b / 8 gives each XCD a contiguous
// range of work items, so the value heads of a key/query group (consecutive
// items) share one L2 for their q and k reads; blocks past the last full round
// of eight keep their own index (a bijection on [0, n)).  Larger grids run in
// rounds, in the order the planner's makespan model assumes (grid order), and
// keep it: remapped, the varlen workload ran 15 % slower.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_work_index(const int b, const int n) {
    if (n > kNumCUs) return b;
    const int per = n / kXcds;
    return b < per * kXcds ? (b % kXcds) * per + b / kXcds : b;
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

// ---------------------------------------------------------------- the forward kernel (8 waves)
// One workgroup of eight waves owns one (segment, v-head).  Waves 0..3, the
// state waves, hold the state: wave w has value columns 32 w .. 32 w + 31 as two
// column tiles of eight 16 x 16 accumulator tiles (v_mfma_f32_16x16x32_bf16:
// lane l holds A row / B column l % 16 with the 8 k-slots 8 (l / 16) .. +7;
// accumulator element j holds row 4 (l / 16) + j, column l % 16).  Two
// accumulator tiles stacked along k read as one B operand see, in a 32-wide k
// step, the k indices 4g..4g+3 and 16+4g..16+4g+3 (g = l / 16), which is also
// the order two transposing LDS reads (ds_read_b64_tr_b16) of 16 rows each
// deliver; every operand of such a k step uses that order.  Every A operand a
// state wave reads from LDS serves both of its column tiles, so each shared
// tile is read by four waves per chunk.  Waves 4..7, the preparation waves,
// hold no state: they load Q, V, g and beta of every chunk straight from HBM
// into LDS (the state waves load K) and run the chunk-local preparation of the
// next chunk (gate scan, K K^T, inverse, W, T diag(beta), P) in step with the
// state pass of the current one, one barrier-separated step at a time, at a
// raised wave priority: their chain of small dependent steps has the longer
// latency, and the state wave that shares their SIMD fills its stalls.
constexpr int NT8 = 512;
constexpr int TS8 = 32 + 4;    // fp32 row stride of the transposed 32 x 32 diagonal blocks
constexpr int TLD = DK + 8;    // bf16 row stride of the K, Q and V tiles: 272 bytes
constexpr int TSLOT = TLD / 8;  // 16-byte slots per tile row: 16 of data, 1 of padding
constexpr int TILE = CH * TLD;  // bf16 elements of one 64-token x 128 tile (K, Q and V alike)
constexpr int TLOADS = CH * TSLOT / 64;  // 1 KB wave loads per tile (17)
static_assert(CH * TSLOT % 64 == 0, "a tile is a whole number of wave loads");
static_assert(DK == DV, "K, Q and V tiles share one layout");

struct __attribute__((aligned(16))) Smem8 {
    bf16 k[2][TILE];                  // K by chunk parity (row = token, padded rows)
    bf16 q[TILE];                     // Q of the chunk being prepared
    bf16 v[TILE];                     // V of the chunk being prepared
    float a[CH * AS];                 // A, inverted in place into T
    bf16x8 tdf[2][6][64];             // diag(dec) T diag(beta) as A fragments [hi, lo][fragment][lane]
    bf16x8 zf[2][6][64];              // (scale P T diag(beta))^T as B fragments [hi, lo][fragment][lane]
    bf16x8 tf[2][6][64];              // T diag(beta) as A fragments (only when v' is stored)
    bf16x8 pf[2][6][64];              // (scale P)^T as B fragments [hi, lo][fragment][lane]
    // the two 32 x 32 diagonal blocks of A, then of T, transposed ([block][col][row])
    float tt[2][32 * TS8];
    float tlo[32 * TS8];              // rows 32..63, columns 0..31 of T (inverse level 2)
    float tlot[32 * TS8];             // the same block transposed ([col][row - 32])
    float gam[2][CH], dec[2][CH];     // e^{G}, e^{G_last - G} (two chunks in flight)
    float graw[2][CH], braw[2][CH];   // g and beta as loaded, by chunk parity
    float gcum[CH], bg[CH];
    float ep[CH], em[CH], rowa[CH];   // e^{G - G_31}, e^{G_31 - G}, beta e^{G - G_31}
};
static_assert(sizeof(Smem8) <= 160 * 1024, "one workgroup's LDS must fit a CU");

// The six 16-row x 32-column tiles of a 64 x 64 lower-triangular matrix that
// hold non-zeros: (row tile, k step) = (0,0) (1,0) (2,0) (3,0) (2,1) (3,1).
__device__ __forceinline__ int frag_rt(int f) { return f < 4 ? f : f - 2; }
__device__ __forceinline__ int frag_ks(int f) { return f < 4 ? 0 : 1; }
__device__ __forceinline__ int frag_of(int rt, int ks) { return ks == 0 ? rt : rt + 2; }
// k slot e of lane group g in the transposed-read order
__device__ __forceinline__ constexpr int kperm(int e, int g) { return (e & 3) + 4 * g + 16 * (e >> 2); }

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two stacked accumulator tiles as the hi and lo bf16 B operand of one k step.
__device__ __forceinline__ void split_pair(const f32x4 &t0, const f32x4 &t1, bf16x8 &hi, bf16x8 &lo) {
    const float x[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
    split8v(x, hi, lo);
}

// ---- 64 x 128 bf16 tiles in LDS with rows of 272 bytes (256 of data and one
// 16-byte pad slot): a row starts 4 banks after the previous one, so sixteen
// consecutive rows at one column (row-fragment reads, 16 bytes a lane) and
// sixteen rows at four column offsets (transposing or 8-byte reads) spread
// over all banks at the minimum number of LDS cycles, and every fragment read
// is a per-lane base address plus a constant offset.
__device__ __forceinline__ int tix(int r, int c) { return r * TLD + c; }

__device__ __forceinline__ bf16x4 tr4(const bf16 *p) {
    typedef short i16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    return __builtin_bit_cast(bf16x4, v);
}

// Fragment (r, k) = X[k0 + k][c0 + r] of a tile X (r = l % 16, k in the
// transposed-read order): lane l reads four columns of row k0 + l / 4 and of
// row k0 + 16 + l / 4, and each transposing read hands every lane its column.
__device__ __forceinline__ bf16x8 frag_t(const bf16 *X, const int c0, const int k0, const int lane) {
    const int r = k0 + (lane >> 2), c = c0 + 4 * (lane & 3);
    const bf16x4 x0 = tr4(X + tix(r, c)), x1 = tr4(X + tix(r + 16, c));
    return bf16x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
}

// Row fragment X[r0 + l % 16][k0 + 8 (l / 16) .. +7]
__device__ __forceinline__ bf16x8 frag_r(const bf16 *X, const int r0, const int k0, const int lane) {
    return lds8(X + tix(r0 + (lane & 15), k0 + 8 * (lane >> 4)));
}

// The same rows at the transposed-read k order: k0 + 4g .. +3, k0 + 16 + 4g .. +3
__device__ __forceinline__ bf16x8 frag_rp(const bf16 *X, const int r0, const int k0, const int lane) {
    const int r = r0 + (lane & 15), g = lane >> 4;
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(X + tix(r, k0 + 4 * g));
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(X + tix(r, k0 + 16 + 4 * g));
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---- direct HBM -> LDS loads (buffer_load ... lds: lane l of a wave writes
// LDS bytes 16 l .. 16 l + 15, or 4 l .. 4 l + 3, past the wave-uniform base).
// Rows beyond a chunk's buffer resource (past the sequence end) arrive as zeros.
typedef __attribute__((address_space(3))) void lds_void;

// The LDS address of a generic pointer into this workgroup's LDS: its low 32
// bits (the shared aperture sits in the high half).  Taken through integers
// rather than an address-space cast, whose null check this compiler can fold
// into an illegal compare against the aperture register.
__device__ __forceinline__ lds_void *lds_ptr(const void *p) {
    return (lds_void *)(uintptr_t)(uint32_t)(uintptr_t)p;
}

// Part `part` of PARTS of a tile: the wave issues loads part, part + PARTS, ...
// of the tile's 17.  Lane l of load i fills 16-byte slot 64 i + l of the
// padded tile, i.e. row (64 i + l) / 17 and piece (64 i + l) % 17; the pad
// piece takes an offset past any buffer and arrives as zeros.  The per-lane
// byte offsets depend only on the row stride, so each wave computes its share
// once and reuses it for every chunk.
template <int PARTS>
struct TileOffs {
    static constexpr int NI = (TLOADS + PARTS - 1) / PARTS;
    unsigned o[NI];
};

template <int PARTS>
__device__ __forceinline__ TileOffs<PARTS> tile_offsets(const unsigned stride, const int part, const int lane) {
    TileOffs<PARTS> t;
#pragma unroll
    for (int n = 0; n < TileOffs<PARTS>::NI; ++n) {
        const int slot = 64 * (part + n * PARTS) + lane;
        const int row = slot / TSLOT, piece = slot - TSLOT * row;
        t.o[n] = (piece < 16 && row < CH) ? (unsigned)row * stride + 16u * (unsigned)piece : 0x80000000u;
    }
    return t;
}

// Chunk c's tile through a buffer resource over the chunk's rows.
template <int PARTS>
__device__ __forceinline__ void dma_tile(bf16 *tile, const char *base, const unsigned stride, const int c,
                                         const int seq_len, const int part, const TileOffs<PARTS> &t) {
    const __amdgpu_buffer_rsrc_t r = chunk_rsrc(base, stride, c, seq_len);
#pragma unroll
    for (int n = 0; n < TileOffs<PARTS>::NI; ++n) {
        const int i = part + n * PARTS;
        if (i < TLOADS) __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(tile + 512 * i), 16, (int)t.o[n], 0, 0, 0);
    }
}

// g (preparation wave 0) and beta (wave 1) of chunk c, one token per lane.
__device__ __forceinline__ void dma_gb(Smem8 &s, const Inputs &in, const int c, const int pw, const int lane) {
    if (pw >= 2) return;
    const __amdgpu_buffer_rsrc_t r = chunk_rsrc(pw == 0 ? in.g : in.b, in.gstride, c, in.seq_len);
    float *dst = (pw == 0) ? s.graw[c & 1] : s.braw[c & 1];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(dst), 4, (int)((unsigned)lane * in.gstride), 0, 0, 0);
}

// This wave's direct loads have landed in LDS (vmcnt(0); other counters untouched).
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// All but this wave's N most recent vector memory operations have completed
// (vmcnt(N); they complete in issue order).
template <int N>
__device__ __forceinline__ void dma_wait_but() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}

// The same for a wave-uniform run-time N (0..15; larger waits for everything).
__device__ __forceinline__ void dma_wait_upto(const int n) {
    switch (n) {
#define GDN_WAIT_CASE(N) \
    case N: dma_wait_but<N>(); break;
        GDN_WAIT_CASE(1) GDN_WAIT_CASE(2) GDN_WAIT_CASE(3) GDN_WAIT_CASE(4) GDN_WAIT_CASE(5)
        GDN_WAIT_CASE(6) GDN_WAIT_CASE(7) GDN_WAIT_CASE(8) GDN_WAIT_CASE(9) GDN_WAIT_CASE(10)
        GDN_WAIT_CASE(11) GDN_WAIT_CASE(12) GDN_WAIT_CASE(13) GDN_WAIT_CASE(14) GDN_WAIT_CASE(15)
#undef GDN_WAIT_CASE
    default: dma_wait(); break;
    }
}

// Wave loads of one tile issued by preparation wave pw (loads pw, pw + 4, ... of 17).
__host__ __device__ constexpr int NTILE4(int pw) { return (TLOADS - pw + 3) / 4; }

// Workgroup barrier for LDS traffic: this wave's own LDS reads and writes are
// complete (lgkmcnt(0)) when it arrives, but its direct HBM -> LDS loads may
// still be in flight (a fenced barrier would wait for them too); the issuing
// wave waits for those itself (dma_wait) before the barrier that publishes
// them.  The memory clobber keeps the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Inclusive wave-wide prefix sum with DPP (row shifts inside each 16-lane row,
// then row broadcasts across rows).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}

// Permutation inside each quad of lanes (quad_perm control)
template <int CTRL>
__device__ __forceinline__ float quad_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}

__device__ __forceinline__ float wave_prefix_sum(float x) {
    x += dpp_f<0x111, 0xf>(x);  // row_shr:1
    x += dpp_f<0x112, 0xf>(x);  // row_shr:2
    x += dpp_f<0x114, 0xf>(x);  // row_shr:4
    x += dpp_f<0x118, 0xf>(x);  // row_shr:8
    x += dpp_f<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
    x += dpp_f<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// ---- preparation step 1 (waves 4..7, pw = wave - 4): the chunk's gate scan
// and decay factors (every preparation wave forms them itself, lane = token,
// and writes identical values to the shared arrays; each reads back only what
// it wrote, so no barrier separates the scan from the products), then for
// pw 0..2 one masked, beta-weighted K K^T 32 x 32 tile each ((0,0) (1,0)
// (1,1)) into s.a, the diagonal ones also transposed into s.tt.
__device__ __forceinline__ void prod9(Smem8 &s, const int lane, const int pw, const int buf) {
    const int m32 = lane & 31, h32 = lane >> 5;
    bool fact;
    {
        const float x = wave_prefix_sum(s.graw[buf][lane]);
        const float glast = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
        const float gref = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
        const float gm = __expf(x);
        const float d = x - gref;
        const float bt = s.braw[buf][lane];
        const float epv = __expf(d);
        s.gcum[lane] = x;
        s.gam[buf][lane] = gm;
        s.dec[buf][lane] = __expf(glast - x);
        s.bg[lane] = bt * gm;
        s.ep[lane] = epv;
        s.em[lane] = __expf(-d);
        s.rowa[lane] = bt * epv;
        fact = __all(fabsf(d) < 80.f);  // the factored decays are finite
    }
    if (pw >= 3) return;
    const bf16 *K = s.k[buf];
    const int rbi = (pw >= 1) ? 1 : 0, rbs = (pw == 2) ? 1 : 0;
    f32x16 acck = {};
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
        bf16x8 xa[4], xb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int col = 8 * h32 + 16 * (4 * k2 + kk);
            xa[kk] = lds8(K + tix(32 * rbi + m32, col));
            xb[kk] = lds8(K + tix(32 * rbs + m32, col));
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the batch of reads ahead of its products
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acck = mfma(xa[kk], xb[kk], acck);
    }
    const int col = 32 * rbs + m32;
    float v[16];
    if (fact) {
        const float cf = s.em[col];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const f32x4 ra4 = *reinterpret_cast<const f32x4 *>(&s.rowa[32 * rbi + 8 * ii + 4 * h32]);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * ii + j] = ra4[j] * cf * acck[4 * ii + j];
        }
    } else {
        const float gs = s.gcum[col];
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
            const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&s.gcum[32 * rbi + 8 * ii + 4 * h32]);
            const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&s.braw[buf][32 * rbi + 8 * ii + 4 * h32]);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[4 * ii + j] = b4[j] * __expf(g4[j] - gs) * acck[4 * ii + j];
        }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int row = 32 * rbi + 8 * (e >> 2) + 4 * h32 + (e & 3);
        v[e] = (col < row) ? v[e] : 0.f;
        s.a[row * AS + col] = v[e];
    }
    if (rbi == rbs) {  // diagonal 32 x 32 block: also store it transposed
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
            *reinterpret_cast<f32x4 *>(&s.tt[rbi][m32 * TS8 + 8 * ii + 4 * h32]) =
                f32x4{v[4 * ii], v[4 * ii + 1], v[4 * ii + 2], v[4 * ii + 3]};
    }
}

// ---- preparation: scale * P, causal and decayed, as the hi/lo A fragment f
// of its non-zero 16 x 16 tiles.  A P fragment (rt, ks) stacks the P^T = K Q^T
// tiles (s tile 2 ks, i tile rt) and (2 ks + 1, rt); the accumulator of each
// tile is the fragment half.  Written once the state pass has consumed the
// previous chunk's P.
__device__ __forceinline__ bool decays_factor(const Smem8 &s, const int lane) {
    return __all(fabsf(s.gcum[lane] - s.gcum[31]) < 80.f);  // as in the gate scan
}

__device__ __forceinline__ void pfrag9(Smem8 &s, const int lane, const int f, const int buf, const float scale,
                                       const bool fact) {
    const int m = lane & 15, g = lane >> 4;
    const bf16 *K = s.k[buf], *Q = s.q;
    const int rt = frag_rt(f), ks = frag_ks(f);
    f32x4 accp[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int st = 2 * ks + half;
        if (st > rt) continue;  // tile entirely above the diagonal
        bf16x8 xa[4], xb[4];
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            xa[kk] = frag_r(K, 16 * st, 32 * kk, lane);
            xb[kk] = frag_r(Q, 16 * rt, 32 * kk, lane);
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the batch of reads ahead of its products
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) accp[half] = mfma16(xa[kk], xb[kk], accp[half]);
    }
    const int i = 16 * rt + m;  // this lane's query row
    float pv[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const int s0 = 32 * ks + 16 * half + 4 * g;  // key rows of this lane's 4 slots
        if (fact) {
            const float cf = scale * s.ep[i];
            const f32x4 e4 = *reinterpret_cast<const f32x4 *>(&s.em[s0]);
#pragma unroll
            for (int j = 0; j < 4; ++j) pv[4 * half + j] = (s0 + j <= i) ? cf * e4[j] * accp[half][j] : 0.f;
        } else {
            const float gi = s.gcum[i];
            const f32x4 g4 = *reinterpret_cast<const f32x4 *>(&s.gcum[s0]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                pv[4 * half + j] = (s0 + j <= i) ? scale * __expf(gi - g4[j]) * accp[half][j] : 0.f;
        }
    }
    bf16x8 hi, lo;
    split8v(pv, hi, lo);
    s.pf[0][f][lane] = hi;
    s.pf[1][f][lane] = lo;
}
// ---- T = (I + A)^{-1} in place in s.a (row-major), with the diagonal 32 x 32
// blocks also kept transposed in s.tt for the merges.
// Level 0 (preparation wave pw: diagonal 16 x 16 block pw): forward
// substitution with lane = 4 c + p; the four lanes of column c split each
// row's dot product over s = p mod 4 and add it with two DPP steps.
__device__ __forceinline__ void inv8_l0(Smem8 &s, const int lane, const int pw) {
    const int c = lane >> 2, p = lane & 3;
    const int bo = 16 * (pw & 1);
    float *tb = s.tt[pw >> 1];  // block pw sits in s.tt[pw / 2] at offset 16 (pw % 2) on both axes
    // this lane's coefficients A[i][p + 4e] for all rows i: rows p + 4e of A^T
    float ac[4][16];
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 x = *reinterpret_cast<const f32x4 *>(&tb[(bo + p + 4 * e4) * TS8 + bo + 4 * q4]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) ac[e4][4 * q4 + jj] = x[jj];
        }
    float t[4] = {0.f, 0.f, 0.f, 0.f};  // T[p + 4 e][c]
#pragma unroll
    for (int ii = 0; ii < 16; ++ii) {
        float part = 0.f;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4)
            if (p + 4 * e4 < ii) part += ac[e4][ii] * t[e4];  // (p + 4 e4 < ii) is lane-dependent
        part += quad_dpp<0xb1>(part);  // quad_perm [1,0,3,2]
        part += quad_dpp<0x4e>(part);  // quad_perm [2,3,0,1]
        const float tv = ((ii == c) ? 1.f : 0.f) - part;
        if (p == (ii & 3)) t[ii >> 2] = tv;
    }
    const int o = 16 * pw;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
        s.a[(o + p + 4 * e4) * AS + o + c] = t[e4];
        tb[(bo + c) * TS8 + bo + p + 4 * e4] = t[e4];
    }
}

// Level 1 (preparation waves 0 and 1, diagonal 32 x 32 block blk):
// T_10 = -T_11 (A_10 T_00), two chained 16 x 16 MFMA products (hi/lo).
__device__ __forceinline__ void inv8_l1(Smem8 &s, const int lane, const int blk) {
    const int m = lane & 15, g = lane >> 4;
    const int b = 32 * blk;
    float *tb = s.tt[blk];
    float av[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (g < 2) {  // k = 0..15 on lane groups 0, 1; groups 2, 3 carry zeros
        const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&s.a[(b + 16 + m) * AS + b + 8 * g]);
        const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&s.a[(b + 16 + m) * AS + b + 8 * g + 4]);
        const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&tb[m * TS8 + 8 * g]);  // T_00[k][m]
        const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&tb[m * TS8 + 8 * g + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            av[e] = a0[e];
            av[4 + e] = a1[e];
            bv[e] = b0[e];
            bv[4 + e] = b1[e];
        }
    }
    bf16x8 ah, al, bh, bl;
    split8v(av, ah, al);
    split8v(bv, bh, bl);
    f32x4 x = {};
    x = mfma16(ah, bh, x);
    x = mfma16(ah, bl, x);
    x = mfma16(al, bh, x);
    // T_11 X: X (rows 4 g + j) is the first half of the B operand's k order,
    // the second half is zero
    const f32x4 t4 = *reinterpret_cast<const f32x4 *>(&s.a[(b + 16 + m) * AS + b + 16 + 4 * g]);
    const float tvv[8] = {t4[0], t4[1], t4[2], t4[3], 0.f, 0.f, 0.f, 0.f};
    const float xv[8] = {x[0], x[1], x[2], x[3], 0.f, 0.f, 0.f, 0.f};
    split8v(tvv, ah, al);
    split8v(xv, bh, bl);
    f32x4 z = {};
    z = mfma16(ah, bh, z);
    z = mfma16(ah, bl, z);
    z = mfma16(al, bh, z);
#pragma unroll
    for (int j = 0; j < 4; ++j) s.a[(b + 16 + 4 * g + j) * AS + b + m] = -z[j];
    *reinterpret_cast<f32x4 *>(&tb[m * TS8 + 16 + 4 * g]) = f32x4{-z[0], -z[1], -z[2], -z[3]};
}

// Level 2 (all four preparation waves, one 16 x 16 quadrant (r, cq) of the
// lower-left 32 x 32 block each, pw = 2 r + cq):
//   T_lo,hi = -T_lo,lo (A_lo,hi T_hi,hi)
// Part a reads every operand (Y = A_lo,hi T_hi,hi[:, 16 cq ..] as two 16 x 16
// tiles, and the T_lo,lo rows of this quadrant); part b writes the quadrant to
// s.tlo, not over A_lo,hi, which the other waves' part a may still be reading,
// so both parts run in one step.
struct L2Regs {
    f32x4 y0, y1;
    bf16x8 th, tl;
};

__device__ __forceinline__ void inv8_l2a(const Smem8 &s, const int lane, const int pw, L2Regs &r2) {
    const int m = lane & 15, g = lane >> 4;
    const int r = pw >> 1, cq = pw & 1;
    float bv[8];
    {
        const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&s.tt[0][(16 * cq + m) * TS8 + 8 * g]);  // T_hi,hi[k][16 cq + m]
        const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&s.tt[0][(16 * cq + m) * TS8 + 8 * g + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bv[e] = b0[e];
            bv[4 + e] = b1[e];
        }
    }
    bf16x8 bh, bl;
    split8v(bv, bh, bl);
    f32x4 y[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const f32x4 a0 = *reinterpret_cast<const f32x4 *>(&s.a[(32 + 16 * i + m) * AS + 8 * g]);
        const f32x4 a1 = *reinterpret_cast<const f32x4 *>(&s.a[(32 + 16 * i + m) * AS + 8 * g + 4]);
        const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
        bf16x8 ah, al;
        split8v(av, ah, al);
        y[i] = f32x4{};
        y[i] = mfma16(ah, bh, y[i]);
        y[i] = mfma16(ah, bl, y[i]);
        y[i] = mfma16(al, bh, y[i]);
    }
    r2.y0 = y[0];
    r2.y1 = y[1];
    // T_lo,lo row 16 r + m at the k order of split_pair(y0, y1)
    const f32x4 t0 = *reinterpret_cast<const f32x4 *>(&s.a[(32 + 16 * r + m) * AS + 32 + 4 * g]);
    const f32x4 t1 = *reinterpret_cast<const f32x4 *>(&s.a[(32 + 16 * r + m) * AS + 48 + 4 * g]);
    const float tv[8] = {t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
    split8v(tv, r2.th, r2.tl);
}

__device__ __forceinline__ void inv8_l2b(Smem8 &s, const int lane, const int pw, const L2Regs &r2) {
    const int m = lane & 15, g = lane >> 4;
    const int r = pw >> 1, cq = pw & 1;
    bf16x8 yh, yl;
    split_pair(r2.y0, r2.y1, yh, yl);
    f32x4 z = {};
    z = mfma16(r2.th, yh, z);
    z = mfma16(r2.th, yl, z);
    z = mfma16(r2.tl, yh, z);
#pragma unroll
    for (int j = 0; j < 4; ++j) s.tlo[(16 * r + 4 * g + j) * TS8 + 16 * cq + m] = -z[j];
    *reinterpret_cast<f32x4 *>(&s.tlot[(16 * cq + m) * TS8 + 16 * r + 4 * g]) = f32x4{-z[0], -z[1], -z[2], -z[3]};
}

// Four consecutive entries T[row][c0 .. c0 + 3] (c0 a multiple of 4): the
// lower-left 32 x 32 block of T sits in s.tlo, the rest in s.a.
__device__ __forceinline__ f32x4 trow4(const Smem8 &s, const int row, const int c0) {
    const float *p = (row >= 32 && c0 < 32) ? &s.tlo[(row - 32) * TS8 + c0] : &s.a[row * AS + c0];
    return *reinterpret_cast<const f32x4 *>(p);
}

// ---- preparation: fragment f of the chunk's WY matrix as MFMA A fragments
// (rows i = 16 rt + l % 16, k = tokens s of token step ks in the
// transposed-read order), hi / lo:
//   s.tdf  diag(dec) T diag(beta)   (the decayed v' of the state update)
//   s.tf   T diag(beta)             (v' itself, only when v' is stored)
// Rows 0..31 of T are final after inverse level 1, rows 32..63 after level 2.
__device__ __forceinline__ void tdfrag(Smem8 &s, const int lane, const int f, const int buf, const bool with_tf,
                                       const bool with_td = true) {
    const int m = lane & 15, g = lane >> 4;
    const int rt = frag_rt(f), ks = frag_ks(f);
    const int c0 = 32 * ks + 4 * g, row = 16 * rt + m;
    const f32x4 t0 = trow4(s, row, c0), t1 = trow4(s, row, c0 + 16);
    const f32x4 b0 = *reinterpret_cast<const f32x4 *>(&s.braw[buf][c0]);
    const f32x4 b1 = *reinterpret_cast<const f32x4 *>(&s.braw[buf][c0 + 16]);
    const float d = s.dec[buf][row];
    float tb[8], td[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        tb[e] = t0[e] * b0[e];
        tb[4 + e] = t1[e] * b1[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) td[e] = d * tb[e];
    bf16x8 hi, lo;
    if (with_td) {
        split8v(td, hi, lo);
        s.tdf[0][f][lane] = hi;
        s.tdf[1][f][lane] = lo;
    }
    if (with_tf) {
        split8v(tb, hi, lo);
        s.tf[0][f][lane] = hi;
        s.tf[1][f][lane] = lo;
    }
}

// ---- preparation: Z^T = (scale P T diag(beta))^T as the hi / lo B fragment f
// of the output product O^T = ... + Y^T Z^T (k = tokens s of token step ks in
// the transposed-read order, columns = query rows i of tile rt).  P v' = P T
// diag(beta) Y, so the output takes the same Y as the state update instead of
// v'.  Each of the fragment's two 16-token tiles st is the MFMA product of
// (T diag(beta))^T (rows s, k = s') and the (scale P)^T fragments (k = s',
// columns i) over the token steps s' between s and i (both factors are
// triangular), hi / lo on both sides.  The columns of T come from its
// transposed blocks (s.tt diagonal blocks, s.tlot lower-left block).  The
// token steps KQ0 <= kq <= KQ1 of the sum are added to acc; zstore splits the
// two tiles and stores the fragment.
template <int KQ0, int KQ1>
__device__ __forceinline__ void zsum(const Smem8 &s, const int lane, const int f, const int buf, f32x4 (&acc)[2]) {
    const int m = lane & 15, g = lane >> 4;
    const int rt = frag_rt(f), ks = frag_ks(f);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int st = 2 * ks + h;  // token tile of the rows s
        if (st > rt) continue;      // above the diagonal: zero
        const int sr = 16 * st + m;
        const float bs = s.braw[buf][sr];
#pragma unroll
        for (int kq = KQ0; kq <= KQ1; ++kq) {
            if (kq < ks || kq > (rt >> 1)) continue;
            const float *src = (kq == 0) ? &s.tt[0][sr * TS8]
                               : (st >= 2) ? &s.tt[1][(sr - 32) * TS8]
                                           : &s.tlot[sr * TS8];
            const f32x4 x0 = *reinterpret_cast<const f32x4 *>(src + 4 * g);
            const f32x4 x1 = *reinterpret_cast<const f32x4 *>(src + 16 + 4 * g);
            const float av[8] = {x0[0] * bs, x0[1] * bs, x0[2] * bs, x0[3] * bs,
                                 x1[0] * bs, x1[1] * bs, x1[2] * bs, x1[3] * bs};
            bf16x8 ah, al;
            split8v(av, ah, al);
            const int pfr = frag_of(rt, kq);
            const bf16x8 ph = s.pf[0][pfr][lane], pl = s.pf[1][pfr][lane];
            acc[h] = mfma16(ah, ph, acc[h]);
            acc[h] = mfma16(ah, pl, acc[h]);
            acc[h] = mfma16(al, ph, acc[h]);
        }
    }
}

__device__ __forceinline__ void zstore(Smem8 &s, const int lane, const int f, const f32x4 (&acc)[2]) {
    bf16x8 hi, lo;
    split_pair(acc[0], acc[1], hi, lo);
    s.zf[0][f][lane] = hi;
    s.zf[1][f][lane] = lo;
}

// ---- state-wave pieces, two column tiles each.  Y = V - diag(gamma) K H of
// a chunk (tokens x this wave's 32 value columns) is held as hi / lo bf16
// pairs [token step ks][column tile ct]: a pair is the B operand of a product
// over tokens (k = tokens in the transposed-read order, columns = value
// columns) and, as the same registers, the A operand of the transposed one
// (rows = value columns, k = tokens).
struct YSplit {
    bf16x8 h[2][2], l[2][2];
};

__device__ __forceinline__ void zero_tiles(f32x4 (&t)[4][2]) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) t[rt][ct] = f32x4{};
}

// X = K H for the chunk in buffers nb (token rows x this wave's value
// columns), from one hi / lo split of the state per k step; the K fragments of
// the next k step are read while the current one's products run.
__device__ __forceinline__ void xk(const Smem8 &s, const f32x4 (&hacc)[2][8], f32x4 (&X)[4][2], const int nb,
                                   const int ln) {
    const bf16 *K = s.k[nb];
    zero_tiles(X);
    bf16x8 ka[2][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) ka[0][rt] = frag_rp(K, 16 * rt, 0, ln);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int b = kk & 1;
        if (kk + 1 < 4) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) ka[b ^ 1][rt] = frag_rp(K, 16 * rt, 32 * (kk + 1), ln);
        }
        __builtin_amdgcn_sched_barrier(0);  // the next step's reads go out ahead of this step's products
        bf16x8 hh[2], hl[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) split_pair(hacc[ct][2 * kk], hacc[ct][2 * kk + 1], hh[ct], hl[ct]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                X[rt][ct] = mfma16(ka[b][rt], hh[ct], X[rt][ct]);
                X[rt][ct] = mfma16(ka[b][rt], hl[ct], X[rt][ct]);
            }
    }
}

// The state term of the output of the chunk in buffers nb,
// qh = (scale diag(gamma) Q H)^T (this wave's value columns x query rows): H
// as the A operand (its bf16 rounding alone for bf16 o: that term reaches only
// o, whose own rounding is the larger error; hi + lo for fp32 o), the Q
// fragments as B operands, read one k step ahead.  Lane (m, g) of tile
// (rt, ct) ends up holding value columns 16 ct + 4 g .. +3 of query row 16 rt + m.
template <bool OF32>
__device__ __forceinline__ void qhq(const Smem8 &s, const f32x4 (&hacc)[2][8], f32x4 (&qh)[4][2], const int nb,
                                    const float scale, const int ln) {
    const int m = ln & 15;
    const bf16 *Q = s.q;
    zero_tiles(qh);
    bf16x8 qa[2][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) qa[0][rt] = frag_rp(Q, 16 * rt, 0, ln);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int b = kk & 1;
        if (kk + 1 < 4) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) qa[b ^ 1][rt] = frag_rp(Q, 16 * rt, 32 * (kk + 1), ln);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const f32x4 &t0 = hacc[ct][2 * kk], &t1 = hacc[ct][2 * kk + 1];
            bf16x8 hh, hl;
            if (OF32) {
                split_pair(t0, t1, hh, hl);
            } else {
                hh = bf16x8{(bf16)t0[0], (bf16)t0[1], (bf16)t0[2], (bf16)t0[3],
                            (bf16)t1[0], (bf16)t1[1], (bf16)t1[2], (bf16)t1[3]};
            }
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                qh[rt][ct] = mfma16(hh, qa[b][rt], qh[rt][ct]);
                if (OF32) qh[rt][ct] = mfma16(hl, qa[b][rt], qh[rt][ct]);
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const float f = scale * s.gam[nb][16 * rt + m];  // this lane's query row
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) qh[rt][ct] *= f;
    }
}

// Y = V - diag(gamma) X of the chunk in buffers nb (the transition-map pass
// has no V: Y = -diag(gamma) X), as hi / lo pairs.  V comes from transposing
// reads of its tile, which hand each lane the rows of its X elements.
__device__ __forceinline__ void yform(const Smem8 &s, const f32x4 (&X)[4][2], YSplit &y, const bool with_v, const int sw,
                                      const int nb, const int ln) {
    const int g = ln >> 4;
    bf16x8 vv[2][2];  // [token step][column tile]
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
            vv[ks][ct] = with_v ? frag_t(s.v, 32 * sw + 16 * ct, 32 * ks, ln) : bf16x8{};
    f32x4 gm[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) gm[rt] = *reinterpret_cast<const f32x4 *>(&s.gam[nb][16 * rt + 4 * g]);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            float yv[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                yv[e] = (float)vv[ks][ct][e] - gm[2 * ks][e] * X[2 * ks][ct][e];
                yv[4 + e] = (float)vv[ks][ct][4 + e] - gm[2 * ks + 1][e] * X[2 * ks + 1][ct][e];
            }
            split8v(yv, y.h[ks][ct], y.l[ks][ct]);
        }
}

// vd = F Y for the hi / lo A fragments F of s.tdf (DECAYED: diag(dec) T
// diag(beta), the decayed v') or s.tf (T diag(beta), v' itself).
__device__ __forceinline__ void tdy(const Smem8 &s, const bool decayed, const YSplit &y, f32x4 (&vd)[4][2],
                                    const int ln) {
    bf16x8 th[6], tl[6];
#pragma unroll
    for (int f = 0; f < 6; ++f) {
        th[f] = decayed ? s.tdf[0][f][ln] : s.tf[0][f][ln];
        tl[f] = decayed ? s.tdf[1][f][ln] : s.tf[1][f][ln];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the batch of reads ahead of its products
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) vd[rt][ct] = f32x4{};
#pragma unroll
    for (int f = 0; f < 6; ++f) {
        const int rt = frag_rt(f), ks = frag_ks(f);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            vd[rt][ct] = mfma16(th[f], y.h[ks][ct], vd[rt][ct]);
            vd[rt][ct] = mfma16(th[f], y.l[ks][ct], vd[rt][ct]);
            vd[rt][ct] = mfma16(tl[f], y.h[ks][ct], vd[rt][ct]);
        }
    }
}

// Step 1 of a chunk's state pass, one loop over the six non-zero fragments
// f = (row tile rt, token step ks), each read one fragment ahead:
//   O^T = (scale diag(gamma) Q H)^T + Y^T Z^T for the two column tiles
//        (acc enters holding the first term; the Y pairs are the A operands,
//        the Z^T fragments the B operands), then stored: lane (m, g) holds value
//        columns 16 ct + 4 g .. +3 of query row 16 rt + m, one 16-byte (fp32) or
//        8-byte (bf16) piece through a buffer resource over the chunk's rows
//        (rows past the sequence end are dropped by the hardware range check),
//        when STORE (a warm-up chunk computes it and stores nothing: one copy
//        of this code in the loop allocates registers without spilling, two
//        copies did not);
//   vd = diag(dec) T diag(beta) Y, the decayed v' of the state update (the
//        fragments of s.tdf as A operands, the Y pairs as B operands).
template <bool OF32>
__device__ __forceinline__ void out_vd(const Smem8 &s, const FwdParams &p, const char *obase, const int seq_len,
                                       const YSplit &y, f32x4 (&acc)[4][2], f32x4 (&vd)[4][2], const bool store,
                                       const int c, const int sw, const int ln) {
    const int m = ln & 15, g = ln >> 4;
    zero_tiles(vd);
    bf16x8 zr[2][2], tr[2][2];  // [fragment parity][hi, lo]
    zr[0][0] = s.zf[0][0][ln];
    zr[0][1] = s.zf[1][0][ln];
    tr[0][0] = s.tdf[0][0][ln];
    tr[0][1] = s.tdf[1][0][ln];
#pragma unroll
    for (int f = 0; f < 6; ++f) {
        const int b = f & 1;
        if (f + 1 < 6) {
            zr[b ^ 1][0] = s.zf[0][f + 1][ln];
            zr[b ^ 1][1] = s.zf[1][f + 1][ln];
            tr[b ^ 1][0] = s.tdf[0][f + 1][ln];
            tr[b ^ 1][1] = s.tdf[1][f + 1][ln];
        }
        // the next fragment's reads go out ahead of this one's products, and
        // no further (registers)
        __builtin_amdgcn_sched_barrier(0);
        const int rt = frag_rt(f), ks = frag_ks(f);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            acc[rt][ct] = mfma16(y.h[ks][ct], zr[b][0], acc[rt][ct]);
            acc[rt][ct] = mfma16(y.l[ks][ct], zr[b][0], acc[rt][ct]);
            acc[rt][ct] = mfma16(y.h[ks][ct], zr[b][1], acc[rt][ct]);
            vd[rt][ct] = mfma16(tr[b][0], y.h[ks][ct], vd[rt][ct]);
            vd[rt][ct] = mfma16(tr[b][0], y.l[ks][ct], vd[rt][ct]);
            vd[rt][ct] = mfma16(tr[b][1], y.h[ks][ct], vd[rt][ct]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if (!store) return;
    const unsigned es = OF32 ? 4u : 2u;
    const unsigned rstride = (unsigned)p.Hv * DV * es;
    const __amdgpu_buffer_rsrc_t ro = chunk_rsrc(obase, rstride, c, seq_len);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const f32x4 w = acc[rt][ct];
            const unsigned off = (unsigned)(16 * rt + m) * rstride + (unsigned)(32 * sw + 16 * ct + 4 * g) * es;
            if (OF32) {
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), ro, (int)off, 0, 0);
            } else {
                const bf16x4 h = {(bf16)w[0], (bf16)w[1], (bf16)w[2], (bf16)w[3]};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), ro, (int)off, 0, 0);
            }
        }
}

// H <- gamma_last H + K^T vd, vd = diag(gamma_last / gamma) v' (as hi / lo).
// LEAN reads the K^T fragments four at a time (the transition-map pass runs
// three waves per SIMD and has fewer registers).
template <bool LEAN>
__device__ __forceinline__ void upd(const Smem8 &s, f32x4 (&hacc)[2][8], const f32x4 (&vd)[4][2], const int buf,
                                    const int ln) {
    const bf16 *K = s.k[buf];
    const float glast = s.gam[buf][CH - 1];
    if (!LEAN) {
        bf16x8 ka[2][8];  // [token step][key-dim tile]
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) ka[ks][dt] = frag_t(K, 16 * dt, 32 * ks, ln);
        __builtin_amdgcn_sched_barrier(0);  // keep the batch of reads ahead of its products
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) hacc[ct][dt] *= glast;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 vh[2], vl[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) split_pair(vd[2 * ks][ct], vd[2 * ks + 1][ct], vh[ct], vl[ct]);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    hacc[ct][dt] = mfma16(ka[ks][dt], vh[ct], hacc[ct][dt]);
                    hacc[ct][dt] = mfma16(ka[ks][dt], vl[ct], hacc[ct][dt]);
                }
        }
    } else {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) hacc[ct][dt] *= glast;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 vh[2], vl[2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) split_pair(vd[2 * ks][ct], vd[2 * ks + 1][ct], vh[ct], vl[ct]);
#pragma unroll
            for (int d4i = 0; d4i < 2; ++d4i) {
                bf16x8 ka[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) ka[d] = frag_t(K, 16 * (4 * d4i + d), 32 * ks, ln);
#pragma unroll
                for (int d = 0; d < 4; ++d)
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        hacc[ct][4 * d4i + d] = mfma16(ka[d], vh[ct], hacc[ct][4 * d4i + d]);
                        hacc[ct][4 * d4i + d] = mfma16(ka[d], vl[ct], hacc[ct][4 * d4i + d]);
                    }
            }
        }
    }
}

// ---- low-level outputs
// First global chunk index of sequence n (chunks of all sequences in order).
__device__ __forceinline__ int seq_chunk_base(const FwdParams &p, int n, int lane) {
    if (!p.cu) return n * seq_chunks(p.T);
    int base = 0;
    for (int n0 = 0; n0 < n; n0 += 64) {
        const int nn = n0 + lane;
        int cnt = (nn < n) ? seq_chunks((int64_t)p.cu[nn + 1] - p.cu[nn]) : 0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
        base += __builtin_amdgcn_readfirstlane(cnt);
    }
    return base;
}

// One chunk's WY matrix T (s.a, complete) as rows of A: preparation wave pw,
// thread t = 64 pw + lane stores row t / 4, columns 16 (t % 4) .. +15.  The
// upper-right 32 x 32 block of s.a is never written by the inverse; its zeros
// are supplied here.  Rows past the sequence end fall outside the chunk's
// buffer resource and are dropped.
__device__ __forceinline__ void store_t8(const Smem8 &s, const FwdParams &p, const char *abase, const int seq_len,
                                         const int c, const int pw, const int lane) {
    const int t = 64 * pw + lane;
    const int row = t >> 2, c0 = 16 * (t & 3);
    const unsigned rstride = (unsigned)p.Hv * CH * 4u;
    const __amdgpu_buffer_rsrc_t ra = chunk_rsrc(abase, rstride, c, seq_len);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int col = c0 + 4 * i;
        f32x4 x = trow4(s, row, col);
        if (row < 32 && col >= 32) x = f32x4{};
        const unsigned off = (unsigned)row * rstride + (unsigned)col * 4u;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), ra, (int)off, 0, 0);
    }
}

// v' of one chunk (all 64 rows, chunk-padded) from state wave sw's registers:
// vp[rt][ct] element jj is row 16 rt + 4 (l / 16) + jj, value column
// 32 sw + 16 ct + l % 16.
__device__ __forceinline__ void store_vn8(const f32x4 (&vp)[4][2], float *dst, const int sw, const int lane) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dst[(16 * rt + 4 * g + jj) * DV + 32 * sw + 16 * ct + m] = vp[rt][ct][jj];
}

// ---- state I/O: K x V fp32 state <-> state wave sw's two column tiles
__device__ __forceinline__ void load_state8(f32x4 (&t)[2][8], const float *src, const int sw, const int lane) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const float *b = src + 32 * sw + 16 * ct + m;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) t[ct][dt][j] = b[(16 * dt + 4 * g + j) * DV];
    }
}

__device__ __forceinline__ void store_state8(const f32x4 (&t)[2][8], float *dst, const int sw, const int lane) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        float *b = dst + 32 * sw + 16 * ct + m;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) b[(16 * dt + 4 * g + j) * DV] = t[ct][dt][j];
    }
}

// The chunk loop of one (segment, v-head).  PRE = false: the forward proper
// (4 state waves, 4 preparation waves).  PRE = true: the exact-CP pre-pass
// (blog, AutoCP: the per-segment M and S) for a segment that does not end its
// sequence -- waves 0..3 run the state pass from a zero state (S), waves 4..7
// the same pass without inputs (U = 0) from the identity (M, the product of the
// chunk maps X -> gamma_last X - K^T diag(gamma_last / gamma) W X; K = V, so M
// has the state's shape), both on the chunk operands the preparation waves
// 8..11 build once; no output, no warm-up.  The segment's end state is then
// M H_start + S.
template <bool PRE, bool OF32>
__device__ __forceinline__ void fwd_pass(const FwdParams &p) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    Smem8 &s = *reinterpret_cast<Smem8 *>(smem_raw);
    constexpr int NSTATE = PRE ? 8 : 4;  // state waves

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const bool state_wave = wave < NSTATE;  // the first NSTATE waves hold states, the rest prepare chunks
    const int sw = PRE ? (wave & 3) : wave;  // column block of a state wave
    const bool mwave = PRE && wave >= 4 && wave < 8;  // pre-pass: this wave carries M
    const int wid = xcd_work_index(blockIdx.x, gridDim.x);
    const int seg = wid / p.Hv;
    const int j = wid % p.Hv;
    if (seg >= p.num_segments) return;
    const SegEntry e = find_segment(p, seg, lane);
    if (e.n < 0) return;  // beyond the planned segments: nothing to do
    if (PRE && e.last) return;  // a last segment's map is never used
    const int i_qk = j / p.group;

    // ---- where this segment's state pass starts
    int c_first = e.c_begin;
    bool from_h0 = (e.c_begin == 0);
    if (!PRE && !from_h0 && p.cp_mode == 2 /* WARMUP */) {
        // gate-driven window: back from the segment start until the summed
        // log-gates reach the fp32 noise floor, or to the sequence start (then
        // the walk begins from the initial state and is exact)
        const int w = gate_window(p.g + e.row0 * p.Hv, p.Hv, j, e.seq_len, e.c_begin - 1, -1, e.c_begin,
                                  p.warmup_cap, lane);
        c_first = __builtin_amdgcn_readfirstlane(e.c_begin - w);
        from_h0 = (c_first == 0);
    }
    const int c_end = e.c_begin + e.c_count;

    const bool has_chunks = c_first < c_end;  // wave-uniform and equal across the workgroup
    if (!has_chunks && !(!PRE && state_wave && e.last && p.ht)) return;

    Inputs in;
    in.kstride = (unsigned)p.Hqk * DK * 2;
    in.vstride = (unsigned)p.Hv * DV * 2;
    in.gstride = (unsigned)p.Hv * 4;
    in.k = reinterpret_cast<const char *>(p.k + (e.row0 * p.Hqk + i_qk) * DK);
    in.q = reinterpret_cast<const char *>(p.q + (e.row0 * p.Hqk + i_qk) * DK);
    in.v = reinterpret_cast<const char *>(p.v + (e.row0 * p.Hv + j) * DV);
    in.g = reinterpret_cast<const char *>(p.g + e.row0 * p.Hv + j);
    in.b = reinterpret_cast<const char *>(p.beta + e.row0 * p.Hv + j);
    in.seq_len = e.seq_len;

    // Iteration c runs the state pass of chunk c (state waves) in step with the
    // preparation of chunk c + 1 (preparation waves); c = c_first - 1 only
    // prepares the first chunk.  With Y = V - diag(gamma) K H (the chunk's
    // v' = U - W H is T diag(beta) Y):
    //   step  state waves                          preparation waves
    //   1     O = scale gamma Q H + Z Y, decayed    gate scan, K K^T; load g, beta of c + 2
    //         v' = diag(dec) T diag(beta) Y
    //   2     H update                             inverse level 0
    //   3     X = K H and Q H of chunk c + 1       inverse level 1 (pw 0, 1), P
    //   4     Y of chunk c + 1; load K of c + 2    inverse level 2; WY fragments of rows 0..31
    //                                              (diag(dec) T diag(beta), Z); load Q of c + 2
    //   5     (optional h store)                   the same for rows 32..63; load V of c + 2
    // K sits in LDS by chunk parity, Q and V for one chunk each; each load is
    // issued once the step that last reads its slot is behind a barrier.  The
    // state waves wait for their K loads before the next iteration's first
    // barrier; the preparation waves wait before the first barrier for their g
    // and beta loads only (the Q and V tiles of steps 4 and 5 stay in flight)
    // and before the third for everything but this iteration's g and beta.
    // Both roles run their own copy of the loop with the same five barriers per
    // iteration (a barrier counts arrivals, wherever they come from), so each
    // role's registers are allocated for its own live values.
    if (state_wave) {
        // ---- state: value columns 32 wave .. +31
        f32x4 hacc[2][8];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) hacc[ct][dt] = f32x4{};
        if (PRE) {
            if (mwave) {  // identity: key row 16 dt + 4 g + jj, column 32 sw + 16 ct + l % 16
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj)
                            hacc[ct][dt][jj] =
                                (16 * dt + 4 * (lane >> 4) + jj == 32 * sw + 16 * ct + (lane & 15)) ? 1.f : 0.f;
            }
        } else {
            const float *src = nullptr;
            if (from_h0 && p.h0) src = p.h0 + ((int64_t)e.n * p.Hv + j) * DK * DV;
            if (!from_h0 && p.cp_mode == 1 /* EXACT */) src = p.ws_h + ((int64_t)seg * p.Hv + j) * DK * DV;
            if (src) load_state8(hacc, src, wave, lane);
        }
        const int64_t oes = OF32 ? 4 : 2;
        const char *obase = static_cast<const char *>(p.o) + ((int64_t)e.row0 * p.Hv + j) * DV * oes;
        f32x4 qh[4][2];  // scale diag(gamma) Q H of the next chunk, transposed
        f32x4 vd[4][2];  // decayed v' of this chunk
        f32x4 X[4][2];   // K H of the next chunk
        YSplit ysp;      // Y of the chunk whose state pass comes next
        const int cbase = (!PRE && (p.h_out || p.vn_out)) ? seq_chunk_base(p, e.n, lane) : 0;
        const TileOffs<NSTATE> koffs = tile_offsets<NSTATE>(in.kstride, wave, lane);  // this wave's share of K
        for (int c = c_first - 1; has_chunks && c < c_end; ++c) {
            const bool chain = c >= c_first;  // state pass of chunk c
            const bool prep = c + 1 < c_end;  // chunk c + 1 follows
            const bool out = !PRE && c >= e.c_begin;             // chunk c produces output
            const bool qnext = !PRE && prep && c + 1 >= e.c_begin;  // chunk c + 1 produces output
            const int b = c & 1, nb = (c + 1) & 1;
            dma_wait();
            lds_barrier();
            // A fresh opaque lane index per step keeps the compiler from
            // hoisting lane-derived LDS addresses out of their steps and
            // holding them all live at once.
            auto lane_now = []() {
                int t = threadIdx.x;
                asm volatile("" : "+v"(t));
                return t & 63;
            };
            // Every value carried from one step to a later one is defined on
            // both sides of its step's branch: a value defined on one side only
            // would stay live around the whole loop (the compiler cannot tell
            // that the later step's branch takes the same side), and the
            // registers would spill.
            if (chain) {
                if (PRE) tdy(s, true, ysp, vd, lane_now());  // the pre-pass has no output
                else out_vd<OF32>(s, p, obase, e.seq_len, ysp, qh, vd, out, c, wave, lane_now());
                if (out && p.vn_out) {
                    f32x4 vp[4][2];
                    tdy(s, false, ysp, vp, lane_now());
                    store_vn8(vp, p.vn_out + ((int64_t)(cbase + c) * p.Hv + j) * CH * DV, wave, lane_now());
                }
            } else {
                zero_tiles(vd);
            }
            lds_barrier();
            if (chain) upd<PRE>(s, hacc, vd, b, lane_now());
            lds_barrier();
            // h of chunk c + 1 (the state is final after the update) goes out
            // before the K loads below, whose wait then also covers these
            // stores, two steps later than a store after the Q H product
            if (qnext && p.h_out)
                store_state8(hacc, p.h_out + ((int64_t)(cbase + c + 1) * p.Hv + j) * DK * DV, wave, lane_now());
            // the K tile of chunk c is free since the H update: the loads of
            // chunk c + 2 have three steps to land (the compiler makes this
            // wave wait for them before its next transposing LDS read, in step 4)
            if (c + 2 < c_end) dma_tile<NSTATE>(s.k[b], in.k, in.kstride, c + 2, e.seq_len, wave, koffs);
            if (prep) xk(s, hacc, X, nb, lane_now());
            else zero_tiles(X);
            lds_barrier();
            if (prep) yform(s, X, ysp, !mwave, sw, nb, lane_now());
            else ysp = YSplit{};
            lds_barrier();
            if (qnext) qhq<OF32>(s, hacc, qh, nb, p.scale, lane_now());
            else zero_tiles(qh);
        }
        if (PRE) {
            store_state8(hacc, (mwave ? p.ws_m : p.ws_s) + ((int64_t)seg * p.Hv + j) * DK * DV, sw, lane);
        } else if (e.last && p.ht) {
            store_state8(hacc, p.ht + ((int64_t)e.n * p.Hv + j) * DK * DV, wave, lane);
        }
    } else {
        __builtin_amdgcn_s_setprio(2);
        // Each preparation wave's share (tile rows, k steps, fragments) is
        // fixed by its index pw; the loop is compiled once per pw, so that the
        // share's LDS offsets and branches are constants.
        auto prep_role = [&](auto pw_c) {
            constexpr int pw = decltype(pw_c)::value;
            const TileOffs<4> kqoffs = tile_offsets<4>(in.kstride, pw, lane);  // this wave's share of K and Q
            const TileOffs<4> voffs = tile_offsets<4>(in.vstride, pw, lane);   // and of V
            const char *abase = (!PRE && p.a_out) ? reinterpret_cast<const char *>(p.a_out + ((int64_t)e.row0 * p.Hv + j) * CH)
                                        : nullptr;
            const bool with_tf = !PRE && p.vn_out;
            if (has_chunks) {
                dma_tile<4>(s.k[c_first & 1], in.k, in.kstride, c_first, e.seq_len, pw, kqoffs);
                dma_gb(s, in, c_first, pw, lane);
                dma_tile<4>(s.v, in.v, in.vstride, c_first, e.seq_len, pw, voffs);
            }
            // vector memory operations this wave issued after its g / beta load
            // of the previous iteration (the A stores and the V tile of its last
            // step): left in flight by the wait before the first barrier
            int after_gb = 0;
            for (int c = c_first - 1; has_chunks && c < c_end; ++c) {
                // with the wave's share fixed at compile time, its lane-derived
                // LDS addresses are few enough to stay in registers across the
                // loop (the state loop re-derives its own every step instead)
                const int ln = lane;
                const bool prep = c + 1 < c_end;   // preparation of chunk c + 1
                const bool ahead = c + 2 < c_end;  // loads of chunk c + 2
                const int nb = (c + 1) & 1;
                const bool pout = !PRE && prep && c + 1 >= e.c_begin;  // chunk c + 1 produces output: P, Z needed
                dma_wait_upto(after_gb);
                lds_barrier();
                // Q of chunk c + 1: its tile is free since the state waves' Q H
                // of chunk c (the previous iteration's last step)
                if (pout) dma_tile<4>(s.q, in.q, in.kstride, c + 1, e.seq_len, pw, kqoffs);
                if (ahead) dma_gb(s, in, c + 2, pw, ln);
                if (prep) prod9(s, ln, pw, nb);
                lds_barrier();
                if (prep) inv8_l0(s, ln, pw);
                // Q of chunk c + 1 (read by P in the next step) and V of chunk
                // c + 1 (read by the state waves' Y in step 4): every load but
                // this iteration's g or beta
                if (ahead && pw < 2) dma_wait_but<1>();
                else dma_wait();
                lds_barrier();
                if (prep && pw < 2) {
                    inv8_l1(s, ln, pw);
                    // rows 0..31 of T are final once block 0's level 1 (this
                    // step, wave 0's own writes) and level 0 (the last step)
                    // are: wave 0 forms fragment 1 (rows 16..31) after its
                    // level 1, wave 1 fragment 0 (rows 0..15, level 0 only);
                    // their T diag(beta) copies (v' stored) wait for the next step
                    tdfrag(s, ln, 1 - pw, nb, false);
                }
                if (pout && pw < 2) pfrag9(s, ln, pw + 1, nb, p.scale, decays_factor(s, ln));  // fragments 1, 2
                if (pout && pw >= 2) {
                    const bool fact = decays_factor(s, ln);
                    pfrag9(s, ln, pw == 2 ? 5 : 3, nb, p.scale, fact);
                    pfrag9(s, ln, pw == 2 ? 0 : 4, nb, p.scale, fact);
                }
                lds_barrier();
                // Z^T fragment 2 + pw (pw < 2) over two steps: the token step
                // of T's first diagonal block now, the lower-left block (level
                // 2) in the next step
                f32x4 zacc[2] = {f32x4{}, f32x4{}};
                if (prep) {
                    L2Regs l2;
                    inv8_l2a(s, ln, pw, l2);
                    inv8_l2b(s, ln, pw, l2);
                    if (with_tf && pw < 2) tdfrag(s, ln, 1 - pw, nb, true, false);
                    // Z^T fragments 4 and 5 read only T's diagonal blocks
                    if (pout) {
                        f32x4 z[2] = {f32x4{}, f32x4{}};
                        if (pw < 2) {
                            zsum<0, 1>(s, ln, pw, nb, z);
                            zstore(s, ln, pw, z);
                            zsum<0, 0>(s, ln, 2 + pw, nb, zacc);
                        } else {
                            zsum<1, 1>(s, ln, 2 + pw, nb, z);
                            zstore(s, ln, 2 + pw, z);
                        }
                    }
                }
                lds_barrier();
                const bool astore = !PRE && prep && p.a_out && c + 1 >= e.c_begin;
                if (astore) store_t8(s, p, abase, e.seq_len, c + 1, pw, ln);
                if (ahead) dma_tile<4>(s.v, in.v, in.vstride, c + 2, e.seq_len, pw, voffs);
                after_gb = ahead ? ((astore ? 4 : 0) + NTILE4(pw)) : 0;
                if (prep) {
                    // rows 32..63: fragments 2..5 on waves 2 and 3, while waves
                    // 0 and 1 finish their Z^T fragments (the waves share SIMDs
                    // with the state waves one to one, so each step's work is
                    // spread evenly over them)
                    if (pw >= 2) {
                        tdfrag(s, ln, pw, nb, with_tf);
                        tdfrag(s, ln, pw + 2, nb, with_tf);
                    } else if (pout) {
                        zsum<1, 1>(s, ln, 2 + pw, nb, zacc);
                        zstore(s, ln, 2 + pw, zacc);
                    }
                }
            }
        };
        switch (wave - NSTATE) {
        case 0: prep_role(std::integral_constant<int, 0>{}); break;
        case 1: prep_role(std::integral_constant<int, 1>{}); break;
        case 2: prep_role(std::integral_constant<int, 2>{}); break;
        default: prep_role(std::integral_constant<int, 3>{}); break;
        }
    }
}


// One workgroup per CU (its LDS footprint): two waves per SIMD for the forward,
// three for the pre-pass.
template <bool OF32>
__global__ void __launch_bounds__(NT8, 1) __attribute__((amdgpu_waves_per_eu(1, 2))) gdn_fwd_main_kernel(FwdParams p) {
    fwd_pass<false, OF32>(p);
}
constexpr int NT_PRE = 768;
__global__ void __launch_bounds__(NT_PRE, 1) gdn_cp_prepass_kernel(FwdParams p) { fwd_pass<true, true>(p); }

// ---------------------------------------------------------------- exact context parallelism
// Combine (sequential over a sequence's segments): H_start[0] = initial state,
// H_start[r+1] = M_r H_start[r] + S_r.  The value columns of H never mix, so
// one workgroup of 8 waves takes one block of 32 value columns of one
// (sequence, v-head): wave w computes rows 16 w .. 16 w + 15 of the block
// (v_mfma_f32_16x16x32_bf16, M rows split hi + lo as the A operand, H as the
// hi / lo B operand from LDS, stored transposed [column][key]).  The operands
// of steps r + 1 and r + 2 (this wave's M rows and S entries, 40 registers a
// step) are in flight while step r runs, so a step waits on the previous
// one's products, not on HBM.
constexpr int CB_COLS = 32;            // value columns per combine workgroup
constexpr int CB_LD = DK + 8;          // bf16 row stride of the transposed H block (272 B)
constexpr int NT_COMB = 512;

struct CombRegs {
    f32x4 m[4][2];   // M row 16 w + l % 16, k = 32 kk + 8 g .. +7 (g = l / 16)
    float x[2][4];   // S entries: rows 16 w + 4 g + j, column 16 ct + l % 16
};

__device__ __forceinline__ void comb_load(CombRegs &R, const float *M, const float *S, const int wave, const int lane,
                                          const int col0) {
    const int m = lane & 15, g = lane >> 4;
    const float *row = M + (int64_t)(16 * wave + m) * DK + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        R.m[kk][0] = *reinterpret_cast<const f32x4 *>(row + 32 * kk);
        R.m[kk][1] = *reinterpret_cast<const f32x4 *>(row + 32 * kk + 4);
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            R.x[ct][jj] = S[(int64_t)(16 * wave + 4 * g + jj) * DV + col0 + 16 * ct + m];
}

// The wave's rows of S + M H for the block's two column tiles (all H operand
// reads issued before the first product, so their latency is paid once)
__device__ __forceinline__ void comb_step(const CombRegs &R, const bf16 *hH, const bf16 *hL, const int lane,
                                          f32x4 (&acc)[2]) {
    const int m = lane & 15, g = lane >> 4;
    bf16x8 bh[4][2], bl[4][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            bh[kk][ct] = lds8(hH + (16 * ct + m) * CB_LD + 32 * kk + 8 * g);
            bl[kk][ct] = lds8(hL + (16 * ct + m) * CB_LD + 32 * kk + 8 * g);
        }
    __builtin_amdgcn_sched_barrier(0);  // keep the batch of reads ahead of its products
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[ct] = f32x4{R.x[ct][0], R.x[ct][1], R.x[ct][2], R.x[ct][3]};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const float av[8] = {R.m[kk][0][0], R.m[kk][0][1], R.m[kk][0][2], R.m[kk][0][3],
                             R.m[kk][1][0], R.m[kk][1][1], R.m[kk][1][2], R.m[kk][1][3]};
        bf16x8 ah, al;
        split8v(av, ah, al);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            acc[ct] = mfma16(ah, bh[kk][ct], acc[ct]);
            acc[ct] = mfma16(ah, bl[kk][ct], acc[ct]);
            acc[ct] = mfma16(al, bh[kk][ct], acc[ct]);
        }
    }
}

// The wave's rows of the block into LDS (hi / lo, transposed) and, if dst,
// into HBM ([key][value] fp32).
__device__ __forceinline__ void comb_put(const f32x4 (&x)[2], bf16 *hH, bf16 *hL, float *dst, const int wave,
                                         const int lane, const int col0) {
    const int m = lane & 15, g = lane >> 4;
    const int k = 16 * wave + 4 * g;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        uint32_t hi0, lo0, hi1, lo1;
        split2(x[ct][0], x[ct][1], hi0, lo0);
        split2(x[ct][2], x[ct][3], hi1, lo1);
        *reinterpret_cast<u32x2 *>(hH + (16 * ct + m) * CB_LD + k) = u32x2{hi0, hi1};
        *reinterpret_cast<u32x2 *>(hL + (16 * ct + m) * CB_LD + k) = u32x2{lo0, lo1};
        if (dst) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) dst[(int64_t)(k + jj) * DV + col0 + 16 * ct + m] = x[ct][jj];
        }
    }
}

__global__ void __launch_bounds__(NT_COMB, 1) gdn_cp_combine_kernel(FwdParams p) {
    // H_start[r] by the parity of r: step r reads one pair and writes the
    // other, so one barrier per step orders both hand-offs
    __shared__ __attribute__((aligned(16))) bf16 hH[2][CB_COLS * CB_LD], hL[2][CB_COLS * CB_LD];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    constexpr int NCB = DV / CB_COLS;
    const int cb = blockIdx.x % NCB;
    const int nj = blockIdx.x / NCB;
    const int n = nj / p.Hv;
    const int j = nj % p.Hv;
    if (n >= p.N) return;
    const int col0 = CB_COLS * cb;
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
    {
        // H_start[0]: the initial state's block (or zeros)
        f32x4 h0v[2];
        const int m = lane & 15, g = lane >> 4;
        const float *src = p.h0 ? p.h0 + ((int64_t)n * p.Hv + j) * DK * DV : nullptr;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                h0v[ct][jj] = src ? src[(int64_t)(16 * wave + 4 * g + jj) * DV + col0 + 16 * ct + m] : 0.f;
        comb_put(h0v, hH[0], hL[0], nullptr, wave, lane, col0);
    }
    auto seg_off = [&](int r) { return ((int64_t)(seg0 + r) * p.Hv + j) * DK * DV; };
    const int steps = R - 1;  // step r makes H_start[r + 1]
    CombRegs C[3];
    // Loads are issued unconditionally (past the last step they re-read the
    // last step's operands, unused): with no branch around them the compiler
    // can count them and waits only for the set a step consumes.
    auto load = [&](CombRegs &X, int r) {
        const int rr = min(r, steps - 1);
        comb_load(X, p.ws_m + seg_off(rr), p.ws_s + seg_off(rr), wave, lane, col0);
    };
    // An LDS-only barrier: a __syncthreads would also wait for every global
    // access in flight, the operand loads of the next two steps included.
    // After it, H_start[r] is complete and every wave is done reading
    // H_start[r - 1], whose pair takes H_start[r + 1].
    auto step = [&](const CombRegs &X, int r) {
        lds_barrier();
        f32x4 acc[2];
        comb_step(X, hH[r & 1], hL[r & 1], lane, acc);
        comb_put(acc, hH[(r + 1) & 1], hL[(r + 1) & 1], p.ws_h + seg_off(r + 1), wave, lane, col0);
    };
    load(C[0], 0);
    load(C[1], 1);
    // three register sets in rotation (unrolled by three so that the sets are
    // fixed registers): the loads of step r + 2 go out before step r
    int r = 0;
    for (; r + 3 <= steps; r += 3) {
        load(C[2], r + 2);
        step(C[0], r);
        load(C[0], r + 3);
        step(C[1], r + 1);
        load(C[1], r + 4);
        step(C[2], r + 2);
    }
    if (r < steps) step(C[0], r);
    if (r + 1 < steps) {
        load(C[2], r + 2);
        step(C[1], r + 1);
    }
}

// ---------------------------------------------------------------- chunk cumsum
// One thread per (row, head); the thread whose row starts a chunk scans that
// chunk in order, reading each g before writing its sum, so out may equal g.
// Offsets are the caller's device data: every range taken from them is
// clamped to the B * T rows of the buffers, so offsets that break the
// contract (past T, decreasing) give wrong sums, never an access outside g or out.
__global__ void __launch_bounds__(256) gdn_chunk_cumsum_kernel(const float *g, float *out, int64_t B, int64_t T,
                                                               int32_t H, int32_t chunk, const int32_t *cu,
                                                               int32_t N) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = B * T * H, total_rows = B * T;
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
        seq0 = min(max((int64_t)cu[lo], (int64_t)0), row);
        seq1 = min((int64_t)cu[lo + 1], total_rows);
    } else {
        seq0 = (row / T) * T;
        seq1 = seq0 + T;
    }
    if ((row - seq0) % chunk != 0) return;
    const int64_t end = min(row + chunk < seq1 ? row + chunk : seq1, total_rows);
    float acc = 0.f;
    for (int64_t r = row; r < end; ++r) {
        acc += g[r * H + hh];
        out[r * H + hh] = acc;
    }
}

// ---------------------------------------------------------------- launchers
int launch_fwd_main(const FwdParams &p, void *stream) {
    static const size_t smem = sizeof(Smem8);
    static const int attr_rc = [] {
        const int rc = (int)hipFuncSetAttribute((const void *)gdn_fwd_main_kernel<false>,
                                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
        return rc ? rc
                  : (int)hipFuncSetAttribute((const void *)gdn_fwd_main_kernel<true>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    }();
    if (attr_rc != 0) return attr_rc;
    const unsigned grid = (unsigned)p.num_segments * (unsigned)p.Hv;
    if (p.o_f32)
        hipLaunchKernelGGL(gdn_fwd_main_kernel<true>, dim3(grid), dim3(NT8), smem, (hipStream_t)stream, p);
    else
        hipLaunchKernelGGL(gdn_fwd_main_kernel<false>, dim3(grid), dim3(NT8), smem, (hipStream_t)stream, p);
    return (int)hipGetLastError();
}

int launch_cp_exact(const FwdParams &p, void *stream) {
    static const size_t smem = sizeof(Smem8);
    static const int attr_rc =
        (int)hipFuncSetAttribute((const void *)gdn_cp_prepass_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)smem);
    if (attr_rc != 0) return attr_rc;
    const unsigned grid = (unsigned)p.num_segments * (unsigned)p.Hv;
    hipLaunchKernelGGL(gdn_cp_prepass_kernel, dim3(grid), dim3(NT_PRE), smem, (hipStream_t)stream, p);
    int err = (int)hipGetLastError();
    if (err) return err;
    hipLaunchKernelGGL(gdn_cp_combine_kernel, dim3((unsigned)p.N * (unsigned)p.Hv * (unsigned)(DV / CB_COLS)),
                       dim3(NT_COMB), 0,
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
