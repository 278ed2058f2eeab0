// HIP kernels of the Gated DeltaNet chunked-prefill forward for gfx950 (MI355X).
//
// What is computed (FlashQLA pages, "FlashQLA: CP-/Bwd-friendly fused linear
// attention kernels for GDN"; the pages name the steps, the formulas are the
// standard chunked WY form of the gated delta rule). For a chunk of 64 tokens
// with incoming state S (d_k x d_v, fp32):
//   gamma = cumsum(g)                      (chunk-local gate log-decay)
//   A[i][j] = beta_i exp(gamma_i - gamma_j) k_i.k_j  (i > j)
//   T = (I + A)^-1,  W = T diag(beta e^gamma) K,  U = T diag(beta) V
//   V' = U - W S                           (pseudo-values)
//   O = scale (diag(e^gamma) Q S + (Q K^T o D) V'),  D[r][i] = e^(gamma_r - gamma_i), i <= r
//   S <- e^gamma_C S + K^T diag(e^(gamma_C - gamma)) V'
//
// Kernels. k_prep solves for T and the chunk-local gate sums of every chunk
// in one wide launch (chunks are independent; this is the state-free half of
// the preparation step). The chain kernels then walk their chunks in order;
// with T at hand they need neither W nor U: V' = U - W S = T Y with
// Y = diag(beta) (V - diag(e^gamma) K S), so the intermediates W, U and S
// never reach HBM (section on optimising GDN chunked prefill). Section
// "Gate-Driven Automatic Intra-Card Context Parallelism (AutoCP)": each
// sequence is cut into segments of L chunks that run as independent
// workgroups; k_cp_prep computes the state at each segment boundary by a
// short warm-up (gates decayed below the noise floor) or the exact state map
// S -> M S + H of the previous segment, k_cp_combine chains the exact maps,
// and k_fwd runs every segment.
//
// Work layout of the chain kernels. A workgroup is 4 waves (256 lanes). Wave
// w owns d_v columns [32w, 32w + 32): its 128 x 32 slice of S, its slice of
// Y / V' and of the output all stay in its registers, so the sequential state
// chain never crosses waves. Operands that every wave needs (Q, K, K^T, V^T,
// T, P = QK^T o D) are staged in LDS. Products use 32x32x16 bf16 MFMAs with
// fp32 accumulation. Values that are not exact bf16 inputs (S, Y, V', T, P)
// enter the MFMA as a hi + lo pair of bf16 (x = hi + lo to about 16 bits),
// giving 2 or 3 MFMAs per product; diagonal gate factors are applied in fp32
// on the accumulators instead of being rounded into operands.
//
// Register layouts (verified on gfx950): 32x32x16 bf16 MFMA, lane l,
//   A operand: row l % 32, 8 k values; B operand: column l % 32, 8 k values
//   C/D: element i holds row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.
// Element e of an operand is placed at k = kb + kperm(h, e), h = l / 32, with
// kperm(h, e) = 4h + e (e < 4) or 8 + 4h + (e - 4); that is exactly where the
// accumulator layout holds rows, so a 32-row accumulator tile serves directly
// as the B operand of two consecutive k steps (elements 0..7 and 8..15), and,
// as the A and B layouts mirror each other, as the A operand of the
// transposed product.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int CH = kChunk;
constexpr int DK = kDim;
constexpr int NTHR = 256;
constexpr int LDQ = 136;   // row stride (elements) of [64][128] bf16 tiles
constexpr int LDKT = 72;   // row stride of [128][64] bf16 tiles
constexpr int LDF = 68;    // row stride of [64][64] fp32 tiles
constexpr int LDP = 72;    // row stride of [64][64] bf16 tiles
constexpr int kMaxFlags = kMaxSegsPerSeq;  // boundary flags the combine kernel keeps in LDS

enum { kCpAuto = 0, kCpOff = 1, kCpExact = 2, kCpWarmup = 3 };

template <typename IO> struct Io;
template <> struct Io<bf16> { static constexpr bool kExact = true; };
template <> struct Io<float> { static constexpr bool kExact = false; };

// ----------------------------------------------------------------------------
// MFMA and operand helpers

__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma16k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The lane index passes through an empty asm, so that the LDS addresses
// derived from it are formed in the function that uses them: otherwise the
// compiler hoists hundreds of loop-invariant addresses out of the chunk loop
// and spills them to scratch. The wave index is wave-uniform (a scalar).
__device__ __forceinline__ int lane_id() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    return l;
}
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Row of accumulator element i for lane half h (32x32 tiles).
__device__ __forceinline__ int acc_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// hi/lo splits. hi is x with its low 16 bits cleared (a bf16 value), lo is
// x - hi (exact in fp32) rounded to nearest bf16, so hi + lo = x to within
// 2^-16 |x|.
__device__ __forceinline__ unsigned pack_rne(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ void split_pair(float x0, float x1, unsigned& hi, unsigned& lo) {
    const unsigned u0 = __float_as_uint(x0), u1 = __float_as_uint(x1);
    hi = (u0 >> 16) | (u1 & 0xffff0000u);
    lo = pack_rne(x0 - __uint_as_float(u0 & 0xffff0000u), x1 - __uint_as_float(u1 & 0xffff0000u));
}
__device__ __forceinline__ void split1(float x, bf16& hi, bf16& lo) {
    const unsigned u = __float_as_uint(x);
    hi = __builtin_bit_cast(bf16, (unsigned short)(u >> 16));
    lo = (bf16)(x - __uint_as_float(u & 0xffff0000u));
}
__device__ __forceinline__ void split4(f32x4 x, bf16x4& hi, bf16x4& lo) {
    unsigned h0, h1, l0, l1;
    split_pair(x[0], x[1], h0, l0);
    split_pair(x[2], x[3], h1, l1);
    hi = __builtin_bit_cast(bf16x4, u32x2{h0, h1});
    lo = __builtin_bit_cast(bf16x4, u32x2{l0, l1});
}

// Elements [B, B + 8) of an accumulator tile as a hi/lo B operand.
template <int B>
__device__ __forceinline__ void split_acc(const f32x16& a, bf16x8& hi, bf16x8& lo) {
    unsigned h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split_pair(a[B + 2 * e], a[B + 2 * e + 1], h[e], l[e]);
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

__device__ __forceinline__ void split_half(const f32x16& a, int half, bf16x8& hi, bf16x8& lo) {
    if (half) split_acc<8>(a, hi, lo);
    else split_acc<0>(a, hi, lo);
}

// bf16 operand tiles in LDS keep their contraction (k) axis in a permuted
// order: within every group of 16, the 4-element blocks 1 and 2 trade places.
// Then the 8 values lane half h needs for one k step (k = kb + kperm(h, e))
// sit contiguously at kb + 8 h and come in one 16-byte read.
__device__ __forceinline__ int pk(int k) {
    const int b = (k >> 2) & 3;
    return (k & ~12) | ((b == 1 ? 2 : (b == 2 ? 1 : b)) << 2);
}
__device__ __forceinline__ bf16x8 lds_op16(const bf16* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}

// Row of the transposed [128][64] LDS tiles (K^T, V^T) that holds column c:
// the low three bits are XORed with bits 3..5 and 6, so that the staging
// stores (sixteen lanes eight columns apart, four consecutive tokens each)
// fall on distinct banks; a bijection on 0..127.
__device__ __forceinline__ int trow(int c) { return (c & ~7) | ((c ^ (c >> 3) ^ (c >> 6)) & 7); }

// B operand from one column of a token-major global tile: element e is token
// kb + kperm(h, e); tokens >= nvalid read as zero.
template <typename IO>
__device__ __forceinline__ void g_col_op(const IO* col0, size_t ts, int kb, int h, int nvalid,
                                         bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int t = kb + ((e < 4) ? (4 * h + e) : (4 + 4 * h + e));
        const float x = (t < nvalid) ? (float)col0[(size_t)t * ts] : 0.f;
        if (Io<IO>::kExact) {
            hi[e] = (bf16)x;
            lo[e] = (bf16)0.f;
        } else {
            bf16 th, tl;
            split1(x, th, tl);
            hi[e] = th;
            lo[e] = tl;
        }
    }
}

// ----------------------------------------------------------------------------
// Work items: segments and chunks

struct SegLoc {
    int seq;          // -1 if the slot is past the last segment
    int s;            // segment index within the sequence
    int P;            // segments of the sequence
    int N;            // chunks of the sequence
    int len;          // tokens of the sequence
    int seg_base;     // global index of the sequence's segment 0
    int chunk_base;   // global index of the sequence's chunk 0
    size_t tok0;      // global token index of the sequence start
};

__device__ __forceinline__ int n_chunks_of(int len) { return (len + CH - 1) / CH; }
__device__ __forceinline__ int n_segs_of(int N, int L) { return N == 0 ? 1 : (N + L - 1) / L; }

__device__ SegLoc locate_segment(const Params& p, int slot) {
    SegLoc o;
    o.seq = -1;
    o.s = o.P = o.N = o.len = o.seg_base = o.chunk_base = 0;
    o.tok0 = 0;
    if (!p.cu) {
        const int N = n_chunks_of(p.seq_len);
        const int P = n_segs_of(N, p.L);
        const int seq = slot / P;
        if (seq < p.n_seqs) {
            o.seq = seq; o.s = slot - seq * P; o.P = P; o.N = N; o.len = p.seq_len;
            o.seg_base = seq * P; o.chunk_base = seq * N; o.tok0 = (size_t)seq * p.seq_len;
        }
        return o;
    }
    int base = 0, cbase = 0;
    for (int n = 0; n < p.n_seqs; ++n) {
        const int a = p.cu[n], len = p.cu[n + 1] - a;
        const int N = n_chunks_of(len), P = n_segs_of(N, p.L);
        if (slot < base + P) {
            o.seq = n; o.s = slot - base; o.P = P; o.N = N; o.len = len;
            o.seg_base = base; o.chunk_base = cbase; o.tok0 = (size_t)a;
            return o;
        }
        base += P;
        cbase += N;
    }
    return o;
}

// Chunk slot -> (sequence, chunk within it); returns false past the end.
__device__ bool locate_chunk(const Params& p, int slot, int& seq, int& c, int& len, size_t& tok0) {
    if (!p.cu) {
        const int N = n_chunks_of(p.seq_len);
        if (N == 0) return false;
        seq = slot / N;
        c = slot - seq * N;
        len = p.seq_len;
        tok0 = (size_t)seq * p.seq_len;
        return seq < p.n_seqs;
    }
    int base = 0;
    for (int n = 0; n < p.n_seqs; ++n) {
        const int a = p.cu[n], l = p.cu[n + 1] - a, N = n_chunks_of(l);
        if (slot < base + N) {
            seq = n; c = slot - base; len = l; tok0 = (size_t)a;
            return true;
        }
        base += N;
    }
    return false;
}

// Inclusive scan of g over the 64 lanes of a wave (lane = token of the chunk).
__device__ __forceinline__ float wave_scan(float s) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(s, d, 64);
        if (lane >= d) s += o;
    }
    return s;
}


// ----------------------------------------------------------------------------
// Chunk preparation kernel: gamma, beta and T = (I + A)^-1 of every (chunk,
// value head). Chunks are independent, so this runs as a wide grid at two
// workgroups per CU; the chain kernels then read T instead of solving the
// triangular system inside their sequential loops.

template <bool EX>
struct __attribute__((aligned(16))) PrepSmem {
    bf16 k_rm[EX ? CH * LDQ : 8];   // K chunk token-major, d_k permuted (bf16 inputs)
    float a[CH * LDF];              // A (strictly lower)
    float t[CH * LDF];              // T = (I + A)^-1
    float gam[CH];
    float beta[CH];
};

// Lower 16x16 tile number job (0..9) -> block row bi >= block column bj.
__device__ __forceinline__ void lower_tile(int job, int& bi, int& bj) {
    bi = (job >= 6) ? 3 : (job >= 3) ? 2 : (job >= 1) ? 1 : 0;
    bj = job - (bi * (bi + 1)) / 2;
}

// The operand a gram lane group reads from a permuted LDS row (8 physical
// elements at 8 g4 within a 32-wide k step), taken from a global fp32 row
// instead: logical elements p[0..3] and p[8..11] with p = row + 32 ks +
// 16 (g4 / 2) + 4 (g4 % 2). Zero if !valid.
__device__ __forceinline__ void g_row8(const float* p, bool valid, bf16x8& hi, bf16x8& lo) {
    if (valid) {
        bf16x4 h0, l0, h1, l1;
        split4(*reinterpret_cast<const f32x4*>(p), h0, l0);
        split4(*reinterpret_cast<const f32x4*>(p + 8), h1, l1);
        hi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
        lo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
        hi = bf16x8{};
        lo = bf16x8{};
    }
}
__device__ __forceinline__ bf16x8 lds_row8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// A[i][j] = beta_i exp(gamma_i - gamma_j) (k_i . k_j) for i > j, else 0, on
// 16x16 tiles (16x16x32 MFMA; lane l: A row l % 16 and B column l % 16, each
// with the 8 consecutive k values 8 (l / 16)..; C rows 4 (l / 16).. of column
// l % 16). The ten lower tiles are jobs first, first + stride, ..., run as
// interleaved chains; each is computed transposed (K rows of block bj against
// K rows of block bi), so a lane ends up with four consecutive columns j of
// one row i and stores them at once.
template <typename IO, int NJOB>
__device__ void gram_a(PrepSmem<Io<IO>::kExact>& sm, const IO* krow0, size_t ts, int nvalid, int first,
                       int stride) {
    constexpr bool EX = Io<IO>::kExact;
    const int lane = lane_id(), n = lane & 15, g4 = lane >> 4;
    f32x4 acc[NJOB];
    int bi[NJOB], bj[NJOB];
#pragma unroll
    for (int t = 0; t < NJOB; ++t) {
        lower_tile(first + stride * t, bi[t], bj[t]);
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int kb = 32 * ks + 8 * g4;                                 // physical (LDS)
        const int kg = 32 * ks + 16 * (g4 >> 1) + 4 * (g4 & 1);          // logical start (HBM rows)
#pragma unroll
        for (int t = 0; t < NJOB; ++t) {
            const int ra = 16 * bj[t] + n, rb = 16 * bi[t] + n;
            if constexpr (EX) {
                acc[t] = mma16k32(lds_row8(sm.k_rm + ra * LDQ + kb), lds_row8(sm.k_rm + rb * LDQ + kb), acc[t]);
            } else {
                bf16x8 ah, al, bh, bl;
                g_row8(krow0 + (size_t)ra * ts + kg, ra < nvalid, ah, al);
                g_row8(krow0 + (size_t)rb * ts + kg, rb < nvalid, bh, bl);
                acc[t] = mma16k32(ah, bh, acc[t]);
                acc[t] = mma16k32(ah, bl, acc[t]);
                acc[t] = mma16k32(al, bh, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NJOB; ++t) {
        const int i = 16 * bi[t] + n, j0 = 16 * bj[t] + 4 * g4;   // row i, columns j0 .. j0 + 3
        const float gi = sm.gam[i], bt = sm.beta[i];
        const f32x4 gj = *reinterpret_cast<const f32x4*>(sm.gam + j0);
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (i > j0 + r) ? bt * __expf(gi - gj[r]) * acc[t][r] : 0.f;
        *reinterpret_cast<f32x4*>(sm.a + i * LDF + j0) = v;
    }
}

// Diagonal 16x16 blocks of T = (I + A)^-1 by forward substitution. Every
// wave solves all four blocks (lane 16 b + j: block b, column j) and writes
// them; the values are identical across waves, so each wave can read the
// blocks back without waiting for the others.
template <bool EX>
__device__ void inv_diag(PrepSmem<EX>& sm) {
    const int lane = lane_id(), b = 16 * (lane >> 4), j = lane & 15;
    const float* A = sm.a + b * LDF + b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float s = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) s = fmaf(-A[i * LDF + m], x[m], s);
        x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.t[(b + i) * LDF + b + j] = x[i];
}

// Block column J of T below the diagonal: T_iJ = -X_i sum_{m=J}^{i-1} A_im T_mJ,
// with 16x16x16 bf16 MFMAs on hi/lo operands (lane l: A row l % 16, k 4 (l/16)..;
// B / C column l % 16, rows 4 (l/16)..). Zeros above the diagonal block.
template <int J, bool EX>
__device__ void inv_col(PrepSmem<EX>& sm) {
    const int lane = lane_id(), n = lane & 15, g4 = lane >> 4;
    f32x4 Tc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) Tc[J][r] = sm.t[(16 * J + 4 * g4 + r) * LDF + 16 * J + n];
#pragma unroll
    for (int i = J + 1; i < 4; ++i) {
        f32x4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = J; m < i; ++m) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(sm.a + (16 * i + n) * LDF + 16 * m + 4 * g4);
            bf16x4 ah, al, bh, bl;
            split4(a, ah, al);
            split4(Tc[m], bh, bl);
            R = mma16(ah, bh, R);
            R = mma16(ah, bl, R);
            R = mma16(al, bh, R);
        }
        const f32x4 xi = *reinterpret_cast<const f32x4*>(sm.t + (16 * i + n) * LDF + 16 * i + 4 * g4);
        bf16x4 xh, xl, rh, rl;
        split4(xi, xh, xl);
        split4(R, rh, rl);
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
        P = mma16(xh, rh, P);
        P = mma16(xh, rl, P);
        P = mma16(xl, rh, P);
        Tc[i] = -P;
    }
#pragma unroll
    for (int i = 0; i < J; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.t[(16 * i + 4 * g4 + r) * LDF + 16 * J + n] = 0.f;
#pragma unroll
    for (int i = J + 1; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.t[(16 * i + 4 * g4 + r) * LDF + 16 * J + n] = Tc[i][r];
}

// Inputs of one chunk for k_prep, prefetched into registers: K rows (bf16;
// thread t: row (t + 256 j) / 16, columns 8 ((t + 256 j) % 16) .. + 8; fp32 K
// is read from HBM by the gram itself) and g, beta of token lane.
template <typename IO> struct PrepIn;
template <> struct PrepIn<bf16> { u32x4 k[4]; float g, b; };
template <> struct PrepIn<float> { float g, b; };

// Loads are unconditional (rows past the end of the sequence read its last
// row) and the values of those rows are replaced by zeros afterwards.
template <typename IO>
__device__ __forceinline__ void prep_fetch(PrepIn<IO>& r, const Params& p, size_t tok0, int nvalid, int h, int hq) {
    const size_t ts = (size_t)p.h_qk * DK;
    if constexpr (Io<IO>::kExact) {
        const IO* kb = static_cast<const IO*>(p.k) + tok0 * ts + (size_t)hq * DK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pc = threadIdx.x + NTHR * j, row = pc >> 4, c8 = (pc & 15) * 8;
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 kv = *reinterpret_cast<const u32x4*>(kb + (size_t)min(row, nvalid - 1) * ts + c8);
            r.k[j] = row < nvalid ? kv : z;
        }
    }
    const int lane = lane_id();
    const size_t idx = (tok0 + min(lane, nvalid - 1)) * (size_t)p.h_v + h;
    const float g = p.g[idx], b = p.beta[idx];
    r.g = lane < nvalid ? g : 0.f;
    r.b = lane < nvalid ? b : 0.f;
}

// Grid (groups of p.prep_cpw consecutive chunk slots, value heads); each
// workgroup walks its chunks, fetching the next chunk's inputs while it works
// on the current one. Per (chunk slot, value head), block b = slot h_v + h:
//   prep_T + b t_stride: T diag(beta) split into bf16 hi and lo, [part][row][k]
//     (2 x 64 x 64), the k (column) axis permuted within each group of 16 as
//     the chain kernels' LDS operands are (zeros above the diagonal);
//   prep_GB + b gb_stride: gamma (64 fp32), then beta (64 fp32).
template <typename IO>
__global__ __launch_bounds__(NTHR, 2) void k_prep(Params p) {
    constexpr bool EX = Io<IO>::kExact;
    __shared__ PrepSmem<EX> sm;
    const int h = blockIdx.y, hq = h / p.group, wave = wave_id(), lane = lane_id();
    const int s0 = blockIdx.x * p.prep_cpw, s1 = min(s0 + p.prep_cpw, p.n_chunks);
    const size_t ts = (size_t)p.h_qk * DK;
    int seq, c, len;
    size_t tok_s;
    if (s0 >= s1 || !locate_chunk(p, s0, seq, c, len, tok_s)) return;
    size_t tok0 = tok_s + (size_t)c * CH;
    int nvalid = min(CH, len - c * CH);
    PrepIn<IO> nxt;
    prep_fetch<IO>(nxt, p, tok0, nvalid, h, hq);
    if (p.sink) {   // (null for the low-level entry, which has no workspace)
        // the loop body's stores (gamma, beta; T) come after its loads; the same
        // stores to the scratch line here make the loop's entry look alike, so
        // that the wait at its head covers the loads only
        float* sk = p.sink + 32 * lane;
        sk[0] = 0.f;
        sk[1] = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(sk + 4 * i) = u32x4{0u, 0u, 0u, 0u};
    }
    for (int slot = s0; slot < s1; ++slot) {
        const size_t tok_cur = tok0;
        const int nv_cur = nvalid;
        const IO* krow0 = static_cast<const IO*>(p.k) + tok_cur * ts + (size_t)hq * DK;
        if constexpr (EX) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int pc = threadIdx.x + NTHR * j, row = pc >> 4, c8 = (pc & 15) * 8;
                *reinterpret_cast<u32x2*>(sm.k_rm + row * LDQ + pk(c8)) = u32x2{nxt.k[j][0], nxt.k[j][1]};
                *reinterpret_cast<u32x2*>(sm.k_rm + row * LDQ + pk(c8 + 4)) = u32x2{nxt.k[j][2], nxt.k[j][3]};
            }
        }
        {   // every wave scans and writes the same values (no branch in the loop)
            const float gam = wave_scan(nxt.g);
            sm.gam[lane] = gam;
            sm.beta[lane] = nxt.b;
            float* gb = p.prep_GB + ((size_t)slot * p.h_v + h) * (size_t)p.gb_stride;
            gb[lane] = gam;
            gb[CH + lane] = nxt.b;
        }
        __syncthreads();
        // always a prefetch (the last slot fetches itself again), so that every
        // iteration has the same memory operations and the compiler's waits on
        // them stay exact across the loop
        if (locate_chunk(p, min(slot + 1, s1 - 1), seq, c, len, tok_s)) {
            tok0 = tok_s + (size_t)c * CH;
            nvalid = min(CH, len - c * CH);
        }
        prep_fetch<IO>(nxt, p, tok0, nvalid, h, hq);
        // the ten tiles: three per wave, the last wave takes one
        if (wave < 3) gram_a<IO, 3>(sm, krow0, ts, nv_cur, wave, 3);
        else gram_a<IO, 1>(sm, krow0, ts, nv_cur, 9, 1);
        __syncthreads();
        inv_diag<EX>(sm);
        // the diagonal blocks this wave reads next are the ones it just wrote
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        switch (wave) {
            case 0: inv_col<0, EX>(sm); break;
            case 1: inv_col<1, EX>(sm); break;
            case 2: inv_col<2, EX>(sm); break;
            default: inv_col<3, EX>(sm); break;
        }
        __syncthreads();
        // (the next chunk's LDS writes touch k_rm and the gate arrays only, all
        // read before the previous barrier; T is rewritten after two more).
        // T diag(beta): thread t takes row t / 4 and the 16 physical k
        // positions 16 (t % 4) ..; physical 4-blocks 0..3 of a 16-group hold
        // logical blocks 0, 2, 1, 3.
        bf16* Tg = reinterpret_cast<bf16*>(p.prep_T + ((size_t)slot * p.h_v + h) * (size_t)p.t_stride);
        {
            const int row = threadIdx.x >> 2, g16 = 16 * (threadIdx.x & 3);
            const float* tr = sm.t + row * LDF + g16;
            const float* br = sm.beta + g16;
            const f32x4 b0 = *reinterpret_cast<const f32x4*>(tr) * *reinterpret_cast<const f32x4*>(br);
            const f32x4 b1 = *reinterpret_cast<const f32x4*>(tr + 8) * *reinterpret_cast<const f32x4*>(br + 8);
            const f32x4 b2 = *reinterpret_cast<const f32x4*>(tr + 4) * *reinterpret_cast<const f32x4*>(br + 4);
            const f32x4 b3 = *reinterpret_cast<const f32x4*>(tr + 12) * *reinterpret_cast<const f32x4*>(br + 12);
            bf16x4 h0, l0, h1, l1, h2, l2, h3, l3;
            split4(b0, h0, l0);
            split4(b1, h1, l1);
            split4(b2, h2, l2);
            split4(b3, h3, l3);
            const bf16x8 hA = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 hB = __builtin_shufflevector(h2, h3, 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 lA = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 lB = __builtin_shufflevector(l2, l3, 0, 1, 2, 3, 4, 5, 6, 7);
            *reinterpret_cast<bf16x8*>(Tg + row * CH + g16) = hA;
            *reinterpret_cast<bf16x8*>(Tg + row * CH + g16 + 8) = hB;
            *reinterpret_cast<bf16x8*>(Tg + (CH + row) * CH + g16) = lA;
            *reinterpret_cast<bf16x8*>(Tg + (CH + row) * CH + g16 + 8) = lB;
        }
    }
}

// ----------------------------------------------------------------------------
// The chain kernels. For a chunk with incoming state S, the same quantities as
// the WY form, evaluated without W and U:
//   Y  = V - diag(e^gamma) K S                    (the prediction error)
//   V' = T diag(beta) Y                           (= U - W S)
//   O  = diag(e^gamma) Q S + P V',  P = (Q K^T) o D  (both times the scale)
//   S <- e^gamma_C S + K^T diag(e^(gamma_C - gamma)) V'
// so each wave needs, besides its own state columns, only K, K^T, V^T, Q, P
// and T from LDS, and the products of different waves never meet.

template <bool EX>
struct __attribute__((aligned(16))) ChainSmem {
    bf16 q_hi[CH * LDQ];                  // Q token-major, d_k permuted
    bf16 q_lo[EX ? 8 : CH * LDQ];
    bf16 k_hi[CH * LDQ];                  // K token-major, d_k permuted
    bf16 k_lo[EX ? 8 : CH * LDQ];
    bf16 kt_hi[DK * LDKT];                // K^T: [d_k][token permuted]
    bf16 kt_lo[EX ? 8 : DK * LDKT];
    bf16 vt[EX ? DK * LDKT : 8];          // V^T (bf16 inputs; fp32 V is read from HBM)
    bf16 p[2 * CH * LDP];                 // P = (Q K^T) o D, causal: hi rows, then lo rows
    bf16 t[2 * CH * LDP];                 // T diag(beta): hi rows, then lo rows (token axis permuted)
    float gam[CH];                        // gamma
    float eg[CH];                         // exp(gamma)
    float egs[CH];                        // scale exp(gamma)
    float egc[CH];                        // exp(gamma_C - gamma)
    float red[8];                         // red[0] = exp(gamma_C); per-chunk gate sums
};

// One chunk's inputs in registers between the global loads and the LDS
// stores, so that the next chunk's loads overlap the current chunk's work.
// K, V: thread t holds token rows 4 (t / 16) + j (j < 4), columns
// 8 (t % 16) .. + 8 (sixteen lanes cover one 256-byte row, and a lane holds
// four consecutive tokens of each of its columns, written to K^T / V^T as
// 8-byte stores). Q: rows t / 16 + 16 j, same columns. T: four 16-byte pieces
// (t + 256 j) of its [part][row][64] image. Gates: gamma, beta of token lane.
template <typename IO> struct Chunk;
template <> struct Chunk<bf16> { u32x4 k[4], v[4], q[4], t[4]; float gl, bl; };
template <> struct Chunk<float> { f32x4 k[8], q[8]; u32x4 t[4]; float gl, bl; };

// Rows past the end of the sequence (last chunk only) read its last row
// again: their values never matter, since such tokens carry beta = 0, which
// zeroes their columns of T diag(beta), so their K, V and Q rows reach
// neither a valid output nor the state. Addresses are a wave-uniform base plus
// 32-bit lane offsets. The chunk loops issue the same loads and stores in
// every iteration (no conditional memory operations), so that the compiler's
// waits on them stay exact across the loop instead of draining every
// outstanding operation.
template <typename IO, bool WANT_Q, bool WANT_V>
__device__ __forceinline__ void fetch_chunk(Chunk<IO>& r, const Params& p, size_t tok0, int nvalid, int h,
                                            int hq, int slot) {
    constexpr bool EX = Io<IO>::kExact;
    const int t = threadIdx.x, m = t >> 4, c8 = (t & 15) * 8;
    const int ts = p.h_qk * DK, tsv = p.h_v * DK;
    const IO* kb = static_cast<const IO*>(p.k) + tok0 * (size_t)ts + (size_t)hq * DK;
    const IO* qb = static_cast<const IO*>(p.q) + tok0 * (size_t)ts + (size_t)hq * DK;
    const IO* vb = static_cast<const IO*>(p.v) + tok0 * (size_t)tsv + (size_t)h * DK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int rk = min(4 * m + j, nvalid - 1), rq = min(m + 16 * j, nvalid - 1);
        const unsigned ok_k = (unsigned)(rk * ts + c8), ok_v = (unsigned)(rk * tsv + c8);
        const unsigned ok_q = (unsigned)(rq * ts + c8);
        if constexpr (EX) {
            r.k[j] = *reinterpret_cast<const u32x4*>(kb + ok_k);
            if (WANT_V) r.v[j] = *reinterpret_cast<const u32x4*>(vb + ok_v);
            if (WANT_Q) r.q[j] = *reinterpret_cast<const u32x4*>(qb + ok_q);
        } else {
            r.k[2 * j] = *reinterpret_cast<const f32x4*>(kb + ok_k);
            r.k[2 * j + 1] = *reinterpret_cast<const f32x4*>(kb + ok_k + 4);
            if (WANT_Q) {
                r.q[2 * j] = *reinterpret_cast<const f32x4*>(qb + ok_q);
                r.q[2 * j + 1] = *reinterpret_cast<const f32x4*>(qb + ok_q + 4);
            }
        }
    }
    const size_t blk = (size_t)slot * p.h_v + h;
    const u32x4* Tg = reinterpret_cast<const u32x4*>(p.prep_T + blk * (size_t)p.t_stride);
#pragma unroll
    for (int j = 0; j < 4; ++j) r.t[j] = Tg[t + NTHR * j];
    const float* gb = p.prep_GB + blk * (size_t)p.gb_stride;
    r.gl = gb[lane_id()];
    r.bl = gb[CH + lane_id()];
}

// Two bf16 of the same column from two rows packed into one 32-bit word.
__device__ __forceinline__ unsigned int pack_col(const u32x4& a, const u32x4& b, int e) {
    const unsigned int wa = a[e >> 1], wb = b[e >> 1];
    return (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
}

// Writes a fetched chunk to LDS: K token-major and transposed (four
// consecutive tokens of a column per 8-byte store), V^T, Q, T and the gate
// factors (tokens past the end of the sequence have g = beta = 0).
template <typename IO, bool WANT_Q, bool WANT_V>
__device__ __forceinline__ void stage_chunk(ChainSmem<Io<IO>::kExact>& sm, const Chunk<IO>& r, float scale) {
    constexpr bool EX = Io<IO>::kExact;
    const int t = threadIdx.x, lane = lane_id(), m = t >> 4, c8 = (t & 15) * 8;
    {   // every wave writes the same values (no branch in the chunk loop)
        const float gc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r.gl), 63));
        const float es = __expf(r.gl);
        sm.gam[lane] = r.gl;
        sm.eg[lane] = es;
        sm.egs[lane] = es * scale;
        sm.egc[lane] = __expf(gc - r.gl);
        sm.red[0] = __expf(gc);
    }
    const int tp = pk(4 * m);   // the four tokens stay contiguous under the permutation
    if constexpr (EX) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 4 * m + j;
            *reinterpret_cast<u32x2*>(sm.k_hi + row * LDQ + pk(c8)) = u32x2{r.k[j][0], r.k[j][1]};
            *reinterpret_cast<u32x2*>(sm.k_hi + row * LDQ + pk(c8 + 4)) = u32x2{r.k[j][2], r.k[j][3]};
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = c8 + e;
            *reinterpret_cast<u32x2*>(sm.kt_hi + trow(c) * LDKT + tp) =
                u32x2{pack_col(r.k[0], r.k[1], e), pack_col(r.k[2], r.k[3], e)};
            if (WANT_V)
                *reinterpret_cast<u32x2*>(sm.vt + trow(c) * LDKT + tp) =
                    u32x2{pack_col(r.v[0], r.v[1], e), pack_col(r.v[2], r.v[3], e)};
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = 4 * m + j;
            bf16x4 ah, al, bh, bl;
            split4(r.k[2 * j], ah, al);
            split4(r.k[2 * j + 1], bh, bl);
            *reinterpret_cast<bf16x4*>(sm.k_hi + row * LDQ + pk(c8)) = ah;
            *reinterpret_cast<bf16x4*>(sm.k_lo + row * LDQ + pk(c8)) = al;
            *reinterpret_cast<bf16x4*>(sm.k_hi + row * LDQ + pk(c8 + 4)) = bh;
            *reinterpret_cast<bf16x4*>(sm.k_lo + row * LDQ + pk(c8 + 4)) = bl;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = c8 + e;
            f32x4 x;
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = r.k[2 * j + (e >> 2)][e & 3];
            bf16x4 xh, xl;
            split4(x, xh, xl);
            *reinterpret_cast<bf16x4*>(sm.kt_hi + trow(c) * LDKT + tp) = xh;
            *reinterpret_cast<bf16x4*>(sm.kt_lo + trow(c) * LDKT + tp) = xl;
        }
    }
    if (WANT_Q) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = m + 16 * j;
            const int o0 = row * LDQ + pk(c8), o1 = row * LDQ + pk(c8 + 4);
            if constexpr (EX) {
                *reinterpret_cast<u32x2*>(sm.q_hi + o0) = u32x2{r.q[j][0], r.q[j][1]};
                *reinterpret_cast<u32x2*>(sm.q_hi + o1) = u32x2{r.q[j][2], r.q[j][3]};
            } else {
                bf16x4 ah, al, bh, bl;
                split4(r.q[2 * j], ah, al);
                split4(r.q[2 * j + 1], bh, bl);
                *reinterpret_cast<bf16x4*>(sm.q_hi + o0) = ah;
                *reinterpret_cast<bf16x4*>(sm.q_lo + o0) = al;
                *reinterpret_cast<bf16x4*>(sm.q_hi + o1) = bh;
                *reinterpret_cast<bf16x4*>(sm.q_lo + o1) = bl;
            }
        }
    }
    // T: piece t + 256 j of the [part][row][64] image -> row part * 64 + row of sm.t
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int pc = t + NTHR * j, prow = pc >> 3, k8 = (pc & 7) * 8;
        *reinterpret_cast<u32x4*>(sm.t + prow * LDP + k8) = r.t[j];
    }
}

// scale P, P = (Q K^T) o D, on the ten lower 16x16 tiles (16x16x32 MFMA, each tile
// computed transposed so that a lane holds four consecutive columns of one
// row), split into hi/lo; the two upper tiles inside the diagonal 32-blocks,
// which the P V' product reads, are zeroed. Jobs first, first + stride, ...
template <bool EX, int NJOB>
__device__ void gram_p(ChainSmem<EX>& sm, int first, int stride, float scale) {
    const int lane = lane_id(), n = lane & 15, g4 = lane >> 4;
    f32x4 acc[NJOB];
    int bi[NJOB], bj[NJOB];
#pragma unroll
    for (int t = 0; t < NJOB; ++t) {
        lower_tile(first + stride * t, bi[t], bj[t]);
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int kb = 32 * ks + 8 * g4;
#pragma unroll
        for (int t = 0; t < NJOB; ++t) {
            const int ra = 16 * bj[t] + n, rb = 16 * bi[t] + n;   // A: K rows of bj; B: Q rows of bi
            const bf16x8 a = lds_row8(sm.k_hi + ra * LDQ + kb);
            const bf16x8 b = lds_row8(sm.q_hi + rb * LDQ + kb);
            acc[t] = mma16k32(a, b, acc[t]);
            if (!EX) {
                acc[t] = mma16k32(a, lds_row8(sm.q_lo + rb * LDQ + kb), acc[t]);
                acc[t] = mma16k32(lds_row8(sm.k_lo + ra * LDQ + kb), b, acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NJOB; ++t) {
        const int i = 16 * bi[t] + n, j0 = 16 * bj[t] + 4 * g4;   // row i, columns j0 .. j0 + 3
        const float gi = sm.gam[i];
        const f32x4 gj = *reinterpret_cast<const f32x4*>(sm.gam + j0);
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (i >= j0 + r) ? scale * __expf(gi - gj[r]) * acc[t][r] : 0.f;
        bf16x4 hi, lo;
        split4(v, hi, lo);
        *reinterpret_cast<bf16x4*>(sm.p + i * LDP + pk(j0)) = hi;
        *reinterpret_cast<bf16x4*>(sm.p + (CH + i) * LDP + pk(j0)) = lo;
    }
}

__device__ __forceinline__ void zero_p_tile(bf16* p, int bi, int bj) {
    // lane: row 16 bi + lane / 4, columns 16 bj + 4 (lane % 4) .. + 4, hi and lo
    const int lane = lane_id(), i = 16 * bi + (lane >> 2), j0 = 16 * bj + 4 * (lane & 3);
    *reinterpret_cast<u32x2*>(p + i * LDP + pk(j0)) = u32x2{0u, 0u};
    *reinterpret_cast<u32x2*>(p + (CH + i) * LDP + pk(j0)) = u32x2{0u, 0u};
}

// The state as hi/lo B operands, one pair per 16-row k step.
struct SplitS {
    bf16x8 hi[8], lo[8];
};
__device__ __forceinline__ void split_state(const f32x16 S[4], SplitS& ss) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) split_half(S[ks >> 1], ks & 1, ss.hi[ks], ss.lo[ks]);
}

// V' = T diag(beta) (V - diag(e^gamma) K S) for this wave's columns.
// KS: A = K rows (token-major LDS), B = S; Y in fp32 on the accumulators
// (V from V^T in LDS, four consecutive tokens per 8-byte read, or from HBM
// for fp32 inputs); then (T diag(beta)) Y with both split hi/lo (T is lower
// triangular: token tile 0 needs k steps 0..1).
template <typename IO, bool WANT_V>
__device__ void chain_vp(const ChainSmem<Io<IO>::kExact>& sm, const SplitS& ss, const IO* vcol, size_t ts,
                         int nvalid, f32x16 Vp[2]) {
    constexpr bool EX = Io<IO>::kExact;
    const int lane = lane_id(), col = lane & 31, h = lane >> 5, n = 32 * wave_id() + col;
    f32x16 KS[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        bf16x8 kh[2], kl[2];
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            kh[ti] = lds_op16(sm.k_hi + (32 * ti + col) * LDQ + 16 * ks + 8 * h);
            if (!EX) kl[ti] = lds_op16(sm.k_lo + (32 * ti + col) * LDQ + 16 * ks + 8 * h);
        }
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) KS[ti] = mma32(kh[ti], ss.hi[ks], KS[ti]);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) KS[ti] = mma32(kh[ti], ss.lo[ks], KS[ti]);
        if (!EX) {
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) KS[ti] = mma32(kl[ti], ss.hi[ks], KS[ti]);
        }
    }
    // Y = V - e^gamma KS on rows 32 ti + 8 q + 4 h + (0..3)
    const int vrow = trow(n) * LDKT;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r0 = 32 * ti + 8 * q + 4 * h;
            const f32x4 eg = *reinterpret_cast<const f32x4*>(sm.eg + r0);
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (WANT_V) {
                if constexpr (EX) {
                    const u32x2 vv = *reinterpret_cast<const u32x2*>(sm.vt + vrow + pk(r0));
                    v = f32x4{__uint_as_float(vv[0] << 16), __uint_as_float(vv[0] & 0xffff0000u),
                              __uint_as_float(vv[1] << 16), __uint_as_float(vv[1] & 0xffff0000u)};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = (r0 + e < nvalid) ? (float)vcol[(size_t)(r0 + e) * ts] : 0.f;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) KS[ti][4 * q + e] = fmaf(-eg[e], KS[ti][4 * q + e], v[e]);
        }
    Vp[0] = Vp[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        bf16x8 yh, yl;
        split_half(KS[ks >> 1], ks & 1, yh, yl);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            if (ti == 0 && ks >= 2) continue;
            const bf16x8 th = lds_op16(sm.t + (32 * ti + col) * LDP + 16 * ks + 8 * h);
            const bf16x8 tl = lds_op16(sm.t + (CH + 32 * ti + col) * LDP + 16 * ks + 8 * h);
            Vp[ti] = mma32(th, yh, Vp[ti]);
            Vp[ti] = mma32(th, yl, Vp[ti]);
            Vp[ti] = mma32(tl, yh, Vp[ti]);
        }
    }
}

// O^T = scale S^T (diag(e^gamma) Q)^T for this wave's d_v rows (token columns): the
// split state serves as the A operand unchanged (the MFMA's A and B register
// layouts mirror each other). Then (chain_pv_out, after P is in LDS) the
// causal part V'^T P^T and the store: a lane holds four consecutive d_v of
// one token per accumulator group, written as one 8- (bf16) or 16-byte
// (fp32) store; rows >= nvalid are not written.
template <bool EX>
__device__ void chain_qs(const ChainSmem<EX>& sm, const SplitS& ss, f32x16 O[2]) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
    O[0] = O[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        bf16x8 qh[2], ql[2];
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            qh[ti] = lds_op16(sm.q_hi + (32 * ti + col) * LDQ + 16 * ks + 8 * h);
            if (!EX) ql[ti] = lds_op16(sm.q_lo + (32 * ti + col) * LDQ + 16 * ks + 8 * h);
        }
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) O[ti] = mma32(ss.hi[ks], qh[ti], O[ti]);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) O[ti] = mma32(ss.lo[ks], qh[ti], O[ti]);
        if (!EX) {
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) O[ti] = mma32(ss.hi[ks], ql[ti], O[ti]);
        }
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) O[ti] *= sm.egs[32 * ti + col];
}

template <typename IO>
__device__ void chain_pv_out(const ChainSmem<Io<IO>::kExact>& sm, const f32x16 Vp[2], f32x16 O[2], IO* orow0,
                             size_t ts, int nvalid, float* sink) {
    constexpr bool EX = Io<IO>::kExact;
    const int lane = lane_id(), col = lane & 31, h = lane >> 5, w = wave_id();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {  // P is causal: token tile 0 needs k steps 0..1
        bf16x8 vh, vl;
        split_half(Vp[ks >> 1], ks & 1, vh, vl);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            if (ti == 0 && ks >= 2) continue;
            const bf16x8 ph = lds_op16(sm.p + (32 * ti + col) * LDP + 16 * ks + 8 * h);
            const bf16x8 pl = lds_op16(sm.p + (CH + 32 * ti + col) * LDP + 16 * ks + 8 * h);
            O[ti] = mma32(vh, ph, O[ti]);
            O[ti] = mma32(vl, ph, O[ti]);
            O[ti] = mma32(vh, pl, O[ti]);
        }
    }
    // rows past the end of the sequence are written to a scratch line (every
    // chunk issues the same stores; see fetch_chunk)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
        const int r = 32 * ti + col;
        IO* dst = (r < nvalid) ? orow0 + (size_t)r * ts + 32 * w + 4 * h
                               : reinterpret_cast<IO*>(sink + 32 * lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 x = f32x4{O[ti][4 * q], O[ti][4 * q + 1], O[ti][4 * q + 2], O[ti][4 * q + 3]};
            if constexpr (EX) {
                *reinterpret_cast<u32x2*>(dst + 8 * q) = u32x2{pack_rne(x[0], x[1]), pack_rne(x[2], x[3])};
            } else {
                *reinterpret_cast<f32x4*>(dst + 8 * q) = x;
            }
        }
    }
}

// S <- e^gamma_C S + K^T diag(e^(gamma_C - gamma)) V' (Vp is scaled in place).
template <bool EX>
__device__ void chain_state(const ChainSmem<EX>& sm, f32x16 S[4], f32x16 Vp[2]) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 e = *reinterpret_cast<const f32x4*>(sm.egc + 32 * ti + 8 * q + 4 * h);
#pragma unroll
            for (int r = 0; r < 4; ++r) Vp[ti][4 * q + r] *= e[r];
        }
    const float ec = sm.red[0];
#pragma unroll
    for (int t = 0; t < 4; ++t) S[t] *= ec;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        bf16x8 vh, vl;
        split_half(Vp[ks >> 1], ks & 1, vh, vl);
        bf16x8 kh[4], kl[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            kh[t] = lds_op16(sm.kt_hi + trow(32 * t + col) * LDKT + 16 * ks + 8 * h);
            if (!EX) kl[t] = lds_op16(sm.kt_lo + trow(32 * t + col) * LDKT + 16 * ks + 8 * h);
        }
        // four independent chains: each tile is touched once per pass
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t] = mma32(kh[t], vh, S[t]);
#pragma unroll
        for (int t = 0; t < 4; ++t) S[t] = mma32(kh[t], vl, S[t]);
        if (!EX) {
#pragma unroll
            for (int t = 0; t < 4; ++t) S[t] = mma32(kl[t], vh, S[t]);
        }
    }
}

// ----------------------------------------------------------------------------
// State tiles in registers: wave w holds columns [32w, 32w + 32) of a
// [128][128] row-major fp32 matrix, as four 32-row accumulator tiles.

__device__ void load_state(const float* Sg, f32x16 S[4]) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5, c = 32 * wave_id() + col;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[t][i] = Sg[(32 * t + acc_row(i, h)) * DK + c];
}
__device__ void store_state(float* Sg, const f32x16 S[4]) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5, c = 32 * wave_id() + col;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) Sg[(32 * t + acc_row(i, h)) * DK + c] = S[t][i];
}
__device__ void zero_state(f32x16 S[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) S[t] = f32x16{};
}
__device__ void identity_state(f32x16 S[4]) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5, c = 32 * wave_id() + col;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[t][i] = (32 * t + acc_row(i, h) == c) ? 1.f : 0.f;
}

__device__ __forceinline__ size_t state_off(int idx, int h_v, int h) {
    return ((size_t)idx * h_v + h) * (size_t)DK * DK;
}

// Runs chunks [c_lo, c_hi) of sequence loc from the state S (no outputs):
// the warm-up scan, the H chain (WANT_V) or the M chain (V = 0, S starts at I).
template <typename IO, bool WANT_V>
__device__ void scan_chunks(ChainSmem<Io<IO>::kExact>& sm, const Params& p, const SegLoc& loc, int h, int hq,
                            int c_lo, int c_hi, f32x16 S[4]) {
    constexpr bool EX = Io<IO>::kExact;
    const size_t ts_v = (size_t)p.h_v * DK;
    Chunk<IO> nxt;
    if (c_lo < c_hi)
        fetch_chunk<IO, false, WANT_V>(nxt, p, loc.tok0 + (size_t)c_lo * CH, min(CH, loc.len - c_lo * CH), h, hq,
                                       loc.chunk_base + c_lo);
    for (int c = c_lo; c < c_hi; ++c) {
        const size_t tok0 = loc.tok0 + (size_t)c * CH;
        const int nvalid = min(CH, loc.len - c * CH);
        stage_chunk<IO, false, WANT_V>(sm, nxt, 1.f);
        __syncthreads();
        {   // always a prefetch (the last chunk fetches itself again): see fetch_chunk
            const int cn = min(c + 1, c_hi - 1);
            fetch_chunk<IO, false, WANT_V>(nxt, p, loc.tok0 + (size_t)cn * CH, min(CH, loc.len - cn * CH), h, hq,
                                           loc.chunk_base + cn);
        }
        f32x16 Vp[2];
        {
            SplitS ss;
            split_state(S, ss);
            const IO* vcol = static_cast<const IO*>(p.v) + tok0 * ts_v + (size_t)h * DK + 32 * wave_id() + (lane_id() & 31);
            chain_vp<IO, WANT_V>(sm, ss, vcol, ts_v, nvalid, Vp);
        }
        chain_state<EX>(sm, S, Vp);
        __syncthreads();
    }
}

// ----------------------------------------------------------------------------
// Kernels

// Low-level chunk preparation, second half: W = (T diag(beta)) diag(e^gamma) K
// and U = (T diag(beta)) V of every (chunk, value head), from T diag(beta)
// (split) and gamma, beta, which k_prep left in the chunk's W_out and U_out
// blocks. Wave w produces columns [32w, 32w + 32) of both.
template <typename IO>
__global__ __launch_bounds__(NTHR) void k_wu(Params p) {
    constexpr bool EX = Io<IO>::kExact;
    __shared__ ChainSmem<EX> sm;
    const int h = blockIdx.y, hq = h / p.group;
    int seq, c, len;
    size_t tok_s;
    if (!locate_chunk(p, blockIdx.x, seq, c, len, tok_s)) return;
    const size_t tok0 = tok_s + (size_t)c * CH;
    const int nvalid = min(CH, len - c * CH);
    float gl;
    {
        Chunk<IO> r;
        fetch_chunk<IO, false, true>(r, p, tok0, nvalid, h, hq, blockIdx.x);
        stage_chunk<IO, false, true>(sm, r, 1.f);
        gl = r.gl;
    }
    __syncthreads();   // every read of T, gamma and beta is done before W and U overwrite them
    const int lane = lane_id(), col = lane & 31, hh = lane >> 5, w = wave_id(), n = 32 * w + col;
    const size_t ts_v = (size_t)p.h_v * DK, ts_k = (size_t)p.h_qk * DK;
    const IO* vcol = static_cast<const IO*>(p.v) + tok0 * ts_v + (size_t)h * DK + n;
    const IO* kcol = static_cast<const IO*>(p.k) + tok0 * ts_k + (size_t)hq * DK + n;
    f32x16 W[2] = {f32x16{}, f32x16{}}, U[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        // B operands: column n, tokens 16 ks + kperm(hh, e) (K scaled by e^gamma of the token)
        const f32x4 eg0 = *reinterpret_cast<const f32x4*>(sm.eg + 16 * ks + 4 * hh);
        const f32x4 eg1 = *reinterpret_cast<const f32x4*>(sm.eg + 16 * ks + 8 + 4 * hh);
        // K and V at those tokens: exact bf16 from LDS, or fp32 from HBM
        f32x4 k0, k1, v0, v1;
        if constexpr (EX) {
            const bf16x8 kh = lds_op16(sm.kt_hi + trow(n) * LDKT + 16 * ks + 8 * hh);
            const bf16x8 vh = lds_op16(sm.vt + trow(n) * LDKT + 16 * ks + 8 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                k0[e] = (float)kh[e];
                k1[e] = (float)kh[4 + e];
                v0[e] = (float)vh[e];
                v1[e] = (float)vh[4 + e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t0 = 16 * ks + 4 * hh + e, t1 = t0 + 8;
                k0[e] = t0 < nvalid ? (float)kcol[(size_t)t0 * ts_k] : 0.f;
                k1[e] = t1 < nvalid ? (float)kcol[(size_t)t1 * ts_k] : 0.f;
                v0[e] = t0 < nvalid ? (float)vcol[(size_t)t0 * ts_v] : 0.f;
                v1[e] = t1 < nvalid ? (float)vcol[(size_t)t1 * ts_v] : 0.f;
            }
        }
        k0 *= eg0;
        k1 *= eg1;
        bf16x4 a0, a1, b0, b1;
        bf16x8 kbh, kbl, vbh, vbl;
        split4(k0, a0, b0);
        split4(k1, a1, b1);
        kbh = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        kbl = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        split4(v0, a0, b0);
        split4(v1, a1, b1);
        vbh = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        vbl = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            if (ti == 0 && ks >= 2) continue;
            const bf16x8 th = lds_op16(sm.t + (32 * ti + col) * LDP + 16 * ks + 8 * hh);
            const bf16x8 tl = lds_op16(sm.t + (CH + 32 * ti + col) * LDP + 16 * ks + 8 * hh);
            W[ti] = mma32(th, kbh, W[ti]);
            W[ti] = mma32(th, kbl, W[ti]);
            W[ti] = mma32(tl, kbh, W[ti]);
            U[ti] = mma32(th, vbh, U[ti]);
            U[ti] = mma32(th, vbl, U[ti]);
            U[ti] = mma32(tl, vbh, U[ti]);
        }
    }
    const size_t base = ((size_t)blockIdx.x * p.h_v + h) * CH;
    if (w == 0) p.prep_gamma[base + lane] = gl;
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const size_t r = base + 32 * ti + acc_row(i, hh);
            p.prep_W[r * DK + n] = W[ti][i];
            p.prep_U[r * DK + n] = U[ti][i];
        }
}

// The map M of a segment, written for the combine kernel: split into hi/lo
// bf16 and laid out as that kernel's MFMA A operands, so that its loads are
// contiguous and it does no splitting on its sequential path. Element
// M[r][k] goes to ((((r / 32) * 8 + k / 16) * 2 + part) * 64 + lane) * 8 + e
// with lane = r % 32 + 32 h, k % 16 = kperm(h, e), part 0 = hi, 1 = lo
// (64 KiB per map). The chunk loop's LDS serves as the staging buffer; the
// caller's chain is finished (behind a barrier) when this starts.
__device__ void store_m_operand(bf16* buf, const f32x16 S[4], bf16* dst) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5, w = wave_id();
    const int kk = col & 15, ks = 2 * w + (col >> 4);
    const int hh = (kk >> 2) & 1, e = (kk & 3) | ((kk & 8) >> 1);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r2 = acc_row(i, h);   // row within the 32-row block t
            const int idx = (((t * 8 + ks) * 2) * 64 + r2 + 32 * hh) * 8 + e;
            bf16 hi, lo;
            split1(S[t][i], hi, lo);
            buf[idx] = hi;
            buf[idx + 64 * 8] = lo;
        }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 16; ++it) {
        const int off = (threadIdx.x + NTHR * it) * 8;
        *reinterpret_cast<u32x4*>(dst + off) = *reinterpret_cast<const u32x4*>(buf + off);
    }
}

// Warm-up or exact segment map for the boundary before segment s >= 1.
// blockIdx.x = 2 * segment slot + part; part 0: warm-up state or H, part 1: M.
template <typename IO>
__global__ __launch_bounds__(NTHR) void k_cp_prep(Params p) {
    __shared__ ChainSmem<Io<IO>::kExact> sm;
    const int slot = blockIdx.x >> 1, part = blockIdx.x & 1, h = blockIdx.y, hq = h / p.group;
    const SegLoc loc = locate_segment(p, slot);
    if (loc.seq < 0 || loc.s == 0) return;
    const int a = loc.s * p.L;  // first chunk of segment s

    // Gate-driven choice: warm up iff the log-decay over the window of w chunks
    // before the boundary is at most log(noise floor) (or the window reaches
    // the sequence start, where the warm-up is exact). The warm-up then scans
    // the shortest run of chunks before the boundary (wq <= w) whose log-decay
    // is already at most log(noise floor); the state it misses is bounded by
    // that decay times the state at the run's start.
    // warm: 0 exact map, 1 warm-up (decayed below the floor, or forced), 2 warm-up
    // from the sequence start (exact)
    int warm, wq = p.w;
    if (p.cp_mode == kCpExact) {
        warm = 0;
    } else if (a - p.w <= 0) {
        warm = 2;
        wq = a;
    } else {
        // chunk a - 1 - j (a full chunk: only a sequence's last chunk is short) -> red[j]
        const int wave = wave_id(), lane = lane_id();
        for (int j = wave; j < p.w; j += 4) {
            float s = p.g[(loc.tok0 + (size_t)(a - 1 - j) * CH + lane) * (size_t)p.h_v + h];
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
            if (lane == 0) sm.red[j] = s;
        }
        __syncthreads();
        float cum = 0.f;
        int found = 0;
        for (int j = 0; j < p.w && !found; ++j) {
            cum += sm.red[j];
            if (cum <= p.log_eps) found = j + 1;
        }
        if (found) {
            warm = 1;
            wq = found;
        } else {
            warm = (p.cp_mode == kCpWarmup) ? 1 : 0;
        }
        __syncthreads();
    }
    if (part == 0 && threadIdx.x == 0) p.warm[(size_t)(loc.seg_base + loc.s) * p.h_v + h] = warm;
    if (warm && part == 1) return;
    // the map of segment 0 is only applied to a nonzero initial state
    if (!warm && part == 1 && loc.s == 1 && !p.s_init) return;

    f32x16 S[4];
    float* dst;
    if (warm) {
        const int c_lo = a - wq;
        if (c_lo == 0 && p.s_init) load_state(p.s_init + state_off(loc.seq, p.h_v, h), S);
        else zero_state(S);
        scan_chunks<IO, true>(sm, p, loc, h, hq, c_lo, a, S);
        dst = p.seg_state + state_off(loc.seg_base + loc.s, p.h_v, h);
    } else if (part == 0) {
        zero_state(S);
        scan_chunks<IO, true>(sm, p, loc, h, hq, a - p.L, a, S);
        dst = p.seg_H + state_off(loc.seg_base + loc.s - 1, p.h_v, h);
    } else {
        identity_state(S);
        scan_chunks<IO, false>(sm, p, loc, h, hq, a - p.L, a, S);
        store_m_operand(reinterpret_cast<bf16*>(&sm), S,
                        reinterpret_cast<bf16*>(p.seg_M + state_off(loc.seg_base + loc.s - 1, p.h_v, h)));
        return;
    }
    store_state(dst, S);
}

// Sequential composition of the exact segment maps for one (sequence, head,
// 32-column block): S0(s) = M_{s-1} S0(s-1) + H_{s-1}, or the warm-up state
// where the boundary warmed up. Wave w computes rows [32w, 32w + 32).
// Each step is one 128 x 32 x 128 product on hi/lo operands. M arrives split
// and in A-operand order (contiguous loads, requested one step ahead); each
// lane writes the split of its rows of the new S0 straight into the B-operand
// slots of the next step (its accumulator rows are exactly that operand's k
// values), so the sequential path has no operand shuffling; the three partial
// products (hi hi, hi lo, lo hi) run as independent MFMA chains. The boundary
// flags come from LDS (the planner keeps segments per sequence within
// kMaxFlags), so no step waits on a global load to branch.
struct CombineIn {
    f32x16 tile;      // H_{s-1} or the warm-up state, this wave's rows
    bf16x8 ah[8], al[8];   // this lane's A operands of M_{s-1}
};

__device__ __forceinline__ void combine_split_out(bf16* sB, const f32x16& acc, int w, int lane) {
    // sB: [ks][part][lane][8]; rows 32w + acc_row(i, h) are k = 16 (2w + i / 8) + kperm(h, i % 8)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        bf16x8 hi, lo;
        split_half(acc, half, hi, lo);
        const int ks = 2 * w + half;
        *reinterpret_cast<bf16x8*>(sB + ((ks * 2 + 0) * 64 + lane) * 8) = hi;
        *reinterpret_cast<bf16x8*>(sB + ((ks * 2 + 1) * 64 + lane) * 8) = lo;
    }
}

__global__ __launch_bounds__(NTHR) void k_cp_combine(Params p) {
    __shared__ __attribute__((aligned(16))) bf16 sB[2][8 * 2 * 64 * 8];  // S0 block as split B operands
    __shared__ int wflag[kMaxFlags];
    const int seq = blockIdx.x >> 2, cb = blockIdx.x & 3, h = blockIdx.y;
    if (seq >= p.n_seqs) return;
    int P, seg_base;
    if (!p.cu) {
        P = n_segs_of(n_chunks_of(p.seq_len), p.L);
        seg_base = seq * P;
    } else {
        seg_base = 0;
        for (int n = 0; n < seq; ++n) seg_base += n_segs_of(n_chunks_of(p.cu[n + 1] - p.cu[n]), p.L);
        P = n_segs_of(n_chunks_of(p.cu[seq + 1] - p.cu[seq]), p.L);
    }
    if (P <= 1 || P > kMaxFlags) return;
    int n_exact = 0;
    for (int s = 1 + (int)threadIdx.x; s < P; s += NTHR) {
        const int f = p.warm[(size_t)(seg_base + s) * p.h_v + h];
        wflag[s] = f;
        n_exact += (f == 0);
    }
    if (!__syncthreads_or(n_exact)) return;

    const int lane = lane_id(), col = lane & 31, hh = lane >> 5, w = wave_id();
    const int cglob = 32 * cb + col;
    {
        f32x16 acc;
        if (p.s_init) {
            const float* S0 = p.s_init + state_off(seq, p.h_v, h);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = S0[(32 * w + acc_row(i, hh)) * DK + cglob];
        } else {
            acc = f32x16{};
        }
        combine_split_out(sB[0], acc, w, lane);
    }
    // Operands of step s1 (boundary s1): the warm-up state or H_{s1-1}, and
    // this lane's A operands of M_{s1-1}.
    // (every step issues the same loads and stores: a step past the end loads
    // the last one again, M is loaded whether or not the step applies it, and
    // the state is stored back also where it is a warm-up state; then the
    // compiler's waits stay exact across the loop and the prefetch works)
    auto tile_src = [&](int s1) {
        s1 = min(s1, P - 1);
        return __builtin_amdgcn_readfirstlane(wflag[s1]) ? p.seg_state + state_off(seg_base + s1, p.h_v, h)
                                                          : p.seg_H + state_off(seg_base + s1 - 1, p.h_v, h);
    };
    auto m_src = [&](int s1) {
        s1 = min(s1, P - 1);
        return reinterpret_cast<const bf16*>(p.seg_M + state_off(seg_base + s1 - 1, p.h_v, h)) +
               (size_t)(w * 8 * 2 * 64 + lane) * 8;
    };
    auto fetch = [&](int s1, CombineIn& in) {
        const float* src = tile_src(s1);
#pragma unroll
        for (int i = 0; i < 16; ++i) in.tile[i] = src[(32 * w + acc_row(i, hh)) * DK + cglob];
        const bf16* mop = m_src(s1);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            in.ah[ks] = *reinterpret_cast<const bf16x8*>(mop + (ks * 2 + 0) * 64 * 8);
            in.al[ks] = *reinterpret_cast<const bf16x8*>(mop + (ks * 2 + 1) * 64 * 8);
        }
    };
    // One step from the operands in `in`, which are refilled with those of
    // step s + 2 as they are consumed (each operand's load is issued right
    // after the MFMAs that read it, so the loads overlap the products): two
    // register sets alternate, and each step's loads have two steps to
    // arrive. The three partial products run as independent chains.
    int buf = 0;
    auto step = [&](int s, CombineIn& in) {
        const int warm = __builtin_amdgcn_readfirstlane(wflag[s]);   // uniform: a scalar branch
        const bool mm = !warm && (s > 1 || p.s_init);
        f32x16 acc = in.tile;
        {
            const float* src = tile_src(s + 2);
#pragma unroll
            for (int i = 0; i < 16; ++i) in.tile[i] = src[(32 * w + acc_row(i, hh)) * DK + cglob];
        }
        const bf16* mop = m_src(s + 2);
        // (the products run also where they are not applied -- a warm-up
        // boundary, or M_0 without an initial state -- and are then dropped:
        // no branch separates the loads from the products)
        const f32x16 base = acc;
        f32x16 hl = f32x16{}, lh = f32x16{};
        const bf16* Bp = sB[buf];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const bf16x8 bh = *reinterpret_cast<const bf16x8*>(Bp + ((ks * 2 + 0) * 64 + lane) * 8);
            const bf16x8 bl = *reinterpret_cast<const bf16x8*>(Bp + ((ks * 2 + 1) * 64 + lane) * 8);
            acc = mma32(in.ah[ks], bh, acc);
            hl = mma32(in.ah[ks], bl, hl);
            lh = mma32(in.al[ks], bh, lh);
            in.ah[ks] = *reinterpret_cast<const bf16x8*>(mop + (ks * 2 + 0) * 64 * 8);
            in.al[ks] = *reinterpret_cast<const bf16x8*>(mop + (ks * 2 + 1) * 64 * 8);
        }
        // instruction order for the scheduler: the tile loads, then per k step
        // two LDS reads, three MFMAs and the two loads that refill their operands
        __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        }
        acc += hl + lh;
        if (!mm) acc = base;
        combine_split_out(sB[buf ^ 1], acc, w, lane);
        {
            float* dst = p.seg_state + state_off(seg_base + s, p.h_v, h);
#pragma unroll
            for (int i = 0; i < 16; ++i) dst[(32 * w + acc_row(i, hh)) * DK + cglob] = acc[i];
        }
        __syncthreads();
        buf ^= 1;
    };
    CombineIn in0, in1;
    fetch(1, in0);
    fetch(2, in1);
    __syncthreads();
    for (int s = 1; s < P; s += 2) {
        step(s, in0);
        if (s + 1 < P) step(s + 1, in1);
    }
}

// The fused forward of one segment: per chunk the P tiles, the state chain and
// the output.
template <typename IO>
__global__ __launch_bounds__(NTHR) void k_fwd(Params p) {
    constexpr bool EX = Io<IO>::kExact;
    __shared__ ChainSmem<EX> sm;
    const int h = blockIdx.y, hq = h / p.group, wave = wave_id();
    const SegLoc loc = locate_segment(p, blockIdx.x);
    if (loc.seq < 0) return;
    f32x16 S[4];
    if (loc.s == 0) {
        if (p.s_init) load_state(p.s_init + state_off(loc.seq, p.h_v, h), S);
        else zero_state(S);
    } else {
        load_state(p.seg_state + state_off(loc.seg_base + loc.s, p.h_v, h), S);
    }
    const int c0 = loc.s * p.L, c1 = min(c0 + p.L, loc.N);
    const size_t ts_v = (size_t)p.h_v * DK;
    Chunk<IO> nxt;
    if (c0 < c1)
        fetch_chunk<IO, true, true>(nxt, p, loc.tok0 + (size_t)c0 * CH, min(CH, loc.len - c0 * CH), h, hq,
                                    loc.chunk_base + c0);
    if (c0 < c1) {   // (the scratch line exists whenever there is a chunk)
        // the loop body ends with the output's eight stores after its loads; the
        // same stores (to the scratch line) here make the loop's entry look
        // alike, so that the wait at its head covers the loads only
        IO* dst = reinterpret_cast<IO*>(p.sink + 32 * lane_id());
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if constexpr (EX) *reinterpret_cast<u32x2*>(dst + 8 * (i & 3)) = u32x2{0u, 0u};
            else *reinterpret_cast<f32x4*>(dst + 8 * (i & 3)) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    for (int c = c0; c < c1; ++c) {
        const size_t tok0 = loc.tok0 + (size_t)c * CH;
        const int nvalid = min(CH, loc.len - c * CH);
        stage_chunk<IO, true, true>(sm, nxt, p.scale);
        __syncthreads();
        {   // always a prefetch (the last chunk fetches itself again): see fetch_chunk
            const int cn = min(c + 1, c1 - 1);
            fetch_chunk<IO, true, true>(nxt, p, loc.tok0 + (size_t)cn * CH, min(CH, loc.len - cn * CH), h, hq,
                                        loc.chunk_base + cn);
        }
        // P tiles: three per wave, the last wave takes one and zeroes the two
        // upper tiles inside the diagonal 32-blocks
        if (wave < 3) {
            gram_p<EX, 3>(sm, wave, 3, p.scale);
        } else {
            gram_p<EX, 1>(sm, 9, 1, p.scale);
            zero_p_tile(sm.p, 0, 1);
            zero_p_tile(sm.p, 2, 3);
        }
        f32x16 Vp[2], O[2];
        {
            SplitS ss;
            split_state(S, ss);
            const IO* vcol = static_cast<const IO*>(p.v) + tok0 * ts_v + (size_t)h * DK + 32 * wave + (lane_id() & 31);
            chain_vp<IO, true>(sm, ss, vcol, ts_v, nvalid, Vp);
            chain_qs<EX>(sm, ss, O);
        }
        __syncthreads();
        chain_pv_out<IO>(sm, Vp, O, static_cast<IO*>(p.out) + tok0 * ts_v + (size_t)h * DK, ts_v, nvalid, p.sink);
        chain_state<EX>(sm, S, Vp);
        __syncthreads();
    }
    if (loc.s == loc.P - 1 && p.s_final) store_state(p.s_final + state_off(loc.seq, p.h_v, h), S);
}

// Per (sequence, head) summary of the boundary choices, over the boundaries
// whose warm-up window does not reach the sequence start: 1 all warm-up,
// 0 all exact, 2 mixed, 3 no such boundary; -1 the sequence was not split.
__global__ void k_debug_path(Params p, int32_t* path) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= p.n_seqs * p.h_v) return;
    const int seq = idx / p.h_v, h = idx - seq * p.h_v;
    int P, seg_base;
    if (!p.cu) {
        P = n_segs_of(n_chunks_of(p.seq_len), p.L);
        seg_base = seq * P;
    } else {
        seg_base = 0;
        for (int n = 0; n < seq; ++n) seg_base += n_segs_of(n_chunks_of(p.cu[n + 1] - p.cu[n]), p.L);
        P = n_segs_of(n_chunks_of(p.cu[seq + 1] - p.cu[seq]), p.L);
    }
    if (P <= 1) {
        path[idx] = -1;
        return;
    }
    int nw = 0, ne = 0;
    for (int s = 1; s < P; ++s) {
        const int f = p.warm[(size_t)(seg_base + s) * p.h_v + h];
        nw += (f == 1);
        ne += (f == 0);
    }
    path[idx] = (nw + ne == 0) ? 3 : (ne == 0 ? 1 : (nw == 0 ? 0 : 2));
}

}  // namespace

// ----------------------------------------------------------------------------
// Launchers

static int launched() { return (int)hipGetLastError(); }

int launch_prep(const Params& p, int io, void* stream) {
    if (p.n_chunks <= 0) return 0;
    const dim3 grid((p.n_chunks + p.prep_cpw - 1) / p.prep_cpw, p.h_v), block(NTHR);
    if (io == kIoBf16) hipLaunchKernelGGL(k_prep<bf16>, grid, block, 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL(k_prep<float>, grid, block, 0, (hipStream_t)stream, p);
    return launched();
}

int launch_wu(const Params& p, int io, void* stream) {
    if (p.n_chunks <= 0) return 0;
    const dim3 grid(p.n_chunks, p.h_v), block(NTHR);
    if (io == kIoBf16) hipLaunchKernelGGL(k_wu<bf16>, grid, block, 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL(k_wu<float>, grid, block, 0, (hipStream_t)stream, p);
    return launched();
}

int launch_cp_prep(const Params& p, int io, void* stream) {
    const dim3 grid(2 * p.n_segments, p.h_v), block(NTHR);
    if (io == kIoBf16) hipLaunchKernelGGL(k_cp_prep<bf16>, grid, block, 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL(k_cp_prep<float>, grid, block, 0, (hipStream_t)stream, p);
    return launched();
}

int launch_cp_combine(const Params& p, void* stream) {
    const dim3 grid(4 * p.n_seqs, p.h_v), block(NTHR);
    hipLaunchKernelGGL(k_cp_combine, grid, block, 0, (hipStream_t)stream, p);
    return launched();
}

int launch_debug_path(const Params& p, int32_t* path_out, void* stream) {
    const int n = p.n_seqs * p.h_v;
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_debug_path, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, p, path_out);
    return launched();
}

int launch_fwd(const Params& p, int io, void* stream) {
    const dim3 grid(p.n_segments, p.h_v), block(NTHR);
    if (io == kIoBf16) hipLaunchKernelGGL(k_fwd<bf16>, grid, block, 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL(k_fwd<float>, grid, block, 0, (hipStream_t)stream, p);
    return launched();
}

}  // namespace gdn
