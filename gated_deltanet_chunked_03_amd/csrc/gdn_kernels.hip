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
// Section on optimising GDN chunked prefill: W, U and S are never written to
// HBM here; the preparation (gamma, A, T, W, U) is recomputed on chip by every
// kernel that needs it. Section "Gate-Driven Automatic Intra-Card Context
// Parallelism (AutoCP)": each sequence is cut into segments of L chunks that
// run as independent workgroups; cp_prep computes the state at each segment
// boundary by a short warm-up (gates decayed below the noise floor) or the
// exact state map S -> M S + H of the previous segment, and cp_combine chains
// the exact maps.
//
// Work layout. A workgroup is 4 waves (256 lanes). Wave w owns d_v columns
// [32w, 32w + 32): its 128 x 32 slice of S, its slice of U / V' and of the
// output all stay in its registers, so the sequential state chain never
// crosses waves. Operands that every wave needs (Q, K^T, -W, P = QK^T o D,
// T) are staged in LDS. Products use 32x32x16 bf16 MFMAs with fp32
// accumulation. Values that are not exact bf16 inputs (S, V', T, W, P) enter
// the MFMA as a hi + lo pair of bf16 (x = hi + lo to about 16 bits), giving
// 2 or 3 MFMAs per product; diagonal gate factors are applied in fp32 on the
// accumulators instead of being rounded into operands.
//
// Register layouts (verified on gfx950): 32x32x16 bf16 MFMA, lane l,
//   A operand: row l % 32, 8 k values; B operand: column l % 32, 8 k values
//   C/D: element i holds row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.
// Element e of an operand is placed at k = kb + kperm(h, e), h = l / 32, with
// kperm(h, e) = 4h + e (e < 4) or 8 + 4h + (e - 4); that is exactly where the
// accumulator layout holds rows, so a 32-row accumulator tile serves directly
// as the B operand of two consecutive k steps (elements 0..7 and 8..15).
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

constexpr int CH = kChunk;
constexpr int DK = kDim;
constexpr int NTHR = 256;
constexpr int LDQ = 132;   // row stride (elements) of [64][128] bf16 tiles
constexpr int LDKT = 68;   // row stride of [128][64] bf16 tiles
constexpr int LDF = 68;    // row stride of [64][64] fp32 tiles
constexpr int LDP = 68;    // row stride of [64][64] bf16 tiles
constexpr int LDC = 132;   // row stride of the combine kernel's [32][128] fp32 tile

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

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// Row of accumulator element i for lane half h (32x32 tiles).
__device__ __forceinline__ int acc_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

__device__ __forceinline__ void split4(f32x4 x, bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const bf16 t = (bf16)x[e];
        hi[e] = t;
        lo[e] = (bf16)(x[e] - (float)t);
    }
}

// Elements [B, B + 8) of an accumulator tile as a hi/lo B operand.
template <int B>
__device__ __forceinline__ void split_acc(const f32x16& a, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float x = a[B + e];
        const bf16 t = (bf16)x;
        hi[e] = t;
        lo[e] = (bf16)(x - (float)t);
    }
}

__device__ __forceinline__ void split_half(const f32x16& a, int half, bf16x8& hi, bf16x8& lo) {
    if (half) split_acc<8>(a, hi, lo);
    else split_acc<0>(a, hi, lo);
}

// Operand from a bf16 row: p = row start + kb + 4h; elements p[0..3], p[8..11].
__device__ __forceinline__ bf16x8 lds_op(const bf16* p) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(p);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(p + 8);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Operand from an fp32 row (same element placement), optionally times a
// per-column scale read at the same offsets, split into hi/lo.
template <bool SCALE>
__device__ __forceinline__ void f32_op(const float* p, const float* sc, bf16x8& hi, bf16x8& lo) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 8);
    if (SCALE) {
        a *= *reinterpret_cast<const f32x4*>(sc);
        b *= *reinterpret_cast<const f32x4*>(sc + 8);
    }
    bf16x4 ah, al, bh, bl;
    split4(a, ah, al);
    split4(b, bh, bl);
    hi = __builtin_shufflevector(ah, bh, 0, 1, 2, 3, 4, 5, 6, 7);
    lo = __builtin_shufflevector(al, bl, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Operand from a global row of 128 io elements (row read as zero if !valid).
__device__ __forceinline__ void g_row_op(const bf16* rowp, bool valid, int kb, int h,
                                         bf16x8& hi, bf16x8& lo) {
    if (valid) {
        hi = lds_op(rowp + kb + 4 * h);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) hi[e] = (bf16)0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) lo[e] = (bf16)0.f;
}
__device__ __forceinline__ void g_row_op(const float* rowp, bool valid, int kb, int h,
                                         bf16x8& hi, bf16x8& lo) {
    if (valid) {
        f32_op<false>(rowp + kb + 4 * h, nullptr, hi, lo);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) { hi[e] = (bf16)0.f; lo[e] = (bf16)0.f; }
    }
}

// B operand from one column of a token-major global tile: element e is token
// kb + kperm(h, e); tokens >= nvalid read as zero.
template <typename IO>
__device__ __forceinline__ void g_col_op(const IO* col0, size_t ts, int kb, int h, int nvalid,
                                         bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int t = kb + ((e < 4) ? (4 * h + e) : (4 + 4 * h + e));
        const float x = (t < nvalid) ? (float)col0[(size_t)t * ts] : 0.f;
        const bf16 th = (bf16)x;
        hi[e] = th;
        lo[e] = Io<IO>::kExact ? (bf16)0.f : (bf16)(x - (float)th);
    }
}

// ----------------------------------------------------------------------------
// Shared memory of the chunk workgroups

template <bool EX>
struct __attribute__((aligned(16))) Smem {
    bf16 q_hi[CH * LDQ];                  // Q chunk, token-major
    bf16 q_lo[EX ? 8 : CH * LDQ];
    bf16 kt_hi[DK * LDKT];                // K chunk transposed: [d_k][token]
    bf16 kt_lo[EX ? 8 : DK * LDKT];
    bf16 p_hi[CH * LDP];                  // P = (Q K^T) o D, causal, split
    bf16 p_lo[CH * LDP];
    float t[CH * LDF];                    // T = (I + A)^-1
    union {
        float a[CH * LDF];                // A (strictly lower), until T is built
        bf16 w[2 * CH * LDQ];             // -W split: hi rows then lo rows
    } x;
    float gam[CH];                        // gamma
    float eg[CH];                         // exp(gamma)
    float egc[CH];                        // exp(gamma_C - gamma)
    float bw[CH];                         // beta exp(gamma)
    float beta[CH];
    float red[64];                        // red[0] = exp(gamma_C); reductions
};

// ----------------------------------------------------------------------------
// Locating work items

struct SegLoc {
    int seq;      // -1 if the slot is past the last segment
    int s;        // segment index within the sequence
    int P;        // segments of the sequence
    int N;        // chunks of the sequence
    int len;      // tokens of the sequence
    int seg_base; // global index of the sequence's segment 0
    size_t tok0;  // global token index of the sequence start
};

__device__ __forceinline__ int n_chunks_of(int len) { return (len + CH - 1) / CH; }
__device__ __forceinline__ int n_segs_of(int N, int L) { return N == 0 ? 1 : (N + L - 1) / L; }

__device__ SegLoc locate_segment(const Params& p, int slot) {
    SegLoc o;
    o.seq = -1;
    o.s = o.P = o.N = o.len = o.seg_base = 0;
    o.tok0 = 0;
    if (!p.cu) {
        const int N = n_chunks_of(p.seq_len);
        const int P = n_segs_of(N, p.L);
        const int seq = slot / P;
        if (seq < p.n_seqs) {
            o.seq = seq; o.s = slot - seq * P; o.P = P; o.N = N; o.len = p.seq_len;
            o.seg_base = seq * P; o.tok0 = (size_t)seq * p.seq_len;
        }
        return o;
    }
    int base = 0;
    for (int n = 0; n < p.n_seqs; ++n) {
        const int a = p.cu[n], len = p.cu[n + 1] - a;
        const int N = n_chunks_of(len), P = n_segs_of(N, p.L);
        if (slot < base + P) {
            o.seq = n; o.s = slot - base; o.P = P; o.N = N; o.len = len;
            o.seg_base = base; o.tok0 = (size_t)a;
            return o;
        }
        base += P;
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

// ----------------------------------------------------------------------------
// Chunk preparation: load, gamma, gram products, inverse, W and U

// Loads K (transposed into kt), optionally Q, and the gates of one chunk.
// Token rows >= nvalid are zero padding (and g = beta = 0 there).
template <typename IO, bool WANT_Q>
__device__ void load_chunk(Smem<Io<IO>::kExact>& sm, const Params& p, size_t tok0, int nvalid,
                           int h, int hq) {
    constexpr bool EX = Io<IO>::kExact;
    const int tid = threadIdx.x;
    const size_t ts = (size_t)p.h_qk * DK;
    const IO* kb = static_cast<const IO*>(p.k) + tok0 * ts + (size_t)hq * DK;
    const IO* qb = static_cast<const IO*>(p.q) + tok0 * ts + (size_t)hq * DK;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int pc = tid + NTHR * it;
        const int row = pc >> 4, c8 = (pc & 15) * 8;
        float kv[8], qv[8];
        if (row < nvalid) {
#pragma unroll
            for (int e = 0; e < 8; ++e) kv[e] = (float)kb[(size_t)row * ts + c8 + e];
            if (WANT_Q) {
#pragma unroll
                for (int e = 0; e < 8; ++e) qv[e] = (float)qb[(size_t)row * ts + c8 + e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) { kv[e] = 0.f; qv[e] = 0.f; }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bf16 th = (bf16)kv[e];
            sm.kt_hi[(c8 + e) * LDKT + row] = th;
            if (!EX) sm.kt_lo[(c8 + e) * LDKT + row] = (bf16)(kv[e] - (float)th);
        }
        if (WANT_Q) {
            bf16x4 h0, h1, l0, l1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                h0[e] = (bf16)qv[e];
                h1[e] = (bf16)qv[4 + e];
                l0[e] = (bf16)(qv[e] - (float)h0[e]);
                l1[e] = (bf16)(qv[4 + e] - (float)h1[e]);
            }
            *reinterpret_cast<bf16x4*>(sm.q_hi + row * LDQ + c8) = h0;
            *reinterpret_cast<bf16x4*>(sm.q_hi + row * LDQ + c8 + 4) = h1;
            if (!EX) {
                *reinterpret_cast<bf16x4*>(sm.q_lo + row * LDQ + c8) = l0;
                *reinterpret_cast<bf16x4*>(sm.q_lo + row * LDQ + c8 + 4) = l1;
            }
        }
    }
    if (wave_id() == 0) {
        const int t = lane_id();
        float gv = 0.f, bv = 0.f;
        if (t < nvalid) {
            const size_t idx = (tok0 + t) * (size_t)p.h_v + h;
            gv = p.g[idx];
            bv = p.beta[idx];
        }
        float s = gv;  // inclusive scan over the 64 lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float o = __shfl_up(s, d, 64);
            if (t >= d) s += o;
        }
        const float gc = __shfl(s, 63, 64);
        const float es = __expf(s);
        sm.gam[t] = s;
        sm.eg[t] = es;
        sm.egc[t] = __expf(gc - s);
        sm.beta[t] = bv;
        sm.bw[t] = bv * es;
        if (t == 0) sm.red[0] = __expf(gc);
    }
}

// One 32x32 tile (ti, tj) of X K^T, X = K (global rows) or Q (LDS rows).
template <typename IO, bool FROM_Q>
__device__ f32x16 gram_tile(const Smem<Io<IO>::kExact>& sm, const IO* krow0, size_t ts, int nvalid,
                            int ti, int tj) {
    constexpr bool EX = Io<IO>::kExact;
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
    const int ra = 32 * ti + col, rb = 32 * tj + col;
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        bf16x8 ah, al, bh, bl;
        if (FROM_Q) {
            ah = lds_op(sm.q_hi + ra * LDQ + 16 * ks + 4 * h);
            if (!EX) al = lds_op(sm.q_lo + ra * LDQ + 16 * ks + 4 * h);
        } else {
            g_row_op(krow0 + (size_t)ra * ts, ra < nvalid, 16 * ks, h, ah, al);
        }
        g_row_op(krow0 + (size_t)rb * ts, rb < nvalid, 16 * ks, h, bh, bl);
        acc = mma32(ah, bh, acc);
        if (!EX) {
            acc = mma32(ah, bl, acc);
            acc = mma32(al, bh, acc);
        }
    }
    return acc;
}

// A[i][j] = beta_i exp(gamma_i - gamma_j) (k_i . k_j) for i > j, else 0.
template <bool EX>
__device__ void store_A(Smem<EX>& sm, const f32x16& acc, int ti, int tj) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
    const int c = 32 * tj + col;
    const float gc = sm.gam[c];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 32 * ti + acc_row(i, h);
        const float d = __expf(sm.gam[r] - gc);
        sm.x.a[r * LDF + c] = (r > c) ? sm.beta[r] * d * acc[i] : 0.f;
    }
}

// P[i][j] = exp(gamma_i - gamma_j) (q_i . k_j) for i >= j, else 0 (hi/lo bf16).
template <bool EX>
__device__ void store_P(Smem<EX>& sm, const f32x16& acc, int ti, int tj) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
    const int c = 32 * tj + col;
    const float gc = sm.gam[c];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 32 * ti + acc_row(i, h);
        const float d = __expf(sm.gam[r] - gc);
        const float v = (r >= c) ? d * acc[i] : 0.f;
        const bf16 th = (bf16)v;
        sm.p_hi[r * LDP + c] = th;
        sm.p_lo[r * LDP + c] = (bf16)(v - (float)th);
    }
}

// Diagonal 16x16 blocks of T = (I + A)^-1 by forward substitution, one block
// per wave; lane j < 16 solves column j.
template <bool EX>
__device__ void inv_diag(Smem<EX>& sm) {
    const int lane = lane_id(), b = 16 * wave_id(), j = lane & 15;
    const float* A = sm.x.a + b * LDF + b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float s = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) s = fmaf(-A[i * LDF + m], x[m], s);
        x[i] = s;
    }
    if (lane < 16) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.t[(b + i) * LDF + b + j] = x[i];
    }
}

// Block column J of T below the diagonal: T_iJ = -X_i sum_{m=J}^{i-1} A_im T_mJ,
// with 16x16x16 bf16 MFMAs on hi/lo operands (lane l: A row l % 16, k 4 (l/16)..;
// B / C column l % 16, rows 4 (l/16)..). Zeros above the diagonal block.
template <int J, bool EX>
__device__ void inv_col(Smem<EX>& sm) {
    const int lane = lane_id(), n = lane & 15, g4 = lane >> 4;
    f32x4 Tc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) Tc[J][r] = sm.t[(16 * J + 4 * g4 + r) * LDF + 16 * J + n];
#pragma unroll
    for (int i = J + 1; i < 4; ++i) {
        f32x4 R = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = J; m < i; ++m) {
            const f32x4 a = *reinterpret_cast<const f32x4*>(sm.x.a + (16 * i + n) * LDF + 16 * m + 4 * g4);
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

// out = T diag(sc) X[:, 32w:32w+32] for X a token-major global tile (V or K).
template <typename IO>
__device__ void wy_tiles(const Smem<Io<IO>::kExact>& sm, const float* sc, const IO* col0, size_t ts,
                         int nvalid, f32x16 out[2]) {
    constexpr bool EX = Io<IO>::kExact;
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
    out[0] = f32x16{};
    out[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        bf16x8 bh, bl;
        g_col_op<IO>(col0, ts, 16 * ks, h, nvalid, bh, bl);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            if (ti == 0 && ks >= 2) continue;  // T is lower triangular
            bf16x8 ah, al;
            f32_op<true>(sm.t + (32 * ti + col) * LDF + 16 * ks + 4 * h, sc + 16 * ks + 4 * h, ah, al);
            out[ti] = mma32(ah, bh, out[ti]);
            out[ti] = mma32(al, bh, out[ti]);
            if (!EX) out[ti] = mma32(ah, bl, out[ti]);
        }
    }
}

// Full chunk preparation after load_chunk and a barrier. On return (before
// the caller's barrier) -W is being written to LDS; U (this wave's columns)
// and, if requested, W's tile for this wave's d_k columns are in registers.
template <typename IO, bool WANT_P>
__device__ void prep_chunk(Smem<Io<IO>::kExact>& sm, const Params& p, size_t tok0, int nvalid,
                           int h, int hq, bool want_U, f32x16 U[2], f32x16 Wt[2]) {
    constexpr bool EX = Io<IO>::kExact;
    const int wave = wave_id(), lane = lane_id(), col = lane & 31, hh = lane >> 5;
    const size_t ts_qk = (size_t)p.h_qk * DK;
    const IO* krow0 = static_cast<const IO*>(p.k) + tok0 * ts_qk + (size_t)hq * DK;

    // gram tiles: A from K K^T, P from Q K^T (lower 32x32 tiles only)
    if (WANT_P) {
        if (wave == 0) {
            store_A<EX>(sm, gram_tile<IO, false>(sm, krow0, ts_qk, nvalid, 0, 0), 0, 0);
            store_A<EX>(sm, gram_tile<IO, false>(sm, krow0, ts_qk, nvalid, 1, 1), 1, 1);
        } else if (wave == 1) {
            store_A<EX>(sm, gram_tile<IO, false>(sm, krow0, ts_qk, nvalid, 1, 0), 1, 0);
        } else if (wave == 2) {
            store_P<EX>(sm, gram_tile<IO, true>(sm, krow0, ts_qk, nvalid, 0, 0), 0, 0);
            store_P<EX>(sm, gram_tile<IO, true>(sm, krow0, ts_qk, nvalid, 1, 1), 1, 1);
        } else {
            store_P<EX>(sm, gram_tile<IO, true>(sm, krow0, ts_qk, nvalid, 1, 0), 1, 0);
        }
    } else {
        if (wave < 3) {
            const int ti = (wave == 0) ? 0 : 1, tj = (wave == 2) ? 1 : 0;
            store_A<EX>(sm, gram_tile<IO, false>(sm, krow0, ts_qk, nvalid, ti, tj), ti, tj);
        }
    }
    __syncthreads();
    inv_diag<EX>(sm);
    __syncthreads();
    switch (wave) {
        case 0: inv_col<0, EX>(sm); break;
        case 1: inv_col<1, EX>(sm); break;
        case 2: inv_col<2, EX>(sm); break;
        default: inv_col<3, EX>(sm); break;
    }
    __syncthreads();
    if (want_U) {
        const size_t ts_v = (size_t)p.h_v * DK;
        const IO* vcol = static_cast<const IO*>(p.v) + tok0 * ts_v + (size_t)h * DK + 32 * wave + col;
        wy_tiles<IO>(sm, sm.beta, vcol, ts_v, nvalid, U);
    } else {
        U[0] = f32x16{};
        U[1] = f32x16{};
    }
    const IO* kcol = krow0 + 32 * wave + col;
    wy_tiles<IO>(sm, sm.bw, kcol, ts_qk, nvalid, Wt);
    // -W as hi/lo into the region that held A (all reads of A are behind the barrier)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 32 * ti + acc_row(i, hh), c = 32 * wave + col;
            const float x = -Wt[ti][i];
            const bf16 th = (bf16)x;
            sm.x.w[r * LDQ + c] = th;
            sm.x.w[CH * LDQ + r * LDQ + c] = (bf16)(x - (float)th);
        }
}

// ----------------------------------------------------------------------------
// The state chain of one chunk (after prep_chunk and a barrier).
//   Vp (holds U on entry): V' = U - W S
//   O (if OUT):            O = diag(e^gamma) Q S + P V'   (scale applied at the store)
//   S:                     S <- e^gamma_C S + K^T diag(e^(gamma_C - gamma)) V'
template <bool EX, bool OUT>
__device__ void chain(const Smem<EX>& sm, f32x16 S[4], f32x16 Vp[2], f32x16 O[2]) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        bf16x8 sh, sl;
        split_half(S[ks >> 1], ks & 1, sh, sl);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            const int r = 32 * ti + col;
            const bf16x8 wh = lds_op(sm.x.w + r * LDQ + 16 * ks + 4 * h);
            const bf16x8 wl = lds_op(sm.x.w + CH * LDQ + r * LDQ + 16 * ks + 4 * h);
            Vp[ti] = mma32(wh, sh, Vp[ti]);
            Vp[ti] = mma32(wh, sl, Vp[ti]);
            Vp[ti] = mma32(wl, sh, Vp[ti]);
            if (OUT) {
                const bf16x8 qh = lds_op(sm.q_hi + r * LDQ + 16 * ks + 4 * h);
                O[ti] = mma32(qh, sh, O[ti]);
                O[ti] = mma32(qh, sl, O[ti]);
                if (!EX) {
                    const bf16x8 ql = lds_op(sm.q_lo + r * LDQ + 16 * ks + 4 * h);
                    O[ti] = mma32(ql, sh, O[ti]);
                }
            }
        }
    }
    if (OUT) {
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int i = 0; i < 16; ++i) O[ti][i] *= sm.eg[32 * ti + acc_row(i, h)];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 vh, vl;
            split_half(Vp[ks >> 1], ks & 1, vh, vl);
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) {
                if (ti == 0 && ks >= 2) continue;  // P is causal
                const int r = 32 * ti + col;
                const bf16x8 ph = lds_op(sm.p_hi + r * LDP + 16 * ks + 4 * h);
                const bf16x8 pl = lds_op(sm.p_lo + r * LDP + 16 * ks + 4 * h);
                O[ti] = mma32(ph, vh, O[ti]);
                O[ti] = mma32(ph, vl, O[ti]);
                O[ti] = mma32(pl, vh, O[ti]);
            }
        }
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int i = 0; i < 16; ++i) Vp[ti][i] *= sm.egc[32 * ti + acc_row(i, h)];
    const float ec = sm.red[0];
#pragma unroll
    for (int t = 0; t < 4; ++t) S[t] *= ec;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        bf16x8 vh, vl;
        split_half(Vp[ks >> 1], ks & 1, vh, vl);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = 32 * t + col;
            const bf16x8 kh = lds_op(sm.kt_hi + r * LDKT + 16 * ks + 4 * h);
            S[t] = mma32(kh, vh, S[t]);
            S[t] = mma32(kh, vl, S[t]);
            if (!EX) {
                const bf16x8 kl = lds_op(sm.kt_lo + r * LDKT + 16 * ks + 4 * h);
                S[t] = mma32(kl, vh, S[t]);
            }
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

// ----------------------------------------------------------------------------
// Kernels

// Low-level chunk preparation: gamma, W, U of every (chunk, value head).
template <typename IO>
__global__ __launch_bounds__(NTHR) void k_chunk_prep(Params p) {
    constexpr bool EX = Io<IO>::kExact;
    __shared__ Smem<EX> sm;
    const int h = blockIdx.y, hq = h / p.group;
    int seq, c, len;
    size_t tok_s;
    if (!locate_chunk(p, blockIdx.x, seq, c, len, tok_s)) return;
    const size_t tok0 = tok_s + (size_t)c * CH;
    const int nvalid = min(CH, len - c * CH);
    load_chunk<IO, false>(sm, p, tok0, nvalid, h, hq);
    __syncthreads();
    f32x16 U[2], Wt[2];
    prep_chunk<IO, false>(sm, p, tok0, nvalid, h, hq, true, U, Wt);
    const int lane = lane_id(), col = lane & 31, hh = lane >> 5, w = wave_id();
    const size_t base = ((size_t)blockIdx.x * p.h_v + h) * CH;
    if (w == 0) p.prep_gamma[base + lane] = sm.gam[lane];
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const size_t r = base + 32 * ti + acc_row(i, hh);
            p.prep_W[r * DK + 32 * w + col] = Wt[ti][i];
            p.prep_U[r * DK + 32 * w + col] = U[ti][i];
        }
}

// Warm-up or exact segment map for the boundary before segment s >= 1.
// blockIdx.x = 2 * segment slot + part; part 0: warm-up state or H, part 1: M.
template <typename IO>
__global__ __launch_bounds__(NTHR) void k_cp_prep(Params p) {
    constexpr bool EX = Io<IO>::kExact;
    __shared__ Smem<EX> sm;
    const int slot = blockIdx.x >> 1, part = blockIdx.x & 1, h = blockIdx.y, hq = h / p.group;
    const SegLoc loc = locate_segment(p, slot);
    if (loc.seq < 0 || loc.s == 0) return;
    const int a = loc.s * p.L;  // first chunk of segment s

    // Gate-driven choice: warm up iff the log-decay over the window of w chunks
    // before the boundary is at most log(noise floor) (or the window reaches
    // the sequence start, where the warm-up is exact).
    // warm: 0 exact map, 1 warm-up (decayed below the floor, or forced), 2 warm-up
    // from the sequence start (exact)
    int warm;
    if (p.cp_mode == kCpExact) {
        warm = 0;
    } else if (a - p.w <= 0) {
        warm = 2;
    } else if (p.cp_mode == kCpWarmup) {
        warm = 1;
    } else {
        const size_t t0 = loc.tok0 + (size_t)(a - p.w) * CH;
        float s = 0.f;
        for (int t = threadIdx.x; t < p.w * CH; t += NTHR) s += p.g[(t0 + t) * (size_t)p.h_v + h];
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
        if (lane_id() == 0) sm.red[8 + wave_id()] = s;
        __syncthreads();
        const float tot = sm.red[8] + sm.red[9] + sm.red[10] + sm.red[11];
        warm = (tot <= p.log_eps) ? 1 : 0;
        __syncthreads();
    }
    if (part == 0 && threadIdx.x == 0) p.warm[(size_t)(loc.seg_base + loc.s) * p.h_v + h] = warm;
    if (warm && part == 1) return;
    // the map of segment 0 is only applied to a nonzero initial state
    if (!warm && part == 1 && loc.s == 1 && !p.s_init) return;

    f32x16 S[4];
    int c_lo, c_hi;
    bool want_U = true;
    if (warm) {
        c_lo = max(a - p.w, 0);
        c_hi = a;
        if (c_lo == 0 && p.s_init) load_state(p.s_init + state_off(loc.seq, p.h_v, h), S);
        else zero_state(S);
    } else {
        c_lo = a - p.L;
        c_hi = a;
        if (part == 0) {
            zero_state(S);
        } else {
            identity_state(S);
            want_U = false;
        }
    }
    for (int c = c_lo; c < c_hi; ++c) {
        const size_t tok0 = loc.tok0 + (size_t)c * CH;
        const int nvalid = min(CH, loc.len - c * CH);
        load_chunk<IO, false>(sm, p, tok0, nvalid, h, hq);
        __syncthreads();
        f32x16 U[2], Wt[2], O[2];
        prep_chunk<IO, false>(sm, p, tok0, nvalid, h, hq, want_U, U, Wt);
        __syncthreads();
        chain<EX, false>(sm, S, U, O);
        __syncthreads();
    }
    float* dst;
    if (warm) dst = p.seg_state + state_off(loc.seg_base + loc.s, p.h_v, h);
    else if (part == 0) dst = p.seg_H + state_off(loc.seg_base + loc.s - 1, p.h_v, h);
    else dst = p.seg_M + state_off(loc.seg_base + loc.s - 1, p.h_v, h);
    store_state(dst, S);
}

// Sequential composition of the exact segment maps for one (sequence, head,
// 32-column block): S0(s) = M_{s-1} S0(s-1) + H_{s-1}, or the warm-up state
// where the boundary warmed up. Wave w computes rows [32w, 32w + 32).
__global__ __launch_bounds__(NTHR) void k_cp_combine(Params p) {
    __shared__ __attribute__((aligned(16))) float sT[2][32 * LDC];  // S0 block, [column][d_k]
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
    if (P <= 1) return;
    bool any_exact = false;
    for (int s = 1; s < P; ++s) any_exact |= (p.warm[(size_t)(seg_base + s) * p.h_v + h] == 0);
    if (!any_exact) return;

    const int lane = lane_id(), col = lane & 31, hh = lane >> 5, w = wave_id();
    const int cglob = 32 * cb + col;
    f32x16 acc;
    if (p.s_init) {
        const float* S0 = p.s_init + state_off(seq, p.h_v, h);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = S0[(32 * w + acc_row(i, hh)) * DK + cglob];
    } else {
        acc = f32x16{};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sT[0][col * LDC + 32 * w + acc_row(i, hh)] = acc[i];
    __syncthreads();
    int buf = 0;
    for (int s = 1; s < P; ++s) {
        float* dst = p.seg_state + state_off(seg_base + s, p.h_v, h);
        const int warm = p.warm[(size_t)(seg_base + s) * p.h_v + h];
        if (warm) {
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = dst[(32 * w + acc_row(i, hh)) * DK + cglob];
        } else {
            const float* Hs = p.seg_H + state_off(seg_base + s - 1, p.h_v, h);
            const float* Ms = p.seg_M + state_off(seg_base + s - 1, p.h_v, h);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = Hs[(32 * w + acc_row(i, hh)) * DK + cglob];
            if (s > 1 || p.s_init) {
                const float* mrow = Ms + (size_t)(32 * w + col) * DK;
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    bf16x8 ah, al, bh, bl;
                    f32_op<false>(mrow + 16 * ks + 4 * hh, nullptr, ah, al);
                    f32_op<false>(&sT[buf][col * LDC + 16 * ks + 4 * hh], nullptr, bh, bl);
                    acc = mma32(ah, bh, acc);
                    acc = mma32(ah, bl, acc);
                    acc = mma32(al, bh, acc);
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) dst[(32 * w + acc_row(i, hh)) * DK + cglob] = acc[i];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[buf ^ 1][col * LDC + 32 * w + acc_row(i, hh)] = acc[i];
        __syncthreads();
        buf ^= 1;
    }
}

// The fused forward of one segment: prep, state chain and output per chunk.
template <typename IO>
__global__ __launch_bounds__(NTHR) void k_fwd(Params p) {
    constexpr bool EX = Io<IO>::kExact;
    __shared__ Smem<EX> sm;
    const int h = blockIdx.y, hq = h / p.group;
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
    const int lane = lane_id(), col = lane & 31, hh = lane >> 5, w = wave_id();
    const size_t ts_v = (size_t)p.h_v * DK;
    for (int c = c0; c < c1; ++c) {
        const size_t tok0 = loc.tok0 + (size_t)c * CH;
        const int nvalid = min(CH, loc.len - c * CH);
        load_chunk<IO, true>(sm, p, tok0, nvalid, h, hq);
        __syncthreads();
        f32x16 U[2], Wt[2];
        prep_chunk<IO, true>(sm, p, tok0, nvalid, h, hq, true, U, Wt);
        __syncthreads();
        f32x16 O[2] = {f32x16{}, f32x16{}};
        chain<EX, true>(sm, S, U, O);
        IO* ocol = static_cast<IO*>(p.out) + tok0 * ts_v + (size_t)h * DK + 32 * w + col;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 32 * ti + acc_row(i, hh);
                if (r < nvalid) ocol[(size_t)r * ts_v] = (IO)(O[ti][i] * p.scale);
            }
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

int launch_chunk_prep(const Params& p, int io, void* stream) {
    if (p.n_chunks <= 0) return 0;
    const dim3 grid(p.n_chunks, p.h_v), block(NTHR);
    if (io == kIoBf16) hipLaunchKernelGGL(k_chunk_prep<bf16>, grid, block, 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL(k_chunk_prep<float>, grid, block, 0, (hipStream_t)stream, p);
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
