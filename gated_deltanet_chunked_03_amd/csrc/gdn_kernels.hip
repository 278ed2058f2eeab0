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
constexpr int LDC = 132;   // row stride of the combine kernel's [32][128] fp32 tile
constexpr int LDO = 136;   // row stride of the staged [64][128] bf16 output tile
constexpr int kMaxFlags = 2048;  // boundary flags the combine kernel keeps in LDS

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
// Shared memory of the chunk workgroups

template <bool EX>
struct __attribute__((aligned(16))) Smem {
    bf16 q_hi[CH * LDQ];                  // Q chunk, token-major
    bf16 q_lo[EX ? 8 : CH * LDQ];
    bf16 kt_hi[DK * LDKT];                // K chunk transposed: [d_k][token]
    bf16 kt_lo[EX ? 8 : DK * LDKT];
    bf16 vt[EX ? DK * LDKT : 8];          // V chunk transposed (bf16 inputs; fp32 V is read from HBM)
    bf16 p_hi[CH * LDP];                  // P = (Q K^T) o D, causal, split
    bf16 p_lo[CH * LDP];
    bf16 tw[EX ? 2 * CH * LDP : 8];       // T diag(beta e^gamma), hi rows then lo rows
    bf16 tu[EX ? 2 * CH * LDP : 8];       // T diag(beta), hi rows then lo rows
    union {
        float t[CH * LDF];                // T = (I + A)^-1
        bf16 k_rm[EX ? CH * LDQ : 8];     // K chunk token-major, until the gram products are done
    } u;
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

// One chunk's inputs in registers between the global load and the LDS store
// (so the next chunk's loads overlap the current chunk's work). Thread t
// holds pieces t + 256 j (j < 4): token row (piece / 16), columns
// 8 (piece % 16) .. + 8 of K, Q and V, so sixteen lanes cover one 256-byte row.
template <typename IO> struct Chunk;
template <> struct Chunk<bf16> { u32x4 k[4], q[4], v[4]; float g, b; };
template <> struct Chunk<float> { f32x4 k[8], q[8]; float g, b; };

template <typename IO, bool WANT_Q>
__device__ __forceinline__ void fetch_chunk(Chunk<IO>& r, const Params& p, size_t tok0, int nvalid,
                                            int h, int hq) {
    constexpr bool EX = Io<IO>::kExact;
    const int t = threadIdx.x;
    const size_t ts = (size_t)p.h_qk * DK, tsv = (size_t)p.h_v * DK;
    const IO* kb = static_cast<const IO*>(p.k) + tok0 * ts + (size_t)hq * DK;
    const IO* qb = static_cast<const IO*>(p.q) + tok0 * ts + (size_t)hq * DK;
    const IO* vb = static_cast<const IO*>(p.v) + tok0 * tsv + (size_t)h * DK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int pc = t + NTHR * j, row = pc >> 4, c8 = (pc & 15) * 8;
        const bool ok = row < nvalid;
        if constexpr (EX) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            r.k[j] = ok ? *reinterpret_cast<const u32x4*>(kb + row * ts + c8) : z;
            if (WANT_Q) r.q[j] = ok ? *reinterpret_cast<const u32x4*>(qb + row * ts + c8) : z;
            r.v[j] = ok ? *reinterpret_cast<const u32x4*>(vb + row * tsv + c8) : z;
        } else {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            r.k[2 * j] = ok ? *reinterpret_cast<const f32x4*>(kb + row * ts + c8) : z;
            r.k[2 * j + 1] = ok ? *reinterpret_cast<const f32x4*>(kb + row * ts + c8 + 4) : z;
            if (WANT_Q) {
                r.q[2 * j] = ok ? *reinterpret_cast<const f32x4*>(qb + row * ts + c8) : z;
                r.q[2 * j + 1] = ok ? *reinterpret_cast<const f32x4*>(qb + row * ts + c8 + 4) : z;
            }
        }
    }
    r.g = 0.f;
    r.b = 0.f;
    if (wave_id() == 0 && lane_id() < nvalid) {
        const size_t idx = (tok0 + lane_id()) * (size_t)p.h_v + h;
        r.g = p.g[idx];
        r.b = p.beta[idx];
    }
}

// Two bf16 of the same column from two rows packed into one 32-bit word.
__device__ __forceinline__ unsigned int pack_col(const u32x4& a, const u32x4& b, int e) {
    const unsigned int wa = a[e >> 1], wb = b[e >> 1];
    return (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
}

// Writes a fetched chunk to LDS and derives the gate quantities. bf16
// inputs: K, Q and V token-major (K in the T area and V in the T'' area,
// both free until the inverse; the gram phase transposes them); fp32 inputs: Q and K^T as hi/lo pairs. Rows
// past the end of the sequence were fetched as zeros (g = beta = 0 there).
template <typename IO, bool WANT_Q>
__device__ __forceinline__ void stage_chunk(Smem<Io<IO>::kExact>& sm, const Chunk<IO>& r) {
    constexpr bool EX = Io<IO>::kExact;
    const int t = threadIdx.x;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int pc = t + NTHR * j, row = pc >> 4, c8 = (pc & 15) * 8;
        if constexpr (EX) {
            const int o0 = row * LDQ + pk(c8), o1 = row * LDQ + pk(c8 + 4);
            *reinterpret_cast<u32x2*>(sm.u.k_rm + o0) = u32x2{r.k[j][0], r.k[j][1]};
            *reinterpret_cast<u32x2*>(sm.u.k_rm + o1) = u32x2{r.k[j][2], r.k[j][3]};
            *reinterpret_cast<u32x2*>(sm.tu + o0) = u32x2{r.v[j][0], r.v[j][1]};
            *reinterpret_cast<u32x2*>(sm.tu + o1) = u32x2{r.v[j][2], r.v[j][3]};
            if (WANT_Q) {
                *reinterpret_cast<u32x2*>(sm.q_hi + o0) = u32x2{r.q[j][0], r.q[j][1]};
                *reinterpret_cast<u32x2*>(sm.q_hi + o1) = u32x2{r.q[j][2], r.q[j][3]};
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                bf16 th, tl;
                split1(r.k[2 * j + (e >> 2)][e & 3], th, tl);
                sm.kt_hi[(c8 + e) * LDKT + pk(row)] = th;
                sm.kt_lo[(c8 + e) * LDKT + pk(row)] = tl;
                if (WANT_Q) {
                    split1(r.q[2 * j + (e >> 2)][e & 3], th, tl);
                    sm.q_hi[row * LDQ + pk(c8 + e)] = th;
                    sm.q_lo[row * LDQ + pk(c8 + e)] = tl;
                }
            }
        }
    }
    if (wave_id() == 0) {
        const int lane = lane_id();
        float s = r.g;  // inclusive scan over the 64 lanes
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float o = __shfl_up(s, d, 64);
            if (lane >= d) s += o;
        }
        const float gc = __shfl(s, 63, 64);
        const float es = __expf(s);
        sm.gam[lane] = s;
        sm.eg[lane] = es;
        sm.egc[lane] = __expf(gc - s);
        sm.beta[lane] = r.b;
        sm.bw[lane] = r.b * es;
        if (lane == 0) sm.red[0] = __expf(gc);
    }
}

// Two bf16 of the same column from two rows packed into one 32-bit word.
__device__ __forceinline__ unsigned pack_col(u32x2 a, u32x2 b, int e) {
    const unsigned wa = a[e >> 1], wb = b[e >> 1];
    return (e & 1) ? ((wa >> 16) | (wb & 0xffff0000u)) : ((wa & 0xffffu) | (wb << 16));
}

// K^T and V^T from the token-major LDS tiles (bf16 inputs; after a barrier):
// thread t packs rows 2 (t % 32), 2 (t % 32) + 1 of column blocks t / 32 and
// t / 32 + 8 into 32-bit words of the transposed tiles.
__device__ __forceinline__ void transpose_kv(Smem<true>& sm) {
    const int t = threadIdx.x, rp = t & 31, cbk = t >> 5;
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
        const int c8 = 8 * (cbk + 8 * jb);
        const int tp = pk(2 * rp);  // the token pair stays adjacent under the permutation
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int o = (2 * rp) * LDQ + pk(c8 + 4 * half);
            const u32x2 ka = *reinterpret_cast<const u32x2*>(sm.u.k_rm + o);
            const u32x2 kb = *reinterpret_cast<const u32x2*>(sm.u.k_rm + o + LDQ);
            const u32x2 va = *reinterpret_cast<const u32x2*>(sm.tu + o);
            const u32x2 vb = *reinterpret_cast<const u32x2*>(sm.tu + o + LDQ);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = c8 + 4 * half + e;
                *reinterpret_cast<unsigned*>(sm.kt_hi + c * LDKT + tp) = pack_col(ka, kb, e);
                *reinterpret_cast<unsigned*>(sm.vt + c * LDKT + tp) = pack_col(va, vb, e);
            }
        }
    }
}

// Gram products on 16x16 tiles (16x16x32 MFMA; lane l: A row l % 16 and
// B column l % 16, each with the 8 consecutive k values 8 (l / 16)..; C rows
// 4 (l / 16).. of column l % 16). The ten lower tiles (bi >= bj) of K K^T and
// of Q K^T are twenty jobs, run as interleaved chains. Each is computed
// transposed (K rows of block bj against K or Q rows of block bi), so a lane
// ends up with four consecutive columns j of one row i and stores them at once.
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

// A[i][j] = beta_i exp(gamma_i - gamma_j) (k_i . k_j) for i > j, else 0 (fp32), and
// P[i][j] = exp(gamma_i - gamma_j) (q_i . k_j) for i >= j, else 0 (hi/lo bf16).
// Jobs first, first + stride, ... (job >= 10: the P tile job - 10).
template <typename IO, int NJOB>
__device__ void gram_jobs(Smem<Io<IO>::kExact>& sm, const IO* krow0, size_t ts, int nvalid, int first,
                          int stride) {
    constexpr bool EX = Io<IO>::kExact;
    const int lane = lane_id(), n = lane & 15, g4 = lane >> 4;
    f32x4 acc[NJOB];
    int bi[NJOB], bj[NJOB];
    bool isq[NJOB];
#pragma unroll
    for (int t = 0; t < NJOB; ++t) {
        const int job = first + stride * t;
        isq[t] = job >= 10;
        lower_tile(isq[t] ? job - 10 : job, bi[t], bj[t]);
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int kb = 32 * ks + 8 * g4;                                 // physical (LDS)
        const int kg = 32 * ks + 16 * (g4 >> 1) + 4 * (g4 & 1);          // logical start (HBM rows)
#pragma unroll
        for (int t = 0; t < NJOB; ++t) {
            const int ra = 16 * bj[t] + n, rb = 16 * bi[t] + n;   // A: K rows of bj; B: rows of bi
            if constexpr (EX) {
                const bf16x8 a = lds_row8(sm.u.k_rm + ra * LDQ + kb);
                const bf16x8 b = lds_row8((isq[t] ? sm.q_hi : sm.u.k_rm) + rb * LDQ + kb);
                acc[t] = mma16k32(a, b, acc[t]);
            } else {
                bf16x8 ah, al, bh, bl;
                g_row8(krow0 + (size_t)ra * ts + kg, ra < nvalid, ah, al);
                if (isq[t]) {
                    bh = lds_row8(sm.q_hi + rb * LDQ + kb);
                    bl = lds_row8(sm.q_lo + rb * LDQ + kb);
                } else {
                    g_row8(krow0 + (size_t)rb * ts + kg, rb < nvalid, bh, bl);
                }
                acc[t] = mma16k32(ah, bh, acc[t]);
                acc[t] = mma16k32(ah, bl, acc[t]);
                acc[t] = mma16k32(al, bh, acc[t]);
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
        for (int r = 0; r < 4; ++r) {
            const float d = __expf(gi - gj[r]);
            v[r] = isq[t] ? ((i >= j0 + r) ? d * acc[t][r] : 0.f) : ((i > j0 + r) ? d * acc[t][r] : 0.f);
        }
        if (!isq[t]) {
            *reinterpret_cast<f32x4*>(sm.x.a + i * LDF + j0) = v * sm.beta[i];
        } else {
            unsigned h0, h1, l0, l1;
            split_pair(v[0], v[1], h0, l0);
            split_pair(v[2], v[3], h1, l1);
            *reinterpret_cast<u32x2*>(sm.p_hi + i * LDP + pk(j0)) = u32x2{h0, h1};
            *reinterpret_cast<u32x2*>(sm.p_lo + i * LDP + pk(j0)) = u32x2{l0, l1};
        }
    }
}

// Zero P on the upper 16x16 tile of a diagonal 32x32 block (read by the P V' product).
template <bool EX>
__device__ void zero_p_tile(Smem<EX>& sm, int bi, int bj) {
    const int lane = lane_id();
    const bf16 z = (bf16)0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int idx = lane + 64 * e, r = 16 * bi + (idx >> 4), c = 16 * bj + (idx & 15);
        sm.p_hi[r * LDP + pk(c)] = z;
        sm.p_lo[r * LDP + pk(c)] = z;
    }
}

// Diagonal 16x16 blocks of T = (I + A)^-1 by forward substitution. Every
// wave solves all four blocks (lane 16 b + j: block b, column j) and writes
// them; the values are identical across waves, so each wave can read the
// blocks back without waiting for the others.
template <bool EX>
__device__ void inv_diag(Smem<EX>& sm) {
    const int lane = lane_id(), b = 16 * (lane >> 4), j = lane & 15;
    const float* A = sm.x.a + b * LDF + b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float s = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) s = fmaf(-A[i * LDF + m], x[m], s);
        x[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.u.t[(b + i) * LDF + b + j] = x[i];
}

// Block column J of T below the diagonal: T_iJ = -X_i sum_{m=J}^{i-1} A_im T_mJ,
// with 16x16x16 bf16 MFMAs on hi/lo operands (lane l: A row l % 16, k 4 (l/16)..;
// B / C column l % 16, rows 4 (l/16)..). Zeros above the diagonal block.
template <int J, bool EX>
__device__ void inv_col(Smem<EX>& sm) {
    const int lane = lane_id(), n = lane & 15, g4 = lane >> 4;
    f32x4 Tc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) Tc[J][r] = sm.u.t[(16 * J + 4 * g4 + r) * LDF + 16 * J + n];
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
        const f32x4 xi = *reinterpret_cast<const f32x4*>(sm.u.t + (16 * i + n) * LDF + 16 * i + 4 * g4);
        bf16x4 xh, xl, rh, rl;
        split4(xi, xh, xl);
        split4(R, rh, rl);
        f32x4 P = {0.f, 0.f, 0.f, 0.f};
        P = mma16(xh, rh, P);
        P = mma16(xh, rl, P);
        P = mma16(xl, rh, P);
        Tc[i] = -P;
    }
    if constexpr (EX) {
        // T's block column J scaled by beta e^gamma (tw) and by beta (tu), split
        const int c = 16 * J + n;
        const float sw = sm.bw[c], su = sm.beta[c];
        const bf16 z = (bf16)0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * i + 4 * g4 + r;
                bf16 wh = z, wl = z, uh = z, ul = z;
                if (i >= J) {
                    split1(Tc[i][r] * sw, wh, wl);
                    split1(Tc[i][r] * su, uh, ul);
                }
                const int o = row * LDP + pk(c);
                sm.tw[o] = wh;
                sm.tw[CH * LDP + o] = wl;
                sm.tu[o] = uh;
                sm.tu[CH * LDP + o] = ul;
            }
    } else {
#pragma unroll
        for (int i = 0; i < J; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.u.t[(16 * i + 4 * g4 + r) * LDF + 16 * J + n] = 0.f;
#pragma unroll
        for (int i = J + 1; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) sm.u.t[(16 * i + 4 * g4 + r) * LDF + 16 * J + n] = Tc[i][r];
    }
}

// U = T diag(beta) V[:, 32w:32w+32] and W = T diag(beta e^gamma) K[:, 32w:32w+32]
// (T is lower triangular, so row tile 0 needs k steps 0..1 only). The B
// operands come from the transposed LDS tiles (fp32 V from HBM); hi and lo
// products accumulate into separate tiles so that four or more independent
// MFMA chains are in flight.
template <typename IO>
__device__ void wy_tiles(const Smem<Io<IO>::kExact>& sm, const IO* vcol, size_t ts, int nvalid,
                         bool want_U, f32x16 U[2], f32x16 W[2]) {
    constexpr bool EX = Io<IO>::kExact;
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
    const int n = 32 * wave_id() + col;
    U[0] = U[1] = W[0] = W[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        bf16x8 kh, kl, vh, vl;
        kh = lds_op16(sm.kt_hi + n * LDKT + 16 * ks + 8 * h);
        if (!EX) kl = lds_op16(sm.kt_lo + n * LDKT + 16 * ks + 8 * h);
        if (want_U) {
            if constexpr (EX) vh = lds_op16(sm.vt + n * LDKT + 16 * ks + 8 * h);
            else g_col_op<IO>(vcol, ts, 16 * ks, h, nvalid, vh, vl);
        }
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            if (ti == 0 && ks >= 2) continue;
            const int r = 32 * ti + col;
            bf16x8 wah, wal, uah, ual;
            if constexpr (EX) {
                wah = lds_op16(sm.tw + r * LDP + 16 * ks + 8 * h);
                wal = lds_op16(sm.tw + CH * LDP + r * LDP + 16 * ks + 8 * h);
                uah = lds_op16(sm.tu + r * LDP + 16 * ks + 8 * h);
                ual = lds_op16(sm.tu + CH * LDP + r * LDP + 16 * ks + 8 * h);
            } else {
                f32_op<true>(sm.u.t + r * LDF + 16 * ks + 4 * h, sm.bw + 16 * ks + 4 * h, wah, wal);
                f32_op<true>(sm.u.t + r * LDF + 16 * ks + 4 * h, sm.beta + 16 * ks + 4 * h, uah, ual);
            }
            W[ti] = mma32(wah, kh, W[ti]);
            if (want_U) U[ti] = mma32(uah, vh, U[ti]);
            W[ti] = mma32(wal, kh, W[ti]);
            if (want_U) U[ti] = mma32(ual, vh, U[ti]);
            if (!EX) {
                W[ti] = mma32(wah, kl, W[ti]);
                if (want_U) U[ti] = mma32(uah, vl, U[ti]);
            }
        }
    }
}

// Chunk preparation, part 1 (after stage_chunk and a barrier): the gram
// products. A = masked beta K K^T goes to LDS, and P = masked Q K^T when the
// output is wanted. The caller then synchronises.
template <typename IO, bool WANT_P>
__device__ void prep_gram(Smem<Io<IO>::kExact>& sm, const Params& p, size_t tok0, int nvalid, int hq) {
    const int wave = wave_id();
    const size_t ts_qk = (size_t)p.h_qk * DK;
    const IO* krow0 = static_cast<const IO*>(p.k) + tok0 * ts_qk + (size_t)hq * DK;
    if constexpr (Io<IO>::kExact) transpose_kv(sm);
    if (WANT_P) {
        gram_jobs<IO, 5>(sm, krow0, ts_qk, nvalid, wave, 4);   // jobs w, w+4, ..., w+16
        if (wave == 0) zero_p_tile(sm, 0, 1);
        if (wave == 1) zero_p_tile(sm, 2, 3);
    } else {
        // the ten K K^T tiles: three per wave, the last wave takes one
        if (wave < 3) gram_jobs<IO, 3>(sm, krow0, ts_qk, nvalid, wave, 3);
        else gram_jobs<IO, 1>(sm, krow0, ts_qk, nvalid, 9, 1);
    }
}

// Chunk preparation, part 2 (after prep_gram and a barrier): T = (I + A)^-1,
// U = T diag(beta) V for this wave's columns and W = T diag(beta e^gamma) K.
// On return (before the caller's barrier) -W is being written to LDS; U and
// this wave's W tile are in registers.
template <typename IO>
__device__ void prep_wy(Smem<Io<IO>::kExact>& sm, const Params& p, size_t tok0, int nvalid, int h,
                        bool want_U, f32x16 U[2], f32x16 Wt[2]) {
    constexpr bool EX = Io<IO>::kExact;
    const int wave = wave_id(), lane = lane_id(), col = lane & 31, hh = lane >> 5;
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
    const size_t ts_v = (size_t)p.h_v * DK;
    const IO* vcol = static_cast<const IO*>(p.v) + tok0 * ts_v + (size_t)h * DK + 32 * wave + col;
    wy_tiles<IO>(sm, vcol, ts_v, nvalid, want_U, U, Wt);
    // -W as hi/lo into the region that held A (all reads of A are behind the barrier)
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int r = 32 * ti + acc_row(i, hh), c = 32 * wave + col;
            bf16 th, tl;
            split1(-Wt[ti][i], th, tl);
            sm.x.w[r * LDQ + pk(c)] = th;
            sm.x.w[CH * LDQ + r * LDQ + pk(c)] = tl;
        }
}

// ----------------------------------------------------------------------------
// The state chain of one chunk (after prep_chunk and a barrier).
//   Vp (holds U on entry): V' = U - W S
//   O (if OUT):            O = diag(e^gamma) Q S + P V'   (scale applied at the store)
//   S:                     S <- e^gamma_C S + K^T diag(e^(gamma_C - gamma)) V'
// The state as hi/lo B operands, one pair per 16-row k step (computed once per
// chunk, used by both products with S).
struct SplitS {
    bf16x8 hi[8], lo[8];
};
__device__ __forceinline__ void split_state(const f32x16 S[4], SplitS& ss) {
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) split_half(S[ks >> 1], ks & 1, ss.hi[ks], ss.lo[ks]);
}

// V' = U - W S (Vp holds U on entry).
template <bool EX>
__device__ void chain_vp(const Smem<EX>& sm, const SplitS& ss, f32x16 Vp[2]) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        bf16x8 wh[2], wl[2];
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            const int r = 32 * ti + col;
            wh[ti] = lds_op16(sm.x.w + r * LDQ + 16 * ks + 8 * h);
            wl[ti] = lds_op16(sm.x.w + CH * LDQ + r * LDQ + 16 * ks + 8 * h);
        }
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) Vp[ti] = mma32(wh[ti], ss.hi[ks], Vp[ti]);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) Vp[ti] = mma32(wh[ti], ss.lo[ks], Vp[ti]);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) Vp[ti] = mma32(wl[ti], ss.hi[ks], Vp[ti]);
    }
}

// O = scale (diag(e^gamma) Q S + P V') for this wave's columns (both 32-row
// tiles, interleaved), stored to the output (rows < nvalid).
template <typename IO>
__device__ void chain_out(const Smem<Io<IO>::kExact>& sm, const SplitS& ss, const f32x16 Vp[2],
                          IO* ocol, size_t ts, int nvalid, float scale) {
    constexpr bool EX = Io<IO>::kExact;
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
    f32x16 O[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        bf16x8 qh[2], ql[2];
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            qh[ti] = lds_op16(sm.q_hi + (32 * ti + col) * LDQ + 16 * ks + 8 * h);
            if (!EX) ql[ti] = lds_op16(sm.q_lo + (32 * ti + col) * LDQ + 16 * ks + 8 * h);
        }
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) O[ti] = mma32(qh[ti], ss.hi[ks], O[ti]);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) O[ti] = mma32(qh[ti], ss.lo[ks], O[ti]);
        if (!EX) {
#pragma unroll
            for (int ti = 0; ti < 2; ++ti) O[ti] = mma32(ql[ti], ss.hi[ks], O[ti]);
        }
    }
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int i = 0; i < 16; ++i) O[ti][i] *= sm.eg[32 * ti + acc_row(i, h)];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {  // P is causal: row tile 0 needs k steps 0..1
        bf16x8 vh, vl;
        split_half(Vp[ks >> 1], ks & 1, vh, vl);
#pragma unroll
        for (int ti = 0; ti < 2; ++ti) {
            if (ti == 0 && ks >= 2) continue;
            const bf16x8 ph = lds_op16(sm.p_hi + (32 * ti + col) * LDP + 16 * ks + 8 * h);
            const bf16x8 pl = lds_op16(sm.p_lo + (32 * ti + col) * LDP + 16 * ks + 8 * h);
            O[ti] = mma32(ph, vh, O[ti]);
            O[ti] = mma32(ph, vl, O[ti]);
            O[ti] = mma32(pl, vh, O[ti]);
        }
    }
    if constexpr (EX) {
        // staged in LDS (the T' / T'' area is free until the next chunk's
        // inverse); written to HBM in 16-byte row pieces by store_out
        bf16* st = const_cast<bf16*>(sm.tw);
        const int c = 32 * wave_id() + col;
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int i = 0; i < 16; ++i) st[(32 * ti + acc_row(i, h)) * LDO + c] = (bf16)(O[ti][i] * scale);
    } else {
#pragma unroll
        for (int ti = 0; ti < 2; ++ti)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = 32 * ti + acc_row(i, h);
                if (row < nvalid) ocol[(size_t)row * ts] = (IO)(O[ti][i] * scale);
            }
    }
}

// Copies the staged bf16 output tile of a chunk to HBM (after a barrier).
__device__ void store_out(const Smem<true>& sm, bf16* orow0, size_t ts, int nvalid) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int pc = threadIdx.x + NTHR * it, row = pc >> 4, c8 = (pc & 15) * 8;
        if (row < nvalid)
            *reinterpret_cast<u32x4*>(orow0 + (size_t)row * ts + c8) =
                *reinterpret_cast<const u32x4*>(sm.tw + row * LDO + c8);
    }
}

// S <- e^gamma_C S + K^T diag(e^(gamma_C - gamma)) V' (Vp is scaled in place).
template <bool EX>
__device__ void chain_state(const Smem<EX>& sm, f32x16 S[4], f32x16 Vp[2]) {
    const int lane = lane_id(), col = lane & 31, h = lane >> 5;
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
        bf16x8 kh[4], kl[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            kh[t] = lds_op16(sm.kt_hi + (32 * t + col) * LDKT + 16 * ks + 8 * h);
            if (!EX) kl[t] = lds_op16(sm.kt_lo + (32 * t + col) * LDKT + 16 * ks + 8 * h);
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
    {
        Chunk<IO> r;
        fetch_chunk<IO, false>(r, p, tok0, nvalid, h, hq);
        stage_chunk<IO, false>(sm, r);
    }
    __syncthreads();
    f32x16 U[2], Wt[2];
    prep_gram<IO, false>(sm, p, tok0, nvalid, hq);
    __syncthreads();
    prep_wy<IO>(sm, p, tok0, nvalid, h, true, U, Wt);
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
    Chunk<IO> nxt;
    if (c_lo < c_hi)
        fetch_chunk<IO, false>(nxt, p, loc.tok0 + (size_t)c_lo * CH, min(CH, loc.len - c_lo * CH), h, hq);
    for (int c = c_lo; c < c_hi; ++c) {
        const size_t tok0 = loc.tok0 + (size_t)c * CH;
        const int nvalid = min(CH, loc.len - c * CH);
        stage_chunk<IO, false>(sm, nxt);
        __syncthreads();
        prep_gram<IO, false>(sm, p, tok0, nvalid, hq);
        __syncthreads();
        if (c + 1 < c_hi)
            fetch_chunk<IO, false>(nxt, p, tok0 + CH, min(CH, loc.len - (c + 1) * CH), h, hq);
        f32x16 U[2], Wt[2];
        prep_wy<IO>(sm, p, tok0, nvalid, h, want_U, U, Wt);
        __syncthreads();
        {
            SplitS ss;
            split_state(S, ss);
            chain_vp<EX>(sm, ss, U);
        }
        chain_state<EX>(sm, S, U);
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
    // boundary choices, staged in LDS so that a step never waits on a global load to branch
    __shared__ int wflag[kMaxFlags];
    int n_exact = 0;
    for (int s = 1 + (int)threadIdx.x; s < P; s += NTHR) {
        const int f = p.warm[(size_t)(seg_base + s) * p.h_v + h];
        if (s < kMaxFlags) wflag[s] = f;
        n_exact += (f == 0);
    }
    if (!__syncthreads_or(n_exact)) return;
    auto warm_of = [&](int s) {
        return s < kMaxFlags ? wflag[s] : p.warm[(size_t)(seg_base + s) * p.h_v + h];
    };

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

    // Operands of step s (boundary s) are fetched one step ahead: the warm-up
    // state, or H_{s-1} and this wave's rows of M_{s-1}.
    int warm_n = 0;
    f32x16 tile_n;
    f32x4 m_n[16];
    auto fetch = [&](int s) {
        warm_n = warm_of(s);
        const float* src = warm_n ? p.seg_state + state_off(seg_base + s, p.h_v, h)
                                  : p.seg_H + state_off(seg_base + s - 1, p.h_v, h);
#pragma unroll
        for (int i = 0; i < 16; ++i) tile_n[i] = src[(32 * w + acc_row(i, hh)) * DK + cglob];
        if (!warm_n && (s > 1 || p.s_init)) {
            const float* mrow = p.seg_M + state_off(seg_base + s - 1, p.h_v, h) + (size_t)(32 * w + col) * DK;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                m_n[2 * ks] = *reinterpret_cast<const f32x4*>(mrow + 16 * ks + 4 * hh);
                m_n[2 * ks + 1] = *reinterpret_cast<const f32x4*>(mrow + 16 * ks + 8 + 4 * hh);
            }
        }
    };
    fetch(1);
    __syncthreads();
    int buf = 0;
    for (int s = 1; s < P; ++s) {
        const int warm = warm_n;
        acc = tile_n;
        f32x4 m[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) m[r] = m_n[r];
        if (s + 1 < P) fetch(s + 1);
        if (!warm) {
            if (s > 1 || p.s_init) {
#pragma unroll
                for (int ks = 0; ks < 8; ++ks) {
                    bf16x4 a0h, a0l, a1h, a1l;
                    split4(m[2 * ks], a0h, a0l);
                    split4(m[2 * ks + 1], a1h, a1l);
                    const bf16x8 ah = __builtin_shufflevector(a0h, a1h, 0, 1, 2, 3, 4, 5, 6, 7);
                    const bf16x8 al = __builtin_shufflevector(a0l, a1l, 0, 1, 2, 3, 4, 5, 6, 7);
                    bf16x8 bh, bl;
                    f32_op<false>(&sT[buf][col * LDC + 16 * ks + 4 * hh], nullptr, bh, bl);
                    acc = mma32(ah, bh, acc);
                    acc = mma32(ah, bl, acc);
                    acc = mma32(al, bh, acc);
                }
            }
            float* dst = p.seg_state + state_off(seg_base + s, p.h_v, h);
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
    const size_t ts_v = (size_t)p.h_v * DK;
    Chunk<IO> nxt;
    if (c0 < c1) fetch_chunk<IO, true>(nxt, p, loc.tok0 + (size_t)c0 * CH, min(CH, loc.len - c0 * CH), h, hq);
    for (int c = c0; c < c1; ++c) {
        const size_t tok0 = loc.tok0 + (size_t)c * CH;
        const int nvalid = min(CH, loc.len - c * CH);
        stage_chunk<IO, true>(sm, nxt);
        __syncthreads();
        prep_gram<IO, true>(sm, p, tok0, nvalid, hq);
        __syncthreads();
        if (c + 1 < c1)
            fetch_chunk<IO, true>(nxt, p, tok0 + CH, min(CH, loc.len - (c + 1) * CH), h, hq);
        f32x16 U[2], Wt[2];
        prep_wy<IO>(sm, p, tok0, nvalid, h, true, U, Wt);
        __syncthreads();
        {
            SplitS ss;
            split_state(S, ss);
            chain_vp<EX>(sm, ss, U);
            IO* ocol = static_cast<IO*>(p.out) + tok0 * ts_v + (size_t)h * DK + 32 * wave_id() + (lane_id() & 31);
            chain_out<IO>(sm, ss, U, ocol, ts_v, nvalid, p.scale);
        }
        chain_state<EX>(sm, S, U);
        __syncthreads();
        if constexpr (EX) store_out(sm, static_cast<bf16*>(p.out) + tok0 * ts_v + (size_t)h * DK, ts_v, nvalid);
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
