// Device-side helpers shared by the HIP sources of the Gated DeltaNet kernels
// (types, MFMA wrappers, operand orders, work-item lookup, the wave scan).
// Each translation unit gets its own internal copy (anonymous namespace).
#pragma once
#include <hip/hip_runtime.h>

#include "gdn_internal.h"
#include "gdn_poison.h"

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
typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int CH = kChunk;
constexpr int DK = kDim;
constexpr int NTHR = 256;      // k_cp_combine, k_decode: 4 waves
constexpr int NTHR_CH = 512;   // chain kernels: 8 waves
constexpr int NW_CH = NTHR_CH / 64;
// Row strides of the LDS tiles. A 16x16x32 operand read has sixteen lanes on
// sixteen rows at one 16-byte column (and four such column groups); on gfx950
// such reads run without bank conflicts when the row stride is 32 bytes past
// a multiple of 64 (measured), hence 288- and 160-byte rows.
constexpr int LDQ = 144;   // row stride (elements) of [64][128] bf16 tiles
constexpr int LDKT = 80;   // row stride of [128][64] bf16 tiles
constexpr int LDF = 72;    // row stride of [64][64] fp32 tiles
constexpr int LDP = 80;    // row stride of [64][64] bf16 tiles
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
// fp16 operands (the forward's chain kernels): 11-bit significands, fp32 accumulation
__device__ __forceinline__ f32x4 mmh(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// two accumulator tiles (4 + 4 values) as one fp16 operand, rounded to nearest even
__device__ __forceinline__ f16x8 pack8h(const f32x4& a, const f32x4& b) {
    return __builtin_convertvector(f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}, f16x8);
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

// hi/lo operand of eight accumulator values: elements 0..3 from a, 4..7 from b.
__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, bf16x8& hi, bf16x8& lo) {
    unsigned h[4], l[4];
    split_pair(a[0], a[1], h[0], l[0]);
    split_pair(a[2], a[3], h[1], l[1]);
    split_pair(b[0], b[1], h[2], l[2]);
    split_pair(b[2], b[3], h[3], l[3]);
    hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
    lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
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

// Position of contraction index x in an LDS operand row: within each block of
// 32, x = 16 b4 + 4 a + e (a < 4, e < 4) sits at 8 a + 4 b4 + e.
__device__ __forceinline__ int kp(int x) {
    return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}

// Transposed tiles (K^T, V^T: row = d_k or d_v index d, 64 tokens) XOR their
// 8-element chunks with (d / 16) mod 8: the staging stores (32 lanes on rows
// four apart) then meet at most two to a bank, and the operand reads (16
// consecutive rows) not at all.
__device__ __forceinline__ int tswz(int d) { return 8 * ((d >> 4) & 7); }

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

template <typename PP>
__device__ SegLoc locate_segment(const PP& p, int slot) {
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
template <typename PP>
__device__ bool locate_chunk(const PP& p, int slot, int& seq, int& c, int& len, size_t& tok0) {
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
// DPP steps: shifts by 1, 2, 4, 8 lanes within each row of 16 (lanes without a
// source add 0), then lane 15 of a row added to the next row (rows 1 and 3),
// then lane 31 added to rows 2 and 3.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float s) {
    return s + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), CTRL, ROW_MASK,
                                                                      0xf, true));
}
__device__ __forceinline__ float wave_scan(float s) {
    s = dpp_add<0x111, 0xf>(s);   // row_shr:1
    s = dpp_add<0x112, 0xf>(s);   // row_shr:2
    s = dpp_add<0x114, 0xf>(s);   // row_shr:4
    s = dpp_add<0x118, 0xf>(s);   // row_shr:8
    s = dpp_add<0x142, 0xa>(s);   // row_bcast:15
    s = dpp_add<0x143, 0xc>(s);   // row_bcast:31
    return s;
}

}  // namespace
}  // namespace gdn
