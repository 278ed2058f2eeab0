// Backward pass of the Gated DeltaNet chunked prefill on MI355X (gfx950).
//
// The FlashQLA pages ("FlashQLA: CP-/Bwd-friendly fused linear attention
// kernels for GDN") promise a backward that runs as long compute chains rather
// than many small stages, but print no backward formulas. The gradients here
// are those of the chunked form the forward evaluates (its formulas are in the
// forward's kernel file), per chunk of C = 64 tokens with incoming state S,
// loss gradient dSn of the outgoing state and dO of the outputs:
//   gamma = cumsum(g), e_r = exp(gamma_r), f_r = exp(gamma_C - gamma_r),
//   A_ri = beta_r exp(gamma_r - gamma_i) k_r.k_i (i < r), T = (I + A)^-1,
//   P_ri = q_r.k_i exp(gamma_r - gamma_i) (i <= r),
//   Y = V - diag(e) K S, V' = T diag(beta) Y.
// Reverse steps:
//   dV' = diag(f) K dSn + scale P^T dO
//   Z = T^T dV', dv = dY = diag(beta) Z, dbeta_r += Z_r . Y_r
//   dS (state entering the chunk) = e_C dSn + scale Q^T diag(e) dO - K^T diag(e) dY
//   dP = scale dO V'^T, Psi = dP o exp(gamma_r - gamma_i) (i <= r)
//   dq = scale diag(e) dO S^T + Psi K
//   dK~ = V' dSn^T;  dk = Psi^T Q + diag(f) dK~ - diag(e) dY S^T + (G + G^T) K
//   dT = dV' (diag(beta) Y)^T, dA = -T^T dT T^T (strictly lower part),
//   G_ri = dA_ri beta_r exp(gamma_r - gamma_i), dbeta_r += sum_i dA_ri A_ri / beta_r
//   dgamma from every exponential it enters (P, e, f, A, e_C), dg = reverse
//   cumulative sum of dgamma over the chunk.
// Kernels: the forward (re-run with the state entering every chunk written
// out), k_bwd_prep (T, P, gamma per chunk and head, and T^T / scale P^T as
// bf16 hi/lo images), the reverse scan of dS over the chunks on the matrix
// cores (k_bwd_chain_mma, in the forward's kernel file, which shares its
// operand layouts), k_bwd_chunk (every other gradient, all chunks in
// parallel, fp32 on the vector ALUs) and k_bwd_sum (query/key gradients
// summed over the value heads of a group). bf16 inputs only.
#include <hip/hip_runtime.h>

#include "gdn_internal.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int CH = kChunk;
constexpr int DK = kDim;
constexpr int NT = 256;
constexpr int LKB = 136;   // bf16 row stride of the [64][128] K, Q tiles
constexpr int LX = 132;    // fp32 row stride of [64][128] tiles
constexpr int LM = 68;     // fp32 row stride of [64][64] tiles

__device__ __forceinline__ int n_chunks_of(int len) { return (len + CH - 1) / CH; }
__device__ __forceinline__ size_t state_off(int idx, int h_v, int h) {
    return ((size_t)idx * h_v + h) * (size_t)DK * DK;
}
__device__ __forceinline__ float bf2f(bf16 x) { return (float)x; }
__device__ __forceinline__ f32x4 bf4(const bf16* x) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(x);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                 __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
}
__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }
__device__ __forceinline__ unsigned pack_rne(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
// Position of token x in an operand row of the matrix-core chain (within each
// block of 32, x = 16 b + 4 a + e sits at 8 a + 4 b + e: the order in which a
// 32-row accumulator pair serves as an MFMA operand).
__device__ __forceinline__ int kp(int x) {
    return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}
// hi = x with its low 16 bits cleared, lo = x - hi rounded to bf16
__device__ __forceinline__ void split1(float x, bf16& hi, bf16& lo) {
    const unsigned u = __float_as_uint(x);
    hi = __builtin_bit_cast(bf16, (unsigned short)(u >> 16));
    lo = (bf16)(x - __uint_as_float(u & 0xffff0000u));
}
// sum over the 32 lanes of a half wave
__device__ __forceinline__ float sum32(float x) {
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// Chunk slot -> (sequence, chunk within it, sequence length, first token).
__device__ bool bwd_locate(const BwdParams& p, int slot, int& seq, int& c, int& len, size_t& tok_s) {
    if (!p.cu) {
        const int N = n_chunks_of(p.seq_len);
        if (N == 0) return false;
        seq = slot / N;
        c = slot - seq * N;
        len = p.seq_len;
        tok_s = (size_t)seq * p.seq_len;
        return seq < p.n_seqs;
    }
    int base = 0;
    for (int n = 0; n < p.n_seqs; ++n) {
        const int a = p.cu[n], l = p.cu[n + 1] - a, N = n_chunks_of(l);
        if (slot < base + N) {
            seq = n; c = slot - base; len = l; tok_s = (size_t)a;
            return true;
        }
        base += N;
    }
    return false;
}

// K and Q rows of a chunk into [64][LKB] bf16 tiles (rows past nv zero).
template <int NTHR = NT>
__device__ void load_kq(const BwdParams& p, size_t tok0, int nv, int hq, bf16 (*kb)[LKB], bf16 (*qb)[LKB]) {
    const size_t ts = (size_t)p.h_qk * DK;
    const bf16* k = static_cast<const bf16*>(p.k) + tok0 * ts + (size_t)hq * DK;
    const bf16* q = static_cast<const bf16*>(p.q) + tok0 * ts + (size_t)hq * DK;
    for (int idx = threadIdx.x; idx < CH * 16; idx += NTHR) {
        const int r = idx >> 4, part = (idx & 15) * 8;
        u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
        if (r < nv) {
            kv = *reinterpret_cast<const u32x4*>(k + (size_t)r * ts + part);
            qv = *reinterpret_cast<const u32x4*>(q + (size_t)r * ts + part);
        }
        *reinterpret_cast<u32x4*>(&kb[r][part]) = kv;
        *reinterpret_cast<u32x4*>(&qb[r][part]) = qv;
    }
}

// ----------------------------------------------------------------------------
// T = (I + A)^-1, P and gamma of one (chunk, value head), fp32.
__global__ __launch_bounds__(NT) void k_bwd_prep(BwdParams p) {
    __shared__ bf16 kb[CH][LKB], qb[CH][LKB];
    __shared__ float am[CH][LM], tm[CH][LM];
    __shared__ float gam[CH], bet[CH];
    // P takes Q's tile once Q K^T is formed (same size: 64 x 136 bf16 = 64 x 68 fp32)
    float (*pmat)[LM] = reinterpret_cast<float (*)[LM]>(&qb[0][0]);
    static_assert(sizeof(qb) == CH * LM * sizeof(float), "P reuses the Q tile");
    const int f = blockIdx.x, h = blockIdx.y, hq = h / p.group, t = threadIdx.x;
    int seq, c, len;
    size_t tok_s;
    if (!bwd_locate(p, f, seq, c, len, tok_s)) return;
    const size_t tok0 = tok_s + (size_t)c * CH;
    const int nv = min(CH, len - c * CH);
    float* out = p.tpg + ((size_t)f * p.h_v + h) * kBwdTpg;
    load_kq(p, tok0, nv, hq, kb, qb);
    if (t < CH) {   // wave 0: inclusive scan of g over the chunk
        float x = t < nv ? p.g[(tok0 + t) * p.h_v + h] : 0.f;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(x, d, 64);
            if (t >= d) x += y;
        }
        gam[t] = x;
        bet[t] = t < nv ? p.beta[(tok0 + t) * p.h_v + h] : 0.f;
        out[2 * CH * CH + t] = x;
    }
    __syncthreads();
    {   // A (strictly lower) and P (lower with the diagonal): row r, columns i0 + 4 ii
        const int r = t >> 2, i0 = t & 3;
        float kk[16], qk[16];
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) kk[ii] = qk[ii] = 0.f;
        for (int d = 0; d < DK; d += 4) {
            const f32x4 kr = bf4(&kb[r][d]), qr = bf4(&qb[r][d]);
#pragma unroll
            for (int ii = 0; ii < 16; ++ii) {
                const f32x4 ki = bf4(&kb[i0 + 4 * ii][d]);
                kk[ii] += dot4(kr, ki);
                qk[ii] += dot4(qr, ki);
            }
        }
        float* P = out + CH * CH;
        __syncthreads();   // every read of Q is done before P overwrites its tile
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) {
            const int i = i0 + 4 * ii;
            const float ex = i <= r ? __expf(gam[r] - gam[i]) : 0.f;
            am[r][i] = i < r ? bet[r] * ex * kk[ii] : 0.f;
            const float pv = i <= r ? ex * qk[ii] : 0.f;
            P[r * CH + i] = pv;
            pmat[r][i] = pv;
        }
    }
    __syncthreads();
    if (t < CH) {   // forward substitution, one column per lane: T[i][c] = d_ic - sum_j A[i][j] T[j][c]
        const int col = t;
        for (int i = 0; i < CH; ++i) {
            // four independent partial sums keep the LDS reads ahead of the adds
            float s0 = (i == col) ? 1.f : 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
            int j = col;
            for (; j + 4 <= i; j += 4) {
                s0 -= am[i][j] * tm[j][col];
                s1 -= am[i][j + 1] * tm[j + 1][col];
                s2 -= am[i][j + 2] * tm[j + 2][col];
                s3 -= am[i][j + 3] * tm[j + 3][col];
            }
            for (; j < i; ++j) s0 -= am[i][j] * tm[j][col];
            tm[i][col] = i >= col ? (s0 + s1) + (s2 + s3) : 0.f;
        }
    }
    __syncthreads();
    for (int idx = t; idx < CH * CH; idx += NT) out[idx] = tm[idx >> 6][idx & 63];
    // T^T and scale P^T as hi/lo bf16 rows with the contraction token in kp order
    // (four consecutive tokens stay consecutive in kp order: one 8-byte store each)
    bf16* img = static_cast<bf16*>(p.tpt) + ((size_t)f * p.h_v + h) * kBwdTpt;
    for (int idx = t; idx < CH * CH / 4; idx += NT) {
        const int r = idx >> 4, m4 = (idx & 15) * 4, o = r * CH + kp(m4);
        bf16 th[4], tl[4], ph[4], pl[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            split1(tm[m4 + e][r], th[e], tl[e]);
            split1(p.scale * pmat[m4 + e][r], ph[e], pl[e]);
        }
        auto pack = [](const bf16 (&x)[4]) {
            return u32x2{(unsigned)__builtin_bit_cast(unsigned short, x[0]) |
                             ((unsigned)__builtin_bit_cast(unsigned short, x[1]) << 16),
                         (unsigned)__builtin_bit_cast(unsigned short, x[2]) |
                             ((unsigned)__builtin_bit_cast(unsigned short, x[3]) << 16)};
        };
        *reinterpret_cast<u32x2*>(img + o) = pack(th);
        *reinterpret_cast<u32x2*>(img + CH * CH + o) = pack(tl);
        *reinterpret_cast<u32x2*>(img + 2 * CH * CH + o) = pack(ph);
        *reinterpret_cast<u32x2*>(img + 3 * CH * CH + o) = pack(pl);
    }
}

// ----------------------------------------------------------------------------
// Every gradient of one (chunk, value head) given the state entering the
// chunk and the gradient of the state leaving it; 8 waves. Thread t owns rows
// 4 (t / 32) .. + 3 and columns 4 (t % 32) .. + 3 of every [64 x 128] result
// (dq and dk accumulate there across the steps); [64 x 64] results are split
// as row t / 8, columns t % 8 + 8 q (q < 8).
constexpr int NTC = 512;
constexpr int RPT = 4;     // rows of a [64 x 128] result per thread
constexpr int QPT = 8;     // columns of a [64 x 64] result per thread
struct ChunkSmem {
    bf16 kb[CH][LKB], qb[CH][LKB];
    float x1[CH][LX];           // Y, then dY
    float x2[CH][LX];           // V', then dV'
    float m1[CH][LM];           // T
    float m2[CH][LM];           // P, then dT T^T, then G
    float m3[CH][LM];           // Psi, then dT, then dA
    float gam[CH], eg[CH], fr[CH], bet[CH], dgam[CH], dbe[CH];
    float dgc;
};

__global__ __launch_bounds__(NTC) void k_bwd_chunk(BwdParams p) {
    __shared__ ChunkSmem sm;
    const int f = blockIdx.x, h = blockIdx.y, hq = h / p.group, t = threadIdx.x;
    int seq, c, len;
    size_t tok_s;
    if (!bwd_locate(p, f, seq, c, len, tok_s)) return;
    const size_t tok0 = tok_s + (size_t)c * CH;
    const int nv = min(CH, len - c * CH);
    const float* S = p.cs + state_off(f, p.h_v, h);
    const float* dSn = p.ds + state_off(f, p.h_v, h);
    const float* tp = p.tpg + ((size_t)f * p.h_v + h) * kBwdTpg;
    const size_t ts_v = (size_t)p.h_v * DK;
    const bf16* V = static_cast<const bf16*>(p.v) + tok0 * ts_v + (size_t)h * DK;
    const bf16* dO = static_cast<const bf16*>(p.dout) + tok0 * ts_v + (size_t)h * DK;
    const float scale = p.scale;

    load_kq<NTC>(p, tok0, nv, hq, sm.kb, sm.qb);
    for (int idx = t; idx < CH * CH / 4; idx += NTC) {
        const int rr = idx >> 4, cc = (idx & 15) * 4;
        *reinterpret_cast<f32x4*>(&sm.m1[rr][cc]) = *reinterpret_cast<const f32x4*>(tp + rr * CH + cc);
        *reinterpret_cast<f32x4*>(&sm.m2[rr][cc]) = *reinterpret_cast<const f32x4*>(tp + CH * CH + rr * CH + cc);
    }
    if (t < CH) {
        const float gm = tp[2 * CH * CH + t];
        sm.gam[t] = gm;
        sm.eg[t] = __expf(gm);
        sm.bet[t] = t < nv ? p.beta[(tok0 + t) * p.h_v + h] : 0.f;
        sm.dgam[t] = 0.f;
        sm.dbe[t] = 0.f;
    }
    if (t == 0) sm.dgc = 0.f;
    __syncthreads();
    if (t < CH) sm.fr[t] = __expf(sm.gam[CH - 1] - sm.gam[t]);
    const float eC = __expf(sm.gam[CH - 1]);
    __syncthreads();

    const int r0 = RPT * (t >> 5), j0 = 4 * (t & 31), lane32 = t & 31;
    // [64 x 64] results: row t / 8, columns t % 8 + 8 q (interleaved, so that the
    // eight lanes of a row group read rows one apart: no LDS bank conflicts)
    const int pr = t >> 3, pi0 = t & 7;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 dq[RPT], dk[RPT];
#pragma unroll
    for (int e = 0; e < RPT; ++e) dq[e] = dk[e] = zero4;
    auto vrow = [&](const bf16* base, int r) { return r < nv ? bf4(base + (size_t)r * ts_v + j0) : zero4; };

    // 1. K S and Q S: Y = V - diag(e) K S; the output's Q S term in dgamma
    {
        f32x4 ks[RPT], qs[RPT];
#pragma unroll
        for (int e = 0; e < RPT; ++e) ks[e] = qs[e] = zero4;
        for (int i = 0; i < DK; ++i) {
            const f32x4 s = *reinterpret_cast<const f32x4*>(S + (size_t)i * DK + j0);
#pragma unroll
            for (int e = 0; e < RPT; ++e) {
                ks[e] += bf2f(sm.kb[r0 + e][i]) * s;
                qs[e] += bf2f(sm.qb[r0 + e][i]) * s;
            }
        }
#pragma unroll
        for (int e = 0; e < RPT; ++e) {
            const int r = r0 + e;
            *reinterpret_cast<f32x4*>(&sm.x1[r][j0]) = vrow(V, r) - sm.eg[r] * ks[e];
            const float part = sum32(dot4(qs[e], vrow(dO, r)));
            if (lane32 == 0) atomicAdd(&sm.dgam[r], scale * sm.eg[r] * part);
        }
    }
    __syncthreads();
    // 2. V' = T diag(beta) Y
    {
        f32x4 a[RPT];
#pragma unroll
        for (int e = 0; e < RPT; ++e) a[e] = zero4;
        for (int i = 0; i < CH; ++i) {
            const f32x4 y = sm.bet[i] * *reinterpret_cast<const f32x4*>(&sm.x1[i][j0]);
#pragma unroll
            for (int e = 0; e < RPT; ++e) a[e] += sm.m1[r0 + e][i] * y;
        }
#pragma unroll
        for (int e = 0; e < RPT; ++e) *reinterpret_cast<f32x4*>(&sm.x2[r0 + e][j0]) = a[e];
    }
    __syncthreads();
    // 3. dK~ = V' dSn^T (into dk with diag(f); its dgamma terms), dP = scale dO V'^T -> Psi
    {
        f32x4 a[RPT];
#pragma unroll
        for (int e = 0; e < RPT; ++e) a[e] = zero4;
        for (int j = 0; j < DK; j += 4) {
            const f32x4 d0 = *reinterpret_cast<const f32x4*>(dSn + (size_t)(j0 + 0) * DK + j);
            const f32x4 d1 = *reinterpret_cast<const f32x4*>(dSn + (size_t)(j0 + 1) * DK + j);
            const f32x4 d2 = *reinterpret_cast<const f32x4*>(dSn + (size_t)(j0 + 2) * DK + j);
            const f32x4 d3 = *reinterpret_cast<const f32x4*>(dSn + (size_t)(j0 + 3) * DK + j);
#pragma unroll
            for (int e = 0; e < RPT; ++e) {
                const f32x4 vv = *reinterpret_cast<const f32x4*>(&sm.x2[r0 + e][j]);
                a[e] += f32x4{dot4(vv, d0), dot4(vv, d1), dot4(vv, d2), dot4(vv, d3)};
            }
        }
#pragma unroll
        for (int e = 0; e < RPT; ++e) {
            const int r = r0 + e;
            dk[e] += sm.fr[r] * a[e];
            const float kap = sum32(sm.fr[r] * dot4(bf4(&sm.kb[r][j0]), a[e]));
            if (lane32 == 0) {
                atomicAdd(&sm.dgam[r], -kap);
                atomicAdd(&sm.dgc, kap);
            }
        }
    }
    {
        float a[QPT];
#pragma unroll
        for (int q = 0; q < QPT; ++q) a[q] = 0.f;
        for (int j = 0; j < DK; j += 4) {
            const f32x4 dov = pr < nv ? bf4(dO + (size_t)pr * ts_v + j) : zero4;
#pragma unroll
            for (int q = 0; q < QPT; ++q) a[q] += dot4(dov, *reinterpret_cast<const f32x4*>(&sm.x2[pi0 + 8 * q][j]));
        }
        float erow = 0.f;
#pragma unroll
        for (int q = 0; q < QPT; ++q) {
            const int i = pi0 + 8 * q;
            float psi = 0.f, E = 0.f;
            if (i <= pr) {
                const float dP = scale * a[q];
                psi = dP * __expf(sm.gam[pr] - sm.gam[i]);
                E = dP * sm.m2[pr][i];
            }
            sm.m3[pr][i] = psi;
            erow += E;
            if (E != 0.f) atomicAdd(&sm.dgam[i], -E);
        }
        atomicAdd(&sm.dgam[pr], erow);
    }
    __syncthreads();
    // 4. dV' = diag(f) K dSn + scale P^T dO; dq += Psi K + scale diag(e) dO S^T; dk += Psi^T Q
    {
        f32x4 a[RPT];
#pragma unroll
        for (int e = 0; e < RPT; ++e) a[e] = zero4;
        for (int i = 0; i < DK; ++i) {
            const f32x4 d = *reinterpret_cast<const f32x4*>(dSn + (size_t)i * DK + j0);
#pragma unroll
            for (int e = 0; e < RPT; ++e) a[e] += bf2f(sm.kb[r0 + e][i]) * d;
        }
#pragma unroll
        for (int e = 0; e < RPT; ++e) a[e] *= sm.fr[r0 + e];
        for (int m = 0; m < nv; ++m) {
            const f32x4 dov = scale * bf4(dO + (size_t)m * ts_v + j0);
#pragma unroll
            for (int e = 0; e < RPT; ++e) a[e] += sm.m2[m][r0 + e] * dov;
        }
#pragma unroll
        for (int e = 0; e < RPT; ++e) *reinterpret_cast<f32x4*>(&sm.x2[r0 + e][j0]) = a[e];
        for (int m = 0; m < CH; ++m) {
            const f32x4 kk = bf4(&sm.kb[m][j0]), qq = bf4(&sm.qb[m][j0]);
#pragma unroll
            for (int e = 0; e < RPT; ++e) {
                dq[e] += sm.m3[r0 + e][m] * kk;
                dk[e] += sm.m3[m][r0 + e] * qq;
            }
        }
        f32x4 b[RPT];
#pragma unroll
        for (int e = 0; e < RPT; ++e) b[e] = zero4;
        for (int j = 0; j < DK; j += 4) {
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(S + (size_t)(j0 + 0) * DK + j);
            const f32x4 s1 = *reinterpret_cast<const f32x4*>(S + (size_t)(j0 + 1) * DK + j);
            const f32x4 s2 = *reinterpret_cast<const f32x4*>(S + (size_t)(j0 + 2) * DK + j);
            const f32x4 s3 = *reinterpret_cast<const f32x4*>(S + (size_t)(j0 + 3) * DK + j);
#pragma unroll
            for (int e = 0; e < RPT; ++e) {
                const int r = r0 + e;
                const f32x4 dov = r < nv ? bf4(dO + (size_t)r * ts_v + j) : zero4;
                b[e] += f32x4{dot4(dov, s0), dot4(dov, s1), dot4(dov, s2), dot4(dov, s3)};
            }
        }
#pragma unroll
        for (int e = 0; e < RPT; ++e) dq[e] += (scale * sm.eg[r0 + e]) * b[e];
    }
    __syncthreads();
    // 5. Z = T^T dV', dY = diag(beta) Z (the dv output), dbeta and dgamma terms; dT = dV' (diag(beta) Y)^T
    f32x4 dy[RPT];
    {
#pragma unroll
        for (int e = 0; e < RPT; ++e) dy[e] = zero4;
        for (int m = 0; m < CH; ++m) {
            const f32x4 d = *reinterpret_cast<const f32x4*>(&sm.x2[m][j0]);
#pragma unroll
            for (int e = 0; e < RPT; ++e) dy[e] += sm.m1[m][r0 + e] * d;
        }
        bf16* dvo = static_cast<bf16*>(p.dv) + tok0 * ts_v + (size_t)h * DK + j0;
#pragma unroll
        for (int e = 0; e < RPT; ++e) {
            const int r = r0 + e;
            const f32x4 y = *reinterpret_cast<const f32x4*>(&sm.x1[r][j0]);
            const float zb = sum32(dot4(dy[e], y));
            dy[e] *= sm.bet[r];
            const float ky = sum32(dot4(vrow(V, r) - y, dy[e]));
            if (lane32 == 0) {
                atomicAdd(&sm.dbe[r], zb);
                atomicAdd(&sm.dgam[r], -ky);
            }
            if (r < nv)
                *reinterpret_cast<u32x2*>(dvo + (size_t)r * ts_v) = u32x2{pack_rne(dy[e][0], dy[e][1]),
                                                                       pack_rne(dy[e][2], dy[e][3])};
        }
        float a[QPT];
#pragma unroll
        for (int q = 0; q < QPT; ++q) a[q] = 0.f;
        for (int j = 0; j < DK; j += 4) {
            const f32x4 d = *reinterpret_cast<const f32x4*>(&sm.x2[pr][j]);
#pragma unroll
            for (int q = 0; q < QPT; ++q) a[q] += dot4(d, *reinterpret_cast<const f32x4*>(&sm.x1[pi0 + 8 * q][j]));
        }
#pragma unroll
        for (int q = 0; q < QPT; ++q) sm.m3[pr][pi0 + 8 * q] = a[q] * sm.bet[pi0 + 8 * q];
    }
    __syncthreads();
    // 6. dY into x1 (Y is no longer read); dT T^T into m2
    {
#pragma unroll
        for (int e = 0; e < RPT; ++e) *reinterpret_cast<f32x4*>(&sm.x1[r0 + e][j0]) = dy[e];
        float a[QPT];
#pragma unroll
        for (int q = 0; q < QPT; ++q) a[q] = 0.f;
        for (int m = 0; m < CH; ++m) {
            const float d = sm.m3[pr][m];
#pragma unroll
            for (int q = 0; q < QPT; ++q) a[q] += d * sm.m1[pi0 + 8 * q][m];
        }
#pragma unroll
        for (int q = 0; q < QPT; ++q) sm.m2[pr][pi0 + 8 * q] = a[q];
    }
    __syncthreads();
    // 7. dA = -T^T (dT T^T), strictly lower, into m3; dk -= diag(e) dY S^T
    {
        float a[QPT];
#pragma unroll
        for (int q = 0; q < QPT; ++q) a[q] = 0.f;
        for (int m = 0; m < CH; ++m) {
            const float tv = sm.m1[m][pr];
#pragma unroll
            for (int q = 0; q < QPT; ++q) a[q] += tv * sm.m2[m][pi0 + 8 * q];
        }
#pragma unroll
        for (int q = 0; q < QPT; ++q) sm.m3[pr][pi0 + 8 * q] = (pi0 + 8 * q < pr) ? -a[q] : 0.f;
        f32x4 b[RPT];
#pragma unroll
        for (int e = 0; e < RPT; ++e) b[e] = zero4;
        for (int j = 0; j < DK; j += 4) {
            const f32x4 s0 = *reinterpret_cast<const f32x4*>(S + (size_t)(j0 + 0) * DK + j);
            const f32x4 s1 = *reinterpret_cast<const f32x4*>(S + (size_t)(j0 + 1) * DK + j);
            const f32x4 s2 = *reinterpret_cast<const f32x4*>(S + (size_t)(j0 + 2) * DK + j);
            const f32x4 s3 = *reinterpret_cast<const f32x4*>(S + (size_t)(j0 + 3) * DK + j);
#pragma unroll
            for (int e = 0; e < RPT; ++e) {
                const f32x4 d = *reinterpret_cast<const f32x4*>(&sm.x1[r0 + e][j]);
                b[e] += f32x4{dot4(d, s0), dot4(d, s1), dot4(d, s2), dot4(d, s3)};
            }
        }
#pragma unroll
        for (int e = 0; e < RPT; ++e) dk[e] -= sm.eg[r0 + e] * b[e];
    }
    __syncthreads();
    // 8. through A: dbeta, dgamma and G (into m2)
    {
        float kk[QPT];
#pragma unroll
        for (int q = 0; q < QPT; ++q) kk[q] = 0.f;
        for (int d = 0; d < DK; d += 4) {
            const f32x4 kr = bf4(&sm.kb[pr][d]);
#pragma unroll
            for (int q = 0; q < QPT; ++q) kk[q] += dot4(kr, bf4(&sm.kb[pi0 + 8 * q][d]));
        }
        float db = 0.f, dgr = 0.f;
#pragma unroll
        for (int q = 0; q < QPT; ++q) {
            const int i = pi0 + 8 * q;
            float G = 0.f;
            if (i < pr) {
                const float ex = __expf(sm.gam[pr] - sm.gam[i]), da = sm.m3[pr][i];
                const float w = da * ex * kk[q];   // dA_ri times dA_ri/dbeta_r
                db += w;
                const float gA = w * sm.bet[pr];   // dA_ri A_ri
                dgr += gA;
                atomicAdd(&sm.dgam[i], -gA);
                G = da * sm.bet[pr] * ex;
            }
            sm.m2[pr][i] = G;
        }
        atomicAdd(&sm.dbe[pr], db);
        atomicAdd(&sm.dgam[pr], dgr);
    }
    {   // dgamma_C from the decay of the state: e_C <S, dSn>
        float part = 0.f;
        for (int idx = t; idx < DK * DK / 4; idx += NTC)
            part += dot4(*reinterpret_cast<const f32x4*>(S + 4 * idx), *reinterpret_cast<const f32x4*>(dSn + 4 * idx));
        part = sum32(part);
        if (lane32 == 0) atomicAdd(&sm.dgc, eC * part);
    }
    __syncthreads();
    // 9. dk += (G + G^T) K
    for (int m = 0; m < CH; ++m) {
        const f32x4 kk = bf4(&sm.kb[m][j0]);
#pragma unroll
        for (int e = 0; e < RPT; ++e) dk[e] += (sm.m2[r0 + e][m] + sm.m2[m][r0 + e]) * kk;
    }
    // outputs: per-head parts of dq and dk; dg as the reverse cumulative sum of dgamma; dbeta
    {
        float* dqp = p.dq_part + (tok0 * p.h_v + h) * DK + j0;
        float* dkp = p.dk_part + (tok0 * p.h_v + h) * DK + j0;
#pragma unroll
        for (int e = 0; e < RPT; ++e) {
            const int r = r0 + e;
            if (r < nv) {
                *reinterpret_cast<f32x4*>(dqp + (size_t)r * ts_v) = dq[e];
                *reinterpret_cast<f32x4*>(dkp + (size_t)r * ts_v) = dk[e];
            }
        }
    }
    if (t < CH) {
        float x = sm.dgam[t] + (t == CH - 1 ? sm.dgc : 0.f);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_down(x, d, 64);
            if (t + d < 64) x += y;
        }
        if (t < nv) {
            p.dg[(tok0 + t) * p.h_v + h] = x;
            p.dbeta[(tok0 + t) * p.h_v + h] = sm.dbe[t];
        }
    }
}

// dq, dk: sum the per-value-head parts over each query/key head's group.
__global__ __launch_bounds__(NT) void k_bwd_sum(BwdParams p, long long n_tokens) {
    const long long idx = (long long)blockIdx.x * NT + threadIdx.x;   // one thread per 4 elements
    const long long per_tok = (long long)p.h_qk * DK / 4;
    if (idx >= n_tokens * per_tok) return;
    const long long tok = idx / per_tok;
    const int rem = (int)(idx - tok * per_tok), hq = rem / (DK / 4), col = (rem % (DK / 4)) * 4;
    f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
    for (int e = 0; e < p.group; ++e) {
        const size_t o = ((size_t)tok * p.h_v + hq * p.group + e) * DK + col;
        a += *reinterpret_cast<const f32x4*>(p.dq_part + o);
        b += *reinterpret_cast<const f32x4*>(p.dk_part + o);
    }
    const size_t oo = ((size_t)tok * p.h_qk + hq) * DK + col;
    *reinterpret_cast<u32x2*>(static_cast<bf16*>(p.dq) + oo) = u32x2{pack_rne(a[0], a[1]), pack_rne(a[2], a[3])};
    *reinterpret_cast<u32x2*>(static_cast<bf16*>(p.dk) + oo) = u32x2{pack_rne(b[0], b[1]), pack_rne(b[2], b[3])};
}

}  // namespace

static int launched() { return (int)hipGetLastError(); }

int launch_bwd(const BwdParams& p, void* stream) {
    const hipStream_t s = (hipStream_t)stream;
    int e;
    if (p.n_chunks > 0) {
        hipLaunchKernelGGL(k_bwd_prep, dim3(p.n_chunks, p.h_v), dim3(NT), 0, s, p);
        if ((e = launched())) return e;
    }
    if ((e = launch_bwd_chain_mma(p, stream))) return e;
    if (p.n_chunks > 0) {
        hipLaunchKernelGGL(k_bwd_chunk, dim3(p.n_chunks, p.h_v), dim3(NTC), 0, s, p);
        if ((e = launched())) return e;
    }
    return 0;
}

int launch_bwd_sum(const BwdParams& p, long long n_tokens, void* stream) {
    if (n_tokens <= 0) return 0;
    const long long n = n_tokens * p.h_qk * DK / 4;
    hipLaunchKernelGGL(k_bwd_sum, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, (hipStream_t)stream, p,
                       n_tokens);
    return launched();
}

}  // namespace gdn
