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
// cores split by the forward's segments (k_bwd_chain_mma, linked by k_cp_combine), every
// other gradient of every chunk in parallel on the matrix cores
// (k_bwd_chunk_mma) -- both in the forward's kernel file, whose operand
// layouts they share -- and k_bwd_sum (query/key gradients summed over the
// value heads of a group). The kernels read bf16 q, k, v, dO; fp32 inputs are
// rounded once to bf16 by k_round_bf16 and their gradients written in fp32.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "gdn_internal.h"
#include "gdn_poison.h"

namespace gdn {
namespace {

typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int CH = kChunk;
constexpr int DK = kDim;
constexpr int NT = 256;
constexpr int LKB = 136;   // bf16 row stride of the [64][128] K, Q tiles
constexpr int LM = 68;     // fp32 row stride of [64][64] tiles

__device__ __forceinline__ int n_chunks_of(int len) { return (len + CH - 1) / CH; }
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

// Item (chunk slot f, value head h) = f h_v + h: the chunk's first token and its
// token count (f < n_chunks: always found).
__device__ __forceinline__ void prep_item(const BwdParams& p, long long item, int& f, int& h, size_t& tok0, int& nv) {
    f = (int)(item / p.h_v);
    h = (int)(item - (long long)f * p.h_v);
    int seq, c, len;
    size_t tok_s;
    bwd_locate(p, f, seq, c, len, tok_s);
    tok0 = tok_s + (size_t)c * CH;
    nv = min(CH, len - c * CH);
}
// One item's inputs from memory, fetched an item ahead so that their latency
// hides behind the previous item's work.
struct PrepIn {
    u32x4 k[4], q[4];   // K, Q row (t + 256 j) / 16, eight columns at 8 ((t + 256 j) % 16) (rows past nv repeat the last)
    float g, b;         // gate and beta of token t % 64 (the last valid one past nv)
};
__device__ __forceinline__ void prep_fetch(const BwdParams& p, long long item, PrepIn& in) {
    int f, h, nv;
    size_t tok0;
    prep_item(p, item, f, h, tok0, nv);
    const int t = threadIdx.x, hq = h / p.group;
    const size_t ts = (size_t)p.h_qk * DK;
    const bf16* k = static_cast<const bf16*>(p.k) + tok0 * ts + (size_t)hq * DK;
    const bf16* q = static_cast<const bf16*>(p.q) + tok0 * ts + (size_t)hq * DK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int idx = t + NT * j, r = min(idx >> 4, nv - 1), part = (idx & 15) * 8;
        in.k[j] = *reinterpret_cast<const u32x4*>(k + (size_t)r * ts + part);
        in.q[j] = *reinterpret_cast<const u32x4*>(q + (size_t)r * ts + part);
    }
    const size_t gi = (tok0 + min(t & 63, nv - 1)) * p.h_v + h;
    in.g = p.g[gi];
    in.b = p.beta[gi];
}

// ----------------------------------------------------------------------------
// T = (I + A)^-1, P and gamma of one (chunk, value head), fp32.
__global__ __launch_bounds__(NT) void k_bwd_prep(BwdParams p) {
    __shared__ __attribute__((aligned(16))) bf16 kb[CH][LKB], qb[CH][LKB];
    __shared__ __attribute__((aligned(16))) float am[CH][LM], tm[CH][LM];
    __shared__ float gam[CH], bet[CH];
    GDN_LDS_POISON_ALL(kb, qb, am, tm, gam, bet);
    // P takes Q's tile once Q K^T is formed (same size: 64 x 136 bf16 = 64 x 68 fp32)
    float (*pmat)[LM] = reinterpret_cast<float (*)[LM]>(&qb[0][0]);
    static_assert(sizeof(qb) == CH * LM * sizeof(float), "P reuses the Q tile");
    // persistent: workgroup b takes items b, b + grid, ... (two per CU)
    const long long n_items = (long long)p.n_chunks * p.h_v;
    long long item = blockIdx.x;
    if (item >= n_items) return;
    PrepIn in;
    prep_fetch(p, item, in);
    for (; item < n_items; item += gridDim.x) {
        // the thread index through an opaque move: the LDS offsets derived from it
        // are formed in each item where they are used, not held through the loop
        int t;
        asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
        int f, h, nv;
        size_t tok0;
        prep_item(p, item, f, h, tok0, nv);
        float* out = p.tpg + ((size_t)f * p.h_v + h) * kBwdTpg;
        __syncthreads();   // the previous item's last LDS reads are done
#pragma unroll
        for (int j = 0; j < 4; ++j) {   // K and Q rows (rows past nv zero)
            const int idx = t + NT * j, r = idx >> 4, part = (idx & 15) * 8;
            *reinterpret_cast<u32x4*>(&kb[r][part]) = r < nv ? in.k[j] : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(&qb[r][part]) = r < nv ? in.q[j] : u32x4{0u, 0u, 0u, 0u};
        }
        if (t < CH) {   // wave 0: inclusive scan of g over the chunk
            float x = t < nv ? in.g : 0.f;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const float y = __shfl_up(x, d, 64);
                if (t >= d) x += y;
            }
            gam[t] = x;
            bet[t] = t < nv ? in.b : 0.f;
            out[CH * CH + t] = x;
        }
        // the next item's inputs, in flight through this one (after the last item,
        // this one's again: every path issues the loads)
        prep_fetch(p, item + gridDim.x < n_items ? item + gridDim.x : item, in);
        __syncthreads();
        {   // K K^T and Q K^T on the ten lower 16x16 tiles (16x16x32 MFMA; lane 16 g + c:
            // A row c and B column c with the k values 8 g .. of each 32-wide step; C rows
            // 4 g .. 4 g + 3 of column c); wave w takes tiles w, w + 4, w + 8
            const int w = t >> 6, lane = t & 63, c = lane & 15, g = lane >> 4;
            f32x4 kk[3], qk[3];
            int tri[3], tii[3];
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const int job = w + 4 * j;
                tri[j] = job >= 6 ? 3 : job >= 3 ? 2 : job >= 1 ? 1 : 0;
                tii[j] = job - tri[j] * (tri[j] + 1) / 2;
                kk[j] = qk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (job >= 10) continue;
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const bf16x8 ak = *reinterpret_cast<const bf16x8*>(&kb[16 * tri[j] + c][32 * s4 + 8 * g]);
                    const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&qb[16 * tri[j] + c][32 * s4 + 8 * g]);
                    const bf16x8 bk = *reinterpret_cast<const bf16x8*>(&kb[16 * tii[j] + c][32 * s4 + 8 * g]);
                    kk[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ak, bk, kk[j], 0, 0, 0);
                    qk[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq, bk, qk[j], 0, 0, 0);
                }
            }
            __syncthreads();   // every read of Q is done before P overwrites its tile
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                if (w + 4 * j >= 10) continue;
                const int i = 16 * tii[j] + c;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * tri[j] + 4 * g + e;
                    const float ex = i <= r ? __expf(gam[r] - gam[i]) : 0.f;
                    am[r][i] = i < r ? bet[r] * ex * kk[j][e] : 0.f;
                    pmat[r][i] = i <= r ? ex * qk[j][e] : 0.f;
                }
            }
        }
        __syncthreads();
        // T = (I + A)^-1 by 16x16 blocks: the diagonal blocks by substitution (wave w,
        // block w, lane c < 16 holds column c in registers), then the blocks below
        // the diagonal one anti-diagonal at a time:
        //   X = sum_{k in blocks j .. i-1} A_ik T_kj (kept in the unused upper block
        //   (j, i) of A), T_ij = -T_ii X.
        {
            const int w = t >> 6, c = t & 63;
            if (c < 16) {
                float tr[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    float s0 = (i == c) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
                    for (int j = 0; j < i; ++j) {
                        if (j & 1) s1 -= am[16 * w + i][16 * w + j] * tr[j];
                        else s0 -= am[16 * w + i][16 * w + j] * tr[j];
                    }
                    tr[i] = i >= c ? s0 + s1 : 0.f;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) tm[16 * w + i][16 * w + c] = tr[i];
            }
        }
        __syncthreads();
        {   // (fully unrolled, four partial sums each: the LDS reads issue together)
            const int a = t >> 4, bb = t & 15;
#pragma unroll
            for (int d = 1; d < 4; ++d) {
#pragma unroll
                for (int j = 0; j + d < 4; ++j) {
                    const int i = j + d;
                    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 16 * j; k < 16 * i; k += 4) {
                        const f32x4 av = *reinterpret_cast<const f32x4*>(&am[16 * i + a][k]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] += av[e] * tm[k + e][16 * j + bb];
                    }
                    am[16 * j + a][16 * i + bb] = (x[0] + x[1]) + (x[2] + x[3]);
                }
                __syncthreads();
#pragma unroll
                for (int j = 0; j + d < 4; ++j) {
                    const int i = j + d;
                    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < 16; m += 4) {
                        const f32x4 tv4 = *reinterpret_cast<const f32x4*>(&tm[16 * i + a][16 * i + m]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) x[e] += tv4[e] * am[16 * j + m + e][16 * i + bb];
                    }
                    tm[16 * i + a][16 * j + bb] = -((x[0] + x[1]) + (x[2] + x[3]));
                }
                __syncthreads();
            }
        }
        // fp32 P (zero above the diagonal; T goes out only as the images below)
        auto tv = [&](int r, int col) { return (col >> 4) > (r >> 4) ? 0.f : tm[r][col]; };
        auto pv = [&](int r, int col) { return col > r ? 0.f : pmat[r][col]; };
        for (int idx = t; idx < CH * CH; idx += NT) {
            out[idx] = pv(idx >> 6, idx & 63);
        }
        // T^T, scale P^T and T as hi/lo bf16 rows with the contraction token in kp order
        // (four consecutive tokens stay consecutive in kp order: one 8-byte store each)
        bf16* img = static_cast<bf16*>(p.tpt) + ((size_t)f * p.h_v + h) * kBwdTpt;
        for (int idx = t; idx < CH * CH / 4; idx += NT) {
            const int r = idx >> 4, m4 = (idx & 15) * 4, o = r * CH + kp(m4);
            bf16 th[4], tl[4], ph[4], pl[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                split1(tv(m4 + e, r), th[e], tl[e]);
                split1(p.scale * pv(m4 + e, r), ph[e], pl[e]);
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
            // T itself: row r, tokens m in kp order
#pragma unroll
            for (int e = 0; e < 4; ++e) split1(tv(r, m4 + e), th[e], tl[e]);
            *reinterpret_cast<u32x2*>(img + 4 * CH * CH + o) = pack(th);
            *reinterpret_cast<u32x2*>(img + 5 * CH * CH + o) = pack(tl);
        }
    }
}

// ----------------------------------------------------------------------------
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
        a += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.dq_part + o));   // (read once)
        b += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.dk_part + o));
    }
    const size_t oo = ((size_t)tok * p.h_qk + hq) * DK + col;
    if (p.out_f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.dq) + oo) = a;
        *reinterpret_cast<f32x4*>(static_cast<float*>(p.dk) + oo) = b;
        return;
    }
    *reinterpret_cast<u32x2*>(static_cast<bf16*>(p.dq) + oo) = u32x2{pack_rne(a[0], a[1]), pack_rne(a[2], a[3])};
    *reinterpret_cast<u32x2*>(static_cast<bf16*>(p.dk) + oo) = u32x2{pack_rne(b[0], b[1]), pack_rne(b[2], b[3])};
}

// dv = diag(beta) Z in fp32 (for fp32 inputs; the bf16 dv is written by the
// state-gradient scan as it forms Z). One workgroup per (chunk, value head).
__global__ __launch_bounds__(NT) void k_bwd_dv32(BwdParams p) {
    const int f = blockIdx.x, h = blockIdx.y;
    int seq, c, len;
    size_t tok_s;
    if (!bwd_locate(p, f, seq, c, len, tok_s)) return;
    const size_t tok0 = tok_s + (size_t)c * CH;
    const int nv = min(CH, len - c * CH);
    const float* z = p.z + ((size_t)f * p.h_v + h) * CH * DK;
    float* dv = static_cast<float*>(p.dv) + tok0 * p.h_v * DK + (size_t)h * DK;
    for (int idx = threadIdx.x; idx < CH * DK / 4; idx += NT) {
        const int r = idx / (DK / 4), col = (idx % (DK / 4)) * 4;
        if (r >= nv) break;
        const float b = p.beta[(tok0 + r) * p.h_v + h];
        *reinterpret_cast<f32x4*>(dv + (size_t)r * p.h_v * DK + col) =
            b * *reinterpret_cast<const f32x4*>(z + r * DK + col);
    }
}

// fp32 -> bf16 with round-to-nearest-even, four elements per thread.
__global__ __launch_bounds__(NT) void k_round_bf16(const float* x, bf16* y, long long n4) {
    const long long i = (long long)blockIdx.x * NT + threadIdx.x;
    if (i >= n4) return;
    const f32x4 a = *reinterpret_cast<const f32x4*>(x + 4 * i);
    *reinterpret_cast<u32x2*>(y + 4 * i) = u32x2{pack_rne(a[0], a[1]), pack_rne(a[2], a[3])};
}

}  // namespace

static int launched() { return (int)hipGetLastError(); }

int launch_bwd(const BwdParams& p, void* stream) {
    const hipStream_t s = (hipStream_t)stream;
    int e;
    if (p.n_chunks > 0) {
        // two workgroups per CU (their LDS), persistent over the items
        int dev = 0, n_cu = 0;
        hipError_t he = hipGetDevice(&dev);
        if (he == hipSuccess) he = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (he != hipSuccess) return (int)he;
        const long long items = (long long)p.n_chunks * p.h_v;
        const unsigned grid = (unsigned)std::min<long long>(items, 2LL * std::max(n_cu, 1));
        hipLaunchKernelGGL(k_bwd_prep, dim3(grid), dim3(NT), 0, s, p);
        if ((e = launched())) return e;
    }
    if ((e = launch_bwd_chain_mma(p, stream))) return e;
    if (p.n_chunks > 0 && p.out_f32) {
        hipLaunchKernelGGL(k_bwd_dv32, dim3(p.n_chunks, p.h_v), dim3(NT), 0, s, p);
        if ((e = launched())) return e;
    }
    if (p.n_chunks > 0) {
        if ((e = launch_bwd_chunk_mma(p, stream))) return e;
    }
    return 0;
}

int launch_round_bf16(const float* x, void* y, long long n, void* stream) {
    if (n <= 0) return 0;
    const long long n4 = n / 4;
    hipLaunchKernelGGL(k_round_bf16, dim3((unsigned)((n4 + NT - 1) / NT)), dim3(NT), 0, (hipStream_t)stream, x,
                       static_cast<bf16*>(y), n4);
    return launched();
}

int launch_bwd_sum(const BwdParams& p, long long n_tokens, void* stream) {
    if (n_tokens <= 0) return 0;
    const long long n = n_tokens * p.h_qk * DK / 4;
    hipLaunchKernelGGL(k_bwd_sum, dim3((unsigned)((n + NT - 1) / NT)), dim3(NT), 0, (hipStream_t)stream, p,
                       n_tokens);
    return launched();
}

}  // namespace gdn
