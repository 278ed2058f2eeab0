// The forward's chain kernels on fp16 matrix-core operands (gfx950).
//
// What is computed: the chunked WY form of the gated delta rule (FlashQLA
// pages, "FlashQLA: CP-/Bwd-friendly fused linear attention kernels for GDN",
// section on optimising GDN chunked prefill), per chunk of 64 tokens with
// incoming state S (d_k x d_v, fp32):
//   Y  = V - diag(e^gamma) K S                  (prediction error)
//   V' = T diag(beta) Y                         (= U - W S; T = (I + A)^-1 from k_prep)
//   O  = scale (diag(e^gamma) Q S + (Q K^T o D) V'),  D[r][i] = e^(gamma_r - gamma_i), i <= r
//   S <- e^gamma_C S + K^T diag(e^(gamma_C - gamma)) V'
// and the intra-card context parallelism of the AutoCP section: segment
// boundary states from a warm-up scan (gates decayed below the noise floor)
// or from the exact segment maps S -> M S + H chained by k_combine16.
//
// Precision. Every product runs on 16x16x32 fp16 MFMAs with fp32
// accumulation: the bf16 inputs q, k, v are exact in fp16 (within its
// range), and the derived operands (S, Y, V', T diag(beta), P) are rounded
// once to fp16 (11-bit significand, 8x finer than bf16); gate factors are
// applied to fp32 accumulators. The state itself stays fp32.
//
// Work layouts. The bf16 forward runs the warp-specialised kernel k_fwd_ws
// (state waves beside staging waves; described at its definition). The CP
// preprocessing (k_cp_prep16) and the fp32 forward (k_fwd16<float>) use the
// symmetric layout: a workgroup is 8 waves, two per SIMD; wave w owns the d_v
// columns [16 w, 16 w + 16): its 128 x 16 slice of S (eight accumulator
// tiles), of Y, V' and of the output stay in its registers, and the state
// chain never crosses waves. Each wave issues a VALU instruction only every
// ~7 cycles (measured), so two waves per SIMD are what keep its VALU and
// matrix pipes busy; the LDS, which serves > 300 bytes per cycle per CU to
// 16-byte reads (measured; writes about 75), absorbs every wave reading the
// whole chunk operands. A chunk's
// K, K^T and Q (converted to fp16), its V rows (as they are) and T diag(beta)
// (from k_prep, already in operand layout) are staged in LDS by all 512
// threads; the next chunk's inputs are loaded into registers a chunk and a
// half ahead. The causal matrix P = scale (Q K^T) o D is formed once per
// chunk, each wave computing two of its 16 tiles, through LDS.
//
// Register layouts (16x16x32 MFMA, lane l = 16 g + c): A row c, B column c,
// each with the k slots 8 g .. 8 g + 7; C/D rows 4 g .. 4 g + 3 of column c.
// Two C tiles stacked along the contraction axis give lane group g the rows
// 4 g + e and 16 + 4 g + e: the k slots of an operand once the contraction
// axis of every LDS operand is stored in the order kp (gdn_device.h). V
// reaches the accumulator layout through an identity product on the matrix
// cores. The output is formed transposed (O^T = S^T Q^T + V'^T P^T, the same
// registers in swapped operand roles), so that a lane holds four consecutive
// d_v of one token and writes them with one 8-byte store.
#include "gdn_device.h"

namespace gdn {
namespace {

constexpr int NW8 = 8;           // waves per chain workgroup
constexpr int NT8 = 64 * NW8;
constexpr int LQ = 144;          // K, Q rows (fp16): 288 bytes, conflict-free operand reads
constexpr int LT = 80;           // K^T rows: 160 bytes
constexpr int LP = 80;           // P rows
constexpr int LV = 136;          // V rows (elements of the input type): 272 / 544 bytes
constexpr int LMI = 144;         // rows of the map image staged for the combine
constexpr float kLog2e = 1.4426950408889634f;

// The six nonzero T diag(beta) fragments (token tile m, k step j): 0 (0,0),
// 1 (1,0), 2 (2,0), 3 (2,1), 4 (3,0), 5 (3,1) -- the same (m, j) pairs as
// the causal P V' product.
__device__ __forceinline__ int tb_frag(int m, int j) { return m < 2 ? m : 2 + 2 * (m - 2) + j; }

// LDS of the chain kernels. OUT: the forward (Q and P as well). K, Q, V and
// T diag(beta) are read in the first half of a chunk step only and restaged
// after the step's first barrier; K^T is read in the second half, so it has
// two buffers (the next chunk's is written while this one's is read).
template <typename IO, bool OUT>
struct __attribute__((aligned(16))) Smem16 {
    f16 k[CH * LQ];                       // K token-major, d_k in kp order
    f16 kt[2][DK * LT];                   // K^T: row d_k, tokens in kp order, 16-byte pieces XOR tswz(row)
    f16 q[OUT ? CH * LQ : 8];             // Q token-major, d_k in kp order
    IO v[CH * LV];                        // V rows as given
    f16 tb[kTbHalfs];                     // T diag(beta) fragments (k_prep's image)
    f16 p[OUT ? CH * LP : 8];             // P: row r, columns i in kp order
    float gam[2][CH];                     // gamma log2(e)
    float eg[2][CH];                      // e^gamma
    float egc[2][CH];                     // e^(gamma_C - gamma)
    float ec[2][4];                       // e^gamma_C
};

// One chunk's inputs in registers between the loads and the LDS stores:
// thread t holds tokens 4 (t / 32) + j (j < 4), columns 4 (t % 32) .. + 4 of
// K, Q and V; piece t of the T diag(beta) image (t < 384); the gate of token
// `lane`.
template <typename IO> struct In16;
template <> struct In16<bf16> { u32x2 k[4], q[4], v[4]; u32x4 tb; float g; };
template <> struct In16<float> { f32x4 k[4], q[4], v[4]; u32x4 tb; float g; };

// Buffer descriptors (raw, 32-bit offsets; word 3 selects 32-bit data on
// gfx9-family chips). Each chunk gets descriptors whose base is its first row
// and whose range ends at its last valid row: loads past a sequence's end
// then return zeros and stores there are dropped by the range check, so the
// per-lane offsets never change across chunks and no row is clamped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Per-lane byte offsets of a chain workgroup's loads and stores, the same for
// every chunk (thread t: tokens 4 (t / 32) + j, columns 4 (t % 32) .. + 4).
struct Lanes {
    unsigned kq[4];   // K, Q rows
    unsigned v[4];    // V rows
    unsigned g;       // gate of token `lane`
    unsigned o[4];    // output: token 16 m + c, d_v 16 w + 4 g
};

template <typename IO>
__device__ Lanes make_lanes(const Params& p) {
    Lanes L;
    const int t = threadIdx.x, lane = lane_id(), c = lane & 15, g = lane >> 4, w = wave_id();
    const unsigned es = sizeof(IO), ts = (unsigned)p.h_qk * DK, tsv = (unsigned)p.h_v * DK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const unsigned row = 4 * (t >> 5) + j;
        L.kq[j] = (row * ts + 4 * (t & 31)) * es;
        L.v[j] = (row * tsv + 4 * (t & 31)) * es;
        L.o[j] = ((16 * j + c) * tsv + 16 * w + 4 * g) * es;
    }
    L.g = (unsigned)lane * p.h_v * 4;
    return L;
}

// Loads one chunk's inputs: the gate first (wave 0's scan waits for it),
// then K, Q, V, T diag(beta).
template <typename IO, bool WANT_Q, bool WANT_V>
__device__ __forceinline__ void fetch16(In16<IO>& r, const Params& p, const Lanes& L, size_t tok0, int nvalid,
                                        int h, int hq, int slot) {
    const int t = threadIdx.x;
    const unsigned es = sizeof(IO), nv = (unsigned)nvalid;
    const size_t ts = (size_t)p.h_qk * DK, tsv = (size_t)p.h_v * DK;
    r.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                        rsrc(p.g + tok0 * p.h_v + h, nv * p.h_v * 4), (int)L.g, 0, 0));
    const auto rk = rsrc(static_cast<const IO*>(p.k) + tok0 * ts + (size_t)hq * DK, nv * (unsigned)ts * es);
    const auto rq = rsrc(static_cast<const IO*>(p.q) + tok0 * ts + (size_t)hq * DK, nv * (unsigned)ts * es);
    const auto rv = rsrc(static_cast<const IO*>(p.v) + tok0 * tsv + (size_t)h * DK, nv * (unsigned)tsv * es);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (Io<IO>::kExact) {
            r.k[j] = __builtin_amdgcn_raw_buffer_load_b64(rk, (int)L.kq[j], 0, 0);
            if (WANT_Q) r.q[j] = __builtin_amdgcn_raw_buffer_load_b64(rq, (int)L.kq[j], 0, 0);
            if (WANT_V) r.v[j] = __builtin_amdgcn_raw_buffer_load_b64(rv, (int)L.v[j], 0, 0);
        } else {
            r.k[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)L.kq[j], 0, 0));
            if (WANT_Q) r.q[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)L.kq[j], 0, 0));
            if (WANT_V) r.v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)L.v[j], 0, 0));
        }
    }
    // (threads past the 384 pieces load piece t - 384 again; only t < 384 store)
    const u32x4* tb = reinterpret_cast<const u32x4*>(static_cast<const f16*>(p.tb16) +
                                                     ((size_t)slot * p.h_v + h) * (size_t)kTbHalfs);
    r.tb = tb[t < kTbHalfs / 8 ? t : t - kTbHalfs / 8];
}

__device__ __forceinline__ f16x4 to_h4(const f32x4& x) { return __builtin_convertvector(x, f16x4); }

// Writes a fetched chunk to LDS (K^T into buffer b): K token-major and
// transposed, Q, V, T diag(beta), and (wave 0) the gate factors. Thread t's
// columns 4 (t % 32) .. + 4 are the kp positions pk .. pk + 3; its four tokens
// 4 (t / 32) .. + 4 the kp positions pt .. pt + 3.
template <typename IO, bool OUT, bool WANT_V>
__device__ __forceinline__ void stage16(Smem16<IO, OUT>& sm, const In16<IO>& r, int b) {
    const int t = threadIdx.x, lane = lane_id(), cq = t & 31, rq = t >> 5;
    if (wave_id() == 0) {
        const float gam = wave_scan(r.g);
        const float gc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gam), 63));
        sm.gam[b][lane] = gam * kLog2e;   // (P's decay factors are formed as powers of two)
        sm.eg[b][lane] = __expf(gam);
        sm.egc[b][lane] = __expf(gc - gam);
        if (lane == 0) sm.ec[b][0] = __expf(gc);
    }
    const int pk = 32 * (cq >> 3) + 8 * (cq & 3) + 4 * ((cq >> 2) & 1);
    const int pt = 32 * (rq >> 3) + 8 * (rq & 3) + 4 * ((rq >> 2) & 1);
    f16x4 kr[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kr[j] = to_h4(r.k[j]);
        *reinterpret_cast<f16x4*>(sm.k + (4 * rq + j) * LQ + pk) = kr[j];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int d = 4 * cq + e;
        *reinterpret_cast<f16x4*>(sm.kt[b] + d * LT + (pt ^ tswz(d))) = f16x4{kr[0][e], kr[1][e], kr[2][e], kr[3][e]};
    }
    if constexpr (OUT) {
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<f16x4*>(sm.q + (4 * rq + j) * LQ + pk) = to_h4(r.q[j]);
    }
    if constexpr (WANT_V) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (Io<IO>::kExact) *reinterpret_cast<u32x2*>(sm.v + (4 * rq + j) * LV + 4 * cq) = r.v[j];
            else *reinterpret_cast<f32x4*>(sm.v + (4 * rq + j) * LV + 4 * cq) = r.v[j];
        }
    }
    if (t < kTbHalfs / 8) *reinterpret_cast<u32x4*>(sm.tb + 8 * t) = r.tb;
}

// ----------------------------------------------------------------------------
// State tiles: wave w, tile i: rows 16 i + 4 g + e, column 16 w + c. In HBM the
// segment states and H maps use the "tile order" of these registers: 128 x 128
// fp32 as [i][u = 16-column tile][lane][4] (a 16-byte load or store per tile
// and lane); the caller's initial and final states are row-major [128][128].

__device__ __forceinline__ size_t tiles_off(int idx, int h_v, int h) {
    return ((size_t)idx * h_v + h) * (size_t)DK * DK;
}

__device__ void load_rm(const float* Sg, f32x4 S[8]) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, w = wave_id();
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[i][e] = Sg[(16 * i + 4 * g + e) * DK + 16 * w + c];
}
__device__ void store_rm(float* Sg, const f32x4 S[8]) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, w = wave_id();
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) Sg[(16 * i + 4 * g + e) * DK + 16 * w + c] = S[i][e];
}
__device__ void load_tiles(const float* Sg, f32x4 S[8]) {
    const int lane = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < 8; ++i) S[i] = *reinterpret_cast<const f32x4*>(Sg + ((i * 8 + w) * 64 + lane) * 4);
}
__device__ void store_tiles(float* Sg, const f32x4 S[8]) {
    const int lane = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<f32x4*>(Sg + ((i * 8 + w) * 64 + lane) * 4) = S[i];
}
__device__ void set_state(f32x4 S[8], bool identity) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, w = wave_id();
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[i][e] = (identity && 16 * i + 4 * g + e == 16 * w + c) ? 1.f : 0.f;
}

// ----------------------------------------------------------------------------
// One chunk step of the chain. OUT: the forward (output rows written to
// orow + r * ts_v, rows past nvalid to the scratch line); else the scan
// without output: the warm-up and H chains (WANT_V) or the M chain (V = 0).
// The chunk is in LDS (K^T in buffer b); `nxt`, the next chunk's inputs, is
// staged after the first barrier.
template <typename IO, bool OUT, bool WANT_V, int b>
__device__ __forceinline__ void chain_step16(Smem16<IO, OUT>& sm, const In16<IO>& nxt, f32x4 S[8], float scale,
                                             float log2_scale, const Lanes& L, __amdgpu_buffer_rsrc_t ro) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, w = wave_id();
    // the state as fp16 operands, one per k step j
    f16x8 Sb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) Sb[j] = pack8h(S[2 * j], S[2 * j + 1]);

    // K S, Q S (transposed) and this wave's two tiles of P, k step by k step:
    // tiles (r block w / 2, i blocks ib0, ib0 + 1), ib0 = 2 (w % 2)
    const int rb = w >> 1, ib0 = 2 * (w & 1);
    f32x4 Y[4], O[4], Pt[2];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        Y[m] = f32x4{0.f, 0.f, 0.f, 0.f};
        O[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    Pt[0] = Pt[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f16x8 kf[4], qf[4], qw, kw0, kw1;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            kf[m] = *reinterpret_cast<const f16x8*>(sm.k + (16 * m + c) * LQ + 32 * j + 8 * g);
            if constexpr (OUT) qf[m] = *reinterpret_cast<const f16x8*>(sm.q + (16 * m + c) * LQ + 32 * j + 8 * g);
        }
        if constexpr (OUT) {
            // (the P operands at wave-dependent rows, read again rather than picked by a branch)
            qw = *reinterpret_cast<const f16x8*>(sm.q + (16 * rb + c) * LQ + 32 * j + 8 * g);
            kw0 = *reinterpret_cast<const f16x8*>(sm.k + (16 * ib0 + c) * LQ + 32 * j + 8 * g);
            kw1 = *reinterpret_cast<const f16x8*>(sm.k + (16 * ib0 + 16 + c) * LQ + 32 * j + 8 * g);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) Y[m] = mmh(kf[m], Sb[j], Y[m]);
        if constexpr (OUT) {
#pragma unroll
            for (int m = 0; m < 4; ++m) O[m] = mmh(Sb[j], qf[m], O[m]);
            Pt[0] = mmh(kw0, qw, Pt[0]);
            Pt[1] = mmh(kw1, qw, Pt[1]);
        }
    }
    if constexpr (OUT) {
        // P[r][i] = scale e^(gamma_r - gamma_i) (q_r . k_i), i <= r, else 0; the
        // tiles hold P^T: lane (g, c) has r = 16 rb + c and i = 16 ib + 4 g + e
        // (gamma is kept times log2(e): the factor is 2^(gr - gi), the scale folded in)
        const int r = 16 * rb + c;
        const float gr = sm.gam[b][r] + log2_scale;
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2) {
            const int ib = ib0 + e2, i0 = 16 * ib + 4 * g;
            const f32x4 gi = *reinterpret_cast<const f32x4*>(sm.gam[b] + i0);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (i0 + e <= r) ? __builtin_amdgcn_exp2f(gr - gi[e]) * Pt[e2][e] : 0.f;
            *reinterpret_cast<f16x4*>(sm.p + r * LP + 32 * (ib >> 1) + 8 * g + 4 * (ib & 1)) =
                __builtin_convertvector(v, f16x4);
        }
    }
    // Y = V - e^gamma (K S) on rows 16 m + 4 g + e; V enters through the
    // identity product V[:, 16 w + (0..15)] = V_rows E (32 columns of V as the
    // A operand, E selecting this wave's 16)
#pragma unroll
    for (int m = 0; m < 4; ++m) Y[m] *= -*reinterpret_cast<const f32x4*>(sm.eg[b] + 16 * m + 4 * g);
    if constexpr (WANT_V) {
        const int vc = 32 * (w >> 1) + 8 * g;
        if constexpr (Io<IO>::kExact) {
            bf16x8 E;
#pragma unroll
            for (int s = 0; s < 8; ++s) E[s] = (bf16)((8 * g + s == 16 * (w & 1) + c) ? 1.f : 0.f);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                Y[m] = mma16k32(*reinterpret_cast<const bf16x8*>(sm.v + (16 * m + c) * LV + vc), E, Y[m]);
        } else {
            f16x8 E;
#pragma unroll
            for (int s = 0; s < 8; ++s) E[s] = (f16)((8 * g + s == 16 * (w & 1) + c) ? 1.f : 0.f);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                // fp32 rows as hi + lo fp16 (exact to about 2^-22)
                const f32x4 a0 = *reinterpret_cast<const f32x4*>(sm.v + (16 * m + c) * LV + vc);
                const f32x4 a1 = *reinterpret_cast<const f32x4*>(sm.v + (16 * m + c) * LV + vc + 4);
                const f16x8 hi = pack8h(a0, a1);
                f32x4 l0, l1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    l0[e] = a0[e] - (float)hi[e];
                    l1[e] = a1[e] - (float)hi[4 + e];
                }
                Y[m] = mmh(hi, E, Y[m]);
                Y[m] = mmh(pack8h(l0, l1), E, Y[m]);
            }
        }
    }
    // V' = (T diag(beta)) Y; T diag(beta) is lower triangular
    f32x4 Vp[4];
    {
        const f16x8 Yb0 = pack8h(Y[0], Y[1]), Yb1 = pack8h(Y[2], Y[3]);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f16x8 t0 = *reinterpret_cast<const f16x8*>(sm.tb + (tb_frag(m, 0) * 64 + lane) * 8);
            Vp[m] = mmh(t0, Yb0, f32x4{0.f, 0.f, 0.f, 0.f});
            if (m >= 2) {
                const f16x8 t1 = *reinterpret_cast<const f16x8*>(sm.tb + (tb_frag(m, 1) * 64 + lane) * 8);
                Vp[m] = mmh(t1, Yb1, Vp[m]);
            }
        }
    }
    if constexpr (OUT) {
#pragma unroll
        for (int m = 0; m < 4; ++m) O[m] *= scale * sm.eg[b][16 * m + c];
    }
    __syncthreads();   // P complete; K, Q, V, T diag(beta) and K^T[b ^ 1] free for the next chunk
    f16x8 Vb[2];
    Vb[0] = pack8h(Vp[0], Vp[1]);
    Vb[1] = pack8h(Vp[2], Vp[3]);
    if constexpr (OUT) {
        // O^T += V'^T P^T (P causal: token tiles 0 and 1 need k step 0 only)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (j == 1 && m < 2) continue;
                const f16x8 pf = *reinterpret_cast<const f16x8*>(sm.p + (16 * m + c) * LP + 32 * j + 8 * g);
                O[m] = mmh(Vb[j], pf, O[m]);
            }
        // lane (g, c) of tile m: token 16 m + c, d_v 16 w + 4 g + (0..3) (rows
        // past the sequence's end fall outside the descriptor's range: dropped)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if constexpr (Io<IO>::kExact)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_rne(O[m][0], O[m][1]), pack_rne(O[m][2], O[m][3])}, ro,
                                                      (int)L.o[m], 0, 0);
            else
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, O[m]), ro, (int)L.o[m], 0, 0);
        }
    }
    stage16<IO, OUT, WANT_V>(sm, nxt, b ^ 1);
    // S <- e^gamma_C S + K^T diag(e^(gamma_C - gamma)) V'
#pragma unroll
    for (int m = 0; m < 4; ++m) Vp[m] *= *reinterpret_cast<const f32x4*>(sm.egc[b] + 16 * m + 4 * g);
    Vb[0] = pack8h(Vp[0], Vp[1]);
    Vb[1] = pack8h(Vp[2], Vp[3]);
    const float ec = sm.ec[b][0];
#pragma unroll
    for (int i = 0; i < 8; ++i) S[i] *= ec;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        f16x8 ktf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            ktf[i] = *reinterpret_cast<const f16x8*>(sm.kt[b] + (16 * i + c) * LT + ((32 * j + 8 * g) ^ tswz(16 * i)));
#pragma unroll
        for (int i = 0; i < 8; ++i) S[i] = mmh(ktf[i], Vb[j], S[i]);
    }
    __syncthreads();   // the next chunk staged
}

// Runs chunks [c_lo, c_hi) of sequence loc from the state S: the forward of a
// segment (OUT) or a scan without output. Two register sets of chunk inputs
// alternate (the loop is unrolled by two, with no branch in its body, so
// every iteration issues the same memory operations and the compiler's waits
// on them stay exact): step c stages the set holding chunk c + 1, and that
// set is then refilled with chunk c + 3, a chunk and a half ahead of its use.
template <typename IO, bool OUT, bool WANT_V>
__device__ void run_chunks16(Smem16<IO, OUT>& sm, const Params& p, const SegLoc& loc, int h, int c_lo, int c_hi,
                             f32x4 S[8]) {
    if (c_lo >= c_hi) return;
    const int hq = h / p.group;
    const size_t ts_v = (size_t)p.h_v * DK;
    const Lanes L = make_lanes<IO>(p);
    const float log2_scale = __log2f(p.scale);
    In16<IO> A, B;
    auto fetch = [&](In16<IO>& r, int c) {
        c = min(c, c_hi - 1);
        fetch16<IO, OUT, WANT_V>(r, p, L, loc.tok0 + (size_t)c * CH, min(CH, loc.len - c * CH), h, hq,
                                 loc.chunk_base + c);
    };
    auto orsrc = [&](int c) {
        return rsrc(OUT ? static_cast<IO*>(p.out) + (loc.tok0 + (size_t)c * CH) * ts_v + (size_t)h * DK : nullptr,
                    OUT ? (unsigned)min(CH, loc.len - c * CH) * (unsigned)(ts_v * sizeof(IO)) : 0u);
    };
    fetch(A, c_lo);
    stage16<IO, OUT, WANT_V>(sm, A, 0);
    fetch(B, c_lo + 1);
    fetch(A, c_lo + 2);
    __syncthreads();
    int c = c_lo;
    for (; c + 1 < c_hi; c += 2) {
        chain_step16<IO, OUT, WANT_V, 0>(sm, B, S, p.scale, log2_scale, L, orsrc(c));
        fetch(B, c + 3);
        chain_step16<IO, OUT, WANT_V, 1>(sm, A, S, p.scale, log2_scale, L, orsrc(c + 1));
        fetch(A, c + 4);
    }
    if (c < c_hi) chain_step16<IO, OUT, WANT_V, 0>(sm, B, S, p.scale, log2_scale, L, orsrc(c));
}

// ----------------------------------------------------------------------------
// CP preprocessing: one 8-wave workgroup per (boundary, part). For an exact
// boundary s (between segments s - 1 and s): part 0 runs segment s - 1 from
// zero (H_{s-1}, tile order), part 1 from the identity with V = 0 (M_{s-1},
// written as the combine's fp16 A-operand image); M_0 only matters with a
// nonzero initial state. A warm-up boundary (part 0 only) scans its window
// from zero (or from the initial state where the window starts at the
// sequence start) and writes the boundary state. Work order as planned
// (exact boundaries first, or head-major).

// Class of boundary pair q = slot h_v + head: -1 (a sequence's first
// segment), 0 exact, 1 or 2 warm-up (window length in bits 8 and up).
__device__ __forceinline__ int pair_class16(const Params& p, int q, int& wq) {
    const SegLoc loc = locate_segment(p, q / p.h_v);
    const int v = p.warm[q];
    wq = v >> 8;
    return (loc.seq < 0 || loc.s == 0) ? -1 : (v & 255);
}

// Block-wide exclusive prefix sum (NW waves).
template <int NW>
__device__ __forceinline__ int block_excl_scan(int x, int* red, int& total) {
    const int lane = lane_id(), w = threadIdx.x >> 6;
    int v = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(v, d, 64);
        if (lane >= d) v += y;
    }
    if (lane == 63) red[w] = v;
    __syncthreads();
    int off = 0;
    total = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        const int r = red[i];
        if (i < w) off += r;
        total += r;
    }
    return off + v - x;
}

// The boundary pair (slot h_v + head) that workgroup i of the CP
// preprocessing takes, and its part; -1: none (uniform over the workgroup).
// An exact boundary takes PX workgroups (parts 0 .. PX - 1), a warm-up one
// part 0 of one. Order as planned: exact boundaries first, then the warm-up
// ones, each in pair order; or head-major (PX workgroups per pair). With
// PX = 2 the two parts of a pair are workgroups 8 apart (pair index
// (i % 8) + 8 (i / 16), part (i / 8) % 2): the XCDs are dealt workgroups
// round-robin, so both run on one XCD and share its L2 for the chunks they
// both stage; the exact region is padded to whole groups of 16, and the grid
// has 16 ceil(pairs / 8) + 16 workgroups. red: 2 NW + 4 ints of LDS.
template <int NW, int PX>
__device__ int cp_pick(const Params& p, int i, int* red, int& part) {
    constexpr int NT = 64 * NW;
    static_assert(PX == 1 || PX == 2, "one or two workgroups per pair");
    const int n_pairs = p.n_segments * p.h_v;
    if (!p.cp_order) {
        int pi = i;
        part = 0;
        if (PX == 2) {
            pi = (i & 7) + 8 * (i >> 4);
            part = (i >> 3) & 1;
        }
        if (pi >= n_pairs) return -1;
        return (pi % p.n_segments) * p.h_v + pi / p.n_segments;
    }
    const int per = (n_pairs + NT - 1) / NT, q0 = threadIdx.x * per, q1 = min(q0 + per, n_pairs);
    int n_ex = 0, n_wu = 0;
    for (int q = q0; q < q1; ++q) {
        int wq;
        const int c = pair_class16(p, q, wq);
        n_ex += c == 0;
        n_wu += c > 0;
    }
    if (threadIdx.x == 0) red[2 * NW] = -1;   // (ordered before its use by the scans' barriers)
    int tot_ex, tot_wu;
    const int pre_ex = block_excl_scan<NW>(n_ex, red, tot_ex);
    const int pre_wu = block_excl_scan<NW>(n_wu, red + NW, tot_wu);
    const int ex_wgs = PX == 2 ? 16 * ((tot_ex + 7) / 8) : tot_ex;   // the exact region (padded with PX = 2)
    const bool want_ex = i < ex_wgs;
    const int r = want_ex ? (PX == 2 ? (i & 7) + 8 * (i >> 4) : i) : i - ex_wgs;
    part = want_ex && PX == 2 ? (i >> 3) & 1 : 0;
    if (r >= (want_ex ? tot_ex : tot_wu)) return -1;   // (uniform: every thread has the totals)
    const int pre = want_ex ? pre_ex : pre_wu, cnt = want_ex ? n_ex : n_wu;
    if (r >= pre && r < pre + cnt) {
        int k = pre;
        for (int q = q0; q < q1; ++q) {
            int wq;
            const int c = pair_class16(p, q, wq);
            if (want_ex ? c == 0 : c > 0) {
                if (k == r) {
                    red[2 * NW] = q;
                    break;
                }
                ++k;
            }
        }
    }
    __syncthreads();
    const int q = red[2 * NW];
    return (q < 0 || q >= n_pairs) ? -1 : q;   // (q < 0 cannot happen: the ranks partition the boundaries)
}

// M (tile registers, columns 16 w + c) -> the combine's A-operand image:
// fragment (row tile mt, k step j), lane (g', c') holds row 16 mt + c' at the
// k slots 8 g' .. + 8, the columns of block j in kp order. Staged through LDS
// (row i, columns in kp order), then copied out.
template <typename IO>
__device__ void store_map_image(Smem16<IO, false>& sm, const f32x4 M[8], f16* dst) {
    f16* img = reinterpret_cast<f16*>(&sm);   // 128 rows of LMI fp16 (36 KiB) over the chunk buffers
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, w = wave_id();
    __syncthreads();   // the chain's last LDS reads are done
    // column k = 16 w + c -> kp position 32 (w / 2) + 8 (c / 4) + 4 (w % 2) + c % 4
    const int col = 32 * (w >> 1) + 8 * (c >> 2) + 4 * (w & 1) + (c & 3);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) img[(16 * i + 4 * g + e) * LMI + col] = (f16)M[i][e];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j)   // fragment F = 4 w + j: row tile w, k step j
        *reinterpret_cast<f16x8*>(dst + ((size_t)(4 * w + j) * 64 + lane) * 8) =
            *reinterpret_cast<const f16x8*>(img + (16 * w + c) * LMI + 32 * j + 8 * g);
}

template <typename IO>
__device__ void cp_item16(const Params& p, Smem16<IO, false>& sm, int slot, int part, int h) {
    const SegLoc loc = locate_segment(p, slot);
    int wq;
    const int cls = pair_class16(p, slot * p.h_v + h, wq);
    if (cls < 0) return;
    const int a = loc.s * p.L;   // first chunk of segment s
    if (cls && part == 1) return;
    if (!cls && part == 1 && loc.s == 1 && !p.s_init) return;
    f32x4 S[8];
    if (cls || part == 0) {
        const int c_lo = cls ? a - wq : a - p.L;
        if (cls && c_lo == 0 && p.s_init) load_rm(p.s_init + tiles_off(loc.seq, p.h_v, h), S);
        else set_state(S, false);
        run_chunks16<IO, false, true>(sm, p, loc, h, c_lo, a, S);
        store_tiles(cls ? p.seg_state + tiles_off(loc.seg_base + loc.s, p.h_v, h)
                        : p.seg_H + tiles_off(loc.seg_base + loc.s - 1, p.h_v, h), S);
    } else {
        set_state(S, true);
        run_chunks16<IO, false, false>(sm, p, loc, h, a - p.L, a, S);
        // (the image is 128 x 128 fp16: the same element count as a state block)
        store_map_image<IO>(sm, S, reinterpret_cast<f16*>(p.seg_M) + tiles_off(loc.seg_base + loc.s - 1, p.h_v, h));
    }
}

template <typename IO>
__global__ __launch_bounds__(NT8) void k_cp_prep16(Params p) {
    __shared__ Smem16<IO, false> sm;
    __shared__ int rank_red[2 * NW8 + 4];
    GDN_LDS_POISON_ALL(sm, rank_red);
    int part;
    const int q = cp_pick<NW8, 2>(p, (int)blockIdx.x, rank_red, part);
    if (q < 0) return;
    cp_item16<IO>(p, sm, q / p.h_v, part, q % p.h_v);
}

// ----------------------------------------------------------------------------
// The segment combine: the boundary states S0(s) of the exact boundaries from
// the segment maps, in 4-wave workgroups, each over one 16-column tile of the
// state (the columns evolve independently).
constexpr int NTC = 256;
// Boundary count, first segment slot and boundary flags (LDS, 0 exact) of a
// (sequence, head); false if no boundary is exact (nothing to chain).
__device__ bool comb_setup(const Params& p, int seq, int h, int* flags, int& P, int& seg_base) {
    if (!p.cu) {
        P = n_segs_of(n_chunks_of(p.seq_len), p.L);
        seg_base = seq * P;
    } else {
        seg_base = 0;
        for (int n = 0; n < seq; ++n) seg_base += n_segs_of(n_chunks_of(p.cu[n + 1] - p.cu[n]), p.L);
        P = n_segs_of(n_chunks_of(p.cu[seq + 1] - p.cu[seq]), p.L);
    }
    if (P <= 1 || P > kMaxSegsPerSeq) return false;
    int any_exact = 0;
    for (int s = 1 + (int)threadIdx.x; s < P; s += NTC) {
        const int f = p.warm[(size_t)(seg_base + s) * p.h_v + h] & 255;
        flags[s] = f;
        any_exact |= f == 0;
    }
    return __syncthreads_or(any_exact);
}

// Column tile u of a row-major 128 x 128 state (row tiles 2 r, 2 r + 1 of wave r).
__device__ __forceinline__ void comb_load_rm_tile(const float* S0, int u, f32x4 cur[2]) {
    const int r = wave_id(), lane = lane_id(), c = lane & 15, g = lane >> 4;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) cur[tt][e] = S0[(16 * (2 * r + tt) + 4 * g + e) * DK + 16 * u + c];
}
// The state tile X (row tiles 2 r, 2 r + 1 of column tile u, in registers) as
// this wave's k step of the next product's B operand.
__device__ __forceinline__ void comb_put(f16* xb, const f32x4 cur[2]) {
    *reinterpret_cast<f16x8*>(xb + (wave_id() * 64 + lane_id()) * 8) = pack8h(cur[0], cur[1]);
}
// ... from a block in tile order
__device__ __forceinline__ void comb_load_tile(const float* src, int u, f32x4 cur[2]) {
    const int r = wave_id(), lane = lane_id();
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) cur[tt] = *reinterpret_cast<const f32x4*>(src + (((2 * r + tt) * 8 + u) * 64 + lane) * 4);
}

struct CombOps {
    f32x4 add[2];   // H_{b-1} or the warm-up state, row tiles 2 r, 2 r + 1
    u32x4 m[8];     // M_{b-1} fragments (row tile 2 r + f / 4, k step f % 4)
};

// The chain over boundaries [b_lo, b_hi) of one (sequence, head) for column
// tile u, from X(b_lo - 1), which the caller has put in xb[0]; on return cur
// holds X(b_hi - 1). An exact boundary maps X(b) = M_{b-1} X(b-1) + add (M_0
// only to an initial state), a warm-up one sets X(b) = add. KIND 0: add = H_{b-1}
// or the warm-up state, every X(b) stored as the boundary state; KIND 1 (a
// group's composed map CM): add = 0; KIND 2 (its CH): as KIND 0, nothing stored.
// Wave r owns rows [32 r, 32 r + 32) of the tile -- exactly the k step r of the
// next product's B operand -- and hands its fp16 rows to the others through
// LDS once per step, so a step is eight MFMAs per wave plus one exchange. Each
// step's operands are loaded two steps ahead, and every step issues the same
// memory operations (both cases evaluated and selected).
template <int KIND>
__device__ void comb_chain(const Params& p, const int* flags, f16 (*xb)[4 * 64 * 8], int seg_base, int h, int u,
                           int b_lo, int b_hi, f32x4 cur[2]) {
    const int lane = lane_id(), r = wave_id();
    auto fetch = [&](CombOps& o, int b) {
        b = min(b, b_hi - 1);
        const int f = __builtin_amdgcn_readfirstlane(flags[b]);   // (uniform: a branch-free select)
        const float* src = f ? p.seg_state + tiles_off(seg_base + b, p.h_v, h)
                             : p.seg_H + tiles_off(seg_base + b - 1, p.h_v, h);
        if (KIND != 1) {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                o.add[tt] = *reinterpret_cast<const f32x4*>(src + (((2 * r + tt) * 8 + u) * 64 + lane) * 4);
        }
        const u32x4* mi = reinterpret_cast<const u32x4*>(reinterpret_cast<const f16*>(p.seg_M) +
                                                          tiles_off(seg_base + b - 1, p.h_v, h));
#pragma unroll
        for (int f8 = 0; f8 < 8; ++f8) o.m[f8] = mi[(8 * r + f8) * 64 + lane];
    };
    auto step = [&](int b, const CombOps& o, int buf) {
        __syncthreads();   // the previous X's B operand is in xb[buf]
        const bool exact = __builtin_amdgcn_readfirstlane(flags[b]) == 0;
        const bool mm = exact && (b > 1 || p.s_init);
        f16x8 Sb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) Sb[j] = *reinterpret_cast<const f16x8*>(xb[buf] + (j * 64 + lane) * 8);
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) acc[tt] = mmh(__builtin_bit_cast(f16x8, o.m[4 * tt + j]), Sb[j], acc[tt]);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            // (a select, not a product with 0: the maps of warm-up boundaries and
            // M_0 without an initial state are never written and may hold NaNs)
            const f32x4 add = KIND == 1 ? f32x4{0.f, 0.f, 0.f, 0.f} : o.add[tt];
            cur[tt] = mm ? add + acc[tt] : add;
        }
        if (KIND == 0) {
            float* dst = p.seg_state + tiles_off(seg_base + b, p.h_v, h);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
                *reinterpret_cast<f32x4*>(dst + (((2 * r + tt) * 8 + u) * 64 + lane) * 4) = cur[tt];
        }
        comb_put(xb[buf ^ 1], cur);
    };
    CombOps A, B;
    fetch(A, b_lo);
    fetch(B, b_lo + 1);
    int b = b_lo;
    for (; b + 1 < b_hi; b += 2) {
        step(b, A, 0);
        fetch(A, b + 2);
        step(b + 1, B, 1);
        fetch(B, b + 3);
    }
    if (b < b_hi) step(b, A, 0);
}

// The segment combine as one chain: one 4-wave workgroup per (sequence, value
// head, 16-column tile u), the eight tiles of a (sequence, head) on one XCD.
// Boundary s (1 <= s < P): exact, S0(s) = M_{s-1} S0(s-1) + H_{s-1} (the map
// product on fp16 operands: the M image as A, the state column tile as B; M_0
// only with an initial state); warm-up, S0(s) is the warm-up state the CP
// preprocessing wrote.
__global__ __launch_bounds__(NTC) void k_combine16(Params p) {
    __shared__ int flags[kMaxSegsPerSeq];
    __shared__ __attribute__((aligned(16))) f16 xb[2][4 * 64 * 8];   // the state tile as B operands, per k step
    GDN_LDS_POISON_ALL(flags, xb);
    // workgroup id = XCD slot (q % 8) + 8 (column tile + 8 (q / 8)), q = seq h_v + head:
    // the eight column tiles of a (sequence, head) run on one XCD (workgroups
    // are dealt to the XCDs round-robin), so each M image is fetched into one
    // L2 instead of eight
    const int id = (int)blockIdx.x, u = (id >> 3) & 7, q = 8 * (id >> 6) + (id & 7);
    if (q >= p.n_seqs * p.h_v) return;
    const int seq = q / p.h_v, h = q % p.h_v;
    int P, seg_base;
    if (!comb_setup(p, seq, h, flags, P, seg_base)) return;
    f32x4 cur[2];
    if (p.s_init) comb_load_rm_tile(p.s_init + tiles_off(seq, p.h_v, h), u, cur);
    else cur[0] = cur[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    comb_put(xb[0], cur);
    comb_chain<0>(p, flags, xb, seg_base, h, u, 1, P, cur);
}

// The combine in two launches over groups of G = comb_G consecutive
// boundaries (group j: boundaries [1 + j G, min(1 + (j + 1) G, P)); its last,
// e_j): 2 G + J - 2 steps in sequence instead of P - 1.
//   k_comb16_groups  group 0 as a chain from S0(0); every later group, in 16
//                    column tiles of X = [CM | CH] from [I | 0], composes its
//                    boundaries' affine maps into one, S -> CM S + CH (CM as an
//                    fp16 A-operand image, CH in tile order);
//   k_comb16_apply   every group j >= 1: S0(e_{j-1}) from S0(e_0) through
//                    CM_i, CH_i (i = 1 .. j - 1), then its boundaries in turn.
// The (sequence, head, group) bundles' workgroups share an XCD.
__device__ __forceinline__ int comb_group_end(int j, int G, int P) { return min((j + 1) * G, P - 1); }

__global__ __launch_bounds__(NTC) void k_comb16_groups(Params p) {
    __shared__ int flags[kMaxSegsPerSeq];
    __shared__ __attribute__((aligned(16))) f16 xb[2][4 * 64 * 8];
    GDN_LDS_POISON_ALL(flags, xb);
    const int id = (int)blockIdx.x, k = (id >> 3) & 15, x = 8 * (id >> 7) + (id & 7);
    const int J = p.comb_J, G = p.comb_G;
    if (x >= p.n_seqs * p.h_v * J) return;
    const int j = x % J, q = x / J, seq = q / p.h_v, h = q % p.h_v;
    if (j == 0 && k >= 8) return;
    int P, seg_base;
    if (!comb_setup(p, seq, h, flags, P, seg_base)) return;
    const int b_lo = 1 + j * G, b_hi = min(b_lo + G, P);
    if (b_lo >= P) return;
    const int u = k & 7, r = wave_id(), lane = lane_id(), c = lane & 15, g = lane >> 4;
    f32x4 cur[2];
    if (j == 0) {
        if (p.s_init) comb_load_rm_tile(p.s_init + tiles_off(seq, p.h_v, h), u, cur);
        else cur[0] = cur[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        comb_put(xb[0], cur);
        comb_chain<0>(p, flags, xb, seg_base, h, u, b_lo, b_hi, cur);
        return;
    }
    const size_t grp = (size_t)(seq * J + j) * p.h_v + h;
    if (k < 8) {   // CM from I
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) cur[tt][e] = (32 * r + 16 * tt + 4 * g + e == 16 * u + c) ? 1.f : 0.f;
        comb_put(xb[0], cur);
        comb_chain<1>(p, flags, xb, seg_base, h, u, b_lo, b_hi, cur);
        // X[row][16 u + c] -> the A-operand image (fragment 4 (row / 16) + u / 2; lane
        // 16 (c / 4) + row % 16; slot 4 (u % 2) + c % 4: the kp order of the chain)
        f16* img = reinterpret_cast<f16*>(p.seg_GM) + grp * (size_t)DK * DK;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 32 * r + 16 * tt + 4 * g + e;
                img[((4 * (row >> 4) + (u >> 1)) * 64 + 16 * (c >> 2) + (row & 15)) * 8 + 4 * (u & 1) + (c & 3)] =
                    (f16)cur[tt][e];
            }
    } else {       // CH from 0
        cur[0] = cur[1] = f32x4{0.f, 0.f, 0.f, 0.f};
        comb_put(xb[0], cur);
        comb_chain<2>(p, flags, xb, seg_base, h, u, b_lo, b_hi, cur);
        float* dst = p.seg_GH + grp * (size_t)DK * DK;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
            *reinterpret_cast<f32x4*>(dst + (((2 * r + tt) * 8 + u) * 64 + lane) * 4) = cur[tt];
    }
}

__global__ __launch_bounds__(NTC) void k_comb16_apply(Params p) {
    __shared__ int flags[kMaxSegsPerSeq];
    __shared__ __attribute__((aligned(16))) f16 xb[2][4 * 64 * 8];
    GDN_LDS_POISON_ALL(flags, xb);
    const int id = (int)blockIdx.x, u = (id >> 3) & 7, x = 8 * (id >> 6) + (id & 7);
    const int J = p.comb_J, G = p.comb_G;
    if (x >= p.n_seqs * p.h_v * J) return;
    const int j = x % J, q = x / J, seq = q / p.h_v, h = q % p.h_v;
    if (j == 0) return;
    int P, seg_base;
    if (!comb_setup(p, seq, h, flags, P, seg_base)) return;
    const int b_lo = 1 + j * G, b_hi = min(b_lo + G, P);
    if (b_lo >= P) return;
    const int r = wave_id(), lane = lane_id();
    // S0(e_{j-1}): from S0(e_0) through the composed maps of groups 1 .. j - 1
    f32x4 cur[2];
    comb_load_tile(p.seg_state + tiles_off(seg_base + comb_group_end(0, G, P), p.h_v, h), u, cur);
    comb_put(xb[0], cur);
    struct LinkOps { f32x4 add[2]; u32x4 m[8]; };
    auto fetch = [&](LinkOps& o, int jj) {
        jj = min(jj, j - 1);
        const size_t grp = (size_t)(seq * J + jj) * p.h_v + h;
        comb_load_tile(p.seg_GH + grp * (size_t)DK * DK, u, o.add);
        const u32x4* mi = reinterpret_cast<const u32x4*>(reinterpret_cast<const f16*>(p.seg_GM) + grp * (size_t)DK * DK);
#pragma unroll
        for (int f8 = 0; f8 < 8; ++f8) o.m[f8] = mi[(8 * r + f8) * 64 + lane];
    };
    auto step = [&](const LinkOps& o, int buf) {
        __syncthreads();
        f16x8 Sb[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) Sb[kk] = *reinterpret_cast<const f16x8*>(xb[buf] + (kk * 64 + lane) * 8);
        f32x4 acc[2] = {o.add[0], o.add[1]};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) acc[tt] = mmh(__builtin_bit_cast(f16x8, o.m[4 * tt + kk]), Sb[kk], acc[tt]);
        cur[0] = acc[0];
        cur[1] = acc[1];
        comb_put(xb[buf ^ 1], cur);
    };
    if (j > 1) {
        LinkOps A, B;
        fetch(A, 1);
        fetch(B, 2);
        int jj = 1;
        for (; jj + 1 < j; jj += 2) {
            step(A, 0);
            fetch(A, jj + 2);
            step(B, 1);
            fetch(B, jj + 3);
        }
        if (jj < j) step(A, 0);
        __syncthreads();   // every wave's last step is done: the state goes to xb[0]
        comb_put(xb[0], cur);
    }
    // then the group's boundaries, every state stored
    comb_chain<0>(p, flags, xb, seg_base, h, u, b_lo, b_hi, cur);
}

// ----------------------------------------------------------------------------
// The fused forward of one segment per (segment slot, value head): from its
// initial state (the caller's for segment 0, else the boundary state), every
// chunk's output and state update; the last segment writes the final state.
template <typename IO>
__global__ __launch_bounds__(NT8) void k_fwd16(Params p) {
    __shared__ Smem16<IO, true> sm;
    GDN_LDS_POISON_ALL(sm);
    const int h = blockIdx.y;
    const SegLoc loc = locate_segment(p, blockIdx.x);
    if (loc.seq < 0) return;
    f32x4 S[8];
    if (loc.s == 0) {
        if (p.s_init) load_rm(p.s_init + tiles_off(loc.seq, p.h_v, h), S);
        else set_state(S, false);
    } else {
        load_tiles(p.seg_state + tiles_off(loc.seg_base + loc.s, p.h_v, h), S);
    }
    const int c0 = loc.s * p.L, c1 = min(c0 + p.L, loc.N);
    run_chunks16<IO, true, true>(sm, p, loc, h, c0, c1, S);
    if (loc.s == loc.P - 1 && p.s_final) store_rm(p.s_final + tiles_off(loc.seq, p.h_v, h), S);
}

// ----------------------------------------------------------------------------
// The fused forward with specialised waves (bf16 inputs). Waves 0-3 (state
// waves) own the d_v columns [32 w, 32 w + 32) of S in registers and produce
// the same columns of the output; waves 4-7 (staging waves) compute P and
// stage every operand, one per SIMD beside a state wave. Per chunk n:
//   state:   O^T = S^T Q^T and Y = K S from the state's fp16 copy,
//            S <- e^gamma_C S, Y = V - e^gamma Y (V through the identity
//            product, its rows loaded a chunk and a half ahead),
//            V' = T diag(beta) Y, O^T scaled by scale e^gamma
//   staging: the next chunk's gate factors; its row block of P
//   -- barrier --
//   state:   O^T += V'^T P^T, stores; S += K~^T V' with
//            K~ = diag(e^(gamma_C - gamma)) K (staged scaled)
//   staging: the next chunk's K, K~^T, Q and T diag(beta); loads for the
//            one after
//   -- barrier --
// The state and V' stay in the state waves' registers: LDS carries only
// the staged inputs and P. K~^T and the gate factors are double-buffered;
// K, Q and T diag(beta) single (their readers are past the first barrier
// when they are restaged). The gate factors come from k_prep, per chunk and
// head.
//
// LDS layouts (row strides chosen by measurement: each operand read and
// staging write runs at the LDS's full rate):
//   K, Q   [64 tokens][128 d_k in kp order, + 16]
//   K~^T   [128 d_k][64 tokens in kp order, + 16], 16-byte pieces of row d
//          at piece ^ tswz(d)
//   P      [64 rows][64 columns in kp order, + 8]
constexpr int kWsRow = 144;                                   // halfs per K / Q row
constexpr int kWsRowT = 80;                                   // halfs per K~^T row
constexpr int kWsRowP = 72;                                   // halfs per P row
__device__ __forceinline__ int kq_at(int r, int piece) { return r * kWsRow + 8 * piece; }
__device__ __forceinline__ int p_at(int r, int piece) { return r * kWsRowP + 8 * piece; }

struct __attribute__((aligned(16))) SmemWS {
    f16 k[CH * kWsRow];                   // K
    f16 q[CH * kWsRow];                   // Q
    f16 kt[2][DK * kWsRowT];              // K~^T
    f16 tb[kTbHalfs];                     // T diag(beta) fragments (k_prep's image)
    f16 p[CH * kWsRowP];                  // P
    float gf[2][kGfFloats];               // gamma log2(e), e^gamma, e^(gamma_C - gamma), e^gamma_C
};

__device__ __forceinline__ f16x8 to_h8(const u32x4& x) {
    return __builtin_convertvector(
        f32x8{__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xffff0000u), __uint_as_float(x[1] << 16),
              __uint_as_float(x[1] & 0xffff0000u), __uint_as_float(x[2] << 16), __uint_as_float(x[2] & 0xffff0000u),
              __uint_as_float(x[3] << 16), __uint_as_float(x[3] & 0xffff0000u)},
        f16x8);
}

// Staging map of thread t < 256 of the staging waves: tokens 4 (t / 16) + j
// (j < 4), d_k 8 (t % 16) .. + 8; in kp order the d_k are the positions
// ws_p0(t) .. + 4 and ws_p0(t) + 8 .. + 12, the tokens ws_pt(t) .. + 4.
__device__ __forceinline__ int ws_p0(int t) { return 32 * ((t & 15) >> 2) + 16 * (t & 1) + 4 * ((t >> 1) & 1); }
__device__ __forceinline__ int ws_pt(int t) {
    const int rq = (t >> 4) & 15;
    return 32 * (rq >> 3) + 8 * (rq & 3) + 4 * ((rq >> 2) & 1);
}
// rows of one chunk's [tokens][heads][128] bf16 input in the staging map
// (rows past the sequence's end read as zeros)
__device__ __forceinline__ void ws_load_rows(u32x4 (&x)[4], const void* base, size_t tok0, size_t ts, int hd,
                                             int nvalid, int t) {
    const auto r = rsrc(static_cast<const bf16*>(base) + tok0 * ts + (size_t)hd * DK, (unsigned)nvalid * (unsigned)ts * 2);
#pragma unroll
    for (int j = 0; j < 4; ++j)
        x[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(((4 * ((t >> 4) & 15) + j) * ts + 8 * (t & 15)) * 2), 0, 0);
}
__device__ __forceinline__ void ws_put_rows(f16* dst, const u32x4 (&x)[4], int t) {
    const int p0 = ws_p0(t), r0 = 4 * ((t >> 4) & 15);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f16x8 h = to_h8(x[j]);
        f16* d = dst + (r0 + j) * kWsRow;
        *reinterpret_cast<f16x4*>(d + p0) = f16x4{h[0], h[1], h[2], h[3]};
        *reinterpret_cast<f16x4*>(d + p0 + 8) = f16x4{h[4], h[5], h[6], h[7]};
    }
}

// State wave over chunks [c_lo, c_hi) owning the NC 16-column tiles from
// column col (a multiple of 16 NC): S[8][NC] (tiles [i][n], rows 16 i + 4 g + e,
// column col + 16 n + c) in registers.
template <int NC>
__device__ void ws_state(SmemWS& sm, const Params& p, const SegLoc& loc, int h, int c_lo, int c_hi, int col,
                         f32x4 S[8][NC]) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const size_t tsv = (size_t)p.h_v * DK;
    // K~^T operand offsets: kt_at(16 i + c, 4 j + g) splits into this lane's
    // part for i % 4 and a constant (the swizzle XORs bits 3-5 of the piece
    // offset with 8 i)
    int ktl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ktl[r] = c * kWsRowT + ((8 * g) ^ (8 * r));
    // V rows of the 32 columns around this wave's, as the A operands of the
    // identity product: token 16 m + c, d_v v32 + 8 g .. + 8 (rows past the end
    // read as zeros); E[n] picks column tile e0 + n of the 32
    const int v32 = col & ~31, e0 = (col >> 4) & 1;
    auto vfetch = [&](u32x4 V[4], int cc) {
        cc = min(cc, c_hi - 1);
        const auto rv = rsrc(static_cast<const bf16*>(p.v) + (loc.tok0 + (size_t)cc * CH) * tsv + (size_t)h * DK,
                             (unsigned)min(CH, loc.len - cc * CH) * (unsigned)tsv * 2);
#pragma unroll
        for (int m = 0; m < 4; ++m)
            V[m] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(((16 * m + c) * tsv + v32 + 8 * g) * 2), 0, 0);
    };
    bf16x8 E[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n)
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) E[n][s2] = (bf16)((8 * g + s2 == 16 * (e0 + n) + c) ? 1.f : 0.f);
    u32x4 VA[4], VB[4];
    vfetch(VA, c_lo);
    vfetch(VB, c_lo + 1);
    __syncthreads();   // (0) the first chunk's gate factors staged
    __syncthreads();   // (1) the first chunk staged
    auto step = [&](int b, const u32x4 (&V)[4], int cc) {
        const float* gf = sm.gf[b];
        // O^T = S^T Q^T and Y = K S from the state's fp16 copy
        f32x4 O[NC][4], Y[4][NC];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < NC; ++n) O[n][m] = Y[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f16x8 sb[NC], kf[4], qf[4];
#pragma unroll
            for (int n = 0; n < NC; ++n) sb[n] = pack8h(S[2 * j][n], S[2 * j + 1][n]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                kf[m] = *reinterpret_cast<const f16x8*>(sm.k + kq_at(16 * m + c, 4 * j + g));
                qf[m] = *reinterpret_cast<const f16x8*>(sm.q + kq_at(16 * m + c, 4 * j + g));
            }
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    Y[m][n] = mmh(kf[m], sb[n], Y[m][n]);
                    O[n][m] = mmh(sb[n], qf[m], O[n][m]);
                }
            __builtin_amdgcn_sched_barrier(0);   // (bounds the operand reads in flight)
        }
        // the decay of this chunk's state update, ahead of it
        const float ec = gf[3 * CH];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int n = 0; n < NC; ++n) S[i][n] *= ec;
        // Y = V - e^gamma (K S)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 eg = *reinterpret_cast<const f32x4*>(gf + CH + 16 * m + 4 * g);
#pragma unroll
            for (int n = 0; n < NC; ++n) Y[m][n] = mma16k32(__builtin_bit_cast(bf16x8, V[m]), E[n], Y[m][n] * -eg);
        }
        // V' = (T diag(beta)) Y
        f16x8 Vb[2][NC];
        {
            f16x8 Yb[2][NC], tf[6];
#pragma unroll
            for (int f = 0; f < 6; ++f) tf[f] = *reinterpret_cast<const f16x8*>(sm.tb + (f * 64 + lane) * 8);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int n = 0; n < NC; ++n) Yb[j][n] = pack8h(Y[2 * j][n], Y[2 * j + 1][n]);
            f32x4 Vp[4][NC];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    Vp[m][n] = mmh(tf[tb_frag(m, 0)], Yb[0][n], f32x4{0.f, 0.f, 0.f, 0.f});
                    if (m >= 2) Vp[m][n] = mmh(tf[tb_frag(m, 1)], Yb[1][n], Vp[m][n]);
                }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int n = 0; n < NC; ++n) Vb[j][n] = pack8h(Vp[2 * j][n], Vp[2 * j + 1][n]);
        }
        // O^T scaled per token by scale e^gamma
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float es = p.scale * gf[CH + 16 * m + c];
#pragma unroll
            for (int n = 0; n < NC; ++n) O[n][m] *= es;
        }
        __syncthreads();   // (2) P complete; the readers of K, Q and T diag(beta) are past
        // O^T += V'^T P^T (P causal: token tiles 0 and 1 need k step 0 only)
        {
            f16x8 pf[6];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (j == 1 && m < 2) continue;
                    pf[tb_frag(m, j)] = *reinterpret_cast<const f16x8*>(sm.p + p_at(16 * m + c, 4 * j + g));
                }
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if (j == 1 && m < 2) continue;
#pragma unroll
                    for (int n = 0; n < NC; ++n) O[n][m] = mmh(Vb[j][n], pf[tb_frag(m, j)], O[n][m]);
                }
        }
        // lane (g, c) of tile (n, m): token 16 m + c, d_v col + 16 n + 4 g + (0..3)
        // (rows past the sequence's end fall outside the descriptor: dropped)
        const auto ro = rsrc(static_cast<bf16*>(p.out) + (loc.tok0 + (size_t)cc * CH) * tsv + (size_t)h * DK,
                             (unsigned)min(CH, loc.len - cc * CH) * (unsigned)tsv * 2);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < NC; ++n)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_rne(O[n][m][0], O[n][m][1]), pack_rne(O[n][m][2], O[n][m][3])},
                                                      ro, (int)(((16 * m + c) * tsv + col + 16 * n + 4 * g) * 2), 0, 0);
        // S += K~^T V'
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            f16x8 ktf[8];
#pragma unroll
            for (int i = 0; i < 8; ++i)
                ktf[i] = *reinterpret_cast<const f16x8*>(sm.kt[b] + ktl[i & 3] + 16 * i * kWsRowT + ((32 * j) ^ (32 * (i >> 2))));
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int n = 0; n < NC; ++n) S[i][n] = mmh(ktf[i], Vb[j][n], S[i][n]);
        }
        __syncthreads();   // (3) the next chunk staged
    };
    int cc = c_lo;
    for (; cc + 1 < c_hi; cc += 2) {
        step(0, VA, cc);
        vfetch(VA, cc + 2);
        step(1, VB, cc + 1);
        vfetch(VB, cc + 3);
    }
    if (cc < c_hi) step(0, VA, cc);
}

// Staging wave cw over chunks [c_lo, c_hi) (threads t = 64 cw + lane): P's
// row block [16 cw, 16 cw + 16) and the staging of every operand. Chunk c's
// inputs are held in register set c % 2 (of the loop's parity b) between their
// loads and their staging: during the step of chunk n the set of chunk n + 2
// (free since chunk n was staged) is filled half in the first part of the
// step (K rows, T diag(beta)) and half after the first barrier (Q rows), so
// the memory pipe's time for the loads is spread over both halves, beside
// the P product and beside the staging of chunk n + 1.
struct WsIn {
    u32x4 kr[4], qr[4], tbr[2];
};
__device__ void ws_stage(SmemWS& sm, const Params& p, const SegLoc& loc, int h, int c_lo, int c_hi, int cw) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, t = 64 * cw + lane;
    const int hq = h / p.group;
    const size_t ts = (size_t)p.h_qk * DK;
    const float log2_scale = __log2f(p.scale);
    WsIn R[2];
    auto rows_of = [&](int& cc, size_t& tok0, int& nv) {
        cc = min(cc, c_hi - 1);
        tok0 = loc.tok0 + (size_t)cc * CH;
        nv = min(CH, loc.len - cc * CH);
    };
    // K rows and T diag(beta) of chunk cc
    auto fetch_a = [&](WsIn& r, int cc) {
        size_t tok0;
        int nv;
        rows_of(cc, tok0, nv);
        ws_load_rows(r.kr, p.k, tok0, ts, hq, nv, t);
        const size_t blk = (size_t)(loc.chunk_base + cc) * p.h_v + h;
        const u32x4* tb = reinterpret_cast<const u32x4*>(static_cast<const f16*>(p.tb16) + blk * (size_t)kTbHalfs);
        r.tbr[0] = tb[t];
        r.tbr[1] = tb[t < 128 ? 256 + t : t];   // (pieces 256..383; the rest load piece t again)
    };
    // Q rows of chunk cc
    auto fetch_b = [&](WsIn& r, int cc) {
        size_t tok0;
        int nv;
        rows_of(cc, tok0, nv);
        ws_load_rows(r.qr, p.q, tok0, ts, hq, nv, t);
    };
    // gate factors, loaded two chunks ahead of their staging
    auto gfetch = [&](int cc) {
        cc = min(cc, c_hi - 1);
        return p.gf16[((size_t)(loc.chunk_base + cc) * p.h_v + h) * kGfFloats + t];
    };
    // K, K~^T (into kt[b], from the gate factors in gf[b]), Q and T diag(beta)
    auto stage = [&](int b, const WsIn& r) {
        // (the factors are read ahead of the writes: an LDS read waits for
        // every LDS access issued before it)
        const f32x4 kfac = *reinterpret_cast<const f32x4*>(sm.gf[b] + 2 * CH + 4 * ((t >> 4) & 15));
        __builtin_amdgcn_sched_barrier(0);
        ws_put_rows(sm.k, r.kr, t);
        ws_put_rows(sm.q, r.qr, t);
        *reinterpret_cast<u32x4*>(sm.tb + 8 * t) = r.tbr[0];
        if (t < 128) *reinterpret_cast<u32x4*>(sm.tb + 8 * (256 + t)) = r.tbr[1];
        const int pt = ws_pt(t);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = 8 * (t & 15) + e;
            f32x4 col;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned wv = r.kr[j][e >> 1];
                col[j] = __uint_as_float((e & 1) ? (wv & 0xffff0000u) : (wv << 16)) * kfac[j];
            }
            *reinterpret_cast<f16x4*>(sm.kt[b] + d * kWsRowT + (pt ^ tswz(d))) = __builtin_convertvector(col, f16x4);
        }
    };
    // (loads issue in the loop's order: operands, then gate factors)
    float gfr[2];
    sm.gf[0][t] = gfetch(c_lo);
    gfr[1] = gfetch(c_lo + 1);
    fetch_a(R[0], c_lo);
    fetch_b(R[0], c_lo);
    __syncthreads();   // (0)
    stage(0, R[0]);
    fetch_a(R[1], c_lo + 1);
    fetch_b(R[1], c_lo + 1);
    gfr[0] = gfetch(c_lo + 2);
    __syncthreads();   // (1)
    auto step = [&](int b, int cc) {
        const float* gf = sm.gf[b];
        // the next chunk's gate factors (their buffer's last readers passed
        // the previous step's end)
        sm.gf[b ^ 1][t] = gfr[b ^ 1];
        // P's row block: P^T tiles k_i . q_r, i block ib
        f32x4 Pt[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) Pt[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f16x8 kf[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) kf[m] = *reinterpret_cast<const f16x8*>(sm.k + kq_at(16 * m + c, 4 * j + g));
            const f16x8 qw = *reinterpret_cast<const f16x8*>(sm.q + kq_at(16 * cw + c, 4 * j + g));
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) Pt[ib] = mmh(kf[ib], qw, Pt[ib]);
        }
        // chunk cc + 2 into the set chunk cc left (staged in the previous step)
        fetch_a(R[b], cc + 2);
        {
            // P[r][i] = scale 2^(gamma_r - gamma_i) (q_r . k_i), i <= r (gamma times log2 e)
            const int r = 16 * cw + c;
            const float gr = gf[r] + log2_scale;
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                const int i0 = 16 * ib + 4 * g;
                const f32x4 gi = *reinterpret_cast<const f32x4*>(gf + i0);
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (i0 + e <= r) ? __builtin_amdgcn_exp2f(gr - gi[e]) * Pt[ib][e] : 0.f;
                *reinterpret_cast<f16x4*>(sm.p + p_at(r, 4 * (ib >> 1) + g) + 4 * (ib & 1)) =
                    __builtin_convertvector(v, f16x4);
            }
        }
        __syncthreads();   // (2)
        stage(b ^ 1, R[b ^ 1]);
        fetch_b(R[b], cc + 2);
        gfr[b ^ 1] = gfetch(cc + 3);
        __syncthreads();   // (3)
    };
    int cc = c_lo;
    for (; cc + 1 < c_hi; cc += 2) {
        step(0, cc);
        step(1, cc + 1);
    }
    if (cc < c_hi) step(0, cc);
}

// The fused forward, grid (segment slot, value head, column block): column
// block cb of p.dv_split covers the d_v columns [cb 128 / dv_split, ...); NSW
// state waves own NC 16-column tiles each (NSW 16 NC = 128 / dv_split), the
// four staging waves follow them.
template <int NSW, int NC>
__global__ __launch_bounds__(64 * (NSW + 4)) void k_fwd_ws(Params p) {
    __shared__ SmemWS sm;
    GDN_LDS_POISON_ALL(sm);
    const int h = blockIdx.y, w = wave_id();
    const SegLoc loc = locate_segment(p, blockIdx.x);
    if (loc.seq < 0) return;
    const int c0 = loc.s * p.L, c1 = min(c0 + p.L, loc.N);
    if (w < NSW) {
        const int lane = lane_id(), c = lane & 15, g = lane >> 4;
        const int col = (int)blockIdx.z * (16 * NC * NSW) + 16 * NC * w;
        f32x4 S[8][NC];
        const float* src = loc.s == 0 ? p.s_init : p.seg_state;
        if (loc.s == 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int n = 0; n < NC; ++n)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        S[i][n][e] = src ? src[tiles_off(loc.seq, p.h_v, h) + (16 * i + 4 * g + e) * DK + col + 16 * n + c] : 0.f;
        } else {
            const float* sg = src + tiles_off(loc.seg_base + loc.s, p.h_v, h);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int n = 0; n < NC; ++n)
                    S[i][n] = *reinterpret_cast<const f32x4*>(sg + ((i * 8 + (col >> 4) + n) * 64 + lane) * 4);
        }
        if (c0 < c1) ws_state<NC>(sm, p, loc, h, c0, c1, col, S);
        if (loc.s == loc.P - 1 && p.s_final) {
            float* dst = p.s_final + tiles_off(loc.seq, p.h_v, h);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int n = 0; n < NC; ++n)
#pragma unroll
                    for (int e = 0; e < 4; ++e) dst[(16 * i + 4 * g + e) * DK + col + 16 * n + c] = S[i][n][e];
        }
    } else if (c0 < c1) {
        ws_stage(sm, p, loc, h, c0, c1, w - NSW);
    }
}

// ----------------------------------------------------------------------------
// CP preprocessing with specialised waves (bf16 inputs). Four state waves
// (each owning 32 d_v columns) run the state: from zero over the previous
// segment (H of an exact boundary) or over the warm-up window (from zero, or
// from the initial state where the window starts at the sequence start).
// Four map waves run the map of an exact boundary's previous segment from
// the identity with V = 0 (M, 32 columns each). Four staging waves stage K,
// K~^T, V, T diag(beta) and the gate factors of every chunk, all
// double-buffered in LDS, so a chunk step needs one barrier and the chain
// waves issue no global loads. Two layouts: the state and map waves of an
// exact boundary in one 12-wave workgroup on the same staged chunks, or
// (SPLIT) in two 8-wave workgroups, one chain wave per SIMD with the whole
// register file's share. The chunk step of a state or map wave is the
// forward's without the output: Y = K S, S <- e^gamma_C S, Y = V - e^gamma Y
// (V = 0 for M), V' = T diag(beta) Y, S += K~^T V'.
struct __attribute__((aligned(16))) SmemCP {
    // (the small buffers first: more of the operand reads reach their
    // addresses through the LDS instructions' 16-bit offsets)
    float gf[2][kGfFloats];               // gate factors (as in the fused forward)
    f16 tb[2][kTbHalfs];                  // T diag(beta) fragments
    f16 k[2][CH * kWsRow];                // K (the map image overlays both at the end)
    f16 kt[2][DK * kWsRowT];              // K~^T
    bf16 v[2][CH * kWsRow];               // V rows, d_v in natural order
};
static_assert(sizeof(f16) * 2 * CH * kWsRow >= sizeof(f16) * DK * LMI, "map image fits over K");
constexpr int kCpWaves = 12;

// State (WANT_V) or map wave over chunks [c_lo, c_hi), 32 columns from col:
// S[i][n] is the tile of rows 16 i + 4 g + e, column col + 16 n + c. WIDE:
// the register budget of an 8-wave workgroup (operand reads run ahead).
template <bool WANT_V, bool WIDE>
__device__ void cp_state(SmemCP& sm, int c_lo, int c_hi, int col, f32x4 S[8][2]) {
    constexpr int NC = 2;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    // K~^T operand offsets: kt_at(16 i + c, 4 j + g) splits into this lane's
    // part for i % 4 and a constant (the swizzle XORs bits 3-5 of the piece
    // offset with 8 i)
    int ktl[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) ktl[r] = c * kWsRowT + ((8 * g) ^ (8 * r));
    bf16x8 E[NC];
#pragma unroll
    for (int n = 0; n < NC; ++n)
#pragma unroll
        for (int s2 = 0; s2 < 8; ++s2) E[n][s2] = (bf16)((8 * g + s2 == 16 * n + c) ? 1.f : 0.f);
    __syncthreads();   // the first chunk staged
    auto step = [&](int b) {
        const float* gf = sm.gf[b];
        // Y = K S from the state's fp16 copy
        f32x4 Y[4][NC];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int n = 0; n < NC; ++n) Y[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f16x8 sb[NC], kf[4];
#pragma unroll
            for (int n = 0; n < NC; ++n) sb[n] = pack8h(S[2 * j][n], S[2 * j + 1][n]);
#pragma unroll
            for (int m = 0; m < 4; ++m) kf[m] = *reinterpret_cast<const f16x8*>(sm.k[b] + kq_at(16 * m + c, 4 * j + g));
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < NC; ++n) Y[m][n] = mmh(kf[m], sb[n], Y[m][n]);
            if constexpr (!WIDE) __builtin_amdgcn_sched_barrier(0);   // (bounds the operand reads in flight)
        }
        const float ec = gf[3 * CH];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int n = 0; n < NC; ++n) S[i][n] *= ec;
        // Y = V - e^gamma (K S); V through the identity product (A: token
        // 16 m + c, d_v col + 8 g .. + 8)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f32x4 eg = *reinterpret_cast<const f32x4*>(gf + CH + 16 * m + 4 * g);
            if constexpr (WANT_V) {
                const bf16x8 vr = *reinterpret_cast<const bf16x8*>(sm.v[b] + (16 * m + c) * kWsRow + col + 8 * g);
#pragma unroll
                for (int n = 0; n < NC; ++n) Y[m][n] = mma16k32(vr, E[n], Y[m][n] * -eg);
            } else {
#pragma unroll
                for (int n = 0; n < NC; ++n) Y[m][n] *= -eg;
            }
        }
        // V' = (T diag(beta)) Y
        f16x8 Vb[2][NC];
        {
            f16x8 Yb[2][NC], tf[6];
#pragma unroll
            for (int f = 0; f < 6; ++f) tf[f] = *reinterpret_cast<const f16x8*>(sm.tb[b] + (f * 64 + lane) * 8);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int n = 0; n < NC; ++n) Yb[j][n] = pack8h(Y[2 * j][n], Y[2 * j + 1][n]);
            f32x4 Vp[4][NC];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int n = 0; n < NC; ++n) {
                    Vp[m][n] = mmh(tf[tb_frag(m, 0)], Yb[0][n], f32x4{0.f, 0.f, 0.f, 0.f});
                    if (m >= 2) Vp[m][n] = mmh(tf[tb_frag(m, 1)], Yb[1][n], Vp[m][n]);
                }
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int n = 0; n < NC; ++n) Vb[j][n] = pack8h(Vp[2 * j][n], Vp[2 * j + 1][n]);
        }
        // S += K~^T V'
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            f16x8 ktf[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) ktf[i] = *reinterpret_cast<const f16x8*>(sm.kt[b] + ktl[i & 3] + 16 * i * kWsRowT + ((32 * j) ^ (32 * (i >> 2))));
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int n = 0; n < NC; ++n) S[i][n] = mmh(ktf[i], Vb[j][n], S[i][n]);
            if constexpr (!WIDE) __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();   // the next chunk staged; this one's buffers free
    };
    int cc = c_lo;
    for (; cc + 1 < c_hi; cc += 2) {
        step(0);
        step(1);
    }
    if (cc < c_hi) step(0);
}

// Staging wave cw of the CP preprocessing (threads t = 64 cw + lane): during
// the step of chunk n it stages chunk n + 1 into the other buffers and loads
// chunk n + 3 into the register set chunk n + 1 left (two sets: the loads have
// two steps to land; past the last chunk, the last one again: staged, never
// read). want_v: stage V (no map-only workgroup reads it).
struct CpIn {
    u32x4 kr[4], vr[4], tbr[2];
    float gfr;
    f32x4 kfac;   // e^(gamma_C - gamma) of this thread's four tokens
};
__device__ void cp_stage(SmemCP& sm, const Params& p, const SegLoc& loc, int h, int c_lo, int c_hi, int cw,
                         bool want_v) {
    const int t = 64 * cw + lane_id();
    const int hq = h / p.group;
    const size_t ts = (size_t)p.h_qk * DK, tsv = (size_t)p.h_v * DK;
    CpIn R[2];
    auto fetch = [&](CpIn& r, int cc) {
        cc = min(cc, c_hi - 1);
        const size_t tok0 = loc.tok0 + (size_t)cc * CH;
        const int nv = min(CH, loc.len - cc * CH);
        ws_load_rows(r.kr, p.k, tok0, ts, hq, nv, t);
        if (want_v) ws_load_rows(r.vr, p.v, tok0, tsv, h, nv, t);
        const size_t blk = (size_t)(loc.chunk_base + cc) * p.h_v + h;
        const u32x4* tb = reinterpret_cast<const u32x4*>(static_cast<const f16*>(p.tb16) + blk * (size_t)kTbHalfs);
        r.tbr[0] = tb[t];
        r.tbr[1] = tb[t < 128 ? 256 + t : t];   // (pieces 256..383; the rest load piece t again)
        const float* gfb = p.gf16 + blk * (size_t)kGfFloats;
        r.gfr = gfb[t];
        r.kfac = *reinterpret_cast<const f32x4*>(gfb + 2 * CH + 4 * ((t >> 4) & 15));
    };
    auto stage = [&](int b, const CpIn& r) {
        ws_put_rows(sm.k[b], r.kr, t);
        if (want_v) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x4*>(sm.v[b] + (4 * ((t >> 4) & 15) + j) * kWsRow + 8 * (t & 15)) = r.vr[j];
        }
        *reinterpret_cast<u32x4*>(sm.tb[b] + 8 * t) = r.tbr[0];
        if (t < 128) *reinterpret_cast<u32x4*>(sm.tb[b] + 8 * (256 + t)) = r.tbr[1];
        sm.gf[b][t] = r.gfr;
        const int pt = ws_pt(t);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = 8 * (t & 15) + e;
            f32x4 col;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned wv = r.kr[j][e >> 1];
                col[j] = __uint_as_float((e & 1) ? (wv & 0xffff0000u) : (wv << 16)) * r.kfac[j];
            }
            *reinterpret_cast<f16x4*>(sm.kt[b] + d * kWsRowT + (pt ^ tswz(d))) = __builtin_convertvector(col, f16x4);
        }
    };
    fetch(R[0], c_lo);
    fetch(R[1], c_lo + 1);
    stage(0, R[0]);
    fetch(R[0], c_lo + 2);
    __syncthreads();   // the first chunk staged
    int cc = c_lo;
    for (; cc + 1 < c_hi; cc += 2) {
        stage(1, R[1]);
        fetch(R[1], cc + 3);
        __syncthreads();
        stage(0, R[0]);
        fetch(R[0], cc + 4);
        __syncthreads();
    }
    if (cc < c_hi) {
        stage(1, R[1]);
        __syncthreads();
    }
}

// One workgroup per boundary pair (order as planned, see cp_pick), or with
// SPLIT one per part: an exact boundary's H and M then run in two 8-wave
// workgroups (four state or map waves, four staging waves), each with a
// SIMD's matrix pipe to one chain wave. Output: exact boundary s (between
// segments s - 1 and s): H_{s-1} (tile order) and, where it matters (s > 1
// or an initial state), M_{s-1} as the combine's fp16 A-operand image;
// warm-up boundary: its state (tile order).
template <bool SPLIT>
__global__ __launch_bounds__(64 * (SPLIT ? 8 : kCpWaves)) void k_cp_ws(Params p) {
    constexpr int NW = SPLIT ? 8 : kCpWaves;
    __shared__ SmemCP sm;
    __shared__ int rank_red[2 * NW + 4];
    GDN_LDS_POISON_ALL(sm, rank_red);
    int part;
    const int q = cp_pick<NW, SPLIT ? 2 : 1>(p, (int)blockIdx.x, rank_red, part);
    if (q < 0) return;
    const int slot = q / p.h_v, h = q % p.h_v;
    const SegLoc loc = locate_segment(p, slot);
    int wq;
    const int cls = pair_class16(p, q, wq);
    if (cls < 0) return;
    const int a = loc.s * p.L;   // first chunk of segment s
    const int c_lo = cls ? a - wq : a - p.L, c_hi = a;
    const bool want_m = cls == 0 && (loc.s > 1 || p.s_init);
    if (SPLIT && part == 1 && !want_m) return;
    // waves: [0, 4) state (or, with SPLIT and part 1, map); without SPLIT
    // [4, 8) map; the last four staging
    const bool run_h = !SPLIT || part == 0, run_m = SPLIT ? part == 1 : want_m;
    const int w = wave_id(), lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int role = w >= NW - 4 ? 2 : (SPLIT ? (run_h ? 0 : 1) : (w < 4 ? 0 : 1));
    if (role == 0) {
        const int col = 32 * (w & 3);
        f32x4 S[8][2];
        const bool from_init = cls && c_lo == 0 && p.s_init;
        const float* s0 = from_init ? p.s_init + tiles_off(loc.seq, p.h_v, h) : nullptr;
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[i][n][e] = s0 ? s0[(16 * i + 4 * g + e) * DK + col + 16 * n + c] : 0.f;
        cp_state<true, SPLIT>(sm, c_lo, c_hi, col, S);
        float* dst = cls ? p.seg_state + tiles_off(loc.seg_base + loc.s, p.h_v, h)
                         : p.seg_H + tiles_off(loc.seg_base + loc.s - 1, p.h_v, h);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int n = 0; n < 2; ++n)
                *reinterpret_cast<f32x4*>(dst + ((i * 8 + (col >> 4) + n) * 64 + lane) * 4) = S[i][n];
    } else if (role == 1) {
        if (!run_m) {
            for (int k = c_lo; k <= c_hi; ++k) __syncthreads();   // (the chain's barriers)
            return;
        }
        const int wm = w & 3, col = 32 * wm;
        f32x4 S[8][2];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[i][n][e] = (16 * i + 4 * g + e == col + 16 * n + c) ? 1.f : 0.f;
        cp_state<false, SPLIT>(sm, c_lo, c_hi, col, S);
        // M -> the combine's A-operand image: fragment F = 4 rt + j holds, in
        // lane (g, c), row 16 rt + c at the kp positions 32 j + 8 g .. + 8 --
        // columns of block j, which are this wave's when j = wm. Staged through
        // LDS (row i, columns in kp order) over the K buffers, whose last
        // readers passed the chain's last barrier; each wave reads back only
        // what it wrote.
        f16* img = &sm.k[0][0];
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int n = 0; n < 2; ++n)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    img[(16 * i + 4 * g + e) * LMI + col + 8 * (c >> 2) + 4 * n + (c & 3)] = (f16)S[i][n][e];
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        f16* dst = reinterpret_cast<f16*>(p.seg_M) + tiles_off(loc.seg_base + loc.s - 1, p.h_v, h);
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
            *reinterpret_cast<f16x8*>(dst + ((size_t)(4 * rt + wm) * 64 + lane) * 8) =
                *reinterpret_cast<const f16x8*>(img + (16 * rt + c) * LMI + col + 8 * g);
    } else {
        cp_stage(sm, p, loc, h, c_lo, c_hi, w - (NW - 4), run_h);
    }
}

// Boundary states in tile order -> row-major (debug copies).
__global__ __launch_bounds__(64) void k_tiles_to_rm(const float* src, float* dst) {
    const size_t blk = blockIdx.x;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const float* s = src + blk * DK * DK;
    float* d = dst + blk * DK * DK;
    for (int tu = 0; tu < 64; ++tu) {
        const int t = tu >> 3, u = tu & 7;
        const f32x4 v = *reinterpret_cast<const f32x4*>(s + (tu * 64 + lane) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) d[(16 * t + 4 * g + e) * DK + 16 * u + c] = v[e];
    }
}

int launched16() { return (int)hipGetLastError(); }

}  // namespace

int launch_cp_prep16(const Params& p, int io, void* stream) {
    if (io == kIoBf16) {
        if (p.cp_split)
            hipLaunchKernelGGL(k_cp_ws<true>, dim3((unsigned)(16 * ((p.n_segments * p.h_v + 7) / 8) + 16)),
                               dim3(64 * 8), 0, (hipStream_t)stream, p);
        else
            hipLaunchKernelGGL(k_cp_ws<false>, dim3((unsigned)(p.n_segments * p.h_v)), dim3(64 * kCpWaves), 0,
                               (hipStream_t)stream, p);
    } else {
        hipLaunchKernelGGL(k_cp_prep16<float>, dim3((unsigned)(16 * ((p.n_segments * p.h_v + 7) / 8) + 16)), dim3(NT8), 0,
                           (hipStream_t)stream, p);
    }
    return launched16();
}

int launch_combine16(const Params& p, void* stream) {
    const hipStream_t s = (hipStream_t)stream;
    const dim3 block(NTC);
    const unsigned heads = (unsigned)((p.n_seqs * p.h_v + 7) / 8);
    if (p.comb_G <= 0) {
        hipLaunchKernelGGL(k_combine16, dim3(64 * heads), block, 0, s, p);
        return launched16();
    }
    const unsigned bundles = (unsigned)(((long long)p.n_seqs * p.h_v * p.comb_J + 7) / 8);
    hipLaunchKernelGGL(k_comb16_groups, dim3(128 * bundles), block, 0, s, p);
    const int e = launched16();
    if (e) return e;
    hipLaunchKernelGGL(k_comb16_apply, dim3(64 * bundles), block, 0, s, p);
    return launched16();
}

int launch_fwd16(const Params& p, int io, void* stream) {
    const unsigned s_dv = io == kIoBf16 ? (unsigned)p.dv_split : 1u;
    const dim3 grid((unsigned)p.n_segments, (unsigned)p.h_v, s_dv);
    hipStream_t hs = (hipStream_t)stream;
    if (io != kIoBf16) hipLaunchKernelGGL(k_fwd16<float>, grid, dim3(NT8), 0, hs, p);
    else if (s_dv == 1) hipLaunchKernelGGL((k_fwd_ws<4, 2>), grid, dim3(64 * 8), 0, hs, p);
    else if (s_dv == 2) hipLaunchKernelGGL((k_fwd_ws<4, 1>), grid, dim3(64 * 8), 0, hs, p);
    else if (s_dv == 4) hipLaunchKernelGGL((k_fwd_ws<2, 1>), grid, dim3(64 * 6), 0, hs, p);
    else return (int)hipErrorInvalidValue;
    return launched16();
}

int launch_tiles_to_rm(const float* src, float* dst, long long n_blocks, void* stream) {
    if (n_blocks <= 0) return 0;
    hipLaunchKernelGGL(k_tiles_to_rm, dim3((unsigned)n_blocks), dim3(64), 0, (hipStream_t)stream, src, dst);
    return launched16();
}

}  // namespace gdn
