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
// Work layout of the chain kernels. A workgroup is 8 waves (512 lanes). Wave
// w owns d_v columns [16w, 16w + 16): its 128 x 16 slice of S, its slice of
// Y / V' and of the output all stay in its registers, so the sequential state
// chain never crosses waves; two waves share each SIMD. Operands that every
// wave needs (Q, K, K^T, V^T, T, P = QK^T o D) are staged in LDS. Products use
// 16x16x32 bf16 MFMAs with fp32 accumulation. Values that are not exact bf16
// inputs (S, Y, V', T, P) enter the MFMA as a hi + lo pair of bf16 (x = hi +
// lo to about 16 bits), giving 2 or 3 MFMAs per product; diagonal gate
// factors are applied in fp32 on the accumulators instead of being rounded
// into operands.
//
// Register layouts (gfx950), 16x16x32 bf16 MFMA, lane l = 16 g + c:
//   A operand: row c, k values 8g .. 8g + 7; B operand: column c, the same k;
//   C/D: rows 4g .. 4g + 3 of column c.
// Two C tiles stacked (rows 0..15 and 16..31) hand lane group g the rows
// 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3; with the contraction axis of every
// LDS operand stored in the order kp (below), that is exactly a B (or,
// mirrored, an A) operand, so accumulator tiles feed the next product without
// shuffles. The segment combine and the 16x16 block products of the prep use
// 32x32x16 and 16x16x16 MFMAs with their own layouts, described there.
#include "gdn_device.h"

namespace gdn {
namespace {



// ----------------------------------------------------------------------------
// Chunk preparation kernel: gamma, beta and T = (I + A)^-1 of every (chunk,
// value head). Chunks are independent, so one wave solves one chunk on its
// own: its K rows come from HBM straight into MFMA operand registers, the
// gram tiles below the diagonal stay in registers as the operands of the
// block inversion, and only T (and A's diagonal blocks, for the substitution)
// pass through the wave's own LDS. No barriers; eight one-wave workgroups per
// CU. The chain kernels then read T instead of solving the triangular system
// inside their sequential loops.

// LDS of one prep wave (about 18.5 KiB: eight waves per CU).
constexpr int kPrepWaves = 8;
struct __attribute__((aligned(16))) PrepSmem {
    float t[CH * LDF];      // T = (I + A)^-1 on and below the diagonal blocks; four of the
                            // blocks above hold A's diagonal blocks (prep_ad)
    float gam[CH];
    float beta[CH];
};

// A's diagonal 16x16 block b, transposed (row m holds column m of the block,
// row stride LDF), kept in an upper block of t, which T never uses: block b
// goes to block (0, b + 1) for b < 3 and block 3 to (1, 3).
__device__ __forceinline__ float* prep_ad(PrepSmem& sm, int b) {
    return sm.t + (b == 3 ? 16 * LDF + 48 : 16 * (b + 1));
}

// Lower 16x16 tile number job (0..9) -> block row bi >= block column bj.
__device__ __forceinline__ void lower_tile(int job, int& bi, int& bj) {
    bi = (job >= 6) ? 3 : (job >= 3) ? 2 : (job >= 1) ? 1 : 0;
    bj = job - (bi * (bi + 1)) / 2;
}
__device__ __forceinline__ bf16x8 lds_row8(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

// One chunk's K rows as 16x16x32 MFMA operands: lane 16 g + n holds row
// 16 rb + n, d_k 32 ks + 8 g .. + 7 (the natural k order: both operands of the
// gram use it). bf16: loaded raw (rows past the end read the last row again,
// zeroed at use, so that the loads need no wait until then).
template <typename IO> struct PrepIn;
template <> struct PrepIn<bf16> { u32x4 k[4][4]; float g, b; int nv; };
template <> struct PrepIn<float> { float g, b; int nv; };

template <typename IO>
__device__ __forceinline__ void prep_fetch(PrepIn<IO>& r, const Params& p, size_t tok0, int nvalid, int h, int hq) {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
    if constexpr (Io<IO>::kExact) {
        const size_t ts = (size_t)p.h_qk * DK;
        const IO* kb = static_cast<const IO*>(p.k) + tok0 * ts + (size_t)hq * DK + 8 * g;
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const unsigned off = (unsigned)(min(16 * rb + n, nvalid - 1) * (int)ts);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) r.k[rb][ks] = *reinterpret_cast<const u32x4*>(kb + off + 32 * ks);
        }
    }
    const size_t idx = (tok0 + min(lane, nvalid - 1)) * (size_t)p.h_v + h;
    r.g = p.g[idx];
    r.b = p.beta[idx];
    r.nv = nvalid;
}

// The ten lower gram tiles of the chunk, each computed transposed (K rows of
// block bj against K rows of block bi): lane 16 g + n ends up with
// k_(16 bi + n) . k_(16 bj + 4 g + e), e < 4 -- row i = 16 bi + n of A, four
// consecutive columns, which is the A-operand layout of a 16x16x16 MFMA.
template <typename IO>
__device__ __forceinline__ void prep_gram(const PrepIn<IO>& r, const Params& p, size_t tok0, int hq, f32x4 acc[10]) {
    const int lane = lane_id(), n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int t = 0; t < 10; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (Io<IO>::kExact) {
        bf16x8 op[4][4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const bool ok = 16 * rb + n < r.nv;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                op[rb][ks] = __builtin_bit_cast(bf16x8, ok ? r.k[rb][ks] : u32x4{0u, 0u, 0u, 0u});
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int t = 0; t < 10; ++t) {
                int bi, bj;
                lower_tile(t, bi, bj);
                acc[t] = mma16k32(op[bj][ks], op[bi][ks], acc[t]);
            }
    } else {
        // fp32 inputs: rows loaded at use and split hi/lo (three products per k step)
        const size_t ts = (size_t)p.h_qk * DK;
        const float* kb = static_cast<const float*>(p.k) + tok0 * ts + (size_t)hq * DK + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 hi[4], lo[4];
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int row = 16 * rb + n;
                const float* src = kb + (size_t)min(row, r.nv - 1) * ts + 32 * ks;
                f32x4 x0 = *reinterpret_cast<const f32x4*>(src), x1 = *reinterpret_cast<const f32x4*>(src + 4);
                if (row >= r.nv) x0 = x1 = f32x4{0.f, 0.f, 0.f, 0.f};
                split8(x0, x1, hi[rb], lo[rb]);
            }
#pragma unroll
            for (int t = 0; t < 10; ++t) {
                int bi, bj;
                lower_tile(t, bi, bj);
                acc[t] = mma16k32(hi[bj], hi[bi], acc[t]);
                acc[t] = mma16k32(hi[bj], lo[bi], acc[t]);
                acc[t] = mma16k32(lo[bj], hi[bi], acc[t]);
            }
        }
    }
}

// Diagonal 16x16 blocks of T by forward substitution, column by column: lane
// 16 b + j solves column j of block b in registers; step m fixes x_m and
// removes its share from the rows below, reading column m of the block (one
// LDS row of the transposed block, a broadcast within the lane's block).
__device__ void prep_inv_diag(PrepSmem& sm) {
    const int lane = lane_id(), b = 16 * (lane >> 4), j = lane & 15;
    const float* ad = prep_ad(sm, lane >> 4);
    float s[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
    for (int m = 0; m < 15; ++m) {
        const float* col = ad + m * LDF;   // A[b + i][b + m] at col[i], i > m
        f32x4 c4[4];
#pragma unroll
        for (int q = (m + 1) / 4; q < 4; ++q) c4[q] = *reinterpret_cast<const f32x4*>(col + 4 * q);
#pragma unroll
        for (int i = m + 1; i < 16; ++i) s[i] = fmaf(-c4[i / 4][i % 4], s[m], s[i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.t[(b + i) * LDF + b + j] = s[i];
}

// 16x16 block products on hi/lo bf16 operands (16x16x16 MFMA; lane l: A row
// l % 16 with k 4 (l / 16) .. + 4; B and C column l % 16 with rows 4 (l / 16) .. + 4).
__device__ __forceinline__ f32x4 mm_split(const bf16x4& ah, const bf16x4& al, const f32x4& bv, f32x4 acc) {
    bf16x4 bh, bl;
    split4(bv, bh, bl);
    acc = mma16(ah, bh, acc);
    acc = mma16(ah, bl, acc);
    return mma16(al, bh, acc);
}
// ... with the A operand the LDS block at (r0, c0) of an fp32 [64][LDF] matrix
__device__ __forceinline__ f32x4 mm_lds(const float* m, int r0, int c0, const f32x4& bv, f32x4 acc) {
    const int lane = lane_id(), n = lane & 15, g4 = lane >> 4;
    bf16x4 ah, al;
    split4(*reinterpret_cast<const f32x4*>(m + (r0 + n) * LDF + c0 + 4 * g4), ah, al);
    return mm_split(ah, al, bv, acc);
}
// The LDS block at (r0, c0) in the C (B operand) layout, and back.
__device__ __forceinline__ f32x4 blk_c(const float* m, int r0, int c0) {
    const int lane = lane_id(), n = lane & 15, g4 = lane >> 4;
    f32x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = m[(r0 + 4 * g4 + r) * LDF + c0 + n];
    return v;
}
__device__ __forceinline__ void blk_store(float* m, int r0, int c0, const f32x4& v) {
    const int lane = lane_id(), n = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) m[(r0 + 4 * g4 + r) * LDF + c0 + n] = v[r];
}

// The six blocks below the diagonal by 2 x 2 block inversion of the 32-row
// halves. With P, R the inverses of the upper-left and lower-right halves:
//   T_10 = -T_11 A_10 T_00,  T_32 = -T_33 A_32 T_22,
//   X = A_bl P (X_a0 = A_a0 T_00 + A_a1 T_10, X_a1 = A_a1 T_11, a = 2, 3),
//   lower-left half = -R X (T_2j = -T_22 X_2j, T_3j = -(T_32 X_2j + T_33 X_3j)).
// A's blocks come from registers (hi/lo, tiles 1, 3, 4, 6, 7, 8 of the gram);
// T's blocks enter as A operands from LDS and as B operands in the C layout.
__device__ void prep_inv_off(PrepSmem& sm, const bf16x4 ah[10], const bf16x4 al[10]) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const f32x4 t00 = blk_c(sm.t, 0, 0), t11 = blk_c(sm.t, 16, 16), t22 = blk_c(sm.t, 32, 32);
    const f32x4 t10 = -mm_lds(sm.t, 16, 16, mm_split(ah[1], al[1], t00, z), z);
    const f32x4 t32 = -mm_lds(sm.t, 48, 48, mm_split(ah[8], al[8], t22, z), z);
    blk_store(sm.t, 16, 0, t10);
    blk_store(sm.t, 48, 32, t32);
    const f32x4 x20 = mm_split(ah[4], al[4], t10, mm_split(ah[3], al[3], t00, z));
    const f32x4 x21 = mm_split(ah[4], al[4], t11, z);
    const f32x4 x30 = mm_split(ah[7], al[7], t10, mm_split(ah[6], al[6], t00, z));
    const f32x4 x31 = mm_split(ah[7], al[7], t11, z);
    // T_32 is read back as an A operand: the wave's own stores above come first
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    blk_store(sm.t, 32, 0, -mm_lds(sm.t, 32, 32, x20, z));
    blk_store(sm.t, 32, 16, -mm_lds(sm.t, 32, 32, x21, z));
    blk_store(sm.t, 48, 0, -mm_lds(sm.t, 48, 48, x30, mm_lds(sm.t, 48, 32, x20, z)));
    blk_store(sm.t, 48, 16, -mm_lds(sm.t, 48, 48, x31, mm_lds(sm.t, 48, 32, x21, z)));
}

// Gate-driven choice for the boundary at chunk a of a sequence (the start
// of segment a / L): warm up iff the log-decay over the window of w chunks
// before the boundary is at most log(noise floor) (or the window reaches the
// sequence start, where the warm-up is exact). The warm-up then scans the
// shortest run of chunks before the boundary (wq <= w) whose log-decay is
// already at most log(noise floor); the state it misses is bounded by that
// decay times the state at the run's start. Chunk log-decays are the gate
// sums in the order of the gamma scan (the chunks before a boundary are
// whole; tok_last is the first token of chunk a - 1). Written to the
// boundary flags as class | wq << 8, class 0 (exact map), 1 (warm-up) or
// 2 (warm-up from the sequence start, exact); k_cp_prep and the combine read
// them.
__device__ void classify_boundary(const Params& p, int seq, int N, int a, int h, size_t tok_last) {
    const int lane = lane_id();
    int cls = 0, wq = p.w;
    if (p.cp_mode == kCpExact) {
        cls = 0;
    } else if (a - p.w <= 0) {
        cls = 2;
        wq = a;
    } else {
        float gl[8], sums[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)   // chunks a - 1 - j >= a - w >= 1 for j < w
            gl[j] = j < p.w ? p.g[(tok_last - (size_t)j * CH + lane) * (size_t)p.h_v + h] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            sums[j] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_scan(gl[j])), 63));
        float cum = 0.f;
        int found = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            cum += sums[j];
            if (!found && j < p.w && cum <= p.log_eps) found = j + 1;
        }
        if (found) {
            cls = 1;
            wq = found;
        } else {
            cls = (p.cp_mode == kCpWarmup) ? 1 : 0;
        }
    }
    int seg_base = 0;
    if (!p.cu) {
        seg_base = seq * n_segs_of(N, p.L);
    } else {
        for (int n = 0; n < seq; ++n) seg_base += n_segs_of(n_chunks_of(p.cu[n + 1] - p.cu[n]), p.L);
    }
    if (lane == 0) p.warm[(size_t)(seg_base + a / p.L) * p.h_v + h] = cls == 0 ? 0 : (cls | (wq << 8));
}

// Work items are (value head, chunk slot) pairs, item f = slot h_v + h (the
// value heads that share a key head are neighbours: their K rows come from
// the same cache lines);
// wave b (wave b % 8 of workgroup b / 8; the waves share nothing) walks items
// [b prep_cpw, (b + 1) prep_cpw), fetching the next item's inputs while it
// works on the current one. (Eight waves per workgroup: one-wave workgroups
// are dispatched too slowly to fill the chip at once.) Per (chunk slot,
// value head), block b = slot h_v + h:
//   prep_T + b t_stride: T diag(beta) split into bf16 hi and lo, [part][row][k]
//     (2 x 64 x 64), the k (column) axis in the kp order of the chain
//     kernels' LDS operands (zeros above the diagonal);
//   prep_GB + b gb_stride: gamma (64 fp32), then beta (64 fp32).
// With F16 the kernel writes instead, per (chunk slot, value head), the image
// tb16 + b * kTbHalfs of T diag(beta) in fp16 as the six nonzero A operands
// (16x16x32) of the product T diag(beta) Y: fragment f <-> (token tile m,
// k step j) = (0,0), (1,0), (2,0), (2,1), (3,0), (3,1); lane 16 g + c holds
// row 16 m + c at the k slots 8 g .. 8 g + 7, i.e. the columns
// 32 j + 16 (s / 4) + 4 g + s % 4 (s < 8) of the kp order, and nothing of
// gamma or beta (the chain kernels scan the gates themselves).
template <typename IO, bool F16>
__global__ __launch_bounds__(64 * kPrepWaves) void k_prep(Params p) {
    __shared__ PrepSmem sm_all[kPrepWaves];
    GDN_LDS_POISON_ALL(sm_all);
    PrepSmem& sm = sm_all[wave_id()];
    const int lane = lane_id();
    const long long n_items = (long long)p.n_chunks * p.h_v;
    const long long wv = (long long)blockIdx.x * kPrepWaves + wave_id();
    const long long f0 = wv * p.prep_cpw, f1 = min(f0 + (long long)p.prep_cpw, n_items);
    if (f0 >= f1) return;
    // item f -> head, chunk slot and the slot's tokens
    int h, slot, nvalid, seq, c, len;
    size_t tok0;
    auto locate = [&](long long f) {
        slot = (int)(f / p.h_v);
        h = (int)(f - (long long)slot * p.h_v);
        size_t tok_s;
        locate_chunk(p, slot, seq, c, len, tok_s);   // slot < n_chunks: always found
        tok0 = tok_s + (size_t)c * CH;
        nvalid = min(CH, len - c * CH);
    };
    // the last chunk before a segment boundary classifies the boundary; done
    // first, so that its loads overlap those of the first item, and outside
    // the item loop, whose memory operations then stay branch-free
    if (p.warm) {
        for (long long f = f0; f < f1; ++f) {
            locate(f);
            const int N = n_chunks_of(len);
            if ((c + 1) % p.L == 0 && c + 1 < N) classify_boundary(p, seq, N, c + 1, h, tok0);
        }
    }
    // Items come in groups of the value heads (in this wave's range) that
    // share a chunk and a key head: the gram of the group's K rows is formed
    // once (its tiles stay in registers through the group, so the next
    // group's K rows load after it). Each item's gates load one item ahead.
    float g_nx, b_nx;
    {
        locate(f0);
        const size_t idx = (tok0 + min(lane, nvalid - 1)) * (size_t)p.h_v + h;
        g_nx = p.g[idx];
        b_nx = p.beta[idx];
    }
    if (p.sink) {   // (null for the low-level entry, which has no workspace)
        // the loop body's stores (gamma, beta; T) come after its loads; the same
        // number of stores to the scratch line here make the loop's entry look
        // alike, so that the wait at its head covers the loads only
        float* sk = p.sink + 32 * lane;
        sk[0] = 0.f;
        sk[1] = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) *reinterpret_cast<u32x4*>(sk + 4 * (i & 3)) = u32x4{0u, 0u, 0u, 0u};
    }
    for (long long fg = f0; fg < f1;) {
        locate(fg);
        const int hq_cur = h / p.group, slot_cur = slot, nv_cur = nvalid;
        const size_t tok_cur = tok0;
        const long long g_end = min(f1, (long long)slot_cur * p.h_v + (long long)(hq_cur + 1) * p.group);
        PrepIn<IO> kin;
        prep_fetch<IO>(kin, p, tok_cur, nv_cur, h, hq_cur);
        f32x4 acc[10];
        kin.nv = nv_cur;
        prep_gram<IO>(kin, p, tok_cur, hq_cur, acc);
    for (long long f = fg; f < g_end; ++f) {
        const int h_cur = (int)(f - (long long)slot_cur * p.h_v);
        const float g_cur = g_nx, b_cur = b_nx;
        {
            // the next item's gates (the last item loads its own again)
            const long long fn = min(f + 1, f1 - 1);
            locate(fn);
            const size_t idx = (tok0 + min(lane, nvalid - 1)) * (size_t)p.h_v + h;
            g_nx = p.g[idx];
            b_nx = p.beta[idx];
        }
        {
            const bool ok = lane < nv_cur;
            const float gam = wave_scan(ok ? g_cur : 0.f), bt = ok ? b_cur : 0.f;
            sm.gam[lane] = gam;
            sm.beta[lane] = bt;
            if constexpr (!F16) {
                float* gb = p.prep_GB + ((size_t)slot_cur * p.h_v + h_cur) * (size_t)p.gb_stride;
                gb[lane] = gam;
                gb[CH + lane] = bt;
            } else {
                // the chain kernels' gate factors: gamma log2(e), e^gamma,
                // e^(gamma_C - gamma), e^gamma_C (padding tokens carry g = 0)
                const float gc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gam), 63));
                float* gf = p.gf16 + ((size_t)slot_cur * p.h_v + h_cur) * (size_t)kGfFloats;
                gf[lane] = gam * 1.4426950408889634f;
                gf[CH + lane] = __expf(gam);
                gf[2 * CH + lane] = __expf(gc - gam);
                gf[3 * CH + lane] = __expf(gc);
            }
        }
        // A = beta_i exp(gamma_i - gamma_j) k_i . k_j below the diagonal: the
        // off-diagonal tiles stay as hi/lo A operands, the diagonal ones go to
        // LDS transposed (prep_ad(b): position (i - 16 b, j - 16 b) holds A[j][i], j > i)
        bf16x4 ah[10], al[10];
        {
            const int n = lane & 15, g4 = lane >> 4;
#pragma unroll
            for (int t = 0; t < 10; ++t) {
                int bi, bj;
                lower_tile(t, bi, bj);
                const int i = 16 * bi + n, j0 = 16 * bj + 4 * g4;
                const float gi = sm.gam[i];
                const f32x4 gj = *reinterpret_cast<const f32x4*>(sm.gam + j0);
                f32x4 v;
                if (bi == bj) {
                    const f32x4 bj4 = *reinterpret_cast<const f32x4*>(sm.beta + j0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = (j0 + r > i) ? bj4[r] * __expf(gj[r] - gi) * acc[t][r] : 0.f;
                    *reinterpret_cast<f32x4*>(prep_ad(sm, bi) + n * LDF + 4 * g4) = v;
                } else {
                    const float bt = sm.beta[i];
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = bt * __expf(gi - gj[r]) * acc[t][r];
                    split4(v, ah[t], al[t]);
                }
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        prep_inv_diag(sm);
        // the off-diagonal blocks read the diagonal ones just written
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        prep_inv_off(sm, ah, al);
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        // T diag(beta) with its column (token) axis in kp order: lane l takes
        // rows 16 u + l / 4 and the physical 8-element pieces 32 q + 8 a,
        // q = (l / 2) % 2, a = 2 (l % 2) + (0, 1); piece 32 q + 8 a holds
        // logical columns 32 q + 4 a + (0..3) (block 2 q) and
        // 32 q + 16 + 4 a + (0..3) (block 2 q + 1). Blocks above the diagonal
        // (column block > row block u) are written as zeros, not read.
        if constexpr (F16) {
            f16* Tg = static_cast<f16*>(p.tb16) + ((size_t)slot_cur * p.h_v + h_cur) * (size_t)kTbHalfs;
            const int c = lane & 15, g = lane >> 4;
#pragma unroll
            for (int f = 0; f < 6; ++f) {
                const int m = f < 2 ? f : 2 + ((f - 2) >> 1), j = f < 2 ? 0 : ((f - 2) & 1);
                const int r = 16 * m + c, x0 = 32 * j + 4 * g, x1 = x0 + 16;
                const f32x4 t0 = *reinterpret_cast<const f32x4*>(sm.t + r * LDF + x0);
                const f32x4 t1 = *reinterpret_cast<const f32x4*>(sm.t + r * LDF + x1);
                const f32x4 b0 = *reinterpret_cast<const f32x4*>(sm.beta + x0);
                const f32x4 b1 = *reinterpret_cast<const f32x4*>(sm.beta + x1);
                f32x4 v0, v1;
#pragma unroll
                for (int e = 0; e < 4; ++e) {   // T is lower triangular; its upper blocks hold other data
                    v0[e] = (x0 + e <= r) ? t0[e] * b0[e] : 0.f;
                    v1[e] = (x1 + e <= r) ? t1[e] * b1[e] : 0.f;
                }
                *reinterpret_cast<f16x8*>(Tg + (f * 64 + lane) * 8) = pack8h(v0, v1);
            }
            continue;
        }
        bf16* Tg = reinterpret_cast<bf16*>(p.prep_T + ((size_t)slot_cur * p.h_v + h_cur) * (size_t)p.t_stride);
        {
            const int q = (lane >> 1) & 1;
            f32x4 bcol[4];
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2) {
                const int l0 = 32 * q + 4 * (2 * (lane & 1) + a2);
                bcol[2 * a2] = *reinterpret_cast<const f32x4*>(sm.beta + l0);
                bcol[2 * a2 + 1] = *reinterpret_cast<const f32x4*>(sm.beta + l0 + 16);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int row = 16 * u + (lane >> 2);
#pragma unroll
                for (int a2 = 0; a2 < 2; ++a2) {
                    const int a = 2 * (lane & 1) + a2, l0 = 32 * q + 4 * a, l1 = l0 + 16;
                    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    const f32x4 x0 = 2 * q <= u ? *reinterpret_cast<const f32x4*>(sm.t + row * LDF + l0) * bcol[2 * a2] : z;
                    const f32x4 x1 = 2 * q + 1 <= u ? *reinterpret_cast<const f32x4*>(sm.t + row * LDF + l1) * bcol[2 * a2 + 1] : z;
                    bf16x8 hi, lo;
                    split8(x0, x1, hi, lo);
                    *reinterpret_cast<bf16x8*>(Tg + row * CH + 32 * q + 8 * a) = hi;
                    *reinterpret_cast<bf16x8*>(Tg + (CH + row) * CH + 32 * q + 8 * a) = lo;
                }
            }
        }
    }
        fg = g_end;
    }
}

// ----------------------------------------------------------------------------
// The chain kernels. For a chunk with incoming state S, the same quantities as
// the WY form, evaluated without W and U:
//   Y  = V - diag(e^gamma) K S                    (the prediction error)
//   V' = T diag(beta) Y                           (= U - W S)
//   O  = diag(e^gamma) Q S + P V',  P = (Q K^T) o D  (both times the scale)
//   S <- e^gamma_C S + K^T diag(e^(gamma_C - gamma)) V'
// Every product keeps the d_v columns apart, so a workgroup of 8 waves gives
// wave w the columns [16w, 16w + 16): its 128 x 16 slice of S, its slices of
// Y, V' and the output stay in its registers, and the state chain never
// crosses waves. Two waves share each SIMD, so one wave's splits and scalings
// run while the other's MFMAs do. Operands that every wave needs (K, K^T, V^T,
// Q, T, P) are staged in LDS.
//
// 16x16x32 bf16 MFMA, lane l = 16 g + c: A row c, B column c, each with the
// eight k values 8g .. 8g + 7; C/D rows 4g .. 4g + 3 of column c. Two C tiles
// stacked (rows 0..15 and 16..31) therefore hand lane group g the rows
// 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3: that is the k order of a B (or,
// mirrored, an A) operand once the contraction axis of every LDS operand is
// stored in the order kp below, and accumulator tiles feed the next product
// without any shuffle.


template <bool EX>
struct __attribute__((aligned(16))) ChainSmem {
    // What the state update reads (K^T and its gate factors) comes in NB
    // buffers: with two (bf16 inputs), the next chunk is staged while the
    // current one finishes its state update, and a chunk takes two barriers
    // instead of three. fp32 inputs need the LDS for the lo halves instead.
    static constexpr int NB = EX ? 2 : 1;
    bf16 k_hi[CH * LDQ];                  // K token-major, d_k in kp order
    bf16 k_lo[EX ? 8 : CH * LDQ];
    bf16 q_hi[CH * LDQ];                  // Q token-major, d_k in kp order
    bf16 q_lo[EX ? 8 : CH * LDQ];
    bf16 kt_hi[NB][DK * LDKT];            // K^T: row d_k, tokens in kp order (chunks swizzled)
    bf16 kt_lo[EX ? 8 : DK * LDKT];
    bf16 vt[EX ? DK * LDKT : 8];          // V^T: row d_v, tokens in order (chunks swizzled)
    bf16 t[2 * CH * LDP];                 // T diag(beta): hi rows, then lo rows; tokens in kp order
    bf16 p[2 * CH * LDP];                 // P: hi rows, then lo rows; columns in kp order
    float gam[CH];                        // gamma
    float eg[CH];                         // exp(gamma)
    float egs[CH];                        // scale exp(gamma)
    float egc[NB][CH];                    // exp(gamma_C - gamma)
    float ec[NB];                         // exp(gamma_C)
    float red[8];                         // per-chunk gate sums (boundary choice)
};

// One chunk's inputs in registers between the global loads and the LDS
// stores, so that the next chunk's loads overlap the current chunk's work.
// K, V, Q: thread t holds tokens 4 (t / 32) + j (j < 4), columns
// 4 (t % 32) .. + 4 (32 lanes cover one 256-byte row, and a lane holds four
// consecutive tokens of each of its columns, written to K^T / V^T as 8-byte
// stores). T: pieces t and t + 512 of its [part][row][64] image (16 bytes
// each). Gates: gamma, beta of token lane.
template <typename IO> struct Chunk;
template <> struct Chunk<bf16> { u32x2 k[4], v[4], q[4]; u32x4 t[2]; float gl, bl; };
template <> struct Chunk<float> { f32x4 k[4], q[4]; u32x4 t[2]; float gl, bl; };

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
    const int t = threadIdx.x, m = t >> 5, c4 = (t & 31) * 4;
    const int ts = p.h_qk * DK, tsv = p.h_v * DK;
    const IO* kb = static_cast<const IO*>(p.k) + tok0 * (size_t)ts + (size_t)hq * DK;
    const IO* qb = static_cast<const IO*>(p.q) + tok0 * (size_t)ts + (size_t)hq * DK;
    const IO* vb = static_cast<const IO*>(p.v) + tok0 * (size_t)tsv + (size_t)h * DK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = min(4 * m + j, nvalid - 1);
        const unsigned ok = (unsigned)(row * ts + c4), ov = (unsigned)(row * tsv + c4);
        if constexpr (EX) {
            r.k[j] = *reinterpret_cast<const u32x2*>(kb + ok);
            if (WANT_V) r.v[j] = *reinterpret_cast<const u32x2*>(vb + ov);
            if (WANT_Q) r.q[j] = *reinterpret_cast<const u32x2*>(qb + ok);
        } else {
            r.k[j] = *reinterpret_cast<const f32x4*>(kb + ok);
            if (WANT_Q) r.q[j] = *reinterpret_cast<const f32x4*>(qb + ok);
        }
    }
    const size_t blk = (size_t)slot * p.h_v + h;
    const u32x4* Tg = reinterpret_cast<const u32x4*>(p.prep_T + blk * (size_t)p.t_stride);
#pragma unroll
    for (int j = 0; j < 2; ++j) r.t[j] = Tg[t + NTHR_CH * j];
    const float* gb = p.prep_GB + blk * (size_t)p.gb_stride;
    r.gl = gb[lane_id()];
    r.bl = gb[CH + lane_id()];
}

// Element e (0..3) of four bf16 rows, packed two tokens to a 32-bit word.
__device__ __forceinline__ u32x2 pack_col4(const u32x2 (&a)[4], int e) {
    const int w = e >> 1, sh = 16 * (e & 1);
    const unsigned x0 = (a[0][w] >> sh) & 0xffffu, x1 = (a[1][w] >> sh) & 0xffffu;
    const unsigned x2 = (a[2][w] >> sh) & 0xffffu, x3 = (a[3][w] >> sh) & 0xffffu;
    return u32x2{x0 | (x1 << 16), x2 | (x3 << 16)};
}

// Writes a fetched chunk to LDS: K token-major and transposed (four
// consecutive tokens of a column per 8-byte store), V^T, Q, T and the gate
// factors (tokens past the end of the sequence have g = beta = 0).
template <typename IO, bool WANT_Q, bool WANT_V>
__device__ __forceinline__ void stage_chunk(ChainSmem<Io<IO>::kExact>& sm, const Chunk<IO>& r, float scale,
                                            int b) {
    constexpr bool EX = Io<IO>::kExact;
    const int t = threadIdx.x, lane = lane_id(), m = t >> 5, c4 = (t & 31) * 4;
    if (wave_id() == 0) {   // the gate factors: one wave (a scalar branch)
        const float gc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r.gl), 63));
        const float es = __expf(r.gl);
        sm.gam[lane] = r.gl;
        sm.eg[lane] = es;
        sm.egs[lane] = es * scale;
        sm.egc[b][lane] = __expf(gc - r.gl);
        sm.ec[b] = __expf(gc);
    }
    const int kc = kp(c4), tk = kp(4 * m) ^ tswz(c4), tv = (4 * m) ^ tswz(c4);
    if constexpr (EX) {
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(sm.k_hi + (4 * m + j) * LDQ + kc) = r.k[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            *reinterpret_cast<u32x2*>(sm.kt_hi[b] + (c4 + e) * LDKT + tk) = pack_col4(r.k, e);
            if (WANT_V) *reinterpret_cast<u32x2*>(sm.vt + (c4 + e) * LDKT + tv) = pack_col4(r.v, e);
        }
        if (WANT_Q) {
#pragma unroll
            for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(sm.q_hi + (4 * m + j) * LDQ + kc) = r.q[j];
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x4 hi, lo;
            split4(r.k[j], hi, lo);
            *reinterpret_cast<bf16x4*>(sm.k_hi + (4 * m + j) * LDQ + kc) = hi;
            *reinterpret_cast<bf16x4*>(sm.k_lo + (4 * m + j) * LDQ + kc) = lo;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x4 x = {r.k[0][e], r.k[1][e], r.k[2][e], r.k[3][e]};
            bf16x4 hi, lo;
            split4(x, hi, lo);
            *reinterpret_cast<bf16x4*>(sm.kt_hi[b] + (c4 + e) * LDKT + tk) = hi;
            *reinterpret_cast<bf16x4*>(sm.kt_lo + (c4 + e) * LDKT + tk) = lo;
        }
        if (WANT_Q) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x4 hi, lo;
                split4(r.q[j], hi, lo);
                *reinterpret_cast<bf16x4*>(sm.q_hi + (4 * m + j) * LDQ + kc) = hi;
                *reinterpret_cast<bf16x4*>(sm.q_lo + (4 * m + j) * LDQ + kc) = lo;
            }
        }
    }
    // T: piece t + 512 j of the [part][row][64] image -> row part * 64 + row of sm.t
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int pc = t + NTHR_CH * j, prow = pc >> 3, k8 = (pc & 7) * 8;
        *reinterpret_cast<u32x4*>(sm.t + prow * LDP + k8) = r.t[j];
    }
}

// One tile of scale P, P = (Q K^T) o D: the lower 16x16 tile `job` (0..9),
// computed transposed (K rows against Q rows) so that a lane ends up with four
// consecutive columns of one row of P, stored split into hi/lo. The two upper
// tiles inside the diagonal 32-blocks, which the P V' product reads, stay zero
// (cleared once per kernel).
template <bool EX>
__device__ __forceinline__ void gram_tile(ChainSmem<EX>& sm, int job, float scale) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    int ri, ii;
    lower_tile(job, ri, ii);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int kb = 32 * s + 8 * g;
        const bf16x8 a = lds_row8(sm.k_hi + (16 * ii + c) * LDQ + kb);
        const bf16x8 b = lds_row8(sm.q_hi + (16 * ri + c) * LDQ + kb);
        acc = mma16k32(a, b, acc);
        if (!EX) {
            acc = mma16k32(a, lds_row8(sm.q_lo + (16 * ri + c) * LDQ + kb), acc);
            acc = mma16k32(lds_row8(sm.k_lo + (16 * ii + c) * LDQ + kb), b, acc);
        }
    }
    const int r = 16 * ri + c, i0 = 16 * ii + 4 * g;   // row r of P, columns i0 .. i0 + 3
    const float gr = sm.gam[r];
    const f32x4 gi = *reinterpret_cast<const f32x4*>(sm.gam + i0);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (i0 + e <= r) ? scale * __expf(gr - gi[e]) * acc[e] : 0.f;
    bf16x4 hi, lo;
    split4(v, hi, lo);
    *reinterpret_cast<bf16x4*>(sm.p + r * LDP + kp(i0)) = hi;
    *reinterpret_cast<bf16x4*>(sm.p + (CH + r) * LDP + kp(i0)) = lo;
}

// The P tiles of a chunk: one per wave, waves 0 and 1 take a second.
template <bool EX>
__device__ __forceinline__ void gram_p(ChainSmem<EX>& sm, float scale) {
    const int w = wave_id();
    gram_tile<EX>(sm, w, scale);
    if (w < 2) gram_tile<EX>(sm, NW_CH + w, scale);
}

// The state as hi/lo B operands, one pair per 32-row k step.
struct SplitS {
    bf16x8 hi[4], lo[4];
};
__device__ __forceinline__ void split_state(const f32x4 S[8], SplitS& ss) {
#pragma unroll
    for (int s = 0; s < 4; ++s) split8(S[2 * s], S[2 * s + 1], ss.hi[s], ss.lo[s]);
}

// V' = T diag(beta) (V - diag(e^gamma) K S) for this wave's columns.
// KS: A = K rows (token-major LDS), B = S; Y in fp32 on the accumulators
// (V from V^T in LDS, four consecutive tokens per 8-byte read, or from HBM
// for fp32 inputs); then (T diag(beta)) Y with both split hi/lo (T is lower
// triangular: token tiles 0 and 1 need k step 0 only).
template <typename IO, bool WANT_V>
__device__ void chain_vp(const ChainSmem<Io<IO>::kExact>& sm, const SplitS& ss, const IO* vcol, size_t ts,
                         int nvalid, f32x4 Vp[4], f32x4* Yout = nullptr) {
    constexpr bool EX = Io<IO>::kExact;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, n = 16 * wave_id() + c;
    f32x4 KS[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) KS[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x8 kh[4], kl[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            kh[rt] = lds_op16(sm.k_hi + (16 * rt + c) * LDQ + 32 * s + 8 * g);
            if (!EX) kl[rt] = lds_op16(sm.k_lo + (16 * rt + c) * LDQ + 32 * s + 8 * g);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) KS[rt] = mma16k32(kh[rt], ss.hi[s], KS[rt]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) KS[rt] = mma16k32(kh[rt], ss.lo[s], KS[rt]);
        if (!EX) {
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) KS[rt] = mma16k32(kl[rt], ss.hi[s], KS[rt]);
        }
    }
    // Y = V - e^gamma KS on rows 16 rt + 4 g + (0..3)
    const int vrow = n * LDKT, sw = tswz(n);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
        const int r0 = 16 * rt + 4 * g;
        const f32x4 eg = *reinterpret_cast<const f32x4*>(sm.eg + r0);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (WANT_V) {
            if constexpr (EX) {
                const u32x2 vv = *reinterpret_cast<const u32x2*>(sm.vt + vrow + (r0 ^ sw));
                v = f32x4{__uint_as_float(vv[0] << 16), __uint_as_float(vv[0] & 0xffff0000u),
                          __uint_as_float(vv[1] << 16), __uint_as_float(vv[1] & 0xffff0000u)};
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = (r0 + e < nvalid) ? (float)vcol[(size_t)(r0 + e) * ts] : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) KS[rt][e] = fmaf(-eg[e], KS[rt][e], v[e]);
        if (Yout) Yout[rt] = KS[rt];
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) Vp[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        bf16x8 yh, yl;
        split8(KS[2 * s], KS[2 * s + 1], yh, yl);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (s == 1 && rt < 2) continue;
            const bf16x8 th = lds_op16(sm.t + (16 * rt + c) * LDP + 32 * s + 8 * g);
            const bf16x8 tl = lds_op16(sm.t + (CH + 16 * rt + c) * LDP + 32 * s + 8 * g);
            Vp[rt] = mma16k32(th, yh, Vp[rt]);
            Vp[rt] = mma16k32(th, yl, Vp[rt]);
            Vp[rt] = mma16k32(tl, yh, Vp[rt]);
        }
    }
}

// O^T = scale S^T (diag(e^gamma) Q)^T for this wave's d_v rows (token columns):
// the split state serves as the A operand unchanged (the MFMA's A and B
// register layouts mirror each other). Then (chain_pv_out, after P is in
// LDS) the causal part V'^T P^T and the store: a lane holds four consecutive
// d_v of one token per tile, written as one 8- (bf16) or 16-byte (fp32)
// store.
template <bool EX>
__device__ void chain_qs(const ChainSmem<EX>& sm, const SplitS& ss, f32x4 O[4]) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) O[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x8 qh[4], ql[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            qh[ct] = lds_op16(sm.q_hi + (16 * ct + c) * LDQ + 32 * s + 8 * g);
            if (!EX) ql[ct] = lds_op16(sm.q_lo + (16 * ct + c) * LDQ + 32 * s + 8 * g);
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) O[ct] = mma16k32(ss.hi[s], qh[ct], O[ct]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) O[ct] = mma16k32(ss.lo[s], qh[ct], O[ct]);
        if (!EX) {
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) O[ct] = mma16k32(ss.hi[s], ql[ct], O[ct]);
        }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) O[ct] *= sm.egs[16 * ct + c];
}

template <typename IO>
__device__ void chain_pv_out(const ChainSmem<Io<IO>::kExact>& sm, const f32x4 Vp[4], f32x4 O[4], IO* orow0,
                             size_t ts, int nvalid, float* sink) {
    constexpr bool EX = Io<IO>::kExact;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, w = wave_id();
#pragma unroll
    for (int s = 0; s < 2; ++s) {  // P is causal: token tiles 0 and 1 need k step 0 only
        bf16x8 vh, vl;
        split8(Vp[2 * s], Vp[2 * s + 1], vh, vl);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            if (s == 1 && ct < 2) continue;
            const bf16x8 ph = lds_op16(sm.p + (16 * ct + c) * LDP + 32 * s + 8 * g);
            const bf16x8 pl = lds_op16(sm.p + (CH + 16 * ct + c) * LDP + 32 * s + 8 * g);
            O[ct] = mma16k32(vh, ph, O[ct]);
            O[ct] = mma16k32(vl, ph, O[ct]);
            O[ct] = mma16k32(vh, pl, O[ct]);
        }
    }
    // rows past the end of the sequence are written to a scratch line (every
    // chunk issues the same stores; see fetch_chunk)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
        const int r = 16 * ct + c;
        IO* dst = (r < nvalid) ? orow0 + (size_t)r * ts + 16 * w + 4 * g : reinterpret_cast<IO*>(sink + 32 * lane);
        if constexpr (EX) {
            *reinterpret_cast<u32x2*>(dst) = u32x2{pack_rne(O[ct][0], O[ct][1]), pack_rne(O[ct][2], O[ct][3])};
        } else {
            *reinterpret_cast<f32x4*>(dst) = O[ct];
        }
    }
}

// S <- e^gamma_C S + K^T diag(e^(gamma_C - gamma)) V' (Vp is scaled in place).
template <bool EX>
__device__ void chain_state(const ChainSmem<EX>& sm, f32x4 S[8], f32x4 Vp[4], int b) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) Vp[rt] *= *reinterpret_cast<const f32x4*>(sm.egc[b] + 16 * rt + 4 * g);
    const float ec = sm.ec[b];
#pragma unroll
    for (int i = 0; i < 8; ++i) S[i] *= ec;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        bf16x8 vh, vl;
        split8(Vp[2 * s], Vp[2 * s + 1], vh, vl);
        bf16x8 kh[8], kl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int off = (16 * i + c) * LDKT + ((32 * s + 8 * g) ^ (8 * i));
            kh[i] = lds_op16(sm.kt_hi[b] + off);
            if (!EX) kl[i] = lds_op16(sm.kt_lo + off);
        }
        // eight independent chains: each tile is touched once per pass
#pragma unroll
        for (int i = 0; i < 8; ++i) S[i] = mma16k32(kh[i], vh, S[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) S[i] = mma16k32(kh[i], vl, S[i]);
        if (!EX) {
#pragma unroll
            for (int i = 0; i < 8; ++i) S[i] = mma16k32(kl[i], vh, S[i]);
        }
    }
}

// ----------------------------------------------------------------------------
// State tiles in registers: wave w holds columns [16w, 16w + 16) of a
// [128][128] row-major fp32 matrix as eight 16-row accumulator tiles (tile i,
// lane 16 g + c: rows 16 i + 4 g + (0..3), column 16 w + c).

__device__ void load_state(const float* Sg, f32x4 S[8]) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, col = 16 * wave_id() + c;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[i][e] = Sg[(16 * i + 4 * g + e) * DK + col];
}
__device__ void store_state(float* Sg, const f32x4 S[8]) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, col = 16 * wave_id() + c;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) Sg[(16 * i + 4 * g + e) * DK + col] = S[i][e];
}
__device__ void zero_state(f32x4 S[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}
__device__ void identity_state(f32x4 S[8]) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, col = 16 * wave_id() + c;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) S[i][e] = (16 * i + 4 * g + e == col) ? 1.f : 0.f;
}

__device__ __forceinline__ size_t state_off(int idx, int h_v, int h) {
    return ((size_t)idx * h_v + h) * (size_t)DK * DK;
}

// Runs chunks [c_lo, c_hi) of sequence loc from the state S (no outputs):
// the warm-up scan, the H chain (WANT_V) or the M chain (V = 0, S starts at I).
// With two K^T buffers a chunk is: V' from the staged chunk | barrier | stage
// the next chunk (other K^T buffer), fetch the one after, state update |
// barrier. Every iteration issues the same loads (the last ones fetch the
// last chunk again): see fetch_chunk.
template <typename IO, bool WANT_V>
__device__ void scan_chunks(ChainSmem<Io<IO>::kExact>& sm, const Params& p, const SegLoc& loc, int h, int hq,
                            int c_lo, int c_hi, f32x4 S[8]) {
    constexpr bool EX = Io<IO>::kExact;
    constexpr bool DB = ChainSmem<EX>::NB == 2;
    if (c_lo >= c_hi) return;
    const size_t ts_v = (size_t)p.h_v * DK;
    Chunk<IO> nxt;
    auto fetch = [&](int c) {
        c = min(c, c_hi - 1);
        fetch_chunk<IO, false, WANT_V>(nxt, p, loc.tok0 + (size_t)c * CH, min(CH, loc.len - c * CH), h, hq,
                                       loc.chunk_base + c);
    };
    auto chunk_vp = [&](int c, f32x4 Vp[4]) {
        const size_t tok0 = loc.tok0 + (size_t)c * CH;
        SplitS ss;
        split_state(S, ss);
        const IO* vcol = static_cast<const IO*>(p.v) + tok0 * ts_v + (size_t)h * DK + 16 * wave_id() + (lane_id() & 15);
        chain_vp<IO, WANT_V>(sm, ss, vcol, ts_v, min(CH, loc.len - c * CH), Vp);
    };
    fetch(c_lo);
    if constexpr (DB) {
        stage_chunk<IO, false, WANT_V>(sm, nxt, 1.f, 0);
        fetch(c_lo + 1);
        __syncthreads();
        for (int c = c_lo; c < c_hi; ++c) {
            const int b = (c - c_lo) & 1;
            f32x4 Vp[4];
            chunk_vp(c, Vp);
            __syncthreads();
            stage_chunk<IO, false, WANT_V>(sm, nxt, 1.f, b ^ 1);
            fetch(c + 2);
            chain_state<EX>(sm, S, Vp, b);
            __syncthreads();
        }
    } else {
        for (int c = c_lo; c < c_hi; ++c) {
            stage_chunk<IO, false, WANT_V>(sm, nxt, 1.f, 0);
            __syncthreads();
            fetch(c + 1);
            f32x4 Vp[4];
            chunk_vp(c, Vp);
            chain_state<EX>(sm, S, Vp, 0);
            __syncthreads();
        }
    }
}

// ----------------------------------------------------------------------------
// Kernels

// Low-level chunk preparation, second half: W = (T diag(beta)) diag(e^gamma) K
// and U = (T diag(beta)) V of every (chunk, value head), from T diag(beta)
// (split) and gamma, beta, which k_prep left in the chunk's W_out and U_out
// blocks. Wave w produces columns [16w, 16w + 16) of both.
template <typename IO>
__global__ __launch_bounds__(NTHR_CH) void k_wu(Params p) {
    constexpr bool EX = Io<IO>::kExact;
    __shared__ ChainSmem<EX> sm;
    GDN_LDS_POISON_ALL(sm);
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
        stage_chunk<IO, false, true>(sm, r, 1.f, 0);
        gl = r.gl;
    }
    __syncthreads();   // every read of T, gamma and beta is done before W and U overwrite them
    const int lane = lane_id(), cc = lane & 15, g = lane >> 4, w = wave_id(), n = 16 * w + cc;
    const size_t ts_v = (size_t)p.h_v * DK, ts_k = (size_t)p.h_qk * DK;
    const IO* vcol = static_cast<const IO*>(p.v) + tok0 * ts_v + (size_t)h * DK + n;
    const IO* kcol = static_cast<const IO*>(p.k) + tok0 * ts_k + (size_t)hq * DK + n;
    f32x4 W[4], U[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) W[rt] = U[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        // B operands: column n, tokens t0 + (0..3) and t1 + (0..3) (K scaled by e^gamma of the token)
        const int t0 = 32 * s + 4 * g, t1 = t0 + 16;
        f32x4 k0, k1, v0, v1;
        if constexpr (EX) {
            const bf16x8 kh = lds_op16(sm.kt_hi[0] + n * LDKT + ((32 * s + 8 * g) ^ tswz(n)));
            const u32x2 va = *reinterpret_cast<const u32x2*>(sm.vt + n * LDKT + (t0 ^ tswz(n)));
            const u32x2 vb = *reinterpret_cast<const u32x2*>(sm.vt + n * LDKT + (t1 ^ tswz(n)));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                k0[e] = (float)kh[e];
                k1[e] = (float)kh[4 + e];
            }
            v0 = f32x4{__uint_as_float(va[0] << 16), __uint_as_float(va[0] & 0xffff0000u),
                       __uint_as_float(va[1] << 16), __uint_as_float(va[1] & 0xffff0000u)};
            v1 = f32x4{__uint_as_float(vb[0] << 16), __uint_as_float(vb[0] & 0xffff0000u),
                       __uint_as_float(vb[1] << 16), __uint_as_float(vb[1] & 0xffff0000u)};
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                k0[e] = t0 + e < nvalid ? (float)kcol[(size_t)(t0 + e) * ts_k] : 0.f;
                k1[e] = t1 + e < nvalid ? (float)kcol[(size_t)(t1 + e) * ts_k] : 0.f;
                v0[e] = t0 + e < nvalid ? (float)vcol[(size_t)(t0 + e) * ts_v] : 0.f;
                v1[e] = t1 + e < nvalid ? (float)vcol[(size_t)(t1 + e) * ts_v] : 0.f;
            }
        }
        k0 *= *reinterpret_cast<const f32x4*>(sm.eg + t0);
        k1 *= *reinterpret_cast<const f32x4*>(sm.eg + t1);
        bf16x8 kbh, kbl, vbh, vbl;
        split8(k0, k1, kbh, kbl);
        split8(v0, v1, vbh, vbl);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            if (s == 1 && rt < 2) continue;
            const bf16x8 th = lds_op16(sm.t + (16 * rt + cc) * LDP + 32 * s + 8 * g);
            const bf16x8 tl = lds_op16(sm.t + (CH + 16 * rt + cc) * LDP + 32 * s + 8 * g);
            W[rt] = mma16k32(th, kbh, W[rt]);
            W[rt] = mma16k32(th, kbl, W[rt]);
            W[rt] = mma16k32(tl, kbh, W[rt]);
            U[rt] = mma16k32(th, vbh, U[rt]);
            U[rt] = mma16k32(th, vbl, U[rt]);
            U[rt] = mma16k32(tl, vbh, U[rt]);
        }
    }
    const size_t base = ((size_t)blockIdx.x * p.h_v + h) * CH;
    if (w == 0) p.prep_gamma[base + lane] = gl;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t r = base + 16 * rt + 4 * g + e;
            p.prep_W[r * DK + n] = W[rt][e];
            p.prep_U[r * DK + n] = U[rt][e];
        }
}

// The map M of a segment, written for the combine kernel: split into hi/lo
// bf16 and laid out as that kernel's MFMA A operands (32x32x16), so that its
// loads are contiguous and it does no splitting on its sequential path.
// Element M[r][k] goes to ((((r / 32) * 8 + k / 16) * 2 + part) * 64 + lane) * 8 + e
// with lane = r % 32 + 32 h, k % 16 = kperm(h, e), part 0 = hi, 1 = lo
// (64 KiB per map). The chunk loop's LDS serves as the staging buffer; the
// caller's chain is finished (behind a barrier) when this starts.
__device__ void store_m_operand(bf16* buf, const f32x4 S[8], bf16* dst) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4, w = wave_id();
    // column k = 16 w + c: k step w, k % 16 = c
    const int hh = (c >> 2) & 1, e = (c & 3) | ((c & 8) >> 1);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = 16 * i + 4 * g + q;
            const int idx = ((((r >> 5) * 8 + w) * 2) * 64 + (r & 31) + 32 * hh) * 8 + e;
            bf16 hi, lo;
            split1(S[i][q], hi, lo);
            buf[idx] = hi;
            buf[idx + 64 * 8] = lo;
        }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
        const int off = (threadIdx.x + NTHR_CH * it) * 8;
        *reinterpret_cast<u32x4*>(dst + off) = *reinterpret_cast<const u32x4*>(buf + off);
    }
}

// Class of boundary pair q = slot h_v + head from the flags k_prep wrote:
// -1 (no boundary: a sequence's first segment), 0 exact, 1 or 2 warm-up
// (window length in bits 8 and up).
__device__ __forceinline__ int pair_class(const Params& p, int q, int& wq) {
    const SegLoc loc = locate_segment(p, q / p.h_v);
    const int v = p.warm[q];
    wq = v >> 8;
    return (loc.seq < 0 || loc.s == 0) ? -1 : (v & 255);
}

// Block-wide exclusive prefix sum of one int per thread (512 threads).
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
    for (int i = 0; i < NW_CH; ++i) {
        const int r = red[i];
        if (i < w) off += r;
        total += r;
    }
    return off + v - x;
}

// Warm-up or exact segment map for one boundary. The grid has a workgroup
// for every (segment slot, part, head); part 0: the warm-up state or H,
// part 1: M. Which boundaries need the long exact chains shows only on the
// device (k_prep classifies them from the gates). The plan picks the order
// in which the workgroups take the items:
//   exact first (cp_order 1, when the exact chains should fit in about one
//   round): every workgroup ranks the boundary flags (one load each), then
//   workgroup i < 2 E takes part i % 2 of the (i / 2)-th exact boundary (E of
//   them), the next ones the warm-up boundaries (part 0 only), and the rest
//   exit; workgroups start in index order, so no exact chain waits behind
//   warm-ups, whatever heads they belong to;
//   head-major (cp_order 0): workgroup i takes head i / (2 n_segments), then
//   slot and part, which spreads the short warm-ups among the rounds of exact
//   chains.
// Boundaries are enumerated as q = slot h_v + head.
// One (segment slot, part, head) item of k_cp_prep.
template <typename IO>
__device__ void cp_prep_item(const Params& p, ChainSmem<Io<IO>::kExact>& sm, int slot, int part, int h) {
    const int hq = h / p.group;
    const SegLoc loc = locate_segment(p, slot);
    int wq;
    const int warm = pair_class(p, slot * p.h_v + h, wq);
    if (warm < 0) return;
    const int a = loc.s * p.L;  // first chunk of segment s
    if (warm && part == 1) return;
    // the map of segment 0 is only applied to a nonzero initial state
    if (!warm && part == 1 && loc.s == 1 && !p.s_init) return;

    f32x4 S[8];
    if (warm || part == 0) {
        // the warm-up state (from the sequence's initial state where the window
        // starts there), or H: the previous segment run from zero
        const int c_lo = warm ? a - wq : a - p.L;
        if (warm && c_lo == 0 && p.s_init) load_state(p.s_init + state_off(loc.seq, p.h_v, h), S);
        else zero_state(S);
        scan_chunks<IO, true>(sm, p, loc, h, hq, c_lo, a, S);
        store_state(warm ? p.seg_state + state_off(loc.seg_base + loc.s, p.h_v, h)
                         : p.seg_H + state_off(loc.seg_base + loc.s - 1, p.h_v, h), S);
    } else {
        identity_state(S);
        scan_chunks<IO, false>(sm, p, loc, h, hq, a - p.L, a, S);
        store_m_operand(reinterpret_cast<bf16*>(&sm), S,
                        reinterpret_cast<bf16*>(p.seg_M + state_off(loc.seg_base + loc.s - 1, p.h_v, h)));
    }
}

template <typename IO>
__global__ __launch_bounds__(NTHR_CH) void k_cp_prep(Params p) {
    __shared__ ChainSmem<Io<IO>::kExact> sm;
    __shared__ int rank_red[2 * NW_CH + 4];
    GDN_LDS_POISON_ALL(sm, rank_red);
    const int i = (int)blockIdx.x;
    if (!p.cp_order) {   // head-major order
        cp_prep_item<IO>(p, sm, (i % (2 * p.n_segments)) >> 1, i & 1, i / (2 * p.n_segments));
        return;
    }
    const int n_pairs = p.n_segments * p.h_v;
    const int per = (n_pairs + NTHR_CH - 1) / NTHR_CH, q0 = threadIdx.x * per, q1 = min(q0 + per, n_pairs);
    int n_ex = 0, n_wu = 0;
    for (int q = q0; q < q1; ++q) {
        int wq;
        const int c = pair_class(p, q, wq);
        n_ex += c == 0;
        n_wu += c > 0;
    }
    if (threadIdx.x == 0) rank_red[2 * NW_CH] = -1;   // (ordered before its use by the scans' barriers)
    int tot_ex, tot_wu;
    const int pre_ex = block_excl_scan(n_ex, rank_red, tot_ex);
    const int pre_wu = block_excl_scan(n_wu, rank_red + NW_CH, tot_wu);
    const bool want_ex = i < 2 * tot_ex;
    const int r = want_ex ? i >> 1 : i - 2 * tot_ex;
    if (!want_ex && r >= tot_wu) return;   // (uniform: every thread has the totals)
    // the thread whose range holds rank r of the wanted class names the boundary
    const int pre = want_ex ? pre_ex : pre_wu, cnt = want_ex ? n_ex : n_wu;
    if (r >= pre && r < pre + cnt) {
        int k = pre;
        for (int q = q0; q < q1; ++q) {
            int wq;
            const int c = pair_class(p, q, wq);
            if (want_ex ? c == 0 : c > 0) {
                if (k == r) {
                    rank_red[2 * NW_CH] = q;
                    break;
                }
                ++k;
            }
        }
    }
    __syncthreads();
    const int q = rank_red[2 * NW_CH];
    if (q < 0 || q >= n_pairs) return;   // (cannot happen: the ranks partition the boundaries)
    cp_prep_item<IO>(p, sm, q / p.h_v, want_ex ? (i & 1) : 0, q % p.h_v);
}

// Chains over the segment boundaries of one (sequence, head, 32-column
// block). Boundary s (1 <= s < P) maps S0(s - 1) to S0(s): an exact boundary
// applies the previous segment's map, S0(s) = M_{s-1} S0(s-1) + H_{s-1} (M_0
// only to a nonzero initial state); a warm-up boundary takes its warm-up
// state. Wave w computes rows [32w, 32w + 32). Each step is one
// 128 x 32 x 128 product on hi/lo operands. M arrives split and in A-operand
// order (contiguous loads, requested two steps ahead); each lane writes the
// split of its rows of the new state straight into the B-operand slots of the
// next step (its accumulator rows are exactly that operand's k values), so the
// sequential path has no operand shuffling. The boundary flags come from LDS
// (the planner keeps segments per sequence within kMaxFlags), so no step
// waits on a global load to branch.
//
// With many boundaries the chain runs in three launches over groups of G
// consecutive boundaries (group j: boundaries [1 + jG, min(1 + (j+1) G, P))):
//   kCombHead   group 0 as a chain from S0(0), writing its states; every later
//               group composes its boundary maps, X <- F_s(X) from X = [I | 0]
//               over 256 columns (eight 32-column blocks), into the affine map
//               (CM_j, CH_j) of the whole group;
//   kCombGroups the state at the end of each group from the end of the one
//               before, S0 <- CM_j S0 + CH_j, j = 1 .. J - 2;
//   kCombApply  every group j >= 1 as a chain from the state at the end of
//               group j - 1, writing its states;
// about 2G + P/G steps in sequence instead of P - 1. kCombAll is the single
// chain (few boundaries).
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

enum { kCombAll = 0, kCombHead = 1, kCombGroups = 2, kCombApply = 3 };

template <int MODE>
__global__ __launch_bounds__(NTHR) void k_cp_combine(Params p) {
    __shared__ __attribute__((aligned(16))) bf16 sB[2][8 * 2 * 64 * 8];  // the state block as split B operands
    __shared__ int wflag[kMaxFlags];
    GDN_LDS_POISON_ALL(sB, wflag);
    const int h = blockIdx.y;
    int seq, j = 0, cb;   // cb: 32-column block (0..7 when composing: 0..3 the M part, 4..7 the H part)
    if (MODE == kCombAll || MODE == kCombGroups) {
        seq = blockIdx.x >> 2;
        cb = blockIdx.x & 3;
    } else if (MODE == kCombHead) {
        seq = blockIdx.x / (8 * p.comb_J);
        const int r = blockIdx.x - seq * 8 * p.comb_J;
        j = r >> 3;
        cb = r & 7;
    } else {
        seq = blockIdx.x / (4 * (p.comb_J - 1));
        const int r = blockIdx.x - seq * 4 * (p.comb_J - 1);
        j = 1 + (r >> 2);
        cb = r & 3;
    }
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
    const int G = p.comb_G, J = (MODE == kCombAll) ? 1 : (P - 1 + G - 1) / G;
    const bool compose = MODE == kCombHead && j > 0;
    if ((MODE == kCombHead || MODE == kCombApply) && j >= J) return;
    if (MODE == kCombHead && j == 0 && cb >= 4) return;
    if (MODE == kCombGroups && J < 3) return;
    int n_exact = 0;
    for (int s = 1 + (int)threadIdx.x; s < P; s += NTHR) {
        const int f = p.warm[(size_t)(seg_base + s) * p.h_v + h];
        wflag[s] = f;
        n_exact += (f == 0);
    }
    if (!__syncthreads_or(n_exact)) return;   // every boundary warmed up: nothing to chain
    // the steps: boundaries [s_lo, s_hi), or groups [1, J - 1) for kCombGroups
    int s_lo = 1, s_hi = P;
    if (MODE == kCombHead || MODE == kCombApply) {
        s_lo = 1 + j * G;
        s_hi = min(1 + (j + 1) * G, P);
        // a group's last state (but the last group's) comes from kCombGroups,
        // and the next group's kCombApply reads it: kCombApply leaves it alone
        if (MODE == kCombApply && j < J - 1) s_hi -= 1;
    } else if (MODE == kCombGroups) {
        s_hi = J - 1;
    }

    const int lane = lane_id(), col = lane & 31, hh = lane >> 5, w = wave_id();
    const int cglob = 32 * (cb & 3) + col;
    const size_t grp_base = ((size_t)seq * p.comb_J) * p.h_v + h;   // + j * h_v: group j's block
    {
        f32x16 acc;
        const float* S0 = nullptr;
        if (MODE == kCombAll || (MODE == kCombHead && j == 0)) {
            if (p.s_init) S0 = p.s_init + state_off(seq, p.h_v, h);
        } else if (MODE == kCombGroups) {
            S0 = p.seg_state + state_off(seg_base + G, p.h_v, h);          // end of group 0
        } else if (MODE == kCombApply) {
            S0 = p.seg_state + state_off(seg_base + j * G, p.h_v, h);      // end of group j - 1
        }
        if (S0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = S0[(32 * w + acc_row(i, hh)) * DK + cglob];
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i)   // composing: [I | 0]; else a zero initial state
                acc[i] = (compose && cb < 4 && 32 * w + acc_row(i, hh) == cglob) ? 1.f : 0.f;
        }
        combine_split_out(sB[0], acc, w, lane);
    }
    // Operands of step s1: the tile added (H_{s1-1}, the warm-up state, or CH_j)
    // and this lane's A operands of the map (M_{s1-1} or CM_j).
    // (every step issues the same loads and stores: a step past the end loads
    // the last one again, the map is loaded whether or not the step applies it,
    // and the state is stored back also where it is a warm-up state; then the
    // compiler's waits stay exact across the loop and the prefetch works)
    auto warm_of = [&](int s1) {
        return MODE == kCombGroups ? 0 : __builtin_amdgcn_readfirstlane(wflag[s1]);
    };
    auto tile_src = [&](int s1) -> const float* {
        s1 = min(s1, s_hi - 1);
        if (MODE == kCombGroups) return p.seg_GH + (grp_base + (size_t)s1 * p.h_v) * (2 * DK * DK);
        return warm_of(s1) ? p.seg_state + state_off(seg_base + s1, p.h_v, h)
                           : p.seg_H + state_off(seg_base + s1 - 1, p.h_v, h);
    };
    auto m_src = [&](int s1) {
        s1 = min(s1, s_hi - 1);
        const bf16* base = (MODE == kCombGroups)
            ? reinterpret_cast<const bf16*>(p.seg_GM + (grp_base + (size_t)s1 * p.h_v) * (DK * DK))
            : reinterpret_cast<const bf16*>(p.seg_M + state_off(seg_base + s1 - 1, p.h_v, h));
        return base + (size_t)(w * 8 * 2 * 64 + lane) * 8;
    };
    // the M part of a composition adds no tile
    const float tscale = (compose && cb < 4) ? 0.f : 1.f;
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
    // where step s1's state goes; composing, the group's CH block (its H part:
    // the last step leaves CH there) or the scratch half beside it (M part)
    auto dst_of = [&](int s1) -> float* {
        if (MODE == kCombGroups) return p.seg_state + state_off(seg_base + (s1 + 1) * G, p.h_v, h);
        if (compose) return p.seg_GH + (grp_base + (size_t)j * p.h_v) * (2 * DK * DK) + (cb < 4 ? DK * DK : 0);
        return p.seg_state + state_off(seg_base + s1, p.h_v, h);
    };
    // One step from the operands in `in`, which are refilled with those of
    // step s + 2 as they are consumed (each operand's load is issued right
    // after the MFMAs that read it, so the loads overlap the products): two
    // register sets alternate, and each step's loads have two steps to
    // arrive. The three partial products run as independent chains.
    int buf = 0;
    f32x16 last;
    auto step = [&](int s, CombineIn& in) {
        const int warm = warm_of(s);   // uniform: a scalar branch
        const bool mm = !warm && (s > 1 || p.s_init || MODE == kCombGroups);
        f32x16 acc = in.tile * tscale;
        const bf16* mop = m_src(s + 2);
        // (the products run also where they are not applied -- a warm-up
        // boundary, or M_0 without an initial state -- and are then dropped:
        // no branch separates the loads from the products)
        const f32x16 base = acc;
        f32x16 hl = f32x16{}, lh = f32x16{};
        const bf16* Bp = sB[buf];
        bf16x8 bh[8], bl[8];
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            bh[ks] = *reinterpret_cast<const bf16x8*>(Bp + ((ks * 2 + 0) * 64 + lane) * 8);
            bl[ks] = *reinterpret_cast<const bf16x8*>(Bp + ((ks * 2 + 1) * 64 + lane) * 8);
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            acc = mma32(in.ah[ks], bh[ks], acc);
            hl = mma32(in.ah[ks], bl[ks], hl);
            lh = mma32(in.al[ks], bh[ks], lh);
            in.ah[ks] = *reinterpret_cast<const bf16x8*>(mop + (ks * 2 + 0) * 64 * 8);
            in.al[ks] = *reinterpret_cast<const bf16x8*>(mop + (ks * 2 + 1) * 64 * 8);
        }
        {
            const float* src = tile_src(s + 2);
#pragma unroll
            for (int i = 0; i < 16; ++i) in.tile[i] = src[(32 * w + acc_row(i, hh)) * DK + cglob];
        }
        // instruction order for the scheduler: all sixteen LDS reads of the B
        // operands first (they arrive while the first products run), then per k
        // step three MFMAs and the two loads that refill their operands, then
        // the tile loads
        __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);
        acc += hl + lh;
        if (!mm) acc = base;
        combine_split_out(sB[buf ^ 1], acc, w, lane);
        {
            float* dst = dst_of(s);
#pragma unroll
            for (int i = 0; i < 16; ++i) dst[(32 * w + acc_row(i, hh)) * DK + cglob] = acc[i];
        }
        last = acc;
        __syncthreads();
        buf ^= 1;
    };
    CombineIn in0, in1;
    fetch(s_lo, in0);
    fetch(s_lo + 1, in1);
    __syncthreads();
    for (int s = s_lo; s < s_hi; s += 2) {
        step(s, in0);
        if (s + 1 < s_hi) step(s + 1, in1);
    }
    if (compose && cb < 4) {
        // the group's CM: split and laid out as the A operands of kCombGroups
        // (as k_cp_prep lays out M); columns 32 cb + col are k steps 2 cb, 2 cb + 1
        bf16* dstm = reinterpret_cast<bf16*>(p.seg_GM + (grp_base + (size_t)j * p.h_v) * (DK * DK));
        const int kk = col & 15, h2 = (kk >> 2) & 1, e = (kk & 3) | ((kk & 8) >> 1);
        const int ks = 2 * cb + (col >> 4);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int idx = (((w * 8 + ks) * 2) * 64 + acc_row(i, hh) + 32 * h2) * 8 + e;
            bf16 hi, lo;
            split1(last[i], hi, lo);
            dstm[idx] = hi;
            dstm[idx + 64 * 8] = lo;
        }
    }
}

// The fused forward of one segment: per chunk the P tiles, the state chain and
// the output. With two K^T buffers (bf16 inputs) a chunk is: P, V' and Q S
// from the staged chunk | barrier | stage the next chunk, fetch the one
// after, P V' and the output, state update | barrier. All waves take the
// steps in the same order: the two waves of a SIMD then tend to reach their
// VALU and their MFMA runs together, which issues faster than interleaving
// (a 16x16x32 MFMA leaves little room for VALU work beside it).
// With ST (the backward's re-run) the kernel instead writes, per chunk, the
// entering state, Y and V' and the output's state part as its dot with dO (the
// backward recomputes its chunk gradients from these), and neither forms the
// P tiles nor the output.
template <typename IO, bool ST>
__global__ __launch_bounds__(NTHR_CH) void k_fwd(Params p) {
    constexpr bool EX = Io<IO>::kExact;
    constexpr bool DB = ChainSmem<EX>::NB == 2;
    __shared__ ChainSmem<EX> sm;
    GDN_LDS_POISON_ALL(sm);
    const int h = blockIdx.y, hq = h / p.group, wave = wave_id();
    const SegLoc loc = locate_segment(p, blockIdx.x);
    if (loc.seq < 0) return;
    // P's upper tiles inside the diagonal 32-blocks stay zero (the chunk loop
    // writes the ten lower tiles only); the first barrier below orders this
    // before every read
    for (int i = threadIdx.x; i < 2 * CH * LDP / 8; i += NTHR_CH)
        *reinterpret_cast<u32x4*>(sm.p + 8 * i) = u32x4{0u, 0u, 0u, 0u};
    f32x4 S[8];
    if (loc.s == 0) {
        if (p.s_init) load_state(p.s_init + state_off(loc.seq, p.h_v, h), S);
        else zero_state(S);
    } else {
        load_state(p.seg_state + state_off(loc.seg_base + loc.s, p.h_v, h), S);
    }
    const int c0 = loc.s * p.L, c1 = min(c0 + p.L, loc.N);
    const size_t ts_v = (size_t)p.h_v * DK;
    if (c0 < c1) {
        Chunk<IO> nxt;
        auto fetch = [&](int c) {
            c = min(c, c1 - 1);
            fetch_chunk<IO, true, true>(nxt, p, loc.tok0 + (size_t)c * CH, min(CH, loc.len - c * CH), h, hq,
                                        loc.chunk_base + c);
        };
        // the loop body's loads are followed by the output's four stores; the
        // same stores (to the scratch line) after the loads before the loop
        // make its entry look alike, so that the waits stay exact
        auto sink_stores = [&]() {
            if constexpr (ST) return;   // (no output stores in the loop)
            IO* dst = reinterpret_cast<IO*>(p.sink + 32 * lane_id());
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (EX) *reinterpret_cast<u32x2*>(dst + 4 * i) = u32x2{0u, 0u};
                else *reinterpret_cast<f32x4*>(dst + 4 * i) = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        };
        // first half of chunk c: V' and the Q S part of the output (and P)
        auto half1 = [&](int c, f32x4 Vp[4], f32x4 O[4]) {
            const size_t tok0 = loc.tok0 + (size_t)c * CH;
            const IO* vcol = static_cast<const IO*>(p.v) + tok0 * ts_v + (size_t)h * DK + 16 * wave + (lane_id() & 15);
            SplitS ss;
            split_state(S, ss);
            if constexpr (ST) {
                // for the backward: Y and V' of this chunk (token rows, fp32), and
                // the output's state part scale e^gamma Q S as its dot with dO
                const int l = lane_id(), cc = l & 15, g = l >> 4;
                const int nv = min(CH, loc.len - c * CH);
                // dO for the state term's dot products below, loaded first so that it
                // arrives during the products (rows past the end read the last row;
                // the reader masks them)
                const unsigned short* dob = static_cast<const unsigned short*>(p.bwd_dout) + tok0 * ts_v +
                                            (size_t)h * DK + 16 * wave + 4 * g;
                u32x2 dw[4];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
                    dw[ct] = *reinterpret_cast<const u32x2*>(dob + (size_t)min(16 * ct + cc, nv - 1) * ts_v);
                f32x4 Y[4];
                chain_vp<IO, true>(sm, ss, vcol, ts_v, nv, Vp, Y);
                chain_qs<EX>(sm, ss, O);
                const size_t blk = ((size_t)(loc.chunk_base + c) * p.h_v + h) * CH * DK;
#pragma unroll
                for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const size_t o = blk + (size_t)(16 * rt + 4 * g + e) * DK + 16 * wave + cc;
                        p.bwd_y[o] = Y[rt][e];
                        p.bwd_vp[o] = Vp[rt][e];
                    }
                // the output's state term enters the gradients only through its dot
                // product with dO per token (the dgamma sums): this wave's 16
                // columns, summed over the lane groups, one partial per wave
                float* part = p.bwd_oi + ((size_t)(loc.chunk_base + c) * p.h_v + h) * (NW_CH * CH) + wave * CH;
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const u32x2 d = dw[ct];
                    float sdot = O[ct][0] * __uint_as_float(d[0] << 16) + O[ct][1] * __uint_as_float(d[0] & 0xffff0000u) +
                                 O[ct][2] * __uint_as_float(d[1] << 16) + O[ct][3] * __uint_as_float(d[1] & 0xffff0000u);
                    sdot += __shfl_xor(sdot, 16, 64);
                    sdot += __shfl_xor(sdot, 32, 64);
                    if (g == 0) part[16 * ct + cc] = sdot;
                }
            } else {
                chain_vp<IO, true>(sm, ss, vcol, ts_v, min(CH, loc.len - c * CH), Vp);
                chain_qs<EX>(sm, ss, O);
            }
            if constexpr (!ST) gram_p<EX>(sm, p.scale);
        };
        // the output: O += P V' and the rows stored (not in the re-run for the
        // backward, which needs only the state part's dot with dO)
        auto out_part = [&](int c, const f32x4 Vp[4], f32x4 O[4]) {
            if constexpr (ST) return;
            const size_t tok0 = loc.tok0 + (size_t)c * CH;
            chain_pv_out<IO>(sm, Vp, O, static_cast<IO*>(p.out) + tok0 * ts_v + (size_t)h * DK, ts_v,
                             min(CH, loc.len - c * CH), p.sink);
        };
        fetch(c0);
        if constexpr (DB) {
            stage_chunk<IO, true, true>(sm, nxt, p.scale, 0);
            fetch(c0 + 1);
            sink_stores();
            __syncthreads();
            for (int c = c0; c < c1; ++c) {
                const int b = (c - c0) & 1;
                if constexpr (ST) store_state(p.chunk_states + state_off(loc.chunk_base + c, p.h_v, h), S);
                f32x4 Vp[4], O[4];
                half1(c, Vp, O);
                __syncthreads();
                stage_chunk<IO, true, true>(sm, nxt, p.scale, b ^ 1);
                fetch(c + 2);
                out_part(c, Vp, O);
                chain_state<EX>(sm, S, Vp, b);
                __syncthreads();
            }
        } else {
            sink_stores();
            for (int c = c0; c < c1; ++c) {
                if constexpr (ST) store_state(p.chunk_states + state_off(loc.chunk_base + c, p.h_v, h), S);
                stage_chunk<IO, true, true>(sm, nxt, p.scale, 0);
                __syncthreads();
                fetch(c + 1);
                f32x4 Vp[4], O[4];
                half1(c, Vp, O);
                __syncthreads();
                out_part(c, Vp, O);
                chain_state<EX>(sm, S, Vp, 0);
                __syncthreads();
            }
        }
    }
    if (loc.s == loc.P - 1 && p.s_final) store_state(p.s_final + state_off(loc.seq, p.h_v, h), S);
}

// ----------------------------------------------------------------------------
// Backward: the reverse scan of the state gradient dS over the chunks of one
// sequence and value head on the matrix cores (the formulas are in
// gdn_bwd.hip). Per chunk, with dS the gradient of the state leaving it:
//   X   = diag(f) K dS + scale P^T dO          (dV'; K dS as the forward's K S)
//   Z   = T^T X,  Y' = -diag(e^gamma beta) Z
//   dS <- e^gamma_C dS + Q^T (scale diag(e^gamma) dO) + K^T Y'
// Eight waves; wave w keeps columns [16w, 16w + 16) of dS in registers in the
// forward's state layout, so dS, X, dO and Y' serve as MFMA operands directly
// (tokens in kp order). T^T and scale P^T come as hi/lo images from the
// backward prep; K (token-major, d_k in kp order), K^T and Q^T are staged as
// in the forward. The next chunk's inputs are loaded during the current one.
struct BwdChainSmem {
    bf16 k_hi[CH * LDQ];                  // K token-major, d_k in kp order
    bf16 kt[DK * LDKT];                   // K^T: row d_k, tokens in kp order (chunks swizzled)
    bf16 qt[DK * LDKT];                   // Q^T, same layout
    bf16 tt[2 * CH * LDP];                // T^T: hi rows, then lo rows; tokens in kp order
    bf16 pt[2 * CH * LDP];                // scale P^T, same
    bf16 dot[DK * LDKT];                  // dO^T: row d_v, tokens in kp order (chunks swizzled), rows past the end zero
    float fr[CH];                         // exp(gamma_C - gamma)
    float egb[CH];                        // -exp(gamma) beta
    float egs[CH];                        // scale exp(gamma)
    float bet[CH];                        // beta (0 past the end)
    float ec;                             // exp(gamma_C)
};

struct BwdChainIn {
    u32x2 k[4], q[4];                     // tokens 4 (t / 32) + j, d_k 4 (t % 32) .. + 3
    u32x2 d[4];                           // dO: tokens 4 (t / 32) + j, d_v 4 (t % 32) .. + 3
    u32x4 img[4];                         // pieces t + 512 j of the T^T / P^T images
    float gl, bl;                         // gamma, beta of token lane
    int nv;                               // valid tokens of the chunk
};

template <bool WANT_DO>
__device__ void bwd_chain_fetch(const BwdParams& p, BwdChainIn& in, int f, size_t tok0, int nv, int h, int hq) {
    const int t = threadIdx.x, m = t >> 5, c4 = (t & 31) * 4, lane = lane_id();
    const size_t ts = (size_t)p.h_qk * DK, ts_v = (size_t)p.h_v * DK;
    const bf16* kb = static_cast<const bf16*>(p.k) + tok0 * ts + (size_t)hq * DK + c4;
    const bf16* qb = static_cast<const bf16*>(p.q) + tok0 * ts + (size_t)hq * DK + c4;
    const bf16* db = static_cast<const bf16*>(p.dout) + tok0 * ts_v + (size_t)h * DK + c4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {   // rows past the end read the last row (K, Q: their values never
        const int row = min(4 * m + j, nv - 1);   // matter; dO: zeroed when staged)
        in.k[j] = *reinterpret_cast<const u32x2*>(kb + (size_t)row * ts);
        in.q[j] = *reinterpret_cast<const u32x2*>(qb + (size_t)row * ts);
        if (WANT_DO) in.d[j] = *reinterpret_cast<const u32x2*>(db + (size_t)row * ts_v);
    }
    const u32x4* img = reinterpret_cast<const u32x4*>(static_cast<const bf16*>(p.tpt) + ((size_t)f * p.h_v + h) * kBwdTpt);
#pragma unroll
    for (int j = 0; j < 4; ++j) in.img[j] = img[t + NTHR_CH * j];
    in.gl = p.tpg[((size_t)f * p.h_v + h) * kBwdTpg + CH * CH + lane];
    in.bl = p.beta[(tok0 + min(lane, nv - 1)) * p.h_v + h];
    in.nv = nv;   // (the masking waits for the loads: it happens when the chunk is staged)
}

template <bool WANT_DO>
__device__ void bwd_chain_stage(BwdChainSmem& sm, const BwdChainIn& in, float scale) {
    const int t = threadIdx.x, lane = lane_id(), m = t >> 5, c4 = (t & 31) * 4;
    if (wave_id() == 0) {   // the gate factors: one wave (a scalar branch)
        const float gc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, in.gl), 63));
        const float es = __expf(in.gl);
        sm.fr[lane] = __expf(gc - in.gl);
        sm.egb[lane] = lane < in.nv ? -es * in.bl : 0.f;
        sm.bet[lane] = lane < in.nv ? in.bl : 0.f;
        sm.egs[lane] = es * scale;
        sm.ec = __expf(gc);
    }
    const int kc = kp(c4), tk = kp(4 * m) ^ tswz(c4);
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x2*>(sm.k_hi + (4 * m + j) * LDQ + kc) = in.k[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<u32x2*>(sm.kt + (c4 + e) * LDKT + tk) = pack_col4(in.k, e);
        *reinterpret_cast<u32x2*>(sm.qt + (c4 + e) * LDKT + tk) = pack_col4(in.q, e);
    }
    if (WANT_DO) {
        u32x2 d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) d[j] = 4 * m + j < in.nv ? in.d[j] : u32x2{0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) *reinterpret_cast<u32x2*>(sm.dot + (c4 + e) * LDKT + tk) = pack_col4(d, e);
    }
    // images: piece idx -> part idx / 512 (T hi, T lo, P hi, P lo), row (idx / 8) % 64, 8 elements at 8 (idx % 8)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int idx = t + NTHR_CH * j, part = idx >> 9, row = (idx >> 3) & 63, k8 = (idx & 7) * 8;
        bf16* dst = (part < 2 ? sm.tt : sm.pt) + ((part & 1) * CH + row) * LDP + k8;
        *reinterpret_cast<u32x4*>(dst) = in.img[j];
    }
}

// The scan over chunks [c_lo, c_hi) of one sequence, from D (the gradient of
// the state leaving chunk c_hi - 1). WANT_DO: the output terms (P^T dO and
// Q^T dO'); without them the scan applies the homogeneous map only.
// WRITE_DS: store the gradient of the state leaving every chunk.
template <bool WANT_DO, bool WRITE_DS>
__device__ void bwd_chain_run(const BwdParams& p, BwdChainSmem& sm, const SegLoc& loc, int c_lo, int c_hi, int h,
                              f32x4 D[8]) {
    const int hq = h / p.group, lane = lane_id(), c = lane & 15, g = lane >> 4;
    BwdChainIn in;
    auto fetch = [&](int cc) {
        bwd_chain_fetch<WANT_DO>(p, in, loc.chunk_base + cc, loc.tok0 + (size_t)cc * CH, min(CH, loc.len - cc * CH),
                                 h, hq);
    };
    if (c_lo < c_hi) fetch(c_hi - 1);
    for (int cc = c_hi - 1; cc >= c_lo; --cc) {
        // stage first: its wait then covers the prefetched loads only, not the
        // stores below (loads and stores share one counter)
        bwd_chain_stage<WANT_DO>(sm, in, p.scale);
        const int in_nv = in.nv;
        if (WRITE_DS) store_state(p.ds + state_off(loc.chunk_base + cc, p.h_v, h), D);
        __syncthreads();
        if (cc > c_lo) fetch(cc - 1);
        // X = diag(f) K dS + scale P^T dO
        f32x4 X[4];
        {
            SplitS ss;
            split_state(D, ss);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) X[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 kh[4];
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) kh[rt] = lds_op16(sm.k_hi + (16 * rt + c) * LDQ + 32 * s + 8 * g);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) X[rt] = mma16k32(kh[rt], ss.hi[s], X[rt]);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) X[rt] = mma16k32(kh[rt], ss.lo[s], X[rt]);
            }
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) X[rt] *= *reinterpret_cast<const f32x4*>(sm.fr + 16 * rt + 4 * g);
        // this lane's dO as B operands (column 16 w + c, the tokens of k step s in kp
        // order: 32 s + 4 g + 0..3 and 32 s + 16 + 4 g + 0..3), bf16 pairs
        unsigned dO[8];
        if (WANT_DO) {
            const int col = 16 * wave_id() + c;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const u32x4 v = __builtin_bit_cast(u32x4, lds_op16(sm.dot + col * LDKT + ((32 * s + 8 * g) ^ tswz(col))));
#pragma unroll
                for (int i = 0; i < 4; ++i) dO[4 * s + i] = v[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) dO[i] = 0u;
        }
        if (WANT_DO) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const bf16x8 db = __builtin_bit_cast(bf16x8, u32x4{dO[4 * s], dO[4 * s + 1], dO[4 * s + 2], dO[4 * s + 3]});
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    if (s == 0 && rt >= 2) continue;   // P^T[r][m] = 0 for m < r
                    const bf16x8 ph = lds_op16(sm.pt + (16 * rt + c) * LDP + 32 * s + 8 * g);
                    const bf16x8 pl = lds_op16(sm.pt + (CH + 16 * rt + c) * LDP + 32 * s + 8 * g);
                    X[rt] = mma16k32(ph, db, X[rt]);
                    X[rt] = mma16k32(pl, db, X[rt]);
                }
            }
        }
        if (WRITE_DS) {   // dV' for the chunk gradients
            float* xb = p.dvp + ((size_t)(loc.chunk_base + cc) * p.h_v + h) * CH * DK + 16 * wave_id() + c + 4 * g * DK;
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) xb[(16 * rt + e) * DK] = X[rt][e];
        }
        // Z = T^T X, then Y' = -diag(e^gamma beta) Z
        f32x4 Z[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) Z[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 xh, xl;
            split8(X[2 * s], X[2 * s + 1], xh, xl);
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                if (s == 0 && rt >= 2) continue;   // T^T[r][m] = 0 for m < r
                const bf16x8 th = lds_op16(sm.tt + (16 * rt + c) * LDP + 32 * s + 8 * g);
                const bf16x8 tl = lds_op16(sm.tt + (CH + 16 * rt + c) * LDP + 32 * s + 8 * g);
                Z[rt] = mma16k32(th, xh, Z[rt]);
                Z[rt] = mma16k32(th, xl, Z[rt]);
                Z[rt] = mma16k32(tl, xh, Z[rt]);
            }
        }
        if (WRITE_DS) {   // for the chunk gradients: Z (fp32) and the output dv = diag(beta) Z
            float* zb = p.z + ((size_t)(loc.chunk_base + cc) * p.h_v + h) * CH * DK + 16 * wave_id() + c + 4 * g * DK;
            const unsigned ts_v = (unsigned)(p.h_v * DK);
            bf16* dv = static_cast<bf16*>(p.dv) + (loc.tok0 + (size_t)cc * CH) * ts_v + (size_t)h * DK + 16 * wave_id() + c;
            const int dv_rows = p.out_f32 ? 0 : in_nv;   // fp32 dv: formed from Z afterwards
#pragma unroll
            for (int rt = 0; rt < 4; ++rt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * rt + 4 * g + e;
                    zb[(16 * rt + e) * DK] = Z[rt][e];
                    if (r < dv_rows) dv[r * ts_v] = (bf16)(sm.bet[r] * Z[rt][e]);
                }
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) Z[rt] *= *reinterpret_cast<const f32x4*>(sm.egb + 16 * rt + 4 * g);
        // dS <- e^gamma_C dS + Q^T (scale e^gamma dO) + K^T Y'
        {
            const float ec = sm.ec;
#pragma unroll
            for (int i = 0; i < 8; ++i) D[i] *= ec;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            bf16x8 yh, yl, oh, ol;
            split8(Z[2 * s], Z[2 * s + 1], yh, yl);
            if (WANT_DO) {
                const f32x4 e0 = *reinterpret_cast<const f32x4*>(sm.egs + 32 * s + 4 * g);
                const f32x4 e1 = *reinterpret_cast<const f32x4*>(sm.egs + 32 * s + 16 + 4 * g);
                const unsigned a0 = dO[4 * s], a1 = dO[4 * s + 1], b0 = dO[4 * s + 2], b1 = dO[4 * s + 3];
                const f32x4 o0 = f32x4{__uint_as_float(a0 << 16), __uint_as_float(a0 & 0xffff0000u),
                                       __uint_as_float(a1 << 16), __uint_as_float(a1 & 0xffff0000u)} * e0;
                const f32x4 o1 = f32x4{__uint_as_float(b0 << 16), __uint_as_float(b0 & 0xffff0000u),
                                       __uint_as_float(b1 << 16), __uint_as_float(b1 & 0xffff0000u)} * e1;
                split8(o0, o1, oh, ol);
            }
            // two row tiles at a time: few operands live, two independent chains
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const int o0 = (16 * i + c) * LDKT + ((32 * s + 8 * g) ^ (8 * i));
                const int o1 = (16 * (i + 1) + c) * LDKT + ((32 * s + 8 * g) ^ (8 * (i + 1)));
                const bf16x8 k0 = lds_op16(sm.kt + o0), k1 = lds_op16(sm.kt + o1);
                if (WANT_DO) {
                    const bf16x8 q0 = lds_op16(sm.qt + o0), q1 = lds_op16(sm.qt + o1);
                    D[i] = mma16k32(q0, oh, D[i]);
                    D[i + 1] = mma16k32(q1, oh, D[i + 1]);
                    D[i] = mma16k32(q0, ol, D[i]);
                    D[i + 1] = mma16k32(q1, ol, D[i + 1]);
                }
                D[i] = mma16k32(k0, yh, D[i]);
                D[i + 1] = mma16k32(k1, yh, D[i + 1]);
                D[i] = mma16k32(k0, yl, D[i]);
                D[i + 1] = mma16k32(k1, yl, D[i + 1]);
            }
        }
        __syncthreads();
    }
}

// MODE kBwdWhole: one workgroup per (sequence, head) over all its chunks.
// With segments (the forward's plan): kBwdMaps, per (segment s >= 1, part,
// head): part 0 scans the segment from zero (from dS_final for the last
// segment) into seg_H[s], part 1 from the identity without output terms into
// seg_M[s] (the segment's map, not needed for the last); kBwdRerun, per
// (segment, head): the scan from the gradient at the segment's end (seg_state
// from the linking pass, dS_final for the last), writing every chunk's.
enum { kBwdWhole = 0, kBwdMaps = 1, kBwdRerun = 2 };

template <int MODE>
__global__ __launch_bounds__(NTHR_CH) void k_bwd_chain_mma(BwdParams p) {
    __shared__ BwdChainSmem sm;
    GDN_LDS_POISON_ALL(sm);
    const int h = blockIdx.y;
    f32x4 D[8];
    if (MODE == kBwdWhole) {
        const SegLoc loc = locate_segment(p, blockIdx.x);   // (L covers the longest sequence: one segment each)
        if (loc.seq < 0) return;
        if (p.dfinal) load_state(p.dfinal + state_off(loc.seq, p.h_v, h), D);
        else zero_state(D);
        bwd_chain_run<true, true>(p, sm, loc, 0, loc.N, h, D);
        if (p.dinit) store_state(p.dinit + state_off(loc.seq, p.h_v, h), D);
    } else if (MODE == kBwdMaps) {
        // segment s goes to slot r = P - 1 - s: the segment ends are then linked
        // by the forward's segment combine (boundary r + 1 applies M[r], H[r]),
        // which runs the boundaries in increasing order
        const int part = blockIdx.x & 1;
        const SegLoc loc = locate_segment(p, blockIdx.x >> 1);
        if (loc.seq < 0 || loc.s == 0) return;
        const bool last = loc.s == loc.P - 1;
        if (part == 1 && last) return;
        const int c0 = loc.s * p.L, c1 = min(c0 + p.L, loc.N), r = loc.P - 1 - loc.s;
        if (part == 0) {
            if (last && p.dfinal) load_state(p.dfinal + state_off(loc.seq, p.h_v, h), D);
            else zero_state(D);
            bwd_chain_run<true, false>(p, sm, loc, c0, c1, h, D);
            store_state(p.seg_H + state_off(loc.seg_base + r, p.h_v, h), D);
            if (threadIdx.x == 0) p.warm[(size_t)(loc.seg_base + r + 1) * p.h_v + h] = 0;   // exact
        } else {
            identity_state(D);
            bwd_chain_run<false, false>(p, sm, loc, c0, c1, h, D);
            // (the scan ended behind a barrier: its LDS is free for the staging)
            store_m_operand(reinterpret_cast<bf16*>(&sm), D,
                            reinterpret_cast<bf16*>(p.seg_M + state_off(loc.seg_base + r, p.h_v, h)));
        }
    } else {
        const SegLoc loc = locate_segment(p, blockIdx.x);
        if (loc.seq < 0) return;
        if (loc.s == loc.P - 1) {
            if (p.dfinal) load_state(p.dfinal + state_off(loc.seq, p.h_v, h), D);
            else zero_state(D);
        } else {
            load_state(p.seg_state + state_off(loc.seg_base + loc.P - 1 - loc.s, p.h_v, h), D);
        }
        const int c0 = loc.s * p.L, c1 = min(c0 + p.L, loc.N);
        bwd_chain_run<true, true>(p, sm, loc, c0, c1, h, D);
        if (loc.s == 0 && p.dinit) store_state(p.dinit + state_off(loc.seq, p.h_v, h), D);
    }
}

// ----------------------------------------------------------------------------
// Backward, every gradient of one (chunk, value head) on the matrix cores.
// The forward re-run left Y, V' and scale e^gamma Q S of the chunk, the state
// scan left dV', Z = T^T dV' (and dv); what remains contracts over d_v or
// over the chunk's tokens (formulas in gdn_bwd.hip):
//   dq = diag(scale e^gamma) dO S^T + Psi K
//   dk = diag(f) V' dSn^T - diag(e^gamma) dY S^T + Psi^T Q + (G + G^T) K
//   dP = scale dO V'^T -> Psi, dT = dV' (diag(beta) Y)^T -> W1 = dT T^T,
//   dA = -T^T W1 -> G, and the dbeta / dgamma row and column sums.
// Eight waves; wave w owns d_k columns [16w, 16w + 16) of dq and dk (all 64
// tokens) and two of the sixteen 16x16 tiles of every 64 x 64 product (row
// tile w / 2, column tiles 2 (w % 2) + 0, 1). Operands over d_v are read from
// HBM / L2 straight into the kp order (two 16-byte loads per lane and k step);
// K^T, Q^T and the 64 x 64 images (T, T^T, Psi, Psi^T, dT, W1^T, G, G^T; hi/lo
// bf16) go through LDS.
struct BwdChunkSmem {
    bf16 kt[DK * LDKT];                   // K^T: row d_k, tokens in kp order (chunks swizzled)
    bf16 qt[DK * LDKT];                   // Q^T, same layout
    bf16 tim[2 * CH * LDP];               // T: rows r, tokens in kp order; hi rows, then lo rows
    bf16 ttim[2 * CH * LDP];              // T^T
    bf16 sa[2 * CH * LDP];                // Psi, then G
    bf16 sb[2 * CH * LDP];                // Psi^T, then G^T
    bf16 sc[2 * CH * LDP];                // dT, then W1^T
    float gam[CH], eg[CH], fr[CH], bet[CH], dgam[CH], dbe[CH];
    float dgc;
};

__device__ __forceinline__ float dot4v(f32x4 a, f32x4 b) { return (a[0] * b[0] + a[1] * b[1]) + (a[2] * b[2] + a[3] * b[3]); }
// Accumulator element (row 16 rt + 4 g + e, column 16 ct + c) of a 64 x 64 tile
// into an image: at [row][kp(col)] (scalar) or transposed at [col][kp(row)]
// (the four rows of a lane are consecutive in kp order: one 8-byte store).
__device__ __forceinline__ void put_img(bf16* img, int rt, int ct, int c, int g, const f32x4& x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bf16 hi, lo;
        split1(x[e], hi, lo);
        const int o = (16 * rt + 4 * g + e) * LDP + kp(16 * ct + c);
        img[o] = hi;
        img[CH * LDP + o] = lo;
    }
}
__device__ __forceinline__ void put_img_t(bf16* img, int rt, int ct, int c, int g, const f32x4& x) {
    bf16x4 hi, lo;
    split4(x, hi, lo);
    const int o = (16 * ct + c) * LDP + kp(16 * rt + 4 * g);
    *reinterpret_cast<bf16x4*>(img + o) = hi;
    *reinterpret_cast<bf16x4*>(img + CH * LDP + o) = lo;
}
// column sums of a 16x16 tile over its 16 rows (e, then lane groups g)
__device__ __forceinline__ float tile_colsum(const f32x4& x) {
    float s = (x[0] + x[1]) + (x[2] + x[3]);
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    return s;
}
// Row sums of N values at once (N = 4, 8 or 16), each over the 16 lanes c of a
// lane group, as a reduce-scatter: at each exchange a lane keeps one half of its
// values, adds its partner's copy of that half and sends the other half, so N
// sums take N - 1 exchanges in four dependent rounds. Lane c returns the sum of
// value (c * N) / 16 (for N < 16 the lanes c that share it hold the same sum).
template <int N, int M>
__device__ __forceinline__ void rowsum_round(float* a, int c) {
    if constexpr (M >= 1) {
        if constexpr (N > 1) {
            const bool up = (c & M) != 0;
#pragma unroll
            for (int i = 0; i < N / 2; ++i) {
                const float send = up ? a[i] : a[i + N / 2];
                const float keep = up ? a[i + N / 2] : a[i];
                a[i] = keep + __shfl_xor(send, M, 64);
            }
            rowsum_round<N / 2, M / 2>(a, c);
        } else {
            a[0] += __shfl_xor(a[0], M, 64);
            rowsum_round<1, M / 2>(a, c);
        }
    }
}
template <int N>
__device__ __forceinline__ float tile_rowsums(float (&a)[N], int c) {
    static_assert(N == 4 || N == 8 || N == 16, "four, eight or sixteen values");
    rowsum_round<N, 8>(a, c);
    return a[0];
}

// One item's operands that the staging and step 1 read from memory. They are
// fetched an item ahead, during the previous item's last steps (few memory
// operations there), so that their latency hides behind that work.
struct BwdItemIn {
    u32x2 kk[4], qq[4];   // K, Q rows 4 (t / 32) + j, columns 4 (t % 32) ..
    u32x4 img[4];         // pieces t, t + 512 of the T^T and T image parts
    float gm, b, qo1;     // gamma, beta of token t (t < 64); the output term's partial sum
    f32x4 y1[4], z1[4];   // Y, Z: row t / 8, columns 16 (t % 8) ..
    u32x2 v1[4];          // V: the same
};

// Items: (chunk slot f, value head h) = (item / h_v, item % h_v), so that the
// value heads of a chunk (which share K and Q rows) run at the same time.
__device__ __forceinline__ void bwd_item_fetch(const BwdParams& p, long long item, BwdItemIn& in) {
    const int f = (int)(item / p.h_v), h = (int)(item - (long long)f * p.h_v), hq = h / p.group, t = threadIdx.x;
    int seq, cidx, len;
    size_t tok_s;
    locate_chunk(p, f, seq, cidx, len, tok_s);   // item < n_chunks h_v: always found
    const size_t tok0 = tok_s + (size_t)cidx * CH;
    const int nv = min(CH, len - cidx * CH);
    const size_t ts = (size_t)p.h_qk * DK, ts_v = (size_t)p.h_v * DK;
    const size_t blk = ((size_t)f * p.h_v + h) * CH * DK;
    const bf16* Kg = static_cast<const bf16*>(p.k) + tok0 * ts + (size_t)hq * DK;
    const bf16* Qg = static_cast<const bf16*>(p.q) + tok0 * ts + (size_t)hq * DK;
    const int m = t >> 5, c4 = (t & 31) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int row = min(4 * m + j, nv - 1);
        in.kk[j] = *reinterpret_cast<const u32x2*>(Kg + (size_t)row * ts + c4);
        in.qq[j] = *reinterpret_cast<const u32x2*>(Qg + (size_t)row * ts + c4);
    }
    const u32x4* img = reinterpret_cast<const u32x4*>(static_cast<const bf16*>(p.tpt) + ((size_t)f * p.h_v + h) * kBwdTpt);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        in.img[2 * j] = img[t + NTHR_CH * j];
        in.img[2 * j + 1] = img[t + NTHR_CH * j + 2048];
    }
    const int tt = min(t, CH - 1);
    in.gm = p.tpg[((size_t)f * p.h_v + h) * kBwdTpg + CH * CH + tt];
    in.b = p.beta[(tok0 + min(tt, nv - 1)) * p.h_v + h];
    const int r1 = t >> 3, c01 = (t & 7) * 16;
    in.qo1 = p.oi[((size_t)f * p.h_v + h) * (NW_CH * CH) + (t & 7) * CH + r1];
    const bf16* Vg = static_cast<const bf16*>(p.v) + tok0 * ts_v + (size_t)h * DK;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        const int col = c01 + 4 * q4;
        in.y1[q4] = *reinterpret_cast<const f32x4*>(p.y + blk + (size_t)r1 * DK + col);
        in.z1[q4] = *reinterpret_cast<const f32x4*>(p.z + blk + (size_t)r1 * DK + col);
        in.v1[q4] = *reinterpret_cast<const u32x2*>(Vg + (size_t)min(r1, nv - 1) * ts_v + col);
    }
}

// One workgroup per CU (its LDS allows no second), walking the items
// blockIdx.x, blockIdx.x + gridDim.x, ...
__global__ __launch_bounds__(NTHR_CH) void k_bwd_chunk_mma(BwdParams p) {
    __shared__ BwdChunkSmem sm;
    GDN_LDS_POISON_ALL(sm);
    const long long n_items = (long long)p.n_chunks * p.h_v;
    long long item = blockIdx.x;
    if (item >= n_items) return;
    BwdItemIn in;
    bwd_item_fetch(p, item, in);
    for (; item < n_items; item += gridDim.x) {
        // the thread index through an opaque move: the many LDS offsets derived
        // from it are then formed in each item where they are used, instead of
        // being hoisted out of the loop and held in registers throughout
        int t;
        asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
        const int w = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63, c = lane & 15, g = lane >> 4;
        const int f = (int)(item / p.h_v), h = (int)(item - (long long)f * p.h_v), hq = h / p.group;
        int seq, cidx, len;
        size_t tok_s;
        locate_chunk(p, f, seq, cidx, len, tok_s);
        const size_t tok0 = tok_s + (size_t)cidx * CH;
        const int nv = min(CH, len - cidx * CH);
        const size_t ts = (size_t)p.h_qk * DK, ts_v = (size_t)p.h_v * DK;
        const size_t blk = ((size_t)f * p.h_v + h) * CH * DK;
        const float* S = p.cs + state_off(f, p.h_v, h);
        const float* dSn = p.ds + state_off(f, p.h_v, h);
        const float* Yb = p.y + blk;
        const float* Vpb = p.vp + blk;
        const float* dVb = p.dvp + blk;
        const float* Zb = p.z + blk;
        const bf16* Kg = static_cast<const bf16*>(p.k) + tok0 * ts + (size_t)hq * DK;
        const bf16* dOg = static_cast<const bf16*>(p.dout) + tok0 * ts_v + (size_t)h * DK;
        const float* tp = p.tpg + ((size_t)f * p.h_v + h) * kBwdTpg;
        const float scale = p.scale;
        const int r1 = t >> 3;
        __syncthreads();   // the previous item's last LDS reads are done
        // ---- staging: K^T, Q^T (rows past the end repeat the last; harmless, see the products), images, gates
        {
            const int m = t >> 5, c4 = (t & 31) * 4, tk = kp(4 * m) ^ tswz(c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                *reinterpret_cast<u32x2*>(sm.kt + (c4 + e) * LDKT + tk) = pack_col4(in.kk, e);
                *reinterpret_cast<u32x2*>(sm.qt + (c4 + e) * LDKT + tk) = pack_col4(in.qq, e);
            }
            // pieces of the [T^T hi, T^T lo, P^T hi, P^T lo, T hi, T lo] image: parts 0, 1 and 4, 5
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int idx = t + NTHR_CH * j, part = idx >> 9, row = (idx >> 3) & 63, k8 = (idx & 7) * 8;
                *reinterpret_cast<u32x4*>(sm.ttim + (part * CH + row) * LDP + k8) = in.img[2 * j];
                *reinterpret_cast<u32x4*>(sm.tim + (part * CH + row) * LDP + k8) = in.img[2 * j + 1];
            }
            if (t < CH) {
                sm.gam[t] = in.gm;
                sm.eg[t] = __expf(in.gm);
                sm.bet[t] = t < nv ? in.b : 0.f;
            }
            if (t == 0) sm.dgc = 0.f;
        }
        // step 2's dO and Z pieces and this wave's S row (every k step), in flight through
        // step 1 (dO rows past the end repeat the last)
        const float* Srow = S + (size_t)(16 * w + c) * DK;
        const float* Drow = dSn + (size_t)(16 * w + c) * DK;
        u32x2 dox[4];
        f32x4 zx[4], srow[4][2];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            srow[ks][0] = *reinterpret_cast<const f32x4*>(Srow + 32 * ks + 4 * g);
            srow[ks][1] = *reinterpret_cast<const f32x4*>(Srow + 32 * ks + 16 + 4 * g);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int idx = t + NTHR_CH * j, r = idx >> 5, c4 = (idx & 31) * 4;
            dox[j] = *reinterpret_cast<const u32x2*>(dOg + (size_t)min(r, nv - 1) * ts_v + c4);
            zx[j] = *reinterpret_cast<const f32x4*>(Zb + (size_t)r * DK + c4);
        }
        __syncthreads();
        if (t < CH) sm.fr[t] = __expf(sm.gam[CH - 1] - sm.gam[t]);
        // ---- 1. row sums over d_v: thread t takes row t / 8, columns 16 (t % 8) .. + 15
        {
            const int r = r1;
            const bool ok = r < nv;
            float zb = 0.f, vy = 0.f;
            // the output's state term . dO over this thread's 16 columns (the forward
            // re-run's partial sum of wave t % 8, whose columns these are)
            float qo = in.qo1;
            const float br = sm.bet[r];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 y = in.y1[q4], z = in.z1[q4];
                const u32x2 vw = in.v1[q4];
                const f32x4 v = {__uint_as_float(vw[0] << 16), __uint_as_float(vw[0] & 0xffff0000u),
                                 __uint_as_float(vw[1] << 16), __uint_as_float(vw[1] & 0xffff0000u)};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    zb += z[e] * y[e];
                    vy += (v[e] - y[e]) * (br * z[e]);
                }
            }
#pragma unroll
            for (int m = 1; m < 8; m <<= 1) {
                zb += __shfl_xor(zb, m, 64);
                vy += __shfl_xor(vy, m, 64);
                qo += __shfl_xor(qo, m, 64);
            }
            if ((t & 7) == 0) {
                sm.dbe[r] = ok ? zb : 0.f;       // dbeta: Z . Y (through V' = T diag(beta) Y)
                sm.dgam[r] = ok ? qo - vy : 0.f; // dgamma: the output's e^gamma Q S term, the e^gamma K S term of Y
            }
        }
        __syncthreads();
        // step 3's tiles: this wave's row tile and pair of column tiles
        const int prt = w >> 1, pct0 = 2 * (w & 1), ra = 16 * prt + c;
        // the operands read from memory (K rows ra and rb, dV' row ra, Y rows rb), one k step ahead
        struct Ops3 {
            u32x2 ka[2], kb[2][2];
            f32x4 dv[2], y[2][2];
        };
        const float brb[2] = {sm.bet[16 * pct0 + c], sm.bet[16 * (pct0 + 1) + c]};
        auto load3 = [&](Ops3& o, int ks) {
            const bf16* kra = Kg + (size_t)min(ra, nv - 1) * ts + 32 * ks + 4 * g;
            o.ka[0] = *reinterpret_cast<const u32x2*>(kra);
            o.ka[1] = *reinterpret_cast<const u32x2*>(kra + 16);
            const float* dvr = dVb + (size_t)ra * DK + 32 * ks + 4 * g;
            o.dv[0] = *reinterpret_cast<const f32x4*>(dvr);
            o.dv[1] = *reinterpret_cast<const f32x4*>(dvr + 16);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int rb = 16 * (pct0 + j) + c;
                const float* yr = Yb + (size_t)rb * DK + 32 * ks + 4 * g;
                o.y[j][0] = *reinterpret_cast<const f32x4*>(yr);
                o.y[j][1] = *reinterpret_cast<const f32x4*>(yr + 16);
                const bf16* krb = Kg + (size_t)min(rb, nv - 1) * ts + 32 * ks + 4 * g;
                o.kb[j][0] = *reinterpret_cast<const u32x2*>(krb);
                o.kb[j][1] = *reinterpret_cast<const u32x2*>(krb + 16);
            }
        };
        Ops3 cur;   // its first k step's operands, issued at the end of step 2
        // ---- 2. d_k-column products: dq = diag(scale e^gamma) dO S^T, dk = diag(f) V' dSn^T - diag(e^gamma) dY S^T.
        // The token-row operands (dO, dY = diag(beta) Z, V'), which every wave needs, are staged once in LDS
        // (rows with d_v in kp order; the image slots sa .. sc are free until step 3): first dO and dY, then V'.
        f32x4 dq[4], dk[4];
        {
            bf16* st = sm.sa;                          // 60 KiB: sa, sb, sc
            bf16* st_do = st;                          // [64][LDQ] dO (kept through step 3's dP)
            bf16* st_x = st + CH * LDQ;                // [128][LDQ] dY, then V': hi rows, then lo rows
            static_assert(sizeof(sm.sa) + sizeof(sm.sb) + sizeof(sm.sc) >= 3 * CH * LDQ * sizeof(bf16), "staging fits");
            // hi and lo bf16 rows of fp32 pieces held in registers
            auto put_f32 = [&](bf16* dst, const f32x4 (&x)[4]) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {   // piece t + 512 j: row / 32, four d_v at 4 (piece % 32)
                    const int idx = t + NTHR_CH * j, r = idx >> 5, c4 = (idx & 31) * 4;
                    bf16x4 hi, lo;
                    split4(x[j], hi, lo);
                    *reinterpret_cast<bf16x4*>(dst + r * LDQ + kp(c4)) = hi;
                    *reinterpret_cast<bf16x4*>(dst + (CH + r) * LDQ + kp(c4)) = lo;
                }
            };
#pragma unroll
            for (int j = 0; j < 4; ++j) {   // dO, rows past the end zero; dY = diag(beta) Z
                const int idx = t + NTHR_CH * j, r = idx >> 5, c4 = (idx & 31) * 4;
                *reinterpret_cast<u32x2*>(st_do + r * LDQ + kp(c4)) = r < nv ? dox[j] : u32x2{0u, 0u};
                zx[j] *= sm.bet[r];
            }
            put_f32(st_x, zx);
            f32x4 aq[4], a1[4], a2[4];
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) aq[rt] = a1[rt] = a2[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
            // this thread's V' pieces and this wave's dSn row, in flight through the dO and dY products
            f32x4 vpx[4], drow[4][2];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int idx = t + NTHR_CH * j;
                vpx[j] = *reinterpret_cast<const f32x4*>(Vpb + (size_t)(idx >> 5) * DK + (idx & 31) * 4);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                drow[ks][0] = *reinterpret_cast<const f32x4*>(Drow + 32 * ks + 4 * g);
                drow[ks][1] = *reinterpret_cast<const f32x4*>(Drow + 32 * ks + 16 + 4 * g);
            }
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 sh, sl;
                split8(srow[ks][0], srow[ks][1], sh, sl);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int o = (16 * rt + c) * LDQ + 32 * ks + 8 * g;
                    const bf16x8 ao = lds_op16(st_do + o);
                    aq[rt] = mma16k32(ao, sh, aq[rt]);
                    aq[rt] = mma16k32(ao, sl, aq[rt]);
                    const bf16x8 yh = lds_op16(st_x + o), yl = lds_op16(st_x + CH * LDQ + o);
                    a2[rt] = mma16k32(yh, sh, a2[rt]);
                    a2[rt] = mma16k32(yh, sl, a2[rt]);
                    a2[rt] = mma16k32(yl, sh, a2[rt]);
                }
            }
            // dgamma_C from the decay of the state, e^gamma_C <S, dSn>: this wave's 16 rows
            // of both are in its registers (this lane's part; summed with the kappas below)
            float sdp = 0.f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) sdp += dot4v(srow[ks][0], drow[ks][0]) + dot4v(srow[ks][1], drow[ks][1]);
            __syncthreads();   // dY read by every wave: V' takes its place
            put_f32(st_x, vpx);
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 dh, dl;
                split8(drow[ks][0], drow[ks][1], dh, dl);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int o = (16 * rt + c) * LDQ + 32 * ks + 8 * g;
                    const bf16x8 vh = lds_op16(st_x + o), vl = lds_op16(st_x + CH * LDQ + o);
                    a1[rt] = mma16k32(vh, dh, a1[rt]);
                    a1[rt] = mma16k32(vh, dl, a1[rt]);
                    a1[rt] = mma16k32(vl, dh, a1[rt]);
                }
            }
            load3(cur, 0);
            float kps[16];   // this wave's 16 columns' parts of kappa for row 16 rt + 4 g + e, at 4 rt + e
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int r0 = 16 * rt + 4 * g;
                const f32x4 eg = *reinterpret_cast<const f32x4*>(sm.eg + r0);
                const f32x4 fr = *reinterpret_cast<const f32x4*>(sm.fr + r0);
                dq[rt] = (scale * eg) * aq[rt];
                dk[rt] = fr * a1[rt] - eg * a2[rt];
                // kappa_r = f_r K_r . dK~_r: through the decay factors of K~
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = r0 + e;
                    // K[r][16 w + c] from the staged K^T (rows past the end hold the last row, as in Kg)
                    const int dkc = 16 * w + c;
                    const float kv = (float)sm.kt[dkc * LDKT + ((kp(r & ~3) ^ tswz(dkc)) | (r & 3))];
                    kps[4 * rt + e] = fr[e] * kv * a1[rt][e];
                }
            }
            {   // lane c holds kappa of row 16 (c / 4) + 4 g + c % 4; dgamma_C takes every kappa
                const float kap = tile_rowsums(kps, c);
                const int r = 16 * (c >> 2) + 4 * g + (c & 3);
                if (r < nv) atomicAdd(&sm.dgam[r], -kap);
                float part = __expf(sm.gam[CH - 1]) * sdp + (r < nv ? kap : 0.f);
#pragma unroll
                for (int m = 1; m < 64; m <<= 1) part += __shfl_xor(part, m, 64);
                if (lane == 0) atomicAdd(&sm.dgc, part);
            }
        }
        // ---- 3. 64 x 64 tiles: dP -> Psi (images), dT (image), K K^T (kept)
        f32x4 kkt[2];
        {
            f32x4 dp[2], dt[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) dp[j] = dt[j] = kkt[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            const bf16* st_do = sm.sa;                       // staged in step 2 (dO, then V' hi / lo rows)
            const bf16* st_v = sm.sa + CH * LDQ;
            // the fp32 P entries of this wave's dP tiles (for dP o P after the loop),
            // loaded in the last k step in place of that step's operands
            float pP[2][4];
            Ops3 nxt;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks < 3) {
                    load3(nxt, ks + 1);
                } else {
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            pP[j][e] = tp[(16 * prt + 4 * g + e) * CH + 16 * (pct0 + j) + c];
                }
                const bf16x8 ao = lds_op16(st_do + ra * LDQ + 32 * ks + 8 * g);
                const bf16x8 ak = __builtin_bit_cast(bf16x8, u32x4{cur.ka[0][0], cur.ka[0][1], cur.ka[1][0], cur.ka[1][1]});
                bf16x8 adh, adl;
                split8(cur.dv[0], cur.dv[1], adh, adl);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int rb = 16 * (pct0 + j) + c;
                    bf16x8 yh, yl;
                    const bf16x8 vh = lds_op16(st_v + rb * LDQ + 32 * ks + 8 * g);
                    const bf16x8 vl = lds_op16(st_v + (CH + rb) * LDQ + 32 * ks + 8 * g);
                    dp[j] = mma16k32(ao, vh, dp[j]);
                    dp[j] = mma16k32(ao, vl, dp[j]);
                    split8(cur.y[j][0] * brb[j], cur.y[j][1] * brb[j], yh, yl);
                    dt[j] = mma16k32(adh, yh, dt[j]);
                    dt[j] = mma16k32(adh, yl, dt[j]);
                    dt[j] = mma16k32(adl, yh, dt[j]);
                    const bf16x8 bk =
                        __builtin_bit_cast(bf16x8, u32x4{cur.kb[j][0][0], cur.kb[j][0][1], cur.kb[j][1][0], cur.kb[j][1][1]});
                    kkt[j] = mma16k32(ak, bk, kkt[j]);
                }
                if (ks < 3) cur = nxt;
            }
            __syncthreads();   // the staging area becomes the image slots again
            float es[4] = {0.f, 0.f, 0.f, 0.f};   // row 16 prt + 4 g + e's part of dP o P, both tiles
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int ct = pct0 + j, m = 16 * ct + c;
                f32x4 psi, E;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * prt + 4 * g + e;
                    const float d = scale * dp[j][e];
                    const bool low = m <= r;
                    psi[e] = low ? d * __expf(sm.gam[r] - sm.gam[m]) : 0.f;
                    E[e] = low ? d * pP[j][e] : 0.f;   // dP o P (P is the fp32 copy)
                }
                put_img(sm.sa, prt, ct, c, g, psi);
                put_img_t(sm.sb, prt, ct, c, g, psi);
                put_img(sm.sc, prt, ct, c, g, dt[j]);
#pragma unroll
                for (int e = 0; e < 4; ++e) es[e] += E[e];
                const float cs = tile_colsum(E);
                if (g == 0) atomicAdd(&sm.dgam[m], -cs);
            }
            const float rs = tile_rowsums(es, c);   // row 16 prt + 4 g + c / 4
            if ((c & 3) == 0) atomicAdd(&sm.dgam[16 * prt + 4 * g + (c >> 2)], rs);
        }
        __syncthreads();
        // ---- 4. W1 = dT T^T (tiles); dq += Psi K; dk += Psi^T Q
        f32x4 w1[2];
        {
#pragma unroll
            for (int j = 0; j < 2; ++j) w1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int oa = (16 * prt + c) * LDP + 32 * ks + 8 * g;
                const bf16x8 ah = lds_op16(sm.sc + oa), al = lds_op16(sm.sc + CH * LDP + oa);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int ob = (16 * (pct0 + j) + c) * LDP + 32 * ks + 8 * g;
                    const bf16x8 bh = lds_op16(sm.tim + ob), bl = lds_op16(sm.tim + CH * LDP + ob);
                    w1[j] = mma16k32(ah, bh, w1[j]);
                    w1[j] = mma16k32(ah, bl, w1[j]);
                    w1[j] = mma16k32(al, bh, w1[j]);
                }
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int ob = (16 * w + c) * LDKT + ((32 * ks + 8 * g) ^ (8 * w));
                const bf16x8 kb = lds_op16(sm.kt + ob), qb = lds_op16(sm.qt + ob);
#pragma unroll
                for (int rt = 0; rt < 4; ++rt) {
                    const int oa = (16 * rt + c) * LDP + 32 * ks + 8 * g;
                    dq[rt] = mma16k32(lds_op16(sm.sa + oa), kb, dq[rt]);
                    dq[rt] = mma16k32(lds_op16(sm.sa + CH * LDP + oa), kb, dq[rt]);
                    dk[rt] = mma16k32(lds_op16(sm.sb + oa), qb, dk[rt]);
                    dk[rt] = mma16k32(lds_op16(sm.sb + CH * LDP + oa), qb, dk[rt]);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < 2; ++j) put_img_t(sm.sc, prt, pct0 + j, c, g, w1[j]);   // W1^T
        __syncthreads();
            // the next item's staging and step-1 operands, in flight through steps 5 and 6
        // (after the last item, this one's again: every path issues the loads, so
        // that the operands are dead through steps 2 to 4)
        bwd_item_fetch(p, item + gridDim.x < n_items ? item + gridDim.x : item, in);
        // ---- 5. dA = -T^T W1 (strictly lower) -> dbeta, dgamma, G, G^T (images)
        {
            f32x4 da[2];
            float rsum[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // row 16 prt + 4 g + e: dbeta at e, dgamma at 4 + e
#pragma unroll
            for (int j = 0; j < 2; ++j) da[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int oa = (16 * prt + c) * LDP + 32 * ks + 8 * g;
                const bf16x8 ah = lds_op16(sm.ttim + oa), al = lds_op16(sm.ttim + CH * LDP + oa);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int ob = (16 * (pct0 + j) + c) * LDP + 32 * ks + 8 * g;
                    const bf16x8 bh = lds_op16(sm.sc + ob), bl = lds_op16(sm.sc + CH * LDP + ob);
                    da[j] = mma16k32(ah, bh, da[j]);
                    da[j] = mma16k32(ah, bl, da[j]);
                    da[j] = mma16k32(al, bh, da[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int ct = pct0 + j, i = 16 * ct + c;
                f32x4 G, gA;
                float dbr[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * prt + 4 * g + e;
                    const bool low = i < r;
                    const float ex = low ? __expf(sm.gam[r] - sm.gam[i]) : 0.f;
                    const float dA = low ? -da[j][e] : 0.f;
                    const float wv = dA * ex * kkt[j][e];   // dA_ri times dA_ri / dbeta_r
                    dbr[e] = wv;
                    gA[e] = wv * sm.bet[r];                 // dA_ri A_ri
                    G[e] = dA * sm.bet[r] * ex;
                }
                put_img(sm.sa, prt, ct, c, g, G);
                put_img_t(sm.sb, prt, ct, c, g, G);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    rsum[e] += dbr[e];
                    rsum[4 + e] += gA[e];
                }
                const float cs = tile_colsum(gA);
                if (g == 0) atomicAdd(&sm.dgam[i], -cs);
            }
            // lane c: the sum of value c / 2 (dbeta parts, then dgamma parts) of row 16 prt + 4 g + (c / 2) % 4
            const float rs = tile_rowsums(rsum, c);
            if ((c & 1) == 0) atomicAdd((c < 8 ? sm.dbe : sm.dgam) + 16 * prt + 4 * g + ((c >> 1) & 3), rs);
        }
        __syncthreads();
        // ---- 6. dk += (G + G^T) K
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 kb = lds_op16(sm.kt + (16 * w + c) * LDKT + ((32 * ks + 8 * g) ^ (8 * w)));
#pragma unroll
            for (int rt = 0; rt < 4; ++rt) {
                const int oa = (16 * rt + c) * LDP + 32 * ks + 8 * g;
                dk[rt] = mma16k32(lds_op16(sm.sa + oa), kb, dk[rt]);
                dk[rt] = mma16k32(lds_op16(sm.sa + CH * LDP + oa), kb, dk[rt]);
                dk[rt] = mma16k32(lds_op16(sm.sb + oa), kb, dk[rt]);
                dk[rt] = mma16k32(lds_op16(sm.sb + CH * LDP + oa), kb, dk[rt]);
            }
        }
        // ---- outputs: per-value-head dq, dk parts; dg (reverse cumulative sum of dgamma), dbeta
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * rt + 4 * g + e;
                if (r < nv) {
                    const size_t o = ((tok0 + r) * p.h_v + h) * DK + 16 * w + c;
                    p.dq_part[o] = dq[rt][e];
                    p.dk_part[o] = dk[rt][e];
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
        nw += ((f & 255) == 1);
        ne += (f == 0);
    }
    path[idx] = (nw + ne == 0) ? 3 : (ne == 0 ? 1 : (nw == 0 ? 0 : 2));
}

// ----------------------------------------------------------------------------
// Recurrent decode: the gated delta rule applied token by token to a state
// already in HBM, the step that follows a prefill once generation starts
// (the pages' edge-side agent inference: a long prompt, then one token at a
// time). Per token and (sequence, value head):
//     a = S^T k, u = beta (v - alpha a), S <- alpha S + k u^T,
//     o = scale S^T q = scale (alpha S_old^T q + (k.q) u).
// One workgroup per (sequence, value head), four waves; wave w owns d_v
// columns [32w, 32w + 32) of S and lane l holds rows 16 (l >> 3) .. +15 of
// columns 32w + 4 (l & 7) .. +3 in registers (64 floats). The contractions
// over d_k (S^T k, S^T q and k.q) finish across the eight row groups of a
// wave by lane swaps, so no step needs LDS or a barrier. The kernel is bound
// by the state's HBM traffic: 64 KiB read and 64 KiB written per (sequence,
// head) and call, whatever the number of tokens. The state moves with
// nontemporal loads and stores: each line is touched once, and on MI355X
// the streaming hint took a 256-row call from 3.2 to 5.2 TB/s (measured).
template <typename IO> struct DecIn;
template <> struct DecIn<bf16> { u32x4 k[2], q[2]; u32x2 v; float g, b; };
template <> struct DecIn<float> { f32x4 k[4], q[4], v; float g, b; };

template <typename IO>
__device__ __forceinline__ void dec_load(DecIn<IO>& in, const Params& p, size_t tok, int hq, int h, int row0,
                                         int col) {
    const size_t qk = (tok * p.h_qk + hq) * DK + row0, vo = (tok * p.h_v + h) * DK + col;
    if constexpr (Io<IO>::kExact) {
        const u32x4* kk = reinterpret_cast<const u32x4*>(static_cast<const bf16*>(p.k) + qk);
        const u32x4* qq = reinterpret_cast<const u32x4*>(static_cast<const bf16*>(p.q) + qk);
        in.k[0] = kk[0]; in.k[1] = kk[1];
        in.q[0] = qq[0]; in.q[1] = qq[1];
        in.v = *reinterpret_cast<const u32x2*>(static_cast<const bf16*>(p.v) + vo);
    } else {
        const f32x4* kk = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.k) + qk);
        const f32x4* qq = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.q) + qk);
#pragma unroll
        for (int i = 0; i < 4; ++i) { in.k[i] = kk[i]; in.q[i] = qq[i]; }
        in.v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.v) + vo);
    }
    in.g = p.g[tok * p.h_v + h];
    in.b = p.beta[tok * p.h_v + h];
}

// Element i of sixteen consecutive values (bf16: two u32x4, element 2w in the
// low half of word w).
__device__ __forceinline__ float dec_elem(const u32x4 (&x)[2], int i) {
    const unsigned w = x[i >> 3][(i >> 1) & 3];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
}
__device__ __forceinline__ float dec_elem(const f32x4 (&x)[4], int i) { return x[i >> 2][i & 3]; }
__device__ __forceinline__ f32x4 dec_v(const u32x2& v) {
    return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                 __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 dec_v(const f32x4& v) { return v; }

template <typename IO>
__global__ __launch_bounds__(NTHR) void k_decode(Params p) {
    const int seq = blockIdx.x, h = blockIdx.y, hq = h / p.group;
    const int l = threadIdx.x & 63, rg = l >> 3, row0 = 16 * rg;
    const int col = 32 * (threadIdx.x >> 6) + 4 * (l & 7);
    const size_t soff = state_off(seq, p.h_v, h) + (size_t)row0 * DK + col;
    f32x4 S[16];
    if (p.s_init) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            S[i] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p.s_init + soff + (size_t)i * DK));
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int T = p.seq_len;
    DecIn<IO> cur;
    if (T > 0) dec_load<IO>(cur, p, (size_t)seq * T, hq, h, row0, col);
    for (int t = 0; t < T; ++t) {
        const size_t tok = (size_t)seq * T + t;
        DecIn<IO> nxt = cur;
        if (t + 1 < T) dec_load<IO>(nxt, p, tok + 1, hq, h, row0, col);
        f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float ki = dec_elem(cur.k, i), qi = dec_elem(cur.q, i);
            a += ki * S[i];
            b += qi * S[i];
            kq += ki * qi;
        }
        // sum over the eight row groups (lane bits 3..5)
#pragma unroll
        for (int m = 8; m < 64; m <<= 1) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a[e] += __shfl_xor(a[e], m, 64);
                b[e] += __shfl_xor(b[e], m, 64);
            }
            kq += __shfl_xor(kq, m, 64);
        }
        const float al = __expf(cur.g);
        const f32x4 u = cur.b * (dec_v(cur.v) - al * a);
        const f32x4 o = p.scale * (al * b + kq * u);
        if (rg == 0) {
            const size_t oo = (tok * p.h_v + h) * DK + col;
            if constexpr (Io<IO>::kExact)
                *reinterpret_cast<u32x2*>(static_cast<bf16*>(p.out) + oo) = u32x2{pack_rne(o[0], o[1]),
                                                                                 pack_rne(o[2], o[3])};
            else
                *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + oo) = o;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) S[i] = al * S[i] + dec_elem(cur.k, i) * u;
        cur = nxt;
    }
    if (p.s_final) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            __builtin_nontemporal_store(S[i], reinterpret_cast<f32x4*>(p.s_final + soff + (size_t)i * DK));
    }
}

}  // namespace

// ----------------------------------------------------------------------------
// Launchers

static int launched() { return (int)hipGetLastError(); }

int launch_prep(const Params& p, int io, void* stream) {
    if (p.n_chunks <= 0) return 0;
    const long long items = (long long)p.n_chunks * p.h_v, waves = (items + p.prep_cpw - 1) / p.prep_cpw;
    const dim3 grid((unsigned)((waves + kPrepWaves - 1) / kPrepWaves)), block(64 * kPrepWaves);
    if (p.tb16) {
        if (io == kIoBf16) hipLaunchKernelGGL((k_prep<bf16, true>), grid, block, 0, (hipStream_t)stream, p);
        else hipLaunchKernelGGL((k_prep<float, true>), grid, block, 0, (hipStream_t)stream, p);
    } else {
        if (io == kIoBf16) hipLaunchKernelGGL((k_prep<bf16, false>), grid, block, 0, (hipStream_t)stream, p);
        else hipLaunchKernelGGL((k_prep<float, false>), grid, block, 0, (hipStream_t)stream, p);
    }
    return launched();
}

int launch_wu(const Params& p, int io, void* stream) {
    if (p.n_chunks <= 0) return 0;
    const dim3 grid(p.n_chunks, p.h_v), block(NTHR_CH);
    if (io == kIoBf16) hipLaunchKernelGGL(k_wu<bf16>, grid, block, 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL(k_wu<float>, grid, block, 0, (hipStream_t)stream, p);
    return launched();
}

int launch_cp_prep(const Params& p, int io, void* stream) {
    // one workgroup per (segment slot, part, head); k_cp_prep hands them out
    const dim3 grid((unsigned)(2LL * p.n_segments * p.h_v)), block(NTHR_CH);
    if (io == kIoBf16) hipLaunchKernelGGL(k_cp_prep<bf16>, grid, block, 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL(k_cp_prep<float>, grid, block, 0, (hipStream_t)stream, p);
    return launched();
}

int launch_cp_combine(const Params& p, void* stream) {
    const dim3 block(NTHR);
    const hipStream_t s = (hipStream_t)stream;
    if (p.comb_G <= 0) {
        hipLaunchKernelGGL(k_cp_combine<kCombAll>, dim3(4 * p.n_seqs, p.h_v), block, 0, s, p);
        return launched();
    }
    hipLaunchKernelGGL(k_cp_combine<kCombHead>, dim3(8 * p.comb_J * p.n_seqs, p.h_v), block, 0, s, p);
    int e = launched();
    if (e) return e;
    if (p.comb_J >= 3) {
        hipLaunchKernelGGL(k_cp_combine<kCombGroups>, dim3(4 * p.n_seqs, p.h_v), block, 0, s, p);
        if ((e = launched())) return e;
    }
    if (p.comb_J >= 2) {
        hipLaunchKernelGGL(k_cp_combine<kCombApply>, dim3(4 * (p.comb_J - 1) * p.n_seqs, p.h_v), block, 0, s, p);
        e = launched();
    }
    return e;
}

int launch_debug_path(const Params& p, int32_t* path_out, void* stream) {
    const int n = p.n_seqs * p.h_v;
    if (n <= 0) return 0;
    hipLaunchKernelGGL(k_debug_path, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream, p, path_out);
    return launched();
}

int launch_fwd(const Params& p, int io, void* stream) {
    const dim3 grid(p.n_segments, p.h_v), block(NTHR_CH);
    if (io == kIoBf16) hipLaunchKernelGGL((k_fwd<bf16, false>), grid, block, 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL((k_fwd<float, false>), grid, block, 0, (hipStream_t)stream, p);
    return launched();
}

int launch_fwd_states(const Params& p, int io, void* stream) {
    const dim3 grid(p.n_segments, p.h_v), block(NTHR_CH);
    if (io == kIoBf16) hipLaunchKernelGGL((k_fwd<bf16, true>), grid, block, 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL((k_fwd<float, true>), grid, block, 0, (hipStream_t)stream, p);
    return launched();
}

int launch_decode(const Params& p, int io, void* stream) {
    if (p.n_seqs <= 0) return 0;
    const dim3 grid(p.n_seqs, p.h_v), block(NTHR);
    if (io == kIoBf16) hipLaunchKernelGGL(k_decode<bf16>, grid, block, 0, (hipStream_t)stream, p);
    else hipLaunchKernelGGL(k_decode<float>, grid, block, 0, (hipStream_t)stream, p);
    return launched();
}

int launch_bwd_chain_mma(const BwdParams& p, void* stream) {
    const hipStream_t s = (hipStream_t)stream;
    if (p.n_segments <= 0) return 0;
    if (!p.seg_state) {   // one segment per sequence
        hipLaunchKernelGGL(k_bwd_chain_mma<kBwdWhole>, dim3(p.n_segments, p.h_v), dim3(NTHR_CH), 0, s, p);
        return launched();
    }
    hipLaunchKernelGGL(k_bwd_chain_mma<kBwdMaps>, dim3(2 * p.n_segments, p.h_v), dim3(NTHR_CH), 0, s, p);
    int e = launched();
    if (e) return e;
    // the segment ends: G(P - 2) = H_(P-1), G(s - 1) = M_s G(s) + H_s, in the
    // reversed slots the maps pass wrote, by the forward's segment combine
    // (no initial state: its first boundary takes H alone)
    Params c{};
    c.cu = p.cu;
    c.n_seqs = p.n_seqs;
    c.seq_len = p.seq_len;
    c.h_qk = p.h_qk;
    c.h_v = p.h_v;
    c.group = p.group;
    c.L = p.L;
    c.n_segments = p.n_segments;
    c.warm = p.warm;
    c.seg_state = p.seg_state;
    c.seg_M = p.seg_M;
    c.seg_H = p.seg_H;
    c.seg_GM = p.seg_GM;
    c.seg_GH = p.seg_GH;
    c.comb_G = p.comb_G;
    c.comb_J = p.comb_J;
    if ((e = launch_cp_combine(c, stream))) return e;
    hipLaunchKernelGGL(k_bwd_chain_mma<kBwdRerun>, dim3(p.n_segments, p.h_v), dim3(NTHR_CH), 0, s, p);
    return launched();
}

int launch_bwd_chunk_mma(const BwdParams& p, void* stream) {
    if (p.n_chunks <= 0) return 0;
    // one workgroup per CU (persistent over the items)
    int dev = 0, n_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return (int)e;
    const long long items = (long long)p.n_chunks * p.h_v;
    const unsigned grid = (unsigned)std::min<long long>(items, std::max(n_cu, 1));
    hipLaunchKernelGGL(k_bwd_chunk_mma, dim3(grid), dim3(NTHR_CH), 0, (hipStream_t)stream, p);
    return launched();
}

}  // namespace gdn
