// Internal launch parameters shared by the host code (gdn_api.cpp) and the
// kernels (gdn_kernels.hip). Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kDim = 128;    // d_k == d_v
constexpr int kMaxSegsPerSeq = 2048;  // the combine kernel keeps one flag per segment in LDS
constexpr int kTbHalfs = 6 * 64 * 8;  // fp16 per (chunk, value head) in the T diag(beta) image (6 KiB)
constexpr int kGfFloats = 4 * 64;     // fp32 per (chunk, value head): gate factors of the chain kernels

struct Params {
    // inputs
    const void* q;            // [tokens][h_qk][128]
    const void* k;
    const void* v;            // [tokens][h_v][128]
    const float* g;           // [tokens][h_v]
    const float* beta;        // [tokens][h_v]
    const float* s_init;      // [n_seqs][h_v][128][128] or null (zeros)
    const int32_t* cu;        // [n_seqs + 1] or null (uniform sequences of seq_len)
    // outputs
    void* out;                // [tokens][h_v][128]
    float* s_final;           // [n_seqs][h_v][128][128] or null
    // workspace (segments numbered sequence by sequence)
    float* seg_state;         // [n_segments][h_v][128][128] initial state of segment s >= 1
    float* seg_M;             // [n_segments][h_v][128][128] state map of segment s: S -> M S + H
    float* seg_H;
    int32_t* warm;            // [n_segments][h_v] 1 if the boundary before segment s warms up
    float* seg_GM;            // [n_seqs][comb_J][h_v] a group's composed map CM (combine operands, 64 KiB)
    float* seg_GH;            // [n_seqs][comb_J][h_v] its CH (128 x 128 fp32) and a scratch block of the same size
    int32_t comb_G;           // boundaries per combine group; 0: one chain over all boundaries
    int32_t comb_J;           // combine groups of the longest sequence
    float* prep_T;            // [n_chunks][h_v] blocks of t_stride floats: T split hi/lo (16 KiB) first
    int64_t t_stride;         // floats between consecutive T blocks (>= 64 * 64)
    float* prep_GB;           // [n_chunks][h_v] blocks of gb_stride floats: gamma (64), beta (64)
    int64_t gb_stride;        // floats between consecutive gamma/beta blocks (>= 128)
    int32_t prep_cpw;         // (head, chunk) items per k_prep wave
    float* sink;              // 8 KiB scratch line for stores of rows past a sequence's end
    void* tb16;               // [n_chunks][h_v] fp16 images of T diag(beta) (kTbHalfs each), or null:
                              //   k_prep then writes the split T and gamma, beta (prep_T, prep_GB)
    float* gf16;              // with tb16: [n_chunks][h_v][4][64] gamma log2(e), e^gamma,
                              //   e^(gamma_C - gamma), e^gamma_C (all 64 the same)
    float* chunk_states;      // [n_chunks][h_v][128][128] state entering each chunk (backward recompute)
    float* bwd_y;             // with chunk_states: per (chunk, head) [64][128] fp32 Y = V - diag(e^gamma) K S,
    float* bwd_vp;            //   and V'; and per (chunk, head) [8 waves][64] partial sums over d_v of
    float* bwd_oi;            //   (scale diag(e^gamma) Q S) o dO per token (the output's state term . dO)
    const void* bwd_dout;     //   with chunk_states: the loss gradient of the output (bf16)
    // low-level chunk-prep outputs
    float* prep_gamma;        // [n_chunks][h_v][64]
    float* prep_W;            // [n_chunks][h_v][64][128]
    float* prep_U;
    // sizes and options
    int32_t n_seqs;
    int32_t seq_len;          // tokens per sequence when cu == null (decode: tokens per row)
    int32_t h_qk, h_v, group; // group = h_v / h_qk
    int32_t L;                // chunks per segment
    int32_t dv_split;         // column blocks of d_v in the fused forward (1, 2 or 4; bf16 inputs)
    int32_t w;                // warm-up chunks
    int32_t cp_mode;          // gdn_cp_mode
    int32_t n_segments;
    int32_t n_chunks;
    int32_t cp_order;         // k_cp_prep work order: 1 exact boundaries first, 0 head-major
    int32_t cp_split;         // bf16 CP preprocessing: 1 H and M of an exact boundary in two workgroups
    float log_eps;            // log(noise floor)
    float scale;
};

enum IoType { kIoBf16 = 0, kIoF32 = 1 };

// Records a failed call's message for gdn_last_error (printf format) and
// returns status (a gdn_status value).
int record_error(int status, const char* fmt, ...);

// Backward pass (gdn_bwd.hip). Chunks are numbered sequence by sequence as in
// the forward; states are [128][128] fp32 blocks in the API layout.
constexpr int kBwdTpg = kChunk * kChunk + kChunk;       // floats per (chunk, head): P, gamma
constexpr int kBwdTpt = 6 * kChunk * kChunk;            // bf16 per (chunk, head) in the T^T / P^T / T images

struct BwdParams {
    const void* q;            // [tokens][h_qk][128] bf16 (fp32 inputs: their bf16 rounding)
    const void* k;
    const void* v;            // [tokens][h_v][128] bf16
    const float* g;           // [tokens][h_v]
    const float* beta;
    const void* dout;         // [tokens][h_v][128] bf16: loss gradient of the output
    const float* dfinal;      // [n_seqs][h_v][128][128] loss gradient of the final state, or null
    const int32_t* cu;        // [n_seqs + 1] or null (uniform sequences of seq_len)
    void* dq;                 // [tokens][h_qk][128] bf16, fp32 if out_f32
    void* dk;
    void* dv;                 // [tokens][h_v][128] bf16, fp32 if out_f32
    float* dg;                // [tokens][h_v]
    float* dbeta;
    float* dinit;             // [n_seqs][h_v][128][128] or null
    // workspace
    const float* cs;          // [n_chunks][h_v] state entering each chunk (from the forward)
    float* ds;                // [n_chunks][h_v] loss gradient of the state leaving each chunk
    float* tpg;               // [n_chunks][h_v] blocks of kBwdTpg floats: P (row-major 64 x 64), gamma
    void* tpt;                // [n_chunks][h_v] bf16 images for the matrix cores: [T^T hi, T^T lo,
                              // scale P^T hi, lo, T hi, lo], rows of 64, contraction token in kp order
    const float* y;           // [n_chunks][h_v][64][128] fp32 from the forward re-run: Y, V', scale e^gamma Q S
    const float* vp;
    const float* oi;
    float* dvp;               // [n_chunks][h_v][64][128] fp32 from the state-gradient scan: dV', Z = T^T dV'
    float* z;
    float* dq_part;           // [tokens][h_v][128] per-value-head parts of dq and dk
    float* dk_part;
    // segments of the state-gradient scan (the forward's plan); seg_state null: one per sequence
    float* seg_state;         // [n_segments][h_v] gradient of the state leaving segment s (s < P - 1)
    float* seg_M;             // [n_segments][h_v] map of segment s >= 1 (gradient at its end -> at its start)
    float* seg_H;             // [n_segments][h_v] the scan of segment s >= 1 from zero (last: from dS_final)
                              // (seg_M, seg_H: segment s in slot P - 1 - s of its sequence, M in the
                              // combine's operand layout; seg_state: gradient leaving s in slot P - 1 - s)
    int32_t* warm;            // [n_segments][h_v] boundary flags for the combine (all exact)
    float* seg_GM;            // the combine's group maps (comb_G > 0)
    float* seg_GH;
    int32_t comb_G, comb_J;   // the forward plan's combine grouping
    int32_t L, n_segments;    // chunks per segment, segments over all sequences
    int32_t n_seqs, seq_len, h_qk, h_v, group, n_chunks;
    int32_t out_f32;          // dq, dk, dv written as fp32 (the caller's inputs were fp32)
    float scale;
};

int launch_bwd(const BwdParams& p, void* stream);                       // prep, chain, chunk gradients
int launch_bwd_sum(const BwdParams& p, long long n_tokens, void* stream);  // dq, dk group sums
int launch_bwd_chain_mma(const BwdParams& p, void* stream);                // dS scan on matrix cores
int launch_bwd_chunk_mma(const BwdParams& p, void* stream);                // chunk gradients on matrix cores
int launch_round_bf16(const float* x, void* y, long long n, void* stream);  // fp32 -> bf16 (RNE), n % 4 == 0

// Kernel launchers (gdn_kernels.hip). Return 0 or a hipError_t value.
int launch_prep(const Params& p, int io, void* stream);
int launch_wu(const Params& p, int io, void* stream);
int launch_cp_prep(const Params& p, int io, void* stream);
int launch_cp_combine(const Params& p, void* stream);
int launch_fwd(const Params& p, int io, void* stream);
int launch_fwd_states(const Params& p, int io, void* stream);
int launch_debug_path(const Params& p, int32_t* path_out, void* stream);
int launch_decode(const Params& p, int io, void* stream);

// The forward's fp16 chain kernels (gdn_fwd16.hip); k_prep writes their
// T diag(beta) images when Params::tb16 is set.
int launch_cp_prep16(const Params& p, int io, void* stream);
int launch_combine16(const Params& p, void* stream);
int launch_fwd16(const Params& p, int io, void* stream);
int launch_tiles_to_rm(const float* src, float* dst, long long n_blocks, void* stream);

}  // namespace gdn
