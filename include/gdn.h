/*
 * gdn.h -- C ABI of the Gated DeltaNet chunked-prefill forward for AMD MI355X
 * (gfx950), with gate-driven intra-card context parallelism.
 *
 * Sources (the FlashQLA pages, "FlashQLA: CP-/Bwd-friendly fused linear
 * attention kernels for GDN"):
 *   - section on optimising GDN chunked prefill: the prefill evaluates the
 *     Gated DeltaNet recurrence chunk by chunk; the intermediates W, U and S
 *     should not round-trip through HBM, and the per-(batch, head) recurrence
 *     alone cannot fill the GPU at small batch or under tensor parallelism;
 *   - section "Gate-Driven Automatic Intra-Card Context Parallelism (AutoCP)":
 *     each sequence is cut into segments ("CP ranks") of L = lambda * sqrt(N)
 *     chunks (N = chunks in the sequence); a segment's initial state comes from
 *     the exact correction matrix M or, for heads whose gate decay drives the
 *     old state below a noise floor, from a 6-8 chunk warm-up;
 *   - section "Implementation & requirements": a high-level API with FLA's
 *     argument order plus low-level entry points.
 * The recurrence (gated delta rule, state stored d_k x d_v):
 *     S_t = exp(g_t) S_{t-1} + beta_t k_t (v_t - exp(g_t) S_{t-1}^T k_t)^T
 *     o_t = scale * S_t^T q_t
 * Value head h reads query/key head h / (h_v / h_qk).
 *
 * Every entry point returns a gdn_status; none throws or aborts. A failed call
 * leaves a message readable with gdn_last_error() (per thread). Calls that
 * launch work do so asynchronously on the caller's HIP stream and never
 * synchronise the host; faults inside kernels surface at the caller's next
 * synchronisation. The library keeps no pointer after a call returns and
 * allocates no device memory: all scratch lives in the caller's workspace.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL_ARG = 1,        /* a required pointer is NULL */
    GDN_ERR_BAD_SHAPE = 2,       /* sizes negative/inconsistent, h_v % h_qk != 0, bad seqlens */
    GDN_ERR_UNSUPPORTED_DIM = 3, /* d_k or d_v other than 128 */
    GDN_ERR_BAD_DTYPE = 4,       /* io_dtype not a gdn_dtype */
    GDN_ERR_MISALIGNED = 5,      /* a tensor pointer not 16-byte aligned */
    GDN_ERR_BAD_SCALE = 6,       /* scale not finite */
    GDN_ERR_WORKSPACE_TOO_SMALL = 7,
    GDN_ERR_BAD_OPTION = 8,      /* cp_mode, lambda, warmup_chunks or noise_floor out of range */
    GDN_ERR_HIP = 9              /* a HIP runtime call or kernel launch failed */
} gdn_status;

/* Element type of q, k, v and out. g, beta and every state are always fp32. */
typedef enum { GDN_BF16 = 0, GDN_F32 = 1 } gdn_dtype;

/* How segment initial states are obtained when a sequence is split. */
typedef enum {
    GDN_CP_AUTO = 0,    /* split only if (sequences x heads) leave CUs idle; path per head from the gates */
    GDN_CP_OFF = 1,     /* one segment per sequence */
    GDN_CP_EXACT = 2,   /* split; every head uses the exact (M, H) composition */
    GDN_CP_WARMUP = 3   /* split; every head uses the warm-up (approximate for slow-decay heads) */
} gdn_cp_mode;

/* Problem descriptor.
 * Layouts (row-major, contiguous):
 *   q, k          [B, T, h_qk, d_k]      io_dtype
 *   v, out        [B, T, h_v, d_v]       io_dtype
 *   g, beta       [B, T, h_v]            fp32; g = log(alpha) must be finite and <= 0
 *   states        [n_seqs, h_v, d_k, d_v] fp32 (initial_state, final_state)
 *   cu_seqlens    [n_seqs + 1] int32 token offsets, 0 = c_0 <= c_1 <= ... = T;
 *                 only with B == 1 (packed variable-length sequences).
 * Without cu_seqlens the B rows are the sequences (n_seqs == B). */
typedef struct {
    int32_t B, T, h_qk, h_v, d_k, d_v;
    int32_t n_seqs;                    /* B, or len(cu_seqlens) - 1 */
    const int32_t* host_cu_seqlens;    /* host copy of cu_seqlens; set = packed sequences */
    int32_t io_dtype;                  /* gdn_dtype */
    int32_t cp_mode;                   /* gdn_cp_mode */
    float lambda;                      /* L = lambda * sqrt(N); 0 = library default */
    int32_t warmup_chunks;             /* warm-up window in chunks, 1..8; 0 = default (6) */
    float noise_floor;                 /* warm-up accepted if window decay <= this; 0 = default 1e-4 */
    int32_t n_cu;                      /* compute units to plan for; 0 = query the current device */
    int32_t dv_split;                  /* column blocks of d_v the forward runs in parallel: 1, 2 or 4
                                          (bf16 inputs, without a context-parallel split: cp_mode
                                          AUTO or OFF); 0 = the planner decides (see gdn_plan) */
    int32_t cp_layout;                 /* workgroups of the boundary preprocessing (bf16 inputs; fp32
                                          inputs have one layout and ignore it): 1 = one per boundary,
                                          an exact boundary's H and M chains sharing its staged chunks;
                                          2 = H and M of an exact boundary in two workgroups; 0 = the
                                          planner decides (2 when every boundary of the plan fits on
                                          the CUs at once, else 1) */
} gdn_desc;

/* Result of planning (host-only arithmetic on the descriptor). */
typedef struct {
    int32_t chunk;           /* chunk length in tokens (64) */
    int32_t n_chunks_total;  /* chunks over all sequences */
    int32_t n_chunks_max;    /* chunks of the longest sequence (N in L = lambda sqrt(N)) */
    int32_t cp_on;           /* 1 if any sequence is split into more than one segment */
    int32_t L;               /* chunks per segment */
    int32_t n_segments;      /* segments over all sequences (workgroups per head in the forward) */
    int32_t P_max;           /* most segments of one sequence */
    int32_t warmup_chunks;
    int32_t n_cu;
    float lambda;
    float noise_floor;
    size_t workspace_bytes;  /* what gdn_fwd needs for this descriptor */
    int32_t combine_group;   /* boundaries per group of the forward's grouped combine (0: one chain) */
    int32_t combine_groups;  /* its groups in the longest sequence (0: one chain) */
    int32_t dv_split;        /* column blocks of d_v in the forward (1: none) */
    int32_t cp_layout;       /* boundary preprocessing layout run (1 or 2, as in gdn_desc); 0 without
                                a context-parallel split or with fp32 inputs */
} gdn_plan_info;

/* Plan a forward (section "Gate-Driven Automatic Intra-Card Context
 * Parallelism (AutoCP)" for the split; the section on optimising GDN chunked
 * prefill for why one (sequence, head) per workgroup leaves CUs idle): chunk
 * counts, the segment length L <= lambda sqrt(N) (N = chunks of the longest
 * sequence) and the workspace size. When sequences x value heads alone leave
 * CUs idle, AUTO either splits the sequences into segments (L chosen so that
 * the segments fill the CUs in whole rounds) or, for bf16 inputs, splits d_v
 * into 2 or 4 column blocks (the columns of the state evolve independently)
 * when that fills the CUs and its estimated time is lower. Host arithmetic
 * only, except that n_cu == 0 queries the current device's compute-unit count. */
gdn_status gdn_plan(const gdn_desc* desc, gdn_plan_info* out);

/* Workspace bytes gdn_fwd needs for desc (0 and a message on an invalid desc):
 * the plan's per-chunk T diag(beta) images and gate factors, and with an
 * AutoCP split (section "Gate-Driven Automatic Intra-Card Context Parallelism
 * (AutoCP)") the boundary states, maps and flags. */
size_t gdn_fwd_workspace_bytes(const gdn_desc* desc);

/* The forward pass (the chunked-prefill forward of the FlashQLA pages, section on
 * optimising GDN chunked prefill, with the AutoCP split of the AutoCP section).
 *   q, k, v, g, beta   device inputs (layouts above), 16-byte aligned
 *   scale              read-out scale (callers usually pass d_k^-1/2)
 *   initial_state      device [n_seqs, h_v, d_k, d_v] fp32, or NULL for zeros
 *   cu_seqlens         device int32 [n_seqs + 1]; required exactly when
 *                      desc->host_cu_seqlens is set (the same values on the host)
 *   out                device output, same layout and dtype as v
 *   final_state        device [n_seqs, h_v, d_k, d_v] fp32, or NULL to skip
 *   workspace          device scratch of at least gdn_fwd_workspace_bytes(desc) bytes,
 *                      256-byte aligned; its contents on entry are ignored. It holds
 *                      T = (I + A)^-1 (16 KiB) and the chunk's gate sums and beta
 *                      (512 bytes) per (chunk, value head), and with a split the
 *                      segment states, the maps M and H (64 KiB per segment and
 *                      value head each), the boundary flags and, with a grouped
 *                      combine, each group's composed map (192 KiB per group and
 *                      value head)
 *   stream             the hipStream_t to launch on (NULL = default stream)
 * All buffers stay owned by the caller and must stay valid until the stream
 * has run the launched kernels. Arguments are validated before any launch. */
gdn_status gdn_fwd(const gdn_desc* desc,
                   const void* q, const void* k, const void* v,
                   const float* g, const float* beta, float scale,
                   const float* initial_state, const int32_t* cu_seqlens,
                   void* out, float* final_state,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. gdn_fwd with the same arguments except the workspace, which
 * lives in a scratch array the library holds on every device it runs on
 * (GDN_NOALLOC_SCRATCH_BYTES per device, kept until the process ends). A
 * descriptor whose gdn_fwd_workspace_bytes exceed it fails with
 * GDN_ERR_WORKSPACE_TOO_SMALL before any launch. The call allocates nothing
 * (the array's device address is looked up on the first call on each device).
 * Every call on one device shares that device's array, which keeps the last
 * call's contents (gdn_fwd reads no workspace byte it has not written, so
 * nothing needs clearing): calls that can overlap on one device -- on
 * different streams, or from host threads without ordering -- race and must
 * be serialised by the caller. Same ownership and error behaviour as gdn_fwd. */
#define GDN_NOALLOC_SCRATCH_BYTES (80u << 20)
gdn_status gdn_fwd_noalloc(const gdn_desc* desc,
                           const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float scale,
                           const float* initial_state, const int32_t* cu_seqlens,
                           void* out, float* final_state, void* stream);

/* gdn_fwd, then copies of what the context-parallel step decided (section
 * "Gate-Driven Automatic Intra-Card Context Parallelism (AutoCP)"):
 *   seg_state_out  device fp32 [n_segments, h_v, d_k, d_v]: the initial state of
 *                  every segment (segments numbered sequence by sequence) as the
 *                  forward used it; NULL to skip
 *   path_out       device int32 [n_seqs, h_v], over the boundaries whose
 *                  warm-up window does not reach the sequence start (those
 *                  warm up from the initial state, which is exact):
 *                  1 = all warmed up, 0 = all exact, 2 = mixed, 3 = no such
 *                  boundary, -1 = the sequence was not split; NULL to skip
 * Same ownership and error behaviour as gdn_fwd. */
gdn_status gdn_fwd_debug(const gdn_desc* desc,
                         const void* q, const void* k, const void* v,
                         const float* g, const float* beta, float scale,
                         const float* initial_state, const int32_t* cu_seqlens,
                         void* out, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream,
                         float* seg_state_out, int32_t* path_out);

/* Low-level entry: the chunk-preparation step alone (gate cumsum, masked
 * beta K K^T, triangular inverse, WY factors; the "fused kernel 1" role of the
 * section on optimising GDN chunked prefill), written out for inspection:
 *   gamma_out  device fp32 [n_chunks_total, h_v, 64]: chunk-local cumulative sum of g
 *   W_out      device fp32 [n_chunks_total, h_v, 64, d_k]: T diag(beta exp(gamma)) K
 *   U_out      device fp32 [n_chunks_total, h_v, 64, d_v]: T diag(beta) V
 * with T = (I + A)^-1, A[i][j] = beta_i exp(gamma_i - gamma_j) k_i.k_j for i > j.
 * Chunks are numbered sequence by sequence; rows past the end of a short final
 * chunk are what zero padding (g = beta = 0, k = v = 0) gives. The forward
 * itself never writes these to memory. */
gdn_status gdn_chunk_prep(const gdn_desc* desc,
                          const void* k, const void* v,
                          const float* g, const float* beta, const int32_t* cu_seqlens,
                          float* gamma_out, float* W_out, float* U_out, void* stream);

/* Calibration of lambda (the AutoCP segment length L = lambda * sqrt(N) of the
 * section "Gate-Driven Automatic Intra-Card Context Parallelism (AutoCP)";
 * the pages fix no lambda): times the forward on the caller's inputs for each
 * candidate and returns the fastest, for the caller to put into later
 * descriptors. Each candidate runs once untimed, then reps times between two
 * HIP events on the stream; the call synchronises the host on those events.
 *   desc, q, k, v, g, beta, scale, cu_seqlens, out   as for gdn_fwd (no states)
 *   workspace          at least gdn_fwd_workspace_bytes for every candidate
 *   lambdas            host array of n_lambdas (1..64) finite values > 0
 *   reps               timed forwards per candidate (1..1000)
 *   ms_out             host float[n_lambdas]: mean ms per forward, or NULL
 *   best_lambda        host float: the fastest candidate
 * Candidates are validated (descriptor, workspace) before anything runs. */
gdn_status gdn_calibrate_lambda(const gdn_desc* desc,
                                const void* q, const void* k, const void* v,
                                const float* g, const float* beta, float scale,
                                const int32_t* cu_seqlens, void* out,
                                void* workspace, size_t workspace_bytes,
                                const float* lambdas, int32_t n_lambdas, int32_t reps,
                                void* stream, float* ms_out, float* best_lambda);

/* Backward pass: the gradients of gdn_fwd's outputs with respect to its
 * inputs (the FlashQLA pages' title promises a backward-friendly design; they
 * print no backward formulas, so this is the exact gradient of the gated delta
 * rule, evaluated on the chunked form). Given the loss gradient of the output
 * and, optionally, of the final state, returns those of q, k, v, g, beta and,
 * optionally, of the initial state. Internally the forward runs again (same
 * plan, so with AutoCP the warm-up boundaries carry the same approximation as
 * gdn_fwd), writing the state that enters every chunk; the state gradient is
 * then scanned backwards over the chunks and every chunk's gradients are
 * formed in parallel.
 *   desc, q, k, v, g, beta, scale, initial_state, cu_seqlens   as for gdn_fwd
 *                      (GDN_F32: q, k, v and d_out are rounded once to bf16 in the
 *                      workspace and the bf16 computation runs on them; the
 *                      gradients are then written in fp32)
 *   d_out              device [B, T, h_v, d_v] io_dtype, loss gradient of the output
 *   d_final_state      device [n_seqs, h_v, d_k, d_v] fp32, or NULL for zero
 *   dq, dk             device [B, T, h_qk, d_k] io_dtype (summed over the value
 *                      heads that share a query/key head)
 *   dv                 device [B, T, h_v, d_v] io_dtype
 *   dg, dbeta          device [B, T, h_v] fp32
 *   d_initial_state    device [n_seqs, h_v, d_k, d_v] fp32, or NULL to skip
 *   workspace          device scratch of at least gdn_bwd_workspace_bytes(desc)
 *                      bytes, 256-byte aligned (the forward's workspace, then per
 *                      (chunk, value head) two 64 KiB states, 16.25 KiB of P and
 *                      gamma, 48 KiB of bf16 images of T^T, P^T and T, four 32 KiB
 *                      intermediates and 2 KiB of output-term sums, and per token
 *                      and value head 1 KiB;
 *                      GDN_F32 adds the bf16 copies of q, k, v and d_out)
 * Same ownership and error behaviour as gdn_fwd. */
size_t gdn_bwd_workspace_bytes(const gdn_desc* desc);
gdn_status gdn_bwd(const gdn_desc* desc,
                   const void* q, const void* k, const void* v,
                   const float* g, const float* beta, float scale,
                   const float* initial_state, const int32_t* cu_seqlens,
                   const void* d_out, const float* d_final_state,
                   void* dq, void* dk, void* dv, float* dg, float* dbeta,
                   float* d_initial_state,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Recurrent decode: the gated delta rule of the section on optimising GDN
 * chunked prefill applied token by token, continuing from a state a prefill
 * (gdn_fwd's final_state) or an earlier decode call left, as generation does
 * after the prompt (the pages' opening: edge-side agent inference, where a
 * long prefill is followed by token-by-token output). Per token and value
 * head: S <- exp(g) S + beta k (v - exp(g) S^T k)^T, o = scale S^T q, with the
 * updated S. desc gives B rows (sequences) of T tokens each (T = 1 for one
 * token; T = 0 only copies the state); desc->host_cu_seqlens must be NULL and
 * the context-parallel options are ignored.
 *   q, k, v, g, beta  device inputs in the gdn_fwd layouts with B rows of T tokens
 *   scale             read-out scale
 *   state_in          device [B, h_v, d_k, d_v] fp32 state before the first token,
 *                     or NULL for zeros
 *   state_out         device [B, h_v, d_k, d_v] fp32 state after the last token, or
 *                     NULL to skip; may be the same pointer as state_in (updated in
 *                     place) but must not overlap it otherwise
 *   out               device output, layout and dtype of v
 *   stream            the hipStream_t to launch on (NULL = default stream)
 * One kernel launch, no workspace. Reads and writes each state once per call
 * (the state stays in registers across the T tokens). Same ownership and
 * error behaviour as gdn_fwd. */
gdn_status gdn_decode(const gdn_desc* desc,
                      const void* q, const void* k, const void* v,
                      const float* g, const float* beta, float scale,
                      const float* state_in, float* state_out, void* out, void* stream);

/* Measurement support. While enabled (on != 0), every gdn_fwd / gdn_fwd_debug
 * call records HIP events on its stream before its first launch and after
 * each of its kernels; gdn_profile_read then waits for the last call's events
 * and returns elapsed milliseconds:
 *   ms[0] chunk preparation (T of every chunk), ms[1] cp_prep,
 *   ms[2] cp_combine, ms[3] forward kernel, ms[4] whole call
 * (phases that did not run read 0). Process-wide state, not thread-safe; the
 * events are created on the first enable, on the current device. */
gdn_status gdn_profile_enable(int on);
gdn_status gdn_profile_read(float ms[5]);

/* Static text for a status code. */
const char* gdn_status_string(gdn_status status);

/* Detail of the last failed call on this thread ("" if none). */
const char* gdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
