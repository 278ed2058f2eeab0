// C ABI of the Gated DeltaNet chunked-prefill forward: validation, the AutoCP
// planner and kernel launches. Host code only; see include/gdn.h.
#include "gdn.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "gdn_internal.h"

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

}  // namespace

int gdn::record_error(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

namespace {

constexpr float kDefaultLambda = 1.0f;
constexpr int kDefaultWarmup = 6;
constexpr int kMaxWarmup = 8;
constexpr float kDefaultNoiseFloor = 1e-4f;
constexpr size_t kStateElems = (size_t)gdn::kDim * gdn::kDim;
// Relative time of one chunk step of a forward workgroup over 128 / s_dv
// columns (index s_dv) against the full 128 columns, all CUs busy: 0.50 for
// four blocks (measured at the TP1 B=4 shape: 2.1 against 4.2 us; the operand
// staging, P and the dependent chain do not shrink with the columns), 0.65
// for two (estimated between).
constexpr double kColStep[5] = {0.0, 1.0, 0.65, 0.0, 0.50};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Byte offsets of the workspace arrays of one forward pipeline.
struct FwdLayout {
    size_t off_sink = 0, off_T = 0, off_GB = 0, off_state = 0, off_M = 0, off_H = 0, off_warm = 0;
    size_t off_GM = 0, off_GH = 0, bytes = 0;
};

struct Plan {
    int n_seqs = 0;
    std::vector<int> len;       // tokens per sequence
    int n_chunks_total = 0, n_chunks_max = 0;
    int L = 1, n_segments = 0, P_max = 0, cp_on = 0, w = kDefaultWarmup, n_cu = 0, cp_order = 0, cp_split = 0;
    int s_dv = 1;                 // column blocks of d_v in the fused forward
    float lambda = kDefaultLambda, eps = kDefaultNoiseFloor;
    int comb_G = 0, comb_J = 0;   // grouped combine of the backward's forward re-run (0: one chain)
    int g16_G = 0, g16_J = 0;     // grouped combine of the forward (0: one chain)
    FwdLayout fw;                 // the forward (fp16 chain kernels)
    FwdLayout re;                 // the backward's forward re-run (split bf16 chain kernels)
    size_t ws_bytes = 0;          // == fw.bytes
};

int n_chunks_of(int len) { return (len + gdn::kChunk - 1) / gdn::kChunk; }
int n_segs_of(int N, int L) { return N == 0 ? 1 : (N + L - 1) / L; }

gdn_status validate_desc(const gdn_desc* d) {
    if (!d) return fail(GDN_ERR_NULL_ARG, "desc is NULL");
    if (d->B < 1 || d->T < 0 || d->h_qk < 1 || d->h_v < 1)
        return fail(GDN_ERR_BAD_SHAPE, "need B >= 1, T >= 0, h_qk >= 1, h_v >= 1 (got B=%d T=%d h_qk=%d h_v=%d)",
                    d->B, d->T, d->h_qk, d->h_v);
    if (d->h_v % d->h_qk != 0)
        return fail(GDN_ERR_BAD_SHAPE, "h_v (%d) must be a multiple of h_qk (%d)", d->h_v, d->h_qk);
    if (d->h_v > 65535) return fail(GDN_ERR_BAD_SHAPE, "h_v (%d) exceeds 65535", d->h_v);
    if (d->d_k != gdn::kDim || d->d_v != gdn::kDim)
        return fail(GDN_ERR_UNSUPPORTED_DIM, "only d_k = d_v = 128 is supported (got %d, %d)", d->d_k, d->d_v);
    if (d->io_dtype != GDN_BF16 && d->io_dtype != GDN_F32)
        return fail(GDN_ERR_BAD_DTYPE, "io_dtype %d is not GDN_BF16 or GDN_F32", d->io_dtype);
    if (d->cp_mode < GDN_CP_AUTO || d->cp_mode > GDN_CP_WARMUP)
        return fail(GDN_ERR_BAD_OPTION, "cp_mode %d out of range", d->cp_mode);
    if (!(d->lambda >= 0.f) || !std::isfinite(d->lambda))
        return fail(GDN_ERR_BAD_OPTION, "lambda must be finite and >= 0");
    if (d->warmup_chunks < 0 || d->warmup_chunks > kMaxWarmup)
        return fail(GDN_ERR_BAD_OPTION, "warmup_chunks must be in 0..%d (got %d)", kMaxWarmup, d->warmup_chunks);
    if (!(d->noise_floor >= 0.f && d->noise_floor < 1.f))
        return fail(GDN_ERR_BAD_OPTION, "noise_floor must be in [0, 1)");
    if (d->n_cu < 0) return fail(GDN_ERR_BAD_OPTION, "n_cu must be >= 0");
    if (d->dv_split != 0 && d->dv_split != 1 && d->dv_split != 2 && d->dv_split != 4)
        return fail(GDN_ERR_BAD_OPTION, "dv_split must be 0 (planner), 1, 2 or 4 (got %d)", d->dv_split);
    if (d->cp_layout < 0 || d->cp_layout > 2)
        return fail(GDN_ERR_BAD_OPTION, "cp_layout must be 0 (planner), 1 or 2 (got %d)", d->cp_layout);
    if (d->dv_split > 1 && d->io_dtype != GDN_BF16)
        return fail(GDN_ERR_BAD_OPTION, "dv_split > 1 needs bf16 inputs");
    if (d->dv_split > 1 && d->cp_mode != GDN_CP_AUTO && d->cp_mode != GDN_CP_OFF)
        return fail(GDN_ERR_BAD_OPTION, "dv_split > 1 runs without a context-parallel split (cp_mode AUTO or OFF)");
    if ((long long)d->B * d->T > 0x7fffffffLL)
        return fail(GDN_ERR_BAD_SHAPE, "B * T exceeds 2^31 - 1 tokens");
    if (d->host_cu_seqlens) {
        if (d->B != 1) return fail(GDN_ERR_BAD_SHAPE, "cu_seqlens requires B == 1 (got B=%d)", d->B);
        if (d->n_seqs < 1) return fail(GDN_ERR_BAD_SHAPE, "n_seqs must be >= 1 with cu_seqlens");
        const int32_t* cu = d->host_cu_seqlens;
        if (cu[0] != 0) return fail(GDN_ERR_BAD_SHAPE, "cu_seqlens[0] must be 0");
        for (int n = 0; n < d->n_seqs; ++n)
            if (cu[n + 1] < cu[n]) return fail(GDN_ERR_BAD_SHAPE, "cu_seqlens must be non-decreasing (at %d)", n);
        if (cu[d->n_seqs] != d->T)
            return fail(GDN_ERR_BAD_SHAPE, "cu_seqlens[n_seqs] (%d) must equal T (%d)", cu[d->n_seqs], d->T);
    } else if (d->n_seqs != d->B) {
        return fail(GDN_ERR_BAD_SHAPE, "n_seqs (%d) must equal B (%d) without cu_seqlens", d->n_seqs, d->B);
    }
    return GDN_OK;
}

gdn_status query_cu_count(int* n_cu) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "querying the CU count failed: %s", hipGetErrorString(e));
    return GDN_OK;
}

// Grouping of the segment combine over nb boundaries with `heads` chains
// (see make_plan): the G with the least estimated steps, or G = 0 (one chain)
// when none beats nb steps; J_max > 0 caps the group count (the workspace
// holds that many group maps).
void combine_grouping(int nb, long long heads, int n_cu, int J_max, int32_t* G_out, int32_t* J_out) {
    *G_out = 0;
    *J_out = 0;
    double best = nb;
    for (int G = 2; G < nb; ++G) {
        const int J = (nb + G - 1) / G;
        if (J < 2) break;
        if (J_max > 0 && J > J_max) continue;
        const long long wgs = 8LL * (J - 1) * heads, rounds = (wgs + n_cu - 1) / n_cu;
        const double slow = 2 * wgs <= n_cu ? 1.0 : 2.5;
        const double steps = slow * (G * rounds + G - 1) + std::max(J - 2, 0) + 4;
        if (steps < best) {
            best = steps;
            *G_out = G;
            *J_out = J;
        }
    }
}

// The forward's (fp16) combine grouping: G boundaries per group when its two
// launches' steps -- G composing steps, then J - 2 + G linking and replaying
// steps, each stretched by the workgroups beyond one per CU (16 per group and
// exact (sequence, head) composing, 8 replaying: a combine step is bound by its
// operand loads, which workgroups sharing a CU share) -- plus about eight steps
// for the extra launch, come to less than 0.8 of the single chain's nb steps
// (measured: a launch costs about as much as eight boundary steps; with more
// composing workgroups than CUs the grouped combine lost to the chain).
void combine16_grouping(int nb, long long exact_heads, int n_cu, int32_t* G_out, int32_t* J_out) {
    *G_out = 0;
    *J_out = 0;
    double best = 0.8 * nb;
    const double cus = std::max(n_cu, 1);
    for (int G = 2; G < nb; ++G) {
        const int J = (nb + G - 1) / G;
        if (J < 2) break;
        const double load1 = std::max(1.0, 16.0 * (J - 1) * exact_heads / cus);
        const double load2 = std::max(1.0, 8.0 * (J - 1) * exact_heads / cus);
        const double steps = G * load1 + (J - 2 + G) * load2 + 8;
        if (steps < best) {
            best = steps;
            *G_out = G;
            *J_out = J;
        }
    }
}

// The AutoCP planner (section "Gate-Driven Automatic Intra-Card Context
// Parallelism (AutoCP)": L = lambda sqrt(N) chunks per segment). Readings:
// N is the chunk count of the longest sequence; lambda sqrt(N), rounded
// half-up, is the largest L considered; below it L is chosen for the hardware
// (every CU gets a workgroup, and whole rounds of workgroups: see the cost
// model below); AUTO keeps a sequence whole when (sequences x heads) already
// cover the CUs or when the sequence is shorter than two warm-up windows. L is
// raised where needed so that no sequence has more than kMaxSegsPerSeq
// segments.
//
// Workspace: an 8 KiB scratch line (stores of rows past a sequence's end land
// there), T (split hi/lo, 16 KiB) and gamma, beta (512 bytes) per (chunk,
// value head); with a split, the segment states, the maps M and H, and the
// boundary flags.
gdn_status make_plan(const gdn_desc* d, Plan* pl, bool column_split = true) {
    gdn_status st = validate_desc(d);
    if (st != GDN_OK) return st;
    Plan P;
    P.n_seqs = d->host_cu_seqlens ? d->n_seqs : d->B;
    P.len.resize(P.n_seqs);
    for (int n = 0; n < P.n_seqs; ++n)
        P.len[n] = d->host_cu_seqlens ? d->host_cu_seqlens[n + 1] - d->host_cu_seqlens[n] : d->T;
    long long nct = 0;
    for (int n = 0; n < P.n_seqs; ++n) {
        const int N = n_chunks_of(P.len[n]);
        nct += N;
        P.n_chunks_max = std::max(P.n_chunks_max, N);
    }
    if (nct > 0x7fffffffLL) return fail(GDN_ERR_BAD_SHAPE, "too many chunks");
    P.n_chunks_total = (int)nct;
    P.w = d->warmup_chunks ? d->warmup_chunks : kDefaultWarmup;
    P.lambda = d->lambda > 0.f ? d->lambda : kDefaultLambda;
    P.eps = d->noise_floor > 0.f ? d->noise_floor : kDefaultNoiseFloor;
    if (d->n_cu > 0) P.n_cu = d->n_cu;
    else if ((st = query_cu_count(&P.n_cu)) != GDN_OK) return st;

    const int Nm = P.n_chunks_max;
    auto total_segs = [&](int L) {
        long long s = 0;
        for (int n = 0; n < P.n_seqs; ++n) s += n_segs_of(n_chunks_of(P.len[n]), L);
        return s;
    };
    bool split = d->cp_mode != GDN_CP_OFF && Nm > 1;
    if (split && d->cp_mode == GDN_CP_AUTO &&
        ((long long)P.n_seqs * d->h_v >= P.n_cu || Nm < 2 * (P.w + 1)))
        split = false;
    if (column_split && d->dv_split > 1) {   // forced column split: no segments
        P.s_dv = d->dv_split;
        split = false;
    }
    // AUTO may split d_v instead of the sequences (bf16 inputs): chosen below
    // when it fills the CUs and its estimated time is lower
    const bool try_columns = column_split && d->dv_split == 0 && split && d->cp_mode == GDN_CP_AUTO &&
                             d->io_dtype == GDN_BF16;
    if (!split) {
        P.L = std::max(Nm, 1);
    } else {
        const int L_lam = std::min(std::max(1, (int)std::floor(P.lambda * std::sqrt((double)Nm) + 0.5)), Nm);
        // Among L <= L_lam whose segments fill every CU (or L = 1), the one with
        // the least estimated time in chunk steps: the forward runs
        // ceil(workgroups / CUs) rounds of L chunks, the exact maps L more, and
        // the combine one short step (about a quarter chunk) per boundary.
        int best_L = 1;
        double best = 0.0;
        bool found = false;
        for (int L = L_lam; L >= 1; --L) {
            const long long segs = total_segs(L), wg = segs * d->h_v;
            if (wg < P.n_cu && L > 1) continue;
            if (n_segs_of(Nm, L) > gdn::kMaxSegsPerSeq) break;
            const long long rounds = (wg + P.n_cu - 1) / P.n_cu;
            const double cost = (double)rounds * L + 0.5 * L + 0.25 * (n_segs_of(Nm, L) - 1);
            if (!found || cost < best) {   // ties keep the longer segments
                found = true;
                best = cost;
                best_L = L;
            }
        }
        int L = best_L;
        while (n_segs_of(Nm, L) > gdn::kMaxSegsPerSeq) ++L;
        P.L = L;
        if (try_columns) {
            // Column blocks instead: the whole sequence per workgroup, d_v in
            // the fewest blocks (2 or 4) that fill the CUs, each chunk step
            // costing kColStep[s_dv] of a full one; taken when cheaper than
            // the split's estimate.
            const long long seq_heads = (long long)P.n_seqs * d->h_v;
            for (int s_dv : {2, 4}) {
                const long long wg = seq_heads * s_dv;
                if (wg < P.n_cu) continue;
                const long long rounds = (wg + P.n_cu - 1) / P.n_cu;
                const double cost = kColStep[s_dv] * (double)rounds * Nm;
                if (cost < best) {
                    P.s_dv = s_dv;
                    P.L = std::max(Nm, 1);
                }
                break;
            }
        }
    }
    long long ns = 0;
    for (int n = 0; n < P.n_seqs; ++n) {
        const int s = n_segs_of(n_chunks_of(P.len[n]), P.L);
        ns += s;
        P.P_max = std::max(P.P_max, s);
    }
    if (ns > 0x7fffffffLL / 2) return fail(GDN_ERR_BAD_SHAPE, "too many segments");
    P.n_segments = (int)ns;
    P.cp_on = P.P_max > 1;
    const size_t nch = (size_t)P.n_chunks_total * d->h_v, nsg = (size_t)P.n_segments * d->h_v;
    const size_t st_bytes = nsg * kStateElems * sizeof(float);
    // k_cp_prep puts the exact boundaries' workgroups (two each) first when,
    // with the share of exact heads the pages report (most heads forget fast:
    // 30 % exact, to the nearest), they fit in about one round (2 E <= 5/4 CUs);
    // with more, head-major order measured faster.
    // With bf16 inputs (cp_layout 0) an exact boundary's H and M run in two
    // 8-wave workgroups when there are no more boundary pairs than CUs (each chain
    // wave then has a SIMD's matrix pipe to itself: TP8 CP preprocessing
    // 40 -> 32 us), else in one 12-wave workgroup sharing the staged chunks
    // (fewer workgroups: TP2 95 -> 69 us, TP1 66 -> 46 us, measured).
    if (P.cp_on) {
        const long long pairs = (long long)(P.n_segments - P.n_seqs) * d->h_v, est = (3 * pairs + 5) / 10;
        P.cp_order = 4 * (2 * est) <= 5LL * P.n_cu ? 1 : 0;
        // (cp_mode EXACT: every pair takes two workgroups)
        const long long wgs = (long long)P.n_segments * d->h_v * (d->cp_mode == GDN_CP_EXACT ? 2 : 1);
        P.cp_split = d->cp_layout == 2 || (d->cp_layout == 0 && wgs <= P.n_cu) ? 1 : 0;
    }
    {
        // The forward: an 8 KiB scratch line (stores of rows past a sequence's
        // end land there), T diag(beta) as fp16 operand images (6 KiB per chunk
        // and value head) and the chunk's gate factors (1 KiB); with a split, the boundary states and H maps (fp32,
        // 64 KiB, in the chain kernels' tile order), the M maps as the combine's
        // fp16 A operands (32 KiB) and the boundary flags.
        FwdLayout& F = P.fw;
        size_t off = 0;
        if (P.n_chunks_total > 0) { F.off_sink = off; off += 8192; }
        F.off_T = off;  off = align_up(off + nch * gdn::kTbHalfs * 2, 256);
        F.off_GB = off; off = align_up(off + nch * gdn::kGfFloats * sizeof(float), 256);
        if (P.cp_on) {
            F.off_state = off; off = align_up(off + st_bytes, 256);
            F.off_H = off;     off = align_up(off + st_bytes, 256);
            F.off_M = off;     off = align_up(off + st_bytes / 2, 256);
            F.off_warm = off;  off = align_up(off + nsg * sizeof(int32_t), 256);
            // the grouped combine: per (sequence, group, head) the composed map CM
            // (fp16 image, 32 KiB) and CH (fp32, 64 KiB)
            const long long heads = std::max(1LL, ((long long)P.n_seqs * d->h_v * 3 + 5) / 10);
            combine16_grouping(P.P_max - 1, heads, P.n_cu, &P.g16_G, &P.g16_J);
            if (P.g16_G) {
                const size_t grp = (size_t)P.n_seqs * P.g16_J * d->h_v * kStateElems;
                F.off_GM = off; off = align_up(off + grp * 2, 256);
                F.off_GH = off; off = align_up(off + grp * sizeof(float), 256);
            }
        }
        F.bytes = off;
    }
    {
        // The backward's re-run of the forward: T split hi/lo (16 KiB) and
        // gamma, beta (512 bytes) per (chunk, value head); with a split, the
        // segment states, maps M (split operands) and H, the boundary flags and
        // the grouped combine's group maps. The combine chains the boundaries of
        // a sequence, P - 1 steps in a row; grouped (groups of G boundaries
        // composed in parallel, then linked, then replayed in parallel) it takes
        // about G + (J - 2) + (G - 1) steps, J = ceil((P - 1) / G), in three
        // launches; the re-run links every head (all exact).
        FwdLayout& R = P.re;
        size_t off = 0;
        const size_t blk = (size_t)gdn::kChunk * gdn::kChunk * sizeof(float);
        if (P.n_chunks_total > 0) { R.off_sink = off; off += 8192; }
        R.off_T = off;  off = align_up(off + nch * blk, 256);
        R.off_GB = off; off = align_up(off + nch * 2 * gdn::kChunk * sizeof(float), 256);
        if (P.cp_on) {
            R.off_state = off; off = align_up(off + st_bytes, 256);
            R.off_M = off;     off = align_up(off + st_bytes, 256);
            R.off_H = off;     off = align_up(off + st_bytes, 256);
            R.off_warm = off;  off = align_up(off + nsg * sizeof(int32_t), 256);
            const long long heads = std::max(1LL, ((long long)P.n_seqs * d->h_v * 3 + 5) / 10);
            combine_grouping(P.P_max - 1, heads, P.n_cu, 0, &P.comb_G, &P.comb_J);
            if (P.comb_G) {
                const size_t grp = (size_t)P.n_seqs * P.comb_J * d->h_v * kStateElems * sizeof(float);
                R.off_GM = off; off = align_up(off + grp, 256);
                R.off_GH = off; off = align_up(off + 2 * grp, 256);
            }
        }
        R.bytes = off;
    }
    P.ws_bytes = P.fw.bytes;
    *pl = std::move(P);
    return GDN_OK;
}

// Profiling events (gdn_profile_enable / gdn_profile_read).
constexpr int kProfEvents = 5;   // before prep, after prep, cp_prep, cp_combine, forward
struct Profiler {
    bool on = false, created = false, recorded = false, ran[4] = {false, false, false, false};
    hipEvent_t ev[kProfEvents];
};
Profiler g_prof;

void prof_mark(int i, hipStream_t s) {
    if (g_prof.on) (void)hipEventRecord(g_prof.ev[i], s);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

gdn_status check_ptr(const void* p, const char* name, bool required, size_t align = 16) {
    if (!p) {
        if (required) return fail(GDN_ERR_NULL_ARG, "%s is NULL", name);
        return GDN_OK;
    }
    if (!aligned(p, align)) return fail(GDN_ERR_MISALIGNED, "%s is not %zu-byte aligned", name, align);
    return GDN_OK;
}

gdn::Params base_params(const gdn_desc* d, const Plan& P) {
    gdn::Params p{};
    p.n_seqs = P.n_seqs;
    p.seq_len = d->T;
    p.h_qk = d->h_qk;
    p.h_v = d->h_v;
    p.group = d->h_v / d->h_qk;
    p.L = P.L;
    p.dv_split = P.s_dv;
    p.w = P.w;
    p.cp_mode = d->cp_mode;
    p.n_segments = P.n_segments;
    p.n_chunks = P.n_chunks_total;
    p.cp_order = P.cp_order;
    p.cp_split = P.cp_split;
    p.log_eps = std::log(P.eps);
    p.t_stride = (int64_t)gdn::kChunk * gdn::kChunk;
    p.gb_stride = 2 * gdn::kChunk;
    // (head, chunk) items per k_prep wave: one round of eight waves (one
    // workgroup) per CU (at most 32 items each; larger inputs take more rounds)
    const long long items = (long long)P.n_chunks_total * d->h_v, slots = 8LL * std::max(P.n_cu, 1);
    p.prep_cpw = (int)std::min<long long>(std::max<long long>((items + slots - 1) / slots, 1), 32);
    return p;
}

// Validation shared by the forward entry points (pointers, sizes, workspace).
gdn_status check_fwd_args(const gdn_desc* d, const Plan& P, const void* q, const void* k, const void* v,
                          const float* g, const float* beta, float scale, const float* s_init, const int32_t* cu,
                          const void* out, const float* s_final, const void* ws, size_t ws_bytes,
                          size_t need_bytes) {
    const bool varlen = d->host_cu_seqlens != nullptr;
    if (varlen && !cu) return fail(GDN_ERR_NULL_ARG, "cu_seqlens is NULL but desc->host_cu_seqlens is set");
    if (!varlen && cu) return fail(GDN_ERR_NULL_ARG, "desc->host_cu_seqlens is required with cu_seqlens");
    const bool any = (long long)d->B * d->T > 0;
    gdn_status st;
    if ((st = check_ptr(q, "q", any)) || (st = check_ptr(k, "k", any)) || (st = check_ptr(v, "v", any)) ||
        (st = check_ptr(g, "g", any)) || (st = check_ptr(beta, "beta", any)) ||
        (st = check_ptr(out, "out", any)) || (st = check_ptr(s_init, "initial_state", false)) ||
        (st = check_ptr(s_final, "final_state", false)) || (st = check_ptr(cu, "cu_seqlens", false, 4)))
        return st;
    if (!std::isfinite(scale)) return fail(GDN_ERR_BAD_SCALE, "scale is not finite");
    if (ws_bytes < need_bytes)
        return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", ws_bytes, need_bytes);
    if (need_bytes > 0 && (st = check_ptr(ws, "workspace", true, 256))) return st;
    (void)P;
    return GDN_OK;
}

void set_layout(gdn::Params& p, const FwdLayout& F, const Plan& P, char* w8) {
    if (P.n_chunks_total > 0) p.sink = reinterpret_cast<float*>(w8 + F.off_sink);
    if (P.cp_on) {
        p.seg_state = reinterpret_cast<float*>(w8 + F.off_state);
        p.seg_M = reinterpret_cast<float*>(w8 + F.off_M);
        p.seg_H = reinterpret_cast<float*>(w8 + F.off_H);
        p.warm = reinterpret_cast<int32_t*>(w8 + F.off_warm);
    }
}

// The forward: k_prep (T diag(beta) images, boundary classes) | k_cp_prep16
// (boundary states or maps) | k_combine16 (exact boundaries) | k_fwd16.
// GDN_LOG=1 in the environment: one line per forward call on stderr with the
// plan it runs (read once per process).
bool log_enabled() {
    static const bool on = [] {
        const char* e = std::getenv("GDN_LOG");
        return e && *e && std::strcmp(e, "0") != 0;
    }();
    return on;
}

void log_plan(const gdn_desc* d, const Plan& P) {
    std::fprintf(stderr,
                 "[gdn] fwd B=%d T=%d h_qk=%d h_v=%d io=%s cp_mode=%d: chunks=%d (max %d) cp_on=%d L=%d "
                 "segments=%d (max %d per sequence) dv_split=%d w=%d eps=%g lambda=%g n_cu=%d cp_order=%d "
                 "cp_split=%d combine_G=%d combine_J=%d workspace=%zu\n",
                 d->B, d->T, d->h_qk, d->h_v, d->io_dtype == GDN_BF16 ? "bf16" : "f32", d->cp_mode,
                 P.n_chunks_total, P.n_chunks_max, P.cp_on, P.L, P.n_segments, P.P_max, P.s_dv, P.w,
                 (double)P.eps, (double)P.lambda, P.n_cu, P.cp_order, P.cp_split, P.g16_G, P.g16_J, P.ws_bytes);
}

gdn_status run_fwd(const gdn_desc* d, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, float scale, const float* s_init, const int32_t* cu, void* out,
                   float* s_final, void* ws, size_t ws_bytes, void* stream, float* seg_out, int32_t* path_out) {
    Plan P;
    gdn_status st = make_plan(d, &P);
    if (st != GDN_OK) return st;
    if (log_enabled()) log_plan(d, P);
    if ((st = check_fwd_args(d, P, q, k, v, g, beta, scale, s_init, cu, out, s_final, ws, ws_bytes, P.fw.bytes)))
        return st;
    if ((st = check_ptr(seg_out, "seg_state_out", false)) || (st = check_ptr(path_out, "path_out", false, 4)))
        return st;
    gdn::Params p = base_params(d, P);
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.s_init = s_init; p.cu = cu;
    p.out = out; p.s_final = s_final; p.scale = scale;
    char* w8 = static_cast<char*>(ws);
    set_layout(p, P.fw, P, w8);
    if (P.n_chunks_total > 0) {
        p.tb16 = w8 + P.fw.off_T;
        p.gf16 = reinterpret_cast<float*>(w8 + P.fw.off_GB);
    }
    p.comb_G = P.g16_G;
    p.comb_J = P.g16_J;
    if (P.cp_on && P.g16_G) {
        p.seg_GM = reinterpret_cast<float*>(w8 + P.fw.off_GM);
        p.seg_GH = reinterpret_cast<float*>(w8 + P.fw.off_GH);
    }
    const int io = d->io_dtype == GDN_BF16 ? gdn::kIoBf16 : gdn::kIoF32;
    const hipStream_t hs = (hipStream_t)stream;
    int e;
    prof_mark(0, hs);
    if ((e = gdn::launch_prep(p, io, stream)))
        return fail(GDN_ERR_HIP, "prep launch: %s", hipGetErrorString((hipError_t)e));
    prof_mark(1, hs);
    if (P.cp_on) {
        if ((e = gdn::launch_cp_prep16(p, io, stream)))
            return fail(GDN_ERR_HIP, "cp_prep launch: %s", hipGetErrorString((hipError_t)e));
        prof_mark(2, hs);
        if ((e = gdn::launch_combine16(p, stream)))
            return fail(GDN_ERR_HIP, "combine launch: %s", hipGetErrorString((hipError_t)e));
        prof_mark(3, hs);
    }
    if ((e = gdn::launch_fwd16(p, io, stream)))
        return fail(GDN_ERR_HIP, "fwd launch: %s", hipGetErrorString((hipError_t)e));
    prof_mark(4, hs);
    if (g_prof.on) {
        g_prof.recorded = true;
        g_prof.ran[0] = true;
        g_prof.ran[1] = g_prof.ran[2] = P.cp_on != 0;
        g_prof.ran[3] = true;
    }

    if (seg_out || path_out) {
        const size_t per_seg = (size_t)d->h_v * kStateElems;
        hipError_t he = hipSuccess;
        if (seg_out) {
            // boundary states (tile order in the workspace) -> row-major; each
            // sequence's segment 0 takes its initial state
            if (P.cp_on && (e = gdn::launch_tiles_to_rm(p.seg_state, seg_out, (long long)P.n_segments * d->h_v, stream)))
                return fail(GDN_ERR_HIP, "debug copy: %s", hipGetErrorString((hipError_t)e));
            int base = 0;
            for (int n = 0; n < P.n_seqs && he == hipSuccess; ++n) {
                float* dst = seg_out + (size_t)base * per_seg;
                if (s_init)
                    he = hipMemcpyAsync(dst, s_init + (size_t)n * per_seg, per_seg * sizeof(float),
                                        hipMemcpyDeviceToDevice, hs);
                else
                    he = hipMemsetAsync(dst, 0, per_seg * sizeof(float), hs);
                base += n_segs_of(n_chunks_of(P.len[n]), P.L);
            }
        }
        if (he != hipSuccess) return fail(GDN_ERR_HIP, "debug copy: %s", hipGetErrorString(he));
        if (path_out && (e = gdn::launch_debug_path(p, path_out, stream)))
            return fail(GDN_ERR_HIP, "debug path launch: %s", hipGetErrorString((hipError_t)e));
    }
    g_last_error.clear();
    return GDN_OK;
}

// The backward's re-run of the forward (split bf16 chain kernels, which also
// write the state entering every chunk, Y, V' and the output's state term
// dotted with dO), in the re-run layout of the workspace.
gdn_status run_fwd_rerun(const gdn_desc* d, const Plan& P, const void* q, const void* k, const void* v,
                         const float* g, const float* beta, float scale, const float* s_init, const int32_t* cu,
                         char* w8, void* stream, float* chunk_states, float* bwd_y, float* bwd_vp,
                         float* bwd_oi, const void* bwd_dout) {
    gdn::Params p = base_params(d, P);
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.s_init = s_init; p.cu = cu;
    p.out = nullptr;   // (the backward needs no output, only the per-chunk blocks below)
    p.s_final = nullptr; p.scale = scale;
    set_layout(p, P.re, P, w8);
    if (P.n_chunks_total > 0) {
        p.prep_T = reinterpret_cast<float*>(w8 + P.re.off_T);
        p.prep_GB = reinterpret_cast<float*>(w8 + P.re.off_GB);
    }
    if (P.cp_on && P.comb_G) {
        p.seg_GM = reinterpret_cast<float*>(w8 + P.re.off_GM);
        p.seg_GH = reinterpret_cast<float*>(w8 + P.re.off_GH);
    }
    p.comb_G = P.comb_G;
    p.comb_J = P.comb_J;
    const int io = gdn::kIoBf16;
    int e;
    if ((e = gdn::launch_prep(p, io, stream)))
        return fail(GDN_ERR_HIP, "prep launch: %s", hipGetErrorString((hipError_t)e));
    if (P.cp_on) {
        if ((e = gdn::launch_cp_prep(p, io, stream)))
            return fail(GDN_ERR_HIP, "cp_prep launch: %s", hipGetErrorString((hipError_t)e));
        if ((e = gdn::launch_cp_combine(p, stream)))
            return fail(GDN_ERR_HIP, "cp_combine launch: %s", hipGetErrorString((hipError_t)e));
    }
    p.chunk_states = chunk_states;
    p.bwd_y = bwd_y;
    p.bwd_vp = bwd_vp;
    p.bwd_oi = bwd_oi;
    p.bwd_dout = bwd_dout;
    if ((e = gdn::launch_fwd_states(p, io, stream)))
        return fail(GDN_ERR_HIP, "fwd launch: %s", hipGetErrorString((hipError_t)e));
    return GDN_OK;
}

// Workspace of the backward: the forward's (for its re-run, which writes no
// output), then the state entering every chunk, the gradient of the state leaving
// every chunk, T / P / gamma per chunk and head (fp32, and T^T / scale P^T / T
// as bf16 hi/lo images), per chunk and head Y, V', scale e^gamma Q S (from the
// re-run) and dV', T^T dV' (from the state-gradient scan), and the
// per-value-head parts of dq and dk.
struct BwdLayout {
    size_t off_cs = 0, off_ds = 0, off_tpg = 0, off_tpt = 0, off_dq = 0, off_dk = 0, bytes = 0;
    size_t off_y = 0, off_vp = 0, off_oi = 0, off_dvp = 0, off_z = 0;
    size_t off_q = 0, off_k = 0, off_v = 0, off_do = 0;   // bf16 copies of fp32 inputs
    size_t tokens = 0;
};

BwdLayout bwd_layout(const gdn_desc* d, const Plan& P) {
    BwdLayout L;
    for (int n = 0; n < P.n_seqs; ++n) L.tokens += (size_t)P.len[n];
    const size_t st = (size_t)P.n_chunks_total * d->h_v * kStateElems * sizeof(float);
    size_t off = align_up(P.re.bytes, 256);
    L.off_cs = off;  off = align_up(off + st, 256);
    L.off_ds = off;  off = align_up(off + st, 256);
    L.off_tpg = off; off = align_up(off + (size_t)P.n_chunks_total * d->h_v * gdn::kBwdTpg * sizeof(float), 256);
    L.off_tpt = off; off = align_up(off + (size_t)P.n_chunks_total * d->h_v * gdn::kBwdTpt * 2, 256);
    const size_t blk = (size_t)P.n_chunks_total * d->h_v * gdn::kChunk * gdn::kDim * sizeof(float);
    L.off_y = off;   off = align_up(off + blk, 256);
    L.off_vp = off;  off = align_up(off + blk, 256);
    // the output's state term only as its per-token dot products with dO, eight partial sums
    L.off_oi = off;  off = align_up(off + (size_t)P.n_chunks_total * d->h_v * 8 * gdn::kChunk * sizeof(float), 256);
    L.off_dvp = off; off = align_up(off + blk, 256);
    L.off_z = off;   off = align_up(off + blk, 256);
    L.off_dq = off;  off = align_up(off + L.tokens * d->h_v * gdn::kDim * sizeof(float), 256);
    L.off_dk = off;  off = align_up(off + L.tokens * d->h_v * gdn::kDim * sizeof(float), 256);
    if (d->io_dtype == GDN_F32) {
        L.off_q = off;  off = align_up(off + L.tokens * d->h_qk * gdn::kDim * 2, 256);
        L.off_k = off;  off = align_up(off + L.tokens * d->h_qk * gdn::kDim * 2, 256);
        L.off_v = off;  off = align_up(off + L.tokens * d->h_v * gdn::kDim * 2, 256);
        L.off_do = off; off = align_up(off + L.tokens * d->h_v * gdn::kDim * 2, 256);
    }
    L.bytes = off;
    return L;
}

}  // namespace

extern "C" {

size_t gdn_bwd_workspace_bytes(const gdn_desc* desc) {
    Plan P;
    if (make_plan(desc, &P, false) != GDN_OK) return 0;
    if (desc->io_dtype == GDN_F32) {   // planned as the bf16 run it becomes
        gdn_desc d16 = *desc;
        d16.io_dtype = GDN_BF16;
        if (make_plan(&d16, &P, false) != GDN_OK) return 0;
    }
    return bwd_layout(desc, P).bytes;
}

gdn_status gdn_bwd(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, float scale, const float* initial_state, const int32_t* cu_seqlens,
                   const void* d_out, const float* d_final_state, void* dq, void* dk, void* dv, float* dg,
                   float* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                   void* stream) {
    Plan P;
    gdn_status st = make_plan(desc, &P, false);   // (the re-run keeps all columns together)
    if (st != GDN_OK) return st;
    // fp32 inputs: q, k, v and d_out are rounded once to bf16 in the workspace,
    // everything after runs as for bf16 inputs (so it is planned as that run),
    // and dq, dk, dv are written in fp32
    const bool f32 = desc->io_dtype == GDN_F32;
    gdn_desc d16 = *desc;
    d16.io_dtype = GDN_BF16;
    if (f32 && (st = make_plan(&d16, &P, false)) != GDN_OK) return st;
    const bool varlen = desc->host_cu_seqlens != nullptr;
    if (varlen && !cu_seqlens) return fail(GDN_ERR_NULL_ARG, "cu_seqlens is NULL but desc->host_cu_seqlens is set");
    if (!varlen && cu_seqlens) return fail(GDN_ERR_NULL_ARG, "desc->host_cu_seqlens is required with cu_seqlens");
    const bool any = (long long)desc->B * desc->T > 0;
    if ((st = check_ptr(q, "q", any)) || (st = check_ptr(k, "k", any)) || (st = check_ptr(v, "v", any)) ||
        (st = check_ptr(g, "g", any)) || (st = check_ptr(beta, "beta", any)) ||
        (st = check_ptr(d_out, "d_out", any)) || (st = check_ptr(dq, "dq", any)) ||
        (st = check_ptr(dk, "dk", any)) || (st = check_ptr(dv, "dv", any)) || (st = check_ptr(dg, "dg", any)) ||
        (st = check_ptr(dbeta, "dbeta", any)) || (st = check_ptr(initial_state, "initial_state", false)) ||
        (st = check_ptr(d_final_state, "d_final_state", false)) ||
        (st = check_ptr(d_initial_state, "d_initial_state", false)) ||
        (st = check_ptr(cu_seqlens, "cu_seqlens", false, 4)))
        return st;
    if (!std::isfinite(scale)) return fail(GDN_ERR_BAD_SCALE, "scale is not finite");
    const BwdLayout L = bwd_layout(desc, P);
    if (workspace_bytes < L.bytes)
        return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, need %zu", workspace_bytes, L.bytes);
    if (L.bytes > 0 && (st = check_ptr(workspace, "workspace", true, 256))) return st;
    char* w8 = static_cast<char*>(workspace);
    if (f32 && L.tokens > 0) {
        const long long nq = (long long)L.tokens * desc->h_qk * gdn::kDim, nv = (long long)L.tokens * desc->h_v * gdn::kDim;
        int e = gdn::launch_round_bf16(static_cast<const float*>(q), w8 + L.off_q, nq, stream);
        if (!e) e = gdn::launch_round_bf16(static_cast<const float*>(k), w8 + L.off_k, nq, stream);
        if (!e) e = gdn::launch_round_bf16(static_cast<const float*>(v), w8 + L.off_v, nv, stream);
        if (!e) e = gdn::launch_round_bf16(static_cast<const float*>(d_out), w8 + L.off_do, nv, stream);
        if (e) return fail(GDN_ERR_HIP, "bf16 rounding launch: %s", hipGetErrorString((hipError_t)e));
        q = w8 + L.off_q;
        k = w8 + L.off_k;
        v = w8 + L.off_v;
        d_out = w8 + L.off_do;
    }
    // the forward again, keeping the state entering every chunk
    if (P.n_chunks_total > 0) {
        st = run_fwd_rerun(&d16, P, q, k, v, g, beta, scale, initial_state, cu_seqlens, w8, stream,
                           reinterpret_cast<float*>(w8 + L.off_cs), reinterpret_cast<float*>(w8 + L.off_y),
                           reinterpret_cast<float*>(w8 + L.off_vp), reinterpret_cast<float*>(w8 + L.off_oi), d_out);
        if (st != GDN_OK) return st;
    }
    gdn::BwdParams b{};
    b.q = q; b.k = k; b.v = v; b.g = g; b.beta = beta; b.dout = d_out; b.dfinal = d_final_state;
    b.cu = cu_seqlens; b.dq = dq; b.dk = dk; b.dv = dv; b.dg = dg; b.dbeta = dbeta; b.dinit = d_initial_state;
    b.cs = reinterpret_cast<const float*>(w8 + L.off_cs);
    b.ds = reinterpret_cast<float*>(w8 + L.off_ds);
    b.tpg = reinterpret_cast<float*>(w8 + L.off_tpg);
    b.tpt = w8 + L.off_tpt;
    b.y = reinterpret_cast<const float*>(w8 + L.off_y);
    b.vp = reinterpret_cast<const float*>(w8 + L.off_vp);
    b.oi = reinterpret_cast<const float*>(w8 + L.off_oi);
    b.dvp = reinterpret_cast<float*>(w8 + L.off_dvp);
    b.z = reinterpret_cast<float*>(w8 + L.off_z);
    b.dq_part = reinterpret_cast<float*>(w8 + L.off_dq);
    b.dk_part = reinterpret_cast<float*>(w8 + L.off_dk);
    // the state-gradient scan splits the sequences as the forward did; the
    // forward's segment arrays are free once its re-run has finished
    b.L = P.cp_on ? P.L : std::max(P.n_chunks_max, 1);
    b.n_segments = P.cp_on ? P.n_segments : P.n_seqs;
    if (P.cp_on) {
        b.seg_state = reinterpret_cast<float*>(w8 + P.re.off_state);
        b.seg_M = reinterpret_cast<float*>(w8 + P.re.off_M);
        b.seg_H = reinterpret_cast<float*>(w8 + P.re.off_H);
        b.warm = reinterpret_cast<int32_t*>(w8 + P.re.off_warm);
        // the backward links every head's segment ends (all exact); grouped only
        // within the group maps the forward's workspace holds
        if (P.comb_G)
            combine_grouping(P.P_max - 1, (long long)P.n_seqs * desc->h_v, P.n_cu, P.comb_J, &b.comb_G, &b.comb_J);
        if (b.comb_G) {
            b.seg_GM = reinterpret_cast<float*>(w8 + P.re.off_GM);
            b.seg_GH = reinterpret_cast<float*>(w8 + P.re.off_GH);
        }
    }
    b.n_seqs = P.n_seqs;
    b.seq_len = desc->T;
    b.h_qk = desc->h_qk;
    b.h_v = desc->h_v;
    b.group = desc->h_v / desc->h_qk;
    b.n_chunks = P.n_chunks_total;
    b.out_f32 = f32;
    b.scale = scale;
    int e = gdn::launch_bwd(b, stream);
    if (!e) e = gdn::launch_bwd_sum(b, (long long)L.tokens, stream);
    if (e) return fail(GDN_ERR_HIP, "backward launch: %s", hipGetErrorString((hipError_t)e));
    g_last_error.clear();
    return GDN_OK;
}

gdn_status gdn_plan(const gdn_desc* desc, gdn_plan_info* out) {
    if (!out) return fail(GDN_ERR_NULL_ARG, "out is NULL");
    Plan P;
    gdn_status st = make_plan(desc, &P);
    if (st != GDN_OK) return st;
    out->chunk = gdn::kChunk;
    out->n_chunks_total = P.n_chunks_total;
    out->n_chunks_max = P.n_chunks_max;
    out->cp_on = P.cp_on;
    out->L = P.L;
    out->n_segments = P.n_segments;
    out->P_max = P.P_max;
    out->warmup_chunks = P.w;
    out->n_cu = P.n_cu;
    out->lambda = P.lambda;
    out->noise_floor = P.eps;
    out->workspace_bytes = P.ws_bytes;
    out->combine_group = P.g16_G;
    out->combine_groups = P.g16_J;
    out->dv_split = P.s_dv;
    out->cp_layout = P.cp_on && desc->io_dtype == GDN_BF16 ? (P.cp_split ? 2 : 1) : 0;
    g_last_error.clear();
    return GDN_OK;
}

size_t gdn_fwd_workspace_bytes(const gdn_desc* desc) {
    Plan P;
    if (make_plan(desc, &P) != GDN_OK) return 0;
    return P.ws_bytes;
}

gdn_status gdn_calibrate_lambda(const gdn_desc* desc, const void* q, const void* k, const void* v,
                                const float* g, const float* beta, float scale, const int32_t* cu_seqlens,
                                void* out, void* workspace, size_t workspace_bytes, const float* lambdas,
                                int32_t n_lambdas, int32_t reps, void* stream, float* ms_out, float* best_lambda) {
    if (!desc) return fail(GDN_ERR_NULL_ARG, "desc is NULL");
    if (!lambdas || !best_lambda) return fail(GDN_ERR_NULL_ARG, "lambdas and best_lambda are required");
    if (n_lambdas < 1 || n_lambdas > 64) return fail(GDN_ERR_BAD_OPTION, "n_lambdas must be in 1..64");
    if (reps < 1 || reps > 1000) return fail(GDN_ERR_BAD_OPTION, "reps must be in 1..1000");
    gdn_desc d = *desc;
    // every candidate is checked (descriptor, pointers, workspace) before anything runs
    for (int i = 0; i < n_lambdas; ++i) {
        if (!(lambdas[i] > 0.f) || !std::isfinite(lambdas[i]))
            return fail(GDN_ERR_BAD_OPTION, "lambdas[%d] must be finite and > 0", i);
        d.lambda = lambdas[i];
        Plan P;
        gdn_status st = make_plan(&d, &P);
        if (st != GDN_OK) return st;
        if (workspace_bytes < P.ws_bytes)
            return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "workspace of %zu bytes, lambda %g needs %zu", workspace_bytes,
                        (double)lambdas[i], P.ws_bytes);
    }
    hipEvent_t ev[2];
    hipError_t e = hipEventCreate(&ev[0]);
    if (e == hipSuccess && (e = hipEventCreate(&ev[1])) != hipSuccess) (void)hipEventDestroy(ev[0]);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
    const hipStream_t hs = (hipStream_t)stream;
    float best_ms = 0.f;
    gdn_status st = GDN_OK;
    for (int i = 0; i < n_lambdas && st == GDN_OK; ++i) {
        d.lambda = lambdas[i];
        // one untimed run, then reps timed ones between two events on the stream
        st = run_fwd(&d, q, k, v, g, beta, scale, nullptr, cu_seqlens, out, nullptr, workspace, workspace_bytes,
                     stream, nullptr, nullptr);
        if (st != GDN_OK) break;
        if ((e = hipEventRecord(ev[0], hs)) != hipSuccess) { st = fail(GDN_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e)); break; }
        for (int r = 0; r < reps && st == GDN_OK; ++r)
            st = run_fwd(&d, q, k, v, g, beta, scale, nullptr, cu_seqlens, out, nullptr, workspace, workspace_bytes,
                         stream, nullptr, nullptr);
        if (st != GDN_OK) break;
        float ms = 0.f;
        if ((e = hipEventRecord(ev[1], hs)) != hipSuccess || (e = hipEventSynchronize(ev[1])) != hipSuccess ||
            (e = hipEventElapsedTime(&ms, ev[0], ev[1])) != hipSuccess) {
            st = fail(GDN_ERR_HIP, "timing: %s", hipGetErrorString(e));
            break;
        }
        ms /= (float)reps;
        if (ms_out) ms_out[i] = ms;
        if (i == 0 || ms < best_ms) {
            best_ms = ms;
            *best_lambda = lambdas[i];
        }
    }
    (void)hipEventDestroy(ev[0]);
    (void)hipEventDestroy(ev[1]);
    if (st == GDN_OK) g_last_error.clear();
    return st;
}

gdn_status gdn_fwd(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, float scale, const float* initial_state, const int32_t* cu_seqlens,
                   void* out, float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    return run_fwd(desc, q, k, v, g, beta, scale, initial_state, cu_seqlens, out, final_state, workspace,
                   workspace_bytes, stream, nullptr, nullptr);
}

gdn_status gdn_fwd_debug(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float scale, const float* initial_state,
                         const int32_t* cu_seqlens, void* out, float* final_state, void* workspace,
                         size_t workspace_bytes, void* stream, float* seg_state_out, int32_t* path_out) {
    return run_fwd(desc, q, k, v, g, beta, scale, initial_state, cu_seqlens, out, final_state, workspace,
                   workspace_bytes, stream, seg_state_out, path_out);
}

gdn_status gdn_decode(const gdn_desc* desc, const void* q, const void* k, const void* v, const float* g,
                      const float* beta, float scale, const float* state_in, float* state_out, void* out,
                      void* stream) {
    gdn_status st = validate_desc(desc);
    if (st != GDN_OK) return st;
    if (desc->host_cu_seqlens)
        return fail(GDN_ERR_BAD_SHAPE, "decode takes B rows of T tokens; host_cu_seqlens must be NULL");
    const bool any = (long long)desc->B * desc->T > 0;
    if ((st = check_ptr(q, "q", any)) || (st = check_ptr(k, "k", any)) || (st = check_ptr(v, "v", any)) ||
        (st = check_ptr(g, "g", any)) || (st = check_ptr(beta, "beta", any)) ||
        (st = check_ptr(out, "out", any)) || (st = check_ptr(state_in, "state_in", false)) ||
        (st = check_ptr(state_out, "state_out", false)))
        return st;
    if (!std::isfinite(scale)) return fail(GDN_ERR_BAD_SCALE, "scale is not finite");
    if (state_in && state_out && state_in != state_out) {
        // each workgroup reads its whole (sequence, head) block before writing
        // it, so only the same pointer or disjoint buffers are safe
        const size_t bytes = (size_t)desc->B * desc->h_v * gdn::kDim * gdn::kDim * sizeof(float);
        const uintptr_t a = (uintptr_t)state_in, b = (uintptr_t)state_out;
        if (a < b + bytes && b < a + bytes)
            return fail(GDN_ERR_BAD_SHAPE, "state_in and state_out overlap without being the same buffer");
    }
    gdn::Params p{};
    p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta;
    p.s_init = state_in; p.s_final = state_out; p.out = out; p.scale = scale;
    p.n_seqs = desc->B;
    p.seq_len = desc->T;
    p.h_qk = desc->h_qk;
    p.h_v = desc->h_v;
    p.group = desc->h_v / desc->h_qk;
    const int io = desc->io_dtype == GDN_BF16 ? gdn::kIoBf16 : gdn::kIoF32;
    if (const int e = gdn::launch_decode(p, io, stream))
        return fail(GDN_ERR_HIP, "decode launch: %s", hipGetErrorString((hipError_t)e));
    g_last_error.clear();
    return GDN_OK;
}

gdn_status gdn_chunk_prep(const gdn_desc* desc, const void* k, const void* v, const float* g,
                          const float* beta, const int32_t* cu_seqlens, float* gamma_out, float* W_out,
                          float* U_out, void* stream) {
    Plan P;
    gdn_status st = make_plan(desc, &P);
    if (st != GDN_OK) return st;
    const bool varlen = desc->host_cu_seqlens != nullptr;
    if (varlen && !cu_seqlens) return fail(GDN_ERR_NULL_ARG, "cu_seqlens is NULL but desc->host_cu_seqlens is set");
    if (!varlen && cu_seqlens) return fail(GDN_ERR_NULL_ARG, "desc->host_cu_seqlens is required with cu_seqlens");
    const bool any = P.n_chunks_total > 0;
    if ((st = check_ptr(k, "k", any)) || (st = check_ptr(v, "v", any)) || (st = check_ptr(g, "g", any)) ||
        (st = check_ptr(beta, "beta", any)) || (st = check_ptr(gamma_out, "gamma_out", any)) ||
        (st = check_ptr(W_out, "W_out", any)) || (st = check_ptr(U_out, "U_out", any)) ||
        (st = check_ptr(cu_seqlens, "cu_seqlens", false, 4)))
        return st;
    gdn::Params p = base_params(desc, P);
    p.k = k; p.v = v; p.g = g; p.beta = beta; p.cu = cu_seqlens;
    p.prep_gamma = gamma_out; p.prep_W = W_out; p.prep_U = U_out;
    // T (split) goes to the start of each chunk's W_out block and gamma, beta to the
    // start of its U_out block; the second kernel reads them and then
    // overwrites the blocks with W and U
    p.prep_T = W_out;
    p.prep_GB = U_out;
    p.t_stride = (int64_t)gdn::kChunk * gdn::kDim;
    p.gb_stride = (int64_t)gdn::kChunk * gdn::kDim;
    const int io = desc->io_dtype == GDN_BF16 ? gdn::kIoBf16 : gdn::kIoF32;
    int e = gdn::launch_prep(p, io, stream);
    if (!e) e = gdn::launch_wu(p, io, stream);
    if (e) return fail(GDN_ERR_HIP, "chunk_prep launch: %s", hipGetErrorString((hipError_t)e));
    g_last_error.clear();
    return GDN_OK;
}

gdn_status gdn_profile_enable(int on) {
    if (on && !g_prof.created) {
        for (int i = 0; i < kProfEvents; ++i) {
            const hipError_t e = hipEventCreate(&g_prof.ev[i]);
            if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
        }
        g_prof.created = true;
    }
    g_prof.on = on != 0;
    g_prof.recorded = false;
    g_last_error.clear();
    return GDN_OK;
}

gdn_status gdn_profile_read(float ms[5]) {
    if (!ms) return fail(GDN_ERR_NULL_ARG, "ms is NULL");
    if (!g_prof.recorded) return fail(GDN_ERR_BAD_OPTION, "no profiled call since gdn_profile_enable");
    hipError_t e = hipEventSynchronize(g_prof.ev[4]);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipEventSynchronize: %s", hipGetErrorString(e));
    // phase i runs from event from[i] to event to[i]; without a split the
    // forward follows the prep directly
    const int from[5] = {0, 1, 2, 3, 0}, to[5] = {1, 2, 3, 4, 4};
    for (int i = 0; i < 5; ++i) {
        ms[i] = 0.f;
        if (i < 4 && !g_prof.ran[i]) continue;
        const int a = (i == 3 && !g_prof.ran[1]) ? 1 : from[i];
        e = hipEventElapsedTime(&ms[i], g_prof.ev[a], g_prof.ev[to[i]]);
        if (e != hipSuccess) return fail(GDN_ERR_HIP, "hipEventElapsedTime: %s", hipGetErrorString(e));
    }
    g_last_error.clear();
    return GDN_OK;
}

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL_ARG: return "GDN_ERR_NULL_ARG: a required pointer is NULL";
        case GDN_ERR_BAD_SHAPE: return "GDN_ERR_BAD_SHAPE: inconsistent sizes";
        case GDN_ERR_UNSUPPORTED_DIM: return "GDN_ERR_UNSUPPORTED_DIM: only d_k = d_v = 128";
        case GDN_ERR_BAD_DTYPE: return "GDN_ERR_BAD_DTYPE: unknown io dtype";
        case GDN_ERR_MISALIGNED: return "GDN_ERR_MISALIGNED: pointer alignment";
        case GDN_ERR_BAD_SCALE: return "GDN_ERR_BAD_SCALE: scale is not finite";
        case GDN_ERR_WORKSPACE_TOO_SMALL: return "GDN_ERR_WORKSPACE_TOO_SMALL";
        case GDN_ERR_BAD_OPTION: return "GDN_ERR_BAD_OPTION: option out of range";
        case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP runtime error";
    }
    return "unknown gdn_status";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
