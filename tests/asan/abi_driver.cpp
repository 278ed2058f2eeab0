// Host-only driver of the C ABI's validation and planning paths, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (no GPU: every case either
// fails validation before any launch or reaches the stand-in launchers).
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gdn.h"

namespace gdn { extern int g_launches; }

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            std::fprintf(stderr, "FAILED %s:%d: %s (%s)\n", __FILE__, __LINE__, \
                         #cond, gdn_last_error());                               \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

static gdn_desc make(int B, int T, int h_qk, int h_v) {
    gdn_desc d;
    std::memset(&d, 0, sizeof d);
    d.B = B; d.T = T; d.h_qk = h_qk; d.h_v = h_v; d.d_k = 128; d.d_v = 128;
    d.n_seqs = B; d.io_dtype = GDN_BF16; d.cp_mode = GDN_CP_AUTO; d.n_cu = 256;
    return d;
}

int main() {
    // planning over many shapes (heap buffers of the planner under ASan)
    const int Ts[] = {0, 1, 63, 64, 65, 1000, 4096, 32768, 262144};
    const int heads[][2] = {{1, 1}, {2, 8}, {8, 24}, {16, 16}, {16, 64}};
    const int modes[] = {GDN_CP_AUTO, GDN_CP_OFF, GDN_CP_EXACT, GDN_CP_WARMUP};
    for (int T : Ts)
        for (auto& hh : heads)
            for (int m : modes)
                for (int B : {1, 3}) {
                    gdn_desc d = make(B, T, hh[0], hh[1]);
                    d.cp_mode = m;
                    gdn_plan_info info;
                    CHECK(gdn_plan(&d, &info) == GDN_OK);
                    CHECK(gdn_fwd_workspace_bytes(&d) == info.workspace_bytes);
                    CHECK(info.L >= 1 && info.n_segments >= B && info.dv_split >= 1);
                    CHECK(gdn_bwd_workspace_bytes(&d) >= info.workspace_bytes);
                }
    // packed sequences, including empty ones
    {
        std::vector<int32_t> cu = {0, 0, 700, 701, 701, 5000};
        gdn_desc d = make(1, 5000, 2, 8);
        d.host_cu_seqlens = cu.data();
        d.n_seqs = (int)cu.size() - 1;
        gdn_plan_info info;
        CHECK(gdn_plan(&d, &info) == GDN_OK);
        cu[3] = 5;    // decreasing
        CHECK(gdn_plan(&d, &info) == GDN_ERR_BAD_SHAPE);
        CHECK(std::strlen(gdn_last_error()) > 0);
    }
    // invalid descriptors
    {
        gdn_plan_info info;
        gdn_desc d = make(1, 64, 3, 8);
        CHECK(gdn_plan(&d, &info) == GDN_ERR_BAD_SHAPE);
        d = make(1, 64, 2, 8); d.d_k = 64;
        CHECK(gdn_plan(&d, &info) == GDN_ERR_UNSUPPORTED_DIM);
        d = make(1, 64, 2, 8); d.io_dtype = 5;
        CHECK(gdn_plan(&d, &info) == GDN_ERR_BAD_DTYPE);
        d = make(1, 64, 2, 8); d.lambda = NAN;
        CHECK(gdn_plan(&d, &info) == GDN_ERR_BAD_OPTION);
        d = make(1, 64, 2, 8); d.dv_split = 3;
        CHECK(gdn_plan(&d, &info) == GDN_ERR_BAD_OPTION);
        d = make(1, 64, 2, 8); d.cp_layout = 3;
        CHECK(gdn_plan(&d, &info) == GDN_ERR_BAD_OPTION);
        CHECK(gdn_plan(nullptr, &info) == GDN_ERR_NULL_ARG);
        CHECK(gdn_fwd_workspace_bytes(nullptr) == 0);
    }
    // forward argument checks (pointers, alignment, workspace) before any launch
    {
        gdn_desc d = make(1, 4096, 2, 8);
        const size_t need = gdn_fwd_workspace_bytes(&d);
        std::vector<unsigned char> host(4096);
        void* p = (void*)(((uintptr_t)host.data() + 255) & ~(uintptr_t)255);
        const int before = gdn::g_launches;
        CHECK(gdn_fwd(&d, nullptr, p, p, (float*)p, (float*)p, 0.1f, nullptr, nullptr, p, nullptr, p, need,
                      nullptr) == GDN_ERR_NULL_ARG);
        CHECK(gdn_fwd(&d, (char*)p + 4, p, p, (float*)p, (float*)p, 0.1f, nullptr, nullptr, p, nullptr, p, need,
                      nullptr) == GDN_ERR_MISALIGNED);
        CHECK(gdn_fwd(&d, p, p, p, (float*)p, (float*)p, NAN, nullptr, nullptr, p, nullptr, p, need, nullptr) ==
              GDN_ERR_BAD_SCALE);
        CHECK(gdn_fwd(&d, p, p, p, (float*)p, (float*)p, 0.1f, nullptr, nullptr, p, nullptr, p, need - 1,
                      nullptr) == GDN_ERR_WORKSPACE_TOO_SMALL);
        CHECK(gdn::g_launches == before);
        // a valid call reaches the launchers (stand-ins here)
        CHECK(gdn_fwd(&d, p, p, p, (float*)p, (float*)p, 0.1f, nullptr, nullptr, p, nullptr, p, need, nullptr) ==
              GDN_OK);
        CHECK(gdn::g_launches > before);
    }
    // backward: bf16 and fp32 inputs (the fp32 workspace adds bf16 copies of q, k, v, d_out)
    for (int io : {GDN_BF16, GDN_F32}) {
        gdn_desc d = make(1, 4096, 2, 8);
        d.io_dtype = io;
        const size_t need = gdn_bwd_workspace_bytes(&d);
        CHECK(need > 0);
        if (io == GDN_F32) {
            gdn_desc d16 = make(1, 4096, 2, 8);
            CHECK(need >= gdn_bwd_workspace_bytes(&d16) + (size_t)4096 * (2 + 8) * 128 * 2 * 2);
        }
        std::vector<unsigned char> host(4096);
        void* p = (void*)(((uintptr_t)host.data() + 255) & ~(uintptr_t)255);
        float* f = (float*)p;
        const int before = gdn::g_launches;
        CHECK(gdn_bwd(&d, p, p, p, f, f, 0.1f, nullptr, nullptr, p, nullptr, p, p, p, f, f, nullptr, p, need - 1,
                      nullptr) == GDN_ERR_WORKSPACE_TOO_SMALL);
        CHECK(gdn::g_launches == before);
        CHECK(gdn_bwd(&d, p, p, p, f, f, 0.1f, nullptr, nullptr, p, nullptr, p, p, p, f, f, nullptr, p, need,
                      nullptr) == GDN_OK);
        CHECK(gdn::g_launches > before);
    }
    // status strings
    for (int s = 0; s <= 9; ++s) CHECK(std::strlen(gdn_status_string((gdn_status)s)) > 0);
    CHECK(gdn_status_string((gdn_status)99) != nullptr);
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("ok\n");
    return 0;
}
