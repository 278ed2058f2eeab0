// Kernel-launch stand-ins for the host-only sanitizer build of gdn_api.cpp:
// the validation and planning code runs for real, the launchers record that
// they were reached and launch nothing.
#include "gdn_internal.h"

namespace gdn {
int g_launches = 0;
static int reached() {
    ++g_launches;
    return 0;
}
int launch_bwd(const BwdParams&, void*) { return reached(); }
int launch_bwd_sum(const BwdParams&, long long, void*) { return reached(); }
int launch_bwd_chain_mma(const BwdParams&, void*) { return reached(); }
int launch_bwd_chunk_mma(const BwdParams&, void*) { return reached(); }
int launch_round_bf16(const float*, void*, long long, void*) { return reached(); }
int launch_prep(const Params&, int, void*) { return reached(); }
int launch_wu(const Params&, int, void*) { return reached(); }
int launch_cp_prep(const Params&, int, void*) { return reached(); }
int launch_cp_combine(const Params&, void*) { return reached(); }
int launch_fwd(const Params&, int, void*) { return reached(); }
int launch_fwd_states(const Params&, int, void*) { return reached(); }
int launch_debug_path(const Params&, int32_t*, void*) { return reached(); }
int launch_decode(const Params&, int, void*) { return reached(); }
int launch_cp_prep16(const Params&, int, void*) { return reached(); }
int launch_combine16(const Params&, void*) { return reached(); }
int launch_fwd16(const Params&, int, void*) { return reached(); }
int launch_tiles_to_rm(const float*, float*, long long, void*) { return reached(); }
}  // namespace gdn
