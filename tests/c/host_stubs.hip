// Stand-in launchers for a host-only build of the C entry points (csrc/capi.hip): they record
// that a launch was requested and return success without touching a GPU, so a sanitized build
// of the host validation runs on a machine with no GPU. Test infrastructure only.
#include "sa_internal.h"

#include <cstdio>

extern "C" int sa_stub_launches = 0;

namespace {
// Reports at exit how many launches the validation let through (the C client expects none).
struct Report {
    ~Report() { std::fprintf(stderr, "stub launches: %d\n", sa_stub_launches); }
} report;
}  // namespace

namespace sa {

hipError_t launch_attn_fwd(const AttnArgs&, hipStream_t) {
    ++sa_stub_launches;
    return hipSuccess;
}
int64_t attn_workspace_bytes(int d) { return (int64_t)2 * 256 * 8 * 64 * (2 * (d / 32) + 1) * 16; }
int64_t attn_scratch_bytes() { return attn_workspace_bytes(128); }
hipError_t attn_scratch(void** out) {
    static char fake[16];
    *out = fake;
    return hipSuccess;
}
hipError_t launch_qk_norm_rope(const NormRopeArgs&, hipStream_t) {
    ++sa_stub_launches;
    return hipSuccess;
}
hipError_t launch_copy_rows(const CopyArgs&, hipStream_t) {
    ++sa_stub_launches;
    return hipSuccess;
}

}  // namespace sa
