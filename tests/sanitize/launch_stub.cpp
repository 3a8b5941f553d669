// Host-only stand-ins for the HIP launchers, linked with attn_api.cpp into a
// sanitizer build of the C-ABI front end (no GPU code).  The CPU tests call
// the entry points only with arguments that the validation rejects or that
// describe empty problems, so these are never reached; if one is, it reports
// a refused launch.
#include "../../exact_attention_121_amd/csrc/attn_launch.h"

namespace attn {
int launch_forward(const LaunchArgs&, void*) { return 1; }
int launch_forward_d64_one_block(const LaunchArgs&, void*) { return 1; }
int launch_decode(const DecodeArgs&, void*) { return 1; }
int launch_backward(const BwdArgs&, void*) { return 1; }
int launch_backward_noalloc(const BwdArgs&, void*) { return 1; }
}  // namespace attn
