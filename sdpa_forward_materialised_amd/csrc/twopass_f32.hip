// Two-sweep kernel instantiations for f32 inputs.
#include "twopass.h"

namespace sdpa {

int launch_twopass_f32(int D, int mask_kind, int waves, bool vec, bool drop, const FwdArgs& a, void* stream) {
    return launch_twopass_t<float>(D, mask_kind, waves, vec, drop, a, stream);
}

bool twopass_nl_ok_f32(int D, int mask_kind) { return twopass_nl_ok_t<float>(D, mask_kind); }

}  // namespace sdpa
