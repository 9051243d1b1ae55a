// Two-sweep kernel instantiations for f16 inputs.
#include "twopass.h"

namespace sdpa {

int launch_twopass_f16(int D, int mask_kind, int waves, bool vec, bool drop, const FwdArgs& a, void* stream) {
    return launch_twopass_t<_Float16>(D, mask_kind, waves, vec, drop, a, stream);
}

bool twopass_nl_ok_f16(int D, int mask_kind) { return twopass_nl_ok_t<_Float16>(D, mask_kind); }

}  // namespace sdpa
