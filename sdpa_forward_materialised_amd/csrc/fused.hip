// Fused single-sweep kernel (scores kept on chip). Not built yet.
#include "sdpa_device.h"

namespace sdpa {

int launch_fused(int, int, int, int, bool, const FwdArgs&, void*) { return (int)hipErrorNotSupported; }

}  // namespace sdpa
