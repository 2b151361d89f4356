// prefill_fast.hip -- matrix-core (bf16 MFMA) chunked prefill for Dk = Dv = 128.
#include "internal.h"

namespace dn {

bool prefill_fast_supported(const PrefillArgs&) { return false; }
size_t prefill_fast_workspace_bytes(const PrefillArgs&) { return 0; }
hipError_t launch_prefill_fast(const PrefillArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace dn
