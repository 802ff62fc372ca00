// Chunked prefill (placeholder until the MFMA kernels land).
#include "kda_device.h"
#include "kda_internal.h"

namespace kda {

int64_t prefill_workspace_bytes(const PrefillParams&, int) { return 0; }

int launch_prefill(const PrefillParams&, int, int, int, hipStream_t) {
  return fail(KDA_ERR_UNSUPPORTED, "prefill not built yet");
}

}  // namespace kda
