// kda_prefill.hip -- chunked prefill (placeholder until the chunked kernels land).
#include "kda_internal.h"

namespace kda {

size_t prefill_workspace_bytes(int, int, int, int, int, int) { return 0; }

kda_status launch_prefill(const PrefillParams &, int, int, kda_dtype, hipStream_t) {
    return KDA_ERR_UNSUPPORTED;
}

}  // namespace kda
