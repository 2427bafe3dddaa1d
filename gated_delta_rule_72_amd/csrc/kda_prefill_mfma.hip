// kda_prefill_mfma.hip -- bf16-input chunkwise prefill (dispatch).
#include "kda_internal.h"

namespace kda {

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    return launch_prefill_valu_bf16(a, stream);
}

}  // namespace kda
