// fp16 instantiations of the matrix-core prefill kernel.
#include "prefill_mfma.h"

namespace sdpa {
hipError_t launch_prefill_f16(const AttnParams& p, int D, bool causal, int mask, bool varlen,
                              hipStream_t stream) {
    return launch_prefill_t<F16>(p, D, causal, mask, varlen, stream);
}
}  // namespace sdpa
