// Prefill path of the expert FFN (grouped bf16 MFMA GEMM).  Not built yet:
// the ABI reports MOE_ERR_UNSUPPORTED for MOE_PATH_PREFILL.
#include "qmoe_internal.h"

namespace qmoe {

size_t prefill_workspace_bytes(int T, int k, int H, int I) {
    (void)H;
    return ((size_t)T * k * I * 2 + 255) & ~(size_t)255;
}

hipError_t launch_ffn_prefill_q4k(const FfnArgs& a, hipStream_t s) {
    (void)a;
    (void)s;
    return hipErrorNotSupported;
}

}  // namespace qmoe
