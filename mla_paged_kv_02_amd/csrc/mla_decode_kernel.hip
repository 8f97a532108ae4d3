// mla_decode_kernel.hip - dispatch of the decode kernel chosen by the plan.
#include "mla_internal.h"

namespace mla {

hipError_t launch_decode(const Plan& plan, const DecodeArgs& args, hipStream_t stream) {
    switch (plan.kernel) {
        case DecodeKernel::Rows16: return launch_decode_rows16(plan, args, stream);
        case DecodeKernel::WaveSplit: return launch_decode_ws(plan, args, stream);
        case DecodeKernel::Rows16Fp8: return launch_decode_rows16_fp8(plan, args, stream);
        case DecodeKernel::FusedWave: return launch_decode_fw(plan, args, stream);
        case DecodeKernel::WaveSplitFp8: return launch_decode_ws_fp8(plan, args, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace mla
