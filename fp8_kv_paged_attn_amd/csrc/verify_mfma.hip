// verify_mfma.hip - MFMA verify kernel for gfx950 (placeholder until built).
#include "pa_internal.h"

namespace pa {

hipError_t launch_verify_mfma(const VerifyArgs &, int, bool, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace pa
