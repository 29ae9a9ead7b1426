// attn_fwd_d64_int8.hip -- the attention kernel's variants for d = 64 and
// INT8 P~V (templates in attn_fwd_kernel.h; one translation unit per mode so
// that the variants compile in parallel).
#include "attn_fwd_kernel.h"

namespace sage {
template hipError_t attn_launch_dp<64, kPvInt8>(const AttnArgs&, hipStream_t);
}  // namespace sage
