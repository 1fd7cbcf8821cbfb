// fa_lowbit.hip -- low-bit path (int8 Q.K^T, fp8 e4m3 P.V) and its quantiser.
#include "fa_internal.h"

namespace fa {

hipError_t launch_attn_lowbit(const AttnArgs &, int, int, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_quant_lowbit(const QuantArgs &, hipStream_t) { return hipErrorNotSupported; }

}  // namespace fa

extern "C" fa_status fa_quantize_lowbit(const fa_layout *, const fa_io *, const fa_io *, int32_t,
                                        fa_hip_stream) {
  return FA_ERR_UNSUPPORTED;
}
