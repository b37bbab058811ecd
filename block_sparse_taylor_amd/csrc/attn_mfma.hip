// Fused PISA forward for bf16 inputs on gfx950 MFMA (placeholder: routes to the VALU kernel).
#include "common.h"

namespace pisa {

hipError_t launch_attn_fwd_mfma(const Geom& g, const pisa_params_t* p, const void* q, const void* k,
                                const void* v, const pisa_stats_t* st, const int32_t* idx,
                                const float* wgate, void* o, hipStream_t stream) {
    return launch_attn_fwd_valu(g, PISA_BF16, p, q, k, v, st, idx, wgate, o, stream);
}

}  // namespace pisa
