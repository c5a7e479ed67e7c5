// Matrix-core decode attention for grouped query heads (placeholder until the
// kernel lands: reports no support, so the vector kernel handles every case).
#include "pf_attn.h"
#include "pf_internal.h"

namespace pf {
bool mfma_supports(int) { return false; }
int launch_mfma_f16(const AttnArgs&, int, hipStream_t) { return PF_ERR_UNSUPPORTED; }
int launch_mfma_bf16(const AttnArgs&, int, hipStream_t) { return PF_ERR_UNSUPPORTED; }
}  // namespace pf
