// Tiled (prefill-shaped) grouped GEMM of the routed experts: not built yet; the host
// layer reports W4A8_ERR_UNSUPPORTED for token counts the streaming kernel cannot take.
#include "common.h"
#include "kernels.h"

namespace w4a8 {

bool prefill_available() { return false; }
size_t prefill_gemm2_partial_bytes(int T, int H) { return (size_t)2 * T * H * sizeof(float); }
void launch_moe_prefill(const MoeGemmParams&, bool, hipStream_t) {}

}  // namespace w4a8
