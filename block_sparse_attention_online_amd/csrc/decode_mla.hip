// Split-KV skip-softmax decode over a shared latent cache (many query heads,
// one 576-wide latent KV row whose first 512 columns are the value).
// Not built yet: decode_mla_supported() reports no support, and
// ss_attn_decode() returns SS_ERR_UNSUPPORTED for these shapes.

#include "device_common.h"
#include "launch.h"

namespace ssattn {

bool decode_mla_supported(int, int, int, bool) { return false; }

int decode_mla_max_tiles(int) { return 1; }

hipError_t launch_decode_mla(const DecodeArgs&, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace ssattn
