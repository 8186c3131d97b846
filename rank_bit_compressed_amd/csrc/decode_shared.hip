// decode_shared.hip -- decode attention over a block-shared latent (placeholder until implemented).
#include "kvc_common.hpp"

namespace kvc {
bool shared_supported(const kvc_layout&) { return false; }
size_t shared_ws_bytes(const kvc_layout&, int, int) { return 0; }
hipError_t launch_decode_shared(const kvc_layout&, const kvc_cache&, const kvc_decode_in&, float*, void*, int, int,
                                hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace kvc
