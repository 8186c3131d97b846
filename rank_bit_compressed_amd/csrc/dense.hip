// dense.hip -- dense bf16 paged decode attention (placeholder until implemented).
#include "kvc_common.hpp"

namespace kvc {
kvc_status dense_impl(const kvc_dense_in&, float*, void*, size_t, hipStream_t, size_t*) { return KVC_ERR_UNSUPPORTED; }
}  // namespace kvc
