#include "decode.h"
namespace gdla {
size_t decode_workspace_bytes(const gdla_config*, int) { return 256; }
hipError_t decode_step(const gdla_config*, const gdla_weights*, int, const void*, void*, void*, const int32_t*, int,
                       void*, hipStream_t) {
  return hipErrorNotSupported;
}
}  // namespace gdla
