// Decode kernel instances for q dtype / cache dtype BF16 / I8.
#include "pa_internal.h"

namespace pa {

hipError_t decode_bf16_i8(const DecodeParams &p, int64_t max_entries, hipStream_t s) {
  return dispatch_decode<PA_BF16, PA_I8>(p, max_entries, s);
}

}  // namespace pa
