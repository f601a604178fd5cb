// Decode kernel instances for q dtype / cache dtype BF16 / BF16.
#include "pa_internal.h"

namespace pa {

hipError_t decode_bf16_bf16(const DecodeParams &p, int64_t max_entries, hipStream_t s) {
  return dispatch_decode<PA_BF16, PA_BF16>(p, max_entries, s);
}

}  // namespace pa
