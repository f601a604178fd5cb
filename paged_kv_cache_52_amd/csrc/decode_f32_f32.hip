// Decode kernel instances for q dtype / cache dtype F32 / F32.
#include "pa_internal.h"

namespace pa {

hipError_t decode_f32_f32(const DecodeParams &p, int64_t max_entries, hipStream_t s) {
  return dispatch_decode<PA_F32, PA_F32>(p, max_entries, s);
}

}  // namespace pa
