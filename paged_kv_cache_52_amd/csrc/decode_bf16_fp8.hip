// Decode kernel instances for q dtype / cache dtype BF16 / FP8 (OCP E4M3).
#include "pa_internal.h"

namespace pa {

hipError_t decode_bf16_fp8(const DecodeParams &p, int64_t max_entries, hipStream_t s) {
  return dispatch_decode<PA_BF16, PA_FP8>(p, max_entries, s);
}

}  // namespace pa
