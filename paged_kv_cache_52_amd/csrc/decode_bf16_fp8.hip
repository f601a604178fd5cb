// Decode kernel instances for q dtype / cache dtype BF16 / FP8 (OCP E4M3).
#include "pa_internal.h"

namespace pa {

hipError_t decode_bf16_fp8(const DecodeParams &p, int grid_splits, hipStream_t s) {
  return dispatch_decode<PA_BF16, PA_FP8>(p, grid_splits, s);
}

}  // namespace pa
