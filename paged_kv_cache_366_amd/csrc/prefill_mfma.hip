// Placeholder until the matrix-core prefill kernel lands.
#include "attention_common.h"

namespace pkv {
pkv_status launch_prefill_mfma(const AttnArgs&, pkv_dtype, int, int, int, hipStream_t) {
  return fail(PKV_ERR_UNSUPPORTED, "MFMA prefill not built");
}
}  // namespace pkv
