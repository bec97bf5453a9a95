// decode_mfma.hip — placeholder until the matrix-core decode kernel lands.
#include "internal.h"

namespace mla {

bool mfma_supports(const mla_decode_desc*) { return false; }

mla_status launch_decode_mfma(const DecodeArgs&, hipStream_t) {
  return fail(MLA_ERR_UNSUPPORTED, "mfma decode not built");
}

}  // namespace mla
