// msa_route_score, batched form: placeholder until the MFMA scan lands.
#include "msa_internal.h"

namespace msa {

int launch_scan_mfma(const uint16_t*, const RouteGeom&, const uint16_t*, int64_t, int32_t, float*,
                     hipStream_t) {
  return fail(MSA_ERR_UNSUPPORTED, "MFMA routing scan not built");
}

}  // namespace msa
