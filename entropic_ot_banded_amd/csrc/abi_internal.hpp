// Helpers of the C-ABI layer shared by the entry points in api.cpp and
// noalloc.hip (host code only).
#pragma once

#include <hip/hip_runtime_api.h>

#include "../../include/sinkattn.h"
#include "geom.hpp"

namespace sinkattn {

// Validate a shape descriptor and fill the band geometry for band width W
// (SINKATTN_OK, SINKATTN_EINVAL or SINKATTN_EUNSUPPORTED).
int make_geom(const sinkattn_shape* s, int W, Geom* g);
bool aligned16(const void* p);
// SINKATTN_OK for hipSuccess, else SINKATTN_EHIP (recording the HIP error
// for sinkattn_last_hip_error).
int hip_status(hipError_t e);
// SINKATTN_DEBUG is set: the forward entry points check their results.
bool debug_checks();
// Status of a forward launch, with the debug check's findings.
int forward_status(hipError_t e, int flags);

}  // namespace sinkattn
