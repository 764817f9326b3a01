// Internal entry into the attention call of api.cpp for callers that bring their own scratch at
// fixed places (the no-allocation entry point in noalloc.hip). Not part of the C ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pdecode.h"

namespace pdk {

// A scratch area split into a counter region (split arrivals and job-queue counters, which must be
// zero before a call and which every call leaves at zero) and a partial-state region.
struct FixedScratch {
  int* counters;
  size_t counter_bytes;
  float* partials;
  size_t partial_bytes;
};

// pdecode_attention with the counters and partial states in `fixed`. Plans needing more than
// either region holds return PDECODE_ERR_WORKSPACE_TOO_SMALL before anything is launched.
// check_only: run every host-side check and return without launching (fixed may then hold null
// pointers).
pdecode_status attention_fixed_scratch(const pdecode_desc* d, const void* q, const void* pages,
                                       const int32_t* page_indptr, const int32_t* page_values,
                                       const int32_t* length_info, const pdecode_rope* rope,
                                       float sm_scale, void* out, float* lse,
                                       const FixedScratch* fixed, void* stream, bool check_only);

}  // namespace pdk
