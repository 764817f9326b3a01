// Launchers implemented in the .hip translation units and called by the C ABI (api.cpp).
#pragma once

#include <hip/hip_runtime.h>

#include "device.hpp"

namespace pdk {

hipError_t launch_decode_valu(const DecodeParams& p, int kv_dtype, int D, int PS, int gp,
                              unsigned grid, hipStream_t st);
// persistent: grid = the jobs upper bound (units x num_chunks), capped at the workgroups that fit
// on the device; otherwise one workgroup per (chunk, unit) and grid is that count.
// rope: apply RoPE (bf16 or fp8 KV).
hipError_t launch_decode_mfma(const DecodeParams& p, int kv_dtype, int D, int PS, int gp,
                              bool persistent, bool rope, long long grid, hipStream_t st);
hipError_t launch_merge_state(const MergeParams& p, int v_dtype, hipStream_t st);
hipError_t launch_append(const AppendParams& p, int in_dtype, int kv_dtype, hipStream_t st);

}  // namespace pdk
