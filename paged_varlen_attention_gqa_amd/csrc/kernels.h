// Launch entry points of the HIP kernels (host side, internal to librelattn).
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace relattn {

// Each returns 0 on success, -1 when the launch was rejected.
int launch_general(const AttnParams& P, int dtype_bf16, int head_dim, hipStream_t stream);
int launch_decode(const AttnParams& P, int head_dim, hipStream_t stream);
// Whether the decode kernel handles this call's dtype / head_dim / block_size.
bool decode_supported(const AttnParams& P, int dtype_bf16, int head_dim);
// Prefill kernel for requests with more than kDecodeMaxRows packed rows.
bool prefill_supported(const AttnParams& P, int dtype_bf16, int head_dim);
int launch_prefill(const AttnParams& P, hipStream_t stream);
int launch_combine(const AttnParams& P, int dtype_bf16, int head_dim, hipStream_t stream);

// Largest S_b * G the decode kernel handles (one 16-row MFMA tile).
constexpr int kDecodeMaxRows = 16;

}  // namespace relattn
