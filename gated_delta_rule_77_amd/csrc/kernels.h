// Launch entry points of the gfx950 kernels, called by the host layer after
// argument validation.  Not a public header.
#pragma once
#include <hip/hip_runtime.h>

#include "pdn.h"

namespace pdn {

// Single-token state update for every (b,h); returns a hipError_t.
hipError_t launch_decode(const pdn_decode_args& a, hipStream_t stream);

// Chunkwise prefill; returns a hipError_t.
hipError_t launch_chunk_fwd(const pdn_chunk_fwd_args& a, hipStream_t stream);

// Throughput prefill for per-token scalar decay and gain, bf16, dk = 128.
bool chunk_fact_supported(const pdn_chunk_fwd_args& a);
hipError_t launch_chunk_fact(const pdn_chunk_fwd_args& a, hipStream_t stream);

// Throughput prefill for per-channel gates and the preconditioner, bf16,
// dk = 128; needs chunk_vec_workspace_bytes() of workspace.
bool chunk_vec_supported(const pdn_chunk_fwd_args& a);
size_t chunk_vec_workspace_bytes(const pdn_chunk_fwd_args& a);
hipError_t launch_chunk_vec(const pdn_chunk_fwd_args& a, hipStream_t stream);

// Scratch bytes the prefill needs for these (valid) arguments.
size_t chunk_fwd_workspace_bytes(const pdn_chunk_fwd_args& a);

// Backward of the prefill (any q/k/v dtype, dk in {64, 128}, dv % 32 == 0).
size_t chunk_bwd_workspace_bytes(const pdn_chunk_bwd_args& a);
hipError_t launch_chunk_bwd(const pdn_chunk_bwd_args& a, hipStream_t stream);

}  // namespace pdn
