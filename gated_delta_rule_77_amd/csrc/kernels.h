// Launch entry points of the gfx950 kernels, called by the host layer after
// argument validation.  Not a public header.
#pragma once
#include <hip/hip_runtime.h>

#include "pdn.h"

namespace pdn {

// Compute units of the current device (hipDeviceGetAttribute; 256 on an
// MI355X), used to size persistent grids and to choose tile widths.
int device_cu_count();

// Workgroups are dealt to the XCDs of an MI355X (eight, each with its own
// L2) in turn.  Launches place the workgroups that read the same head's rows
// on one XCD by this count; it decides L2 locality only, never results.
constexpr int kXcds = 8;

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

// Sequence segments, after the segment runs (either prefill kernel): the
// segments' start states S_{g+1} = Phi_g S_g + N_g from the end states nst
// [nbh][nseg][128][dv] (segment 0 run from the real start state, the others
// from zero) and transitions phi [nbh][nseg][128][128], kept in sst and the
// last one written to ST; then o_t += (Phi_t^T q_t)^T S_g for the tokens of
// segments g >= 1 (qh [nbh][T][128]: the identity-start columns' outputs).
// Segment g holds tokens [g seg_tokens, (g + 1) seg_tokens); dv % 32 == 0.
hipError_t launch_seg_finish(const float* nst, const float* phi, float* sst, float* ST, const float* qh,
                             float* o, long nbh, long T, int nseg, long seg_tokens, int dv,
                             hipStream_t stream);

// Scalar-gate prefill workspace (sequence segments for few heads; else 0).
size_t chunk_fact_workspace_bytes(const pdn_chunk_fwd_args& a);

// Scratch bytes the prefill needs for these (valid) arguments.
size_t chunk_fwd_workspace_bytes(const pdn_chunk_fwd_args& a);

// Backward of the prefill (any q/k/v dtype, dk in {64, 128}, dv % 32 == 0).
size_t chunk_bwd_workspace_bytes(const pdn_chunk_bwd_args& a);
hipError_t launch_chunk_bwd(const pdn_chunk_bwd_args& a, hipStream_t stream);

}  // namespace pdn
