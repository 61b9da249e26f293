// Chunkwise prefill (placeholder until the kernel lands).
#include "common.h"
#include "kernels.h"

namespace pdn {
size_t chunk_fwd_workspace_bytes(const pdn_chunk_fwd_args&) { return 0; }
hipError_t launch_chunk_fwd(const pdn_chunk_fwd_args&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace pdn
