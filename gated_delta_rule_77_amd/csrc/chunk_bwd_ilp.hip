// The backward kernels built with the instruction-level-parallelism
// scheduler (see build.py): the state passes on 32-column tiles and the
// gradient kernel.  Kernels in chunk_bwd.h; the launch sequence in
// chunk_bwd.hip.
#include "chunk_bwd.h"

namespace pdn {

template <int DK>
void launch_bwd_states_wide(const BwdParams& p, unsigned grid, long units, hipStream_t s) {
    bwd_states_kernel<DK, JT><<<grid, NT, 0, s>>>(p, units);
}

template <int DK, bool BF16>
void launch_bwd_grads(const BwdParams& p, unsigned grid, hipStream_t s) {
    bwd_grads_kernel<DK, BF16><<<grid, NT, 0, s>>>(p);
}

template void launch_bwd_states_wide<64>(const BwdParams&, unsigned, long, hipStream_t);
template void launch_bwd_states_wide<128>(const BwdParams&, unsigned, long, hipStream_t);
template void launch_bwd_grads<64, false>(const BwdParams&, unsigned, hipStream_t);
template void launch_bwd_grads<64, true>(const BwdParams&, unsigned, hipStream_t);
template void launch_bwd_grads<128, false>(const BwdParams&, unsigned, hipStream_t);
template void launch_bwd_grads<128, true>(const BwdParams&, unsigned, hipStream_t);

}  // namespace pdn
