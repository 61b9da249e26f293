// The per-channel-gate preparation kernel with symmetric keys and per-channel
// decay and gain, built with the instruction-level-parallelism scheduler (see
// build.py).  Kernels in chunk_vec.h; the launch sequence in chunk_vec.hip.
#include "chunk_vec.h"

namespace pdn {

template <bool PRE>
void launch_vec_prep_sym_vec(const PrepParams& p, unsigned grid, hipStream_t s) {
    vec_prep_kernel<true, true, PRE, PDN_KEY_SYMMETRIC, false><<<grid, 256, 0, s>>>(p);
}

template void launch_vec_prep_sym_vec<false>(const PrepParams&, unsigned, hipStream_t);
template void launch_vec_prep_sym_vec<true>(const PrepParams&, unsigned, hipStream_t);

}  // namespace pdn
