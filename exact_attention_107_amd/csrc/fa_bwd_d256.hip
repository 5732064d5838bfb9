// Kernel instances of the attention backward for head dimension 256.
#include "fa_bwd_kernel.hpp"

namespace fa_detail {

BwdKernels select_bwd_d256(bool causal, bool packed) { return select_bwd<256>(causal, packed); }

}  // namespace fa_detail
