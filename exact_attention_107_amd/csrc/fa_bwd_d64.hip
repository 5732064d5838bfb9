// Kernel instances of the attention backward for head dimension 64.
#include "fa_bwd_kernel.hpp"

namespace fa_detail {

BwdKernels select_bwd_d64(bool causal, bool packed) { return select_bwd<64>(causal, packed); }

}  // namespace fa_detail
