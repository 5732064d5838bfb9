// Kernel instances of the attention backward for head dimension 128.
#include "fa_bwd_kernel.hpp"

namespace fa_detail {

BwdKernels select_bwd_d128(bool causal, bool packed) { return select_bwd<128>(causal, packed); }

}  // namespace fa_detail
