// Kernel instances of the attention forward for head dimension 256.
#include "fa_kernel.hpp"

namespace fa_detail {

KernelFn select_d256(bool causal, bool varlen, int exp_mode, int rescale_mode) {
    return select_kernel<256>(causal, varlen, exp_mode, rescale_mode);
}

KernelFn select_split_d256(bool causal, bool varlen) { return select_split<256>(causal, varlen); }

KernelFn select_mods_d256(bool varlen) { return select_mods<256>(varlen); }

}  // namespace fa_detail
