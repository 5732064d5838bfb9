// Kernel instances of the attention forward for head dimension 64.
#include "fa_kernel.hpp"

namespace fa_detail {

KernelFn select_d64(bool causal, bool varlen, int exp_mode, int rescale_mode) {
    return select_kernel<64>(causal, varlen, exp_mode, rescale_mode);
}

KernelFn select_split_d64(bool causal, bool varlen) { return select_split<64>(causal, varlen); }

KernelFn select_mods_d64(bool varlen) { return select_mods<64>(varlen); }

}  // namespace fa_detail
