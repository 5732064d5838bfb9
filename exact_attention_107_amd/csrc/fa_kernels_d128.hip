// Kernel instances of the attention forward for head dimension 128.
#include "fa_kernel.hpp"

namespace fa_detail {

KernelFn select_d128(bool causal, bool varlen, int exp_mode, int rescale_mode) {
    return select_kernel<128>(causal, varlen, exp_mode, rescale_mode);
}

KernelFn select_split_d128(bool causal, bool varlen) { return select_split<128>(causal, varlen); }

KernelFn select_mods_d128(bool varlen) { return select_mods<128>(varlen); }

KernelFn select_count_d128(bool causal, bool varlen, int rescale_mode) {
    return select_count<128>(causal, varlen, rescale_mode);
}

KernelFn select_ping_d128(bool causal, bool varlen) { return select_ping<128>(causal, varlen); }

KernelFn select_quad_d128(bool causal, bool varlen) { return select_quad<128>(causal, varlen); }

}  // namespace fa_detail
