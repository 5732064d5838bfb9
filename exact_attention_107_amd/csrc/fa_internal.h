// Declarations shared by the kernel translation units (one per head
// dimension) and the C ABI unit of libfa.so.
#pragma once

#include <stdint.h>

namespace fa_detail {

// Kernel arguments.
struct Params {
    const uint16_t *q, *k, *v;  // bf16 bit patterns
    uint16_t *o;
    float *lse;
    const int32_t *cu;  // packed offsets, or nullptr (dense)
    int B, H, N;        // N: sequence length (dense) or total tokens (packed)
    int n_qt;           // dense: query tiles per sequence
    float cs;           // scale * log2(e)
};

using KernelFn = void (*)(Params);

// Launch geometry shared by every instance.
constexpr int kWorkgroupWaves = 4;               // waves per workgroup
constexpr int kTileRows = kWorkgroupWaves * 32;  // query rows per workgroup
constexpr int kTileKeys = 64;                    // keys per K/V tile

// Kernel instance for head dimension D (defined in fa_kernels_d<D>.hip).
KernelFn select_d64(bool causal, bool varlen, int exp_mode, int rescale_mode);
KernelFn select_d128(bool causal, bool varlen, int exp_mode, int rescale_mode);
KernelFn select_d256(bool causal, bool varlen, int exp_mode, int rescale_mode);

}  // namespace fa_detail
