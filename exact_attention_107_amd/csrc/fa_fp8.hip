// FP8 (E4M3) attention forward instances and the per-head quantisation
// launches (device code in fa_fp8_kernel.hpp).
#include "fa_fp8_kernel.hpp"

namespace fa_detail {

KernelFp8Fn select_fp8_d64(bool causal, bool packed) { return select_fp8<64>(causal, packed); }
KernelFp8Fn select_fp8_d128(bool causal, bool packed) { return select_fp8<128>(causal, packed); }
KernelFp8Fn select_fp8_d256(bool causal, bool packed) { return select_fp8<256>(causal, packed); }

int launch_quant(const QuantParams &qp, void *stream) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const long long bh = static_cast<long long>(qp.B) * qp.H;
    if (qp.cu) {
        // packed: one workgroup per (sequence, head) for both steps
        if (bh > 0x7fffffffLL) return -1;
        hipLaunchKernelGGL(fa_fp8_amax_packed_kernel, dim3(static_cast<unsigned>(bh)), dim3(256), 0, st, qp);
        if (hipGetLastError() != hipSuccess) return -1;
        hipLaunchKernelGGL(fa_fp8_quant_packed_kernel, dim3(static_cast<unsigned>(bh)), dim3(256), 0, st, qp);
        return hipGetLastError() == hipSuccess ? 0 : -1;
    }
    const long long tokens = qp.transpose ? (qp.N + 63) / 64 * 64 : qp.N;
    const long long items = bh * tokens * (qp.d / 4);
    const long long grid = (items + 255) / 256;
    if (bh > 0x7fffffffLL || grid > 0x7fffffffLL) return -1;
    hipLaunchKernelGGL(fa_fp8_amax_kernel, dim3(static_cast<unsigned>(bh)), dim3(256), 0, st, qp);
    if (hipGetLastError() != hipSuccess) return -1;
    hipLaunchKernelGGL(fa_fp8_quant_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, st, qp);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace fa_detail
