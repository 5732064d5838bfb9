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
    // token slices per (sequence, head) of the amax (and packed code) kernels:
    // 256 tokens each (dense); packed, twice the average sequence's count
    long long slices;
    if (qp.cu) {
        const long long avg = (static_cast<long long>(qp.N) + 256LL * qp.B - 1) / (256LL * qp.B);
        slices = avg * 2 < 1 ? 1 : (avg * 2 > 1024 ? 1024 : avg * 2);
    } else {
        slices = (static_cast<long long>(qp.N) + 255) / 256;
    }
    const long long sgrid = bh * slices;
    const long long bgrid = (bh + 255) / 256;
    const long long qgrid = qp.cu ? sgrid
                            : qp.transpose ? bh * ((qp.N + 63) / 64)        // 64-key tiles
                                           : (bh * qp.N * (qp.d / 8) + 255) / 256;
    if (sgrid > 0x7fffffffLL || qgrid > 0x7fffffffLL) return -1;
    hipLaunchKernelGGL(fa_fp8_amax_init_kernel, dim3(static_cast<unsigned>(bgrid)), dim3(256), 0, st, qp);
    if (hipGetLastError() != hipSuccess) return -1;
    hipLaunchKernelGGL(fa_fp8_amax_kernel, dim3(static_cast<unsigned>(sgrid)), dim3(256), 0, st, qp);
    if (hipGetLastError() != hipSuccess) return -1;
    if (qp.cu)
        hipLaunchKernelGGL(fa_fp8_quant_packed_kernel, dim3(static_cast<unsigned>(qgrid)), dim3(256), 0, st, qp);
    else if (qp.transpose)
        hipLaunchKernelGGL(fa_fp8_quant_t_kernel, dim3(static_cast<unsigned>(qgrid)), dim3(256), 0, st, qp);
    else
        hipLaunchKernelGGL(fa_fp8_quant_kernel, dim3(static_cast<unsigned>(qgrid)), dim3(256), 0, st, qp);
    if (hipGetLastError() != hipSuccess) return -1;
    hipLaunchKernelGGL(fa_fp8_descale_kernel, dim3(static_cast<unsigned>(bgrid)), dim3(256), 0, st, qp);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace fa_detail
