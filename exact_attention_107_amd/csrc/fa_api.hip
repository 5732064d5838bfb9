// C ABI of libfa.so: argument validation, kernel selection and launch of the
// fused exact-attention forward (declarations and contract in include/fa.h).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_internal.h"

using namespace fa_detail;

namespace {

constexpr float kLog2e = 1.44269504088896340736f;

KernelFn pick(int d, bool causal, bool varlen, int expm, int rsm) {
    switch (d) {
        case 64: return select_d64(causal, varlen, expm, rsm);
        case 128: return select_d128(causal, varlen, expm, rsm);
        default: return select_d256(causal, varlen, expm, rsm);
    }
}

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

}  // namespace

extern "C" {

const char *fa_strerror(int code) {
    switch (code) {
        case FA_OK: return "success";
        case FA_ERR_NULLPTR: return "a required pointer argument is NULL";
        case FA_ERR_SHAPE: return "invalid shape: B, H and N must be >= 1 and the sizes must fit";
        case FA_ERR_HEAD_DIM: return "unsupported head dimension (expected 64, 128 or 256)";
        case FA_ERR_SCALE: return "scale must be finite and > 0";
        case FA_ERR_ALIGN: return "misaligned pointer (q, k, v, o need 16 bytes; lse, cu_seqlens 4)";
        case FA_ERR_VARIANT: return "exp_mode or rescale_mode out of range";
        case FA_ERR_ALIAS: return "an output overlaps an input or the other output";
        case FA_ERR_HIP: return "HIP kernel launch failed";
        default: return "unknown fa status code";
    }
}

int fa_tile_rows(int d) { return tile_rows_for(d); }

int fa_tile_keys(int d) { return (d == 64 || d == 128 || d == 256) ? kTileKeys : 0; }

int fa_fwd_variant(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                   int N, int d, float scale, int causal, const int32_t *cu_seqlens,
                   hipStream_t stream, int exp_mode, int rescale_mode) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && d != 256) return FA_ERR_HEAD_DIM;
    if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
    if (exp_mode < FA_EXP_HW || exp_mode > FA_EXP_MIXED) return FA_ERR_VARIANT;
    if (rescale_mode < FA_RESCALE_ALWAYS || rescale_mode > FA_RESCALE_THRESHOLD) return FA_ERR_VARIANT;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) ||
        misaligned(lse, 4) || misaligned(cu_seqlens, 4))
        return FA_ERR_ALIGN;

    const bool varlen = cu_seqlens != nullptr;
    const long long tokens = varlen ? static_cast<long long>(N) : static_cast<long long>(B) * N;
    const long long elems = tokens * H * d;
    if (elems <= 0 || elems > (1LL << 46)) return FA_ERR_SHAPE;
    const size_t tensor_bytes = static_cast<size_t>(elems) * 2;
    const size_t lse_bytes = static_cast<size_t>(tokens * H) * 4;
    if (overlap(o, tensor_bytes, q, tensor_bytes) || overlap(o, tensor_bytes, k, tensor_bytes) ||
        overlap(o, tensor_bytes, v, tensor_bytes) || overlap(lse, lse_bytes, q, tensor_bytes) ||
        overlap(lse, lse_bytes, k, tensor_bytes) || overlap(lse, lse_bytes, v, tensor_bytes) ||
        overlap(lse, lse_bytes, o, tensor_bytes))
        return FA_ERR_ALIAS;

    Params prm;
    prm.q = static_cast<const uint16_t *>(q);
    prm.k = static_cast<const uint16_t *>(k);
    prm.v = static_cast<const uint16_t *>(v);
    prm.o = static_cast<uint16_t *>(o);
    prm.lse = lse;
    prm.cu = cu_seqlens;
    prm.B = B;
    prm.H = H;
    prm.N = N;
    prm.cs = scale * kLog2e;
    const int rows = tile_rows_for(d);
    const long long n_qt = (static_cast<long long>(N) + rows - 1) / rows;
    prm.n_qt = static_cast<int>(n_qt);
    long long grid;
    if (varlen) {
        grid = static_cast<long long>(H) * (n_qt + B);  // bound on sum_b ceil(n_b / rows)
    } else {
        grid = static_cast<long long>(B) * H * n_qt;
    }
    if (grid <= 0 || grid > 0x7fffffffLL) return FA_ERR_SHAPE;

    KernelFn fn = pick(d, causal != 0, varlen, exp_mode, rescale_mode);
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(grid)), dim3(kWorkgroupWaves * 64), 0, stream, prm);
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    return FA_OK;
}

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N,
           int d, float scale, int causal, const int32_t *cu_seqlens, hipStream_t stream) {
    return fa_fwd_variant(q, k, v, o, lse, B, H, N, d, scale, causal, cu_seqlens, stream,
                          FA_EXP_HW, FA_RESCALE_STRICT);
}

}  // extern "C"
