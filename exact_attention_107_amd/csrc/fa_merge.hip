// Merge of split-KV partial results: for each query row, the key ranges'
// normalised outputs O_s and log-sum-exps LSE_s combine into the result over
// all keys as  LSE = ln sum_s exp(LSE_s),  O = sum_s exp(LSE_s - LSE) O_s
// (the rescaling that a split of the key/value sequence needs: FlashAttention
// 1-4 post, FlashAttention-2 section, parallelism along the sequence).
//
// Bandwidth-bound: per row it reads nsplit * (d + 1) fp32 values and writes d
// bf16 values and one fp32 LSE.  Threads own 4 consecutive columns of one row
// (one 16-byte load per split); rows are taken in LSE order (b, h, i) so the
// LSE reads and writes of a workgroup are contiguous, while each row's d
// columns stay one contiguous segment of O.

#include <hip/hip_runtime.h>

#include "fa_kernel.hpp"

namespace fa_detail {

namespace {

constexpr int kMergeThreads = 256;

template <int D>
__global__ void __launch_bounds__(kMergeThreads) fa_merge_kernel(MergeParams mp) {
    constexpr int TPR = D / 4;                 // threads per row
    constexpr int RPB = kMergeThreads / TPR;   // rows per workgroup
    const long long r = static_cast<long long>(blockIdx.x) * RPB + threadIdx.x / TPR;
    if (r >= mp.rows) return;
    const int part = threadIdx.x % TPR;
    // r = (b * H + h) * N + i: the LSE index; O row (b * N + i) * H + h
    const long long bh = r / mp.N;
    const int i = static_cast<int>(r - bh * mp.N);
    const int h = static_cast<int>(bh % mp.H);
    const long long b = bh / mp.H;
    const long long orow = (b * mp.N + i) * mp.H + h;

    float m = -INFINITY;
    for (int s = 0; s < mp.nsplit; ++s) m = fmaxf(m, mp.lp[s * mp.lstride + r]);
    const float ref = (m == -INFINITY) ? 0.0f : m;  // no key at all: every weight is 0
    constexpr float kLog2e = 1.44269504088896340736f;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float wsum = 0.0f;
    for (int s = 0; s < mp.nsplit; ++s) {
        const float w = __builtin_amdgcn_exp2f((mp.lp[s * mp.lstride + r] - ref) * kLog2e);
        if (w != 0.0f) {  // a range without keys contributes nothing; skip its read
            const f32x4 v = *reinterpret_cast<const f32x4 *>(mp.op + s * mp.ostride + orow * D + part * 4);
            acc += w * v;
            wsum += w;
        }
    }
    const float inv = wsum > 0.0f ? 1.0f / wsum : 0.0f;
    const u32x2 packed = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv)};
    *reinterpret_cast<u32x2 *>(mp.o + orow * D + part * 4) = packed;
    if (part == 0) mp.lse[r] = wsum > 0.0f ? ref + log2f(wsum) * kLn2 : -INFINITY;
}

template <int D>
int launch(const MergeParams &mp, void *stream) {
    constexpr int RPB = kMergeThreads / (D / 4);
    const long long grid = (mp.rows + RPB - 1) / RPB;
    if (grid <= 0 || grid > 0x7fffffffLL) return -1;
    hipLaunchKernelGGL(fa_merge_kernel<D>, dim3(static_cast<unsigned>(grid)), dim3(kMergeThreads), 0,
                       static_cast<hipStream_t>(stream), mp);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_merge(const MergeParams &mp, int d, void *stream) {
    switch (d) {
        case 64: return launch<64>(mp, stream);
        case 128: return launch<128>(mp, stream);
        case 256: return launch<256>(mp, stream);
        default: return -1;
    }
}

}  // namespace fa_detail
