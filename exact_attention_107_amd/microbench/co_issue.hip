// Issue-rate microbenchmarks of one gfx950 SIMD: dense BF16 MFMA, the VALU
// instructions the attention softmax issues per score (FMA, exp, add, max3,
// bf16 pack), and the two mixed in one instruction stream or split between
// the SIMD's waves.  Each wave times its own loop with s_memtime (shader
// clock cycles), so the figures do not depend on the clock under load.
//
// Loop body, per iteration: NM MFMAs (v_mfma_f32_32x32x16_bf16, NC
// independent accumulator chains) and, after each MFMA, NV VALU
// instructions of kind KIND over 16 rotating registers (no instruction reads
// a register written fewer than 8 instructions before).  ROLE splits the
// work between the two waves of a SIMD: 0 = both run the same mix, 1 = even
// waves run only the MFMAs and odd waves only the VALU instructions.
//
// Results: one line per configuration, cycles per iteration per SIMD
// (median over waves).  Built and run by run_co_issue.py.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Kind { FMA = 0, EXP = 1, ADD = 2, MAX3 = 3, CVT = 4, MIX = 5 };

template <int KIND>
__device__ __forceinline__ void valu(float (&r)[16], int k, float c1, float c2) {
    float &dst = r[k & 15];
    const float src = r[(k + 8) & 15];
    if constexpr (KIND == FMA) {
        asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(dst) : "v"(src), "v"(c1), "v"(c2));
    } else if constexpr (KIND == EXP) {
        asm volatile("v_exp_f32 %0, %1" : "=v"(dst) : "v"(src));
    } else if constexpr (KIND == ADD) {
        asm volatile("v_add_f32 %0, %1, %2" : "=v"(dst) : "v"(src), "v"(c1));
    } else if constexpr (KIND == MAX3) {
        asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(dst) : "v"(src), "v"(c1), "v"(c2));
    } else if constexpr (KIND == CVT) {
        asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(dst) : "v"(src), "v"(c1));
    } else {
        // the softmax's per-score mix: FMA, exp, add, and a max3 / pack on
        // alternate scores (4 instructions per 2 VALU slots of this loop)
        if ((k & 3) == 0) asm volatile("v_fma_f32 %0, %1, %2, %3" : "=v"(dst) : "v"(src), "v"(c1), "v"(c2));
        else if ((k & 3) == 1) asm volatile("v_exp_f32 %0, %1" : "=v"(dst) : "v"(src));
        else if ((k & 3) == 2) asm volatile("v_add_f32 %0, %1, %2" : "=v"(dst) : "v"(src), "v"(c1));
        else if ((k & 7) == 3) asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(dst) : "v"(src), "v"(c1), "v"(c2));
        else asm volatile("v_cvt_pk_bf16_f32 %0, %1, %2" : "=v"(dst) : "v"(src), "v"(c1));
    }
}

template <int AGPR>
__device__ __forceinline__ void mfma(f32x16 &acc, bf16x8 x, bf16x8 y) {
    if constexpr (AGPR)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(x), "v"(y));
    else
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(x), "v"(y));
}

// ROLE 0: every wave runs the mixed stream.  ROLE 1 / 2: the SIMD's first
// wave (waves 0-3 of the workgroup; waves w and w + 4 share a SIMD) runs only
// the MFMAs, the second only the VALU instructions, each in a loop of its
// own (the role is chosen once, outside the loop); ROLE 2 also raises the
// MFMA wave's priority (s_setprio 1).
template <int NM, int NC, int NV, int KIND, int ROLE, int AGPR>
__global__ void __launch_bounds__(512) probe(unsigned long long *cycles, float *sink, int iters) {
    f32x16 acc[4] = {};
    bf16x8 x, y;
    for (int i = 0; i < 8; ++i) {
        x[i] = (__bf16)(1e-3f * (threadIdx.x + i));
        y[i] = (__bf16)(2e-3f * i);
    }
    float r[16];
    for (int i = 0; i < 16; ++i) r[i] = 1e-3f * (threadIdx.x + i);
    const float c1 = 0.999f, c2 = 1e-7f;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    __syncthreads();
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    if constexpr (ROLE == 0) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                mfma<AGPR>(acc[m % NC], x, y);
#pragma unroll
                for (int k = 0; k < NV; ++k) valu<KIND>(r, m * NV + k, c1, c2);
            }
        }
    } else if ((wave & 4) == 0) {
        if constexpr (ROLE == 2) __builtin_amdgcn_s_setprio(1);
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int m = 0; m < NM; ++m) mfma<AGPR>(acc[m % NC], x, y);
        }
        if constexpr (ROLE == 2) __builtin_amdgcn_s_setprio(0);
    } else {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int k = 0; k < NM * NV; ++k) valu<KIND>(r, k, c1, c2);
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += r[i];
    for (int c = 0; c < 4; ++c)
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
    if ((threadIdx.x & 63) == 0) cycles[blockIdx.x * (blockDim.x / 64) + wave] = t1 - t0;
}

struct Result {
    double per_iter;
};

template <int NM, int NC, int NV, int KIND, int ROLE, int AGPR>
void run(const char *name, int waves_per_simd, int iters, unsigned long long *dcyc, float *dsink) {
    const int blocks = 256, threads = 256 * waves_per_simd;
    auto k = probe<NM, NC, NV, KIND, ROLE, AGPR>;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), 0, 0, dcyc, dsink, 4);
    hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), 0, 0, dcyc, dsink, iters);
    if (hipDeviceSynchronize() != hipSuccess) {
        printf("%s: launch failed\n", name);
        exit(1);
    }
    const int nw = blocks * threads / 64;
    std::vector<unsigned long long> h(nw);
    hipMemcpy(h.data(), dcyc, nw * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    std::sort(h.begin(), h.end());
    const double med = static_cast<double>(h[nw / 2]) / iters;
    const int mfma_per_simd = NM * (ROLE == 0 ? waves_per_simd : 1);
    const int valu_per_simd = NM * NV * (ROLE == 0 ? waves_per_simd : 1);  // roles: one wave each
    printf("%-34s waves/SIMD %d | per SIMD and iteration: %2d MFMA %3d VALU | %7.1f cycles "
           "(MFMA alone %4d) | MFMA busy %5.1f%%\n",
           name, waves_per_simd, mfma_per_simd, valu_per_simd, med, 32 * mfma_per_simd,
           100.0 * 32 * mfma_per_simd / med);
}

int main() {
    unsigned long long *dcyc;
    float *dsink;
    if (hipMalloc(&dcyc, 256 * 8 * sizeof(unsigned long long)) != hipSuccess ||
        hipMalloc(&dsink, 256 * 512 * sizeof(float)) != hipSuccess)
        return 1;
    const int it = 4000;
    printf("# s_memtime cycles; v_mfma_f32_32x32x16_bf16 = 32768 flop, 32 cycles at 1024 flop/clk/SIMD\n");
    for (int w : {1, 2}) {
        run<4, 4, 0, FMA, 0, 0>("mfma only, 4 chains", w, it, dcyc, dsink);
        run<4, 1, 0, FMA, 0, 0>("mfma only, 1 chain", w, it, dcyc, dsink);
        run<4, 4, 0, FMA, 0, 1>("mfma only, 4 chains, AGPR", w, it, dcyc, dsink);
    }
    printf("# VALU alone (1 wave/SIMD; 32 VALU + 1 MFMA per iteration)\n");
    run<1, 1, 32, FMA, 0, 0>("fma", 1, it, dcyc, dsink);
    run<1, 1, 32, EXP, 0, 0>("exp", 1, it, dcyc, dsink);
    run<1, 1, 32, ADD, 0, 0>("add", 1, it, dcyc, dsink);
    run<1, 1, 32, MAX3, 0, 0>("max3", 1, it, dcyc, dsink);
    run<1, 1, 32, CVT, 0, 0>("cvt_pk_bf16", 1, it, dcyc, dsink);
    run<1, 1, 32, MIX, 0, 0>("softmax mix", 1, it, dcyc, dsink);
    printf("# MFMA with VALU after each MFMA, same wave (4 chains)\n");
    for (int w : {1, 2}) {
        run<4, 4, 2, FMA, 0, 0>("mfma + 2 fma", w, it, dcyc, dsink);
        run<4, 4, 4, FMA, 0, 0>("mfma + 4 fma", w, it, dcyc, dsink);
        run<4, 4, 6, FMA, 0, 0>("mfma + 6 fma", w, it, dcyc, dsink);
        run<4, 4, 8, FMA, 0, 0>("mfma + 8 fma", w, it, dcyc, dsink);
        run<4, 4, 2, EXP, 0, 0>("mfma + 2 exp", w, it, dcyc, dsink);
        run<4, 4, 4, EXP, 0, 0>("mfma + 4 exp", w, it, dcyc, dsink);
        run<4, 4, 4, MIX, 0, 0>("mfma + 4 softmax mix", w, it, dcyc, dsink);
        run<4, 4, 5, MIX, 0, 0>("mfma + 5 softmax mix", w, it, dcyc, dsink);
        run<4, 4, 6, MIX, 0, 0>("mfma + 6 softmax mix", w, it, dcyc, dsink);
        run<4, 4, 8, MIX, 0, 0>("mfma + 8 softmax mix", w, it, dcyc, dsink);
    }
    printf("# split roles on one SIMD: one wave only MFMA, the other only VALU (2 waves/SIMD)\n");
    run<4, 4, 4, FMA, 1, 0>("split: 4 mfma | 16 fma", 2, it, dcyc, dsink);
    run<4, 4, 6, FMA, 1, 0>("split: 4 mfma | 24 fma", 2, it, dcyc, dsink);
    run<4, 4, 8, FMA, 1, 0>("split: 4 mfma | 32 fma", 2, it, dcyc, dsink);
    run<4, 4, 4, MIX, 1, 0>("split: 4 mfma | 16 softmax mix", 2, it, dcyc, dsink);
    run<4, 4, 5, MIX, 1, 0>("split: 4 mfma | 20 softmax mix", 2, it, dcyc, dsink);
    run<4, 4, 6, MIX, 1, 0>("split: 4 mfma | 24 softmax mix", 2, it, dcyc, dsink);
    run<4, 4, 8, MIX, 1, 0>("split: 4 mfma | 32 softmax mix", 2, it, dcyc, dsink);
    run<4, 4, 5, MIX, 2, 0>("split+prio: 4 mfma | 20 mix", 2, it, dcyc, dsink);
    run<4, 4, 6, MIX, 2, 0>("split+prio: 4 mfma | 24 mix", 2, it, dcyc, dsink);
    run<4, 4, 8, MIX, 2, 0>("split+prio: 4 mfma | 32 mix", 2, it, dcyc, dsink);
    run<4, 4, 6, MIX, 1, 1>("split: 4 mfma AGPR | 24 mix", 2, it, dcyc, dsink);
    run<4, 4, 6, EXP, 1, 0>("split: 4 mfma | 24 exp", 2, it, dcyc, dsink);
    (void)hipFree(dcyc);
    (void)hipFree(dsink);
    return 0;
}
