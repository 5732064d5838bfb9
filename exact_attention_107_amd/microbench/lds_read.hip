// LDS read bandwidth of one gfx950 CU: 16-byte reads (ds_read_b128, the K
// fragment reads of the score product) and 8-byte transposing reads
// (ds_read_b64_tr_b16, the V fragment reads of P V), bank-conflict-free
// address patterns, 4 or 8 waves per workgroup, one workgroup per CU.
// Every value read is folded into a register with XOR (v_xor3_b32: one VALU
// instruction per 16 bytes read), so no read is dead.  Each wave times its
// own loop with s_memtime; bytes per cycle per CU are summed over the waves.
// Build: hipcc --offload-arch=gfx950 -O3 lds_read.hip -o lds_read.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kLdsBytes = 64 * 1024;

template <int TR, int UNROLL>
__global__ void __launch_bounds__(512) lds_probe(unsigned long long *cycles, uint32_t *sink, int iters) {
    __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
    for (int i = threadIdx.x * 16; i < kLdsBytes; i += blockDim.x * 16)
        *reinterpret_cast<u32x4 *>(lds + i) = u32x4{uint32_t(i), uint32_t(i + 1), uint32_t(i + 2), uint32_t(i + 3)};
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t acc = 0;
    // b128: 64 consecutive 16-byte chunks per read (1 KB, every bank once per
    // 256 bytes).  tr16: within 16 lanes, 4 rows x 4 chunks of 8 bytes, rows
    // 256 bytes apart and XOR-swizzled as in the forward kernel's V tile.
    int base;
    if (TR) {
        const int s16 = lane & 15, g16 = lane >> 4;
        const int row = (g16 >> 1) * 4 + (s16 >> 2);
        const int chunk = ((g16 & 1) * 2 + ((s16 & 3) >> 1)) ^ ((row & 3) << 2);
        base = row * 256 + chunk * 16 + (s16 & 1) * 8;
    } else {
        base = lane * 16;
    }
    base += wave * 2048;
    const unsigned long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int off = (base + u * 4096 + it * 64) & (kLdsBytes - 1);
            if (TR) {
                const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) v4i16 *)(lds + off));
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                const u32x2 w = __builtin_bit_cast(u32x2, r);
                acc ^= w[0] ^ w[1];
            } else {
                const u32x4 r = *reinterpret_cast<const u32x4 *>(lds + off);
                acc ^= r[0] ^ r[1] ^ r[2] ^ r[3];
            }
        }
    }
    const unsigned long long t1 = __builtin_amdgcn_s_memtime();
    sink[blockIdx.x * blockDim.x + threadIdx.x] = acc;
    if (lane == 0) cycles[blockIdx.x * (blockDim.x / 64) + wave] = t1 - t0;
}

template <int TR>
void run(const char *name, int waves, int iters, unsigned long long *dcyc, uint32_t *dsink) {
    constexpr int UNROLL = 8;
    auto k = lds_probe<TR, UNROLL>;
    const int blocks = 256, threads = 64 * waves;
    hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), 0, 0, dcyc, dsink, 4);
    hipLaunchKernelGGL(k, dim3(blocks), dim3(threads), 0, 0, dcyc, dsink, iters);
    if (hipDeviceSynchronize() != hipSuccess) {
        printf("%s: launch failed\n", name);
        exit(1);
    }
    std::vector<unsigned long long> h(blocks * waves), per_block(blocks);
    if (hipMemcpy(h.data(), dcyc, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess) exit(1);
    for (int b = 0; b < blocks; ++b) per_block[b] = *std::max_element(h.begin() + b * waves, h.begin() + (b + 1) * waves);
    std::sort(per_block.begin(), per_block.end());
    const double cyc = static_cast<double>(per_block[blocks / 2]);
    const double bytes = static_cast<double>(waves) * iters * UNROLL * 64 * (TR ? 8 : 16);
    printf("%-28s %d waves/CU | %6.1f bytes/cycle/CU\n", name, waves, bytes / cyc);
}

int main() {
    unsigned long long *dcyc;
    uint32_t *dsink;
    if (hipMalloc(&dcyc, 256 * 8 * sizeof(unsigned long long)) != hipSuccess ||
        hipMalloc(&dsink, 256 * 512 * sizeof(uint32_t)) != hipSuccess)
        return 1;
    for (int w : {4, 8}) {
        run<0>("ds_read_b128", w, 2000, dcyc, dsink);
        run<1>("ds_read_b64_tr_b16", w, 2000, dcyc, dsink);
    }
    (void)hipFree(dcyc);
    (void)hipFree(dsink);
    return 0;
}
