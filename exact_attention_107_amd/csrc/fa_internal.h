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
    // split of the key sequence (split-KV instances only)
    float *op;          // partial outputs, [nsplit][B*N][H][d] fp32
    float *lp;          // partial LSEs, [nsplit][B][H][N] fp32
    int nsplit;         // number of key ranges per query tile
    // window mask and linear bias (masked instances only)
    int wl, wr;          // key j visible to query i iff i - wl <= j <= i + wr (< 0: unbounded)
    const float *alibi;  // per-head slopes [H], or nullptr
    float inv_scale;     // 1 / scale
    // rescale statistics (counting instances only): [0] wave-steps after the
    // first tile, [1] of them with an O rescale, [2] rows whose reference max
    // moved, [3] rows updated
    unsigned long long *counts;
};

using KernelFn = void (*)(Params);

// Launch geometry.  K/V tiles of 64 keys; each wave owns kBlocks blocks of
// 32 query rows and a workgroup has kWaves waves; kSimdWaves waves fit per
// SIMD (registers).  At d = 128 (two waves per SIMD) an eight-wave workgroup
// per CU shares each K/V tile among twice the rows of a four-wave one,
// halving the direct loads and L2 requests per flop (measured 2-5 % faster
// on long sequences).  At d = 64 three waves fit per SIMD, which only
// four-wave workgroups can fill; d = 256 runs one wave per SIMD.  (Two blocks
// per wave would let each K/V fragment read from LDS feed two MFMAs, but at
// d = 128 the kernel then needs more than the 512 registers of a wave.)
constexpr int kTileKeys = 64;
template <int D> struct Geometry {
    static constexpr int kBlocks = 1;
    static constexpr int kWaves = D == 128 ? 8 : 4;
    static constexpr int kSimdWaves = D == 64 ? 3 : (D == 128 ? 2 : 1);
    static constexpr int kRows = kWaves * 32 * kBlocks;  // query rows per workgroup
    static constexpr int kResident = 4 * kSimdWaves / kWaves;  // workgroups per CU
};
inline int tile_rows_for(int d) {
    switch (d) {
        case 64: return Geometry<64>::kRows;
        case 128: return Geometry<128>::kRows;
        case 256: return Geometry<256>::kRows;
        default: return 0;
    }
}
inline int resident_for(int d) {
    switch (d) {
        case 64: return Geometry<64>::kResident;
        case 128: return Geometry<128>::kResident;
        case 256: return Geometry<256>::kResident;
        default: return 0;
    }
}
inline int waves_for(int d) {
    switch (d) {
        case 64: return Geometry<64>::kWaves;
        case 128: return Geometry<128>::kWaves;
        case 256: return Geometry<256>::kWaves;
        default: return 0;
    }
}

// Kernel instance for head dimension D (defined in fa_kernels_d<D>.hip).
KernelFn select_d64(bool causal, bool varlen, int exp_mode, int rescale_mode);
KernelFn select_d128(bool causal, bool varlen, int exp_mode, int rescale_mode);
KernelFn select_d256(bool causal, bool varlen, int exp_mode, int rescale_mode);
// Instance that also counts rescales (head dimension 128, hardware exp2).
KernelFn select_count_d128(bool causal, bool varlen, int rescale_mode);
// The default forward (hardware exp2, strict rescale) with the two halves of
// the eight-wave workgroup run half a key tile apart (head dimension 128).
KernelFn select_ping_d128(bool causal, bool varlen);
// The default forward at head dimension 128 in four-wave (128-row)
// workgroups, for grids that would leave compute units idle.
KernelFn select_quad_d128(bool causal, bool varlen);
// Window-mask / linear-bias instance (dense or packed layout).
KernelFn select_mods_d64(bool varlen);
KernelFn select_mods_d128(bool varlen);
KernelFn select_mods_d256(bool varlen);
// Split-KV instance (dense or packed layout, partial results into Params::op / lp).
KernelFn select_split_d64(bool causal, bool varlen);
KernelFn select_split_d128(bool causal, bool varlen);
KernelFn select_split_d256(bool causal, bool varlen);

// Merge of split-KV partials (fa_merge.hip).
struct MergeParams {
    const float *op, *lp;  // partials, layouts as in Params
    uint16_t *o;           // bf16 [B*N][H][d]
    float *lse;            // [B][H][N]
    long long rows;        // B*N*H
    long long ostride;     // elements between splits of op
    long long lstride;     // elements between splits of lp
    int H, N, nsplit;
};
int launch_merge(const MergeParams &mp, int d, void *stream);

// Backward pass (fa_bwd_kernel.hpp).
struct BwdParams {
    const uint16_t *q, *k, *v, *o, *dout;  // bf16 [B, N, H, d], packed [T, H, d]
    const float *lse;                      // [B, H, N], packed [H, T]; natural log
    const int32_t *cu;                     // packed: sequence offsets [B + 1]; dense: null
    uint16_t *dq, *dk, *dv;                // bf16, layout of q
    float *stats;                          // two floats per LSE entry, same index:
                                           // LSE*log2(e), delta
    int B, H, N;                           // packed: B sequences, N = T tokens
    float cs;                              // scale * log2(e)
    float scale;
};
using BwdKernelFn = void (*)(BwdParams);
struct BwdKernels {
    BwdKernelFn prep, dkdv, dq;
};
BwdKernels select_bwd_d64(bool causal, bool packed);
BwdKernels select_bwd_d128(bool causal, bool packed);
BwdKernels select_bwd_d256(bool causal, bool packed);

// FP8 (E4M3) forward and quantisation (fa_fp8_kernel.hpp).
struct Fp8Params {
    const uint8_t *q, *k;   // E4M3 codes [B, N, H, d] (packed: [T, H, d])
    const uint8_t *vt;      // E4M3 codes of V transposed, [B, H, d, Np],
                            // Np = ceil(N / 64) * 64, zero padded (packed:
                            // [H, d, vts], each sequence padded to 64 keys)
    const float *dq, *dk, *dv;  // per-(b, h) descales [B * H]
    uint16_t *o;            // bf16 [B, N, H, d] (packed: [T, H, d])
    float *lse;             // [B, H, N] (packed: [H, T])
    const int32_t *cu;      // packed offsets [B + 1], or nullptr (dense)
    int B, H, N;            // N: sequence length (dense) or total tokens T (packed)
    int vts;                // packed: V^T row length in keys
    float cs;               // scale * log2(e)
};
using KernelFp8Fn = void (*)(Fp8Params);
// query rows per FP8 workgroup (32 per wave).  Four waves: an FP8 tile is
// half the bytes of a bf16 one, and eight-wave workgroups measured 5-8 %
// slower here (one barrier couples twice the waves).
template <int D> struct Fp8Geometry {
    static constexpr int kWaves = 4;
    static constexpr int kRows = kWaves * 32;
};
inline int fp8_rows_for(int d) {
    return d == 64 ? Fp8Geometry<64>::kRows : d == 128 ? Fp8Geometry<128>::kRows : Fp8Geometry<256>::kRows;
}
KernelFp8Fn select_fp8_d64(bool causal, bool packed);
KernelFp8Fn select_fp8_d128(bool causal, bool packed);
KernelFp8Fn select_fp8_d256(bool causal, bool packed);
struct QuantParams {
    const uint16_t *x;      // bf16 [B, N, H, d] (packed: [T, H, d])
    uint8_t *x8;            // E4M3 codes [B, N, H, d] or [B, H, d, Np] (packed: [T, H, d] or [H, d, vts])
    float *descale;         // [B * H]
    const int32_t *cu;      // packed offsets [B + 1], or nullptr (dense)
    int B, H, N, d, transpose;
    int vts;                // packed V^T row length in keys
};
int launch_quant(const QuantParams &qp, void *stream);

}  // namespace fa_detail
