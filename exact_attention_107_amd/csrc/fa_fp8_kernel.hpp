// Device code of the FP8 (E4M3) attention forward for gfx950 and of the
// per-head E4M3 quantisation that feeds it (fa_fp8.hip).
//
// The FlashAttention-3 notes of "FlashAttention 1-4 explained" run the
// forward's two products on FP8 matrix units; here both run as
// v_mfma_f32_32x32x64_f8f6f4 with E4M3 operands and fp32 accumulation:
//  * S^T = K Q^T per 32-key block and 64-wide k step: K (A operand) from LDS,
//    each lane reading 32 consecutive bytes of its key's row; Q (B operand)
//    held in VGPRs for the whole kernel.  Each lane again owns one query row.
//  * P = 2^(s c - m) (strict rescale: m is the running row max, so P <= 1) is
//    computed directly as 2^8 P = 2^(s c - (m - 8)) and rounded to E4M3
//    (v_cvt_pk_fp8_f32, nearest even): the factor keeps values down to 2^-18
//    of the row max out of the flush-to-zero range, and 2^8 P <= 256 stays
//    below the E4M3 maximum 448.  The row sum l is accumulated from the fp32
//    weights.
//  * O^T += V^T P^T takes P as the B operand, whose 64 keys must sit as 32
//    consecutive keys per lane half.  The accumulator gives lane half hh the
//    keys 8g + 4hh + r of both 32-key blocks; one v_permlane32_swap per
//    register pair moves block 0's keys to the lower half and block 1's to
//    the upper half, after which packing four keys per register is exactly
//    the operand order.  V is read from a transposed copy (V^T,
//    [B, H, d, Np] with rows padded with zero codes to Np = ceil(N/64)*64) so
//    that its A operand is again 32 consecutive bytes of one LDS row.
//  * Scores are scaled by scale * descale_q * descale_k (folded into c) and
//    the output by descale_v / l.
//  * Software pipeline as in the bf16 kernel: the S(j+1) MFMAs are issued
//    before the weights of S(j) are computed, the P V(j) MFMAs before the row
//    max of S(j+1).
// LDS rows are 64, 128 or 256 bytes; their 16-byte chunks are XOR-permuted
// so that the 16 rows of one fragment read cover 16 distinct bank groups.
//
// Packed sequences (cu_seqlens): each sequence is its own problem with its
// own per-head scales; work items are decoded like the bf16 packed forward's.
// V^T is [H, d, vts] with each sequence's keys starting at a multiple of 64
// (the sum of the padded lengths of the sequences before it), so that a
// 64-key tile again never crosses a sequence and its tail holds zero codes.

#pragma once

#include "fa_kernel.hpp"

namespace fa_detail {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kFp8Keys = 64;            // keys per K / V^T tile
constexpr float kFp8PScale = 256.0f;    // P is stored as E4M3(2^8 P)

// chunk permutation of row r for rows of RB bytes (RB = 64, 128 or 256)
template <int RB>
__device__ __forceinline__ int fp8_swz(int r) {
    if constexpr (RB == 256) return r & 15;             // one row per 256-byte bank window
    else if constexpr (RB == 128) return (r >> 1) & 7;  // 2 rows per window
    else return (r >> 2) & 3;                           // 4 rows per window
}

// 4 E4M3 codes of a, b, c, d (nearest even; |x| <= 448 required)
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
}

// Column of sequence b's first key in a packed V^T row: the sum of
// ceil(n / 64) * 64 over the sequences before it, summed 64 sequences at a
// time by the wave.  Well-formed offsets keep the sum below the row length
// vts (the host bounds vts below 2^31); the caller skips a sequence whose
// padded keys would end past vts (only malformed offsets, e.g. overlapping
// sequences, get there), and the running sum is capped at vts so it cannot
// overflow.
__device__ __forceinline__ int fp8_packed_vt_start(const int32_t *cu, int b, int T, int vts) {
    const int lane = threadIdx.x & 63;
    int s = 0;
    for (int o0 = 0; o0 < b; o0 += 64) {
        const int o = o0 + lane;
        int v = o < b ? (seq_len(cu, o, T) + 63) / 64 * 64 : 0;
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
        s = min(s + v, vts);
    }
    return __builtin_amdgcn_readfirstlane(s);
}

template <int D, bool CAUSAL, bool PACKED>
__global__ void __launch_bounds__(Fp8Geometry<D>::kWaves * 64) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2)))
fa_fp8_fwd_kernel(Fp8Params p) {
    constexpr int NW = Fp8Geometry<D>::kWaves, BC = kFp8Keys, BR = NW * 32;
    constexpr int KS = D / 64;          // 64-wide k steps of Q K^T
    constexpr int NDB = D / 32;         // 32-wide d blocks of O^T
    constexpr int KRB = D;              // bytes per K row
    constexpr int VRB = BC;             // bytes per V^T row (64 keys)
    constexpr int KT = BC * KRB;        // bytes of a K tile
    constexpr int VT = D * VRB;         // bytes of a V^T tile
    constexpr int KBLK = KT / 1024, VBLK = VT / 1024;
    static_assert(KBLK % NW == 0 && VBLK % NW == 0, "tiles must split over the waves");

    __shared__ __attribute__((aligned(1024))) char k_lds0[KT], k_lds1[KT], v_lds0[VT], v_lds1[VT];

    // work item (sequence b, head h, query tile qt), in the bf16 forward's
    // order: dense causal longest first, dense non-causal in per-XCD runs,
    // packed by sequence through cu_seqlens (surplus workgroups exit)
    Work w;
    {
        Params wp{};
        wp.B = p.B;
        wp.H = p.H;
        wp.N = p.N;
        wp.cu = p.cu;
        wp.n_qt = (p.N + BR - 1) / BR;
        if (!decode_work<CAUSAL, PACKED, BR, false>(wp, w)) return;
    }
    const int b = w.b, h = w.h, qt = w.qt, n = w.n;
    const int bh = b * p.H + h;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, hh = lane >> 5;
    const int q0 = qt * BR;
    const int wrow0 = q0 + wave * 32;
    const int rs = p.H * D;                                   // token stride of q8, k8 (bytes)
    const long long base8 = (w.t0 * p.H + h) * D;             // token 0 of the sequence, head h
    // V^T: row stride np (bytes), the sequence's first key in the head's row
    // 0 at vt, and the bytes from there to the end of the head's rows
    int np;
    const uint8_t *vt;
    long long vspan;
    if constexpr (PACKED) {
        np = p.vts;
        const int start = fp8_packed_vt_start(p.cu, b, p.N, p.vts);
        if (start + (n + 63) / 64 * 64 > np) return;   // malformed offsets only
        vt = p.vt + static_cast<long long>(h) * D * np + start;
        vspan = static_cast<long long>(D) * np - start;
    } else {
        np = (n + 63) / 64 * 64;
        vt = p.vt + static_cast<long long>(bh) * D * np;
        vspan = static_cast<long long>(D) * np;
    }

    // per-(b, h) scales: scores by scale * dq * dk (log2 units), output by dv
    const float cs = p.cs * p.dq[bh] * p.dk[bh];
    const float dv = p.dv[bh];

    // Q of this wave's rows, B operand: lane (c, hh) holds bytes
    // 64 ks + 32 hh .. +32 of row wrow0 + c
    i32x8 qf[KS];
    {
        const auto qrs = make_rsrc(p.q + base8 + static_cast<long long>(wrow0) * rs, (long long)(n - wrow0) * rs);
        const int vo = c * rs + hh * 32;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(qrs, vo + ks * 64, 0, 0);
            const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(qrs, vo + ks * 64 + 16, 0, 0);
            qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    }

    // direct loads: lane l of 1 KB load I fills row r = (1024 I + 16 l) / RB,
    // physical chunk pc, with logical chunk pc ^ swz(r); swz depends on I only
    // through I mod NW here, so one per-lane offset serves a wave's loads
    int kvo, vvo;
    {
        const int pos = wave * 1024 + lane * 16;
        const int kr = pos / KRB, kpc = (pos % KRB) / 16;
        kvo = kr * rs + ((kpc ^ fp8_swz<KRB>(kr)) << 4);
        const int vr = pos / VRB, vpc = (pos % VRB) / 16;
        vvo = vr * np + ((vpc ^ fp8_swz<VRB>(vr)) << 4);
    }
    // fragment reads: lane (c, hh) reads 32 bytes = chunks 2 kh', 2 kh' + 1
    // of a row (kh' = 4 ks + ... for K, hh for V^T)
    auto row32 = [&](const char *tile, int row, int chunk0, auto rb_) __attribute__((always_inline)) -> i32x8 {
        constexpr int RB = decltype(rb_)::value;
        const int s = fp8_swz<RB>(row);
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(tile + row * RB + ((chunk0 ^ s) << 4));
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(tile + row * RB + (((chunk0 + 1) ^ s) << 4));
        return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    using KRBc = std::integral_constant<int, KRB>;
    using VRBc = std::integral_constant<int, VRB>;

    const int kv_end = CAUSAL ? min(n, q0 + BR) : n;
    const int nkv = (kv_end + BC - 1) / BC;
    const int nkv_w = CAUSAL ? min(nkv, (wrow0 + 31) / BC + 1) : nkv;

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    // m_run: running row max (log2 units); the weights are 2^(s c - m + 8) =
    // 2^8 P, so l_run sums 2^8 P as well
    float m_run = -INFINITY, l_run = 0.0f, m_use8 = 0.0f, alpha = 1.0f;
    bool rescale_o = false;

    // S^T of one 64-key tile: lane (c, hh) register 4 g + r of s[kb] holds
    // key 32 kb + 8 g + 4 hh + r of query wrow0 + c
    auto s_mfma = [&](f32x16 (&s)[2], const char *ktile) __attribute__((always_inline)) {
        s[0] = f32x16{};
        s[1] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    row32(ktile, kb * 32 + c, 4 * ks + 2 * hh, KRBc{}), qf[ks], s[kb], 0, 0, 0, 0, 0, 0);
    };
    auto need_mask = [&](int j) { return (CAUSAL && j * BC + BC - 1 > wrow0) || j * BC + BC > n; };
    auto s_mask = [&](f32x16 (&s)[2], int j) __attribute__((always_inline)) {
        const int kv0 = j * BC;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = kv0 + kb * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
                const bool off = key >= n || (CAUSAL && key > wrow0 + c);
                s[kb][e] = off ? -INFINITY : s[kb][e];
            }
    };
    // running max update from the tile's raw row max (strict: the reference
    // is always the exact running max, so P <= 1)
    auto s_update = [&](const f32x16 (&s)[2]) __attribute__((always_inline)) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
        mx = xhalf_max(mx);
        const float mt = (mx == -INFINITY) ? -INFINITY : mx * cs;
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        rescale_o = __ballot(m_new > m_run) != 0;
        m_run = m_new;
        m_use8 = m_use - 8.0f;
        l_run *= alpha;
    };
    // O rescale of the strict rule: a wave-uniform branch at the top of a
    // step, before the P V MFMAs accumulate onto O
    auto o_rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
    };
    // 2^8 P in E4M3 and its sum, regrouped into operand order
    auto p_exp = [&](const f32x16 (&s)[2], i32x8 &pb) __attribute__((always_inline)) {
        int pk[2][4];
        float rsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float pv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][4 * g + r], cs, -m_use8));
                    rsum += pv[r];
                }
                pk[kb][g] = pack_fp8x4(pv[0], pv[1], pv[2], pv[3]);
            }
        l_run += rsum;
        // lower half takes block 0's keys, upper half block 1's, in key order
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const auto sw = __builtin_amdgcn_permlane32_swap(pk[0][g], pk[1][g], false, false);
            pb[2 * g] = sw[0];
            pb[2 * g + 1] = sw[1];
        }
    };
    // O^T += V^T P^T
    auto pv_mfma = [&](const char *vtile, const i32x8 &pb) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            oacc[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(row32(vtile, db * 32 + c, 2 * hh, VRBc{}), pb,
                                                                      oacc[db], 0, 0, 0, 0, 0, 0);
    };

    // Pipeline: LDS holds K(j+1) and V(j) while K(j+2) and V(j+1) stream in
    // (into the buffers of K(j) and V(j-1), both consumed before the previous
    // barrier).  A step j issues those loads, the S(j+1) MFMAs, the weights of
    // S(j) (VALU, independent of them, in the same basic block so that the two
    // interleave) and the P V(j) MFMAs, then the row max of S(j+1).  The
    // steady-state steps carry no branch: the mask, the last tile and the
    // tiles past a wave's causal horizon have steps of their own.
    f32x16 sa[2], sb[2];
    auto dma_k = [&](int j, char *kd) __attribute__((always_inline)) {
        const int kv0 = j * BC;
        // load i starts NW i (1024 / KRB) rows past the lane offset's row: its
        // resource is based there (the size check covers the lane offset only)
#pragma unroll
        for (int i = 0; i < KBLK / NW; ++i) {
            const int r0 = kv0 + NW * i * (1024 / KRB);
            const auto krs = make_rsrc(p.k + base8 + static_cast<long long>(r0) * rs, (long long)(n - r0) * rs);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, LDS_PTR(void, kd + (wave + NW * i) * 1024), 16, kvo, 0, 0,
                                                     0);
        }
    };
    auto dma_v = [&](int j, char *vd) __attribute__((always_inline)) {
        const int kv0 = j * BC;
        // V^T rows are np bytes apart, so a 64-key tile never crosses a row;
        // keys past n hold the zero padding.  The scalar offset (d rows) stays
        // inside the head's D x np bytes, which the resource spans.
        const auto vrs = make_rsrc(vt + kv0, vspan - kv0);
#pragma unroll
        for (int i = 0; i < VBLK / NW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, LDS_PTR(void, vd + (wave + NW * i) * 1024), 16, vvo,
                                                     NW * i * (1024 / VRB) * np, 0, 0);
    };
    dma_k(0, k_lds0);
    dma_v(0, v_lds0);
    if (nkv > 1) dma_k(1, k_lds1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nkv_w > 0) {
        s_mfma(sa, k_lds0);
        if (need_mask(0)) s_mask(sa, 0);
        s_update(sa);
    }
    __syncthreads();  // K(0)'s buffer takes K(2) next

    auto issue_loads = [&](int j, char *kbuf_j, char *vbuf_n) __attribute__((always_inline)) {
        if (j + 2 < nkv) dma_k(j + 2, kbuf_j);
        if (j + 1 < nkv) dma_v(j + 1, vbuf_n);
    };
    auto end_iteration = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    // a step whose tiles j and j + 1 this wave both computes; PAR = j & 1
    // selects the LDS buffers, MASK whether S(j+1) needs the tail or causal mask
    auto full_step = [&](auto par_, auto mask_, f32x16 (&cur)[2], f32x16 (&nxt)[2], int j)
                         __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_)::value;
        char *kbuf_j = PAR ? k_lds1 : k_lds0;       // held K(j), takes K(j+2)
        char *kbuf_n = PAR ? k_lds0 : k_lds1;       // holds K(j+1)
        char *vbuf_j = PAR ? v_lds1 : v_lds0;       // holds V(j)
        char *vbuf_n = PAR ? v_lds0 : v_lds1;       // held V(j-1), takes V(j+1)
        issue_loads(j, kbuf_j, vbuf_n);
        if (rescale_o) o_rescale();
        __builtin_amdgcn_sched_barrier(0);
        s_mfma(nxt, kbuf_n);
        i32x8 pb;
        p_exp(cur, pb);
        pv_mfma(vbuf_j, pb);
        if constexpr (decltype(mask_)::value) s_mask(nxt, j + 1);
        s_update(nxt);
        __builtin_amdgcn_sched_barrier(0);
        end_iteration();
    };
    // the wave's last tile: no next S
    auto drain_step = [&](auto par_, const f32x16 (&cur)[2], int j) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_)::value;
        issue_loads(j, PAR ? k_lds1 : k_lds0, PAR ? v_lds0 : v_lds1);
        if (rescale_o) o_rescale();
        i32x8 pb;
        p_exp(cur, pb);
        pv_mfma(PAR ? v_lds1 : v_lds0, pb);
        end_iteration();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;
    // first tile that needs a mask (tail: n / BC; causal: (wrow0 + 1) / BC)
    const int jm = CAUSAL ? min(n / BC, (wrow0 + 1) / BC) : n / BC;
    const int lim = min(nkv_w, jm);
    int j = 0;
    for (; j + 2 < lim; j += 2) {
        full_step(I0{}, NoMask{}, sa, sb, j);
        full_step(I1{}, NoMask{}, sb, sa, j + 1);
    }
    for (; j + 2 < nkv_w; j += 2) {
        full_step(I0{}, Mask{}, sa, sb, j);
        full_step(I1{}, Mask{}, sb, sa, j + 1);
    }
    if (j + 1 < nkv_w) {
        full_step(I0{}, Mask{}, sa, sb, j);
        ++j;
    }
    if (j < nkv_w) {
        if (j & 1) drain_step(I1{}, sb, j);
        else drain_step(I0{}, sa, j);
        ++j;
    }
    // tiles past this wave's causal horizon: keep loading for the other waves
    for (; j < nkv; ++j) {
        if (j & 1) issue_loads(j, k_lds1, v_lds0);
        else issue_loads(j, k_lds0, v_lds1);
        end_iteration();
    }

    // epilogue: O = O^T dv / l (l sums 2^8 P like O), LSE = (m + log2 l - 8) ln 2
    const float l = xhalf_sum(l_run);
    const float inv = l > 0.0f ? dv / l : 0.0f;
    const long long obase = (w.t0 * p.H + h) * D;
    const auto ors = make_rsrc(p.o + obase + static_cast<long long>(wrow0) * p.H * D,
                               (long long)(n - wrow0) * p.H * D * 2);
    const int voff_o = c * p.H * D * 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int col = db * 32 + g4 * 8 + hh * 4;
            const u32x2 v2 = {pack_bf16x2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv),
                              pack_bf16x2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv)};
            __builtin_amdgcn_raw_buffer_store_b64(v2, ors, voff_o + col * 2, 0, 0);
        }
    const int qrow = wrow0 + c;
    // LSE row of the sequence's first token: dense [B, H, N], packed [H, T]
    const long long lrow0 = PACKED ? static_cast<long long>(h) * p.N + w.t0 : static_cast<long long>(bh) * n;
    if (qrow < n && hh == 0)
        p.lse[lrow0 + qrow] = l > 0.0f ? (m_run + log2f(l) - 8.0f) * kLn2 : -INFINITY;
}

// ---------------------------------------------------------------------------
// Quantisation: descale[bh] = amax / 448 (1 for an all-zero head), codes =
// E4M3(x * (1 / descale)), every step in fp32 with IEEE rounding.
//
// Four launches on the stream.  Until the last one the descale array holds
// each (sequence, head)'s running amax as a bit pattern: |x| >= 0, so the
// integer order of the bits is the float order and an atomic maximum over
// the workgroups of a head is exact whatever their order.  The array is
// zeroed; each workgroup reduces one slice of the tokens of one (sequence,
// head) and merges its maximum; the codes are written from the finished
// amax; the amax is turned into the descale.  The amax and packed code
// kernels run (sequence, head) x slices workgroups, slices = grid / (B H).

__device__ __forceinline__ float fp8_descale_of(float amax) { return amax > 0.0f ? amax / 448.0f : 1.0f; }

// tokens of sequence b: the first one on the token axis and the count
__device__ __forceinline__ void fp8_quant_seq(const QuantParams &p, int b, long long &t0, int &n) {
    if (p.cu) {
        int a, e;
        seq_span(p.cu, b, p.N, a, e);
        t0 = a;
        n = e - a;
    } else {
        t0 = static_cast<long long>(b) * p.N;
        n = p.N;
    }
}

// slice s of n tokens cut into `slices` near-equal parts: [lo, hi)
__device__ __forceinline__ void fp8_quant_slice(int n, int s, int slices, int &lo, int &hi) {
    const long long per = (static_cast<long long>(n) + slices - 1) / slices;
    lo = static_cast<int>(min(static_cast<long long>(n), s * per));
    hi = static_cast<int>(min(static_cast<long long>(n), lo + per));
}

__global__ void __launch_bounds__(256) fa_fp8_amax_init_kernel(QuantParams p) {
    const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
    if (i < static_cast<long long>(p.B) * p.H) p.descale[i] = 0.0f;
}

__global__ void __launch_bounds__(256) fa_fp8_amax_kernel(QuantParams p) {
    const int slices = static_cast<int>(gridDim.x / (static_cast<unsigned>(p.B) * p.H));
    const int bh = blockIdx.x / slices, s = blockIdx.x - bh * slices;
    const int b = bh / p.H, h = bh - b * p.H;
    long long t0;
    int n, lo, hi;
    fp8_quant_seq(p, b, t0, n);
    fp8_quant_slice(n, s, slices, lo, hi);
    // each thread keeps one 16-byte column chunk and steps over the rows
    const int chunks = p.d / 8;
    const int step = 256 / chunks;
    const long long rs = static_cast<long long>(p.H) * p.d;
    const uint16_t *xs = p.x + ((t0 + lo) * p.H + h) * p.d + (threadIdx.x % chunks) * 8;
    float m = 0.0f;
#pragma unroll 4
    for (int i = threadIdx.x / chunks; i < hi - lo; i += step) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(xs + i * rs);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            m = fmaxf(m, fabsf(__uint_as_float(w[k] << 16)));
            m = fmaxf(m, fabsf(__uint_as_float(w[k] & 0xffff0000u)));
        }
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    __shared__ float red[4];
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        if (m > 0.0f) atomicMax(reinterpret_cast<unsigned int *>(p.descale) + bh, __float_as_uint(m));
    }
}

__global__ void __launch_bounds__(256) fa_fp8_descale_kernel(QuantParams p) {
    const long long i = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
    if (i < static_cast<long long>(p.B) * p.H) p.descale[i] = fp8_descale_of(p.descale[i]);
}

// 8 codes of 8 consecutive bf16 values (one 16-byte read; two 4-byte writes,
// the codes being only 4-byte aligned)
__device__ __forceinline__ void fp8_quant8(const uint16_t *src, uint8_t *dst, float inv) {
    const u32x4 w = *reinterpret_cast<const u32x4 *>(src);
    uint32_t out[2];
    out[0] = static_cast<uint32_t>(
        pack_fp8x4(__uint_as_float(w[0] << 16) * inv, __uint_as_float(w[0] & 0xffff0000u) * inv,
                   __uint_as_float(w[1] << 16) * inv, __uint_as_float(w[1] & 0xffff0000u) * inv));
    out[1] = static_cast<uint32_t>(
        pack_fp8x4(__uint_as_float(w[2] << 16) * inv, __uint_as_float(w[2] & 0xffff0000u) * inv,
                   __uint_as_float(w[3] << 16) * inv, __uint_as_float(w[3] & 0xffff0000u) * inv));
    reinterpret_cast<uint32_t *>(dst)[0] = out[0];
    reinterpret_cast<uint32_t *>(dst)[1] = out[1];
}

// codes in x's layout, one thread per (token, head, 8 columns)
__global__ void __launch_bounds__(256) fa_fp8_quant_kernel(QuantParams p) {
    const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
    const int g8 = p.d / 8;
    // t = ((b * N + i) * H + h) * g8 + q: lanes run along columns
    const int q = static_cast<int>(t % g8);
    const long long r = t / g8;
    const int h = static_cast<int>(r % p.H);
    const long long bh = (r / p.H / p.N) * p.H + h;
    if (bh >= static_cast<long long>(p.B) * p.H) return;
    fp8_quant8(p.x + r * p.d + q * 8, p.x8 + r * p.d + q * 8, 1.0f / fp8_descale_of(p.descale[bh]));
}

// Transposed codes of one 64-key tile of one (sequence, head), through LDS.
// A thread takes four consecutive keys of 8 columns (16-byte reads, the
// lanes of a column group reading whole rows), packs each column's four
// codes into one dword of `tile` (column-major, rows padded to kTRow bytes so
// that the column groups of a wave fall in different banks), and each of the
// d V^T rows then receives one 64-byte run.  xs: the tile's first token,
// head h; keys: its tokens present (the rest of the 64 are zero padding
// codes); dst: V^T row 0 at the tile's first key; stride: V^T row length.
constexpr int kTRow = 68;

__device__ __forceinline__ void fp8_quant_t_tile(const QuantParams &p, float inv, const uint16_t *xs, int keys,
                                                 uint8_t *dst, long long stride, uint8_t *tile) {
    const int g8 = p.d / 8;
    const long long rs = static_cast<long long>(p.H) * p.d;
    for (int c = threadIdx.x; c < 16 * g8; c += 256) {
        const int q = c % g8, rg = c / g8;
        uint32_t col[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
            const int r = 4 * rg + k4;
            if (r < keys) {
                const u32x4 w = *reinterpret_cast<const u32x4 *>(xs + r * rs + q * 8);
                const uint32_t lo = static_cast<uint32_t>(
                    pack_fp8x4(__uint_as_float(w[0] << 16) * inv, __uint_as_float(w[0] & 0xffff0000u) * inv,
                               __uint_as_float(w[1] << 16) * inv, __uint_as_float(w[1] & 0xffff0000u) * inv));
                const uint32_t hi = static_cast<uint32_t>(
                    pack_fp8x4(__uint_as_float(w[2] << 16) * inv, __uint_as_float(w[2] & 0xffff0000u) * inv,
                               __uint_as_float(w[3] << 16) * inv, __uint_as_float(w[3] & 0xffff0000u) * inv));
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    col[k] |= ((lo >> (8 * k)) & 0xffu) << (8 * k4);
                    col[4 + k] |= ((hi >> (8 * k)) & 0xffu) << (8 * k4);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) *reinterpret_cast<uint32_t *>(tile + (q * 8 + j) * kTRow + 4 * rg) = col[j];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < p.d * 16; c += 256) {
        const int cl = c >> 4, part = c & 15;
        *reinterpret_cast<uint32_t *>(dst + cl * stride + part * 4) =
            *reinterpret_cast<const uint32_t *>(tile + cl * kTRow + part * 4);
    }
    __syncthreads();  // before the next tile overwrites `tile`
}

// transposed codes [B, H, d, np], np = ceil(N / 64) * 64: one workgroup per
// 64-key tile of one (b, h)
__global__ void __launch_bounds__(256) fa_fp8_quant_t_kernel(QuantParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[256 * kTRow];
    const int np = (p.N + 63) / 64 * 64;
    const int tiles = np / 64;
    const long long bh = blockIdx.x / tiles;
    const int t = static_cast<int>(blockIdx.x - bh * tiles);
    const int b = static_cast<int>(bh / p.H), h = static_cast<int>(bh % p.H);
    const float inv = 1.0f / fp8_descale_of(p.descale[bh]);
    const int k0 = t * 64;
    fp8_quant_t_tile(p, inv, p.x + ((static_cast<long long>(b) * p.N + k0) * p.H + h) * p.d, min(64, p.N - k0),
                     p.x8 + bh * p.d * np + k0, np, tile);
}

// Packed sequences: the codes of one token slice of one (sequence, head):
// [T, H, d] in place of x, or the slice's 64-key tiles of the packed V^T
// rows (the sequence's last tile carries the zero codes up to the next
// multiple of 64 keys; columns past the last sequence's padding are not
// written).
__global__ void __launch_bounds__(256) fa_fp8_quant_packed_kernel(QuantParams p) {
    __shared__ __attribute__((aligned(16))) uint8_t tile[256 * kTRow];
    const int slices = static_cast<int>(gridDim.x / (static_cast<unsigned>(p.B) * p.H));
    const int bh = blockIdx.x / slices, s = blockIdx.x - bh * slices;
    const int b = bh / p.H, h = bh - b * p.H;
    long long t0;
    int n;
    fp8_quant_seq(p, b, t0, n);
    const float inv = 1.0f / fp8_descale_of(p.descale[bh]);
    if (!p.transpose) {
        int lo, hi;
        fp8_quant_slice(n, s, slices, lo, hi);
        const int g8 = p.d / 8;
        const long long off = ((t0 + lo) * p.H + h) * p.d + (threadIdx.x % g8) * 8;
        const long long rs = static_cast<long long>(p.H) * p.d;
        for (int i = threadIdx.x / g8; i < hi - lo; i += 256 / g8)
            fp8_quant8(p.x + off + i * rs, p.x8 + off + i * rs, inv);
        return;
    }
    // transposed: the slice's share of the sequence's 64-key tiles
    const int pad = (n + 63) / 64 * 64;
    const int start = fp8_packed_vt_start(p.cu, b, p.N, p.vts);
    if (start + pad > p.vts) return;   // malformed offsets only
    int lo, hi;
    fp8_quant_slice(pad / 64, s, slices, lo, hi);
    for (int t = lo; t < hi; ++t)
        fp8_quant_t_tile(p, inv, p.x + ((t0 + t * 64) * p.H + h) * p.d, min(64, n - t * 64),
                         p.x8 + static_cast<long long>(h) * p.d * p.vts + start + t * 64, p.vts, tile);
}

template <int D>
KernelFp8Fn select_fp8(bool causal, bool packed) {
    if (packed) return causal ? fa_fp8_fwd_kernel<D, true, true> : fa_fp8_fwd_kernel<D, false, true>;
    return causal ? fa_fp8_fwd_kernel<D, true, false> : fa_fp8_fwd_kernel<D, false, false>;
}

}  // namespace fa_detail
