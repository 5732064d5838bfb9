// Fused exact-attention forward for AMD Instinct MI355X (gfx950 / CDNA4).
//
// O = softmax(Q K^T * scale) V with the online softmax of the FlashAttention-1
// derivation ("FlashAttention 1-4 explained", online softmax equation block):
// per query row the kernel carries the running max m, the running sum l and
// the unnormalised output, and divides by l once at the end (FlashAttention-2
// deferred normalisation).  S and P live only in registers.
//
// Mapping onto CDNA4:
//  * Each wave owns 32 query rows.  Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: K (from LDS) is the A
//    operand and Q (held in VGPRs for the whole kernel) the B operand.  In the
//    32x32 accumulator layout lane l holds column l%32, i.e. one query row, so
//    the row max and row sum are in-lane reductions plus one exchange between
//    lanes l and l+32 (v_permlane32_swap).
//  * The P tile is converted to bf16 in place and is directly the B operand
//    of O^T += V^T P^T: its register order fixes a permutation of the 16 keys
//    of each MFMA, and V is read from LDS in that order with the transposing
//    ds_read_b64_tr_b16, so P never leaves the VGPRs.  The O^T accumulator
//    again gives each lane one query row, so the rescale by exp(m_old - m_new)
//    is a per-lane scalar multiply.
//  * K and V tiles are staged global -> VGPR -> LDS, double-buffered: the
//    global loads of tile j+1 are in flight while tile j is computed.  The
//    LDS rows are padded so that both the K reads (8 lanes, 8 rows, one
//    16-byte chunk) and the transposing V reads (16 lanes, 4 rows, 32 bytes)
//    touch distinct banks.
//  * exp is evaluated as exp2 of (s * scale * log2 e - m) with the hardware
//    v_exp_f32, or with a degree-3 polynomial on the FMA units (section 3.2
//    of the FlashAttention V4 explainer), or half and half.
//  * Conditional rescale (FlashAttention-4 section of the 1-4 post): a wave
//    skips the O multiply when no row max grew, or, in threshold mode, keeps
//    its reference max until a row max exceeds it by more than 8.
//  * Causal tiles that are fully masked are never visited (FlashAttention-2
//    engineering notes); the tile order puts the longest tiles first and keeps
//    the work items of one (sequence, head) on one XCD so that its K/V stream
//    is shared through that XCD's L2.
//
// Every function of the library's C ABI is declared in include/fa.h.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "fa.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
// Threshold rescale: P~ = 2^(s*c - m) may reach 2^kTau before m moves.
constexpr float kTau = 8.0f;

struct Params {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    const int32_t *cu;  // packed offsets, or nullptr
    int B, H, N;        // N: sequence length (dense) or total tokens (packed)
    int n_qt;           // dense: query tiles per sequence
    float cs;           // scale * log2(e)
};

// ---------------------------------------------------------------------------
// exp2 evaluations

// 2^x with x = n + f, n = floor(x), f in [0, 1): p(f) = 1 + f(c1 + f(c2 + f c3))
// is a minimax fit of 2^f with p(0) = 1 exactly (coefficients derived by
// gen_exp2_poly.py, max relative error 8.6e-5), and 2^n is added to the
// exponent field.  x is clamped to -127 first: there n = -127, p = 1 and the
// sum of the fields is exactly +0, so masked (-inf) scores give 0 and the
// exponent add never wraps.
__device__ __forceinline__ float exp2_poly(float x) {
    x = fmaxf(x, -127.0f);
    const float n = __builtin_floorf(x);
    const float f = x - n;
    float p = __builtin_fmaf(f, 7.706703991e-02f, 2.276449949e-01f);
    p = __builtin_fmaf(f, p, 6.951167583e-01f);
    p = __builtin_fmaf(f, p, 1.0f);
    const int bits = __float_as_int(p) + (static_cast<int>(n) << 23);
    return __int_as_float(bits);
}

template <int EXPM>
__device__ __forceinline__ float exp2_sel(float x, int idx) {
    if constexpr (EXPM == FA_EXP_HW) {
        return __builtin_amdgcn_exp2f(x);
    } else if constexpr (EXPM == FA_EXP_POLY) {
        return exp2_poly(x);
    } else {
        return (idx & 1) ? exp2_poly(x) : __builtin_amdgcn_exp2f(x);
    }
}

// ---------------------------------------------------------------------------
// LDS tile layout: [rows][D] bf16 with padded rows.  K rows are padded by
// 16 bytes, so the 8 lanes of one 16-byte K read (8 consecutive rows, same
// column) start 4 banks apart; V rows by 32 bytes, so the 4 rows x 32 bytes
// read by each 16-lane group of the transposing V read start 8 banks apart.
// Both reads are then free of bank conflicts on 32 banks x 4 bytes, and every
// address is a per-lane base plus a compile-time offset.

template <int D> struct Lds {
    static constexpr int KSTR = D * 2 + 16;  // bytes per K row
    static constexpr int VSTR = D * 2 + 32;  // bytes per V row
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

// Max of x over lanes l and l ^ 32.
__device__ __forceinline__ float xhalf_max(float x) {
    const uint32_t u = __float_as_uint(x);
    auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float xhalf_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// ---------------------------------------------------------------------------
// Work decode: one workgroup = (sequence b, head h, query tile qt).

struct Work {
    int b, h, qt, n;  // n: length of sequence b
    long long t0;     // first token of sequence b
};

template <bool CAUSAL, bool VARLEN, int BR>
__device__ __forceinline__ bool decode_work(const Params &p, Work &w) {
    const int wg = blockIdx.x;
    if constexpr (!VARLEN) {
        const int BH = p.B * p.H;
        int bh, qt;
        if constexpr (CAUSAL) {
            // longest tiles (highest query tile) first; wg % 8 picks the XCD,
            // so with BH % 8 == 0 all tiles of one head stay on one XCD
            qt = p.n_qt - 1 - wg / BH;
            bh = wg % BH;
        } else {
            // equal work: give each XCD a contiguous run of items so the
            // workgroups resident on one XCD stream the same head's K/V
            const int G = gridDim.x, x = wg & 7, s = wg >> 3;
            const int per = G >> 3, rem = G & 7;
            const int item = x * per + (x < rem ? x : rem) + s;
            bh = item / p.n_qt;
            qt = item - bh * p.n_qt;
        }
        w.b = bh / p.H;
        w.h = bh - w.b * p.H;
        w.qt = qt;
        w.n = p.N;
        w.t0 = static_cast<long long>(w.b) * p.N;
        return true;
    } else {
        // Items are (sequence, query tile) pairs ordered by query-tile index,
        // highest first (for causal masks the work of a tile grows with its
        // index); ties in sequence order.  Each wave decodes independently
        // with ballots over up to 64 sequences at a time.
        const int lane = threadIdx.x & 63;
        w.h = wg % p.H;
        int r = wg / p.H;
        int lmax = 0;
        for (int base = 0; base < p.B; base += 64) {
            const int b = base + lane;
            int nt = 0;
            if (b < p.B) nt = (p.cu[b + 1] - p.cu[b] + BR - 1) / BR;
            for (int off = 32; off > 0; off >>= 1) nt = max(nt, __shfl_xor(nt, off));
            lmax = max(lmax, nt);
        }
        for (int L = lmax - 1; L >= 0; --L) {
            int cnt = 0;
            for (int base = 0; base < p.B; base += 64) {
                const int b = base + lane;
                bool on = false;
                if (b < p.B) on = (p.cu[b + 1] - p.cu[b] + BR - 1) / BR > L;
                cnt += __popcll(__ballot(on));
            }
            if (r < cnt) {
                for (int base = 0; base < p.B; base += 64) {
                    const int b = base + lane;
                    bool on = false;
                    if (b < p.B) on = (p.cu[b + 1] - p.cu[b] + BR - 1) / BR > L;
                    unsigned long long m = __ballot(on);
                    const int c = __popcll(m);
                    if (r < c) {
                        // position of the r-th set bit of m
                        for (int i = 0; i < r; ++i) m &= m - 1;
                        const int bsel = base + __ffsll(static_cast<long long>(m)) - 1;
                        w.b = bsel;
                        w.qt = L;
                        w.t0 = p.cu[bsel];
                        w.n = p.cu[bsel + 1] - p.cu[bsel];
                        return true;
                    }
                    r -= c;
                }
            }
            r -= cnt;
        }
        return false;  // surplus workgroup of the grid bound
    }
}

// ---------------------------------------------------------------------------
// The kernel.  NW waves x 32 rows = BR query rows per workgroup; BC keys per
// K/V tile.

template <int D, int BC, int NW, bool CAUSAL, bool VARLEN, int EXPM, int RSM>
__global__ void __launch_bounds__(NW * 64)
fa_fwd_kernel(Params p) {
    constexpr int NT = NW * 64;
    constexpr int BR = NW * 32;
    constexpr int KK = D / 16;           // MFMA k-steps of Q K^T
    constexpr int NKB = BC / 32;         // 32-key blocks per tile
    constexpr int NDB = D / 32;          // 32-wide d blocks of O^T
    constexpr int NT16 = BC / 16;        // 16-key chunks (PV k-steps)
    constexpr int KSTR = Lds<D>::KSTR, VSTR = Lds<D>::VSTR;
    constexpr int KBYTES = BC * KSTR, VBYTES = BC * VSTR;
    constexpr int STAGE = KBYTES + VBYTES;  // one K tile + one V tile
    constexpr int CHUNKS = BC * D / 8;   // 16-byte chunks per K (or V) tile
    constexpr int PER = CHUNKS / NT;     // chunks per thread per tile
    static_assert(CHUNKS % NT == 0, "tile must split evenly over threads");

    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    Work w;
    if (!decode_work<CAUSAL, VARLEN, BR>(p, w)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int c = lane & 31, hh = lane >> 5;
    const int n = w.n;
    const int q0 = w.qt * BR;
    const long long rs = static_cast<long long>(p.H) * D;  // token stride (elements)
    const long long base = (w.t0 * p.H + w.h) * D;
    const uint16_t *qg = p.q + base;
    const uint16_t *kg = p.k + base;
    const uint16_t *vg = p.v + base;

    const int wrow0 = q0 + wave * 32;  // first row of this wave
    const int qrow = wrow0 + c;        // this lane's row

    // Q fragments: B operand of S^T = K Q^T, lane (c, hh) holds
    // Q[qrow][kk*16 + hh*8 .. +8].
    bf16x8 qf[KK];
    if (qrow < n) {
        const uint16_t *src = qg + qrow * rs + hh * 8;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qf[kk] = *reinterpret_cast<const bf16x8 *>(src + kk * 16);
    } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) qf[kk] = bf16x8{};
    }

    const int kv_end = CAUSAL ? min(n, q0 + BR) : n;
    const int nkv = (kv_end + BC - 1) / BC;

    u32x4 kreg[PER], vreg[PER];
    auto gload = [&](int j) {
        const int kv0 = j * BC;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int qc = tid + i * NT;
            const int row = qc / (D / 8), ch = qc % (D / 8);
            if (kv0 + row < n) {
                const long long off = (kv0 + row) * rs + ch * 8;
                kreg[i] = *reinterpret_cast<const u32x4 *>(kg + off);
                vreg[i] = *reinterpret_cast<const u32x4 *>(vg + off);
            } else {
                kreg[i] = u32x4{};
                vreg[i] = u32x4{};
            }
        }
    };
    auto lstore = [&](int s) {
        char *kb = smem + s * STAGE;
        char *vb = kb + KBYTES;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int qc = tid + i * NT;
            const int row = qc / (D / 8), ch = qc % (D / 8);
            *reinterpret_cast<u32x4 *>(kb + row * KSTR + ch * 16) = kreg[i];
            *reinterpret_cast<u32x4 *>(vb + row * VSTR + ch * 16) = vreg[i];
        }
    };

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    float m_run = -INFINITY;  // reference max, scaled log2 units
    float l_run = 0.0f;       // this lane's partial row sum

    const float cs = p.cs;

    if (nkv > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();

    for (int j = 0; j < nkv; ++j) {
        if (j + 1 < nkv) gload(j + 1);
        const char *kb = smem + (j & 1) * STAGE;
        const char *vb = kb + KBYTES;
        const int kv0 = j * BC;
        const bool active = !CAUSAL || kv0 <= wrow0 + 31;
        if (active) {
            // ---- S^T = K Q^T ------------------------------------------------
            f32x16 sacc[NKB];
#pragma unroll
            for (int i = 0; i < NKB; ++i) sacc[i] = f32x16{};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
                for (int kb2 = 0; kb2 < NKB; ++kb2) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        kb + (kb2 * 32 + c) * KSTR + (kk * 16 + hh * 8) * 2);
                    sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kk], sacc[kb2], 0, 0, 0);
                }
            }
            // ---- mask: tail keys, and keys after the query when causal -------
            const bool need_mask = (CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > n);
            if (need_mask) {
#pragma unroll
                for (int kb2 = 0; kb2 < NKB; ++kb2) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kv0 + kb2 * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
                        const bool off = key >= n || (CAUSAL && key > qrow);
                        sacc[kb2][r] = off ? -INFINITY : sacc[kb2][r];
                    }
                }
            }
            // ---- row max (raw scores), then in scaled log2 units --------------
            float mx = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb2][r]);
            mx = xhalf_max(mx);
            const float mt = (mx == -INFINITY) ? -INFINITY : mx * cs;

            float m_new;
            bool grow;
            if constexpr (RSM == FA_RESCALE_THRESHOLD) {
                grow = mt > m_run + kTau;  // also true for the first finite tile
                m_new = grow ? mt : m_run;
            } else {
                m_new = fmaxf(m_run, mt);
                grow = m_new > m_run;
            }
            const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);  // 0 when m_run = -inf
            bool rescale_o;
            if constexpr (RSM == FA_RESCALE_ALWAYS) {
                rescale_o = true;
            } else {
                rescale_o = __ballot(grow) != 0;
            }
            // rows that did not grow have alpha == 1 exactly
            l_run *= alpha;
            m_run = m_new;
            if (rescale_o) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
            }

            // ---- P~ = 2^(s*cs - m), row sum, bf16 B operand ------------------
            bf16x8 pf[NT16];
            float rsum = 0.0f;
#pragma unroll
            for (int t = 0; t < NT16; ++t) {
                const int kb2 = t >> 1, r0 = (t & 1) * 8;
                uint32_t pk[4];
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const float e0 = exp2_sel<EXPM>(__builtin_fmaf(sacc[kb2][r0 + i], cs, -m_use), i);
                    const float e1 = exp2_sel<EXPM>(__builtin_fmaf(sacc[kb2][r0 + i + 1], cs, -m_use), i + 1);
                    rsum += e0 + e1;
                    pk[i >> 1] = pack_bf16x2(e0, e1);
                }
                u32x4 pv = {pk[0], pk[1], pk[2], pk[3]};
                pf[t] = __builtin_bit_cast(bf16x8, pv);
            }
            l_run += rsum;

            // ---- O^T += V^T P^T ----------------------------------------------
            // The k-slot order of pf[t] for lane half hh is keys
            // t*16 + hh*4 + {0..3}, then t*16 + 8 + hh*4 + {0..3}; each half is
            // one transposing read of 4 V rows x 16 columns per 16-lane group.
            const int g = lane >> 4, s16 = lane & 15;
#pragma unroll
            for (int t = 0; t < NT16; ++t) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int col = db * 32 + (g & 1) * 16 + (s16 & 3) * 4;
                    const int row0 = t * 16 + hh * 4 + (s16 >> 2);
                    const char *src = vb + row0 * VSTR + col * 2;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, src));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, src + 8 * VSTR));
                    const i16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    const bf16x8 a = __builtin_bit_cast(bf16x8, both);
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[t], oacc[db], 0, 0, 0);
                }
            }
        }
        if (j + 1 < nkv) lstore((j + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: O / l, LSE = (m + log2 l) ln 2 ----------------------------
    const float l = xhalf_sum(l_run);
    if (qrow < n) {
        const float inv = l > 0.0f ? 1.0f / l : 0.0f;
        uint16_t *og = p.o + base + qrow * rs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int col = db * 32 + g4 * 8 + hh * 4;
                u32x2 v2 = {pack_bf16x2(oacc[db][g4 * 4 + 0] * inv, oacc[db][g4 * 4 + 1] * inv),
                            pack_bf16x2(oacc[db][g4 * 4 + 2] * inv, oacc[db][g4 * 4 + 3] * inv)};
                *reinterpret_cast<u32x2 *>(og + col) = v2;
            }
        }
        if (hh == 0) {
            const float lse = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
            long long li;
            if constexpr (VARLEN) {
                li = static_cast<long long>(w.h) * p.N + w.t0 + qrow;
            } else {
                li = (static_cast<long long>(w.b) * p.H + w.h) * p.N + qrow;
            }
            p.lse[li] = lse;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side

constexpr int kWaves = 4;
constexpr int kRows = kWaves * 32;

template <int D>
constexpr int keys_per_tile() { return 64; }

using KernelFn = void (*)(Params);

template <int D, bool CAUSAL, bool VARLEN, int EXPM, int RSM>
KernelFn pick5() { return fa_fwd_kernel<D, keys_per_tile<D>(), kWaves, CAUSAL, VARLEN, EXPM, RSM>; }

template <int D, bool CAUSAL, bool VARLEN, int EXPM>
KernelFn pick4(int rsm) {
    switch (rsm) {
        case FA_RESCALE_ALWAYS: return pick5<D, CAUSAL, VARLEN, EXPM, FA_RESCALE_ALWAYS>();
        case FA_RESCALE_STRICT: return pick5<D, CAUSAL, VARLEN, EXPM, FA_RESCALE_STRICT>();
        default: return pick5<D, CAUSAL, VARLEN, EXPM, FA_RESCALE_THRESHOLD>();
    }
}

template <int D, bool CAUSAL, bool VARLEN>
KernelFn pick3(int expm, int rsm) {
    switch (expm) {
        case FA_EXP_HW: return pick4<D, CAUSAL, VARLEN, FA_EXP_HW>(rsm);
        case FA_EXP_POLY: return pick4<D, CAUSAL, VARLEN, FA_EXP_POLY>(rsm);
        default: return pick4<D, CAUSAL, VARLEN, FA_EXP_MIXED>(rsm);
    }
}

template <int D>
KernelFn pick2(bool causal, bool varlen, int expm, int rsm) {
    if (causal) return varlen ? pick3<D, true, true>(expm, rsm) : pick3<D, true, false>(expm, rsm);
    return varlen ? pick3<D, false, true>(expm, rsm) : pick3<D, false, false>(expm, rsm);
}

KernelFn pick(int d, bool causal, bool varlen, int expm, int rsm) {
    switch (d) {
        case 64: return pick2<64>(causal, varlen, expm, rsm);
        case 128: return pick2<128>(causal, varlen, expm, rsm);
        default: return pick2<256>(causal, varlen, expm, rsm);
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

int fa_tile_rows(int d) { return (d == 64 || d == 128 || d == 256) ? kRows : 0; }

int fa_tile_keys(int d) {
    switch (d) {
        case 64: return keys_per_tile<64>();
        case 128: return keys_per_tile<128>();
        case 256: return keys_per_tile<256>();
        default: return 0;
    }
}

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
    const long long n_qt = (static_cast<long long>(N) + kRows - 1) / kRows;
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
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(grid)), dim3(kWaves * 64), 0, stream, prm);
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    return FA_OK;
}

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N,
           int d, float scale, int causal, const int32_t *cu_seqlens, hipStream_t stream) {
    return fa_fwd_variant(q, k, v, o, lse, B, H, N, d, scale, causal, cu_seqlens, stream,
                          FA_EXP_HW, FA_RESCALE_STRICT);
}

}  // extern "C"
