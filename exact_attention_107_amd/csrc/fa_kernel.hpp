// Device code of the fused exact-attention forward for gfx950, included by one
// translation unit per head dimension (fa_kernels_d*.hip).
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
//  * K and V tiles go from global memory straight into LDS (buffer loads with
//    the LDS destination), two K and two V tiles: K_{j+2} and V_{j+1} stream
//    in while tile j is computed.  The 16-byte chunks of each LDS row are
//    XOR-permuted so that the K reads (16 consecutive rows, one chunk) and
//    the transposing V reads (4 rows x 4 chunks) touch distinct banks.
//  * exp is evaluated as exp2 of (s * scale * log2 e - m) with the hardware
//    v_exp_f32, or with a degree-3 polynomial on the FMA units (section 3.2
//    of the FlashAttention V4 explainer), or half and half.
//  * Conditional rescale (FlashAttention-4 section of the 1-4 post): a wave
//    skips the O multiply when no row max grew (strict, the default), or, in
//    threshold mode, keeps its reference max until a row max exceeds it by
//    more than 8 and then divides O by the sum of the bf16 weights it used.
//  * Causal tiles that are fully masked are never visited (FlashAttention-2
//    engineering notes); causal work is ordered longest first, non-causal
//    work gives each XCD a contiguous run of items (the query tiles of one
//    head, whose K/V stream its L2 then serves), and packed sequences go
//    longest first with the heads of one query tile together.
//
// Every function of the library's C ABI is declared in include/fa.h.

#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa.h"
#include "fa_internal.h"

namespace fa_detail {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
// Threshold rescale: P~ = 2^(s*c - m) may reach 2^kTau before m moves.
constexpr float kTau = 8.0f;
// LDS fragment reads in flight ahead of the MFMA that uses them (K in the
// score phase, V in the P V phase)
constexpr int kKLookahead = 2;
constexpr int kVLookahead = 2;


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
// LDS tile layouts (the LDS has 64 banks of 4 bytes = 16 groups of 16 bytes).
// Tiles are filled by direct global->LDS loads, each writing 64 lanes x 16
// bytes contiguously; where a lane's 16 bytes land is fixed, so layouts are
// chosen by which global chunk each lane fetches.
//  * K, in planes of 8 chunks: chunks 8p..8p+7 of the 64 rows form plane p
//    (64 rows x 128 bytes), and within a row the chunks are XOR-permuted by
//    g(r) = (r >> 1) & 7.  A K fragment read (16 lanes per cycle, 16
//    consecutive rows, one chunk) then covers all 16 bank groups: row parity
//    picks the half of the 64 banks, g(r) the group within it.  Each direct
//    load covers 8 whole rows of a plane (8 x 128 contiguous global bytes).
//  * V, row-major with the 16-byte chunks of row r XOR-permuted by f_V(r).
//    The transposing 8-byte V read serves 32 lanes per cycle covering 4
//    consecutive rows x 4 consecutive chunks; f_V gives the 4 rows disjoint
//    sets of 4 bank groups.

template <int D> struct Swz {
    static constexpr int RB = D * 2;  // bytes per row
    static __device__ __forceinline__ int gk(int r) { return (r >> 1) & 7; }
    static __device__ __forceinline__ int fv(int r) {
        if constexpr (D == 64) return ((r >> 1) & 1) << 2;  // 8 chunks/row: rows pair up in 16 groups
        else return (r & 3) << 2;
    }
};

// Raw buffer resource over `bytes` bytes at `base` (gfx9 word 3); loads past
// the end return zeros (also into LDS) and stores past the end are dropped.
// The hardware checks only the per-lane offset (plus the immediate) against
// the size, never the scalar offset: a row offset must therefore go into the
// base and size of the resource (rows_rsrc), and the scalar offset may only
// hold a column offset that stays inside a row the lane offset has
// already bounded.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, long long bytes) {
    const long long lim = bytes < 0 ? 0 : (bytes > 0xffffffffLL ? 0xffffffffLL : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                             static_cast<int>(static_cast<uint32_t>(lim)),
                                             0x00020000);
}

// Resource over rows row0 .. min(n, row0 + 64) - 1 of a bf16 tensor whose
// rows are row_elems elements apart (`base` points at row 0): rows at or
// past n read as zeros.  No access through it reaches 64 rows past row0, and
// row_elems * 2 <= 2^23 (the library's token-stride limit), so the size is
// computed in 32-bit scalar arithmetic (a 64-bit clamp compiles to vector
// compares feeding scalar selects, a slow chain in front of every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t *base, long long row_elems,
                                                            int row0, int n) {
    int rows = n - row0;
    rows = rows < 0 ? 0 : (rows > 64 ? 64 : rows);
    // the operands are wave-uniform; say so, or the clamp may land in a
    // vector register and every load through the resource becomes a loop
    // over the lanes' distinct values
    rows = __builtin_amdgcn_readfirstlane(rows);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base + row0 * row_elems), (short)0,
                                             rows * static_cast<int>(row_elems) * 2, 0x00020000);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
    return __builtin_bit_cast(uint32_t, v);
}

// Transposing LDS read, issued through inline assembly: the compiler then
// does not treat it as a possible reader of the direct global->LDS loads in
// flight (it would otherwise wait for all of them first).  The caller owns
// the LDS wait: lgkm_wait<N>(v) waits until at most N LDS operations are
// outstanding and ties the wait to v, so uses of v stay after it.
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) char *)(p)));
}
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16(uint32_t addr) {
    u32x2 v;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}
// Keeps the computation of v inside the current scheduling region: the empty
// volatile asm consumes v, and volatile asm statements keep their order
// relative to the region boundaries.
__device__ __forceinline__ void anchor(float v) { asm volatile("" ::"v"(v)); }

template <int N>
__device__ __forceinline__ void lgkm_wait(bf16x8 &v) {
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "i"(N));
}

// Max of x over lanes l and l ^ 32.
// max of two floats that are never signalling NaNs: a plain v_max_f32, without
// the quieting of the inputs that fmaxf implies
__device__ __forceinline__ float vmax(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

__device__ __forceinline__ float xhalf_max(float x) {
    const uint32_t u = __float_as_uint(x);
    auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return vmax(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ float xhalf_sum(float x) {
    const uint32_t u = __float_as_uint(x);
    auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ---------------------------------------------------------------------------
// Packed sequence b spans tokens [s0, s1) of T.  The offsets are read on the
// device and not validated; clamping them to [0, T] leaves well-formed ones
// unchanged and turns malformed ones (decreasing, negative, past T) into
// empty or shortened sequences inside the buffers, never into accesses past
// them.
__device__ __forceinline__ void seq_span(const int32_t *cu, int b, int T, int &s0, int &s1) {
    s0 = min(max(cu[b], 0), T);
    s1 = min(max(cu[b + 1], s0), T);
}
__device__ __forceinline__ int seq_len(const int32_t *cu, int b, int T) {
    int s0, s1;
    seq_span(cu, b, T, s0, s1);
    return s1 - s0;
}

// ---------------------------------------------------------------------------
// Work decode: one workgroup = (sequence b, head h, query tile qt).

struct Work {
    int b, h, qt, n;  // n: length of sequence b
    long long t0;     // first token of sequence b
    int split;        // key range (split-KV instances)
};

template <bool CAUSAL, bool VARLEN, int BR, bool SPLIT, bool MODS = false>
__device__ __forceinline__ bool decode_work(const Params &p, Work &w) {
    int wg = blockIdx.x;
    w.split = 0;
    if constexpr (SPLIT && !VARLEN) {
        // Items are (b, h, key range, query tile); the ranges of one query
        // tile hold equal work.  Causal: highest query tile first (it sees the
        // most keys).  Non-causal: each XCD
        // gets a contiguous run of items, i.e. the query tiles of one
        // (b, h, range) and so one K/V range in its L2.
        const int BH = p.B * p.H, S = p.nsplit;
        int bh, qt, s;
        if constexpr (CAUSAL) {
            const int level = BH * S;
            qt = p.n_qt - 1 - wg / level;
            const int r = wg - (wg / level) * level;
            s = r / BH;
            bh = r - s * BH;
        } else {
            const int G = gridDim.x, x = wg & 7, sx = wg >> 3;
            const int per = G >> 3, rem = G & 7;
            const int item = x * per + (x < rem ? x : rem) + sx;
            const int per_bh = S * p.n_qt;
            bh = item / per_bh;
            const int r = item - bh * per_bh;
            s = r / p.n_qt;
            qt = r - s * p.n_qt;
        }
        w.b = bh / p.H;
        w.h = bh - w.b * p.H;
        w.qt = qt;
        w.split = s;
        w.n = p.N;
        w.t0 = static_cast<long long>(w.b) * p.N;
        return true;
    } else if constexpr (!VARLEN) {
        const int BH = p.B * p.H;
        int bh, qt;
        // a window with a right edge makes the work grow with the query tile
        // like the causal mask does
        if (CAUSAL || (MODS && p.wr >= 0)) {
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
        // packed with key ranges: the ranges of one (sequence, head, query
        // tile) are consecutive workgroups, the item order below for the rest
        if constexpr (SPLIT) {
            w.split = wg % p.nsplit;
            wg /= p.nsplit;
        }
        const int lane = threadIdx.x & 63;
        w.h = wg % p.H;
        int r = wg / p.H;
        if (p.B <= 64) {
            // Items are ordered by sequence, longest first (ties by index),
            // and within a sequence by query tile, highest first; the head
            // varies fastest, so the tiles of one (sequence, head) run at
            // about the same time on one XCD (wg % 8) and share its L2.
            // Lane b computes where sequence b's tiles start in that order.
            const int b = lane;
            const int len = b < p.B ? seq_len(p.cu, b, p.N) : 0;
            const int tiles = (len + BR - 1) / BR;
            int pos = 0;
            for (int o = 0; o < p.B; ++o) {
                const int lo = seq_len(p.cu, o, p.N);
                const bool before = lo > len || (lo == len && o < b);
                pos += before ? (lo + BR - 1) / BR : 0;
            }
            const bool mine = b < p.B && r >= pos && r < pos + tiles;
            const unsigned long long m = __ballot(mine);
            if (m == 0) return false;  // surplus workgroup of the grid bound
            const int bsel = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(m)) - 1);
            const int pos_sel = __builtin_amdgcn_readfirstlane(__shfl(pos, bsel));
            const int tiles_sel = __builtin_amdgcn_readfirstlane(__shfl(tiles, bsel));
            w.b = bsel;
            w.qt = tiles_sel - 1 - (r - pos_sel);
            int s0, s1;
            seq_span(p.cu, bsel, p.N, s0, s1);
            s0 = __builtin_amdgcn_readfirstlane(s0);
            s1 = __builtin_amdgcn_readfirstlane(s1);
            w.t0 = s0;
            w.n = s1 - s0;
            return true;
        }
        // More than 64 sequences: items ordered by query-tile index, highest
        // first (for causal masks the work of a tile grows with its index),
        // ties in sequence order; ballots over 64 sequences at a time.
        int lmax = 0;
        for (int base = 0; base < p.B; base += 64) {
            const int b = base + lane;
            int nt = 0;
            if (b < p.B) nt = (seq_len(p.cu, b, p.N) + BR - 1) / BR;
            for (int off = 32; off > 0; off >>= 1) nt = max(nt, __shfl_xor(nt, off));
            lmax = max(lmax, __builtin_amdgcn_readfirstlane(nt));
        }
        for (int L = lmax - 1; L >= 0; --L) {
            int cnt = 0;
            for (int base = 0; base < p.B; base += 64) {
                const int b = base + lane;
                bool on = false;
                if (b < p.B) on = (seq_len(p.cu, b, p.N) + BR - 1) / BR > L;
                cnt += __popcll(__ballot(on));
            }
            if (r < cnt) {
                for (int base = 0; base < p.B; base += 64) {
                    const int b = base + lane;
                    bool on = false;
                    if (b < p.B) on = (seq_len(p.cu, b, p.N) + BR - 1) / BR > L;
                    unsigned long long m = __ballot(on);
                    const int c = __popcll(m);
                    if (r < c) {
                        // position of the r-th set bit of m
                        for (int i = 0; i < r; ++i) m &= m - 1;
                        // every value here is wave-uniform; say so to the compiler
                        const int bsel = __builtin_amdgcn_readfirstlane(
                            base + __ffsll(static_cast<long long>(m)) - 1);
                        w.b = bsel;
                        w.qt = __builtin_amdgcn_readfirstlane(L);
                        int s0, s1;
                        seq_span(p.cu, bsel, p.N, s0, s1);
                        s0 = __builtin_amdgcn_readfirstlane(s0);
                        s1 = __builtin_amdgcn_readfirstlane(s1);
                        w.t0 = s0;
                        w.n = s1 - s0;
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
// The kernel.  NW waves, each owning QB blocks of 32 query rows, so a
// workgroup covers BR = NW * QB * 32 rows; BC keys per K/V tile.  With QB = 2
// every K or V fragment read from LDS feeds two MFMAs.
//
// Each wave runs a two-stage software pipeline over the K/V tiles so that its
// MFMAs overlap its own softmax arithmetic:
//   [A_j]  MFMA  S_{j+1} = K_{j+1} Q^T  ||  VALU  first half of P_j = 2^(S_j c - m_j)
//   [B_j]  MFMA  O^T += V_j^T P_j^T     ||  VALU  second half of P_j, row max of
//                                              S_{j+1}
// after which the reference max, the rescale factor and l are updated.  LDS
// holds two K and two V tiles; at the start of iteration j the direct loads
// of K_{j+2} and V_{j+1} are issued into the tiles of K_j and V_{j-1} (both
// consumed before the previous barrier); the barrier that ends the iteration
// makes them visible.

template <int D, int BC, int NW, int QB, bool CAUSAL, bool VARLEN, int EXPM, int RSM, bool SPLIT = false,
          bool MODS = false, bool COUNT = false, bool PING = false>
__global__ void __launch_bounds__(NW * 64)
fa_fwd_kernel(Params p) {
    using SW = Swz<D>;
    constexpr int RW = QB * 32;          // query rows per wave
    constexpr int BR = NW * RW;          // query rows per workgroup
    constexpr int KK = D / 16;           // MFMA k-steps of Q K^T
    constexpr int NKB = BC / 32;         // 32-key blocks per tile
    constexpr int NDB = D / 32;          // 32-wide d blocks of O^T
    constexpr int NT16 = BC / 16;        // 16-key chunks (PV k-steps)
    constexpr int RB = SW::RB;
    constexpr int TB = BC * RB;          // bytes per K (or V) tile
    constexpr int BLK = TB / 1024;       // 1 KB direct-load blocks per tile
    constexpr int MS = KK * NKB;         // fragment steps of one S tile (= of one PV pass)
    constexpr int NE = NKB * 16;         // S elements per lane per query block
    static_assert(MS == NT16 * NDB, "phase shapes");

    // Two K and two V tiles, as separate objects so that the compiler can see
    // that reads of one tile never alias the direct loads filling another.
    __shared__ __attribute__((aligned(1024))) char k_lds0[TB], k_lds1[TB], v_lds0[TB], v_lds1[TB];

    Work w;
    if (!decode_work<CAUSAL, VARLEN, BR, SPLIT, MODS>(p, w)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int c = lane & 31, hh = lane >> 5;
    const int n = w.n;
    const int q0 = w.qt * BR;
    const long long rs = static_cast<long long>(p.H) * D;  // token stride (elements)
    const long long base = (w.t0 * p.H + w.h) * D;
    const uint16_t *qg = p.q + base;
    const uint16_t *kg = p.k + base;
    const uint16_t *vg = p.v + base;

    const int wrow0 = q0 + wave * RW;  // first row of this wave; block b starts at wrow0 + 32 b

    // Q fragments: B operand of S^T = K Q^T, lane (c, hh) of block b holds
    // Q[wrow0 + 32 b + c][kk*16 + hh*8 .. +8]; rows >= n read as zeros.
    bf16x8 qf[QB][KK];
    {
        const int voff = (c * static_cast<int>(rs) + hh * 8) * 2;
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            const auto qrs = rows_rsrc(qg, rs, wrow0 + 32 * b, n);
#pragma unroll
            for (int kk = 0; kk < KK; ++kk)
                qf[b][kk] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, voff + kk * 32, 0, 0));
        }
    }

    // keys past kv_end are invisible to every row of the workgroup: the causal
    // diagonal, or the right edge of a window
    const int kv_end = MODS ? (p.wr < 0 ? n : min(n, q0 + BR + p.wr)) : (CAUSAL ? min(n, q0 + BR) : n);
    // Tiles are numbered from kt0, the first tile of this workgroup's key
    // range (0 unless the key sequence is split or a window's left edge
    // hides the first tiles); tile j covers keys (kt0 + j) * BC ...
    // The split divides the tiles this query tile sees (all of the sequence,
    // or up to the diagonal when causal) into nsplit near-equal ranges.
    const int tiles_seen = (kv_end + BC - 1) / BC;
    const int kt0 = SPLIT ? w.split * tiles_seen / p.nsplit
                          : (MODS && p.wl >= 0 ? max(0, q0 - p.wl) / BC : 0);
    const int kt_end = SPLIT ? (w.split + 1) * tiles_seen / p.nsplit : tiles_seen;
    const int nkv = max(kt_end - kt0, 0);
    // tiles this wave computes: the causal diagonal (or the window's right
    // edge) ends its work earlier
    int w_end = kt_end;
    if (CAUSAL) w_end = min(kt_end, (wrow0 + RW - 1) / BC + 1);
    if (MODS && p.wr >= 0) w_end = min(kt_end, (wrow0 + RW - 1 + p.wr) / BC + 1);
    const int nkv_w = max(w_end - kt0, 0);

    // ---- direct global -> LDS loads ---------------------------------------------
    // K: the tile is 8*D/64 loads of 1 KB (8 rows of one 128-byte plane each);
    // wave w issues loads w, w + NW, ...  Lane l of load I fills row
    // 8 (I % 8) + l / 8 of plane I / 8, slot l % 8, with logical chunk
    // (l % 8) ^ g(row); g depends on I only through I % 2, which is the same
    // for all of a wave's loads, so one per-lane offset serves them all.
    // V: wave w fills 1 KB blocks w, w + NW, ...; lane l of block b fills tile
    // bytes b*1024 + 16 l = chunk slot pc of row r with logical chunk pc ^ f_V(r)
    // (f_V depends only on l).
    // Ping-pong (PING instances, eight-wave workgroups): waves 0..3 form
    // group 0 and waves 4..7 group 1, so every SIMD holds one wave of each.
    // Group 1 runs half a key tile behind group 0, with a workgroup barrier
    // every half tile: while one group issues its loads, rescales O and waits
    // at the barrier, the other group's matrix products keep the SIMD's
    // matrix unit busy.  Group 0 issues every K tile's loads, group 1 every V
    // tile's.  (Measured 2-5 % slower than both groups in step: a single
    // wave issues vector instructions too slowly to fill the matrix unit's
    // shadow on its own, so the default keeps both waves of a SIMD
    // interleaving products and softmax.)
    static_assert(!PING || NW == 8, "the ping-pong pairs the two waves of a SIMD");
    constexpr bool PP = PING;
    constexpr int LW = PP ? NW / 2 : NW;  // waves that share one tile's loads
    const int grp = PP ? (wave >= LW ? 1 : 0) : 0;
    const int li = wave - grp * LW;       // this wave's index among them
    static_assert(BC == 64, "K planes are 64 rows");
    static_assert(LW == 4 || LW == 8, "each wave's K loads must share one row parity");
    constexpr int KLD = D / 8;            // 1 KB K loads per tile
    constexpr int KPW = KLD / LW;         // K loads per loading wave
    constexpr int VPW = BLK / LW;         // V loads per loading wave
    static_assert(KLD % LW == 0 && BLK % LW == 0, "loads must split evenly");
    const int rs_bytes = static_cast<int>(rs) * 2;
    int koff;
    {
        const int r = 8 * (li % 8) + lane / 8;
        koff = r * rs_bytes + (((lane % 8) ^ Swz<D>::gk(r)) << 4);
    }
    int voff;
    {
        const int pos = li * 1024 + lane * 16;
        const int r = pos / RB, pc = (pos % RB) / 16;
        voff = r * rs_bytes + ((pc ^ Swz<D>::fv(r)) << 4);
    }
    // A load whose rows start past the wave's first rows gets a resource
    // based at those rows (the size check covers the lane offset only); the
    // scalar offset carries just the plane's column offset.
    // With eight loading waves a tile needs at most two lane offsets per
    // tensor, so each tile gets one resource and the row offset of a load
    // goes into its lane offset (precomputed, checked against the size);
    // with four, a tile's loads reach up to eight row groups and each gets a
    // resource of its own instead (scalar work, no vector registers).
    constexpr int VROWS = 1024 / RB;     // V rows per 1 KB block
    constexpr bool ONE_RSRC = LW == 8;
    const int voff_hi = voff + LW * VROWS * rs_bytes;   // V loads i = 1 (eight loading waves)
    auto dma_k = [&](char *tile, int j) {
        const int kv0 = (kt0 + j) * BC;
        const auto rsrc = rows_rsrc(kg, rs, kv0, n);
#pragma unroll
        for (int i = 0; i < KPW; ++i) {
            const int I = li + LW * i;                // load index within the tile
            const int di = (I % 8) - (li % 8);        // rows of this load past the wave's first / 8
            if constexpr (ONE_RSRC)                   // di = 0: I % 8 = li % 8
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, tile + I * 1024), 16, koff,
                                                         (I / 8) * 128, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(kg, rs, kv0 + 8 * di, n),
                                                         LDS_PTR(void, tile + I * 1024), 16, koff, (I / 8) * 128, 0, 0);
        }
    };
    auto dma_v = [&](char *tile, int j) {
        const int kv0 = (kt0 + j) * BC;
        const auto rsrc = rows_rsrc(vg, rs, kv0, n);
#pragma unroll
        for (int i = 0; i < VPW; ++i) {
            if constexpr (ONE_RSRC) {
                static_assert(!ONE_RSRC || VPW <= 2, "two V lane offsets");
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, LDS_PTR(void, tile + (li + LW * i) * 1024), 16,
                                                         i == 0 ? voff : voff_hi, 0, 0, 0);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(vg, rs, kv0 + LW * i * VROWS, n),
                                                         LDS_PTR(void, tile + (li + LW * i) * 1024), 16, voff, 0, 0,
                                                         0);
            }
        }
    };
    // The half-tile barrier of the ping-pong: no wait for the direct loads in
    // flight (they are waited for before the end-of-step barrier); the empty
    // asm keeps the compiler from moving memory accesses across it.
    auto half_barrier = [&]() {
        if constexpr (PP) {
            __builtin_amdgcn_sched_barrier(0);
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- LDS fragment reads --------------------------------------------------------
    // K fragment of S step (kk, kb2): rows kb2*32 + c, chunk 2 kk + hh, i.e.
    // plane kk / 4, in-plane chunk 2 (kk % 4) + hh.
    int kaddr[4];
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) kaddr[bb] = c * 128 + (((2 * bb + hh) ^ Swz<D>::gk(c)) << 4);
    auto kfrag = [&](const char *kb, int kk, int kb2) -> bf16x8 {
        return *reinterpret_cast<const bf16x8 *>(kb + kaddr[kk % 4] + (kk / 4) * 8192 + kb2 * 32 * 128);
    };
    // V fragment of PV step (t, db): rows t*16 + hh*4 + s/4 (+8 for the upper
    // half), columns db*32 + (g&1)*16 + (s&3)*4, for lane group g, s = lane%16.
    const int g16 = lane >> 4, s16 = lane & 15;
    constexpr int NVA = NDB < 4 ? NDB : 4;
    int vaddr[NVA];
    {
        const int vr = hh * 4 + (s16 >> 2);
        const int x = (g16 & 1) * 2 + ((s16 & 3) >> 1);
#pragma unroll
        for (int bb = 0; bb < NVA; ++bb)
            vaddr[bb] = vr * RB + (((4 * bb + x) ^ Swz<D>::fv(vr)) << 4) + (s16 & 1) * 8;
    }
    // Issues the two transposing reads of a V fragment; the caller waits.
    auto vfrag_issue = [&](const char *vb, auto t_, auto db_) -> bf16x8 {
        constexpr int t = decltype(t_)::value, db = decltype(db_)::value;
        const uint32_t a = lds_offset(vb) + vaddr[db % NVA];
        constexpr int off = (db / NVA) * 256 + t * 16 * RB;
        const u32x2 lo = ds_read_tr16<off>(a);
        const u32x2 hi = ds_read_tr16<off + 8 * RB>(a);
        const u32x4 both = {lo[0], lo[1], hi[0], hi[1]};
        return __builtin_bit_cast(bf16x8, both);
    };

    // ---- per-wave softmax state (per query block) ---------------------------------
    f32x16 oacc[QB][NDB];
#pragma unroll
    for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int i = 0; i < NDB; ++i) oacc[b][i] = f32x16{};
    // Threshold rescale: the reference max may trail a row's true max by up to
    // 8, so a row dominated by one key gives that key a weight up to 2^8, which
    // bf16 rounds by up to 2^-9; dividing O by the sum of the bf16 weights the
    // P V product actually uses keeps O a weighted mean of V rows (the LSE
    // keeps the fp32 sum).  Under the strict and always rules the dominant
    // weight is exactly 1 and O is divided by the fp32 sum.
    constexpr bool kBf16Norm = RSM == FA_RESCALE_THRESHOLD;
    float m_run[QB], l_run[QB], lb_run[QB], m_use[QB], alpha[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        m_run[b] = -INFINITY;  // reference max, scaled log2 units
        l_run[b] = 0.0f;       // this lane's partial row sum (fp32 weights: the LSE)
        lb_run[b] = 0.0f;      // the same over the bf16 weights P V uses (divides O)
        m_use[b] = 0.0f;       // subtrahend of the tile being exponentiated
        alpha[b] = 1.0f;       // pending rescale of O for that tile
    }
    bool rescale_o = false;    // wave-uniform: some row's reference moved
    const float cs = p.cs;

    // -inf for tail keys (>= n) and, when causal, keys after the query.
    auto need_mask = [&](int j) {
        const int kv0 = (kt0 + j) * BC;
        if constexpr (MODS)
            return p.alibi != nullptr || (p.wl >= 0 && kv0 < wrow0 + RW - 1 - p.wl) ||
                   (p.wr >= 0 && kv0 + BC - 1 > wrow0 + p.wr) || kv0 + BC > n;
        return (CAUSAL && kv0 + BC - 1 > wrow0) || kv0 + BC > n;
    };
    const float bias_coef = MODS && p.alibi ? p.alibi[w.h] * p.inv_scale : 0.0f;
    // linear bias of block b: slope (j - i) on the scaled score = slope / scale
    // on the raw one; j - i = (k0 - qrow) + C
    auto s_bias_block = [&](f32x16 (&s)[QB][NKB], int b, int k0, int qrow) {
        const float base = static_cast<float>(k0 - qrow);
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int C = kb2 * 32 + (r >> 2) * 8 + (r & 3);
                s[b][kb2][r] = __builtin_fmaf(bias_coef, base + static_cast<float>(C), s[b][kb2][r]);
            }
    };
    // the bias alone, for tiles that no window edge or tail cuts
    auto s_bias = [&](f32x16 (&s)[QB][NKB], int j) {
        const int k0 = (kt0 + j) * BC + 4 * hh;
#pragma unroll
        for (int b = 0; b < QB; ++b) s_bias_block(s, b, k0, wrow0 + 32 * b + c);
    };
    auto s_mask = [&](f32x16 (&s)[QB][NKB], int j) {
        const int kv0 = (kt0 + j) * BC;
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            const int qrow = wrow0 + 32 * b + c;
            if constexpr (!MODS) {
                // key = kv0 + 4 hh + C with C = 32 kb2 + 8 (r >> 2) + (r & 3) fixed per
                // element: the key is visible iff C < lim, one compare with an inline
                // constant per element (measured +3 % on short causal runs)
                int lim = n - kv0 - 4 * hh;
                if (CAUSAL) lim = min(lim, qrow - kv0 - 4 * hh + 1);
#pragma unroll
                for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int C = kb2 * 32 + (r >> 2) * 8 + (r & 3);
                        s[b][kb2][r] = C < lim ? s[b][kb2][r] : -INFINITY;
                    }
                continue;
            }
            // windows: key = kv0 + 4 hh + C is visible iff lo <= C < hi, two
            // compares per element against per-lane limits (a chain of
            // short-circuit tests per element would compile to branches)
            const int k0 = kv0 + 4 * hh;
            int hi = n - k0;
            if (CAUSAL) hi = min(hi, qrow - k0 + 1);
            if (p.wr >= 0) hi = min(hi, qrow + p.wr - k0 + 1);
            const int lo = p.wl >= 0 ? qrow - p.wl - k0 : -BC;
            if (p.alibi != nullptr) s_bias_block(s, b, k0, qrow);
#pragma unroll
            for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int C = kb2 * 32 + (r >> 2) * 8 + (r & 3);
                    s[b][kb2][r] = ((C >= lo) & (C < hi)) ? s[b][kb2][r] : -INFINITY;
                }
        }
    };
    // Reference max update of every block from its tile's raw row max
    // (`tally`: counted by the counting instances; not for the first tile).
    auto s_update = [&](float (&mx)[QB], bool tally = true) {
        bool grow_any = false;
        unsigned grown = 0;
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            const float x = xhalf_max(mx[b]);
            const float mt = x * cs;  // cs > 0: -inf stays -inf
            float m_new;
            bool grow;
            if constexpr (RSM == FA_RESCALE_THRESHOLD) {
                grow = mt > m_run[b] + kTau;  // also true for the first finite tile
                m_new = grow ? mt : m_run[b];
            } else {
                m_new = vmax(m_run[b], mt);
                grow = m_new > m_run[b];
            }
            // a row with no visible key so far keeps m = -inf; its subtrahend is then a
            // large finite value, so that -inf - m_use is -inf and never NaN
            float mu;
            asm("v_max_f32 %0, 0xf149f2ca, %1" : "=v"(mu) : "v"(m_new));  // max(m_new, -1e30)
            m_use[b] = mu;
            alpha[b] = __builtin_amdgcn_exp2f(m_run[b] - m_use[b]);  // 1 if unchanged, 0 from -inf
            l_run[b] *= alpha[b];
            if constexpr (kBf16Norm) lb_run[b] *= alpha[b];
            m_run[b] = m_new;
            grow_any = grow_any || grow;
            if constexpr (COUNT) grown += __popcll(__ballot(grow)) / 2;  // each row sits in two lanes
        }
        if constexpr (COUNT) {
            if (tally && lane == 0) {
                atomicAdd(&p.counts[2], static_cast<unsigned long long>(grown));
                atomicAdd(&p.counts[3], static_cast<unsigned long long>(32 * QB));
            }
        }
        if constexpr (RSM == FA_RESCALE_ALWAYS) {
            rescale_o = true;
        } else {
            rescale_o = __ballot(grow_any) != 0;
        }
    };
    auto s_rowmax = [&](const f32x16 (&s)[QB][NKB], float (&mx)[QB]) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            mx[b] = -INFINITY;
#pragma unroll
            for (int kb2 = 0; kb2 < NKB; ++kb2)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx[b] = fmaxf(mx[b], s[b][kb2][r]);
        }
    };
    // S^T = K Q^T alone (prologue).
    auto s_mfma = [&](f32x16 (&s)[QB][NKB], const char *kb) {
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int i = 0; i < NKB; ++i) s[b][i] = f32x16{};
#pragma unroll
        for (int m = 0; m < MS; ++m) {
            const int kb2 = m % NKB, kk = m / NKB;
            const bf16x8 kf = kfrag(kb, kk, kb2);
#pragma unroll
            for (int b = 0; b < QB; ++b)
                s[b][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[b][kk], s[b][kb2], 0, 0, 0);
        }
    };
    // P~ element e (0..NE-1) of block b: e = kb2*16 + r, pf[b][t] holds e = 8t..8t+7.
    bf16x8 pf[QB][NT16];
    float pe[QB][NE];
    auto p_elem = [&](const f32x16 (&s)[QB][NKB], int b, int e) {
        pe[b][e] = exp2_sel<EXPM>(__builtin_fmaf(s[b][e >> 4][e & 15], cs, -m_use[b]), e);
    };
    const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
    auto p_pack = [&](int b, int t, float &rsum) {
        uint32_t pk[4];
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            rsum += pe[b][8 * t + i] + pe[b][8 * t + i + 1];
            pk[i >> 1] = pack_bf16x2(pe[b][8 * t + i], pe[b][8 * t + i + 1]);
            if constexpr (kBf16Norm)
                lb_run[b] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk[i >> 1]), ones,
                                                            lb_run[b], false);
        }
        u32x4 pv = {pk[0], pk[1], pk[2], pk[3]};
        pf[b][t] = __builtin_bit_cast(bf16x8, pv);
    };
    auto p_exp = [&](const f32x16 (&s)[QB][NKB]) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            float rsum = 0.0f;
#pragma unroll
            for (int e = 0; e < NE; ++e) {
                p_elem(s, b, e);
                if ((e & 7) == 7) p_pack(b, e >> 3, rsum);
            }
            l_run[b] += rsum;
        }
    };
    auto o_rescale = [&]() {
#pragma unroll
        for (int b = 0; b < QB; ++b)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) oacc[b][db][r] *= alpha[b];
    };
    // PV product: O^T += V^T P^T, step order t-major (all d blocks of key chunk
    // t, then chunk t+1), V fragments read two steps ahead, QB MFMAs per step.
    // `work(m)` is VALU work placed after step m; it may produce pf[.][t] for a
    // later t.
    auto pv_run = [&](const char *vb, auto &&work) {
        constexpr int LA = kVLookahead < MS ? kVLookahead : MS;  // fragments in flight
        bf16x8 vf[MS];
        static_for<0, LA>([&](auto m) {
            vf[m] = vfrag_issue(vb, std::integral_constant<int, m / NDB>{},
                                std::integral_constant<int, m % NDB>{});
        });
        static_for<0, MS>([&](auto m) {
            constexpr int t = m / NDB, db = m % NDB;
            // two LDS reads per fragment; the later fragments may stay in flight
            constexpr int later = (LA - 1 < MS - 1 - m) ? LA - 1 : MS - 1 - m;
            lgkm_wait<2 * later>(vf[m]);
#pragma unroll
            for (int b = 0; b < QB; ++b)
                oacc[b][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[m], pf[b][t], oacc[b][db], 0, 0, 0);
            if constexpr (m + LA < MS)
                vf[m + LA] = vfrag_issue(vb, std::integral_constant<int, (m + LA) / NDB>{},
                                         std::integral_constant<int, (m + LA) % NDB>{});
            work(m);
        });
    };
    auto pv_mfma = [&](const char *vb) { pv_run(vb, [](auto) {}); };

    // The exponentials of S_j are split between the two phases: [A] does key
    // chunks 0 .. NT16/2-1 of every block, [B] the rest, chunk NT16/2 + i during
    // PV steps i*NDB .. (i+1)*NDB-1, i.e. before the first step that needs it.
    // [B] then takes the row max of S_{j+1}.  The sched_group_barrier sequences
    // spread the VALU work evenly between the MFMAs (a wave issues in order; a
    // burst of exponentials between two MFMAs would hold back the second), and
    // anchor() keeps [A]'s exponentials inside [A].
    constexpr int HALF = NE / 2;          // elements per block per phase
    constexpr int AE = QB * HALF;         // [A] elements (all blocks)
    float rsum_a[QB];

    // [A]: S_{j+1} MFMAs interleaved with the first half of the exponentials of S_j.
    // The first KLA K fragments are read by the caller (k_prefetch) at the
    // top of the step, so that their LDS latency passes under the load issue
    // and the O rescale instead of stalling the first MFMA.
    constexpr int KLA = kKLookahead < MS ? kKLookahead : MS;  // fragments in flight
    auto k_prefetch = [&](bf16x8 (&kf)[KLA + 1], const char *kb) {
        // step order alternates the NKB accumulator chains
        static_for<0, KLA>([&](auto i) { kf[i] = kfrag(kb, i / NKB, i % NKB); });
    };
    auto phase_a = [&](f32x16 (&nxt)[QB][NKB], const f32x16 (&cur)[QB][NKB], const char *kb,
                       bf16x8 (&kf)[KLA + 1]) {
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            rsum_a[b] = 0.0f;
#pragma unroll
            for (int i = 0; i < NKB; ++i) nxt[b][i] = f32x16{};
        }
        constexpr int LA = KLA;
        static_for<0, MS>([&](auto m) {
            constexpr int kb2 = m % NKB, kk = m / NKB;
            if constexpr (m + LA < MS) kf[(m + LA) % (LA + 1)] = kfrag(kb, (m + LA) / NKB, (m + LA) % NKB);
#pragma unroll
            for (int b = 0; b < QB; ++b)
                nxt[b][kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[m % (LA + 1)], qf[b][kk], nxt[b][kb2], 0, 0, 0);
            // elements [m*AE/MS, (m+1)*AE/MS) of the list (b, e), b-major
#pragma unroll
            for (int x = m * AE / MS; x < (m + 1) * AE / MS; ++x) {
                const int b = x / HALF, e = x % HALF;
                p_elem(cur, b, e);
                anchor(pe[b][e]);
                if ((e & 7) == 7) p_pack(b, e >> 3, rsum_a[b]);
            }
        });
#pragma unroll
        for (int b = 0; b < QB; ++b) anchor(rsum_a[b]);
        static_for<0, MS>([&](auto m) {
            constexpr int ne = (m + 1) * AE / MS - m * AE / MS;  // elements of this step
            __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);  // MFMA
            if constexpr (m + LA < MS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            if constexpr (ne > 0) __builtin_amdgcn_sched_group_barrier(0x402, 3 * ne + (ne + 1) / 2, 0);
        });
    };
    // [B]: PV MFMAs interleaved with the second half of the exponentials of
    // S_j and the row max of S_{j+1}.
    auto phase_b = [&](const f32x16 (&nxt)[QB][NKB], const f32x16 (&cur)[QB][NKB], const char *vb,
                       float (&mx)[QB]) {
        constexpr int EB = QB * 8 / NDB;                // exp elements per step, first half of [B]
        constexpr int MB = QB * NE / (MS - MS / 2);     // max elements per step, second half
        static_assert((QB * 8) % NDB == 0 && (QB * NE) % (MS - MS / 2) == 0, "element split");
        float rsum[QB];
#pragma unroll
        for (int b = 0; b < QB; ++b) {
            rsum[b] = rsum_a[b];
            mx[b] = -INFINITY;
        }
        pv_run(vb, [&](auto m) {
            if constexpr (m < MS / 2) {
                // chunk NT16/2 + m / NDB of every block: elements (b, 8 t + i)
#pragma unroll
                for (int x = m * EB; x < (m + 1) * EB; ++x) {
                    const int t = NT16 / 2 + x / (QB * 8);
                    const int b = (x / 8) % QB, i = x % 8;
                    const int e = 8 * t + i;
                    p_elem(cur, b, e);
                    if (i == 7) p_pack(b, t, rsum[b]);
                }
            } else {
#pragma unroll
                for (int x = (m - MS / 2) * MB; x < (m - MS / 2 + 1) * MB; ++x) {
                    const int b = x / NE, e = x % NE;
                    mx[b] = fmaxf(mx[b], nxt[b][e >> 4][e & 15]);
                }
            }
        });
        static_for<0, MS>([&](auto m) {
            __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);  // MFMA
            if constexpr (m < MS / 2) __builtin_amdgcn_sched_group_barrier(0x402, 3 * EB + (EB + 1) / 2, 0);
            else __builtin_amdgcn_sched_group_barrier(0x402, (MB + 1) / 2, 0);
        });
#pragma unroll
        for (int b = 0; b < QB; ++b) l_run[b] += rsum[b];
    };

    // ---- prologue: K_0, V_0, K_1 into LDS; S_0 and its row max ------------------
    f32x16 sa[QB][NKB], sb[QB][NKB];
    // (a key range with no visible key for the workgroup skips straight to the
    // epilogue and stores the empty result)
    if (nkv > 0) {
    if (!PP || grp == 0) {
        dma_k(k_lds0, 0);
        if (nkv > 1) dma_k(k_lds1, 1);
    }
    if (!PP || grp == 1) dma_v(v_lds0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (nkv_w > 0) {
        s_mfma(sa, k_lds0);
        if (need_mask(0)) s_mask(sa, 0);
        float mx[QB];
        s_rowmax(sa, mx);
        s_update(mx, false);
    }
    __syncthreads();  // K tile 0 is reloaded at the start of iteration 0

    // Direct loads that belong to iteration j: K_{j+2} over K_j, V_{j+1} over
    // V_{j-1} (both consumed before the previous barrier).
    // (ping-pong: group 0 issues the K loads in its half tile, group 1 the V
    // loads in the next; each tile then has one full step to land)
    auto issue_loads = [&](int j, char *k_dst, char *v_dst) {
        if ((!PP || grp == 0) && j + 2 < nkv) dma_k(k_dst, j + 2);
        if ((!PP || grp == 1) && j + 1 < nkv) dma_v(v_dst, j + 1);
    };
    auto end_iteration = [&]() {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads have landed
        __syncthreads();
    };
    // A full pipeline iteration (tiles j and j+1 both computed by this wave);
    // PAR = j & 1 selects the LDS tiles statically.  MASK: tile j+1 needs the
    // tail/causal mask (kept out of the hot loop so that nothing separates
    // phase [A] from phase [B]).
    // counting instances: the O-rescale decision of step j (tile S_j), j >= 1
    auto tally_step = [&](int j) {
        if constexpr (COUNT) {
            if (j > 0 && lane == 0) {
                atomicAdd(&p.counts[0], 1ull);
                if (rescale_o) atomicAdd(&p.counts[1], 1ull);
            }
        }
    };
    auto full_step = [&](auto par, auto mask, f32x16 (&cur)[QB][NKB], f32x16 (&nxt)[QB][NKB], int j) {
        constexpr int PAR = decltype(par)::value;
        bf16x8 kf[KLA + 1];
        k_prefetch(kf, (PAR ? k_lds0 : k_lds1));  // K_{j+1}, in LDS since the last barrier
        issue_loads(j, (PAR ? k_lds1 : k_lds0), (PAR ? v_lds0 : v_lds1));
        tally_step(j);
        if (rescale_o) o_rescale();
        __builtin_amdgcn_sched_barrier(0);
        // the score MFMAs go first when the SIMD's two waves compete for
        // issue (measured +1 %)
        __builtin_amdgcn_s_setprio(1);
        phase_a(nxt, cur, (PAR ? k_lds0 : k_lds1), kf);  // K_{j+1}
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(mask)::value == 1) s_mask(nxt, j + 1);
        else if constexpr (decltype(mask)::value == 2) s_bias(nxt, j + 1);
        half_barrier();
        float mx[QB];
        phase_b(nxt, cur, (PAR ? v_lds1 : v_lds0), mx);  // V_j
        s_update(mx);
        __builtin_amdgcn_sched_barrier(0);
        end_iteration();
    };
    // The wave's last tile: no next S.
    auto drain_step = [&](const f32x16 (&cur)[QB][NKB], int j) {
        const int par = j & 1;
        issue_loads(j, (par ? k_lds1 : k_lds0), (par ? v_lds0 : v_lds1));
        tally_step(j);
        if (rescale_o) o_rescale();
        p_exp(cur);
        half_barrier();
        pv_mfma((par ? v_lds1 : v_lds0));
        end_iteration();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    // what a step does to its next tile's scores: nothing, the tail / causal /
    // window mask (with the bias, if any), or the bias alone
    using NoMask = std::integral_constant<int, 0>;
    using Mask = std::integral_constant<int, 1>;
    using BiasOnly = std::integral_constant<int, 2>;

    // first tile that needs a mask (tail: n / BC; causal: (wrow0 + 1) / BC)
    // (windows: the right edge plays the diagonal's part, the left edge masks
    // the first tiles, jh of them rounded up to a pair; a bias goes on every
    // tile, with the mask or alone)
    int jm = (CAUSAL ? min(n / BC, (wrow0 + 1) / BC) : n / BC) - kt0;
    int jh = 0;
    if constexpr (MODS) {
        jm = (p.wr >= 0 ? min(n / BC, (wrow0 + p.wr + 1) / BC) : n / BC) - kt0;
        if (p.wl >= 0) jh = max(0, (wrow0 + RW - 1 - p.wl - kt0 * BC + BC) / BC);
        jh = (jh + 1) & ~1;
    }
    const int lim = min(nkv_w, jm);
    int j = 0;
    // ping-pong: group 1 starts half a tile behind group 0
    if (PP && grp == 1) half_barrier();
    // leading pairs whose next tiles a window's left edge cuts
    for (; j + 1 < jh && j + 2 < nkv_w; j += 2) {
        full_step(I0{}, Mask{}, sa, sb, j);
        full_step(I1{}, Mask{}, sb, sa, j + 1);
    }
    // hot loop: pairs of full steps whose next tiles need no mask (with a
    // bias: the bias alone)
    if constexpr (MODS) {
        if (p.alibi != nullptr) {
            for (; j + 2 < lim; j += 2) {
                full_step(I0{}, BiasOnly{}, sa, sb, j);
                full_step(I1{}, BiasOnly{}, sb, sa, j + 1);
            }
        }
    }
    for (; j + 2 < lim; j += 2) {
        full_step(I0{}, NoMask{}, sa, sb, j);
        full_step(I1{}, NoMask{}, sb, sa, j + 1);
    }
    // the wave's last few full steps, masked (a mask on an interior tile
    // changes nothing); still in pairs so S_j and S_{j+1} keep their registers
    for (; j + 2 < nkv_w; j += 2) {
        full_step(I0{}, Mask{}, sa, sb, j);
        full_step(I1{}, Mask{}, sb, sa, j + 1);
    }
    if (j + 1 < nkv_w) {
        full_step(I0{}, Mask{}, sa, sb, j);
        ++j;
    }
    if (j < nkv_w) {
        if (j & 1) drain_step(sb, j);
        else drain_step(sa, j);
        ++j;
    }
    // tiles past this wave's causal horizon: keep loading for the other waves
    for (; j < nkv; ++j) {
        issue_loads(j, ((j & 1) ? k_lds1 : k_lds0), ((j & 1) ? v_lds0 : v_lds1));
        half_barrier();
        end_iteration();
    }
    // ping-pong: group 0 waits for group 1's last half tile
    if (PP && grp == 0) half_barrier();
    }  // nkv > 0

    // ---- epilogue: O / l, LSE = (m + log2 l) ln 2 ----------------------------
#pragma unroll
    for (int b = 0; b < QB; ++b) {
        const int rowb = wrow0 + 32 * b;
        const float l = xhalf_sum(l_run[b]);
        const float lb = kBf16Norm ? xhalf_sum(lb_run[b]) : l;
        // rows >= n fall outside the buffer and are dropped
        const float inv = lb > 0.0f ? 1.0f / lb : 0.0f;
        if constexpr (SPLIT) {
            // normalised fp32 partial O of this key range, and its LSE
            // ([S, tokens, H, D] and [S, B, H, N], packed [S, H, T])
            const long long tokens = VARLEN ? static_cast<long long>(p.N) : static_cast<long long>(p.B) * p.N;
            const long long sbase = static_cast<long long>(w.split) * tokens * p.H * D + base;
            const auto prs = make_rsrc(p.op + sbase + rowb * rs, (long long)(n - rowb) * rs * 4);
            const int voff_p = c * static_cast<int>(rs) * 4;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int col = db * 32 + g4 * 8 + hh * 4;
                    const f32x4 v4 = {oacc[b][db][g4 * 4 + 0] * inv, oacc[b][db][g4 * 4 + 1] * inv,
                                      oacc[b][db][g4 * 4 + 2] * inv, oacc[b][db][g4 * 4 + 3] * inv};
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v4), prs,
                                                           voff_p + col * 4, 0, 0);
                }
            }
            const int qrow = rowb + c;
            if (qrow < n && hh == 0) {
                const float lse = l > 0.0f ? (m_run[b] + log2f(l)) * kLn2 : -INFINITY;
                long long li;
                if constexpr (VARLEN) {
                    li = (static_cast<long long>(w.split) * p.H + w.h) * p.N + w.t0 + qrow;
                } else {
                    li = (static_cast<long long>(w.split) * p.B * p.H + static_cast<long long>(w.b) * p.H + w.h) *
                             p.N + qrow;
                }
                p.lp[li] = lse;
            }
            continue;
        }
        const auto ors = make_rsrc(p.o + base + rowb * rs, (long long)(n - rowb) * rs * 2);
        const int voff_o = c * static_cast<int>(rs) * 2;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int col = db * 32 + g4 * 8 + hh * 4;
                u32x2 v2 = {pack_bf16x2(oacc[b][db][g4 * 4 + 0] * inv, oacc[b][db][g4 * 4 + 1] * inv),
                            pack_bf16x2(oacc[b][db][g4 * 4 + 2] * inv, oacc[b][db][g4 * 4 + 3] * inv)};
                __builtin_amdgcn_raw_buffer_store_b64(v2, ors, voff_o + col * 2, 0, 0);
            }
        }
        const int qrow = rowb + c;
        if (qrow < n && hh == 0) {
            const float lse = l > 0.0f ? (m_run[b] + log2f(l)) * kLn2 : -INFINITY;
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

template <int D, bool CAUSAL, bool VARLEN, int EXPM>
KernelFn select_rsm(int rsm) {
    constexpr int BC = kTileKeys, NW = Geometry<D>::kWaves, QB = Geometry<D>::kBlocks;
    switch (rsm) {
        case FA_RESCALE_ALWAYS: return fa_fwd_kernel<D, BC, NW, QB, CAUSAL, VARLEN, EXPM, FA_RESCALE_ALWAYS>;
        case FA_RESCALE_STRICT: return fa_fwd_kernel<D, BC, NW, QB, CAUSAL, VARLEN, EXPM, FA_RESCALE_STRICT>;
        default: return fa_fwd_kernel<D, BC, NW, QB, CAUSAL, VARLEN, EXPM, FA_RESCALE_THRESHOLD>;
    }
}

template <int D, bool CAUSAL, bool VARLEN>
KernelFn select_exp(int expm, int rsm) {
    switch (expm) {
        case FA_EXP_HW: return select_rsm<D, CAUSAL, VARLEN, FA_EXP_HW>(rsm);
        case FA_EXP_POLY: return select_rsm<D, CAUSAL, VARLEN, FA_EXP_POLY>(rsm);
        default: return select_rsm<D, CAUSAL, VARLEN, FA_EXP_MIXED>(rsm);
    }
}

template <int D>
KernelFn select_count(bool causal, bool varlen, int rsm) {
    constexpr int BC = kTileKeys, NW = Geometry<D>::kWaves, QB = Geometry<D>::kBlocks;
    constexpr int HW = FA_EXP_HW, ST = FA_RESCALE_STRICT, TH = FA_RESCALE_THRESHOLD;
    if (rsm == FA_RESCALE_STRICT) {
        if (causal) return varlen ? fa_fwd_kernel<D, BC, NW, QB, true, true, HW, ST, false, false, true>
                                  : fa_fwd_kernel<D, BC, NW, QB, true, false, HW, ST, false, false, true>;
        return varlen ? fa_fwd_kernel<D, BC, NW, QB, false, true, HW, ST, false, false, true>
                      : fa_fwd_kernel<D, BC, NW, QB, false, false, HW, ST, false, false, true>;
    }
    if (causal) return varlen ? fa_fwd_kernel<D, BC, NW, QB, true, true, HW, TH, false, false, true>
                              : fa_fwd_kernel<D, BC, NW, QB, true, false, HW, TH, false, false, true>;
    return varlen ? fa_fwd_kernel<D, BC, NW, QB, false, true, HW, TH, false, false, true>
                  : fa_fwd_kernel<D, BC, NW, QB, false, false, HW, TH, false, false, true>;
}

template <int D>
KernelFn select_ping(bool causal, bool varlen) {
    constexpr int BC = kTileKeys, NW = Geometry<D>::kWaves, QB = Geometry<D>::kBlocks;
    constexpr int HW = FA_EXP_HW, ST = FA_RESCALE_STRICT;
    if (causal) return varlen ? fa_fwd_kernel<D, BC, NW, QB, true, true, HW, ST, false, false, false, true>
                              : fa_fwd_kernel<D, BC, NW, QB, true, false, HW, ST, false, false, false, true>;
    return varlen ? fa_fwd_kernel<D, BC, NW, QB, false, true, HW, ST, false, false, false, true>
                  : fa_fwd_kernel<D, BC, NW, QB, false, false, HW, ST, false, false, false, true>;
}

template <int D>
KernelFn select_mods(bool varlen) {
    constexpr int BC = kTileKeys, NW = Geometry<D>::kWaves, QB = Geometry<D>::kBlocks;
    if (varlen) return fa_fwd_kernel<D, BC, NW, QB, false, true, FA_EXP_HW, FA_RESCALE_THRESHOLD, false, true>;
    return fa_fwd_kernel<D, BC, NW, QB, false, false, FA_EXP_HW, FA_RESCALE_THRESHOLD, false, true>;
}

// The default forward (hardware exp2, strict rescale) in four-wave
// workgroups of 128 rows, for shapes whose eight-wave grid would leave
// compute units idle; each wave's rows see the same tiles in the same order,
// so its results are bitwise those of the eight-wave instance.
template <int D>
KernelFn select_quad(bool causal, bool varlen) {
    constexpr int BC = kTileKeys;
    if (causal) return varlen ? fa_fwd_kernel<D, BC, 4, 1, true, true, FA_EXP_HW, FA_RESCALE_STRICT>
                              : fa_fwd_kernel<D, BC, 4, 1, true, false, FA_EXP_HW, FA_RESCALE_STRICT>;
    return varlen ? fa_fwd_kernel<D, BC, 4, 1, false, true, FA_EXP_HW, FA_RESCALE_STRICT>
                  : fa_fwd_kernel<D, BC, 4, 1, false, false, FA_EXP_HW, FA_RESCALE_STRICT>;
}

template <int D>
KernelFn select_split(bool causal, bool varlen) {
    constexpr int BC = kTileKeys, NW = Geometry<D>::kWaves, QB = Geometry<D>::kBlocks;
    if (varlen) {
        if (causal) return fa_fwd_kernel<D, BC, NW, QB, true, true, FA_EXP_HW, FA_RESCALE_THRESHOLD, true>;
        return fa_fwd_kernel<D, BC, NW, QB, false, true, FA_EXP_HW, FA_RESCALE_THRESHOLD, true>;
    }
    if (causal) return fa_fwd_kernel<D, BC, NW, QB, true, false, FA_EXP_HW, FA_RESCALE_THRESHOLD, true>;
    return fa_fwd_kernel<D, BC, NW, QB, false, false, FA_EXP_HW, FA_RESCALE_THRESHOLD, true>;
}

template <int D>
KernelFn select_kernel(bool causal, bool varlen, int expm, int rsm) {
    if (causal) return varlen ? select_exp<D, true, true>(expm, rsm) : select_exp<D, true, false>(expm, rsm);
    return varlen ? select_exp<D, false, true>(expm, rsm) : select_exp<D, false, false>(expm, rsm);
}

}  // namespace fa_detail
