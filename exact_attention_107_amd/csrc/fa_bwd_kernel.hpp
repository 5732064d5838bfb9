// Device code of the exact-attention backward for gfx950, included by one
// translation unit per head dimension (fa_bwd_d*.hip).
//
// The gradients of O = softmax(scale Q K^T) V for an upstream dO, with the
// attention weights recomputed from the forward's log-sum-exp instead of
// being stored (the recomputation of the FlashAttention-1 backward, summary
// table of "FlashAttention 1-4 explained"; section 2.2 of "Understanding
// FlashAttention V4"):
//
//     P  = exp(scale Q K^T - LSE)          (recomputed, never in HBM)
//     dV = P^T dO,   dP = dO V^T,   dS = P * (dP - delta),
//     delta_i = sum_d dO_id O_id,   dQ = scale dS K,   dK = scale dS^T Q.
//
// Three kernels, none with atomics, so every result is bitwise reproducible
// (the deterministic mode of section 3.3 of the V4 explainer):
//  * prep: delta and LSE * log2(e) per query row, stored as a pair at the
//    row's LSE index (dense [B, H, N] or packed [H, T]).
//  * dK/dV: a workgroup owns 128 keys (32 per wave) and walks over the query
//    blocks; dK^T and dV^T accumulate in registers.  S = Q K^T and dP = dO V^T
//    put one key per lane, so P and dS, converted to bf16 in place, are
//    directly the B operands of dV^T += dO^T P and dK^T += Q^T dS (the k
//    order of those products is the register order of the 32x32 accumulator,
//    matched by reading dO and Q transposed from LDS).
//  * dQ: a workgroup owns 128 query rows (32 per wave) and walks over the K/V
//    tiles like the forward: S^T = K Q^T, dP^T = V dO^T, then
//    dQ^T += K^T dS^T with K read transposed.
//
// LDS tiles that are read both by rows (MFMA operands of Q K^T and the like)
// and transposed (ds_read_b64_tr_b16) use one row-major layout whose 16-byte
// chunks are XOR-permuted by sg(r): a row read (16 lanes, 16 rows, one
// chunk) and a transposed read (32 lanes, 4 rows x 4 chunks) both touch 16
// distinct bank groups.
//
// Packed sequences (cu_seqlens, the layout of the packed forward): every
// sequence is its own attention problem; a workgroup's tile is counted from
// its sequence's first token, loads are clipped at the sequence end and the
// masks use the sequence's length.

#pragma once

#include "fa_kernel.hpp"

namespace fa_detail {

constexpr int kBwdWaves = 4;
constexpr int kBwdKeysPerWave = 32;
constexpr int kBwdKeyTile = kBwdWaves * kBwdKeysPerWave;  // keys per dK/dV workgroup
constexpr int kBwdQBlock = 32;                             // query rows per dK/dV step
constexpr int kBwdQTile = kBwdWaves * 32;                  // query rows per dQ workgroup
constexpr int kBwdKvTile = 64;                             // keys per dQ step

// Row-major tile of D-wide bf16 rows with XOR-permuted 16-byte chunks.
template <int D> struct BwdTile {
    static constexpr int RB = D * 2;  // bytes per row
    // Row reads: 16 consecutive rows must give 16 distinct values.  Transposed
    // reads: the 4 rows 4i..4i+3 must differ in the bits above the lowest two
    // (which the 4 chunks of one read span); for D = 64 a 256-byte bank window
    // holds two rows, so row parity already separates half the groups.
    static __device__ __forceinline__ int sg(int r) {
        if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
        else return ((r & 3) << 2) | ((r >> 2) & 3);
    }
};

// Direct global->LDS loads of ROWS rows into a BwdTile: 1 KB per load, the
// workgroup's NW waves take loads wave, wave + NW, ...  Lane l of load I
// fills row r = (1024 I + 16 l) / RB, physical chunk pc, with logical chunk
// pc ^ sg(r); sg depends on r mod 16 only.  A wave's loads are NW * RPB rows
// apart: for D <= 128 a multiple of 16, so one per-lane offset serves them
// all; for D = 256 (two rows per load, eight rows apart) loads of even and
// odd index take two offsets.
template <int D, int ROWS, int NW> struct BwdDma {
    static constexpr int RB = D * 2;
    static constexpr int BLK = ROWS * RB / 1024;
    static constexpr int PER = BLK / NW;
    static constexpr int RPB = 1024 / RB;  // rows per load
    static constexpr int NV = (NW * RPB) % 16 == 0 ? 1 : 2;  // lane offsets per wave
    static_assert(BLK % NW == 0, "tile must split evenly over the waves");
    static_assert((NV * NW * RPB) % 16 == 0, "a wave's loads must take at most two swizzles");
    struct Off {
        int v[NV];
    };
    static __device__ __forceinline__ Off voff(int wave, int lane, int rs_bytes) {
        const int pos = wave * 1024 + lane * 16;
        const int r = pos / RB, pc = (pos % RB) / 16;
        Off o;
#pragma unroll
        for (int i = 0; i < NV; ++i)   // the row offset is the first load's; the swizzle load i's
            o.v[i] = r * rs_bytes + ((pc ^ BwdTile<D>::sg(r + NW * i * RPB)) << 4);
        return o;
    }
    // Rows row0 .. row0 + ROWS - 1 of the tensor at g (row stride rs
    // elements); rows at or past n read as zeros.  Load i covers rows
    // NW i RPB .. further on than the lane offset says, so it gets a resource
    // based at those rows: the size check covers the lane offset only.
    static __device__ __forceinline__ void load(const uint16_t *g, long long rs, int row0, int n, char *tile,
                                                int wave, const Off &vo) {
#pragma unroll
        for (int i = 0; i < PER; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(g, rs, row0 + NW * i * RPB, n),
                                                     LDS_PTR(void, tile + (wave + NW * i) * 1024), 16,
                                                     vo.v[i % NV], 0, 0, 0);
    }
};

// Per-lane byte offsets of the two MFMA operand patterns in a BwdTile,
// kept as two bases plus an XOR term each and completed at every use (one
// or two VALU operations instead of a register per fragment).
//  * Row fragment of k step ks: lane (c, hh) reads row c of a block, chunk
//    (2 ks + hh) ^ sg(c) = (2 ks ^ (sg & ~1)) | ((hh ^ sg) & 1).
//  * Transposed fragment of d block db, half `half`: rows 4 hh + s/4 (+8 for
//    the upper half) of a 16-row k step, columns db*32 + (g&1)*16 + (s&3)*4
//    for lane group g, s = lane % 16: chunk (4 db + x) ^ sg(r) =
//    (4 db ^ (sg & ~3)) | ((x ^ sg) & 3), x = (g&1)*2 + (s&3)/2.
// Any block of rows that starts at a multiple of 16 has the same sg.
template <int D> struct BwdAddr {
    static constexpr int RB = D * 2;
    int rb, rx;          // row fragments: rb | ((ks << 5) ^ rx)
    int tb[2], tx[2];    // transposed fragments: tb[half] | ((db << 6) ^ tx[half])
    __device__ __forceinline__ void init(int lane) {
        const int c = lane & 31, hh = lane >> 5;
        const int sgc = BwdTile<D>::sg(c);
        rb = c * RB | (((hh ^ sgc) & 1) << 4);
        rx = (sgc & ~1) << 4;
        const int g16 = lane >> 4, s16 = lane & 15;
        const int x = (g16 & 1) * 2 + ((s16 & 3) >> 1);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int r = hh * 4 + (s16 >> 2) + 8 * half;
            const int sgr = BwdTile<D>::sg(r);
            tb[half] = r * RB + (s16 & 1) * 8 + (((x ^ sgr) & 3) << 4);
            tx[half] = (sgr & ~3) << 4;
        }
    }
    // Redefines the bases inside a loop so that the compiler does not hoist
    // every per-fragment address out of it (one register each).
    __device__ __forceinline__ void refresh() {
        asm volatile("" : "+v"(rb), "+v"(rx), "+v"(tb[0]), "+v"(tb[1]), "+v"(tx[0]), "+v"(tx[1]));
    }
    __device__ __forceinline__ int row(int ks) const { return rb | ((ks << 5) ^ rx); }
    __device__ __forceinline__ int tr(int db, int half) const { return tb[half] | ((db << 6) ^ tx[half]); }
};

__device__ __forceinline__ bf16x8 lds_row(const char *tile, int off) {
    return *reinterpret_cast<const bf16x8 *>(tile + off);
}

// Transposed fragment (two ds_read_b64_tr_b16) at tile + off_lo / off_hi +
// OFF; the caller waits with lgkm_wait.
template <int OFF>
__device__ __forceinline__ bf16x8 lds_tr(const char *tile, int off_lo, int off_hi) {
    const uint32_t a = lds_offset(tile);
    const u32x2 lo = ds_read_tr16<OFF>(a + off_lo);
    const u32x2 hi = ds_read_tr16<OFF>(a + off_hi);
    const u32x4 both = {lo[0], lo[1], hi[0], hi[1]};
    return __builtin_bit_cast(bf16x8, both);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------------------
// prep: delta_i = sum_d dO_id O_id and LSE_i * log2(e), one thread per LSE
// entry t, stored as the pair stats[2 t], stats[2 t + 1].

template <int D>
__global__ void __launch_bounds__(256) fa_bwd_prep_kernel(BwdParams p) {
    const long long t = static_cast<long long>(blockIdx.x) * 256 + threadIdx.x;
    const long long rows = static_cast<long long>(p.cu ? 1 : p.B) * p.H * p.N;
    if (t >= rows) return;
    // token and head of LSE entry t: packed [H, T], dense [B, H, N]
    long long tok;
    int h;
    if (p.cu) {
        h = static_cast<int>(t / p.N);
        tok = t - static_cast<long long>(h) * p.N;
    } else {
        const long long bh = t / p.N;
        const int b = static_cast<int>(bh / p.H);
        h = static_cast<int>(bh - static_cast<long long>(b) * p.H);
        tok = static_cast<long long>(b) * p.N + (t - bh * p.N);
    }
    const long long base = (tok * p.H + h) * D;
    const u32x4 *dq = reinterpret_cast<const u32x4 *>(p.dout + base);
    const u32x4 *oq = reinterpret_cast<const u32x4 *>(p.o + base);
    float acc = 0.0f;
#pragma unroll
    for (int cch = 0; cch < D / 8; ++cch) {
        const u32x4 a = dq[cch], o = oq[cch];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            acc = __builtin_fmaf(bf16_lo(a[w]), bf16_lo(o[w]), acc);
            acc = __builtin_fmaf(bf16_hi(a[w]), bf16_hi(o[w]), acc);
        }
    }
    const u32x2 st = {__float_as_uint(p.lse[t] * kLog2e), __float_as_uint(acc)};
    *reinterpret_cast<u32x2 *>(p.stats + 2 * t) = st;
}

// ---------------------------------------------------------------------------
// Work items: head h and tile `tile` (of TILE keys or rows, counted from the
// first token of the sequence) of one sequence of length n starting at token
// t0; lrow is the LSE index of the sequence's first row for head h.

struct BwdItem {
    int h, tile, n;
    long long t0, lrow;
};

// Packed sequences: items are ordered by sequence and, within it, by tile,
// with the head varying fastest (the tiles of one sequence and head run at
// about the same time, on one XCD).  Up to 64 sequences the longest go
// first; beyond that they keep their order.  HIGH_FIRST numbers a
// sequence's tiles from its end.  Returns false for a surplus workgroup of
// the grid bound H * (ceil(T / TILE) + B).
template <int TILE, bool HIGH_FIRST>
__device__ __forceinline__ bool bwd_packed_item(const BwdParams &p, BwdItem &it) {
    const int lane = threadIdx.x & 63;
    const int r = static_cast<int>(blockIdx.x) / p.H;
    it.h = static_cast<int>(blockIdx.x) - r * p.H;
    int sel = -1, local = 0, tiles_sel = 0;
    if (p.B <= 64) {
        // lane b: where sequence b's tiles start when longer sequences (ties:
        // lower index) come first
        const int b = lane;
        const int len = b < p.B ? seq_len(p.cu, b, p.N) : 0;
        const int tiles = (len + TILE - 1) / TILE;
        int pos = 0;
        for (int o = 0; o < p.B; ++o) {
            const int lo = seq_len(p.cu, o, p.N);
            pos += (lo > len || (lo == len && o < b)) ? (lo + TILE - 1) / TILE : 0;
        }
        const unsigned long long m = __ballot(b < p.B && r >= pos && r < pos + tiles);
        if (m == 0) return false;
        sel = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(m)) - 1);
        local = r - __builtin_amdgcn_readfirstlane(__shfl(pos, sel));
        tiles_sel = __builtin_amdgcn_readfirstlane(__shfl(tiles, sel));
    } else {
        int pos = 0;  // tiles of the sequences before this chunk of 64
        for (int c0 = 0; c0 < p.B; c0 += 64) {
            const int b = c0 + lane;
            const int tiles = b < p.B ? (seq_len(p.cu, b, p.N) + TILE - 1) / TILE : 0;
            int incl = tiles;  // inclusive prefix sum over the lanes
            for (int off = 1; off < 64; off <<= 1) {
                const int x = __shfl_up(incl, off);
                if (lane >= off) incl += x;
            }
            const int total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
            if (r < pos + total) {
                const unsigned long long m = __ballot(r >= pos + incl - tiles && r < pos + incl);
                const int l = __builtin_amdgcn_readfirstlane(__ffsll(static_cast<long long>(m)) - 1);
                sel = c0 + l;
                local = r - pos - __builtin_amdgcn_readfirstlane(__shfl(incl - tiles, l));
                tiles_sel = __builtin_amdgcn_readfirstlane(__shfl(tiles, l));
                break;
            }
            pos += total;
        }
        if (sel < 0) return false;
    }
    it.tile = HIGH_FIRST ? tiles_sel - 1 - local : local;
    int s0, s1;
    seq_span(p.cu, sel, p.N, s0, s1);
    s0 = __builtin_amdgcn_readfirstlane(s0);
    s1 = __builtin_amdgcn_readfirstlane(s1);
    it.t0 = s0;
    it.n = s1 - s0;
    it.lrow = static_cast<long long>(it.h) * p.N + s0;
    return true;
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = (b, h, key tile of 128 keys).

template <int D, bool CAUSAL, bool PACKED>
__global__ void __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2)))
fa_bwd_dkdv_kernel(BwdParams p) {
    constexpr int NW = kBwdWaves, KW = kBwdKeysPerWave, BK = kBwdKeyTile, BQ = kBwdQBlock;
    constexpr int KK = D / 16, NDB = D / 32, RB = D * 2;
    constexpr int QT = BQ * RB;   // bytes of a Q or dO block
    constexpr int VT = BK * RB;   // bytes of the V tile
    using QDMA = BwdDma<D, BQ, NW>;
    using VDMA = BwdDma<D, BK, NW>;

    __shared__ __attribute__((aligned(1024))) char q_lds0[QT], q_lds1[QT], do_lds0[QT], do_lds1[QT];
    __shared__ __attribute__((aligned(1024))) char v_lds[VT];
    __shared__ __attribute__((aligned(256))) float st_lds0[64], st_lds1[64];

    BwdItem it;
    if constexpr (PACKED) {
        // causal: a sequence's low key tiles see the most query blocks
        if (!bwd_packed_item<BK, false>(p, it)) return;
    } else {
        const int BH = p.B * p.H;
        const int n_kt = (p.N + BK - 1) / BK;
        int bh, kt;
        if constexpr (CAUSAL) {
            // low key tiles see the most query blocks: they go first
            kt = blockIdx.x / BH;
            bh = blockIdx.x - kt * BH;
        } else {
            // each XCD (blockIdx % 8) takes a contiguous run of items, so the key
            // tiles of one (b, h) share that XCD's L2 for their Q and dO stream
            const int G = gridDim.x, x = blockIdx.x & 7, sx = blockIdx.x >> 3;
            const int per = G >> 3, rem = G & 7;
            const int item = x * per + (x < rem ? x : rem) + sx;
            bh = item / n_kt;
            kt = item - bh * n_kt;
        }
        const int b = bh / p.H;
        it.h = bh - b * p.H;
        it.tile = kt;
        it.n = p.N;
        it.t0 = static_cast<long long>(b) * p.N;
        it.lrow = static_cast<long long>(bh) * p.N;
    }
    const int n = it.n, kt = it.tile, h = it.h;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, hh = lane >> 5;
    const int j0 = kt * BK;
    const int kw0 = j0 + wave * KW;  // this wave's first key
    const long long rs = static_cast<long long>(p.H) * D;
    const int rs_bytes = static_cast<int>(rs) * 2;
    const long long base = (it.t0 * p.H + h) * D;  // token 0 of the sequence, head h

    // K of this wave's keys, B operand of S = Q K^T: lane (c, hh) holds
    // K[kw0 + c][16 ks + 8 hh .. +8]; keys >= n read as zeros.
    bf16x8 kf[KK];
    {
        const auto krs = make_rsrc(p.k + base + kw0 * rs, (long long)(n - kw0) * rs_bytes);
        const int vo = (c * static_cast<int>(rs) + hh * 8) * 2;
#pragma unroll
        for (int ks = 0; ks < KK; ++ks)
            kf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, vo + ks * 32, 0, 0));
    }

    BwdAddr<D> ad;
    ad.init(lane);
    const auto qvoff = QDMA::voff(wave, lane, rs_bytes);
    const auto vvoff = VDMA::voff(wave, lane, rs_bytes);
    // (LSE*log2e, delta) pairs of the sequence's rows; lane l < 32 fetches
    // row l's LSE, lane 32 + l its delta: st_lds = [32 x LSE*log2e | 32 x delta]
    const float *stats_seq = p.stats + 2 * it.lrow;
    const int st_off = lane < 32 ? lane * 8 : (lane - 32) * 8 + 4;

    // query blocks: causal starts at the tile's first key
    const int qb0 = CAUSAL ? j0 / BQ : 0;
    const int nqb = (n + BQ - 1) / BQ;
    auto dma_block = [&](int qb, char *qd, char *dd, float *sd) __attribute__((always_inline)) {
        const int q0 = qb * BQ;
        QDMA::load(p.q + base, rs, q0, n, qd, wave, qvoff);
        QDMA::load(p.dout + base, rs, q0, n, dd, wave, qvoff);
        if (wave == 0) {
            // rows past the sequence read (0, 0); the mask gives them P = 0
            const auto srs = make_rsrc(stats_seq + 2 * q0, (long long)(n - q0) * 8);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, LDS_PTR(void, sd), 4, st_off, 0, 0, 0);
        }
    };
    VDMA::load(p.v + base, rs, j0, n, v_lds, wave, vvoff);
    if (qb0 < nqb) dma_block(qb0, q_lds0, do_lds0, st_lds0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) {
        dkacc[i] = f32x16{};
        dvacc[i] = f32x16{};
    }
    const float cs = p.cs;
    const bool key_tail = kw0 + KW > n;
    const int vrow = wave * KW * RB;  // this wave's rows of the V tile

    // One query block: q0 = first row; MASK: causal diagonal or key tail.
    auto block = [&](const char *qb_lds, const char *db_lds, const float *st, int q0, bool need_mask) __attribute__((always_inline)) {
        ad.refresh();
        // S = Q K^T and dP = dO V^T; the fragments of step ks + 1 are read
        // while step ks multiplies (the scheduling barriers keep the compiler
        // from hoisting every read of the block and running out of registers)
        f32x16 s = f32x16{}, dp = f32x16{};
        bf16x8 qa[2], da[2], vb[2];
        qa[0] = lds_row(qb_lds, ad.row(0));
        da[0] = lds_row(db_lds, ad.row(0));
        vb[0] = lds_row(v_lds + vrow, ad.row(0));
        static_for<0, KK>([&](auto ks_) {
            constexpr int ks = decltype(ks_)::value, cur = ks & 1, nxt = cur ^ 1;
            if constexpr (ks + 1 < KK) {
                qa[nxt] = lds_row(qb_lds, ad.row(ks + 1));
                da[nxt] = lds_row(db_lds, ad.row(ks + 1));
                vb[nxt] = lds_row(v_lds + vrow, ad.row(ks + 1));
            }
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[cur], kf[ks], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[cur], vb[cur], dp, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
        // lane (c, hh), register 4 g + r: key kw0 + c, query q0 + 8 g + 4 hh + r
        bf16x8 pf[2], sf[2];
        auto elementwise = [&](auto mask_) __attribute__((always_inline)) {
            constexpr bool MASK = decltype(mask_)::value;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint32_t pk[4], sk[4];
#pragma unroll
                for (int gg = 0; gg < 2; ++gg) {
                    const int g = 2 * t + gg;
                    const f32x4 l4 = *reinterpret_cast<const f32x4 *>(st + 8 * g + 4 * hh);
                    const f32x4 d4 = *reinterpret_cast<const f32x4 *>(st + 32 + 8 * g + 4 * hh);
                    float pv[4], sv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int e = 4 * g + r;
                        float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], cs, -l4[r]));
                        if constexpr (MASK) {
                            const int key = kw0 + c, qry = q0 + 8 * g + 4 * hh + r;
                            // (query rows past the sequence: P = 0 whatever the
                            // tile's rows past it hold)
                            const bool off = key >= n || qry >= n || (CAUSAL && key > qry);
                            pe = off ? 0.0f : pe;
                        }
                        pv[r] = pe;
                        sv[r] = pe * (dp[e] - d4[r]);
                    }
                    pk[2 * gg] = pack_bf16x2(pv[0], pv[1]);
                    pk[2 * gg + 1] = pack_bf16x2(pv[2], pv[3]);
                    sk[2 * gg] = pack_bf16x2(sv[0], sv[1]);
                    sk[2 * gg + 1] = pack_bf16x2(sv[2], sv[3]);
                }
                const u32x4 pu = {pk[0], pk[1], pk[2], pk[3]};
                const u32x4 su = {sk[0], sk[1], sk[2], sk[3]};
                pf[t] = __builtin_bit_cast(bf16x8, pu);
                sf[t] = __builtin_bit_cast(bf16x8, su);
            }
        };
        if (need_mask) elementwise(std::true_type{});
        else elementwise(std::false_type{});
        __builtin_amdgcn_sched_barrier(0);
        // dV^T += dO^T P, dK^T += Q^T dS (dO, Q read transposed); step m =
        // (d block m / 2, k step m % 2), fragments read one step ahead
        constexpr int MS = 2 * NDB;
        bf16x8 ta[2], tq[2];
        ta[0] = lds_tr<0>(db_lds, ad.tr(0, 0), ad.tr(0, 1));
        tq[0] = lds_tr<0>(qb_lds, ad.tr(0, 0), ad.tr(0, 1));
        static_for<0, MS>([&](auto m_) {
            constexpr int m = decltype(m_)::value, db = m / 2, t = m % 2, cur = m & 1, nxt = cur ^ 1;
            if constexpr (m + 1 < MS) {
                constexpr int db1 = (m + 1) / 2, t1 = (m + 1) % 2;
                ta[nxt] = lds_tr<t1 * 16 * RB>(db_lds, ad.tr(db1, 0), ad.tr(db1, 1));
                tq[nxt] = lds_tr<t1 * 16 * RB>(qb_lds, ad.tr(db1, 0), ad.tr(db1, 1));
                lgkm_wait<4>(ta[cur]);
                lgkm_wait<4>(tq[cur]);
            } else {
                lgkm_wait<0>(ta[cur]);
                lgkm_wait<0>(tq[cur]);
            }
            dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[cur], pf[t], dvacc[db], 0, 0, 0);
            dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[cur], sf[t], dkacc[db], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // one query block; PAR selects the LDS buffers statically
    auto step = [&](auto par_, int qb) __attribute__((always_inline)) {
        constexpr int PAR = decltype(par_)::value;
        char *qcur = PAR ? q_lds1 : q_lds0;
        char *dcur = PAR ? do_lds1 : do_lds0;
        float *scur = PAR ? st_lds1 : st_lds0;
        if (qb + 1 < nqb) dma_block(qb + 1, PAR ? q_lds0 : q_lds1, PAR ? do_lds0 : do_lds1, PAR ? st_lds0 : st_lds1);
        const int q0 = qb * BQ;
        // causal: queries q0 .. q0+31 all precede this wave's keys -> nothing
        // to add.  Only D = 64 skips such a block; for D = 128 and 256 it runs
        // fully masked (P = dS = 0 add exact zeros; the first `wave` blocks of
        // waves 1..3, about 1 % of a long causal run's blocks): branching round
        // it makes the compiler spill the accumulators (d = 128: 136 VGPRs,
        // 3.7 times slower)
        if (!CAUSAL || D != 64 || q0 + BQ - 1 >= kw0) {
            block(qcur, dcur, scur, q0, key_tail || q0 + BQ > n || (CAUSAL && q0 < kw0 + KW));
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    int qb = qb0;
    for (; qb + 1 < nqb; qb += 2) {
        step(std::integral_constant<int, 0>{}, qb);
        step(std::integral_constant<int, 1>{}, qb + 1);
    }
    if (qb < nqb) step(std::integral_constant<int, 0>{}, qb);

    // epilogue: lane (c, hh) register 4 g + r of block db holds column
    // d = db*32 + 8 g + 4 hh + r of key kw0 + c; keys >= n are dropped
    const auto krs_out = make_rsrc(p.dk + base + kw0 * rs, (long long)(n - kw0) * rs_bytes);
    const auto vrs_out = make_rsrc(p.dv + base + kw0 * rs, (long long)(n - kw0) * rs_bytes);
    const int vo = c * rs_bytes;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int col = db * 32 + g * 8 + hh * 4;
            const u32x2 kv = {pack_bf16x2(dkacc[db][4 * g] * sc, dkacc[db][4 * g + 1] * sc),
                              pack_bf16x2(dkacc[db][4 * g + 2] * sc, dkacc[db][4 * g + 3] * sc)};
            const u32x2 vv = {pack_bf16x2(dvacc[db][4 * g], dvacc[db][4 * g + 1]),
                              pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3])};
            __builtin_amdgcn_raw_buffer_store_b64(kv, krs_out, vo + col * 2, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b64(vv, vrs_out, vo + col * 2, 0, 0);
        }
    }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = (b, h, query tile of 128 rows), like the forward.

template <int D, bool CAUSAL, bool PACKED>
__global__ void __launch_bounds__(kBwdWaves * 64) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2)))
fa_bwd_dq_kernel(BwdParams p) {
    constexpr int NW = kBwdWaves, BR = kBwdQTile, BC = kBwdKvTile;
    constexpr int KK = D / 16, NDB = D / 32, RB = D * 2, NKB = BC / 32;
    constexpr int TT = BC * RB;  // bytes of a K or V tile
    using KDMA = BwdDma<D, BC, NW>;

    __shared__ __attribute__((aligned(1024))) char k_lds0[TT], k_lds1[TT], v_lds0[TT], v_lds1[TT];

    BwdItem it;
    if constexpr (PACKED) {
        // causal: a sequence's high query tiles see the most keys
        if (!bwd_packed_item<BR, CAUSAL>(p, it)) return;
    } else {
        const int BH = p.B * p.H;
        const int n_qt = (p.N + BR - 1) / BR;
        int bh, qt;
        if constexpr (CAUSAL) {
            qt = n_qt - 1 - static_cast<int>(blockIdx.x) / BH;  // longest first
            bh = blockIdx.x - (n_qt - 1 - qt) * BH;
        } else {
            const int G = gridDim.x, x = blockIdx.x & 7, sx = blockIdx.x >> 3;
            const int per = G >> 3, rem = G & 7;
            const int item = x * per + (x < rem ? x : rem) + sx;
            bh = item / n_qt;
            qt = item - bh * n_qt;
        }
        const int b = bh / p.H;
        it.h = bh - b * p.H;
        it.tile = qt;
        it.n = p.N;
        it.t0 = static_cast<long long>(b) * p.N;
        it.lrow = static_cast<long long>(bh) * p.N;
    }
    const int n = it.n, qt = it.tile, h = it.h;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane & 31, hh = lane >> 5;
    const int q0 = qt * BR;
    const int wrow0 = q0 + wave * 32;
    const long long rs = static_cast<long long>(p.H) * D;
    const int rs_bytes = static_cast<int>(rs) * 2;
    const long long base = (it.t0 * p.H + h) * D;

    // Q and dO of this wave's rows, B operands of S^T = K Q^T, dP^T = V dO^T
    bf16x8 qf[KK], df[KK];
    {
        const auto qrs = make_rsrc(p.q + base + wrow0 * rs, (long long)(n - wrow0) * rs_bytes);
        const auto drs = make_rsrc(p.dout + base + wrow0 * rs, (long long)(n - wrow0) * rs_bytes);
        const int vo = (c * static_cast<int>(rs) + hh * 8) * 2;
#pragma unroll
        for (int ks = 0; ks < KK; ++ks) {
            qf[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(qrs, vo + ks * 32, 0, 0));
            df[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(drs, vo + ks * 32, 0, 0));
        }
    }
    // this lane's query row: LSE * log2(e) and delta; rows past n take +inf
    // and 0, so their P = 0
    const bool row_ok = wrow0 + c < n;
    const float *st = p.stats + 2 * (it.lrow + (row_ok ? wrow0 + c : 0));
    const float lse2 = row_ok ? st[0] : INFINITY;
    const float delta = row_ok ? st[1] : 0.0f;

    BwdAddr<D> ad;
    ad.init(lane);
    const auto kvoff = KDMA::voff(wave, lane, rs_bytes);
    const int kv_end = CAUSAL ? min(n, q0 + BR) : n;
    const int nkv = (kv_end + BC - 1) / BC;
    const int nkv_w = CAUSAL ? min(nkv, (wrow0 + 31) / BC + 1) : nkv;

    auto dma_tile = [&](int j, char *kd, char *vd) __attribute__((always_inline)) {
        const int kv0 = j * BC;
        KDMA::load(p.k + base, rs, kv0, n, kd, wave, kvoff);
        KDMA::load(p.v + base, rs, kv0, n, vd, wave, kvoff);
    };
    dma_tile(0, k_lds0, v_lds0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x16 dqacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dqacc[i] = f32x16{};
    const float cs = p.cs;

    auto tile = [&](const char *kb, const char *vb, int j, auto mask_) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_)::value;
        ad.refresh();
        const int kv0 = j * BC;
        bf16x8 sf[2 * NKB];
#pragma unroll
        for (int kb2 = 0; kb2 < NKB; ++kb2) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KK; ++ks) {
                const bf16x8 ka = lds_row(kb + kb2 * 32 * RB, ad.row(ks));
                const bf16x8 va = lds_row(vb + kb2 * 32 * RB, ad.row(ks));
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, df[ks], dp, 0, 0, 0);
            }
            // lane (c, hh), register 4 g + r: query wrow0 + c, key
            // kv0 + kb2*32 + 8 g + 4 hh + r
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                uint32_t sk[4];
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    float v2[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int e = 8 * t + i + u;
                        float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[e], cs, -lse2));
                        if constexpr (MASK) {
                            const int key = kv0 + kb2 * 32 + 8 * (e >> 2) + 4 * hh + (e & 3);
                            const bool off = key >= n || (CAUSAL && key > wrow0 + c);
                            pe = off ? 0.0f : pe;
                        }
                        v2[u] = pe * (dp[e] - delta);
                    }
                    sk[i >> 1] = pack_bf16x2(v2[0], v2[1]);
                }
                const u32x4 su = {sk[0], sk[1], sk[2], sk[3]};
                sf[2 * kb2 + t] = __builtin_bit_cast(bf16x8, su);
            }
        }
        // dQ^T += K^T dS^T (K read transposed): step m = (d block m / T16, k
        // step m % T16 of 16 keys); the next step's fragment is read while
        // this one multiplies (two reads in flight at the wait)
        constexpr int T16 = 2 * NKB, MS = NDB * T16;
        bf16x8 kt[2];
        kt[0] = lds_tr<0>(kb, ad.tr(0, 0), ad.tr(0, 1));
        static_for<0, MS>([&](auto m_) {
            constexpr int m = decltype(m_)::value, db = m / T16, t16 = m % T16, cur = m & 1;
            if constexpr (m + 1 < MS) {
                constexpr int db1 = (m + 1) / T16, t1 = (m + 1) % T16;
                kt[cur ^ 1] = lds_tr<t1 * 16 * RB>(kb, ad.tr(db1, 0), ad.tr(db1, 1));
                lgkm_wait<2>(kt[cur]);
            } else {
                lgkm_wait<0>(kt[cur]);
            }
            dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[cur], sf[t16], dqacc[db], 0, 0, 0);
        });
    };

    using Yes = std::integral_constant<bool, true>;
    using No = std::integral_constant<bool, false>;
    for (int j = 0; j < nkv; ++j) {
        const int par = j & 1;
        char *kcur = par ? k_lds1 : k_lds0;
        char *vcur = par ? v_lds1 : v_lds0;
        if (j + 1 < nkv) dma_tile(j + 1, par ? k_lds0 : k_lds1, par ? v_lds0 : v_lds1);
        if (j < nkv_w) {
            const int kv0 = j * BC;
            const bool need_mask = (CAUSAL && kv0 + BC - 1 > wrow0) || kv0 + BC > n;
            if (need_mask) tile(kcur, vcur, j, Yes{});
            else tile(kcur, vcur, j, No{});
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    }

    // epilogue: lane (c, hh) register 4 g + r of block db holds column
    // db*32 + 8 g + 4 hh + r of query wrow0 + c; rows >= n are dropped
    const auto ors = make_rsrc(p.dq + base + wrow0 * rs, (long long)(n - wrow0) * rs_bytes);
    const int vo = c * rs_bytes;
    const float sc = p.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int col = db * 32 + g * 8 + hh * 4;
            const u32x2 v2 = {pack_bf16x2(dqacc[db][4 * g] * sc, dqacc[db][4 * g + 1] * sc),
                              pack_bf16x2(dqacc[db][4 * g + 2] * sc, dqacc[db][4 * g + 3] * sc)};
            __builtin_amdgcn_raw_buffer_store_b64(v2, ors, vo + col * 2, 0, 0);
        }
    }
}

template <int D>
BwdKernels select_bwd(bool causal, bool packed) {
    if (packed) {
        if (causal) return {fa_bwd_prep_kernel<D>, fa_bwd_dkdv_kernel<D, true, true>, fa_bwd_dq_kernel<D, true, true>};
        return {fa_bwd_prep_kernel<D>, fa_bwd_dkdv_kernel<D, false, true>, fa_bwd_dq_kernel<D, false, true>};
    }
    if (causal) return {fa_bwd_prep_kernel<D>, fa_bwd_dkdv_kernel<D, true, false>, fa_bwd_dq_kernel<D, true, false>};
    return {fa_bwd_prep_kernel<D>, fa_bwd_dkdv_kernel<D, false, false>, fa_bwd_dq_kernel<D, false, false>};
}

}  // namespace fa_detail
