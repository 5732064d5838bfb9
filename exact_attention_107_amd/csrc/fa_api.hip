// C ABI of libfa.so: argument validation, kernel selection and launch of the
// fused exact-attention forward (declarations and contract in include/fa.h).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_internal.h"

using namespace fa_detail;

// Scratch of fa_fwd_splitkv_static (the split partials: o_part, then
// lse_part).  Every GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` is only a stand-in for the symbol:
// its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) char scratch[FA_STATIC_SCRATCH_BYTES];

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

// The kernels address up to 64 rows of one tile with 32-bit byte offsets of
// fp32 data: H * d * 4 * 64 must stay below 2^31.
bool token_stride_ok(int H, int d) { return static_cast<long long>(H) * d <= (1LL << 22); }

int key_tiles(int N) { return (N + kTileKeys - 1) / kTileKeys; }

// Longest sequence of the window-mask forward: row + window edge (each below
// N after clamping) plus a tile must fit in an int.
constexpr int kMaskedMaxN = 1 << 30;

// Device address of the current GPU's scratch array, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_for_current_device(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FA_OK;
}

// Compute units of the current GPU, asked once per device and kept (0 when
// HIP cannot say).  Only the choice of workgroup shape depends on it.
std::atomic<int> g_cus[kMaxDevices];

int cus_of_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int n = g_cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 0)
            n = 0;
        g_cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Rows per workgroup of the default forward.  At d = 128 an eight-wave
// workgroup (256 rows) is the fastest shape once the grid covers the GPU
// several times over; four-wave workgroups (128 rows, two resident per
// compute unit) win when the eight-wave grid would leave compute units idle
// or end in a short last round: a non-causal grid of at most half a workgroup
// per compute unit, or of one to three rounds whose last round is at most
// half full; a causal grid of at most one and a half per compute unit, whose
// tiles of unequal length the finer grid balances.
int default_rows(int B, int H, int N, int d, bool causal, bool packed, int num_cus) {
    if (d != 128) return tile_rows_for(d);
    const long long cus = num_cus > 0 ? num_cus : 256;
    const long long items = (packed ? 1LL : static_cast<long long>(B)) * H * ((N + 255LL) / 256);
    bool four;
    if (causal) {
        four = 2 * items <= 3 * cus;
    } else {
        const long long last = items % cus;  // workgroups of the last round
        four = 2 * items <= cus || (items > cus && items < 3 * cus && last > 0 && 2 * last <= cus);
    }
    return four ? 128 : 256;
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
        case FA_ERR_SPLIT: return "num_splits out of range (1 .. ceil(N / tile keys))";
        case FA_ERR_SCRATCH: return "the split partials exceed the static scratch (FA_STATIC_SCRATCH_BYTES)";
        default: return "unknown fa status code";
    }
}

int fa_tile_rows(int d) { return tile_rows_for(d); }

int fa_tile_keys(int d) { return (d == 64 || d == 128 || d == 256) ? kTileKeys : 0; }

int fa_fwd_tile_rows(int B, int H, int N, int d, int causal, int packed, int num_cus) {
    if (tile_rows_for(d) == 0) return 0;
    if (B < 1 || H < 1 || N < 1) return tile_rows_for(d);
    return default_rows(B, H, N, d, causal != 0, packed != 0, num_cus);
}

// Validation and launch of the forward; `counts` selects the counting
// instance (d = 128, hardware exp2) and receives its statistics; `adapt`
// lets the shape of the grid choose the workgroup shape (fa_fwd).
static int fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                    int N, int d, float scale, int causal, const int32_t *cu_seqlens,
                    hipStream_t stream, int exp_mode, int rescale_mode, unsigned long long *counts,
                    bool ping = false, bool adapt = false) {
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
    if (elems <= 0 || elems > (1LL << 46) || !token_stride_ok(H, d)) return FA_ERR_SHAPE;
    const size_t tensor_bytes = static_cast<size_t>(elems) * 2;
    const size_t lse_bytes = static_cast<size_t>(tokens * H) * 4;
    if (overlap(o, tensor_bytes, q, tensor_bytes) || overlap(o, tensor_bytes, k, tensor_bytes) ||
        overlap(o, tensor_bytes, v, tensor_bytes) || overlap(lse, lse_bytes, q, tensor_bytes) ||
        overlap(lse, lse_bytes, k, tensor_bytes) || overlap(lse, lse_bytes, v, tensor_bytes) ||
        overlap(lse, lse_bytes, o, tensor_bytes))
        return FA_ERR_ALIAS;

    Params prm{};
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
    // fa_fwd picks its workgroup shape for the grid; fa_fwd_variant (the
    // default instance included), the counting and the ping-pong instances
    // keep theirs
    const bool plain = adapt && !counts && !ping && exp_mode == FA_EXP_HW && rescale_mode == FA_RESCALE_STRICT;
    const int rows = plain ? default_rows(B, H, N, d, causal != 0, varlen, cus_of_current_device())
                           : tile_rows_for(d);
    const bool quad = d == 128 && rows == 128;
    const long long n_qt = (static_cast<long long>(N) + rows - 1) / rows;
    prm.n_qt = static_cast<int>(n_qt);
    long long grid;
    if (varlen) {
        grid = static_cast<long long>(H) * (n_qt + B);  // bound on sum_b ceil(n_b / rows)
    } else {
        grid = static_cast<long long>(B) * H * n_qt;
    }
    if (grid <= 0 || grid > 0x7fffffffLL) return FA_ERR_SHAPE;

    prm.counts = counts;
    KernelFn fn = counts ? select_count_d128(causal != 0, varlen, rescale_mode)
                  : ping ? select_ping_d128(causal != 0, varlen)
                  : quad ? select_quad_d128(causal != 0, varlen)
                         : pick(d, causal != 0, varlen, exp_mode, rescale_mode);
    const int threads = (quad ? 4 : waves_for(d)) * 64;
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(grid)), dim3(threads), 0, stream, prm);
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    return FA_OK;
}

int fa_split_range(int N, int d, int causal, int num_splits, int s, int row, int *key_lo, int *key_hi) {
    if (!key_lo || !key_hi) return FA_ERR_NULLPTR;
    if (N < 1 || row < 0 || row >= N) return FA_ERR_SHAPE;
    if (tile_rows_for(d) == 0) return FA_ERR_HEAD_DIM;
    if (num_splits < 1 || num_splits > key_tiles(N) || s < 0 || s >= num_splits) return FA_ERR_SPLIT;
    // keys the row's query tile sees: all, or up to the tile's last row
    const long long rows = tile_rows_for(d);
    const long long q_end = (row / rows + 1) * rows;
    const long long seen = causal ? (q_end < N ? q_end : N) : N;
    const long long t = (seen + kTileKeys - 1) / kTileKeys;
    const long long lo = s * t / num_splits * kTileKeys, hi = (s + 1) * t / num_splits * kTileKeys;
    *key_lo = static_cast<int>(lo);
    *key_hi = static_cast<int>(hi < seen ? hi : seen);
    return FA_OK;
}

int fa_num_splits(int B, int H, int N, int d, int causal, int num_cus) {
    if (B < 1 || H < 1 || N < 1 || tile_rows_for(d) == 0) return 1;
    const long long cus = num_cus > 0 ? num_cus : 256;
    // workgroups resident per compute unit (registers): 3, 1, 1 at d = 64,
    // 128, 256
    const long long slots = static_cast<long long>(resident_for(d)) * cus;
    const long long n_qt = (static_cast<long long>(N) + tile_rows_for(d) - 1) / tile_rows_for(d);
    // causal: the average query tile sees half the keys
    const long long wgs = static_cast<long long>(B) * H * n_qt / (causal ? 2 : 1);
    if (wgs >= slots) return 1;
    // with one workgroup per compute unit already, splitting pays only when
    // each range stays long next to the partials it writes
    if (wgs >= cus && N < 8192) return 1;
    long long s = (slots + wgs - 1) / (wgs > 0 ? wgs : 1);
    const long long cap = key_tiles(N) / 16 > 1 ? key_tiles(N) / 16 : 1;  // >= 1024 keys a range
    if (s > cap) s = cap;
    if (s > 32) s = 32;
    return static_cast<int>(s < 1 ? 1 : s);
}

int fa_merge(const float *o_part, const float *lse_part, int num_splits, int B, int H, int N, int d,
             void *o, float *lse, hipStream_t stream) {
    if (!o_part || !lse_part || !o || !lse) return FA_ERR_NULLPTR;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && d != 256) return FA_ERR_HEAD_DIM;
    if (num_splits < 1) return FA_ERR_SPLIT;
    if (misaligned(o_part, 16) || misaligned(o, 16) || misaligned(lse_part, 4) || misaligned(lse, 4))
        return FA_ERR_ALIGN;
    const long long rows = static_cast<long long>(B) * N * H;
    const long long elems = rows * d;
    if (elems <= 0 || elems > (1LL << 46) || elems * num_splits > (1LL << 46)) return FA_ERR_SHAPE;
    const size_t ob = static_cast<size_t>(elems) * 2, lb = static_cast<size_t>(rows) * 4;
    const size_t opb = static_cast<size_t>(elems) * num_splits * 4, lpb = static_cast<size_t>(rows) * num_splits * 4;
    if (overlap(o, ob, o_part, opb) || overlap(o, ob, lse_part, lpb) || overlap(lse, lb, o_part, opb) ||
        overlap(lse, lb, lse_part, lpb) || overlap(o, ob, lse, lb))
        return FA_ERR_ALIAS;
    MergeParams mp;
    mp.op = o_part;
    mp.lp = lse_part;
    mp.o = static_cast<uint16_t *>(o);
    mp.lse = lse;
    mp.rows = rows;
    mp.ostride = elems;
    mp.lstride = rows;
    mp.H = H;
    mp.N = N;
    mp.nsplit = num_splits;
    (void)hipGetLastError();
    return launch_merge(mp, d, stream) == 0 ? FA_OK : FA_ERR_HIP;
}

// Validation shared by the two split-KV entry points (everything but the
// workspaces).
// (Packed: cu_seqlens != nullptr and N = T tokens; rows = T H.)
static int splitkv_check(const void *q, const void *k, const void *v, void *o, float *lse, const int32_t *cu,
                         int B, int H, int N, int d, float scale, int num_splits) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && d != 256) return FA_ERR_HEAD_DIM;
    if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
    if (num_splits < 1 || num_splits > key_tiles(N)) return FA_ERR_SPLIT;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(lse, 4) ||
        misaligned(cu, 4))
        return FA_ERR_ALIGN;
    const long long rows = cu ? static_cast<long long>(N) * H : static_cast<long long>(B) * N * H;
    const long long elems = rows * d;
    if (elems <= 0 || elems * num_splits > (1LL << 46) || !token_stride_ok(H, d)) return FA_ERR_SHAPE;
    const size_t tb = static_cast<size_t>(elems) * 2, lb = static_cast<size_t>(rows) * 4;
    const void *ins[3] = {q, k, v};
    for (const void *in : ins)
        if (overlap(o, tb, in, tb) || overlap(lse, lb, in, tb)) return FA_ERR_ALIAS;
    if (overlap(o, tb, lse, lb)) return FA_ERR_ALIAS;
    if (cu) {
        const size_t cb = static_cast<size_t>(B + 1) * 4;
        if (overlap(o, tb, cu, cb) || overlap(lse, lb, cu, cb)) return FA_ERR_ALIAS;
    }
    return FA_OK;
}

// The split forward and the merge on validated arguments.
static int splitkv_launch(const void *q, const void *k, const void *v, void *o, float *lse, const int32_t *cu,
                          int B, int H, int N, int d, float scale, int causal, int num_splits, float *o_part,
                          float *lse_part, hipStream_t stream) {
    const bool packed = cu != nullptr;
    const long long rows = packed ? static_cast<long long>(N) * H : static_cast<long long>(B) * N * H;
    const long long elems = rows * d;
    Params prm{};
    prm.q = static_cast<const uint16_t *>(q);
    prm.k = static_cast<const uint16_t *>(k);
    prm.v = static_cast<const uint16_t *>(v);
    prm.o = static_cast<uint16_t *>(o);
    prm.lse = lse;
    prm.cu = cu;
    prm.B = B;
    prm.H = H;
    prm.N = N;
    prm.cs = scale * kLog2e;
    const int rows_per_tile = tile_rows_for(d);
    const long long n_qt = (static_cast<long long>(N) + rows_per_tile - 1) / rows_per_tile;
    prm.n_qt = static_cast<int>(n_qt);
    prm.op = o_part;
    prm.lp = lse_part;
    prm.nsplit = num_splits;
    // packed: a bound on sum_b ceil(n_b / rows) query tiles, surplus workgroups exit
    const long long items = packed ? static_cast<long long>(H) * (n_qt + B) : static_cast<long long>(B) * H * n_qt;
    const long long grid = items * num_splits;
    if (grid <= 0 || grid > 0x7fffffffLL) return FA_ERR_SHAPE;

    KernelFn fn;
    switch (d) {
        case 64: fn = select_split_d64(causal != 0, packed); break;
        case 128: fn = select_split_d128(causal != 0, packed); break;
        default: fn = select_split_d256(causal != 0, packed); break;
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(grid)), dim3(waves_for(d) * 64), 0, stream, prm);
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;

    // the merge is per row: packed [T, H, d] / [H, T] is the dense layout
    // of one sequence of T tokens
    MergeParams mp;
    mp.op = o_part;
    mp.lp = lse_part;
    mp.o = static_cast<uint16_t *>(o);
    mp.lse = lse;
    mp.rows = rows;
    mp.ostride = elems;
    mp.lstride = rows;
    mp.H = H;
    mp.N = N;
    mp.nsplit = num_splits;
    return launch_merge(mp, d, stream) == 0 ? FA_OK : FA_ERR_HIP;
}

// Caller workspaces: validation and launch (dense or packed).
static int splitkv_ws(const void *q, const void *k, const void *v, void *o, float *lse, const int32_t *cu, int B,
                      int H, int N, int d, float scale, int causal, int num_splits, float *o_part, float *lse_part,
                      hipStream_t stream) {
    if (!o_part || !lse_part) return FA_ERR_NULLPTR;
    const int rc = splitkv_check(q, k, v, o, lse, cu, B, H, N, d, scale, num_splits);
    if (rc != FA_OK) return rc;
    if (misaligned(o_part, 16) || misaligned(lse_part, 4)) return FA_ERR_ALIGN;
    const long long rows = cu ? static_cast<long long>(N) * H : static_cast<long long>(B) * N * H;
    const long long elems = rows * d;
    const size_t tb = static_cast<size_t>(elems) * 2, lb = static_cast<size_t>(rows) * 4;
    const size_t opb = static_cast<size_t>(elems) * num_splits * 4, lpb = static_cast<size_t>(rows) * num_splits * 4;
    const void *ins[3] = {q, k, v};
    for (const void *in : ins)
        if (overlap(o_part, opb, in, tb) || overlap(lse_part, lpb, in, tb)) return FA_ERR_ALIAS;
    if (overlap(o_part, opb, o, tb) || overlap(o_part, opb, lse, lb) || overlap(lse_part, lpb, o, tb) ||
        overlap(lse_part, lpb, lse, lb) || overlap(o_part, opb, lse_part, lpb))
        return FA_ERR_ALIAS;
    if (cu) {
        const size_t cb = static_cast<size_t>(B + 1) * 4;
        if (overlap(o_part, opb, cu, cb) || overlap(lse_part, lpb, cu, cb)) return FA_ERR_ALIAS;
    }
    return splitkv_launch(q, k, v, o, lse, cu, B, H, N, d, scale, causal, num_splits, o_part, lse_part, stream);
}

int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                   int N, int d, float scale, int causal, int num_splits, float *o_part,
                   float *lse_part, hipStream_t stream) {
    return splitkv_ws(q, k, v, o, lse, nullptr, B, H, N, d, scale, causal, num_splits, o_part, lse_part, stream);
}

int fa_fwd_splitkv_packed(const void *q, const void *k, const void *v, void *o, float *lse,
                          const int32_t *cu_seqlens, int B, int H, int T, int d, float scale, int causal,
                          int num_splits, float *o_part, float *lse_part, hipStream_t stream) {
    if (!cu_seqlens) return FA_ERR_NULLPTR;
    return splitkv_ws(q, k, v, o, lse, cu_seqlens, B, H, T, d, scale, causal, num_splits, o_part, lse_part,
                      stream);
}

int fa_fwd_splitkv_static(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                          int N, int d, float scale, int causal, int num_splits, hipStream_t stream) {
    const int rc = splitkv_check(q, k, v, o, lse, nullptr, B, H, N, d, scale, num_splits);
    if (rc != FA_OK) return rc;
    // partials: o_part [S, B, N, H, d] then lse_part [S, B, H, N], fp32;
    // rows * d * 4 is a multiple of 256, so lse_part stays aligned
    const long long rows = static_cast<long long>(B) * N * H;
    const long long need = static_cast<long long>(num_splits) * rows * (d + 1) * 4;
    if (need > static_cast<long long>(FA_STATIC_SCRATCH_BYTES)) return FA_ERR_SCRATCH;
    void *base = nullptr;
    const int sc = scratch_for_current_device(&base);
    if (sc != FA_OK) return sc;
    float *o_part = static_cast<float *>(base);
    float *lse_part = o_part + static_cast<long long>(num_splits) * rows * d;
    return splitkv_launch(q, k, v, o, lse, nullptr, B, H, N, d, scale, causal, num_splits, o_part, lse_part,
                          stream);
}

long long fa_bwd_workspace_floats(int B, int H, int N) {
    if (B < 1 || H < 1 || N < 1) return 0;
    return 2LL * B * H * N;
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
           void *dq, void *dk, void *dv, int B, int H, int N, int d, float scale, int causal,
           const int32_t *cu_seqlens, float *workspace, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace) return FA_ERR_NULLPTR;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && d != 256) return FA_ERR_HEAD_DIM;
    if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
    const void *t16[] = {q, k, v, o, dout, dq, dk, dv, workspace};
    for (const void *t : t16)
        if (misaligned(t, 16)) return FA_ERR_ALIGN;
    if (misaligned(lse, 4) || misaligned(cu_seqlens, 4)) return FA_ERR_ALIGN;
    const bool packed = cu_seqlens != nullptr;
    const long long tokens = packed ? static_cast<long long>(N) : static_cast<long long>(B) * N;
    const long long rows = tokens * H;
    const long long elems = rows * d;
    if (elems <= 0 || elems > (1LL << 46) || !token_stride_ok(H, d)) return FA_ERR_SHAPE;
    const size_t tb = static_cast<size_t>(elems) * 2, lb = static_cast<size_t>(rows) * 4;
    const size_t wb = static_cast<size_t>(rows) * 8;  // two floats per LSE entry
    const void *outs[] = {dq, dk, dv, workspace};
    const size_t out_bytes[] = {tb, tb, tb, wb};
    const void *ins[] = {q, k, v, o, dout, lse};
    const size_t in_bytes[] = {tb, tb, tb, tb, tb, lb};
    for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlap(outs[i], out_bytes[i], ins[j], in_bytes[j])) return FA_ERR_ALIAS;
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], out_bytes[i], outs[j], out_bytes[j])) return FA_ERR_ALIAS;
    }

    BwdParams bp{};
    bp.q = static_cast<const uint16_t *>(q);
    bp.k = static_cast<const uint16_t *>(k);
    bp.v = static_cast<const uint16_t *>(v);
    bp.o = static_cast<const uint16_t *>(o);
    bp.dout = static_cast<const uint16_t *>(dout);
    bp.lse = lse;
    bp.cu = cu_seqlens;
    bp.dq = static_cast<uint16_t *>(dq);
    bp.dk = static_cast<uint16_t *>(dk);
    bp.dv = static_cast<uint16_t *>(dv);
    bp.stats = workspace;
    bp.B = B;
    bp.H = H;
    bp.N = N;
    bp.cs = scale * kLog2e;
    bp.scale = scale;
    const BwdKernels ks = d == 64    ? select_bwd_d64(causal != 0, packed)
                          : d == 128 ? select_bwd_d128(causal != 0, packed)
                                     : select_bwd_d256(causal != 0, packed);
    // key tiles of the dK/dV kernel and query tiles of the dQ kernel: 128
    // each; packed: a bound on sum_b ceil(n_b / 128), surplus workgroups exit
    const long long tiles = (static_cast<long long>(N) + 127) / 128;
    const long long prep_grid = (rows + 255) / 256;
    const long long kv_grid = packed ? static_cast<long long>(H) * (tiles + B) : static_cast<long long>(B) * H * tiles;
    const long long q_grid = kv_grid;
    if (prep_grid > 0x7fffffffLL || kv_grid > 0x7fffffffLL || q_grid > 0x7fffffffLL) return FA_ERR_SHAPE;
    (void)hipGetLastError();
    hipLaunchKernelGGL(ks.prep, dim3(static_cast<unsigned>(prep_grid)), dim3(256), 0, stream, bp);
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    hipLaunchKernelGGL(ks.dkdv, dim3(static_cast<unsigned>(kv_grid)), dim3(256), 0, stream, bp);
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    hipLaunchKernelGGL(ks.dq, dim3(static_cast<unsigned>(q_grid)), dim3(256), 0, stream, bp);
    if (hipGetLastError() != hipSuccess) return FA_ERR_HIP;
    return FA_OK;
}

// Masked forward, dense (cu_seqlens == nullptr) or packed (N = T tokens).
static int masked_impl(const void *q, const void *k, const void *v, void *o, float *lse, const int32_t *cu_seqlens,
                       int B, int H, int N, int d, float scale, int window_left, int window_right,
                       const float *alibi_slopes, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_NULLPTR;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && d != 256) return FA_ERR_HEAD_DIM;
    if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
    if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16) || misaligned(lse, 4) ||
        misaligned(alibi_slopes, 4) || misaligned(cu_seqlens, 4))
        return FA_ERR_ALIGN;
    const bool packed = cu_seqlens != nullptr;
    const long long rows = packed ? static_cast<long long>(N) * H : static_cast<long long>(B) * N * H;
    const long long elems = rows * d;
    // window edges are added to row and key indices in 32-bit arithmetic
    if (elems <= 0 || elems > (1LL << 46) || !token_stride_ok(H, d) || N > kMaskedMaxN) return FA_ERR_SHAPE;
    const size_t tb = static_cast<size_t>(elems) * 2, lb = static_cast<size_t>(rows) * 4;
    const size_t sb = static_cast<size_t>(H) * 4;
    const void *ins[] = {q, k, v};
    for (const void *in : ins)
        if (overlap(o, tb, in, tb) || overlap(lse, lb, in, tb)) return FA_ERR_ALIAS;
    if (overlap(o, tb, lse, lb)) return FA_ERR_ALIAS;
    if (alibi_slopes && (overlap(o, tb, alibi_slopes, sb) || overlap(lse, lb, alibi_slopes, sb))) return FA_ERR_ALIAS;
    if (packed) {
        const size_t cb = static_cast<size_t>(B + 1) * 4;
        if (overlap(o, tb, cu_seqlens, cb) || overlap(lse, lb, cu_seqlens, cb)) return FA_ERR_ALIAS;
    }

    Params prm{};
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
    // an edge at N - 1 or beyond hides no key (packed: no sequence is longer
    // than T = N): clamp it there, so that the kernel's index arithmetic
    // (row + edge) stays far from overflow
    prm.wl = window_left < 0 ? -1 : (window_left < N ? window_left : N - 1);
    prm.wr = window_right < 0 ? -1 : (window_right < N ? window_right : N - 1);
    prm.alibi = alibi_slopes;
    prm.inv_scale = 1.0f / scale;
    const int rows_per_tile = tile_rows_for(d);
    const long long n_qt = (static_cast<long long>(N) + rows_per_tile - 1) / rows_per_tile;
    prm.n_qt = static_cast<int>(n_qt);
    // packed: a bound on sum_b ceil(n_b / rows), surplus workgroups exit
    const long long grid = packed ? static_cast<long long>(H) * (n_qt + B) : static_cast<long long>(B) * H * n_qt;
    if (grid <= 0 || grid > 0x7fffffffLL) return FA_ERR_SHAPE;
    const KernelFn fn = d == 64    ? select_mods_d64(packed)
                        : d == 128 ? select_mods_d128(packed)
                                   : select_mods_d256(packed);
    (void)hipGetLastError();
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(grid)), dim3(waves_for(d) * 64), 0, stream, prm);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_masked(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N, int d,
                  float scale, int window_left, int window_right, const float *alibi_slopes, hipStream_t stream) {
    return masked_impl(q, k, v, o, lse, nullptr, B, H, N, d, scale, window_left, window_right, alibi_slopes, stream);
}

int fa_fwd_masked_packed(const void *q, const void *k, const void *v, void *o, float *lse,
                         const int32_t *cu_seqlens, int B, int H, int T, int d, float scale, int window_left,
                         int window_right, const float *alibi_slopes, hipStream_t stream) {
    if (!cu_seqlens) return FA_ERR_NULLPTR;
    return masked_impl(q, k, v, o, lse, cu_seqlens, B, H, T, d, scale, window_left, window_right, alibi_slopes,
                       stream);
}

int fa_fp8_vt_stride(int N) { return N < 1 ? 0 : (N + 63) / 64 * 64; }

int fa_fp8_vt_stride_packed(int T, int B) {
    if (T < 1 || B < 1) return 0;
    const long long s = (static_cast<long long>(T) + 63) / 64 * 64 + 64LL * B;
    return s > 0x7fffffffLL ? 0 : static_cast<int>(s);
}

// Quantisation, dense (cu_seqlens == nullptr: x [B, N, H, d]) or packed
// (x [T, H, d], N = T, B sequences).
static int quant_impl(const void *x, void *x8, float *descale, const int32_t *cu_seqlens, int B, int H, int N,
                      int d, int transpose, hipStream_t stream) {
    if (!x || !x8 || !descale) return FA_ERR_NULLPTR;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && d != 256) return FA_ERR_HEAD_DIM;
    if (misaligned(x, 16) || misaligned(x8, 4) || misaligned(descale, 4) || misaligned(cu_seqlens, 4))
        return FA_ERR_ALIGN;
    const bool packed = cu_seqlens != nullptr;
    const long long rows = packed ? static_cast<long long>(N) * H : static_cast<long long>(B) * N * H;
    long long x8_elems;
    if (!transpose) {
        x8_elems = rows * d;
    } else if (packed) {
        const int vts = fa_fp8_vt_stride_packed(N, B);
        if (vts == 0 || static_cast<long long>(d) * vts > 0x7fffffffLL) return FA_ERR_SHAPE;
        x8_elems = static_cast<long long>(H) * d * vts;
    } else {
        x8_elems = static_cast<long long>(B) * H * d * fa_fp8_vt_stride(N);
    }
    if (rows * d <= 0 || rows * d > (1LL << 46) || x8_elems > (1LL << 46) || !token_stride_ok(H, d))
        return FA_ERR_SHAPE;
    const size_t xb = static_cast<size_t>(rows) * d * 2, x8b = static_cast<size_t>(x8_elems);
    const size_t db = static_cast<size_t>(B) * H * 4, cb = packed ? static_cast<size_t>(B + 1) * 4 : 0;
    if (overlap(x8, x8b, x, xb) || overlap(descale, db, x, xb) || overlap(descale, db, x8, x8b) ||
        (packed && (overlap(x8, x8b, cu_seqlens, cb) || overlap(descale, db, cu_seqlens, cb))))
        return FA_ERR_ALIAS;
    QuantParams qp;
    qp.x = static_cast<const uint16_t *>(x);
    qp.x8 = static_cast<uint8_t *>(x8);
    qp.descale = descale;
    qp.cu = cu_seqlens;
    qp.B = B;
    qp.H = H;
    qp.N = N;
    qp.d = d;
    qp.transpose = transpose != 0;
    qp.vts = packed ? fa_fp8_vt_stride_packed(N, B) : 0;
    (void)hipGetLastError();
    return launch_quant(qp, stream) == 0 ? FA_OK : FA_ERR_HIP;
}

int fa_quantize_fp8(const void *x, void *x8, float *descale, int B, int H, int N, int d, int transpose,
                    hipStream_t stream) {
    return quant_impl(x, x8, descale, nullptr, B, H, N, d, transpose, stream);
}

int fa_quantize_fp8_packed(const void *x, void *x8, float *descale, const int32_t *cu_seqlens, int B, int H,
                           int T, int d, int transpose, hipStream_t stream) {
    if (!cu_seqlens) return FA_ERR_NULLPTR;
    return quant_impl(x, x8, descale, cu_seqlens, B, H, T, d, transpose, stream);
}

// FP8 forward, dense or packed (as quant_impl).
static int fwd_fp8_impl(const void *q8, const void *k8, const void *vt8, const float *descale_q,
                        const float *descale_k, const float *descale_v, void *o, float *lse,
                        const int32_t *cu_seqlens, int B, int H, int N, int d, float scale, int causal,
                        hipStream_t stream) {
    if (!q8 || !k8 || !vt8 || !descale_q || !descale_k || !descale_v || !o || !lse) return FA_ERR_NULLPTR;
    if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
    if (d != 64 && d != 128 && d != 256) return FA_ERR_HEAD_DIM;
    if (!(scale > 0.0f) || !isfinite(scale)) return FA_ERR_SCALE;
    if (misaligned(q8, 16) || misaligned(k8, 16) || misaligned(vt8, 16) || misaligned(o, 16) ||
        misaligned(lse, 4) || misaligned(descale_q, 4) || misaligned(descale_k, 4) || misaligned(descale_v, 4) ||
        misaligned(cu_seqlens, 4))
        return FA_ERR_ALIGN;
    const bool packed = cu_seqlens != nullptr;
    const long long rows = packed ? static_cast<long long>(N) * H : static_cast<long long>(B) * N * H;
    const long long elems = rows * d;
    const int vts = packed ? fa_fp8_vt_stride_packed(N, B) : fa_fp8_vt_stride(N);
    const long long vt_elems = packed ? static_cast<long long>(H) * d * vts : static_cast<long long>(B) * H * d * vts;
    // a head's V^T rows are addressed by one buffer resource (32-bit size)
    if (elems <= 0 || elems > (1LL << 46) || !token_stride_ok(H, d) || vts == 0 ||
        static_cast<long long>(d) * vts > 0x7fffffffLL || vt_elems > (1LL << 46))
        return FA_ERR_SHAPE;
    const size_t qb = static_cast<size_t>(elems), vb = static_cast<size_t>(vt_elems);
    const size_t ob = static_cast<size_t>(elems) * 2, lb = static_cast<size_t>(rows) * 4;
    const size_t sb = static_cast<size_t>(B) * H * 4;
    const void *ins[] = {q8, k8, vt8, descale_q, descale_k, descale_v};
    const size_t in_bytes[] = {qb, qb, vb, sb, sb, sb};
    for (int i = 0; i < 6; ++i)
        if (overlap(o, ob, ins[i], in_bytes[i]) || overlap(lse, lb, ins[i], in_bytes[i])) return FA_ERR_ALIAS;
    if (overlap(o, ob, lse, lb)) return FA_ERR_ALIAS;
    if (packed) {
        const size_t cb = static_cast<size_t>(B + 1) * 4;
        if (overlap(o, ob, cu_seqlens, cb) || overlap(lse, lb, cu_seqlens, cb)) return FA_ERR_ALIAS;
    }

    Fp8Params fp{};
    fp.q = static_cast<const uint8_t *>(q8);
    fp.k = static_cast<const uint8_t *>(k8);
    fp.vt = static_cast<const uint8_t *>(vt8);
    fp.dq = descale_q;
    fp.dk = descale_k;
    fp.dv = descale_v;
    fp.o = static_cast<uint16_t *>(o);
    fp.lse = lse;
    fp.cu = cu_seqlens;
    fp.B = B;
    fp.H = H;
    fp.N = N;
    fp.vts = packed ? vts : 0;
    fp.cs = scale * kLog2e;
    const int rows_per_tile = fp8_rows_for(d);
    const long long n_qt = (static_cast<long long>(N) + rows_per_tile - 1) / rows_per_tile;
    // packed: a bound on sum_b ceil(n_b / rows), surplus workgroups exit
    const long long grid = packed ? static_cast<long long>(H) * (n_qt + B) : static_cast<long long>(B) * H * n_qt;
    if (grid <= 0 || grid > 0x7fffffffLL) return FA_ERR_SHAPE;
    const KernelFp8Fn fn = d == 64    ? select_fp8_d64(causal != 0, packed)
                           : d == 128 ? select_fp8_d128(causal != 0, packed)
                                      : select_fp8_d256(causal != 0, packed);
    (void)hipGetLastError();
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(grid)), dim3(rows_per_tile * 2), 0, stream, fp);
    return hipGetLastError() == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8(const void *q8, const void *k8, const void *vt8, const float *descale_q, const float *descale_k,
               const float *descale_v, void *o, float *lse, int B, int H, int N, int d, float scale, int causal,
               hipStream_t stream) {
    return fwd_fp8_impl(q8, k8, vt8, descale_q, descale_k, descale_v, o, lse, nullptr, B, H, N, d, scale, causal,
                        stream);
}

int fa_fwd_fp8_packed(const void *q8, const void *k8, const void *vt8, const float *descale_q,
                      const float *descale_k, const float *descale_v, void *o, float *lse,
                      const int32_t *cu_seqlens, int B, int H, int T, int d, float scale, int causal,
                      hipStream_t stream) {
    if (!cu_seqlens) return FA_ERR_NULLPTR;
    return fwd_fp8_impl(q8, k8, vt8, descale_q, descale_k, descale_v, o, lse, cu_seqlens, B, H, T, d, scale,
                        causal, stream);
}

int fa_fwd_variant(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                   int N, int d, float scale, int causal, const int32_t *cu_seqlens,
                   hipStream_t stream, int exp_mode, int rescale_mode) {
    return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, cu_seqlens, stream, exp_mode, rescale_mode,
                    nullptr);
}

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N,
           int d, float scale, int causal, const int32_t *cu_seqlens, hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, cu_seqlens, stream, FA_EXP_HW, FA_RESCALE_STRICT,
                    nullptr, false, true);
}

int fa_fwd_pingpong(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int N,
                    int d, float scale, int causal, const int32_t *cu_seqlens, hipStream_t stream) {
    if (d != 128 && (d == 64 || d == 256)) return FA_ERR_HEAD_DIM;
    return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, cu_seqlens, stream, FA_EXP_HW, FA_RESCALE_STRICT,
                    nullptr, d == 128);
}

int fa_fwd_rescale_counts(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
                          int N, int d, float scale, int causal, const int32_t *cu_seqlens,
                          hipStream_t stream, int rescale_mode, unsigned long long *counts) {
    if (!counts) return FA_ERR_NULLPTR;
    if (misaligned(counts, 8)) return FA_ERR_ALIGN;
    if (d != 128) return FA_ERR_HEAD_DIM;
    if (rescale_mode != FA_RESCALE_STRICT && rescale_mode != FA_RESCALE_THRESHOLD) return FA_ERR_VARIANT;
    const long long tokens = cu_seqlens ? static_cast<long long>(N) : static_cast<long long>(B) * N;
    const long long elems = tokens * H * d;
    if (B >= 1 && H >= 1 && N >= 1 && elems > 0 && elems <= (1LL << 46)) {
        const size_t tb = static_cast<size_t>(elems) * 2, lb = static_cast<size_t>(tokens * H) * 4;
        const void *bufs[] = {q, k, v, o};
        for (const void *b : bufs)
            if (b && overlap(counts, 32, b, tb)) return FA_ERR_ALIAS;
        if (lse && overlap(counts, 32, lse, lb)) return FA_ERR_ALIAS;
    }
    return fwd_impl(q, k, v, o, lse, B, H, N, d, scale, causal, cu_seqlens, stream, FA_EXP_HW, rescale_mode,
                    counts);
}

}  // extern "C"
