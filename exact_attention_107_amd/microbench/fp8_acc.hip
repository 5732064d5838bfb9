// Accumulation error of the gfx950 FP8 matrix product that the FP8 forward
// uses (v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands, fp32
// accumulator starting at 0): each 32x32 output element is a 64-term dot
// product of E4M3 values.  The host decodes the codes from the OCP E4M3
// definition (bias 7, 3 mantissa bits, subnormals) and sums the exact
// products in double (each product has at most 8 significant bits and the
// exponents span < 40 bits, so the 64-term sums are exact), then reports
// max |mfma - exact| / sum_k |a_k b_k| over many dot products, for codes
// drawn uniformly over all finite codes and for codes of normally
// distributed values scaled to amax = 448, and one constructed case of a
// large product next to many small ones.
// Build: hipcc --offload-arch=gfx950 -O3 fp8_acc.hip -o fp8_acc.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                          \
    do {                                                                                  \
        hipError_t e_ = (x);                                                              \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));                       \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

// One wave per group g: A and B are 32 rows of 64 codes each ([G][32][64]
// bytes).  Lane l supplies row l % 32, bytes 32 (l / 32) .. +32 of both; the
// product is D[i][j] = sum_k A[i][k] B[j][k], and accumulator element r of
// lane l is D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
__global__ void __launch_bounds__(64) fp8_dot(const uint8_t *a, const uint8_t *b, float *d) {
    const int g = blockIdx.x, l = threadIdx.x;
    const long long off = (static_cast<long long>(g) * 32 + (l & 31)) * 64 + 32 * (l >> 5);
    const u32x4 a0 = *reinterpret_cast<const u32x4 *>(a + off), a1 = *reinterpret_cast<const u32x4 *>(a + off + 16);
    const u32x4 b0 = *reinterpret_cast<const u32x4 *>(b + off), b1 = *reinterpret_cast<const u32x4 *>(b + off + 16);
    const i32x8 av = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8 bv = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    f32x16 acc = {};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
    for (int r = 0; r < 16; ++r)
        d[static_cast<long long>(g) * 1024 + (8 * (r / 4) + 4 * (l >> 5) + r % 4) * 32 + (l & 31)] = acc[r];
}

static double e4m3(uint8_t c) {
    const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    const double v = e == 0 ? m * ldexp(1.0, -9) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
    return s ? -v : v;
}

// nearest E4M3 code of x (|x| <= 448), ties to the even code
static uint8_t encode(double x) {
    uint8_t best = 0;
    double bd = 1e300;
    for (int c = 0; c < 0x7f; ++c) {
        const double dd = fabs(e4m3(static_cast<uint8_t>(c)) - fabs(x));
        if (dd < bd || (dd == bd && (c & 1) == 0)) {
            bd = dd;
            best = static_cast<uint8_t>(c);
        }
    }
    return x < 0 ? best | 0x80 : best;
}

struct Result {
    double worst;     // max |err| / sum |products|
    double mean;
    long long n;
};

static Result run(const std::vector<uint8_t> &A, const std::vector<uint8_t> &B, int G) {
    uint8_t *da, *db;
    float *dd;
    CHECK(hipMalloc(&da, A.size()));
    CHECK(hipMalloc(&db, B.size()));
    CHECK(hipMalloc(&dd, static_cast<size_t>(G) * 1024 * 4));
    CHECK(hipMemcpy(da, A.data(), A.size(), hipMemcpyHostToDevice));
    CHECK(hipMemcpy(db, B.data(), B.size(), hipMemcpyHostToDevice));
    hipLaunchKernelGGL(fp8_dot, dim3(G), dim3(64), 0, 0, da, db, dd);
    CHECK(hipGetLastError());
    std::vector<float> D(static_cast<size_t>(G) * 1024);
    CHECK(hipMemcpy(D.data(), dd, D.size() * 4, hipMemcpyDeviceToHost));
    CHECK(hipFree(da));
    CHECK(hipFree(db));
    CHECK(hipFree(dd));
    Result r{0.0, 0.0, 0};
    for (int g = 0; g < G; ++g)
        for (int i = 0; i < 32; ++i)
            for (int j = 0; j < 32; ++j) {
                double exact = 0.0, mag = 0.0;
                for (int k = 0; k < 64; ++k) {
                    const double p = e4m3(A[(static_cast<size_t>(g) * 32 + i) * 64 + k]) *
                                     e4m3(B[(static_cast<size_t>(g) * 32 + j) * 64 + k]);
                    exact += p;
                    mag += fabs(p);
                }
                if (mag == 0.0) continue;
                const double rel = fabs(D[static_cast<size_t>(g) * 1024 + i * 32 + j] - exact) / mag;
                r.worst = rel > r.worst ? rel : r.worst;
                r.mean += rel;
                ++r.n;
            }
    r.mean /= r.n > 0 ? r.n : 1;
    return r;
}

int main() {
    const int G = 64;   // 64 groups x 1024 dot products
    std::mt19937_64 rng(20261203);
    std::vector<uint8_t> A(static_cast<size_t>(G) * 2048), B(A.size());
    // all finite codes, uniformly (0x7f and 0xff are NaN)
    std::uniform_int_distribution<int> code(0, 253);
    auto draw = [&]() {
        const int c = code(rng);
        return static_cast<uint8_t>(c >= 0x7f ? c + 1 : c);
    };
    for (auto &x : A) x = draw();
    for (auto &x : B) x = draw();
    const Result u = run(A, B, G);
    // normally distributed values scaled so that the largest is 448, as the
    // per-head quantisation produces
    std::normal_distribution<double> nd(0.0, 1.0);
    std::vector<double> va(A.size()), vb(B.size());
    double ma = 0.0, mb = 0.0;
    for (size_t i = 0; i < va.size(); ++i) {
        va[i] = nd(rng);
        vb[i] = nd(rng);
        ma = fmax(ma, fabs(va[i]));
        mb = fmax(mb, fabs(vb[i]));
    }
    for (size_t i = 0; i < va.size(); ++i) {
        A[i] = encode(va[i] * 448.0 / ma);
        B[i] = encode(vb[i] * 448.0 / mb);
    }
    const Result nrm = run(A, B, G);
    // one product 256 x 256 = 65536 and 63 products 2^-3 x 2^-3 = 2^-6
    std::vector<uint8_t> A1(2048, 0), B1(2048, 0);
    A1[0] = B1[0] = 0x78;                       // 256
    for (int k = 1; k < 64; ++k) A1[k] = B1[k] = 0x20;  // 2^-3
    uint8_t *da, *db;
    float *dd;
    CHECK(hipMalloc(&da, 2048));
    CHECK(hipMalloc(&db, 2048));
    CHECK(hipMalloc(&dd, 4096));
    CHECK(hipMemcpy(da, A1.data(), 2048, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(db, B1.data(), 2048, hipMemcpyHostToDevice));
    hipLaunchKernelGGL(fp8_dot, dim3(1), dim3(64), 0, 0, da, db, dd);
    CHECK(hipGetLastError());
    float d00;
    CHECK(hipMemcpy(&d00, dd, 4, hipMemcpyDeviceToHost));
    CHECK(hipFree(da));
    CHECK(hipFree(db));
    CHECK(hipFree(dd));
    printf("# v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3, fp32 accumulate from 0: 64-term dot products\n");
    printf("uniform finite codes   %lld dot products | max |err|/sum|prod| = 2^%.2f | mean 2^%.2f\n", u.n,
           log2(u.worst), log2(u.mean));
    printf("normal values, amax 448 %lld dot products | max |err|/sum|prod| = 2^%.2f | mean 2^%.2f\n", nrm.n,
           log2(nrm.worst), log2(nrm.mean));
    printf("65536 + 63 x 2^-6: exact %.6f, mfma %.6f\n", 65536.0 + 63.0 / 64.0, d00);
    return 0;
}
