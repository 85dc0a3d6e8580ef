// Measures how exactly gfx950's E4M3 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4,
// unit scales) sums the 128 products of one block: one wave multiplies seeded
// random E4M3 operands (every finite code) and the host compares each of the
// 256 outputs with the exact sum of its products.  Prints one JSON line:
// the largest |gpu - exact| / sum |product| over all trials, and the result
// of a block of one product of 448 and 127 of 2^-9 * 1 (exact: 448.248046875).
// The FP8 layer's per-token parity tolerance rests on the first number.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <random>
#include <vector>

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

// A, B: 64 lanes x 32 codes; lane l holds row / column l % 16 and the 32
// k-values 32 * (l / 16) .. +31.  out: lane l, register r = C[4 (l / 16) + r][l % 16].
__global__ __launch_bounds__(64) void block_sum(const int* a, const int* b, float* out) {
  const int l = threadIdx.x;
  i32x8_t A, B;
  for (int i = 0; i < 8; ++i) {
    A[i] = a[l * 8 + i];
    B[i] = b[l * 8 + i];
  }
  const floatx4_t c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
      A, B, floatx4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
  for (int r = 0; r < 4; ++r) out[l * 4 + r] = c[r];
}

static double e4m3(unsigned c) {
  const double s = (c & 0x80) ? -1.0 : 1.0;
  const int e = (c >> 3) & 15, m = c & 7;
  return e == 0 ? s * m / 8.0 * std::ldexp(1.0, -6) : s * (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
}

#define CHECK(x)                                                         \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

int main() {
  int *da = nullptr, *db = nullptr;
  float* dout = nullptr;
  CHECK(hipMalloc(&da, 64 * 32));
  CHECK(hipMalloc(&db, 64 * 32));
  CHECK(hipMalloc(&dout, 256 * sizeof(float)));
  std::vector<unsigned char> ha(64 * 32), hb(64 * 32);
  std::vector<float> ho(256);
  auto run = [&]() -> hipError_t {
    hipError_t e = hipMemcpy(da, ha.data(), ha.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(db, hb.data(), hb.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(block_sum, dim3(1), dim3(64), 0, 0, da, db, dout);
    e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(ho.data(), dout, ho.size() * sizeof(float), hipMemcpyDeviceToHost);
    return e;
  };
  // one large product among small ones
  for (auto& v : ha) v = 0x38;  // 1.0
  for (auto& v : hb) v = 0x01;  // 2^-9
  hb[0] = 0x7E;                 // 448 at lane 0, k = 0: output column 0
  CHECK(run());
  const float big = ho[0];
  // random finite codes
  std::mt19937 rng(12345);
  auto code = [&]() {
    unsigned c;
    do c = rng() & 0xFFu; while ((c & 0x7Fu) == 0x7Fu);
    return (unsigned char)c;
  };
  double worst = 0.0;
  for (int trial = 0; trial < 16; ++trial) {
    for (auto& v : ha) v = code();
    for (auto& v : hb) v = code();
    CHECK(run());
    for (int l = 0; l < 64; ++l)
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * (l / 16) + r, col = l % 16;
        double s = 0.0, sa = 0.0;
        for (int k = 0; k < 128; ++k) {
          const double p = e4m3(ha[(row + 16 * (k / 32)) * 32 + k % 32]) *
                           e4m3(hb[(col + 16 * (k / 32)) * 32 + k % 32]);
          s += p;
          sa += std::fabs(p);
        }
        if (sa > 0.0) worst = std::fmax(worst, std::fabs(ho[l * 4 + r] - s) / sa);
      }
  }
  std::printf("{\"max_err_over_abs_sum\": %.6e, \"one_large_block\": %.9g, \"exact\": 448.248046875}\n",
              worst, big);
  return 0;
}
