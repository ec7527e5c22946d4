// The r Gaussian hyperplanes per head that the hash uses (HA page,
// "Algorithm", Definition 1: a Hamming-sorted LSH; read here as signs of
// projections on Gaussian hyperplanes).
//
// Entry (k, t) of head h is the Box-Muller normal of gaussian.h from two
// counter-based draws of SplitMix64 (Steele, Lea and Flood, OOPSLA 2014),
// purpose 1, node 0, counters 2e and 2e + 1 with e = k d + t, rounded to fp32
// and then to the nearest bfloat16 (ties to even; a bf16 input times a
// hyperplane entry is then exact in fp32). gaussian.h uses binary64 basic
// operations only, so the device computes the same bits as the host: every
// call draws its hyperplanes on the device, on the caller's stream, into the
// caller's workspace, and the library keeps nothing between calls.
#include "common.h"
#include "device_util.h"
#include "gaussian.h"

namespace ha {

namespace {

constexpr int kPlaneThreads = 256;

// One thread per entry of the bf16 layout [heads][16][d]; rows k < r also go
// to the fp32 layout [heads][r][d]. Rows r..15 of the bf16 layout are zero.
__global__ __launch_bounds__(kPlaneThreads) void planes_kernel(uint64_t key, int heads, int r,
                                                               int d, float* __restrict__ G,
                                                               bf16_t* __restrict__ Gb) {
  const int64_t i = int64_t(blockIdx.x) * kPlaneThreads + threadIdx.x;
  if (i >= int64_t(heads) * 16 * d) return;
  const int t = int(i % d);
  const int k = int((i / d) % 16);
  const int h = int(i / (int64_t(16) * d));
  bf16_t v = 0;
  if (k < r) {
    const uint64_t e = uint64_t(k) * d + t;
    const double g = gauss::box_muller(draw(key, 1, h, 0, 2 * e), draw(key, 1, h, 0, 2 * e + 1));
    v = gauss::to_bf16_bits(g);
    G[(int64_t(h) * r + k) * d + t] = __uint_as_float(uint32_t(v) << 16);
  }
  Gb[i] = v;
}

}  // namespace

void host_hyperplanes(uint64_t seed, int heads, int r, int d, float* G) {
  const uint64_t key = mix64(seed);
  for (int h = 0; h < heads; ++h)
    for (int k = 0; k < r; ++k)
      for (int t = 0; t < d; ++t) {
        const uint64_t e = uint64_t(k) * d + t;
        const double g = gauss::box_muller(draw(key, 1, h, 0, 2 * e), draw(key, 1, h, 0, 2 * e + 1));
        const uint32_t u = uint32_t(gauss::to_bf16_bits(g)) << 16;
        G[(int64_t(h) * r + k) * d + t] = __builtin_bit_cast(float, u);
      }
}

void host_gaussians(const uint64_t* a, const uint64_t* b, int64_t count, double* out) {
  for (int64_t i = 0; i < count; ++i) out[i] = gauss::box_muller(a[i], b[i]);
}

int64_t hyperplane_stage_bytes(int heads, int r, int d) {
  return align256(int64_t(heads) * (r > 0 ? r : 1) * d * 4) + int64_t(heads) * 16 * d * 2;
}

int launch_hyperplanes(uint64_t seed, int heads, int r, int d, void* stage, hipStream_t s,
                       const float** out, const uint16_t** out_bf16) {
  char* base = static_cast<char*>(stage);
  float* G = reinterpret_cast<float*>(base);
  bf16_t* Gb = reinterpret_cast<bf16_t*>(base + align256(int64_t(heads) * (r > 0 ? r : 1) * d * 4));
  *out = G;
  if (out_bf16) *out_bf16 = Gb;
  const int64_t total = int64_t(heads) * 16 * d;
  if (r == 0 || total == 0) return HA_OK;   // the local block mask reads no hyperplanes
  ProfRange pr("hyperplanes", s);
  hipLaunchKernelGGL(planes_kernel, dim3(unsigned(ceil_div(total, kPlaneThreads))),
                     dim3(kPlaneThreads), 0, s, mix64(seed), heads, r, d, G, Gb);
  HA_LAUNCH_CHECK("hyperplanes");
  return HA_OK;
}

}  // namespace ha
