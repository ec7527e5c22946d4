// Rotary position embedding of Q and K on the device, fused with the sortLSH
// hash for bf16 rows (the long-context workloads rotate Q and K before
// attention, and the hash must see the rotated rows: HA page, "Algorithm",
// Definition 1 applied to the rows the attention uses).
//
// Rotation (the usual rotary form): pairs (t, t + d/2) for t < d/2, frequency
// theta_t = base^(-2t/d), row i at position i:
//   x'_t       = x_t cos(i theta_t) - x_{t+d/2} sin(i theta_t)
//   x'_{t+d/2} = x_t sin(i theta_t) + x_{t+d/2} cos(i theta_t)
// in fp32 with every product and sum rounded once (no fused multiply-add),
// then, for bf16 rows, rounded to the nearest bf16. cos and sin come from a
// table the caller passes in device memory, filled by rope_table on the host
// with the C library's pow, cos and sin (fp64, rounded once to fp32), so the
// rotated rows are fixed numbers, not just close ones.
//
// bf16 rows: rope_hash_kernel. Lane l of a wave owns row l%16 of the wave's
// 16 rows and the 16-byte chunks at elements 32s + 8(l/16), s < d/32 (the
// layout of the MFMA hash); chunk s and chunk s + d/64 hold the two members of
// eight pairs, so the rotation needs no data exchange. A work-group keeps its
// 64 rows' table entries in registers and loops over every head and both of
// Q and K; each rotated row is written out and hashed from registers.
// Signs the fp32 MFMA projection cannot settle are recomputed in fp64 in
// order t from the raw row and the table (the rotation is recomputed exactly).
// fp32 rows, and rotation without hashing: rope_kernel.
// Backward: rope_adjoint_kernel applies the transpose of each pair's rotation
// (a turn by -i theta_t, same table and rounding) to dQ and dK in place, so
// that they become the gradients of the rows before rotation.
#include <cmath>
#include <vector>

#include "common.h"
#include "device_util.h"

namespace ha {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 16;
constexpr int kRopeRows = kThreads / 64 * kRowsPerWave;   // rows per work-group

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One rotated pair in fp32, each operation rounded separately.
__device__ __forceinline__ void rotate_pair(float x1, float x2, float c, float s, float& y1,
                                            float& y2) {
#pragma clang fp contract(off)
  const float a = x1 * c;
  const float b = x2 * s;
  const float e = x1 * s;
  const float f = x2 * c;
  y1 = a - b;
  y2 = e + f;
}

// ------------------------------------------------ rotation only (any type)
// Thread: one row, four consecutive pairs t0..t0+3; a work-group covers
// kThreads / (d/8) rows and loops over the heads and the given sides.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void rope_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, T* __restrict__ Qr, T* __restrict__ Kr,
    const float* __restrict__ tab, int64_t n, int heads, int sides) {
  constexpr int TPR = D / 8;                  // threads per row
  constexpr int RPB = kThreads / TPR;         // rows per work-group
  const int64_t row = int64_t(blockIdx.x) * RPB + threadIdx.x / TPR;
  const int t0 = (threadIdx.x % TPR) * 4;
  if (row >= n) return;
  float c[4], s[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = tab[(row * (D / 2) + t0 + j) * 2];
    s[j] = tab[(row * (D / 2) + t0 + j) * 2 + 1];
  }
  for (int z = 0; z < sides; ++z)
    for (int h = 0; h < heads; ++h) {
      const int64_t base = (int64_t(h) * n + row) * D;
      const T* x = (z == 0 ? Q : K) + base;
      T* y = (z == 0 ? Qr : Kr) + base;
      T lo[4], hi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = x[t0 + j];
        hi[j] = x[t0 + j + D / 2];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y1, y2;
        rotate_pair(to_f32<T>(lo[j]), to_f32<T>(hi[j]), c[j], s[j], y1, y2);
        lo[j] = from_f32<T>(y1);
        hi[j] = from_f32<T>(y2);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        y[t0 + j] = lo[j];
        y[t0 + j + D / 2] = hi[j];
      }
    }
}

// ------------------------------------------------- adjoint of the rotation
// Gradients of the rows before rotation from those of the rotated rows, in
// place: the rotation of each pair is orthogonal, so its adjoint rotates by
// -i theta_t:
//   g_t       =  g'_t cos(i theta_t) + g'_{t+d/2} sin(i theta_t)
//   g_{t+d/2} = -g'_t sin(i theta_t) + g'_{t+d/2} cos(i theta_t)
// in fp32 (each product and sum rounded once), then to the row type. Thread
// layout as rope_kernel's; X holds `sides` tensors one after another.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void rope_adjoint_kernel(T* X0, T* X1,
                                                                const float* __restrict__ tab,
                                                                int64_t n, int heads) {
  constexpr int TPR = D / 8;
  constexpr int RPB = kThreads / TPR;
  const int64_t row = int64_t(blockIdx.x) * RPB + threadIdx.x / TPR;
  const int t0 = (threadIdx.x % TPR) * 4;
  if (row >= n) return;
  float c[4], s[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c[j] = tab[(row * (D / 2) + t0 + j) * 2];
    s[j] = -tab[(row * (D / 2) + t0 + j) * 2 + 1];
  }
  for (int z = 0; z < 2; ++z)
    for (int h = 0; h < heads; ++h) {
      T* x = (z == 0 ? X0 : X1) + (int64_t(h) * n + row) * D;
      T lo[4], hi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        lo[j] = x[t0 + j];
        hi[j] = x[t0 + j + D / 2];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y1, y2;
        rotate_pair(to_f32<T>(lo[j]), to_f32<T>(hi[j]), c[j], s[j], y1, y2);
        lo[j] = from_f32<T>(y1);
        hi[j] = from_f32<T>(y2);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[t0 + j] = lo[j];
        x[t0 + j + D / 2] = hi[j];
      }
    }
}

// ------------------------------------------- rotation + hash (bf16 rows)
// Rotated value of element t of a raw bf16 row (for the exact-sign fallback).
template <int D>
__device__ __forceinline__ double rotated_at(const bf16_t* __restrict__ xr,
                                             const float* __restrict__ trow, int t) {
  const int p = t < D / 2 ? t : t - D / 2;
  float y1, y2;
  rotate_pair(bf16_to_f32(xr[p]), bf16_to_f32(xr[p + D / 2]), trow[2 * p], trow[2 * p + 1], y1,
              y2);
  return double(bf16_to_f32(f32_to_bf16(t < D / 2 ? y1 : y2)));
}

// grid: ceil(n / kRopeRows); codes_q/codes_k: [heads][n]
template <int D>
__global__ __launch_bounds__(kThreads) void rope_hash_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, bf16_t* __restrict__ Qr,
    bf16_t* __restrict__ Kr, const float* __restrict__ tab, const float* __restrict__ G,
    const bf16_t* __restrict__ Gb, int r, int64_t n, int heads, uint8_t* __restrict__ codes_q,
    uint8_t* __restrict__ codes_k) {
  constexpr int KS = D / 32;                  // 16-byte chunks per lane and row
  constexpr int KH = KS / 2;                  // chunks holding first members of pairs
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int64_t wbase = int64_t(blockIdx.x) * kRopeRows + wave * kRowsPerWave;
  const int64_t row = wbase + col;            // the row this lane loads
  const bool live = row < n;
  // table entries of this lane's pairs: t = 32s + 8kq + j, s < KH
  float c[KH][8], s[KH][8];
#pragma unroll
  for (int k = 0; k < KH; ++k)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = 32 * k + 8 * kq + j;
      c[k][j] = live ? tab[(row * (D / 2) + t) * 2] : 0.f;
      s[k][j] = live ? tab[(row * (D / 2) + t) * 2 + 1] : 0.f;
    }
  constexpr float u = 0x1p-24f;
  constexpr float gamma = (D * u) / (1.f - D * u);
  // iterations it = z * heads + h (z = 0: Q, 1: K); the rows of iteration
  // it + 1 are loaded while iteration it is rotated and hashed
  const int iters = 2 * heads;
  auto load_rows = [&](int it, uint4* dst) __attribute__((always_inline)) {
    const int z = it >= heads;
    const int h = it - z * heads;
    const bf16_t* X = (z == 0 ? Q : K) + int64_t(h) * n * D;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      dst[k] = live ? *reinterpret_cast<const uint4*>(X + row * D + 32 * k + 8 * kq)
                    : make_uint4(0, 0, 0, 0);
  };
  uint4 nxt[KS];
  load_rows(0, nxt);
  for (int it = 0; it < iters; ++it) {
    const int z = it >= heads;
    const int h = it - z * heads;
    const int64_t hoff = int64_t(h) * n;
    const bf16_t* X = (z == 0 ? Q : K) + hoff * D;
    bf16_t* Y = (z == 0 ? Qr : Kr) + hoff * D;
    uint8_t* codes = (z == 0 ? codes_q : codes_k) + hoff;
    uint4 xa[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k) xa[k] = nxt[k];
    if (it + 1 < iters) load_rows(it + 1, nxt);
    // rotate the eight pairs of chunks (k, k + KH) in registers
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      const uint32_t a[4] = {xa[k].x, xa[k].y, xa[k].z, xa[k].w};
      const uint32_t b[4] = {xa[k + KH].x, xa[k + KH].y, xa[k + KH].z, xa[k + KH].w};
      uint32_t ya[4], yb[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float y1, y2, y3, y4;
        rotate_pair(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), c[k][2 * w],
                    s[k][2 * w], y1, y2);
        rotate_pair(__uint_as_float(a[w] & 0xFFFF0000u), __uint_as_float(b[w] & 0xFFFF0000u),
                    c[k][2 * w + 1], s[k][2 * w + 1], y3, y4);
        ya[w] = uint32_t(f32_to_bf16(y1)) | (uint32_t(f32_to_bf16(y3)) << 16);
        yb[w] = uint32_t(f32_to_bf16(y2)) | (uint32_t(f32_to_bf16(y4)) << 16);
      }
      xa[k] = make_uint4(ya[0], ya[1], ya[2], ya[3]);
      xa[k + KH] = make_uint4(yb[0], yb[1], yb[2], yb[3]);
    }
    if (live) {
#pragma unroll
      for (int k = 0; k < KS; ++k)
        *reinterpret_cast<uint4*>(Y + row * D + 32 * k + 8 * kq) = xa[k];
    }
    if (r == 0) {                           // no hyperplanes: every code is 0
      if (kq == 0 && live) codes[row] = 0;
      continue;
    }
    // sign pattern of the rotated rows (the MFMA projection of the hash)
    const float* Gh = G + int64_t(h) * r * D;
    const bf16_t* Gbh = Gb + int64_t(h) * 16 * D;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, aabs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const uint4 g = *reinterpret_cast<const uint4*>(Gbh + col * D + 32 * k + 8 * kq);
      const uint4 ga = make_uint4(g.x & 0x7FFF7FFFu, g.y & 0x7FFF7FFFu, g.z & 0x7FFF7FFFu,
                                  g.w & 0x7FFF7FFFu);
      const uint4 v = xa[k];
      const uint4 va = make_uint4(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu,
                                  v.w & 0x7FFF7FFFu);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v),
                                                    __builtin_bit_cast(bf16x8_t, g), acc, 0, 0,
                                                    0);
      aabs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va),
                                                     __builtin_bit_cast(bf16x8_t, ga), aabs,
                                                     0, 0, 0);
    }
    uint64_t bpos[4], buns[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool sure = fabsf(acc[i]) > 3.f * gamma * aabs[i] + 0x1p-100f;
      bpos[i] = __ballot(col < r && sure && acc[i] > 0.f);
      buns[i] = __ballot(col < r && !sure);
    }
    // lane l < 16 owns row l: C row 4(l/4) + l%4 sits in ballot l%4 at bit 16(l/4)
    const int64_t orow = wbase + lane;
    if (lane < 16 && orow < n) {
      const int i = lane & 3;
      const int sh = 16 * (lane >> 2);
      const uint64_t bp = i == 0 ? bpos[0] : i == 1 ? bpos[1] : i == 2 ? bpos[2] : bpos[3];
      const uint64_t bu = i == 0 ? buns[0] : i == 1 ? buns[1] : i == 2 ? buns[2] : buns[3];
      uint32_t bits = uint32_t(bp >> sh) & 0xFFu;
      const uint32_t unsure = uint32_t(bu >> sh) & 0xFFu;
      if (unsure) {
        // fp64 sums in order t over the rotated row, recomputed from the raw row
        const bf16_t* xr = X + orow * D;
        const float* trow = tab + orow * (D / 2) * 2;
        double acc8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int t = 0; t < D; ++t) {
          const double x = rotated_at<D>(xr, trow, t);
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if ((unsure >> k) & 1u) acc8[k] = fma(x, double(Gh[k * D + t]), acc8[k]);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if ((unsure >> k) & 1u) bits = acc8[k] > 0.0 ? (bits | (1u << k)) : (bits & ~(1u << k));
      }
      uint32_t g = bits;        // Gray rank: bit k = parity of bits k..7
      g ^= g >> 1;
      g ^= g >> 2;
      g ^= g >> 4;
      codes[orow] = uint8_t(g);
    }
    }
}

}  // namespace

void host_rope_table(int64_t n, int d, double base, float* out) {
  // called through pointers, so that the C library's functions are used as
  // they are (no folding or vector variants)
  double (*volatile pw)(double, double) = std::pow;
  double (*volatile cs)(double) = std::cos;
  double (*volatile sn)(double) = std::sin;
  const int half = d / 2;
  std::vector<double> theta(half);
  for (int t = 0; t < half; ++t) theta[t] = pw(base, -2.0 * t / d);
  for (int64_t i = 0; i < n; ++i)
    for (int t = 0; t < half; ++t) {
      const double a = double(i) * theta[t];
      out[(i * half + t) * 2] = float(cs(a));
      out[(i * half + t) * 2 + 1] = float(sn(a));
    }
}

// Rotates Q and K into Qr and Kr; with hash, also writes the sortLSH codes
// of the rotated rows into the plan's code regions (bf16: one fused pass;
// fp32: rotation, then the hash kernel over the rotated rows).
int launch_rope_adjoint(void* dQ, void* dK, int64_t n, int d, int heads, int dtype,
                        const float* tab, hipStream_t s) {
  if (n == 0 || heads == 0) return HA_OK;
  ProfRange pr("rope_adjoint", s);
  const int tpr = d / 8;
  const dim3 grid(unsigned(ceil_div(n, int64_t(kThreads / tpr))));
  if (dtype == HA_BF16) {
    auto k = d == 128 ? rope_adjoint_kernel<bf16_t, 128> : rope_adjoint_kernel<bf16_t, 64>;
    hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, static_cast<bf16_t*>(dQ),
                       static_cast<bf16_t*>(dK), tab, n, heads);
  } else {
    auto k = d == 128 ? rope_adjoint_kernel<float, 128> : rope_adjoint_kernel<float, 64>;
    hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, static_cast<float*>(dQ),
                       static_cast<float*>(dK), tab, n, heads);
  }
  HA_LAUNCH_CHECK("rope_adjoint");
  return HA_OK;
}

int launch_rope(const Plan& p, const void* Q, const void* K, void* Qr, void* Kr,
                const float* tab, bool hash, const float* G, const uint16_t* Gb, void* ws,
                hipStream_t s) {
  char* w = static_cast<char*>(ws);
  if (hash && p.dtype == HA_BF16) {
    ProfRange pr("rope_hash", s);
    const dim3 grid(unsigned(ceil_div(p.n, int64_t(kRopeRows))));
    auto* cq = reinterpret_cast<uint8_t*>(w + p.off[HA_WS_CODES_Q]);
    auto* ck = reinterpret_cast<uint8_t*>(w + p.off[HA_WS_CODES_K]);
    auto* q = static_cast<const bf16_t*>(Q);
    auto* k = static_cast<const bf16_t*>(K);
    auto* qr = static_cast<bf16_t*>(Qr);
    auto* kr = static_cast<bf16_t*>(Kr);
    auto* gb = reinterpret_cast<const bf16_t*>(Gb);
    if (p.d == 128)
      hipLaunchKernelGGL(rope_hash_kernel<128>, grid, dim3(kThreads), 0, s, q, k, qr, kr, tab, G,
                         gb, p.r, p.n, p.heads, cq, ck);
    else
      hipLaunchKernelGGL(rope_hash_kernel<64>, grid, dim3(kThreads), 0, s, q, k, qr, kr, tab, G,
                         gb, p.r, p.n, p.heads, cq, ck);
    HA_LAUNCH_CHECK("rope_hash");
    return HA_OK;
  }
  {
    ProfRange pr("rope", s);
    const int rpb = kThreads / (p.d / 8);
    const dim3 grid(unsigned(ceil_div(p.n, int64_t(rpb))));
    if (p.dtype == HA_BF16) {
      auto* q = static_cast<const bf16_t*>(Q);
      auto* k = static_cast<const bf16_t*>(K);
      auto* qr = static_cast<bf16_t*>(Qr);
      auto* kr = static_cast<bf16_t*>(Kr);
      if (p.d == 128)
        hipLaunchKernelGGL((rope_kernel<bf16_t, 128>), grid, dim3(kThreads), 0, s, q, k, qr, kr,
                           tab, p.n, p.heads, 2);
      else
        hipLaunchKernelGGL((rope_kernel<bf16_t, 64>), grid, dim3(kThreads), 0, s, q, k, qr, kr,
                           tab, p.n, p.heads, 2);
    } else {
      auto* q = static_cast<const float*>(Q);
      auto* k = static_cast<const float*>(K);
      auto* qr = static_cast<float*>(Qr);
      auto* kr = static_cast<float*>(Kr);
      if (p.d == 128)
        hipLaunchKernelGGL((rope_kernel<float, 128>), grid, dim3(kThreads), 0, s, q, k, qr, kr,
                           tab, p.n, p.heads, 2);
      else
        hipLaunchKernelGGL((rope_kernel<float, 64>), grid, dim3(kThreads), 0, s, q, k, qr, kr,
                           tab, p.n, p.heads, 2);
    }
    HA_LAUNCH_CHECK("rope");
  }
  if (hash) return launch_hash(p, Qr, Kr, nullptr, G, Gb, ws, s);
  return HA_OK;
}

}  // namespace ha
