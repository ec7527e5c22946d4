// Front end of the pass: the Hamming-sorted LSH of every Q and K row and the
// squared row norms of V, then the integer V-norm sampling weights and their
// prefix sums.
//
// Hash (HA page, "Algorithm", Definition 1, as read here): bit k of a row x
// is the sign of <x, g_k> for the head's hyperplane g_k, where the sign is
// that of the fp64 sum of x_t g_kt in order t = 0..d-1; the code is the Gray
// rank of the bit pattern. The kernel first forms the projection in fp32
// (16 lanes per row, reduced across lanes). Any order of fp32 summation is
// within gamma_d * sum_t |x_t g_kt| <= gamma_d |x| |g_k| of the exact value,
// gamma_d = d u / (1 - d u), u = 2^-24 (the classical dot-product bound), and
// the fp64 sequential sum is far closer still. So when
// |p32| > 4 gamma_d |x| |g_k| (plus a floor against underflow), the fp32 sign
// is the sign of the exact value and of the fp64 sequential sum; otherwise
// the row's first lane recomputes the fp64 sequential sum itself. Every code
// therefore equals the definition's, not just with high probability.
//
// V norms (HA page, "Method overview" / "Algorithm": sample rows of V by
// their squared l2 norms): a_j = fp64 sum of v_jt^2 in order t (each square
// is exact in fp64), one thread per row. Integer weights
// W_j = ceil(2^32 a_j / max_j a_j) and their exclusive prefix sums P make
// sampling exact integer arithmetic.
#include "common.h"
#include "device_util.h"

namespace ha {

namespace {

struct VBlock {
  double amax;
  unsigned long long wsum;
};

constexpr int kThreads = 256;

template <typename T, int D>
__device__ void hash_rows(const T* __restrict__ X, const float* __restrict__ Gh, int r,
                          int64_t n, int64_t row0, uint8_t* __restrict__ codes) {
  constexpr int LPR = D / 8;          // lanes per row, 8 elements each
  constexpr int RPW = 64 / LPR;       // rows per wave step
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int c = lane % LPR;
  const int sub = lane / LPR;

  float g[8][8];
  float gn[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k < r) {
#pragma unroll
      for (int j = 0; j < 8; ++j) g[k][j] = Gh[k * D + c * 8 + j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) g[k][j] = 0.f;
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += g[k][j] * g[k][j];
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    gn[k] = sqrtf(s);
  }
  constexpr float u = 0x1p-24f;
  constexpr float gamma = (D * u) / (1.f - D * u);
  const int64_t end = row0 + kThreads < n ? row0 + kThreads : n;

  for (int64_t rb = row0 + int64_t(wave) * RPW; rb < end; rb += 4 * RPW) {
    const int64_t row = rb + sub;
    const bool valid = row < end;
    float x[8];
    if (valid) {
      load8<T>(X + row * D + c * 8, x);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = 0.f;
    }
    float p[8];
    float sx = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) sx += x[j] * x[j];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) a += x[j] * g[k][j];
      p[k] = a;
    }
#pragma unroll
    for (int o = LPR / 2; o > 0; o >>= 1) {
      sx += __shfl_xor(sx, o, 64);
#pragma unroll
      for (int k = 0; k < 8; ++k) p[k] += __shfl_xor(p[k], o, 64);
    }
    const bool row_unsure = !(sx >= 0x1p-100f && sx <= 3.0e38f);
    const float nx = sqrtf(sx);
    uint32_t bits = 0, unsure = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if (k < r) {
        const float thr = 4.f * gamma * nx * gn[k] + 0x1p-100f;
        if (row_unsure || !(fabsf(p[k]) > thr))
          unsure |= 1u << k;
        else if (p[k] > 0.f)
          bits |= 1u << k;
      }
    }
    if (valid && c == 0) {
      if (unsure) {
        const T* xr = X + row * D;
        for (int k = 0; k < r; ++k) {
          if (!((unsure >> k) & 1u)) continue;
          double acc = 0.0;
          for (int t = 0; t < D; ++t)
            acc = fma(double(to_f32<T>(xr[t])), double(Gh[k * D + t]), acc);
          if (acc > 0.0) bits |= 1u << k;
        }
      }
      uint32_t h = bits;        // Gray rank: bit k = parity of bits k..7
      h ^= h >> 1;
      h ^= h >> 2;
      h ^= h >> 4;
      codes[row] = uint8_t(h);
    }
  }
}

template <typename T, int D>
__device__ void vnorm_rows(const T* __restrict__ V, int64_t n, int64_t row0,
                           double* __restrict__ va, VBlock* __restrict__ blk) {
  __shared__ double wmax[kThreads / 64];
  const int64_t row = row0 + threadIdx.x;
  double a = 0.0;
  if (row < n) {
    const T* vr = V + row * D;
    for (int c = 0; c < D / 8; ++c) {
      float v[8];
      load8<T>(vr + c * 8, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) a = fma(double(v[j]), double(v[j]), a);
    }
    va[row] = a;
  }
  const double wm = wave_max(a);
  if (lane_id() == 0) wmax[threadIdx.x >> 6] = wm;
  __syncthreads();
  if (threadIdx.x == 0) {
    double mx = wmax[0];
    for (int w = 1; w < kThreads / 64; ++w) mx = wmax[w] > mx ? wmax[w] : mx;
    blk->amax = mx;
  }
}

// grid: (ceil(n/256), heads, 2 or 3); z = 0: hash Q, 1: hash K, 2: V norms
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void hash_vnorm_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const float* __restrict__ G, int r, int64_t n, uint8_t* __restrict__ codes_q,
    uint8_t* __restrict__ codes_k, double* __restrict__ va, VBlock* __restrict__ vblk) {
  const int head = blockIdx.y;
  const int side = blockIdx.z;
  const int64_t row0 = int64_t(blockIdx.x) * kThreads;
  const int64_t hoff = int64_t(head) * n;
  if (side == 2) {
    vnorm_rows<T, D>(V + hoff * D, n, row0, va + hoff,
                     vblk + int64_t(head) * gridDim.x + blockIdx.x);
    return;
  }
  const T* X = (side == 0 ? Q : K) + hoff * D;
  uint8_t* codes = (side == 0 ? codes_q : codes_k) + hoff;
  hash_rows<T, D>(X, G + int64_t(head) * r * D, r, n, row0, codes);
}

__device__ __forceinline__ double block_max_f64(double x, double* sh) {
  x = wave_max(x);
  if (lane_id() == 0) sh[threadIdx.x >> 6] = x;
  __syncthreads();
  double m = sh[0];
  for (int w = 1; w < kThreads / 64; ++w) m = sh[w] > m ? sh[w] : m;
  __syncthreads();
  return m;
}

__device__ __forceinline__ uint64_t block_sum_u64(uint64_t x, uint64_t* sh) {
  x = wave_sum(x);
  if (lane_id() == 0) sh[threadIdx.x >> 6] = x;
  __syncthreads();
  uint64_t s = 0;
  for (int w = 0; w < kThreads / 64; ++w) s += sh[w];
  __syncthreads();
  return s;
}

// grid: (vblocks, heads). W_j = ceil(2^32 * (a_j / M)), M = max over the head.
__global__ __launch_bounds__(kThreads) void vnorm_weights_kernel(
    int64_t n, const double* __restrict__ va, VBlock* __restrict__ vblk,
    uint64_t* __restrict__ W) {
  __shared__ double shd[kThreads / 64];
  __shared__ uint64_t shu[kThreads / 64];
  const int64_t nb = gridDim.x;
  const VBlock* hb = vblk + int64_t(blockIdx.y) * nb;
  double M = 0.0;
  for (int64_t b = threadIdx.x; b < nb; b += kThreads) M = hb[b].amax > M ? hb[b].amax : M;
  M = block_max_f64(M, shd);
  const int64_t row = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  uint64_t w = 0;
  if (row < n) {
    const double a = va[int64_t(blockIdx.y) * n + row];
    if (M > 0.0) w = uint64_t(ceil(ldexp(a / M, 32)));
    W[int64_t(blockIdx.y) * n + row] = w;
  }
  const uint64_t s = block_sum_u64(w, shu);
  if (threadIdx.x == 0) vblk[int64_t(blockIdx.y) * nb + blockIdx.x].wsum = s;
}

// grid: (vblocks, heads). P[j] = sum_{i<j} W_i, P[n] = total.
__global__ __launch_bounds__(kThreads) void vnorm_prefix_kernel(
    int64_t n, const VBlock* __restrict__ vblk, const uint64_t* __restrict__ W,
    uint64_t* __restrict__ P) {
  __shared__ uint64_t shu[kThreads / 64];
  __shared__ uint64_t wtot[kThreads / 64];
  const int64_t nb = gridDim.x;
  const VBlock* hb = vblk + int64_t(blockIdx.y) * nb;
  uint64_t pre = 0;
  for (int64_t b = threadIdx.x; b < blockIdx.x; b += kThreads) pre += hb[b].wsum;
  pre = block_sum_u64(pre, shu);
  const int64_t row = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const uint64_t w = row < n ? W[int64_t(blockIdx.y) * n + row] : 0;
  const uint64_t incl_w = wave_incl_scan(w);
  const int wave = threadIdx.x >> 6;
  if (lane_id() == 63) wtot[wave] = incl_w;
  __syncthreads();
  uint64_t before = 0;
  for (int i = 0; i < wave; ++i) before += wtot[i];
  const uint64_t incl = pre + before + incl_w;
  uint64_t* Ph = P + int64_t(blockIdx.y) * (n + 1);
  if (row < n) Ph[row] = incl - w;
  if (row == n - 1) Ph[n] = incl;
}

template <typename T, int D>
void launch_hash_t(dim3 grid, hipStream_t s, const void* Q, const void* K, const void* V,
                   const float* G, int r, int64_t n, uint8_t* cq, uint8_t* ck, double* va,
                   VBlock* vb) {
  hipLaunchKernelGGL((hash_vnorm_kernel<T, D>), grid, dim3(kThreads), 0, s,
                     static_cast<const T*>(Q), static_cast<const T*>(K),
                     static_cast<const T*>(V), G, r, n, cq, ck, va, vb);
}

void dispatch_hash(int dtype, int d, dim3 grid, hipStream_t s, const void* Q, const void* K,
                   const void* V, const float* G, int r, int64_t n, uint8_t* cq, uint8_t* ck,
                   double* va, VBlock* vb) {
  if (dtype == HA_BF16) {
    if (d == 128) launch_hash_t<bf16_t, 128>(grid, s, Q, K, V, G, r, n, cq, ck, va, vb);
    else launch_hash_t<bf16_t, 64>(grid, s, Q, K, V, G, r, n, cq, ck, va, vb);
  } else {
    if (d == 128) launch_hash_t<float, 128>(grid, s, Q, K, V, G, r, n, cq, ck, va, vb);
    else launch_hash_t<float, 64>(grid, s, Q, K, V, G, r, n, cq, ck, va, vb);
  }
}

}  // namespace

int launch_hash(const Plan& p, const void* Q, const void* K, const void* V, const float* G,
                void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  dim3 grid(unsigned(p.vblocks), unsigned(p.heads), p.product ? 3u : 2u);
  ProfRange pr("hash_vnorm", s);
  dispatch_hash(p.dtype, p.d, grid, s, Q, K, V, G, p.r, p.n,
                reinterpret_cast<uint8_t*>(w + p.off[HA_WS_CODES_Q]),
                reinterpret_cast<uint8_t*>(w + p.off[HA_WS_CODES_K]),
                p.product ? reinterpret_cast<double*>(w + p.off[HA_WS_VNORM_A]) : nullptr,
                p.product ? reinterpret_cast<VBlock*>(w + p.off[HA_WS_VNORM_BLK]) : nullptr);
  HA_LAUNCH_CHECK("hash_vnorm");
  return HA_OK;
}

int launch_hash_one(const void* X, int64_t n, int d, int heads, int r, int dtype,
                    const float* G, uint8_t* codes, hipStream_t s) {
  dim3 grid(unsigned(ceil_div(n, kThreads)), unsigned(heads), 1u);
  ProfRange pr("hash_vnorm", s);
  dispatch_hash(dtype, d, grid, s, X, X, X, G, r, n, codes, codes, nullptr, nullptr);
  HA_LAUNCH_CHECK("hash_vnorm");
  return HA_OK;
}

int launch_vnorm_scan(const Plan& p, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  dim3 grid(unsigned(p.vblocks), unsigned(p.heads));
  auto* va = reinterpret_cast<const double*>(w + p.off[HA_WS_VNORM_A]);
  auto* vb = reinterpret_cast<VBlock*>(w + p.off[HA_WS_VNORM_BLK]);
  auto* W = reinterpret_cast<uint64_t*>(w + p.off[HA_WS_VNORM_W]);
  auto* P = reinterpret_cast<uint64_t*>(w + p.off[HA_WS_VNORM_P]);
  {
    ProfRange pr("vnorm_weights", s);
    hipLaunchKernelGGL(vnorm_weights_kernel, grid, dim3(kThreads), 0, s, p.n, va, vb, W);
    HA_LAUNCH_CHECK("vnorm_weights");
  }
  {
    ProfRange pr("vnorm_prefix", s);
    hipLaunchKernelGGL(vnorm_prefix_kernel, grid, dim3(kThreads), 0, s, p.n, vb, W, P);
    HA_LAUNCH_CHECK("vnorm_prefix");
  }
  return HA_OK;
}

}  // namespace ha
