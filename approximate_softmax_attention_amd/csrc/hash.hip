// Front end of the pass: the Hamming-sorted LSH of every Q and K row and the
// squared row norms of V, then the integer V-norm sampling weights and their
// prefix sums.
//
// Hash (HA page, "Algorithm", Definition 1, as read here): bit k of a row x
// is the sign of <x, g_k> for the head's hyperplane g_k, where the sign is
// that of the fp64 sum of x_t g_kt in order t = 0..d-1; the code is the Gray
// rank of the bit pattern. The kernel first forms the projection in fp32
// (bf16 inputs: on MFMA, below; fp32 inputs: 16 lanes per row, reduced
// across lanes). Any order of fp32 summation is
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
constexpr int kHashRows = 1024;   // rows hashed per work-group

// Sum over the D/8 consecutive lanes that hold one row (8 or 16 lanes), by
// DPP butterflies inside a 16-lane row: swap neighbours, swap pairs, mirror
// within 8, mirror within 16. Every lane of the group ends with the total.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int LANES>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);          // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);          // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);         // row_half_mirror
  if (LANES == 16) x += dpp<0x140>(x);   // row_mirror
  return x;
}

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
    gn[k] = sqrtf(group_sum<LPR>(s));
  }
  constexpr float u = 0x1p-24f;
  constexpr float gamma = (D * u) / (1.f - D * u);
  const int64_t end = row0 + kThreads < n ? row0 + kThreads : n;

  // each wave takes row groups wave, wave+4, ...; NG groups per batch with
  // all of the batch's loads issued before any arithmetic
  constexpr int NG = 4;
  for (int64_t rb0 = row0 + int64_t(wave) * RPW; rb0 < end; rb0 += NG * 4 * RPW) {
    float x[NG][8];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int64_t row = rb0 + int64_t(gi) * 4 * RPW + sub;
      if (row < end) {
        load8<T>(X + row * D + c * 8, x[gi]);
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[gi][j] = 0.f;
      }
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int64_t row = rb0 + int64_t(gi) * 4 * RPW + sub;
      const bool valid = row < end;
      float p[8];
      float sx = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) sx += x[gi][j] * x[gi][j];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a += x[gi][j] * g[k][j];
        p[k] = a;
      }
      sx = group_sum<LPR>(sx);
#pragma unroll
      for (int k = 0; k < 8; ++k) p[k] = group_sum<LPR>(p[k]);
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
}

// bf16 rows: the projections X G^T are a small contraction (d x 8), done on
// v_mfma_f32_16x16x32_bf16. Every hyperplane entry is a bf16 value, so each
// product is exact in fp32; a second MFMA over |X| |G|^T yields
// S_k = sum_t |x_t g_kt| (all terms positive). The unit's internal rounding
// is not specified by the ISA, so the margin is chosen to hold under either
// of two models: (A) every internal addition faithfully rounded (relative
// error < 2u) in any order, giving |p32 - p| <= 2 gamma_d S_k; (B) each
// instruction aligning its 33 addends to the largest, keeping >= 23 fraction
// bits, truncating, adding exactly and rounding once, giving
// |p32 - p| < 68 u (d/32) S_k ~ 2.13 gamma_d S_k. In both the computed S_k is
// within a factor (1 - 2.13 gamma_d) of the true one, so
// |p32| > 3 gamma_d S_k + 2^-100 fixes the sign of p and of its fp64
// sequential sum. Rows with an uncertain bit recompute it in fp64 in order t.
// Each wave takes 16 rows per step: A = 16 rows x 32 elements (lane l: row
// l%16, elements 8(l/16)..+7 of the step), B = the hyperplanes (lane l:
// hyperplane l%16, zero when >= r). C gives lane l hyperplane l%16 of rows
// 4(l/16)..+3; per row the r sign bits are gathered with wave ballots.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
__device__ void hash_rows_mfma(const bf16_t* __restrict__ X, const float* __restrict__ Gh,
                               const bf16_t* __restrict__ Gbh, int r, int64_t n, int64_t row0,
                               uint8_t* __restrict__ codes) {
  constexpr int KS = D / 32;
  constexpr int STEPS = 4;                     // 4 x 16 rows per wave and batch
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int kq = lane >> 4;
  bf16x8_t gb[KS], gab[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const uint4 v = *reinterpret_cast<const uint4*>(Gbh + col * D + 32 * s + 8 * kq);
    gb[s] = __builtin_bit_cast(bf16x8_t, v);
    gab[s] = __builtin_bit_cast(bf16x8_t, make_uint4(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu,
                                                     v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
  }
  constexpr float u = 0x1p-24f;
  constexpr float gamma = (D * u) / (1.f - D * u);
  for (int batch = 0; batch < kHashRows / kThreads; ++batch) {
  const int64_t rbatch = row0 + int64_t(batch) * kThreads;
  const int64_t end = rbatch + kThreads < n ? rbatch + kThreads : n;
  const int64_t wbase = rbatch + 64 * wave;
  uint4 xa[STEPS][KS];
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    const int64_t row = wbase + 16 * st + col;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      xa[st][s] = row < end ? *reinterpret_cast<const uint4*>(X + row * D + 32 * s + 8 * kq)
                            : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int st = 0; st < STEPS; ++st) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f}, aabs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const uint4 v = xa[st][s];
      const uint4 va = make_uint4(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu, v.z & 0x7FFF7FFFu,
                                  v.w & 0x7FFF7FFFu);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, v), gb[s], acc,
                                                    0, 0, 0);
      aabs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, va), gab[s],
                                                     aabs, 0, 0, 0);
    }
    uint64_t bpos[4], buns[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool sure = fabsf(acc[i]) > 3.f * gamma * aabs[i] + 0x1p-100f;
      bpos[i] = __ballot(col < r && sure && acc[i] > 0.f);
      buns[i] = __ballot(col < r && !sure);
    }
    // lane l < 16 owns row l of the step: C row 4*(l/4) + l%4 sits in ballot
    // l%4 at bit offset 16*(l/4)
    const int64_t row = wbase + 16 * st + lane;
    if (lane < 16 && row < end) {
      const int i = lane & 3;
      const int sh = 16 * (lane >> 2);
      const uint64_t bp = i == 0 ? bpos[0] : i == 1 ? bpos[1] : i == 2 ? bpos[2] : bpos[3];
      const uint64_t bu = i == 0 ? buns[0] : i == 1 ? buns[1] : i == 2 ? buns[2] : buns[3];
      uint32_t bits = uint32_t(bp >> sh) & 0xFFu;
      const uint32_t unsure = uint32_t(bu >> sh) & 0xFFu;
      if (unsure) {
        // fp64 sums in order t for the uncertain hyperplanes, one pass over the row
        const uint4* xr = reinterpret_cast<const uint4*>(X + row * D);
        double acc8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        for (int c = 0; c < D / 8; ++c) {
          const uint4 v = xr[c];
          const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const uint32_t half = (j & 1) ? (wd[j >> 1] & 0xFFFF0000u) : (wd[j >> 1] << 16);
            const double x = double(__uint_as_float(half));
#pragma unroll
            for (int k = 0; k < 8; ++k)
              if ((unsure >> k) & 1u) acc8[k] = fma(x, double(Gh[k * D + 8 * c + j]), acc8[k]);
          }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if ((unsure >> k) & 1u) bits = acc8[k] > 0.0 ? (bits | (1u << k)) : (bits & ~(1u << k));
      }
      uint32_t h = bits;        // Gray rank: bit k = parity of bits k..7
      h ^= h >> 1;
      h ^= h >> 2;
      h ^= h >> 4;
      codes[row] = uint8_t(h);
    }
  }
  }
}

// Squared row norms of 256 rows (one per thread), summed in fp64 in order
// t = 0..d-1. bf16 rows are first brought into LDS with coalesced 16-byte
// loads (each wave stages 32 rows at a time; the chunks of a row are
// XOR-swizzled so that 32 lanes reading the same chunk of 32 different rows
// spread over the banks), then each lane walks its own row.
template <typename T, int D>
__device__ void vnorm_rows(const T* __restrict__ V, int64_t n, int64_t row0,
                           double* __restrict__ va, VBlock* __restrict__ blk) {
  __shared__ double wmax[kThreads / 64];
  const int64_t row = row0 + threadIdx.x;
  double a = 0.0;
  if constexpr (sizeof(T) == 2) {
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    __shared__ uint4 tile[kThreads / 64][32 * CPR];
    const int wave = threadIdx.x >> 6, lane = lane_id();
    uint4* tw = tile[wave];
    constexpr int PER = 32 * CPR / 64;         // 16-byte chunks per lane per half
    uint4 buf[2][PER];
    auto load_half = [&](int half, uint4* dst) {
      const int64_t rbase = row0 + 64 * wave + 32 * half;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int q = i * 64 + lane;           // chunk index within the 32 rows
        const int rr = q / CPR, c = q % CPR;
        dst[i] = rbase + rr < n ? *reinterpret_cast<const uint4*>(V + (rbase + rr) * D + c * 8)
                                : make_uint4(0, 0, 0, 0);
      }
    };
    load_half(0, buf[0]);
    load_half(1, buf[1]);                      // both halves in flight
#pragma unroll
    for (int half = 0; half < 2; ++half) {     // rows 32*half .. 32*half+31 of this wave
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int q = i * 64 + lane;
        const int rr = q / CPR, c = q % CPR;
        tw[rr * CPR + (c ^ (rr % CPR))] = buf[half][i];
      }
      __builtin_amdgcn_s_waitcnt(0);           // the wave's own LDS writes
      __builtin_amdgcn_wave_barrier();
      if ((lane >> 5) == half) {
        const int rr = lane & 31;
#pragma unroll
        for (int c = 0; c < CPR; ++c) {
          const uint4 v = tw[rr * CPR + (c ^ (rr % CPR))];
          const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const double lo = double(__uint_as_float(wd[j] << 16));
            const double hi = double(__uint_as_float(wd[j] & 0xFFFF0000u));
            a = fma(lo, lo, a);
            a = fma(hi, hi, a);
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (row >= n) a = 0.0;
  } else {
    if (row < n) {
      const T* vr = V + row * D;
      for (int c = 0; c < D / 8; ++c) {
        float v[8];
        load8<T>(vr + c * 8, v);
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fma(double(v[j]), double(v[j]), a);
      }
    }
  }
  if (row < n) va[row] = a;
  const double wm = wave_max(a);
  if (lane_id() == 0) wmax[threadIdx.x >> 6] = wm;
  __syncthreads();
  if (threadIdx.x == 0) {
    double mx = wmax[0];
    for (int w = 1; w < kThreads / 64; ++w) mx = wmax[w] > mx ? wmax[w] : mx;
    blk->amax = mx;
  }
}

// grid: (ceil(n/256), heads)
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void vnorm_rows_kernel(
    const T* __restrict__ V, int64_t n, double* __restrict__ va, VBlock* __restrict__ vblk) {
  const int64_t hoff = int64_t(blockIdx.y) * n;
  vnorm_rows<T, D>(V + hoff * D, n, int64_t(blockIdx.x) * kThreads, va + hoff,
                   vblk + int64_t(blockIdx.y) * gridDim.x + blockIdx.x);
}

// grid: (ceil(n/1024), heads, 2 or 1); z = 0 hashes Q, z = 1 hashes K
// bf16 rows fit in 128 registers, four waves per SIMD: 1024 resident
// work-groups, so that 2048 of them (n = 131072 at 8 heads, or n = 32768 at
// 32) run as two full rounds instead of two and a part. The fp32 path keeps
// its registers.
template <typename T> struct HashWaves { static constexpr int value = sizeof(T) == 2 ? 4 : 1; };

template <typename T, int D>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(HashWaves<T>::value))) void hash_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const float* __restrict__ G,
    const bf16_t* __restrict__ Gb, int r, int64_t n, uint8_t* __restrict__ codes_q,
    uint8_t* __restrict__ codes_k) {
  const int head = blockIdx.y;
  const int side = blockIdx.z;
  const int64_t row0 = int64_t(blockIdx.x) * kHashRows;
  const int64_t hoff = int64_t(head) * n;
  const T* X = (side == 0 ? Q : K) + hoff * D;
  uint8_t* codes = (side == 0 ? codes_q : codes_k) + hoff;
  if constexpr (sizeof(T) == 2) {
    hash_rows_mfma<D>(X, G + int64_t(head) * r * D, Gb + int64_t(head) * 16 * D, r, n, row0,
                      codes);
  } else {
    for (int b = 0; b < kHashRows / kThreads; ++b)
      hash_rows<T, D>(X, G + int64_t(head) * r * D, r, n, row0 + int64_t(b) * kThreads, codes);
  }
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

// r = 0 (no hyperplanes): every code is GrayRank(0) = 0. codes[z] is a
// [heads][n] array; blockIdx.y is the head, z the side.
__global__ __launch_bounds__(kThreads) void zero_codes_kernel(uint8_t* __restrict__ cq,
                                                              uint8_t* __restrict__ ck,
                                                              int64_t n) {
  uint8_t* c = (blockIdx.z == 0 ? cq : ck) + int64_t(blockIdx.y) * n;
  const int64_t i0 = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * 16;
  if (i0 + 16 <= n && (reinterpret_cast<uintptr_t>(c + i0) & 15) == 0) {
    *reinterpret_cast<uint4*>(c + i0) = make_uint4(0, 0, 0, 0);
  } else {
    const int64_t i1 = i0 + 16 < n ? i0 + 16 : n;
    for (int64_t i = i0; i < i1; ++i) c[i] = 0;
  }
}

int launch_zero_codes(uint8_t* cq, uint8_t* ck, int64_t n, int heads, int sides,
                      hipStream_t s) {
  const dim3 grid(unsigned(ceil_div(n, int64_t(kThreads) * 16)), unsigned(heads),
                  unsigned(sides));
  hipLaunchKernelGGL(zero_codes_kernel, grid, dim3(kThreads), 0, s, cq, ck, n);
  HA_LAUNCH_CHECK("hash");
  return HA_OK;
}

template <typename T, int D>
void launch_hash_t(dim3 grid, hipStream_t s, const void* Q, const void* K, const float* G,
                   const uint16_t* Gb, int r, int64_t n, uint8_t* cq, uint8_t* ck) {
  hipLaunchKernelGGL((hash_kernel<T, D>), grid, dim3(kThreads), 0, s, static_cast<const T*>(Q),
                     static_cast<const T*>(K), G, Gb, r, n, cq, ck);
}

template <typename T, int D>
void launch_vnorm_t(dim3 grid, hipStream_t s, const void* V, int64_t n, double* va, VBlock* vb) {
  hipLaunchKernelGGL((vnorm_rows_kernel<T, D>), grid, dim3(kThreads), 0, s,
                     static_cast<const T*>(V), n, va, vb);
}

void dispatch_hash(int dtype, int d, dim3 grid, hipStream_t s, const void* Q, const void* K,
                   const float* G, const uint16_t* Gb, int r, int64_t n, uint8_t* cq,
                   uint8_t* ck) {
  if (dtype == HA_BF16) {
    if (d == 128) launch_hash_t<bf16_t, 128>(grid, s, Q, K, G, Gb, r, n, cq, ck);
    else launch_hash_t<bf16_t, 64>(grid, s, Q, K, G, Gb, r, n, cq, ck);
  } else {
    if (d == 128) launch_hash_t<float, 128>(grid, s, Q, K, G, Gb, r, n, cq, ck);
    else launch_hash_t<float, 64>(grid, s, Q, K, G, Gb, r, n, cq, ck);
  }
}

void dispatch_vnorm(int dtype, int d, dim3 grid, hipStream_t s, const void* V, int64_t n,
                    double* va, VBlock* vb) {
  if (dtype == HA_BF16) {
    if (d == 128) launch_vnorm_t<bf16_t, 128>(grid, s, V, n, va, vb);
    else launch_vnorm_t<bf16_t, 64>(grid, s, V, n, va, vb);
  } else {
    if (d == 128) launch_vnorm_t<float, 128>(grid, s, V, n, va, vb);
    else launch_vnorm_t<float, 64>(grid, s, V, n, va, vb);
  }
}

}  // namespace

int launch_hash(const Plan& p, const void* Q, const void* K, const void* V, const float* G,
                const uint16_t* Gb, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  if (Q) {
    ProfRange pr("hash", s);
    auto* cq = reinterpret_cast<uint8_t*>(w + p.off[HA_WS_CODES_Q]);
    auto* ck = reinterpret_cast<uint8_t*>(w + p.off[HA_WS_CODES_K]);
    if (p.r == 0) {
      if (int rc = launch_zero_codes(cq, ck, p.n, p.heads, 2, s)) return rc;
    } else {
      dispatch_hash(p.dtype, p.d,
                    dim3(unsigned(ceil_div(p.n, kHashRows)), unsigned(p.heads), 2u), s, Q, K,
                    G, Gb, p.r, p.n, cq, ck);
      HA_LAUNCH_CHECK("hash");
    }
  }
  if (p.product && V) {
    ProfRange pr("vnorm_rows", s);
    dispatch_vnorm(p.dtype, p.d, dim3(unsigned(p.vblocks), unsigned(p.heads)), s, V, p.n,
                   reinterpret_cast<double*>(w + p.off[HA_WS_VNORM_A]),
                   reinterpret_cast<VBlock*>(w + p.off[HA_WS_VNORM_BLK]));
    HA_LAUNCH_CHECK("vnorm_rows");
  }
  return HA_OK;
}

int launch_hash_one(const void* X, int64_t n, int d, int heads, int r, int dtype,
                    const float* G, const uint16_t* Gb, uint8_t* codes, hipStream_t s) {
  ProfRange pr("hash", s);
  if (r == 0) return launch_zero_codes(codes, codes, n, heads, 1, s);
  dispatch_hash(dtype, d, dim3(unsigned(ceil_div(n, kHashRows)), unsigned(heads), 1u), s, X, X,
                G, Gb, r, n, codes, codes);
  HA_LAUNCH_CHECK("hash");
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
