// Device building blocks of the MFMA attention kernels (gfx950), shared by
// the forward kernels and the backward kernels: key tiles in LDS with
// XOR-swizzled 16-byte chunks, their loaders (buffer loads with LDS
// destination for bf16), the register fragments of the rows a wave owns,
// the per-lane LDS offsets of the MFMA fragment reads, and the per-XCD work
// queues of persistent launches.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16): a wave computes a 32 x 32 block
// X Y^T with the A operand (32 rows of X, 16 elements of the reduction per
// step) read from an LDS tile and the B operand (the wave's own 32 rows of
// Y) held in registers, so lane l owns column l & 31 of the result, and
// accumulator element i of lane l is row 8(i/4) + 4(l/32) + i%4. The
// transposing LDS read (ds_read_b64_tr_b16) gives the A operand of a product
// whose reduction runs over the tile's rows, in the order of those
// accumulator rows, so a block of probabilities feeds the next product
// directly as its B operand.
#pragma once

#include <cmath>

#include "common.h"
#include "device_util.h"

namespace ha {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kQW = 32;   // queries per wave; kAttnQ = kWaves * kQW
static_assert(kAttnQ == kWaves * kQW, "query tile");
// Wave priority while issuing an MFMA chain: the SIMD's arbiter then keeps
// the matrix unit fed from that wave while the other wave's softmax work
// fills the VALU.
constexpr int kMfmaPrio = 1;
constexpr int kSlotCap = 1024;   // key slots staged in LDS per window (gathered modes)


// ------------------------------------------------------------ tile buffers
template <typename T, int D> struct Buf;

// bf16: KT rows of K and V, D elements each, 16-byte chunks XOR-swizzled.
template <int D>
struct alignas(16) Buf<bf16_t, D> {
  static constexpr int KT = 128;
  static constexpr int CPR = D / 8;                    // 16-byte chunks per row
  // Physical chunk = logical chunk XOR swz(row). swz is a bijection on the
  // rows that share one 256-byte bank window pattern (16 rows for d = 128,
  // 8 row pairs for d = 64), so the rows of a K fragment read hit distinct
  // banks; its high bits follow the row's low bits, so the four consecutive
  // rows of one transposing V read fall in four different 64-byte bank
  // groups.
  __device__ static int swz(int row) {
    if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    const int u = (row >> 1) & 7;
    return ((u & 1) << 2) | (((u >> 2) & 1) << 1) | ((u >> 1) & 1);
  }
  // Tiles read by 16x16 transposing reads (the backward pass's key-major
  // kernels, d = 128): the same bijection with the row quarter bit-reversed
  // in the low bits, so that in any 8 aligned rows swz_t >> 1 is distinct as
  // well. A half-wave reads 8 rows x two adjacent chunks there, and under
  // swz rows r and r + 4 share one chunk pair (a 2-way bank conflict).
  __device__ static int swz_t(int row) {
    if (D == 128) return ((row & 3) << 2) | ((row >> 3) & 1) | (((row >> 2) & 1) << 1);
    return swz(row);
  }
  bf16_t k[KT * D];
  bf16_t v[KT * D];
  float w[KT];                                         // per-slot weight
};

// fp32: padded K rows and a padded V^T tile.
template <int D>
struct alignas(16) Buf<float, D> {
  static constexpr int KT = D == 128 ? 64 : 128;
  static constexpr int KS = D + 4;
  static constexpr int VS = KT + 4;
  static constexpr int CPR = D / 4;                    // 16-byte chunks per row
  static_assert((KT / 4) * CPR == kThreads, "one 4-key x 16-byte item per thread");
  float k[KT * KS];
  float v[D * VS];
  float w[KT];
};


__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(x[l], x[l ^ 32]) for every lane l
__device__ __forceinline__ float half_swap_max(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Raw buffer resource over one head's [n][d] tensor: loads take 32-bit byte
// offsets, and offsets past the end return zeros (used for masked rows).
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Logical work-group index with consecutive indices placed on the same XCD
// (work-groups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int64_t xcd_remap(int64_t x, int64_t n) {
  constexpr int64_t kXcd = 8;
  if (n % kXcd) return x;
  return (x % kXcd) * (n / kXcd) + x / kXcd;
}

// ---------------------------------------------------------------- loaders
// Pipe<T, D>::issue(buf, ...) starts loading one key tile; commit(buf) makes
// it complete in LDS (before the barrier that publishes it). RowFn maps a tile
// row to a key row of the head (-1: masked, zero-filled); WFn gives the
// slot's weight. bf16 tiles are laid out with Buf::swz, or with Buf::swz_t
// when issued as issue<true> (tiles read by 16x16 transposing reads).
template <typename T, int D> struct Pipe;

template <int D>
struct Pipe<bf16_t, D> {
  using B = Buf<bf16_t, D>;
  template <bool kTr = false, typename RowFn, typename WFn>
  __device__ __forceinline__ void issue(B& b, __amdgpu_buffer_rsrc_t Kr, __amdgpu_buffer_rsrc_t Vr,
                                        bool with_v, const RowFn& rowidx, const WFn& weight) {
    constexpr int PER = B::KT * B::CPR / kThreads;
    constexpr uint32_t RB = D * 2;
    const int wave = threadIdx.x >> 6;
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p0 = i * kThreads + wave * 64;           // wave-uniform chunk index
      const int p = p0 + lane;
      const int row = p / B::CPR;
      const int c = (p % B::CPR) ^ (kTr ? B::swz_t(row) : B::swz(row));   // chunk landing here
      const int r = rowidx(row);
      const uint32_t off = r >= 0 ? uint32_t(r) * RB + uint32_t(c) * 16u : kOob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(Kr, (lds_void_t*)(b.k + p0 * 8), 16, off, 0, 0, 0);
      if (with_v)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(Vr, (lds_void_t*)(b.v + p0 * 8), 16, off, 0, 0,
                                                 0);
    }
    if (threadIdx.x < B::KT) b.w[threadIdx.x] = weight(int(threadIdx.x));
  }
  __device__ __forceinline__ void commit(B&, bool) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
};

template <int D>
struct Pipe<float, D> {
  using B = Buf<float, D>;
  uint4 k[4], v[4];
  float w[4];
  template <typename RowFn, typename WFn>
  __device__ __forceinline__ void issue(B&, __amdgpu_buffer_rsrc_t Kr, __amdgpu_buffer_rsrc_t Vr,
                                        bool with_v, const RowFn& rowidx, const WFn& weight) {
    const int kg = threadIdx.x / B::CPR;
    const uint32_t cb = (threadIdx.x % B::CPR) * 16u;
    uint32_t off[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rowidx(4 * kg + i);
      w[i] = weight(4 * kg + i);
      off[i] = r >= 0 ? uint32_t(r) * (D * 4u) + cb : kOob;
      k[i] = buf_load16(Kr, off[i]);
    }
    if (with_v) {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = buf_load16(Vr, off[i]);
    }
  }
  __device__ __forceinline__ void commit(B& b, bool with_v) {
    const int kg = threadIdx.x / B::CPR;
    const int ch = threadIdx.x % B::CPR;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&b.k[(4 * kg + i) * B::KS + ch * 4]) = k[i];
    if (ch == 0) *reinterpret_cast<float4*>(&b.w[4 * kg]) = make_float4(w[0], w[1], w[2], w[3]);
    if (!with_v) return;
    // V^T[d][key]: the four keys' element j of this chunk as one 16-byte piece
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        e[i] = j == 0 ? v[i].x : j == 1 ? v[i].y : j == 2 ? v[i].z : v[i].w;
      *reinterpret_cast<uint4*>(&b.v[(ch * 4 + j) * B::VS + 4 * kg]) =
          make_uint4(e[0], e[1], e[2], e[3]);
    }
  }
};

// ------------------------------------------------------------ per-wave core
template <typename T, int D> struct QFrag;
template <int D> struct QFrag<bf16_t, D> { bf16x8_t v[D / 16]; };
template <int D> struct QFrag<float, D> { float v[D / 2]; };

template <typename T, int D>
__device__ __forceinline__ void load_q(QFrag<T, D>& q, __amdgpu_buffer_rsrc_t Qr, int64_t row) {
  const int g = lane_id() >> 5;
  constexpr uint32_t RB = D * sizeof(T);
  const uint32_t base = row >= 0 ? uint32_t(row) * RB : kOob;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      q.v[st] = __builtin_bit_cast(bf16x8_t, buf_load16(Qr, base + (16 * st + 8 * g) * 2));
  } else {
#pragma unroll
    for (int st = 0; st < D / 2; ++st)
      q.v[st] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              Qr, base + (2 * st + g) * 4, 0, 0));
  }
}

// Per-lane LDS byte offsets of the MFMA fragments within one bf16 tile:
//   k[st]:    K row ql of key block 0, chunk 2st+g (key block kb adds kb*32*D*2)
//   v[h][db]: transposing-read address for keys 4g + (i16>>2) + 8h of a
//             16-key step, columns 32db + 16*((lane>>4)&1) + 4*(i16&3)
//             (step st of key block kb adds (32kb + 16st)*D*2)
template <typename T, int D> struct LaneOffs { };
template <int D>
struct LaneOffs<bf16_t, D> {
  using B = Buf<bf16_t, D>;
  uint32_t k[D / 16];
  uint32_t v[2][D / 32];
  // Derived from a copy of the lane id that the compiler cannot see through,
  // so that the offsets are formed per work item rather than held in
  // registers across a persistent kernel's item loop.
  __device__ __forceinline__ void init() {
    int lane = lane_id();
    asm volatile("" : "+v"(lane));
    const int ql = lane & 31, g = lane >> 5, i16 = lane & 15;
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      k[st] = uint32_t(ql * B::CPR + ((2 * st + g) ^ B::swz(ql))) * 16u;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 4 * g + (i16 >> 2) + 8 * h;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int d = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (i16 & 3);
        v[h][db] = uint32_t(row * B::CPR + ((d >> 3) ^ B::swz(row))) * 16u + uint32_t(d & 7) * 2u;
      }
    }
  }
};
template <int D>
struct LaneOffs<float, D> {
  __device__ __forceinline__ void init() {}
};


__device__ __forceinline__ int key_of(int kb, int i, int g) {
  return 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
}


// threadIdx.x through a copy the compiler cannot see through: the epilogue's
// per-thread offsets are then formed where they are used instead of being
// hoisted out of a persistent kernel's item loop, where they would hold
// registers across the tile loop.
__device__ __forceinline__ int opaque_tid() {
  int t = int(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}


// 16 raw bytes <-> E values of T as floats
template <typename T>
__device__ __forceinline__ void unpack16(uint4 raw, float* v) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    v[0] = __uint_as_float(raw.x); v[1] = __uint_as_float(raw.y);
    v[2] = __uint_as_float(raw.z); v[3] = __uint_as_float(raw.w);
  }
}
template <typename T>
__device__ __forceinline__ uint4 pack16(const float* v) {
  if constexpr (sizeof(T) == 2) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = uint32_t(f32_to_bf16(v[2 * i])) | (uint32_t(f32_to_bf16(v[2 * i + 1])) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3]));
  }
}

// Waves per SIMD to aim for: with bf16 and d = 64 two work-groups fit a
// CU's LDS, so those kernels keep to the 128 registers that four waves per
// SIMD allow.
template <typename T, int D> struct WavesPerEu {
  static constexpr int value = sizeof(T) == 2 && D == 64 ? 4 : 2;
};

// ------------------------------------------------------------- work queues
// A persistent launch runs one work-group per resident slot of the device.
// Work items are split into kQueues contiguous ranges, one per XCD; a
// work-group takes items from the queue of the XCD it runs on and, once that
// one is empty, from the others in turn. Neighbouring items (which share key
// blocks or sample lists) so run on the same XCD and share its L2, and no
// work-group waits for the in-order dispatch of others. The next item's
// counter is fetched while the current item runs.
__device__ __forceinline__ int hw_xcc() {
  // HW_REG_XCC_ID (hardware register 20), all 32 bits
  return int(__builtin_amdgcn_s_getreg((31 << 11) | 20)) & (kQueues - 1);
}

// Item for counter value `taken` of queue qi, or the next free item of the
// following queues; -1 when every queue is empty. Called by one thread.
__device__ __forceinline__ int64_t queue_resolve(uint32_t* ctr, uint32_t items, int& qi,
                                              uint32_t taken) {
  const uint32_t per = (items + kQueues - 1) / kQueues;
  for (int k = 0; k < kQueues; ++k) {
    const uint32_t lo = min(items, uint32_t(qi) * per);
    const uint32_t hi = min(items, lo + per);
    if (taken < hi - lo) return int64_t(lo + taken);
    if (k + 1 == kQueues) break;
    qi = (qi + 1) & (kQueues - 1);
    taken = atomicAdd(&ctr[qi], 1u);
  }
  return -1;
}


// Work-groups of kernel k (kThreads threads each) that the device holds at
// once, cached per device and kernel.
template <typename Kern>
int resident_groups(Kern k) {
  return resident_groups_of(reinterpret_cast<const void*>(k), kThreads);
}


// Runs item_fn over this work-group's items: one (from the linear block
// index, remapped so that neighbouring items share an XCD) when the launch
// has no queue, else
// items taken from the queues until all are done. item_fn must contain a
// barrier before it returns.
// Args: a launch's arguments with `queue` (counters, or null) and `items`.
template <typename Args, typename ItemFn>
__device__ __forceinline__ void run_items(const Args& a, int64_t& s_item,
                                          const ItemFn& item_fn) {
  int qi = hw_xcc();
  int64_t item;
  if (!a.queue) {
    item = xcd_remap(int64_t(blockIdx.y) * gridDim.x + blockIdx.x,
                     int64_t(gridDim.x) * gridDim.y);
  } else {
    if (threadIdx.x == 0)
      s_item = queue_resolve(a.queue, a.items, qi, atomicAdd(&a.queue[qi], 1u));
    __syncthreads();
    item = s_item;
  }
  while (item >= 0) {
    uint32_t pre = 0;
    if (a.queue && threadIdx.x == 0) pre = atomicAdd(&a.queue[qi], 1u);
    item_fn(item);
    if (!a.queue) break;
    if (threadIdx.x == 0) s_item = queue_resolve(a.queue, a.items, qi, pre);
    __syncthreads();
    item = s_item;
  }
}

__global__ void queue_reset_kernel(uint32_t* ctr) {
  if (threadIdx.x < kQueues) ctr[threadIdx.x] = 0u;
}


// Zeroes a queue's counters (a kernel rather than a memset, so that the
// sequence may be captured in a graph).
int reset_queue(uint32_t* ctr, hipStream_t s) {
  hipLaunchKernelGGL(queue_reset_kernel, dim3(1), dim3(64), 0, s, ctr);
  HA_LAUNCH_CHECK("queue_reset");
  return HA_OK;
}

}  // namespace

}  // namespace ha
