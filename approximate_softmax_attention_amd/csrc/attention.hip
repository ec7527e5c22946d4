// Attention kernels on MFMA (gfx950): one flash-style core (online softmax,
// fp32 accumulation) used in three modes.
//
//  EXACT  — Att = D^-1 exp(QK^T / sqrt(d)) V over contiguous key blocks,
//           causal or not (HA page, "Method overview"). With block < n it is
//           the causal recursion's base case (HA page, "Algorithm", Figure 2;
//           "Monkey-patching": exact attention below the base size), and its
//           epilogue merges the row's off-diagonal partial results by
//           log-sum-exp ("Single self-attention layer": merge the outputs).
//  BUCKET — one sortLSH bucket of one sub-problem (Algorithms 1-3): the
//           bucket's queries against (a) the bucket's keys (weight 1 in both
//           the row sum and the product), (b) the uniform column sample
//           (weight n_k/m in the row sum only) and (c) the V-norm sample
//           (weight 1/(m p_j) in the product only); (b) and (c) drop keys
//           that lie in the query's own bucket.
//  ROWSUM — (a) and (b) only, producing log d~ (Algorithm 2 alone).
//
// Layout: a work-group of 4 waves owns 128 query rows, 32 per wave. Each
// wave computes S^T = K Q^T for a key tile with v_mfma_f32_32x32x16_bf16
// (A = K rows from LDS, B = the wave's Q rows held in registers), so every
// lane owns one query column of S^T and the softmax statistics of that query
// need only one cross-lane exchange (lane l with lane l^32). The probabilities
// then feed O^T += V^T P^T directly as the B operand (same lane layout), with
// V^T staged transposed in LDS. fp32 inputs use v_mfma_f32_32x32x2f32 with the
// same structure.
//
// Pipelining: key tiles are double-buffered in LDS. While a wave computes on
// tile t, its share of tile t+1 is already in flight from HBM into registers
// and the key indices of tile t+2 (gathered modes) are being fetched; one
// barrier per tile. The running maximum is only moved (and O, l rescaled)
// when a score exceeds it by more than 2^8, so most tiles skip the rescale.
// Work-group ids are remapped so that consecutive logical tiles (which share
// key blocks or sample lists) run on the same XCD and share its L2.
#include <cmath>

#include "common.h"
#include "device_util.h"

namespace ha {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kQW = 32;   // queries per wave; kAttnQ = kWaves * kQW
static_assert(kAttnQ == kWaves * kQW, "query tile");
constexpr float kTau = 8.f;   // lazy-rescale threshold (log2 units)

enum { MODE_EXACT = 0, MODE_BUCKET = 1, MODE_ROWSUM = 2 };
enum { KIND_PLAIN = 0, KIND_SUM_W = 1, KIND_PV_W = 2 };

template <typename T, int D> struct TileCfg;
template <> struct TileCfg<bf16_t, 128> { static constexpr int KT = 64, KPAD = 8, VPAD = 4; };
template <> struct TileCfg<bf16_t, 64> { static constexpr int KT = 128, KPAD = 8, VPAD = 4; };
template <> struct TileCfg<float, 128> { static constexpr int KT = 32, KPAD = 4, VPAD = 4; };
template <> struct TileCfg<float, 64> { static constexpr int KT = 64, KPAD = 4, VPAD = 4; };

template <typename T, int D>
struct alignas(16) Buf {
  static constexpr int KT = TileCfg<T, D>::KT;
  static constexpr int KS = D + TileCfg<T, D>::KPAD;   // K row stride (elements)
  static constexpr int VS = KT + TileCfg<T, D>::VPAD;  // V^T row stride (elements)
  static constexpr int EPC = 16 / int(sizeof(T));      // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                  // chunks per row
  static_assert((KT / 4) * CPR == kThreads, "one 4-key x 16-byte item per thread");
  alignas(16) T k[KT * KS];
  alignas(16) T vt[D * VS];
  alignas(16) float w[KT];     // per-slot weight (sample segments)
};

constexpr int kSlotCap = 1024;   // key slots staged in LDS per window (gathered modes)

template <typename T, int D>
struct Smem {
  Buf<T, D> buf[2];
};

template <typename T, int D>
struct SmemG {
  Buf<T, D> buf[2];
  alignas(16) int32_t srow[kSlotCap];
  alignas(16) float sw[kSlotCap];
};

struct SlotInfo {
  int32_t row;   // key row within the head, or -1 (masked, zero-filled)
  float w;       // weight of the slot in its segment
};

// One thread's share of a tile between HBM and LDS: 4 consecutive slots,
// one 16-byte chunk of each K and V row.
struct Staged {
  uint4 k[4];
  uint4 v[4];
  float w[4];
};

struct AttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* lse;
  int64_t n;
  int heads;
  float scale_log2;        // log2(e) / sqrt(d)
  // EXACT
  int64_t block;           // key/query block size (n for plain exact attention)
  int64_t tiles_per_block; // ceil(block / 128)
  int causal;
  int merge_levels;        // base case: number of levels to merge (0: none)
  const void* part_o;      // [L][heads][S][d]
  const float* part_lse;   // [L][heads][S]
  int64_t S;
  // BUCKET / ROWSUM
  LevelTable table;
  int m;
  int64_t nodes;
  const int32_t* perm_q;
  const int32_t* perm_k;
  const int32_t* u_idx;
  const int32_t* u_bkt;
  const int32_t* v_idx;
  const int32_t* v_bkt;
  const float* v_w;
  const int32_t* meta;
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Logical work-group index with consecutive indices placed on the same XCD
// (work-groups are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int64_t xcd_remap(int64_t x, int64_t n) {
  constexpr int64_t kXcd = 8;
  if (n % kXcd) return x;
  return (x % kXcd) * (n / kXcd) + x / kXcd;
}

// ---------------------------------------------------------------- tiles
template <typename T, int D>
__device__ __forceinline__ void fetch(Staged& st, const SlotInfo* si, const T* __restrict__ Kh,
                                      const T* __restrict__ Vh, bool with_v) {
  constexpr int EPC = Buf<T, D>::EPC;
  const int ch = threadIdx.x % Buf<T, D>::CPR;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    st.w[i] = si[i].w;
    const int64_t r = si[i].row;
    st.k[i] = r >= 0 ? *reinterpret_cast<const uint4*>(Kh + r * D + ch * EPC)
                     : make_uint4(0, 0, 0, 0);
  }
  if (with_v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = si[i].row;
      st.v[i] = r >= 0 ? *reinterpret_cast<const uint4*>(Vh + r * D + ch * EPC)
                       : make_uint4(0, 0, 0, 0);
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void stash(Buf<T, D>& b, const Staged& st, bool with_v) {
  constexpr int KS = Buf<T, D>::KS;
  constexpr int VS = Buf<T, D>::VS;
  constexpr int EPC = Buf<T, D>::EPC;
  const int kg = threadIdx.x / Buf<T, D>::CPR;
  const int ch = threadIdx.x % Buf<T, D>::CPR;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<uint4*>(&b.k[(4 * kg + i) * KS + ch * EPC]) = st.k[i];
  if (ch == 0)
    *reinterpret_cast<float4*>(&b.w[4 * kg]) = make_float4(st.w[0], st.w[1], st.w[2], st.w[3]);
  if (!with_v) return;
  if constexpr (sizeof(T) == 2) {
    // V^T[d][key]: element j of the chunk is 16-bit half (j & 1) of word j/2
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = wi == 0 ? st.v[i].x : wi == 1 ? st.v[i].y : wi == 2 ? st.v[i].z : st.v[i].w;
      const uint2 lo = make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x05040100u),
                                  __builtin_amdgcn_perm(w[3], w[2], 0x05040100u));
      const uint2 hi = make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x07060302u),
                                  __builtin_amdgcn_perm(w[3], w[2], 0x07060302u));
      *reinterpret_cast<uint2*>(&b.vt[(ch * 8 + 2 * wi) * VS + 4 * kg]) = lo;
      *reinterpret_cast<uint2*>(&b.vt[(ch * 8 + 2 * wi + 1) * VS + 4 * kg]) = hi;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        e[i] = j == 0 ? st.v[i].x : j == 1 ? st.v[i].y : j == 2 ? st.v[i].z : st.v[i].w;
      *reinterpret_cast<uint4*>(&b.vt[(ch * 4 + j) * VS + 4 * kg]) =
          make_uint4(e[0], e[1], e[2], e[3]);
    }
  }
}

// ------------------------------------------------------------ per-wave core
template <typename T, int D> struct QFrag;
template <int D> struct QFrag<bf16_t, D> { bf16x8_t v[D / 16]; };
template <int D> struct QFrag<float, D> { float v[D / 2]; };

template <typename T, int D>
__device__ __forceinline__ void load_q(QFrag<T, D>& q, const T* __restrict__ Qh, int64_t row) {
  const int g = lane_id() >> 5;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      uint4 raw = row >= 0 ? *reinterpret_cast<const uint4*>(Qh + row * D + 16 * st + 8 * g)
                           : make_uint4(0, 0, 0, 0);
      q.v[st] = __builtin_bit_cast(bf16x8_t, raw);
    }
  } else {
#pragma unroll
    for (int st = 0; st < D / 2; ++st) q.v[st] = row >= 0 ? Qh[row * D + 2 * st + g] : 0.f;
  }
}

template <typename T, int D>
struct WaveState {
  f32x16 o[D / 32];
  float m;      // running reference maximum (log2 units)
  float l;      // this lane's part of the row sum (its 16 keys per block)
};

template <typename T, int D>
__device__ __forceinline__ void init_state(WaveState<T, D>& ws) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) ws.o[db] = zero16();
  ws.m = -INFINITY;
  ws.l = 0.f;
}

// S^T for key block kb of the tile: s[i] = score of key 32kb + 8(i/4) + 4g + i%4
template <typename T, int D>
__device__ __forceinline__ f32x16 scores(const Buf<T, D>& b, const QFrag<T, D>& q, int kb) {
  constexpr int KS = Buf<T, D>::KS;
  const int lane = lane_id();
  const int ql = lane & 31, g = lane >> 5;
  f32x16 acc = zero16();
  const T* krow = &b.k[(32 * kb + ql) * KS];
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(krow + 16 * st + 8 * g);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q.v[st], acc, 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int st = 0; st < D / 2; ++st)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * st + g], q.v[st], acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ int key_of(int kb, int i, int g) {
  return 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
}

// O^T += V^T P^T for key block kb, p[i] the (weighted) probability of key_of(kb, i)
template <typename T, int D>
__device__ __forceinline__ void accumulate_pv(const Buf<T, D>& b, WaveState<T, D>& ws,
                                              const f32x16& p, int kb) {
  constexpr int VS = Buf<T, D>::VS;
  const int lane = lane_id();
  const int ql = lane & 31, g = lane >> 5;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8_t pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = (__bf16)p[8 * st + j];
      const int k0 = 32 * kb + 16 * st + 4 * g;      // keys k0..k0+3, k0+8..k0+11
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16_t* vr = &b.vt[(32 * db + ql) * VS];
        const uint2 lo = *reinterpret_cast<const uint2*>(vr + k0);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + k0 + 8);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        ws.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, ws.o[db], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int key = key_of(kb, st, g);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const float a = b.vt[(32 * db + ql) * VS + key];
        ws.o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[st], ws.o[db], 0, 0, 0);
      }
    }
  }
}

// One LDS tile for this wave, processed as 32-key blocks, each with its own
// online-softmax step (fewer live registers than one step per tile).
//   KIND_PLAIN: row sum and product, weight 1; KIND_SUM_W: row sum only,
//   weighted by b.w; KIND_PV_W: product only, weighted by b.w.
// masked: keys >= nvalid (and, if causal, keys after the query) score -inf.
template <typename T, int D, int KIND, bool kCausal>
__device__ __forceinline__ void compute_tile(const Buf<T, D>& b, const QFrag<T, D>& q,
                                             WaveState<T, D>& ws, float c, bool masked,
                                             int nvalid, int64_t key0, int64_t qrow) {
  constexpr int KT = Buf<T, D>::KT;
  constexpr int NB = KT / 32;
  const int g = lane_id() >> 5;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
    if (masked && 32 * kb >= nvalid) break;            // rest of the tile is empty
    f32x16 s = scores<T, D>(b, q, kb);
    if (masked) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key_of(kb, i, g);
        bool ok = key < nvalid;
        if (kCausal) ok = ok && (key0 + key <= qrow);
        s[i] = ok ? s[i] : -INFINITY;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
    const bool need = mx > ws.m + kTau;
    if (__ballot(need)) {
      const float m_new = need ? mx : ws.m;
      const float f = (m_new == -INFINITY || m_new == ws.m) ? 1.f : fast_exp2(ws.m - m_new);
      ws.l *= f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) ws.o[db][i] *= f;
      ws.m = m_new;
    }
    const float mref = ws.m == -INFINITY ? 0.f : ws.m;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(fmaf(s[i], c, -mref));
      if (KIND == KIND_PLAIN) {
        lsum += p;
        s[i] = p;
      } else if (KIND == KIND_SUM_W) {
        lsum = fmaf(b.w[key_of(kb, i, g)], p, lsum);
      } else {
        s[i] = b.w[key_of(kb, i, g)] * p;
      }
    }
    if (KIND != KIND_PV_W) ws.l += lsum;
    if (KIND != KIND_SUM_W) accumulate_pv<T, D>(b, ws, s, kb);
  }
}

// Normalised output of this lane's query; returns lse (natural log).
template <typename T, int D>
__device__ __forceinline__ float finalize(WaveState<T, D>& ws) {
  const float l = ws.l + __shfl_xor(ws.l, 32, 64);
  const float inv = 1.f / l;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) ws.o[db][i] *= inv;
  return (ws.m + __log2f(l)) * 0.69314718055994531f;
}

// d index of accumulator (db, i) for lane group g: 32db + 8(i/4) + 4g + i%4
template <typename T, int D>
__device__ __forceinline__ void store_row(const WaveState<T, D>& ws, T* __restrict__ out) {
  const int g = lane_id() >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * g;
      if constexpr (sizeof(T) == 2) {
        const uint32_t a = uint32_t(f32_to_bf16(ws.o[db][4 * q4])) |
                           (uint32_t(f32_to_bf16(ws.o[db][4 * q4 + 1])) << 16);
        const uint32_t b = uint32_t(f32_to_bf16(ws.o[db][4 * q4 + 2])) |
                           (uint32_t(f32_to_bf16(ws.o[db][4 * q4 + 3])) << 16);
        *reinterpret_cast<uint2*>(out + d0) = make_uint2(a, b);
      } else {
        *reinterpret_cast<float4*>(out + d0) =
            make_float4(ws.o[db][4 * q4], ws.o[db][4 * q4 + 1], ws.o[db][4 * q4 + 2],
                        ws.o[db][4 * q4 + 3]);
      }
    }
}

// Merge a normalised partial (po, plse) into (ws.o, lse).
template <typename T, int D>
__device__ __forceinline__ float merge_partial(WaveState<T, D>& ws, float lse,
                                               const T* __restrict__ po, float plse) {
  const int g = lane_id() >> 5;
  const float mx = fmaxf(lse, plse);
  const float wa = __expf(lse - mx);
  const float wb = __expf(plse - mx);
  const float inv = 1.f / (wa + wb);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * g;
      float v[4];
      if constexpr (sizeof(T) == 2) {
        const uint2 raw = *reinterpret_cast<const uint2*>(po + d0);
        v[0] = __uint_as_float(raw.x << 16);
        v[1] = __uint_as_float(raw.x & 0xFFFF0000u);
        v[2] = __uint_as_float(raw.y << 16);
        v[3] = __uint_as_float(raw.y & 0xFFFF0000u);
      } else {
        const float4 raw = *reinterpret_cast<const float4*>(po + d0);
        v[0] = raw.x; v[1] = raw.y; v[2] = raw.z; v[3] = raw.w;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ws.o[db][4 * q4 + j] = (ws.o[db][4 * q4 + j] * wa + v[j] * wb) * inv;
    }
  return mx + __logf(wa + wb);
}

// ------------------------------------------------------------- EXACT kernel
// grid: (blocks_per_head * tiles_per_block, heads). Causal tiles are visited
// from the longest (last) to the shortest for load balance.
template <typename T, int D, bool kCausal>
__global__ __launch_bounds__(kThreads, 2) void exact_kernel(AttnArgs a) {
  __shared__ Smem<T, D> sm;
  constexpr int KT = Buf<T, D>::KT;
  const int64_t nx = int64_t(gridDim.x) * gridDim.y;
  const int64_t lin = xcd_remap(int64_t(blockIdx.y) * gridDim.x + blockIdx.x, nx);
  const int head = int(lin / gridDim.x);
  const int64_t bx = lin % gridDim.x;
  const int64_t tpb = a.tiles_per_block;
  const int64_t blk = bx / tpb;
  const int64_t tile = kCausal ? tpb - 1 - bx % tpb : bx % tpb;
  const int64_t b_lo = blk * a.block;
  const int64_t b_hi = b_lo + a.block < a.n ? b_lo + a.block : a.n;
  const int64_t q0 = b_lo + tile * kAttnQ;
  const int64_t q_end = q0 + kAttnQ < b_hi ? q0 + kAttnQ : b_hi;
  const int wave = threadIdx.x >> 6;
  const int ql = lane_id() & 31;
  const int64_t qw0 = q0 + wave * kQW;              // first query of this wave
  const int64_t qr = qw0 + ql;
  const int64_t qrow = qr < q_end ? qr : -1;

  const int64_t hoff = int64_t(head) * a.n * D;
  const T* Qh = static_cast<const T*>(a.Q) + hoff;
  const T* Kh = static_cast<const T*>(a.K) + hoff;
  const T* Vh = static_cast<const T*>(a.V) + hoff;
  QFrag<T, D> q;
  load_q<T, D>(q, Qh, qrow);
  WaveState<T, D> ws;
  init_state<T, D>(ws);

  const int64_t k_end = kCausal ? q_end : b_hi;
  const int ntiles = int((k_end - b_lo + KT - 1) / KT);
  const int kg = threadIdx.x / Buf<T, D>::CPR;
  auto slots = [&](int t, SlotInfo* si) {
    const int64_t k0 = b_lo + int64_t(t) * KT;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t r = k0 + 4 * kg + i;
      si[i] = SlotInfo{r < k_end ? int32_t(r) : -1, 1.f};
    }
  };
  Staged st;
  SlotInfo si[4];
  slots(0, si);
  fetch<T, D>(st, si, Kh, Vh, true);
  stash<T, D>(sm.buf[0], st, true);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) {
      slots(t + 1, si);
      fetch<T, D>(st, si, Kh, Vh, true);
    }
    const int64_t k0 = b_lo + int64_t(t) * KT;
    const int nvalid = int(k_end - k0 < KT ? k_end - k0 : KT);
    const bool skip = kCausal && k0 > qw0 + kQW - 1;       // wholly above the diagonal
    if (!skip) {
      const bool masked = nvalid < KT || (kCausal && k0 + KT - 1 > qw0);
      compute_tile<T, D, KIND_PLAIN, kCausal>(sm.buf[t & 1], q, ws, a.scale_log2, masked,
                                              nvalid, k0, qrow);
    }
    if (t + 1 < ntiles) stash<T, D>(sm.buf[(t + 1) & 1], st, true);
    __syncthreads();
  }
  float lse = finalize<T, D>(ws);
  if (qrow < 0) return;
  if (a.merge_levels > 0) {
    for (int lv = 0; lv < a.merge_levels; ++lv) {
      const int64_t hl = a.n >> (lv + 1);
      if (((qrow / hl) & 1) == 0) continue;
      const int64_t slot = (qrow / (2 * hl)) * hl + (qrow % hl);
      const int64_t idx = (int64_t(lv) * a.heads + head) * a.S + slot;
      lse = merge_partial<T, D>(ws, lse, static_cast<const T*>(a.part_o) + idx * D,
                                a.part_lse[idx]);
    }
  }
  store_row<T, D>(ws, static_cast<T*>(a.O) + hoff + qrow * D);
  if (a.lse && (lane_id() >> 5) == 0) a.lse[int64_t(head) * a.n + qrow] = lse;
}

// ------------------------------------------------------ BUCKET / ROWSUM kernel
// The key tiles of a work-group form one sequence: the bucket's own keys,
// then the uniform sample, then (BUCKET) the V-norm sample, each segment
// padded to whole tiles. The rows and weights of up to kSlotCap slots (a
// window of tiles) are staged in LDS up front, so the tile loop issues no
// dependent index loads.
template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads, 2) void bucket_kernel(AttnArgs a) {
  __shared__ SmemG<T, D> sm;
  constexpr int KT = Buf<T, D>::KT;
  constexpr int kWin = kSlotCap / KT;           // tiles per slot window
  constexpr bool kProduct = MODE == MODE_BUCKET;
  const int64_t w = xcd_remap(blockIdx.x, gridDim.x);
  int lv = 0;
  for (int l = 1; l < a.table.count; ++l)
    if (w >= a.table.lv[l].att_wg0) lv = l;
  const Level& L = a.table.lv[lv];
  int64_t rem = w - L.att_wg0;
  const int64_t qc = rem % L.att_qch;
  rem /= L.att_qch;
  const int64_t bucket = rem % L.nbucket;
  rem /= L.nbucket;
  const int64_t seg = rem % L.nseg;
  const int head = int(rem / L.nseg);
  const int b_eff = L.b_eff;
  const int64_t h = L.h;

  const int64_t slot0 = (int64_t(lv) * a.heads + head) * a.S + seg * h + bucket * b_eff;
  const int wave = threadIdx.x >> 6;
  const int ql = lane_id() & 31;
  const int64_t qi = qc * kAttnQ + wave * kQW + ql;
  const int64_t qrow = qi < b_eff ? int64_t(a.perm_q[slot0 + qi]) : -1;

  const int64_t node = (int64_t(1) << lv) + seg;
  const int64_t rec = int64_t(head) * a.nodes + (node - 1);
  const int32_t* meta = a.meta + rec * 4;
  const int ucount = meta[0];
  const int vcount = kProduct ? meta[1] : 0;
  const float alpha = __int_as_float(meta[2]);

  const int64_t hoff = int64_t(head) * a.n * D;
  const T* Qh = static_cast<const T*>(a.Q) + hoff;
  const T* Kh = static_cast<const T*>(a.K) + hoff;
  const T* Vh = kProduct ? static_cast<const T*>(a.V) + hoff : nullptr;
  QFrag<T, D> q;
  load_q<T, D>(q, Qh, qrow);
  WaveState<T, D> ws;
  init_state<T, D>(ws);

  const int t_b = (b_eff + KT - 1) / KT;
  const int t_u = (ucount + KT - 1) / KT;
  const int t_v = (vcount + KT - 1) / KT;
  const int ntiles = t_b + t_u + t_v;
  // segment of tile t (0 bucket, 1 uniform, 2 V-norm), its first slot, its size
  auto seg_of = [&](int t, int& j0, int& cnt) {
    if (t < t_b) { j0 = t * KT; cnt = b_eff; return 0; }
    if (t < t_b + t_u) { j0 = (t - t_b) * KT; cnt = ucount; return 1; }
    j0 = (t - t_b - t_u) * KT; cnt = vcount; return 2;
  };
  // stage slots of tiles [t0, t0 + kWin) in LDS
  auto fill = [&](int t0) {
    const int32_t* pk = a.perm_k + slot0;
    const int32_t* ui = a.u_idx + rec * a.m;
    const int32_t* ub = a.u_bkt + rec * a.m;
    for (int e = threadIdx.x; e < kSlotCap; e += kThreads) {
      const int t = t0 + e / KT;
      int32_t row = -1;
      float wt = 0.f;
      if (t < ntiles) {
        int j0, cnt;
        const int sg = seg_of(t, j0, cnt);
        const int j = j0 + e % KT;
        if (j < cnt) {
          if (sg == 0) {
            row = pk[j];
            wt = 1.f;
          } else if (sg == 1) {
            row = ui[j];
            wt = ub[j] != bucket ? alpha : 0.f;
          } else {
            row = a.v_idx[rec * a.m + j];
            wt = a.v_bkt[rec * a.m + j] != bucket ? a.v_w[rec * a.m + j] : 0.f;
          }
        }
      }
      sm.srow[e] = row;
      sm.sw[e] = wt;
    }
  };
  const int kg = threadIdx.x / Buf<T, D>::CPR;
  auto slots = [&](int t, SlotInfo* si) {
    const int e0 = (t % kWin) * KT + 4 * kg;
    const int4 r = *reinterpret_cast<const int4*>(&sm.srow[e0]);
    const float4 wt = *reinterpret_cast<const float4*>(&sm.sw[e0]);
    si[0] = SlotInfo{r.x, wt.x};
    si[1] = SlotInfo{r.y, wt.y};
    si[2] = SlotInfo{r.z, wt.z};
    si[3] = SlotInfo{r.w, wt.w};
  };
  auto needs_v = [&](int t) { return kProduct && (t < t_b || t >= t_b + t_u); };

  Staged st;
  SlotInfo si[4];
  fill(0);
  __syncthreads();
  slots(0, si);
  fetch<T, D>(st, si, Kh, Vh, needs_v(0));
  stash<T, D>(sm.buf[0], st, needs_v(0));
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) {
      if ((t + 1) % kWin == 0) {      // next window of slots
        fill(t + 1);
        __syncthreads();
      }
      slots(t + 1, si);
      fetch<T, D>(st, si, Kh, Vh, needs_v(t + 1));
    }
    int j0, cnt;
    const int sg = seg_of(t, j0, cnt);
    const int nvalid = cnt - j0 < KT ? cnt - j0 : KT;
    const bool masked = nvalid < KT;
    const Buf<T, D>& b = sm.buf[t & 1];
    if (sg == 0) {
      if (kProduct)
        compute_tile<T, D, KIND_PLAIN, false>(b, q, ws, a.scale_log2, masked, nvalid, 0, qrow);
      else
        compute_tile<T, D, KIND_SUM_W, false>(b, q, ws, a.scale_log2, masked, nvalid, 0, qrow);
    } else if (sg == 1) {
      compute_tile<T, D, KIND_SUM_W, false>(b, q, ws, a.scale_log2, masked, nvalid, 0, qrow);
    } else if (kProduct) {
      compute_tile<T, D, KIND_PV_W, false>(b, q, ws, a.scale_log2, masked, nvalid, 0, qrow);
    }
    if (t + 1 < ntiles) stash<T, D>(sm.buf[(t + 1) & 1], st, needs_v(t + 1));
    __syncthreads();
  }
  const float lse = finalize<T, D>(ws);
  if (qrow < 0) return;
  const bool first = (lane_id() >> 5) == 0;
  if (MODE == MODE_ROWSUM) {
    if (first) a.lse[int64_t(head) * a.n + qrow] = lse;
    return;
  }
  if (a.table.causal) {
    const int64_t slot = (qrow / (2 * h)) * h + (qrow % h);
    const int64_t idx = (int64_t(lv) * a.heads + head) * a.S + slot;
    store_row<T, D>(ws, static_cast<T*>(a.O) + idx * D);
    if (first) a.lse[idx] = lse;
  } else {
    store_row<T, D>(ws, static_cast<T*>(a.O) + hoff + qrow * D);
    if (first && a.lse) a.lse[int64_t(head) * a.n + qrow] = lse;
  }
}

template <typename T, int D>
void launch_exact_t(const AttnArgs& a, dim3 grid, hipStream_t s) {
  if (a.causal)
    hipLaunchKernelGGL((exact_kernel<T, D, true>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((exact_kernel<T, D, false>), grid, dim3(kThreads), 0, s, a);
}

template <typename T, int D>
void launch_bucket_t(const AttnArgs& a, dim3 grid, bool product, hipStream_t s) {
  if (product)
    hipLaunchKernelGGL((bucket_kernel<T, D, MODE_BUCKET>), grid, dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((bucket_kernel<T, D, MODE_ROWSUM>), grid, dim3(kThreads), 0, s, a);
}

}  // namespace

int launch_exact(const void* Q, const void* K, const void* V, void* O, float* lse, int64_t n,
                 int d, int heads, int causal, int dtype, int64_t block, const Plan* merge,
                 const void* ws, hipStream_t s) {
  AttnArgs a{};
  a.Q = Q; a.K = K; a.V = V; a.O = O; a.lse = lse;
  a.n = n;
  a.heads = heads;
  a.scale_log2 = float(1.4426950408889634 / std::sqrt(double(d)));
  a.block = block;
  a.tiles_per_block = ceil_div(block, kAttnQ);
  a.causal = causal;
  if (merge && merge->L > 0) {
    const char* w = static_cast<const char*>(ws);
    a.merge_levels = merge->L;
    a.part_o = w + merge->off[HA_WS_PART_O];
    a.part_lse = reinterpret_cast<const float*>(w + merge->off[HA_WS_PART_LSE]);
    a.S = merge->S;
  }
  const int64_t blocks = ceil_div(n, block);
  dim3 grid(unsigned(blocks * a.tiles_per_block), unsigned(heads));
  ProfRange pr(merge ? "exact_base_merge" : "exact_attention", s);
  if (dtype == HA_BF16) {
    if (d == 128) launch_exact_t<bf16_t, 128>(a, grid, s);
    else launch_exact_t<bf16_t, 64>(a, grid, s);
  } else {
    if (d == 128) launch_exact_t<float, 128>(a, grid, s);
    else launch_exact_t<float, 64>(a, grid, s);
  }
  HA_LAUNCH_CHECK("exact_attention");
  return HA_OK;
}

int launch_bucket_attention(const Plan& p, const void* Q, const void* K, const void* V, void* O,
                            float* lse, void* ws, hipStream_t s) {
  if (p.att_wgs == 0) return HA_OK;
  char* w = static_cast<char*>(ws);
  AttnArgs a{};
  a.Q = Q; a.K = K; a.V = V;
  a.n = p.n;
  a.heads = p.heads;
  a.scale_log2 = float(1.4426950408889634 / std::sqrt(double(p.d)));
  a.table = p.table;
  a.m = p.m;
  a.nodes = p.nodes;
  a.S = p.S;
  a.perm_q = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_PERM_Q]);
  a.perm_k = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_PERM_K]);
  a.u_idx = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_U_IDX]);
  a.u_bkt = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_U_BKT]);
  a.meta = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_NODE_META]);
  if (p.product) {
    a.v_idx = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_V_IDX]);
    a.v_bkt = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_V_BKT]);
    a.v_w = reinterpret_cast<const float*>(w + p.off[HA_WS_V_W]);
  }
  if (p.product && p.causal) {
    a.O = w + p.off[HA_WS_PART_O];
    a.lse = reinterpret_cast<float*>(w + p.off[HA_WS_PART_LSE]);
  } else {
    a.O = O;
    a.lse = lse;
  }
  dim3 grid(unsigned(p.att_wgs));
  ProfRange pr(p.product ? "bucket_attention" : "bucket_rowsum", s);
  if (p.dtype == HA_BF16) {
    if (p.d == 128) launch_bucket_t<bf16_t, 128>(a, grid, p.product, s);
    else launch_bucket_t<bf16_t, 64>(a, grid, p.product, s);
  } else {
    if (p.d == 128) launch_bucket_t<float, 128>(a, grid, p.product, s);
    else launch_bucket_t<float, 64>(a, grid, p.product, s);
  }
  HA_LAUNCH_CHECK("bucket_attention");
  return HA_OK;
}

}  // namespace ha
