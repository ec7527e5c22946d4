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

enum { MODE_EXACT = 0, MODE_BUCKET = 1, MODE_ROWSUM = 2 };

template <typename T, int D> struct TileCfg;
template <> struct TileCfg<bf16_t, 128> { static constexpr int KT = 64, KPAD = 8, VPAD = 4; };
template <> struct TileCfg<bf16_t, 64> { static constexpr int KT = 128, KPAD = 8, VPAD = 4; };
template <> struct TileCfg<float, 128> { static constexpr int KT = 32, KPAD = 4, VPAD = 4; };
template <> struct TileCfg<float, 64> { static constexpr int KT = 64, KPAD = 4, VPAD = 4; };

template <typename T, int D>
struct alignas(16) Smem {
  static constexpr int KT = TileCfg<T, D>::KT;
  static constexpr int KS = D + TileCfg<T, D>::KPAD;   // K row stride (elements)
  static constexpr int VS = KT + TileCfg<T, D>::VPAD;  // V^T row stride (elements)
  alignas(16) T k[KT * KS];
  alignas(16) T vt[D * VS];
  float wd[KT];
  float wn[KT];
  int valid[KT];
};

struct KeySlot {
  int64_t row;    // key row within the head, or -1 (masked, zero-filled)
  float wd, wn;   // weight in the row sum and in the product
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

// ---------------------------------------------------------------- tiles
// Loads key slots [0, KT) of a tile into LDS: K rows as they are, V rows
// transposed, plus each slot's weights and validity. Threads take groups of
// 4 consecutive slots x one 16-byte chunk of the row.
template <typename T, int D, bool kV, typename Src>
__device__ __forceinline__ void load_tile(Smem<T, D>& sm, const T* __restrict__ Kh,
                                          const T* __restrict__ Vh, const Src& src) {
  constexpr int KT = Smem<T, D>::KT;
  constexpr int KS = Smem<T, D>::KS;
  constexpr int VS = Smem<T, D>::VS;
  constexpr int EPC = 16 / int(sizeof(T));   // elements per 16-byte chunk
  constexpr int CPR = D / EPC;               // chunks per row
  for (int u = threadIdx.x; u < (KT / 4) * CPR; u += kThreads) {
    const int kg = u / CPR;
    const int ch = u % CPR;
    int64_t rows[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const KeySlot s = src(4 * kg + i);
      rows[i] = s.row;
      if (ch == 0) {
        sm.valid[4 * kg + i] = s.row >= 0;
        sm.wd[4 * kg + i] = s.wd;
        sm.wn[4 * kg + i] = s.wn;
      }
    }
    uint4 kv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kv[i] = rows[i] >= 0 ? *reinterpret_cast<const uint4*>(Kh + rows[i] * D + ch * EPC)
                           : make_uint4(0, 0, 0, 0);
    }
    uint4 vv[4];
    if (kV) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vv[i] = rows[i] >= 0 ? *reinterpret_cast<const uint4*>(Vh + rows[i] * D + ch * EPC)
                             : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&sm.k[(4 * kg + i) * KS + ch * EPC]) = kv[i];
    if (kV) {
      if constexpr (sizeof(T) == 2) {
        // element j of the 8-element chunk of key i sits in 16-bit half
        // (j & 1) of word (j >> 1); write the 4 keys' element j as 8 bytes
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          uint32_t e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t wv = (j >> 1) == 0 ? vv[i].x : (j >> 1) == 1 ? vv[i].y
                                : (j >> 1) == 2 ? vv[i].z : vv[i].w;
            e[i] = (j & 1) ? (wv >> 16) : (wv & 0xFFFFu);
          }
          uint2 out = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
          *reinterpret_cast<uint2*>(&sm.vt[(ch * 8 + j) * VS + 4 * kg]) = out;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            e[i] = j == 0 ? vv[i].x : j == 1 ? vv[i].y : j == 2 ? vv[i].z : vv[i].w;
          *reinterpret_cast<uint4*>(&sm.vt[(ch * 4 + j) * VS + 4 * kg]) =
              make_uint4(e[0], e[1], e[2], e[3]);
        }
      }
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
  float m;      // running max (log2 units)
  float l;      // this lane's part of the row sum (its 16 keys per block)
};

// S^T for key block kb of the tile: s[i] = score of key 32kb + 8(i/4) + 4g + i%4
template <typename T, int D>
__device__ __forceinline__ f32x16 scores(const Smem<T, D>& sm, const QFrag<T, D>& q, int kb) {
  constexpr int KS = Smem<T, D>::KS;
  const int lane = lane_id();
  const int ql = lane & 31, g = lane >> 5;
  f32x16 acc = zero16();
  const T* krow = &sm.k[(32 * kb + ql) * KS];
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
__device__ __forceinline__ void accumulate_pv(const Smem<T, D>& sm, WaveState<T, D>& ws,
                                              const f32x16& p, int kb) {
  constexpr int VS = Smem<T, D>::VS;
  const int lane = lane_id();
  const int ql = lane & 31, g = lane >> 5;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      bf16x8_t b;
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = (__bf16)p[8 * st + j];
      const int k0 = 32 * kb + 16 * st + 4 * g;      // keys k0..k0+3, k0+8..k0+11
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16_t* vr = &sm.vt[(32 * db + ql) * VS];
        const uint2 lo = *reinterpret_cast<const uint2*>(vr + k0);
        const uint2 hi = *reinterpret_cast<const uint2*>(vr + k0 + 8);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        ws.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, ws.o[db], 0, 0, 0);
      }
    }
  } else {
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int key = key_of(kb, st, g);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const float a = sm.vt[(32 * db + ql) * VS + key];
        ws.o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[st], ws.o[db], 0, 0, 0);
      }
    }
  }
}

// Process one LDS tile for this wave. kWeights: use the tile's wd/wn;
// kPV: accumulate the product; kSum: accumulate the row sum.
template <typename T, int D, bool kWeights, bool kPV, bool kSum, bool kCausal>
__device__ __forceinline__ void process_tile(const Smem<T, D>& sm, const QFrag<T, D>& q,
                                             WaveState<T, D>& ws, float scale_log2,
                                             int64_t key0, int64_t qrow, int nvalid) {
  constexpr int KT = Smem<T, D>::KT;
  constexpr int NB = KT / 32;
  const int g = lane_id() >> 5;
  f32x16 s[NB];
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) s[kb] = scores<T, D>(sm, q, kb);
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key_of(kb, i, g);
      bool ok;
      if (kWeights) ok = sm.valid[key] != 0;
      else ok = key < nvalid;
      if (kCausal) ok = ok && (key0 + key <= qrow);
      const float x = ok ? s[kb][i] * scale_log2 : -INFINITY;
      s[kb][i] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float m_new = fmaxf(ws.m, mx);
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float factor = exp2f(ws.m - m_use);
  ws.m = m_new;
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = exp2f(s[kb][i] - m_use);
      if (kWeights) {
        const int key = key_of(kb, i, g);
        if (kSum) lsum += sm.wd[key] * p;
        s[kb][i] = kPV ? sm.wn[key] * p : 0.f;
      } else {
        lsum += p;
        s[kb][i] = p;
      }
    }
  }
  ws.l = ws.l * factor + (kSum ? lsum : 0.f);
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) ws.o[db][i] *= factor;
  if (kPV) {
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) accumulate_pv<T, D>(sm, ws, s[kb], kb);
  }
}

// Normalised output of this lane's query: fills out[db][i] and returns lse.
template <typename T, int D>
__device__ __forceinline__ float finalize(WaveState<T, D>& ws) {
  const float l = ws.l + __shfl_xor(ws.l, 32, 64);
  const float inv = 1.f / l;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) ws.o[db][i] *= inv;
  return (ws.m + log2f(l)) * 0.69314718055994531f;
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

template <typename T, int D>
__device__ __forceinline__ void init_state(WaveState<T, D>& ws) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) ws.o[db] = zero16();
  ws.m = -INFINITY;
  ws.l = 0.f;
}

// ------------------------------------------------------------- EXACT kernel
// grid: (blocks_per_head * tiles_per_block, heads). Causal tiles are visited
// from the longest (last) to the shortest for load balance.
template <typename T, int D, bool kCausal>
__global__ __launch_bounds__(kThreads) void exact_kernel(AttnArgs a) {
  __shared__ Smem<T, D> sm;
  constexpr int KT = Smem<T, D>::KT;
  const int head = blockIdx.y;
  const int64_t tpb = a.tiles_per_block;
  const int64_t blk = int64_t(blockIdx.x) / tpb;
  const int64_t tile = kCausal ? tpb - 1 - int64_t(blockIdx.x) % tpb : int64_t(blockIdx.x) % tpb;
  const int64_t b_lo = blk * a.block;
  const int64_t b_hi = b_lo + a.block < a.n ? b_lo + a.block : a.n;
  const int64_t q0 = b_lo + tile * kAttnQ;
  const int64_t q_end = q0 + kAttnQ < b_hi ? q0 + kAttnQ : b_hi;
  const int wave = threadIdx.x >> 6;
  const int ql = lane_id() & 31;
  const int64_t qr = q0 + wave * kQW + ql;
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
  for (int64_t k0 = b_lo; k0 < k_end; k0 += KT) {
    const int nvalid = int(k_end - k0 < KT ? k_end - k0 : KT);
    load_tile<T, D, true>(sm, Kh, Vh, [&](int i) {
      return KeySlot{i < nvalid ? k0 + i : -1, 1.f, 1.f};
    });
    __syncthreads();
    process_tile<T, D, false, true, true, kCausal>(sm, q, ws, a.scale_log2, k0, qrow, nvalid);
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
template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads) void bucket_kernel(AttnArgs a) {
  __shared__ Smem<T, D> sm;
  constexpr int KT = Smem<T, D>::KT;
  constexpr bool kProduct = MODE == MODE_BUCKET;
  const int64_t w = blockIdx.x;
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

  // (a) the bucket's own keys
  const int32_t* pk = a.perm_k + slot0;
  for (int k0 = 0; k0 < b_eff; k0 += KT) {
    load_tile<T, D, kProduct>(sm, Kh, Vh, [&](int i) {
      const int j = k0 + i;
      return KeySlot{j < b_eff ? int64_t(pk[j]) : -1, 1.f, 1.f};
    });
    __syncthreads();
    process_tile<T, D, true, kProduct, true, false>(sm, q, ws, a.scale_log2, 0, qrow, 0);
    __syncthreads();
  }
  // (b) uniform column sample: row sum only
  const int32_t* ui = a.u_idx + rec * a.m;
  const int32_t* ub = a.u_bkt + rec * a.m;
  for (int k0 = 0; k0 < ucount; k0 += KT) {
    load_tile<T, D, false>(sm, Kh, Vh, [&](int i) {
      const int j = k0 + i;
      if (j >= ucount) return KeySlot{-1, 0.f, 0.f};
      return KeySlot{int64_t(ui[j]), ub[j] != bucket ? alpha : 0.f, 0.f};
    });
    __syncthreads();
    process_tile<T, D, true, false, true, false>(sm, q, ws, a.scale_log2, 0, qrow, 0);
    __syncthreads();
  }
  // (c) V-row-norm sample: product only
  if (kProduct) {
    const int32_t* vi = a.v_idx + rec * a.m;
    const int32_t* vb = a.v_bkt + rec * a.m;
    const float* vw = a.v_w + rec * a.m;
    for (int k0 = 0; k0 < vcount; k0 += KT) {
      load_tile<T, D, true>(sm, Kh, Vh, [&](int i) {
        const int j = k0 + i;
        if (j >= vcount) return KeySlot{-1, 0.f, 0.f};
        return KeySlot{int64_t(vi[j]), 0.f, vb[j] != bucket ? vw[j] : 0.f};
      });
      __syncthreads();
      process_tile<T, D, true, true, false, false>(sm, q, ws, a.scale_log2, 0, qrow, 0);
      __syncthreads();
    }
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
