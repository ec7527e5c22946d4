// Backward pass of exact attention and of the HyperAttention estimator on
// MFMA (gfx950).
//
// What is differentiated (HA page, "Single self-attention layer", which
// times the forward and backward passes together; the page states no
// formula, so the backward pass is the exact derivative of the forward
// pass's estimator with its buckets and samples held fixed): every row i of
// the output is O_i = N_i / Z_i with N_i = sum_j w_ij e^{s_ij} V_j and
// Z_i = sum_j u_ij e^{s_ij} over the key slots row i evaluates, and
// ln Z_i = Lambda_i is its final lse. With Delta_i = dO_i . O_i and
// E_ij = e^{s_ij - Lambda_i}:
//   ds_ij = E_ij (w_ij dO_i . V_j - u_ij Delta_i),   dV_j += w_ij E_ij dO_i,
//   dq_i += ds_ij k_j / sqrt(d),                      dk_j += ds_ij q_i / sqrt(d).
// Slot weights (w, u): a bucket or base-case key (1, 1); a uniform sample
// (0, n_k/m); a V-norm sample (its weight, 0); a sample inside the query's
// bucket (0, 0).
//
// Two kinds of kernels, on the forward kernels' tiles and fragments:
//  query-major (dQ): a wave owns 32 query rows (their Q and dO fragments in
//    registers) and streams the rows' key slots through LDS: S^T = K Q^T,
//    dP^T = V dO^T, then dQ^T += K^T dS^T with the transposing read of K.
//  key-major (dK, dV): a wave owns a group of key slots (K and V
//    fragments) and streams the queries that use them: S = Q K^T,
//    dP = dO V^T, then dV^T += dO^T (w E) and dK^T += Q^T dS with
//    transposing reads of the dO and Q tiles, both gradients in one sweep.
//    32 slots a wave on v_mfma_f32_32x32x16_bf16 at d = 64; 16 slots a wave
//    on v_mfma_f32_16x16x32_bf16 at d = 128, where the fragments and
//    accumulators of 32 slots would not fit a wave's registers.
// HyperAttention: the query-major kernel takes each bucket's queries against
// the bucket's keys and the node's two samples; the key-major kernel takes
// each bucket's keys against the bucket's queries, and, separately, every
// sample slot of a node against chunks of the node's queries in sorted
// order (a query's bucket is its sorted position / b_eff). The chunks'
// partial slot gradients stay apart and the bucket kernel adds them, with
// every other slot drawn on the same key row in slot order, to that row's
// gradient: no floating-point atomics, so results are deterministic.
// Causal recursion: the bucket kernels write per-level partial gradients
// (bf16 rows, as the forward pass's partial outputs) and the base case
// kernels add them in fp32 to the rows of their diagonal blocks, as the
// forward pass's base case merges partial outputs.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "device_util.h"
#include "mfma_tile.h"

namespace ha {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int KT = Buf<bf16_t, 128>::KT;   // rows per LDS tile (both d)

enum { BW_EXACT = 0, BW_BUCKET = 1, BW_SAMPLE = 2 };
// slot weights of a query-major tile: (1, 1), (0, u) or (w, 0)
enum { SK_FULL = 0, SK_SUM = 1, SK_PROD = 2 };

// One LDS tile: the rows of two tensors (t.k, t.v) and per-row scalars.
// Query-major: K and V rows, t.w = w, w2 = u of each key slot.
// Key-major: Q and dO rows, t.w = Lambda_i log2(e) (+inf for no row),
// w2 = Delta_i.
template <int D>
struct BwdBuf {
  Buf<bf16_t, D> t;
  float w2[KT];
};

template <int D>
struct BwdSmem {
  BwdBuf<D> buf[2];
  alignas(16) int32_t srow[kSlotCap];
  alignas(16) float sw[kSlotCap];
  alignas(16) float sw2[kSlotCap];
  int64_t item;            // next work item (persistent launches)
};

struct BwdArgs {
  const bf16_t* Q;
  const bf16_t* K;
  const bf16_t* V;
  const bf16_t* dO;
  const float* lse;
  const float* delta;
  bf16_t* dQ;
  bf16_t* dK;
  bf16_t* dV;
  int64_t n;
  int heads;
  float scale_log2;        // log2(e) / sqrt(d)
  float scale;             // 1 / sqrt(d)
  // EXACT
  int64_t block;
  uint32_t tiles_per_block;
  uint32_t items_per_head;
  int merge_levels;
  int64_t S;
  bf16_t* part_dq;         // [L][heads][S][d]
  bf16_t* part_dk;
  bf16_t* part_dv;
  // BUCKET / SAMPLE
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
  const int32_t* slot_first;   // [L][heads][S]
  const int32_t* slot_next;    // [heads][nodes][2m]
  float* slot_dk;              // [sample items][kAttnQ][d]
  float* slot_dv;
  // work queue of a persistent launch
  uint32_t* queue;             // [kQueues] counters, zero at launch
  uint32_t items;              // total work items
};

// ------------------------------------------------------------ MFMA helpers
// acc[i] = <tile row key_of(kb, i, g), the lane's fragment row> over the 32
// rows of block kb of the tile array (A: tile rows from LDS, B: fragment).
// kAhead: every fragment read of the block is issued before the MFMA chain
// (the empty asm keeps the compiler from sinking them between the MFMAs), so
// the chain waits on LDS latency once; it holds D/4 more registers.
template <int D, bool kAhead = false>
__device__ __forceinline__ f32x16 tile_dot(const bf16_t* arr, const LaneOffs<bf16_t, D>& lo,
                                           const QFrag<bf16_t, D>& f, int kb,
                                           f32x16 acc = zero16()) {
  const char* base = reinterpret_cast<const char*>(arr) + kb * 32 * D * 2;
  if constexpr (kAhead) {
    bf16x8_t x[D / 16];
#pragma unroll
    for (int st = 0; st < D / 16; ++st) x[st] = *reinterpret_cast<const bf16x8_t*>(base + lo.k[st]);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[st], f.v[st], acc, 0, 0, 0);
  } else {
    __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      const bf16x8_t x = *reinterpret_cast<const bf16x8_t*>(base + lo.k[st]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, f.v[st], acc, 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
  return acc;
}

// acc[db] += (rows of block kb)^T p: element i of acc[db] (column
// 32db + 8(i/4) + 4g + i%4 of the tile) gains the sum over the block's rows
// of tile[row][column] * p(row), with p packed as pb[i / 8][i % 8] for
// row key_of(kb, i, g).
template <int D, bool kAhead = false>
__device__ __forceinline__ void tile_tr_acc(const bf16_t* arr, const LaneOffs<bf16_t, D>& lo,
                                            f32x16* acc, const bf16x8_t* pb, int kb) {
  if constexpr (kAhead) {
    v4i16_t x[2][D / 32][2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const char* base = reinterpret_cast<const char*>(arr) + (32 * kb + 16 * st) * D * 2;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          x[st][db][h] =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + lo.v[h][db]));
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(x[st][db][0], x[st][db][1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], acc[db], 0, 0, 0);
      }
    __builtin_amdgcn_s_setprio(0);
    return;
  }
  __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    const char* base = reinterpret_cast<const char*>(arr) + (32 * kb + 16 * st) * D * 2;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const v4i16_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + lo.v[0][db]));
      const v4i16_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + lo.v[1][db]));
      const bf16x8_t a =
          __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], acc[db], 0, 0, 0);
    }
  }
  __builtin_amdgcn_s_setprio(0);
}

// The per-row values of block kb that this lane's accumulator elements
// need: v[i] = arr[key_of(kb, i, g)], read as four 16-byte LDS loads.
template <typename T>
__device__ __forceinline__ void rows16(const T* arr, int kb, int g, T* v) {
  static_assert(sizeof(T) == 4, "32-bit values");
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint4 x = *reinterpret_cast<const uint4*>(arr + 32 * kb + 8 * j + 4 * g);
    v[4 * j] = __builtin_bit_cast(T, x.x);
    v[4 * j + 1] = __builtin_bit_cast(T, x.y);
    v[4 * j + 2] = __builtin_bit_cast(T, x.z);
    v[4 * j + 3] = __builtin_bit_cast(T, x.w);
  }
}

__device__ __forceinline__ void pack_bf16(const float* x, bf16x8_t* pb) {
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int j = 0; j < 8; ++j) pb[st][j] = (__bf16)x[8 * st + j];
}

// Four consecutive floats of a row <-> the lane's accumulator chunk
// (db, q4): columns 32db + 8q4 + 4g + j, j < 4.
__device__ __forceinline__ int chunk_col(int db, int q4, int g) { return 32 * db + 8 * q4 + 4 * g; }

template <int D>
__device__ __forceinline__ void add_row_f32(f32x16* acc, const float* row) {
  const int g = lane_id() >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const float4 v = *reinterpret_cast<const float4*>(row + chunk_col(db, q4, g));
      acc[db][4 * q4] += v.x;
      acc[db][4 * q4 + 1] += v.y;
      acc[db][4 * q4 + 2] += v.z;
      acc[db][4 * q4 + 3] += v.w;
    }
}

// Level partials are bf16 rows, like the forward pass's partial outputs.
__device__ __forceinline__ float bf16_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

template <int D>
__device__ __forceinline__ void add_row_bf16(f32x16* acc, const bf16_t* row) {
  const int g = lane_id() >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint2 v = *reinterpret_cast<const uint2*>(row + chunk_col(db, q4, g));
      acc[db][4 * q4] += bf16_lo(v.x);
      acc[db][4 * q4 + 1] += bf16_hi(v.x);
      acc[db][4 * q4 + 2] += bf16_lo(v.y);
      acc[db][4 * q4 + 3] += bf16_hi(v.y);
    }
}

template <int D>
__device__ __forceinline__ void store_row_f32(const f32x16* acc, float* row) {
  const int g = lane_id() >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      *reinterpret_cast<float4*>(row + chunk_col(db, q4, g)) =
          make_float4(acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2],
                      acc[db][4 * q4 + 3]);
}

template <int D>
__device__ __forceinline__ void store_row_bf16(const f32x16* acc, bf16_t* row) {
  const int g = lane_id() >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const uint32_t lo = uint32_t(f32_to_bf16(acc[db][4 * q4])) |
                          (uint32_t(f32_to_bf16(acc[db][4 * q4 + 1])) << 16);
      const uint32_t hi = uint32_t(f32_to_bf16(acc[db][4 * q4 + 2])) |
                          (uint32_t(f32_to_bf16(acc[db][4 * q4 + 3])) << 16);
      *reinterpret_cast<uint2*>(row + chunk_col(db, q4, g)) = make_uint2(lo, hi);
    }
}

template <int D>
__device__ __forceinline__ void scale_acc(f32x16* acc, float f) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] *= f;
}

template <int D>
__device__ __forceinline__ void zero_acc(f32x16* acc) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = zero16();
}

// Slot of row `row` in level lv's partial buffers for base block blk whose
// rows lie in that level's node: in its second half (queries, want_query)
// or its first half (keys). Returns -1 when the block is in the other half.
__device__ __forceinline__ int64_t level_slot(const BwdArgs& a, int lv, uint32_t blk,
                                              int64_t b_lo, int64_t row, bool want_query,
                                              int head) {
  const int sh = a.merge_levels - 1 - lv;
  const bool second = ((blk >> sh) & 1u) != 0;
  if (second != want_query) return -1;
  const int64_t hl = a.block << sh;
  const int64_t slot = int64_t(blk >> (sh + 1)) * hl +
                       int64_t(blk & ((1u << sh) - 1u)) * a.block + (row - b_lo);
  return (int64_t(lv) * a.heads + head) * a.S + slot;
}

// Fragment reads issued ahead of their MFMA chains (see tile_dot) in the
// query-major kernels, which have the registers for it.
constexpr bool kQAhead = true;

// ------------------------------------------------------ query-major tiles
// One LDS tile of key slots for the wave's 32 queries: dQ^T += K^T dS^T.
// masked: a slot is valid iff its index is < nvalid and (causal) <= lim.
template <int D, int KIND, bool kCausal>
__device__ __forceinline__ void q_tile(const BwdBuf<D>& b, const LaneOffs<bf16_t, D>& lo,
                                       const QFrag<bf16_t, D>& qf, const QFrag<bf16_t, D>& df,
                                       f32x16* dq, float c, float lam2, float dlt, bool masked,
                                       int nvalid, int lim) {
  const int g = lane_id() >> 5;
#pragma unroll
  for (int kb = 0; kb < KT / 32; ++kb) {
    if (masked && 32 * kb >= nvalid) break;
    float wt[16];
    if (KIND == SK_SUM) rows16(b.w2, kb, g, wt);
    if (KIND == SK_PROD) rows16(b.t.w, kb, g, wt);
    const f32x16 s = tile_dot<D, kQAhead>(b.t.k, lo, qf, kb);
    f32x16 dp;
    if (KIND != SK_SUM) dp = tile_dot<D, kQAhead>(b.t.v, lo, df, kb);
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = key_of(kb, i, g);
      bool ok = true;
      if (masked) {
        ok = r < nvalid;
        if (kCausal) ok = ok && r <= lim;
      }
      // masked entries take exp2(-inf) = 0 (a select, not a branch)
      const float e = fast_exp2(ok ? fmaf(s[i], c, -lam2) : -INFINITY);
      if (KIND == SK_FULL) x[i] = e * (dp[i] - dlt);
      else if (KIND == SK_SUM) x[i] = -(e * wt[i]) * dlt;
      else x[i] = (e * wt[i]) * dp[i];
    }
    bf16x8_t pb[2];
    pack_bf16(x, pb);
    tile_tr_acc<D, kQAhead>(b.t.k, lo, dq, pb, kb);
  }
}

// -------------------------------------------------------- key-major tiles
// 32 key slots a wave (d = 64): K, V, dK and dV of 32 keys take 96 registers
// there, so one sweep computes both gradients. (At d = 128 they would take
// 192 and the kernels use the 16-key layout below.)

// One LDS tile of queries for the wave's 32 key slots (weights om, nu):
// dV^T += dO^T (w E) and dK^T += Q^T dS. Rows without a query carry
// t.w = +inf (E = 0). kUnit: om = nu = 1 (base case and bucket keys), when
// dP's accumulator starts at -Delta so that it ends at dP - Delta and no
// separate Delta values are held. kCausal: query index r valid iff r >= lim;
// kBucketMask: valid iff r < mlo or r >= mhi (the tile rows inside the
// slot's own bucket, a contiguous range since queries come in sorted order).
// use_dp: some slot of the wave has om != 0 (else dP is not needed).
template <int D, bool kCausal, bool kBucketMask, bool kUnit>
__device__ __forceinline__ void kv_tile(const BwdBuf<D>& b, const LaneOffs<bf16_t, D>& lo,
                                        const QFrag<bf16_t, D>& kf, const QFrag<bf16_t, D>& vf,
                                        f32x16* dk, f32x16* dv, float c, float om, float nu,
                                        int mlo, int mhi, bool use_dp, int nvalid, int lim,
                                        int skip_below) {
  const int g = lane_id() >> 5;
#pragma unroll
  for (int qb = 0; qb < KT / 32; ++qb) {
    if (32 * qb >= nvalid) break;
    if (kCausal && 32 * qb + 31 < skip_below) continue;   // the wave's keys all follow
    float lw[16], dl[16];
    rows16(b.t.w, qb, g, lw);
    rows16(b.w2, qb, g, dl);
    const f32x16 s = tile_dot<D>(b.t.k, lo, kf, qb);
    f32x16 dp = zero16();
    if (kUnit) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dp[i] = -dl[i];
      dp = tile_dot<D>(b.t.v, lo, vf, qb, dp);
    } else if (use_dp) {
      dp = tile_dot<D>(b.t.v, lo, vf, qb);
    }
    float e[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = key_of(qb, i, g);
      bool ok = true;
      if (kCausal) ok = r >= lim;
      if (kBucketMask) ok = ok && (r < mlo || r >= mhi);
      // rows without a query carry +inf; masked entries take exp2(-inf) = 0
      e[i] = fast_exp2(ok ? fmaf(s[i], c, -lw[i]) : -INFINITY);
    }
    bf16x8_t pb[2];
    if (kUnit || use_dp) {
      float pv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pv[i] = om * e[i];
      pack_bf16(pv, pb);
      tile_tr_acc<D>(b.t.v, lo, dv, pb, qb);
    }
    float pk[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      pk[i] = kUnit ? e[i] * dp[i] : e[i] * (om * dp[i] - nu * dl[i]);
    pack_bf16(pk, pb);
    tile_tr_acc<D>(b.t.k, lo, dk, pb, qb);
  }
}

// ------------------------------------------- key-major tiles, 16 keys a wave
// v_mfma_f32_16x16x32_bf16: A is 16 rows x 32 (lane l holds row l % 16,
// elements 8(l/16) .. +7), B is 32 x 16 (lane l holds column l % 16, rows
// 8(l/16) .. +7), the result 16 x 16 (lane l holds column l % 16, rows
// 4(l/16) .. +3). A wave owns 16 key slots: K and V of its slots are the B
// operands of S = Q K^T and dP = dO V^T over 16-query sub-blocks, and
// dK^T, dV^T (16 columns of d per product, keys as the result's columns)
// take 32-query blocks through transposing reads of the Q and dO tiles.
// K, V, dK and dV of 16 keys take 96 registers at d = 128, so one sweep
// computes both gradients (the 32-key layout would need 192 and two sweeps).
typedef float f32x4 __attribute__((ext_vector_type(4)));

// The k index of step st runs over 16-byte chunks st + 4(l/16) of the row
// (elements 8st + 32(l/16) .. +7), in both operands of S and dP: then the
// 16 lanes of each quarter read one chunk column of 16 rows and the next
// quarter the chunk 4 further, which the LDS serves without bank conflicts
// (chunks 4st + l/16 put every row's two chunks into one conflicting pair).
template <int D>
struct Frag16 {
  bf16x8_t v[D / 32];   // v[st]: row elements 8st + 32(l/16) .. +7
};

template <int D>
struct Acc16 {
  f32x4 a[D / 16];      // a[mb][i]: column 16mb + 4(l/16) + i of the lane's key row
};

template <int D>
__device__ __forceinline__ void load_frag16(Frag16<D>& f, __amdgpu_buffer_rsrc_t r, int64_t row) {
  const int g = lane_id() >> 4;
  const uint32_t base = row >= 0 ? uint32_t(row) * (D * 2u) : kOob;
#pragma unroll
  for (int st = 0; st < D / 32; ++st)
    f.v[st] = __builtin_bit_cast(bf16x8_t, buf_load16(r, base + (8 * st + 32 * g) * 2));
}

// Per-lane LDS byte offsets within one bf16 tile (Buf<bf16_t, D> layout):
//   rd[st]: A operand of S / dP, row l % 16 of a 16-row sub-block, chunk
//           st + 4(l/16) (a sub-block 16 rows further adds 16 rows: the
//           swizzle repeats every 16 rows);
//   tr[mb]: transposing read of rows 4(l/16) + (l%16)/4 (then 16 rows
//           further), columns 16mb + 4(l % 4): lane l receives column
//           16mb + l % 16 of four consecutive rows.
template <int D>
struct Offs16 {
  using B = Buf<bf16_t, D>;
  static_assert(D == 128, "the swizzle repeats every 16 rows for d = 128");
  uint32_t rd[D / 32];
  uint32_t tr[D / 16];
  __device__ __forceinline__ void init() {
    int lane = lane_id();
    asm volatile("" : "+v"(lane));
    const int r16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int st = 0; st < D / 32; ++st)
      rd[st] = uint32_t(r16 * B::CPR + ((st + 4 * g) ^ B::swz_t(r16))) * 16u;
    const int row = 4 * g + (r16 >> 2);
#pragma unroll
    for (int mb = 0; mb < D / 16; ++mb) {
      const int d = 16 * mb + 4 * (r16 & 3);
      tr[mb] = uint32_t(row * B::CPR + ((d >> 3) ^ B::swz_t(row))) * 16u + uint32_t(d & 7) * 2u;
    }
  }
};

// S (or dP) for the 16-row sub-block at row r0 of the tile array.
template <int D>
__device__ __forceinline__ f32x4 dot16(const bf16_t* arr, const Offs16<D>& o,
                                       const Frag16<D>& f, int r0, f32x4 acc) {
  const char* base = reinterpret_cast<const char*>(arr) + r0 * D * 2;
  bf16x8_t x[D / 32];
#pragma unroll
  for (int st = 0; st < D / 32; ++st) x[st] = *reinterpret_cast<const bf16x8_t*>(base + o.rd[st]);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
  for (int st = 0; st < D / 32; ++st)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[st], f.v[st], acc, 0, 0, 0);
  __builtin_amdgcn_s_setprio(0);
  return acc;
}

// acc.a[mb] += (rows [r0, r0 + 32) of the tile array)^T p, p packed with
// element j of the lane's B operand for row r0 + 4(l/16) + j (j < 4) and
// r0 + 16 + 4(l/16) + j - 4 (j >= 4).
template <int D>
__device__ __forceinline__ void tr_acc16(const bf16_t* arr, const Offs16<D>& o, Acc16<D>& acc,
                                         bf16x8_t p, int r0) {
  const char* base = reinterpret_cast<const char*>(arr) + r0 * D * 2;
  // the transposing reads of kGroup column blocks are issued ahead of their
  // MFMAs (4 kGroup registers in flight; all eight at d = 128 measured
  // best, with four the kernels were about 1% slower)
  constexpr int kGroup = 8;
#pragma unroll
  for (int m0 = 0; m0 < D / 16; m0 += kGroup) {
    v4i16_t x[kGroup][2];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      x[j][0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + o.tr[m0 + j]));
      x[j][1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16_t*)(base + o.tr[m0 + j] + 16 * D * 2));
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const bf16x8_t a = __builtin_bit_cast(
          bf16x8_t, __builtin_shufflevector(x[j][0], x[j][1], 0, 1, 2, 3, 4, 5, 6, 7));
      acc.a[m0 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, p, acc.a[m0 + j], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  }
}

// One LDS tile of queries for the wave's 16 key slots: dV^T += dO^T (w E),
// dK^T += Q^T dS in one pass (arguments as kv_tile's).
template <int D, bool kCausal, bool kBucketMask, bool kUnit>
__device__ __forceinline__ void kv_tile16(const BwdBuf<D>& b, const Offs16<D>& o,
                                          const Frag16<D>& kf, const Frag16<D>& vf,
                                          Acc16<D>& dk, Acc16<D>& dv, float c, float om,
                                          float nu, int mlo, int mhi, bool use_dp, int nvalid,
                                          int lim, int skip_below) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int qb = 0; qb < KT / 32; ++qb) {
    if (32 * qb >= nvalid) break;
    if (kCausal && 32 * qb + 31 < skip_below) continue;   // the wave's keys all follow
    float pv[8], pk[8];
#pragma unroll
    for (int sq = 0; sq < 2; ++sq) {
      const int r0 = 32 * qb + 16 * sq;
      const float4 lw = *reinterpret_cast<const float4*>(b.t.w + r0 + 4 * g);
      const float4 dl = *reinterpret_cast<const float4*>(b.w2 + r0 + 4 * g);
      const float lwa[4] = {lw.x, lw.y, lw.z, lw.w};
      const float dla[4] = {dl.x, dl.y, dl.z, dl.w};
      const f32x4 s = dot16<D>(b.t.k, o, kf, r0, f32x4{0.f, 0.f, 0.f, 0.f});
      f32x4 dp = {0.f, 0.f, 0.f, 0.f};
      if (kUnit) dp = dot16<D>(b.t.v, o, vf, r0, f32x4{-dla[0], -dla[1], -dla[2], -dla[3]});
      else if (use_dp) dp = dot16<D>(b.t.v, o, vf, r0, dp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + 4 * g + i;
        bool ok = true;
        if (kCausal) ok = r >= lim;
        if (kBucketMask) ok = ok && (r < mlo || r >= mhi);
        const float e = fast_exp2(ok ? fmaf(s[i], c, -lwa[i]) : -INFINITY);
        pv[4 * sq + i] = om * e;
        pk[4 * sq + i] = kUnit ? e * dp[i] : e * (om * dp[i] - nu * dla[i]);
      }
    }
    bf16x8_t p;
    if (kUnit || use_dp) {
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = (__bf16)pv[j];
      tr_acc16<D>(b.t.v, o, dv, p, 32 * qb);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = (__bf16)pk[j];
    tr_acc16<D>(b.t.k, o, dk, p, 32 * qb);
  }
}

template <int D>
__device__ __forceinline__ void zero16(Acc16<D>& a) {
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) a.a[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int D>
__device__ __forceinline__ void scale16(Acc16<D>& a, float f) {
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) a.a[mb] *= f;
}

template <int D>
__device__ __forceinline__ void add_row16(Acc16<D>& a, const float* row) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) {
    const float4 v = *reinterpret_cast<const float4*>(row + 16 * mb + 4 * g);
    a.a[mb][0] += v.x;
    a.a[mb][1] += v.y;
    a.a[mb][2] += v.z;
    a.a[mb][3] += v.w;
  }
}

template <int D>
__device__ __forceinline__ void add_row16_bf16(Acc16<D>& a, const bf16_t* row) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) {
    const uint2 v = *reinterpret_cast<const uint2*>(row + 16 * mb + 4 * g);
    a.a[mb][0] += bf16_lo(v.x);
    a.a[mb][1] += bf16_hi(v.x);
    a.a[mb][2] += bf16_lo(v.y);
    a.a[mb][3] += bf16_hi(v.y);
  }
}

template <int D>
__device__ __forceinline__ void store_row16_f32(const Acc16<D>& a, float* row) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb)
    *reinterpret_cast<float4*>(row + 16 * mb + 4 * g) =
        make_float4(a.a[mb][0], a.a[mb][1], a.a[mb][2], a.a[mb][3]);
}

template <int D>
__device__ __forceinline__ void store_row16_bf16(const Acc16<D>& a, bf16_t* row) {
  const int g = lane_id() >> 4;
#pragma unroll
  for (int mb = 0; mb < D / 16; ++mb) {
    const uint32_t lo = uint32_t(f32_to_bf16(a.a[mb][0])) | (uint32_t(f32_to_bf16(a.a[mb][1])) << 16);
    const uint32_t hi = uint32_t(f32_to_bf16(a.a[mb][2])) | (uint32_t(f32_to_bf16(a.a[mb][3])) << 16);
    *reinterpret_cast<uint2*>(row + 16 * mb + 4 * g) = make_uint2(lo, hi);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const bf16_t* base, int head, int64_t n,
                                                          int d) {
  return head_rsrc(base + int64_t(head) * n * d, n * d * 2);
}

// ------------------------------------------------------------- EXACT items
// Work item lin = head * items_per_head + blk * tiles_per_block + t: tile t
// (kAttnQ rows) of diagonal or full block blk.

// dQ of query tile t (causal: longest tiles first).
template <int D, bool kCausal>
__device__ __forceinline__ void q_exact_item(const BwdArgs& a, BwdSmem<D>& sm, uint32_t lin) {
  const uint32_t gx = a.items_per_head;
  const int head = int(lin / gx);
  const uint32_t bx = lin - uint32_t(head) * gx;
  const uint32_t tpb = a.tiles_per_block;
  const uint32_t blk = bx / tpb;
  const uint32_t tl = bx - blk * tpb;
  const int64_t tile = kCausal ? int64_t(tpb - 1 - tl) : int64_t(tl);
  const int64_t b_lo = blk * a.block;
  const int64_t b_hi = b_lo + a.block < a.n ? b_lo + a.block : a.n;
  const int64_t q0 = b_lo + tile * kAttnQ;
  const int64_t q_end = q0 + kAttnQ < b_hi ? q0 + kAttnQ : b_hi;
  const int wave = threadIdx.x >> 6;
  const int ql = lane_id() & 31;
  const int64_t qw0 = q0 + wave * kQW;
  const int64_t qrow = qw0 + ql < q_end ? qw0 + ql : -1;

  const auto Qr = rsrc_of(a.Q, head, a.n, D);
  const auto Kr = rsrc_of(a.K, head, a.n, D);
  const auto Vr = rsrc_of(a.V, head, a.n, D);
  const auto dOr = rsrc_of(a.dO, head, a.n, D);
  QFrag<bf16_t, D> qf, df;
  load_q<bf16_t, D>(qf, Qr, qrow);
  load_q<bf16_t, D>(df, dOr, qrow);
  LaneOffs<bf16_t, D> lo;
  lo.init();
  float lam2 = INFINITY, dlt = 0.f;
  if (qrow >= 0) {
    lam2 = a.lse[int64_t(head) * a.n + qrow] * kLog2e;
    dlt = a.delta[int64_t(head) * a.n + qrow];
  }
  f32x16 dq[D / 32];
  zero_acc<D>(dq);

  const int64_t k_end = kCausal ? q_end : b_hi;
  const int ntiles = int((k_end - b_lo + KT - 1) / KT);
  Pipe<bf16_t, D> pipe;
  auto issue = [&](int t) {
    const int64_t k0 = b_lo + int64_t(t) * KT;
    const int nv = int(k_end - k0 < KT ? k_end - k0 : KT);
    pipe.issue(sm.buf[t & 1].t, Kr, Vr, true,
               [&](int row) { return row < nv ? int(k0 + row) : -1; },
               [](int) { return 1.f; });
  };
  issue(0);
  pipe.commit(sm.buf[0].t, true);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) issue(t + 1);
    const int64_t k0 = b_lo + int64_t(t) * KT;
    const int nvalid = int(k_end - k0 < KT ? k_end - k0 : KT);
    const bool skip = kCausal && k0 > qw0 + kQW - 1;
    if (!skip) {
      const bool masked = nvalid < KT || (kCausal && k0 + KT - 1 > qw0);
      const int64_t dl = qrow - k0;
      const int lim = dl < 0 ? -1 : (dl > KT ? KT : int(dl));
      q_tile<D, SK_FULL, kCausal>(sm.buf[t & 1], lo, qf, df, dq, a.scale_log2, lam2, dlt, masked,
                                  nvalid, lim);
    }
    if (t + 1 < ntiles) pipe.commit(sm.buf[(t + 1) & 1].t, true);
    __syncthreads();
  }
  if (qrow < 0) return;
  scale_acc<D>(dq, a.scale);
  for (int lv = 0; lv < a.merge_levels; ++lv) {
    const int64_t idx = level_slot(a, lv, blk, b_lo, qrow, true, head);
    if (idx >= 0) add_row_bf16<D>(dq, a.part_dq + idx * D);
  }
  store_row_bf16<D>(dq, a.dQ + (int64_t(head) * a.n + qrow) * D);
}

// One sweep of the block's queries [q_lo, b_hi) for the wave's keys.
template <int D, bool kCausal>
__device__ __forceinline__ void kv_exact_sweep(const BwdArgs& a, BwdSmem<D>& sm, int head,
                                               int64_t q_lo, int64_t b_hi, int64_t kw0,
                                               int64_t krow, const QFrag<bf16_t, D>& kf,
                                               const QFrag<bf16_t, D>& vf, f32x16* dk,
                                               f32x16* dv) {
  const auto Qr = rsrc_of(a.Q, head, a.n, D);
  const auto dOr = rsrc_of(a.dO, head, a.n, D);
  LaneOffs<bf16_t, D> lo;
  lo.init();
  const int ntiles = int((b_hi - q_lo + KT - 1) / KT);
  const float* lse = a.lse + int64_t(head) * a.n;
  const float* dl = a.delta + int64_t(head) * a.n;
  Pipe<bf16_t, D> pipe;
  auto issue = [&](int t) {
    const int64_t r0 = q_lo + int64_t(t) * KT;
    const int nv = int(b_hi - r0 < KT ? b_hi - r0 : KT);
    BwdBuf<D>& b = sm.buf[t & 1];
    pipe.issue(b.t, Qr, dOr, true, [&](int row) { return row < nv ? int(r0 + row) : -1; },
               [&](int row) { return row < nv ? lse[r0 + row] * kLog2e : INFINITY; });
    if (threadIdx.x < KT) b.w2[threadIdx.x] = int(threadIdx.x) < nv ? dl[r0 + threadIdx.x] : 0.f;
  };
  issue(0);
  pipe.commit(sm.buf[0].t, true);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) issue(t + 1);
    const int64_t r0 = q_lo + int64_t(t) * KT;
    const int nvalid = int(b_hi - r0 < KT ? b_hi - r0 : KT);
    // causal: query r0 + r is valid for key krow iff r >= krow - r0
    const int64_t dk0 = (krow >= 0 ? krow : kw0) - r0;
    const int lim = dk0 < 0 ? 0 : (dk0 > KT ? KT : int(dk0));
    const int64_t sb = kw0 - r0;
    const int skip_below = sb < 0 ? 0 : (sb > KT ? KT : int(sb));
    kv_tile<D, kCausal, false, true>(sm.buf[t & 1], lo, kf, vf, dk, dv, a.scale_log2, 1.f, 1.f,
                                     0, 0, true, nvalid, lim, skip_below);
    if (t + 1 < ntiles) pipe.commit(sm.buf[(t + 1) & 1].t, true);
    __syncthreads();
  }
}

// Adds the level partials of key row krow (base block blk) and stores it.
template <int D>
__device__ __forceinline__ void finish_exact_key(const BwdArgs& a, f32x16* acc, bool is_k,
                                                 uint32_t blk, int64_t b_lo, int64_t krow,
                                                 int head) {
  if (is_k) scale_acc<D>(acc, a.scale);
  for (int lv = 0; lv < a.merge_levels; ++lv) {
    const int64_t idx = level_slot(a, lv, blk, b_lo, krow, false, head);
    if (idx >= 0) add_row_bf16<D>(acc, (is_k ? a.part_dk : a.part_dv) + idx * D);
  }
  store_row_bf16<D>(acc, (is_k ? a.dK : a.dV) + (int64_t(head) * a.n + krow) * D);
}

// dK, dV of key tile t (kAttnQ keys) against the block's queries (causal:
// the queries at or after the tile's first key).
template <int D, bool kCausal>
__device__ __forceinline__ void kv_exact_item(const BwdArgs& a, BwdSmem<D>& sm, uint32_t lin) {
  const uint32_t gx = a.items_per_head;
  const int head = int(lin / gx);
  const uint32_t bx = lin - uint32_t(head) * gx;
  const uint32_t tpb = a.tiles_per_block;
  const uint32_t blk = bx / tpb;
  const int64_t tile = bx - blk * tpb;
  const int64_t b_lo = blk * a.block;
  const int64_t b_hi = b_lo + a.block < a.n ? b_lo + a.block : a.n;
  const int64_t k0 = b_lo + tile * kAttnQ;
  const int64_t k_end = k0 + kAttnQ < b_hi ? k0 + kAttnQ : b_hi;
  const int wave = threadIdx.x >> 6;
  const int ql = lane_id() & 31;
  const int64_t kw0 = k0 + wave * kQW;
  const int64_t krow = kw0 + ql < k_end ? kw0 + ql : -1;
  const int64_t q_lo = kCausal ? k0 : b_lo;
  const auto Kr = rsrc_of(a.K, head, a.n, D);
  const auto Vr = rsrc_of(a.V, head, a.n, D);
  QFrag<bf16_t, D> kf, vf;
  load_q<bf16_t, D>(kf, Kr, krow);
  load_q<bf16_t, D>(vf, Vr, krow);
  f32x16 dk[D / 32], dv[D / 32];
  zero_acc<D>(dk);
  zero_acc<D>(dv);
  kv_exact_sweep<D, kCausal>(a, sm, head, q_lo, b_hi, kw0, krow, kf, vf, dk, dv);
  if (krow < 0) return;
  finish_exact_key<D>(a, dv, false, blk, b_lo, krow, head);
  finish_exact_key<D>(a, dk, true, blk, b_lo, krow, head);
}

// ------------------------------------------------------ bucket item decode
struct BucketItem {
  int lv;
  int head;
  int64_t seg;
  int64_t bucket;
  int64_t chunk;      // chunk of kAttnQ rows within the bucket
  int64_t slot0;      // first sorted position of the bucket in perm_q / perm_k
  int64_t rec;        // head * nodes + node - 1
};

__device__ __forceinline__ BucketItem decode_bucket(const BwdArgs& a, int64_t w) {
  BucketItem it;
  int lv = 0;
  for (int l = 1; l < a.table.count; ++l)
    if (w >= a.table.lv[l].att_wg0) lv = l;
  const Level& L = a.table.lv[lv];
  uint32_t rem = uint32_t(w - L.att_wg0);
  const uint32_t nq = uint32_t(L.att_qch), nbk = uint32_t(L.nbucket), nsg = uint32_t(L.nseg);
  uint32_t quo = rem / nq;
  it.chunk = rem - quo * nq;
  rem = quo;
  quo = rem / nbk;
  it.bucket = rem - quo * nbk;
  rem = quo;
  quo = rem / nsg;
  it.seg = rem - quo * nsg;
  it.head = int(quo);
  it.lv = lv;
  it.slot0 = (int64_t(lv) * a.heads + it.head) * a.S + it.seg * L.h + it.bucket * L.b_eff;
  it.rec = int64_t(it.head) * a.nodes + ((int64_t(1) << lv) + it.seg - 1);
  return it;
}

// dQ of one bucket chunk's queries: the bucket's keys (1, 1), the uniform
// sample (0, alpha), the V-norm sample (weight, 0); samples inside the
// bucket weigh (0, 0). Slot rows and weights of up to kSlotCap slots (a
// window of tiles) are staged in LDS up front.
template <int D>
__device__ __forceinline__ void q_bucket_item(const BwdArgs& a, BwdSmem<D>& sm, int64_t w) {
  constexpr int kWin = kSlotCap / KT;
  const BucketItem it = decode_bucket(a, w);
  const Level& L = a.table.lv[it.lv];
  const int b_eff = L.b_eff;
  const int64_t h = L.h;
  const int wave = threadIdx.x >> 6;
  const int ql = lane_id() & 31;
  const int64_t qi = it.chunk * kAttnQ + wave * kQW + ql;
  const int64_t qrow = qi < b_eff ? int64_t(a.perm_q[it.slot0 + qi]) : -1;
  const int ucount = L.u_cnt;
  const int vcount = a.meta[it.rec * 4 + 1];
  const float alpha = L.alpha;
  const int64_t bucket = it.bucket;

  const auto Qr = rsrc_of(a.Q, it.head, a.n, D);
  const auto Kr = rsrc_of(a.K, it.head, a.n, D);
  const auto Vr = rsrc_of(a.V, it.head, a.n, D);
  const auto dOr = rsrc_of(a.dO, it.head, a.n, D);
  QFrag<bf16_t, D> qf, df;
  load_q<bf16_t, D>(qf, Qr, qrow);
  load_q<bf16_t, D>(df, dOr, qrow);
  LaneOffs<bf16_t, D> lo;
  lo.init();
  float lam2 = INFINITY, dlt = 0.f;
  if (qrow >= 0) {
    lam2 = a.lse[int64_t(it.head) * a.n + qrow] * kLog2e;
    dlt = a.delta[int64_t(it.head) * a.n + qrow];
  }
  f32x16 dq[D / 32];
  zero_acc<D>(dq);

  const int t_b = (b_eff + KT - 1) / KT;
  const int t_u = (ucount + KT - 1) / KT;
  const int t_v = (vcount + KT - 1) / KT;
  const int ntiles = t_b + t_u + t_v;
  auto seg_of = [&](int t, int& j0, int& cnt) {
    if (t < t_b) { j0 = t * KT; cnt = b_eff; return 0; }
    if (t < t_b + t_u) { j0 = (t - t_b) * KT; cnt = ucount; return 1; }
    j0 = (t - t_b - t_u) * KT; cnt = vcount; return 2;
  };
  auto fill = [&](int t0) {
    const int32_t* pk = a.perm_k + it.slot0;
    const int32_t* ui = a.u_idx + it.rec * a.m;
    const int32_t* ub = a.u_bkt + it.rec * a.m;
    const int32_t* vi = a.v_idx + it.rec * a.m;
    const int32_t* vb = a.v_bkt + it.rec * a.m;
    const float* vw = a.v_w + it.rec * a.m;
    for (int e = threadIdx.x; e < kSlotCap; e += kThreads) {
      const int t = t0 + e / KT;
      int32_t row = -1;
      float om = 0.f, nu = 0.f;
      if (t < ntiles) {
        int j0, cnt;
        const int sg = seg_of(t, j0, cnt);
        const int j = j0 + e % KT;
        if (j < cnt) {
          if (sg == 0) {
            row = pk[j];
            om = nu = 1.f;
          } else if (sg == 1) {
            row = ui[j];
            if (ub[j] != bucket) nu = alpha;
          } else {
            row = vi[j];
            if (vb[j] != bucket) om = vw[j];
          }
        }
      }
      sm.srow[e] = row;
      sm.sw[e] = om;
      sm.sw2[e] = nu;
    }
  };
  auto needs_v = [&](int t) { return t < t_b || t >= t_b + t_u; };
  Pipe<bf16_t, D> pipe;
  auto issue = [&](int t) {
    const int e0 = (t % kWin) * KT;
    BwdBuf<D>& b = sm.buf[t & 1];
    pipe.issue(b.t, Kr, Vr, needs_v(t), [&](int row) { return int(sm.srow[e0 + row]); },
               [&](int slot) { return sm.sw[e0 + slot]; });
    if (threadIdx.x < KT) b.w2[threadIdx.x] = sm.sw2[e0 + threadIdx.x];
  };
  fill(0);
  __syncthreads();
  issue(0);
  pipe.commit(sm.buf[0].t, needs_v(0));
  __syncthreads();
  // one loop per segment, each with its own slot weights
  auto step = [&](int t, auto kind) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kind)::value;
    if (t + 1 < ntiles) {
      if ((t + 1) % kWin == 0) {
        fill(t + 1);
        __syncthreads();
      }
      issue(t + 1);
    }
    int j0, cnt;
    seg_of(t, j0, cnt);
    const int nvalid = cnt - j0 < KT ? cnt - j0 : KT;
    q_tile<D, KIND, false>(sm.buf[t & 1], lo, qf, df, dq, a.scale_log2, lam2, dlt, nvalid < KT,
                           nvalid, KT);
    if (t + 1 < ntiles) pipe.commit(sm.buf[(t + 1) & 1].t, needs_v(t + 1));
    __syncthreads();
  };
  int t = 0;
  for (; t < t_b; ++t) step(t, std::integral_constant<int, SK_FULL>{});
  for (; t < t_b + t_u; ++t) step(t, std::integral_constant<int, SK_SUM>{});
  for (; t < ntiles; ++t) step(t, std::integral_constant<int, SK_PROD>{});
  if (qrow < 0) return;
  scale_acc<D>(dq, a.scale);
  if (a.table.causal) {
    // queries of sub-problem seg are rows [2 seg h + h, 2 seg h + 2h); their
    // slot is seg h + (row - 2 seg h - h)
    const int64_t slot = (int64_t(it.lv) * a.heads + it.head) * a.S + (qrow - (it.seg + 1) * h);
    store_row_bf16<D>(dq, a.part_dq + slot * D);
  } else {
    store_row_bf16<D>(dq, a.dQ + (int64_t(it.head) * a.n + qrow) * D);
  }
}

// Stages query positions [p0, p0 + count) of a sorted segment (perm_q at
// `perm`) for the key-major kernels: rows, Lambda log2(e) and Delta.
template <int D>
__device__ __forceinline__ void fill_queries(const BwdArgs& a, BwdSmem<D>& sm, const int32_t* perm,
                                             int64_t p0, int64_t count, int head) {
  const float* lse = a.lse + int64_t(head) * a.n;
  const float* dl = a.delta + int64_t(head) * a.n;
  for (int e = threadIdx.x; e < kSlotCap; e += kThreads) {
    int32_t row = -1;
    float l2 = INFINITY, dt = 0.f;
    if (e < count) {
      row = perm[p0 + e];
      l2 = lse[row] * kLog2e;
      dt = dl[row];
    }
    sm.srow[e] = row;
    sm.sw[e] = l2;
    sm.sw2[e] = dt;
  }
}

// Key-major sweep over `count` queries at sorted positions [p0, p0 + count)
// of `perm` for the wave's key slots. kMask: a query in bucket bkt (its
// position / b_eff) is skipped.
template <int D, bool kMask>
__device__ __forceinline__ void kv_sorted_loop(const BwdArgs& a, BwdSmem<D>& sm,
                                               const int32_t* perm, int64_t p0, int64_t count,
                                               int b_eff, int head, const QFrag<bf16_t, D>& kf,
                                               const QFrag<bf16_t, D>& vf, f32x16* dk,
                                               f32x16* dv, float om, float nu, int bkt,
                                               bool use_dp) {
  constexpr int kWin = kSlotCap / KT;
  const auto Qr = rsrc_of(a.Q, head, a.n, D);
  const auto dOr = rsrc_of(a.dO, head, a.n, D);
  LaneOffs<bf16_t, D> lo;
  lo.init();
  const int ntiles = int((count + KT - 1) / KT);
  Pipe<bf16_t, D> pipe;
  auto issue = [&](int t) {
    const int e0 = (t % kWin) * KT;
    BwdBuf<D>& b = sm.buf[t & 1];
    pipe.issue(b.t, Qr, dOr, true, [&](int row) { return int(sm.srow[e0 + row]); },
               [&](int row) { return sm.sw[e0 + row]; });
    if (threadIdx.x < KT) b.w2[threadIdx.x] = sm.sw2[e0 + threadIdx.x];
  };
  fill_queries(a, sm, perm, p0, count, head);
  __syncthreads();
  issue(0);
  pipe.commit(sm.buf[0].t, true);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) {
      if ((t + 1) % kWin == 0) {
        fill_queries(a, sm, perm, p0 + int64_t(t + 1) * KT, count - int64_t(t + 1) * KT, head);
        __syncthreads();
      }
      issue(t + 1);
    }
    const int64_t left = count - int64_t(t) * KT;
    const int nvalid = int(left < KT ? left : KT);
    // tile rows inside the slot's bucket: sorted positions
    // [bkt b_eff, (bkt + 1) b_eff), clamped to the tile
    int mlo = 0, mhi = 0;
    if (kMask && bkt >= 0) {
      const int64_t first = int64_t(bkt) * b_eff - (p0 + int64_t(t) * KT);
      const int64_t last = first + b_eff;
      mlo = int(first < 0 ? 0 : (first > KT ? KT : first));
      mhi = int(last < 0 ? 0 : (last > KT ? KT : last));
    }
    // bucket keys (no mask) have om = nu = 1
    kv_tile<D, false, kMask, !kMask>(sm.buf[t & 1], lo, kf, vf, dk, dv, a.scale_log2, om, nu,
                                     mlo, mhi, use_dp, nvalid, 0, 0);
    if (t + 1 < ntiles) pipe.commit(sm.buf[(t + 1) & 1].t, true);
    __syncthreads();
  }
}

// Adds the node's sample slots drawn on key row krow (their partials over
// every query chunk, slots in increasing order) to the row's dK (is_k) or
// dV, then stores it: a level partial (causal) or the output.
template <int D>
__device__ __forceinline__ void finish_bucket_key(const BwdArgs& a, const BucketItem& it,
                                                  f32x16* acc, bool is_k, int64_t krow) {
  const Level& L = a.table.lv[it.lv];
  const int64_t h = L.h;
  if (is_k) scale_acc<D>(acc, a.scale);
  const int64_t k_lo = a.table.causal ? 2 * it.seg * h : 0;
  const int64_t kslot = (int64_t(it.lv) * a.heads + it.head) * a.S + it.seg * h + (krow - k_lo);
  const int64_t nqc = L.smp_nqc;
  const int64_t item0 = L.smp_wg0 + (int64_t(it.head) * L.nseg + it.seg) * L.smp_nsc * nqc;
  const float* part = is_k ? a.slot_dk : a.slot_dv;
  for (int t = a.slot_first[kslot]; t >= 0; t = a.slot_next[it.rec * 2 * a.m + t]) {
    const int64_t sc = t / kAttnQ;
    const int tt = t - int(sc) * kAttnQ;
    for (int64_t qc = 0; qc < nqc; ++qc)
      add_row_f32<D>(acc, part + ((item0 + sc * nqc + qc) * kAttnQ + tt) * D);
  }
  if (a.table.causal)
    store_row_bf16<D>(acc, (is_k ? a.part_dk : a.part_dv) + kslot * D);
  else
    store_row_bf16<D>(acc, (is_k ? a.dK : a.dV) + (int64_t(it.head) * a.n + krow) * D);
}

// dK, dV of one bucket chunk's keys against the bucket's queries, plus the
// node's sample slots drawn on these key rows.
template <int D>
__device__ __forceinline__ void kv_bucket_item(const BwdArgs& a, BwdSmem<D>& sm, int64_t w) {
  const BucketItem it = decode_bucket(a, w);
  const int b_eff = a.table.lv[it.lv].b_eff;
  const int wave = threadIdx.x >> 6;
  const int ql = lane_id() & 31;
  const int64_t ki = it.chunk * kAttnQ + wave * kQW + ql;
  const int64_t krow = ki < b_eff ? int64_t(a.perm_k[it.slot0 + ki]) : -1;
  const auto Kr = rsrc_of(a.K, it.head, a.n, D);
  const auto Vr = rsrc_of(a.V, it.head, a.n, D);
  QFrag<bf16_t, D> kf, vf;
  load_q<bf16_t, D>(kf, Kr, krow);
  load_q<bf16_t, D>(vf, Vr, krow);
  f32x16 dk[D / 32], dv[D / 32];
  zero_acc<D>(dk);
  zero_acc<D>(dv);
  kv_sorted_loop<D, false>(a, sm, a.perm_q, it.slot0, b_eff, b_eff, it.head, kf, vf, dk, dv,
                           1.f, 1.f, 0, true);
  if (krow < 0) return;
  finish_bucket_key<D>(a, it, dv, false, krow);
  finish_bucket_key<D>(a, it, dk, true, krow);
}

// Partial dK, dV of kAttnQ sample slots of one node (uniform list then
// V-norm list) against one chunk of the node's queries in sorted order.
template <int D>
__device__ __forceinline__ void kv_sample_item(const BwdArgs& a, BwdSmem<D>& sm, int64_t w) {
  int lv = 0;
  for (int l = 1; l < a.table.count; ++l)
    if (w >= a.table.lv[l].smp_wg0) lv = l;
  const Level& L = a.table.lv[lv];
  uint32_t rem = uint32_t(w - L.smp_wg0);
  const uint32_t nqc = uint32_t(L.smp_nqc), nsc = uint32_t(L.smp_nsc), nsg = uint32_t(L.nseg);
  uint32_t quo = rem / nqc;
  const int64_t qc = rem - quo * nqc;
  rem = quo;
  quo = rem / nsc;
  const int64_t sc = rem - quo * nsc;
  rem = quo;
  quo = rem / nsg;
  const int64_t seg = rem - quo * nsg;
  const int head = int(quo);
  const int64_t h = L.h;
  const int64_t rec = int64_t(head) * a.nodes + ((int64_t(1) << lv) + seg - 1);
  const int ucount = a.meta[rec * 4];
  const int vcount = a.meta[rec * 4 + 1];
  const int wave = threadIdx.x >> 6;
  const int ql = lane_id() & 31;
  const int64_t t = sc * kAttnQ + wave * kQW + ql;
  int64_t krow = -1;
  float om = 0.f, nu = 0.f;
  int bkt = -1;
  if (t < ucount) {
    krow = a.u_idx[rec * a.m + t];
    bkt = a.u_bkt[rec * a.m + t];
    nu = L.alpha;
  } else if (t - ucount < vcount) {
    krow = a.v_idx[rec * a.m + (t - ucount)];
    bkt = a.v_bkt[rec * a.m + (t - ucount)];
    om = a.v_w[rec * a.m + (t - ucount)];
  }
  const auto Kr = rsrc_of(a.K, head, a.n, D);
  const auto Vr = rsrc_of(a.V, head, a.n, D);
  QFrag<bf16_t, D> kf, vf;
  load_q<bf16_t, D>(kf, Kr, krow);
  const int64_t p0 = qc * kBwdQChunk;
  const int64_t count = h - p0 < kBwdQChunk ? h - p0 : kBwdQChunk;
  const int64_t seg0 = (int64_t(lv) * a.heads + head) * a.S + seg * h;
  const int64_t idx = w * kAttnQ + wave * kQW + ql;
  const int32_t* perm = a.perm_q + seg0;
  // uniform slots have om = 0: no dV and no dP for them
  const bool wave_om = __ballot(om != 0.f) != 0;
  load_q<bf16_t, D>(vf, Vr, krow);
  f32x16 dk[D / 32], dv[D / 32];
  zero_acc<D>(dk);
  zero_acc<D>(dv);
  kv_sorted_loop<D, true>(a, sm, perm, p0, count, L.b_eff, head, kf, vf, dk, dv, om, nu, bkt,
                          wave_om);
  if (krow < 0) return;
  scale_acc<D>(dk, a.scale);
  store_row_f32<D>(dk, a.slot_dk + idx * D);
  store_row_f32<D>(dv, a.slot_dv + idx * D);
}

// ------------------------------------- key-major items, 16 keys a wave (d = 128)
// A work-group owns kAttnQ / 2 = 128 key slots (8 waves x 16). Bucket and
// sample items are the halves of the 256-slot items above: item w covers
// slots [128 (w mod 2), 128 (w mod 2) + 128) of item w / 2.
constexpr int kKW16 = 16;
constexpr int kKeys16 = kWaves * kKW16;
// At d = 128 the key-major kernels take the 16-key layout (one sweep for
// dK and dV). A bucket item keeps 256 key slots per work-group as two
// halves that share the bucket's query tiles.
template <int D, int MODE> constexpr bool kKv16 = D == 128;

template <int D, bool kCausal>
__device__ __forceinline__ void kv16_exact_sweep(const BwdArgs& a, BwdSmem<D>& sm, int head,
                                                 int64_t q_lo, int64_t b_hi, int64_t kw0,
                                                 int64_t krow, const Frag16<D>& kf,
                                                 const Frag16<D>& vf, Acc16<D>& dk,
                                                 Acc16<D>& dv) {
  const auto Qr = rsrc_of(a.Q, head, a.n, D);
  const auto dOr = rsrc_of(a.dO, head, a.n, D);
  Offs16<D> o;
  o.init();
  const int ntiles = int((b_hi - q_lo + KT - 1) / KT);
  const float* lse = a.lse + int64_t(head) * a.n;
  const float* dl = a.delta + int64_t(head) * a.n;
  Pipe<bf16_t, D> pipe;
  auto issue = [&](int t) {
    const int64_t r0 = q_lo + int64_t(t) * KT;
    const int nv = int(b_hi - r0 < KT ? b_hi - r0 : KT);
    BwdBuf<D>& b = sm.buf[t & 1];
    pipe.template issue<true>(b.t, Qr, dOr, true,
                              [&](int row) { return row < nv ? int(r0 + row) : -1; },
                              [&](int row) { return row < nv ? lse[r0 + row] * kLog2e : INFINITY; });
    if (threadIdx.x < KT) b.w2[threadIdx.x] = int(threadIdx.x) < nv ? dl[r0 + threadIdx.x] : 0.f;
  };
  issue(0);
  pipe.commit(sm.buf[0].t, true);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) issue(t + 1);
    const int64_t r0 = q_lo + int64_t(t) * KT;
    const int nvalid = int(b_hi - r0 < KT ? b_hi - r0 : KT);
    const int64_t dk0 = (krow >= 0 ? krow : kw0) - r0;
    const int lim = dk0 < 0 ? 0 : (dk0 > KT ? KT : int(dk0));
    const int64_t sb = kw0 - r0;
    const int skip_below = sb < 0 ? 0 : (sb > KT ? KT : int(sb));
    kv_tile16<D, kCausal, false, true>(sm.buf[t & 1], o, kf, vf, dk, dv, a.scale_log2, 1.f, 1.f,
                                       0, 0, true, nvalid, lim, skip_below);
    if (t + 1 < ntiles) pipe.commit(sm.buf[(t + 1) & 1].t, true);
    __syncthreads();
  }
}

// dK, dV of key tile `tile` (128 keys) of block blk against its queries.
template <int D, bool kCausal>
__device__ __forceinline__ void kv16_exact_keys(const BwdArgs& a, BwdSmem<D>& sm, int head,
                                                uint32_t blk, int64_t tile) {
  const int64_t b_lo = blk * a.block;
  const int64_t b_hi = b_lo + a.block < a.n ? b_lo + a.block : a.n;
  const int64_t k0 = b_lo + tile * kKeys16;
  const int64_t k_end = k0 + kKeys16 < b_hi ? k0 + kKeys16 : b_hi;
  const int wave = threadIdx.x >> 6;
  const int64_t kw0 = k0 + wave * kKW16;
  const int64_t kr = kw0 + (lane_id() & 15);
  const int64_t krow = kr < k_end ? kr : -1;
  const int64_t q_lo = kCausal ? k0 : b_lo;
  Frag16<D> kf, vf;
  load_frag16<D>(kf, rsrc_of(a.K, head, a.n, D), krow);
  load_frag16<D>(vf, rsrc_of(a.V, head, a.n, D), krow);
  Acc16<D> dk, dv;
  zero16<D>(dk);
  zero16<D>(dv);
  kv16_exact_sweep<D, kCausal>(a, sm, head, q_lo, b_hi, kw0, krow, kf, vf, dk, dv);
  if (krow < 0) return;
  scale16<D>(dk, a.scale);
  for (int lv = 0; lv < a.merge_levels; ++lv) {
    const int64_t idx = level_slot(a, lv, blk, b_lo, krow, false, head);
    if (idx >= 0) {
      add_row16_bf16<D>(dk, a.part_dk + idx * D);
      add_row16_bf16<D>(dv, a.part_dv + idx * D);
    }
  }
  store_row16_bf16<D>(dk, a.dK + (int64_t(head) * a.n + krow) * D);
  store_row16_bf16<D>(dv, a.dV + (int64_t(head) * a.n + krow) * D);
}

// Work item lin = head * items_per_head + blk * per_block + j. Non-causal:
// key tile j (per_block = tiles_per_block). Causal: key tiles j and
// tiles_per_block - 1 - j (per_block = ceil(tiles_per_block / 2)), one after
// the other, so that every item sweeps the same number of query tiles (key
// tile j sees the queries from its own rows to the block's end); each sweep
// ends with a barrier, after which the tile buffers are free.
template <int D, bool kCausal>
__device__ __forceinline__ void kv16_exact_item(const BwdArgs& a, BwdSmem<D>& sm, uint32_t lin) {
  const uint32_t gx = a.items_per_head;
  const int head = int(lin / gx);
  const uint32_t bx = lin - uint32_t(head) * gx;
  const uint32_t tpb = a.tiles_per_block;
  if constexpr (kCausal) {
    const uint32_t ppb = (tpb + 1) / 2;
    const uint32_t blk = bx / ppb;
    const uint32_t j = bx - blk * ppb;
    kv16_exact_keys<D, kCausal>(a, sm, head, blk, int64_t(j));
    if (tpb - 1 - j != j) kv16_exact_keys<D, kCausal>(a, sm, head, blk, int64_t(tpb - 1 - j));
  } else {
    const uint32_t blk = bx / tpb;
    kv16_exact_keys<D, kCausal>(a, sm, head, blk, int64_t(bx - blk * tpb));
  }
}

// Sweep over `count` queries at sorted positions [p0, p0 + count) of `perm`
// (kv_sorted_loop's arguments).
template <int D, bool kMask>
__device__ __forceinline__ void kv16_sorted_loop(const BwdArgs& a, BwdSmem<D>& sm,
                                                 const int32_t* perm, int64_t p0, int64_t count,
                                                 int b_eff, int head, const Frag16<D>& kf,
                                                 const Frag16<D>& vf, Acc16<D>& dk,
                                                 Acc16<D>& dv, float om, float nu, int bkt,
                                                 bool use_dp) {
  constexpr int kWin = kSlotCap / KT;
  const auto Qr = rsrc_of(a.Q, head, a.n, D);
  const auto dOr = rsrc_of(a.dO, head, a.n, D);
  Offs16<D> o;
  o.init();
  const int ntiles = int((count + KT - 1) / KT);
  Pipe<bf16_t, D> pipe;
  auto issue = [&](int t) {
    const int e0 = (t % kWin) * KT;
    BwdBuf<D>& b = sm.buf[t & 1];
    pipe.template issue<true>(b.t, Qr, dOr, true,
                              [&](int row) { return int(sm.srow[e0 + row]); },
                              [&](int row) { return sm.sw[e0 + row]; });
    if (threadIdx.x < KT) b.w2[threadIdx.x] = sm.sw2[e0 + threadIdx.x];
  };
  fill_queries(a, sm, perm, p0, count, head);
  __syncthreads();
  issue(0);
  pipe.commit(sm.buf[0].t, true);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) {
      if ((t + 1) % kWin == 0) {
        fill_queries(a, sm, perm, p0 + int64_t(t + 1) * KT, count - int64_t(t + 1) * KT, head);
        __syncthreads();
      }
      issue(t + 1);
    }
    const int64_t left = count - int64_t(t) * KT;
    const int nvalid = int(left < KT ? left : KT);
    int mlo = 0, mhi = 0;
    if (kMask && bkt >= 0) {
      const int64_t first = int64_t(bkt) * b_eff - (p0 + int64_t(t) * KT);
      const int64_t last = first + b_eff;
      mlo = int(first < 0 ? 0 : (first > KT ? KT : first));
      mhi = int(last < 0 ? 0 : (last > KT ? KT : last));
    }
    kv_tile16<D, false, kMask, !kMask>(sm.buf[t & 1], o, kf, vf, dk, dv, a.scale_log2, om, nu,
                                       mlo, mhi, use_dp, nvalid, 0, 0);
    if (t + 1 < ntiles) pipe.commit(sm.buf[(t + 1) & 1].t, true);
    __syncthreads();
  }
}

// Slot of key row krow among this item's level partials.
__device__ __forceinline__ int64_t bucket_kslot(const BwdArgs& a, const BucketItem& it,
                                                int64_t krow) {
  const int64_t h = a.table.lv[it.lv].h;
  const int64_t k_lo = a.table.causal ? 2 * it.seg * h : 0;
  return (int64_t(it.lv) * a.heads + it.head) * a.S + it.seg * h + (krow - k_lo);
}

// dK (scaled) and dV of a bucket key: adds the key's sample-slot partials
// (the slots on its list, first = slot_first of its slot, loaded by the
// caller ahead of the tile loop) and stores the level partials (causal) or
// the final rows. One walk of the list serves both gradients; each adds its
// rows in list order.
template <int D>
__device__ __forceinline__ void finish_bucket_keys16(const BwdArgs& a, const BucketItem& it,
                                                     Acc16<D>& dk, Acc16<D>& dv, int64_t krow,
                                                     int first) {
  const Level& L = a.table.lv[it.lv];
  scale16<D>(dk, a.scale);
  const int64_t kslot = bucket_kslot(a, it, krow);
  const int64_t nqc = L.smp_nqc;
  const int64_t item0 = L.smp_wg0 + (int64_t(it.head) * L.nseg + it.seg) * L.smp_nsc * nqc;
  for (int t = first; t >= 0; t = a.slot_next[it.rec * 2 * a.m + t]) {
    const int64_t sc = t / kAttnQ;
    const int tt = t - int(sc) * kAttnQ;
    for (int64_t qc = 0; qc < nqc; ++qc) {
      const int64_t row = ((item0 + sc * nqc + qc) * kAttnQ + tt) * D;
      add_row16<D>(dk, a.slot_dk + row);
      add_row16<D>(dv, a.slot_dv + row);
    }
  }
  if (a.table.causal) {
    store_row16_bf16<D>(dv, a.part_dv + kslot * D);
    store_row16_bf16<D>(dk, a.part_dk + kslot * D);
  } else {
    store_row16_bf16<D>(dv, a.dV + (int64_t(it.head) * a.n + krow) * D);
    store_row16_bf16<D>(dk, a.dK + (int64_t(it.head) * a.n + krow) * D);
  }
}

// dK, dV of one bucket item's 256 key slots (two halves of 128, one after the
// other) against the bucket's queries. When the bucket has at most 2 KT
// queries both query tiles are loaded once and serve both halves; larger
// buckets stream the queries once per half.
template <int D>
__device__ __forceinline__ void kv16_bucket_item(const BwdArgs& a, BwdSmem<D>& sm, int64_t w) {
  const BucketItem it = decode_bucket(a, w);
  const int b_eff = a.table.lv[it.lv].b_eff;
  const int wave = threadIdx.x >> 6;
  const auto Kr = rsrc_of(a.K, it.head, a.n, D);
  const auto Vr = rsrc_of(a.V, it.head, a.n, D);
  const int64_t kbase = it.chunk * kAttnQ + wave * kKW16 + (lane_id() & 15);
  if (b_eff > 2 * KT) {
    for (int half = 0; half < 2; ++half) {
      const int64_t ki = kbase + half * kKeys16;
      const int64_t krow = ki < b_eff ? int64_t(a.perm_k[it.slot0 + ki]) : -1;
      const int first = krow >= 0 ? a.slot_first[bucket_kslot(a, it, krow)] : -1;
      Frag16<D> kf, vf;
      load_frag16<D>(kf, Kr, krow);
      load_frag16<D>(vf, Vr, krow);
      Acc16<D> dk, dv;
      zero16<D>(dk);
      zero16<D>(dv);
      kv16_sorted_loop<D, false>(a, sm, a.perm_q, it.slot0, b_eff, b_eff, it.head, kf, vf, dk,
                                 dv, 1.f, 1.f, 0, true);
      if (krow >= 0) finish_bucket_keys16<D>(a, it, dk, dv, krow, first);
    }
    return;
  }
  // both query tiles resident
  const auto Qr = rsrc_of(a.Q, it.head, a.n, D);
  const auto dOr = rsrc_of(a.dO, it.head, a.n, D);
  const int ntiles = (b_eff + KT - 1) / KT;
  fill_queries(a, sm, a.perm_q, it.slot0, b_eff, it.head);
  __syncthreads();
  Pipe<bf16_t, D> pipe;
  for (int t = 0; t < ntiles; ++t) {
    BwdBuf<D>& b = sm.buf[t];
    const int e0 = t * KT;
    pipe.template issue<true>(b.t, Qr, dOr, true,
                              [&](int row) { return int(sm.srow[e0 + row]); },
                              [&](int row) { return sm.sw[e0 + row]; });
    if (threadIdx.x < KT) b.w2[threadIdx.x] = sm.sw2[e0 + threadIdx.x];
  }
  Offs16<D> o;
  o.init();
  // both halves' key rows and slot-list heads first, then each half's K and
  // V fragments one half ahead, so that no half waits on a dependent load
  int64_t krows[2];
  int firsts[2];
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int64_t ki = kbase + half * kKeys16;
    krows[half] = ki < b_eff ? int64_t(a.perm_k[it.slot0 + ki]) : -1;
  }
#pragma unroll
  for (int half = 0; half < 2; ++half)
    firsts[half] = krows[half] >= 0 ? a.slot_first[bucket_kslot(a, it, krows[half])] : -1;
  Frag16<D> kf, vf, kf1, vf1;
  load_frag16<D>(kf, Kr, krows[0]);
  load_frag16<D>(vf, Vr, krows[0]);
  pipe.commit(sm.buf[0].t, true);
  __syncthreads();
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (half == 0) {
      load_frag16<D>(kf1, Kr, krows[1]);
      load_frag16<D>(vf1, Vr, krows[1]);
    } else {
      kf = kf1;
      vf = vf1;
    }
    Acc16<D> dk, dv;
    zero16<D>(dk);
    zero16<D>(dv);
    for (int t = 0; t < ntiles; ++t) {
      const int left = b_eff - t * KT;
      kv_tile16<D, false, false, true>(sm.buf[t], o, kf, vf, dk, dv, a.scale_log2, 1.f, 1.f, 0,
                                       0, true, left < KT ? left : KT, 0, 0);
    }
    if (krows[half] >= 0) finish_bucket_keys16<D>(a, it, dk, dv, krows[half], firsts[half]);
  }
  __syncthreads();   // the tiles are read until here
}

template <int D>
__device__ __forceinline__ void kv16_sample_item(const BwdArgs& a, BwdSmem<D>& sm, int64_t w) {
  const int64_t w2 = w >> 1;
  int lv = 0;
  for (int l = 1; l < a.table.count; ++l)
    if (w2 >= a.table.lv[l].smp_wg0) lv = l;
  const Level& L = a.table.lv[lv];
  uint32_t rem = uint32_t(w2 - L.smp_wg0);
  const uint32_t nqc = uint32_t(L.smp_nqc), nsc = uint32_t(L.smp_nsc), nsg = uint32_t(L.nseg);
  uint32_t quo = rem / nqc;
  const int64_t qc = rem - quo * nqc;
  rem = quo;
  quo = rem / nsc;
  const int64_t sc = rem - quo * nsc;
  rem = quo;
  quo = rem / nsg;
  const int64_t seg = rem - quo * nsg;
  const int head = int(quo);
  const int64_t h = L.h;
  const int64_t rec = int64_t(head) * a.nodes + ((int64_t(1) << lv) + seg - 1);
  const int ucount = a.meta[rec * 4];
  const int vcount = a.meta[rec * 4 + 1];
  const int wave = threadIdx.x >> 6;
  const int64_t slot = (w & 1) * kKeys16 + wave * kKW16 + (lane_id() & 15);
  const int64_t t = sc * kAttnQ + slot;
  int64_t krow = -1;
  float om = 0.f, nu = 0.f;
  int bkt = -1;
  if (t < ucount) {
    krow = a.u_idx[rec * a.m + t];
    bkt = a.u_bkt[rec * a.m + t];
    nu = L.alpha;
  } else if (t - ucount < vcount) {
    krow = a.v_idx[rec * a.m + (t - ucount)];
    bkt = a.v_bkt[rec * a.m + (t - ucount)];
    om = a.v_w[rec * a.m + (t - ucount)];
  }
  Frag16<D> kf, vf;
  load_frag16<D>(kf, rsrc_of(a.K, head, a.n, D), krow);
  load_frag16<D>(vf, rsrc_of(a.V, head, a.n, D), krow);
  Acc16<D> dk, dv;
  zero16<D>(dk);
  zero16<D>(dv);
  const int64_t p0 = qc * kBwdQChunk;
  const int64_t count = h - p0 < kBwdQChunk ? h - p0 : kBwdQChunk;
  const int64_t seg0 = (int64_t(lv) * a.heads + head) * a.S + seg * h;
  // uniform slots have om = 0: no dV and no dP for a wave of them
  const bool wave_om = __ballot(om != 0.f) != 0;
  kv16_sorted_loop<D, true>(a, sm, a.perm_q + seg0, p0, count, L.b_eff, head, kf, vf, dk, dv, om,
                            nu, bkt, wave_om);
  if (krow < 0) return;
  scale16<D>(dk, a.scale);
  const int64_t idx = w2 * kAttnQ + slot;
  store_row16_f32<D>(dk, a.slot_dk + idx * D);
  store_row16_f32<D>(dv, a.slot_dv + idx * D);
}

// ------------------------------------------------------------------ kernels
// kPersistent: the work-group takes items from the queues until all are
// done; else it runs the one item of its (XCD-remapped) block index. The
// two are separate instantiations because the item loop changes register
// allocation (values hoisted out of it stay live across items).
template <int D, int MODE, bool kCausal, bool kPersistent>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_q_kernel(BwdArgs a) {
  __shared__ BwdSmem<D> sm;
  auto item_fn = [&](int64_t item) __attribute__((always_inline)) {
    if (MODE == BW_EXACT) q_exact_item<D, kCausal>(a, sm, uint32_t(item));
    else q_bucket_item<D>(a, sm, item);
  };
  if constexpr (kPersistent) {
    run_items(a, sm.item, [&](int64_t item) __attribute__((always_inline)) {
      item_fn(item);
      __syncthreads();
    });
  } else {
    item_fn(xcd_remap(int64_t(blockIdx.x), int64_t(gridDim.x)));
  }
}

template <int D, int MODE, bool kCausal, bool kPersistent>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_kv_kernel(BwdArgs a) {
  __shared__ BwdSmem<D> sm;
  auto item_fn = [&](int64_t item) __attribute__((always_inline)) {
    if constexpr (kKv16<D, MODE>) {
      if (MODE == BW_EXACT) kv16_exact_item<D, kCausal>(a, sm, uint32_t(item));
      else if (MODE == BW_BUCKET) kv16_bucket_item<D>(a, sm, item);
      else kv16_sample_item<D>(a, sm, item);
    } else {
      if (MODE == BW_EXACT) kv_exact_item<D, kCausal>(a, sm, uint32_t(item));
      else if (MODE == BW_BUCKET) kv_bucket_item<D>(a, sm, item);
      else kv_sample_item<D>(a, sm, item);
    }
  };
  if constexpr (kPersistent) {
    run_items(a, sm.item, [&](int64_t item) __attribute__((always_inline)) {
      item_fn(item);
      __syncthreads();
    });
  } else {
    item_fn(xcd_remap(int64_t(blockIdx.x), int64_t(gridDim.x)));
  }
}

// delta[row] = O[row] . dO[row]: CPR lanes per row, 16 bytes each.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(const bf16_t* O, const bf16_t* dO,
                                                    float* delta, int64_t rows) {
  constexpr int CPR = D / 8;
  const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid / CPR;
  const int ch = int(gid % CPR);
  float acc = 0.f;
  if (row < rows) {
    float o[8], g[8];
    load8<bf16_t>(O + row * D + ch * 8, o);
    load8<bf16_t>(dO + row * D + ch * 8, g);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(o[j], g[j], acc);
  }
#pragma unroll
  for (int o = CPR / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (row < rows && ch == 0) delta[row] = acc;
}

// Per node (grid: nodes x heads): slot_first[key row of the node] = least
// sample slot on that row (-1: none), slot_next[t] = next slot on t's row.
// Slots: the uniform list (t < ucount) then the V-norm list.
constexpr int kLinkThreads = 512;
__global__ __launch_bounds__(kLinkThreads) void links_kernel(BwdArgs a) {
  __shared__ int32_t rows[2 * kBwdMaxM];
  const int64_t node = int64_t(blockIdx.x) + 1;
  const int head = blockIdx.y;
  const int lv = 63 - __clzll(node);
  const int64_t seg = node - (int64_t(1) << lv);
  const Level& L = a.table.lv[lv];
  const int64_t h = L.h;
  const int64_t k_lo = a.table.causal ? 2 * seg * h : 0;
  int32_t* first = const_cast<int32_t*>(a.slot_first) + (int64_t(lv) * a.heads + head) * a.S +
                   seg * h;
  const int64_t rec = int64_t(head) * a.nodes + (node - 1);
  int32_t* next = const_cast<int32_t*>(a.slot_next) + rec * 2 * a.m;
  const int ucount = a.meta[rec * 4];
  const int vcount = a.meta[rec * 4 + 1];
  const int T = ucount + vcount;
  for (int64_t k = threadIdx.x; k < h; k += kLinkThreads) first[k] = -1;
  for (int t = threadIdx.x; t < T; t += kLinkThreads)
    rows[t] = t < ucount ? a.u_idx[rec * a.m + t] : a.v_idx[rec * a.m + (t - ucount)];
  __syncthreads();
  for (int t = threadIdx.x; t < T; t += kLinkThreads) {
    const int32_t r = rows[t];
    int nx = -1;
    bool lead = true;
    for (int u = 0; u < T; ++u) {
      if (rows[u] != r) continue;
      if (u < t) lead = false;
      else if (u > t && nx < 0) nx = u;
    }
    next[t] = nx;
    if (lead) first[r - k_lo] = t;
  }
}

BwdArgs base_args(const BwdIO& io, int64_t n, int d, int heads) {
  BwdArgs a{};
  a.Q = static_cast<const bf16_t*>(io.Q);
  a.K = static_cast<const bf16_t*>(io.K);
  a.V = static_cast<const bf16_t*>(io.V);
  a.dO = static_cast<const bf16_t*>(io.dO);
  a.lse = io.lse;
  a.delta = io.delta;
  a.dQ = static_cast<bf16_t*>(io.dQ);
  a.dK = static_cast<bf16_t*>(io.dK);
  a.dV = static_cast<bf16_t*>(io.dV);
  a.n = n;
  a.heads = heads;
  a.scale_log2 = float(1.4426950408889634 / std::sqrt(double(d)));
  a.scale = float(1.0 / std::sqrt(double(d)));
  return a;
}

void plan_args(BwdArgs& a, const Plan& p, void* ws) {
  char* w = static_cast<char*>(ws);
  a.table = p.table;
  a.m = p.m;
  a.nodes = p.nodes;
  a.S = p.S;
  a.perm_q = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_PERM_Q]);
  a.perm_k = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_PERM_K]);
  a.u_idx = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_U_IDX]);
  a.u_bkt = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_U_BKT]);
  a.v_idx = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_V_IDX]);
  a.v_bkt = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_V_BKT]);
  a.v_w = reinterpret_cast<const float*>(w + p.off[HA_WS_V_W]);
  a.meta = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_NODE_META]);
  a.slot_first = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_SLOT_FIRST]);
  a.slot_next = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_SLOT_NEXT]);
  a.slot_dk = reinterpret_cast<float*>(w + p.off[HA_WS_SLOT_DK]);
  a.slot_dv = reinterpret_cast<float*>(w + p.off[HA_WS_SLOT_DV]);
  a.queue = reinterpret_cast<uint32_t*>(w + p.off[HA_WS_SCHED]);
  if (p.causal && p.L > 0) {
    a.part_dq = reinterpret_cast<bf16_t*>(w + p.off[HA_WS_PART_DQ]);
    a.part_dk = reinterpret_cast<bf16_t*>(w + p.off[HA_WS_PART_DK]);
    a.part_dv = reinterpret_cast<bf16_t*>(w + p.off[HA_WS_PART_DV]);
  }
}

// A launch of kernel k over `items` work items. persistent: one work-group
// per resident slot (at most one per item) taking items from the queues,
// whose counters are zeroed first; else one work-group per item in the
// dispatcher's order. Measured on the long-context causal workload, the
// queues help the sample-slot and base-case dQ launches (whose items differ
// in length) and slow the others, so each launch chooses.
template <typename Kern>
int launch_items(Kern k, BwdArgs a, int64_t items, bool persistent, const char* name,
                 hipStream_t s) {
  if (items == 0) return HA_OK;
  if (items >= (int64_t(1) << 31))
    return fail(HA_ERR_SHAPE, "%lld work items of %s exceed the launch limit", (long long)items,
                name);
  a.items = uint32_t(items);
  unsigned grid = a.items;
  if (persistent) {
    const int r = resident_groups(k);
    if (r <= 0) return fail(HA_ERR_HIP, "could not query the device's occupancy");
    if (int rc = reset_queue(a.queue, s)) return rc;
    grid = unsigned(r) < a.items ? unsigned(r) : a.items;
  } else {
    a.queue = nullptr;
  }
  ProfRange pr(name, s);
  pr.groups = grid;
  hipLaunchKernelGGL(k, dim3(grid), dim3(kThreads), 0, s, a);
  HA_LAUNCH_CHECK(name);
  return HA_OK;
}

}  // namespace

int launch_delta(const void* O, const void* dO, float* delta, int64_t rows, int d,
                 hipStream_t s) {
  if (rows == 0) return HA_OK;
  const int64_t threads = rows * (d / 8);
  const int64_t blocks = ceil_div(threads, 256);
  if (blocks >= (int64_t(1) << 31)) return fail(HA_ERR_SHAPE, "too many rows for delta");
  ProfRange pr("bwd_delta", s);
  auto k = d == 128 ? delta_kernel<128> : delta_kernel<64>;
  hipLaunchKernelGGL(k, dim3(unsigned(blocks)), dim3(256), 0, s, static_cast<const bf16_t*>(O),
                     static_cast<const bf16_t*>(dO), delta, rows);
  HA_LAUNCH_CHECK("bwd_delta");
  return HA_OK;
}

int launch_bwd_links(const Plan& p, void* ws, hipStream_t s) {
  if (p.nodes == 0 || p.heads == 0) return HA_OK;
  BwdArgs a{};
  a.heads = p.heads;
  a.n = p.n;
  plan_args(a, p, ws);
  ProfRange pr("bwd_links", s);
  hipLaunchKernelGGL(links_kernel, dim3(unsigned(p.nodes), unsigned(p.heads)),
                     dim3(kLinkThreads), 0, s, a);
  HA_LAUNCH_CHECK("bwd_links");
  return HA_OK;
}

int launch_bwd_samples(const Plan& p, const BwdIO& io, void* ws, hipStream_t s) {
  BwdArgs a = base_args(io, p.n, p.d, p.heads);
  plan_args(a, p, ws);
  auto k = p.d == 128 ? bwd_kv_kernel<128, BW_SAMPLE, false, true> : bwd_kv_kernel<64, BW_SAMPLE, false, true>;
  return launch_items(k, a, p.d == 128 ? 2 * p.smp_wgs : p.smp_wgs, true, "bwd_sample_kv", s);
}

int launch_bwd_bucket(const Plan& p, const BwdIO& io, void* ws, hipStream_t s) {
  BwdArgs a = base_args(io, p.n, p.d, p.heads);
  plan_args(a, p, ws);
  auto kq = p.d == 128 ? bwd_q_kernel<128, BW_BUCKET, false, false> : bwd_q_kernel<64, BW_BUCKET, false, false>;
  if (int rc = launch_items(kq, a, p.att_wgs, false, "bwd_bucket_q", s)) return rc;
  auto kkv =
      p.d == 128 ? bwd_kv_kernel<128, BW_BUCKET, false, false>
                 : bwd_kv_kernel<64, BW_BUCKET, false, false>;
  return launch_items(kkv, a, p.att_wgs, false, "bwd_bucket_kv", s);
}

int launch_bwd_exact(const BwdIO& io, int64_t n, int d, int heads, int causal, int64_t block,
                     const Plan* merge, const void* ws, uint32_t* queue, hipStream_t s) {
  BwdArgs a = base_args(io, n, d, heads);
  a.block = block;
  a.queue = queue;
  const int64_t tpb = ceil_div(block, kAttnQ);
  const int64_t per_head = ceil_div(n, block) * tpb;
  const int64_t items = per_head * heads;
  if (items >= (int64_t(1) << 31))
    return fail(HA_ERR_SHAPE, "%lld tiles exceed the launch limit", (long long)items);
  a.tiles_per_block = uint32_t(tpb);
  a.items_per_head = uint32_t(per_head);
  if (merge && merge->L > 0) {
    if ((block << merge->L) != n)
      return fail(HA_ERR_SHAPE, "base block %lld times 2^%d differs from n = %lld",
                  (long long)block, merge->L, (long long)n);
    const char* w = static_cast<const char*>(ws);
    a.merge_levels = merge->L;
    a.S = merge->S;
    a.part_dq = reinterpret_cast<bf16_t*>(const_cast<char*>(w) + merge->off[HA_WS_PART_DQ]);
    a.part_dk = reinterpret_cast<bf16_t*>(const_cast<char*>(w) + merge->off[HA_WS_PART_DK]);
    a.part_dv = reinterpret_cast<bf16_t*>(const_cast<char*>(w) + merge->off[HA_WS_PART_DV]);
  }
  const char* nq = merge ? "bwd_base_q" : "bwd_exact_q";
  const char* nkv = merge ? "bwd_base_kv" : "bwd_exact_kv";
  int rc;
  if (d == 128) {
    rc = launch_items(causal ? bwd_q_kernel<128, BW_EXACT, true, true> : bwd_q_kernel<128, BW_EXACT, false, true>,
                      a, items, true, nq, s);
    // the key-major items are tiles of 128 keys (16 per wave)
    BwdArgs akv = a;
    const int64_t tpb_kv = ceil_div(block, kKeys16);
    // causal items are pairs of key tiles (kv16_exact_item)
    const int64_t per_head_kv = ceil_div(n, block) * (causal ? (tpb_kv + 1) / 2 : tpb_kv);
    akv.tiles_per_block = uint32_t(tpb_kv);
    akv.items_per_head = uint32_t(per_head_kv);
    if (!rc && per_head_kv * heads >= (int64_t(1) << 31))
      rc = fail(HA_ERR_SHAPE, "%lld key tiles exceed the launch limit",
                (long long)(per_head_kv * heads));
    if (!rc)
      rc = launch_items(causal ? bwd_kv_kernel<128, BW_EXACT, true, false>
                               : bwd_kv_kernel<128, BW_EXACT, false, false>,
                        akv, per_head_kv * heads, false, nkv, s);
  } else {
    rc = launch_items(causal ? bwd_q_kernel<64, BW_EXACT, true, true> : bwd_q_kernel<64, BW_EXACT, false, true>,
                      a, items, true, nq, s);
    if (!rc)
      rc = launch_items(causal ? bwd_kv_kernel<64, BW_EXACT, true, false>
                               : bwd_kv_kernel<64, BW_EXACT, false, false>,
                        a, items, false, nkv, s);
  }
  return rc;
}

}  // namespace ha
