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
// Layout: a work-group of 8 waves owns 256 query rows, 32 per wave. Each
// wave computes S^T = K Q^T for a key tile with v_mfma_f32_32x32x16_bf16
// (A = K rows from LDS, B = the wave's Q rows held in registers), so every
// lane owns one query column of S^T and the softmax statistics of that query
// need only one cross-lane exchange (lane l with lane l^32, a permlane swap).
// The probabilities then feed O^T += V^T P^T directly as the B operand (same
// lane layout).
//
// bf16 tiles: K and V rows go from HBM straight into LDS (buffer loads with
// the LDS destination, 16 bytes per lane, no register staging), unpadded with
// the 16-byte chunks of each row XOR-swizzled by the row index so that the
// fragment reads of 16 consecutive rows hit distinct banks. V's A operand is
// read with gfx950's transposing LDS read (ds_read_b64_tr_b16): within each
// 16-lane group, lane i receives element i%4 of what lane 4j + i/4 addressed
// as its element j, so pointing lane L at V[key0 + L/4][d0 + 4(L%4)] hands
// lane i the four keys key0..key0+3 of column d0 + i. All per-lane LDS byte
// offsets are computed once per kernel.
// fp32 tiles (a correctness path): v_mfma_f32_32x32x2f32, K padded, V
// transposed through registers.
//
// Pipelining: key tiles are double-buffered in LDS; while a wave computes on
// tile t the loads of tile t+1 are in flight; one barrier per tile. The
// running maximum is only moved (and O, l rescaled) when a score exceeds it
// by more than 2^8, so most tiles skip the rescale. Work-group ids are
// remapped so that consecutive logical tiles (which share key blocks or
// sample lists) run on the same XCD and share its L2.
#include <cmath>
#include <type_traits>

#include "common.h"
#include "device_util.h"
#include "mfma_tile.h"

namespace ha {

namespace {

constexpr float kTau = 8.f;   // lazy-rescale threshold (log2 units)

enum { MODE_EXACT = 0, MODE_BUCKET = 1, MODE_ROWSUM = 2 };
enum { KIND_PLAIN = 0, KIND_SUM_W = 1, KIND_PV_W = 2 };

template <typename T, int D>
struct Smem {
  Buf<T, D> buf[2];
  float slse[kAttnQ];      // epilogue: lse of each staged row
  int64_t item;            // next work item (persistent launches)
};

template <typename T, int D>
struct SmemG {
  Buf<T, D> buf[2];
  alignas(16) int32_t srow[kSlotCap];
  alignas(16) float sw[kSlotCap];
  float slse[kAttnQ];      // epilogue: lse of each staged row
  int64_t sdst[kAttnQ];    // epilogue: destination row of each staged row (-1: none)
  int64_t item;            // next work item (persistent launches)
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
  int64_t tiles_per_block; // ceil(block / kAttnQ)
  uint32_t items_per_head; // work items per head (exact_item)
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
  // work queue of a persistent launch
  uint32_t* queue;         // [kQueues] counters, zero at launch; nullptr: one item per group
  uint32_t items;          // total work items
};

template <typename T, int D>
struct WaveState {
  f32x16 o[D / 32];
  float m;      // running reference maximum (log2 units; 0 until the row has one)
  float l;      // this lane's part of the row sum (its 16 keys per block)
  float thr;    // raw score that moves the reference: (m + kTau) / c; -inf before
                // the row's first reference, +inf for a lane without a row
};

// valid: the lane's query row exists (rows past the end never take a reference)
template <typename T, int D>
__device__ __forceinline__ void init_state(WaveState<T, D>& ws, bool valid) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db) ws.o[db] = zero16();
  ws.m = 0.f;
  ws.l = 0.f;
  ws.thr = valid ? -INFINITY : INFINITY;
}

// S^T for key block kb of the tile: s[i] = score of key 32kb + 8(i/4) + 4g + i%4
template <typename T, int D>
__device__ __forceinline__ f32x16 scores(const Buf<T, D>& b, const LaneOffs<T, D>& lo,
                                         const QFrag<T, D>& q, int kb) {
  f32x16 acc = zero16();
  if constexpr (sizeof(T) == 2) {
    const char* base = reinterpret_cast<const char*>(b.k) + kb * 32 * D * 2;
    // every fragment read is issued before the chain starts (the empty asm
    // keeps the compiler from sinking them between the MFMAs), so the chain
    // waits on LDS latency once instead of once per step
    // (d = 128 only: the d = 64 kernels run four waves per SIMD and have no
    // registers to spare, so they read each fragment just ahead of its MFMA)
    if constexpr (D == 128) {
      bf16x8_t kf[D / 16];
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        kf[st] = *reinterpret_cast<const bf16x8_t*>(base + lo.k[st]);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], q.v[st], acc, 0, 0, 0);
    } else {
      __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(base + lo.k[st]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q.v[st], acc, 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  } else {
    const int lane = lane_id();
    const float* krow = &b.k[(32 * kb + (lane & 31)) * Buf<T, D>::KS];
#pragma unroll
    for (int st = 0; st < D / 2; ++st)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[2 * st + (lane >> 5)], q.v[st], acc, 0,
                                                 0, 0);
  }
  return acc;
}

// O^T += V^T P^T for key block kb, p[i] the (weighted) probability of
// key_of(kb, i); bf16 tiles take it as the packed pb[i / 8][i % 8].
template <typename T, int D>
__device__ __forceinline__ void accumulate_pv(const Buf<T, D>& b, const LaneOffs<T, D>& lo,
                                              WaveState<T, D>& ws, const f32x16& p,
                                              const bf16x8_t* pb, int kb) {
  if constexpr (sizeof(T) == 2) {
    if constexpr (D == 128) {
      // all transposing reads of the block first, as for the score chain
      v4i16_t vx[2][D / 32][2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const char* base = reinterpret_cast<const char*>(b.v) + (32 * kb + 16 * st) * D * 2;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            vx[st][db][h] =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + lo.v[h][db]));
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t,
              __builtin_shufflevector(vx[st][db][0], vx[st][db][1], 0, 1, 2, 3, 4, 5, 6, 7));
          ws.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], ws.o[db], 0, 0, 0);
        }
      }
    } else {
      __builtin_amdgcn_s_setprio(kMfmaPrio);
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const char* base = reinterpret_cast<const char*>(b.v) + (32 * kb + 16 * st) * D * 2;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const v4i16_t x0 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + lo.v[0][db]));
          const v4i16_t x1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(base + lo.v[1][db]));
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
          ws.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[st], ws.o[db], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
  } else {
    const int lane = lane_id();
    const int ql = lane & 31, g = lane >> 5;
#pragma unroll
    for (int st = 0; st < 16; ++st) {
      const int key = key_of(kb, st, g);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const float a = b.v[(32 * db + ql) * Buf<T, D>::VS + key];
        ws.o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[st], ws.o[db], 0, 0, 0);
      }
    }
  }
}

// One LDS tile for this wave, processed as 32-key blocks, each with its own
// online-softmax step.
//   KIND_PLAIN: row sum and product, weight 1; KIND_SUM_W: row sum only,
//   weighted by b.w; KIND_PV_W: product only, weighted by b.w.
// masked: a key is valid iff its index in the tile is < nvalid and, if causal,
// at most lim (= query row - first key row of the tile).
template <typename T, int D, int KIND, bool kCausal>
__device__ __forceinline__ void compute_tile(const Buf<T, D>& b, const LaneOffs<T, D>& lo,
                                             const QFrag<T, D>& q, WaveState<T, D>& ws, float c,
                                             bool masked, int nvalid, int lim) {
  constexpr int NB = Buf<T, D>::KT / 32;
  constexpr bool kPack = sizeof(T) == 2 && KIND != KIND_SUM_W;   // bf16 P feeds the product
  const int g = lane_id() >> 5;
  const float inv_c = 1.f / c;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
    if (masked && 32 * kb >= nvalid) break;            // rest of the tile is empty
    f32x16 s = scores<T, D>(b, lo, q, kb);
    if (masked) {
      // key_of(kb, i, g) = 32kb + 4g + (8(i/4) + i%4): compare the immediate
      // part against per-lane limits
      const int vlim = nvalid - 32 * kb - 4 * g;
      const int clim = lim - 32 * kb - 4 * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 8 * (i >> 2) + (i & 3);
        bool ok = kk < vlim;
        if (kCausal) ok = ok && kk <= clim;
        s[i] = ok ? s[i] : -INFINITY;
      }
    }
    // The reference moves only when some lane's raw maximum passes its
    // threshold; then both halves of each row take the row maximum (one
    // permlane swap) and rescale if it exceeds the reference by kTau.
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int i = 2; i < 16; ++i) mx = fmaxf(mx, s[i]);
    if (__ballot(mx > ws.thr)) {
      mx = half_swap_max(mx) * c;
      const bool fresh = ws.thr == -INFINITY;
      if (fresh ? mx > -INFINITY : mx > ws.m + kTau) {
        const float f = fresh ? 1.f : fast_exp2(ws.m - mx);
        ws.l *= f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) ws.o[db][i] *= f;
        ws.m = mx;
        ws.thr = (mx + kTau) * inv_c;
      }
    }
    // (Weighted) probabilities in place, their bf16 pairs, and this lane's
    // block sum of what the row sum takes: the bf16 values that feed the
    // product (one dot2 per pair), else the fp32 ones.
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = fast_exp2(fmaf(s[i], c, -ws.m));
      if (KIND != KIND_PLAIN) s[i] *= b.w[key_of(kb, i, g)];
    }
    bf16x8_t pb[2];
    float a0 = 0.f, a1 = 0.f;
    if constexpr (kPack) {
      bf16x2_t one;
      one[0] = (__bf16)1.f;
      one[1] = (__bf16)1.f;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int j = 0; j < 8; ++j) pb[st][j] = (__bf16)s[8 * st + j];
        // (pairs by constant shuffles: element access on a bit_cast of the
        // vector came out wrong, every pair read as the first)
        const bf16x8_t v = pb[st];
        a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, a0, false);
        a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, a1, false);
        a0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, a0, false);
        a1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, a1, false);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i & 1) a1 += s[i];
        else a0 += s[i];
      }
    }
    const float bsum = a0 + a1;
    if (KIND != KIND_PV_W) ws.l += bsum;
    if (KIND != KIND_SUM_W) accumulate_pv<T, D>(b, lo, ws, s, pb, kb);
  }
}

// Normalised output of this lane's query; returns lse (natural log).
template <typename T, int D>
__device__ __forceinline__ float finalize(WaveState<T, D>& ws) {
  const float l = half_swap_sum(ws.l);
  const float inv = 1.f / l;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) ws.o[db][i] *= inv;
  return (ws.m + __log2f(l)) * 0.69314718055994531f;
}

// ------------------------------------------------------- epilogue staging
// After the tile loop the tile buffers are free; the epilogue stages the
// work-group's output rows there (in T, row-major, 16-byte chunks
// XOR-swizzled by row) and then reads and writes global memory a row at a
// time: 16 contiguous bytes per lane, four rows per instruction, instead of
// the MFMA layout's 8 or 16 bytes from each of 32 rows.
template <typename T, int D>
struct Stage {
  static constexpr int E = 16 / int(sizeof(T));          // elements per chunk
  static constexpr int CPR = D / E;                      // chunks per row
  static constexpr int RB = D * int(sizeof(T));          // bytes per row
  static constexpr int NCH = kAttnQ * CPR / kThreads;    // chunks per thread
  static_assert(kAttnQ * RB <= int(sizeof(Buf<T, D>)) * 2, "stage fits the tile buffers");
  static_assert(kAttnQ * CPR % kThreads == 0, "whole chunks per thread");
  __device__ static int off(int row, int ch) { return row * RB + ((ch ^ (row & (CPR - 1))) << 4); }
};

// This lane's part of its output row (accumulator layout: d = 32db + 8q4 +
// 4g + j) into staged row `row`.
template <typename T, int D>
__device__ __forceinline__ void stage_row(const WaveState<T, D>& ws, char* st, int row) {
  using S = Stage<T, D>;
  const int g = lane_id() >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d0 = 32 * db + 8 * q4 + 4 * g;
      if constexpr (sizeof(T) == 2) {
        const uint32_t lo = uint32_t(f32_to_bf16(ws.o[db][4 * q4])) |
                            (uint32_t(f32_to_bf16(ws.o[db][4 * q4 + 1])) << 16);
        const uint32_t hi = uint32_t(f32_to_bf16(ws.o[db][4 * q4 + 2])) |
                            (uint32_t(f32_to_bf16(ws.o[db][4 * q4 + 3])) << 16);
        *reinterpret_cast<uint2*>(st + S::off(row, d0 >> 3) + (d0 & 7) * 2) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<float4*>(st + S::off(row, d0 >> 2)) =
            make_float4(ws.o[db][4 * q4], ws.o[db][4 * q4 + 1], ws.o[db][4 * q4 + 2],
                        ws.o[db][4 * q4 + 3]);
      }
    }
}

// ------------------------------------------------------------- EXACT kernel
// Query tile `tile` of key block blk; desc: its key tiles in descending order.
template <typename T, int D, bool kCausal>
__device__ __forceinline__ void exact_tile(const AttnArgs& a, Smem<T, D>& sm, int head,
                                           uint32_t blk, int64_t tile, bool desc) {
  constexpr int KT = Buf<T, D>::KT;
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
  const int64_t hbytes = a.n * D * int64_t(sizeof(T));
  const auto Qr = head_rsrc(static_cast<const T*>(a.Q) + hoff, hbytes);
  const auto Kr = head_rsrc(static_cast<const T*>(a.K) + hoff, hbytes);
  const auto Vr = head_rsrc(static_cast<const T*>(a.V) + hoff, hbytes);
  QFrag<T, D> q;
  load_q<T, D>(q, Qr, qrow);
  LaneOffs<T, D> lo;
  lo.init();
  WaveState<T, D> ws;
  init_state<T, D>(ws, qrow >= 0);

  const int64_t k_end = kCausal ? q_end : b_hi;
  const int ntiles = int((k_end - b_lo + KT - 1) / KT);
  Pipe<T, D> pipe;
  // step t of the loop takes key tile kt(t); its buffer is t & 1
  auto kt = [&](int t) { return desc ? ntiles - 1 - t : t; };
  auto issue = [&](int t) {
    const int64_t k0 = b_lo + int64_t(kt(t)) * KT;
    const int nv = int(k_end - k0 < KT ? k_end - k0 : KT);
    pipe.issue(sm.buf[t & 1], Kr, Vr, true,
               [&](int row) { return row < nv ? int(k0 + row) : -1; },
               [](int) { return 1.f; });
  };
  issue(0);
  pipe.commit(sm.buf[0], true);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) issue(t + 1);
    const int64_t k0 = b_lo + int64_t(kt(t)) * KT;
    const int nvalid = int(k_end - k0 < KT ? k_end - k0 : KT);
    const bool skip = kCausal && k0 > qw0 + kQW - 1;       // wholly above the diagonal
    if (!skip) {
      const bool masked = nvalid < KT || (kCausal && k0 + KT - 1 > qw0);
      const int64_t dl = qrow - k0;
      const int lim = dl < 0 ? -1 : (dl > KT ? KT : int(dl));
      compute_tile<T, D, KIND_PLAIN, kCausal>(sm.buf[t & 1], lo, q, ws, a.scale_log2, masked,
                                              nvalid, lim);
    }
    if (t + 1 < ntiles) pipe.commit(sm.buf[(t + 1) & 1], true);
    __syncthreads();
  }
  const float lse = finalize<T, D>(ws);
  // stage the rows, then merge and store them a row at a time
  using S = Stage<T, D>;
  char* st = reinterpret_cast<char*>(&sm.buf[0]);
  stage_row<T, D>(ws, st, wave * kQW + ql);
  if ((lane_id() >> 5) == 0) sm.slse[wave * kQW + ql] = lse;
  __syncthreads();
  const int nrows = int(q_end - q0);
  const int tid = opaque_tid();
  float acc[S::NCH][S::E], l[S::NCH];
#pragma unroll
  for (int k = 0; k < S::NCH; ++k) {
    const int c = tid + k * kThreads;
    const int row = c / S::CPR, ch = c % S::CPR;
    unpack16<T>(*reinterpret_cast<const uint4*>(st + S::off(row, ch)), acc[k]);
    l[k] = sm.slse[row];
  }
  if (a.merge_levels > 0) {
    // The base block blk lies in the second half of its level-lv node (and
    // so has a partial there) iff bit L-1-lv of blk is set; the node's half
    // size is block << (L-1-lv). The partial of row b_lo + r sits at slot
    // (blk >> (L-lv)) * hl + (blk mod 2^(L-1-lv)) * block + r, so a tile's
    // partials are contiguous.
    const int L = a.merge_levels;
    for (int lv = 0; lv < L; ++lv) {
      const int sh = L - 1 - lv;
      if (((blk >> sh) & 1u) == 0) continue;
      const int64_t hl = a.block << sh;
      const int64_t slot0 = int64_t(blk >> (sh + 1)) * hl +
                            int64_t(blk & ((1u << sh) - 1u)) * a.block + (q0 - b_lo);
      const int64_t idx0 = (int64_t(lv) * a.heads + head) * a.S + slot0;
      const T* po = static_cast<const T*>(a.part_o) + idx0 * D;
      const float* pls = a.part_lse + idx0;
      uint4 raw[S::NCH];
      float pl[S::NCH];
#pragma unroll
      for (int k = 0; k < S::NCH; ++k) {
        const int c = tid + k * kThreads;
        const int row = c / S::CPR, ch = c % S::CPR;
        raw[k] = make_uint4(0, 0, 0, 0);
        pl[k] = -INFINITY;
        if (row < nrows) {
          raw[k] = *reinterpret_cast<const uint4*>(po + int64_t(row) * D + ch * S::E);
          pl[k] = pls[row];
        }
      }
#pragma unroll
      for (int k = 0; k < S::NCH; ++k) {
        float v[S::E];
        unpack16<T>(raw[k], v);
        const float mx = fmaxf(l[k], pl[k]);
        const float wa = __expf(l[k] - mx);
        const float wb = __expf(pl[k] - mx);
        const float inv = 1.f / (wa + wb);
#pragma unroll
        for (int j = 0; j < S::E; ++j) acc[k][j] = (acc[k][j] * wa + v[j] * wb) * inv;
        l[k] = mx + __logf(wa + wb);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < S::NCH; ++k) {
    const int c = tid + k * kThreads;
    const int row = c / S::CPR, ch = c % S::CPR;
    if (row >= nrows) continue;
    const int64_t grow = q0 + row;
    *reinterpret_cast<uint4*>(static_cast<T*>(a.O) + hoff + grow * D + ch * S::E) =
        pack16<T>(acc[k]);
    if (ch == 0 && a.lse) a.lse[int64_t(head) * a.n + grow] = l[k];
  }
}

// Work item lin = head * items_per_head + blk * per_block + j. Non-causal:
// query tile j of key block blk (per_block = tiles_per_block). Causal: the
// pair of query tiles j and tiles_per_block - 1 - j (per_block =
// ceil(tiles_per_block / 2)), so every item of a block sees the same number
// of key tiles; the first takes its key tiles in ascending order, the second
// in descending order. At any moment the items of one block that started
// together then read only two of the block's key tiles (tile tau of the
// first sweeps, tile 2 tiles_per_block + 1 - tau of the second), and the
// XCD's L2 serves the rest of them.
template <typename T, int D, bool kCausal>
__device__ __forceinline__ void exact_item(const AttnArgs& a, Smem<T, D>& sm, uint32_t lin) {
  // 32-bit division: far cheaper than 64-bit, and the counts fit
  const uint32_t gx = a.items_per_head;
  const int head = int(lin / gx);
  const uint32_t bx = lin - uint32_t(head) * gx;
  const uint32_t tpb = uint32_t(a.tiles_per_block);
  if constexpr (kCausal) {
    const uint32_t ppb = (tpb + 1) / 2;
    const uint32_t blk = bx / ppb;
    const uint32_t j = bx - blk * ppb;
    exact_tile<T, D, kCausal>(a, sm, head, blk, int64_t(j), false);
    if (tpb - 1 - j != j) {
      __syncthreads();   // the first tile's epilogue reads the buffers the second loads into
      exact_tile<T, D, kCausal>(a, sm, head, blk, int64_t(tpb - 1 - j), true);
    }
  } else {
    const uint32_t blk = bx / tpb;
    exact_tile<T, D, kCausal>(a, sm, head, blk, int64_t(bx - blk * tpb), false);
  }
}

template <typename T, int D, bool kCausal>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WavesPerEu<T, D>::value)))
void exact_kernel(AttnArgs a) {
  __shared__ Smem<T, D> sm;
  run_items(a, sm.item, [&](int64_t item) __attribute__((always_inline)) {
    exact_item<T, D, kCausal>(a, sm, uint32_t(item));
  });
}

// ------------------------------------------------------ BUCKET / ROWSUM kernel
// Work item w (ordered by level, head, segment, bucket, query chunk): one
// query chunk of one sortLSH bucket. Its key tiles form one sequence: the
// bucket's own keys, then the uniform sample, then (BUCKET) the V-norm
// sample, each segment padded to whole tiles. The rows and weights of up to
// kSlotCap slots (a window of tiles) are staged in LDS up front, so the tile
// loop issues no dependent index loads.
template <typename T, int D, int MODE>
__device__ __forceinline__ void bucket_item(const AttnArgs& a, SmemG<T, D>& sm, int64_t w) {
  constexpr int KT = Buf<T, D>::KT;
  constexpr int kWin = kSlotCap / KT;           // tiles per slot window
  constexpr bool kProduct = MODE == MODE_BUCKET;
  int lv = 0;
  for (int l = 1; l < a.table.count; ++l)
    if (w >= a.table.lv[l].att_wg0) lv = l;
  const Level& L = a.table.lv[lv];
  // 32-bit division: far cheaper than 64-bit, and the counts fit
  uint32_t rem = uint32_t(w - L.att_wg0);
  const uint32_t nq = uint32_t(L.att_qch), nbk = uint32_t(L.nbucket), nsg = uint32_t(L.nseg);
  uint32_t quo = rem / nq;
  const int64_t qc = rem - quo * nq;
  rem = quo;
  quo = rem / nbk;
  const int64_t bucket = rem - quo * nbk;
  rem = quo;
  quo = rem / nsg;
  const int64_t seg = rem - quo * nsg;
  const int head = int(quo);
  const int b_eff = L.b_eff;
  const int64_t h = L.h;
  const int64_t slot0 = (int64_t(lv) * a.heads + head) * a.S + seg * h + bucket * b_eff;
  const int wave = threadIdx.x >> 6;
  const int ql = lane_id() & 31;
  const int64_t qi = qc * kAttnQ + wave * kQW + ql;
  const int64_t qrow = qi < b_eff ? int64_t(a.perm_q[slot0 + qi]) : -1;

  const int64_t node = (int64_t(1) << lv) + seg;
  const int64_t rec = int64_t(head) * a.nodes + (node - 1);
  // List lengths and the uniform weight are fixed per level, so the slot
  // loads below need not wait for the node record; only an empty V-norm list
  // (all of the node's V rows zero) is read from it, after they are issued.
  const int ucount = L.u_cnt;
  const int vcap = kProduct ? L.v_cap : 0;
  const float alpha = L.alpha;

  const int64_t hoff = int64_t(head) * a.n * D;
  const int64_t hbytes = a.n * D * int64_t(sizeof(T));
  const auto Qr = head_rsrc(static_cast<const T*>(a.Q) + hoff, hbytes);
  const auto Kr = head_rsrc(static_cast<const T*>(a.K) + hoff, hbytes);
  const auto Vr = head_rsrc(kProduct ? static_cast<const T*>(a.V) + hoff
                                     : static_cast<const T*>(a.K) + hoff, hbytes);
  QFrag<T, D> q;
  load_q<T, D>(q, Qr, qrow);
  LaneOffs<T, D> lo;
  lo.init();
  WaveState<T, D> ws;
  init_state<T, D>(ws, qrow >= 0);

  const int t_b = (b_eff + KT - 1) / KT;
  const int t_u = (ucount + KT - 1) / KT;
  const int t_vcap = (vcap + KT - 1) / KT;
  const int ntiles_cap = t_b + t_u + t_vcap;
  // segment of tile t (0 bucket, 1 uniform, 2 V-norm), its first slot, its size
  auto seg_of = [&](int t, int& j0, int& cnt) {
    if (t < t_b) { j0 = t * KT; cnt = b_eff; return 0; }
    if (t < t_b + t_u) { j0 = (t - t_b) * KT; cnt = ucount; return 1; }
    j0 = (t - t_b - t_u) * KT; cnt = vcap; return 2;
  };
  // stage slots of tiles [t0, t0 + kWin) in LDS; all of a thread's index
  // loads are issued before any of them is used
  auto fill = [&](int t0) {
    constexpr int NI = kSlotCap / kThreads;
    const int32_t* pk = a.perm_k + slot0;
    const int32_t* ui = a.u_idx + rec * a.m;
    const int32_t* ub = a.u_bkt + rec * a.m;
    const int32_t* vi = a.v_idx + rec * a.m;
    const int32_t* vb = a.v_bkt + rec * a.m;
    const float* vw = a.v_w + rec * a.m;
    int kind[NI], jj[NI];
    int32_t row[NI], bk[NI];
    float wv[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int e = int(threadIdx.x) + i * kThreads;
      const int t = t0 + e / KT;
      kind[i] = -1;
      jj[i] = 0;
      if (t < ntiles_cap) {
        int j0, cnt;
        const int sg = seg_of(t, j0, cnt);
        const int j = j0 + e % KT;
        if (j < cnt) {
          kind[i] = sg;
          jj[i] = j;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      row[i] = -1;
      bk[i] = int32_t(bucket);
      wv[i] = 1.f;
      if (kind[i] >= 0) row[i] = (kind[i] == 0 ? pk : kind[i] == 1 ? ui : vi)[jj[i]];
      if (kind[i] >= 1) bk[i] = (kind[i] == 1 ? ub : vb)[jj[i]];
      if (kind[i] == 2) wv[i] = vw[jj[i]];
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int e = int(threadIdx.x) + i * kThreads;
      float wt = 0.f;
      if (kind[i] == 0) wt = 1.f;
      else if (kind[i] >= 1 && bk[i] != bucket) wt = kind[i] == 1 ? alpha : wv[i];
      sm.srow[e] = row[i];
      sm.sw[e] = wt;
    }
  };
  auto needs_v = [&](int t) { return kProduct && (t < t_b || t >= t_b + t_u); };
  Pipe<T, D> pipe;
  auto issue = [&](int t) {
    const int e0 = (t % kWin) * KT;
    pipe.issue(sm.buf[t & 1], Kr, Vr, needs_v(t),
               [&](int row) { return int(sm.srow[e0 + row]); },
               [&](int slot) { return sm.sw[e0 + slot]; });
  };

  fill(0);
  const int ntiles = kProduct && a.meta[rec * 4 + 1] == 0 ? t_b + t_u : ntiles_cap;
  __syncthreads();
  issue(0);
  pipe.commit(sm.buf[0], needs_v(0));
  __syncthreads();
  // one loop per segment, each with its own weighting of the tiles
  auto step = [&](int t, auto kind) __attribute__((always_inline)) {
    constexpr int KIND = decltype(kind)::value;
    if (t + 1 < ntiles) {
      if ((t + 1) % kWin == 0) {      // next window of slots
        fill(t + 1);
        __syncthreads();
      }
      issue(t + 1);
    }
    int j0, cnt;
    seg_of(t, j0, cnt);
    const int nvalid = cnt - j0 < KT ? cnt - j0 : KT;
    compute_tile<T, D, KIND, false>(sm.buf[t & 1], lo, q, ws, a.scale_log2, nvalid < KT,
                                    nvalid, KT);
    if (t + 1 < ntiles) pipe.commit(sm.buf[(t + 1) & 1], needs_v(t + 1));
    __syncthreads();
  };
  using Plain = std::integral_constant<int, KIND_PLAIN>;
  using SumW = std::integral_constant<int, KIND_SUM_W>;
  using PvW = std::integral_constant<int, KIND_PV_W>;
  int t = 0;
  if (kProduct)
    for (; t < t_b; ++t) step(t, Plain{});
  else
    for (; t < t_b; ++t) step(t, SumW{});
  for (; t < t_b + t_u; ++t) step(t, SumW{});
  if (kProduct)
    for (; t < ntiles; ++t) step(t, PvW{});
  const float lse = finalize<T, D>(ws);
  // stage the rows with their destinations, then store them a row at a time
  using S = Stage<T, D>;
  char* st = reinterpret_cast<char*>(&sm.buf[0]);
  const int srow = wave * kQW + ql;
  if (MODE != MODE_ROWSUM) stage_row<T, D>(ws, st, srow);
  if ((lane_id() >> 5) == 0) {
    int64_t dst = -1;
    if (qrow >= 0) {
      if (MODE != MODE_ROWSUM && a.table.causal)
        // the sub-problem's queries are rows [2 seg h + h, 2 seg h + 2h) of
        // the head; their slot is seg h + (row - 2 seg h - h)
        dst = (int64_t(lv) * a.heads + head) * a.S + (qrow - (seg + 1) * h);
      else
        dst = int64_t(head) * a.n + qrow;
    }
    sm.slse[srow] = lse;
    sm.sdst[srow] = dst;
  }
  __syncthreads();
  const int tid = opaque_tid();
#pragma unroll
  for (int k = 0; k < S::NCH; ++k) {
    const int c = tid + k * kThreads;
    const int row = c / S::CPR, ch = c % S::CPR;
    const int64_t dst = sm.sdst[row];
    if (dst < 0) continue;
    if (MODE != MODE_ROWSUM)
      *reinterpret_cast<uint4*>(static_cast<T*>(a.O) + dst * D + ch * S::E) =
          *reinterpret_cast<const uint4*>(st + S::off(row, ch));
    if (ch == 0 && a.lse) a.lse[dst] = sm.slse[row];
  }
}

template <typename T, int D, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(WavesPerEu<T, D>::value)))
void bucket_kernel(AttnArgs a) {
  __shared__ SmemG<T, D> sm;
  run_items(a, sm.item, [&](int64_t item) __attribute__((always_inline)) {
    bucket_item<T, D, MODE>(a, sm, item);
  });
}

// Grid of a launch: every item when there is no queue (rows of `per_row`
// items), else the resident work-groups (at most one per item).
template <typename Kern>
int launch_grid(Kern k, const AttnArgs& a, unsigned per_row, dim3& grid) {
  if (!a.queue) {
    grid = dim3(per_row, a.items / per_row);
    return HA_OK;
  }
  const int r = resident_groups(k);
  if (r <= 0) return fail(HA_ERR_HIP, "could not query the device's occupancy");
  grid = dim3(unsigned(r) < a.items ? unsigned(r) : a.items);
  return HA_OK;
}

template <typename T, int D>
int launch_exact_t(const AttnArgs& a, hipStream_t s, ProfRange& pr) {
  auto k = a.causal ? exact_kernel<T, D, true> : exact_kernel<T, D, false>;
  dim3 grid;
  if (int rc = launch_grid(k, a, a.items_per_head, grid)) return rc;
  pr.groups = int64_t(grid.x) * grid.y;
  hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, a);
  return HA_OK;
}

template <typename T, int D>
int launch_bucket_t(const AttnArgs& a, bool product, hipStream_t s, ProfRange& pr) {
  auto k = product ? bucket_kernel<T, D, MODE_BUCKET> : bucket_kernel<T, D, MODE_ROWSUM>;
  dim3 grid;
  if (int rc = launch_grid(k, a, a.items, grid)) return rc;
  pr.groups = int64_t(grid.x) * grid.y;
  hipLaunchKernelGGL(k, grid, dim3(kThreads), 0, s, a);
  return HA_OK;
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
  // causal items are pairs of query tiles (exact_item)
  const int64_t per_block = causal ? (a.tiles_per_block + 1) / 2 : a.tiles_per_block;
  const int64_t items = ceil_div(n, block) * per_block * heads;
  if (items >= (int64_t(1) << 31))
    return fail(HA_ERR_SHAPE, "%lld query tiles exceed the launch limit", (long long)items);
  a.items_per_head = uint32_t(ceil_div(n, block) * per_block);
  a.items = uint32_t(items);
  if (merge && merge->L > 0) {
    // the merge epilogue locates partials by shifts of the base-block index
    if ((block << merge->L) != n)
      return fail(HA_ERR_SHAPE, "base block %lld times 2^%d differs from n = %lld",
                  (long long)block, merge->L, (long long)n);
    const char* w = static_cast<const char*>(ws);
    a.merge_levels = merge->L;
    a.part_o = w + merge->off[HA_WS_PART_O];
    a.part_lse = reinterpret_cast<const float*>(w + merge->off[HA_WS_PART_LSE]);
    a.S = merge->S;
    a.queue = reinterpret_cast<uint32_t*>(const_cast<char*>(w) + merge->off[HA_WS_SCHED]) +
              kQueues;
    if (int rc = reset_queue(a.queue, s)) return rc;
  }
  if (items == 0) return HA_OK;
  ProfRange pr(merge ? "exact_base_merge" : "exact_attention", s);
  int rc;
  if (dtype == HA_BF16)
    rc = d == 128 ? launch_exact_t<bf16_t, 128>(a, s, pr) : launch_exact_t<bf16_t, 64>(a, s, pr);
  else
    rc = d == 128 ? launch_exact_t<float, 128>(a, s, pr) : launch_exact_t<float, 64>(a, s, pr);
  if (rc) return rc;
  HA_LAUNCH_CHECK("exact_attention");
  return HA_OK;
}

int launch_bucket_attention(const Plan& p, const void* Q, const void* K, const void* V, void* O,
                            float* lse, void* ws, hipStream_t s) {
  if (p.att_wgs == 0) return HA_OK;
  if (p.att_wgs >= (int64_t(1) << 31))
    return fail(HA_ERR_SHAPE, "%lld bucket work items exceed the launch limit",
                (long long)p.att_wgs);
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
  a.items = uint32_t(p.att_wgs);
  a.queue = reinterpret_cast<uint32_t*>(w + p.off[HA_WS_SCHED]);
  if (int rc = reset_queue(a.queue, s)) return rc;
  ProfRange pr(p.product ? "bucket_attention" : "bucket_rowsum", s);
  int rc;
  if (p.dtype == HA_BF16)
    rc = p.d == 128 ? launch_bucket_t<bf16_t, 128>(a, p.product, s, pr)
                    : launch_bucket_t<bf16_t, 64>(a, p.product, s, pr);
  else
    rc = p.d == 128 ? launch_bucket_t<float, 128>(a, p.product, s, pr)
                    : launch_bucket_t<float, 64>(a, p.product, s, pr);
  if (rc) return rc;
  HA_LAUNCH_CHECK("bucket_attention");
  return HA_OK;
}

}  // namespace ha
