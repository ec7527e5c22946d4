// sortLSH ordering (HA page, "Algorithm", Algorithm 1: keys and queries are
// sorted by their Hamming-sorted hash and cut into equal-size buckets).
//
// Every (level, head, side, sub-problem) segment is sorted stably by
// (code, index) with a counting sort over the 2^r <= 256 code values. All
// segments of all levels are independent once the codes exist, so each of
// the two passes covers every segment in one launch:
//   1. per chunk of kSortChunk elements: a 256-bin histogram (LDS counters);
//   2. per chunk: its exclusive offsets (bin-major over the segment, then
//      chunk-minor), summed from the segment's chunk histograms by one thread
//      per bin; stable ranks (wave ballots find the earlier lanes with the
//      same code, per-wave LDS counts carry the order across batches and
//      waves); then perm (sorted position -> row) written in sorted order
//      from an LDS copy of the chunk, and rank (slot -> sorted position, keys
//      only).
// The chunks of one segment run on one XCD (chunk_of), so the short runs
// that neighbouring chunks write into each bin of perm meet in one L2.
#include "common.h"
#include "device_util.h"

namespace ha {

namespace {

constexpr int kThreads = 256;

struct SortArgs {
  LevelTable table;
  int heads;
  int sides;
  int64_t n;
  int64_t S;                    // slots per level per head
  const uint8_t* codes[2];      // [heads][n] per side
  int32_t* perm[2];             // [L][heads][S] per side
  int32_t* rank;                // [L][heads][S] for side 1, or null
  uint32_t* hist;               // [chunks][256]
};

struct ChunkRef {
  int lv, head, side;
  int64_t seg, chunk, h;
};

__device__ __forceinline__ int find_level(const LevelTable& t, int64_t w) {
  int lv = 0;
  for (int l = 1; l < t.count; ++l)
    if (w >= t.lv[l].sort_wg0) lv = l;
  return lv;
}

// Chunk processed by work-group x of a grid of n: work-groups are dealt to
// the 8 XCDs round-robin, so XCD j is given the j-th eighth of the chunks,
// in order, and a segment's chunks share one L2.
__device__ __forceinline__ int64_t chunk_of(int64_t x, int64_t n) {
  constexpr int64_t kXcd = 8;
  const int64_t per = n / kXcd, rem = n % kXcd;
  const int64_t xcd = x % kXcd, k = x / kXcd;
  // XCD j takes per (+1 for j < rem) consecutive chunks
  return xcd * per + (xcd < rem ? xcd : rem) + k;
}

// Work-group counts fit in 32 bits, and 32-bit division is far cheaper than
// 64-bit.
__device__ __forceinline__ ChunkRef decode_chunk(const SortArgs& a, int64_t w) {
  ChunkRef c;
  c.lv = find_level(a.table, w);
  const Level& L = a.table.lv[c.lv];
  uint32_t rem = uint32_t(w - L.sort_wg0);
  const uint32_t cps = uint32_t(L.sort_cps), nseg = uint32_t(L.nseg);
  const uint32_t sides = uint32_t(a.sides);
  uint32_t q = rem / cps;
  c.chunk = rem - q * cps;
  rem = q;
  q = rem / nseg;
  c.seg = rem - q * nseg;
  rem = q;
  q = rem / sides;
  c.side = int(rem - q * sides);
  c.head = int(q);
  c.h = L.h;
  return c;
}

// Global row of element t of a segment: queries sit in the second half of
// their block, keys in the first (non-causal: both cover [0, n)).
__device__ __forceinline__ int64_t seg_row(const SortArgs& a, int side, int64_t seg,
                                           int64_t h, int64_t t) {
  if (!a.table.causal) return t;
  return 2 * seg * h + (side == 0 ? h : 0) + t;
}

constexpr int kPer = kSortChunk / kThreads;      // elements per thread and chunk

__global__ __launch_bounds__(kThreads) void sort_hist_kernel(SortArgs a) {
  __shared__ uint32_t hist[kSortBins];
  // the scatter's chunk-to-XCD mapping: a chunk's histogram and codes are
  // in the L2 of the XCD that ranks it
  const int64_t w = chunk_of(blockIdx.x, gridDim.x);
  const ChunkRef c = decode_chunk(a, w);
  hist[threadIdx.x] = 0;
  const uint8_t* codes = a.codes[c.side] + int64_t(c.head) * a.n +
                         seg_row(a, c.side, c.seg, c.h, 0);
  const int64_t t0 = c.chunk * kSortChunk;
  const int64_t t1 = t0 + kSortChunk < c.h ? t0 + kSortChunk : c.h;
  // all of this thread's codes are loaded before any is counted
  uint32_t v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t t = t0 + i * kThreads + threadIdx.x;
    v[i] = t < t1 ? codes[t] : kSortBins;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (v[i] < kSortBins) atomicAdd(&hist[v[i]], 1u);
  __syncthreads();
  a.hist[w * kSortBins + threadIdx.x] = hist[threadIdx.x];
}

// Wave wv owns the chunk's elements [wv * kWaveSpan, (wv + 1) * kWaveSpan)
// (kPer batches of 64), so stable ranks need no barrier inside the wave: a
// batch's equal codes are found by ballots and the wave's running count per
// code lives in its own LDS row. Elements are then placed at their sorted
// position within the chunk in LDS and written out in that order, so lanes
// next to each other write runs of one bin's consecutive global positions.
constexpr int kWaves = kThreads / 64;
constexpr int kWaveSpan = kSortChunk / kWaves;

__global__ __launch_bounds__(kThreads) void sort_scatter_kernel(SortArgs a) {
  __shared__ uint32_t base[kSortBins];             // chunk's first global position per bin
  __shared__ uint32_t lstart[kSortBins];           // chunk's first local position per bin
  __shared__ uint32_t wcnt[kWaves][kSortBins];     // per-wave counts, then wave prefixes
  __shared__ uint32_t wtot[kWaves];
  __shared__ int32_t srow[kSortChunk];
  __shared__ uint32_t spos[kSortChunk];
  const int64_t w = chunk_of(blockIdx.x, gridDim.x);
  const ChunkRef c = decode_chunk(a, w);
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  {
    // This chunk's first position per bin: the lower bins over the whole
    // segment, plus this bin's count in the segment's earlier chunks (the
    // chunks of a segment are consecutive, the first at w - chunk).
    const int64_t cps = a.table.lv[c.lv].sort_cps;
    const uint32_t* __restrict__ h = a.hist + (w - c.chunk) * kSortBins + tid;
    uint32_t total = 0, before = 0;
#pragma unroll 8
    for (int64_t k = 0; k < cps; ++k) {
      const uint32_t v = h[k * kSortBins];
      total += v;
      before += k < c.chunk ? v : 0u;
    }
    const uint32_t incl = uint32_t(wave_incl_scan(uint64_t(total)));
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t below = 0;
    for (int i = 0; i < wave; ++i) below += wtot[i];
    base[tid] = below + incl - total + before;
  }
#pragma unroll
  for (int i = 0; i < kWaves; ++i) wcnt[i][tid] = 0;
  const uint8_t* codes = a.codes[c.side] + int64_t(c.head) * a.n;
  const int64_t slot0 = (int64_t(c.lv) * a.heads + c.head) * a.S + c.seg * c.h;
  int32_t* perm = a.perm[c.side] + slot0;
  int32_t* rank = (a.rank && c.side == 1) ? a.rank + slot0 : nullptr;
  const int64_t t0 = c.chunk * kSortChunk;
  const int64_t t1 = t0 + kSortChunk < c.h ? t0 + kSortChunk : c.h;
  const int64_t tw = t0 + wave * kWaveSpan;          // this wave's first element
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  // all of this thread's codes are loaded before any is ranked
  uint32_t cv[kPer];
#pragma unroll
  for (int b = 0; b < kPer; ++b) {
    const int64_t t = tw + b * 64 + lane;
    cv[b] = t < t1 ? codes[seg_row(a, c.side, c.seg, c.h, t)] : 0u;
  }
  __syncthreads();
  // rank within the wave: earlier batches (the wave's count row) plus the
  // earlier lanes of this batch with the same code
  uint32_t inw[kPer];
#pragma unroll
  for (int b = 0; b < kPer; ++b) {
    const bool valid = tw + b * 64 + lane < t1;
    const uint32_t code = cv[b];
    uint64_t eq = __ballot(valid);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const bool bit = (code >> k) & 1u;
      const uint64_t bk = __ballot(valid && bit);
      eq &= bit ? bk : ~bk;
    }
    const uint32_t local = __popcll(eq & lt_mask);
    const uint32_t before = valid ? wcnt[wave][code] : 0u;
    inw[b] = before + local;
    // every lane has read before the leader of each code writes (one wave,
    // LDS operations in program order)
    __builtin_amdgcn_wave_barrier();
    if (valid && local == 0) wcnt[wave][code] = before + uint32_t(__popcll(eq));
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  // per bin: prefixes over the waves, and the chunk's exclusive scan over bins
  {
    uint32_t run = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const uint32_t v = wcnt[i][tid];
      wcnt[i][tid] = run;
      run += v;
    }
    const uint32_t incl = uint32_t(wave_incl_scan(uint64_t(run)));
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int i = 0; i < wave; ++i) before += wtot[i];
    lstart[tid] = before + incl - run;
  }
  __syncthreads();
#pragma unroll
  for (int b = 0; b < kPer; ++b) {
    const int64_t t = tw + b * 64 + lane;
    if (t < t1) {
      const uint32_t code = cv[b];
      const uint32_t r = wcnt[wave][code] + inw[b];   // rank among the chunk's equal codes
      const uint32_t pos = base[code] + r;
      srow[lstart[code] + r] = int32_t(seg_row(a, c.side, c.seg, c.h, t));
      spos[lstart[code] + r] = pos;
      if (rank) rank[t] = int32_t(pos);
    }
  }
  __syncthreads();
  const int nv = int(t1 - t0);
  for (int j = tid; j < nv; j += kThreads) perm[spos[j]] = srow[j];
}

// Recompute the chunk offsets of the table for the given side count.
int64_t retable(LevelTable& t, int heads, int sides) {
  int64_t chunks = 0;
  for (int l = 0; l < t.count; ++l) {
    Level& v = t.lv[l];
    v.sort_wg0 = chunks;
    chunks += int64_t(heads) * sides * v.nseg * v.sort_cps;
  }
  return chunks;
}

int run_sort(SortArgs& a, int64_t chunks, hipStream_t s) {
  if (chunks == 0) return HA_OK;
  {
    ProfRange pr("sort_hist", s);
    hipLaunchKernelGGL(sort_hist_kernel, dim3(unsigned(chunks)), dim3(kThreads), 0, s, a);
    HA_LAUNCH_CHECK("sort_hist");
  }
  {
    ProfRange pr("sort_scatter", s);
    hipLaunchKernelGGL(sort_scatter_kernel, dim3(unsigned(chunks)), dim3(kThreads), 0, s, a);
    HA_LAUNCH_CHECK("sort_scatter");
  }
  return HA_OK;
}

}  // namespace

int launch_sort(const Plan& p, void* ws, int sides, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  SortArgs a;
  a.table = p.table;
  a.heads = p.heads;
  a.sides = sides;
  a.n = p.n;
  a.S = p.S;
  a.codes[0] = reinterpret_cast<const uint8_t*>(w + p.off[HA_WS_CODES_Q]);
  a.codes[1] = reinterpret_cast<const uint8_t*>(w + p.off[HA_WS_CODES_K]);
  a.perm[0] = reinterpret_cast<int32_t*>(w + p.off[HA_WS_PERM_Q]);
  a.perm[1] = reinterpret_cast<int32_t*>(w + p.off[HA_WS_PERM_K]);
  a.rank = reinterpret_cast<int32_t*>(w + p.off[HA_WS_RANK_K]);
  a.hist = reinterpret_cast<uint32_t*>(w + p.off[HA_WS_SORT_HIST]);
  return run_sort(a, retable(a.table, p.heads, sides), s);
}

size_t sort_single_scratch_bytes(int64_t n, int heads) {
  const int64_t chunks = int64_t(heads) * ceil_div(n, kSortChunk);
  return size_t(align256(chunks * kSortBins * 4));
}

int launch_sort_single(const uint8_t* codes, int64_t n, int heads, int32_t* perm,
                       void* scratch, hipStream_t s) {
  SortArgs a;
  a.table.count = 1;
  a.table.causal = 0;
  a.table.n = n;
  Level& v = a.table.lv[0];
  v.h = n;
  v.nseg = 1;
  v.b_eff = 1;
  v.nbucket = n;
  v.sort_cps = ceil_div(n, kSortChunk);
  v.att_wg0 = 0;
  v.att_qch = 0;
  a.heads = heads;
  a.sides = 1;
  a.n = n;
  a.S = n;
  a.codes[0] = a.codes[1] = codes;
  a.perm[0] = a.perm[1] = perm;
  a.rank = nullptr;
  a.hist = static_cast<uint32_t*>(scratch);
  return run_sort(a, retable(a.table, heads, 1), s);
}

}  // namespace ha
