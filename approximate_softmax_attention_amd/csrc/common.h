// Internal declarations shared by the library's translation units: the plan
// (sizes, recursion levels, workspace carve-up), element-type helpers, error
// reporting and the kernel launchers. Nothing here is part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/hyperattn.h"

namespace ha {

constexpr int kMaxLevels = 21;      // 20 halvings + 1
constexpr int kSortChunk = 4096;     // elements per sort work-group
constexpr int kSortBins = 256;       // codes are < 2^r <= 256

// ---------------------------------------------------------------- errors
void set_error(const char* fmt, ...);
int fail(int code, const char* fmt, ...);
#define HA_HIP_TRY(expr)                                                     \
  do {                                                                       \
    hipError_t e_ = (expr);                                                  \
    if (e_ != hipSuccess)                                                    \
      return ::ha::fail(HA_ERR_HIP, "%s failed: %s (%s:%d)", #expr,          \
                        hipGetErrorString(e_), __FILE__, __LINE__);          \
  } while (0)
#define HA_LAUNCH_CHECK(name)                                                \
  do {                                                                       \
    hipError_t e_ = hipGetLastError();                                       \
    if (e_ != hipSuccess)                                                    \
      return ::ha::fail(HA_ERR_HIP, "launch of %s failed: %s", name,         \
                        hipGetErrorString(e_));                              \
  } while (0)

// ------------------------------------------------------------- profiling
// Brackets one launch with events on its stream when profiling is enabled.
// `groups` (set by the launcher) is the launch's work-group count.
struct ProfRange {
  ProfRange(const char* name, hipStream_t s);
  ~ProfRange();
  int slot;
  hipStream_t stream;
  int64_t groups = 0;
};

// Work-groups of `threads` threads of the kernel `kernel` that the current
// device holds at once (occupancy query, cached per device and kernel); 0 if
// the query fails.
int resident_groups_of(const void* kernel, int threads);

// ------------------------------------------------------- level geometry
// One level of the flattened causal recursion (or the single non-causal
// sub-problem). Level l (0-based) has nseg sub-problems of size h: the
// queries of sub-problem s are rows [2sh + h, 2sh + 2h), its keys rows
// [2sh, 2sh + h) (non-causal: both [0, n)). The node id is 2^l + s.
struct Level {
  int64_t h;          // sub-problem size n_k
  int64_t nseg;       // sub-problems at this level
  int b_eff;          // bucket size min(b, h)
  int64_t nbucket;    // h / b_eff
  int64_t sort_cps;   // sort chunks per segment
  int64_t sort_wg0;   // first sort chunk work-group of this level
  int64_t att_wg0;    // first attention work-group of this level
  int64_t att_qch;    // query chunks per bucket
  // Sample lists of every sub-problem at this level: the uniform list holds
  // u_cnt = min(m, n_k) entries of weight alpha (n_k / m, or 1 when the list
  // is exhaustive); the V-norm list holds v_cap entries, or none when the
  // node's V rows are all zero (recorded per node by the sampler).
  int u_cnt;
  int v_cap;
  float alpha;
  // Backward pass: the gradient of the node's sample slots (uniform list
  // then V-norm list, u_cnt + v_cap slots) is computed by items of kAttnQ
  // slots times kBwdQChunk query positions.
  int smp_nsc;        // slot chunks per node
  int64_t smp_nqc;    // query chunks per node
  int64_t smp_wg0;    // first sample-slot item of this level
};

struct LevelTable {
  int count;
  int causal;
  int64_t n;
  Level lv[kMaxLevels];
};

struct Plan {
  int64_t n = 0;
  int d = 0, heads = 0, causal = 0, b = 0, m = 0, base = 0, r = 0, dtype = 0;
  int esize = 0;              // bytes per input element
  bool product = true;        // false for rowsum_estimate (no V)
  int L = 0;                  // sub-problem levels (0: causal with n <= base)
  int64_t S = 0;              // slots per level per head: n or n / 2
  int64_t nodes = 0;          // 2^L - 1 (causal) or 1
  int64_t base_block = 0;     // causal diagonal block size n >> L
  int64_t vblocks = 0;        // V-norm blocks per head
  int64_t sort_wgs = 0;       // sort chunk work-groups (all levels/heads/sides)
  int64_t att_wgs = 0;        // bucket attention work-groups
  bool backward = false;      // workspace of the backward pass
  int64_t smp_wgs = 0;        // sample-slot gradient items (backward)
  LevelTable table{};
  int64_t off[HA_WS_COUNT] = {};
  int64_t bytes[HA_WS_COUNT] = {};
  size_t total = 0;
};

constexpr int kVnormBlock = 256;     // rows per V-norm work-group
constexpr int kAttnQ = 256;          // query rows per attention work-group
constexpr int kQueues = 8;           // work queues of the persistent attention kernels (one per XCD)
constexpr int kBwdQChunk = 8192;     // query positions per sample-slot gradient item
constexpr int kBwdMaxM = 2048;       // largest m of the backward pass (slot lists staged in LDS)

int make_plan(Plan& p, int64_t n, int d, int heads, int causal, int b, int m,
              int base, int r, int dtype, bool product, bool backward = false);
int check_workspace(const Plan& p, const void* ws, size_t ws_bytes);

// Hyperplanes of (seed, heads, r, d), drawn on the device into `stage`
// (hyperplane_stage_bytes bytes, the workspace region HA_WS_PLANES) on
// stream s. *out: fp32 values [heads][r][d]; *out_bf16 (optional): the same
// values as bf16 bit patterns in [heads][16][d], hyperplanes r..15 zero.
int launch_hyperplanes(uint64_t seed, int heads, int r, int d, void* stage, hipStream_t s,
                       const float** out, const uint16_t** out_bf16 = nullptr);
int64_t hyperplane_stage_bytes(int heads, int r, int d);
// The same values computed on the host ([heads][r][d] floats).
void host_hyperplanes(uint64_t seed, int heads, int r, int d, float* G);
// Box-Muller normals (binary64, before rounding) from pairs of draws.
void host_gaussians(const uint64_t* a, const uint64_t* b, int64_t count, double* out);

// --------------------------------------------------------------- launchers
// All return HA_OK or HA_ERR_HIP; arguments are validated by the caller.
// Q (with K) null: no hash; V null: no V norms.
int launch_hash(const Plan& p, const void* Q, const void* K, const void* V,
                const float* G, const uint16_t* Gb, void* ws, hipStream_t s);
// Rotary embedding of Q and K into Qr and Kr (rope.hip); with hash, also the
// sortLSH codes of the rotated rows. tab: the caller's cos/sin table
// [>= n][d/2][2] in device memory.
int launch_rope(const Plan& p, const void* Q, const void* K, void* Qr, void* Kr,
                const float* tab, bool hash, const float* G, const uint16_t* Gb, void* ws,
                hipStream_t s);
// In place: the gradients of the rows before rotation (dQ, dK [heads][n][d])
// from those of the rotated rows, i.e. the adjoint rotation by -i theta_t.
int launch_rope_adjoint(void* dQ, void* dK, int64_t n, int d, int heads, int dtype,
                        const float* tab, hipStream_t s);
// cos and sin of i * base^(-2t/d) for rows i < n and pairs t < d/2, as
// [n][d/2][2], fp64 from the C library rounded to fp32 (host).
void host_rope_table(int64_t n, int d, double base, float* out);
int launch_hash_one(const void* X, int64_t n, int d, int heads, int r, int dtype,
                    const float* G, const uint16_t* Gb, uint8_t* codes, hipStream_t s);
int launch_vnorm_scan(const Plan& p, void* ws, hipStream_t s);
int launch_sort(const Plan& p, void* ws, int sides, hipStream_t s);
int launch_sort_single(const uint8_t* codes, int64_t n, int heads, int32_t* perm,
                       void* scratch, hipStream_t s);
int launch_samples(const Plan& p, uint64_t seed, void* ws, hipStream_t s);
int launch_bucket_attention(const Plan& p, const void* Q, const void* K,
                            const void* V, void* O, float* lse, void* ws,
                            hipStream_t s);
int launch_exact(const void* Q, const void* K, const void* V, void* O, float* lse,
                 int64_t n, int d, int heads, int causal, int dtype,
                 int64_t block, const Plan* merge, const void* ws, hipStream_t s);

size_t sort_single_scratch_bytes(int64_t n, int heads);

// ------------------------------------------------------------ backward pass
// Inputs and outputs of one backward call (device pointers, bf16 tensors
// [heads][n][d]; lse and delta fp32 [heads][n]).
struct BwdIO {
  const void* Q;
  const void* K;
  const void* V;
  const void* dO;
  const float* lse;       // final log-normaliser of each row (forward output)
  const float* delta;     // dO_i . O_i (launch_delta's output)
  void* dQ;
  void* dK;
  void* dV;
};
// delta[row] = sum_t O[row][t] dO[row][t] for rows * d elements (bf16)
int launch_delta(const void* O, const void* dO, float* delta, int64_t rows, int d,
                 hipStream_t s);
// Per node: which sample slots share a key row (first slot per key row of the
// node, next slot with the same row).
int launch_bwd_links(const Plan& p, void* ws, hipStream_t s);
// Gradient of every sample slot's key and value rows, partial per query chunk.
int launch_bwd_samples(const Plan& p, const BwdIO& io, void* ws, hipStream_t s);
// dQ of every bucket's queries, and dK, dV of every bucket's keys plus the
// node's sample slots on those rows: per-level partials (causal) or the
// outputs (non-causal).
int launch_bwd_bucket(const Plan& p, const BwdIO& io, void* ws, hipStream_t s);
// Exact attention's gradients over key/query blocks of `block` rows; with
// merge, the base case of the causal recursion, adding every level's partials.
// queue: kQueues work-queue counters (device memory; zeroed here).
int launch_bwd_exact(const BwdIO& io, int64_t n, int d, int heads, int causal, int64_t block,
                     const Plan* merge, const void* ws, uint32_t* queue, hipStream_t s);

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace ha
