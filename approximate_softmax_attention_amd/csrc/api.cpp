// The C ABI declared in include/hyperattn.h: argument validation, the launch
// sequence of each entry point, the thread-local error message and the
// event-based kernel timing.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace ha {

namespace {
thread_local std::string g_error;
}

void set_error(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
}

int fail(int code, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

// ------------------------------------------------------------ profiling
namespace {

struct ProfRecord {
  int name;
  hipEvent_t start, stop;
  int device;
  int64_t groups;
};

struct ProfName {
  std::string name;
  int64_t launches = 0;
  double total_ms = 0.0;
  int64_t groups = 0;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRecord> g_pending;
std::vector<ProfRecord> g_free;
std::vector<ProfName> g_names;

int name_index(const char* name) {
  for (size_t i = 0; i < g_names.size(); ++i)
    if (g_names[i].name == name) return int(i);
  g_names.push_back(ProfName{name});
  return int(g_names.size() - 1);
}

}  // namespace

ProfRange::ProfRange(const char* name, hipStream_t s) : slot(-1), stream(s) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  if (!g_prof_on) return;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return;
  ProfRecord r{};
  bool have = false;
  for (size_t i = 0; i < g_free.size(); ++i)
    if (g_free[i].device == dev) {
      r = g_free[i];
      g_free.erase(g_free.begin() + i);
      have = true;
      break;
    }
  if (!have) {
    if (hipEventCreate(&r.start) != hipSuccess) return;
    if (hipEventCreate(&r.stop) != hipSuccess) {
      (void)hipEventDestroy(r.start);
      return;
    }
    r.device = dev;
  }
  r.name = name_index(name);
  if (hipEventRecord(r.start, s) != hipSuccess) {
    g_free.push_back(r);
    return;
  }
  g_pending.push_back(r);
  slot = int(g_pending.size() - 1);
}

ProfRange::~ProfRange() {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lock(g_prof_mu);
  if (size_t(slot) < g_pending.size()) {
    g_pending[slot].groups = groups;
    (void)hipEventRecord(g_pending[slot].stop, stream);
  }
}

// ------------------------------------------------------------ occupancy
namespace {
struct Resident {
  int device;
  const void* kernel;
  int threads;
  int groups;
};
std::mutex g_res_mu;
std::vector<Resident> g_resident;
}  // namespace

int resident_groups_of(const void* kernel, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(g_res_mu);
  for (const Resident& r : g_resident)
    if (r.device == dev && r.kernel == kernel && r.threads == threads) return r.groups;
  // The queries enqueue nothing; while the caller captures a stream in the
  // global mode, this thread takes the relaxed mode for them so that they do
  // not invalidate the capture.
  hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
  if (hipThreadExchangeStreamCaptureMode(&mode) != hipSuccess) return 0;
  int per_cu = 0, cus = 0;
  const bool ok =
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess;
  (void)hipThreadExchangeStreamCaptureMode(&mode);
  if (!ok) return 0;
  const int groups = (per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  g_resident.push_back(Resident{dev, kernel, threads, groups});
  return groups;
}

// ------------------------------------------------------------ overlaps
namespace {

struct Span {
  const void* p;
  size_t bytes;
  const char* name;
};

bool overlap(const Span& a, const Span& b) {
  if (!a.p || !b.p || !a.bytes || !b.bytes) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

}  // namespace

// Every written range (outputs and the workspace) must be disjoint from
// every read range and from the other written ranges; inputs may share
// memory with each other.
int check_disjoint(std::initializer_list<Span> written, std::initializer_list<Span> read) {
  for (const Span* o = written.begin(); o != written.end(); ++o) {
    for (const Span& i : read)
      if (overlap(*o, i)) return fail(HA_ERR_SHAPE, "%s overlaps the input %s", o->name, i.name);
    for (const Span* o2 = o + 1; o2 != written.end(); ++o2)
      if (overlap(*o, *o2)) return fail(HA_ERR_SHAPE, "%s overlaps %s", o->name, o2->name);
  }
  return HA_OK;
}

}  // namespace ha

using namespace ha;

extern "C" {

const char* hyperattn_last_error(void) { return g_error.c_str(); }

size_t hyperattn_workspace_bytes(int64_t n, int d, int heads, int causal, int b, int m,
                                 int recursion_base, int r, int dtype) {
  g_error.clear();
  Plan p;
  if (make_plan(p, n, d, heads, causal, b, m, recursion_base, r, dtype, true) != HA_OK) return 0;
  return p.total;
}

int hyperattn_workspace_layout(int64_t n, int d, int heads, int causal, int b, int m,
                               int recursion_base, int r, int dtype, int64_t* offsets,
                               int64_t* bytes) {
  g_error.clear();
  if (!offsets || !bytes) return fail(HA_ERR_NULL, "offsets and bytes must not be NULL");
  Plan p;
  const int rc = make_plan(p, n, d, heads, causal, b, m, recursion_base, r, dtype, true);
  if (rc != HA_OK) return rc;
  for (int i = 0; i < HA_WS_COUNT; ++i) {
    offsets[i] = p.off[i];
    bytes[i] = p.bytes[i];
  }
  return HA_OK;
}

int sortlsh_hyperplanes(uint64_t seed, int heads, int r, int d, float* G_host) {
  g_error.clear();
  if (r < 0 || r > 8) return fail(HA_ERR_UNSUPPORTED, "r=%d not in [0, 8]", r);
  if (!G_host && r > 0) return fail(HA_ERR_NULL, "G_host is NULL");
  if (d != 64 && d != 128) return fail(HA_ERR_UNSUPPORTED, "d=%d not 64 or 128", d);
  if (heads < 0 || heads >= (1 << 16)) return fail(HA_ERR_SHAPE, "heads=%d out of range", heads);
  host_hyperplanes(seed, heads, r, d, G_host);
  return HA_OK;
}

int exact_attention_forward(const void* Q, const void* K, const void* V, void* O, float* lse,
                            int64_t n, int d, int heads, int causal, int dtype, void* stream) {
  g_error.clear();
  if (dtype != HA_F32 && dtype != HA_BF16)
    return fail(HA_ERR_UNSUPPORTED, "dtype %d is not HA_F32 or HA_BF16", dtype);
  if (d != 64 && d != 128) return fail(HA_ERR_UNSUPPORTED, "d=%d not 64 or 128", d);
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(HA_ERR_SHAPE, "n=%lld out of range", (long long)n);
  if (heads < 0 || heads >= (1 << 16)) return fail(HA_ERR_SHAPE, "heads=%d out of range", heads);
  if (n * d * (dtype == HA_BF16 ? 2 : 4) >= (int64_t(1) << 31))
    return fail(HA_ERR_SHAPE, "one head of n=%lld rows exceeds 2 GiB", (long long)n);
  if (n == 0 || heads == 0) return HA_OK;
  if (!Q || !K || !V || !O) return fail(HA_ERR_NULL, "Q, K, V and O must not be NULL");
  {
    const size_t t = size_t(n) * d * heads * (dtype == HA_BF16 ? 2 : 4);
    const int rc = check_disjoint({{O, t, "O"}, {lse, size_t(n) * heads * 4, "lse"}},
                                  {{Q, t, "Q"}, {K, t, "K"}, {V, t, "V"}});
    if (rc != HA_OK) return rc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return launch_exact(Q, K, V, O, lse, n, d, heads, causal ? 1 : 0, dtype, n, nullptr, nullptr, s);
}

namespace {

// The forward pass; with rope set, Q and K are first rotated into Qr and Kr
// (in the pass that hashes them) and the attention reads those.
struct Rope {
  void* Qr;
  void* Kr;
  const float* tab;   // caller's cos/sin table [rows][d/2][2] (device)
  int64_t rows;
};

int forward_impl(const void* Q, const void* K, const void* V, void* O, float* lse, int64_t n,
                 int d, int heads, int causal, int b, int m, int recursion_base, int r,
                 uint64_t seed, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream, const Rope* rope) {
  Plan p;
  int rc = make_plan(p, n, d, heads, causal, b, m, recursion_base, r, dtype, true);
  if (rc != HA_OK) return rc;
  if (n == 0 || heads == 0) return HA_OK;
  if (!Q || !K || !V || !O) return fail(HA_ERR_NULL, "Q, K, V and O must not be NULL");
  if (rope && (!rope->Qr || !rope->Kr)) return fail(HA_ERR_NULL, "Q_rot and K_rot must not be NULL");
  if (rope && !rope->tab) return fail(HA_ERR_NULL, "the cos/sin table must not be NULL");
  if (rope && rope->rows < n)
    return fail(HA_ERR_SHAPE, "the cos/sin table has %lld rows, n = %lld", (long long)rope->rows,
                (long long)n);
  // the single-block causal case uses no workspace; otherwise it is checked first
  const bool single = p.causal && p.L == 0;
  if (!single && (rc = check_workspace(p, workspace, workspace_bytes)) != HA_OK) return rc;
  {
    const size_t t = size_t(n) * d * heads * p.esize;
    rc = check_disjoint({{O, t, "O"}, {lse, size_t(n) * heads * 4, "lse"},
                         {rope ? rope->Qr : nullptr, t, "Q_rot"},
                         {rope ? rope->Kr : nullptr, t, "K_rot"},
                         {single ? nullptr : workspace, p.total, "workspace"}},
                        {{Q, t, "Q"}, {K, t, "K"}, {V, t, "V"},
                         {rope ? rope->tab : nullptr, rope ? size_t(rope->rows) * d * 4 : 0,
                          "cos_sin"}});
    if (rc != HA_OK) return rc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* tab = rope ? rope->tab : nullptr;
  if (p.causal && p.L == 0) {  // the whole sequence is one base block
    if (rope) {
      if ((rc = launch_rope(p, Q, K, rope->Qr, rope->Kr, tab, false, nullptr, nullptr, nullptr,
                            s)) != HA_OK)
        return rc;
      Q = rope->Qr;
      K = rope->Kr;
    }
    return launch_exact(Q, K, V, O, lse, n, d, heads, 1, dtype, n, nullptr, nullptr, s);
  }
  const float* G = nullptr;
  const uint16_t* Gb = nullptr;
  if ((rc = launch_hyperplanes(seed, heads, r, d, static_cast<char*>(workspace) + p.off[HA_WS_PLANES],
                               s, &G, &Gb)) != HA_OK)
    return rc;
  if (rope) {
    if ((rc = launch_rope(p, Q, K, rope->Qr, rope->Kr, tab, true, G, Gb, workspace, s)) != HA_OK)
      return rc;
    Q = rope->Qr;
    K = rope->Kr;
    rc = launch_hash(p, nullptr, nullptr, V, G, Gb, workspace, s);
  } else {
    rc = launch_hash(p, Q, K, V, G, Gb, workspace, s);
  }
  if (rc != HA_OK) return rc;
  if ((rc = launch_vnorm_scan(p, workspace, s)) != HA_OK) return rc;
  if ((rc = launch_sort(p, workspace, 2, s)) != HA_OK) return rc;
  if ((rc = launch_samples(p, seed, workspace, s)) != HA_OK) return rc;
  if ((rc = launch_bucket_attention(p, Q, K, V, O, lse, workspace, s)) != HA_OK) return rc;
  if (p.causal)
    rc = launch_exact(Q, K, V, O, lse, n, d, heads, 1, dtype, p.base_block, &p, workspace, s);
  return rc;
}

}  // namespace

int hyperattn_forward(const void* Q, const void* K, const void* V, void* O, float* lse,
                      int64_t n, int d, int heads, int causal, int b, int m, int recursion_base,
                      int r, uint64_t seed, int dtype, void* workspace, size_t workspace_bytes,
                      void* stream) {
  g_error.clear();
  return forward_impl(Q, K, V, O, lse, n, d, heads, causal, b, m, recursion_base, r, seed,
                      dtype, workspace, workspace_bytes, stream, nullptr);
}

int hyperattn_forward_rope(const void* Q, const void* K, const void* V, const float* cos_sin,
                           int64_t cos_sin_rows, void* Q_rot, void* K_rot, void* O, float* lse,
                           int64_t n, int d, int heads, int causal, int b, int m,
                           int recursion_base, int r, uint64_t seed, int dtype, void* workspace,
                           size_t workspace_bytes, void* stream) {
  g_error.clear();
  const Rope rope{Q_rot, K_rot, cos_sin, cos_sin_rows};
  return forward_impl(Q, K, V, O, lse, n, d, heads, causal, b, m, recursion_base, r, seed,
                      dtype, workspace, workspace_bytes, stream, &rope);
}

int rope_table(int64_t n, int d, double rope_base, float* table_host) {
  g_error.clear();
  if (d != 64 && d != 128) return fail(HA_ERR_UNSUPPORTED, "d=%d not 64 or 128", d);
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(HA_ERR_SHAPE, "n=%lld out of range", (long long)n);
  if (!(rope_base > 1.0 && std::isfinite(rope_base)))
    return fail(HA_ERR_UNSUPPORTED, "rope_base=%g must be a finite number above 1", rope_base);
  if (n == 0) return HA_OK;
  if (!table_host) return fail(HA_ERR_NULL, "table_host is NULL");
  host_rope_table(n, d, rope_base, table_host);
  return HA_OK;
}

int rowsum_estimate(const void* Q, const void* K, int64_t n, int d, int heads, int b, int m, int r,
                    uint64_t seed, int dtype, float* log_d, void* workspace,
                    size_t workspace_bytes, void* stream) {
  g_error.clear();
  Plan p;
  int rc = make_plan(p, n, d, heads, 0, b, m, 1, r, dtype, false);
  if (rc != HA_OK) return rc;
  if (n == 0 || heads == 0) return HA_OK;
  if (!Q || !K || !log_d) return fail(HA_ERR_NULL, "Q, K and log_d must not be NULL");
  // the caller sizes the workspace with hyperattn_workspace_bytes(..., causal=0, ...),
  // which covers this plan's smaller carve-up region by region
  Plan full;
  rc = make_plan(full, n, d, heads, 0, b, m, 1, r, dtype, true);
  if (rc != HA_OK) return rc;
  rc = check_workspace(full, workspace, workspace_bytes);
  if (rc != HA_OK) return rc;
  {
    const size_t t = size_t(n) * d * heads * p.esize;
    rc = check_disjoint({{log_d, size_t(n) * heads * 4, "log_d"}, {workspace, full.total, "workspace"}},
                        {{Q, t, "Q"}, {K, t, "K"}});
    if (rc != HA_OK) return rc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* G = nullptr;
  const uint16_t* Gb = nullptr;
  if ((rc = launch_hyperplanes(seed, heads, r, d,
                               static_cast<char*>(workspace) + full.off[HA_WS_PLANES], s, &G,
                               &Gb)) != HA_OK)
    return rc;
  if ((rc = launch_hash(p, Q, K, nullptr, G, Gb, workspace, s)) != HA_OK) return rc;
  if ((rc = launch_sort(p, workspace, 2, s)) != HA_OK) return rc;
  if ((rc = launch_samples(p, seed, workspace, s)) != HA_OK) return rc;
  return launch_bucket_attention(p, Q, K, nullptr, nullptr, log_d, workspace, s);
}

size_t hyperattn_backward_workspace_bytes(int64_t n, int d, int heads, int causal, int b, int m,
                                          int recursion_base, int r, int dtype) {
  g_error.clear();
  Plan p;
  if (make_plan(p, n, d, heads, causal, b, m, recursion_base, r, dtype, true, true) != HA_OK)
    return 0;
  return p.total;
}

namespace {
int backward_impl(const void* Q, const void* K, const void* V, const void* O, const float* lse,
                  const void* dO, void* dQ, void* dK, void* dV, int64_t n, int d, int heads,
                  int causal, int b, int m, int recursion_base, int r, uint64_t seed, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream,
                  const void* extra = nullptr, size_t extra_bytes = 0);
}  // namespace

int hyperattn_backward(const void* Q, const void* K, const void* V, const void* O,
                       const float* lse, const void* dO, void* dQ, void* dK, void* dV, int64_t n,
                       int d, int heads, int causal, int b, int m, int recursion_base, int r,
                       uint64_t seed, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
  g_error.clear();
  return backward_impl(Q, K, V, O, lse, dO, dQ, dK, dV, n, d, heads, causal, b, m,
                       recursion_base, r, seed, dtype, workspace, workspace_bytes, stream);
}

int hyperattn_backward_rope(const void* Q_rot, const void* K_rot, const void* V, const void* O,
                            const float* lse, const void* dO, const float* cos_sin,
                            int64_t cos_sin_rows, void* dQ, void* dK, void* dV, int64_t n,
                            int d, int heads, int causal, int b, int m, int recursion_base,
                            int r, uint64_t seed, int dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  g_error.clear();
  if (n > 0 && heads > 0) {
    if (!cos_sin) return fail(HA_ERR_NULL, "the cos/sin table must not be NULL");
    if (cos_sin_rows < n)
      return fail(HA_ERR_SHAPE, "the cos/sin table has %lld rows, n = %lld",
                  (long long)cos_sin_rows, (long long)n);
  }
  int rc = backward_impl(Q_rot, K_rot, V, O, lse, dO, dQ, dK, dV, n, d, heads, causal, b, m,
                         recursion_base, r, seed, dtype, workspace, workspace_bytes, stream,
                         cos_sin, size_t(cos_sin_rows > 0 ? cos_sin_rows : 0) * d * 4);
  if (rc != HA_OK || n == 0 || heads == 0) return rc;
  return launch_rope_adjoint(dQ, dK, n, d, heads, dtype, cos_sin,
                             static_cast<hipStream_t>(stream));
}

namespace {
int backward_impl(const void* Q, const void* K, const void* V, const void* O, const float* lse,
                  const void* dO, void* dQ, void* dK, void* dV, int64_t n, int d, int heads,
                  int causal, int b, int m, int recursion_base, int r, uint64_t seed, int dtype,
                  void* workspace, size_t workspace_bytes, void* stream, const void* extra,
                  size_t extra_bytes) {
  Plan p;
  int rc = make_plan(p, n, d, heads, causal, b, m, recursion_base, r, dtype, true, true);
  if (rc != HA_OK) return rc;
  if (n == 0 || heads == 0) return HA_OK;
  if (!Q || !K || !V || !O || !lse || !dO || !dQ || !dK || !dV)
    return fail(HA_ERR_NULL, "Q, K, V, O, lse, dO, dQ, dK and dV must not be NULL");
  rc = check_workspace(p, workspace, workspace_bytes);
  if (rc != HA_OK) return rc;
  {
    const size_t t = size_t(n) * d * heads * 2;
    rc = check_disjoint({{dQ, t, "dQ"}, {dK, t, "dK"}, {dV, t, "dV"},
                         {workspace, p.total, "workspace"}},
                        {{Q, t, "Q"}, {K, t, "K"}, {V, t, "V"}, {O, t, "O"},
                         {lse, size_t(n) * heads * 4, "lse"}, {dO, t, "dO"},
                         {extra, extra_bytes, "cos_sin"}});
    if (rc != HA_OK) return rc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  float* delta = reinterpret_cast<float*>(w + p.off[HA_WS_DELTA]);
  const BwdIO io{Q, K, V, dO, lse, delta, dQ, dK, dV};
  uint32_t* queue = reinterpret_cast<uint32_t*>(w + p.off[HA_WS_SCHED]);
  if ((rc = launch_delta(O, dO, delta, n * heads, d, s)) != HA_OK) return rc;
  if (p.causal && p.L == 0)   // the whole sequence is one base block
    return launch_bwd_exact(io, n, d, heads, 1, n, nullptr, nullptr, queue, s);
  // the forward pass's buckets and sample lists, recomputed from the seed
  const float* G = nullptr;
  const uint16_t* Gb = nullptr;
  if ((rc = launch_hyperplanes(seed, heads, r, d, w + p.off[HA_WS_PLANES], s, &G, &Gb)) != HA_OK)
    return rc;
  if ((rc = launch_hash(p, Q, K, V, G, Gb, workspace, s)) != HA_OK) return rc;
  if ((rc = launch_vnorm_scan(p, workspace, s)) != HA_OK) return rc;
  if ((rc = launch_sort(p, workspace, 2, s)) != HA_OK) return rc;
  if ((rc = launch_samples(p, seed, workspace, s)) != HA_OK) return rc;
  if ((rc = launch_bwd_links(p, workspace, s)) != HA_OK) return rc;
  if ((rc = launch_bwd_samples(p, io, workspace, s)) != HA_OK) return rc;
  if ((rc = launch_bwd_bucket(p, io, workspace, s)) != HA_OK) return rc;
  if (p.causal) rc = launch_bwd_exact(io, n, d, heads, 1, p.base_block, &p, workspace, queue, s);
  return rc;
}
}  // namespace

size_t exact_attention_backward_workspace_bytes(int64_t n, int heads) {
  g_error.clear();
  if (n < 0 || heads < 0) return 0;
  return size_t(align256(n * heads * 4) + 256);   // Delta, then the work-queue counters
}

int exact_attention_backward(const void* Q, const void* K, const void* V, const void* O,
                             const float* lse, const void* dO, void* dQ, void* dK, void* dV,
                             int64_t n, int d, int heads, int causal, int dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  g_error.clear();
  if (dtype != HA_BF16) return fail(HA_ERR_UNSUPPORTED, "the backward pass takes bf16 tensors only");
  if (d != 64 && d != 128) return fail(HA_ERR_UNSUPPORTED, "d=%d not 64 or 128", d);
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(HA_ERR_SHAPE, "n=%lld out of range", (long long)n);
  if (heads < 0 || heads >= (1 << 16)) return fail(HA_ERR_SHAPE, "heads=%d out of range", heads);
  if (n * d * 2 >= (int64_t(1) << 31))
    return fail(HA_ERR_SHAPE, "one head of n=%lld rows exceeds 2 GiB", (long long)n);
  if (n == 0 || heads == 0) return HA_OK;
  if (!Q || !K || !V || !O || !lse || !dO || !dQ || !dK || !dV)
    return fail(HA_ERR_NULL, "Q, K, V, O, lse, dO, dQ, dK and dV must not be NULL");
  const size_t need = size_t(align256(n * heads * 4) + 256);
  if (!workspace) return fail(HA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(HA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(HA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  {
    const size_t t = size_t(n) * d * heads * 2;
    const int rc = check_disjoint({{dQ, t, "dQ"}, {dK, t, "dK"}, {dV, t, "dV"},
                                   {workspace, need, "workspace"}},
                                  {{Q, t, "Q"}, {K, t, "K"}, {V, t, "V"}, {O, t, "O"},
                                   {lse, size_t(n) * heads * 4, "lse"}, {dO, t, "dO"}});
    if (rc != HA_OK) return rc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* delta = static_cast<float*>(workspace);
  uint32_t* queue = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                                align256(n * heads * 4));
  const BwdIO io{Q, K, V, dO, lse, delta, dQ, dK, dV};
  int rc = launch_delta(O, dO, delta, n * heads, d, s);
  if (rc != HA_OK) return rc;
  return launch_bwd_exact(io, n, d, heads, causal ? 1 : 0, n, nullptr, nullptr, queue, s);
}

namespace {
// sortlsh_hash's workspace: the hyperplanes, then (with perm) the sort's
// scratch at the next 256-byte boundary.
size_t hash_ws_bytes(int64_t n, int d, int heads, int r, bool with_perm) {
  return size_t(align256(hyperplane_stage_bytes(heads, r, d))) +
         (with_perm ? sort_single_scratch_bytes(n, heads) : 0);
}
}  // namespace

size_t sortlsh_hash_workspace_bytes(int64_t n, int d, int heads, int r, int with_perm) {
  g_error.clear();
  if (n < 0 || heads < 0 || heads >= (1 << 16) || r < 0 || r > 8 || (d != 64 && d != 128)) {
    set_error("invalid sizes for sortlsh_hash (n=%lld, d=%d, heads=%d, r=%d)", (long long)n, d,
              heads, r);
    return 0;
  }
  return hash_ws_bytes(n, d, heads, r, with_perm != 0);
}

int sortlsh_hash(const void* X, int64_t n, int d, int heads, int r, uint64_t seed, int dtype,
                 uint8_t* codes, int32_t* perm, void* workspace, size_t workspace_bytes,
                 void* stream) {
  g_error.clear();
  if (dtype != HA_F32 && dtype != HA_BF16)
    return fail(HA_ERR_UNSUPPORTED, "dtype %d is not HA_F32 or HA_BF16", dtype);
  if (d != 64 && d != 128) return fail(HA_ERR_UNSUPPORTED, "d=%d not 64 or 128", d);
  if (r < 0 || r > 8) return fail(HA_ERR_UNSUPPORTED, "r=%d not in [0, 8]", r);
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(HA_ERR_SHAPE, "n=%lld out of range", (long long)n);
  if (heads < 0 || heads >= (1 << 16)) return fail(HA_ERR_SHAPE, "heads=%d out of range", heads);
  if (n * d * (dtype == HA_BF16 ? 2 : 4) >= (int64_t(1) << 31))
    return fail(HA_ERR_SHAPE, "one head of n=%lld rows exceeds 2 GiB", (long long)n);
  if (n == 0 || heads == 0) return HA_OK;
  if (!X || !codes) return fail(HA_ERR_NULL, "X and codes must not be NULL");
  const size_t need = hash_ws_bytes(n, d, heads, r, perm != nullptr);
  if (!workspace) return fail(HA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(HA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(HA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  int rc = check_disjoint({{codes, size_t(n) * heads, "codes"},
                           {perm, size_t(n) * heads * 4, "perm"},
                           {workspace, need, "workspace"}},
                          {{X, size_t(n) * d * heads * (dtype == HA_BF16 ? 2 : 4), "X"}});
  if (rc != HA_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* G = nullptr;
  const uint16_t* Gb = nullptr;
  if ((rc = launch_hyperplanes(seed, heads, r, d, workspace, s, &G, &Gb)) != HA_OK) return rc;
  if ((rc = launch_hash_one(X, n, d, heads, r, dtype, G, Gb, codes, s)) != HA_OK) return rc;
  if (perm)
    rc = launch_sort_single(codes, n, heads, perm,
                            static_cast<char*>(workspace) +
                                align256(hyperplane_stage_bytes(heads, r, d)),
                            s);
  return rc;
}

int sortlsh_gaussians(const uint64_t* a, const uint64_t* b, int64_t count, double* out) {
  g_error.clear();
  if (count < 0) return fail(HA_ERR_SHAPE, "count=%lld is negative", (long long)count);
  if (count == 0) return HA_OK;
  if (!a || !b || !out) return fail(HA_ERR_NULL, "a, b and out must not be NULL");
  host_gaussians(a, b, count, out);
  return HA_OK;
}

int hyperattn_debug_artifacts(const void* Q, const void* K, const void* V, int64_t n, int d,
                              int heads, int causal, int b, int m, int recursion_base, int r,
                              uint64_t seed, int dtype, void* workspace, size_t workspace_bytes,
                              void* stream, const ha_artifacts* out) {
  g_error.clear();
  Plan p;
  int rc = make_plan(p, n, d, heads, causal, b, m, recursion_base, r, dtype, true);
  if (rc != HA_OK) return rc;
  if (!out) return fail(HA_ERR_NULL, "out must not be NULL");
  if (n == 0 || heads == 0) return HA_OK;
  if (!Q || !K || !V) return fail(HA_ERR_NULL, "Q, K and V must not be NULL");
  if ((rc = check_workspace(p, workspace, workspace_bytes)) != HA_OK) return rc;
  {
    const size_t t = size_t(n) * d * heads * p.esize;
    rc = check_disjoint({{workspace, p.total, "workspace"}},
                        {{Q, t, "Q"}, {K, t, "K"}, {V, t, "V"}});
    if (rc != HA_OK) return rc;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(workspace);
  const float* G = nullptr;
  const uint16_t* Gb = nullptr;
  if ((rc = launch_hyperplanes(seed, heads, r, d, w + p.off[HA_WS_PLANES], s, &G, &Gb)) != HA_OK)
    return rc;
  if ((rc = launch_hash(p, Q, K, V, G, Gb, workspace, s)) != HA_OK) return rc;
  if ((rc = launch_vnorm_scan(p, workspace, s)) != HA_OK) return rc;
  const bool subs = !(p.causal && p.L == 0);
  if (subs) {
    if ((rc = launch_sort(p, workspace, 2, s)) != HA_OK) return rc;
    if ((rc = launch_samples(p, seed, workspace, s)) != HA_OK) return rc;
  }
  const struct {
    void* host;
    int region;
  } copies[] = {
      {out->codes_q, HA_WS_CODES_Q}, {out->codes_k, HA_WS_CODES_K},
      {out->vnorm_w, HA_WS_VNORM_W}, {out->vnorm_p, HA_WS_VNORM_P},
      {out->perm_q, HA_WS_PERM_Q},   {out->perm_k, HA_WS_PERM_K},
      {out->rank_k, HA_WS_RANK_K},   {out->u_idx, HA_WS_U_IDX},
      {out->u_bkt, HA_WS_U_BKT},     {out->v_idx, HA_WS_V_IDX},
      {out->v_bkt, HA_WS_V_BKT},     {out->v_w, HA_WS_V_W},
      {out->node_meta, HA_WS_NODE_META},
  };
  for (const auto& c : copies) {
    if (!c.host || p.bytes[c.region] == 0) continue;
    if (!subs && c.region != HA_WS_CODES_Q && c.region != HA_WS_CODES_K &&
        c.region != HA_WS_VNORM_W && c.region != HA_WS_VNORM_P)
      continue;
    HA_HIP_TRY(hipMemcpyAsync(c.host, w + p.off[c.region], size_t(p.bytes[c.region]),
                              hipMemcpyDeviceToHost, s));
  }
  HA_HIP_TRY(hipStreamSynchronize(s));
  return HA_OK;
}

// ------------------------------------------------------------ profiling
int hyperattn_profile_enable(int on) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  g_prof_on = on != 0;
  return HA_OK;
}

int hyperattn_profile_collect(void) {
  g_error.clear();
  std::lock_guard<std::mutex> lock(g_prof_mu);
  int cur = 0;
  HA_HIP_TRY(hipGetDevice(&cur));
  for (ProfRecord& r : g_pending) {
    HA_HIP_TRY(hipSetDevice(r.device));
    HA_HIP_TRY(hipEventSynchronize(r.stop));
    float ms = 0.f;
    HA_HIP_TRY(hipEventElapsedTime(&ms, r.start, r.stop));
    g_names[r.name].launches += 1;
    g_names[r.name].total_ms += ms;
    g_names[r.name].groups += r.groups;
    g_free.push_back(r);
  }
  g_pending.clear();
  HA_HIP_TRY(hipSetDevice(cur));
  return HA_OK;
}

int hyperattn_profile_reset(void) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  for (ProfName& nm : g_names) {
    nm.launches = 0;
    nm.total_ms = 0.0;
    nm.groups = 0;
  }
  return HA_OK;
}

int hyperattn_profile_count(void) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  return int(g_names.size());
}

const char* hyperattn_profile_name(int i) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  return (i >= 0 && size_t(i) < g_names.size()) ? g_names[i].name.c_str() : "";
}

int64_t hyperattn_profile_launches(int i) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  return (i >= 0 && size_t(i) < g_names.size()) ? g_names[i].launches : 0;
}

int64_t hyperattn_profile_groups(int i) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  return (i >= 0 && size_t(i) < g_names.size()) ? g_names[i].groups : 0;
}

double hyperattn_profile_total_ms(int i) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  return (i >= 0 && size_t(i) < g_names.size()) ? g_names[i].total_ms : 0.0;
}

}  // extern "C"
