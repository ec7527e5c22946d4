// The r Gaussian hyperplanes per head that the hash uses (HA page,
// "Algorithm", Definition 1: a Hamming-sorted LSH; read here as signs of
// projections on Gaussian hyperplanes).
//
// Each element comes from two counter-based draws of SplitMix64 (Steele, Lea
// and Flood, OOPSLA 2014), turned into one normal by the Box-Muller transform
// (Box and Muller, 1958) in fp64 with the C library's log, sqrt and cos,
// rounded to fp32 and then to the nearest bfloat16 (a bf16 input times a
// hyperplane entry is then exact in fp32). They are generated on the host so that the values are
// fixed by the C library, and kept on each device for up to 16 keys
// (seed, heads, r, d); further keys are staged through the caller's workspace
// on the caller's stream.
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"

namespace ha {

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

uint64_t mix64(uint64_t x) {
  uint64_t z = x + kGamma;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t draw(uint64_t key, uint64_t purpose, uint64_t head, uint64_t node,
              uint64_t counter) {
  return mix64(key ^ ((purpose << 60) | (head << 44) | (node << 24) | counter));
}

struct Entry {
  int device;
  uint64_t seed;
  int heads, r, d;
  float* ptr;          // fp32 [heads][r][d]
  uint16_t* ptr_bf16;  // bf16 [heads][16][d], rows >= r zero
  uint64_t stamp;
};

std::mutex g_mu;
std::vector<Entry> g_cache;
uint64_t g_clock = 0;
constexpr size_t kCacheEntries = 16;

// Nearest bfloat16 of an fp32 value (ties to even), kept as an fp32 value.
float round_bf16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u = ((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16) << 16;
  float y;
  std::memcpy(&y, &u, 4);
  return y;
}

}  // namespace

void host_hyperplanes(uint64_t seed, int heads, int r, int d, float* G) {
#pragma clang fp contract(off)
  const uint64_t key = mix64(seed);
  const double two_pi = 2.0 * M_PI;
  for (int h = 0; h < heads; ++h)
    for (int k = 0; k < r; ++k)
      for (int t = 0; t < d; ++t) {
        const uint64_t e = uint64_t(k) * d + t;
        const uint64_t a = draw(key, 1, h, 0, 2 * e);
        const uint64_t b = draw(key, 1, h, 0, 2 * e + 1);
        const double u1 = double((a >> 11) + 1) * 0x1p-53;
        const double u2 = double(b >> 11) * 0x1p-53;
        const double g = std::sqrt(-2.0 * std::log(u1)) * std::cos(two_pi * u2);
        G[(int64_t(h) * r + k) * d + t] = round_bf16(static_cast<float>(g));
      }
}

int64_t hyperplane_stage_bytes(int heads, int r, int d) {
  return align256(int64_t(heads) * r * d * 4) + int64_t(heads) * 16 * d * 2;
}

namespace {

// fp32 values [heads][r][d] and their bf16 bit patterns [heads][16][d]
// (hyperplanes r..15 zero)
void fill_host(uint64_t seed, int heads, int r, int d, float* f32, uint16_t* b16) {
  host_hyperplanes(seed, heads, r, d, f32);
  std::memset(b16, 0, size_t(heads) * 16 * d * sizeof(uint16_t));
  for (int h = 0; h < heads; ++h)
    for (int k = 0; k < r; ++k)
      for (int t = 0; t < d; ++t) {
        uint32_t u;
        std::memcpy(&u, &f32[(size_t(h) * r + k) * d + t], 4);
        b16[(size_t(h) * 16 + k) * d + t] = uint16_t(u >> 16);   // exact: bf16 values
      }
}

// Pinned host buffer per device from which staged hyperplanes are copied;
// `done` marks the end of the last copy out of it.
struct Staging {
  int device;
  void* host;
  size_t bytes;
  hipEvent_t done;
  bool pending;
};
std::vector<Staging> g_staging;

int stage_hyperplanes(int dev, uint64_t seed, int heads, int r, int d, void* stage,
                      hipStream_t s, const float** out, const uint16_t** out_bf16) {
  Staging* st = nullptr;
  for (Staging& e : g_staging)
    if (e.device == dev) st = &e;
  if (!st) {
    Staging e{dev, nullptr, 0, nullptr, false};
    HA_HIP_TRY(hipEventCreateWithFlags(&e.done, hipEventDisableTiming));
    g_staging.push_back(e);
    st = &g_staging.back();
  }
  if (st->pending) {          // the previous copy must have left the buffer
    HA_HIP_TRY(hipEventSynchronize(st->done));
    st->pending = false;
  }
  const size_t need = size_t(hyperplane_stage_bytes(heads, r, d));
  if (st->bytes < need) {
    if (st->host) HA_HIP_TRY(hipHostFree(st->host));
    st->host = nullptr;
    st->bytes = 0;
    HA_HIP_TRY(hipHostMalloc(&st->host, need));
    st->bytes = need;
  }
  const size_t off16 = size_t(align256(int64_t(heads) * r * d * 4));
  char* h = static_cast<char*>(st->host);
  fill_host(seed, heads, r, d, reinterpret_cast<float*>(h), reinterpret_cast<uint16_t*>(h + off16));
  HA_HIP_TRY(hipMemcpyAsync(stage, h, need, hipMemcpyHostToDevice, s));
  HA_HIP_TRY(hipEventRecord(st->done, s));
  st->pending = true;
  *out = static_cast<const float*>(stage);
  if (out_bf16) *out_bf16 = reinterpret_cast<const uint16_t*>(static_cast<char*>(stage) + off16);
  return HA_OK;
}

}  // namespace

int device_hyperplanes(uint64_t seed, int heads, int r, int d, const float** out,
                       const uint16_t** out_bf16, void* stage, hipStream_t s) {
  int dev = 0;
  HA_HIP_TRY(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_mu);
  size_t held = 0;
  for (Entry& e : g_cache) {
    if (e.device != dev) continue;
    ++held;
    if (e.seed == seed && e.heads == heads && e.r == r && e.d == d) {
      e.stamp = ++g_clock;
      *out = e.ptr;
      if (out_bf16) *out_bf16 = e.ptr_bf16;
      return HA_OK;
    }
  }
  if (held >= kCacheEntries) {
    if (stage) return stage_hyperplanes(dev, seed, heads, r, d, stage, s, out, out_bf16);
    // no staging area: replace this device's least recently used entry;
    // earlier launches may still read it, so the device is drained first
    size_t old = g_cache.size();
    for (size_t i = 0; i < g_cache.size(); ++i)
      if (g_cache[i].device == dev && (old == g_cache.size() || g_cache[i].stamp < g_cache[old].stamp))
        old = i;
    HA_HIP_TRY(hipDeviceSynchronize());
    HA_HIP_TRY(hipFree(g_cache[old].ptr));
    HA_HIP_TRY(hipFree(g_cache[old].ptr_bf16));
    g_cache.erase(g_cache.begin() + old);
  }
  const size_t count = size_t(heads) * r * d;
  const size_t count16 = size_t(heads) * 16 * d;
  std::vector<float> host(count ? count : 1);
  std::vector<uint16_t> host16(count16);
  fill_host(seed, heads, r, d, host.data(), host16.data());
  float* ptr = nullptr;
  uint16_t* ptr16 = nullptr;
  // (at least one element, so that r = 0 still yields a valid pointer)
  HA_HIP_TRY(hipMalloc(&ptr, (count ? count : 1) * sizeof(float)));
  hipError_t e = hipMalloc(&ptr16, count16 * sizeof(uint16_t));
  if (e == hipSuccess)
    e = hipMemcpy(ptr, host.data(), count * sizeof(float), hipMemcpyHostToDevice);
  if (e == hipSuccess)
    e = hipMemcpy(ptr16, host16.data(), count16 * sizeof(uint16_t), hipMemcpyHostToDevice);
  if (e != hipSuccess) {
    (void)hipFree(ptr);
    if (ptr16) (void)hipFree(ptr16);
    return fail(HA_ERR_HIP, "copy of hyperplanes to the device failed: %s",
                hipGetErrorString(e));
  }
  g_cache.push_back(Entry{dev, seed, heads, r, d, ptr, ptr16, ++g_clock});
  *out = ptr;
  if (out_bf16) *out_bf16 = ptr16;
  return HA_OK;
}

}  // namespace ha
