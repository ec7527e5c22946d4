// Host-side planning: argument validation, the flattened causal recursion
// (HA page, "Algorithm", Figure 2 / Algorithm 4: a block larger than the base
// size splits into two diagonal halves plus the lower-left block A_21), and
// the carve-up of the caller's workspace into regions.
#include <cstdarg>
#include <cstdio>

#include "common.h"

namespace ha {

namespace {

int64_t add_region(Plan& p, int id, int64_t bytes) {
  p.off[id] = static_cast<int64_t>(p.total);
  p.bytes[id] = bytes;
  p.total += static_cast<size_t>(align256(bytes));
  return p.off[id];
}

}  // namespace

int make_plan(Plan& p, int64_t n, int d, int heads, int causal, int b, int m,
              int base, int r, int dtype, bool product, bool backward) {
  p = Plan();
  if (dtype != HA_F32 && dtype != HA_BF16)
    return fail(HA_ERR_UNSUPPORTED, "dtype %d is not HA_F32 (0) or HA_BF16 (1)", dtype);
  if (d != 64 && d != 128)
    return fail(HA_ERR_UNSUPPORTED, "head dimension d=%d not supported (64 or 128)", d);
  if (r < 0 || r > 8)
    return fail(HA_ERR_UNSUPPORTED, "r=%d hyperplanes not supported (0..8)", r);
  if (n < 0 || n >= (int64_t(1) << 31))
    return fail(HA_ERR_SHAPE, "n=%lld out of range [0, 2^31)", (long long)n);
  if (heads < 0 || heads >= (1 << 16))
    return fail(HA_ERR_SHAPE, "heads=%d out of range [0, 65536)", heads);
  if (n * d * (dtype == HA_BF16 ? 2 : 4) >= (int64_t(1) << 31))
    return fail(HA_ERR_SHAPE, "one head of n=%lld rows exceeds 2 GiB", (long long)n);
  if (b < 1) return fail(HA_ERR_SHAPE, "bucket size b=%d must be >= 1", b);
  if (m < 1 || m >= (1 << 24))
    return fail(HA_ERR_SHAPE, "sample count m=%d out of range [1, 2^24)", m);
  if (causal && base < 1)
    return fail(HA_ERR_SHAPE, "recursion_base=%d must be >= 1", base);
  if (backward && dtype != HA_BF16)
    return fail(HA_ERR_UNSUPPORTED, "the backward pass takes bf16 tensors only");
  if (backward && m > kBwdMaxM)
    return fail(HA_ERR_UNSUPPORTED, "the backward pass takes m <= %d (m=%d)", kBwdMaxM, m);

  p.n = n; p.d = d; p.heads = heads; p.causal = causal ? 1 : 0; p.b = b; p.m = m;
  p.base = base; p.r = r; p.dtype = dtype; p.product = product; p.backward = backward;
  p.esize = dtype == HA_BF16 ? 2 : 4;
  if (n == 0 || heads == 0) return HA_OK;

  if (p.causal) {
    int64_t size = n;
    int L = 0;
    while (size > base) {
      if (size % 2)
        return fail(HA_ERR_SHAPE,
                    "causal recursion: block of odd size %lld (> recursion_base=%d) "
                    "cannot be halved", (long long)size, base);
      size /= 2;
      ++L;
    }
    if (L > 20)
      return fail(HA_ERR_SHAPE, "causal recursion needs %d levels (at most 20)", L);
    p.L = L;
    p.base_block = size;
    p.S = L ? n / 2 : 0;
    p.nodes = (int64_t(1) << L) - 1;
  } else {
    p.L = 1;
    p.S = n;
    p.nodes = 1;
  }
  LevelTable& t = p.table;
  t.count = p.L;
  t.causal = p.causal;
  t.n = n;
  for (int l = 0; l < p.L; ++l) {
    Level& v = t.lv[l];
    v.h = p.causal ? (n >> (l + 1)) : n;
    v.nseg = p.causal ? (int64_t(1) << l) : 1;
    v.b_eff = static_cast<int>(v.h < b ? v.h : b);
    if (v.h % v.b_eff)
      return fail(HA_ERR_SHAPE,
                  "bucket size %d does not divide the sub-problem size %lld (level %d)",
                  v.b_eff, (long long)v.h, l);
    v.nbucket = v.h / v.b_eff;
    v.sort_cps = ceil_div(v.h, kSortChunk);
    v.sort_wg0 = p.sort_wgs;
    p.sort_wgs += int64_t(heads) * 2 * v.nseg * v.sort_cps;
    v.att_qch = ceil_div(v.b_eff, kAttnQ);
    const bool exhaustive = int64_t(m) >= v.h;
    v.u_cnt = exhaustive ? static_cast<int>(v.h) : m;
    v.v_cap = v.u_cnt;
    v.alpha = exhaustive ? 1.f : static_cast<float>(double(v.h) / double(m));
    v.att_wg0 = p.att_wgs;
    p.att_wgs += int64_t(heads) * v.nseg * v.nbucket * v.att_qch;
    v.smp_nsc = static_cast<int>(ceil_div(v.u_cnt + v.v_cap, kAttnQ));
    v.smp_nqc = ceil_div(v.h, kBwdQChunk);
    v.smp_wg0 = p.smp_wgs;
    p.smp_wgs += int64_t(heads) * v.nseg * v.smp_nsc * v.smp_nqc;
  }
  p.vblocks = ceil_div(n, kVnormBlock);

  const int64_t H = heads;
  const int64_t slots = int64_t(p.L) * H * p.S;
  add_region(p, HA_WS_CODES_Q, H * n);
  add_region(p, HA_WS_CODES_K, H * n);
  if (product) {
    add_region(p, HA_WS_VNORM_A, H * n * 8);
    add_region(p, HA_WS_VNORM_W, H * n * 8);
    add_region(p, HA_WS_VNORM_P, H * (n + 1) * 8);
    add_region(p, HA_WS_VNORM_BLK, H * p.vblocks * 16);
  }
  add_region(p, HA_WS_PERM_Q, slots * 4);
  add_region(p, HA_WS_PERM_K, slots * 4);
  add_region(p, HA_WS_RANK_K, slots * 4);
  add_region(p, HA_WS_SORT_HIST, p.sort_wgs * kSortBins * 4);
  const int64_t samples = H * p.nodes * m;
  add_region(p, HA_WS_U_IDX, samples * 4);
  add_region(p, HA_WS_U_BKT, samples * 4);
  if (product) {
    add_region(p, HA_WS_V_IDX, samples * 4);
    add_region(p, HA_WS_V_BKT, samples * 4);
    add_region(p, HA_WS_V_W, samples * 4);
  }
  add_region(p, HA_WS_NODE_META, H * p.nodes * 16);
  if (product && p.causal && p.L > 0 && !backward) {
    add_region(p, HA_WS_PART_O, slots * d * p.esize);
    add_region(p, HA_WS_PART_LSE, slots * 4);
  }
  add_region(p, HA_WS_SCHED, 2 * kQueues * 4);
  add_region(p, HA_WS_PLANES, hyperplane_stage_bytes(heads, r, d));
  if (backward) {
    add_region(p, HA_WS_DELTA, H * n * 4);
    if (p.causal && p.L > 0) {
      add_region(p, HA_WS_PART_DQ, slots * d * 2);
      add_region(p, HA_WS_PART_DK, slots * d * 2);
      add_region(p, HA_WS_PART_DV, slots * d * 2);
    }
    add_region(p, HA_WS_SLOT_FIRST, slots * 4);
    add_region(p, HA_WS_SLOT_NEXT, H * p.nodes * 2 * m * 4);
    add_region(p, HA_WS_SLOT_DK, p.smp_wgs * kAttnQ * d * 4);
    add_region(p, HA_WS_SLOT_DV, p.smp_wgs * kAttnQ * d * 4);
  }
  return HA_OK;
}

int check_workspace(const Plan& p, const void* ws, size_t ws_bytes) {
  if (p.total == 0) return HA_OK;
  if (!ws) return fail(HA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", p.total);
  if (reinterpret_cast<uintptr_t>(ws) % 256)
    return fail(HA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < p.total)
    return fail(HA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, p.total);
  return HA_OK;
}

}  // namespace ha
