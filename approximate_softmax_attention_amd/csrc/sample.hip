// The two sample lists of every sub-problem (node).
//
// HA page, "Algorithm": ApproxD (Algorithm 2) adds a randomly chosen subset of
// the columns of A to the entries under the sortLSH mask; "Method overview"
// and "Algorithm": the product with V is estimated by sampling rows of V by
// their squared l2 norms. Readings taken: m draws with replacement per list,
// shared by every query of the node.
//   uniform: l_t = lo + floor(u_t n_k / 2^32), u_t = top 32 bits of
//            draw(purpose 2, head, node, t); each weighs n_k / m.
//   V-norm:  U_t = floor(R_t T / 2^64), R_t = draw(purpose 3, head, node, t),
//            T = P[lo + n_k] - P[lo]; j_t = least j with P[j+1] - P[lo] > U_t
//            (binary search on the integer prefix sums P); weight
//            T / (m W_j) computed in fp64 and rounded to fp32.
//   m >= n_k: every key of the range once, weight 1. T = 0: no V samples.
// Each entry also records the sortLSH bucket of its key in this node, so the
// attention kernel can drop samples that fall inside the query's bucket.
#include "common.h"
#include "device_util.h"

namespace ha {

namespace {

constexpr int kThreads = 256;

struct SampleArgs {
  LevelTable table;
  int heads, m;
  int64_t n, S, nodes;
  uint64_t key;                 // mix64(seed)
  const int32_t* rank_k;        // [L][heads][S]
  const uint64_t* P;            // [heads][n+1] or null (no V list)
  int32_t *u_idx, *u_bkt, *v_idx, *v_bkt;
  float* v_w;
  int32_t* meta;                // [heads][nodes][4]
};

// grid: (nodes, heads)
__global__ __launch_bounds__(kThreads) void samples_kernel(SampleArgs a) {
  const int64_t node = int64_t(blockIdx.x) + 1;
  const int head = blockIdx.y;
  const int lv = 63 - __clzll(node);
  const int64_t seg = node - (int64_t(1) << lv);
  const Level& L = a.table.lv[lv];
  const int64_t h = L.h;
  const int64_t lo = a.table.causal ? 2 * seg * h : 0;
  const int32_t* rank = a.rank_k + (int64_t(lv) * a.heads + head) * a.S + seg * h;
  const int64_t rec = int64_t(head) * a.nodes + (node - 1);
  int32_t* uidx = a.u_idx + rec * a.m;
  int32_t* ubkt = a.u_bkt + rec * a.m;
  const int b_eff = L.b_eff;
  const bool exhaustive = int64_t(a.m) >= h;

  const int ucount = exhaustive ? int(h) : a.m;
  for (int t = threadIdx.x; t < ucount; t += kThreads) {
    int64_t j;
    if (exhaustive) {
      j = t;
    } else {
      const uint64_t u = draw(a.key, 2, head, node, t) >> 32;
      j = int64_t((u * uint64_t(h)) >> 32);
    }
    uidx[t] = int32_t(lo + j);
    ubkt[t] = rank[j] / b_eff;
  }

  int vcount = 0;
  if (a.P) {
    const uint64_t* P = a.P + int64_t(head) * (a.n + 1);
    const uint64_t base = P[lo];
    const uint64_t T = P[lo + h] - base;
    vcount = exhaustive ? int(h) : (T == 0 ? 0 : a.m);
    int32_t* vidx = a.v_idx + rec * a.m;
    int32_t* vbkt = a.v_bkt + rec * a.m;
    float* vw = a.v_w + rec * a.m;
    for (int t = threadIdx.x; t < vcount; t += kThreads) {
      int64_t j;
      float w;
      if (exhaustive) {
        j = t;
        w = 1.f;
      } else {
        const uint64_t R = draw(a.key, 3, head, node, t);
        const uint64_t U = __umul64hi(R, T);
        int64_t lo_j = 0, hi_j = h - 1;     // answer in [0, h-1]
        while (lo_j < hi_j) {
          const int64_t mid = (lo_j + hi_j) >> 1;
          if (P[lo + mid + 1] - base > U) hi_j = mid;
          else lo_j = mid + 1;
        }
        j = lo_j;
        const uint64_t Wj = P[lo + j + 1] - P[lo + j];
        w = float(double(T) / (double(a.m) * double(Wj)));
      }
      vidx[t] = int32_t(lo + j);
      vbkt[t] = rank[j] / b_eff;
      vw[t] = w;
    }
  }
  if (threadIdx.x == 0) {
    int32_t* mt = a.meta + rec * 4;
    mt[0] = ucount;
    mt[1] = vcount;
    const float alpha = exhaustive ? 1.f : float(double(h) / double(a.m));
    mt[2] = __float_as_int(alpha);
    mt[3] = b_eff;
  }
}


}  // namespace

int launch_samples(const Plan& p, uint64_t seed, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  SampleArgs a;
  a.table = p.table;
  a.heads = p.heads;
  a.m = p.m;
  a.n = p.n;
  a.S = p.S;
  a.nodes = p.nodes;
  a.key = mix64(seed);
  a.rank_k = reinterpret_cast<const int32_t*>(w + p.off[HA_WS_RANK_K]);
  a.P = p.product ? reinterpret_cast<const uint64_t*>(w + p.off[HA_WS_VNORM_P]) : nullptr;
  a.u_idx = reinterpret_cast<int32_t*>(w + p.off[HA_WS_U_IDX]);
  a.u_bkt = reinterpret_cast<int32_t*>(w + p.off[HA_WS_U_BKT]);
  a.v_idx = p.product ? reinterpret_cast<int32_t*>(w + p.off[HA_WS_V_IDX]) : nullptr;
  a.v_bkt = p.product ? reinterpret_cast<int32_t*>(w + p.off[HA_WS_V_BKT]) : nullptr;
  a.v_w = p.product ? reinterpret_cast<float*>(w + p.off[HA_WS_V_W]) : nullptr;
  a.meta = reinterpret_cast<int32_t*>(w + p.off[HA_WS_NODE_META]);
  ProfRange pr("samples", s);
  hipLaunchKernelGGL(samples_kernel, dim3(unsigned(p.nodes), unsigned(p.heads)),
                     dim3(kThreads), 0, s, a);
  HA_LAUNCH_CHECK("samples");
  return HA_OK;
}

}  // namespace ha
