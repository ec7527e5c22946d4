/*
 * hyperattn.h — C ABI of the MI355X (gfx950) HyperAttention library.
 *
 * Source of every operation below: the Japanese article on HyperAttention at
 * nearauto.com/p/20145.html (a summary of arXiv 2310.05869), cited as
 * "HA page" with its section:
 *   "Method overview"  — Att = D^-1 A V, A = exp(QK^T), D = diag(A 1);
 *                        product sampled by the row norms of V; D estimated
 *                        with uniform column sampling.
 *   "Algorithm"        — Definition 1 (Hamming-sorted LSH), Algorithm 1
 *                        (sortLSH buckets), Algorithm 2 (ApproxD), Algorithm 3
 *                        (HyperAttention), Figure 2 / Algorithm 4 (causal
 *                        recursion into two diagonal blocks and A_21).
 *   "Monkey-patching"  — recursion to a small exact base case; b = m = 256.
 *   "Single self-attention layer" — causal mode splits Q, K, V and merges
 *                        the attention outputs.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are [heads][n][d], row-major, d contiguous, batch folded into
 *   heads. Element type is given by `dtype`: HA_F32 (float) or HA_BF16
 *   (bfloat16 bit patterns, 2 bytes). d must be 64 or 128.
 * - Scores are s_ij = <q_i, k_j> / sqrt(d). lse outputs are the natural log
 *   of the row's normaliser in these units (fp32, [heads][n]).
 * - Pointers named Q, K, V, O, lse, codes, perm, log_d and workspace are
 *   DEVICE pointers owned by the caller; the library never frees them and
 *   keeps no pointer to them after the call returns. G_host is a host pointer.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream). All
 *   device work is enqueued on it asynchronously; entry points return once
 *   the work is enqueued. The caller synchronises before reading outputs.
 * - Return value: HA_OK (0) or a negative HA_ERR_* code. Arguments are
 *   validated on the host before anything is enqueued; on error nothing is
 *   enqueued and hyperattn_last_error() describes the problem. No C++
 *   exception crosses this boundary.
 * - Results are deterministic: the same inputs, sizes and seed give
 *   bit-identical outputs (no floating-point atomics are used).
 * - Workspaces must be 256-byte aligned and at least the size the matching
 *   *_workspace_bytes function returns; their contents on entry do not matter.
 * - Written ranges (outputs and the workspace) must not overlap any input or
 *   each other; inputs may share memory (Q, K and V may be one tensor).
 *   Overlaps are refused with HA_ERR_SHAPE before anything is enqueued.
 * - n == 0 or heads == 0 is valid and enqueues nothing.
 */
#ifndef HYPERATTN_H
#define HYPERATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ha_dtype { HA_F32 = 0, HA_BF16 = 1 };

enum ha_status {
  HA_OK = 0,
  HA_ERR_NULL = -1,        /* a required pointer is NULL                     */
  HA_ERR_SHAPE = -2,       /* sizes inconsistent (see each entry point)      */
  HA_ERR_UNSUPPORTED = -3, /* d not in {64,128}, r not in [1,8], bad dtype   */
  HA_ERR_WORKSPACE = -4,   /* workspace NULL/too small/misaligned            */
  HA_ERR_HIP = -5          /* a HIP runtime call failed (message has detail) */
};

/*
 * hyperattn_forward — HyperAttention forward pass (HA page, "Algorithm",
 * Algorithms 1-3; causal: Figure 2 / Algorithm 4 with the base case of
 * "Monkey-patching" and the merge of "Single self-attention layer").
 *
 * Per head, with r Gaussian hyperplanes drawn from `seed`:
 *  1. sortLSH: hash every row of Q and K (Gray rank of the hyperplane sign
 *     pattern), then, per sub-problem, sort queries and keys stably by
 *     (code, index) and cut both into buckets of b_eff = min(b, n_k) rows.
 *  2. ApproxD: d~_i = sum over the keys in i's bucket of e^{s_ij}
 *       + (n_k/m) * sum over m uniform key samples outside i's bucket.
 *  3. Product: N_i = sum over bucket keys of e^{s_ij} V_j
 *       + sum over m V-row-norm samples j_t (p_j ∝ |V_j|^2) outside i's
 *         bucket of (1/(m p_j)) e^{s_ij} V_j;   O_i = N_i / d~_i.
 *     When m >= n_k both samples are every key of the range, weight 1.
 *  r = 0 takes a predefined mask instead of sortLSH (HA page, "Algorithm":
 *  Algorithms 2 and 3 accept any mask of the large entries): every code is 0,
 *  so the stable sort keeps index order and bucket k of a sub-problem holds
 *  its query rows and key rows [k b_eff, (k+1) b_eff), a block-diagonal local
 *  mask. Q and K are then not read for hashing.
 *  Non-causal: one sub-problem with queries and keys [0, n).
 *  Causal: while a diagonal block is larger than recursion_base, split it in
 *  halves; the lower-left block (queries of the second half, keys of the
 *  first) is a sub-problem as above; blocks of size <= recursion_base get
 *  exact causal attention; every row merges its partial results by
 *  log-sum-exp.
 *
 * Q, K, V: inputs [heads][n][d]. O: output [heads][n][d], same dtype.
 * lse: optional output [heads][n] fp32 (log d~ merged over the row's parts).
 * b >= 1 bucket size; m >= 1 samples per estimator; recursion_base >= 1
 * (ignored when causal == 0); r in [0, 8] hyperplanes (0: the local block
 * mask above); seed selects hyperplanes and samples.
 * HA_ERR_SHAPE if b_eff does not divide a sub-problem size, if a causal block
 * to be split has odd size, or if one head (n * d elements) exceeds 2 GiB.
 * workspace: >= hyperattn_workspace_bytes(...) with the same arguments.
 */
int hyperattn_forward(const void* Q, const void* K, const void* V, void* O,
                      float* lse, int64_t n, int d, int heads, int causal,
                      int b, int m, int recursion_base, int r, uint64_t seed,
                      int dtype, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * hyperattn_forward_noalloc — hyperattn_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * hosts that forbid allocation): it takes no workspace and allocates nothing.
 * Its workspace is a fixed array of hyperattn_noalloc_scratch_bytes() bytes
 * (64 MiB) in the library's device code, one per GPU, held by each GPU the
 * library runs on until the process ends; its address is looked up once per
 * device on that device's first call. Sizes whose workspace
 * (hyperattn_workspace_bytes) exceeds it are refused with HA_ERR_WORKSPACE
 * before anything is enqueued. All calls on one GPU share its array: calls
 * that overlap on one GPU (other streams or threads) race and must be
 * serialised by the caller. Arguments, outputs and other errors as
 * hyperattn_forward; the same inputs and seed give the same bytes as
 * hyperattn_forward.
 */
int hyperattn_forward_noalloc(const void* Q, const void* K, const void* V,
                              void* O, float* lse, int64_t n, int d, int heads,
                              int causal, int b, int m, int recursion_base,
                              int r, uint64_t seed, int dtype, void* stream);
size_t hyperattn_noalloc_scratch_bytes(void);

/*
 * hyperattn_forward_rope — hyperattn_forward on Q and K that still need their
 * rotary position embedding, applied on the device in the pass that hashes
 * them (the long-context layers rotate Q and K before attention, and the
 * hash must see the rotated rows: HA page, "Algorithm", Definition 1 applied
 * to the rows the attention uses).
 * Rotation: pairs (t, t + d/2) for t < d/2, row i at position i, with
 * c = cos_sin[(i * d/2 + t) * 2] and s = cos_sin[(i * d/2 + t) * 2 + 1]:
 *   x'_t = x_t c - x_{t+d/2} s,   x'_{t+d/2} = x_t s + x_{t+d/2} c,
 * in fp32 with each product and sum rounded once, then (bf16 rows) rounded
 * to the nearest bf16, ties to even.
 * cos_sin: DEVICE table owned by the caller, at least cos_sin_rows >= n rows
 * of d floats ([rows][d/2][2]); rope_table fills it on the host (theta_t =
 * rope_base^(-2t/d), angle i theta_t). Rows are positions, so one table of
 * the longest n serves every shorter call. The library only reads it.
 * Q_rot, K_rot: outputs [heads][n][d] in the input dtype, the rotated rows
 * (the attention then reads them). All other arguments, outputs and errors
 * as hyperattn_forward, with the same workspace size; HA_ERR_NULL if
 * cos_sin is NULL, HA_ERR_SHAPE if cos_sin_rows < n.
 */
int hyperattn_forward_rope(const void* Q, const void* K, const void* V,
                           const float* cos_sin, int64_t cos_sin_rows,
                           void* Q_rot, void* K_rot, void* O, float* lse,
                           int64_t n, int d, int heads, int causal, int b,
                           int m, int recursion_base, int r, uint64_t seed,
                           int dtype, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * rope_table — host-only: the cos/sin table hyperattn_forward_rope and
 * hyperattn_backward_rope read (the caller copies it to the device).
 * table_host[(i * d/2 + t) * 2 + 0] = cos(i * theta_t) and [... + 1] =
 * sin(i * theta_t), with theta_t = pow(rope_base, -2t/d), the angle, cos and
 * sin in fp64 from the C library, each entry rounded once to fp32.
 * table_host holds n * d floats. rope_base must be a finite number above 1
 * (HA_ERR_UNSUPPORTED).
 */
int rope_table(int64_t n, int d, double rope_base, float* table_host);

/* Bytes of workspace hyperattn_forward needs for these sizes (0 on invalid
 * arguments; hyperattn_last_error() then says why). */
size_t hyperattn_workspace_bytes(int64_t n, int d, int heads, int causal,
                                 int b, int m, int recursion_base, int r,
                                 int dtype);

/*
 * sortlsh_hash — the Hamming-sorted LSH of Definition 1 (HA page,
 * "Algorithm") applied to every row of X, and optionally Algorithm 1's
 * stable sort of each head's rows by (code, index).
 * codes[h][i] = GrayRank(sum_k [<x_i, g_hk> > 0] 2^k), where the sign is that
 * of the fp64 sum of x_it * g_hkt taken in order t = 0..d-1 and g_hk are the
 * hyperplanes sortlsh_hyperplanes(seed, heads, r, d) returns (drawn on the
 * device into the workspace by this call).
 * r in [0, 8]; with r = 0 every code is 0 and perm is the identity.
 * codes: output [heads][n] uint8. perm: optional output [heads][n] int32,
 * perm[h][p] = the row at sorted position p.
 * workspace: >= sortlsh_hash_workspace_bytes(n, d, heads, r, perm != NULL).
 */
int sortlsh_hash(const void* X, int64_t n, int d, int heads, int r,
                 uint64_t seed, int dtype, uint8_t* codes, int32_t* perm,
                 void* workspace, size_t workspace_bytes, void* stream);
size_t sortlsh_hash_workspace_bytes(int64_t n, int d, int heads, int r,
                                    int with_perm);

/*
 * exact_attention_forward — Att = D^-1 A V with A = exp(QK^T / sqrt(d)) and
 * D = diag(A 1) (HA page, "Method overview"); causal == 1 applies the mask
 * j <= i (Figure 2's M^C). Needs no workspace.
 * O: output [heads][n][d], same dtype; lse: optional output [heads][n].
 */
int exact_attention_forward(const void* Q, const void* K, const void* V,
                            void* O, float* lse, int64_t n, int d, int heads,
                            int causal, int dtype, void* stream);

/*
 * rowsum_estimate — Algorithm 2 (ApproxD) alone, non-causal (HA page,
 * "Algorithm"): log_d[h][i] = log d~_i with d~ as in hyperattn_forward step 2
 * (same hyperplanes, buckets and uniform samples for the same seed).
 * log_d: output [heads][n] fp32.
 * workspace: >= hyperattn_workspace_bytes(n, d, heads, 0, b, m, 1, r, dtype).
 */
int rowsum_estimate(const void* Q, const void* K, int64_t n, int d, int heads,
                    int b, int m, int r, uint64_t seed, int dtype,
                    float* log_d, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * hyperattn_backward — gradients of hyperattn_forward's output: dQ, dK, dV
 * of the loss L = sum(dO * O) for the O that hyperattn_forward returns with
 * the same arguments. The HA page times the forward and backward passes
 * together ("Single self-attention layer") but states no formula; this is
 * the exact derivative of the forward pass's estimator with its buckets,
 * sample lists and sample weights held fixed (they are piecewise constant in
 * Q, K and V). Row i's output is O_i = N_i / Z_i, where
 * N_i = sum_j w_ij e^{s_ij} V_j and Z_i = sum_j u_ij e^{s_ij} run over the
 * key slots row i evaluates. The slot weights (w, u) are:
 *   a bucket or base-case key         (1, 1)
 *   a uniform sample                  (0, n_k/m)
 *   a V-norm sample                   (its weight, 0)
 *   a sample inside the query's bucket (0, 0)
 * With E_ij = e^{s_ij - lse_i} and Delta_i = dO_i . O_i:
 *   ds_ij = E_ij (w_ij dO_i . V_j - u_ij Delta_i),
 *   dV_j += w_ij E_ij dO_i,
 *   dQ_i += ds_ij K_j / sqrt(d),
 *   dK_j += ds_ij Q_i / sqrt(d).
 * A key drawn several times counts once per draw.
 * Q, K, V, dO: inputs [heads][n][d] bf16. O and lse: hyperattn_forward's
 * outputs for these inputs and arguments (lse is required).
 * dQ, dK, dV: outputs [heads][n][d] bf16.
 * The buckets and samples are recomputed from `seed` on the device, so the
 * arguments must be those of the forward call. Accumulation is in fp32
 * (a causal level's partial gradient is rounded to bf16 once before the base
 * case adds it), and every sum runs in a fixed order with no atomics, so
 * results are deterministic.
 * bf16 only (HA_ERR_UNSUPPORTED for HA_F32), m <= 2048; other arguments and
 * errors as hyperattn_forward.
 * workspace: >= hyperattn_backward_workspace_bytes(...) with the same
 * arguments. It is larger than the forward's: it holds per-level bf16
 * partial gradients (rounded like the forward's partial outputs) and the
 * sample slots' fp32 partial gradients.
 */
int hyperattn_backward(const void* Q, const void* K, const void* V,
                       const void* O, const float* lse, const void* dO,
                       void* dQ, void* dK, void* dV, int64_t n, int d,
                       int heads, int causal, int b, int m,
                       int recursion_base, int r, uint64_t seed, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);
size_t hyperattn_backward_workspace_bytes(int64_t n, int d, int heads,
                                          int causal, int b, int m,
                                          int recursion_base, int r,
                                          int dtype);

/*
 * hyperattn_backward_rope — hyperattn_backward for a call of
 * hyperattn_forward_rope: dQ and dK are the gradients of the rows BEFORE
 * their rotary embedding. Q_rot and K_rot are the rotated rows that
 * hyperattn_forward_rope returned. The library runs hyperattn_backward on
 * them, then applies the adjoint of the rotation to the two gradients in
 * place. The rotation of each pair is orthogonal, so its adjoint rotates by
 * -i theta_t:
 *   g_t = g'_t c + g'_{t+d/2} s,   g_{t+d/2} = -g'_t s + g'_{t+d/2} c,
 * in fp32 with each product and sum rounded once, with c and s from the
 * caller's cos_sin table (as hyperattn_forward_rope), then rounded to bf16.
 * The rounding of the rotated rows to bf16 is piecewise constant and, as
 * with the sketch, carries no gradient.
 * Other arguments, outputs, workspace and errors as hyperattn_backward;
 * cos_sin and cos_sin_rows as hyperattn_forward_rope.
 */
int hyperattn_backward_rope(const void* Q_rot, const void* K_rot,
                            const void* V, const void* O, const float* lse,
                            const void* dO, const float* cos_sin,
                            int64_t cos_sin_rows, void* dQ, void* dK, void* dV,
                            int64_t n, int d, int heads, int causal, int b,
                            int m, int recursion_base, int r, uint64_t seed,
                            int dtype, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * exact_attention_backward — gradients of exact_attention_forward (HA page,
 * "Method overview"; causal: mask M^C): with P = D^-1 A and Delta_i =
 * dO_i . O_i, dV = P^T dO, dS = P (dO V^T - Delta 1^T), dQ = dS K / sqrt(d),
 * dK = dS^T Q / sqrt(d). O and lse are the forward call's outputs (lse
 * required). bf16 only. workspace: >=
 * exact_attention_backward_workspace_bytes(n, heads) bytes (Delta and the
 * work-queue counters of the persistent launches).
 */
int exact_attention_backward(const void* Q, const void* K, const void* V,
                             const void* O, const float* lse, const void* dO,
                             void* dQ, void* dK, void* dV, int64_t n, int d,
                             int heads, int causal, int dtype,
                             void* workspace, size_t workspace_bytes,
                             void* stream);
size_t exact_attention_backward_workspace_bytes(int64_t n, int heads);

/*
 * sortlsh_hyperplanes — host-only: the r Gaussian hyperplanes per head the
 * hash uses (HA page, "Algorithm", Definition 1; hash family as read here).
 * G_host[h][k][t] (fp32 holding a bf16 value) = the Box-Muller normal g that
 * sortlsh_gaussians computes from two counter-based SplitMix64 draws
 * (purpose 1, head h, node 0, counters 2e and 2e+1 with e = k*d + t), rounded
 * to fp32 and then to the nearest bf16 (ties to even). Every entry point
 * that hashes draws the same values on the device from the seed, bit for bit.
 * Touches no device. G_host must hold heads*r*d floats (r = 0: nothing is
 * written and G_host may be NULL).
 */
int sortlsh_hyperplanes(uint64_t seed, int heads, int r, int d, float* G_host);

/*
 * sortlsh_gaussians — host-only: out[i] = the binary64 Box-Muller normal of
 * the draws a[i] and b[i], before any rounding:
 *   g = sqrt(-2 ln u1) cos(2 pi u2), u1 = ((a >> 11) + 1) 2^-53,
 *   u2 = (b >> 11) 2^-53,
 * with ln, sqrt and cos evaluated by fixed series and Newton steps in
 * correctly rounded binary64 additions, subtractions, multiplications and
 * divisions only (no fused multiply-add, no library function), so that every
 * IEEE-754 platform, the GPU included, computes the same bits:
 *   ln u:   u = f 2^e, f in [1,2); if f > sqrt 2: f = f/2, e = e+1;
 *           s = (f-1)/(f+1), z = s s, p = Horner in z of 1/(2k+1) for
 *           k = 11..0, ln u = e ln2 + (2s) p;
 *   sqrt y: y = m 2^e, m in [1,2); if e odd: m = 2m, e = e-1;
 *           x = (1+m)/2, then x = (x + m/x)/2 six times; result x 2^(e/2)
 *           (y <= 0 gives 0);
 *   cos 2 pi u, u = B 2^-53: q = (B + 2^50) >> 51, r = (B - q 2^51) 2^-51,
 *           theta = r (pi/2), t = theta^2, C = Horner in t of (-1)^k/(2k)!
 *           for k = 9..0, S = theta times Horner in t of (-1)^k/(2k+1)! for
 *           k = 8..0; result C, -S, -C, S for q mod 4 = 0, 1, 2, 3.
 * Constants are the binary64 values nearest to ln 2, sqrt 2, pi/2 and the
 * coefficients. a, b and out are host arrays of count elements.
 */
int sortlsh_gaussians(const uint64_t* a, const uint64_t* b, int64_t count,
                      double* out);

/*
 * hyperattn_workspace_layout — where hyperattn_forward keeps its
 * intermediate results inside the workspace (for inspection after a call:
 * hash codes, sorts and sample lists). Fills offsets[i] and bytes[i] for
 * i < HA_WS_COUNT (bytes 0 for a region the call does not use).
 * Returns HA_OK or an error as hyperattn_workspace_bytes would.
 *
 * Region contents (L = number of levels: 1 if non-causal, else the number
 * of halvings; S = n if non-causal, else n/2; node ids run 1 .. 2^L-1;
 * regions not listed are scratch):
 *   HA_WS_CODES_Q, HA_WS_CODES_K  uint8 [heads][n]
 *   HA_WS_VNORM_W                 uint64 [heads][n]   integer weights W_j
 *   HA_WS_VNORM_P                 uint64 [heads][n+1] exclusive prefix of W
 *   HA_WS_PERM_Q, HA_WS_PERM_K    int32 [L][heads][S] global row at each sorted
 *                                 position; level l's segments of size
 *                                 h = n >> (l+1) (n if non-causal) are stored
 *                                 one after another
 *   HA_WS_RANK_K                  int32 [L][heads][S] sorted position (within
 *                                 its segment) of each key slot
 *   HA_WS_U_IDX, HA_WS_U_BKT      int32 [heads][nodes][m] uniform samples and
 *                                 the key bucket of each
 *   HA_WS_V_IDX, HA_WS_V_BKT      int32 [heads][nodes][m] V-norm samples, bucket
 *   HA_WS_V_W                     float [heads][nodes][m] V-norm sample weights
 *   HA_WS_NODE_META               int32 [heads][nodes][4]: uniform count,
 *                                 V-norm count, alpha (float bits), b_eff
 *   HA_WS_SCHED                   uint32 [2][8] work-queue counters of the
 *                                 attention kernels (scratch, reset by each call)
 *   HA_WS_PLANES                  the call's hyperplanes, drawn on the device
 *                                 from the seed: fp32 [heads][r][d], then at
 *                                 the next 256-byte boundary bf16
 *                                 [heads][16][d] (rows r..15 zero)
 *   HA_WS_DELTA ... HA_WS_SLOT_DV backward pass only (hyperattn_backward's
 *                                 workspace; bytes 0 in the forward layout):
 *                                 HA_WS_DELTA float [heads][n] = dO_i . O_i
 */
enum ha_ws_region {
  HA_WS_CODES_Q = 0, HA_WS_CODES_K,
  HA_WS_VNORM_A, HA_WS_VNORM_W, HA_WS_VNORM_P, HA_WS_VNORM_BLK,
  HA_WS_PERM_Q, HA_WS_PERM_K, HA_WS_RANK_K,
  HA_WS_SORT_HIST,
  HA_WS_U_IDX, HA_WS_U_BKT, HA_WS_V_IDX, HA_WS_V_BKT, HA_WS_V_W,
  HA_WS_NODE_META,
  HA_WS_PART_O, HA_WS_PART_LSE,
  HA_WS_SCHED, HA_WS_PLANES,
  HA_WS_DELTA, HA_WS_PART_DQ, HA_WS_PART_DK, HA_WS_PART_DV,
  HA_WS_SLOT_FIRST, HA_WS_SLOT_NEXT, HA_WS_SLOT_DK, HA_WS_SLOT_DV,
  HA_WS_COUNT
};
int hyperattn_workspace_layout(int64_t n, int d, int heads, int causal, int b,
                               int m, int recursion_base, int r, int dtype,
                               int64_t* offsets, int64_t* bytes);

/*
 * hyperattn_debug_artifacts — the intermediate results of hyperattn_forward
 * with the same arguments, copied to host memory for inspection: the sortLSH
 * codes (Definition 1), the V-norm weights and prefix sums, every level's
 * sorted order of queries and keys (Algorithm 1), and every node's uniform
 * and V-norm sample lists with their key buckets and weights (Algorithms 2
 * and 3) (HA page, "Algorithm"). It runs the forward pass's front end (the
 * hyperplanes, hash, V norms, sort and samples) on `stream` into the
 * workspace, copies each requested region, and waits for `stream` before it
 * returns (a debugging call; nothing else is waited for). No attention is
 * computed.
 * Every field of `out` is a HOST pointer or NULL (region not copied); each
 * must hold the bytes hyperattn_workspace_layout reports for its region, in
 * the layout described there. A causal call with n <= recursion_base (one
 * exact block) has no sub-problems: only the codes, W and P are produced.
 * Arguments, workspace and errors as hyperattn_forward (Q, K, V, dtype and
 * workspace size); workspace: >= hyperattn_workspace_bytes(...).
 */
typedef struct ha_artifacts {
  uint8_t* codes_q;    /* HA_WS_CODES_Q  uint8  [heads][n]            */
  uint8_t* codes_k;    /* HA_WS_CODES_K  uint8  [heads][n]            */
  uint64_t* vnorm_w;   /* HA_WS_VNORM_W  uint64 [heads][n]            */
  uint64_t* vnorm_p;   /* HA_WS_VNORM_P  uint64 [heads][n+1]          */
  int32_t* perm_q;     /* HA_WS_PERM_Q   int32  [L][heads][S]         */
  int32_t* perm_k;     /* HA_WS_PERM_K   int32  [L][heads][S]         */
  int32_t* rank_k;     /* HA_WS_RANK_K   int32  [L][heads][S]         */
  int32_t* u_idx;      /* HA_WS_U_IDX    int32  [heads][nodes][m]     */
  int32_t* u_bkt;      /* HA_WS_U_BKT    int32  [heads][nodes][m]     */
  int32_t* v_idx;      /* HA_WS_V_IDX    int32  [heads][nodes][m]     */
  int32_t* v_bkt;      /* HA_WS_V_BKT    int32  [heads][nodes][m]     */
  float* v_w;          /* HA_WS_V_W      float  [heads][nodes][m]     */
  int32_t* node_meta;  /* HA_WS_NODE_META int32 [heads][nodes][4]     */
} ha_artifacts;
int hyperattn_debug_artifacts(const void* Q, const void* K, const void* V,
                              int64_t n, int d, int heads, int causal, int b,
                              int m, int recursion_base, int r, uint64_t seed,
                              int dtype, void* workspace,
                              size_t workspace_bytes, void* stream,
                              const ha_artifacts* out);

/* Message for the last error on the calling thread ("" if none); valid until
 * the next call into the library on this thread. */
const char* hyperattn_last_error(void);

/*
 * Kernel timing for measurement. When enabled, every kernel the library
 * launches is bracketed by two hipEvents recorded on the launch stream.
 * hyperattn_profile_collect() waits for all recorded events, adds their
 * durations to per-kernel totals and recycles them. Totals persist until
 * hyperattn_profile_reset(). Not meant to be used from several threads.
 */
int hyperattn_profile_enable(int on);
int hyperattn_profile_collect(void);
int hyperattn_profile_reset(void);
int hyperattn_profile_count(void);                 /* number of kernel names */
const char* hyperattn_profile_name(int i);
int64_t hyperattn_profile_launches(int i);
/* work-groups launched under name i, summed over its launches (persistent
 * launches: the resident work-groups the occupancy query gave) */
int64_t hyperattn_profile_groups(int i);
double hyperattn_profile_total_ms(int i);

#ifdef __cplusplus
}
#endif

#endif /* HYPERATTN_H */
