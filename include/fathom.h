/*
 * fathom.h — C ABI of the MI355X (gfx950) Fathom key scan.
 *
 * The method: "Fathom: Per-Query Read Depth for Sparse Decoding over
 * Offloaded KV Caches" (papers.paperslantern.ai/papers/2609.17652, abstract
 * and §3.2–§3.3; restated with its equations in the jaehun.me review of the
 * same paper, "Bit-Plane K Cache", "Per-Query Read Depth" and the
 * Appendix A walkthrough).  A decode step ranks every cached key before a
 * top-k sparse attention step:
 *
 *   fathom_encode : fp16 K  -> 4 bit planes + fp16 block scales    (§3.2)
 *   fathom_plan   : q group, channel variances, bit budget -> depths (§3.3, Eq. 4)
 *   fathom_scan   : planes, depths, q group -> approximate scores   (§3.3, §7)
 *   fathom_topk   : scores, k -> top-k key indices per query head   (§2)
 *
 * and around them: fathom_plan_fixed (the fixed-depth reads the pages
 * compare against, §2 and §5), fathom_scan_topk (scan and selection in one
 * call), fathom_gather (the runs a plan reads, from a host-resident store,
 * §3.6) and fathom_klt_* (the rotated store of §3.5).
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer owned by the caller, except the
 *     host store of fathom_gather (pinned host memory).  The library
 *     allocates nothing, keeps no pointer after a call returns and holds no
 *     state between calls, apart from the fixed per-GPU scratch of
 *     fathom_topk_noalloc (and its looked-up device address), the host-side
 *     call counters that tag the messages between workgroups of one launch
 *     (fathom_topk, fathom_scan_topk) and the settings of
 *     fathom_test_cut_hooks.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously on it; no call synchronises the host
 *     with the device.  Calls are reentrant; calls on different streams are
 *     independent.
 *   - All arrays are dense, row-major, with the layouts stated per call.
 *   - d (channels per KV head) must be 128; G (query heads per KV head) must
 *     be in [1, 8]; token counts must be positive multiples of 64 and below
 *     2^31; "groups" is the number of KV heads in the call (KV heads x layers
 *     x sessions, all with the same n).
 *   - Arguments are checked on the host before any HIP call; a failed check
 *     returns an error status and enqueues nothing.  Pointers must be
 *     aligned to their element size, k to 16 bytes and the top-k workspace
 *     to 256 bytes.  groups (and top-k rows) must be at most 65535.
 *   - Return value: FATHOM_OK (0) or a negative status below;
 *     fathom_status_string() names it.
 */
#ifndef FATHOM_H_
#define FATHOM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FATHOM_ABI_VERSION 9   /* 2: fathom_plan_fixed; 3: fathom_scan_topk; 4: fathom_gather;
                                  5: fathom_klt_*; 6: fathom_scan_timed;
                                  7: fathom_topk_noalloc; 8: fathom_test_cut_hooks;
                                  9: fathom_append_plan */

enum fathom_status {
  FATHOM_OK = 0,
  FATHOM_ERR_NULL_ARG = -1,        /* a required pointer is NULL            */
  FATHOM_ERR_BAD_SHAPE = -2,       /* d, G, n, groups or strides invalid    */
  FATHOM_ERR_BAD_RANGE = -3,       /* k, budget or plan parameter invalid   */
  FATHOM_ERR_WORKSPACE = -4,       /* workspace smaller than required       */
  FATHOM_ERR_HIP = -5,             /* a HIP launch or runtime call failed   */
  FATHOM_ERR_NO_DEVICE = -6,       /* no HIP device is visible              */
  FATHOM_ERR_ALIGNMENT = -7,       /* a pointer lacks its required alignment */
  FATHOM_ERR_NOT_PINNED = -8,      /* host memory the device cannot address  */
  FATHOM_ERR_TOO_LARGE = -9        /* beyond the fixed no-allocation scratch */
};

/* Number of bit planes per channel and tokens per block (fixed by §3.2). */
#define FATHOM_PLANES 4
#define FATHOM_BLOCK 64

/*
 * fathom_encode — quantize fp16 keys into the channel-major bit-plane store.
 *
 * Defined by §3.2 "Bit-Plane K Cache" (both pages): per channel j and 64-token
 * block b, a = max_i |k_ij| over the block, cell width s = a/8, 4-bit code
 * c = clamp(floor(k/s) + 8, 0, 15) (code 8 is zero, the MSB is the sign;
 * floor is fixed by the Appendix A codes).  Bit p of the codes (p = 0 is the
 * MSB) of the 64 tokens is packed into one 64-bit word, token i of the block
 * in bit i.  An all-zero block stores a = 0 and codes 8.
 *
 *   k      [groups][n][d]          fp16 bit patterns (input)
 *   planes [groups][d][4][nb_store] uint64 (output) — for fixed (group, j) the
 *          first t planes over all blocks are one contiguous run (§3.6)
 *   scales [groups][d][nb_store]   fp16 bit pattern of a (output)
 *
 * The n/64 blocks of `k` are written to block slots
 * [block_offset, block_offset + n/64) of a store holding nb_store blocks per
 * channel, so a decode loop can append one block at a time.  Requires
 * block_offset >= 0 and block_offset + n/64 <= nb_store.
 *
 * nonfinite_flag (nullable, device uint32): if any input element of a block is
 * Inf or NaN the kernel ORs 1 into *nonfinite_flag; that block's output is
 * unspecified.  The flag is never cleared by the library.
 */
int fathom_encode(const uint16_t* k, int64_t groups, int64_t n, int32_t d,
                  int64_t nb_store, int64_t block_offset, uint64_t* planes,
                  uint16_t* scales, uint32_t* nonfinite_flag, void* stream);

/*
 * fathom_plan — per query group read depths by integer reverse water-filling.
 *
 * Defined by §3.3 "Per-Query Read Depth" (Eq. 4) and the Appendix A
 * walkthrough: importance g_j = (sum_h q_hj^2) * Var_j (fp64), depth
 * t_j = clip(round(log4(g_j/theta)), 0, 4) with halves rounded up, i.e.
 * t_j = #{m in 1..4 : g_j >= 2^(2m-1) * theta} (0 when g_j = 0).  theta is
 * found by 30 steps of log-bisection (geometric midpoints) for the smallest
 * theta with sum_j t_j <= budget_bits, bracket [min_{g>0} g / 256, max g];
 * the depths at the feasible end are returned.  Special cases without
 * bisection: budget >= 4 * #{g_j > 0} gives t_j = 4 on every g_j > 0
 * (theta = min_{g>0} g / 256); max g = 0 or budget 0 gives all zeros
 * (theta = max g).  The plan is shared by the G heads of the group.
 *
 *   q         [groups][G][d] fp32  query heads of each KV head (finite)
 *   var       [groups][d]    fp32  per-channel key variance (>= 0, finite)
 *   depths    [groups][d]    uint8 output, values 0..4
 *   theta     [groups]       fp64  output water line (nullable)
 *   bits_used [groups]       int32 output sum_j t_j (nullable)
 *   0 <= budget_bits <= 4*d.
 */
int fathom_plan(const float* q, const float* var, int64_t groups, int32_t G,
                int32_t d, int32_t budget_bits, uint8_t* depths, double* theta,
                int32_t* bits_used, void* stream);

/*
 * fathom_append_plan — a decode step's store append (§3.2) and plan (§3.3,
 * Eq. 4) in one call: exactly fathom_encode(k, groups, n, d, nb_store,
 * block_offset, planes, scales, nonfinite_flag) and then fathom_plan(q, var,
 * groups, G, d, budget_bits, depths, theta, bits_used), the same outputs bit
 * for bit.  The two read and write disjoint data, so when the append is at
 * most 64 blocks per group (n <= 4096, the decode-time append) they run as
 * one launch, the plan's groups first; longer appends run as the two
 * launches.  Arguments, layouts and errors are those of the two calls (a
 * failed check of either returns before anything is enqueued); q, var and
 * depths must not overlap k, planes or scales.
 */
int fathom_append_plan(const uint16_t* k, int64_t groups, int64_t n, int32_t d,
                       int64_t nb_store, int64_t block_offset, uint64_t* planes,
                       uint16_t* scales, uint32_t* nonfinite_flag, const float* q,
                       const float* var, int32_t G, int32_t budget_bits, uint8_t* depths,
                       double* theta, int32_t* bits_used, void* stream);

/*
 * fathom_plan_fixed — fixed-depth plans, the pages' comparison points read
 * through the same store and fathom_scan.
 *
 * The 2-bit thumbnail baseline of §2 reads every channel at two planes (288
 * bits per token with the scales); SparQ (§2) keeps, per query, the channels
 * with the largest |q_j|, summed over the query heads that share a KV head,
 * here at 4 bits (r = 16 and 32 give the 68- and 136-bit scans of Table 1);
 * Double Sparsity (§2) keeps a fixed set chosen offline from a calibration
 * statistic.
 *
 *   mode FATHOM_PLAN_UNIFORM: t_j = param for every channel, 0 <= param <= 4.
 *   mode FATHOM_PLAN_SPARQ:   s_j = sum_h |q_hj| (fp64, heads in order);
 *                             t_j = 4 on the param channels with the largest
 *                             s_j, 0 elsewhere, 0 <= param <= d.
 *   mode FATHOM_PLAN_TOPSTAT: the same with s_j = stat[group][j] (fp32).
 * Ties in s_j go to the lower channel index.
 *
 *   q     [groups][G][d] fp32 (read by SPARQ; finite), may be null otherwise
 *   stat  [groups][d]    fp32 (read by TOPSTAT; finite), may be null otherwise
 *   depths [groups][d]   uint8 output
 */
#define FATHOM_PLAN_UNIFORM 1
#define FATHOM_PLAN_SPARQ 2
#define FATHOM_PLAN_TOPSTAT 3
int fathom_plan_fixed(const float* q, const float* stat, int64_t groups, int32_t G, int32_t d,
                      int32_t mode, int32_t param, uint8_t* depths, void* stream);

/*
 * fathom_scan — approximate scores from the prefix planes the depths select.
 *
 * Defined by §3.2 (reading the first t planes gives c' = c >> (4-t), value
 * (c' + 0.5 - 2^(t-1)) * a / 2^(t-1), the t-bit mid-rise quantizer) and §3.3
 * (channels with t_j = 0 are skipped; one plan per group, read once for all
 * G heads).  Score of token i for head h:
 *     S_hi = sum_{j : t_j > 0} q_hj * khat_ij.
 * Only the planes p < t_j of active channels and their scales are read.
 *
 * fp32 evaluation order (fixed so results are reproducible bit for bit):
 *   U_hi = +0; for each active j: U_hi = fma(w_hj, m_ij, U_hi),
 *          w_hj = q_hj * 2^(11 - t_j), m_ij = a_bj * c'_ij * 2^-10 (both exact);
 *   o_hb = +0; for each active j: o_hb = fma(e_hj, a_bj, o_hb),
 *          e_hj = fl32(q_hj * (2^-t_j - 1));
 *   S_hi = fl32(U_hi + o_hb),
 * where "each active j" takes the channels of depth 4 first, then 3, 2 and
 * 1, ascending j within a depth.  Depth values above 4 read as 4.
 *
 *   planes, scales as written by fathom_encode with nb_store blocks/channel
 *   (scales must be 4-byte aligned here); blocks [0, n/64) are scanned.
 *   depths [groups][d] uint8 (0..4), q [groups][G][d] fp32,
 *   scores [groups][G][n] fp32 output.
 *
 * Any capacity and alignment the arguments allow take the same kernels:
 * whole runs of 2048 keys in the main kernel, the blocks after the last
 * whole run in a small tail kernel.  Scale rows load as 16-byte vectors
 * when nb_store is a multiple of 8 and scales is 16-byte aligned, else one
 * 2-byte load per block (a few loads more per workgroup; no other
 * difference).  Only a group whose plane array exceeds 4 GiB (nb_store
 * beyond 2^20 - 1, i.e. 67M keys) is scanned by the tail kernel alone.
 */
int fathom_scan(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                const uint8_t* depths, const float* q, int64_t groups, int32_t G,
                int32_t d, int64_t n, float* scores, void* stream);

/*
 * fathom_scan_timed — fathom_scan, the same work and results, with the time
 * its kernels take recorded in two caller-created HIP events (hipEvent_t
 * passed as void*, both non-null): start_event takes the start timestamp of
 * the scan's first kernel and stop_event the end timestamp of its last, from
 * the kernels' own dispatches, so no marker packet is added to the stream
 * between the scan and the work around it (the HIP runtime still ends a
 * timed dispatch with a system-scope release, a few microseconds of idle
 * GPU around the scan).  hipEventElapsedTime(start, stop) then gives the
 * scan's duration once stop_event has completed.  For callers that time the
 * scan inside a pipeline (the benchmark's roofline).  Errors as fathom_scan;
 * a null event is FATHOM_ERR_NULL_ARG.
 */
int fathom_scan_timed(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                      const uint8_t* depths, const float* q, int64_t groups, int32_t G,
                      int32_t d, int64_t n, float* scores, void* start_event, void* stop_event,
                      void* stream);

/*
 * fathom_topk — the k highest scores of every row (per query head, §2).
 *
 * Order: score descending, ties broken by the lower index; -0 equals +0.
 * Output: the selected indices of each row in ascending index order.
 * Scores must be finite.
 *
 *   scores  [rows][n] fp32 (rows = groups * G for fathom_scan output)
 *   indices [rows][k] int32 output
 *   workspace: device scratch of at least fathom_topk_workspace_bytes(rows,
 *   n, k) bytes, 256-byte aligned; its contents on entry do not matter.
 *   1 <= k <= n, n < 2^31 (any n, not only multiples of 64).
 */
size_t fathom_topk_workspace_bytes(int64_t rows, int64_t n, int32_t k);
int fathom_topk(const float* scores, int64_t rows, int64_t n, int32_t k,
                int32_t* indices, void* workspace, size_t workspace_bytes,
                void* stream);

/*
 * fathom_topk_noalloc — fathom_topk for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same selection, bit for bit, with the workspace
 * taken from a fixed scratch array the library holds in device memory, one
 * per GPU it runs on, until the process ends.  The call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).
 *
 *   scores, rows, n, k, indices, stream: as fathom_topk.
 *   The scratch is fathom_topk_noalloc_max_bytes() bytes (64 MiB); a call
 *   whose fathom_topk_workspace_bytes(rows, n, k) exceeds it returns
 *   FATHOM_ERR_TOO_LARGE and enqueues nothing (32 rows of 2^20 keys need
 *   about 21 MB).
 *   The scratch of a GPU is shared by every call on that GPU and keeps the
 *   last call's contents (the selection writes everything it reads, so
 *   nothing has to start cleared): calls that overlap on one GPU (two
 *   streams, two host threads) race and must be serialised by the caller.
 *   The scratch's device address is looked up once per GPU, on the first
 *   call that runs there (the device of `stream`, or the current device for
 *   the null stream).
 */
size_t fathom_topk_noalloc_max_bytes(void);
int fathom_topk_noalloc(const float* scores, int64_t rows, int64_t n, int32_t k,
                        int32_t* indices, void* stream);

/*
 * fathom_scan_topk — fathom_scan followed by fathom_topk on its scores, with
 * the top-k candidates taken by the scan itself instead of by a second pass
 * over the scores, and the scores written only when the caller wants them.
 *
 * Results are those of the two calls, bit for bit: scores as fathom_scan
 * writes them (when `scores` is non-null), indices as fathom_topk selects
 * them (§2 order, ascending).  When 65536 <= n <= 2^21 (and the group's
 * plane array is under 4 GiB): 8 runs of 1024 keys spread evenly over each
 * row are scored first, a cut tau per row is taken from that sample (inside
 * the scan's launch), and the scan then writes every score >= tau, in index
 * order, to the row's candidate buffer (pooled per 2048-key round, which
 * holds 512 of them; the blocks after the last whole round per 512-key
 * tile, 128 each, the last tile possibly partial), from which the selection
 * is made.  A row whose candidates cannot give the selection (fewer than k
 * of them, or a round with more than its region holds: heavy ties, or top
 * keys crowded past a quarter of a round) is selected from its scores: from
 * `scores`, or, when `scores` is null, from a second scan of its group into
 * the workspace.
 * Otherwise the two calls run as they are (into the workspace when `scores`
 * is null).
 *
 *   planes, scales, nb_store, depths, q, groups, G, d, n: as fathom_scan
 *   scores  [groups][G][n] fp32 output, or NULL (no scores are written to
 *           caller memory; the fused path then writes none at all unless a
 *           row needs them)
 *   indices [groups * G][k] int32 output
 *   workspace: device scratch of at least fathom_scan_topk_workspace_bytes(
 *   groups, G, n, k) bytes (it includes room for every row's scores),
 *   256-byte aligned; contents on entry do not matter.
 *   1 <= k <= n.
 */
size_t fathom_scan_topk_workspace_bytes(int64_t groups, int32_t G, int64_t n, int32_t k);
int fathom_scan_topk(const uint64_t* planes, const uint16_t* scales, int64_t nb_store,
                     const uint8_t* depths, const float* q, int64_t groups, int32_t G, int32_t d,
                     int64_t n, int32_t k, float* scores, int32_t* indices, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * fathom_gather — copy the runs a plan reads from a host-resident store into
 * the device store (§3.6: the first t_j planes of channel j are one run of
 * t_j * n / 8 bytes; Fig. 10: contiguous copies run at the link rate).
 *
 * For every group and channel with t_j > 0: planes p < t_j and the scale row,
 * blocks [0, n/64), from host_planes / host_scales to planes / scales at the
 * same positions.  Nothing else of the device store is written (the scan
 * never reads it).  The depths stay in device memory: no host round trip.
 *
 *   host_planes, host_scales: store layout of fathom_encode, in pinned host
 *     memory the device can address (hipHostMalloc; torch pin_memory)
 *   planes, scales: device store of the same nb_store
 *   depths [groups][d] uint8 (device)
 *   nb_store a multiple of 8 blocks; all four store pointers 16-byte aligned.
 *   FATHOM_ERR_NOT_PINNED if the host store is not memory the device can
 *   address.
 */
int fathom_gather(const uint64_t* host_planes, const uint16_t* host_scales, int64_t nb_store,
                  const uint8_t* depths, int64_t groups, int32_t d, int64_t n, uint64_t* planes,
                  uint16_t* scales, void* stream);

/*
 * The KLT-rotated store (§3.5 "rotated variant"; the calibration-free fit of
 * Appendix D).  For keys whose variance is not concentrated in few raw
 * channels the store holds the planes of (k - mu) V, V the eigenbasis of the
 * keys' covariance, and the plan uses g_j = sum_h ((q_h V)_j)^2 lambda_j.
 * With these calls the rotated variant is
 *   fathom_klt_fit -> fathom_klt_rotate_keys -> fathom_encode     (store)
 *   fathom_klt_rotate_queries -> fathom_plan(q V, lambda) -> fathom_scan(q V)
 * and its scores are q . (k - mu) up to the quantisation: the per-row
 * constant q . mu is left out (it moves no key across the top-k boundary).
 *
 * fathom_klt_fit — per group: mu_c = mean of the n binary16 keys of channel
 * c; C = (k - mu)^T (k - mu) / (n - 1), all in fp64 (sum order unspecified);
 * its eigenpairs by cyclic Jacobi (fp64 covariance, fp32 accumulated
 * rotation), eigenvalues descending (equal values: lower Jacobi index
 * first), each eigenvector signed so its first component of magnitude at
 * least 1/(2 sqrt(d)) is positive; eigenvalues below 0 read as 0.
 *   k      [groups][n][d] binary16 (16-byte aligned), n >= 64, n % 64 == 0
 *   mu     [groups][d]    fp32 output
 *   basis  [groups][d][d] fp32 output, eigenvector j in column j (row c =
 *          raw channel c)
 *   lambda [groups][d]    fp32 output (the rotated channels' variances)
 *   workspace: device scratch of fathom_klt_fit_workspace_bytes(groups, n, d)
 *          bytes, 256-byte aligned (0 from the query for invalid shapes).
 *
 * fathom_klt_rotate_keys — k_rot[g][i][j] = binary16 (nearest-even) of the
 * fp32 fold over c = 0 .. d-1 ascending, from +0, of
 * fma(fl32(k_ic - mu_c), basis[c][j], acc).  k, k_rot 16-byte aligned,
 * basis 16-byte aligned.  |k_rot| beyond the binary16 range gives Inf, which
 * fathom_encode then flags.
 *
 * fathom_klt_rotate_queries — q_rot[g][h][j] = the fp32 fold over c
 * ascending, from +0, of fma(q_hc, basis[c][j], acc).  q, q_rot
 * [groups][G][d] fp32; basis 16-byte aligned.
 */
size_t fathom_klt_fit_workspace_bytes(int64_t groups, int64_t n, int32_t d);
int fathom_klt_fit(const uint16_t* k, int64_t groups, int64_t n, int32_t d, float* mu,
                   float* basis, float* lambda, void* workspace, size_t workspace_bytes,
                   void* stream);
int fathom_klt_rotate_keys(const uint16_t* k, const float* mu, const float* basis,
                           int64_t groups, int64_t n, int32_t d, uint16_t* k_rot, void* stream);
int fathom_klt_rotate_queries(const float* q, const float* basis, int64_t groups, int32_t G,
                              int32_t d, float* q_rot, void* stream);

/* Static, NUL-terminated name of a status code. */
const char* fathom_status_string(int status);
/*
 * fathom_test_cut_hooks — for tests of the fallbacks of fathom_scan_topk
 * and fathom_topk only.  In fathom_scan_topk's fused path the scan's first
 * workgroups publish each row's cut and the scan waves poll for it a
 * bounded number of times; a row whose cut is still missing then is flagged
 * and selected by the fallback.  In fathom_topk the first workgroups of the
 * compaction publish the cuts in the same way, and a chunk whose cut does
 * not come in time sends its row to the selection from the scores.
 * publish = 0 makes those workgroups store the cut without publishing it,
 * so that every waiting wave reaches its poll limit; spin_limit (1 to 16384
 * polls of about 0.2 us) sets the limit.  (1, 2048) are the defaults.  Host-side settings
 * of the calling process, read by later calls; FATHOM_ERR_BAD_RANGE for a
 * publish other than 0 or 1 or a limit outside the range.
 */
int fathom_test_cut_hooks(int32_t publish, int32_t spin_limit);

/* FATHOM_ABI_VERSION of the loaded library. */
int fathom_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FATHOM_H_ */
