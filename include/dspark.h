/*
 * dspark.h -- C ABI of libdspark.so: the data-parallel hot path of one DSpark
 * speculative-decoding round on an MI355X (gfx950) GPU.
 *
 * Method (the DSpark pages; cited by page and section):
 *  [P3] papercache.org summary of "DSpark: Confidence-Scheduled Speculative
 *       Decoding with Semi-Autoregressive Generation" (arXiv 2607.05147).
 *  [P1] backyes.github.io "MTP algorithm survey", section 2.2 (rejection sampling).
 *  [P2] bevisy.github.io DeepSpec analysis, section 2.2 (DFlash = rank 0) and
 *       section 5.4 (DSpark in SGLang): verify modes static / compact /
 *       cap-accept, ragged verify padded to captured graph tiers.
 *  [P4] modelscope/CSDN DSpark article, section 3.3 (flatten + marker tensors).
 *
 * Conventions shared by every entry point
 *  - Every pointer is a DEVICE pointer unless marked (host).  The caller owns
 *    all memory; no call allocates, frees or synchronises.  Each call checks
 *    its scalar arguments on the host, then enqueues kernels on `stream` and
 *    returns; outputs are valid once the stream reaches the call.
 *  - A call that returns an error other than DSPARK_E_HIP has enqueued nothing.
 *    DSPARK_E_HIP means a kernel launch failed; the stream state is then the
 *    HIP runtime's.
 *  - The library keeps no state between calls other than a per-device cache
 *    of immutable device facts (compute-unit count, occupancy) and the test
 *    switches of dspark_set_switch.  Calls that share a workspace must be
 *    ordered on one stream (or otherwise serialised).
 *  - R = requests in the batch, gamma = block size (draft positions per
 *    request), V = vocabulary, r = Markov rank, d = backbone hidden size,
 *    T = sampling temperature (T == 0 selects greedy decoding).
 *  - Row-major layouts.  Token ids are int32 in [0, V).
 *  - Random numbers come from Philox4x32-10 (Salmon et al., SC'11) with
 *    key (lo32 seed, hi32 seed) and counter (idx/4, k | tag<<16, request,
 *    lo32 round); `round` must change between rounds that reuse a seed.
 *    Sampling from softmax(score) uses the chunked Gumbel-max rule with
 *    chunks of DSPARK_CHUNK consecutive vocabulary entries (exact sampling).
 *  - Limits: 1 <= gamma <= 32; r == 0 or r a multiple of 16 up to 512;
 *    1 <= V < 2^31; T >= 0 and finite; R * gamma <= 16384 for the scheduler.
 *    R == 0 is a valid empty batch (nothing is enqueued).
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSPARK_CHUNK 128

typedef enum {
    DSPARK_OK = 0,
    DSPARK_E_INVALID = 1,      /* null pointer, negative size, T < 0, bad layout  */
    DSPARK_E_UNSUPPORTED = 2,  /* outside the limits above                         */
    DSPARK_E_WORKSPACE = 3,    /* ws_bytes < dspark_workspace_bytes(...)           */
    DSPARK_E_HIP = 4           /* a kernel launch failed                           */
} dspark_status;

/* Element type of a tensor argument: a plain 32-bit integer, so that any value
 * a caller passes is well defined to receive and check (values other than
 * these two are rejected with DSPARK_E_INVALID). */
typedef int32_t dspark_dtype;
enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 };

/* Device-side condition flags, OR-ed into the workspace status word. */
#define DSPARK_FLAG_NONFINITE 1u   /* a non-finite logit or score was seen        */
#define DSPARK_FLAG_BAD_LEN   2u   /* a pack length outside [0, width] was clamped */
#define DSPARK_FLAG_BAD_TOKEN 4u   /* a token id outside [0, V) was read           */
#define DSPARK_FLAG_BARRIER   8u   /* a grid barrier of the persistent draft gave
                                      up waiting (its outputs are then invalid)   */
#define DSPARK_FLAG_TIER     16u   /* a tiered pack's total exceeded every tier
                                      (N_pad = N)                                 */

/*
 * Tracing: every call in this header that takes a stream, and dspark_get_status, opens
 * a roctx range named after itself for its host-side span (shown by
 * `rocprofv3 --marker-trace`); without a profiler attached the ranges cost
 * two calls that return at once.
 */

/*
 * (host) Test and measurement switches.  They select among schedules that give
 * the same results (or bound a wait); they never change what is computed.
 * Their start values are read once from the environment, the first time the
 * library needs them: DSPARK_DRAFT_KERNEL=steps (FORCE_PER_STEP = 1),
 * DSPARK_DRAFT_KERNEL=pipe (DRAFT_KERNEL = 1), DSPARK_RNN_CELL_VALU set
 * (RNN_CELL_VALU = 1), DSPARK_BARRIER_SPINS=n (BARRIER_SPINS = n),
 * DSPARK_PERSIST_LAUNCH=coop (PERSIST_LAUNCH = 1).  Apart from the
 * per-device cache of device facts and a per-process call counter of the
 * verify these switches are the library's only state; set them between
 * rounds, not while calls are being enqueued on another thread.
 *   FORCE_PER_STEP  1: the per-step draft schedule for every shape
 *   RNN_CELL_VALU   1: the RNN head on the per-step schedule with the
 *                   vector-ALU cell
 *   BARRIER_SPINS   polls before a cross-workgroup wait of a persistent draft
 *                   launch gives up (DSPARK_FLAG_BARRIER); 0 = the default 2^24
 *   DRAFT_KERNEL    persistent Markov draft: 0 one grid barrier per step
 *                   (default), 1 request groups pipelined across steps (no
 *                   grid barrier; slower on the measured shapes)
 *   PERSIST_LAUNCH  launches whose workgroups wait for one another (the
 *                   persistent draft kernels, with grid barriers; grids of
 *                   at most one workgroup per compute unit): 0 plain launch (default; resident at once while
 *                   nothing else occupies the device, otherwise the waits
 *                   last until the other work drains; a wait that gives up
 *                   sets DSPARK_FLAG_BARRIER), 1 cooperative launch (the
 *                   runtime guarantees residency; about 20 us more per
 *                   launch from its synchronisation around the kernel)
 * dspark_set_switch returns DSPARK_E_INVALID for an unknown key or value;
 * dspark_get_switch returns -1 for an unknown key.
 */
#define DSPARK_SWITCH_FORCE_PER_STEP 1
#define DSPARK_SWITCH_RNN_CELL_VALU  2
#define DSPARK_SWITCH_BARRIER_SPINS  3
#define DSPARK_SWITCH_DRAFT_KERNEL   4
#define DSPARK_SWITCH_PERSIST_LAUNCH 5
dspark_status dspark_set_switch(int key, int64_t value);
int64_t dspark_get_switch(int key);

/* (host) Bytes of workspace every entry point below needs for these sizes.
 * Its first 256 bytes (the header: status word, the verify's epoch words and
 * counters) must be zero when a workspace is first used; the calls keep them
 * consistent afterwards, also when a call is captured in a HIP graph and
 * replayed. */
size_t dspark_workspace_bytes(int R, int gamma, int V, int r, int d);

/* (host) Human-readable name of a status code. */
const char* dspark_status_string(dspark_status s);

/* (host) Version string of the library build. */
const char* dspark_version(void);

/* Clears the workspace status word (enqueued on `stream`; no allocation). */
dspark_status dspark_clear_status(void* ws, size_t ws_bytes, hipStream_t stream);

/* (host, synchronous) Reads the workspace status word into *flags (host).  Call
 * after the stream has finished the calls of interest; it blocks on a copy. */
dspark_status dspark_get_status(const void* ws, size_t ws_bytes, uint32_t* flags);

/*
 * Markov draft head over one block ([P3] Method details: causal block
 * distribution p_k(v | x_0, x_<k) = softmax(U_k + B_k)(v); Markov head
 * B(x_{k-1}, .) = W1[x_{k-1}] W2 with W1 in R^{V x r}, W2 in R^{r x V}; the
 * anchor x_0 is the first predicted position's input).  For k = 1..gamma, in
 * order: s = (U_k + W1[x_{k-1}] W2) / T over the whole vocabulary, an exact
 * softmax, and x_k sampled from it; T == 0 takes the first argmax of
 * U_k + W1[x_{k-1}] W2.  r == 0 is the DFlash case: independent per-position
 * sampling from softmax(U_k / T) ([P2] 2.2).
 *   U      [R][gamma][V]   base logits U_1..U_gamma (U_dt)
 *   W1     [V][r]          embedding table (W_dt); unused if r == 0
 *   W2t    [V][r]          W2 TRANSPOSED: W2t[v][i] = W2[i][v], the weight
 *                          layout of a linear layer r -> V (W_dt);
 *                          dspark_w2_transpose converts W2 [r][V] into it
 *   x0     [R]             anchors
 *   x      out [R][gamma+1]  x[i][0] = x0[i], x[i][k] = drafted token k
 *   logp_d out [R][gamma]    log p_k(x_k) of the tempered draft (0 if T == 0)
 *   lse_d  out [R][gamma]    log-normaliser of s (max score if T == 0)
 *   margin out nullable [R][gamma]  gap between the two best Gumbel keys
 *                          (debug; smaller of the chunk and in-chunk gaps)
 * W_dt == DSPARK_BF16 runs the bias contraction on MFMA (fp32 accumulation);
 * DSPARK_F32 weights run it on the vector ALU.  With bf16 U and weights,
 * r in {64, 128, 256}, 16-byte aligned tables, V a multiple of 8 and at most
 * 512 vocabulary entries per compute unit, all gamma steps run as one
 * launch whose workgroups are all resident at once (at most one per compute
 * unit; plain launch, or cooperative with DSPARK_SWITCH_PERSIST_LAUNCH) that
 * keeps W2 on chip (grid barriers between steps; DSPARK_FLAG_BARRIER reports
 * a barrier that gave up waiting); other shapes
 * run two launches per step, and r == 0 (independent positions) two launches
 * in all.  The schedules give the same results.  DSPARK_SWITCH_FORCE_PER_STEP
 * forces the per-step schedule.
 */
dspark_status dspark_draft_markov(int R, int gamma, int V, int r, float T,
                                  uint64_t seed, uint64_t round,
                                  const void* U, dspark_dtype U_dt,
                                  const void* W1, const void* W2t, dspark_dtype W_dt,
                                  const int32_t* x0, int32_t* x, float* logp_d, float* lse_d,
                                  float* margin, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * W2 in the method's own layout ([P3] Method details: W2 in R^{r x V}) into
 * the W2t layout every entry point here reads: W2t[v][i] = W2[i][v].  The
 * draft keeps each compute unit's slice of vocabulary entries in registers
 * with an entry's r values contiguous, and its picks read a chunk's 128
 * entries as 128 contiguous rows, so W2t is the resident format; convert once
 * per weight update.  Element bits are copied unchanged.
 *   W2   [r][V]   (W_dt)
 *   W2t  out [V][r] (W_dt); must not overlap W2
 * r == 0 enqueues nothing.  DSPARK_E_INVALID for negative r, V < 1, a null
 * or overlapping buffer or an unknown W_dt.
 */
dspark_status dspark_w2_transpose(int r, int V, const void* W2, void* W2t, dspark_dtype W_dt,
                                  hipStream_t stream);

/*
 * dspark_draft_markov for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument; the draft's scratch (status word, chunk statistics,
 * barrier flags, per-slice records) lives in a static device array of
 * DSPARK_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds until
 * the process ends.  The call allocates and frees nothing.  Same kernels and
 * results as dspark_draft_markov; rank 0 takes one statistics launch per
 * position (the all-rows region of the workspace is not there).
 *   flags   out nullable (device uint32): the DSPARK_FLAG_* word of this call,
 *           written when the stream reaches the end of the call
 *   other arguments as for dspark_draft_markov
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller.  The array keeps the last call's contents; the call clears what has
 * to start at zero.  Returns DSPARK_E_WORKSPACE when the shape needs more than
 * the array: 256 + 12 R ceil(V/128) + 4096 + 32 R ceil(V/512) bytes, each term
 * rounded up to 256.
 */
#define DSPARK_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
dspark_status dspark_draft_markov_noalloc(int R, int gamma, int V, int r, float T,
                                          uint64_t seed, uint64_t round,
                                          const void* U, dspark_dtype U_dt,
                                          const void* W1, const void* W2t, dspark_dtype W_dt,
                                          const int32_t* x0, int32_t* x, float* logp_d,
                                          float* lse_d, float* margin, uint32_t* flags,
                                          hipStream_t stream);

/*
 * Instrumented dspark_draft_markov for performance measurement: identical
 * results; additionally records events on `stream` around the draft's
 * dominant kernel.  With the persistent schedule (one launch for all gamma
 * steps) that is ev_begin[0] / ev_end[0] around the launch and
 * *n_timed = 1; with the per-step schedule ev_begin[k-1] / ev_end[k-1] bracket
 * the per-chunk statistics kernel of step k and *n_timed = gamma; at r == 0
 * (independent positions: one statistics launch over all R gamma rows, then
 * one pick launch) ev_begin[0] / ev_end[0] bracket the statistics launch and
 * *n_timed = 1.
 *   ev_begin, ev_end  (host) arrays of gamma events created by the caller
 *   n_timed           (host, nullable) number of event pairs recorded
 * Returns DSPARK_E_INVALID if either array is null.
 */
dspark_status dspark_draft_markov_profiled(int R, int gamma, int V, int r, float T,
                                           uint64_t seed, uint64_t round,
                                           const void* U, dspark_dtype U_dt,
                                           const void* W1, const void* W2t, dspark_dtype W_dt,
                                           const int32_t* x0, int32_t* x, float* logp_d,
                                           float* lse_d, float* margin, void* ws, size_t ws_bytes,
                                           hipStream_t stream, hipEvent_t* ev_begin,
                                           hipEvent_t* ev_end, int* n_timed);

/*
 * Confidence head ([P3] Method details, confidence head and STS calibration):
 * c[i][k-1] = sigmoid((w_h . h_k + w_e . W1[x_{k-1}]) / t_k), k = 1..gamma.
 *   h      [R][gamma][d]   backbone hidden states (h_dt)
 *   W1     [V][r]          embedding table (W_dt); unused if r == 0
 *   w      [d + r]         confidence vector [w_h ; w_e] (w_dt)
 *   sts_T  nullable [gamma] per-position temperatures (default 1)
 *   x      [R][gamma+1]    anchor + drafted tokens
 *   c      out [R][gamma]  float32 confidences
 */
dspark_status dspark_confidence(int R, int gamma, int d, int r, int V,
                                const void* h, dspark_dtype h_dt,
                                const void* W1, dspark_dtype W_dt,
                                const void* w, dspark_dtype w_dt,
                                const float* sts_T, const int32_t* x, float* c,
                                hipStream_t stream);

/*
 * Hardware-aware prefix scheduler ([P3] Method details, "greedy solution and
 * causality", Algorithm 1).  a[i][j] = prod_{q<=j} c[i][q] (float32, left to
 * right); candidates (i, j) with a > 0 are taken in order of a descending
 * (ties: i, then j ascending); starting from B = R, tau = R,
 * Theta_best = R * SPS(R), each candidate adds 1 to B and a to tau, and
 * Theta = tau * SPS(B) must strictly improve or the scan stops (early stop).
 * tau is summed in 2^-32 fixed point (exact, order-free); Theta is a double.
 * B > N_max counts as Theta = 0 (capacity exceeded).
 *   c          [R][gamma]   confidences, in [0, 1] (the confidence head's
 *                           sigmoid outputs; outside [0, 1] a request's
 *                           admitted positions need not form a prefix and
 *                           ell, N_out and Theta are unspecified)
 *   sps        [N_max+1]    SPS(B), engine steps per second at batch B (double)
 *   enabled    0: ell = gamma for every request (static verification; then
 *              N_max must hold the whole block, N_max >= R (gamma + 1), else
 *              DSPARK_E_INVALID)
 *   ell        out [R]      scheduled verify lengths in [0, gamma]
 *   a          out nullable [R][gamma]  survival products
 *   N_out      out nullable (device scalar)  sum_i (1 + ell_i)
 *   theta_best out nullable (device scalar)  Theta of the returned schedule
 * Needs R <= N_max and R * gamma <= 16384 (one workgroup, LDS-resident sort).
 */
dspark_status dspark_prefix_schedule(int R, int gamma, const float* c, const double* sps,
                                     int N_max, int enabled, int32_t* ell, float* a,
                                     int32_t* N_out, double* theta_best, hipStream_t stream);

/*
 * Asynchronous prefix scheduler, the production form ([P3] Supplementary
 * details, the hardware-aware prefix scheduler in production; [P1] 4.2.5 and
 * 8.5).  The candidates and their order are those of dspark_prefix_schedule.
 * One sort of this round's candidates serves two decisions:
 *   admission  the first min(*K_in, N_max) - R candidates are admitted
 *              (dynamic top-K: none if that count is <= 0, all if it exceeds
 *              their number); no Theta test, no early stop.
 *   planning   q* = the first q in 0..|E| maximising Theta_q = tau_q SPS(R + q)
 *              over the sorted candidates (global search; Theta = 0 past
 *              N_max); *K_plan = R + q*.  A round two rounds later passes it
 *              back as K_in.
 * Because the capacity a round admits with was fixed from confidences two
 * rounds old, the batch size does not depend on this round's tokens, and the
 * host can read it (copied asynchronously) before the round is enqueued.
 *   c, sps, N_max   as for dspark_prefix_schedule; SPS values finite, >= 0
 *   K_in       (device scalar) verify capacity in tokens, anchors included;
 *              the caller seeds the first two rounds (e.g. with
 *              min(R (gamma + 1), N_max), the static block)
 *   K_plan     out (device scalar) the capacity planned from this round.  May
 *              be the same address as K_in: K_in is read before K_plan is
 *              written (a two-slot ring indexed by round parity works).
 *   ell        out [R]  scheduled verify lengths (admitted prefix per request)
 *   a          out nullable [R][gamma] survival products
 *   N_out      out nullable (device scalar) sum_i (1 + ell_i)
 *   theta      out nullable (device scalar) Theta of the admitted schedule
 *   theta_plan out nullable (device scalar) Theta_{q*}
 * Needs R <= N_max and R * gamma <= 16384, like dspark_prefix_schedule.
 */
dspark_status dspark_async_schedule(int R, int gamma, const float* c, const double* sps,
                                    int N_max, const int32_t* K_in, int32_t* K_plan, int32_t* ell,
                                    float* a, int32_t* N_out, double* theta, double* theta_plan,
                                    hipStream_t stream);

/*
 * Scheduler and verify-batch pack in one launch ([P3] Method details, the
 * prefix scheduler, and Supplementary details, variable-length routing; [P4]
 * 3.3): the schedule of dspark_prefix_schedule (mode 0: static, every
 * request verifies its whole block; mode 1: greedy with early stop) or of
 * dspark_async_schedule (mode 2), then the pack of dspark_pack with rows = x,
 * len = the ell just decided, len_offset = 1, by the same workgroup.  Every
 * output equals that of the two calls in sequence.
 *   mode       0 static, 1 greedy, 2 asynchronous (K_in, K_plan required)
 *   c, sps, N_max, K_in, K_plan, ell, a, theta, theta_plan
 *              as for the schedulers (theta = theta_best in modes 0 and 1;
 *              theta_plan is written in mode 2 only)
 *   x          [R][gamma+1] anchor + drafted tokens
 *   N_out      out nullable (device scalar) sum_i (1 + ell_i) = cu[R]
 *   cu, flat, marker_req, marker_pos  as for dspark_pack with width gamma+1
 * Needs R <= N_max and R * gamma <= 16384 (mode 0: N_max >= R (gamma + 1)).
 */
dspark_status dspark_schedule_pack(int R, int gamma, int mode, const float* c, const double* sps,
                                   int N_max, const int32_t* K_in, int32_t* K_plan,
                                   const int32_t* x, int32_t* ell, float* a, int32_t* N_out,
                                   double* theta, double* theta_plan, int32_t* cu, int32_t* flat,
                                   int32_t* marker_req, int32_t* marker_pos, hipStream_t stream);

/*
 * Ragged pack ([P3] Supplementary details, variable-length routing; [P4] 3.3):
 * row i contributes its first len[i] + len_offset tokens; all of them are
 * flattened back to back as independent elements, with offsets and marker
 * tensors (owning request, position in the block).
 *   rows       [R][width]   token rows (e.g. x with width gamma+1)
 *   len        [R]          lengths (e.g. ell with len_offset 1, or tau with 0);
 *                           an effective length outside [0, width] is clamped
 *                           and flagged (DSPARK_FLAG_BAD_LEN) when ws != NULL
 *   cu         out [R+1]    offsets, cu[0] = 0, cu[R] = N
 *   flat       out [R*width] packed tokens; slots >= N hold -1
 *   marker_req out nullable [R*width] owning request (-1 past N)
 *   marker_pos out nullable [R*width] position inside the block (-1 past N)
 *   N_out      out nullable (device scalar)
 */
dspark_status dspark_pack(int R, int width, const int32_t* rows, const int32_t* len,
                          int len_offset, int32_t* cu, int32_t* flat, int32_t* marker_req,
                          int32_t* marker_pos, int32_t* N_out, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * Ragged pack padded to a captured graph tier ([P2] 5.4, DSpark in SGLang: ragged verify packs the
 * requests into one compact buffer whose total is rounded up to a captured
 * CUDA-graph tier, so a fixed graph replays a batch of any smaller size).
 * The pack is dspark_pack's; then N_pad = the smallest tier >= N, or N when
 * no tier holds it (DSPARK_FLAG_TIER, when ws != NULL).  Slots [N, N_pad)
 * hold pad_token with markers -1; slots [N_pad, slots) hold -1.
 *   tiers      (host) [n_tiers] strictly ascending, each in [1, slots];
 *              copied into the launch (at most 32)
 *   slots      length of flat / marker_req / marker_pos, >= R * width
 *   N_pad      out nullable (device scalar)
 *   other arguments as for dspark_pack
 */
dspark_status dspark_pack_tiered(int R, int width, const int32_t* rows, const int32_t* len,
                                 int len_offset, const int32_t* tiers, int n_tiers, int pad_token,
                                 int64_t slots, int32_t* cu, int32_t* flat, int32_t* marker_req,
                                 int32_t* marker_pos, int32_t* N_out, int32_t* N_pad, void* ws,
                                 size_t ws_bytes, hipStream_t stream);

/*
 * Lossless rejection-sampling verification ([P3] Background: x_k accepted with
 * probability min(1, p_t(x_k) / p_d(x_k)), left to right, the first rejection
 * drops the rest; [P1] 2.2: at the first rejection a token is resampled from
 * norm(max(0, p_t - p_d)), after a fully accepted prefix a bonus token is
 * drawn from the next target distribution, tau = m + 1; at T == 0 the test is
 * x_k == argmax p_t and the correction is the argmax).
 * Request i verifies positions 1..ell[i].  Its verify row j (input token x_j,
 * target distribution p_t^{j+1}), j = 0..ell[i], is read from
 *   target_layout 0: packed [N][V], row cu[i] + j (cu from dspark_pack with
 *                    rows = x, len = ell, len_offset = 1)
 *   target_layout 1: dense [R][gamma+1][V], row i*(gamma+1) + j
 * Accept test: log u < log p_t(x_k) - logp_d[i][k-1] with u in (0,1).
 * Zero residual mass (p_t == p_d up to rounding) falls back to p_t.
 *   x, logp_d, lse_d  the draft's outputs;  U, W1, W2t the draft's inputs
 *                     (used to rebuild p_d at a rejected position)
 *   m           out [R]        accepted draft tokens
 *   tau         out [R]        m + 1 emitted tokens
 *   emitted     out [R][gamma+1] x_1..x_m then the resampled / bonus token; -1 after
 *   next_anchor out [R]        the last emitted token (next round's x_0)
 *   logp_t      out nullable [R][gamma]  log p_t(x_k) for k <= ell[i], else 0
 */
dspark_status dspark_verify(int R, int gamma, int V, int r, float T,
                            uint64_t seed, uint64_t round,
                            const int32_t* ell, const int32_t* cu,
                            const void* target, dspark_dtype t_dt, int target_layout,
                            const int32_t* x, const float* logp_d, const float* lse_d,
                            const void* U, dspark_dtype U_dt,
                            const void* W1, const void* W2t, dspark_dtype W_dt,
                            int32_t* m, int32_t* tau, int32_t* emitted, int32_t* next_anchor,
                            float* logp_t, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Single-step acceptance rate of every block position, a diagnostic pass
 * over the whole block ([P3] Method details, confidence head: the head is
 * supervised with c*_k = 1 - TV(p_d^k, p_t^k)):
 *   c*_k = sum_v min(p_d^k(v), p_t^k(v)),  k = 1..gamma,
 * with p_d^k the tempered draft distribution of position k given x_{k-1}
 * (rebuilt from U, W1, W2t and normalised by lse_d, as at a rejection) and
 * p_t^k = softmax(row / T) of dense target row i*(gamma+1) + k-1.  T == 0:
 * point masses, c*_k = 1 if x_k is the first argmax of that target row, else 0.
 *   target   dense [R][gamma+1][V] (t_dt, equal to U_dt); rows 0..gamma-1 are read
 *   x, lse_d the draft's outputs; U, W1, W2t the draft's inputs
 *   c_star   out [R][gamma] float32
 * Uses the workspace like dspark_verify (same size); enqueues about 3 gamma
 * kernels.
 */
dspark_status dspark_acceptance_rate(int R, int gamma, int V, int r, float T, const void* target,
                                     dspark_dtype t_dt, const int32_t* x, const float* lse_d,
                                     const void* U, dspark_dtype U_dt, const void* W1,
                                     const void* W2t, dspark_dtype W_dt, float* c_star, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/*
 * Sequential temperature scaling fit of the confidence head ([P3] Method
 * details, post-hoc calibration; [P1] 4.2.3).  Held-out data: n blocks with
 * raw confidence logits z (c_k = sigmoid(z_k / t_k); e.g. from
 * dspark_confidence_logits) and the number m of drafts the target accepted
 * under whole-block verification.  Left to right, k = 1..gamma, with t_1..t_{k-1}
 * fixed: for every candidate t of the grid the cumulative product
 * A_k = A_{k-1} sigmoid(z_k / t) (A_0 = 1) is scored by its expected
 * calibration error against y_k = [m >= k],
 *   ECE = (1/n) sum_b | sum_{i in bin b} (A_i - y_i) |,
 * nbins equal-width bins of [0, 1], bin = min(floor(A nbins), nbins - 1);
 * t_k = the first grid value with the smallest ECE.  Evaluated in double,
 * deterministic.  The result feeds dspark_confidence's sts_T.
 *   z        [n][gamma] float32 logits;  m  [n] int32
 *   grid     (host) [G] candidate temperatures, each > 0 and finite, G <= 256
 *   nbins    1..64 (15 is the usual choice)
 *   t_out    out [gamma] float32 (a grid value per position)
 *   ece_out  out nullable [gamma] double: ECE at the chosen temperature
 *   ws       workspace of dspark_sts_workspace_bytes(n) bytes (8 n + 4 MiB and a
 *            little), 16-byte aligned
 */
size_t dspark_sts_workspace_bytes(int n);
dspark_status dspark_sts_fit(int n, int gamma, const float* z, const int32_t* m, const float* grid,
                             int G, int nbins, float* t_out, double* ece_out, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * Confidence logits: z_k = w . [h_k ; W1[x_{k-1}]] (dspark_confidence before the
 * temperature and the sigmoid), the input of the STS fit.  Arguments as for
 * dspark_confidence; z out [R][gamma] float32.
 */
dspark_status dspark_confidence_logits(int R, int gamma, int d, int r, int V,
                                       const void* h, dspark_dtype h_dt,
                                       const void* W1, dspark_dtype W_dt,
                                       const void* w, dspark_dtype w_dt,
                                       const int32_t* x, float* z, hipStream_t stream);

/*
 * Cap-accept verification ([P2] 5.4, DSpark in SGLang, the verify modes:
 * verify the whole window, commit only the scheduler's truncated window; used
 * to observe the acceptance a schedule leaves on the table).  Request i is
 * verified over its window ell[i] exactly as by dspark_verify (same random
 * streams, same accept tests), giving m_full accepted drafts.  With
 * C = cap[i] clamped to [0, ell[i]] (a negative cap is flagged
 * DSPARK_FLAG_BAD_LEN), the committed sequence is the first min(m_full, C) + 1
 * tokens of the verification's sequence: when m_full > C those are
 * x_1..x_{C+1}, the last being an accepted draft, and no correction or bonus
 * token is drawn; otherwise the outputs equal dspark_verify's.  A prefix of a
 * lossless sequence, so the committed tokens keep the target's law.
 *   ell      [R] verified window (typically gamma: the static block)
 *   cap      [R] commit window (typically the scheduler's ell)
 *   m, tau, emitted, next_anchor  the committed result (m = min(m_full, C))
 *   m_full   out nullable [R] accepted drafts over the whole window
 *   other arguments as for dspark_verify (logp_t covers the whole window)
 */
dspark_status dspark_verify_cap_accept(int R, int gamma, int V, int r, float T, uint64_t seed,
                                       uint64_t round, const int32_t* ell, const int32_t* cap,
                                       const int32_t* cu, const void* target, dspark_dtype t_dt,
                                       int target_layout, const int32_t* x, const float* logp_d,
                                       const float* lse_d, const void* U, dspark_dtype U_dt,
                                       const void* W1, const void* W2t, dspark_dtype W_dt,
                                       int32_t* m, int32_t* tau, int32_t* emitted,
                                       int32_t* next_anchor, int32_t* m_full, float* logp_t,
                                       void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * (host) Bytes of workspace dspark_draft_rnn needs for these sizes: the
 * shared workspace of dspark_workspace_bytes plus the h part of the cell's
 * projection ([R gamma][3r] float32) and the states when `state` is NULL
 * ([R][gamma][r] float32).  The first dspark_workspace_bytes bytes are laid
 * out as for every other entry point, so the same buffer serves the round.
 */
size_t dspark_rnn_workspace_bytes(int R, int gamma, int V, int r, int d);

/*
 * RNN draft head over one block ([P3] Method details, RNN head: a gated
 * recurrent state carries the whole in-block prefix, so the transition bias
 * of position k depends on every earlier draft, not only on x_{k-1}).  With
 * z_k = [s_{k-1} ; W1[x_{k-1}] ; h_k] (length 2r + d, s_0 = 0) and
 * Wr = [Wr_g ; Wr_c ; Wr_o] (3r rows, no bias terms):
 *   g_k = sigmoid(Wr_g z_k),  s_k = g_k * s_{k-1} + (1 - g_k) * tanh(Wr_c z_k),
 *   e_k = tanh(Wr_o z_k),     bias_k = W2^T e_k (e_k rounded to W_dt),
 * then x_k is drawn from softmax((U_k + bias_k) / T) by the same rule and
 * random stream as dspark_draft_markov (T == 0: first argmax).
 *   U, W1, W2t, x0, x, logp_d, lse_d, margin  as for dspark_draft_markov
 *   Wr     [3r][2r + d]     (W_dt) rows 0..r-1 gate, r..2r-1 candidate,
 *                           2r..3r-1 output; columns [s ; W1 row ; h]
 *   h      [R][gamma][d]    backbone hidden states (h_dt)
 *   feat   out [R][gamma][r]  e_1..e_gamma in W_dt (the bias features; pass
 *                           them to dspark_verify_features)
 *   state  out nullable [R][gamma][r] float32  s_1..s_gamma
 *   ws     at least dspark_rnn_workspace_bytes(R, gamma, V, r, d) bytes
 * r must be a multiple of 16 in [16, 512].  The h part of the projection is one
 * contraction over all positions before the chain (MFMA when h and Wr are
 * bf16 with d a multiple of 8 and 16-byte aligned tables).  With bf16 U,
 * weights and h, r in {64, 128, 256}, 2r + d a multiple of 8 and the shape
 * limits of dspark_draft_markov's persistent launch, all gamma steps (cell,
 * statistics, pick) run in one co-resident launch with two grid barriers per
 * step (DSPARK_FLAG_BARRIER as there).  Other shapes run three launches per
 * step: the cell (MFMA with the fp32 state split into exact bf16 parts for
 * bf16 weights, fp32 vector ALU otherwise), the per-chunk statistics and the
 * pick.  The schedules give the same results.  DSPARK_SWITCH_FORCE_PER_STEP
 * forces the per-step schedule, DSPARK_SWITCH_RNN_CELL_VALU the per-step
 * schedule with the vector-ALU cell.
 */
dspark_status dspark_draft_rnn(int R, int gamma, int V, int r, int d, float T,
                               uint64_t seed, uint64_t round,
                               const void* U, dspark_dtype U_dt,
                               const void* W1, const void* W2t, dspark_dtype W_dt,
                               const void* Wr, const void* h, dspark_dtype h_dt,
                               const int32_t* x0, int32_t* x, float* logp_d, float* lse_d,
                               float* margin, void* feat, float* state,
                               void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * dspark_acceptance_rate for drafts whose bias is carried by per-position
 * features (the RNN head): p_d^k = softmax((U_k + W2^T e_k) / T) with e_k from
 * feat row i*gamma + k-1 ([P3] Method details, confidence head: c*_k is the
 * single-step acceptance rate of the draft actually sampled).
 *   feat   [R][gamma][r] (W_dt) the draft's features; W1 is not read
 *   other arguments as for dspark_acceptance_rate (r >= 16)
 */
dspark_status dspark_acceptance_rate_features(int R, int gamma, int V, int r, float T,
                                              const void* target, dspark_dtype t_dt,
                                              const int32_t* x, const float* lse_d,
                                              const void* U, dspark_dtype U_dt,
                                              const void* feat, const void* W2t, dspark_dtype W_dt,
                                              float* c_star, void* ws, size_t ws_bytes,
                                              hipStream_t stream);

/*
 * dspark_verify_cap_accept for drafts whose bias is carried by per-position
 * features (the RNN head): the whole-window verification rebuilds p_d of a
 * rejected position from feat row i*gamma + k-1, as dspark_verify_features.
 *   feat   [R][gamma][r] (W_dt) the draft's features; W1 is not read
 *   other arguments as for dspark_verify_cap_accept (r >= 16)
 */
dspark_status dspark_verify_cap_accept_features(int R, int gamma, int V, int r, float T,
                                                uint64_t seed, uint64_t round, const int32_t* ell,
                                                const int32_t* cap, const int32_t* cu,
                                                const void* target, dspark_dtype t_dt,
                                                int target_layout, const int32_t* x,
                                                const float* logp_d, const float* lse_d,
                                                const void* U, dspark_dtype U_dt, const void* feat,
                                                const void* W2t, dspark_dtype W_dt, int32_t* m,
                                                int32_t* tau, int32_t* emitted,
                                                int32_t* next_anchor, int32_t* m_full,
                                                float* logp_t, void* ws, size_t ws_bytes,
                                                hipStream_t stream);

/*
 * Instrumented dspark_draft_rnn for performance measurement: identical
 * results; additionally records events on `stream` around the draft's
 * dominant kernel.  With the persistent schedule (cell, statistics and pick
 * of all gamma steps in one launch) that is ev_begin[0] /
 * ev_end[0] around the launch and *n_timed = 1; with the per-step schedule
 * ev_begin[k-1] / ev_end[k-1] bracket the per-chunk statistics kernel of
 * step k and *n_timed = gamma.
 *   ev_begin, ev_end  (host) arrays of gamma events created by the caller
 *   n_timed           (host, nullable) number of event pairs recorded
 * Returns DSPARK_E_INVALID if either array is null.
 */
dspark_status dspark_draft_rnn_profiled(int R, int gamma, int V, int r, int d, float T,
                                        uint64_t seed, uint64_t round,
                                        const void* U, dspark_dtype U_dt,
                                        const void* W1, const void* W2t, dspark_dtype W_dt,
                                        const void* Wr, const void* h, dspark_dtype h_dt,
                                        const int32_t* x0, int32_t* x, float* logp_d,
                                        float* lse_d, float* margin, void* feat, float* state,
                                        void* ws, size_t ws_bytes, hipStream_t stream,
                                        hipEvent_t* ev_begin, hipEvent_t* ev_end, int* n_timed);

/*
 * dspark_verify for drafts whose bias is carried by per-position features
 * (the RNN head above): identical accept tests and random streams; at a
 * rejected position k the draft distribution is rebuilt as
 * softmax((U_k + W2^T e_k) / T) from feat row i*gamma + k-1 instead of
 * W1[x_{k-1}] W2 ([P1] 2.2: the residual needs the p_d actually sampled).
 *   feat   [R][gamma][r] (W_dt) the draft's features; W1 is not read
 *   other arguments as for dspark_verify (r >= 16)
 */
dspark_status dspark_verify_features(int R, int gamma, int V, int r, float T,
                                     uint64_t seed, uint64_t round,
                                     const int32_t* ell, const int32_t* cu,
                                     const void* target, dspark_dtype t_dt, int target_layout,
                                     const int32_t* x, const float* logp_d, const float* lse_d,
                                     const void* U, dspark_dtype U_dt,
                                     const void* feat, const void* W2t, dspark_dtype W_dt,
                                     int32_t* m, int32_t* tau, int32_t* emitted,
                                     int32_t* next_anchor, float* logp_t,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * One whole round with the Markov head in one call ([P3] Method details: draft
 * the block, score it with the confidence head, schedule the verify prefix,
 * verify, emit): enqueues on `stream`, in this order and with the same
 * results as the calls made one by one,
 *   dspark_draft_markov      (margin not produced)
 *   dspark_confidence
 *   dspark_schedule_pack     (mode = sched_mode)
 *   dspark_verify
 *   dspark_pack              (emitted, tau, len_offset 0 -> cu_out, flat_out,
 *                             N_out; no markers)
 * with the fields of `a` as those calls' arguments of the same names (c, ell,
 * N, theta, ... are the intermediate buffers they hand to one another; `a` is
 * the score buffer of the scheduler).  (host) `a` is read during the call
 * only.  Every call's argument checks run before anything is enqueued, so an
 * error other than DSPARK_E_HIP leaves the stream untouched; the status is the
 * first failing call's.  ws, ws_bytes: one workspace of
 * dspark_workspace_bytes(R, gamma, V, r, d) bytes shared by the five calls.
 */
typedef struct dspark_round_markov_args {
  int R, gamma, V, r, d;
  float T;
  uint64_t seed, round;
  int sched_mode;                 /* 0 static block, 1 Algorithm 1, 2 asynchronous */
  int N_max;
  int target_layout;
  dspark_dtype U_dt, W_dt, h_dt, w_dt, t_dt;
  /* inputs */
  const void* U;
  const void* W1;
  const void* W2t;
  const int32_t* x0;
  const void* h;
  const void* w;
  const float* sts_T;             /* nullable */
  const double* sps;
  const void* target;
  const int32_t* K_in;            /* sched_mode 2 only */
  int32_t* K_plan;                /* sched_mode 2 only */
  /* intermediate buffers and outputs */
  int32_t* x;
  float* logp_d;
  float* lse_d;
  float* c;
  int32_t* ell;
  float* a;                       /* nullable */
  int32_t* N;                     /* nullable */
  double* theta;                  /* nullable */
  double* theta_plan;             /* nullable */
  int32_t* cu;
  int32_t* flat;
  int32_t* marker_req;            /* nullable */
  int32_t* marker_pos;            /* nullable */
  int32_t* m;
  int32_t* tau;
  int32_t* emitted;
  int32_t* next_anchor;
  float* logp_t;                  /* nullable */
  int32_t* cu_out;
  int32_t* flat_out;
  int32_t* N_out;                 /* nullable */
} dspark_round_markov_args;
dspark_status dspark_round_markov(const dspark_round_markov_args* a, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
