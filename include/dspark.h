/*
 * dspark.h -- C ABI of the MI355X (gfx950) library for one DSpark draft/verify round.
 *
 * The round, per batch of B requests (sources cited by short name):
 *   [XTL]   "[DeepSeek-6] DSpark: From Draft Models to Serving-Aware Speculative
 *           Decoding" (xutianle.me), sections 1-7.
 *   [CSDN]  "DSpark: Confidence-Scheduled Speculative Decoding with Semi-Autoregressive
 *           Generation -- 研读报告" (devpress.csdn.net), key formulas Eq. 4, 7, 8 and the
 *           throughput objective Theta = tau * SPS(B).
 *   [AIMSG] "DeepSeek DSpark 深度解读：系统工程与模型协同的极致优化" (aimsg.uk), concepts 2, 8, 9.
 *
 *   1. dspark_draft_markov   Markov-head draft: gamma sequential softmax + sampling steps
 *                            over base logits plus a rank-r transition bias  [CSDN Eq. 4; XTL §3-4]
 *   2. dspark_confidence     c_k = sigmoid(w . [h_k ; W1[x_{k-1}]])          [CSDN Eq. 7; XTL §5]
 *      dspark_sts_calibrate  per-position temperatures for it, fitted on held-out data, and
 *      dspark_confidence_calibrated, the head with them applied          [XTL §5; AIMSG]
 *   3. dspark_schedule       greedy prefix scheduler maximising tau * SPS(N)  [XTL §6; CSDN]
 *      dspark_schedule_topk  its production form: top-K admission, K from history [XTL §7]
 *   4. dspark_verify         lossless rejection-sampling verification         [XTL §1; AIMSG 2]
 *   5. dspark_accept_rate_tv analytic accept rate 1 - |p_d - p_t|_1 / 2       [CSDN Eq. 8; XTL §5]
 *   7. dspark_closed_loop    rounds 1-5 chained on the GPU with a synthetic Markov target,
 *                            the accepted length tau per round           [CSDN Eq. 1]
 * and, on the training side of the same heads:
 *   6. dspark_draft_loss     distribution-matching loss (CE + L1 + confidence BCE, position
 *                            weights) and its gradients                   [XTL §9, §5, §8]
 *
 * Conventions shared by every call:
 *   - Tensor arguments are DEVICE pointers to row-major contiguous arrays owned by the
 *     caller.  The library never allocates or frees memory and never reads device memory
 *     on the host.  Scratch memory is the caller's `ws` buffer of at least
 *     dspark_workspace_bytes(op, dims) bytes; its contents are undefined afterwards.
 *   - Calls enqueue kernels on `stream` (a hipStream_t; NULL = the default stream) and
 *     return without synchronising.  Arguments are validated on the host first: on any
 *     error a non-zero dspark_status is returned and nothing is enqueued.  Faults inside
 *     kernels surface at the caller's next synchronisation, as usual in HIP.
 *   - Token ids are int32 in [0, V).  Ids out of range are the caller's error; wherever a
 *     kernel uses an id as an index it is clamped into [0, V), so bad ids never fault.
 *     Inputs containing NaN give unspecified (but finite-time) results; a draft position
 *     whose logits are all -inf or NaN reports token -1 and logp NaN.
 *   - Identical inputs give bit-identical outputs (all cross-workgroup reductions have a
 *     fixed order or are order-free).  The calls keep no state between invocations and
 *     may run concurrently on different streams with different workspaces.
 *   - Randomness: u(seed, b, k, s, v) = (2 * (W >> 9) + 1) * 2^-24 where W is word
 *     (v mod 4) of Philox4x32-10 (Salmon et al., SC'11) applied to counter
 *     (v div 4, k, b, s) with key (seed mod 2^32, seed div 2^32).  b is the request row,
 *     k the 1-based position, s the stream: 0 draft sample, 1 accept test (v = 0),
 *     2 residual/bonus sample.  Gumbel noise is G = -ln(-ln u).
 *
 * Shapes: B = batch, gamma = draft length, V = vocabulary, r = Markov rank, d = hidden.
 * Limits: 1 <= B <= 65535, 1 <= gamma <= 64, 2 <= V <= 2^28, r a multiple of 8 with
 * 8 <= r <= 1024, 0 <= d <= 65536; dspark_schedule also needs B * gamma <= 4096.
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSPARK_OK = 0,
    DSPARK_E_NULL = 1,        /* a required pointer is NULL                               */
    DSPARK_E_SHAPE = 2,       /* a dimension is out of the supported range                */
    DSPARK_E_DTYPE = 3,       /* unknown dtype code                                       */
    DSPARK_E_VALUE = 4,       /* temperature <= 0 or not finite, unknown scheduler mode   */
    DSPARK_E_WORKSPACE = 5,   /* ws is NULL or ws_bytes < dspark_workspace_bytes(...)     */
    DSPARK_E_HIP = 6          /* the HIP runtime refused a launch                         */
} dspark_status;

typedef enum { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;

/* GREEDY and FULL: see dspark_schedule.  TOPK_DELAYED: dspark_closed_loop only (see there). */
typedef enum {
    DSPARK_SCHED_GREEDY = 0, DSPARK_SCHED_FULL = 1, DSPARK_SCHED_TOPK_DELAYED = 2
} dspark_sched_mode;

typedef enum {
    DSPARK_OP_DRAFT = 0, DSPARK_OP_CONFIDENCE = 1, DSPARK_OP_SCHEDULE = 2,
    DSPARK_OP_VERIFY = 3, DSPARK_OP_TV = 4
} dspark_op;

typedef struct {
    int32_t batch;   /* B */
    int32_t gamma;   /* draft length */
    int32_t vocab;   /* V */
    int32_t rank;    /* r */
    int32_t hidden;  /* d (only dspark_confidence reads it) */
} dspark_dims;

/* Scratch bytes the call `op` needs for `dims` (0 when it needs none).  Returns 0 for an
 * unknown op or invalid dims (the call itself then reports the error). */
size_t dspark_workspace_bytes(int op, const dspark_dims* dims);

/* Human-readable name of a status code (static storage). */
const char* dspark_status_string(int status);

/* Library version as 10000 * major + 100 * minor + patch. */
int dspark_version(void);

/*
 * Markov-head draft [CSDN Eq. 4; XTL §3 "Semi-Autoregressive", §4 "Markov Head"].
 * For k = 1..gamma (sequentially) and every request b:
 *   prev_b = x_{b,k-1}, with x_{b,0} = anchor[b] (the anchor is the first predicted
 *            position, [XTL §3]), or forced[b][k-2] when `forced` is not NULL;
 *   z_v    = (U[b][k-1][v] + sum_i W1[prev_b][i] * W2t[v][i]) / temperature;
 *   lse    = log sum_v exp(z_v);
 *   x_{b,k}= argmax_v (z_v + G(seed, b, k, 0, v)) -- a draw from p = softmax(z)
 *            (Gumbel-max; the lowest v wins exact ties);
 *   logp   = z_{x_{b,k}} - lse.
 * Arguments:
 *   U        [B][gamma][V] fp32 base logits of the parallel backbone.
 *   W1       [V][r] Markov embedding (`wdt`: F32 or BF16).
 *   W2t      [V][r] = W2 transposed, W2 being the [r][V] bias-free projection (same dtype).
 *   anchor   [B] int32 anchor tokens.
 *   forced   [B][gamma] int32 or NULL: teacher forcing -- position k conditions on
 *            forced[b][k-2] instead of the token drawn at k-1 (scores a given block; the
 *            call still draws and outputs its own tokens).
 *   tokens   out [B][gamma] int32 drawn tokens x_{b,1..gamma}.
 *   logp     out [B][gamma] fp32 log p_d(x_{b,k}).
 *   lse      out [B][gamma] fp32 log-partition of z at each position.
 */
dspark_status dspark_draft_markov(const dspark_dims* dims, const float* U, const void* W1,
                                  const void* W2t, int wdt, const int32_t* anchor,
                                  const int32_t* forced, float temperature, uint64_t seed,
                                  int32_t* tokens, float* logp, float* lse, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * dspark_draft_markov for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same computation,
 * kernels and results, bit for bit, with the same arguments except the workspace.  Its
 * scratch (the per-position packed winners and softmax partials) is a 32 MiB array in
 * device memory that the library holds on every GPU it runs on until the process ends;
 * the call itself allocates nothing and calls no allocating routine.  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (several streams or
 * host threads) race and give undefined results, so serialise them.  The array keeps the
 * last call's contents; each call clears what it needs cleared with a kernel (no memset),
 * so the call can be captured in a graph.
 * Returns DSPARK_E_WORKSPACE (nothing enqueued) when the draft's scratch for `dims` exceeds
 * 32 MiB; dspark_workspace_bytes(DSPARK_OP_DRAFT, dims) <= 32 MiB guarantees it fits (e.g.
 * B = 128, gamma = 16, V = 151936 needs 8.4 MB).  DSPARK_E_HIP if the array's device
 * address cannot be looked up.  Other errors as for dspark_draft_markov.
 */
dspark_status dspark_draft_markov_noalloc(const dspark_dims* dims, const float* U,
                                          const void* W1, const void* W2t, int wdt,
                                          const int32_t* anchor, const int32_t* forced,
                                          float temperature, uint64_t seed, int32_t* tokens,
                                          float* logp, float* lse, void* stream);

/*
 * Confidence head [CSDN Eq. 7; XTL §5 "Confidence Head"]:
 *   c[b][k-1] = 1 / (1 + exp(-(sum_j w[j] h[b][k-1][j] + sum_i w[d+i] W1[x_{b,k-1}][i])))
 * with x_{b,0} = anchor[b] and x_{b,k-1} = tokens[b][k-2]; no bias term.
 *   h [B][gamma][d] (`hdt`), W1 [V][r] (`wdt`), w [d + r] (`wvdt`, order [h ; W1-row]),
 *   tokens [B][gamma] int32, c out [B][gamma] fp32.  Needs no workspace.
 */
dspark_status dspark_confidence(const dspark_dims* dims, const void* h, int hdt,
                                const void* W1, int wdt, const void* w, int wvdt,
                                const int32_t* anchor, const int32_t* tokens, float* c,
                                void* stream);

/*
 * The calibrated confidence head [XTL §5, sequential temperature scaling]:
 *   c[b][k-1] = 1 / (1 + exp(-logit_{b,k} / temps[k-1]))
 * with logit_{b,k} the argument of the sigmoid of dspark_confidence (computed the same
 * way) and temps [gamma] fp64 > 0 per-position temperatures, for instance those of
 * dspark_sts_calibrate.  temps NULL: DSPARK_E_NULL.  Other arguments as there.
 */
dspark_status dspark_confidence_calibrated(const dspark_dims* dims, const void* h, int hdt,
                                           const void* W1, int wdt, const void* w, int wvdt,
                                           const int32_t* anchor, const int32_t* tokens,
                                           const double* temps, float* c, void* stream);

/*
 * Sequential temperature scaling [XTL §5: the scheduler needs confidences whose values
 * match acceptance rates, so the product of confidences is calibrated on held-out data
 * from left to right; AIMSG, on STS: per position a 1-D grid search over the temperature,
 * minimising the expected calibration error (ECE) of the cumulative product against the
 * empirical prefix acceptance; scaling by a temperature keeps the confidences' order].
 *   n         held-out drafted blocks, 1 <= n <= 2^22.
 *   logit     [n][gamma] fp32 confidence logits (c = sigmoid(logit)).
 *   n_accept  [n] int32 accepted prefix length of each block; the label of position k is
 *             y_k = [n_accept >= k].
 *   temps     [n_t] fp64 candidate temperatures (> 0), 1 <= n_t <= 65535.
 *   n_bins    equal-width ECE bins on [0, 1], 1..256; p lies in bin
 *             min(floor(p * n_bins), n_bins - 1).
 *   t_out     out [gamma] fp64 chosen temperature per position.
 *   ece_out   out [gamma] fp64 ECE of the cumulative product at the chosen temperatures.
 * For k = 1..gamma, with t_1..t_{k-1} chosen:
 *   p_{s,k}(t) = prod_{i<k} sigmoid(logit_{s,i} / t_i) * sigmoid(logit_{s,k} / t)   (fp64)
 *   ECE_k(t)   = sum over bins of (|bin| / n) |mean p - mean y_k| = sum |sum p - sum y| / n
 *   t_k        = the grid value with the smallest ECE_k (the first on exact ties).
 * The bin sums are accumulated as integers (p in units of 2^-40), so the result does not
 * depend on the order of accumulation.  Workspace: dspark_sts_workspace_bytes(n, n_t,
 * n_bins) bytes.
 */
size_t dspark_sts_workspace_bytes(int32_t n, int32_t n_t, int32_t n_bins);
dspark_status dspark_sts_calibrate(int32_t n, int32_t gamma, const float* logit,
                                   const int32_t* n_accept, const double* temps, int32_t n_t,
                                   int32_t n_bins, double* t_out, double* ece_out, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * Hardware-aware prefix scheduler [XTL §6; CSDN throughput objective and the quotes of
 * paper Sec. 3.2.2 in its roundtable], run entirely on the GPU.
 *   a_{b,j} = prod_{i<=j} c_{b,i}   (fp64, multiplied left to right from 1)
 *   N       = sum_b (ell_b + 1)     (the +1 is the target's bonus/corrected slot)
 *   tau     = sum_b (1 + sum_{j<=ell_b} a_{b,j})
 *   Theta   = tau * sps[N]
 * GREEDY: candidates (b, j) ordered by a descending, then b ascending, then j ascending,
 * are admitted one at a time from ell = 0 (tau = B, N = B), tau and Theta updated in fp64
 * in that order; the walk stops at the first candidate whose Theta <= the best Theta so
 * far.  FULL: every candidate is admitted (ell_b = gamma).  Other modes: DSPARK_E_VALUE.
 *   c      [B][gamma] fp32 confidences in [0, 1] (sigmoid outputs).  Values above 1 are
 *          not rejected: the order and the walk are still exact, but a can then grow
 *          along a request, and ell_b is the largest admitted j, which need not be a
 *          prefix of what was admitted.
 *   sps    [B*(gamma+1)+1] fp64 target steps per second at N verify tokens.
 *   ell    out [B] int32 verify lengths in 0..gamma.
 *   theta  out [1] fp64 final Theta; n_total out [1] int32 final N.
 * Needs no workspace (pass NULL, 0); B * gamma <= 4096.
 */
dspark_status dspark_schedule(int32_t batch, int32_t gamma, const float* c, const double* sps,
                              int mode, int32_t* ell, double* theta, int32_t* n_total,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * Dynamic top-K admission [XTL §7, the production form of the scheduler: candidates are
 * still ordered by the latest confidences, but the truncation length is predicted from
 * the confidences of two steps earlier, so the next batch size is known ahead and the
 * admission depends on history only].
 *   k_admit  number of draft tokens to admit beyond the B bonus slots (for instance
 *            n_total - B of a dspark_schedule made two steps earlier); values above
 *            B * gamma admit everything.  Negative: DSPARK_E_VALUE.
 * The first k_admit candidates in dspark_schedule's order (a descending, b ascending,
 * j ascending; a in fp64 as there) are admitted; tau accumulates along them in that order
 * and Theta = tau * sps[N] with N = B + k_admit.  Since a never increases along a request
 * (c <= 1), every admission is a prefix: ell_b = the largest admitted j of request b.
 * c, sps, ell, theta and n_total as for dspark_schedule; needs no workspace (NULL, 0);
 * B * gamma <= 4096.
 */
dspark_status dspark_schedule_topk(int32_t batch, int32_t gamma, const float* c,
                                   const double* sps, int32_t k_admit, int32_t* ell,
                                   double* theta, int32_t* n_total, void* ws, size_t ws_bytes,
                                   void* stream);

/*
 * Rejection-sampling verification [XTL §1; AIMSG concept 2; accept probability
 * min(1, p_t/p_d) as quoted in the CSDN roundtable].  For every request b, with
 * p_t,k = softmax(T[b][k-1] / temperature) and p_d,k the draft distribution:
 *   for k = 1..ell_b: accept x_k iff u(seed, b, k, 1, 0) * p_d,k(x_k) < p_t,k(x_k),
 *                     with p_d,k(x_k) = exp(logp[b][k-1]); stop at the first rejection;
 *   n_b = number of leading accepts;
 *   if n_b < ell_b:   j = n_b + 1, y = argmax_{v: rho_v > 0} (ln rho_v + G(seed,b,j,2,v))
 *                     where rho = max(0, p_t,j - p_d,j) (the normalised residual; p_d,j is
 *                     recomputed from U, W1, W2t with lse[b][j-1]); if rounding leaves
 *                     every rho_v = 0, y is drawn from p_t,j with the same noise;
 *   else:             y = argmax_v (T[b][ell_b][v] / temperature + G(seed, b, ell_b+1, 2, v)),
 *                     the bonus token drawn from p_t at position ell_b + 1.
 * Arguments:
 *   U, W1, W2t, wdt, anchor, tokens as for the draft; logp, lse: the draft's outputs.
 *   T          [B][gamma+1][V] fp32 target logits (row k-1 is position k).
 *   ell        [B] int32 verify lengths (e.g. from dspark_schedule).
 *   n_accept   out [B] int32.
 *   out_tokens out [B][gamma+1] int32: x_1..x_{n_b}, y, then -1.
 *   pt_tok     out [B][gamma] fp32 p_t,k(x_k) for k <= ell_b (NaN elsewhere), or NULL.
 */
dspark_status dspark_verify(const dspark_dims* dims, const float* U, const void* W1,
                            const void* W2t, int wdt, const int32_t* anchor,
                            const int32_t* tokens, const float* logp, const float* lse,
                            const float* T, const int32_t* ell, float temperature,
                            uint64_t seed, int32_t* n_accept, int32_t* out_tokens,
                            float* pt_tok, void* ws, size_t ws_bytes, void* stream);

/*
 * Analytic accept rate [CSDN Eq. 8; XTL §5: 1 - |p_d - p_t|_1 / 2, computed on the
 * softmaxed draft and target logits]:
 *   alpha[b][k-1] = sum_v min(p_d,k(v), p_t,k(v)),   k = 1..gamma,
 * with the tempered draft distribution of position k given tokens (p_d,k = exp(z - lse),
 * lse from the draft) and p_t,k = softmax(T[b][k-1] / temperature).
 */
dspark_status dspark_accept_rate_tv(const dspark_dims* dims, const float* U, const void* W1,
                                    const void* W2t, int wdt, const int32_t* anchor,
                                    const int32_t* tokens, const float* lse, const float* T,
                                    float temperature, float* alpha, void* ws,
                                    size_t ws_bytes, void* stream);

/*
 * A closed loop of `rounds` rounds on `stream`, with no host synchronisation between them.
 * Round t (0-based) drafts from anchor_t (anchor_0 = anchor, later the last token the
 * previous round emitted), scores the block with the confidence head, schedules it
 * (sched_mode as for dspark_schedule), builds the stand-in target logits and verifies,
 * each call as documented above with seed_t = seed + t.  sched_mode GREEDY or FULL schedules
 * every round with dspark_schedule; TOPK_DELAYED is the production form of [XTL §7]: round
 * t admits the first K_t candidates in dspark_schedule's order of its own confidences
 * (dspark_schedule_topk), where K_t = N - B of the greedy schedule of round t - 2's
 * confidences, read on the device, so the admitted count of a round is known two rounds
 * ahead and depends on history only; rounds 0 and 1, which have no such history, take
 * K from their own greedy schedule, i.e. are scheduled greedily.  ell, theta and n_total
 * report the admission made.  The accepted length of request b
 * in round t is n_accept + 1 tokens; the latency per token of the speculative loop is
 * (T_draft + T_verify) / tau [CSDN Eq. 1].
 * Stand-in target (a synthetic Markov chain over tokens, not part of the method): position
 * j + 1 (j = 0..gamma) of request b has logits
 *   T[b][j][v] = U[b][min(j, gamma-1)][v] + target_sigma sqrt(3) (2 u - 1),
 *   u = u(target_seed, prev, 0, 3, v),   prev = anchor_t[b] (j = 0) or tokens[b][j-1],
 * a zero-mean transition term of variance target_sigma^2 keyed by the previous token.
 * Arguments: dims, U, W1, W2t, wdt, temperature as for dspark_draft_markov; h, hdt, w, wvdt
 * as for dspark_confidence; sps, sched_mode as for dspark_schedule; target_sigma >= 0.
 * Outputs, one slice per round (row-major, round first):
 *   anchors [R][B] (or NULL), tokens [R][B][gamma], c [R][B][gamma], ell [R][B],
 *   theta [R] (or NULL), n_total [R], n_accept [R][B], out_tokens [R][B][gamma+1],
 *   pt_tok [R][B][gamma] (or NULL).
 * rounds in 1..65536; B * gamma <= 4096 (the scheduler's limit), else DSPARK_E_SHAPE before
 * anything is enqueued.  Workspace: dspark_loop_workspace_bytes(dims) bytes (it holds one
 * round's target logits, B (gamma+1) V floats).
 */
size_t dspark_loop_workspace_bytes(const dspark_dims* dims);
dspark_status dspark_closed_loop(const dspark_dims* dims, const float* U, const void* W1,
                                 const void* W2t, int wdt, const void* h, int hdt,
                                 const void* w, int wvdt, const int32_t* anchor,
                                 const double* sps, int sched_mode, float temperature,
                                 uint64_t seed, float target_sigma, uint64_t target_seed,
                                 int32_t rounds, int32_t* anchors, int32_t* tokens, float* c,
                                 int32_t* ell, double* theta, int32_t* n_total,
                                 int32_t* n_accept, int32_t* out_tokens, float* pt_tok,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * The closed loop's stand-in target on its own (not a step of the method; measurement and
 * test support): T [B][gamma+1][V] fp32 with
 *   T[b][j][v] = U[b][min(j, gamma-1)][v] + target_sigma sqrt(3) (2 u - 1),
 *   u = u(target_seed, prev, 0, 3, v),   prev = anchor[b] (j = 0) or tokens[b][j-1],
 * exactly the logits dspark_closed_loop verifies against, so that the target side of a
 * round can be timed apart from the loop.  U, anchor, tokens as for dspark_draft_markov;
 * target_sigma >= 0 (else DSPARK_E_VALUE).  Needs no workspace.
 */
dspark_status dspark_markov_target(const dspark_dims* dims, const float* U,
                                   const int32_t* anchor, const int32_t* tokens,
                                   float target_sigma, uint64_t target_seed, float* T,
                                   void* stream);

/*
 * Distribution-matching training loss of the draft and confidence heads, forward and
 * backward [XTL §9: a cross-entropy term on the true next token, an L1 (total-variation)
 * term between the draft and target distributions, a binary cross-entropy term training
 * the confidence head on the soft accept rate, position weights exp(-(k-1)/gamma); XTL §5:
 * the soft label 1 - |p_d - p_t|_1 / 2 from the two softmaxes; XTL §8: the open
 * configuration weighs the terms 0.1, 0.9 and 1.0].  For each row (b, k), k = 1..gamma:
 *   p_d = softmax(zd[b][k-1]), p_t = softmax(zt[b][k-1]), y = labels[b][k-1]
 *   ce  = -log p_d(y),  l1 = sum_v |p_d(v) - p_t(v)|,  a = 1 - l1 / 2 (a fixed target)
 *   bce = log(1 + exp(l)) - a l,  l = conf_logit[b][k-1],  c = sigmoid(l)
 *   loss = sum_{b,k} w_k (alpha_ce ce + alpha_l1 l1 + alpha_conf bce) / (B sum_k w_k),
 *          w_k = exp(-(k-1)/gamma)
 *   grad_zd[j]  = w_k / (B sum w) (alpha_ce (p_d(j) - [j = y]) + alpha_l1 p_d(j) (s_j - S)),
 *                 s_j = sign(p_d(j) - p_t(j)) (0 at equality), S = sum_v s_v p_d(v)
 *   grad_conf   = w_k / (B sum w) alpha_conf (c - a)
 * The soft label is held fixed: the confidence term sends no gradient into zd.
 *   zd, zt      [B][gamma][V] fp32 draft and target logits, 1 <= V <= 2^22.
 *   labels      [B][gamma] int32 true next tokens (clamped into [0, V) where used).
 *   conf_logit  [B][gamma] fp32 confidence-head logits.
 *   alpha_*     finite term weights (else DSPARK_E_VALUE).
 *   loss        out [1] fp64; NaN if the workgroups of a row failed to meet (see below).
 *   terms       out [B][gamma][3] fp32 (ce, l1, bce) per row, or NULL.
 *   grad_zd     out [B][gamma][V] fp32, or NULL (forward only).
 *   grad_conf   out [B][gamma] fp32, or NULL.
 * One cooperative launch: the vocabulary of a row is split over up to 1024 workgroups that
 * exchange partial sums through the workspace and wait for each other with bounded polls;
 * DSPARK_E_HIP if the device cannot run the grid resident at once.  Rows run in a fixed
 * order and every sum has a fixed order, so results are bit-reproducible.  Workspace:
 * dspark_loss_workspace_bytes(B, gamma, V) bytes.
 */
size_t dspark_loss_workspace_bytes(int32_t batch, int32_t gamma, int32_t vocab);
dspark_status dspark_draft_loss(int32_t batch, int32_t gamma, int32_t vocab, const float* zd,
                                const float* zt, const int32_t* labels,
                                const float* conf_logit, double alpha_ce, double alpha_l1,
                                double alpha_conf, double* loss, float* terms,
                                float* grad_zd, float* grad_conf, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * The uniforms of the random-number definition above, for checking the generator:
 *   out[i] = u(seed, b, k, s, v0 + i), i < n   (fp32; every value is exact in fp32).
 */
dspark_status dspark_rng_uniforms(uint64_t seed, uint32_t b, uint32_t k, uint32_t s,
                                  uint32_t v0, int64_t n, float* out, void* stream);

/*
 * The Gumbel transform of the random-number definition above, as the kernels evaluate it
 * in fp32, on the whole lattice of uniforms (for checking it exhaustively):
 *   out[m], m = 0 .. 2^23 - 1 (out holds 2^23 floats), for u = (2m + 1) * 2^-24;
 *   form 0: G = -ln(-ln u), the form of the row kernels;
 *   form 1: -log2(-log2 u), the base-2 score offset of the matrix-core kernels (it equals
 *           G / ln 2 - log2(ln 2); the constant shifts every candidate of a race alike).
 * Both use the hardware base-2 logarithm.  Measured against fp64 on every lattice point,
 * the error is within 3 * 2^-23 * (1 + |value|) (ULP-scale: about 3.6e-7 absolute near 0
 * and 2.2e-5 relative to |value| ~ 17 at u -> 1) -- far inside the 1e-4 score gap below
 * which a sampled token may differ from an exact sampler's.
 * Errors: DSPARK_E_NULL, DSPARK_E_VALUE (form not 0 or 1), DSPARK_E_HIP.
 */
dspark_status dspark_gumbel_lattice(int form, float* out, void* stream);

/*
 * Launch timing (measurement support, not part of the method).  Between
 * dspark_profile_start and dspark_profile_stop the launches of the sampling kernel of
 * each dspark_draft_markov call (one launch per draft position, or one launch for all
 * positions of the call) are bracketed by one pair of HIP events on the call's stream, for
 * at most max_launches launches (1..65536; events are created on the first call and
 * kept).  dspark_profile_stop waits for the recorded events and returns the mean duration
 * per launch in milliseconds (the bracketed time over the number of launches, so the
 * dispatch gaps between a call's consecutive launches are counted in), the number of
 * launches, and the mean number of draft positions one launch covered.  Not thread-safe; meant for
 * one timing loop at a time.  Errors: DSPARK_E_VALUE (max_launches out of range),
 * DSPARK_E_NULL, DSPARK_E_HIP (event creation or timing failed).
 */
dspark_status dspark_profile_start(int max_launches);
dspark_status dspark_profile_stop(double* mean_ms, int* launches,
                                  double* positions_per_launch);

/*
 * Failure-path testing (not part of the method, not for production use).  The cooperative
 * kernels (the resident draft of dspark_draft_markov for up to 16 requests, and
 * dspark_draft_loss) bound every wait on other workgroups: a wait that runs past its poll
 * limit raises the call's fault word, every workgroup leaves, and the call reports its
 * failure in its outputs (draft: every token -1, logp and lse NaN; loss: NaN).  With
 * polls >= 0, later calls in this process limit each such wait to `polls` polls and make
 * the completion it looks for unreachable, so that every wait gives up and the failure is
 * reported while every kernel still ends; polls < 0 restores normal operation (2^22 polls,
 * reachable completions).  Process-wide, on every device.  Always DSPARK_OK.
 */
dspark_status dspark_test_wait_limit(int32_t polls);

/*
 * Achievable HBM read rate (measurement support, not part of the method).  Times `reps`
 * launches of a plain streaming-read kernel (16-byte loads, every byte read once, nothing
 * written) on `stream`; launch i reads the i-th of the buf_bytes / launch_bytes regions of
 * `buf` in turn, so that consecutive launches do not hit data left in the caches.  Writes
 * the mean duration of one launch in milliseconds to *mean_ms; waits for its own events.
 * buf: device memory, 16-byte aligned, owned by the caller; launch_bytes: a multiple of 16,
 * 16 <= launch_bytes <= buf_bytes; reps: 1..10000; sink: one device float the kernel may
 * write.  Errors: DSPARK_E_NULL, DSPARK_E_SHAPE (sizes or alignment), DSPARK_E_VALUE
 * (reps), DSPARK_E_HIP (launch or events).
 */
dspark_status dspark_stream_read_probe(const void* buf, size_t buf_bytes, size_t launch_bytes,
                                       int reps, float* sink, double* mean_ms, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H */
