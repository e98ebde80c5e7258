/*
 * dspark_oracle.c -- plain, slow, fp64 CPU oracle for one DSpark draft/verify round.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load or call this file:
 * only the test-suite, the smoke check and the benchmark's CPU-baseline leg do.  It
 * shares no code, header, table or helper with the HIP library; the two meet only in
 * the seeded input generator and in the published definition of the random-number
 * generator, which each side implements on its own.
 *
 * Sources (web pages describing DSpark; cited by short name below):
 *   [XTL]   "[DeepSeek-6] DSpark: From Draft Models to Serving-Aware Speculative
 *           Decoding" (xutianle.me), numbered sections 1-13.
 *   [CSDN]  "DSpark: Confidence-Scheduled Speculative Decoding with Semi-Autoregressive
 *           Generation -- 研读报告" (devpress.csdn.net), "关键公式与解释": Eq. 1, 4, 7, 8
 *           and the throughput objective; roundtable quotes of paper Sec. 3.2.2.
 *   [AIMSG] "DeepSeek DSpark 深度解读：系统工程与模型协同的极致优化" (aimsg.uk),
 *           concepts 1-10.
 *   [SALMON] J. Salmon, M. Moraes, R. Dror, D. Shaw, "Parallel Random Numbers: As Easy
 *           as 1, 2, 3", SC'11 -- definition of Philox4x32.
 *
 * Everything is computed in IEEE double precision, one element at a time, in the order
 * the definitions state.  Build with contraction off (-ffp-contract=off) so that every
 * product and sum rounds on its own.
 *
 * Parity status of each function (what pins it is listed in the test-suite):
 *   ora_philox4x32, ora_uniform ........ pinned (published known-answer vectors, uniformity)
 *   ora_draft .......................... pinned (normalisation, W2=0 softmax special case,
 *                                        Gumbel-max sampling law by chi-square)
 *   ora_confidence ..................... pinned (w=0, unit-vector w special cases)
 *   ora_schedule ....................... pinned (brute force over all prefix lengths,
 *                                        closed-form special cases)
 *   ora_schedule_topk .................. pinned (brute force over all prefix lengths of a
 *                                        given total, agreement with ora_schedule at its
 *                                        own admitted count, Monte-Carlo losslessness)
 *   ora_sts_calibrate .................. pinned (recovery of known per-position
 *                                        temperatures, hand-computed ECE, one-value grids)
 *   ora_markov_target .................. pinned (depends on the previous token only,
 *                                        moments of the uniform transition term); the
 *                                        closed loop's stand-in target, not a step of
 *                                        the method
 *   ora_draft_loss ..................... pinned (central finite differences of the loss,
 *                                        p_d = p_t and one-hot special cases)
 *   ora_verify ......................... pinned (Monte-Carlo losslessness against the
 *                                        target law, special cases)
 *   ora_accept_tv ...................... pinned (TV identity, Monte-Carlo acceptance rate)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------ */
/* Random numbers: Philox4x32 with 10 rounds [SALMON], used as a counter-based hash.     */
/* ------------------------------------------------------------------------------------ */
#define ORA_PHILOX_ROUNDS 10

/* One Philox4x32 evaluation [SALMON, Sec. on Philox]: each round multiplies counter words
 * 0 and 2 by the two Philox constants, and the new counter is (hi(p1) ^ c1 ^ k0, lo(p1),
 * hi(p0) ^ c3 ^ k1, lo(p0)); the key is bumped by the two Weyl constants between rounds. */
void ora_philox4x32(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < ORA_PHILOX_ROUNDS; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)p1;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The uniform keyed on (seed, request, position, stream, vocab index):
 *   W = word (v mod 4) of Philox4x32-10(counter = (v div 4, k, b, s), key = (seed lo, seed hi))
 *   u = (2 * (W >> 9) + 1) * 2^-24,
 * an odd multiple of 2^-24 strictly inside (0, 1); it is exact in fp32 and fp64.
 * Streams: 0 = draft sample, 1 = accept test (v = 0), 2 = residual / bonus sample. */
double ora_uniform(uint64_t seed, uint32_t b, uint32_t k, uint32_t s, uint32_t v)
{
    uint32_t ctr[4] = { v >> 2, k, b, s };
    uint32_t key[2] = { (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32) };
    uint32_t w[4];
    ora_philox4x32(ctr, key, w);
    uint32_t word = w[v & 3u];
    return ldexp(2.0 * (double)(word >> 9) + 1.0, -24);
}

/* Standard Gumbel variate from the uniform: G = -ln(-ln u). */
static double ora_gumbel(uint64_t seed, uint32_t b, uint32_t k, uint32_t s, uint32_t v)
{
    return -log(-log(ora_uniform(seed, b, k, s, v)));
}

/* Convenience loop for tests: out[i] = u(seed, b, k, s, v0 + i), i < n. */
void ora_uniform_fill(uint64_t seed, uint32_t b, uint32_t k, uint32_t s, uint32_t v0,
                      int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = ora_uniform(seed, b, k, s, v0 + (uint32_t)i);
}

/* ------------------------------------------------------------------------------------ */
/* Shared shape of the round.                                                            */
/* ------------------------------------------------------------------------------------ */
typedef struct {
    int32_t batch;   /* B: number of requests passed in (rows of every [B][...] array)   */
    int32_t gamma;   /* draft length                                                       */
    int32_t vocab;   /* V                                                                  */
    int32_t rank;    /* r: Markov-head rank                                                */
    int32_t hidden;  /* d: backbone hidden size                                            */
} ora_dims;

/* Global request id of row b (the id keys the random numbers). */
static uint32_t gid_of(const int32_t* gid, int b) { return gid ? (uint32_t)gid[b] : (uint32_t)b; }

/* Token that position k (1-based) conditions on: the anchor for k = 1, else x_{k-1}
 * ([XTL §3]: the anchor is the first predicted position, so x_0 = anchor). */
static int32_t prev_token(const int32_t* anchor, const int32_t* tokens, int gamma, int b, int k)
{
    return (k == 1) ? anchor[b] : tokens[(size_t)b * gamma + (k - 2)];
}

/* Draft logits of one position [CSDN Eq. 4; XTL §4 Markov head]:
 *   z_v = (U_k(v) + sum_i W1[prev, i] * W2[i, v]) / temperature,
 * with W2 stored transposed as W2t[v][i] (the weight of a bias-free linear map r -> V). */
static void draft_logits(const ora_dims* dm, const double* Urow, const double* W1,
                         const double* W2t, int32_t prev, double temperature, double* z)
{
    const int V = dm->vocab, r = dm->rank;
    const double* a = W1 + (size_t)prev * r;
    for (int v = 0; v < V; ++v) {
        const double* w = W2t + (size_t)v * r;
        double bias = 0.0;
        for (int i = 0; i < r; ++i) bias += a[i] * w[i];
        z[v] = (Urow[v] + bias) / temperature;
    }
}

/* log sum_v exp(z_v), shifted by the maximum. */
static double logsumexp(const double* z, int V)
{
    double m = -INFINITY;
    for (int v = 0; v < V; ++v) if (z[v] > m) m = z[v];
    double s = 0.0;
    for (int v = 0; v < V; ++v) s += exp(z[v] - m);
    return m + log(s);
}

/* ------------------------------------------------------------------------------------ */
/* Draft: gamma sequential Markov-head steps, each a full softmax and a Gumbel-max draw.  */
/* ------------------------------------------------------------------------------------ */
/* For k = 1..gamma and every request b:
 *   prev = x_{k-1}  (anchor at k = 1, or forced[b][k-2] when a forced prefix is given),
 *   z    = draft logits of position k given prev,
 *   lse  = log sum_v exp z_v,   p_v = exp(z_v - lse),
 *   x_k  = argmax_v (z_v + G(seed, b, k, 0, v)), lowest v on exact ties (Gumbel-max: the
 *          argmax is distributed as p),
 *   logp = z_{x_k} - lse.
 * gap[b][k] is the score margin between the best and second-best candidates (used to
 * excuse near-tie mismatches).  probs, when not NULL, receives every p row [B][gamma][V]. */
void ora_draft(const ora_dims* dm, const double* U, const double* W1, const double* W2t,
               const int32_t* anchor, const int32_t* forced, const int32_t* gid,
               double temperature, uint64_t seed, int32_t* tokens, double* logp,
               double* lse_out, double* gap, double* probs)
{
    const int B = dm->batch, G = dm->gamma, V = dm->vocab;
    double* z = (double*)malloc(sizeof(double) * (size_t)V);
    for (int b = 0; b < B; ++b) {
        for (int k = 1; k <= G; ++k) {
            int32_t prev = prev_token(anchor, forced ? forced : tokens, G, b, k);
            const double* Urow = U + ((size_t)b * G + (k - 1)) * V;
            draft_logits(dm, Urow, W1, W2t, prev, temperature, z);
            double lse = logsumexp(z, V);
            double best = -INFINITY, second = -INFINITY;
            int32_t arg = 0;
            for (int v = 0; v < V; ++v) {
                double score = z[v] + ora_gumbel(seed, gid_of(gid, b), (uint32_t)k, 0u, (uint32_t)v);
                if (score > best) { second = best; best = score; arg = v; }
                else if (score > second) { second = score; }
            }
            size_t o = (size_t)b * G + (k - 1);
            tokens[o] = arg;
            logp[o] = z[arg] - lse;
            lse_out[o] = lse;
            if (gap) gap[o] = best - second;
            if (probs) {
                double* p = probs + o * V;
                for (int v = 0; v < V; ++v) p[v] = exp(z[v] - lse);
            }
        }
    }
    free(z);
}

/* ------------------------------------------------------------------------------------ */
/* Confidence head [CSDN Eq. 7; XTL §5]: c_k = sigmoid(w . [h_k ; W1[x_{k-1}]]).          */
/* ------------------------------------------------------------------------------------ */
/* w has d + r entries in the concatenation order [h ; W1 row]; there is no bias term. */
/* With temps (may be NULL) the head is the calibrated one [XTL §5, sequential temperature
 * scaling]: c = 1 / (1 + exp(-logit / temps[k-1])). */
void ora_confidence(const ora_dims* dm, const double* h, const double* W1, const double* w,
                    const int32_t* anchor, const int32_t* tokens, const double* temps,
                    double* c)
{
    const int B = dm->batch, G = dm->gamma, d = dm->hidden, r = dm->rank;
    for (int b = 0; b < B; ++b) {
        for (int k = 1; k <= G; ++k) {
            const double* hk = h + ((size_t)b * G + (k - 1)) * d;
            const double* e = W1 + (size_t)prev_token(anchor, tokens, G, b, k) * r;
            double logit = 0.0;
            for (int j = 0; j < d; ++j) logit += w[j] * hk[j];
            for (int i = 0; i < r; ++i) logit += w[d + i] * e[i];
            if (temps) logit = logit / temps[k - 1];
            c[(size_t)b * G + (k - 1)] = 1.0 / (1.0 + exp(-logit));
        }
    }
}

/* ------------------------------------------------------------------------------------ */
/* Hardware-aware prefix scheduler [XTL §6; CSDN throughput objective; paper Sec. 3.2.2  */
/* as quoted in the CSDN roundtable].                                                    */
/* ------------------------------------------------------------------------------------ */
typedef struct { double a; int32_t b; int32_t j; } ora_cand;

/* Candidate order: survival a descending, then request ascending, then position ascending. */
static int cand_cmp(const void* x, const void* y)
{
    const ora_cand* p = (const ora_cand*)x;
    const ora_cand* q = (const ora_cand*)y;
    if (p->a > q->a) return -1;
    if (p->a < q->a) return 1;
    if (p->b != q->b) return p->b < q->b ? -1 : 1;
    if (p->j != q->j) return p->j < q->j ? -1 : 1;
    return 0;
}

/* Inputs: c[B][gamma] confidences (the fp32 values, widened exactly), sps[N] for
 * N = 0..B*(gamma+1) (target steps per second at N verify tokens), mode 0 = greedy with
 * early stop, mode 1 = full block.
 *   a_{b,j} = prod_{i<=j} c_{b,i}            (prefix survival, multiplied left to right)
 *   N       = sum_b (ell_b + 1)              (the +1 is the target's bonus/corrected slot)
 *   tau     = sum_b (1 + sum_{j<=ell_b} a_{b,j})   (expected output tokens)
 *   Theta   = tau * SPS(N)
 * Greedy: start from ell = 0 (N = B, tau = B); take candidates in order, each adding one
 * verify token; stop at the first candidate whose Theta' <= best Theta so far.
 * Outputs ell[B], theta (the final Theta) and n_total (the final N). */
void ora_schedule(int32_t B, int32_t gamma, const double* c, const double* sps, int32_t mode,
                  int32_t* ell, double* theta, int32_t* n_total)
{
    size_t n = (size_t)B * gamma;
    ora_cand* cand = (ora_cand*)malloc(sizeof(ora_cand) * (n ? n : 1));
    for (int b = 0; b < B; ++b) {
        double a = 1.0;
        for (int j = 1; j <= gamma; ++j) {
            a = a * c[(size_t)b * gamma + (j - 1)];
            cand[(size_t)b * gamma + (j - 1)] = (ora_cand){ a, b, j };
        }
        ell[b] = 0;
    }
    qsort(cand, n, sizeof(ora_cand), cand_cmp);
    int32_t N = B;
    double tau = (double)B;
    double best = tau * sps[N];
    for (size_t t = 0; t < n; ++t) {
        double tau_next = tau + cand[t].a;
        double theta_next = tau_next * sps[N + 1];
        if (mode == 0 && theta_next <= best) break;
        tau = tau_next;
        N = N + 1;
        best = theta_next;
        /* with every c <= 1 a request's candidates are taken in j order, so this is its
         * newest j; above 1 (outside the sigmoid's range) it is the largest admitted j */
        if (cand[t].j > ell[cand[t].b]) ell[cand[t].b] = cand[t].j;
    }
    *theta = best;
    *n_total = N;
    free(cand);
}

/* Dynamic top-K admission [XTL §7: in production the candidates are still ordered by the
 * latest confidences, but the truncation length is predicted from the confidences of two
 * steps earlier, so that the next batch size is known ahead and admission depends on
 * history only].  K is that length: the number of draft tokens admitted beyond the B
 * bonus slots, supplied by the caller (for instance n_total - B of a schedule made two
 * steps earlier) and clamped to [0, B*gamma].  The first K candidates in the order of
 * ora_schedule are admitted; tau, N and Theta accumulate along them exactly as there. */
void ora_schedule_topk(int32_t B, int32_t gamma, const double* c, const double* sps, int32_t K,
                       int32_t* ell, double* theta, int32_t* n_total)
{
    size_t n = (size_t)B * gamma;
    size_t take = K < 0 ? 0 : ((size_t)K > n ? n : (size_t)K);
    ora_cand* cand = (ora_cand*)malloc(sizeof(ora_cand) * (n ? n : 1));
    for (int b = 0; b < B; ++b) {
        double a = 1.0;
        for (int j = 1; j <= gamma; ++j) {
            a = a * c[(size_t)b * gamma + (j - 1)];
            cand[(size_t)b * gamma + (j - 1)] = (ora_cand){ a, b, j };
        }
        ell[b] = 0;
    }
    qsort(cand, n, sizeof(ora_cand), cand_cmp);
    int32_t N = B;
    double tau = (double)B;
    for (size_t t = 0; t < take; ++t) {
        tau = tau + cand[t].a;
        N = N + 1;
        if (cand[t].j > ell[cand[t].b]) ell[cand[t].b] = cand[t].j;
    }
    *theta = tau * sps[N];
    *n_total = N;
    free(cand);
}

/* ------------------------------------------------------------------------------------ */
/* Sequential temperature scaling of the confidence head [XTL §5: the scheduler needs     */
/* confidences whose values match acceptance rates, not only their order, so the product  */
/* of confidences is calibrated on held-out data from left to right; AIMSG, on STS: a     */
/* 1-D grid search per position over the cumulative product, minimising the expected      */
/* calibration error against the empirical prefix acceptance; temperature scaling keeps   */
/* the order of the confidences].                                                        */
/* ------------------------------------------------------------------------------------ */
/* n held-out drafted blocks: logit[s][k-1] is the confidence logit of position k
 * (c = 1 / (1 + exp(-logit))), n_accept[s] the accepted prefix length, so the label of
 * position k is y_{s,k} = [n_accept[s] >= k].  temps[0..n_t) is the grid, n_bins the
 * number of equal-width bins on [0, 1] (p falls in bin min(floor(p n_bins), n_bins - 1)).
 * For k = 1..gamma in order, with t_1..t_{k-1} already chosen:
 *   p_{s,k}(t) = prod_{i<k} c_{s,i}(t_i) * c_{s,k}(t),   c_{s,i}(t) = 1/(1+exp(-logit/t))
 *   ECE_k(t)   = sum over bins m of (|m| / n) * | mean_{s in m} p - mean_{s in m} y_k |
 *   t_k        = the grid value with the smallest ECE_k (the first one on exact ties).
 * Outputs t_out[k-1], ece_out[k-1] = ECE_k(t_k) and, if gap is not NULL, gap[k-1] = the
 * second-smallest ECE_k over the grid minus the smallest (+inf for a one-value grid). */
void ora_sts_calibrate(int32_t n, int32_t gamma, const double* logit, const int32_t* n_accept,
                       const double* temps, int32_t n_t, int32_t n_bins, double* t_out,
                       double* ece_out, double* gap)
{
    double* q = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    double* sp = (double*)malloc(sizeof(double) * (size_t)n_bins);
    double* sy = (double*)malloc(sizeof(double) * (size_t)n_bins);
    double* cnt = (double*)malloc(sizeof(double) * (size_t)n_bins);
    for (int s = 0; s < n; ++s) q[s] = 1.0;
    for (int k = 1; k <= gamma; ++k) {
        double best = INFINITY, second = INFINITY;
        int best_i = 0;
        for (int ti = 0; ti < n_t; ++ti) {
            const double t = temps[ti];
            for (int m = 0; m < n_bins; ++m) sp[m] = sy[m] = cnt[m] = 0.0;
            for (int s = 0; s < n; ++s) {
                const double c = 1.0 / (1.0 + exp(-logit[(size_t)s * gamma + (k - 1)] / t));
                const double p = q[s] * c;
                int m = (int)floor(p * n_bins);
                if (m >= n_bins) m = n_bins - 1;
                if (m < 0) m = 0;
                sp[m] += p;
                sy[m] += n_accept[s] >= k ? 1.0 : 0.0;
                cnt[m] += 1.0;
            }
            double ece = 0.0;
            for (int m = 0; m < n_bins; ++m)
                if (cnt[m] > 0.0) ece += (cnt[m] / n) * fabs(sp[m] / cnt[m] - sy[m] / cnt[m]);
            if (ece < best) {
                second = best;
                best = ece;
                best_i = ti;
            } else if (ece < second) {
                second = ece;
            }
        }
        t_out[k - 1] = temps[best_i];
        ece_out[k - 1] = best;
        if (gap) gap[k - 1] = second - best;
        for (int s = 0; s < n; ++s)
            q[s] = q[s] * (1.0 / (1.0 + exp(-logit[(size_t)s * gamma + (k - 1)] / t_out[k - 1])));
    }
    free(q);
    free(sp);
    free(sy);
    free(cnt);
}

/* ------------------------------------------------------------------------------------ */
/* Stand-in target for a closed loop of rounds (not a step of the method).  A synthetic   */
/* Markov target: the logits of position k = j + 1 (j = 0..gamma) of request b are the   */
/* draft's base logits plus a transition term that depends only on the previous token:   */
/*   T[b][j][v] = U[b][min(j, gamma-1)][v] + sigma sqrt(3) (2 u - 1),                     */
/*   u = u(seed, prev, 0, 3, v),  prev = anchor[b] (j = 0) or tokens[b][j-1],             */
/* with the random-number definition above (stream s = 3 reserved for it): a zero-mean    */
/* uniform term of variance sigma^2 per (previous token, next token) pair.               */
/* ------------------------------------------------------------------------------------ */
void ora_markov_target(int32_t B, int32_t gamma, int32_t V, const double* U,
                       const int32_t* anchor, const int32_t* tokens, double sigma,
                       uint64_t seed, double* T)
{
    const double scale = sigma * sqrt(3.0);
    for (int b = 0; b < B; ++b) {
        for (int j = 0; j <= gamma; ++j) {
            int prev = j == 0 ? anchor[b] : tokens[(size_t)b * gamma + (j - 1)];
            if (prev < 0) prev = 0;
            if (prev >= V) prev = V - 1;
            const int row = j < gamma ? j : gamma - 1;
            const double* base = U + ((size_t)b * gamma + row) * V;
            double* out = T + ((size_t)b * (gamma + 1) + j) * V;
            for (int v = 0; v < V; ++v) {
                const double u = ora_uniform(seed, (uint32_t)prev, 0u, 3u, (uint32_t)v);
                out[v] = base[v] + scale * (2.0 * u - 1.0);
            }
        }
    }
}

/* ------------------------------------------------------------------------------------ */
/* Distribution-matching training loss of the draft and confidence heads [XTL §9: a       */
/* cross-entropy term on the true next token, an L1 (total-variation) term between the    */
/* draft and target distributions, a binary cross-entropy term training the confidence    */
/* head on the soft accept rate 1 - |p_d - p_t|_1 / 2, position weights exp(-(k-1)/gamma);*/
/* XTL §8: the open configuration weights them 0.1, 0.9 and 1.0].                         */
/* ------------------------------------------------------------------------------------ */
/* Rows (b, k), k = 1..gamma, of draft logits zd and target logits zt ([B][gamma][V]):
 *   p_d = softmax(zd), p_t = softmax(zt)
 *   ce  = -log p_d(y)                       y = labels[b][k-1], the true next token
 *   l1  = sum_v |p_d(v) - p_t(v)|           (twice the total-variation distance)
 *   a   = 1 - l1 / 2                        the soft accept rate (a fixed target)
 *   bce = -(a log c + (1 - a) log(1 - c)),  c = sigmoid(conf_logit[b][k-1]),
 *         evaluated as log(1 + exp(l)) - a l
 *   w_k = exp(-(k-1)/gamma),  W = B * sum_k w_k
 *   loss = sum_{b,k} w_k (alpha_ce ce + alpha_l1 l1 + alpha_conf bce) / W
 * Gradients (a and p_t held fixed):
 *   dloss/dzd[j]  = w_k/W (alpha_ce (p_d(j) - [j = y]) + alpha_l1 p_d(j) (s_j - S)),
 *                   s_j = sign(p_d(j) - p_t(j)) (0 at equality), S = sum_v s_v p_d(v)
 *   dloss/dconf_logit = w_k/W alpha_conf (c - a)
 * terms[row][0..2] = (ce, l1, bce) when terms is not NULL. */
void ora_draft_loss(int32_t B, int32_t gamma, int32_t V, const double* zd, const double* zt,
                    const int32_t* labels, const double* conf_logit, double alpha_ce,
                    double alpha_l1, double alpha_conf, double* loss, double* terms,
                    double* grad_zd, double* grad_conf)
{
    double* pd = (double*)malloc(sizeof(double) * (size_t)V);
    double* pt = (double*)malloc(sizeof(double) * (size_t)V);
    double wsum = 0.0;
    for (int k = 1; k <= gamma; ++k) wsum += exp(-(double)(k - 1) / gamma);
    const double W = B * wsum;
    double total = 0.0;
    for (int b = 0; b < B; ++b) {
        for (int k = 1; k <= gamma; ++k) {
            const size_t row = (size_t)b * gamma + (k - 1);
            const double* xd = zd + row * V;
            const double* xt = zt + row * V;
            double md = xd[0], mt = xt[0];
            for (int v = 1; v < V; ++v) {
                if (xd[v] > md) md = xd[v];
                if (xt[v] > mt) mt = xt[v];
            }
            double sd = 0.0, st = 0.0;
            for (int v = 0; v < V; ++v) {
                sd += exp(xd[v] - md);
                st += exp(xt[v] - mt);
            }
            const double lse_d = md + log(sd), lse_t = mt + log(st);
            double l1 = 0.0, S = 0.0;
            for (int v = 0; v < V; ++v) {
                pd[v] = exp(xd[v] - lse_d);
                pt[v] = exp(xt[v] - lse_t);
                const double diff = pd[v] - pt[v];
                l1 += fabs(diff);
                S += (diff > 0.0 ? 1.0 : (diff < 0.0 ? -1.0 : 0.0)) * pd[v];
            }
            int y = labels[row];
            if (y < 0) y = 0;
            if (y >= V) y = V - 1;
            const double ce = lse_d - xd[y];
            const double a = 1.0 - 0.5 * l1;
            const double l = conf_logit[row];
            const double softplus = l > 0.0 ? l + log1p(exp(-l)) : log1p(exp(l));
            const double bce = softplus - a * l;
            const double c = 1.0 / (1.0 + exp(-l));
            const double wk = exp(-(double)(k - 1) / gamma) / W;
            total += wk * (alpha_ce * ce + alpha_l1 * l1 + alpha_conf * bce);
            if (terms) {
                terms[row * 3 + 0] = ce;
                terms[row * 3 + 1] = l1;
                terms[row * 3 + 2] = bce;
            }
            if (grad_zd) {
                for (int v = 0; v < V; ++v) {
                    const double diff = pd[v] - pt[v];
                    const double sv = diff > 0.0 ? 1.0 : (diff < 0.0 ? -1.0 : 0.0);
                    grad_zd[row * V + v] =
                        wk * (alpha_ce * (pd[v] - (v == y ? 1.0 : 0.0)) + alpha_l1 * pd[v] * (sv - S));
                }
            }
            if (grad_conf) grad_conf[row] = wk * alpha_conf * (c - a);
        }
    }
    *loss = total;
    free(pd);
    free(pt);
}

/* ------------------------------------------------------------------------------------ */
/* Verification by rejection sampling [XTL §1; AIMSG concept 2; CSDN roundtable on the   */
/* accept probability min(1, p_t/p_d)].                                                  */
/* ------------------------------------------------------------------------------------ */
/* For each request b, with p_d,k the draft distribution of position k given the drafted
 * prefix (recomputed here) and p_t,k = softmax(T[b][k] / temperature):
 *   for k = 1..ell_b: accept x_k iff u(seed, b, k, 1, 0) * p_d,k(x_k) < p_t,k(x_k),
 *                     i.e. with probability min(1, p_t/p_d); stop at the first rejection;
 *   n_b = number of leading accepts;
 *   if n_b < ell_b:   j = n_b + 1, rho = max(0, p_t,j - p_d,j) (the normalised residual),
 *                     y = argmax_{v: rho_v > 0} (ln rho_v + G(seed, b, j, 2, v));
 *                     when every rho_v is 0 (reachable only through rounding) y is drawn
 *                     from p_t,j with the same Gumbel numbers instead;
 *   else:             j = ell_b + 1, y = argmax_v (ln p_t,j(v) + G(seed, b, j, 2, v)), the
 *                     bonus token;
 *   output x_1..x_{n_b}, y, then -1 padding up to gamma + 1 entries.
 * Diagnostics (any may be NULL): pt_tok[b][k-1] = p_t,k(x_k) for k <= ell_b (NaN after);
 * margin[b][k-1] = |u p_d(x_k) - p_t(x_k)| / p_t(x_k) of each test made (NaN otherwise);
 * gap[b] = top-2 score margin of the final draw; kind[b] = 0 bonus, 1 residual,
 * 2 residual that fell back to p_t. */
void ora_verify(const ora_dims* dm, const double* U, const double* W1, const double* W2t,
                const int32_t* anchor, const int32_t* tokens, const double* T,
                const int32_t* ell, const int32_t* gid, double temperature, uint64_t seed,
                int32_t* n_accept, int32_t* out_tokens, double* pt_tok, double* margin,
                double* gap, int32_t* kind)
{
    const int B = dm->batch, G = dm->gamma, V = dm->vocab;
    double* zd = (double*)malloc(sizeof(double) * (size_t)V);
    double* zt = (double*)malloc(sizeof(double) * (size_t)V);
    for (int b = 0; b < B; ++b) {
        const uint32_t gb = gid_of(gid, b);
        const int L = ell[b];
        for (int k = 1; k <= G; ++k) {
            if (pt_tok) pt_tok[(size_t)b * G + (k - 1)] = NAN;
            if (margin) margin[(size_t)b * G + (k - 1)] = NAN;
        }
        int n = 0, rejected = 0;
        for (int k = 1; k <= L; ++k) {
            const int32_t x = tokens[(size_t)b * G + (k - 1)];
            const double* Trow = T + ((size_t)b * (G + 1) + (k - 1)) * V;
            for (int v = 0; v < V; ++v) zt[v] = Trow[v] / temperature;
            double pt = exp(zt[x] - logsumexp(zt, V));
            if (pt_tok) pt_tok[(size_t)b * G + (k - 1)] = pt;
            if (rejected) continue;
            draft_logits(dm, U + ((size_t)b * G + (k - 1)) * V, W1, W2t,
                         prev_token(anchor, tokens, G, b, k), temperature, zd);
            double pd = exp(zd[x] - logsumexp(zd, V));
            double u = ora_uniform(seed, gb, (uint32_t)k, 1u, 0u);
            if (margin) margin[(size_t)b * G + (k - 1)] = fabs(u * pd - pt) / pt;
            if (u * pd < pt) ++n;
            else rejected = 1;
        }
        int32_t* out = out_tokens + (size_t)b * (G + 1);
        for (int i = 0; i <= G; ++i) out[i] = -1;
        for (int i = 0; i < n; ++i) out[i] = tokens[(size_t)b * G + i];

        const int j = (n < L) ? n + 1 : L + 1;
        const double* Trow = T + ((size_t)b * (G + 1) + (j - 1)) * V;
        for (int v = 0; v < V; ++v) zt[v] = Trow[v] / temperature;
        const double lt = logsumexp(zt, V);
        int mode = 0;
        if (n < L) {
            draft_logits(dm, U + ((size_t)b * G + (j - 1)) * V, W1, W2t,
                         prev_token(anchor, tokens, G, b, j), temperature, zd);
            const double ld = logsumexp(zd, V);
            mode = 2;
            for (int v = 0; v < V; ++v) {
                double rho = exp(zt[v] - lt) - exp(zd[v] - ld);
                zd[v] = rho > 0.0 ? rho : 0.0;
                if (zd[v] > 0.0) mode = 1;
            }
        }
        double best = -INFINITY, second = -INFINITY;
        int32_t arg = 0;
        for (int v = 0; v < V; ++v) {
            double base;
            if (mode == 1) {
                if (!(zd[v] > 0.0)) continue;
                base = log(zd[v]);
            } else {
                base = zt[v] - lt;
            }
            double score = base + ora_gumbel(seed, gb, (uint32_t)j, 2u, (uint32_t)v);
            if (score > best) { second = best; best = score; arg = v; }
            else if (score > second) { second = score; }
        }
        out[n] = arg;
        n_accept[b] = n;
        if (gap) gap[b] = best - second;
        if (kind) kind[b] = mode;
    }
    free(zd);
    free(zt);
}

/* ------------------------------------------------------------------------------------ */
/* Analytic accept rate [CSDN Eq. 8; XTL §5]: c*_k = 1 - 1/2 || p_d,k - p_t,k ||_1.         */
/* ------------------------------------------------------------------------------------ */
/* alpha[b][k-1] = sum_v min(p_d,k(v), p_t,k(v)) for k = 1..gamma, with p_d,k given the
 * drafted prefix and p_t,k = softmax(T[b][k] / temperature) (the same tempered
 * distributions that verification compares).  l1form, when not NULL, receives
 * 1 - 1/2 sum_v |p_d - p_t| computed separately, for the identity check. */
void ora_accept_tv(const ora_dims* dm, const double* U, const double* W1, const double* W2t,
                   const int32_t* anchor, const int32_t* tokens, const double* T,
                   double temperature, double* alpha, double* l1form)
{
    const int B = dm->batch, G = dm->gamma, V = dm->vocab;
    double* zd = (double*)malloc(sizeof(double) * (size_t)V);
    double* zt = (double*)malloc(sizeof(double) * (size_t)V);
    for (int b = 0; b < B; ++b) {
        for (int k = 1; k <= G; ++k) {
            draft_logits(dm, U + ((size_t)b * G + (k - 1)) * V, W1, W2t,
                         prev_token(anchor, tokens, G, b, k), temperature, zd);
            const double* Trow = T + ((size_t)b * (G + 1) + (k - 1)) * V;
            for (int v = 0; v < V; ++v) zt[v] = Trow[v] / temperature;
            double ld = logsumexp(zd, V), lt = logsumexp(zt, V);
            double smin = 0.0, sabs = 0.0;
            for (int v = 0; v < V; ++v) {
                double pd = exp(zd[v] - ld), pt = exp(zt[v] - lt);
                smin += pd < pt ? pd : pt;
                sabs += fabs(pd - pt);
            }
            alpha[(size_t)b * G + (k - 1)] = smin;
            if (l1form) l1form[(size_t)b * G + (k - 1)] = 1.0 - 0.5 * sabs;
        }
    }
    free(zd);
    free(zt);
}
