/*
 * Runs every function of the fp64 oracle on small and edge-case shapes, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_sanitizers.py builds and runs
 * it).  It checks nothing numerically -- the pins do that -- it only drives every code path
 * (forced prefixes, global ids, gamma = 1, V = 2, empty and full budgets, every scheduler
 * mode, NULL diagnostics) so that an out-of-bounds access, a leak or undefined arithmetic
 * aborts the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct { int32_t batch, gamma, vocab, rank, hidden; } ora_dims;

void ora_philox4x32(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
double ora_uniform(uint64_t seed, uint32_t b, uint32_t k, uint32_t s, uint32_t v);
void ora_uniform_fill(uint64_t seed, uint32_t b, uint32_t k, uint32_t s, uint32_t v0,
                      int64_t n, double* out);
void ora_draft(const ora_dims* dm, const double* U, const double* W1, const double* W2t,
               const int32_t* anchor, const int32_t* forced, const int32_t* gid,
               double temperature, uint64_t seed, int32_t* tokens, double* logp,
               double* lse_out, double* gap, double* probs);
void ora_confidence(const ora_dims* dm, const double* h, const double* W1, const double* w,
                    const int32_t* anchor, const int32_t* tokens, const double* temps,
                    double* c);
void ora_schedule(int32_t B, int32_t gamma, const double* c, const double* sps, int32_t mode,
                  int32_t* ell, double* theta, int32_t* n_total);
void ora_schedule_topk(int32_t B, int32_t gamma, const double* c, const double* sps, int32_t K,
                       int32_t* ell, double* theta, int32_t* n_total);
void ora_sts_calibrate(int32_t n, int32_t gamma, const double* logit, const int32_t* n_accept,
                       const double* temps, int32_t n_t, int32_t n_bins, double* t_out,
                       double* ece_out, double* gap);
void ora_markov_target(int32_t B, int32_t gamma, int32_t V, const double* U,
                       const int32_t* anchor, const int32_t* tokens, double sigma,
                       uint64_t seed, double* T);
void ora_draft_loss(int32_t B, int32_t gamma, int32_t V, const double* zd, const double* zt,
                    const int32_t* labels, const double* conf_logit, double alpha_ce,
                    double alpha_l1, double alpha_conf, double* loss, double* terms,
                    double* grad_zd, double* grad_conf);
void ora_verify(const ora_dims* dm, const double* U, const double* W1, const double* W2t,
                const int32_t* anchor, const int32_t* tokens, const double* T,
                const int32_t* ell, const int32_t* gid, double temperature, uint64_t seed,
                int32_t* n_accept, int32_t* out_tokens, double* pt_tok, double* margin,
                double* gap, int32_t* kind);
void ora_accept_tv(const ora_dims* dm, const double* U, const double* W1, const double* W2t,
                   const int32_t* anchor, const int32_t* tokens, const double* T,
                   double temperature, double* alpha, double* l1form);

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double unif(void) {   /* xorshift64*: test inputs only */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (double)((rng_state * 0x2545F4914F6CDD1Dull) >> 11) * 0x1p-53;
}
static double* dvec(size_t n, double s) {
    double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = s * (2.0 * unif() - 1.0);
    return p;
}
static int32_t* ivec(size_t n, int32_t hi) {
    int32_t* p = (int32_t*)malloc(sizeof(int32_t) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) p[i] = (int32_t)(unif() * hi);
    return p;
}

static void round_case(int B, int G, int V, int r, int d, double temp, int diagnostics) {
    ora_dims dm = {B, G, V, r, d};
    double* U = dvec((size_t)B * G * V, 3.0);
    double* W1 = dvec((size_t)V * r, 0.5);
    double* W2t = dvec((size_t)V * r, 0.5);
    double* h = dvec((size_t)B * G * d, 1.0);
    double* w = dvec((size_t)d + r, 0.3);
    int32_t* anchor = ivec(B, V);
    int32_t* gid = ivec(B, 1 << 20);
    int32_t* tok = ivec((size_t)B * G, V);
    double* logp = dvec((size_t)B * G, 0), *lse = dvec((size_t)B * G, 0);
    double* gap = dvec((size_t)B * G, 0);
    double* probs = dvec((size_t)B * G * V, 0);
    ora_draft(&dm, U, W1, W2t, anchor, NULL, NULL, temp, 7, tok, logp, lse,
              diagnostics ? gap : NULL, diagnostics ? probs : NULL);
    int32_t* forced = ivec((size_t)B * G, V);
    ora_draft(&dm, U, W1, W2t, anchor, forced, gid, temp, 8, tok, logp, lse, gap, probs);
    double* c = dvec((size_t)B * G, 0);
    double* temps = dvec(G, 0);
    for (int k = 0; k < G; ++k) temps[k] = 0.5 + k;
    ora_confidence(&dm, h, W1, w, anchor, tok, NULL, c);
    ora_confidence(&dm, h, W1, w, anchor, tok, temps, c);
    const int nsps = B * (G + 1) + 1;
    double* sps = dvec(nsps, 0);
    for (int i = 0; i < nsps; ++i) sps[i] = 1000.0 / (10.0 + 0.05 * i);
    int32_t* ell = ivec(B, 1);
    double theta;
    int32_t n_total;
    for (int mode = 0; mode < 2; ++mode) ora_schedule(B, G, c, sps, mode, ell, &theta, &n_total);
    const int ks[5] = {-3, 0, 1, B * G, B * G + 5};
    for (int i = 0; i < 5; ++i) ora_schedule_topk(B, G, c, sps, ks[i], ell, &theta, &n_total);
    double* T = dvec((size_t)B * (G + 1) * V, 3.0);
    ora_markov_target(B, G, V, U, anchor, tok, 0.5, 11, T);
    int32_t* nacc = ivec(B, 1), *out = ivec((size_t)B * (G + 1), 1), *kind = ivec(B, 1);
    double* pt = dvec((size_t)B * G, 0), *margin = dvec((size_t)B * G, 0), *vgap = dvec(B, 0);
    for (int b = 0; b < B; ++b) ell[b] = b % (G + 1);
    ora_verify(&dm, U, W1, W2t, anchor, tok, T, ell, NULL, temp, 9, nacc, out, NULL, NULL,
               NULL, NULL);
    for (int b = 0; b < B; ++b) ell[b] = G;
    ora_verify(&dm, U, W1, W2t, anchor, tok, T, ell, gid, temp, 9, nacc, out, pt, margin, vgap,
               kind);
    double* alpha = dvec((size_t)B * G, 0), *l1 = dvec((size_t)B * G, 0);
    ora_accept_tv(&dm, U, W1, W2t, anchor, tok, T, temp, alpha, NULL);
    ora_accept_tv(&dm, U, W1, W2t, anchor, tok, T, temp, alpha, l1);
    double loss;
    double* terms = dvec((size_t)B * G * 3, 0), *gz = dvec((size_t)B * G * V, 0);
    double* gc = dvec((size_t)B * G, 0);
    double* zd = dvec((size_t)B * G * V, 2.0);
    ora_draft_loss(B, G, V, zd, U, tok, c, 0.1, 0.9, 1.0, &loss, terms, gz, gc);
    ora_draft_loss(B, G, V, zd, U, tok, c, 0.1, 0.9, 1.0, &loss, NULL, NULL, NULL);
    free(U); free(W1); free(W2t); free(h); free(w); free(anchor); free(gid); free(tok);
    free(logp); free(lse); free(gap); free(probs); free(forced); free(c); free(temps);
    free(sps); free(ell); free(T); free(nacc); free(out); free(kind); free(pt); free(margin);
    free(vgap); free(alpha); free(l1); free(terms); free(gz); free(gc); free(zd);
}

int main(void) {
    uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, o[4];
    ora_philox4x32(ctr, key, o);
    double u[37];
    ora_uniform_fill(~0ull, 65535, 64, 2, 0xFFFFFFF0u, 37, u);   /* v wraps past 2^32 */
    (void)ora_uniform(0, 0, 0, 0, 0);
    round_case(4, 4, 64, 8, 16, 1.0, 1);
    round_case(1, 1, 2, 8, 0, 0.7, 0);      /* gamma = 1, V = 2, no hidden state */
    round_case(3, 5, 101, 16, 7, 2.0, 1);   /* odd sizes */
    /* calibration: grid of one, bins of one and many, a position nobody reaches */
    const int n = 50, G = 3;
    double* logit = dvec((size_t)n * G, 3.0);
    int32_t* nacc = ivec(n, G + 1);
    double grid[4] = {0.5, 1.0, 2.0, 4.0}, t[3], e[3], g[3];
    ora_sts_calibrate(n, G, logit, nacc, grid, 4, 15, t, e, g);
    ora_sts_calibrate(n, G, logit, nacc, grid, 1, 1, t, e, g);
    for (int i = 0; i < n; ++i) nacc[i] = 0;
    ora_sts_calibrate(n, G, logit, nacc, grid, 4, 256, t, e, g);
    free(logit);
    free(nacc);
    printf("oracle driver: every function ran\n");
    return 0;
}
