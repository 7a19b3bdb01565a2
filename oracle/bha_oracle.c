/*
 * Block-hybrid attention: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the correctness reference that the
 * HIP library is checked against. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does. It
 * shares no code, header, table or helper with the HIP library.
 *
 * Sources (the paper is "Retrofitting Linear Attention into Diffusion Language
 * Models", Kim, Roh, Kim):
 *   [GS]  gist.science explainer of the paper, "Technical Summary",
 *         section "Methodology: Block-Hybrid Attention", list "Architecture
 *         Design" (within-block softmax, cross-block Hedgehog linear
 *         attention, the S_n / Z_n states, the shared-normaliser merge).
 *   [ML]  mlsanity.com index of the paper, "Abstract (arXiv)" (the cost the
 *         method removes: every denoising step attends to all previous blocks).
 *   [PR]  pith.science review of the paper, "The reading", paragraph "What
 *         carries the argument" (the formulas for phi, S_n and Z_n; the per
 *         query O(F d) read), and "Circularity Check" (state sizes).
 *   The exact merge (where the gate and the row maximum m sit) is not printed
 *   on the pages; the form used here is the one fixed for this library:
 *     y_i = ( sum_j e^{s_ij - m_i} v_j + g e^{-m_i} phi(q_i)^T S )
 *         / ( sum_j e^{s_ij - m_i}     + g e^{-m_i} phi(q_i)^T Z ),
 *     s_ij = c q_i . k_j,  m_i = max_j s_ij,  c = 1/sqrt(d) unless given.
 *
 * Everything is computed in double precision with plain loops, in the order
 * the definitions are written. There is no blocking, no fusion and no
 * reordering beyond what the definitions state.
 *
 * Plain layouts used by every function here (all arrays row-major, fp64):
 *   x, q, k, v, out : [n][d]       one row per token
 *   w               : [FW][d]      row j holds column j of the d x FW matrix W
 *   phi             : [n][2*FW]    first FW entries softmax(xW), then softmax(-xW)
 *   S               : [2*FW][d]    S = sum_t phi(k_t) v_t^T
 *   Z               : [2*FW]       Z = sum_t phi(k_t)
 * Parity status: every function below is pinned by the CPU test suite (closed
 * forms, library softmax / attention, brute force, invariants).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------------
 * Hedgehog feature map, [GS] Architecture Design (cross-block bullet) and [PR]
 * "What carries the argument": phi(x) = [softmax(xW), softmax(-xW)], a positive
 * map of dimension 2*FW. The softmax runs over the FW entries of xW for one
 * token; no bias and no scaling of x.
 * ------------------------------------------------------------------------- */
void bha_ref_phi(const double* x, const double* w, int d, int fw, double* phi)
{
    double* u = (double*)malloc(sizeof(double) * (size_t)fw);
    for (int j = 0; j < fw; ++j) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += x[c] * w[(size_t)j * d + c];
        u[j] = acc;
    }
    /* first half: softmax(u) */
    double mx = u[0];
    for (int j = 1; j < fw; ++j) if (u[j] > mx) mx = u[j];
    double sum = 0.0;
    for (int j = 0; j < fw; ++j) { phi[j] = exp(u[j] - mx); sum += phi[j]; }
    for (int j = 0; j < fw; ++j) phi[j] /= sum;
    /* second half: softmax(-u) */
    double mn = -u[0];
    for (int j = 1; j < fw; ++j) if (-u[j] > mn) mn = -u[j];
    sum = 0.0;
    for (int j = 0; j < fw; ++j) { phi[fw + j] = exp(-u[j] - mn); sum += phi[fw + j]; }
    for (int j = 0; j < fw; ++j) phi[fw + j] /= sum;
    free(u);
}

/* phi for n tokens: x [n][d] -> phi [n][2*FW]. */
void bha_ref_feature_map(int n, int d, int fw, const double* x, const double* w, double* phi)
{
    for (int t = 0; t < n; ++t)
        bha_ref_phi(x + (size_t)t * d, w, d, fw, phi + (size_t)t * 2 * fw);
}

/* ---------------------------------------------------------------------------
 * State commit, [GS] Architecture Design (state-compression bullet: the states
 * change only when a block is committed) and [PR] "What carries the argument"
 * (S_n and Z_n sum phi(k_t) v_t^T and phi(k_t) over every token of every
 * committed block):  S += sum_t phi(k_t) v_t^T,  Z += sum_t phi(k_t).
 * k, v: [nt][d]; S: [2FW][d]; Z: [2FW]; updated in place.
 * ------------------------------------------------------------------------- */
void bha_ref_state_commit(int nt, int d, int fw, const double* k, const double* v,
                          const double* w, double* S, double* Z)
{
    const int F = 2 * fw;
    double* ph = (double*)malloc(sizeof(double) * (size_t)F);
    for (int t = 0; t < nt; ++t) {
        bha_ref_phi(k + (size_t)t * d, w, d, fw, ph);
        for (int f = 0; f < F; ++f) {
            Z[f] += ph[f];
            for (int c = 0; c < d; ++c) S[(size_t)f * d + c] += ph[f] * v[(size_t)t * d + c];
        }
    }
    free(ph);
}

/* State of a prefix built from nothing: S = 0, Z = 0, then one commit of all
 * nt prefix tokens (the sums do not depend on how tokens are grouped in blocks). */
void bha_ref_state_build(int nt, int d, int fw, const double* k, const double* v,
                         const double* w, double* S, double* Z)
{
    const int F = 2 * fw;
    memset(S, 0, sizeof(double) * (size_t)F * d);
    memset(Z, 0, sizeof(double) * (size_t)F);
    bha_ref_state_commit(nt, d, fw, k, v, w, S, Z);
}

/* ---------------------------------------------------------------------------
 * Block forward for one (request, head): exact bidirectional softmax over the B
 * tokens of the active block ([GS] Architecture Design, within-block bullet:
 * no mask inside the block), plus the linear read phi(q)^T S, phi(q)^T Z of the
 * committed state ([PR] "What carries the argument": each query reads it in
 * O(F d)), merged under one normaliser with the scalar gate g ([GS] merging
 * bullet) in the form written at the top of this file.
 * q, k, v, out: [B][d]; S: [2FW][d]; Z: [2FW].
 * ------------------------------------------------------------------------- */
void bha_ref_block_forward(int B, int d, int fw, const double* q, const double* k,
                           const double* v, const double* w, double gamma, double scale,
                           const double* S, const double* Z, double* out)
{
    const int F = 2 * fw;
    const double c = (scale > 0.0) ? scale : 1.0 / sqrt((double)d);
    double* s = (double*)malloc(sizeof(double) * (size_t)B);
    double* ph = (double*)malloc(sizeof(double) * (size_t)F);
    double* lin = (double*)malloc(sizeof(double) * (size_t)d);
    for (int i = 0; i < B; ++i) {
        const double* qi = q + (size_t)i * d;
        /* block logits and their row maximum */
        for (int j = 0; j < B; ++j) {
            double acc = 0.0;
            for (int e = 0; e < d; ++e) acc += qi[e] * k[(size_t)j * d + e];
            s[j] = c * acc;
        }
        double m = s[0];
        for (int j = 1; j < B; ++j) if (s[j] > m) m = s[j];
        /* linear read of the committed state */
        bha_ref_phi(qi, w, d, fw, ph);
        double lin_den = 0.0;
        for (int f = 0; f < F; ++f) lin_den += ph[f] * Z[f];
        for (int e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int f = 0; f < F; ++f) acc += ph[f] * S[(size_t)f * d + e];
            lin[e] = acc;
        }
        /* merge under one normaliser */
        const double g = gamma * exp(-m);
        double den = 0.0;
        for (int j = 0; j < B; ++j) den += exp(s[j] - m);
        den += g * lin_den;
        for (int e = 0; e < d; ++e) {
            double num = 0.0;
            for (int j = 0; j < B; ++j) num += exp(s[j] - m) * v[(size_t)j * d + e];
            num += g * lin[e];
            out[(size_t)i * d + e] = num / den;
        }
    }
    free(lin);
    free(ph);
    free(s);
}

/* ---------------------------------------------------------------------------
 * Softmax attention over the whole prefix, the path block-hybrid attention
 * replaces ([ML] abstract and [GS] Problem Statement: with KV caching, every
 * denoising step of the active block still attends to all previous blocks).
 * Each query of the block attends with one softmax to the np prefix tokens
 * (kp, vp: [np][d]) and to the B keys of the block itself (no mask):
 *   y_i = sum_t e^{c q_i.k_t} v_t / sum_t e^{c q_i.k_t}  over t in prefix + block.
 * The row maximum is subtracted before exponentiating (the value is the same).
 * q, k, v, out: [B][d].
 * ------------------------------------------------------------------------- */
void bha_ref_prefix_attention(int B, int np, int d, const double* q, const double* k, const double* v,
                              const double* kp, const double* vp, double scale, double* out)
{
    const double c = (scale > 0.0) ? scale : 1.0 / sqrt((double)d);
    const int nk = np + B;
    double* s = (double*)malloc(sizeof(double) * (size_t)(nk > 0 ? nk : 1));
    for (int i = 0; i < B; ++i) {
        const double* qi = q + (size_t)i * d;
        for (int t = 0; t < nk; ++t) {
            const double* kt = t < np ? kp + (size_t)t * d : k + (size_t)(t - np) * d;
            double acc = 0.0;
            for (int e = 0; e < d; ++e) acc += qi[e] * kt[e];
            s[t] = c * acc;
        }
        double m = s[0];
        for (int t = 1; t < nk; ++t) if (s[t] > m) m = s[t];
        double den = 0.0;
        for (int t = 0; t < nk; ++t) den += exp(s[t] - m);
        for (int e = 0; e < d; ++e) {
            double num = 0.0;
            for (int t = 0; t < nk; ++t) {
                const double* vt = t < np ? vp + (size_t)t * d : v + (size_t)(t - np) * d;
                num += exp(s[t] - m) * vt[e];
            }
            out[(size_t)i * d + e] = num / den;
        }
    }
    free(s);
}

/* ---------------------------------------------------------------------------
 * Batched drivers: the same per-pair functions applied to every (request, head)
 * pair, spread over plain pthreads. Pair-major plain layouts:
 *   q, k, v, out : [R][H][B][d]     w : [H][FW][d]     gamma : [H]
 *   S : [R][H][2FW][d]              Z : [R][H][2FW]
 * ------------------------------------------------------------------------- */
typedef struct {
    int kind; /* 0 = forward, 1 = commit */
    int R, H, B, d, fw;
    const double *q, *k, *v, *w, *gamma;
    double scale;
    double *S, *Z, *out;
    const double *Sc, *Zc;
    int64_t next;     /* shared pair counter */
    pthread_mutex_t lock;
} batch_job;

static void run_pair(batch_job* jb, int64_t p)
{
    const int F = 2 * jb->fw;
    const int h = (int)(p % jb->H);
    const size_t tok = (size_t)p * jb->B * jb->d;
    const double* wh = jb->w + (size_t)h * jb->fw * jb->d;
    if (jb->kind == 0) {
        bha_ref_block_forward(jb->B, jb->d, jb->fw, jb->q + tok, jb->k + tok, jb->v + tok, wh,
                              jb->gamma[h], jb->scale, jb->Sc + (size_t)p * F * jb->d,
                              jb->Zc + (size_t)p * F, jb->out + tok);
    } else {
        bha_ref_state_commit(jb->B, jb->d, jb->fw, jb->k + tok, jb->v + tok, wh,
                             jb->S + (size_t)p * F * jb->d, jb->Z + (size_t)p * F);
    }
}

static void* worker(void* arg)
{
    batch_job* jb = (batch_job*)arg;
    const int64_t total = (int64_t)jb->R * jb->H;
    for (;;) {
        pthread_mutex_lock(&jb->lock);
        int64_t p = jb->next++;
        pthread_mutex_unlock(&jb->lock);
        if (p >= total) break;
        run_pair(jb, p);
    }
    return NULL;
}

static void run_batch(batch_job* jb, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    jb->next = 0;
    pthread_mutex_init(&jb->lock, NULL);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, jb);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&jb->lock);
}

void bha_ref_block_forward_batch(int R, int H, int B, int d, int fw, const double* q,
                                 const double* k, const double* v, const double* w,
                                 const double* gamma, double scale, const double* S,
                                 const double* Z, double* out, int nthreads)
{
    batch_job jb;
    memset(&jb, 0, sizeof(jb));
    jb.kind = 0; jb.R = R; jb.H = H; jb.B = B; jb.d = d; jb.fw = fw;
    jb.q = q; jb.k = k; jb.v = v; jb.w = w; jb.gamma = gamma; jb.scale = scale;
    jb.Sc = S; jb.Zc = Z; jb.out = out;
    run_batch(&jb, nthreads);
}

void bha_ref_state_commit_batch(int R, int H, int B, int d, int fw, const double* k,
                                const double* v, const double* w, double* S, double* Z,
                                int nthreads)
{
    batch_job jb;
    memset(&jb, 0, sizeof(jb));
    jb.kind = 1; jb.R = R; jb.H = H; jb.B = B; jb.d = d; jb.fw = fw;
    jb.k = k; jb.v = v; jb.w = w; jb.S = S; jb.Z = Z;
    run_batch(&jb, nthreads);
}
