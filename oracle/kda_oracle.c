/*
 * kda_oracle.c -- plain, slow CPU oracle for the KDA layer path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library and must never be used as a
 * fallback for it.
 *
 * What it computes (Kimi Delta Attention, per sequence and per head, token by
 * token).  Per head, a KDA layer carries a matrix of fixed size that every
 * token updates, and beside it the recent inputs of a short causal
 * convolution; caching a prefix means keeping both ("Kimi K3 + vLLM: Inside
 * the Day-0 Production Integration", section "Kimi Delta Attention: When
 * Prefix Caching Meets Recurrent State"; "Kimi K3 on vLLM: Up to 370
 * Tokens/sec", section "Kimi Delta Attention: a hybrid recurrent +
 * full-attention stack").  The pages give no equation for the update; the
 * oracle takes the gated delta rule with per-key-channel decay as the
 * plainest reading:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t,            alpha_t = exp(g_t)
 *
 * with S a d_k x d_v matrix (rows = key channels), the decay applied first,
 * the delta-rule correction taken against the decayed state, and the output
 * read from the updated state.  Everything is evaluated literally in the
 * order written, one token at a time.
 *
 * Interval checkpoints follow the retention policy of the Day-0 Integration
 * page (section "Interval-Based and Marconi-Style Retention"): the state is
 * saved after every absolute position p that is a multiple of the interval
 * and lies strictly inside the sequence; the final state is returned
 * separately.
 *
 * The short causal convolution (same page, "Separate Prefill/Decode Code
 * Paths", where the fused decode kernel folds it in) is depthwise over the
 * channel axis with the current token on the last tap:
 *
 *     y[t, c] = bias[c] + sum_{j=0}^{W-1} w[c, j] * xbar[t - (W-1) + j, c]
 *
 * where xbar is the carried state (the last W-1 raw inputs, oldest first)
 * followed by the sequence's tokens; optional SiLU on the result.  The new
 * carried state is the last W-1 raw inputs.
 *
 * Arithmetic type: `real` (double by default; -DORACLE_REAL_FLOAT builds an
 * fp32 variant).  Inputs arrive as float32 arrays (bf16 values upcast
 * exactly by the caller).  OpenMP spreads independent (sequence, head) pairs
 * over threads; each pair's arithmetic is serial and in the order above.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#ifdef ORACLE_REAL_FLOAT
typedef float real;
#define REXP expf
#else
typedef double real;
#define REXP exp
#endif

/* Planted mistakes (mutation testing of the pins).  0 = the oracle as is. */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

int oracle_real_bytes(void) { return (int)sizeof(real); }

int oracle_mutant(void) { return ORACLE_MUTANT; }

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_get_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Checkpoint positions of one sequence occupying absolute positions
 * [start, start + len): every p = m * interval with start < p < start + len,
 * found by walking the tokens one by one.  Writes at most `cap` positions to
 * `pos` (if not NULL) and returns how many there are.
 */
static int64_t ckpt_walk(int64_t start, int64_t len, int64_t interval, int32_t *pos, int64_t cap) {
    int64_t n = 0;
    if (interval <= 0) return 0;
    for (int64_t i = 0; i < len; ++i) {
        int64_t after = start + i + 1;           /* tokens consumed so far, absolute */
        if (after % interval == 0 && after < start + len) {
            if (pos && n < cap) pos[n] = (int32_t)after;
            ++n;
        }
    }
    return n;
}

/*
 * Enumerate the checkpoints of a packed batch.  ckpt_cu [n_seq+1] receives the
 * prefix counts; ckpt_pos (capacity cap) the positions.  Returns the total.
 */
int64_t oracle_ckpt_enumerate(const int32_t *cu_seqlens, const int32_t *start_pos, int32_t n_seq,
                              int32_t interval, int32_t *ckpt_cu, int32_t *ckpt_pos, int64_t cap) {
    int64_t total = 0;
    if (ckpt_cu) ckpt_cu[0] = 0;
    for (int32_t s = 0; s < n_seq; ++s) {
        int64_t len = (int64_t)cu_seqlens[s + 1] - cu_seqlens[s];
        int64_t start = start_pos ? start_pos[s] : 0;
        int64_t room = cap - total;
        int64_t n = ckpt_walk(start, len, interval, ckpt_pos ? ckpt_pos + total : NULL,
                              room > 0 ? room : 0);
        total += n;
        if (ckpt_cu) ckpt_cu[s + 1] = (int32_t)total;
    }
    return total;
}

/* One token of the recurrence on state S (dk x dv, row-major).  */
static void kda_token(real *S, real *w, int dk, int dv, const float *q, const float *k,
                      const float *v, const float *g, float beta, real scale, real *o_out) {
    /* Diag(alpha_t) S: row r (key channel r) scaled by exp(g[r]). */
    for (int r = 0; r < dk; ++r) {
#if ORACLE_MUTANT == 1
        real a = 1;                                  /* mistake: decay dropped */
        (void)g;
#else
        real a = REXP((real)g[r]);
#endif
        for (int c = 0; c < dv; ++c) {
#if ORACLE_MUTANT == 2
            S[(size_t)r * dv + c] *= REXP((real)g[c % dk]);   /* mistake: decay on value axis */
            (void)a;
#else
            S[(size_t)r * dv + c] *= a;
#endif
        }
    }
#if ORACLE_MUTANT == 6
    for (int c = 0; c < dv; ++c) {
        real acc = 0;
        for (int r = 0; r < dk; ++r) acc += S[(size_t)r * dv + c] * (real)q[r];
        o_out[c] = scale * acc;
    }
#endif
    /* w = S^T k (the decayed state's prediction for key k). */
    for (int c = 0; c < dv; ++c) {
        real acc = 0;
        for (int r = 0; r < dk; ++r) {
#if ORACLE_MUTANT == 3
            acc += S[(size_t)c % dk * dv + r % dv] * (real)k[r];   /* mistake: S k, transposed */
#else
            acc += S[(size_t)r * dv + c] * (real)k[r];
#endif
        }
        w[c] = acc;
    }
    /* S += beta k (v - w)^T, i.e. (I - beta k k^T)(Diag(alpha) S) + beta k v^T. */
    for (int r = 0; r < dk; ++r) {
        real bk = (real)beta * (real)k[r];
        for (int c = 0; c < dv; ++c) {
#if ORACLE_MUTANT == 4
            S[(size_t)r * dv + c] += bk * ((real)v[c] + w[c]);     /* mistake: sign of correction */
#else
            S[(size_t)r * dv + c] += bk * ((real)v[c] - w[c]);
#endif
        }
    }
#if ORACLE_MUTANT == 6
    return;                                          /* mistake: output read before the update */
#endif
    /* o = scale * S_t^T q, from the updated state. */
    for (int c = 0; c < dv; ++c) {
        real acc = 0;
        for (int r = 0; r < dk; ++r) acc += S[(size_t)r * dv + c] * (real)q[r];
        o_out[c] = scale * acc;
    }
}

/*
 * Varlen recurrence over a packed batch.
 *
 *   q, k, g : [T_tot, H, dk] float32 (contiguous)
 *   v       : [T_tot, H, dv] float32
 *   beta    : [T_tot, H]     float32
 *   cu_seqlens [n_seq+1], start_pos [n_seq] or NULL (absolute position of the
 *   sequence's first token; only checkpoint placement depends on it)
 *   init    : [n_seq, H, dk, dv] real or NULL; has_init [n_seq] or NULL
 *             (sequence s starts from init[s] when has_init[s] != 0, else 0)
 *   o       : [T_tot, H, dv] real (written for the computed pairs)
 *   final   : [n_seq, H, dk, dv] real or NULL
 *   ckpt    : [n_ckpt, H, dk, dv] real or NULL, ordered as
 *             oracle_ckpt_enumerate; ckpt_cap = rows available
 *   pairs   : [n_pairs, 2] (seq, head) to compute, or NULL for all
 *   o_skip  : if nonzero, outputs are not written (state-only runs)
 *
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int oracle_kda_varlen(const float *q, const float *k, const float *v, const float *g,
                      const float *beta, const int32_t *cu_seqlens, const int32_t *start_pos,
                      int32_t n_seq, int32_t H, int32_t dk, int32_t dv, double scale,
                      const real *init, const int32_t *has_init, real *o, real *final,
                      int32_t ckpt_interval, real *ckpt, int64_t ckpt_cap,
                      const int32_t *pairs, int64_t n_pairs, int32_t o_skip) {
    if (n_seq < 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    int64_t *ck_off = (int64_t *)calloc((size_t)n_seq + 1, sizeof(int64_t));
    if (!ck_off) return -1;
    for (int32_t s = 0; s < n_seq; ++s) {
        int64_t len = (int64_t)cu_seqlens[s + 1] - cu_seqlens[s];
        int64_t start = start_pos ? start_pos[s] : 0;
        ck_off[s + 1] = ck_off[s] + ckpt_walk(start, len, ckpt_interval, NULL, 0);
    }
    int64_t total_pairs = pairs ? n_pairs : (int64_t)n_seq * H;
    const size_t SS = (size_t)dk * dv;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pi = 0; pi < total_pairs; ++pi) {
        int32_t s = pairs ? pairs[2 * pi] : (int32_t)(pi / H);
        int32_t h = pairs ? pairs[2 * pi + 1] : (int32_t)(pi % H);
        if (s < 0 || s >= n_seq || h < 0 || h >= H) {
#pragma omp atomic write
            status = -1;
            continue;
        }
        real *S = (real *)malloc(SS * sizeof(real));
        real *w = (real *)malloc((size_t)dv * sizeof(real));
        real *ob = (real *)malloc((size_t)dv * sizeof(real));
        if (!S || !w || !ob) {
            free(S); free(w); free(ob);
#pragma omp atomic write
            status = -1;
            continue;
        }
        if (init && (!has_init || has_init[s]))
            memcpy(S, init + ((size_t)s * H + h) * SS, SS * sizeof(real));
        else
            memset(S, 0, SS * sizeof(real));
        int64_t bos = cu_seqlens[s], eos = cu_seqlens[s + 1];
        int64_t start = start_pos ? start_pos[s] : 0;
        int64_t nck = 0;
        for (int64_t t = bos; t < eos; ++t) {
            size_t th = (size_t)t * H + h;
            kda_token(S, w, dk, dv, q + th * dk, k + th * dk, v + th * dv, g + th * dk,
                      beta[th], (real)scale, ob);
            if (!o_skip) memcpy(o + th * dv, ob, (size_t)dv * sizeof(real));
            int64_t after = start + (t - bos) + 1;
            if (ckpt_interval > 0 && after % ckpt_interval == 0 && after < start + (eos - bos)) {
                int64_t row = ck_off[s] + nck;
                if (ckpt && row < ckpt_cap)
                    memcpy(ckpt + ((size_t)row * H + h) * SS, S, SS * sizeof(real));
                ++nck;
            }
        }
        if (final) memcpy(final + ((size_t)s * H + h) * SS, S, SS * sizeof(real));
        free(S); free(w); free(ob);
    }
    free(ck_off);
    return status;
}

/*
 * Speculative verification: each of n_seq sequences holds T_spec candidate
 * tokens (position 0 = the token already accepted, then the drafts).  The
 * recurrence runs over all T_spec tokens from init (outputs for every
 * position), and the state after exactly accepted_len[s] tokens is returned in
 * committed [n_seq, H, dk, dv].  accepted_len outside [0, T_spec] marks the
 * sequence as rejected: committed_len[s] = -1 and committed[s] is untouched.
 * accepted_len = 0 commits init itself.
 *
 *   q, k, g [n_seq, T_spec, H, dk]; v [n_seq, T_spec, H, dv]; beta [n_seq, T_spec, H]
 *   init [n_seq, H, dk, dv] real; o [n_seq, T_spec, H, dv] real or NULL
 */
int oracle_kda_verify(const float *q, const float *k, const float *v, const float *g,
                      const float *beta, int32_t n_seq, int32_t T_spec, int32_t H, int32_t dk,
                      int32_t dv, double scale, const real *init, const int32_t *accepted_len,
                      real *o, real *committed, int32_t *committed_len) {
    if (n_seq < 0 || T_spec <= 0 || H <= 0 || dk <= 0 || dv <= 0) return -1;
    const size_t SS = (size_t)dk * dv;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pi = 0; pi < (int64_t)n_seq * H; ++pi) {
        int32_t s = (int32_t)(pi / H), h = (int32_t)(pi % H);
        real *S = (real *)malloc(SS * sizeof(real));
        real *w = (real *)malloc((size_t)dv * sizeof(real));
        real *ob = (real *)malloc((size_t)dv * sizeof(real));
        if (!S || !w || !ob) {
            free(S); free(w); free(ob);
#pragma omp atomic write
            status = -1;
            continue;
        }
        memcpy(S, init + ((size_t)s * H + h) * SS, SS * sizeof(real));
        int32_t L = accepted_len ? accepted_len[s] : T_spec;
        int valid = (L >= 0 && L <= T_spec);
        if (h == 0 && committed_len) committed_len[s] = valid ? L : -1;
        if (valid && L == 0 && committed)
            memcpy(committed + ((size_t)s * H + h) * SS, S, SS * sizeof(real));
        for (int32_t j = 0; j < T_spec; ++j) {
            size_t th = ((size_t)s * T_spec + j) * H + h;
            kda_token(S, w, dk, dv, q + th * dk, k + th * dk, v + th * dv, g + th * dk,
                      beta[th], (real)scale, ob);
            if (o) memcpy(o + th * dv, ob, (size_t)dv * sizeof(real));
            if (valid && j + 1 == L && committed)
                memcpy(committed + ((size_t)s * H + h) * SS, S, SS * sizeof(real));
        }
        free(S); free(w); free(ob);
    }
    return status;
}

/*
 * Short causal depthwise convolution over a packed batch.
 *
 *   x      : [T_tot, C] float32, row stride x_stride (elements)
 *   w      : [C, W] float32; bias [C] or NULL; act: 0 none, 1 SiLU
 *   state  : [n_seq, C, W-1] float32 or NULL (the carried raw inputs, oldest
 *            first); has_state [n_seq] or NULL (0 -> zero history)
 *   adv    : [n_seq] or NULL.  The new state is taken after adv[s] tokens of
 *            the sequence (all of them when NULL); outputs cover every token.
 *   y      : [T_tot, C] real
 *   new_state : [n_seq, C, W-1] real or NULL
 */
int oracle_conv_short(const float *x, int64_t x_stride, const float *w, const float *bias,
                      int32_t act, const int32_t *cu_seqlens, int32_t n_seq, int32_t C,
                      int32_t W, const float *state, const int32_t *has_state,
                      const int32_t *adv, real *y, real *new_state) {
    if (n_seq < 0 || C <= 0 || W < 1) return -1;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t pi = 0; pi < (int64_t)n_seq * C; ++pi) {
        int32_t s = (int32_t)(pi / C), c = (int32_t)(pi % C);
        int64_t bos = cu_seqlens[s], eos = cu_seqlens[s + 1];
        int64_t len = eos - bos;
        int64_t hist = W - 1;
        /* xbar = carried state ++ tokens of this channel */
        real *xb = (real *)malloc((size_t)(hist + len + 1) * sizeof(real));
        if (!xb) {
#pragma omp atomic write
            status = -1;
            continue;
        }
        for (int64_t j = 0; j < hist; ++j) {
            int use = state && (!has_state || has_state[s]);
            xb[j] = use ? (real)state[((size_t)s * C + c) * hist + j] : 0;
        }
        for (int64_t t = 0; t < len; ++t) xb[hist + t] = (real)x[(size_t)(bos + t) * x_stride + c];
        for (int64_t t = 0; t < len; ++t) {
            real acc = bias ? (real)bias[c] : 0;
            for (int32_t j = 0; j < W; ++j) {
#if ORACLE_MUTANT == 5
                acc += (real)w[(size_t)c * W + (W - 1 - j)] * xb[t + j];  /* mistake: taps reversed */
#else
                acc += (real)w[(size_t)c * W + j] * xb[t + j];
#endif
            }
            if (act == 1) acc = acc / (1 + REXP(-acc));
            y[(size_t)(bos + t) * C + c] = acc;
        }
        if (new_state) {
            int64_t a = adv ? adv[s] : len;
            if (a < 0) a = 0;
            if (a > len) a = len;
            /* last W-1 entries of xbar[0 .. hist + a) */
            for (int64_t j = 0; j < hist; ++j)
                new_state[((size_t)s * C + c) * hist + j] = xb[a + j];
        }
        free(xb);
    }
    return status;
}
