/*
 * Plain fp64 CPU oracle for exact softmax attention and for the W4A16 layer.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the library's compute path may include,
 * link, load or call this file; it exists so that tests, the smoke check and the
 * CPU baseline of the benchmark can compare the GPU kernels with a slow,
 * obviously correct computation. It shares no header, helper or constant with
 * the GPU code.
 *
 * What it computes (sources are the four pages this project follows):
 *
 *  - Standard attention, O = softmax(scale * Q K^T) V, the result FlashAttention-2
 *    keeps "fully equivalent" to ("FlashAttention-2", Systems analysis wiki: lead
 *    paragraph and "Background: the attention problem in transformers").  For a
 *    query row i the allowed keys are J_i = { j < Nk : !causal or
 *    j <= i + Nk - Nq } (causal masking is named only by the FlashAttention-4
 *    summary, "Hardware-Aware FP4 FlashAttention-4"; the bottom-right alignment
 *    for Nq != Nk is this project's reading and equals j <= i when Nq == Nk).
 *    s_ij = scale * sum_c q_ic k_jc ; m_i = max_j s_ij ;
 *    P_ij = exp(s_ij - m_i) / sum_j' exp(s_ij' - m_i) ; O_i = sum_j P_ij v_j ;
 *    LSE_i = m_i + ln sum_j exp(s_ij - m_i).  Rows with no allowed key get O = 0,
 *    LSE = -inf.  Subtracting m_i changes nothing mathematically; it only keeps
 *    exp() finite.
 *
 *  - The per-block partial state and its merge, from "Sequence parallelism and
 *    ring attention" (aiunderstanding.org), sections "Deep dive" and "Technical
 *    insight": a running maximum and running normaliser let attention be built
 *    block by block, the earlier partial sum being rescaled when a larger
 *    maximum appears.  A partial state over a key subset K_b is
 *    (O_b normalised by its own l_b, m_b = max s, l_b = sum exp(s - m_b)); two
 *    states merge as M = max(m_a, m_b), w_x = l_x exp(m_x - M),
 *    O = (w_a O_a + w_b O_b) / (w_a + w_b), l = w_a + w_b, m = M.
 *
 *  - Input decoding: bfloat16 bit patterns (upper half of an IEEE binary32) and
 *    OCP FP8 E4M3 ("e4m3fn": bias 7, no infinities, S.1111.111 is NaN) codes
 *    times a float32 scale per (batch, head, 128-token tile), the block
 *    quantization of "Scaling FlashAttention, multi-GPU training and weight
 *    quantization" (itimpress), section 1, FP8 bullet.  Both decodes are exact in
 *    fp64.
 *
 *  - The gradients of that attention (the backward pass that the training
 *    results of "FlashAttention-2" ("Performance and efficiency") and of the
 *    FlashAttention-4 summary presuppose; the pages give no formula, so this is
 *    the chain rule applied to the definition above).  For one (b, h) and the
 *    loss L = sum_i dO_i . O_i:  dV_j = sum_i P_ij dO_i ;
 *    dP_ij = dO_i . v_j ;  D_i = sum_j P_ij dP_ij ;  dS_ij = P_ij (dP_ij - D_i) ;
 *    dQ_i = scale sum_j dS_ij k_j ;  dK_j = scale sum_i dS_ij q_i.
 *
 *  - The W4A16 linear layer of "Scaling FlashAttention, multi-GPU training and
 *    weight quantization" (itimpress), section 3: weights stored as 4-bit
 *    integers, eight to a 32-bit word, with a scale and a zero point per group,
 *    turned back into 16-bit values as w = (q - z) * s and multiplied with
 *    16-bit activations: y[m][n] = sum_k x[m][k] w[n][k].  The pages do not fix
 *    the order of the eight values in a word; this project's reading (the
 *    library's input format) puts weight k = 8j + e of row n in word j at bits
 *    4 (e / 2) + 16 (e % 2) .. +3, so even e fill the low 16 bits and odd e the
 *    high 16 bits.  Groups are G consecutive k of one row.
 *
 * Layout of every tensor: contiguous [B, H, N, d], d innermost; per-row outputs
 * [B, H, N].  A row subset is given as `rows` (n_rows query indices shared by
 * every (b, h)), or rows == NULL for all Nq rows; outputs are then
 * [B, H, n_rows, d] and [B, H, n_rows].
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- decoding */

/* bfloat16 bits -> value: the 16 bits are the top half of a binary32. */
double oracle_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP E4M3 ("e4m3fn") code -> value. sign | 4-bit exponent (bias 7) | 3-bit
 * mantissa; exponent 0 is subnormal (m/8 * 2^-6); 0x7F and 0xFF are NaN; there
 * is no infinity, so exponent 15 with mantissa < 7 is an ordinary number. */
double oracle_e4m3_value(uint8_t code) {
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double mag;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0) mag = ldexp((double)m / 8.0, -6);
    else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* kind: 0 = float32 values, 1 = bfloat16 bits, 2 = e4m3 codes with scales
 * [B, H, ceil(N / tile)] (float32), each scale applied to `tile` consecutive
 * tokens of one (b, h). */
int oracle_decode(int kind, const void* src, const float* scales, int tile,
                  int64_t B, int64_t H, int64_t N, int64_t d, double* dst) {
    int64_t total = B * H * N * d;
    if (kind == 0) {
        const float* s = (const float*)src;
        for (int64_t i = 0; i < total; ++i) dst[i] = (double)s[i];
        return 0;
    }
    if (kind == 1) {
        const uint16_t* s = (const uint16_t*)src;
        for (int64_t i = 0; i < total; ++i) dst[i] = oracle_bf16_value(s[i]);
        return 0;
    }
    if (kind == 2) {
        const uint8_t* s = (const uint8_t*)src;
        int64_t ntiles = (N + tile - 1) / tile;
        for (int64_t bh = 0; bh < B * H; ++bh)
            for (int64_t n = 0; n < N; ++n) {
                double sc = (double)scales[bh * ntiles + n / tile];
                for (int64_t c = 0; c < d; ++c) {
                    int64_t idx = (bh * N + n) * d + c;
                    dst[idx] = oracle_e4m3_value(s[idx]) * sc;
                }
            }
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------- one query row, all */

/* Attention of one query row q (length d) against the first `count` keys and
 * values of k, v ([Nk, d] each); every allowed key set in this file is such a
 * prefix (causal masks allow keys 0 .. limit).  Writes o (length d),
 * *m_out = max score, *l_out = sum exp(s - max), and optionally the probability
 * row p (length Nk, zero beyond the prefix).  count == 0 gives the empty state
 * O = 0, m = -inf, l = 0. */
static void row_attention(const double* q, const double* k, const double* v,
                          int64_t Nk, int64_t d, int64_t count, double scale,
                          double* s_buf, double* o, double* m_out, double* l_out,
                          double* p) {
    for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
    if (p)
        for (int64_t j = 0; j < Nk; ++j) p[j] = 0.0;
    if (count <= 0) {
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    /* scores s_j = scale * q . k_j */
    for (int64_t j = 0; j < count; ++j) {
        double dot = 0.0;
        for (int64_t c = 0; c < d; ++c) dot += q[c] * k[j * d + c];
        s_buf[j] = scale * dot;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < count; ++j)
        if (s_buf[j] > m) m = s_buf[j];
    double l = 0.0;
    for (int64_t j = 0; j < count; ++j) {
        s_buf[j] = exp(s_buf[j] - m); /* unnormalised probability */
        l += s_buf[j];
    }
    for (int64_t j = 0; j < count; ++j) {
        double pj = s_buf[j] / l;
        if (p) p[j] = pj;
        for (int64_t c = 0; c < d; ++c) o[c] += pj * v[j * d + c];
    }
    *m_out = m;
    *l_out = l;
}

/* Number of keys 0 .. n-1 that satisfy j <= limit. */
static int64_t prefix_count(int64_t limit, int64_t n) {
    if (limit < 0) return 0;
    return limit + 1 < n ? limit + 1 : n;
}

/* ------------------------------------------------------------ full attention */

/* O and LSE of standard softmax attention for the requested rows.
 * q: [B,H,Nq,d]; k, v: [B,H,Nk,d]; o: [B,H,R,d]; lse: [B,H,R];
 * p (optional): [B,H,R,Nk].  R = n_rows (rows != NULL) or Nq. */
int oracle_attention(const double* q, const double* k, const double* v,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                     int causal, double scale, const int64_t* rows, int64_t n_rows,
                     double* o, double* lse, double* p) {
    int64_t R = rows ? n_rows : Nq;
    if (B <= 0 || H <= 0 || Nq < 0 || Nk < 0 || d <= 0) return -1;
    int64_t units = B * H * R;
    int err = 0;
#pragma omp parallel
    {
        double* s_buf = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        if (!s_buf) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t u = 0; u < units; ++u) {
            if (!s_buf) continue;
            int64_t bh = u / R, r = u % R;
            int64_t i = rows ? rows[r] : r;
            /* causal: key j allowed iff j <= i + Nk - Nq */
            int64_t count = causal ? prefix_count(i + Nk - Nq, Nk) : Nk;
            double m, l;
            row_attention(q + (bh * Nq + i) * d, k + bh * Nk * d, v + bh * Nk * d, Nk, d,
                          count, scale, s_buf, o + u * d, &m, &l, p ? p + u * Nk : NULL);
            lse[u] = count > 0 ? m + log(l) : -INFINITY;
        }
        free(s_buf);
    }
    return err;
}

/* ------------------------------------------------------- block partial state */

/* Partial state of the requested query rows against one key/value block of
 * Nkb keys whose global positions are k_pos0 .. k_pos0 + Nkb - 1; query row i
 * sits at global position q_pos0 + i.  With causal set, key j is allowed iff
 * k_pos0 + j <= q_pos0 + i.  o: normalised [B,H,R,d]; m: [B,H,R] (max of
 * scale*q.k, -inf if no key); l: [B,H,R] (sum exp(s - m), 0 if no key). */
int oracle_block_state(const double* q, const double* kb, const double* vb,
                       int64_t B, int64_t H, int64_t Nq, int64_t Nkb, int64_t d,
                       int causal, int64_t q_pos0, int64_t k_pos0, double scale,
                       const int64_t* rows, int64_t n_rows,
                       double* o, double* m, double* l) {
    int64_t R = rows ? n_rows : Nq;
    if (B <= 0 || H <= 0 || Nq < 0 || Nkb < 0 || d <= 0) return -1;
    int64_t units = B * H * R;
    int err = 0;
#pragma omp parallel
    {
        double* s_buf = (double*)malloc(sizeof(double) * (size_t)(Nkb > 0 ? Nkb : 1));
        if (!s_buf) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 4)
        for (int64_t u = 0; u < units; ++u) {
            if (!s_buf) continue;
            int64_t bh = u / R, r = u % R;
            int64_t i = rows ? rows[r] : r;
            /* causal: local key j allowed iff k_pos0 + j <= q_pos0 + i */
            int64_t count = causal ? prefix_count(q_pos0 + i - k_pos0, Nkb) : Nkb;
            row_attention(q + (bh * Nq + i) * d, kb + bh * Nkb * d, vb + bh * Nkb * d,
                          Nkb, d, count, scale, s_buf, o + u * d, &m[u], &l[u], NULL);
        }
        free(s_buf);
    }
    return err;
}

/* Merge state b into state a, in place, for n rows of width d. */
void oracle_merge(double* o_a, double* m_a, double* l_a,
                  const double* o_b, const double* m_b, const double* l_b,
                  int64_t n, int64_t d) {
    for (int64_t r = 0; r < n; ++r) {
        double ma = m_a[r], mb = m_b[r];
        double M = ma > mb ? ma : mb;
        if (M == -INFINITY) { /* both empty: stays the empty state */
            for (int64_t c = 0; c < d; ++c) o_a[r * d + c] = 0.0;
            m_a[r] = -INFINITY;
            l_a[r] = 0.0;
            continue;
        }
        double wa = (ma == -INFINITY) ? 0.0 : l_a[r] * exp(ma - M);
        double wb = (mb == -INFINITY) ? 0.0 : l_b[r] * exp(mb - M);
        double lsum = wa + wb;
        for (int64_t c = 0; c < d; ++c)
            o_a[r * d + c] = (wa * o_a[r * d + c] + wb * o_b[r * d + c]) / lsum;
        m_a[r] = M;
        l_a[r] = lsum;
    }
}

/* Log-sum-exp of a state: m + ln l (natural log), -inf for the empty state. */
void oracle_state_lse(const double* m, const double* l, int64_t n, double* lse) {
    for (int64_t r = 0; r < n; ++r)
        lse[r] = (m[r] == -INFINITY || l[r] <= 0.0) ? -INFINITY : m[r] + log(l[r]);
}

/* ------------------------------------------------------------- gradients */

/* Gradients of L = sum dO . O with respect to q, k and v (formulas in the
 * header).  q, dout: [B,H,Nq,d]; k, v: [B,H,Nk,d].  dq gets the rows q_rows
 * ([B,H,n_q,d]; all Nq rows when q_rows == NULL), dk and dv the key rows
 * k_rows ([B,H,n_k,d]; all Nk rows when k_rows == NULL).  Each (b, h) first
 * computes every query row's log-sum-exp and D_i, then the requested rows
 * one by one, each as a sum over the other side's rows. */
int oracle_attention_bwd(const double* q, const double* k, const double* v, const double* dout,
                         int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                         int causal, double scale,
                         const int64_t* q_rows, int64_t n_q, const int64_t* k_rows, int64_t n_k,
                         double* dq, double* dk, double* dv) {
    if (B <= 0 || H <= 0 || Nq < 0 || Nk < 0 || d <= 0) return -1;
    const int64_t RQ = q_rows ? n_q : Nq, RK = k_rows ? n_k : Nk, BH = B * H;
    double* lse = (double*)malloc(sizeof(double) * (size_t)(BH * Nq > 0 ? BH * Nq : 1));
    double* Dr = (double*)malloc(sizeof(double) * (size_t)(BH * Nq > 0 ? BH * Nq : 1));
    if (!lse || !Dr) {
        free(lse);
        free(Dr);
        return -2;
    }
    int err = 0;
    /* pass 1: per query row, the log-sum-exp and D_i = sum_j P_ij dP_ij */
#pragma omp parallel
    {
        double* s_buf = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double* p_buf = (double*)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
        double* o_buf = (double*)malloc(sizeof(double) * (size_t)d);
        if (!s_buf || !p_buf || !o_buf) {
#pragma omp atomic write
            err = -2;
        }
#pragma omp for schedule(dynamic, 8)
        for (int64_t u = 0; u < BH * Nq; ++u) {
            if (!s_buf || !p_buf || !o_buf) continue;
            const int64_t bh = u / Nq, i = u % Nq;
            const int64_t count = causal ? prefix_count(i + Nk - Nq, Nk) : Nk;
            const double* qi = q + (bh * Nq + i) * d;
            const double* doi = dout + (bh * Nq + i) * d;
            double m, l;
            row_attention(qi, k + bh * Nk * d, v + bh * Nk * d, Nk, d, count, scale, s_buf, o_buf, &m, &l, p_buf);
            lse[u] = count > 0 ? m + log(l) : -INFINITY;
            double D = 0.0;
            for (int64_t j = 0; j < count; ++j) {
                double dp = 0.0;
                for (int64_t c = 0; c < d; ++c) dp += doi[c] * v[(bh * Nk + j) * d + c];
                D += p_buf[j] * dp;
            }
            Dr[u] = D;
        }
        free(s_buf);
        free(p_buf);
        free(o_buf);
    }
    if (err) {
        free(lse);
        free(Dr);
        return err;
    }
    /* P_ij and dS_ij from the row statistics */
#define ORACLE_P(bh, i, j, p_out, ds_out)                                                  \
    do {                                                                                 \
        const double* qi_ = q + ((bh) * Nq + (i)) * d;                                   \
        const double* di_ = dout + ((bh) * Nq + (i)) * d;                                \
        const double* kj_ = k + ((bh) * Nk + (j)) * d;                                   \
        const double* vj_ = v + ((bh) * Nk + (j)) * d;                                   \
        double dot_ = 0.0, dp_ = 0.0;                                                    \
        for (int64_t c_ = 0; c_ < d; ++c_) {                                             \
            dot_ += qi_[c_] * kj_[c_];                                                   \
            dp_ += di_[c_] * vj_[c_];                                                    \
        }                                                                                \
        (p_out) = exp(scale * dot_ - lse[(bh) * Nq + (i)]);                              \
        (ds_out) = (p_out) * (dp_ - Dr[(bh) * Nq + (i)]);                                \
    } while (0)
    /* pass 2: dq rows */
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t u = 0; u < BH * RQ; ++u) {
        const int64_t bh = u / RQ, r = u % RQ, i = q_rows ? q_rows[r] : r;
        double* out = dq + u * d;
        for (int64_t c = 0; c < d; ++c) out[c] = 0.0;
        const int64_t count = causal ? prefix_count(i + Nk - Nq, Nk) : Nk;
        for (int64_t j = 0; j < count; ++j) {
            double P, dS;
            ORACLE_P(bh, i, j, P, dS);
            (void)P;
            for (int64_t c = 0; c < d; ++c) out[c] += scale * dS * k[(bh * Nk + j) * d + c];
        }
    }
    /* pass 3: dk and dv rows; key j is seen by the rows i with j <= i + Nk - Nq */
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t u = 0; u < BH * RK; ++u) {
        const int64_t bh = u / RK, r = u % RK, j = k_rows ? k_rows[r] : r;
        double* gk = dk + u * d;
        double* gv = dv + u * d;
        for (int64_t c = 0; c < d; ++c) gk[c] = gv[c] = 0.0;
        const int64_t i0 = causal ? (j - (Nk - Nq) > 0 ? j - (Nk - Nq) : 0) : 0;
        for (int64_t i = i0; i < Nq; ++i) {
            double P, dS;
            ORACLE_P(bh, i, j, P, dS);
            for (int64_t c = 0; c < d; ++c) {
                gv[c] += P * dout[(bh * Nq + i) * d + c];
                gk[c] += scale * dS * q[(bh * Nq + i) * d + c];
            }
        }
    }
#undef ORACLE_P
    free(lse);
    free(Dr);
    return 0;
}

/* ------------------------------------------------------------ W4A16 layer */

/* The 4-bit value of weight k of a row from its packed words (bit position
 * 4 (e / 2) + 16 (e % 2) for e = k % 8 in word k / 8). */
int oracle_w4_value(const uint32_t* row_words, int64_t k) {
    const int64_t j = k / 8, e = k % 8;
    const int shift = (int)(4 * (e / 2) + 16 * (e % 2));
    return (int)((row_words[j] >> shift) & 0xFu);
}

/* y [M, N] = x [M, K] . W^T with W[n][k] = (q[n][k] - zero[n][k/G]) * scale[n][k/G];
 * packed: [N, K/8] words, zero: [N, K/G], scale: [N, K/G] (already decoded to
 * doubles).  K must be a multiple of 8 and of G. */
int oracle_w4a16(const double* x, const uint32_t* packed, const uint8_t* zero, const double* scale,
                 int64_t M, int64_t N, int64_t K, int64_t G, double* y) {
    if (M < 0 || N < 0 || K <= 0 || G <= 0 || K % 8 || K % G) return -1;
    const int64_t ng = K / G;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t* rw = packed + n * (K / 8);
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int64_t g = k / G;
                const double w = (double)(oracle_w4_value(rw, k) - (int)zero[n * ng + g]) * scale[n * ng + g];
                acc += x[m * K + k] * w;
            }
            y[m * N + n] = acc;
        }
    }
    return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
