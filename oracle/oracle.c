/*
 * fp64 CPU oracle for scaled-dot-product attention and LayerNorm.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the tests, the package smoke check and the benchmark's
 * CPU-baseline leg do.  It shares no code, header or table with the HIP
 * library: it decodes bf16 and e4m3fn bytes with its own routines below.
 *
 * Every result is the plain definition, written out in double precision with
 * plain loops and a fixed summation order per output row (OpenMP splits
 * rows, never a sum):
 *
 *   s_j  = scale * sum_d q_d k_jd + mask_j            (additive mask, added
 *          after scaling: head_dim>128 GQA Flash-Decode kernel, "Input
 *          contract": 0 keeps a key, -inf drops it)
 *   m    = max_j s_j,  Z = sum_j exp(s_j - m)
 *   o_d  = sum_j exp(s_j - m) v_jd / Z,  lse = m + ln Z
 *
 * Non-causal (vit-encoder-neuron-kernels, "Supported shapes and limits":
 * bidirectional self-attention only).  Query head h reads KV head h / G with
 * G = num_kv_groups, i.e. the G query heads sharing a KV head are contiguous
 * (Prefill Context-Parallel Attention POC, "Layout": Q heads that share a KV
 * head are packed together).  A row whose keys are all masked returns o = 0
 * and lse = -inf (the pages do not define this case).
 *
 * LayerNorm is standard LayerNorm (vit-encoder-neuron-kernels, "Supported
 * shapes and limits": standard LayerNorm, not RMSNorm):
 *   mu = sum x / N, var = sum (x - mu)^2 / N (biased), rstd = 1/sqrt(var+eps),
 *   y = (x - mu) * rstd * gamma + beta.
 *
 * The paged prefill gathers logical key j of KV head h from physical block
 * block_table[j / bs], row j % bs, of a [num_blocks, Hkv, bs, D] cache, and
 * drops keys j >= actual_history_len with an additive -inf bias (Prefill
 * Context-Parallel Attention POC, "Layout" and "Benchmark": runtime additive
 * score bias derived from actual_history_len; the final partial block is
 * padded and biased).  Keys are e4m3fn codes times one fp32 scale per tensor.
 * The prefill with current-token attention (oracle_prefill_causal) is the
 * one causal computation here: token t also attends current tokens 0..t.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1, OR_E4M3 = 2, OR_F64 = 3 };

/* bf16 is the top half of an IEEE binary32: widen by shifting left 16. */
double oracle_bf16_to_f64(uint16_t bits) {
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* OCP 8-bit e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
 * infinities, S.1111.111 is NaN, largest finite 448.  Exponent field 0 is
 * subnormal: 2^-6 * m/8. */
double oracle_e4m3_to_f64(uint8_t bits) {
    int s = (bits >> 7) & 1;
    int e = (bits >> 3) & 0xF;
    int m = bits & 0x7;
    double mag;
    if (e == 0xF && m == 0x7) return NAN;
    if (e == 0)
        mag = ldexp((double)m / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -mag : mag;
}

static double load_elem(const void *p, int dtype, int64_t i) {
    switch (dtype) {
    case OR_F32: return (double)((const float *)p)[i];
    case OR_BF16: return oracle_bf16_to_f64(((const uint16_t *)p)[i]);
    case OR_E4M3: return oracle_e4m3_to_f64(((const uint8_t *)p)[i]);
    default: return ((const double *)p)[i];
    }
}

void oracle_decode(const void *src, int dtype, int64_t n, double *dst) {
    for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, dtype, i);
}

/* One attention row: q[D], keys k[j*D], values v[j*D] for j < n, optional
 * additive mask[j].  s is caller scratch of n doubles. */
static void attend_row(const double *q, const double *k, const double *v, const double *mask,
                       int64_t n, int D, double scale, double *s, double *o, double *lse) {
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += q[d] * k[j * D + d];
        s[j] = scale * acc + (mask ? mask[j] : 0.0);
        if (s[j] > m) m = s[j];
    }
    for (int d = 0; d < D; ++d) o[d] = 0.0;
    if (m == -INFINITY) { /* every key masked */
        if (lse) *lse = -INFINITY;
        return;
    }
    double Z = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double e = exp(s[j] - m);
        s[j] = e;
        Z += e;
    }
    for (int64_t j = 0; j < n; ++j) {
        if (s[j] == 0.0) continue; /* exp underflowed or key masked: contributes nothing */
        for (int d = 0; d < D; ++d) o[d] += s[j] * v[j * D + d];
    }
    for (int d = 0; d < D; ++d) o[d] /= Z;
    if (lse) *lse = m + log(Z);
}

/*
 * Dense SDPA.  q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D] contiguous in the given
 * dtypes; mask nullable fp64 [B,Skv] (the [B,1,1,Skv] additive mask with its
 * unit dims dropped).  out [B,Hq,Sq,D] fp64, lse nullable [B,Hq,Sq].
 * Returns 0, or -1 for bad shapes.
 */
int oracle_sdpa(const void *q, int q_dtype, const void *k, int k_dtype, const void *v, int v_dtype,
                const double *mask, int B, int Hq, int Hkv, int Sq, int Skv, int D, double scale,
                double *out, double *lse) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv <= 0 || D <= 0 || Hq % Hkv) return -1;
    const int G = Hq / Hkv;
    const int64_t kv_elems = (int64_t)B * Hkv * Skv * D;
    double *kd = (double *)malloc(sizeof(double) * kv_elems);
    double *vd = (double *)malloc(sizeof(double) * kv_elems);
    if (!kd || !vd) { free(kd); free(vd); return -2; }
    oracle_decode(k, k_dtype, kv_elems, kd);
    oracle_decode(v, v_dtype, kv_elems, vd);
    const int64_t rows = (int64_t)B * Hq * Sq;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * Skv);
        double *qr = (double *)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < rows; ++r) {
            int64_t b = r / ((int64_t)Hq * Sq);
            int h = (int)((r / Sq) % Hq);
            int hk = h / G;
            for (int d = 0; d < D; ++d) qr[d] = load_elem(q, q_dtype, r * D + d);
            const int64_t kv0 = ((b * Hkv + hk) * (int64_t)Skv) * D;
            attend_row(qr, kd + kv0, vd + kv0, mask ? mask + b * Skv : NULL, Skv, D, scale, s,
                       out + r * D, lse ? lse + r : NULL);
        }
        free(s);
        free(qr);
    }
    free(kd);
    free(vd);
    return 0;
}

/*
 * LayerNorm over the last dim of x [rows, N] (fp64).  gamma/beta nullable
 * (affine-free).  y [rows,N], mean/rstd nullable [rows].
 */
int oracle_layernorm(const double *x, int64_t rows, int N, const double *gamma, const double *beta,
                     double eps, double *y, double *mean, double *rstd) {
    if (rows < 0 || N <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * N;
        double mu = 0.0;
        for (int i = 0; i < N; ++i) mu += xr[i];
        mu /= N;
        double var = 0.0;
        for (int i = 0; i < N; ++i) var += (xr[i] - mu) * (xr[i] - mu);
        var /= N;
        double rs = 1.0 / sqrt(var + eps);
        for (int i = 0; i < N; ++i) {
            double t = (xr[i] - mu) * rs;
            y[r * N + i] = t * (gamma ? gamma[i] : 1.0) + (beta ? beta[i] : 0.0);
        }
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = rs;
    }
    return 0;
}

/*
 * Encoder block: attention (Hq == Hkv == H; S_q query tokens over S_kv keys,
 * mask [B, S_kv]), the head outputs laid out token-major as [B, S_q, H*D]
 * (head h owns columns h*D .. h*D+D-1), added to the fp32 residual stream,
 * then LayerNorm over H*D.
 *   attn_out  [B,H,S_q,D] fp64 (nullable)
 *   res_out   [B,S_q,H*D] fp64 = residual + attention
 *   ln_out    [B,S_q,H*D] fp64, mean/rstd [B*S_q] (nullable)
 */
int oracle_encoder_block(const void *q, const void *k, const void *v, int in_dtype, const double *mask,
                         int B, int H, int Sq, int Skv, int D, double scale, const float *residual,
                         const double *gamma, const double *beta, double eps, double *attn_out,
                         double *res_out, double *ln_out, double *mean, double *rstd) {
    const int64_t n_attn = (int64_t)B * H * Sq * D;
    double *o = attn_out ? attn_out : (double *)malloc(sizeof(double) * n_attn);
    if (!o) return -2;
    int rc = oracle_sdpa(q, in_dtype, k, in_dtype, v, in_dtype, mask, B, H, H, Sq, Skv, D, scale, o, NULL);
    if (rc) { if (!attn_out) free(o); return rc; }
    const int N = H * D;
    for (int b = 0; b < B; ++b)
        for (int s = 0; s < Sq; ++s)
            for (int h = 0; h < H; ++h)
                for (int d = 0; d < D; ++d) {
                    int64_t t = ((int64_t)b * Sq + s) * N + (int64_t)h * D + d;
                    res_out[t] = (double)residual[t] + o[(((int64_t)b * H + h) * Sq + s) * D + d];
                }
    if (!attn_out) free(o);
    if (ln_out) rc = oracle_layernorm(res_out, (int64_t)B * Sq, N, gamma, beta, eps, ln_out, mean, rstd);
    return rc;
}

/*
 * History-only paged prefill, evaluated for the query tokens listed in
 * rows[n_rows] and every query head.  q [Hq, Lq, D] (bf16 or other dtype),
 * k_cache/v_cache [num_blocks, Hkv, bs, D] e4m3fn codes, block_table
 * [max_blocks] int32.  out [Hq, n_rows, D] fp64, lse nullable [Hq, n_rows].
 */
int oracle_prefill_paged(const void *q, int q_dtype, const uint8_t *k_cache, const uint8_t *v_cache,
                         double k_scale, double v_scale, const int32_t *block_table, int max_blocks,
                         int num_blocks, int bs, int L_act, double scale, int Hq, int Hkv, int Lq, int D,
                         const int64_t *rows, int n_rows, double *out, double *lse) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || bs <= 0 || D <= 0 || L_act < 0 ||
        L_act > (int64_t)max_blocks * bs)
        return -1;
    const int G = Hq / Hkv;
    /* The additive bias removes every key j >= L_act, so the softmax runs over
     * logical keys 0..L_act-1 gathered through the block table. */
    const int64_t n = L_act;
    double *kd = (double *)malloc(sizeof(double) * (size_t)Hkv * (n ? n : 1) * D);
    double *vd = (double *)malloc(sizeof(double) * (size_t)Hkv * (n ? n : 1) * D);
    if (!kd || !vd) { free(kd); free(vd); return -2; }
    for (int h = 0; h < Hkv; ++h)
        for (int64_t j = 0; j < n; ++j) {
            int32_t phys = block_table[j / bs];
            if (phys < 0 || phys >= num_blocks) { free(kd); free(vd); return -3; }
            int64_t src = (((int64_t)phys * Hkv + h) * bs + j % bs) * D;
            for (int d = 0; d < D; ++d) {
                kd[((int64_t)h * n + j) * D + d] = oracle_e4m3_to_f64(k_cache[src + d]) * k_scale;
                vd[((int64_t)h * n + j) * D + d] = oracle_e4m3_to_f64(v_cache[src + d]) * v_scale;
            }
        }
    const int64_t total = (int64_t)Hq * n_rows;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (n ? n : 1));
        double *qr = (double *)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < total; ++r) {
            int h = (int)(r / n_rows);
            int64_t t = rows[r % n_rows];
            for (int d = 0; d < D; ++d) qr[d] = load_elem(q, q_dtype, ((int64_t)h * Lq + t) * D + d);
            const int64_t kv0 = (int64_t)(h / G) * n * D;
            attend_row(qr, kd + kv0, vd + kv0, NULL, n, D, scale, s, out + r * D, lse ? lse + r : NULL);
        }
        free(s);
        free(qr);
    }
    free(kd);
    free(vd);
    return 0;
}

/*
 * Prefill with current-token attention: query token t of head h attends the
 * L_act history keys of the paged cache (gathered and biased as above),
 * followed by the keys of the current tokens 0..t of its own KV head
 * (causal).  Prefill Context-Parallel Attention POC, introduction: its first
 * version leaves out attention among the current tokens; this adds it.  The
 * current tokens' K/V are k_cur/v_cur [Hkv, Lq, D] in cur_dtype, with no
 * scale.  L_act may be 0 (no history).  The softmax runs over the joined key
 * list in that order: history keys 0..L_act-1, then current keys 0..t.
 * out [Hq, n_rows, D] fp64, lse nullable [Hq, n_rows].
 */
int oracle_prefill_causal(const void *q, int q_dtype, const uint8_t *k_cache, const uint8_t *v_cache,
                          double k_scale, double v_scale, const int32_t *block_table, int max_blocks,
                          int num_blocks, int bs, int L_act, const void *k_cur, const void *v_cur, int cur_dtype,
                          double scale, int Hq, int Hkv, int Lq, int D, const int64_t *rows, int n_rows,
                          double *out, double *lse) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || bs <= 0 || D <= 0 || Lq <= 0 || L_act < 0 ||
        L_act > (int64_t)max_blocks * bs)
        return -1;
    const int G = Hq / Hkv;
    const int64_t n = (int64_t)L_act + Lq; /* keys per KV head in the joined list */
    double *kd = (double *)malloc(sizeof(double) * (size_t)Hkv * n * D);
    double *vd = (double *)malloc(sizeof(double) * (size_t)Hkv * n * D);
    if (!kd || !vd) { free(kd); free(vd); return -2; }
    for (int h = 0; h < Hkv; ++h) {
        for (int64_t j = 0; j < L_act; ++j) {
            int32_t phys = block_table[j / bs];
            if (phys < 0 || phys >= num_blocks) { free(kd); free(vd); return -3; }
            int64_t src = (((int64_t)phys * Hkv + h) * bs + j % bs) * D;
            for (int d = 0; d < D; ++d) {
                kd[((int64_t)h * n + j) * D + d] = oracle_e4m3_to_f64(k_cache[src + d]) * k_scale;
                vd[((int64_t)h * n + j) * D + d] = oracle_e4m3_to_f64(v_cache[src + d]) * v_scale;
            }
        }
        for (int64_t j = 0; j < Lq; ++j)
            for (int d = 0; d < D; ++d) {
                int64_t src = ((int64_t)h * Lq + j) * D + d;
                kd[((int64_t)h * n + L_act + j) * D + d] = load_elem(k_cur, cur_dtype, src);
                vd[((int64_t)h * n + L_act + j) * D + d] = load_elem(v_cur, cur_dtype, src);
            }
    }
    const int64_t total = (int64_t)Hq * n_rows;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * n);
        double *qr = (double *)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < total; ++r) {
            int h = (int)(r / n_rows);
            int64_t t = rows[r % n_rows];
            if (t < 0 || t >= Lq) { bad = 1; continue; }
            for (int d = 0; d < D; ++d) qr[d] = load_elem(q, q_dtype, ((int64_t)h * Lq + t) * D + d);
            const int64_t kv0 = (int64_t)(h / G) * n * D;
            /* the first L_act + t + 1 keys of the joined list: history, then current 0..t */
            attend_row(qr, kd + kv0, vd + kv0, NULL, L_act + t + 1, D, scale, s, out + r * D, lse ? lse + r : NULL);
        }
        free(s);
        free(qr);
    }
    free(kd);
    free(vd);
    return bad ? -4 : 0;
}
