/*
 * Float64 CPU oracle for the forward pass of multi-head scaled dot-product
 * attention.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg are its only callers.  It shares no code,
 * header, table or helper with the GPU library and never calls it.
 *
 * What it computes -- the plain definition, with no tiling and no online
 * softmax:
 *     out = softmax(scale * Q K^T + M) V
 * following
 *   - "Self-Attention" (blog-15c notes), section "Scaled Dot-Product
 *     Attention" (the Attention(Q,K,V) formula) and section "Causal Masking"
 *     (M_ij = 0 for j <= i and -inf for j > i, added before the softmax);
 *   - "Attention from First Principles", section 4 "Tiny example" (scores,
 *     scale, causal mask, row softmax, multiply by V, in that order);
 *   - "Attention from Scratch" (KubeDojo module 1.4.3), Part 2's teaching
 *     implementation (forbidden logits get exactly zero probability, the
 *     softmax runs over the key axis, d_v may differ from d_k) and Part 3
 *     (causal and padding allowed-masks combined by logical AND).
 *
 * Readings where the pages leave a step open:
 *   - a masked key is excluded outright (an exact -inf logit, so exactly zero
 *     weight), never a finite sentinel;
 *   - padding is right padding given by one valid length L_b per sequence,
 *     clamped to [0, Skv]; the queries of sequence b are its last
 *     n_b = min(Sq, L_b) valid positions, so query row i sits at absolute
 *     position p = L_b - n_b + i (bottom-right causal alignment: a single
 *     decode query is the newest token and sees every cached key, as the
 *     "Scaled dot-product attention with masking" page says of decode);
 *   - query rows i >= n_b are padding and their output is exactly 0, and so
 *     is any row with no visible key;
 *   - the softmax subtracts the row maximum before exponentiating, the stable
 *     form that page's Part 7 (debugging) asks for.
 *
 * Explicit allowed-mask: an optional byte array, nonzero where query row i
 * of (b, h) may see key j (the True-means-allowed boolean mask of "Attention
 * from Scratch", KubeDojo module 1.4.3, Part 3), combined with the causal
 * and length rules by logical AND as that part combines its causal and
 * padding masks.  Element (b, h, i, j) is mask[b*sb + h*sh + i*Skv + j];
 * a stride of 0 broadcasts over that axis.
 *
 * Additive bias: an optional array of the inputs' element type added to
 * the scaled logits before the softmax, logit_ij = scale * q_i . k_j +
 * bias_ij -- the float mask that "Attention from Scratch" (KubeDojo module
 * 1.4.3), Part 7 describes as an additive bias, where a boolean mask only
 * allows or forbids.  Element (b, h, i, j) is bias[b*bsb + h*bsh + i*Skv +
 * j].  A bias of -inf forbids the key exactly as a False mask entry does
 * (exactly zero weight; a row whose keys are all forbidden is 0).
 *
 * Grouped heads (GQA / MQA): with H_kv key/value heads for H query heads
 * (H a multiple of H_kv), query head h reads key/value head h / (H / H_kv).
 * That is the grouping of "Attention from First Principles", section "MHA,
 * GQA, MQA -- the KV cache lever" (consecutive query heads share one K/V
 * head), and what the repeat_interleave expansion of K and V along the head
 * axis in "Scaled dot-product attention with masking", section
 * "Grouped-query attention (GQA)", computes.  H_kv = H is multi-head
 * attention.
 *
 * Inputs may be float64, float32 or bfloat16 bit patterns; each element is
 * widened exactly to double before any arithmetic.  All arithmetic is in
 * double, sums in ascending index order.  Built without -ffast-math.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { OR_OK = 0, OR_E_NULL = 1, OR_E_SHAPE = 2, OR_E_DTYPE = 4, OR_E_ARG = 7, OR_E_NOMEM = 9 };
enum { OR_F64 = 0, OR_F32 = 1, OR_BF16 = 2 };

/* Exact widening of one stored element to double. */
static double load_elem(const void* base, int dtype, size_t idx) {
    if (dtype == OR_F64) return ((const double*)base)[idx];
    if (dtype == OR_F32) return (double)((const float*)base)[idx];
    /* bfloat16 is the upper half of an IEEE binary32 */
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

typedef struct {
    const void *q, *k, *v;
    int dtype;
    double* out;      /* [B,H,Sq,dv] */
    double* weights;  /* optional [B,H,Sq,Skv] */
    int B, H, Hkv, Sq, Skv, d, dv;
    double scale;
    int causal;
    const int32_t* kv_lens;
    const uint8_t* mask;  /* optional allowed-mask, see above */
    long long mask_sb, mask_sh;
    const void* bias;     /* optional additive bias (dtype elements), see above */
    long long bias_sb, bias_sh;
    int next_pair;    /* work counter, guarded by mu */
    pthread_mutex_t mu;
} job_t;

/* Valid length of sequence b, clamped to [0, Skv]. */
static int valid_len(const job_t* J, int b) {
    long L = J->kv_lens ? (long)J->kv_lens[b] : (long)J->Skv;
    if (L < 0) L = 0;
    if (L > J->Skv) L = J->Skv;
    return (int)L;
}

/* The additive bias of (b, h, i, j), 0 without one. */
static double bias_at(const job_t* J, int b, int h, int i, int j) {
    if (!J->bias) return 0.0;
    return load_elem(J->bias, J->dtype,
                     (size_t)(b * J->bias_sb + h * J->bias_sh + (long long)i * J->Skv + j));
}

/* Mask M: is key j visible to query row i (absolute position p) of (b, h)? */
static int key_visible(const job_t* J, int b, int h, int i, int j, int p, int L) {
    if (j >= L) return 0;          /* padding: past the valid length */
    if (J->mask && !J->mask[b * J->mask_sb + h * J->mask_sh + (long long)i * J->Skv + j])
        return 0;                  /* the caller's allowed-mask */
    if (bias_at(J, b, h, i, j) == -INFINITY) return 0; /* a -inf bias forbids the key */
    if (!J->causal) return 1;
    return j <= p;                 /* causal: M_pj = 0 iff j <= p */
}

/* scale * (q_row . k_j) + bias, the row's logit for key j */
static double score(const job_t* J, size_t qrow, size_t kbase, int j, double bias) {
    double acc = 0.0;
    for (int c = 0; c < J->d; ++c)
        acc += load_elem(J->q, J->dtype, qrow + c) *
               load_elem(J->k, J->dtype, kbase + (size_t)j * J->d + c);
    return J->scale * acc + bias;
}

/* One query row: out_row[dv] and optionally w_row[Skv]; s is scratch of Skv. */
static void one_row(const job_t* J, int b, int h, int i, double* out_row, double* w_row,
                    double* s) {
    const int Sq = J->Sq, Skv = J->Skv, dv = J->dv;
    const int L = valid_len(J, b);
    const int n = Sq < L ? Sq : L;
    const int hk = h / (J->H / J->Hkv); /* the key/value head of query head h */
    const size_t qrow = (((size_t)b * J->H + h) * Sq + i) * (size_t)J->d;
    const size_t kbase = ((size_t)b * J->Hkv + hk) * (size_t)Skv * J->d;
    const size_t vbase = ((size_t)b * J->Hkv + hk) * (size_t)Skv * dv;

    for (int c = 0; c < dv; ++c) out_row[c] = 0.0;
    if (w_row)
        for (int j = 0; j < Skv; ++j) w_row[j] = 0.0;
    if (i >= n) return;            /* padded query row: exactly zero */
    const int p = (L - n) + i;     /* absolute position of this query */

    /* logits of the visible keys and their maximum */
    double m = -INFINITY;
    int any = 0;
    for (int j = 0; j < Skv; ++j) {
        if (!key_visible(J, b, h, i, j, p, L)) continue;
        s[j] = score(J, qrow, kbase, j, bias_at(J, b, h, i, j));
        if (s[j] > m) m = s[j];
        any = 1;
    }
    if (!any) return;              /* no visible key: exactly zero */

    /* softmax normaliser over the visible keys */
    double l = 0.0;
    for (int j = 0; j < Skv; ++j)
        if (key_visible(J, b, h, i, j, p, L)) l += exp(s[j] - m);

    /* weighted mixture of value rows */
    for (int j = 0; j < Skv; ++j) {
        if (!key_visible(J, b, h, i, j, p, L)) continue;
        const double w = exp(s[j] - m) / l;
        if (w_row) w_row[j] = w;
        for (int c = 0; c < dv; ++c)
            out_row[c] += w * load_elem(J->v, J->dtype, vbase + (size_t)j * dv + c);
    }
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    double* s = (double*)malloc(sizeof(double) * (size_t)J->Skv);
    if (!s) return (void*)1;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        int pair = J->next_pair++;
        pthread_mutex_unlock(&J->mu);
        if (pair >= J->B * J->H) break;
        int b = pair / J->H, h = pair % J->H;
        for (int i = 0; i < J->Sq; ++i) {
            size_t row = ((size_t)b * J->H + h) * J->Sq + i;
            one_row(J, b, h, i, J->out + row * J->dv,
                    J->weights ? J->weights + row * (size_t)J->Skv : NULL, s);
        }
    }
    free(s);
    return NULL;
}

static int run(job_t* J, int nthreads) {
    if (!J->q || !J->k || !J->v || !J->out) return OR_E_NULL;
    if (J->dtype != OR_F64 && J->dtype != OR_F32 && J->dtype != OR_BF16) return OR_E_DTYPE;
    if (J->B <= 0 || J->H <= 0 || J->Sq <= 0 || J->Skv <= 0 || J->d <= 0 || J->dv <= 0 ||
        J->Sq > J->Skv || J->Hkv <= 0 || J->H % J->Hkv != 0)
        return OR_E_SHAPE;
    if (!isfinite(J->scale)) return OR_E_ARG;
    if (nthreads <= 0) {
        long nc = sysconf(_SC_NPROCESSORS_ONLN);
        nthreads = nc > 0 ? (int)nc : 1;
    }
    if (nthreads > J->B * J->H) nthreads = J->B * J->H;
    J->next_pair = 0;
    pthread_mutex_init(&J->mu, NULL);
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
    if (!th) {
        pthread_mutex_destroy(&J->mu);
        return OR_E_NOMEM;
    }
    int started = 0, failed = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&th[t], NULL, worker, J) != 0) break;
        ++started;
    }
    if (started == 0) failed = (worker(J) != NULL);
    for (int t = 0; t < started; ++t) {
        void* rv = NULL;
        pthread_join(th[t], &rv);
        if (rv) failed = 1;
    }
    free(th);
    pthread_mutex_destroy(&J->mu);
    return failed ? OR_E_NOMEM : OR_OK;
}

/* out is [B,H,Sq,dv] float64; q is [B,H,Sq,d], k is [B,Hkv,Skv,d], v is
   [B,Hkv,Skv,dv], row-major, all of one dtype (0 f64, 1 f32, 2 bf16 bits).
   kv_lens is a host int32[B] or NULL (every sequence has Skv valid keys).
   Returns 0, or 1 null pointer, 2 bad shape (a size <= 0, Sq > Skv, or H
   not a multiple of Hkv), 4 bad dtype, 7 non-finite scale, 9 out of memory.
   nthreads <= 0 uses every online core. */
int oracle_attn_fwd_gqa(const void* q, const void* k, const void* v, int dtype, double* out,
                        int B, int H, int Hkv, int Sq, int Skv, int d, int dv, double scale,
                        int causal, const int32_t* kv_lens, int nthreads) {
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dtype = dtype; J.out = out; J.weights = NULL;
    J.B = B; J.H = H; J.Hkv = Hkv; J.Sq = Sq; J.Skv = Skv; J.d = d; J.dv = dv;
    J.scale = scale; J.causal = causal ? 1 : 0; J.kv_lens = kv_lens;
    return run(&J, nthreads);
}

/* As oracle_attn_fwd_gqa, with an allowed-mask (NULL: none) whose element
   (b, h, i, j) is mask[b*mask_sb + h*mask_sh + i*Skv + j], nonzero = allowed.
   Negative strides return 2 (bad shape). */
int oracle_attn_fwd_mask(const void* q, const void* k, const void* v, int dtype, double* out,
                         int B, int H, int Hkv, int Sq, int Skv, int d, int dv, double scale,
                         int causal, const int32_t* kv_lens, const uint8_t* mask,
                         long long mask_sb, long long mask_sh, int nthreads) {
    if (mask_sb < 0 || mask_sh < 0) return OR_E_SHAPE;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dtype = dtype; J.out = out; J.weights = NULL;
    J.B = B; J.H = H; J.Hkv = Hkv; J.Sq = Sq; J.Skv = Skv; J.d = d; J.dv = dv;
    J.scale = scale; J.causal = causal ? 1 : 0; J.kv_lens = kv_lens;
    J.mask = mask; J.mask_sb = mask_sb; J.mask_sh = mask_sh;
    return run(&J, nthreads);
}

/* As oracle_attn_fwd_mask, and also the weight tensor [B,H,Sq,Skv]. */
int oracle_attn_fwd_weights_mask(const void* q, const void* k, const void* v, int dtype,
                                 double* out, double* weights, int B, int H, int Hkv, int Sq,
                                 int Skv, int d, int dv, double scale, int causal,
                                 const int32_t* kv_lens, const uint8_t* mask, long long mask_sb,
                                 long long mask_sh, int nthreads) {
    if (!weights) return OR_E_NULL;
    if (mask_sb < 0 || mask_sh < 0) return OR_E_SHAPE;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dtype = dtype; J.out = out; J.weights = weights;
    J.B = B; J.H = H; J.Hkv = Hkv; J.Sq = Sq; J.Skv = Skv; J.d = d; J.dv = dv;
    J.scale = scale; J.causal = causal ? 1 : 0; J.kv_lens = kv_lens;
    J.mask = mask; J.mask_sb = mask_sb; J.mask_sh = mask_sh;
    return run(&J, nthreads);
}

/* Every option at once: an allowed-mask (as oracle_attn_fwd_mask; NULL:
   none), an additive bias of the inputs' dtype whose element (b, h, i, j) is
   bias[b*bias_sb + h*bias_sh + i*Skv + j] (NULL: none), and optionally the
   weight tensor (weights NULL: not returned).  Negative strides return 2. */
int oracle_attn_fwd_ex(const void* q, const void* k, const void* v, int dtype, double* out,
                       double* weights, int B, int H, int Hkv, int Sq, int Skv, int d, int dv,
                       double scale, int causal, const int32_t* kv_lens, const uint8_t* mask,
                       long long mask_sb, long long mask_sh, const void* bias, long long bias_sb,
                       long long bias_sh, int nthreads) {
    if (mask_sb < 0 || mask_sh < 0 || bias_sb < 0 || bias_sh < 0) return OR_E_SHAPE;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dtype = dtype; J.out = out; J.weights = weights;
    J.B = B; J.H = H; J.Hkv = Hkv; J.Sq = Sq; J.Skv = Skv; J.d = d; J.dv = dv;
    J.scale = scale; J.causal = causal ? 1 : 0; J.kv_lens = kv_lens;
    J.mask = mask; J.mask_sb = mask_sb; J.mask_sh = mask_sh;
    J.bias = bias; J.bias_sb = bias_sb; J.bias_sh = bias_sh;
    return run(&J, nthreads);
}

/* Multi-head attention: oracle_attn_fwd_gqa with Hkv = H. */
int oracle_attn_fwd(const void* q, const void* k, const void* v, int dtype, double* out, int B,
                    int H, int Sq, int Skv, int d, int dv, double scale, int causal,
                    const int32_t* kv_lens, int nthreads) {
    return oracle_attn_fwd_gqa(q, k, v, dtype, out, B, H, H, Sq, Skv, d, dv, scale, causal,
                               kv_lens, nthreads);
}

/* As oracle_attn_fwd_gqa, and also the weight tensor [B,H,Sq,Skv] (float64),
   with every forbidden entry exactly 0. */
int oracle_attn_fwd_weights_gqa(const void* q, const void* k, const void* v, int dtype,
                                double* out, double* weights, int B, int H, int Hkv, int Sq,
                                int Skv, int d, int dv, double scale, int causal,
                                const int32_t* kv_lens, int nthreads) {
    if (!weights) return OR_E_NULL;
    job_t J;
    memset(&J, 0, sizeof J);
    J.q = q; J.k = k; J.v = v; J.dtype = dtype; J.out = out; J.weights = weights;
    J.B = B; J.H = H; J.Hkv = Hkv; J.Sq = Sq; J.Skv = Skv; J.d = d; J.dv = dv;
    J.scale = scale; J.causal = causal ? 1 : 0; J.kv_lens = kv_lens;
    return run(&J, nthreads);
}

/* As oracle_attn_fwd, and also the weight tensor (oracle_attn_fwd_weights_gqa
   with Hkv = H). */
int oracle_attn_fwd_weights(const void* q, const void* k, const void* v, int dtype, double* out,
                            double* weights, int B, int H, int Sq, int Skv, int d, int dv,
                            double scale, int causal, const int32_t* kv_lens, int nthreads) {
    return oracle_attn_fwd_weights_gqa(q, k, v, dtype, out, weights, B, H, H, Sq, Skv, d, dv,
                                       scale, causal, kv_lens, nthreads);
}

/* Number of threads a call with nthreads <= 0 uses. */
int oracle_default_threads(void) {
    long nc = sysconf(_SC_NPROCESSORS_ONLN);
    return nc > 0 ? (int)nc : 1;
}
