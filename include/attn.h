/*
 * attn.h -- C ABI of the MI355X (gfx950) scaled dot-product attention forward.
 *
 * The operation is the forward pass of multi-head scaled dot-product
 * attention with the mask added to the logits before the softmax:
 *
 *     out = softmax(scale * Q K^T + M) V
 *
 * as stated on "Self-Attention" (blog-15c notes), sections "Scaled
 * Dot-Product Attention" and "Causal Masking", and worked by hand on
 * "Attention from First Principles", section 4.  Heads are independent
 * attention computations laid out as a batch-like axis ("Attention from
 * First Principles", section 5, "Why multiple heads").
 *
 * Mask M (the readings taken where the pages leave the rule open):
 *   - kv_lens[b] = L_b is the valid length of sequence b (right padding,
 *     as in the padding-mask example of "Attention from Scratch",
 *     KubeDojo module 1.4.3, Part 3); keys j >= L_b are
 *     invisible to every query.  Values outside [0, Skv] are clamped to it.
 *     kv_lens == NULL means L_b = Skv for every b.
 *   - The queries of sequence b are its last n_b = min(Sq, L_b) valid
 *     positions: query row i is at absolute position p = L_b - n_b + i
 *     (bottom-right alignment; with Sq == 1 the query is the newest token
 *     and sees the whole cache, as "Scaled dot-product attention with
 *     masking" says of decode).  Rows i >= n_b are padding.
 *   - causal != 0 additionally hides keys j > p (M = -inf there, 0 else).
 *   - A padded query row, or a row with no visible key, is written as 0.
 *
 * Layout: q and out are [B][H][Sq][d], k and v are [B][H][Skv][d] (for the
 * _gqa and _ex entry points [B][H_kv][Skv][d]; with attn_fwd_ex's value
 * width d_v, v is [B][H_kv][Skv][d_v] and out [B][H][Sq][d_v]), all
 * row-major, densely packed, of
 * the one element type `dtype`; out has the inputs' type.  At decode Skv is
 * the cache capacity and L_b <= Skv the filled part.  All five base
 * pointers must be 16-byte aligned.
 *
 * Grouped key/value heads (the _gqa entry points): H_kv K/V heads serve H
 * query heads, H a multiple of H_kv, and query head h reads K/V head
 * h / (H / H_kv) -- consecutive query heads share one K/V head, the grouping
 * of "Attention from First Principles", section "MHA, GQA, MQA -- the KV
 * cache lever", and what repeating K and V with repeat_interleave along the
 * head axis computes ("Scaled dot-product attention with masking", section
 * "Grouped-query attention (GQA)").  H_kv = H is multi-head attention (the
 * entry points without _gqa), H_kv = 1 multi-query attention.
 *
 * Pointers: q, k, v, out, kv_lens and workspace are DEVICE pointers on the
 * current HIP device.  stream is a hipStream_t (NULL = the null stream).
 * Every compute call only enqueues work on `stream` and returns; results are
 * ready when that stream's work has completed.  The caller owns every buffer
 * and keeps it alive until then.  q, k, v and kv_lens are only read; out is
 * only written; the padded tails of k and v (rows >= L_b) are never read, so
 * they may hold anything.
 *
 * Errors: every function returns an attn_status and never throws.  All
 * argument checks run on the host before any HIP call; a failed check
 * enqueues nothing and leaves out untouched.  ATTN_E_LAUNCH reports a HIP
 * launch failure, after which out is undefined.
 */
#ifndef TSDA_ATTN_H
#define TSDA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 7

typedef enum {
    ATTN_OK = 0,
    ATTN_E_NULL = 1,        /* q, k, v or out is NULL (or workspace, where required) */
    ATTN_E_SHAPE = 2,       /* a size <= 0, Sq > Skv, H % H_kv != 0, or sizes overflow */
    ATTN_E_UNSUPPORTED = 3, /* valid request outside the kernels' support matrix */
    ATTN_E_DTYPE = 4,       /* dtype is not an attn_dtype value */
    ATTN_E_ALIGN = 5,       /* a base pointer is not 16-byte aligned (mask: 4 bytes) */
    ATTN_E_WORKSPACE = 6,   /* caller workspace smaller than attn_workspace_bytes() */
    ATTN_E_ARG = 7,         /* scale is not finite */
    ATTN_E_LAUNCH = 8,      /* a HIP call or kernel launch failed */
    ATTN_E_NOMEM = 9,       /* the library could not allocate its workspace */
    ATTN_E_SCRATCH = 10     /* attn_fwd_noalloc: the problem needs more temporary memory
                               than the fixed scratch area holds */
} attn_status;

typedef enum {
    ATTN_F32 = 0,  /* IEEE binary32 in and out */
    ATTN_BF16 = 1  /* bfloat16 in and out; fp32 accumulation and softmax */
} attn_dtype;

/*
 * Support matrix (anything else valid returns ATTN_E_UNSUPPORTED -- there is
 * no silent slow fallback, the hazard "Attention from First Principles"
 * section 8 warns of):
 *   ATTN_F32 : any Sq <= Skv, 1 <= d, d_v <= 128           (VALU kernel)
 *   ATTN_BF16: Sq == 1, d and d_v each in {64, 128}          (split-KV decode)
 *              Sq >= 2, d and d_v each in {64, 128}          (MFMA prefill)
 *              and one head's keys under 4 GiB: Skv * max(d, d_v) * 2 < 2^32
 *              (Skv < 16777216 at 128), since rows are addressed with
 *              32-bit byte offsets from the head's base
 * Every path takes grouped K/V heads, an allowed-mask (attn_fwd_ex), an
 * additive bias (attn_fwd_bias) and any finite scale; with a bias or a scale
 * that is not positive the bf16 paths run their general-logit kernels.
 */

/*
 * attn_fwd -- out = softmax(scale * Q K^T + M) V, arguments as above.
 * scale: the logit multiplier, normally 1/sqrt(d) ("Self-Attention",
 * section "Why divide by sqrt(d_k)?"); any finite value (else ATTN_E_ARG).
 * causal: 0 or nonzero.
 * Temporary memory comes from a library-owned workspace kept per (device,
 * stream) pair and grown on demand; the call that grows it first waits for
 * the earlier work on its stream.  Calls on different streams therefore
 * never share temporary memory and may run concurrently.  attn_release
 * frees these workspaces.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int Sq,
             int Skv, int d, float scale, int causal, const int32_t* kv_lens, int dtype,
             void* stream);

/*
 * attn_workspace_bytes -- device bytes attn_fwd_ws needs for this problem
 * (0 when the chosen kernel needs none).  Returns 0 for invalid arguments.
 * Decode needs fp32 (m, l, acc[d]) partials: one per served query head for
 * each (wave, cache) segment of its fixed grid of waves (at most as many
 * waves as the GPU holds, plus one segment per cache), and two wave indices
 * per cache; prefill needs one per query row and key split only when a short query
 * chunk against a long cache leaves CUs idle (fewer than 256 query tiles of
 * 256 rows) and the key range is split.
 */
size_t attn_workspace_bytes(int B, int H, int Sq, int Skv, int d, int dtype);

/*
 * attn_fwd_ws -- attn_fwd with caller-owned temporary memory.  workspace is
 * a device buffer of at least attn_workspace_bytes(...) bytes, 256-byte
 * aligned, not used by any other call until this one's stream work ends.
 * Its contents need no initialisation and are garbage afterwards.  workspace
 * may be NULL only when attn_workspace_bytes(...) is 0.
 */
int attn_fwd_ws(const void* q, const void* k, const void* v, void* out, int B, int H, int Sq,
                int Skv, int d, float scale, int causal, const int32_t* kv_lens, int dtype,
                void* stream, void* workspace, size_t workspace_bytes);

/*
 * attn_fwd_gqa -- attn_fwd with H_kv key/value heads (layout and head
 * grouping above; k and v are [B][H_kv][Skv][d]).  H_kv must divide H, else
 * ATTN_E_SHAPE.  The decode kernel reads each K/V row once for all the query
 * heads it serves (up to 32 per pass), so decode bytes fall by up to H / H_kv.
 * Other arguments, ownership and errors as attn_fwd.
 */
int attn_fwd_gqa(const void* q, const void* k, const void* v, void* out, int B, int H, int H_kv,
                 int Sq, int Skv, int d, float scale, int causal, const int32_t* kv_lens,
                 int dtype, void* stream);

/* attn_workspace_bytes for attn_fwd_gqa_ws (0 also for invalid arguments). */
size_t attn_workspace_bytes_gqa(int B, int H, int H_kv, int Sq, int Skv, int d, int dtype);

/* attn_fwd_gqa with caller-owned temporary memory, as attn_fwd_ws. */
int attn_fwd_gqa_ws(const void* q, const void* k, const void* v, void* out, int B, int H,
                    int H_kv, int Sq, int Skv, int d, float scale, int causal,
                    const int32_t* kv_lens, int dtype, void* stream, void* workspace,
                    size_t workspace_bytes);

/* The host-side checks of attn_fwd_gqa alone (as attn_validate). */
int attn_validate_gqa(const void* q, const void* k, const void* v, void* out, int B, int H,
                      int H_kv, int Sq, int Skv, int d, float scale, int causal, int dtype);

/*
 * attn_fwd_ex -- H_kv key/value heads (as attn_fwd_gqa), a value width d_v
 * that may differ from d (softmax(QK^T) V only needs V's rows to match K's,
 * the d_k = 4, d_v = 2 example of "Attention from Scratch", KubeDojo module
 * 1.4.3, Part 2; see the support matrix), and an explicit allowed-mask ANDed
 * into M:
 * query row i of (b, h) sees key j only if the causal and length rules above
 * allow it AND mask byte (b, h, i, j) is nonzero (the boolean allowed-mask,
 * True = may attend, of "Attention from Scratch", KubeDojo module 1.4.3,
 * Part 3, which combines its causal and padding masks by logical AND; a
 * torch.bool tensor's bytes are such a mask).  It covers key-padding masks
 * of padded cross-attention sources, left padding, per-row query lengths
 * (hide every key of a padded row), and arbitrary patterns.  A row that sees
 * no key, or a padded row (i >= n_b), is written as 0.
 *
 *   mask      DEVICE bytes; byte (b, h, i, j) is
 *             mask[b*mask_sb + h*mask_sh + i*mask_si + j], i indexing the
 *             Sq query rows as given (before the bottom-right offset).  A
 *             stride of 0 broadcasts that axis ([B,1,1,Skv] key padding:
 *             mask_sh = mask_si = 0).  NULL: no mask (attn_fwd_gqa_ws).
 *   mask_s*   strides in bytes, >= 0 (else ATTN_E_SHAPE).
 *   Rows are read as 4-byte words: mask must be 4-byte aligned and the
 *   strides multiples of 4 (else ATTN_E_ALIGN), and each row must be
 *   readable up to Skv rounded up to a multiple of 4 (the bytes past Skv are
 *   ignored).  A dense [B,H,Sq,Skv] mask with Skv a multiple of 4 meets all
 *   of this; otherwise pad its rows.  32 * mask_si + Skv must stay below
 *   2^32 (else ATTN_E_UNSUPPORTED).  The mask is only read.
 *   workspace NULL: the library-owned workspace, as attn_fwd_gqa; else a
 *             caller buffer as for attn_fwd_gqa_ws, of attn_workspace_bytes_ex
 *             bytes (a masked bf16 prefill needs a little more: one byte per
 *             query tile and key tile, which it uses to skip key tiles the
 *             mask hides from a whole query tile when the mask is shared by
 *             all heads).
 * The masked kernels are separate instantiations: calls with mask == NULL
 * run exactly the unmasked code.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* out, int B, int H, int H_kv,
                int Sq, int Skv, int d, int d_v, float scale, int causal, const int32_t* kv_lens,
                const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int64_t mask_si, int dtype,
                void* stream, void* workspace, size_t workspace_bytes);

/*
 * attn_fwd_bias -- attn_fwd_ex plus an additive bias: the logit of query row
 * i and key j of (b, h) is scale * q_i . k_j + bias(b, h, i, j), before the
 * softmax (the float mask that "Attention from Scratch", KubeDojo module
 * 1.4.3, Part 7 calls an additive bias, where a boolean mask only allows or
 * forbids).  A bias of -inf hides the key exactly as a zero mask byte does;
 * the bias is added to keys the rules and the mask leave visible.  Its
 * entries must be finite or -inf (+inf or NaN give undefined results).
 *
 *   bias      DEVICE array of `dtype` elements (bf16 bias for bf16 inputs,
 *             fp32 for fp32); element (b, h, i, j) is
 *             bias[b*bias_sb + h*bias_sh + i*bias_si + j], i the query row as
 *             given.  A stride of 0 broadcasts that axis.  NULL: no bias
 *             (then this is attn_fwd_ex).
 *   bias_s*   strides in ELEMENTS, >= 0 (else ATTN_E_SHAPE) and multiples of
 *             4, with the base 16-byte aligned (else ATTN_E_ALIGN); rows are
 *             read in groups of 4 elements, so each row must be readable up to
 *             Skv rounded up to a multiple of 4.  (32 * bias_si + Skv) times
 *             the element size must stay below 2^32 (else
 *             ATTN_E_UNSUPPORTED).  The bias is only read.
 * The workspace is that of attn_fwd_ex (attn_workspace_bytes_ex); the other
 * arguments, ownership and errors are as there.  Mask checks come before
 * bias checks.
 */
int attn_fwd_bias(const void* q, const void* k, const void* v, void* out, int B, int H, int H_kv,
                  int Sq, int Skv, int d, int d_v, float scale, int causal,
                  const int32_t* kv_lens, const uint8_t* mask, int64_t mask_sb, int64_t mask_sh,
                  int64_t mask_si, const void* bias, int64_t bias_sb, int64_t bias_sh,
                  int64_t bias_si, int dtype, void* stream, void* workspace,
                  size_t workspace_bytes);

/* The host-side checks of attn_fwd_bias alone (as attn_validate). */
int attn_validate_bias(const void* q, const void* k, const void* v, void* out, int B, int H,
                       int H_kv, int Sq, int Skv, int d, int d_v, float scale, int causal,
                       const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int64_t mask_si,
                       const void* bias, int64_t bias_sb, int64_t bias_sh, int64_t bias_si,
                       int dtype);

/* Device bytes attn_fwd_ex needs as caller workspace (masked != 0 when a
   mask is passed: a masked prefill adds key-tile marks, a masked decode a
   visible-tile count and list per (b, K/V head) cache); 0 also for invalid
   arguments. */
size_t attn_workspace_bytes_ex(int B, int H, int H_kv, int Sq, int Skv, int d, int d_v, int dtype,
                               int masked);

/* The host-side checks of attn_fwd_ex alone (as attn_validate; d_v <= 0 is
   ATTN_E_SHAPE, a d_v the dtype's kernels do not take ATTN_E_UNSUPPORTED). */
int attn_validate_ex(const void* q, const void* k, const void* v, void* out, int B, int H,
                     int H_kv, int Sq, int Skv, int d, int d_v, float scale, int causal,
                     const uint8_t* mask, int64_t mask_sb, int64_t mask_sh, int64_t mask_si,
                     int dtype);

/*
 * attn_fwd_noalloc -- attn_fwd_ex for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, whose role is
 * taken by a fixed scratch array of attn_noalloc_scratch_bytes() bytes that
 * the library's code object holds on every device it runs on, from load until
 * the process ends.  The call allocates and frees nothing.  A problem whose
 * temporary memory (attn_workspace_bytes_ex) exceeds the array returns
 * ATTN_E_SCRATCH before enqueueing anything; other errors as attn_fwd_ex.
 * Every call on one device shares that device's array, which keeps the last
 * call's contents: two calls whose work may overlap on one device (calls on
 * different streams, or from different host threads) race on it and give
 * undefined results.  Order such calls on one stream.
 */
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H,
                     int H_kv, int Sq, int Skv, int d, int d_v, float scale, int causal,
                     const int32_t* kv_lens, const uint8_t* mask, int64_t mask_sb,
                     int64_t mask_sh, int64_t mask_si, int dtype, void* stream);

/* Size in bytes of the scratch array attn_fwd_noalloc uses on each device. */
size_t attn_noalloc_scratch_bytes(void);

/*
 * attn_validate -- the host-side checks of attn_fwd alone: returns what
 * attn_fwd would return before enqueueing anything.  Makes no HIP call.
 */
int attn_validate(const void* q, const void* k, const void* v, void* out, int B, int H, int Sq,
                  int Skv, int d, float scale, int causal, int dtype);

/*
 * attn_kernel_for -- name of the kernel family attn_fwd would launch for
 * these sizes ("prefill_bf16_mfma", "decode_bf16_stream", "generic_f32"),
 * or NULL when the request is invalid or unsupported.  Makes no HIP call.
 * The string is static.
 */
const char* attn_kernel_for(int Sq, int Skv, int d, int dtype);

/* Human-readable text for an attn_status value (static string). */
const char* attn_status_string(int status);

/* ATTN_ABI_VERSION of the loaded library. */
int attn_abi_version(void);

/*
 * attn_last_hip_error -- the hipError_t value behind the last ATTN_E_LAUNCH
 * that a call on this thread returned (0, hipSuccess, if none has), kept per
 * thread until the next such failure.  attn_last_hip_error_name -- the HIP
 * runtime's name for it (static string).  Neither makes a GPU call.
 */
int attn_last_hip_error(void);
const char* attn_last_hip_error_name(void);

/*
 * attn_prefill_plan -- how a bf16 prefill of these sizes is launched, for
 * tests and tuning: *key_splits key-range splits per query tile (1 = none),
 * *rows_per_block query rows per block (256, or 128 / 64 on small grids) and
 * *key_groups wave sets per block that split its keys (1 or 2).  masked: an
 * allowed-mask is given; general: a bias, or a scale that is not positive.
 * Output pointers may be NULL.  Returns ATTN_E_SHAPE for invalid sizes and
 * ATTN_E_UNSUPPORTED when the sizes do not take the prefill kernel (Sq == 1,
 * d or d_v outside {64, 128}).  Makes no HIP call.
 */
int attn_prefill_plan(int B, int H, int H_kv, int Sq, int Skv, int d, int d_v, int masked,
                      int general, int* key_splits, int* rows_per_block, int* key_groups);

/*
 * attn_release -- frees the library-owned workspace of every device.  The
 * caller must ensure no enqueued attn_fwd call is still running.
 */
void attn_release(void);

/*
 * Kernel timing, for benchmarks.  While enabled, every kernel the library
 * launches is bracketed by HIP events recorded on the launch stream.
 * attn_profile_read synchronizes on those events and returns, for kernel
 * family `kernel` (the index into the list attn_profile_name enumerates),
 * the number of launches and their summed duration in milliseconds since the
 * last reset.  Enabling or resetting discards earlier records.
 */
int attn_profile_enable(int on);
int attn_profile_reset(void);
int attn_profile_read(int kernel, long* launches, double* total_ms);
const char* attn_profile_name(int kernel); /* NULL past the last kernel */
/* The individual durations (milliseconds, launch order) of the first `cap`
   recorded launches of family `kernel` go to ms[0 .. cap-1]; *launches gets
   the number recorded since the last reset.  Synchronizes on their events. */
int attn_profile_samples(int kernel, double* ms, long cap, long* launches);

#ifdef __cplusplus
}
#endif

#endif /* TSDA_ATTN_H */
