/*
 * orthros.h -- C ABI of the MI355X (gfx950) Orthros attention library.
 *
 * One layer of Orthros phase-aware heterogeneous attention, as described in
 * "Orthros:阶段感知异构注意力精读笔记" (close-reading notes of arXiv
 * 2610.13735; cited below as [N]):
 *
 *   - base stream: causal sliding-window attention (window w, 128 in the
 *     pages) over every base token, [N] §2.3 Eq. (4); it writes every
 *     position's K/V into the layer's cache, [N] §2.1 and §2.6;
 *   - output-only stream: full-history causal cross-attention over that
 *     cache, only at positions that predict a token, masked by the copy's
 *     original position, [N] §2.3 Eq. (5) and §2.4;
 *   - both streams' queries come from one shared projection followed by a
 *     per-stream elementwise scale-offset q * alpha + beta, [N] §2.2.
 *
 * Either side of the attention ([N] §2.1-§2.2): the base stream's K/V come
 * from the base input X at every position and both streams' queries from one
 * shared W_Q; orthros_project computes them and writes K/V into the cache.
 *
 * Modes ([N] §2.5, mode table): prefill has T_in = T-1 base-only tokens and
 * T_out = 1 copy (the last prompt position); decode processes one new base
 * token and one copy per step, the copy reading the whole history.
 *
 * Conventions shared by every call
 *   - Positions are 0-based: the window of base row t is
 *     [max(0, t-w+1), t]; a copy at original position P reads keys [0, P].
 *   - Query head h reads KV head h / (n_q_heads / n_kv_heads).
 *   - Tensors are dense, row-major, in the layouts written next to each
 *     argument; every tensor of one call is stored in desc->dtype
 *     (alpha/beta included).  Arithmetic is fp32 (bf16 storage: bf16 MFMA
 *     operands with fp32 accumulation).  Outputs are written in dtype,
 *     rounded to nearest even.
 *   - Pointers named as device pointers must be device memory of the
 *     current HIP device and 16-byte aligned.  Host pointers are read
 *     before the call returns.
 *   - Ownership: the caller owns every buffer, including the KV cache, the
 *     lengths and the workspace.  The library allocates nothing, frees
 *     nothing and never synchronises: work is queued on `stream` (a
 *     hipStream_t; NULL is the null stream) and the call returns.  (The one
 *     exception to "the caller owns": orthros_decode_step_noalloc keeps its
 *     partials in a scratch array the library holds on each device.)
 *   - Outputs must not alias inputs; k_cache/v_cache must not alias k/v.
 *   - Errors: arguments are validated on the host before anything is
 *     queued; a negative status means nothing was launched.  ORTHROS_E_HIP
 *     reports a failed launch; orthros_last_error() then holds the text.
 *   - Thread safety: calls may be made from several host threads; the only
 *     global state is the per-thread error text and, for
 *     orthros_decode_step_noalloc, one scratch array per device (below).
 */
#ifndef ORTHROS_H
#define ORTHROS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORTHROS_ABI_VERSION 3

typedef enum {
    ORTHROS_OK = 0,
    ORTHROS_E_NULL = -1,      /* a required pointer is NULL                    */
    ORTHROS_E_SHAPE = -2,     /* unsupported or inconsistent sizes             */
    ORTHROS_E_DTYPE = -3,     /* dtype not one of orthros_dtype                */
    ORTHROS_E_POS = -4,       /* a copy position outside [0, T)                */
    ORTHROS_E_CAPACITY = -5,  /* cache capacity too small for the call         */
    ORTHROS_E_WORKSPACE = -6, /* workspace missing or smaller than required    */
    ORTHROS_E_HIP = -7,       /* a HIP launch failed                           */
    ORTHROS_E_ALIGN = -8      /* a device pointer is not 16-byte aligned       */
} orthros_status;

typedef enum { ORTHROS_F32 = 0, ORTHROS_BF16 = 1 } orthros_dtype;

/* Problem description shared by every call.
 *   batch          B >= 1 sequences
 *   n_q_heads      Hq >= 1, a multiple of n_kv_heads
 *   n_kv_heads     Hkv >= 1
 *   head_dim       d: 64 or 128
 *   window         w >= 1 keys in the base stream's window, itself included
 *                  ([N] §2.3: W_t = {max(1, t-w+1), ..., t}; 128 in the pages)
 *   softmax_scale  score scale; 0 means 1/sqrt(d)
 *   dtype          orthros_dtype of every tensor of the call               */
typedef struct {
    int32_t batch, n_q_heads, n_kv_heads, head_dim, window;
    float softmax_scale;
    int32_t dtype;
} orthros_desc;

/* ------------------------------------------------------------- prefill */

/* Workspace bytes orthros_prefill and orthros_global_xattn need for a
 * prompt of T tokens (split-K partials of the copy's query).  0 on an
 * invalid desc or T. */
size_t orthros_prefill_workspace_size(const orthros_desc* desc, int64_t T);

/*
 * One layer's prefill ([N] §2.5, prefill row: T_in = T-1, T_out = 1):
 * orthros_swa_prefill followed by orthros_global_xattn on the same stream.
 *
 *   T          prompt length per sequence, 1 <= T <= cap
 *   q          device [B][T][Hq][d]   base-stream projected queries x W_Q
 *   q_out      device [B][Hq][d]      each sequence's output copy, x' W_Q
 *              (the copy Algorithm 2 appends at the tensor tail)
 *   out_pos    host   [B]             original position of each copy,
 *              0 <= out_pos[b] < T (T-1 for a plain prefill)
 *   k, v       device [B][T][Hkv][d]  this layer's base K/V
 *   alpha, beta          device [Hq][d]  base-stream scale-offset
 *   alpha_out, beta_out  device [Hq][d]  output-stream scale-offset
 *   k_cache, v_cache     device [B][Hkv][cap][d]; slots [0, T) are written,
 *              every other slot is left untouched
 *   o          device [B][T][Hq][d]   Eq. (4) for every base row
 *   o_out      device [B][Hq][d]      Eq. (5) for each copy
 *   workspace  device, >= orthros_prefill_workspace_size(desc, T) bytes
 */
orthros_status orthros_prefill(const orthros_desc* desc, int64_t T,
                               const void* q, const void* q_out, const int64_t* out_pos,
                               const void* k, const void* v,
                               const void* alpha, const void* beta,
                               const void* alpha_out, const void* beta_out,
                               void* k_cache, void* v_cache, int64_t cap,
                               void* o, void* o_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Base stream of a prefill ([N] §2.3 Eq. (4); cache write [N] §2.1, §2.6):
 * banded sliding-window attention for every base row t of every sequence
 * and head, and the copy of k, v into cache slots [0, T).  Arguments as in
 * orthros_prefill.  Needs no workspace.
 */
orthros_status orthros_swa_prefill(const orthros_desc* desc, int64_t T,
                                   const void* q, const void* k, const void* v,
                                   const void* alpha, const void* beta,
                                   void* k_cache, void* v_cache, int64_t cap,
                                   void* o, void* stream);

/*
 * Output stream of a prefill ([N] §2.3 Eq. (5), §2.4): each sequence's copy
 * query, scale-offset by alpha_out/beta_out, attends over cache slots
 * [0, out_pos[b]] (its original position; 0 <= out_pos[b] < T).  Split-K
 * over the cache, then a log-sum-exp merge in a fixed order (results are
 * run-to-run identical).  The cache must already hold slots [0, T) (stream
 * order after orthros_swa_prefill suffices).  Arguments as in
 * orthros_prefill.
 */
orthros_status orthros_global_xattn(const orthros_desc* desc, int64_t T,
                                    const void* q_out, const int64_t* out_pos,
                                    const void* alpha_out, const void* beta_out,
                                    const void* k_cache, const void* v_cache, int64_t cap,
                                    void* o_out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* -------------------------------------------------- many output copies */

/*
 * Output copies at many positions per sequence: the pre-training and
 * fine-tuning modes of [N] §2.5 (mode table: PT copies every position,
 * T_out = T; SFT copies the answer positions).  Copy i of sequence b sits
 * at original position out_pos[b][i]; its query q_out[b][i], scale-offset
 * by alpha_out/beta_out, attends over cache slots [0, out_pos[b][i]]
 * ([N] §2.3 Eq. (5), §2.4: the mask follows the original position, never
 * the copy's slot).  The copies neither write the cache nor see one
 * another.  The cache must already hold slots [0, T) (stream order after
 * orthros_swa_prefill or orthros_prefill suffices).
 *
 *   T          prompt length per sequence, 1 <= T <= cap
 *   T_out      copies per sequence, >= 1
 *   q_out      device [B][T_out][Hq][d]   the copies' projected queries x' W_Q
 *   out_pos    device int32 [B][T_out]    original positions, in any order
 *              (ascending is fastest); 4-byte aligned.  A copy whose
 *              position lies outside [0, T) reads nothing and gets NaN in
 *              o_out (the positions live on the device, so they are checked
 *              there)
 *   alpha_out, beta_out  device [Hq][d]
 *   k_cache, v_cache     device [B][Hkv][cap][d], read only
 *   o_out      device [B][T_out][Hq][d]
 * Needs no workspace.  Results are run-to-run identical.
 */
orthros_status orthros_copies(const orthros_desc* desc, int64_t T, int64_t T_out,
                              const void* q_out, const int32_t* out_pos,
                              const void* alpha_out, const void* beta_out,
                              const void* k_cache, const void* v_cache, int64_t cap,
                              void* o_out, void* stream);

/* ---------------------------------------------------------- projections */

/*
 * The projections on either side of one layer's attention step ([N] §2.1:
 * the base stream's K/V come from the layer's base input X for every
 * position and are that layer's cache rows; §2.2: both streams' queries come
 * from the one shared W_Q, then each stream's elementwise scale-offset).
 * One launch, one pass over the stacked rows [X; X']:
 *   q[b][t]       = (x[b][t] W_Q^T) * alpha + beta
 *   q_out[b][i]   = (x_out[b][i] W_Q^T) * alpha_out + beta_out
 *   k_cache[b][g][t] = (x[b][t] W_K^T) head g,  v_cache likewise with W_V
 * bf16 storage only (ORTHROS_E_DTYPE otherwise); fp32 accumulation, outputs
 * rounded to nearest even.  desc->window and softmax_scale are not used.
 *
 *   T          base rows per sequence, 1 <= T <= cap
 *   T_out      copy rows per sequence, >= 0 (prefill: 1; PT/SFT: the copies)
 *   d_model    the layer's input width, a multiple of 32 in [32, 65536]
 *   x          device [B][T][d_model]       base input X
 *   x_out      device [B][T_out][d_model]   copy inputs X' (may be NULL when T_out = 0)
 *   w_q        device [Hq*d][d_model]       W_Q stored [out][in] (y = x W^T)
 *   w_k, w_v   device [Hkv*d][d_model]
 *   alpha, beta          device [Hq][d] or both NULL: no scale-offset on q
 *   alpha_out, beta_out  device [Hq][d] or both NULL: none on q_out
 *              (pass NULL to feed orthros_prefill / orthros_copies, which
 *              apply the scale-offset themselves)
 *   q          device [B][T][Hq][d]
 *   q_out      device [B][T_out][Hq][d] (may be NULL when T_out = 0)
 *   k_cache, v_cache     device [B][Hkv][cap][d]; slots [0, T) are written,
 *              every other slot is left untouched
 * Needs n_q_heads*d and n_kv_heads*d to be multiples of 128.
 */
orthros_status orthros_project(const orthros_desc* desc, int64_t T, int64_t T_out, int64_t d_model,
                               const void* x, const void* x_out,
                               const void* w_q, const void* w_k, const void* w_v,
                               const void* alpha, const void* beta,
                               const void* alpha_out, const void* beta_out,
                               void* q, void* q_out, void* k_cache, void* v_cache, int64_t cap,
                               void* stream);

/* -------------------------------------------------------------- decode */

/* Workspace bytes orthros_decode_step needs when every cache length is at
 * most max_len.  0 on an invalid desc or max_len.  The workspace begins
 * with the step's arrival counters: it must be zero-filled once before its
 * first step (e.g. hipMemset after allocating it); every step leaves the
 * counters at zero again, so one zero-fill serves any number of steps,
 * replayed graphs included.  Do not share it with other calls. */
size_t orthros_decode_workspace_size(const orthros_desc* desc, int64_t max_len);

/*
 * One decode step of one layer ([N] §2.5, decode row; §2.4 walk-through):
 * for each sequence b with L = cache_len[b] (read on the device):
 *   - the new base token's k_new[b], v_new[b] are written to cache slot L;
 *   - its query q[b] attends over slots [max(0, L-w+1), L] -> o[b];
 *   - its output copy q_out[b] attends over slots [0, L] (the whole
 *     history, the new token included) -> o_out[b];
 *   - cache_len[b] becomes L + 1.
 *
 *   q, q_out          device [B][Hq][d]   projected queries of the token and its copy
 *   k_new, v_new      device [B][Hkv][d]
 *   alpha..beta_out   device [Hq][d]
 *   k_cache, v_cache  device [B][Hkv][cap][d]
 *   cache_len         device int32 [B], lengths before the step; updated in stream order
 *   max_len_hint      host: an upper bound of every cache_len[b]; sizes the
 *                     grid; needs max_len_hint + 1 <= cap
 *   o, o_out          device [B][Hq][d]
 *   workspace         device, >= orthros_decode_workspace_size(desc, max_len_hint) bytes,
 *                     zero-filled before its first step (see above)
 *
 * A sequence whose cache_len[b] is negative or above max_len_hint is not
 * touched (no cache write, no length update) and gets NaN in o[b] and
 * o_out[b].  Successive steps may be queued back to back with no host
 * synchronisation; a step's workspace must not be shared with a step that
 * can run concurrently.
 */
orthros_status orthros_decode_step(const orthros_desc* desc,
                                   const void* q, const void* q_out,
                                   const void* k_new, const void* v_new,
                                   const void* alpha, const void* beta,
                                   const void* alpha_out, const void* beta_out,
                                   void* k_cache, void* v_cache, int64_t cap,
                                   int32_t* cache_len, int64_t max_len_hint,
                                   void* o, void* o_out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * orthros_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments (minus workspace
 * and workspace_bytes), same kernels, same results bit for bit.
 *
 * The split-K partials live instead in a scratch array of 64 MiB that the
 * library holds on every GPU it runs on (a device global, loaded with the
 * library's code and kept until the process ends).  Nothing is allocated or
 * freed per call.  The first call on a device looks the array's address up
 * (hipGetSymbolAddress) with that device current; a caller about to
 * capture can make one call before the capture so that no lookup happens
 * inside it.
 *
 * Limits and errors: a step whose workspace (orthros_decode_workspace_size
 * of desc and max_len_hint) exceeds 64 MiB is rejected with
 * ORTHROS_E_WORKSPACE before anything is queued (the batch-16 step with
 * 128K-key histories needs about 3.3 MB; steps on the lane-parallel
 * kernel -- fp32, and short bf16 steps of groups that are not multiples of
 * 4 -- need far more: about 60 MB for fp32 at batch 16 with 120K-key
 * histories).  Every call on one GPU shares that
 * GPU's array, which keeps the last call's contents; each step writes what
 * it reads, so no clearing is needed, but calls that can overlap on one GPU
 * (other streams, other host threads) race on it: serialise them.
 */
orthros_status orthros_decode_step_noalloc(const orthros_desc* desc,
                                           const void* q, const void* q_out,
                                           const void* k_new, const void* v_new,
                                           const void* alpha, const void* beta,
                                           const void* alpha_out, const void* beta_out,
                                           void* k_cache, void* v_cache, int64_t cap,
                                           int32_t* cache_len, int64_t max_len_hint,
                                           void* o, void* o_out, void* stream);

/* ------------------------------------------------------------ utilities */

/* Static text naming a status code. */
const char* orthros_status_str(int status);
/* Text of the last error on the calling thread ("" when none). */
const char* orthros_last_error(void);
/* ORTHROS_ABI_VERSION of the built library. */
int orthros_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ORTHROS_H */
