// api.hip -- the C ABI of include/orthros.h: argument validation, workspace
// sizing, split-size choice and kernel launches.  Host code only.
//
// Every argument is checked before the first launch, so a negative status
// always means that nothing was queued.  The library allocates nothing and
// never synchronises; all work goes to the caller's stream.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "kernels.h"
#include "orthros.h"

namespace {

thread_local std::string g_err;

orthros_status fail(orthros_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
orthros_status fail(orthros_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

constexpr int64_t kMaxElems = int64_t(1) << 50;   // keeps every byte offset far from overflow

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

orthros_status check_desc(const orthros_desc* d)
{
    if (!d) return fail(ORTHROS_E_NULL, "desc is NULL");
    if (d->dtype != ORTHROS_F32 && d->dtype != ORTHROS_BF16)
        return fail(ORTHROS_E_DTYPE, "dtype %d is neither ORTHROS_F32 nor ORTHROS_BF16", d->dtype);
    if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
        return fail(ORTHROS_E_SHAPE, "batch, n_q_heads and n_kv_heads must be >= 1");
    if (d->n_q_heads % d->n_kv_heads)
        return fail(ORTHROS_E_SHAPE, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", d->n_q_heads,
                    d->n_kv_heads);
    if (d->n_q_heads > 65535 || d->batch > 65535)
        return fail(ORTHROS_E_SHAPE, "batch and n_q_heads must be <= 65535");
    if (d->head_dim != 64 && d->head_dim != 128)
        return fail(ORTHROS_E_SHAPE, "head_dim %d unsupported (64 or 128)", d->head_dim);
    if (d->window < 1) return fail(ORTHROS_E_SHAPE, "window must be >= 1");
    if (!(d->softmax_scale >= 0.f) || std::isinf(d->softmax_scale))
        return fail(ORTHROS_E_SHAPE, "softmax_scale must be finite and >= 0");
    return ORTHROS_OK;
}

float qscale_of(const orthros_desc* d)
{
    const float s = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / std::sqrt((float)d->head_dim);
    return s * 1.4426950408889634f;   // scores go to exp2: fold log2(e) into the query
}

// Smallest power-of-two key chunk >= 256 that keeps about `target` workgroups.
int pick_chunk(int64_t keys, int64_t streams, int64_t target)
{
    const int64_t want = (keys * streams + target - 1) / target;
    int64_t c = 256;
    while (c < want && c < (int64_t(1) << 24)) c <<= 1;
    return (int)c;
}

int64_t streams_of(const orthros_desc* d)
{
    const int G = d->n_q_heads / d->n_kv_heads;
    return (int64_t)d->batch * d->n_kv_heads * (G / orthros::xattn_heads_per_wg(G));
}

constexpr int64_t kPrefillTargetWgs = 2048;
constexpr int64_t kDecodeTargetWgs = 16384;
constexpr size_t kLenBytesAlign = 256;

size_t len_bytes(const orthros_desc* d)
{
    return ((size_t)d->batch * 4 + kLenBytesAlign - 1) / kLenBytesAlign * kLenBytesAlign;
}

struct Split { int chunk, n_split, rec; bool lds, fused = false; size_t bytes; };

// Bytes of the LDS-streamed kernel's per-stream record ranges ([B][streams][3]
// int32, 256-byte aligned), which sit between the lengths and the records;
// 0 for the other kernels.
size_t rng_bytes(const orthros_desc* d, bool lds)
{
    if (!lds) return 0;
    return ((size_t)streams_of(d) * 3 * 4 + kLenBytesAlign - 1) / kLenBytesAlign * kLenBytesAlign;
}

// The LDS-streamed kernel's records: ids over every launch, kinds x 4 heads
// of rec floats each.
size_t lds_record_bytes(const orthros_desc* d, int kinds, int rec)
{
    const int S = (int)(streams_of(d) / d->batch);
    return (size_t)orthros::xattn_lds_records(d->batch, S) * kinds * 4 * rec * 4;
}

orthros::Dt dt_of(const orthros_desc* d) { return d->dtype == ORTHROS_F32 ? orthros::Dt::F32 : orthros::Dt::BF16; }

bool fused_prefill(const orthros_desc* d)
{
    return orthros::ring_applies(dt_of(d), d->n_q_heads, d->n_kv_heads, d->window);
}

// Key splits of the output copy in prefill.  The LDS-streamed kernel cuts
// the keys into equal runs per workgroup (records by id, their ranges per
// stream); the lane-parallel kernel uses power-of-two chunks; the fused path
// (streaming SWA kernel with the copy's query folded in) leaves one partial
// per segment of its launch.  The workspace covers whichever the call takes.
Split prefill_split(const orthros_desc* d, int64_t T)
{
    Split s;
    const bool lds = orthros::xattn_lds_applies(dt_of(d), d->n_q_heads, d->n_kv_heads) &&
                     ((d->n_q_heads / d->n_kv_heads) % 4 == 0 ||
                      T * streams_of(d) >= orthros::kXattnLdsPrefillMinKeys);
    s.lds = lds;
    if (lds) {
        s.chunk = 0;
        s.n_split = 0;
        s.rec = d->head_dim + orthros::kXattnLdsRecPad;
        s.bytes = len_bytes(d) + rng_bytes(d, true) + lds_record_bytes(d, 1, s.rec);
        return s;
    }
    s.chunk = pick_chunk(T, streams_of(d), kPrefillTargetWgs);
    s.n_split = (int)((T + s.chunk - 1) / s.chunk);
    s.rec = d->head_dim + 2;
    s.bytes = len_bytes(d) + (size_t)d->batch * d->n_q_heads * s.n_split * s.rec * 4;
    return s;
}

Split fused_split(const orthros_desc* d, int64_t T)
{
    const orthros::RingGeom r = orthros::ring_geometry(d->batch, d->n_q_heads, d->n_kv_heads, T);
    Split s;
    s.chunk = 32 * r.tps;
    s.n_split = r.n_seg;
    s.rec = d->head_dim + 2;
    s.lds = false;
    s.bytes = len_bytes(d) + (size_t)d->batch * d->n_q_heads * s.n_split * s.rec * 4;
    return s;
}

size_t prefill_ws_bytes(const orthros_desc* d, int64_t T)
{
    const size_t a = prefill_split(d, T).bytes;
    if (!fused_prefill(d)) return a;
    const size_t b = fused_split(d, T).bytes;
    return a > b ? a : b;
}

// Bytes of the decode step's arrival counters at the start of its
// workspace: one per (sequence, KV head, head block of the chunked kernel)
// and one per sequence, 256-byte aligned.
size_t cnt_bytes(const orthros_desc* d)
{
    const size_t n = (size_t)d->batch * (size_t)(streams_of(d) / d->batch + 1);
    return (n * 4 + kLenBytesAlign - 1) / kLenBytesAlign * kLenBytesAlign;
}

Split decode_split(const orthros_desc* d, int64_t max_len)
{
    Split s;
    const int64_t keys = max_len + 1;
    // short bf16 steps: one launch over 128-key chunks (latency-bound, so
    // each workgroup reads its whole chunk in one round trip)
    s.fused = d->dtype == ORTHROS_BF16 &&
              keys <= (int64_t)orthros::kDecodeShortChunk * orthros::kDecodeShortMaxSplits;
    // longer bf16 steps: the LDS-streamed kernel (equal runs of the step's
    // keys per workgroup) for groups that are multiples of 4, and for other
    // groups once the step is long enough for its runs to pay
    s.lds = !s.fused && orthros::xattn_lds_applies(dt_of(d), d->n_q_heads, d->n_kv_heads) &&
            ((d->n_q_heads / d->n_kv_heads) % 4 == 0 || keys * streams_of(d) >= orthros::kXattnLdsDecodeMinKeys ||
             keys >= orthros::kXattnLdsDecodeLongKeys);
    if (s.lds) {
        s.chunk = 0;
        s.n_split = 0;
        s.rec = d->head_dim + orthros::kXattnLdsRecPad;
        s.bytes = cnt_bytes(d) + len_bytes(d) + rng_bytes(d, true) + lds_record_bytes(d, 2, s.rec);
        return s;
    }
    // the rest (fp32, and short bf16 steps of other groups) on the
    // lane-parallel kernel
    s.chunk = s.fused ? orthros::kDecodeShortChunk : pick_chunk(keys, streams_of(d), kDecodeTargetWgs);
    s.n_split = (int)((keys + s.chunk - 1) / s.chunk);
    s.rec = d->head_dim + (s.fused ? 4 : 2);
    s.bytes = cnt_bytes(d) + len_bytes(d) + (size_t)d->batch * d->n_q_heads * 2 * s.n_split * s.rec * 4;
    return s;
}

orthros_status check_T(const orthros_desc* d, int64_t T, int64_t cap)
{
    if (T < 1 || T > INT32_MAX) return fail(ORTHROS_E_SHAPE, "T = %lld outside [1, 2^31)", (long long)T);
    if (cap < T) return fail(ORTHROS_E_CAPACITY, "cap %lld < T %lld", (long long)cap, (long long)T);
    const int64_t rowq = (int64_t)d->n_q_heads * d->head_dim;
    if ((int64_t)d->batch * cap > kMaxElems / rowq || (int64_t)d->batch * T > kMaxElems / rowq)
        return fail(ORTHROS_E_SHAPE, "tensor sizes overflow the library's 2^50-element bound");
    // bf16 SWA grid: B * Hkv * (G / HS) * ceil(T / TQ) workgroups of 256 threads, TQ >= 32
    if ((int64_t)d->batch * d->n_q_heads * ((T + 31) / 32) >= (int64_t(1) << 24))
        return fail(ORTHROS_E_SHAPE, "batch * n_q_heads * T / 32 exceeds the launch grid limit");
    return ORTHROS_OK;
}

orthros_status check_ptrs(std::initializer_list<const void*> ps)
{
    for (const void* p : ps) {
        if (!p) return fail(ORTHROS_E_NULL, "a required pointer is NULL");
        if (!aligned16(p)) return fail(ORTHROS_E_ALIGN, "a device pointer is not 16-byte aligned");
    }
    return ORTHROS_OK;
}

orthros_status hip_status(hipError_t e, const char* what)
{
    if (e == hipSuccess) return ORTHROS_OK;
    return fail(ORTHROS_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

orthros_status validate_swa(const orthros_desc* d, int64_t T, const void* q, const void* k, const void* v,
                            const void* alpha, const void* beta, const void* k_cache, const void* v_cache,
                            int64_t cap, const void* o)
{
    orthros_status st = check_desc(d);
    if (st) return st;
    if ((st = check_T(d, T, cap))) return st;
    return check_ptrs({q, k, v, alpha, beta, k_cache, v_cache, o});
}

orthros_status validate_xattn(const orthros_desc* d, int64_t T, const void* q_out, const int64_t* out_pos,
                              const void* alpha_out, const void* beta_out, const void* k_cache,
                              const void* v_cache, int64_t cap, const void* o_out, const void* ws,
                              size_t ws_bytes)
{
    orthros_status st = check_desc(d);
    if (st) return st;
    if ((st = check_T(d, T, cap))) return st;
    if (!out_pos) return fail(ORTHROS_E_NULL, "out_pos is NULL");
    for (int b = 0; b < d->batch; ++b)
        if (out_pos[b] < 0 || out_pos[b] >= T)
            return fail(ORTHROS_E_POS, "out_pos[%d] = %lld outside [0, T=%lld)", b, (long long)out_pos[b],
                        (long long)T);
    if ((st = check_ptrs({q_out, alpha_out, beta_out, k_cache, v_cache, o_out}))) return st;
    if (!ws) return fail(ORTHROS_E_WORKSPACE, "workspace is NULL");
    if ((st = check_ptrs({ws}))) return st;
    const size_t need = prefill_ws_bytes(d, T);
    if (ws_bytes < need)
        return fail(ORTHROS_E_WORKSPACE, "workspace of %zu bytes < %zu required", ws_bytes, need);
    return ORTHROS_OK;
}

orthros::SwaParams swa_params(const orthros_desc* d, int64_t T, const void* q, const void* k, const void* v,
                              const void* alpha, const void* beta, void* k_cache, void* v_cache, int64_t cap,
                              void* o)
{
    orthros::SwaParams p;
    p.q = q; p.k = k; p.v = v; p.alpha = alpha; p.beta = beta;
    p.k_cache = k_cache; p.v_cache = v_cache; p.o = o;
    p.T = T; p.cap = cap;
    p.B = d->batch; p.Hq = d->n_q_heads; p.Hkv = d->n_kv_heads; p.D = d->head_dim; p.window = d->window;
    p.qscale = qscale_of(d);
    p.dt = dt_of(d);
    return p;
}

orthros::XattnParams xattn_params(const orthros_desc* d, const Split& sp, const void* q_out,
                                  const int64_t* out_pos, const void* alpha_out, const void* beta_out,
                                  const void* k_cache, const void* v_cache, int64_t cap, void* o_out, void* ws)
{
    orthros::XattnParams p;
    p.q_out = q_out; p.alpha_out = alpha_out; p.beta_out = beta_out;
    p.k_cache = k_cache; p.v_cache = v_cache; p.o_out = o_out;
    p.ws_len = (int32_t*)ws;
    p.ws_rng = sp.lds ? (int32_t*)((char*)ws + len_bytes(d)) : nullptr;
    p.ws_part = (float*)((char*)ws + len_bytes(d) + rng_bytes(d, sp.lds));
    p.pos = out_pos;
    p.cap = cap;
    p.B = d->batch; p.Hq = d->n_q_heads; p.Hkv = d->n_kv_heads; p.D = d->head_dim;
    p.chunk = sp.chunk; p.n_split = sp.n_split; p.rec = sp.rec; p.lds = sp.lds ? 1 : 0;
    p.qscale = qscale_of(d);
    p.dt = dt_of(d);
    return p;
}

orthros_status run_swa(const orthros_desc* d, int64_t T, const void* q, const void* k, const void* v,
                       const void* alpha, const void* beta, void* k_cache, void* v_cache, int64_t cap, void* o,
                       hipStream_t s)
{
    const orthros::SwaParams p = swa_params(d, T, q, k, v, alpha, beta, k_cache, v_cache, cap, o);
    return hip_status(orthros::launch_swa(p, s), "sliding-window kernel launch");
}

orthros_status run_xattn(const orthros_desc* d, int64_t T, const void* q_out, const int64_t* out_pos,
                         const void* alpha_out, const void* beta_out, const void* k_cache, const void* v_cache,
                         int64_t cap, void* o_out, void* ws, hipStream_t s)
{
    const orthros::XattnParams p = xattn_params(d, prefill_split(d, T), q_out, out_pos, alpha_out, beta_out,
                                                k_cache, v_cache, cap, o_out, ws);
    return hip_status(orthros::launch_xattn(p, s), "cross-attention kernel launch");
}

orthros_status validate_decode(const orthros_desc* desc, const void* q, const void* q_out, const void* k_new,
                               const void* v_new, const void* alpha, const void* beta, const void* alpha_out,
                               const void* beta_out, const void* k_cache, const void* v_cache, int64_t cap,
                               const int32_t* cache_len, int64_t max_len_hint, const void* o, const void* o_out)
{
    orthros_status st = check_desc(desc);
    if (st) return st;
    if (max_len_hint < 0 || max_len_hint >= INT32_MAX)
        return fail(ORTHROS_E_SHAPE, "max_len_hint %lld outside [0, 2^31 - 1)", (long long)max_len_hint);
    if (cap < max_len_hint + 1)
        return fail(ORTHROS_E_CAPACITY, "cap %lld < max_len_hint + 1 = %lld", (long long)cap,
                    (long long)max_len_hint + 1);
    const int64_t rowq = (int64_t)desc->n_q_heads * desc->head_dim;
    if ((int64_t)desc->batch * cap > kMaxElems / rowq)
        return fail(ORTHROS_E_SHAPE, "cache size overflows the library's 2^50-element bound");
    return check_ptrs({q, q_out, k_new, v_new, alpha, beta, alpha_out, beta_out, k_cache, v_cache, cache_len, o,
                       o_out});
}

orthros_status run_decode(const orthros_desc* desc, const Split& sp, const void* q, const void* q_out,
                          const void* k_new, const void* v_new, const void* alpha, const void* beta,
                          const void* alpha_out, const void* beta_out, void* k_cache, void* v_cache, int64_t cap,
                          int32_t* cache_len, int64_t max_len_hint, void* o, void* o_out, void* workspace,
                          hipStream_t stream)
{
    orthros::DecodeParams p;
    p.q = q; p.q_out = q_out; p.k_new = k_new; p.v_new = v_new;
    p.alpha = alpha; p.beta = beta; p.alpha_out = alpha_out; p.beta_out = beta_out;
    p.k_cache = k_cache; p.v_cache = v_cache; p.cache_len = cache_len; p.o = o; p.o_out = o_out;
    p.ws_cnt = (int32_t*)workspace;
    p.ws_len = (int32_t*)((char*)workspace + cnt_bytes(desc));
    p.ws_rng = sp.lds ? (int32_t*)((char*)workspace + cnt_bytes(desc) + len_bytes(desc)) : nullptr;
    p.ws_part = (float*)((char*)workspace + cnt_bytes(desc) + len_bytes(desc) + rng_bytes(desc, sp.lds));
    p.cap = cap; p.max_len = max_len_hint;
    p.B = desc->batch; p.Hq = desc->n_q_heads; p.Hkv = desc->n_kv_heads; p.D = desc->head_dim;
    p.window = desc->window;
    p.chunk = sp.chunk; p.n_split = sp.n_split; p.rec = sp.rec; p.lds = sp.lds ? 1 : 0; p.fused = sp.fused ? 1 : 0;
    p.qscale = qscale_of(desc);
    p.dt = dt_of(desc);
    return hip_status(orthros::launch_decode(p, stream), "decode kernel launch");
}

// Scratch of the allocation-free decode entry point: the arrival counters,
// per-step lengths and split-K partials that orthros_decode_step keeps in
// the caller's workspace.  The counters start at zero (a device global is
// zero-filled when the library's code is loaded) and every step leaves them
// at zero; every other word a step reads it has written itself, so nothing
// needs clearing between calls.  In host code `scratch` only names
// the variable; its device address (one copy per GPU) comes from
// hipGetSymbolAddress, looked up once per device on that device's first call.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

orthros_status scratch_of_current_device(void** out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ORTHROS_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ORTHROS_E_HIP, "device %d beyond the %d supported", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(ORTHROS_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ORTHROS_OK;
}

}  // namespace

extern "C" {

size_t orthros_prefill_workspace_size(const orthros_desc* desc, int64_t T)
{
    if (check_desc(desc) || T < 1 || T > INT32_MAX) return 0;
    return prefill_ws_bytes(desc, T);
}

size_t orthros_decode_workspace_size(const orthros_desc* desc, int64_t max_len)
{
    if (check_desc(desc) || max_len < 0 || max_len >= INT32_MAX) return 0;
    return decode_split(desc, max_len).bytes;
}

orthros_status orthros_swa_prefill(const orthros_desc* desc, int64_t T, const void* q, const void* k,
                                   const void* v, const void* alpha, const void* beta, void* k_cache,
                                   void* v_cache, int64_t cap, void* o, void* stream)
{
    g_err.clear();
    orthros_status st = validate_swa(desc, T, q, k, v, alpha, beta, k_cache, v_cache, cap, o);
    if (st) return st;
    return run_swa(desc, T, q, k, v, alpha, beta, k_cache, v_cache, cap, o, (hipStream_t)stream);
}

orthros_status orthros_global_xattn(const orthros_desc* desc, int64_t T, const void* q_out,
                                    const int64_t* out_pos, const void* alpha_out, const void* beta_out,
                                    const void* k_cache, const void* v_cache, int64_t cap, void* o_out,
                                    void* workspace, size_t workspace_bytes, void* stream)
{
    g_err.clear();
    orthros_status st = validate_xattn(desc, T, q_out, out_pos, alpha_out, beta_out, k_cache, v_cache, cap,
                                       o_out, workspace, workspace_bytes);
    if (st) return st;
    return run_xattn(desc, T, q_out, out_pos, alpha_out, beta_out, k_cache, v_cache, cap, o_out, workspace,
                     (hipStream_t)stream);
}

orthros_status orthros_prefill(const orthros_desc* desc, int64_t T, const void* q, const void* q_out,
                               const int64_t* out_pos, const void* k, const void* v, const void* alpha,
                               const void* beta, const void* alpha_out, const void* beta_out, void* k_cache,
                               void* v_cache, int64_t cap, void* o, void* o_out, void* workspace,
                               size_t workspace_bytes, void* stream)
{
    g_err.clear();
    orthros_status st = validate_swa(desc, T, q, k, v, alpha, beta, k_cache, v_cache, cap, o);
    if (st) return st;
    st = validate_xattn(desc, T, q_out, out_pos, alpha_out, beta_out, k_cache, v_cache, cap, o_out, workspace,
                        workspace_bytes);
    if (st) return st;
    if (fused_prefill(desc)) {
        // one pass over K/V: the streaming SWA kernel also attends the copy's
        // query to the pairs it brings in, then the LSE merge
        const orthros::SwaParams p = swa_params(desc, T, q, k, v, alpha, beta, k_cache, v_cache, cap, o);
        const orthros::XattnParams x = xattn_params(desc, fused_split(desc, T), q_out, out_pos, alpha_out,
                                                    beta_out, k_cache, v_cache, cap, o_out, workspace);
        return hip_status(orthros::launch_swa_ring_fused(p, x, (hipStream_t)stream), "fused prefill kernel launch");
    }
    st = run_swa(desc, T, q, k, v, alpha, beta, k_cache, v_cache, cap, o, (hipStream_t)stream);
    if (st) return st;
    return run_xattn(desc, T, q_out, out_pos, alpha_out, beta_out, k_cache, v_cache, cap, o_out, workspace,
                     (hipStream_t)stream);
}

orthros_status orthros_copies(const orthros_desc* desc, int64_t T, int64_t T_out, const void* q_out,
                              const int32_t* out_pos, const void* alpha_out, const void* beta_out,
                              const void* k_cache, const void* v_cache, int64_t cap, void* o_out, void* stream)
{
    g_err.clear();
    orthros_status st = check_desc(desc);
    if (st) return st;
    if ((st = check_T(desc, T, cap))) return st;
    if (T_out < 1 || T_out > INT32_MAX)
        return fail(ORTHROS_E_SHAPE, "T_out = %lld outside [1, 2^31)", (long long)T_out);
    const int64_t rowq = (int64_t)desc->n_q_heads * desc->head_dim;
    if ((int64_t)desc->batch * T_out > kMaxElems / rowq)
        return fail(ORTHROS_E_SHAPE, "copy tensors overflow the library's 2^50-element bound");
    if ((st = check_ptrs({q_out, alpha_out, beta_out, k_cache, v_cache, o_out}))) return st;
    if (!out_pos) return fail(ORTHROS_E_NULL, "out_pos is NULL");
    if (reinterpret_cast<uintptr_t>(out_pos) & 3u) return fail(ORTHROS_E_ALIGN, "out_pos is not 4-byte aligned");
    orthros::CopiesParams p;
    p.q_out = q_out; p.pos = out_pos; p.alpha_out = alpha_out; p.beta_out = beta_out;
    p.k_cache = k_cache; p.v_cache = v_cache; p.o_out = o_out;
    p.T = T; p.T_out = T_out; p.cap = cap;
    p.B = desc->batch; p.Hq = desc->n_q_heads; p.Hkv = desc->n_kv_heads; p.D = desc->head_dim;
    p.qscale = qscale_of(desc);
    p.dt = dt_of(desc);
    return hip_status(orthros::launch_copies(p, (hipStream_t)stream), "copies kernel launch");
}

orthros_status orthros_project(const orthros_desc* desc, int64_t T, int64_t T_out, int64_t d_model,
                               const void* x, const void* x_out, const void* w_q, const void* w_k, const void* w_v,
                               const void* alpha, const void* beta, const void* alpha_out, const void* beta_out,
                               void* q, void* q_out, void* k_cache, void* v_cache, int64_t cap, void* stream)
{
    g_err.clear();
    orthros_status st = check_desc(desc);
    if (st) return st;
    if (desc->dtype != ORTHROS_BF16) return fail(ORTHROS_E_DTYPE, "orthros_project takes bf16 tensors only");
    if ((st = check_T(desc, T, cap))) return st;
    if (T_out < 0 || T_out > INT32_MAX)
        return fail(ORTHROS_E_SHAPE, "T_out = %lld outside [0, 2^31)", (long long)T_out);
    if (d_model < 32 || d_model > 65536 || d_model % 32)
        return fail(ORTHROS_E_SHAPE, "d_model = %lld: must be a multiple of 32 in [32, 65536]", (long long)d_model);
    const int64_t nq = (int64_t)desc->n_q_heads * desc->head_dim, nk = (int64_t)desc->n_kv_heads * desc->head_dim;
    if (nq % 128 || nk % 128)
        return fail(ORTHROS_E_SHAPE, "n_q_heads * head_dim (%lld) and n_kv_heads * head_dim (%lld) must be "
                    "multiples of 128", (long long)nq, (long long)nk);
    const int64_t rows = (int64_t)desc->batch * (T + T_out);
    if (rows > kMaxElems / d_model || (int64_t)desc->batch * T_out > kMaxElems / nq)
        return fail(ORTHROS_E_SHAPE, "tensor sizes overflow the library's 2^50-element bound");
    if ((st = check_ptrs({x, w_q, w_k, w_v, q, k_cache, v_cache}))) return st;
    if (T_out > 0 && (st = check_ptrs({x_out, q_out}))) return st;
    if (!alpha != !beta || !alpha_out != !beta_out)
        return fail(ORTHROS_E_NULL, "alpha and beta (and alpha_out and beta_out) must be given together");
    for (const void* v : {alpha, beta, alpha_out, beta_out})
        if (v && !aligned16(v)) return fail(ORTHROS_E_ALIGN, "a device pointer is not 16-byte aligned");
    orthros::ProjParams p;
    p.x = (const uint16_t*)x; p.xo = (const uint16_t*)x_out;
    p.wq = (const uint16_t*)w_q; p.wk = (const uint16_t*)w_k; p.wv = (const uint16_t*)w_v;
    p.alpha = (const uint16_t*)alpha; p.beta = (const uint16_t*)beta;
    p.alpha_out = (const uint16_t*)alpha_out; p.beta_out = (const uint16_t*)beta_out;
    p.q = (uint16_t*)q; p.q_out = (uint16_t*)q_out; p.k_cache = (uint16_t*)k_cache; p.v_cache = (uint16_t*)v_cache;
    p.Mx = (int64_t)desc->batch * T; p.Mo = (int64_t)desc->batch * T_out;
    p.T = T; p.cap = cap; p.K = d_model; p.tiles_b = 0;
    p.Hq = desc->n_q_heads; p.Hkv = desc->n_kv_heads; p.D = desc->head_dim;
    if (!orthros::project_applies(p)) return fail(ORTHROS_E_SHAPE, "shape not supported by the projection kernel");
    return hip_status(orthros::launch_project(p, (hipStream_t)stream), "projection kernel launch");
}

orthros_status orthros_decode_step(const orthros_desc* desc, const void* q, const void* q_out,
                                   const void* k_new, const void* v_new, const void* alpha, const void* beta,
                                   const void* alpha_out, const void* beta_out, void* k_cache, void* v_cache,
                                   int64_t cap, int32_t* cache_len, int64_t max_len_hint, void* o, void* o_out,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    g_err.clear();
    orthros_status st = validate_decode(desc, q, q_out, k_new, v_new, alpha, beta, alpha_out, beta_out, k_cache,
                                        v_cache, cap, cache_len, max_len_hint, o, o_out);
    if (st) return st;
    if (!workspace) return fail(ORTHROS_E_WORKSPACE, "workspace is NULL");
    if ((st = check_ptrs({workspace}))) return st;
    const Split sp = decode_split(desc, max_len_hint);
    if (workspace_bytes < sp.bytes)
        return fail(ORTHROS_E_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, sp.bytes);
    return run_decode(desc, sp, q, q_out, k_new, v_new, alpha, beta, alpha_out, beta_out, k_cache, v_cache, cap,
                      cache_len, max_len_hint, o, o_out, workspace, (hipStream_t)stream);
}

orthros_status orthros_decode_step_noalloc(const orthros_desc* desc, const void* q, const void* q_out,
                                           const void* k_new, const void* v_new, const void* alpha,
                                           const void* beta, const void* alpha_out, const void* beta_out,
                                           void* k_cache, void* v_cache, int64_t cap, int32_t* cache_len,
                                           int64_t max_len_hint, void* o, void* o_out, void* stream)
{
    g_err.clear();
    orthros_status st = validate_decode(desc, q, q_out, k_new, v_new, alpha, beta, alpha_out, beta_out, k_cache,
                                        v_cache, cap, cache_len, max_len_hint, o, o_out);
    if (st) return st;
    const Split sp = decode_split(desc, max_len_hint);
    if (sp.bytes > kScratchBytes)
        return fail(ORTHROS_E_WORKSPACE, "this step needs %zu bytes of scratch, more than the %zu bytes the "
                    "allocation-free entry point holds (use orthros_decode_step with a workspace)", sp.bytes,
                    kScratchBytes);
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws))) return st;
    return run_decode(desc, sp, q, q_out, k_new, v_new, alpha, beta, alpha_out, beta_out, k_cache, v_cache, cap,
                      cache_len, max_len_hint, o, o_out, ws, (hipStream_t)stream);
}

const char* orthros_status_str(int status)
{
    switch (status) {
    case ORTHROS_OK: return "ORTHROS_OK";
    case ORTHROS_E_NULL: return "ORTHROS_E_NULL";
    case ORTHROS_E_SHAPE: return "ORTHROS_E_SHAPE";
    case ORTHROS_E_DTYPE: return "ORTHROS_E_DTYPE";
    case ORTHROS_E_POS: return "ORTHROS_E_POS";
    case ORTHROS_E_CAPACITY: return "ORTHROS_E_CAPACITY";
    case ORTHROS_E_WORKSPACE: return "ORTHROS_E_WORKSPACE";
    case ORTHROS_E_HIP: return "ORTHROS_E_HIP";
    case ORTHROS_E_ALIGN: return "ORTHROS_E_ALIGN";
    default: return "ORTHROS_E_UNKNOWN";
    }
}

const char* orthros_last_error(void) { return g_err.c_str(); }

int orthros_abi_version(void) { return ORTHROS_ABI_VERSION; }

}  // extern "C"
