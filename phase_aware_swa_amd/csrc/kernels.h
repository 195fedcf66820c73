// kernels.h -- internal interface between the C-ABI host code (api.hip) and
// the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthros {

// Storage type of every tensor of a call.
enum class Dt : int32_t { F32 = 0, BF16 = 1 };

// Base-stream sliding-window attention + cache write (prefill).
struct SwaParams {
    const void* q;        // [B][T][Hq][D]
    const void* k;        // [B][T][Hkv][D]
    const void* v;
    const void* alpha;    // [Hq][D]
    const void* beta;
    void* k_cache;        // [B][Hkv][cap][D]
    void* v_cache;
    void* o;              // [B][T][Hq][D]
    int64_t T, cap;
    int32_t B, Hq, Hkv, D, window;
    float qscale;         // softmax_scale * log2(e)
    Dt dt;
};

// Chunked single-query attention over the cache (the output copy, and in
// decode also the base token's window), followed by the LSE merge.
constexpr int kPosPerLaunch = 64;   // batch rows whose copy positions travel in one launch
struct PosBlock { int64_t v[kPosPerLaunch]; };   // passed by value as a kernel argument

struct XattnParams {
    const void* q_out;    // [B][Hq][D]
    const void* alpha_out;
    const void* beta_out;
    const void* k_cache;  // [B][Hkv][cap][D]
    const void* v_cache;
    void* o_out;          // [B][Hq][D]
    int32_t* ws_len;      // workspace: per-sequence last key index
    int32_t* ws_rng;      // workspace (LDS-streamed kernel): record range per stream, [B][streams][3]
    float* ws_part;       // workspace: partials [B][Hq][1][n_split][rec], or the LDS-streamed
                          // kernel's records [id][4][rec]
    const int64_t* pos;   // host [B]: copy positions
    int64_t cap;
    int32_t B, Hq, Hkv, D;
    int32_t chunk, n_split;
    // stride of a partial record in floats: (max, sum, ..., weighted values
    // at rec - D); D + 2, except on the LDS-streamed kernel (D +
    // kXattnLdsRecPad: the values start on a 128-byte line)
    int32_t rec;
    int32_t lds;          // nonzero: the LDS-streamed kernel (chosen with the split)
    float qscale;
    Dt dt;
};

struct DecodeParams {
    const void* q;        // [B][Hq][D]
    const void* q_out;
    const void* k_new;    // [B][Hkv][D]
    const void* v_new;
    const void* alpha;
    const void* beta;
    const void* alpha_out;
    const void* beta_out;
    void* k_cache;        // [B][Hkv][cap][D]
    void* v_cache;
    int32_t* cache_len;   // device [B]
    void* o;              // [B][Hq][D]
    void* o_out;
    int32_t* ws_cnt;      // workspace: arrival counters, [B][Hkv * G / HG] per head block then [B] per
                          // sequence (short-history kernel); zero before a step and after it
    int32_t* ws_len;      // workspace: per-sequence length seen by this step
    int32_t* ws_rng;      // workspace (LDS-streamed kernel): as in XattnParams
    float* ws_part;       // workspace: partials [B][Hq][2][n_split][rec], or the LDS-streamed
                          // kernel's records [id][2][4][rec]
    int64_t cap, max_len;
    int32_t B, Hq, Hkv, D, window;
    int32_t chunk, n_split;
    int32_t rec;          // as in XattnParams
    int32_t lds;          // nonzero: the LDS-streamed kernel (chosen with the split)
    int32_t fused;        // nonzero: the one-launch short-history kernel (chunk = kDecodeShortChunk)
    float qscale;
    Dt dt;
};

// Heads of one KV group that one workgroup of the chunked kernels serves.
__host__ __device__ inline int xattn_heads_per_wg(int G) { return (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1; }

hipError_t launch_swa(const SwaParams& p, hipStream_t s);
// Streaming sliding-window kernel: bf16, window <= kRingMaxWindow, any group
// (blocks of ring_heads_per_block(G) query heads per KV head: 4 for groups
// that are multiples of 4, 2 for other even ones, else 1), with or without
// the output copy's global query folded in.
constexpr int kRingMaxWindow = 129;
inline bool ring_applies(Dt dt, int, int, int window) { return dt == Dt::BF16 && window <= kRingMaxWindow; }
inline int ring_heads_per_block(int G) { return (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1; }
// Launch geometry of the streaming kernel: ceil(T / 32) tiles of 32 rows per
// (sequence, KV head, head block) stream, cut into n_seg segments of tps
// tiles (about two workgroups per CU of the 256).
struct RingGeom { int n_tiles, hblocks, n_seg, tps; };
RingGeom ring_geometry(int B, int Hq, int Hkv, int64_t T);
hipError_t launch_swa_ring(const SwaParams& p, hipStream_t s);
// The streaming kernel with the output copy's global query fused in: each
// workgroup attends the copy's query of its block's heads (a wave each) to
// the pairs it brings in and leaves one partial per head and segment (x.chunk = 32 tps keys, x.n_split =
// n_seg); the LSE merge follows.  x.k_cache / v_cache are not read.
hipError_t launch_swa_ring_fused(const SwaParams& p, const XattnParams& x, hipStream_t s);
hipError_t launch_xattn(const XattnParams& p, hipStream_t s);
// LSE merge of bf16 prefill partials [B][Hq][1][n_split][rec] into o_out.
hipError_t launch_merge(const XattnParams& p, hipStream_t s);
// The LDS-streamed MFMA form of the cross-attention (bf16, any group size:
// streams of xattn_heads_per_wg(G) query heads): a persistent kernel, one
// workgroup per CU (at most kXattnLdsMaxGrid), each taking an equal run of
// the launch's keys (at least kXattnLdsSegMin), then the LSE merge.  A
// launch serves up to kPosPerLaunch sequences; its records take ids
// rbase .. rbase + region - 1 (one per segment: a run's piece of one stream,
// at most streams + grid of them), where launch i has rbase = i * region.
inline bool xattn_lds_applies(Dt dt, int, int) { return dt == Dt::BF16; }
// In prefill the LDS-streamed kernel takes groups that are multiples of 4,
// and other groups when the copies read at least kXattnLdsPrefillMinKeys
// keys over all streams: below that its runs are a few stages long and the
// lane-parallel kernel's many resident workgroups (and cached loads, which
// can hit what the SWA pass just wrote) do better (8K MHA: 67 against 70 us).
constexpr int64_t kXattnLdsPrefillMinKeys = int64_t(1) << 20;
// In decode, past the one-launch short kernel, it takes groups that are
// multiples of 4, and other groups when max_len_hint + 1 keys over all
// streams reach kXattnLdsDecodeMinKeys or one history reaches
// kXattnLdsDecodeLongKeys; below both the lane-parallel kernel's many
// workgroups hide the latency better.  Measured per step, lane-parallel
// against LDS-streamed, MHA d128 with 8K-32K histories: batch 4 62.6
// against 67.2 us, batch 8 150 against 133; batch 1 with 64K-128K
// histories 101 against 89.
constexpr int64_t kXattnLdsDecodeMinKeys = int64_t(3) << 19;
constexpr int64_t kXattnLdsDecodeLongKeys = int64_t(1) << 16;
constexpr int kXattnLdsRecPad = 32;   // floats before the values in a partial record
constexpr int kXattnLdsMaxGrid = 512;
constexpr int64_t kXattnLdsSegMin = 256;
inline int64_t xattn_lds_region(int B, int streams)
{
    return (int64_t)(B < kPosPerLaunch ? B : kPosPerLaunch) * streams + kXattnLdsMaxGrid;
}
inline int64_t xattn_lds_records(int B, int streams)
{
    return (int64_t)((B + kPosPerLaunch - 1) / kPosPerLaunch) * xattn_lds_region(B, streams);
}
hipError_t launch_xattn_lds(const XattnParams& p, hipStream_t s);
// LSE merge of the LDS-streamed kernel's records (the ranges in ws_rng)
// into o_out; in decode into o_out and o with the new token's key L added,
// then that key appended at slot L and cache_len[b] += 1.
hipError_t launch_lds_merge(const XattnParams& p, hipStream_t s);
hipError_t launch_lds_merge(const DecodeParams& p, hipStream_t s);
// The decode step: for bf16 steps of at most kDecodeShortMaxSplits chunks
// of kDecodeShortChunk keys, on the one-launch short-history kernel (fused =
// 1); longer bf16 ones on the LDS-streamed kernel (stream, then the merge
// that adds the new key and appends it) when the rule above takes it; the rest (fp32 among them) on the
// lane-parallel split kernel and a merge kernel.
constexpr int kDecodeShortChunk = 128;
constexpr int kDecodeShortMaxSplits = 32;
hipError_t launch_decode(const DecodeParams& p, hipStream_t s);
// The decode step on the LDS-streamed kernel (bf16, more keys than the
// one-launch short-history kernel takes): the copy and the base token over
// the history 0 .. L - 1 in one streaming pass, then the LSE merge of both
// kinds with the new token's key L from k_new / v_new, which also appends
// that key at slot L and advances cache_len.
hipError_t launch_decode_lds(const DecodeParams& p, hipStream_t s);
// LSE merge of decode partials [B][Hq][2][n_split][rec] into o_out and o,
// then cache_len[b] += 1 for every valid sequence.
hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t s);

// Output copies at many positions per sequence (no workspace).
struct CopiesParams {
    const void* q_out;      // [B][T_out][Hq][D]
    const int32_t* pos;     // device [B][T_out]
    const void* alpha_out;  // [Hq][D]
    const void* beta_out;
    const void* k_cache;    // [B][Hkv][cap][D]
    const void* v_cache;
    void* o_out;            // [B][T_out][Hq][D]
    int64_t T, T_out, cap;
    int32_t B, Hq, Hkv, D;
    float qscale;
    Dt dt;
};
hipError_t launch_copies(const CopiesParams& p, hipStream_t s);
// The MFMA flash form of the copies (bf16, groups of 4 query heads).
bool copies_flash_applies(const CopiesParams& p);
hipError_t launch_copies_flash(const CopiesParams& p, hipStream_t s);

// The projections either side of the attention step (bf16): q and k/v of the
// base rows X, q' of the copy rows X', one shared W_Q.
struct ProjParams {
    const uint16_t* x;          // [Mx][K], Mx = B * T
    const uint16_t* xo;         // [Mo][K], Mo = B * T_out (may be null when Mo = 0)
    const uint16_t* wq;         // [Hq*D][K]
    const uint16_t* wk;         // [Hkv*D][K]
    const uint16_t* wv;
    const uint16_t* alpha;      // [Hq*D]; null (with beta) = no scale-offset
    const uint16_t* beta;
    const uint16_t* alpha_out;  // same, for the copy rows
    const uint16_t* beta_out;
    uint16_t* q;                // [Mx][Hq*D]
    uint16_t* q_out;            // [Mo][Hq*D]
    uint16_t* k_cache;          // [B][Hkv][cap][D]
    uint16_t* v_cache;
    int64_t Mx, Mo, T, cap, K;
    int64_t tiles_b;            // set by the launcher
    int32_t Hq, Hkv, D;
};
// Shapes the tiled kernel takes: Hq*D and Hkv*D multiples of 128, K a
// multiple of 32.
bool project_applies(const ProjParams& p);
hipError_t launch_project(const ProjParams& p, hipStream_t s);

}  // namespace orthros
