// global_xattn.hip -- the output-only stream's full-history causal
// cross-attention (prefill and decode) and the decode step, for gfx950.
//
// "Orthros:阶段感知异构注意力精读笔记" §2.3 Eq. (5): the output copy at
// original position P attends over every cached key j <= P (§2.4: the mask
// follows the original position, never the copy's slot at the tensor tail).
// Its query is q_out * alpha_out + beta_out (§2.2).  In decode (§2.5 decode
// row, §2.4 walk-through) the step also appends the new base token's K/V at
// slot L = cache_len[b], runs the base token's window [L-w+1, L], and the
// copy reads [0, L], the new token included.
//
// One query per (sequence, head) over up to a million keys is a
// memory-bound stream (about 2 flop per cache byte per head), so the work is
// split along the keys (split-K):
//   - a workgroup owns one key chunk of one KV head and serves the HG query
//     heads of that group at once, so each K/V byte is read from HBM once;
//   - inside a wave, D/8 lanes hold one key row (8 head-dim values each, a
//     16-byte load), so a wave reads 4 (d=128) or 8 (d=64) whole 256-byte or
//     128-byte rows per load instruction; the dot product is finished with
//     DPP row moves (no LDS);
//   - each lane keeps an fp32 online-softmax state per head for the keys
//     it saw; the states of a workgroup are merged by lane shuffles, then
//     through LDS, into one (max, sum, unnormalised output) partial per head;
//   - the partials of a (sequence, head) are merged by log-sum-exp in a
//     fixed split order, so results are run-to-run identical: by a second
//     kernel in prefill, and in decode by the last workgroup of the head
//     block to finish (one launch per step).
// The decode step uses the same chunk worker for the copy (range [0, L])
// and the base token (range [L-w+1, L]); the new token's key L is read from
// k_new/v_new, never from the cache slot the same launch is writing.

#include "device.h"
#include "kernels.h"
#include "pair_tile.h"

namespace orthros {
namespace {

constexpr int kUnroll = 4;   // key rows per lane per softmax update

// 8 consecutive head-dim values of one row, kept in storage form until used.
template <typename E> struct Row8;
template <> struct Row8<uint16_t> {
    u32x4 w;
    __device__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
    __device__ void load(const uint16_t* p) { w = *(const u32x4*)p; }
    __device__ float operator[](int e) const { return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]); }
};
template <> struct Row8<float> {
    float4 a, b;
    __device__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ void load(const float* p) { a = *(const float4*)p; b = *(const float4*)(p + 4); }
    __device__ float operator[](int e) const
    {
        const float4& x = e < 4 ? a : b;
        switch (e & 3) { case 0: return x.x; case 1: return x.y; case 2: return x.z; default: return x.w; }
    }
};

// A lane's 8-wide slice of one scale-offset query, and its dot product with
// a key row slice.  bf16 storage: the query slice is rounded to bf16 and the
// product uses v_dot2_f32_bf16 (exact products, fp32 accumulate), as the
// bf16 MFMA path rounds its query operand; fp32 storage: plain fp32 FMAs.
template <typename E> struct QSlice;
template <> struct QSlice<uint16_t> {
    bf16x2 q[4];
    __device__ void set(const float* x)
    {
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = __builtin_bit_cast(bf16x2, pack_bf16x2(x[2 * e], x[2 * e + 1]));
    }
    __device__ float dot(const Row8<uint16_t>& k) const
    {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // copy the lane out of the vector first: a bit_cast applied to a
            // vector element directly reads element 0 with this compiler
            const uint32_t kw = k.w[e];
            acc = __builtin_amdgcn_fdot2_f32_bf16(q[e], __builtin_bit_cast(bf16x2, kw), acc, false);
        }
        return acc;
    }
};
template <> struct QSlice<float> {
    float q[8];
    __device__ void set(const float* x)
    {
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = x[e];
    }
    __device__ float dot(const Row8<float>& k) const
    {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += q[e] * k[e];
        return acc;
    }
};

__device__ __forceinline__ float ld_elem(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ float ld_elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ void st_elem(uint16_t* p, int64_t i, float x) { p[i] = (uint16_t)f32_to_bf16_bits(x); }
__device__ __forceinline__ void st_elem(float* p, int64_t i, float x) { p[i] = x; }

// Scale-offset queries of HG heads into LDS: qs[hh][d] = (q*alpha+beta)*qscale.
template <typename E, int D, int HG>
__device__ __forceinline__ void load_queries(float (*qs)[D], const E* q, const E* alpha, const E* beta,
                             int64_t qrow0, int h0, float qscale)
{
    for (int idx = threadIdx.x; idx < HG * D; idx += blockDim.x) {
        const int hh = idx / D, d = idx % D;
        const int64_t hd = (int64_t)(h0 + hh) * D + d;
        qs[hh][d] = (ld_elem(q, qrow0 + hd) * ld_elem(alpha, hd) + ld_elem(beta, hd)) * qscale;
    }
}

// Online softmax over keys [lo, hi] of one KV head for HG queries; writes
// one partial (max, sum, sum of weighted values) per query head to
// out[hh * out_stride + {0, 1, 2 + d}].  Key rows start at kc + j * D; key
// `lnew` (if >= 0) is read from knew/vnew instead.  256 threads.
template <typename E, int D, int HG>
__device__ __forceinline__ void attend_chunk(const float (*qs)[D], const E* kc, const E* vc,
                             int64_t lnew, const E* knew, const E* vnew,
                             int64_t lo, int64_t hi, float (*red)[HG][D + 2],
                             float* out, int64_t out_stride)
{
    constexpr bool kBf16 = sizeof(E) == 2;
    static_assert(kUnroll % 2 == 0, "keys go in pairs");
    constexpr int LPK = D / 8;        // lanes per key row
    constexpr int KPW = 64 / LPK;     // key rows per wave per step
    constexpr int KPS = 4 * KPW;      // key rows per workgroup per step
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c = lane % LPK, kg = lane / LPK;

    QSlice<E> qr[HG];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) qr[hh].set(&qs[hh][8 * c]);

    float m[HG], l[HG], acc[HG][8];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
        m[hh] = kNegBig;
        l[hh] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = 0.f;
    }

    for (int64_t base = lo; base <= hi; base += (int64_t)KPS * kUnroll) {
        Row8<E> kx[kUnroll], vx[kUnroll];
        bool ok[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = base + (int64_t)u * KPS + wv * KPW + kg;
            ok[u] = j <= hi;
            kx[u].zero();
            vx[u].zero();
            if (ok[u]) {
                const E* kr = (j == lnew) ? knew : kc + j * D;
                const E* vr = (j == lnew) ? vnew : vc + j * D;
                kx[u].load(kr + 8 * c);
                vx[u].load(vr + 8 * c);
            }
        }
        // bf16: V values of keys (u, u+1) paired per head-dim value, shared by the heads
        uint32_t vp[kUnroll / 2][8];
        if constexpr (kBf16) {
#pragma unroll
            for (int u = 0; u < kUnroll; u += 2)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t a0 = vx[u].w[w], a1 = vx[u + 1].w[w];
                    vp[u / 2][2 * w] = (a0 & 0xffffu) | (a1 << 16);
                    vp[u / 2][2 * w + 1] = (a0 >> 16) | (a1 & 0xffff0000u);
                }
        }
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
            float s[kUnroll];
            float mx = m[hh];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const float dot = group_sum<LPK>(qr[hh].dot(kx[u]));
                s[u] = ok[u] ? dot : -INFINITY;
                mx = fmaxf(mx, s[u]);
            }
            const float corr = fast_exp2(m[hh] - mx);
            m[hh] = mx;
            l[hh] *= corr;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[hh][e] *= corr;
            if constexpr (kBf16) {
                // keys in pairs: P as a bf16 pair, V as (key u, key u+1) pairs
                // per head-dim value, one v_dot2_f32_bf16 per value; the row
                // sum takes the same rounded weights
#pragma unroll
                for (int u = 0; u < kUnroll; u += 2) {
                    const uint32_t pp = pack_bf16x2(fast_exp2(s[u] - mx), fast_exp2(s[u + 1] - mx));
                    l[hh] += bf16_lo(pp) + bf16_hi(pp);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        acc[hh][e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, vp[u / 2][e]),
                                                                     __builtin_bit_cast(bf16x2, pp), acc[hh][e],
                                                                     false);
                }
            } else {
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    const float p = fast_exp2(s[u] - mx);
                    l[hh] += p;
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[hh][e] += p * vx[u][e];
                }
            }
        }
    }

    // merge the KPW key slots of a wave (lanes differing in kg)
#pragma unroll
    for (int x = LPK; x < 64; x <<= 1) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
            const float mo = __shfl_xor(m[hh], x);
            const float lo_ = __shfl_xor(l[hh], x);
            const float mx = fmaxf(m[hh], mo);
            const float f = fast_exp2(m[hh] - mx), fo = fast_exp2(mo - mx);
            l[hh] = l[hh] * f + lo_ * fo;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[hh][e] = acc[hh][e] * f + __shfl_xor(acc[hh][e], x) * fo;
            m[hh] = mx;
        }
    }
    if (kg == 0) {
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wv][hh][2 + 8 * c + e] = acc[hh][e];
            if (c == 0) { red[wv][hh][0] = m[hh]; red[wv][hh][1] = l[hh]; }
        }
    }
    __syncthreads();
    // merge the 4 waves in a fixed order
    for (int idx = threadIdx.x; idx < HG * (D + 1); idx += blockDim.x) {
        const int hh = idx / (D + 1), d = idx % (D + 1);   // d == D: the (max, sum) pair
        float M = red[0][hh][0];
#pragma unroll
        for (int w = 1; w < 4; ++w) M = fmaxf(M, red[w][hh][0]);
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = fast_exp2(red[w][hh][0] - M);
            sum += f * (d < D ? red[w][hh][2 + d] : red[w][hh][1]);
        }
        float* o = out + hh * out_stride;
        if (d < D) {
            o[2 + d] = sum;
        } else {
            o[0] = M;
            o[1] = sum;
        }
    }
    __syncthreads();
}

// --------------------------------------------------------------- LSE merge

// Log-sum-exp merge of the partial records s0..s1 of one (sequence, head,
// kind) at pk (record s at pk + s * stride floats: max, sum, ..., weighted
// values at aoff) into out[row .. row + D):
//   o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
// With xv set, one more key takes part: score xm (exp2 units), weight 1,
// values the bf16 row xv (a decode step's new token, which no record holds).
// 256 threads.  Thread t owns head-dim values 4 (t % (D/4)) .. +3 of split
// group t / (D/4); the split groups are then added in a fixed order, so the
// result is run-to-run identical.  Ends with a barrier (LDS reusable).
template <typename E, int D>
__device__ void merge_splits(const float* pk, int64_t stride, int aoff, int s0, int s1, E* out, int64_t row,
                             float xm = 0.f, const uint16_t* xv = nullptr)
{
    constexpr int TPR = D / 4;            // threads per head-dim row
    constexpr int NG = 256 / TPR;         // split groups
    __shared__ float red[NG][D + 1];
    __shared__ float wmax[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int gp = tid / TPR, d4 = tid % TPR;
    // M = max over splits
    float mx = kNegBig;
    for (int s = s0 + tid; s <= s1; s += 256) mx = fmaxf(mx, pk[(int64_t)s * stride]);
#pragma unroll
    for (int x = 32; x > 0; x >>= 1) mx = fmaxf(mx, __shfl_xor(mx, x));
    if (lane == 0) wmax[wv] = mx;
    __syncthreads();
    const float M0 = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float M = xv ? fmaxf(M0, xm) : M0;
    // this thread's split group: weighted sums of 4 head-dim values and of
    // l, eight splits per round with every load of the round issued first
    // (one L2 round trip per round, not per split); a round's splits past
    // s1 read split s1 again with weight 0
    float n0 = 0.f, n1 = 0.f, n2 = 0.f, n3 = 0.f, den = 0.f;
    constexpr int RB = 8;
    for (int s = s0 + gp; s <= s1; s += NG * RB) {
        float ml[RB][2];
        float2 a[RB], c[RB];
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const int sk = s + NG * k <= s1 ? s + NG * k : s1;
            const float* ps = pk + (int64_t)sk * stride;
            ml[k][0] = ps[0];
            ml[k][1] = ps[1];
            a[k] = *(const float2*)(ps + aoff + 4 * d4);
            c[k] = *(const float2*)(ps + aoff + 2 + 4 * d4);
        }
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const float f = s + NG * k <= s1 ? fast_exp2(ml[k][0] - M) : 0.f;
            den += f * ml[k][1];
            n0 += f * a[k].x;
            n1 += f * a[k].y;
            n2 += f * c[k].x;
            n3 += f * c[k].y;
        }
    }
    if (xv && gp == 0) {
        // the extra key, in split group 0
        const float f = fast_exp2(xm - M);
        const u32x2 w = *(const u32x2*)(xv + 4 * d4);
        den += f;
        n0 += f * bf16_lo(w[0]);
        n1 += f * bf16_hi(w[0]);
        n2 += f * bf16_lo(w[1]);
        n3 += f * bf16_hi(w[1]);
    }
    red[gp][4 * d4] = n0;
    red[gp][4 * d4 + 1] = n1;
    red[gp][4 * d4 + 2] = n2;
    red[gp][4 * d4 + 3] = n3;
    if (d4 == 0) red[gp][D] = den;
    __syncthreads();
    for (int d = tid; d < D; d += 256) {
        float num = 0.f, dsum = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            num += red[g][d];
            dsum += red[g][D];
        }
        st_elem(out, row + d, num / dsum);
    }
    __syncthreads();
}

// ------------------------------------------------------ prefill: split-K

template <typename E, int D, int HG>
__global__ __launch_bounds__(256) void xattn_split_kernel(XattnParams p, int b0, int nb, PosBlock pos)
{
    __shared__ float qs[HG][D];
    __shared__ float red[4][HG][D + 2];
    const int s = blockIdx.x;
    const int G = p.Hq / p.Hkv, hblocks = G / HG;
    const int g = blockIdx.y / hblocks, hb = blockIdx.y % hblocks;
    const int bi = blockIdx.z, b = b0 + bi;
    const int64_t P = pos.v[bi];
    if (s == 0 && blockIdx.y == 0 && threadIdx.x == 0) p.ws_len[b] = (int32_t)P;
    const int64_t lo = (int64_t)s * p.chunk;
    if (lo > P) return;
    const int64_t hi = lo + p.chunk - 1 < P ? lo + p.chunk - 1 : P;
    const int h0 = g * G + hb * HG;
    load_queries<E, D, HG>(qs, (const E*)p.q_out, (const E*)p.alpha_out, (const E*)p.beta_out,
                           (int64_t)b * p.Hq * D, h0, p.qscale);
    __syncthreads();
    const int64_t crow = ((int64_t)b * p.Hkv + g) * p.cap * D;
    const int64_t part_stride = (int64_t)p.n_split * (D + 2);
    float* out = p.ws_part + ((int64_t)b * p.Hq + h0) * part_stride + (int64_t)s * (D + 2);
    attend_chunk<E, D, HG>(qs, (const E*)p.k_cache + crow, (const E*)p.v_cache + crow, -1, nullptr,
                           nullptr, lo, hi, red, out, part_stride);
}

// ----------------------------------------------------------- decode: split

// The decode step's split kernel (the two-launch form): a workgroup takes
// split s (keys [s chunk, (s+1) chunk)) of one KV head's HG-head block of
// sequence b, for the copy over [0, L] and the base token over its window;
// the partials and each sequence's length go to the workspace and the merge
// kernel combines them (many splits per row merge fastest there, spread over
// B x Hq workgroups).
template <typename E, int D, int HG>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeParams p)
{
    __shared__ float qs[2][HG][D];
    __shared__ float red[4][HG][D + 2];
    const int s = blockIdx.x;
    const int G = p.Hq / p.Hkv, hblocks = G / HG;
    const int g = blockIdx.y / hblocks, hb = blockIdx.y % hblocks;
    const int b = blockIdx.z;
    const int64_t L = p.cache_len[b];
    if (s == 0 && blockIdx.y == 0 && threadIdx.x == 0) p.ws_len[b] = (int32_t)L;
    if (L < 0 || L > p.max_len) return;

    const int64_t crow = ((int64_t)b * p.Hkv + g) * p.cap * D;
    const E* knew = (const E*)p.k_new + ((int64_t)b * p.Hkv + g) * D;
    const E* vnew = (const E*)p.v_new + ((int64_t)b * p.Hkv + g) * D;
    if (s == 0 && hb == 0) {
        // append the new base token's K/V at slot L (nobody reads slot L from
        // the cache in this launch: readers take key L from k_new / v_new)
        for (int d = threadIdx.x; d < D; d += blockDim.x) {
            ((E*)p.k_cache)[crow + L * D + d] = knew[d];
            ((E*)p.v_cache)[crow + L * D + d] = vnew[d];
        }
    }
    const int64_t lo = (int64_t)s * p.chunk;
    if (lo > L) return;
    const int64_t hi = lo + p.chunk - 1 < L ? lo + p.chunk - 1 : L;
    const int h0 = g * G + hb * HG;
    load_queries<E, D, HG>(qs[0], (const E*)p.q_out, (const E*)p.alpha_out, (const E*)p.beta_out,
                           (int64_t)b * p.Hq * D, h0, p.qscale);
    load_queries<E, D, HG>(qs[1], (const E*)p.q, (const E*)p.alpha, (const E*)p.beta,
                           (int64_t)b * p.Hq * D, h0, p.qscale);
    __syncthreads();
    const int64_t kind_stride = (int64_t)p.n_split * (D + 2);
    const int64_t head_stride = 2 * kind_stride;
    float* out = p.ws_part + ((int64_t)b * p.Hq + h0) * head_stride + (int64_t)s * (D + 2);
    // the output copy: whole history [0, L]
    attend_chunk<E, D, HG>(qs[0], (const E*)p.k_cache + crow, (const E*)p.v_cache + crow, L, knew, vnew,
                           lo, hi, red, out, head_stride);
    // the base token: its window [L - w + 1, L]
    const int64_t wlo = L - p.window + 1 > lo ? L - p.window + 1 : lo;
    if (wlo <= hi)
        attend_chunk<E, D, HG>(qs[1], (const E*)p.k_cache + crow, (const E*)p.v_cache + crow, L, knew,
                               vnew, wlo, hi, red, out + kind_stride, head_stride);
}

// --------------------------------------------- decode: short steps, fused

// Device-scope 16-byte load / store of a partial record quad (sc1: written
// through to, and read from, the level every XCD shares).
__device__ __forceinline__ f32x4 rec_ld(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicySc1));
}
__device__ __forceinline__ void rec_st(f32x4 v, rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kCachePolicySc1);
}

// Maximum and sum over the whole wave, every lane given the result (DPP
// inside rows of 16 lanes, then row broadcasts into lane 63; fixed order).
__device__ __forceinline__ float wave_max(float x)
{
    x = fmaxf(x, dpp_mov<kDppXor1>(x));
    x = fmaxf(x, dpp_mov<kDppXor2>(x));
    x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
    x = fmaxf(x, dpp_mov<kDppMirror>(x));
    return wave_max_of_rows(x);
}
__device__ __forceinline__ float wave_sum(float x)
{
    constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
    x = group_sum<16>(x);
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kRowBcast15, 0xa, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kRowBcast31, 0xc, 0xf, false));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// The merge of a whole head block by one workgroup, from records of D + 4
// floats (max, sum, 0, 0, weighted values) read at device scope.  A head's
// (kind, split) records -- the copy's splits 0 .. s1, then the base token's
// sw0 .. s1, at most 64 -- are indexed k = 0 .. np - 1.  Each of the head's
// W = 4 / HG waves loads every header in one instruction (lane k: record
// k), takes the per-kind maximum and the weights f_k = 2^(max_k - max) by
// wave reductions, and so the denominators; the values are then dealt
// round-robin to the head's groups of D / 4 threads (one 4-value quad
// each), which issue all their loads of a round at once (one memory round
// trip for up to NG RB records) and accumulate f_k-weighted sums with no
// rescaling.  The groups' sums combine in a fixed order (shuffles within a
// wave, LDS across waves), so the result is run-to-run identical.  Every
// thread of the workgroup takes part; with W > 1 there is a barrier.
// `scratch` is LDS for 8 D + 4 x 130 floats.
template <int D, int HG>
__device__ __forceinline__ void merge_block(rsrc_t part, uint32_t head_bytes, uint32_t kind_bytes, int sw0, int s1,
                                            uint16_t* o_out, uint16_t* o, int64_t row0, float* scratch)
{
    constexpr int TPR = D / 4;                   // threads per record
    constexpr int NGW = 64 / TPR;                // groups per wave
    constexpr int W = 4 / HG;                    // waves per head
    constexpr int NG = NGW * W;                  // groups per head
    constexpr int RB = (36 + NG - 1) / NG;       // records per group and round
    constexpr int REC = D + 4;
    static_assert(HG * W == 4 && NGW >= 2, "thread layout");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int hh = wv / W, grp = (wv % W) * NGW + lane / TPR, qd = lane % TPR;
    const int n0 = s1 + 1, np = n0 + (s1 - sw0 + 1);   // the copy's records, then the base token's
    const uint32_t hbase = hh * head_bytes;
    auto rec_off = [&](int k) {
        const int kind = k >= n0, sk = kind ? sw0 + k - n0 : k;
        return hbase + (kind ? kind_bytes : 0u) + (uint32_t)sk * (REC * 4);
    };
    // headers: lane k holds record k's (max, sum); per-kind maxima and sums
    const f32x4 h4 = rec_ld(part, rec_off(lane < np ? lane : np - 1));
    const bool own = lane < np, hk = lane >= n0;
    const float m0 = wave_max(own && !hk ? h4[0] : kNegBig), m1 = wave_max(own && hk ? h4[0] : kNegBig);
    const float f = own ? fast_exp2(h4[0] - (hk ? m1 : m0)) : 0.f;
    const float d0 = wave_sum(hk ? 0.f : f * h4[1]), d1 = wave_sum(hk ? f * h4[1] : 0.f);
    // the weights per kind, [k][kind] in this wave's LDS slot (k = 64: zero),
    // so the value loop needs no per-record lane masks (a wave reads back
    // its own writes in order: no barrier)
    float2* wts = reinterpret_cast<float2*>(scratch + 8 * D) + wv * 65;
    wts[lane] = float2{hk ? 0.f : f, hk ? f : 0.f};
    if (lane == 0) wts[64] = float2{0.f, 0.f};
    // values: group grp takes records grp, grp + NG, ...
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 a0 = zero, a1 = zero;
    for (int p0 = grp; p0 < np; p0 += NG * RB) {
        f32x4 v[RB];
#pragma unroll
        for (int k = 0; k < RB; ++k) v[k] = rec_ld(part, rec_off(min(p0 + NG * k, np - 1)) + 16 + 16 * qd);
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const float2 w = wts[min(p0 + NG * k, 64)];
            a0 += w.x * v[k];
            a1 += w.y * v[k];
        }
    }
    // the groups' sums in a fixed order: lanes 0..31 end with the copy's,
    // 32..63 with the base token's (the swap hands each half the other's)
    if constexpr (TPR == 16)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a0[e] += __shfl_xor(a0[e], 16);
            a1[e] += __shfl_xor(a1[e], 16);
        }
    f32x4 t;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0[e]), __float_as_uint(a1[e]), false, false);
        t[e] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const int kind = lane >> 5;                  // the lanes (lane & 31) < TPR finish quad qd of this kind
    if constexpr (W > 1) {
        auto at = [&](int j) { return scratch + (((hh * W + j) * 2 + kind) * TPR + qd) * 4; };   // [head][wave][kind][quad]
        if ((lane & 31) < TPR) *(f32x4*)at(wv % W) = t;
        __syncthreads();
        if (wv % W == 0) {
            t = *(const f32x4*)at(0);
            for (int j = 1; j < W; ++j) t += *(const f32x4*)at(j);
        }
    }
    if (wv % W == 0 && (lane & 31) < TPR) {
        const float inv = 1.f / (kind ? d1 : d0);
        uint16_t* out = kind ? o : o_out;
        const int64_t row = row0 + (int64_t)hh * D + 4 * qd;
        *(u32x2*)(out + row) = u32x2{pack_bf16x2(t[0] * inv, t[1] * inv), pack_bf16x2(t[2] * inv, t[3] * inv)};
    }
}

// One launch per decode step when the histories are short (bf16, at most
// kDecodeShortMaxSplits chunks of kDecodeShortChunk = 128 keys): the step is
// then a few serial memory round trips long, so the work of a chunk is laid
// out for latency.  A workgroup takes chunk s of one KV head's HG-head block
// of sequence b; wave w takes the chunk's w-th run of kDecodeShortChunk / 128
// 32-key pairs:
//   - its pairs' K and V rows go straight into the wave's own LDS region by
//     direct buffer-to-LDS loads in the pair layout of the streaming kernels
//     (keys past L land as zeros), issued together with the query rows, and
//     the new token's key L is then written over its slot there from
//     k_new / v_new, and the wave of the first head block stores that row
//     into cache slot L (the append);
//   - S^T = K Q^T and O^T = V^T P^T run on v_mfma_f32_16x16x32_bf16 with
//     the copy's HG heads as query columns 0..HG-1 and the base token's as
//     columns HG..2HG-1 (live when the chunk holds keys of its window;
//     keys below the window are masked in those columns); V^T comes from the
//     transposing LDS read; the row sums from an all-ones MFMA;
//   - the 4 waves' states merge through LDS (in a fixed order) into one
//     partial record per (head, kind), D + 4 floats (max, sum, 0, 0,
//     weighted values), stored at device scope in 16-byte quads.
// The workgroup then counts itself in on the block's counter; the last of
// the block's n_split workgroups to arrive counts the block in on the
// sequence's counter (at once, its result read later) and merges the block
// into o_out and o, and the last block of the sequence to arrive then
// advances cache_len[b].  Every workgroup of the grid arrives, those past the history
// too, so cache_len[b] changes only once every workgroup of sequence b has
// read it.  The counters live at the start of the workspace, start at zero
// and are left at zero.
template <int D, int HG>
__global__ __launch_bounds__(256) void decode_short_kernel(DecodeParams p)
{
    using R = PairTile<D>;
    constexpr int NQ = D / 32, ND = D / 16;
    constexpr int NH = 2 * HG;                 // live query columns
    constexpr int PPW = kDecodeShortChunk / 128;   // 32-key pairs per wave
    constexpr int KJ = R::KPART * 2 / 16 / 64; // direct loads per lane for a pair's K (and for its V)
    constexpr int CPR = D / 8;                 // 16-byte chunks of a row
    static_assert(PPW >= 1 && kDecodeShortChunk == 128 * PPW, "chunk of whole pairs per wave");
    static_assert(4 * NH * (D + 2) * 4 <= 4 * PPW * R::SLOT * 2, "the wave combine fits in the pair regions");
    __shared__ __align__(16) uint16_t lds[4 * PPW * R::SLOT];   // the waves' pairs, then the wave combine
    __shared__ int last;
    float (*red)[NH][D + 2] = reinterpret_cast<float (*)[NH][D + 2]>(lds);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;
    const int s = blockIdx.x;
    const int G = p.Hq / p.Hkv, hblocks = G / HG;
    const int nblk = p.Hkv * hblocks;
    const int g = blockIdx.y / hblocks, hb = blockIdx.y % hblocks;
    const int b = blockIdx.z;
    const int64_t L = p.cache_len[b];
    const int h0 = g * G + hb * HG;
    if (L < 0 || L > p.max_len) {
        // a length outside [0, max_len]: NaN outputs, nothing else touched
        if (s == 0)
            for (int idx = tid; idx < HG * D; idx += 256) {
                const int64_t o = ((int64_t)b * p.Hq + h0) * D + idx;
                st_elem((uint16_t*)p.o_out, o, __builtin_nanf(""));
                st_elem((uint16_t*)p.o, o, __builtin_nanf(""));
            }
        return;
    }
    const int64_t crow = ((int64_t)b * p.Hkv + g) * p.cap * D;
    const uint16_t* knew = (const uint16_t*)p.k_new + ((int64_t)b * p.Hkv + g) * D;
    const uint16_t* vnew = (const uint16_t*)p.v_new + ((int64_t)b * p.Hkv + g) * D;
    const int64_t lo = (int64_t)s * kDecodeShortChunk;
    const int64_t wlo = L - p.window + 1 > 0 ? L - p.window + 1 : 0;
    // record offsets in bytes (the head block's records span less than 4 GB)
    const uint32_t kind_bytes = (uint32_t)p.n_split * ((D + 4) * 4), head_bytes = 2 * kind_bytes;
    // this head block's records, through a buffer resource (device-scope 16-byte accesses)
    const rsrc_t prs = make_rsrc(p.ws_part + ((int64_t)b * p.Hq + h0) * (head_bytes / 4), (int64_t)HG * head_bytes);
    const bool any = lo <= L;                                    // the chunk holds keys of the history
    const bool win = any && lo + kDecodeShortChunk - 1 >= wlo;    // ... and of the base token's window
    if (any) {
        // wave wv takes pairs PPW wv .. PPW wv + PPW - 1 of the chunk
        const int64_t kw0 = lo + 32 * PPW * wv;
        const bool mine = kw0 <= L;                              // wave-uniform
        const bool hasL = mine && L - kw0 < 32 * PPW;
        uint16_t* slots = lds + wv * PPW * R::SLOT;
        if (mine) {
            // the pairs' rows through key L (the buffer range ends there, so
            // later keys land as zeros), unit u = 64 j + lane of each part
            const int64_t avail = (L - kw0 + 1) * D * 2;
            const i32x4 rk = buffer_words((const uint16_t*)p.k_cache + crow + kw0 * D, avail);
            const i32x4 rv = buffer_words((const uint16_t*)p.v_cache + crow + kw0 * D, avail);
#pragma unroll
            for (int pp = 0; pp < PPW; ++pp) {
#pragma unroll
                for (int j = 0; j < KJ; ++j) {
                    int r, c;
                    R::k_unit(64 * j + lane, r, c);
                    load_lds16_nt(rk, (uint32_t)(((32 * pp + r) * D + 8 * c) * 2), 0, slots + pp * R::SLOT + 64 * j * 8);
                }
#pragma unroll
                for (int j = 0; j < KJ; ++j) {
                    int r, c;
                    R::v_unit(64 * j + lane, r, c);
                    load_lds16_nt(rv, (uint32_t)(((32 * pp + r) * D + 8 * c) * 2), 0,
                                  slots + pp * R::SLOT + R::KPART + 64 * j * 8);
                }
            }
        }
        // the new token's row chunks (lanes 0 .. 2 CPR - 1: K, then V)
        u32x4 nrow = {0u, 0u, 0u, 0u};
        if (hasL && lane < 2 * CPR) nrow = *(const u32x4*)(lane < CPR ? knew + 8 * lane : vnew + 8 * (lane - CPR));
        // the query rows: lane (n, gq) holds column n, dims 32 i + 8 gq .. + 7
        const bool base = n >= HG;
        const bool live = n < HG || (n < NH && win);
        const int h = h0 + (base ? n - HG : n);
        u32x4 qw[NQ], aw[NQ], bw[NQ];
        if (live) {
            const uint16_t* q = (const uint16_t*)(base ? p.q : p.q_out) + ((int64_t)b * p.Hq + h) * D + 8 * gq;
            const uint16_t* al = (const uint16_t*)(base ? p.alpha : p.alpha_out) + (int64_t)h * D + 8 * gq;
            const uint16_t* be = (const uint16_t*)(base ? p.beta : p.beta_out) + (int64_t)h * D + 8 * gq;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                qw[i] = *(const u32x4*)(q + 32 * i);
                aw[i] = *(const u32x4*)(al + 32 * i);
                bw[i] = *(const u32x4*)(be + 32 * i);
            }
        }
        wait_vmcnt<0>();
        if (hasL && lane < 2 * CPR) {
            const int r = (int)(L - kw0);
            uint16_t* sl = slots + (r >> 5) * R::SLOT;
            uint16_t* dst = lane < CPR ? sl + R::kofs(r & 31, lane) : sl + R::KPART + R::vofs16(r & 31, lane - CPR);
            *(u32x4*)dst = nrow;
            // the append: the new token's K/V row into cache slot L, once per
            // KV head (this launch reads key L from k_new / v_new only)
            if (hb == 0) {
                uint16_t* cache = (uint16_t*)(lane < CPR ? p.k_cache : p.v_cache);
                *(u32x4*)(cache + crow + L * D + 8 * (lane < CPR ? lane : lane - CPR)) = nrow;
            }
        }
        // scale-offset queries in exp2 units as the B operand (zero columns past the live ones)
        bf16x8 qf[NQ];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            u32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = qw[i][e], a = aw[i][e], bb = bw[i][e];
                r[e] = live ? pack_bf16x2(__builtin_fmaf(bf16_lo(w), bf16_lo(a), bf16_lo(bb)) * p.qscale,
                                          __builtin_fmaf(bf16_hi(w), bf16_hi(a), bf16_hi(bb)) * p.qscale)
                            : 0u;
            }
            qf[i] = __builtin_bit_cast(bf16x8, r);
        }
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 oacc[ND];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) oacc[dt] = zero;
        f32x4 lacc = zero;
        float m = kNegBig;
        if (mine) {
            __builtin_amdgcn_s_waitcnt(0xC07F);                  // lgkmcnt(0): key L's slot rewritten
            // S^T per pair: sc[pp][0][r]: key 32 pp + 4 gq + r, sc[pp][1][r]:
            // key 32 pp + 16 + 4 gq + r (from kw0, column n); admissible:
            // <= L, and for the base token's columns >= wlo
            f32x4 sc[PPW][2];
            float mx = -INFINITY;
#pragma unroll
            for (int pp = 0; pp < PPW; ++pp) {
                const uint16_t* kb0 = slots + pp * R::SLOT + R::kofs(n, gq);
                const uint16_t* kb1 = slots + pp * R::SLOT + R::kofs(n, 4 + gq);
                sc[pp][0] = zero;
                sc[pp][1] = zero;
#pragma unroll
                for (int i = 0; i < NQ; ++i) {
                    const uint16_t* kb = ((i & 1) ? kb1 : kb0) + (i >> 1) * R::K_STEP2;
                    const bf16x8 k0 = *(const bf16x8*)kb;
                    const bf16x8 k1 = *(const bf16x8*)(kb + R::K_KEY16);
                    sc[pp][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[i], sc[pp][0], 0, 0, 0);
                    sc[pp][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[i], sc[pp][1], 0, 0, 0);
                }
                const int64_t key0 = kw0 + 32 * pp;
                const int hi_off = (int)(L - key0 < 64 ? (L - key0 > -64 ? L - key0 : -64) : 64) - 4 * gq;
                const int lo_off =
                    (base ? (int)(wlo - key0 > -64 ? (wlo - key0 < 64 ? wlo - key0 : 64) : -64) : -64) - 4 * gq;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (r > hi_off || r < lo_off) sc[pp][0][r] = -INFINITY;
                    if (16 + r > hi_off || 16 + r < lo_off) sc[pp][1][r] = -INFINITY;
                    mx = fmaxf(mx, fmaxf(sc[pp][0][r], sc[pp][1][r]));
                }
            }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            m = fmaxf(mx, kNegBig);
            const bf16x8 kOnes = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
#pragma unroll
            for (int pp = 0; pp < PPW; ++pp) {
                const f32x4 s0 = sc[pp][0], s1 = sc[pp][1];
                const u32x4 pw4 = {pack_bf16x2(fast_exp2(s0[0] - m), fast_exp2(s0[1] - m)),
                                   pack_bf16x2(fast_exp2(s0[2] - m), fast_exp2(s0[3] - m)),
                                   pack_bf16x2(fast_exp2(s1[0] - m), fast_exp2(s1[1] - m)),
                                   pack_bf16x2(fast_exp2(s1[2] - m), fast_exp2(s1[3] - m))};
                const bf16x8 pb = __builtin_bit_cast(bf16x8, pw4);
                lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes, pb, lacc, 0, 0, 0);
                // V^T operands: this lane addresses key rows 4 gq + (n >> 2) and
                // 16 + 4 gq + (n >> 2), dims 16 dt + 4 (n & 3)
                const uint16_t* vb = slots + pp * R::SLOT + R::KPART + R::vofs_tr(4 * gq + (n >> 2), 0, n & 3);
#pragma unroll
                for (int dt = 0; dt < ND; ++dt) {
                    const s16x4 v0 = lds_read_tr(vb + dt * R::V_DT);
                    const s16x4 v1 = lds_read_tr(vb + R::V_KEY16 + dt * R::V_DT);
                    const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
                    oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, oacc[dt], 0, 0, 0);
                }
            }
        }
        __syncthreads();                                         // every wave is done with its pair region
        if (n < NH) {
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[wv][n][2 + 16 * dt + 4 * gq + r] = oacc[dt][r];
            if (gq == 0) {
                red[wv][n][0] = m;
                red[wv][n][1] = lacc[0];
            }
        }
        __syncthreads();
        // the 4 waves in a fixed order; one record per (head, kind) of
        // D + 4 floats (max, sum, 0, 0, weighted values), stored at device
        // scope one 16-byte quad at a time
        const int nr = win ? NH : HG;
        constexpr int NQD = D / 4 + 1;
        for (int idx = tid; idx < nr * NQD; idx += 256) {
            const int r = idx / NQD, qd = idx % NQD;          // column r; qd == 0: the (max, sum) header
            float M = red[0][r][0];
#pragma unroll
            for (int w = 1; w < 4; ++w) M = fmaxf(M, red[w][r][0]);
            float f[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) f[w] = fast_exp2(red[w][r][0] - M);
            f32x4 q4 = zero;
            if (qd == 0) {
                float l = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) l += f[w] * red[w][r][1];
                q4[0] = M;
                q4[1] = l;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float x = 0.f;
#pragma unroll
                    for (int w = 0; w < 4; ++w) x += f[w] * red[w][r][2 + 4 * (qd - 1) + e];
                    q4[e] = x;
                }
            }
            const uint32_t off = (r % HG) * head_bytes + (r >= HG ? kind_bytes : 0u) + (uint32_t)s * ((D + 4) * 4) + 16 * qd;
            rec_st(q4, prs, off);
        }
    }
    // count in once this workgroup's records are written at device scope:
    // the device-scope stores have completed (vmcnt) before the barrier, and
    // the counter moves after it.  No cache-wide fence: the records bypass
    // the non-coherent caches on both sides (device-scope stores here,
    // device-scope loads in the merge).
    wait_vmcnt<0>();
    __syncthreads();
    int* blk_cnt = p.ws_cnt + (int64_t)b * nblk + blockIdx.y;
    int* seq_cnt = p.ws_cnt + (int64_t)p.B * nblk + b;
    int ns = 0;
    if (tid == 0) {
        last = atomicAdd(blk_cnt, 1) == p.n_split - 1;
        // the block's last arrival counts the block in on the sequence's
        // counter at once; the count is read after the merge
        if (last) ns = atomicAdd(seq_cnt, 1) + 1;
    }
    __syncthreads();
    if (!last) return;
    static_assert((8 * D + 4 * 130) * 4 <= 4 * PPW * R::SLOT * 2, "the merge's LDS fits in the pair regions");
    merge_block<D, HG>(prs, head_bytes, kind_bytes, (int)(wlo / kDecodeShortChunk), (int)(L / kDecodeShortChunk),
                       (uint16_t*)p.o_out, (uint16_t*)p.o, ((int64_t)b * p.Hq + h0) * D, reinterpret_cast<float*>(lds));
    if (tid == 0) {
        __hip_atomic_store(blk_cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (ns == nblk) {
            // every block's workgroups have arrived, so all have read L
            // (cache_len[b] is not read by the merges)
            __hip_atomic_store(seq_cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            p.cache_len[b] = (int32_t)(L + 1);
        }
    }
}

// ------------------------------------------------ many copies: general form

// One workgroup per (copy, KV group block, sequence): the copy's HG heads
// attend over keys [0, pos] with the chunk worker, whose one partial stays
// in LDS and is normalised in place.  A position outside [0, T) gives NaN.
template <typename E, int D, int HG>
__global__ __launch_bounds__(256) void copies_simple_kernel(CopiesParams p)
{
    __shared__ float qs[HG][D];
    __shared__ float red[4][HG][D + 2];
    __shared__ float part[HG][D + 2];
    const int64_t i = blockIdx.x;
    const int G = p.Hq / p.Hkv, hblocks = G / HG;
    const int g = blockIdx.y / hblocks, hb = blockIdx.y % hblocks;
    const int b = blockIdx.z;
    const int h0 = g * G + hb * HG;
    const int64_t row = ((int64_t)b * p.T_out + i) * p.Hq * D;     // copy i's query / output row
    const int64_t P = p.pos[(int64_t)b * p.T_out + i];
    if (P < 0 || P >= p.T) {
        for (int idx = threadIdx.x; idx < HG * D; idx += blockDim.x)
            st_elem((E*)p.o_out, row + (int64_t)h0 * D + idx, __builtin_nanf(""));
        return;
    }
    load_queries<E, D, HG>(qs, (const E*)p.q_out, (const E*)p.alpha_out, (const E*)p.beta_out, row, h0,
                           p.qscale);
    __syncthreads();
    const int64_t crow = ((int64_t)b * p.Hkv + g) * p.cap * D;
    attend_chunk<E, D, HG>(qs, (const E*)p.k_cache + crow, (const E*)p.v_cache + crow, -1, nullptr, nullptr, 0, P,
                           red, &part[0][0], D + 2);
    for (int idx = threadIdx.x; idx < HG * D; idx += blockDim.x) {
        const int hh = idx / D, d = idx % D;
        st_elem((E*)p.o_out, row + (int64_t)(h0 + hh) * D + d, part[hh][2 + d] / part[hh][1]);
    }
}

// One workgroup (256 threads) per (sequence, query head): the merge of its
// splits that hold keys of the query's range.  kinds = 1: the copy only
// (prefill); kinds = 2: the copy, then the base token (decode), which also
// advances cache_len.
template <typename E, int D>
__global__ __launch_bounds__(256) void merge_kernel(const float* ws_part, const int32_t* ws_len,
                                                    int32_t* cache_len, int64_t max_len, int window,
                                                    int Hq, int chunk, int n_split, int rec,
                                                    int kinds, E* o_out, E* o)
{
    const int tid = threadIdx.x;
    const int b = blockIdx.x / Hq, h = blockIdx.x % Hq;
    const int64_t L = ws_len[b];
    const int64_t kind_stride = (int64_t)n_split * rec;
    const float* part = ws_part + ((int64_t)b * Hq + h) * kinds * kind_stride;
    const int64_t row = ((int64_t)b * Hq + h) * D;
    if (L < 0 || L > max_len) {
        for (int d = tid; d < D; d += 256) {
            st_elem(o_out, row + d, __builtin_nanf(""));
            if (kinds == 2) st_elem(o, row + d, __builtin_nanf(""));
        }
        return;
    }
    for (int kind = 0; kind < kinds; ++kind) {
        const int64_t lo = kind == 0 ? 0 : (L - window + 1 > 0 ? L - window + 1 : 0);
        merge_splits<E, D>(part + kind * kind_stride, rec, rec - D, (int)(lo / chunk), (int)(L / chunk),
                           kind == 0 ? o_out : o, row);
    }
    if (cache_len && h == 0 && tid == 0) cache_len[b] = (int32_t)(L + 1);
}

// The LDS-streamed kernel's records in prefill: one workgroup per
// (sequence, query head) merges the record ids its stream's range lists
// (ws_rng: first, -, last) -- records [id][1][4 head slots, the block's hg
// used][rec] -- into o_out.
template <int D>
__global__ __launch_bounds__(256) void lds_merge_kernel(const float* ws_part, const int32_t* ws_rng,
                                                        const int32_t* ws_len, int64_t max_len, int Hq, int G,
                                                        int rec, uint16_t* o_out)
{
    const int tid = threadIdx.x;
    const int b = blockIdx.x / Hq, h = blockIdx.x % Hq;
    const int64_t L = ws_len[b];
    const int64_t row = ((int64_t)b * Hq + h) * D;
    if (L < 0 || L > max_len) {
        for (int d = tid; d < D; d += 256) st_elem(o_out, row + d, __builtin_nanf(""));
        return;
    }
    const int hg = xattn_heads_per_wg(G), hblocks = G / hg, S = (Hq / G) * hblocks;
    const int j = (h / G) * hblocks + (h % G) / hg;         // the head's stream: KV head, head block
    const int32_t* rg = ws_rng + ((int64_t)b * S + j) * 3;
    merge_splits<uint16_t, D>(ws_part + (h % G) % hg * rec, (int64_t)4 * rec, rec - D, rg[0], rg[2], o_out, row);
}

// The decode step's merge after the LDS-streamed kernel, which read the
// history 0 .. L - 1: one workgroup per (sequence, query head) merges its
// stream's records of both kinds (the copy's over the whole history, the
// base token's over the segments holding its window) together with the new
// token's key L from k_new / v_new -- its score from the same bf16
// scale-offset query the streaming kernel used -- into o_out and o.  The
// workgroup of head 0 then appends the new token's K/V rows at slot L of
// every KV head of the sequence (nothing reads the cache after the
// streaming kernel) and advances cache_len[b].  A length outside
// [0, max_len] gives NaN outputs and touches nothing.
template <int D>
__global__ __launch_bounds__(256) void lds_decode_merge_kernel(DecodeParams p)
{
    __shared__ float wsum[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int b = blockIdx.x / p.Hq, h = blockIdx.x % p.Hq;
    const int64_t L = p.ws_len[b];
    const int64_t row = ((int64_t)b * p.Hq + h) * D;
    uint16_t* o_out = (uint16_t*)p.o_out;
    uint16_t* o = (uint16_t*)p.o;
    if (L < 0 || L > p.max_len) {
        for (int d = tid; d < D; d += 256) {
            st_elem(o_out, row + d, __builtin_nanf(""));
            st_elem(o, row + d, __builtin_nanf(""));
        }
        return;
    }
    const int G = p.Hq / p.Hkv, hg = xattn_heads_per_wg(G), hblocks = G / hg, S = p.Hkv * hblocks;
    const int g = h / G, j = g * hblocks + (h % G) / hg;     // the head's KV head and stream
    const uint16_t* knew = (const uint16_t*)p.k_new + ((int64_t)b * p.Hkv + g) * D;
    const uint16_t* vnew = (const uint16_t*)p.v_new + ((int64_t)b * p.Hkv + g) * D;
    // the new key's score per kind (thread kind * D + d takes dim d; kind 0
    // the copy's query, kind 1 the base token's), in exp2 units
    float part = 0.f;
    if (tid < 2 * D) {
        const int kind = tid / D, d = tid % D;
        const uint16_t* q = (const uint16_t*)(kind ? p.q : p.q_out) + row + d;
        const uint16_t* al = (const uint16_t*)(kind ? p.alpha : p.alpha_out) + (int64_t)h * D + d;
        const uint16_t* be = (const uint16_t*)(kind ? p.beta : p.beta_out) + (int64_t)h * D + d;
        const float qh = bf16_lo(pack_bf16x2(__builtin_fmaf(bf16_lo(*q), bf16_lo(*al), bf16_lo(*be)) * p.qscale, 0.f));
        part = qh * bf16_lo(knew[d]);
    }
    part = wave_sum(part);
    if (lane == 0) wsum[wv] = part;
    __syncthreads();
    constexpr int WPK = D / 64;                              // waves per kind
    float sk[2];
#pragma unroll
    for (int kind = 0; kind < 2; ++kind) {
        sk[kind] = wsum[kind * WPK];
#pragma unroll
        for (int w = 1; w < WPK; ++w) sk[kind] += wsum[kind * WPK + w];
    }
    const int32_t* rg = p.ws_rng + ((int64_t)b * S + j) * 3;
    const int64_t stride = (int64_t)2 * 4 * p.rec;
#pragma unroll
    for (int kind = 0; kind < 2; ++kind)
        merge_splits<uint16_t, D>(p.ws_part + ((int64_t)kind * 4 + (h % G) % hg) * p.rec, stride, p.rec - D,
                                  kind == 0 ? rg[0] : rg[1], rg[2], kind == 0 ? o_out : o, row, sk[kind], vnew);
    if (h == 0) {
        constexpr int UPR = D / 8;                           // 16-byte units per row
        const int units = p.Hkv * UPR;
        for (int u = tid; u < 2 * units; u += 256) {
            const bool isv = u >= units;
            const int uu = isv ? u - units : u;
            const int gg = uu / UPR, c = uu - gg * UPR;
            const int64_t kv = (int64_t)b * p.Hkv + gg;
            const u32x4 w = *((const u32x4*)((const uint16_t*)(isv ? p.v_new : p.k_new) + kv * D) + c);
            *((u32x4*)((uint16_t*)(isv ? p.v_cache : p.k_cache) + (kv * p.cap + L) * D) + c) = w;
        }
        if (tid == 0) p.cache_len[b] = (int32_t)(L + 1);
    }
}

template <typename E, int D, int HG>
hipError_t launch_xattn_t(const XattnParams& p, hipStream_t st)
{
    const int hblocks = (p.Hq / p.Hkv) / HG;
    for (int b0 = 0; b0 < p.B; b0 += kPosPerLaunch) {
        const int nb = p.B - b0 < kPosPerLaunch ? p.B - b0 : kPosPerLaunch;
        PosBlock pos;
        for (int i = 0; i < nb; ++i) pos.v[i] = p.pos[b0 + i];
        hipLaunchKernelGGL((xattn_split_kernel<E, D, HG>), dim3(p.n_split, p.Hkv * hblocks, nb), dim3(256),
                           0, st, p, b0, nb, pos);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    int64_t max_len = 0;
    for (int b = 0; b < p.B; ++b) max_len = p.pos[b] > max_len ? p.pos[b] : max_len;
    hipLaunchKernelGGL((merge_kernel<E, D>), dim3(p.B * p.Hq), dim3(256), 0, st, p.ws_part, p.ws_len,
                       (int32_t*)nullptr, max_len, 0, p.Hq, p.chunk, p.n_split, p.rec, 1, (E*)p.o_out,
                       (E*)nullptr);
    return hipGetLastError();
}

template <typename E, int D, int HG>
hipError_t launch_decode_t(const DecodeParams& p, hipStream_t st)
{
    const int hblocks = (p.Hq / p.Hkv) / HG;
    const dim3 grid(p.n_split, p.Hkv * hblocks, p.B);
    if constexpr (sizeof(E) == 2) {
        if (p.fused) {
            hipLaunchKernelGGL((decode_short_kernel<D, HG>), grid, dim3(256), 0, st, p);
            return hipGetLastError();
        }
    }
    if (p.fused) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_split_kernel<E, D, HG>), grid, dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_decode_merge(p, st);
}

template <typename E, int D>
hipError_t xattn_by_hg(const XattnParams& p, hipStream_t st)
{
    switch (xattn_heads_per_wg(p.Hq / p.Hkv)) {
    case 4: return launch_xattn_t<E, D, 4>(p, st);
    case 2: return launch_xattn_t<E, D, 2>(p, st);
    default: return launch_xattn_t<E, D, 1>(p, st);
    }
}

template <typename E, int D>
hipError_t decode_by_hg(const DecodeParams& p, hipStream_t st)
{
    switch (xattn_heads_per_wg(p.Hq / p.Hkv)) {
    case 4: return launch_decode_t<E, D, 4>(p, st);
    case 2: return launch_decode_t<E, D, 2>(p, st);
    default: return launch_decode_t<E, D, 1>(p, st);
    }
}

}  // namespace

hipError_t launch_xattn(const XattnParams& p, hipStream_t st)
{
    if (p.lds) return launch_xattn_lds(p, st);
    if (p.dt == Dt::F32) return p.D == 64 ? xattn_by_hg<float, 64>(p, st) : xattn_by_hg<float, 128>(p, st);
    return p.D == 64 ? xattn_by_hg<uint16_t, 64>(p, st) : xattn_by_hg<uint16_t, 128>(p, st);
}

template <typename E, int D>
hipError_t launch_copies_simple(const CopiesParams& p, hipStream_t st)
{
    const int G = p.Hq / p.Hkv, HG = xattn_heads_per_wg(G);
    const dim3 grid((unsigned)p.T_out, (unsigned)(p.Hkv * (G / HG)), (unsigned)p.B);
    if (HG == 4) hipLaunchKernelGGL((copies_simple_kernel<E, D, 4>), grid, dim3(256), 0, st, p);
    else if (HG == 2) hipLaunchKernelGGL((copies_simple_kernel<E, D, 2>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((copies_simple_kernel<E, D, 1>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_copies(const CopiesParams& p, hipStream_t st)
{
    if (copies_flash_applies(p)) return launch_copies_flash(p, st);
    if (p.dt == Dt::F32)
        return p.D == 64 ? launch_copies_simple<float, 64>(p, st) : launch_copies_simple<float, 128>(p, st);
    return p.D == 64 ? launch_copies_simple<uint16_t, 64>(p, st) : launch_copies_simple<uint16_t, 128>(p, st);
}

hipError_t launch_merge(const XattnParams& p, hipStream_t st)
{
    int64_t max_len = 0;
    for (int b = 0; b < p.B; ++b) max_len = p.pos[b] > max_len ? p.pos[b] : max_len;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(p.B * p.Hq), dim3(256), 0, st, p.ws_part, p.ws_len, (int32_t*)nullptr,
                           max_len, 0, p.Hq, p.chunk, p.n_split, p.rec, 1, (uint16_t*)p.o_out,
                           (uint16_t*)nullptr);
    };
    if (p.D == 64) go(merge_kernel<uint16_t, 64>);
    else go(merge_kernel<uint16_t, 128>);
    return hipGetLastError();
}

hipError_t launch_lds_merge(const XattnParams& p, hipStream_t st)
{
    int64_t max_len = 0;
    for (int b = 0; b < p.B; ++b) max_len = p.pos[b] > max_len ? p.pos[b] : max_len;
    if (p.D == 64)
        hipLaunchKernelGGL((lds_merge_kernel<64>), dim3(p.B * p.Hq), dim3(256), 0, st, p.ws_part, p.ws_rng, p.ws_len,
                           max_len, p.Hq, p.Hq / p.Hkv, p.rec, (uint16_t*)p.o_out);
    else
        hipLaunchKernelGGL((lds_merge_kernel<128>), dim3(p.B * p.Hq), dim3(256), 0, st, p.ws_part, p.ws_rng, p.ws_len,
                           max_len, p.Hq, p.Hq / p.Hkv, p.rec, (uint16_t*)p.o_out);
    return hipGetLastError();
}

hipError_t launch_lds_merge(const DecodeParams& p, hipStream_t st)
{
    if (p.dt != Dt::BF16 || (p.D != 64 && p.D != 128)) return hipErrorInvalidValue;
    if (p.D == 64) hipLaunchKernelGGL((lds_decode_merge_kernel<64>), dim3(p.B * p.Hq), dim3(256), 0, st, p);
    else hipLaunchKernelGGL((lds_decode_merge_kernel<128>), dim3(p.B * p.Hq), dim3(256), 0, st, p);
    return hipGetLastError();
}

template <typename E, int D>
void decode_merge_t(const DecodeParams& p, hipStream_t st)
{
    hipLaunchKernelGGL((merge_kernel<E, D>), dim3(p.B * p.Hq), dim3(256), 0, st, p.ws_part, p.ws_len, p.cache_len,
                       p.max_len, p.window, p.Hq, p.chunk, p.n_split, p.rec, 2, (E*)p.o_out, (E*)p.o);
}

hipError_t launch_decode_merge(const DecodeParams& p, hipStream_t st)
{
    if (p.dt == Dt::F32) {
        if (p.D == 64) decode_merge_t<float, 64>(p, st);
        else decode_merge_t<float, 128>(p, st);
    } else {
        if (p.D == 64) decode_merge_t<uint16_t, 64>(p, st);
        else decode_merge_t<uint16_t, 128>(p, st);
    }
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t st)
{
    if (p.lds) return launch_decode_lds(p, st);
    if (p.dt == Dt::F32) return p.D == 64 ? decode_by_hg<float, 64>(p, st) : decode_by_hg<float, 128>(p, st);
    return p.D == 64 ? decode_by_hg<uint16_t, 64>(p, st) : decode_by_hg<uint16_t, 128>(p, st);
}

}  // namespace orthros
