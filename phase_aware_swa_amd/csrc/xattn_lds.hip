// xattn_lds.hip -- the output copy's full-history cross-attention in prefill
// for bf16 and groups of 4 query heads per KV head, for gfx950: the cache
// streams through LDS by direct loads and the contractions run on MFMA.
//
// "Orthros:阶段感知异构注意力精读笔记" §2.3 Eq. (5): the copy at original
// position P attends over every cached key j <= P (§2.4: the mask follows the
// original position); its query is q_out * alpha_out + beta_out (§2.2).
//
// One query per head over the whole cache is a pure stream of K/V bytes
// (about 2 flop per byte per head), so the design is about keeping HBM busy:
//   - the keys of one (sequence, KV head) are cut into chunks (split-K); a
//     workgroup owns one chunk and serves the 4 query heads of a 4-head
//     block at once, so every K/V byte is read from HBM once;
//   - the chunk streams through two 64 KB LDS slots in stages of 4 (d = 128)
//     or 8 (d = 64) 32-key pairs, by buffer loads that write LDS directly
//     (16 per lane per stage, no register staging): while one stage is
//     consumed the next is in flight, one barrier per stage.  The LDS holds
//     one workgroup per CU, which is what the streaming needs;
//   - each load instruction fills 1 KB of a slot in lane order, so each lane
//     fetches the cache chunk that belongs at its 16-byte unit of the pair
//     layout (PairTile's inverse maps); the stage's buffer range ends at the
//     chunk's last key, so keys past it land as zeros;
//   - wave w consumes the stage's pairs w (and 4 + w at d = 64):
//     S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 with the 4
//     heads' queries as columns 0..3 of the B operand (the other 12 are
//     zero: the MFMAs are idle most of the time either way), V^T from the
//     transposing LDS read, online softmax in exp2 units with a lazy rescale;
//   - the 4 waves' states merge through LDS into one (max, sum, weighted sum
//     of values) partial per head, in the layout the LSE merge reads.

#include "device.h"
#include "kernels.h"
#include "pair_tile.h"

namespace orthros {
namespace {

constexpr int kStageBytes = 65536;                 // one LDS slot
constexpr int kLoads = kStageBytes / (256 * 16);   // direct loads per lane per stage
constexpr float kMargin = 8.0f;                    // lazy-rescale margin, log2 units

template <int D>
__global__ __launch_bounds__(256) void xattn_lds_kernel(XattnParams p, int b0, PosBlock pos)
{
    using R = PairTile<D>;
    constexpr int PPW = 128 / D;          // pairs per wave per stage
    constexpr int SK = 128 * PPW;         // keys per stage
    constexpr int PAIRB = 32 * D * 2;     // bytes of one pair's K (or V) rows in the cache
    constexpr int JP = D / 32;            // loads per lane per pair: JH of K, then JH of V
    constexpr int JH = JP / 2;
    constexpr int NQ = D / 32, ND = D / 16;
    constexpr int SLOTE = kStageBytes / 2;  // slot size in bf16 elements
    static_assert(4 * PPW * JP == kLoads && 4 * PPW * R::SLOT == SLOTE, "stage shape");
    __shared__ __align__(16) uint16_t lds[2 * SLOTE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;
    const int s = blockIdx.x;
    const int hblocks = (p.Hq / p.Hkv) / 4;
    const int g = blockIdx.y / hblocks, hb = blockIdx.y % hblocks;
    const int bi = blockIdx.z, b = b0 + bi;
    const int64_t P = pos.v[bi];
    if (s == 0 && blockIdx.y == 0 && tid == 0) p.ws_len[b] = (int32_t)P;
    const int64_t lo = (int64_t)s * p.chunk;
    if (lo > P) return;
    const int64_t hi = lo + p.chunk - 1 < P ? lo + p.chunk - 1 : P;
    const int nst = (int)((hi - lo) / SK) + 1;
    const int h0 = g * (p.Hq / p.Hkv) + hb * 4;

    const int64_t crow = ((int64_t)b * p.Hkv + g) * p.cap * D;
    const uint16_t* kc = (const uint16_t*)p.k_cache + crow;
    const uint16_t* vc = (const uint16_t*)p.v_cache + crow;

    // byte offset, inside one pair's rows, of the chunk this lane fetches for
    // the 16-byte unit 256 jj + 64 wv + lane of the pair's K and V parts
    uint32_t koff[JH], voff[JH];
#pragma unroll
    for (int jj = 0; jj < JH; ++jj) {
        int r, c;
        R::k_unit(256 * jj + 64 * wv + lane, r, c);
        koff[jj] = (uint32_t)((r * D + 8 * c) * 2);
        R::v_unit(256 * jj + 64 * wv + lane, r, c);
        voff[jj] = (uint32_t)((r * D + 8 * c) * 2);
    }
    // stage st -> slot st & 1: load j of wave wv fills units 256 j + 64 wv ..
    // + 63 of the slot, i.e. part (j % JP) of pair j / JP
    auto issue = [&](int st) {
        const int64_t k0 = lo + (int64_t)st * SK;
        const int64_t avail = (hi - k0 + 1) * D * 2;
        const i32x4 rk = buffer_words(kc + k0 * D, avail);
        const i32x4 rv = buffer_words(vc + k0 * D, avail);
        const uint16_t* dst = lds + (st & 1) * SLOTE + 64 * wv * 8;
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
            const int pp = j / JP, jj = j % JP;
            if (jj < JH) load_lds16(rk, koff[jj] + pp * PAIRB, 0, dst + 256 * j * 8);
            else load_lds16(rv, voff[jj - JH] + pp * PAIRB, 0, dst + 256 * j * 8);
        }
    };

    // the 4 heads' scale-offset queries, times qscale (the score scale with
    // log2(e): scores come out of the MFMAs in exp2 units), as B operands:
    // lane (n, gq) holds head h0 + n (n < 4; zero otherwise), dims 32 i + 8 gq .. + 7
    bf16x8 qf[NQ];
    {
        const float qs = p.qscale;
        const int h = h0 + (n < 4 ? n : 0);
        const uint16_t* qrow = (const uint16_t*)p.q_out + ((int64_t)b * p.Hq + h) * D;
        const uint16_t* al = (const uint16_t*)p.alpha_out + (int64_t)h * D;
        const uint16_t* be = (const uint16_t*)p.beta_out + (int64_t)h * D;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int d0 = 32 * i + 8 * gq;
            const u32x4 qw = *(const u32x4*)(qrow + d0);
            const u32x4 av = *(const u32x4*)(al + d0);
            const u32x4 bv = *(const u32x4*)(be + d0);
            u32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = qw[e], aw = av[e], bw = bv[e];
                r[e] = pack_bf16x2(__builtin_fmaf(bf16_lo(w), bf16_lo(aw), bf16_lo(bw)) * qs,
                                   __builtin_fmaf(bf16_hi(w), bf16_hi(aw), bf16_hi(bw)) * qs);
                r[e] = n < 4 ? r[e] : 0u;
            }
            qf[i] = __builtin_bit_cast(bf16x8, r);
        }
    }

    const bf16x8 kOnes = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 oacc[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) oacc[dt] = zero;
    f32x4 lacc = zero;
    float m_run = kNegBig;      // lane (n, .): the running maximum of head h0 + n

    // one pair of the stage in `slot`: keys key0 .. key0 + 31
    auto attend = [&](const uint16_t* slot, int pp, int64_t key0) {
        int ko = pp * R::SLOT + R::kofs(n, gq);
        asm volatile("" : "+v"(ko));
        const uint16_t* kb = slot + ko;
        f32x4 s0 = zero, s1 = zero;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const bf16x8 k0 = *(const bf16x8*)(kb + i * R::K_STEP);
            const bf16x8 k1 = *(const bf16x8*)(kb + i * R::K_STEP + R::K_KEY16);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[i], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[i], s1, 0, 0, 0);
        }
        // s0[r]: key key0 + 4 gq + r, s1[r]: key key0 + 16 + 4 gq + r (head h0 + n)
        if (key0 + 31 > hi) {
            const int lim = (int)(hi - key0) - 4 * gq;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (r > lim) s0[r] = -INFINITY;
                if (16 + r > lim) s1[r] = -INFINITY;
            }
        }
        float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                         fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        if (__any(mx > m_run + kMargin)) {
            const float mn = fmaxf(m_run, mx);
            const float corr = fast_exp2(m_run - mn);
            m_run = mn;
            lacc *= corr;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) oacc[dt] *= corr;
        }
        const u32x4 pw4 = {pack_bf16x2(fast_exp2(s0[0] - m_run), fast_exp2(s0[1] - m_run)),
                           pack_bf16x2(fast_exp2(s0[2] - m_run), fast_exp2(s0[3] - m_run)),
                           pack_bf16x2(fast_exp2(s1[0] - m_run), fast_exp2(s1[1] - m_run)),
                           pack_bf16x2(fast_exp2(s1[2] - m_run), fast_exp2(s1[3] - m_run))};
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw4);
        lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes, pb, lacc, 0, 0, 0);
        // V^T operands: this lane addresses key rows 4 gq + (n >> 2) and
        // 16 + 4 gq + (n >> 2), dims 16 dt + 4 (n & 3)
        int vo = pp * R::SLOT + R::KPART + R::vofs_tr(4 * gq + (n >> 2), 0, n & 3);
        asm volatile("" : "+v"(vo));
        const uint16_t* vb = slot + vo;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const s16x4 v0 = lds_read_tr(vb + dt * R::V_DT);
            const s16x4 v1 = lds_read_tr(vb + R::V_KEY16 + dt * R::V_DT);
            const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
            oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb, oacc[dt], 0, 0, 0);
        }
    };

    issue(0);
    for (int st = 0; st < nst; ++st) {
        // this wave's loads of stage st have landed; after the barrier every
        // wave's have, and every wave is done with stage st - 1's slot
        __builtin_amdgcn_s_waitcnt(0x0F70);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (st + 1 < nst) issue(st + 1);
        const uint16_t* slot = lds + (st & 1) * SLOTE;
#pragma unroll
        for (int t = 0; t < PPW; ++t) {
            const int pp = wv * PPW + t;
            const int64_t key0 = lo + (int64_t)st * SK + 32 * pp;
            if (key0 <= hi) attend(slot, pp, key0);
        }
    }

    // merge the 4 waves' states (fixed order) into the partials of the
    // chunk: out[head][{max, sum, sum of weighted values}]
    __syncthreads();
    float (*red)[4][D + 2] = (float (*)[4][D + 2])lds;    // [wave][head][D + 2]
    if (n < 4) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[wv][n][2 + 16 * dt + 4 * gq + r] = oacc[dt][r];
        if (gq == 0) {
            red[wv][n][0] = m_run;
            red[wv][n][1] = lacc[0];
        }
    }
    __syncthreads();
    const int64_t part_stride = (int64_t)p.n_split * (D + 2);
    float* out = p.ws_part + ((int64_t)b * p.Hq + h0) * part_stride + (int64_t)s * (D + 2);
    for (int idx = tid; idx < 4 * (D + 1); idx += 256) {
        const int hh = idx / (D + 1), d = idx % (D + 1);   // d == D: the (max, sum) pair
        float M = red[0][hh][0];
#pragma unroll
        for (int w = 1; w < 4; ++w) M = fmaxf(M, red[w][hh][0]);
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) sum += fast_exp2(red[w][hh][0] - M) * (d < D ? red[w][hh][2 + d] : red[w][hh][1]);
        float* o = out + hh * part_stride;
        if (d < D) {
            o[2 + d] = sum;
        } else {
            o[0] = M;
            o[1] = sum;
        }
    }
}

}  // namespace

hipError_t launch_xattn_lds(const XattnParams& p, hipStream_t st)
{
    const int hblocks = (p.Hq / p.Hkv) / 4;
    for (int b0 = 0; b0 < p.B; b0 += kPosPerLaunch) {
        const int nb = p.B - b0 < kPosPerLaunch ? p.B - b0 : kPosPerLaunch;
        PosBlock pos;
        for (int i = 0; i < nb; ++i) pos.v[i] = p.pos[b0 + i];
        const dim3 grid((unsigned)p.n_split, (unsigned)(p.Hkv * hblocks), (unsigned)nb);
        if (p.D == 64) hipLaunchKernelGGL((xattn_lds_kernel<64>), grid, dim3(256), 0, st, p, b0, pos);
        else hipLaunchKernelGGL((xattn_lds_kernel<128>), grid, dim3(256), 0, st, p, b0, pos);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_merge(p, st);
}

}  // namespace orthros
