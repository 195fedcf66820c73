// swa_prefill.hip -- base-stream sliding-window attention with the fused
// KV-cache writer (prefill), for gfx950.
//
// Computes, for every sequence b, query head h and base row t,
//   o[b,t,h] = sum_{j in W_t} softmax_j(<q_hat, k_j> * scale) v_j,
//   W_t = [max(0, t-w+1), t],  q_hat = q[b,t,h] * alpha[h] + beta[h],
// ("Orthros:阶段感知异构注意力精读笔记" §2.3 Eq. (4) with the per-stream
// scale-offset of §2.2), and copies k, v rows [0, T) into the layer's cache
// (§2.1: the base stream builds every position's K/V; §2.6: the window
// bounds reads, not storage).
//
// bf16 kernel (the hot path).  The band really is a dense contraction, so
// both products run on bf16 MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulate):
//   - one workgroup = 4 waves = one 32-row query sub-tile per wave; the
//     waves of a workgroup share one KV head: with G = Hq/Hkv >= 4 they are
//     4 heads of the group on the same 32 tokens (K/V read once for the 4),
//     with G = 1 they are 4 consecutive sub-tiles of one head;
//   - the key band [q0-w+1, q0+TQ) is streamed through LDS in 32-key
//     blocks, double-buffered: the next block's global loads are in flight
//     while the current block's MFMAs run;
//   - scores are computed transposed, S^T = K Q^T, so each lane owns one
//     query column and 16 keys: the row softmax is 16 in-lane values plus
//     one swap with the other half-wave, and P^T leaves the accumulator
//     already in the B-operand layout of the next product O^T = V^T P^T;
//   - V is stored transposed in LDS (written from registers, conflict-free)
//     so the A operand of O^T = V^T P^T is two 8-byte LDS reads per lane;
//   - fp32 online softmax in the exp2 domain (log2 e folded into q_hat);
//   - the workgroup that owns a key block (keys [q0, q0+TQ)) writes those
//     K/V rows to the cache from the registers that staged them, so the
//     cache write costs no extra read.
// Workgroup ids are remapped so each XCD walks a contiguous run of tiles
// and the 127-key halo of the next tile is still in its L2.
//
// fp32 kernel: a VALU variant (16 lanes per row, 16 rows of one head per
// workgroup) for fp32 storage, where the tolerance is 1e-4.

#include "device.h"
#include "kernels.h"

namespace orthros {
namespace {

// ------------------------------------------------------------------ bf16

template <int D, int HS>
__global__ __launch_bounds__(256, 2) void swa_bf16_kernel(SwaParams a, int n_tiles, int hblocks)
{
    constexpr int TQ = 32 * (4 / HS);   // base rows per workgroup
    constexpr int KROW = D + 8;         // bf16 per K row in LDS (16 B pad: conflict-free b128 reads)
    constexpr int VROW = 36;            // bf16 per V^T row in LDS (72 B: conflict-free b64 reads)
    constexpr int KBUF = 32 * KROW;
    constexpr int VBUF = D * VROW;
    constexpr int KCH = D / 64;         // 16-byte K chunks per thread per block
    constexpr int NQ = D / 16;          // MFMA k-steps over the head dim
    constexpr int ND = D / 32;          // 32-wide output tiles over the head dim
    __shared__ __align__(16) uint16_t lds[2 * (KBUF + VBUF)];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int64_t id = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int tile = (int)(id % n_tiles);
    int64_t rest = id / n_tiles;
    const int hb = (int)(rest % hblocks);
    rest /= hblocks;
    const int g = (int)(rest % a.Hkv);
    const int b = (int)(rest / a.Hkv);

    const int64_t T = a.T;
    const int G = a.Hq / a.Hkv;
    const int W = a.window;
    const int64_t q0 = (int64_t)tile * TQ;
    const int h = g * G + hb * HS + (wv % HS);
    const int64_t r0 = q0 + 32 * (wv / HS);
    const int n = lane & 31, half = lane >> 5;
    const int64_t t = r0 + n;

    const uint16_t* __restrict__ qg = (const uint16_t*)a.q;
    const uint16_t* __restrict__ kg = (const uint16_t*)a.k;
    const uint16_t* __restrict__ vg = (const uint16_t*)a.v;
    uint16_t* __restrict__ kc = (uint16_t*)a.k_cache;
    uint16_t* __restrict__ vc = (uint16_t*)a.v_cache;

    // ---- q_hat = (q * alpha + beta) * scale * log2(e), as MFMA B operands:
    // lane (n, half) holds q_hat[row t][16 i + 8 half + e], e = 0..7.
    bf16x8 qf[NQ];
    {
        const uint16_t* al = (const uint16_t*)a.alpha + (int64_t)h * D;
        const uint16_t* be = (const uint16_t*)a.beta + (int64_t)h * D;
        const uint16_t* qrow = qg + (((int64_t)b * T + t) * a.Hq + h) * D;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int d0 = 16 * i + 8 * half;
            u32x4 qv = {0u, 0u, 0u, 0u};
            if (t < T) qv = *(const u32x4*)(qrow + d0);
            const u32x4 av = *(const u32x4*)(al + d0);
            const u32x4 bv = *(const u32x4*)(be + d0);
            u32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float x0 = (bf16_lo(qv[e]) * bf16_lo(av[e]) + bf16_lo(bv[e])) * a.qscale;
                float x1 = (bf16_hi(qv[e]) * bf16_hi(av[e]) + bf16_hi(bv[e])) * a.qscale;
                r[e] = pack_bf16x2(x0, x1);
            }
            qf[i] = __builtin_bit_cast(bf16x8, r);
        }
    }

    // ---- key blocks of this workgroup and of this wave
    const int64_t klo = q0 - W + 1 > 0 ? q0 - W + 1 : 0;
    const int64_t khi = (q0 + TQ < T ? q0 + TQ : T) - 1;
    const int64_t kb0 = klo >> 5, kb1 = khi >> 5;
    const bool wave_on = r0 < T;
    const int64_t wlo = r0 - W + 1 > 0 ? r0 - W + 1 : 0;
    const int64_t whi = r0 + 31 < T - 1 ? r0 + 31 : T - 1;
    const bool writer = (hb == 0);

    // ---- staging registers of one key block
    u32x4 kreg[KCH];
    u32x4 vreg[2];
    const int vkp = tid & 15, vdc = tid >> 4;     // V: key pair, 8-wide d chunk
    const bool vthread = vdc < D / 8;

    auto load_block = [&](int64_t kb) {
        const int64_t kbase = kb * 32;
#pragma unroll
        for (int r = 0; r < KCH; ++r) {
            const int c = tid + 256 * r, kk = c / (D / 8), dc = c % (D / 8);
            const int64_t j = kbase + kk;
            kreg[r] = u32x4{0u, 0u, 0u, 0u};
            if (j < T) kreg[r] = *(const u32x4*)(kg + (((int64_t)b * T + j) * a.Hkv + g) * D + 8 * dc);
        }
        vreg[0] = vreg[1] = u32x4{0u, 0u, 0u, 0u};
        if (vthread) {
            const int64_t j = kbase + 2 * vkp;
            if (j < T) vreg[0] = *(const u32x4*)(vg + (((int64_t)b * T + j) * a.Hkv + g) * D + 8 * vdc);
            if (j + 1 < T) vreg[1] = *(const u32x4*)(vg + (((int64_t)b * T + j + 1) * a.Hkv + g) * D + 8 * vdc);
        }
    };

    auto store_block = [&](int buf, int64_t kb) {
        uint16_t* Ks = lds + buf * (KBUF + VBUF);
        uint16_t* Vt = Ks + KBUF;
#pragma unroll
        for (int r = 0; r < KCH; ++r) {
            const int c = tid + 256 * r, kk = c / (D / 8), dc = c % (D / 8);
            *(u32x4*)(Ks + kk * KROW + 8 * dc) = kreg[r];
        }
        if (vthread) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w0 = vreg[0][e], w1 = vreg[1][e];
                *(uint32_t*)(Vt + (8 * vdc + 2 * e) * VROW + 2 * vkp) = (w0 & 0xffffu) | (w1 << 16);
                *(uint32_t*)(Vt + (8 * vdc + 2 * e + 1) * VROW + 2 * vkp) = (w0 >> 16) | (w1 & 0xffff0000u);
            }
        }
        // fused cache writer: this workgroup owns keys [q0, q0 + TQ)
        const int64_t kbase = kb * 32;
        if (writer && kbase >= q0) {
            const int64_t crow = ((int64_t)b * a.Hkv + g) * a.cap;
#pragma unroll
            for (int r = 0; r < KCH; ++r) {
                const int c = tid + 256 * r, kk = c / (D / 8), dc = c % (D / 8);
                const int64_t j = kbase + kk;
                if (j < T) *(u32x4*)(kc + (crow + j) * D + 8 * dc) = kreg[r];
            }
            if (vthread) {
                const int64_t j = kbase + 2 * vkp;
                if (j < T) *(u32x4*)(vc + (crow + j) * D + 8 * vdc) = vreg[0];
                if (j + 1 < T) *(u32x4*)(vc + (crow + j + 1) * D + 8 * vdc) = vreg[1];
            }
        }
    };

    f32x16 oacc[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) oacc[i] = f32x16{};
    float m_run = kNegBig, l_run = 0.f;

    auto compute_block = [&](int buf, int64_t kb) {
        const int64_t kbase = kb * 32;
        if (!wave_on || kbase + 31 < wlo || kbase > whi) return;
        const uint16_t* Ks = lds + buf * (KBUF + VBUF);
        const uint16_t* Vt = Ks + KBUF;

        // S^T[key m][query n] for the 32 keys of the block
        f32x16 s = f32x16{};
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const bf16x8 kf = *(const bf16x8*)(Ks + n * KROW + 16 * i + 8 * half);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[i], s, 0, 0, 0);
        }
        // lane (n, half), register r holds key kbase + 8 (r/4) + 4 half + r%4
        const bool full = (kbase + 31 <= r0) && (kbase >= r0 + 31 - W + 1);
        float mloc = kNegBig;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            if (!full) {
                const int64_t j = kbase + 8 * (r >> 2) + 4 * half + (r & 3);
                if (j > t || j < t - W + 1) s[r] = -INFINITY;
            }
            mloc = fmaxf(mloc, s[r]);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float m_new = fmaxf(m_run, mloc);
        const float corr = fast_exp2(m_run - m_new);
        m_run = m_new;
        float psum = 0.f;
        u32x4 pw[2];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const float p0 = fast_exp2(s[r] - m_new);
            const float p1 = fast_exp2(s[r + 1] - m_new);
            psum += p0 + p1;
            pw[r >> 3][(r & 7) >> 1] = pack_bf16x2(p0, p1);
        }
        l_run = l_run * corr + psum;
#pragma unroll
        for (int i = 0; i < ND; ++i) oacc[i] *= corr;

        // O^T[d][query] += V^T[d][keys] P^T[keys][query]; operand c covers keys
        // 16c + {4half..4half+3, 8+4half..8+4half+3}, matching P^T's registers.
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const uint16_t* vrow = Vt + (32 * dt + n) * VROW;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const u32x2 lo = *(const u32x2*)(vrow + 16 * c + 4 * half);
                const u32x2 hi = *(const u32x2*)(vrow + 16 * c + 8 + 4 * half);
                const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, __builtin_bit_cast(bf16x8, pw[c]),
                                                                   oacc[dt], 0, 0, 0);
            }
        }
    };

    load_block(kb0);
    store_block(0, kb0);
    __syncthreads();
    for (int64_t kb = kb0; kb <= kb1; ++kb) {
        const int buf = (int)((kb - kb0) & 1);
        const bool more = kb < kb1;
        if (more) load_block(kb + 1);
        compute_block(buf, kb);
        if (more) store_block(buf ^ 1, kb + 1);
        __syncthreads();
    }

    // ---- normalise and store: lane (n, half) holds d = 32 dt + 8 i + 4 half
    // + 0..3; a permlane32 swap between the halves for each pair of i leaves
    // it 8 consecutive dims (32 dt + 8 (2 k + half)), stored as 16 bytes
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = 1.f / l_tot;
    u32x4 w[ND][2];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i0 = 2 * k, i1 = 2 * k + 1;
                const auto r = __builtin_amdgcn_permlane32_swap(
                    pack_bf16x2(oacc[dt][4 * i0 + 2 * e] * inv, oacc[dt][4 * i0 + 2 * e + 1] * inv),
                    pack_bf16x2(oacc[dt][4 * i1 + 2 * e] * inv, oacc[dt][4 * i1 + 2 * e + 1] * inv), false, false);
                w[dt][k][e] = r[0];
                w[dt][k][2 + e] = r[1];
            }
    if (wave_on && t < T) {
        uint16_t* orow = (uint16_t*)a.o + (((int64_t)b * T + t) * a.Hq + h) * D;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int k = 0; k < 2; ++k) *(u32x4*)(orow + 32 * dt + 16 * k + 8 * half) = w[dt][k];
    }
}

// ------------------------------------------------------------------- fp32

// fp32 storage (tolerance 1e-4): fp32 FMAs on the VALU.  A workgroup takes
// 16 rows of one query head; each row is served by 16 lanes, lane e of the
// row holding head dims [D/16 e, D/16 (e+1)) of the query and of the output
// accumulator.  The key band [q0 - w + 1, q0 + 15] streams through LDS in
// 32-key blocks (the next block's rows are loaded into registers while the
// current one is used); per key the 16 lanes' partial dot products meet in
// a DPP reduction, so every lane of the row has the score; the block's
// scores are taken first and the online softmax advances once per block.
// The workgroup of the KV group's first query head writes the K/V rows it
// owns ([q0, q0 + 16)) to the cache.
template <int D>
__global__ __launch_bounds__(256) void swa_f32_kernel(SwaParams a, int n_tiles)
{
    constexpr int KB = 32;                  // keys per LDS block
    constexpr int LPR = 16, RW = 256 / LPR; // lanes per row, rows per workgroup
    constexpr int DL = D / LPR;             // head dims per lane
    constexpr int F4 = KB * D / 4 / 256;    // float4 of a K (or V) block per thread
    __shared__ __align__(16) float Ks[KB][D];
    __shared__ __align__(16) float Vs[KB][D];

    const int tid = threadIdx.x;
    const int row = tid / LPR, e = tid % LPR;
    const int tile = blockIdx.x % n_tiles;
    const int h = (blockIdx.x / n_tiles) % a.Hq;
    const int b = blockIdx.x / n_tiles / a.Hq;
    const int G = a.Hq / a.Hkv, g = h / G;
    const int64_t T = a.T;
    const int W = a.window;
    const int64_t q0 = (int64_t)tile * RW, t = q0 + row;
    const float* kg = (const float*)a.k;
    const float* vg = (const float*)a.v;

    float qh[DL], acc[DL];
    {
        const float* al = (const float*)a.alpha + (int64_t)h * D + DL * e;
        const float* be = (const float*)a.beta + (int64_t)h * D + DL * e;
        const float* qrow = (const float*)a.q + (((int64_t)b * T + (t < T ? t : T - 1)) * a.Hq + h) * D + DL * e;
#pragma unroll
        for (int d = 0; d < DL; ++d) {
            qh[d] = (qrow[d] * al[d] + be[d]) * a.qscale;
            acc[d] = 0.f;
        }
    }
    float m_run = kNegBig, l_run = 0.f;

    const int64_t klo = q0 - W + 1 > 0 ? q0 - W + 1 : 0;
    const int64_t khi = (q0 + RW < T ? q0 + RW : T) - 1;
    const bool writer = (h % G) == 0;
    const int64_t kb0 = klo & ~(int64_t)(KB - 1);
    // rows of one block: thread tid holds float4 i of K and V, i = tid + 256 f
    float4 kr[F4], vr[F4];
    auto load_block = [&](int64_t kbase) {
#pragma unroll
        for (int f = 0; f < F4; ++f) {
            const int idx = tid + 256 * f, kk = idx / (D / 4), d4 = idx % (D / 4);
            const int64_t j = kbase + kk;
            kr[f] = vr[f] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (j < T) {
                const int64_t off = (((int64_t)b * T + j) * a.Hkv + g) * D + 4 * d4;
                kr[f] = *(const float4*)(kg + off);
                vr[f] = *(const float4*)(vg + off);
            }
        }
    };
    load_block(kb0);
    for (int64_t kbase = kb0; kbase <= khi; kbase += KB) {
        __syncthreads();                    // the previous block is no longer read
#pragma unroll
        for (int f = 0; f < F4; ++f) {
            const int idx = tid + 256 * f, kk = idx / (D / 4), d4 = idx % (D / 4);
            *(float4*)&Ks[kk][4 * d4] = kr[f];
            *(float4*)&Vs[kk][4 * d4] = vr[f];
            const int64_t j = kbase + kk;
            if (writer && j >= q0 && j <= khi) {
                const int64_t coff = (((int64_t)b * a.Hkv + g) * a.cap + j) * D + 4 * d4;
                *(float4*)((float*)a.k_cache + coff) = kr[f];
                *(float4*)((float*)a.v_cache + coff) = vr[f];
            }
        }
        __syncthreads();
        if (kbase + KB <= khi) load_block(kbase + KB);
        // keys of this block in the row's window [t - w + 1, t]: the block's
        // scores first (independent of one another), one maximum and one
        // rescale per block, then the weighted values into two interleaved
        // accumulator sets (short dependency chains)
        const int lo = (int)((t - W + 1 > kbase ? t - W + 1 : kbase) - kbase);
        const int hi = (int)((t < kbase + KB - 1 ? t : kbase + KB - 1) - kbase);
        float sc[KB];
        float mb = kNegBig;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            float sp = 0.f;
#pragma unroll
            for (int d = 0; d < DL; ++d) sp += qh[d] * Ks[j][DL * e + d];
            const float sj = group_sum<LPR>(sp);
            const bool ok = j >= lo && j <= hi && t < T;   // uniform over the row's lanes
            sc[j] = ok ? sj : -INFINITY;
            mb = fmaxf(mb, sc[j]);
        }
        if (mb > kNegBig) {
            const float m_new = fmaxf(m_run, mb);
            const float corr = fast_exp2(m_run - m_new);
            m_run = m_new;
            float l0 = l_run * corr, l1 = 0.f, acc1[DL];
#pragma unroll
            for (int d = 0; d < DL; ++d) {
                acc[d] *= corr;
                acc1[d] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < KB; j += 2) {
                const float p0 = fast_exp2(sc[j] - m_new), p1 = fast_exp2(sc[j + 1] - m_new);
                l0 += p0;
                l1 += p1;
#pragma unroll
                for (int d = 0; d < DL; ++d) {
                    acc[d] += p0 * Vs[j][DL * e + d];
                    acc1[d] += p1 * Vs[j + 1][DL * e + d];
                }
            }
            l_run = l0 + l1;
#pragma unroll
            for (int d = 0; d < DL; ++d) acc[d] += acc1[d];
        }
    }
    if (t < T) {
        float* orow = (float*)a.o + (((int64_t)b * T + t) * a.Hq + h) * D + DL * e;
        const float inv = 1.f / l_run;
#pragma unroll
        for (int d = 0; d < DL; d += 4)
            *(float4*)(orow + d) = make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
    }
}

template <int D, int HS>
hipError_t launch_bf16(const SwaParams& p, hipStream_t s)
{
    constexpr int TQ = 32 * (4 / HS);
    const int G = p.Hq / p.Hkv;
    const int n_tiles = (int)((p.T + TQ - 1) / TQ);
    const int hblocks = G / HS;
    const int64_t n_wg = (int64_t)p.B * p.Hkv * hblocks * n_tiles;
    hipLaunchKernelGGL((swa_bf16_kernel<D, HS>), dim3((unsigned)n_wg), dim3(256), 0, s, p, n_tiles, hblocks);
    return hipGetLastError();
}

template <int D>
hipError_t launch_f32(const SwaParams& p, hipStream_t s)
{
    const int n_tiles = (int)((p.T + 15) / 16);             // 16 rows per workgroup
    const int64_t n_wg = (int64_t)p.B * p.Hq * n_tiles;
    hipLaunchKernelGGL((swa_f32_kernel<D>), dim3((unsigned)n_wg), dim3(256), 0, s, p, n_tiles);
    return hipGetLastError();
}

}  // namespace

// Heads per workgroup of the bf16 kernel: 4 waves cover HS heads x (4/HS)
// sub-tiles of 32 rows; HS must divide G.
static int swa_heads_per_wg(int G) { return (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1; }

hipError_t launch_swa(const SwaParams& p, hipStream_t s)
{
    if (p.dt == Dt::F32) return p.D == 64 ? launch_f32<64>(p, s) : launch_f32<128>(p, s);
    const int HS = swa_heads_per_wg(p.Hq / p.Hkv);
    if (ring_applies(p.dt, p.Hq, p.Hkv, p.window)) return launch_swa_ring(p, s);
    if (p.D == 64) {
        if (HS == 4) return launch_bf16<64, 4>(p, s);
        if (HS == 2) return launch_bf16<64, 2>(p, s);
        return launch_bf16<64, 1>(p, s);
    }
    if (HS == 4) return launch_bf16<128, 4>(p, s);
    if (HS == 2) return launch_bf16<128, 2>(p, s);
    return launch_bf16<128, 1>(p, s);
}

}  // namespace orthros
