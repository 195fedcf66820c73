// copies_flash.hip -- output copies at many positions per sequence (the PT
// and SFT modes, "Orthros:阶段感知异构注意力精读笔记" §2.5 mode table) for
// bf16 and groups of 4 query heads per KV head: each copy's scale-offset
// query attends over the cached keys [0, pos] of its original position
// (§2.3 Eq. (5), §2.4).  A causal flash kernel over an arbitrary position
// list:
//
//   - a workgroup (4 waves) serves 32 copies of one sequence x the 4 query
//     heads of a 4-head block of one KV group; wave (sub-tile s, head pair
//     p) owns copies 16 s .. 16 s + 15 of both heads of the pair, so every
//     K/V fragment it reads from LDS feeds two MFMAs;
//   - the keys [0, max position of the 32 copies] stream from the cache
//     (one contiguous run of rows per (sequence, KV head)) as 32-key pairs
//     through a 4-slot LDS ring, two pairs per step: while a step computes,
//     the next two pairs are in flight into registers, and the slots they
//     land in are the previous step's, so one barrier per step suffices;
//   - S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 (K layout in
//     pair_tile.h); V stays row-major in LDS and its V^T operands come from
//     the transposing LDS read; keys past a copy's position are masked in the pairs
//     that reach past the smallest position of the wave's copies; a wave
//     skips the pairs past its largest position;
//   - online softmax in the exp2 domain, rescaled only when a block's
//     maximum exceeds the running one by more than 2^8; pair 0 goes first
//     and starts the running maxima and the accumulators (every copy has
//     key 0);
//   - workgroups with the largest positions are dispatched first.
// A copy whose position lies outside [0, T) computes as if at 0 and writes
// NaN.

#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "pair_tile.h"

namespace orthros {
namespace {

constexpr int kNs = 4;                    // pair slots of the ring
constexpr float kMargin = 8.0f;           // lazy-rescale margin, log2 units

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void copies_flash_kernel(
    CopiesParams a, int n_tiles, int hblocks)
{
    using R = PairTile<D>;
    constexpr int NT = 256;
    constexpr int C16 = D / 8;                 // 16-byte chunks per row
    constexpr int NQ = D / 32;                 // MFMA k-steps over the head dim
    constexpr int ND = D / 16;                 // 16-wide d tiles of O^T
    constexpr int KPC = 32 * C16;              // 16-byte chunks of K (and of V) per pair
    constexpr int KCH = KPC / NT;              // per thread and pair
    static_assert(KCH >= 1 && KPC == KCH * NT, "head dim");
    __shared__ __align__(16) uint16_t ring[kNs * R::SLOT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hp = wv & 1, sub = wv >> 1;
    const int n = lane & 15, gq = lane >> 4;
    // heaviest tiles first: the tile index runs slowest and backwards
    const int64_t streams = (int64_t)a.B * a.Hkv * hblocks;
    const int64_t id = blockIdx.x;
    const int tile = n_tiles - 1 - (int)(id / streams);
    int64_t st = id % streams;
    const int hb = (int)(st % hblocks);
    st /= hblocks;
    const int g = (int)(st % a.Hkv);
    const int b = (int)(st / a.Hkv);
    const int G = a.Hq / a.Hkv;
    const int h0 = g * G + hb * 4 + 2 * hp;     // the wave's heads: h0, h0 + 1
    const int64_t T = a.T, T_out = a.T_out;
    const float qs = a.qscale;

    // positions of the workgroup's 32 copies: lane & 31 reads copy 32 tile + (lane & 31)
    const int32_t* posb = a.pos + (int64_t)b * T_out;
    auto pos_of = [&](int64_t c) -> int {
        if (c >= T_out) return -1;                  // no such copy: nothing to read, nothing stored
        const int p = posb[c];
        return (p >= 0 && p < T) ? p : -2;         // -2: invalid position, NaN output
    };
    const int pw = pos_of((int64_t)tile * 32 + (lane & 31));
    int pmax = pw < 0 ? 0 : pw;
#pragma unroll
    for (int x = 1; x < 32; x <<= 1) pmax = max(pmax, __shfl_xor(pmax, x));
    pmax = __builtin_amdgcn_readfirstlane(pmax);          // the workgroup's largest position
    const int64_t c0 = (int64_t)tile * 32 + 16 * sub;     // the wave's first copy
    const int myp_raw = pos_of(c0 + n);
    const int myp = myp_raw < 0 ? 0 : myp_raw;            // lane n's copy position (clamped)
    int wmin = myp, wmax = myp;
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) {
        wmin = min(wmin, __shfl_xor(wmin, x));
        wmax = max(wmax, __shfl_xor(wmax, x));
    }
    wmin = __builtin_amdgcn_readfirstlane(wmin);
    wmax = __builtin_amdgcn_readfirstlane(wmax);

    const int64_t qrow_b = (int64_t)a.Hq * D * 2;
    const int64_t q_seq = (int64_t)b * T_out * a.Hq * D + (int64_t)h0 * D;
    const int64_t c_seq = ((int64_t)b * a.Hkv + g) * a.cap * D;

    // the copies' queries (q' * alpha' + beta') * qscale as MFMA B operands
    // (the score scale, log2(e) included, is folded in here, once per
    // workgroup, so that S comes out of the MFMAs in exp2 units):
    // lane (n, gq) holds copy c0 + n, head dims 32 i + 8 gq .. + 7
    bf16x8 qf[2][NQ];
    {
        const rsrc_t rq = make_rsrc((const uint16_t*)a.q_out + q_seq + c0 * a.Hq * D,
                                    (T_out - c0) * qrow_b - h0 * D * 2);
        const uint16_t* al = (const uint16_t*)a.alpha_out + (int64_t)h0 * D;
        const uint16_t* be = (const uint16_t*)a.beta_out + (int64_t)h0 * D;
#pragma unroll
        for (int hd = 0; hd < 2; ++hd)
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const u32x4 qw = buf_load16(rq, (uint32_t)(n * qrow_b + hd * D * 2 + 64 * i + 16 * gq));
                const int d0 = hd * D + 32 * i + 8 * gq;
                const u32x4 av = *(const u32x4*)(al + d0);
                const u32x4 bv = *(const u32x4*)(be + d0);
                u32x4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = qw[e], aw = av[e], bw = bv[e];
                    r[e] = pack_bf16x2(__builtin_fmaf(bf16_lo(w), bf16_lo(aw), bf16_lo(bw)) * qs,
                                       __builtin_fmaf(bf16_hi(w), bf16_hi(aw), bf16_hi(bw)) * qs);
                }
                qf[hd][i] = __builtin_bit_cast(bf16x8, r);
            }
    }

    // staging of pairs (32 cache rows each): K by LDS unit, thread tid
    // taking units tid + 256 j of the pair's K part (PairTile::k_unit:
    // 8 threads read 128 contiguous bytes of one row, and the LDS stores are
    // contiguous); V item tid + 256 j -> (row, chunk) by PairTile::vitem,
    // item + 256 being the same chunk 16 rows on (KCH is 2 only at d = 128)
    static_assert(KCH == 1 || NT / C16 == 16, "staging step");
    auto load_pair = [&](int64_t pr, u32x4 (&kr)[KCH], u32x4 (&vr)[KCH]) {
        const int64_t kbase = pr * 32;
        const int64_t avail = (T - kbase) * D * 2;
        const rsrc_t rk = make_rsrc((const uint16_t*)a.k_cache + c_seq + kbase * D, avail);
        const rsrc_t rv = make_rsrc((const uint16_t*)a.v_cache + c_seq + kbase * D, avail);
        int vr_row, vr_c;
        R::vitem(tid, vr_row, vr_c);
#pragma unroll
        for (int j = 0; j < KCH; ++j) {
            int kr_row, kr_c;
            R::k_unit(tid + NT * j, kr_row, kr_c);
            kr[j] = buf_load16(rk, (uint32_t)(kr_row * D * 2 + 16 * kr_c));
            vr[j] = buf_load16(rv, (uint32_t)((vr_row + 16 * j) * D * 2 + 16 * vr_c));
        }
    };
    auto store_pair = [&](int64_t pr, const u32x4 (&kr)[KCH], const u32x4 (&vr)[KCH]) {
        uint16_t* Ks = ring + (int)(pr & (kNs - 1)) * R::SLOT;
        uint16_t* Vt = Ks + R::KPART;
        int t = tid;
        asm volatile("" : "+v"(t));
        int vr_row, vr_c;
        R::vitem(t, vr_row, vr_c);
#pragma unroll
        for (int j = 0; j < KCH; ++j) {
            *(u32x4*)(Ks + 8 * (t + NT * j)) = kr[j];
            *(u32x4*)(Vt + R::vofs16(vr_row, vr_c) + j * R::V_KEY16) = vr[j];
        }
    };

    const bf16x8 kOnes = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    f32x4 oacc[2][ND];
    f32x4 lacc[2];
    float m_run[2];
    f32x4 negm[2];      // -m_run of the lane's copy, the first S MFMA's accumulator after pair 0
    // one pair against both heads; FIRST: pair 0, which starts the running
    // maxima and the accumulators.  After it, S comes out of the MFMAs
    // already shifted by the running maximum (exp2 units), so the
    // probabilities are plain exp2 of the scores.
    auto attend = [&](auto first_tag, int64_t pr) {
        constexpr bool FIRST = decltype(first_tag)::value;
        // two K bases per pair, for even and odd k-steps (opaque, so that
        // the steps stay immediate offsets)
        int ko0 = (int)(pr & (kNs - 1)) * R::SLOT + R::kofs(n, gq);
        int ko1 = (int)(pr & (kNs - 1)) * R::SLOT + R::kofs(n, 4 + gq);
        asm volatile("" : "+v"(ko0), "+v"(ko1));
        const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 s[2][2];
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const uint16_t* kb = ring + ((i & 1) ? ko1 : ko0) + (i >> 1) * R::K_STEP2;
            const bf16x8 k0 = *(const bf16x8*)kb;
            const bf16x8 k1 = *(const bf16x8*)(kb + R::K_KEY16);
#pragma unroll
            for (int hd = 0; hd < 2; ++hd) {
                const f32x4 c = FIRST ? zero : negm[hd];
                s[hd][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[hd][i], i ? s[hd][0] : c, 0, 0, 0);
                s[hd][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[hd][i], i ? s[hd][1] : c, 0, 0, 0);
            }
        }
        // s[.][0][r]: key 32 pr + 4 gq + r, s[.][1][r]: key 32 pr + 16 + 4 gq + r; copy c0 + n
        if (pr * 32 + 31 > wmin) {
            const int lim = myp - (int)(pr * 32) - 4 * gq;   // last admissible r (block 0) for this lane
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool m0 = r > lim, m1 = 16 + r > lim;
#pragma unroll
                for (int hd = 0; hd < 2; ++hd) {
                    if (m0) s[hd][0][r] = -INFINITY;
                    if (m1) s[hd][1][r] = -INFINITY;
                }
            }
        }
        bf16x8 pb[2];
#pragma unroll
        for (int hd = 0; hd < 2; ++hd) {
            f32x4 s0 = s[hd][0], s1 = s[hd][1];
            const float lmax = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                                     fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
            if constexpr (FIRST) {
                // scores in exp2 units; their row maximum starts the running maximum
                float rmax = fmaxf(lmax, __shfl_xor(lmax, 16));
                m_run[hd] = fmaxf(rmax, __shfl_xor(rmax, 32));
                s0 -= m_run[hd];
                s1 -= m_run[hd];
                negm[hd] = f32x4{-m_run[hd], -m_run[hd], -m_run[hd], -m_run[hd]};
            } else if (__any(lmax > kMargin)) {
                // scores already relative to m_run: raise it by the row's excess
                float rmax = fmaxf(lmax, __shfl_xor(lmax, 16));
                rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
                const float up = fmaxf(rmax, 0.f);
                const float corr = fast_exp2(-up);
                m_run[hd] += up;
                negm[hd] = f32x4{-m_run[hd], -m_run[hd], -m_run[hd], -m_run[hd]};
                s0 -= up;
                s1 -= up;
                lacc[hd] *= corr;
#pragma unroll
                for (int i = 0; i < ND; ++i) oacc[hd][i] *= corr;
            }
            float p[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[r] = fast_exp2(s0[r]);
                p[4 + r] = fast_exp2(s1[r]);
            }
            const u32x4 pw4 = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                               pack_bf16x2(p[6], p[7])};
            pb[hd] = __builtin_bit_cast(bf16x8, pw4);
            lacc[hd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes, pb[hd], FIRST ? zero : lacc[hd], 0, 0, 0);
        }
        // V^T operands by transposing reads: this lane addresses key row 4 gq + (n >> 2)
        // (block 0) and 16 + 4 gq + (n >> 2) (block 1), dims 16 dt + 4 (n & 3)
        // (one base per pair, opaque, so that the steps stay immediate offsets)
        int vo = (int)(pr & (kNs - 1)) * R::SLOT + R::KPART + R::vofs_tr(4 * gq + (n >> 2), 0, n & 3);
        asm volatile("" : "+v"(vo));
        const uint16_t* vb = ring + vo;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) {
            const s16x4 v0 = lds_read_tr(vb + dt * R::V_DT);
            const s16x4 v1 = lds_read_tr(vb + R::V_KEY16 + dt * R::V_DT);
            const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
            const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
#pragma unroll
            for (int hd = 0; hd < 2; ++hd)
                oacc[hd][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[hd], FIRST ? zero : oacc[hd][dt],
                                                                       0, 0, 0);
        }
    };

    // pairs 0 .. last, two per step
    const int64_t last = pmax >> 5;
    const int64_t wlast = wmax >> 5;
    u32x4 kreg[2][KCH];
    u32x4 vreg[2][KCH];
    load_pair(0, kreg[0], vreg[0]);
    if (last >= 1) load_pair(1, kreg[1], vreg[1]);
    store_pair(0, kreg[0], vreg[0]);
    if (last >= 1) store_pair(1, kreg[1], vreg[1]);
    __syncthreads();
    for (int64_t p0 = 0; p0 <= last; p0 += 2) {
        const bool next0 = p0 + 2 <= last, next1 = p0 + 3 <= last;
        if (next0) load_pair(p0 + 2, kreg[0], vreg[0]);
        if (next1) load_pair(p0 + 3, kreg[1], vreg[1]);
        if (p0 == 0) {
            attend(std::true_type{}, 0);
        } else if (p0 <= wlast) {
            attend(std::false_type{}, p0);
        }
        if (p0 + 1 <= wlast) attend(std::false_type{}, p0 + 1);
        // the slots of pairs p0 + 2, p0 + 3 held pairs p0 - 2, p0 - 1, which
        // every wave finished before the previous barrier
        if (next0) store_pair(p0 + 2, kreg[0], vreg[0]);
        if (next1) store_pair(p0 + 3, kreg[1], vreg[1]);
        __syncthreads();
    }

    // ---- normalise and store (copies past T_out fall outside the resource)
    const rsrc_t ro = make_rsrc((uint16_t*)a.o_out + q_seq + c0 * a.Hq * D, (T_out - c0) * qrow_b - h0 * D * 2);
    // an invalid position's NaN is written as a bit pattern (this file is
    // compiled assuming no NaN arithmetic)
    const uint32_t nan_mask = myp_raw == -2 ? 0xffffffffu : 0u;
    constexpr uint32_t kNanPair = 0x7fc07fc0u;
    // lane (n, gq) holds dims 16 dt + 4 gq .. + 3 of copy n; a permlane16
    // swap between the rows gq and gq ^ 1 of each dt pair leaves it 8
    // consecutive dims (32 m + 8 ((gq & 1) * 2 + (gq >> 1))): 16-byte stores
    // (the NaN mask belongs to the copy, the same in both partner lanes)
#pragma unroll
    for (int hd = 0; hd < 2; ++hd) {
        const float inv = __builtin_amdgcn_rcpf(lacc[hd][0]);
#pragma unroll
        for (int m = 0; m < ND / 2; ++m) {
            const f32x4 oa = oacc[hd][2 * m], ob = oacc[hd][2 * m + 1];
            u32x4 w;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const auto r = __builtin_amdgcn_permlane16_swap(
                    pack_bf16x2(oa[2 * i] * inv, oa[2 * i + 1] * inv),
                    pack_bf16x2(ob[2 * i] * inv, ob[2 * i + 1] * inv), false, false);
                w[i] = (r[0] & ~nan_mask) | (kNanPair & nan_mask);
                w[2 + i] = (r[1] & ~nan_mask) | (kNanPair & nan_mask);
            }
            buf_store16(w, ro, (uint32_t)(n * qrow_b + hd * D * 2 + 2 * (32 * m + 8 * ((gq & 1) * 2 + (gq >> 1)))));
        }
    }
}

}  // namespace

bool copies_flash_applies(const CopiesParams& p)
{
    return p.dt == Dt::BF16 && (p.Hq / p.Hkv) % 4 == 0;
}

hipError_t launch_copies_flash(const CopiesParams& p, hipStream_t s)
{
    const int hblocks = (p.Hq / p.Hkv) / 4;
    const int n_tiles = (int)((p.T_out + 31) / 32);
    const int64_t n_wg = (int64_t)n_tiles * p.B * p.Hkv * hblocks;
    if (p.D == 64)
        hipLaunchKernelGGL((copies_flash_kernel<64>), dim3((unsigned)n_wg), dim3(256), 0, s, p, n_tiles, hblocks);
    else
        hipLaunchKernelGGL((copies_flash_kernel<128>), dim3((unsigned)n_wg), dim3(256), 0, s, p, n_tiles, hblocks);
    return hipGetLastError();
}

}  // namespace orthros
