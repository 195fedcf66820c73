// swa_ring.hip -- streaming variant of the base-stream sliding-window
// attention for bf16 and windows w <= 129 (the pages' w = 128), any group
// size.  Same result as swa_bf16_kernel in swa_prefill.hip
// ("Orthros:阶段感知异构注意力精读笔记" §2.3 Eq. (4), the fused cache
// write of §2.1), organised for HBM streaming:
//
//   - a workgroup of 4 waves walks one segment of one KV head's sequence,
//     32 rows at a time, for the block of query heads it serves: wave
//     (sub-tile s, column c) owns rows 16 s .. 16 s + 15 of its heads.  In
//     blocks of 4 heads (groups that are multiples of 4) column c is a head
//     pair, so every K/V fragment it reads from LDS feeds two MFMAs; in
//     blocks of 2 (other even groups) it is one head; with one head (odd
//     groups) the two columns split the head dims of O (each computes the
//     scores of all of them).  Two workgroups share a CU (2 waves per SIMD,
//     up to 256 registers each);
//   - the window of a 32-row tile spans at most 5 blocks of 32 keys, kept in
//     a 5-slot ring of K and V blocks in LDS (16 KB per slot at d = 128,
//     XOR-swizzled instead of padded so that two workgroups fit in one CU's
//     160 KB): each K/V byte is read from HBM once, and the 128-key halo
//     stays on chip between tiles;
//   - while a tile computes, the next tile's new K/V block and its Q rows
//     are already in flight into registers (one-tile software pipeline);
//   - within a tile the diagonal pair goes first, so the running maxima
//     and the accumulators start from it (no clearing, no rescale), and
//     its causal mask is a fixed bias in the first S MFMA's accumulator;
//   - softmax keeps a running maximum per row but rescales the accumulator
//     only when a block's maximum exceeds it by more than 2^8 (the row sum
//     and the accumulator share the stale maximum, so the final quotient is
//     unchanged; probabilities stay <= 256, well inside bf16 and fp32);
//   - the workgroup that brings a block in writes it to the cache.

#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "pair_tile.h"

namespace orthros {
namespace {

constexpr float kRescaleMargin = 8.0f;   // log2 units

// 16x16x32 form: the window of a 32-row tile spans 10 blocks of 16 keys =
// 5 aligned pairs, kept in a 5-slot ring of 32-key pair slots (pair_tile.h).
template <int D>
struct Pair : PairTile<D> {
    static constexpr int NSLOT = 5;
};

// Output-copy side of the fused kernel: the copy's raw query and its
// scale-offset, where the partials go, and the copy positions of the batch
// rows b0 .. b0 + nb - 1 this launch covers.
struct GlobalArgs {
    const void* q_out;    // [B][Hq][D]
    const void* alpha_out;
    const void* beta_out;
    float* ws_part;       // [B][Hq][1][n_seg][D+2]: m (exp2 units), l, acc
    int32_t* ws_len;      // [B]: the copy position, for the merge
};

template <int D, bool GQ, int HPW, int DS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void swa_ring_kernel(
    SwaParams a, int n_tiles, int hblocks, int n_seg, int tps, int b0, GlobalArgs ga, PosBlock pos)
{
    using R = Pair<D>;
    constexpr int NS = R::NSLOT;
    constexpr int NT = 256;
    constexpr int C16 = D / 8;                 // 16-byte chunks per row
    constexpr int NQ = D / 32;                 // MFMA k-steps over the head dim (32 each)
    constexpr int ND = D / 16;                 // 16-wide d tiles of O^T
    constexpr int NDW = ND / DS;               // ... of one wave
    constexpr int HB = DS == 1 ? 2 * HPW : HPW;   // query heads of the workgroup
    static_assert((HPW == 2 && DS == 1) || (HPW == 1 && (DS == 1 || DS == 2)), "wave layout");
    constexpr int KCH = 32 * C16 / NT;         // K (and V) chunks per thread per pair
    static_assert(KCH >= 1, "head dim");
    __shared__ __align__(16) uint16_t ring[NS * R::SLOT];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    // 16-row sub-tile, and the wave's column of the block: its HPW heads
    // (DS = 1), or its half of the head dims (DS = 2)
    const int hp = wv & 1, sub = wv >> 1;
    const int n = lane & 15, gq = lane >> 4;
    int64_t id = blockIdx.x;
    const int seg = (int)(id % n_seg);
    id /= n_seg;
    const int hb = (int)(id % hblocks);
    id /= hblocks;
    const int g = (int)(id % a.Hkv);
    const int b = b0 + (int)(id / a.Hkv);
    const int G = a.Hq / a.Hkv;
    const int hbase = g * G + hb * HB;
    const int h0 = hbase + (DS == 1 ? HPW * hp : 0);   // the wave's heads: h0 .. h0 + HPW - 1
    const int dt0 = DS == 1 ? 0 : hp * NDW;             // its first 16-wide d tile of O^T
    const int64_t T = a.T;
    const int W = a.window;
    const int t_begin = seg * tps;
    const int t_end = t_begin + tps < n_tiles ? t_begin + tps : n_tiles;
    if (t_begin >= t_end) return;
    const bool writer = (hb == 0);
    const float qs = a.qscale;

    const uint16_t* __restrict__ al = (const uint16_t*)a.alpha + (int64_t)h0 * D;
    const uint16_t* __restrict__ be = (const uint16_t*)a.beta + (int64_t)h0 * D;
    const int64_t qrow_b = (int64_t)a.Hq * D * 2, krow_b = (int64_t)a.Hkv * D * 2;
    const int64_t kv_seq = (int64_t)b * T * a.Hkv * D + (int64_t)g * D;
    const int64_t q_seq = (int64_t)b * T * a.Hq * D + (int64_t)h0 * D;
    const int64_t c_seq = ((int64_t)b * a.Hkv + g) * a.cap * D;

    // staging of one pair (32 new keys): K by LDS unit, thread tid taking
    // units tid + 256 j of the pair's K part (PairTile::k_unit: 8
    // threads read 128 contiguous bytes of a row, and the LDS stores are
    // contiguous); V item tid + 256 j -> (row, chunk) by PairTile::vitem,
    // item + 256 being the same chunk 16 rows on (KCH is 2 only at d = 128)
    static_assert(KCH == 1 || NT / C16 == 16, "staging step");
    auto load_pair = [&](int64_t pr, u32x4 (&kr)[KCH], u32x4 (&vr)[KCH]) {
        const int64_t kbase = pr * 32;
        const int64_t avail = (T - kbase) * krow_b - g * D * 2;
        const rsrc_t rk = make_rsrc((const uint16_t*)a.k + kv_seq + kbase * a.Hkv * D, avail);
        const rsrc_t rv = make_rsrc((const uint16_t*)a.v + kv_seq + kbase * a.Hkv * D, avail);
        int vr_row, vr_c;
        R::vitem(tid, vr_row, vr_c);
#pragma unroll
        for (int j = 0; j < KCH; ++j) {
            int kr_row, kr_c;
            R::k_unit(tid + NT * j, kr_row, kr_c);
            kr[j] = buf_load16(rk, (uint32_t)(kr_row * krow_b + 16 * kr_c));
            vr[j] = buf_load16(rv, (uint32_t)((vr_row + 16 * j) * krow_b + 16 * vr_c));
        }
    };
    auto store_pair = [&](int64_t pr, bool own, const u32x4 (&kr)[KCH], const u32x4 (&vr)[KCH]) {
        uint16_t* Ks = ring + (int)(pr % NS) * R::SLOT;
        uint16_t* Vt = Ks + R::KPART;
        // recompute the thread's LDS offsets here rather than keep them live
        // across the tile (they would only take registers the tile needs)
        int t = tid;
        asm volatile("" : "+v"(t));
        int vr_row, vr_c;
        R::vitem(t, vr_row, vr_c);
#pragma unroll
        for (int j = 0; j < KCH; ++j) {
            *(u32x4*)(Ks + 8 * (t + NT * j)) = kr[j];
            *(u32x4*)(Vt + R::vofs16(vr_row, vr_c) + j * R::V_KEY16) = vr[j];
        }
        if (own && writer) {
            const int64_t kbase = pr * 32;
            const int64_t avail = (T - kbase) * D * 2;
            const rsrc_t ck = make_rsrc((uint16_t*)a.k_cache + c_seq + kbase * D, avail);
            const rsrc_t cv = make_rsrc((uint16_t*)a.v_cache + c_seq + kbase * D, avail);
#pragma unroll
            for (int j = 0; j < KCH; ++j) {
                int kr_row, kr_c;
                R::k_unit(t + NT * j, kr_row, kr_c);
                buf_store16(kr[j], ck, (uint32_t)(kr_row * D * 2 + 16 * kr_c));
                buf_store16(vr[j], cv, (uint32_t)((vr_row + 16 * j) * D * 2 + 16 * vr_c));
            }
        }
    };
    // raw Q rows of the wave's 16-row sub-tile for its heads:
    // lane (n, gq) holds q[row][head][32 i + 8 gq + 0..7]
    auto load_q = [&](int64_t r0, u32x4 (&qr)[HPW][NQ]) {
        const rsrc_t rq = make_rsrc((const uint16_t*)a.q + q_seq + r0 * a.Hq * D,
                                    (T - r0) * qrow_b - h0 * D * 2);
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd)
#pragma unroll
            for (int i = 0; i < NQ; ++i)
                qr[hd][i] = buf_load16(rq, (uint32_t)(n * qrow_b + hd * D * 2 + 64 * i + 16 * gq));
    };
    // q * alpha + beta, packed as MFMA B operands (the softmax scale is
    // applied to the scores inside the exponent instead).  Element e is one
    // v_dot2_f32_bf16 of (q_e masked to its half of the word) with the alpha
    // word, accumulated onto beta_e.  All alpha/beta loads go out together
    // (one L1/L2 round trip); the pair loop's registers are free by then.
    auto scale_offset = [&](const u32x4 (&qr)[HPW][NQ], bf16x8 (&qf)[HPW][NQ]) {
        u32x4 av[HPW][NQ], bv[HPW][NQ];
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd)
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int d0 = hd * D + 32 * i + 8 * gq;
                av[hd][i] = *(const u32x4*)(al + d0);
                bv[hd][i] = *(const u32x4*)(be + d0);
            }
#pragma unroll
        for (int hd = 0; hd < HPW; ++hd)
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                u32x4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = qr[hd][i][e], aw = av[hd][i][e], bw = bv[hd][i][e];
                    const bf16x2 a2 = __builtin_bit_cast(bf16x2, aw);
                    r[e] = pack_bf16x2(
                        __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w & 0xffffu), a2, bf16_lo(bw),
                                                        false),
                        __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w & 0xffff0000u), a2,
                                                        bf16_hi(bw), false));
                }
                qf[hd][i] = __builtin_bit_cast(bf16x8, r);
            }
    };

    u32x4 kreg[KCH];
    u32x4 vreg[KCH];
    u32x4 qraw[HPW][NQ];
    bf16x8 qf[HPW][NQ];
    const bf16x8 kOnes = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});

    // Causal mask of the diagonal pair (keys q0 .. q0 + 31 of a tile against
    // the wave's rows q0 + 16 sub + n): the same for every tile.  -inf where
    // the key is outside the row's window, else 0; it enters the pair's
    // first S MFMA as the accumulator.
    f32x4 dbias[2];
    {
        const int c = n - W + 1 + 16 * sub - 4 * gq;
        const uint32_t wm1 = (uint32_t)(W - 1);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dbias[0][r] = (uint32_t)(r - c) > wm1 ? -INFINITY : 0.f;
            dbias[1][r] = (uint32_t)(16 + r - c) > wm1 ? -INFINITY : 0.f;
        }
    }

    // ---- the output copy's global query (Eq. (5)), fused: wave w < HB
    // serves head hbase + w over every key of the pairs this workgroup
    // brings in (keys j <= P only); the other waves have no copy head.  Lanes (group kg, chunk kc): a group of LPK lanes
    // covers STEPS keys, each lane dotting its 16-byte K chunk with the
    // scaled query for every key of the group, in the order s ^ m with
    // m = kc / 2; a transposing DPP reduction then leaves lane (kg, kc)
    // with the full score of key STEPS kg + m (both lanes of a pair).  The
    // online softmax state (gm) is wave-uniform, gl is per lane (each key
    // counted twice); P goes to scalar registers as bf16 pairs, and lane l
    // accumulates rows l + 64 r of V^T P with v_dot2_f32_bf16, reading its
    // V^T row four keys at a time by transposing LDS reads.
    constexpr int LPK = D / 8;                  // lanes per key (16-byte chunks of a row)
    constexpr int STEPS = 32 * LPK / 64;        // keys of the pair per lane group
    constexpr int RPL = D / 64;                 // V^T rows per lane
    static_assert(STEPS == 8 || STEPS == 4, "head dim");
    const int kg = lane / LPK, kc = lane % LPK, km = kc >> 1;
    u32x4 gqq = u32x4{0u, 0u, 0u, 0u};          // q' * alpha' + beta', d = 8 kc .. 8 kc + 7
    float gm = kNegBig, gl = 0.f, gacc[RPL];
#pragma unroll
    for (int r = 0; r < RPL; ++r) gacc[r] = 0.f;
    int64_t P = -1;
    const bool gwave = GQ && (HB == 4 || wv < HB);   // wave-uniform
    if (gwave) {
        const int hg = hbase + wv;
        P = pos.v[b - b0];
        const int64_t o = (int64_t)hg * D + 8 * kc;
        const u32x4 qw = *(const u32x4*)((const uint16_t*)ga.q_out + (int64_t)b * a.Hq * D + o);
        const u32x4 aw = *(const u32x4*)((const uint16_t*)ga.alpha_out + o);
        const u32x4 bw = *(const u32x4*)((const uint16_t*)ga.beta_out + o);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t w = qw[e], av = aw[e], bv = bw[e];
            gqq[e] = pack_bf16x2(__builtin_fmaf(bf16_lo(w), bf16_lo(av), bf16_lo(bv)),
                                 __builtin_fmaf(bf16_hi(w), bf16_hi(av), bf16_hi(bv)));
        }
    }
    auto global_pair = [&](int64_t pr) {
        const uint16_t* Ks = ring + (int)(pr % NS) * R::SLOT;
        // keys past P only in the pair that holds P: lim = last valid key of the pair
        const int64_t lim64 = P - pr * 32;
        const int lim = lim64 < 31 ? (int)lim64 : 31;
        float v[STEPS];
#pragma unroll
        for (int st = 0; st < STEPS; ++st) {
            const u32x4 kw = *(const u32x4*)(Ks + R::kofs(kg * STEPS + (st ^ km), kc));
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t x = kw[e], y = gqq[e];
                part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y),
                                                       part, false);
            }
            v[st] = part;
        }
        // slot s holds key s ^ m; each stage adds the partner's slot that
        // holds the same key and halves the slots (partner m' = m ^ 4, m ^ 3,
        // m ^ 1, m)
        if constexpr (STEPS == 8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] += dpp_mov<kDppRor8>(v[j + 4]);
        }
        v[0] += dpp_mov<kDppHalfMirror>(v[3]);
        v[1] += dpp_mov<kDppHalfMirror>(v[2]);
        v[0] += dpp_mov<kDppXor2>(v[1]);
        v[0] += dpp_mov<kDppXor1>(v[0]);
        const int key = kg * STEPS + km;
        const float sc = key <= lim ? v[0] : -INFINITY;
        // pair maximum: over the keys of a row of 16 lanes, then over the rows
        float lmax = fmaxf(sc, dpp_mov<kDppXor2>(sc));
        lmax = fmaxf(lmax, dpp_mov<kDppHalfMirror>(lmax));
        lmax = fmaxf(lmax, dpp_mov<kDppRor8>(lmax));
        lmax = wave_max_of_rows(lmax) * qs;
        if (lmax > gm + kRescaleMargin) {
            const float corr = fast_exp2(gm - lmax);
            gm = lmax;
            gl *= corr;
#pragma unroll
            for (int r = 0; r < RPL; ++r) gacc[r] *= corr;
        }
        const float p = fast_exp2(__builtin_fmaf(sc, qs, -gm));
        gl += p;
        // bf16 pairs (keys 2 j, 2 j + 1): the partner m ^ 1 sits at kc ^ 2;
        // lanes with m even hold them in order
        const int wrd = (int)pack_bf16x2(p, dpp_mov<kDppXor2>(p));
        uint32_t pw[16];
#pragma unroll
        for (int j = 0; j < 16; ++j)
            pw[j] = (uint32_t)__builtin_amdgcn_readlane(wrd, LPK * ((2 * j) / STEPS) + 2 * ((2 * j) % STEPS));
        // read i: this lane addresses key 4 i + (n >> 2), dims 16 (gq + 4 r) + 4 (n & 3),
        // and receives keys 4 i .. 4 i + 3 of V^T row lane + 64 r.  One base
        // per pair (opaque, so that the steps stay immediate offsets).
        int vo = (int)(pr % NS) * R::SLOT + R::KPART + R::vofs_tr(n >> 2, gq, n & 3);
        asm volatile("" : "+v"(vo));
        const uint16_t* vb = ring + vo;
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const s16x4 vv =
                    lds_read_tr(vb + (i >> 1) * R::V_KEY8 + (i & 1) * R::V_KEY4 + 4 * r * R::V_DT);
                const u32x2 vw = __builtin_bit_cast(u32x2, vv);
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    // through scalars: a bit_cast of a vector element directly
                    // miscompiles (every dot2 then reads element 0)
                    const uint32_t x = vw[e], y = pw[2 * i + e];
                    gacc[r] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                                              __builtin_bit_cast(bf16x2, y), gacc[r], false);
                }
            }
        }
    };

    {   // prologue: the first tile's window (the halo pairs are not owned),
        // every pair's loads in flight at once
        constexpr int NPRO = (kRingMaxWindow - 1 + 31) / 32 + 1;   // pairs of a window, at most
        static_assert(NPRO <= NS, "ring slots");
        const int64_t q0 = (int64_t)t_begin * 32;
        const int64_t lo = q0 - W + 1 > 0 ? q0 - W + 1 : 0;
        const int64_t p0 = lo >> 5, p1 = q0 >> 5;
        load_q(q0 + 16 * sub, qraw);
        u32x4 kp[NPRO][KCH], vp[NPRO][KCH];
#pragma unroll
        for (int i = 0; i < NPRO; ++i)
            if (p0 + i <= p1) load_pair(p0 + i, kp[i], vp[i]);
#pragma unroll
        for (int i = 0; i < NPRO; ++i)
            if (p0 + i <= p1) store_pair(p0 + i, p0 + i == p1, kp[i], vp[i]);
        scale_offset(qraw, qf);
        __syncthreads();
    }

    for (int tile = t_begin; tile < t_end; ++tile) {
        const int64_t q0 = (int64_t)tile * 32;
        const bool has_next = tile + 1 < t_end;
        if (has_next) {
            load_pair((q0 >> 5) + 1, kreg, vreg);
            load_q(q0 + 32 + 16 * sub, qraw);
        }
        const int64_t lo = q0 - W + 1 > 0 ? q0 - W + 1 : 0;
        const int r0 = 16 * sub;                    // wave's first row relative to q0

        f32x4 oacc[HPW][NDW];
        f32x4 lacc[HPW];                            // row sums of the bf16 P, from an all-ones V^T tile
        float m_run[HPW];                           // running maxima, in scaled (exp2) units
        // One pair of 16-key blocks against the wave's heads.  The diagonal pair
        // goes first: every row has its own key there, so its row maxima
        // start the running maxima, and its MFMAs start the accumulators
        // from zero (no clearing, no rescale).
        auto attend = [&](auto first_tag, int64_t pr) {
            constexpr bool FIRST = decltype(first_tag)::value;
            // two K bases per pair, for even and odd k-steps (opaque, so that
            // the steps stay immediate offsets)
            int ko0 = (int)(pr % NS) * R::SLOT + R::kofs(n, gq);
            int ko1 = (int)(pr % NS) * R::SLOT + R::kofs(n, 4 + gq);
            asm volatile("" : "+v"(ko0), "+v"(ko1));
            const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 s[HPW][2];
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const uint16_t* kb = ring + ((i & 1) ? ko1 : ko0) + (i >> 1) * R::K_STEP2;
                const bf16x8 k0 = *(const bf16x8*)kb;
                const bf16x8 k1 = *(const bf16x8*)(kb + R::K_KEY16);
#pragma unroll
                for (int hd = 0; hd < HPW; ++hd) {
                    const f32x4 c0 = i ? s[hd][0] : (FIRST ? dbias[0] : zero);
                    const f32x4 c1 = i ? s[hd][1] : (FIRST ? dbias[1] : zero);
                    s[hd][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[hd][i], c0, 0, 0, 0);
                    s[hd][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[hd][i], c1, 0, 0, 0);
                }
            }
            // s[.][0][r]: key 32 pr + 4 gq + r, s[.][1][r]: key 32 pr + 16 + 4 gq + r; row r0 + n (relative to q0)
            if constexpr (!FIRST) {
                const int dj = (int)(pr * 32 - q0) - r0;
                const bool full = (dj + 31 <= 0) && (dj >= 15 - W + 1);
                if (!full) {
                    // key dj + 4 gq + e (e = r or 16 + r) is in row n's window iff
                    // n - w + 1 <= key <= n, i.e. (unsigned)(e - c) <= w - 1 with c = n - w + 1 - dj - 4 gq
                    const int c = n - W + 1 - dj - 4 * gq;
                    const uint32_t wm1 = (uint32_t)(W - 1);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool m0 = (uint32_t)(r - c) > wm1, m1 = (uint32_t)(16 + r - c) > wm1;
#pragma unroll
                        for (int hd = 0; hd < HPW; ++hd) {
                            if (m0) s[hd][0][r] = -INFINITY;
                            if (m1) s[hd][1][r] = -INFINITY;
                        }
                    }
                }
            }
            bf16x8 pb[HPW];
#pragma unroll
            for (int hd = 0; hd < HPW; ++hd) {
                const f32x4 s0 = s[hd][0], s1 = s[hd][1];
                float lmax = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                                   fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
                lmax *= qs;
                if constexpr (FIRST) {
                    float rmax = fmaxf(lmax, __shfl_xor(lmax, 16));
                    m_run[hd] = fmaxf(rmax, __shfl_xor(rmax, 32));
                } else if (__any(lmax > m_run[hd] + kRescaleMargin)) {
                    float rmax = fmaxf(lmax, __shfl_xor(lmax, 16));
                    rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
                    const float m_new = fmaxf(m_run[hd], rmax);
                    const float corr = fast_exp2(m_run[hd] - m_new);
                    m_run[hd] = m_new;
                    lacc[hd] *= corr;
#pragma unroll
                    for (int i = 0; i < NDW; ++i) oacc[hd][i] *= corr;
                }
                float p[8];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[r] = fast_exp2(__builtin_fmaf(s0[r], qs, -m_run[hd]));
                    p[4 + r] = fast_exp2(__builtin_fmaf(s1[r], qs, -m_run[hd]));
                }
                const u32x4 pw = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                  pack_bf16x2(p[6], p[7])};
                pb[hd] = __builtin_bit_cast(bf16x8, pw);
                lacc[hd] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kOnes, pb[hd], FIRST ? zero : lacc[hd], 0, 0, 0);
            }
            // V^T operands by transposing reads: this lane addresses key row
            // 4 gq + (n >> 2) of each block, dims 16 (dt0 + dt) + 4 (n & 3).
            // One base per pair (opaque, so that the steps stay immediate
            // offsets).
            int vo = (int)(pr % NS) * R::SLOT + R::KPART + R::vofs_tr(4 * gq + (n >> 2), dt0, n & 3);
            asm volatile("" : "+v"(vo));
            const uint16_t* vb = ring + vo;
#pragma unroll
            for (int dt = 0; dt < NDW; ++dt) {
                const u32x2 w0 = __builtin_bit_cast(u32x2, lds_read_tr(vb + dt * R::V_DT));
                const u32x2 w1 = __builtin_bit_cast(u32x2, lds_read_tr(vb + R::V_KEY16 + dt * R::V_DT));
                const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{w0[0], w0[1], w1[0], w1[1]});
#pragma unroll
                for (int hd = 0; hd < HPW; ++hd)
                    oacc[hd][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pb[hd], FIRST ? zero : oacc[hd][dt],
                                                                           0, 0, 0);
            }
        };
        attend(std::true_type{}, q0 >> 5);
        for (int64_t pr = lo >> 5; pr < (q0 >> 5); ++pr) attend(std::false_type{}, pr);
        // The next tile's scale-offset runs before this tile's O stores: the
        // vector-memory counter retires in issue order, so waiting for the
        // alpha/beta loads after the stores would also wait for the stores.
        __builtin_amdgcn_sched_barrier(0);
        // the copy's step on this tile's own pair (LDS and ALU only) runs
        // while the next tile's Q rows may still be arriving
        if constexpr (GQ) {
            if (gwave && q0 <= P) global_pair(q0 >> 5);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (has_next) scale_offset(qraw, qf);
        __builtin_amdgcn_sched_barrier(0);
        // ---- normalise and store the sub-tile (rows >= T fall outside the resource)
        {
            const int64_t r0g = q0 + r0;
            const rsrc_t ro = make_rsrc((uint16_t*)a.o + q_seq + r0g * a.Hq * D,
                                        (T - r0g) * qrow_b - h0 * D * 2);
            // lane (n, gq) holds dims 16 dt + 4 gq .. + 3 of row n; a
            // permlane16 swap between the rows gq and gq ^ 1 of each dt pair
            // leaves it 8 consecutive dims (32 m + 8 ((gq & 1) * 2 + (gq >> 1))),
            // so the stores are 16 bytes a lane and 64 contiguous bytes a row
#pragma unroll
            for (int hd = 0; hd < HPW; ++hd) {
                const float inv = __builtin_amdgcn_rcpf(lacc[hd][0]);
#pragma unroll
                for (int m = 0; m < NDW / 2; ++m) {
                    const f32x4 oa = oacc[hd][2 * m], ob = oacc[hd][2 * m + 1];
                    u32x4 w;
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const auto r = __builtin_amdgcn_permlane16_swap(
                            pack_bf16x2(oa[2 * i] * inv, oa[2 * i + 1] * inv),
                            pack_bf16x2(ob[2 * i] * inv, ob[2 * i + 1] * inv), false, false);
                        w[i] = r[0];
                        w[2 + i] = r[1];
                    }
                    buf_store16(w, ro, (uint32_t)(n * qrow_b + hd * D * 2 +
                                                  2 * (16 * dt0 + 32 * m + 8 * ((gq & 1) * 2 + (gq >> 1)))));
                }
            }
        }
        __syncthreads();   // every wave is done with the slot the next pair replaces
        if (has_next) store_pair((q0 >> 5) + 1, true, kreg, vreg);
        __syncthreads();
    }
    if (gwave) {
        float* part = ga.ws_part + (((int64_t)b * a.Hq + hbase + wv) * n_seg + seg) * (D + 2);
#pragma unroll
        for (int r = 0; r < RPL; ++r) part[2 + lane + 64 * r] = gacc[r];
        // every key was counted by the two lanes of its pair
        int ln = lane;
        asm volatile("" : "+v"(ln));   // recompute the exchange addresses here, not across the loop
        float lsum = group_sum<16>(gl);
        lsum += lane_xor(lsum, ln, 16);
        lsum += lane_xor(lsum, ln, 32);
        if (lane == 0) {
            part[0] = gm;
            part[1] = 0.5f * lsum;
        }
    }
    if constexpr (GQ) {
        if (seg == 0 && g == 0 && hb == 0 && tid == 0) ga.ws_len[b] = (int32_t)P;
    }
}

}  // namespace

RingGeom ring_geometry(int B, int Hq, int Hkv, int64_t T)
{
    RingGeom r;
    r.hblocks = (Hq / Hkv) / ring_heads_per_block(Hq / Hkv);
    r.n_tiles = (int)((T + 31) / 32);
    const int64_t streams = (int64_t)B * Hkv * r.hblocks;
    constexpr int64_t kTargetWgs = 512;
    int n_seg = (int)((kTargetWgs + streams - 1) / streams);
    if (n_seg > r.n_tiles) n_seg = r.n_tiles;
    if (n_seg < 1) n_seg = 1;
    r.tps = (r.n_tiles + n_seg - 1) / n_seg;
    r.n_seg = (r.n_tiles + r.tps - 1) / r.tps;
    return r;
}

namespace {

template <int D, bool GQ>
void launch_ring_d(dim3 grid, const SwaParams& p, const RingGeom& r, int b0, const GlobalArgs& ga,
                   const PosBlock& pos, hipStream_t s)
{
    // groups of 4k: two heads a wave; of 2: one head a wave; odd: the two
    // waves of a sub-tile split the head dims
    const int hpb = ring_heads_per_block(p.Hq / p.Hkv);
    if (hpb == 4)
        hipLaunchKernelGGL((swa_ring_kernel<D, GQ, 2, 1>), grid, dim3(256), 0, s, p, r.n_tiles, r.hblocks, r.n_seg,
                           r.tps, b0, ga, pos);
    else if (hpb == 2)
        hipLaunchKernelGGL((swa_ring_kernel<D, GQ, 1, 1>), grid, dim3(256), 0, s, p, r.n_tiles, r.hblocks,
                           r.n_seg, r.tps, b0, ga, pos);
    else
        hipLaunchKernelGGL((swa_ring_kernel<D, GQ, 1, 2>), grid, dim3(256), 0, s, p, r.n_tiles, r.hblocks,
                           r.n_seg, r.tps, b0, ga, pos);
}

template <bool GQ>
hipError_t launch_ring(const SwaParams& p, const GlobalArgs& ga, const int64_t* pos_host, hipStream_t s)
{
    const RingGeom r = ring_geometry(p.B, p.Hq, p.Hkv, p.T);
    const int per_launch = GQ ? kPosPerLaunch : p.B;
    for (int b0 = 0; b0 < p.B; b0 += per_launch) {
        const int nb = p.B - b0 < per_launch ? p.B - b0 : per_launch;
        PosBlock pos;
        for (int i = 0; i < kPosPerLaunch; ++i) pos.v[i] = (GQ && i < nb) ? pos_host[b0 + i] : 0;
        const int64_t n_wg = (int64_t)nb * p.Hkv * r.hblocks * r.n_seg;
        if (p.D == 64)
            launch_ring_d<64, GQ>(dim3((unsigned)n_wg), p, r, b0, ga, pos, s);
        else
            launch_ring_d<128, GQ>(dim3((unsigned)n_wg), p, r, b0, ga, pos, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

// Workgroups of the streaming kernel: about two per CU of the 256, each
// walking an equal share of one (sequence, KV head, head block) stream.
hipError_t launch_swa_ring(const SwaParams& p, hipStream_t s)
{
    return launch_ring<false>(p, GlobalArgs{}, nullptr, s);
}

hipError_t launch_swa_ring_fused(const SwaParams& p, const XattnParams& x, hipStream_t s)
{
    const GlobalArgs ga{x.q_out, x.alpha_out, x.beta_out, x.ws_part, x.ws_len};
    const hipError_t e = launch_ring<true>(p, ga, x.pos, s);
    if (e != hipSuccess) return e;
    return launch_merge(x, s);
}

}  // namespace orthros
