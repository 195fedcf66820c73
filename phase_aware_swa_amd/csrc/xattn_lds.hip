// xattn_lds.hip -- the output copy's full-history cross-attention (prefill)
// and the decode step's copy and base token, for bf16, for gfx950: the cache
// streams through LDS by direct loads and the contractions run on MFMA.
//
// "Orthros:阶段感知异构注意力精读笔记" §2.3 Eq. (5): the copy at original
// position P attends over every cached key j <= P (§2.4: the mask follows the
// original position); its query is q_out * alpha_out + beta_out (§2.2).
//
// One query per head over the whole cache is a pure stream of K/V bytes
// (about 2 flop per byte per head), so the design is about keeping HBM busy:
//   - a stream is one (sequence, KV head, block of hg query heads): hg = 4
//     when the group size is a multiple of 4, else 2 or 1; the block's heads
//     are served at once, so every K/V byte is read from HBM once;
//   - the kernel is persistent, one workgroup per CU: the launch's keys, in
//     (sequence, stream, key) order, are cut into one equal run per
//     workgroup, and a run that crosses from one stream into the next is
//     worked as segments, each with its own partial records -- every
//     workgroup gets the same bytes whatever the mix of lengths, and writes
//     records for one to three segments (each wave holds one sequence per
//     lane and finds a segment's sequence with one ballot over the lanes'
//     prefix sums);
//   - a segment's keys stream through two 64 KB LDS slots in stages of 4
//     (d = 128) or 8 (d = 64) 32-key pairs, by buffer loads that write LDS
//     directly (16 per lane per stage, no register staging).  The stage
//     sequence runs on across segments, and stage t + 2 is issued into
//     stage t's slot as soon as every wave is done with it, while stage
//     t + 1 is still landing in the other slot: the load queue never runs
//     dry, and a new segment costs no pipeline refill.  The segment's query
//     rows and their scale-offsets come the same way into a small
//     double-buffered LDS area;
//   - the waits are explicit vmcnt counts: each wave counts what it issued
//     after a stage's loads (the next stage's loads and rows, partial
//     stores), and vector memory operations retire in issue order, so the
//     stage's wait lets exactly those stay in flight;
//   - each load instruction fills 1 KB of a slot in lane order, so each lane
//     fetches the cache chunk that belongs at its 16-byte unit of the pair
//     layout (PairTile's inverse maps: every instruction reads whole
//     128-byte lines, 8 key rows x 128 bytes, which the loads mark
//     non-temporal -- the cache is read once per call); the stage's buffer
//     range ends at the segment's last key, so keys past it land as zeros;
//   - pair p of a stage is consumed by wave p % 4: S^T = K Q^T and
//     O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 with the block's queries as
//     columns 0 .. hg - 1 of the B operand (the rest are zero: the MFMAs are
//     idle most of the time either way), V^T from the transposing LDS read,
//     online softmax per column in exp2 units with a lazy rescale;
//   - at a segment's last stage the 4 waves' states merge through LDS into
//     one (max, sum, weighted sum of values) record per head, in the layout
//     the LSE merge reads, padded so that the values start on a 128-byte
//     line.

#include <atomic>
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "pair_tile.h"

namespace orthros {
namespace {

// s_waitcnt lgkmcnt(0) alone: this wave's LDS accesses are done.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

constexpr float kMargin = 8.0f;                    // lazy-rescale margin, log2 units
constexpr int kStageBytes = 65536;                 // one LDS slot

__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ int64_t readlane64(int64_t x, int l)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)x >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Keys per workgroup when `total` keys are cut into nwg equal runs (at least
// kXattnLdsSegMin, so that a short call uses fewer workgroups).
__device__ __forceinline__ int64_t run_keys(int64_t total, int nwg)
{
    const int64_t e = (total + nwg - 1) / nwg;
    return e > kXattnLdsSegMin ? e : kXattnLdsSegMin;
}

// One segment: keys lo .. hi (len keys) of stream j = (KV head g, the block
// of query heads from h0) of sequence b, hi <= P (the copy's position), nst
// stages, its partial records under record id `id`.  In decode the keys are
// the history 0 .. L - 1 (L = cache_len[b]), and `win` marks a segment that
// holds keys of the base token's window [wlo, L - 1].  Key indices fit 32 bits (positions are below 2^31); cache
// offsets and positions in the launch's key order take 64.
struct Item {
    int b, g, h0, id, nst, len;
    int lo, hi, wlo;
    bool win;
};

// PT = XattnParams: prefill, the copy's positions by value in `pos`.
// PT = DecodeParams: a decode step, L = cache_len[b] read on the device; the
// kernel reads the history 0 .. L - 1 (key L, the new token's, is added by
// the merge from k_new / v_new), and the base token's heads ride along as
// query columns 4 .. 3 + hg of the same MFMAs (their keys are a subset of
// the copy's), leaving a second partial per head for the segments that hold
// its window.  Record ids of this launch start at rbase.
template <int D, typename PT>
__global__ __launch_bounds__(256) void xattn_lds_kernel(PT a, int b0, int nb, int rbase, int hg, int hblocks,
                                                        PosBlock pos)
{
    constexpr bool DEC = std::is_same<PT, DecodeParams>::value;
    using R = PairTile<D>;
    constexpr int NP = 128 / D * 4;       // pairs per stage: 64 KB
    constexpr int SK = 32 * NP;           // keys per stage
    constexpr int PAIRB = 32 * D * 2;     // bytes of one pair's K (or V) rows in the cache
    constexpr int JP = D / 32;            // loads per lane per pair: JH of K, then JH of V
    constexpr int JH = JP / 2;
    constexpr int LPS = NP * JP;          // direct loads per lane per stage
    constexpr int NQ = D / 32, ND = D / 16;
    constexpr int SLOTE = NP * R::SLOT;   // slot size in bf16 elements
    // the item's rows in LDS: 4 head rows of each of q_out, alpha_out,
    // beta_out (then q, alpha, beta of the base token in decode)
    constexpr int NREG = DEC ? 6 : 3;
    constexpr int HRE = 4 * D;            // elements per region
    constexpr int NST = D / 64 + 1;       // partial store instructions per wave, segment and kind
    constexpr int REC = D + kXattnLdsRecPad, AOFF = kXattnLdsRecPad;   // partial record layout
    constexpr int KINDS = DEC ? 2 : 1;    // records per head and id: the copy (then the base token)
    constexpr int NH = DEC ? 8 : 4;       // live query columns
    static_assert(SLOTE * 2 == kStageBytes && LPS == 16, "stage shape");
    __shared__ __align__(16) uint16_t lds[2 * SLOTE];
    __shared__ __align__(16) uint16_t qa[2][NREG * HRE];
    __shared__ __align__(16) float red[4][NH][D + 2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, gq = lane >> 4;
    // a stream is one KV head's block of hg = xattn_heads_per_wg(G) query
    // heads (4, or 2 or 1 when the group size G is not a multiple of 4;
    // hblocks = G / hg blocks per KV head): the block's heads are MFMA query
    // columns 0 .. hg - 1 (and hg more for the base token in decode)
    const int S = a.Hkv * hblocks;        // streams of a sequence
    const uint16_t* k_cache = (const uint16_t*)a.k_cache;
    const uint16_t* v_cache = (const uint16_t*)a.v_cache;

    // lane i < nb: sequence b0 + i, its copy position and its key count
    int Lv = -1;
    if constexpr (DEC) {
        // a length outside [0, max_len] gives the sequence no keys (the
        // merge turns it into NaN outputs and leaves cache_len alone)
        const int Lraw = lane < nb ? a.cache_len[b0 + lane] : -1;
        if (blockIdx.x == 0 && tid < nb) a.ws_len[b0 + tid] = Lraw;
        Lv = Lraw >= 0 && Lraw <= a.max_len ? Lraw : -1;
    } else {
        Lv = lane < nb ? (int)pos.v[lane] : -1;
        if (blockIdx.x == 0 && tid < nb) a.ws_len[b0 + tid] = Lv;
    }
    // Work split: the keys of every stream of the launch, in (sequence,
    // stream, key) order, cut into nwg runs of E consecutive keys; workgroup
    // w takes run w, which may cross from one stream into the next (each
    // piece is a segment with its own records).  Every workgroup gets the
    // same number of keys to within one, whatever the mix of lengths, and
    // writes records for only one or a few segments.  A segment of stream t
    // (t = sequence * S + stream, counted in the launch) in run w has record
    // id rbase + t + w: those of one stream are consecutive, and no two
    // segments share one.
    // keys per stream: the copy's 0 .. P in prefill; in decode the history
    // 0 .. L - 1 (the new token's key L comes from k_new / v_new in the
    // merge, which also appends it to the cache)
    constexpr int KX = DEC ? 0 : 1;
    const int64_t cnt = Lv >= 0 ? (int64_t)(Lv + KX) * S : 0;   // keys of sequence b0 + lane
    int64_t incl = cnt;                   // inclusive prefix sum over the lanes
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) {
        const int64_t t = __shfl_up(incl, x);
        if (lane >= x) incl += t;
    }
    const int64_t excl = incl - cnt;
    const int64_t total = readlane64(incl, 63);
    const int64_t E = run_keys(total, gridDim.x);
    if (blockIdx.x == 0) {
        // each stream's records for the merge: first id, first id holding
        // keys of the base token's window (decode), last id
        for (int t0 = 0; t0 < nb * S; t0 += 256) {
            const int t = t0 + tid;
            const int bl = t / S < 63 ? t / S : 63;
            const int L = __shfl(Lv, bl);
            const int64_t ex = __shfl(excl, bl);
            if (t < nb * S) {
                int32_t* rg = a.ws_rng + ((int64_t)b0 * S + t) * 3;
                const int nk = L + KX;            // the stream's keys
                if (L < 0 || nk == 0) {
                    rg[0] = 0;
                    rg[1] = 0;
                    rg[2] = -1;
                } else {
                    const int64_t P = ex + (int64_t)(t - bl * S) * nk;
                    int wlo = 0;
                    if constexpr (DEC) wlo = L - a.window + 1 > 0 ? L - a.window + 1 : 0;
                    rg[0] = rbase + t + (int)(P / E);
                    rg[2] = rbase + t + (int)((P + nk - 1) / E);
                    // no segment holds window keys when the window is the new key alone
                    rg[1] = wlo <= nk - 1 ? rbase + t + (int)((P + wlo) / E) : rg[2] + 1;
                }
            }
        }
    }
    // this workgroup's run: keys beg .. beg + run - 1 of the order (below
    // 2^30 keys: the launchers check it)
    const int64_t beg = (int64_t)blockIdx.x * E;
    const int run = (int)(beg + E < total ? E : total - beg);

    // the segment that starts at key rel of the run
    auto item_of = [&](int rel, Item& it) {
        const int64_t at = beg + rel;
        // its sequence: the last lane whose exclusive prefix is <= at (a
        // lane with no keys is never the last: the next one shares its prefix)
        const uint64_t m = __ballot(lane < nb && excl <= at);
        const int bl = __popcll(m) - 1;
        it.b = b0 + bl;
        const int L = __builtin_amdgcn_readlane(Lv, bl);
        // the key's place among the sequence's S * (L + KX) keys (below 2^32:
        // the launchers check S * cap)
        const uint32_t off = (uint32_t)(at - readlane64(excl, bl));
        const int j = (int)(off / (uint32_t)(L + KX));
        // (g only addresses the cache: a vector division, so that no scalar
        // reciprocal of hblocks is held across the loop)
        int hbv = hblocks;
        asm volatile("" : "+v"(hbv));
        it.g = (int)((unsigned)j / (unsigned)hbv);
        it.h0 = j * hg;                   // = g * G + (j - g * hblocks) * hg
        it.lo = (int)(off - (uint32_t)j * (uint32_t)(L + KX));
        const int last = L + KX - 1;      // the stream's last key
        it.hi = run - rel > last - it.lo ? last : it.lo + (run - rel) - 1;
        it.len = it.hi - it.lo + 1;
        it.nst = (it.hi - it.lo) / SK + 1;
        it.id = rbase + bl * S + j + (int)blockIdx.x;
        it.wlo = 0;
        it.win = false;
        if constexpr (DEC) {
            it.wlo = L - a.window + 1 > 0 ? L - a.window + 1 : 0;
            it.win = it.hi >= it.wlo;
        }
    };

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
    // stage st of item `it` into slot `sl`: load j of wave wv fills units
    // 256 j + 64 wv .. + 63 of the slot, i.e. part (j % JP) of pair j / JP
    auto issue = [&](const Item& it, int st, int sl) {
        const int64_t crow = ((int64_t)it.b * a.Hkv + it.g) * a.cap * D;
        const int k0 = it.lo + st * SK;
        const int64_t avail = (int64_t)(it.hi - k0 + 1) * D * 2;
        const i32x4 rk = buffer_words(k_cache + crow + (int64_t)k0 * D, avail);
        const i32x4 rv = buffer_words(v_cache + crow + (int64_t)k0 * D, avail);
        const uint16_t* dst = lds + sl * SLOTE + 64 * wv * 8;
#pragma unroll
        for (int j = 0; j < LPS; ++j) {
            const int pp = j / JP, jj = j % JP;
            if (jj < JH) load_lds16_nt(rk, koff[jj] + pp * PAIRB, 0, dst + 256 * j * 8);
            else load_lds16_nt(rv, voff[jj - JH] + pp * PAIRB, 0, dst + 256 * j * 8);
        }
    };
    // the item's query rows and scale-offsets into qa[q]: region i by wave
    // i % 4, one load instruction of D / 2 lanes each
    auto row_src = [&](const Item& it, int r) -> const uint16_t* {
        const int h0 = it.h0;
        const int64_t qrow = ((int64_t)it.b * a.Hq + h0) * D;
        if constexpr (DEC) {
            if (r == 3) return (const uint16_t*)a.q + qrow;
            if (r == 4) return (const uint16_t*)a.alpha + (int64_t)h0 * D;
            if (r == 5) return (const uint16_t*)a.beta + (int64_t)h0 * D;
        }
        return r == 0 ? (const uint16_t*)a.q_out + qrow
                      : (r == 1 ? (const uint16_t*)a.alpha_out : (const uint16_t*)a.beta_out) + (int64_t)h0 * D;
    };
    auto issue_rows = [&](const Item& it, int q) {
        // the wave index read afresh here: the region tests then cost a
        // compare at each call instead of scalar masks held across the loop
        int w0 = wv;
        asm volatile("" : "+s"(w0));
#pragma unroll
        for (int r = w0; r < NREG; r += 4) {
            // the block's hg rows; rows past them read as zeros
            const i32x4 rs = buffer_words(row_src(it, r), (int64_t)hg * D * 2);
            if (lane < HRE / 8) load_lds16(rs, 16 * lane, 0, &qa[q][r * HRE]);
        }
    };

    if (run <= 0) return;
    int pc = 0;                   // the segment being consumed starts at key pc of the run
    Item ci;
    item_of(pc, ci);
    // its record id only addresses the records: a vector register, like the
    // issue cursor's segment below
    asm volatile("" : "+v"(ci.id));
    int sc = 0, qc = 0;           // its stage; qc: parity of its row area
    Item ii = ci;                 // the segment being issued, its next stage and row area
    int pi = pc, si = 0, qi = 0;
    bool more = true;             // the issue cursor has stages left
    auto advance_issue = [&]() {
        if (++si < ii.nst) return;
        pi += ii.len;
        if (pi >= run) {
            more = false;
            return;
        }
        item_of(pi, ii);
        // the issue cursor's segment only feeds address arithmetic: it is
        // kept in vector registers (the same value in every lane), which
        // leaves the scalar file room for the rest without spilling (its
        // stage count and length stay scalar: the cursor's branches must
        // stay uniform)
        asm volatile("" : "+v"(ii.b), "+v"(ii.g), "+v"(ii.h0), "+v"(ii.lo), "+v"(ii.hi));
        si = 0;
        qi ^= 1;
    };
    // vector memory instructions this wave issued after the loads (and
    // rows) of the stage in slot 0 / 1: the stage's wait lets exactly those
    // stay in flight
    int after0 = 0, after1 = 0;
    const int rows_w = (NREG - wv + 3) / 4;   // row loads this wave issues
    auto issue_next = [&](int sl) {
        issue(ii, si, sl);
        const int k = LPS + (si == 0 ? rows_w : 0);
        if (sl == 0) {
            after0 = 0;
            after1 += k;
        } else {
            after1 = 0;
            after0 += k;
        }
        if (si == 0) issue_rows(ii, qi);
        advance_issue();
    };
    issue_next(0);
    if (more) issue_next(1);

    const bf16x8 kOnes = __builtin_bit_cast(bf16x8, u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 qf[NQ];
    f32x4 oacc[ND];
    f32x4 lacc = zero;
    float m_run = kNegBig;        // lane (n, .): the running maximum of head n of the block

    // one pair of the stage in `slot`: keys key0 .. key0 + 31, the last admissible hi
    auto attend = [&](const uint16_t* slot, int pp, int key0, int hi, int wlo, bool win) {
        int ko0 = pp * R::SLOT + R::kofs(n, gq), ko1 = pp * R::SLOT + R::kofs(n, 4 + gq);
        asm volatile("" : "+v"(ko0), "+v"(ko1));
        f32x4 s0 = zero, s1 = zero;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const uint16_t* kb = slot + ((i & 1) ? ko1 : ko0) + (i >> 1) * R::K_STEP2;
            const bf16x8 k0 = *(const bf16x8*)kb;
            const bf16x8 k1 = *(const bf16x8*)(kb + R::K_KEY16);
            s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[i], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[i], s1, 0, 0, 0);
        }
        // s0[r]: key key0 + 4 gq + r, s1[r]: key key0 + 16 + 4 gq + r (column n)
        if (key0 + 31 > hi) {
            const int lim = hi - key0 - 4 * gq;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (r > lim) s0[r] = -INFINITY;
                if (16 + r > lim) s1[r] = -INFINITY;
            }
        }
        if constexpr (DEC) {
            // the base token's columns 4 .. 3 + hg: keys below its window
            if (win && key0 < wlo) {
                const int lim = wlo - key0 < 64 ? wlo - key0 - 4 * gq : 64;
                if ((n >> 2) == 1) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (r < lim) s0[r] = -INFINITY;
                        if (16 + r < lim) s1[r] = -INFINITY;
                    }
                }
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

    for (int t = 0;; ++t) {
        // this wave's loads of stage t (and, at an item's first stage, its
        // rows) have landed -- what it issued after them may still be in
        // flight; after the barrier every wave's have
        wait_stages<1, LPS + 2 + 4 * NST>((t & 1) ? after1 : after0);
        block_barrier();
        const uint16_t* slot = lds + (t & 1) * SLOTE;
        if (sc == 0) {
            // a new item: its scale-offset queries (times qscale, the score
            // scale with log2(e), so scores come out of the MFMAs in exp2
            // units) as B operands -- lane (n, gq) holds head n of the
            // block (n < 4; in decode, n = 4..7: the base token's head
            // n - 4 when the item holds keys of its window; zero
            // otherwise), dims 32 i + 8 gq .. + 7 -- and fresh softmax states
            const float qs = a.qscale;
            const bool live = ((n >> 2) == 0 || (DEC && (n >> 2) == 1 && ci.win)) && (n & 3) < hg;
            const uint16_t* qr = qa[qc] + (DEC && (n >> 2) == 1 ? 3 * HRE : 0) + (n & 3) * D;
#pragma unroll
            for (int i = 0; i < NQ; ++i) {
                const int d0 = 32 * i + 8 * gq;
                const u32x4 qw = *(const u32x4*)(qr + d0);
                const u32x4 av = *(const u32x4*)(qr + HRE + d0);
                const u32x4 bv = *(const u32x4*)(qr + 2 * HRE + d0);
                u32x4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = qw[e], aw = av[e], bw = bv[e];
                    r[e] = pack_bf16x2(__builtin_fmaf(bf16_lo(w), bf16_lo(aw), bf16_lo(bw)) * qs,
                                       __builtin_fmaf(bf16_hi(w), bf16_hi(aw), bf16_hi(bw)) * qs);
                    r[e] = live ? r[e] : 0u;
                }
                qf[i] = __builtin_bit_cast(bf16x8, r);
            }
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) oacc[dt] = zero;
            lacc = zero;
            m_run = kNegBig;
        }
        // pair pp of the stage goes to wave pp % 4
#pragma unroll
        for (int pp = 0; pp < NP; ++pp) {
            const int key0 = ci.lo + sc * SK + 32 * pp;
            if ((pp & 3) == wv && key0 <= ci.hi) attend(slot, pp, key0, ci.hi, ci.wlo, ci.win);
        }
        if (++sc < ci.nst) {
            // every wave is done with slot t & 1: stage t + 2 goes there
            // while stage t + 1 may still be landing in the other slot
            block_barrier();
            if (more) issue_next(t & 1);
            continue;
        }

        // the item's last stage: every wave is done with slot t & 1, so
        // stage t + 2 goes there first and two stages stay in flight while
        // the 4 waves' states merge (fixed order) into the item's partial
        // records (max, sum, 30 unused, weighted values: kXattnLdsRec
        // floats, so that each store of 64 values covers two whole 128-byte
        // lines); wave w writes head w of the block with NST store
        // instructions per kind (decode: the copy, then the base token for
        // chunks that hold keys of its window)
        block_barrier();
        if (more) issue_next(t & 1);
        if (n < NH) {
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[wv][n][2 + 16 * dt + 4 * gq + r] = oacc[dt][r];
            if (gq == 0) {
                red[wv][n][0] = m_run;
                red[wv][n][1] = lacc[0];
            }
        }
        wait_lgkm0();
        block_barrier();
        {
            const int nkind = wv >= hg ? 0 : DEC && ci.win ? 2 : 1;   // wave w writes head w of the block
            // (the wave index read afresh: no record base is held across the loop)
            int w0 = wv;
            asm volatile("" : "+s"(w0));
            for (int kind = 0; kind < nkind; ++kind) {
                const int col = 4 * kind + wv;
                float* o = a.ws_part + (((int64_t)ci.id * KINDS + kind) * 4 + w0) * REC;
                float mw[4], M = kNegBig;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    mw[w] = red[w][col][0];
                    M = fmaxf(M, mw[w]);
                }
                float f[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) f[w] = fast_exp2(mw[w] - M);
#pragma unroll
                for (int h = 0; h < D / 64; ++h) {
                    const int d = lane + 64 * h;
                    float sum = 0.f;
#pragma unroll
                    for (int w = 0; w < 4; ++w) sum += f[w] * red[w][col][2 + d];
                    o[AOFF + d] = sum;
                }
                float l = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) l += f[w] * red[w][col][1];
                if (lane == 0) *(float2*)o = make_float2(M, l);
            }
            after0 += NST * nkind;
            after1 += NST * nkind;
        }
        pc += ci.len;
        if (pc >= run) break;
        item_of(pc, ci);
        asm volatile("" : "+v"(ci.id));
        sc = 0;
        qc ^= 1;
    }
}

// Compute units of the current device (one persistent workgroup each),
// looked up once per device.
int cu_count()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

// Key indices travel as 32-bit integers in the kernel: every cached key,
// plus a stage of overrun, must stay below 2^31.
constexpr int64_t kLdsMaxCap = INT32_MAX - 4096;

// Workgroups of one launch over at most `keys` keys in all: one per CU,
// fewer when runs of kXattnLdsSegMin keys do not fill them; 0 when a run
// would not fit the kernel's 32-bit key counts.
unsigned lds_grid(int64_t keys)
{
    int64_t g = cu_count();
    if (g > kXattnLdsMaxGrid) g = kXattnLdsMaxGrid;
    const int64_t need = (keys + kXattnLdsSegMin - 1) / kXattnLdsSegMin;
    if (need < g) g = need;
    if (g < 1) g = 1;
    return (keys + g - 1) / g < (int64_t(1) << 30) ? (unsigned)g : 0u;
}

}  // namespace

hipError_t launch_xattn_lds(const XattnParams& p, hipStream_t st)
{
    const int G = p.Hq / p.Hkv, hg = xattn_heads_per_wg(G);
    const int S = p.Hkv * (G / hg);
    if (p.rec != p.D + kXattnLdsRecPad || p.cap > kLdsMaxCap || (int64_t)S * p.cap > UINT32_MAX)
        return hipErrorInvalidValue;
    const int64_t region = xattn_lds_region(p.B, S);
    if (xattn_lds_records(p.B, S) >= INT32_MAX) return hipErrorInvalidValue;
    for (int b0 = 0; b0 < p.B; b0 += kPosPerLaunch) {
        const int nb = p.B - b0 < kPosPerLaunch ? p.B - b0 : kPosPerLaunch;
        PosBlock pos;
        int64_t keys = 0;
        for (int i = 0; i < kPosPerLaunch; ++i) {
            pos.v[i] = i < nb ? p.pos[b0 + i] : 0;
            if (i < nb) keys += (pos.v[i] + 1) * S;
        }
        const unsigned grid = lds_grid(keys);
        if (!grid) return hipErrorInvalidValue;
        const int rbase = (int)(b0 / kPosPerLaunch * region);
        if (p.D == 64)
            hipLaunchKernelGGL((xattn_lds_kernel<64, XattnParams>), dim3(grid), dim3(256), 0, st, p, b0, nb, rbase, hg,
                               G / hg, pos);
        else
            hipLaunchKernelGGL((xattn_lds_kernel<128, XattnParams>), dim3(grid), dim3(256), 0, st, p, b0, nb, rbase, hg,
                               G / hg, pos);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return launch_lds_merge(p, st);
}

hipError_t launch_decode_lds(const DecodeParams& p, hipStream_t st)
{
    const int G = p.Hq / p.Hkv, hg = xattn_heads_per_wg(G);
    const int S = p.Hkv * (G / hg);
    const int nb_max = p.B < kPosPerLaunch ? p.B : kPosPerLaunch;
    if ((p.D != 64 && p.D != 128) || p.rec != p.D + kXattnLdsRecPad || p.cap > kLdsMaxCap ||
        (int64_t)S * p.cap > UINT32_MAX || xattn_lds_records(p.B, S) >= INT32_MAX ||
        !lds_grid((int64_t)nb_max * S * (p.max_len + 1)))
        return hipErrorInvalidValue;
    hipError_t e = hipSuccess;
    const int64_t region = xattn_lds_region(p.B, S);
    PosBlock unused{};
    for (int b0 = 0; b0 < p.B; b0 += kPosPerLaunch) {
        const int nb = p.B - b0 < kPosPerLaunch ? p.B - b0 : kPosPerLaunch;
        // keys of this launch, at most (every length at max_len)
        const unsigned grid = lds_grid((int64_t)nb * S * (p.max_len + 1));
        const int rbase = (int)(b0 / kPosPerLaunch * region);
        if (p.D == 64)
            hipLaunchKernelGGL((xattn_lds_kernel<64, DecodeParams>), dim3(grid), dim3(256), 0, st, p, b0, nb, rbase, hg,
                               G / hg, unused);
        else
            hipLaunchKernelGGL((xattn_lds_kernel<128, DecodeParams>), dim3(grid), dim3(256), 0, st, p, b0, nb, rbase,
                               hg, G / hg, unused);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // the merge adds the new token's key L and appends it to the cache
    return launch_lds_merge(p, st);
}

}  // namespace orthros
