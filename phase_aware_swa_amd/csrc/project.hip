// project.hip -- the projections either side of one layer's attention step,
// for gfx950, bf16.
//
// "Orthros:阶段感知异构注意力精读笔记" §2.1-§2.2: the base stream's keys and
// values come from the layer's base input X at every position (k = x W_K,
// v = x W_V; they are the layer's cache rows), and both streams' queries come
// from the one shared W_Q followed by each stream's elementwise scale-offset
// (q = (x W_Q) * alpha + beta for the base rows, q' = (x' W_Q) * alpha' +
// beta' for the output copies).  One launch computes all of it as a single
// tiled product over the stacked rows [X; X']:
//
//   region A: X rows (B*T) against [W_Q; W_K; W_V] (Hq*d + 2*Hkv*d columns),
//   region B: X' rows (B*T_out) against W_Q only,
//
// with the epilogue applied to each 128-column tile by what its columns are:
// the scale-offset of the row's stream and a store into q / q_out, or a store
// straight into k_cache / v_cache at slot t of (sequence, KV head) -- the
// K/V never make a separate trip through HBM.
//
// Kernel design (one workgroup = NW waves = one 256-row x 32*NW-column tile;
// the workload shape runs NW = 8, 256 x 256 tiles, one workgroup per CU):
//   - C^T = W X^T on v_mfma_f32_16x16x32_bf16: the A operand is 16 weight
//     rows (output columns), the B operand 16 token rows, so each lane ends
//     with 4 consecutive output columns of one token row (8-byte stores);
//     wave (wr, wc) owns rows 128 wr .. +127 and columns 64 wc .. +63, i.e.
//     8 x 4 MFMA tiles, 32 MFMAs per 32-deep step against 12 LDS reads, two
//     waves per SIMD;
//   - the K dimension (d_model) streams in 32-deep stages through NS LDS
//     slots filled by buffer loads that write LDS directly (no register
//     staging), NS - 1 stages ahead of the MFMAs, one barrier per stage.  The
//     stage time is bounded by the loads' latency over the prefetch depth,
//     so the depth is what the 160 KB of LDS buys (4 slots of 32 KB for the
//     256-column tile).  The stage loop is unrolled by NS, so every slot is
//     known at compile time;
//   - LDS layout of a slot part (rows x 4 chunks of 16 bytes): chunk c of row
//     r sits at unit 4r + (c ^ ((r >> 2) & 3)).  An MFMA operand read (16 rows,
//     one chunk) then touches 16 distinct 16-byte bank groups, and every read
//     is one per-lane base plus an immediate.  The direct loads write units in
//     lane order, so each lane fetches the global chunk that belongs at its
//     unit (16 rows x 64 contiguous bytes per load instruction);
//   - rows past the end of X / X' read as zeros through the buffer range and
//     are not stored;
//   - logical tile ids are XCD-contiguous with the 128-column tiles of one
//     256-row block adjacent, so a row block (2 MB at d_model 4096) is read
//     from HBM once and reused from its XCD's L2 by every column tile.

#include "device.h"
#include "kernels.h"

namespace orthros {
namespace {

constexpr int kBM = 256;                 // token rows per tile
constexpr int kBK = 32;                  // reduction depth per stage
constexpr int kXU = kBM * 4;             // 16-byte units of a slot's X part
constexpr int kWideNS = 4;               // LDS slots of the 256-column form
constexpr bool kWideFB = true;           // its operand fragments double-buffered in registers

__device__ __forceinline__ int unit_of(int r, int c) { return 4 * r + (c ^ ((r >> 2) & 3)); }

// One tile's columns and where they go.
struct TileKind {
    const uint16_t* w;        // first weight row of the tile ([out][in])
    int kind;                 // 0: queries, 1: keys, 2: values
    int col0;                 // first column within its own matrix (q: Hq*d, k/v: Hkv*d)
};

template <int NW, int NS, bool FB>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void project_kernel(ProjParams p, int64_t tiles_a)
{
    constexpr int NT = 64 * NW;              // threads
    constexpr int kBN = 32 * NW;             // output columns per tile (64 per wave column)
    constexpr int kWU = kBN * 4;             // 16-byte units of a slot's W part
    constexpr int kSlotU = kXU + kWU;
    constexpr int kXL = kXU / NT;            // direct loads per lane per stage (X part)
    constexpr int kWL = kWU / NT;            // (W part)
    constexpr int NC = 4;                    // MFMA column tiles per wave
    constexpr int kL = kXL + kWL;            // loads per lane per stage
    static_assert(kXU % NT == 0 && kWU % NT == 0 && NS >= 2 && (NS - 2) * kL <= 63, "tile shape");
    __shared__ __align__(16) uint16_t slots[NS][kSlotU * 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr = wv & 1, wc = wv >> 1;
    const int n = lane & 15, gq = lane >> 4;
    const int Nq = p.Hq * p.D, Nk = p.Hkv * p.D;
    const int64_t K = p.K;

    // ---- which tile
    const int64_t total = tiles_a + p.tiles_b;
    const int64_t id = xcd_contiguous_id(blockIdx.x, total);
    const bool region_b = id >= tiles_a;
    const int ntiles_n = region_b ? Nq / kBN : (Nq + 2 * Nk) / kBN;
    const int64_t local = region_b ? id - tiles_a : id;
    const int64_t row0 = (local / ntiles_n) * kBM;
    const int colt = (int)(local % ntiles_n) * kBN;          // first column of the stacked [W_Q; W_K; W_V]
    const int64_t M = region_b ? p.Mo : p.Mx;
    const uint16_t* xrows = region_b ? p.xo : p.x;
    TileKind tk;
    if (colt < Nq) {
        tk = {p.wq + (int64_t)colt * K, 0, colt};
    } else if (colt < Nq + Nk) {
        tk = {p.wk + (int64_t)(colt - Nq) * K, 1, colt - Nq};
    } else {
        tk = {p.wv + (int64_t)(colt - Nq - Nk) * K, 2, colt - Nq - Nk};
    }

    // ---- direct-load addressing: lane l of load j writes unit NT j + 64 wave + l of the part
    const i32x4 rx = buffer_words(xrows + row0 * K, (M - row0) * K * 2);
    const i32x4 rw = buffer_words(tk.w, (int64_t)kBN * K * 2);
    uint32_t xoff[kXL], woff[kWL];
#pragma unroll
    for (int j = 0; j < kXL; ++j) {
        const int u = NT * j + 64 * wv + lane, r = u >> 2, c = (u & 3) ^ ((r >> 2) & 3);
        xoff[j] = (uint32_t)(r * K * 2 + 16 * c);
    }
#pragma unroll
    for (int j = 0; j < kWL; ++j) {
        const int u = NT * j + 64 * wv + lane, r = u >> 2, c = (u & 3) ^ ((r >> 2) & 3);
        woff[j] = (uint32_t)(r * K * 2 + 16 * c);
    }
    auto issue = [&](uint16_t* slot, int64_t t) {
        const int kb = (int)(t * kBK * 2);                   // byte offset of the stage along a row
#pragma unroll
        for (int j = 0; j < kXL; ++j) load_lds16(rx, xoff[j], kb, slot + (NT * j + 64 * wv) * 8);
#pragma unroll
        for (int j = 0; j < kWL; ++j) load_lds16(rw, woff[j], kb, slot + (kXU + NT * j + 64 * wv) * 8);
    };

    // ---- operand reads: token rows 128 wr + 16 ri + n, weight rows 64 wc + 16 ci + n, chunk gq
    const int xb = unit_of(128 * wr + n, gq) * 8;            // elements
    const int wb = (kXU + unit_of(64 * wc + n, gq)) * 8;
    f32x4 acc[8][NC];
#pragma unroll
    for (int ri = 0; ri < 8; ++ri)
#pragma unroll
        for (int ci = 0; ci < NC; ++ci) acc[ri][ci] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](const uint16_t* slot) {
        bf16x8 wf[NC];
#pragma unroll
        for (int ci = 0; ci < NC; ++ci) wf[ci] = *(const bf16x8*)(slot + wb + ci * 64 * 8);
#pragma unroll
        for (int ri = 0; ri < 8; ++ri) {
            const bf16x8 xf = *(const bf16x8*)(slot + xb + ri * 64 * 8);
#pragma unroll
            for (int ci = 0; ci < NC; ++ci)
                acc[ri][ci] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[ci], xf, acc[ri][ci], 0, 0, 0);
        }
    };
    // stage t computes from slot t % NS and refills slot (t + NS - 1) % NS (read at t - 1)
    const int64_t nk = K / kBK;
    auto step = [&](uint16_t* cur, uint16_t* refill, int64_t t) {
        if (t >= nk) return;
        // this lane's loads of stage t are done when at most the stages after
        // it that were issued (up to NS - 2 of them) remain
        const int64_t after = nk - 1 - t < NS - 2 ? nk - 1 - t : NS - 2;
        wait_stages<kL, NS - 2>((int)after);
        // A bare barrier: every wave has waited for its own loads of stage t
        // above, and each wave's reads of the slot refilled next were consumed
        // by its MFMAs before it got here.  (__syncthreads' release fence
        // would also wait for the loads of stage t + 1.)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (t + NS - 1 < nk) issue(refill, t + NS - 1);
        compute(cur);
    };
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nk) issue(slots[s], s);
    if constexpr (!FB) {
        for (int64_t t = 0; t < nk; t += NS) {
#pragma unroll
            for (int s = 0; s < NS; ++s) step(slots[s], slots[(s + NS - 1) % NS], t + s);
        }
    } else {
        // FB: the fragments a stage needs first (its 4 weight fragments and its
        // first 2 row fragments) double-buffered in registers.  Step t waits
        // for stage t + 1 and reads that prefix (set (t + 1) % 2) while the
        // MFMAs of stage t run on set t % 2 and on its other row fragments,
        // read during those MFMAs; so no stage starts with the LDS read
        // latency.  The slot refilled at step t held stage t - 1, whose
        // fragments every wave read before it left step t - 1.  The launcher
        // takes this form only when nk is a multiple of NS, so the loop has no
        // partial group and the reads no branch around them (at a branch the
        // compiler would wait for every outstanding LDS read); the last step
        // reads a stale slot it never uses.
        static_assert(NS % 2 == 0 && NS >= 3, "fragment sets alternate with the slots");
        constexpr int XPRE = 2;
        bf16x8 wfb[2][NC], xfb[2][XPRE];
        auto read_frags = [&](int fs, const uint16_t* slot) {
#pragma unroll
            for (int ci = 0; ci < NC; ++ci) wfb[fs][ci] = *(const bf16x8*)(slot + wb + ci * 64 * 8);
#pragma unroll
            for (int ri = 0; ri < XPRE; ++ri) xfb[fs][ri] = *(const bf16x8*)(slot + xb + ri * 64 * 8);
        };
        auto sync_stage = [&](int64_t u) {      // stage u (if any) landed in every wave's view
            const int64_t after = nk - 1 - u < NS - 2 ? nk - 1 - u : NS - 2;
            wait_stages<kL, NS - 2>((int)after);  // nothing to wait for when u = nk
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        };
        auto step_fb = [&](int fs, const uint16_t* cur, const uint16_t* next, uint16_t* refill, int64_t t) {
            sync_stage(t + 1);
            if (t + NS - 1 < nk) issue(refill, t + NS - 1);
            read_frags(fs ^ 1, next);
            // keep this stage's MFMAs after the next stage's reads are issued
            // (the scheduler would otherwise hoist them and serialise the two)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ri = 0; ri < 8; ++ri) {
                const bf16x8 xf = ri < XPRE ? xfb[fs][ri < XPRE ? ri : 0] : *(const bf16x8*)(cur + xb + ri * 64 * 8);
#pragma unroll
                for (int ci = 0; ci < NC; ++ci)
                    acc[ri][ci] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wfb[fs][ci], xf, acc[ri][ci], 0, 0, 0);
            }
        };
        sync_stage(0);
        read_frags(0, slots[0]);
        for (int64_t t = 0; t < nk; t += NS) {
#pragma unroll
            for (int s = 0; s < NS; ++s)
                step_fb(s & 1, slots[s], slots[(s + 1) % NS], slots[(s + NS - 1) % NS], t + s);
        }
    }

    // ---- epilogue: lane (n, gq) holds columns 4 gq .. + 3 of row n of each 16 x 16 tile
#pragma unroll
    for (int ri = 0; ri < 8; ++ri) {
        const int64_t row = row0 + 128 * wr + 16 * ri + n;
        if (row >= M) continue;
#pragma unroll
        for (int ci = 0; ci < NC; ++ci) {
            const int col = tk.col0 + 64 * wc + 16 * ci + 4 * gq;   // within its own matrix
            float v[4] = {acc[ri][ci][0], acc[ri][ci][1], acc[ri][ci][2], acc[ri][ci][3]};
            uint16_t* dst;
            if (tk.kind == 0) {
                const uint16_t* al = region_b ? p.alpha_out : p.alpha;
                const uint16_t* be = region_b ? p.beta_out : p.beta;
                if (al) {
                    const u32x2 aw = *(const u32x2*)(al + col), bw = *(const u32x2*)(be + col);
                    v[0] = __builtin_fmaf(v[0], bf16_lo(aw[0]), bf16_lo(bw[0]));
                    v[1] = __builtin_fmaf(v[1], bf16_hi(aw[0]), bf16_hi(bw[0]));
                    v[2] = __builtin_fmaf(v[2], bf16_lo(aw[1]), bf16_lo(bw[1]));
                    v[3] = __builtin_fmaf(v[3], bf16_hi(aw[1]), bf16_hi(bw[1]));
                }
                dst = (region_b ? p.q_out : p.q) + row * Nq + col;
            } else {
                const int64_t b = row / p.T, t = row - b * p.T;
                const int g = col / p.D, e = col - g * p.D;
                dst = (tk.kind == 1 ? p.k_cache : p.v_cache) + (((int64_t)b * p.Hkv + g) * p.cap + t) * p.D + e;
            }
            *(u32x2*)dst = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
    }
}

}  // namespace

template <int NW, int NS, bool FB>
hipError_t launch_project_t(const ProjParams& p, hipStream_t s)
{
    constexpr int BN = 32 * NW;
    const int Nq = p.Hq * p.D, Nk = p.Hkv * p.D;
    const int64_t tiles_a = (p.Mx + kBM - 1) / kBM * ((Nq + 2 * Nk) / BN);
    ProjParams q = p;
    q.tiles_b = (p.Mo + kBM - 1) / kBM * (Nq / BN);
    const int64_t total = tiles_a + q.tiles_b;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL((project_kernel<NW, NS, FB>), dim3((unsigned)total), dim3(64 * NW), 0, s, q, tiles_a);
    return hipGetLastError();
}

bool project_applies(const ProjParams& p)
{
    return p.D > 0 && (p.Hq * p.D) % 128 == 0 && (p.Hkv * p.D) % 128 == 0 && p.K >= kBK && p.K % kBK == 0;
}

hipError_t launch_project(const ProjParams& p, hipStream_t s)
{
    // 256-column tiles (8 waves, one workgroup per CU, 4 slots) when no tile
    // would straddle the query / key / value columns; else 128-column tiles
    // (4 waves, two workgroups per CU, 3 slots)
    if ((p.Hq * p.D) % 256 == 0 && (p.Hkv * p.D) % 256 == 0) {
        if (kWideFB && (p.K / kBK) % kWideNS == 0) return launch_project_t<8, kWideNS, true>(p, s);
        return launch_project_t<8, kWideNS, false>(p, s);
    }
    return launch_project_t<4, 3, false>(p, s);
}

}  // namespace orthros
