// pair_tile.h -- LDS layout of one 32-key "pair" (two 16-key blocks) of K
// and V for the 16x16x32 bf16 MFMA attention kernels (the streaming SWA
// kernel, the cross-attention stream, the short decode kernel and the
// many-copy kernel).
//
// S^T = K Q^T per 16-key block leaves each lane (n = query, gq = lane/16)
// with keys 4gq..4gq+3 of the block; the P^T operand of O^T = V^T P^T over a
// pair is then [block 0 keys 4gq..+3, block 1 keys 4gq..+3].
//
// K is stored line-aligned: the K part is a run of 16-byte units in blocks
// of 64 (1 KB), each block holding 8 keys x 8 chunks, i.e. 128 contiguous
// bytes of each of 8 key rows.  Filled in unit order -- a direct-to-LDS
// load instruction, or 256 threads' 16-byte stores -- every 8 consecutive
// lanes read 128 contiguous bytes of one cache row (whole lines, which lets
// non-temporal loads stream at the full HBM rate) and the LDS stores are
// contiguous.  Within a 16-key block, keys r and r + 8 take adjacent 8-unit
// rows and chunk c of key r sits at position (c & 7) ^ (r & 7) of its row,
// so the operand read of a k-step (16 keys, one chunk) hits 16 distinct
// 16-byte bank groups, and any 8 consecutive of those keys 8 distinct ones.
//
// V is stored in 256-byte lines of 8 keys x 16 head dims,
// [key / 8][d / 16][key % 8][d % 16], and read with ds_read_b64_tr_b16:
// inside each 16-lane group, output lane l, slot k is element l & 3 of the
// 8-byte chunk that source lane 4k + (l >> 2) addresses.  Source lane
// 4k + q of a group addresses keys' d = 16 dt + 4q .. + 3, so output lane m
// receives V[the group's 4 keys][16 dt + m] -- the V^T operand, transposed
// by the read.  A 32-lane access of 8 keys x 4 chunks then covers one line
// (every LDS bank once), and dt is an immediate offset.
#pragma once

#include <hip/hip_runtime.h>

namespace orthros {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct PairTile {
    static constexpr int KPART = 32 * D;    // bf16: K rows of the two blocks
    static constexpr int VPART = 32 * D;    // bf16: V rows of the two blocks
    static constexpr int SLOT = KPART + VPART;
    // K: element offset of 16-byte chunk c (dims 8c .. 8c + 7) of key r.
    __device__ static int kofs(int r, int c)
    {
        const int row = ((r & 7) << 1) | ((r >> 3) & 1);
        return ((r >> 4) * 2 * D + (c >> 3) * 128 + row * 8 + ((c & 7) ^ (r & 7))) * 8;
    }
    // The operand of k-step i (chunk 4 i + gq of key n of block 0) is at
    // kofs(n, 4 (i & 1) + gq) + (i >> 1) * K_STEP2; block 1 adds K_KEY16.
    static constexpr int K_STEP2 = 128 * 8, K_KEY16 = 2 * D * 8;
    // Inverse map for unit-order filling: key row r and chunk c held by
    // 16-byte unit u of the K part.
    __device__ static void k_unit(int u, int& r, int& c)
    {
        const int row = (u >> 3) & 15;
        r = 16 * (u / (2 * D)) + ((row & 1) << 3) + (row >> 1);
        c = 8 * ((u % (2 * D)) >> 7) + ((u & 7) ^ (r & 7));
    }
    // V: element offset of head dims 16 dt + 4 q .. + 3 of key r (an 8-byte
    // transposing-read chunk), and of 16-byte chunk c (dims 8c .. 8c + 7).
    __device__ static int vofs_tr(int r, int dt, int q) { return (r >> 3) * 8 * D + dt * 128 + (r & 7) * 16 + 4 * q; }
    __device__ static int vofs16(int r, int c) { return (r >> 3) * 8 * D + (c >> 1) * 128 + (r & 7) * 16 + 8 * (c & 1); }
    // Inverse map for loads that write the V part in lane order: the key row
    // r and 16-byte chunk c held by 16-byte unit u (vofs16).
    __device__ static void v_unit(int u, int& r, int& c)
    {
        const int w = u % D;
        r = 8 * (u / D) + ((w >> 1) & 7);
        c = 2 * (w >> 4) + (w & 1);
    }
    // Immediate steps of vofs_tr: dt + 1 is one line on, key r + 16
    // (r < 16) two 8-key groups on, and key r + 4 (r & 7 < 4) half a line.
    static constexpr int V_DT = 128, V_KEY16 = 16 * D, V_KEY8 = 8 * D, V_KEY4 = 64;
    // Staging order of V chunks through registers: item it -> key row,
    // 16-byte chunk.  The 16 lanes of one 16-byte LDS store cover one line
    // (8 keys x 2 chunks), and a wave's global loads cover 8 keys x 128
    // contiguous bytes.
    __device__ static void vitem(int it, int& r, int& c)
    {
        constexpr int LDT = D == 128 ? 3 : 2;        // log2(D / 16)
        r = ((it >> (4 + LDT)) << 3) | ((it >> 1) & 7);
        c = (((it >> 4) & ((1 << LDT) - 1)) << 1) | (it & 1);
    }
};

// Four bf16 of V^T through the transposing read (see above).
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

}  // namespace orthros
