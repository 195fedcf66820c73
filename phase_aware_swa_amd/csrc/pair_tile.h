// pair_tile.h -- LDS layout of one 32-key "pair" (two 16-key blocks) of K
// and V for the 16x16x32 bf16 MFMA attention kernels (the streaming SWA
// kernel and the many-copy kernel).
//
// S^T = K Q^T per 16-key block leaves each lane (n = query, gq = lane/16)
// with keys 4gq..4gq+3 of the block; the P^T operand of O^T = V^T P^T over a
// pair is then [block 0 keys 4gq..+3, block 1 keys 4gq..+3].  V^T rows of a
// pair slot store the 32 keys in exactly that order, so each PV operand is a
// single 16-byte LDS read.  Both parts are XOR-swizzled instead of padded:
// the MFMA operand reads (16 rows x 16 bytes per 16 lanes) hit 16 distinct
// 16-byte bank groups.
#pragma once

namespace orthros {

template <int D>
struct PairTile {
    static constexpr int KPART = 32 * D;    // bf16: K rows of the two blocks
    static constexpr int VPART = D * 32;    // bf16: V^T rows, 32 keys each
    static constexpr int SLOT = KPART + VPART;
    // K: row = key of the pair (0..31); 16-byte chunks XOR-swizzled by row.
    __device__ static int kofs(int r, int c)
    {
        const int sw = (D == 128) ? (r & 15) : ((r >> 1) & 7);
        return r * D + ((c ^ sw) << 3);
    }
    // V^T: row d = 64 bytes = four 16-byte units; unit u holds keys
    // 4u..4u+3 of block 0 then of block 1; XOR by bits 2..3 of d.
    __device__ static int vofs(int d, int u) { return d * 32 + ((u ^ ((d >> 2) & 3)) << 3); }
};

}  // namespace orthros
