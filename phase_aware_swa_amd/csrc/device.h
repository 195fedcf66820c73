// device.h -- small gfx950 device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthros {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// Finite "minus infinity" for running maxima: exp2(x - kNegBig) never
// produces NaN, and exp2(kNegBig - m) underflows to 0 for any real m.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16)
{
    return __uint_as_float(bits16 << 16);
}

// Low / high bf16 of a packed 32-bit pair, as fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Buffer resource over [base, base + bytes): loads past the end return
// zeros and stores past the end are dropped, so tile edges need no branches.
// `base` must be the same for every lane of the wave.  Offsets are 32-bit.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes)
{
    const int64_t n = bytes < 0 ? 0 : (bytes > 0xffffffffll ? 0xffffffffll : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)(uint32_t)n, 0x00020000);
}
// Cache-policy operand of the buffer builtins marking an access
// non-temporal (nt): a stream read once.  On this GPU it is what lets a
// one-workgroup-per-CU read stream reach the HBM rate of a many-wave copy.
constexpr int kCachePolicyNt = 2;

template <int CP = 0>
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP));
}
__device__ __forceinline__ void buf_store16(u32x4 v, rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store8(u32x2 v, rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, (int)off, 0, 0);
}

// Cache-policy operand of the buffer load / store builtins selecting device
// scope (sc1): the access is coherent across the XCDs' L2 caches.
constexpr int kCachePolicySc1 = 16;

typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor words for [base, base + bytes) (raw buffer, no swizzle;
// out-of-range loads return zeros), as 4 scalar registers.  base and bytes
// must be the same for every lane of the wave: they are taken from the first
// active lane (the compiler's divergence analysis can lose track of uniform
// values joined after a divergent branch, and these words must be scalar).
__device__ __forceinline__ i32x4 buffer_words(const void* base, int64_t bytes)
{
    const uint64_t a = (uint64_t)base;
    const int64_t nb = bytes < 0 ? 0 : (bytes > 0xffffffffll ? 0xffffffffll : bytes);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)nb), 0x00020000};
}

// 16 bytes per lane from the buffer at voffset + soffset into LDS at
// lds + 16 * lane.  Written as inline asm so that the compiler inserts no
// wait of its own for it: it would otherwise wait for every such load before
// any LDS read, since it cannot tell the slots apart.  Completion is waited
// for explicitly (vmcnt); M0 holds the LDS address.
__device__ __forceinline__ void load_lds16(i32x4 rsrc, uint32_t voffset, int soffset, const uint16_t* lds)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void*)lds;
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voffset), "s"(rsrc), "s"(soffset), "s"(m0)
                 : "memory", "m0");
}
// The same, non-temporal (a stream read once; see kCachePolicyNt).
__device__ __forceinline__ void load_lds16_nt(i32x4 rsrc, uint32_t voffset, int soffset, const uint16_t* lds)
{
    const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void*)lds;
    asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds"
                 :
                 : "v"(voffset), "s"(rsrc), "s"(soffset), "s"(m0)
                 : "memory", "m0");
}

// s_waitcnt vmcnt(N) alone (expcnt and lgkmcnt left at their maxima);
// vmcnt is 6 bits, split over the immediate's bits 3:0 and 15:14.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(L * n) for a wave-uniform n >= 0 (the count is an
// immediate of the instruction, hence the unrolled selection); n above NMAX
// waits for vmcnt(L * NMAX), which is more than needed, never less.
template <int L, int NMAX, int I = 0>
__device__ __forceinline__ void wait_stages(int n)
{
    if (n == I || (I == NMAX && n > NMAX)) {
        wait_vmcnt<L * I>();
        return;
    }
    if constexpr (I < NMAX) wait_stages<L, NMAX, I + 1>(n);
}

// DPP lane movement inside a row of 16 lanes.  Every pattern used here
// reads a lane of the same row, so bound_ctrl never applies; written this
// way (old = 0, bound_ctrl set) the compiler folds the move into the DPP
// form of the instruction that consumes it (v_add_f32_dpp).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- 7-i inside each 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <- 15-i inside each 16 lanes
constexpr int kDppRor8 = 0x128;       // lane i <- i ^ 8 inside each 16 lanes (rotate by 8)

// Sum over aligned groups of N lanes (N = 8 or 16); every lane of a group
// ends with the same bits (each step adds a pair in both orders, and fp32
// addition is commutative).
template <int N>
__device__ __forceinline__ float group_sum(float x)
{
    x += dpp_mov<kDppXor1>(x);
    x += dpp_mov<kDppXor2>(x);
    x += dpp_mov<kDppHalfMirror>(x);
    if constexpr (N == 16) x += dpp_mov<kDppMirror>(x);
    return x;
}

// Maximum over the whole wave of a value that is already uniform within each
// row of 16 lanes: two DPP row broadcasts (row 0 -> 1, 2 -> 3, then 1 -> 2, 3)
// leave the total in lane 63.
__device__ __forceinline__ float wave_max_of_rows(float x)
{
    constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), kRowBcast15,
                                                            0xa, 0xf, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), kRowBcast31,
                                                            0xc, 0xf, false)));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Value of lane (lane ^ x) of the wave (x < 64), through ds_bpermute.
__device__ __forceinline__ float lane_xor(float v, int lane, int x)
{
    return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ x) << 2, __float_as_int(v)));
}

// Maps a launch-order workgroup id to a logical id so that the round-robin
// dispatch over the 8 XCDs hands each XCD one contiguous run of logical ids
// (neighbouring tiles then share that XCD's L2).  Ids past the last whole
// multiple of 8 keep their order.
__device__ __forceinline__ int64_t xcd_contiguous_id(int64_t i, int64_t n)
{
    int64_t n8 = n - (n & 7);
    if (i >= n8) return i;
    return (i & 7) * (n8 >> 3) + (i >> 3);
}

}  // namespace orthros
