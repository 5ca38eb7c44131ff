// Device helpers shared by the library's kernels (wave64, gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sko {

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Append the lanes whose `pred` is set to a list whose length lives in
// `counter`: one atomic per wave; returns this lane's slot (or -1).
__device__ __forceinline__ int wave_append(int32_t* counter, bool pred) {
    unsigned long long mask = __ballot(pred);
    if (mask == 0ull) return -1;
    const int lane = lane_id();
    const int leader = __ffsll((long long)mask) - 1;
    int base = 0;
    if (lane == leader) base = atomicAdd(counter, (int32_t)__popcll(mask));
    base = __shfl(base, leader);
    const unsigned long long below = (lane == 0) ? 0ull : (mask & ((~0ull) >> (64 - lane)));
    return pred ? base + (int)__popcll(below) : -1;
}

// Exclusive prefix sum over a block of NT threads (NT a multiple of 64, at
// most 4096).  `scratch` needs NT/64 + 1 ints of LDS.  Returns this thread's
// exclusive prefix; *total receives the block sum.  Contains barriers: every
// thread of the block must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* scratch) {
    constexpr int NW = NT / 64;
    const int lane = lane_id();
    const int wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) scratch[wid] = x;
    __syncthreads();
    if (wid == 0) {
        int w = lane < NW ? scratch[lane] : 0;
        int s = w;
#pragma unroll
        for (int o = 1; o < NW; o <<= 1) {
            int y = __shfl_up(s, o);
            if (lane >= o) s += y;
        }
        if (lane < NW) scratch[lane] = s - w;
        if (lane == NW - 1) scratch[NW] = s;
    }
    __syncthreads();
    const int res = scratch[wid] + x - v;
    *total = scratch[NW];
    __syncthreads();
    return res;
}

// 16-byte load marked nontemporal: data streamed once per step (the
// indexer scan) is not kept in the caches, which lets the loads reach a
// higher share of HBM bandwidth than ordinary loads.
__device__ __forceinline__ uint4 load_nt_u4(const uint4* p) {
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// bf16 pair in one dword -> two floats (exact widening).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Monotone key of a binary32 score (larger score -> larger key).
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u ^ 0x80000000u);
}

// ---- launches kept off one XCD ------------------------------------------
// MI355X deals the blocks of a launch to its 8 XCDs in a fixed stripe:
// block i (linear id, x fastest) runs on XCD (i + o) mod 8, with one offset
// o per launch (the handle checks this at creation).  A launch that must
// stay off XCD `xc` has 8 * ceil(n / 7) blocks for its n work blocks: the
// blocks of the stripe slot that falls on XCD xc leave at once, and the
// others take work blocks 0, 1, ... in order, 7 per group of 8.  xc < 0:
// no split, block i is work block i.
constexpr int kXcds = 8;

__device__ __forceinline__ int xcc_id() {
    int v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(v));
    return v;
}

// Work block of linear block `lin`, or -1 for a block on XCD xc.
__device__ __forceinline__ int split_block(int lin, int xc) {
    if (xc < 0) return lin;
    const int x = xcc_id();
    if (x == xc) return -1;
    const int slot = lin & (kXcds - 1);
    const int cslot = (xc - x + slot) & (kXcds - 1);  // the slot on XCD xc
    return (lin >> 3) * (kXcds - 1) + ((slot - cslot - 1) & (kXcds - 1));
}

// Blocks of a launch of n work blocks (n >= 1).
__host__ __device__ inline unsigned split_grid(int64_t n, int xc) {
    return xc < 0 ? (unsigned)n : (unsigned)((n + kXcds - 2) / (kXcds - 1) * kXcds);
}

}  // namespace sko
