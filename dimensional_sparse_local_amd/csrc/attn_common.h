// Device helpers shared by the attention kernels (gfx950): vector types, LDS
// transpose reads and LDS DMA, bf16 conversion, half-wave reductions and the
// XCD-aware workgroup order.
//
// MFMA 32x32 accumulator layout used throughout: lane l, element r holds
// row 8*(r/4) + 4*(l/32) + r%4 and column l%32.  A and B operands: lane l holds
// row (A) / column (B) l%32 and reduction slots 8*(l/32)..8*(l/32)+7 (bf16) or
// slot l/32 (fp32).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "na_internal.h"

namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Load through a global-address-space pointer (a flat load would also count
// against the LDS wait counter).
template <typename T>
__device__ __forceinline__ T gload(const T* ptr) {
    return *(const __attribute__((address_space(1))) T*)(ptr);
}

// Load of read-only, wave-uniform data through the constant address space
// (a scalar load).
template <typename T>
__device__ __forceinline__ T cload(const T* ptr) {
    return *(const __attribute__((address_space(4))) T*)(ptr);
}

typedef int32_t i32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ NaEntry load_entry(const NaEntry* e) {
    const i32x2 v = cload((const i32x2*)e);
    return NaEntry{v[0], v[1]};
}

// Mask words of one query row for one tile: the keep plane (2 words), and with
// BIAS the partner plane of fixed fusion (2 more words).
template <bool BIAS> struct MaskRow { using T = u32x2; };
template <> struct MaskRow<true> { using T = u32x4; };

// Keep score x when bit `bit` of word w is set, else -inf: the bit, extracted
// sign-extended, selects between the two bit patterns (two VALU instructions,
// no compare-and-select through VCC).
__device__ __forceinline__ float keep_if(uint32_t w, int bit, float x) {
    const uint32_t m = (uint32_t)((int32_t)(w << (31 - bit)) >> 31);
    return __builtin_bit_cast(float, (m & __builtin_bit_cast(uint32_t, x)) | (~m & 0xff800000u));
}

// Online softmax in the log2 domain against a reference maximum per row: the
// probabilities of a tile are 2^(c s - reference); the reference moves (and O,
// l are rescaled) only when a row has none yet or when one lane's sum of a
// tile's probabilities, which bounds each of them, passes 2^kSumLog2.  Every
// probability then stays below 2^32, far inside fp32 and bf16 range for O and
// l over any number of keys, and the result is exact after the final division
// by l whatever the reference.
constexpr float kSumLog2 = 32.0f;
constexpr float kSumMax = 4294967296.0f;   // 2^kSumLog2

typedef __attribute__((address_space(3))) bf16x4* lds_bf16x4_ptr;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_ptr)(p));
}

// 16 bytes per lane from global memory into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (lds_void_ptr)(lds), 16, 0, 0);
}

// Wait for all of this wave's vector memory operations (including LDS DMA).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ bf16x8 cvt8(float a0, float a1, float a2, float a3, float a4, float a5,
                                       float a6, float a7) {
    const f32x2 x0 = {a0, a1}, x1 = {a2, a3}, x2 = {a4, a5}, x3 = {a6, a7};
    const bf16x2 y0 = __builtin_convertvector(x0, bf16x2);
    const bf16x2 y1 = __builtin_convertvector(x1, bf16x2);
    const bf16x2 y2 = __builtin_convertvector(x2, bf16x2);
    const bf16x2 y3 = __builtin_convertvector(x3, bf16x2);
    u32x4 w = {__builtin_bit_cast(uint32_t, y0), __builtin_bit_cast(uint32_t, y1),
               __builtin_bit_cast(uint32_t, y2), __builtin_bit_cast(uint32_t, y3)};
    return __builtin_bit_cast(bf16x8, w);
}

// Sum of the 32 values of two 16-element accumulators, as a pairwise tree
// (fp32 adds, depth 5).
__device__ __forceinline__ float tile_sum32(const f32x16& a, const f32x16& b) {
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) t[r] = a[r] + b[r];
#pragma unroll
    for (int w = 8; w >= 1; w /= 2)
#pragma unroll
        for (int r = 0; r < w; ++r) t[r] = t[r] + t[r + w];
    return t[0];
}

// Combine a value across the two half-waves (lanes l and l ^ 32).  The swap
// returns {this lane's vdst, this lane's vsrc}; the partner's value sits in
// the first for lanes 0-31 and in the second for lanes 32-63, and the other
// element holds the lane's own value, so a symmetric reduction of the pair is
// the same on every lane.
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// Logical tile index -> query tile of its (batch, head), in ascending order
// or (desc) descending.  On a causal window the tiles at the start of the
// sequence have the shortest walks; taking them last lets them fill the final
// round of workgroups instead of leaving compute units idle behind
// full-length ones (longest first, as in list scheduling).
__device__ __forceinline__ int tile_of(int wg, int n_q_tiles, int desc) {
    const int t = wg % n_q_tiles;
    return desc ? n_q_tiles - 1 - t : t;
}

// Workgroup index -> logical tile index.  Workgroups are dispatched to the 8
// XCDs round-robin; give each XCD one contiguous range of logical tiles
// (consecutive query tiles of one head) so that the tiles sharing key/value
// tiles share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
    constexpr int kXcd = 8;
    const int q = n / kXcd, r = n % kXcd;
    const int x = bid % kXcd, local = bid / kXcd;
    return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + local;
}

}  // namespace
