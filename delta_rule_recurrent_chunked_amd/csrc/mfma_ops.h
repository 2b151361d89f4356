// mfma_ops.h -- gfx950 matrix-core and LDS helpers shared by the prefill kernels.
//
// MFMA lane layouts (wave64):
//   32x32x16 bf16: lane l supplies A[l%32][8(l/32) + e] and B[8(l/32) + e][l%32],
//                  e < 8; accumulator element e is D[8(e/4) + 4(l/32) + e%4][l%32].
//   16x16x32 bf16: lane l supplies A[l%16][8(l/16) + e] and B[8(l/16) + e][l%16];
//                  accumulator element e is D[4(l/16) + e][l%16].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 ld8(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ void st4(__bf16* p, float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
    *reinterpret_cast<bf16x4*>(p) = v;
}
// Transposed LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane i receives
// element i%4 of the 8-byte rows addressed by lanes i/4, 4 + i/4, 8 + i/4 and 12 + i/4.
// With lane s of the group addressing row base + s/4, column 4*(s%4) of a row-major tile,
// lane i gets column i of rows base .. base+3: four consecutive rows of one column.
__device__ __forceinline__ bf16x4 trld(const __bf16* p) {
    typedef __bf16 v4bf16 __attribute__((__vector_size__(4 * sizeof(__bf16))));
    typedef __attribute__((address_space(3))) v4bf16 lds_v4bf16;
    const v4bf16 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (lds_v4bf16*)((__attribute__((address_space(3))) __bf16*)(p)));
    return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 zero8() {
    bf16x8 z;
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
    return z;
}

// Orders this wave's LDS writes before its later LDS reads of the same data (LDS executes
// one wave's instructions in order; this only stops the compiler from reordering them).
__device__ __forceinline__ void wave_lds_order() { __asm__ volatile("" ::: "memory"); }

// Scheduling fence: the compiler moves no instruction across it (used to issue a step's
// LDS reads together, so that one round trip covers them all).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// Two 16x16 accumulator tiles a (rows 0..15) and b (rows 16..31) of one 32-row block, as
// the B operand of a 16x16x32 MFMA contracting over those 32 rows.  Lane group g = l/16
// holds rows 4g..4g+3 of each tile and needs rows 8g..8g+7 of the block: a swap of lane
// halves between a and b, then of odd and even 16-lane rows, routes each 4-row piece to
// its lane (v_permlane32_swap / v_permlane16_swap), with no trip through LDS.
__device__ __forceinline__ bf16x8 acc_to_b(f32x4 a, f32x4 b) {
    const uint32_t a0 = pack_bf16x2(a[0], a[1]), a1 = pack_bf16x2(a[2], a[3]);
    const uint32_t b0 = pack_bf16x2(b[0], b[1]), b1 = pack_bf16x2(b[2], b[3]);
    const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
    const auto u0 = __builtin_amdgcn_permlane16_swap(s0[0], s0[1], false, false);
    const auto u1 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = {u0[0], u1[0], u0[1], u1[1]};
    return __builtin_bit_cast(bf16x8, w);
}

}  // namespace dn
