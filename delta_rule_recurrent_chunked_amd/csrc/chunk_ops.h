// chunk_ops.h -- device helpers shared by the T/P kernel (chunk_tp.hip) and the chunkwise
// reverse pass (chunk_bwd.hip): MFMA operand fragments out of LDS, tile stores,
// DPP lane sums, the in-chunk decay scan, buffer loads, and the chunk numbering of the
// workspace records.
#pragma once

#include "internal.h"
#include "mfma_ops.h"

namespace dn {
namespace ck {

constexpr int BC = 64;             // chunk
constexpr int BS = 32;             // state columns per slice
constexpr int P64 = BC + 16;       // bf16 pitches (16-byte reads of 16 rows conflict-free)
constexpr int P32 = BS + 16;
constexpr int ADP = 136;           // A's diagonal 16x16 blocks, 120 packed fp16 entries + spare
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// --------------------------------------------------------------------- fragments
__device__ __forceinline__ bf16x8 frag_r(const __bf16* S, int pitch, int r0, int k0, int l16, int q16) {
    return ld8(S + (r0 + l16) * pitch + k0 + 8 * q16);
}
__device__ __forceinline__ bf16x8 frag_c(const __bf16* S, int pitch, int c0, int k0, int l16, int q16) {
    const __bf16* p = S + (k0 + 8 * q16 + (l16 >> 2)) * pitch + c0 + 4 * (l16 & 3);
    return cat(trld(p), trld(p + 4 * pitch));
}
__device__ __forceinline__ bf16x8 scale_r(bf16x8 x, float f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (__bf16)((float)x[e] * f);
    return x;
}
// an accumulator tile C[16 i + 4 q16 + e][16 j + l16] to a bf16 row-major matrix
__device__ __forceinline__ void put_tile(__bf16* S, int pitch, int i, int j, const f32x4& c, int l16, int q16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) S[(16 * i + 4 * q16 + e) * pitch + 16 * j + l16] = (__bf16)c[e];
}
// the same tile transposed (S[16 j + l16][16 i + 4 q16 + e]): one 8-byte write per lane
__device__ __forceinline__ void put_tile_t(__bf16* S, int pitch, int i, int j, const f32x4& c, int l16, int q16) {
    st4(S + (16 * j + l16) * pitch + 16 * i + 4 * q16, c[0], c[1], c[2], c[3]);
}
// DPP lane moves within rows of 16 lanes (every lane has a source)
template <int CTRL>
__device__ __forceinline__ float dpp16(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// sum over the 16 lanes of one q16 group (the tile's columns) of each of the lane's 4 rows:
// lane ^ 1, lane ^ 2 (quad permutes), then the 8- and 16-lane mirrors, in every lane
__device__ __forceinline__ f32x4 row_sum16(f32x4 v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float x = v[e];
        x += dpp16<0xB1>(x);
        x += dpp16<0x4E>(x);
        x += dpp16<0x141>(x);
        x += dpp16<0x140>(x);
        v[e] = x;
    }
    return v;
}
// x as a value the compiler cannot see through: addresses derived from it are computed where
// they are used instead of being hoisted out of loops and held in registers
__device__ __forceinline__ int fresh(int x) {
    __asm__ volatile("" : "+v"(x));
    return x;
}
// sum over the wave, the same value in every lane: the four 16-lane row sums, read out and
// added in row order
__device__ __forceinline__ float wave_sum(float x) {
    x += dpp16<0xB1>(x);
    x += dpp16<0x4E>(x);
    x += dpp16<0x141>(x);
    x += dpp16<0x140>(x);
    const int b = __builtin_bit_cast(int, x);
    return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0)) + __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16))) +
           (__builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32)) + __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48)));
}
// x moved by a DPP control; lanes with no source (or rows outside row_mask) get 0
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or0(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xf, true));
}
// gamma: inclusive scan of g over a chunk on one wave (lane = row), by DPP: shifts right by
// 1, 2, 4, 8 lanes within each 16-lane row, then lane 15 of each row added into the next row
// and lane 31 into the upper two rows; gl = gamma of row 63
__device__ __forceinline__ float gamma_scan(float g, float& gl) {
    g += dpp_or0<0x111, 0xf>(g);   // row_shr:1
    g += dpp_or0<0x112, 0xf>(g);   // row_shr:2
    g += dpp_or0<0x114, 0xf>(g);   // row_shr:4
    g += dpp_or0<0x118, 0xf>(g);   // row_shr:8
    g += dpp_or0<0x142, 0xa>(g);   // row_bcast:15 into rows 1 and 3
    g += dpp_or0<0x143, 0xc>(g);   // row_bcast:31 into rows 2 and 3
    gl = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, g), 63));
    return g;
}
// lower tile u < 10 of a 64 x 64 matrix in 16 x 16 blocks: (ri, ci), ci <= ri
__device__ __forceinline__ void lower_tile(int u, int& ri, int& ci) {
    ri = u < 1 ? 0 : u < 3 ? 1 : u < 6 ? 2 : 3;
    ci = u - ri * (ri + 1) / 2;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ float ld32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// chunk number cid -> sequence n, chunk c of it, the sequence's first token and length;
// false for a number no chunk uses
__device__ __forceinline__ bool chunk_of_id(const PrefillArgs& a, long cid, int& n, long& c, long& bos, long& L) {
    if (a.cu) {   // the last sequence whose first chunk number is <= cid (strictly increasing)
        int lo = 0, hi = a.N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (chunk_id_base(a, mid) <= cid) lo = mid; else hi = mid - 1;
        }
        n = lo;
    } else {
        n = (int)(cid / ((a.T + BC - 1) / BC));
    }
    long eos;
    seq_range(a.cu, n, a.T, bos, eos);
    L = eos - bos;
    c = cid - chunk_id_base(a, n);
    return c * BC < L;
}


}  // namespace ck
}  // namespace dn
