// epilogue.hip -- the readout epilogue over a prefill's output: per (token, value head),
// over the d_v entries of the readout, a normalisation (the frankenstein "DeltaNet
// Attention" page's layer norm of the recurrent readout, or the RMSNorm box that follows
// the Delta Rule box in the mutichung DeltaNet block flowchart), then the silu output
// gate (frankenstein g_proj):
//
//   RMS:    y = o / sqrt(mean(o^2) + eps) * w
//   layer:  y = (o - mean(o)) / sqrt(mean((o - mean(o))^2) + eps) * w + b
//   gate:   y <- y * silu(z)
//
// A row of d_v entries is spread over d_v * sizeof(T) / 16 lanes, one 16-byte piece each;
// the mean and the sum of squares reduce over those lanes with DPP butterflies (two
// passes: the mean first, then squares around it).  The weight, bias and gate of a lane's
// entries are requested with its piece of o, before the first wait.  Each byte of o, z and
// y moves once, in 16-byte nontemporal loads and stores (nothing is read again, so they
// bypass the caches' retention): the kernel is bound by HBM bandwidth.
#include "internal.h"

namespace dn {
namespace {

template <typename T>
__device__ __forceinline__ void ld16(const void* base, long off, float (&x)[16 / sizeof(T)]) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 uv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const T*>(base) + off));
    const uint4 u = make_uint4(uv[0], uv[1], uv[2], uv[3]);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (sizeof(T) == 2) {   // bf16 pair: low half first
            x[2 * j] = __uint_as_float(w[j] << 16);
            x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        } else {
            x[j] = __uint_as_float(w[j]);
        }
    }
}

template <typename T>
__device__ __forceinline__ void st16(void* base, long off, const float (&y)[16 / sizeof(T)]) {
    T* p = static_cast<T*>(base) + off;
    if constexpr (sizeof(T) == 2) {
        __bf16 h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = (__bf16)y[e];
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, h), reinterpret_cast<u32x4*>(p));
    } else {
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(f32x4v{y[0], y[1], y[2], y[3]}, reinterpret_cast<f32x4v*>(p));
    }
}

// DPP move with bound_ctrl (every source lane exists for the patterns used here)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}

// Sum over groups of N consecutive lanes (N a power of two <= 32), in every lane:
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror, then a swap of
// 16-lane halves of 32
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if (N > 1) x += dpp<0xb1>(x);
    if (N > 2) x += dpp<0x4e>(x);
    if (N > 4) x += dpp<0x141>(x);
    if (N > 8) x += dpp<0x140>(x);
    if (N > 16) x += __shfl_xor(x, 16);
    return x;
}

template <typename T, int DV>
__global__ __launch_bounds__(256) void norm_gate_kernel(NormGateArgs a) {
    constexpr int EPV = 16 / (int)sizeof(T);   // entries per 16-byte piece
    constexpr int TPR = DV / EPV;              // lanes per row
    constexpr int RPB = 256 / TPR;             // rows per workgroup
    static_assert(TPR >= 2 && TPR <= 32 && (TPR & (TPR - 1)) == 0, "norm_gate tiling");
    const int tid = threadIdx.x, part = tid % TPR;
    const long row = (long)blockIdx.x * RPB + tid / TPR;
    const bool live = row < a.rows;
    const long off = row * DV + part * EPV;
    float x[EPV], z[EPV], w[EPV], b[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
        x[e] = z[e] = b[e] = 0.f;
        w[e] = 1.f;
    }
    if (live) {
        ld16<T>(a.o, off, x);
        if (a.ep.gate) ld16<T>(a.ep.gate, off, z);
    }
    if (a.ep.w) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) w[e] = a.ep.w[part * EPV + e];
    }
    if (a.ep.b) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) b[e] = a.ep.b[part * EPV + e];
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) s += x[e];
    s = group_sum<TPR>(s);
    const float c = a.ep.kind == 1 ? s * (1.f / DV) : 0.f;   // layer norm: the mean
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) q += (x[e] - c) * (x[e] - c);
    q = group_sum<TPR>(q);
    const float r = rsqrtf(q * (1.f / DV) + a.ep.eps);
    if (!live) return;
    float y[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
        float t = (x[e] - c) * r * w[e] + b[e];
        if (a.ep.gate) t *= silu(z[e]);
        y[e] = t;
    }
    st16<T>(a.y, off, y);
}

template <typename T>
hipError_t launch_t(const NormGateArgs& a, hipStream_t s) {
    auto go = [&](auto kern, int rpb) {
        const long blocks = (a.rows + rpb - 1) / rpb;
        if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, a);
        return hipGetLastError();
    };
    constexpr int EPV = 16 / (int)sizeof(T);
    switch (a.Dv) {
        case 16: return go(norm_gate_kernel<T, 16>, 256 / (16 / EPV));
        case 32: return go(norm_gate_kernel<T, 32>, 256 / (32 / EPV));
        case 64: return go(norm_gate_kernel<T, 64>, 256 / (64 / EPV));
        case 128: return go(norm_gate_kernel<T, 128>, 256 / (128 / EPV));
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_norm_gate(const NormGateArgs& a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    return a.bf16 ? launch_t<__bf16>(a, s) : launch_t<float>(a, s);
}

}  // namespace dn
