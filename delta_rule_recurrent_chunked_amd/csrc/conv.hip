// conv.hip -- the short causal depthwise convolution (+ silu) in front of the rule (the
// mutichung DeltaNet block flowchart's "Conv" and "SiLU" boxes on the q/k and v branches;
// depthwise, generalising the shift SSM).  Per channel c:
//
//   y_t[c] = act(b[c] + sum_{j<W} w[c][j] x_{t-W+1+j}[c])
//
// with the inputs before a sequence's first token taken from its conv state (the W - 1
// inputs before it, oldest first) or zero, and the sequence's last W - 1 inputs written out
// as its final state.
//
// Prompt: a thread owns 8 consecutive channels (one 16-byte piece of bf16) over a block of
// 32 consecutive tokens of the packed stream, and slides a window of the last W - 1 inputs
// through them in registers: each input is read once (plus W - 1 at the block start) and
// each output written once; the lanes of a wave read one token's consecutive channels.
// A block that crosses sequence starts refills the window from the next sequence's state.
// The same kernel serves the fused prologue (dn_conv_qkv): the q, k and v channel ranges go
// to their own tensors, and q and k are L2-normalised per head, the head's Dk / 8 lanes
// adding their squares by DPP lane moves, so the rule's inputs are ready in one pass.
// Decode step: a thread owns 8 channels of one sequence and shifts their state in place.
#include "internal.h"

namespace dn {
namespace {

constexpr int CG = 8;      // channels per thread
constexpr int TB = 32;     // tokens per thread (prompt)
constexpr int NTH = 256;   // threads per workgroup

template <typename T>
__device__ __forceinline__ void ld8(const T* p, float (&v)[CG]) {
    if constexpr (sizeof(T) == 2) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// 8 outputs, in nontemporal stores (nothing reads them again in this kernel)
template <typename T>
__device__ __forceinline__ void st8(T* p, const float (&v)[CG]) {
    if constexpr (sizeof(T) == 2) {
        __bf16 h[CG];
#pragma unroll
        for (int e = 0; e < CG; ++e) h[e] = (__bf16)v[e];
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, h), reinterpret_cast<u32x4*>(p));
    } else {
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store(f32x4v{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4v*>(p));
        __builtin_nontemporal_store(f32x4v{v[4], v[5], v[6], v[7]}, reinterpret_cast<f32x4v*>(p + 4));
    }
}

__device__ __forceinline__ void seq_of(const ConvArgs& a, long t, int& n, long& bos, long& eos) {
    if (a.cu) {   // the sequence holding token t: the largest n with cu[n] <= t
        int lo = 0, hi = a.N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
    } else {
        n = (int)(t / a.T);
    }
    seq_range(a.cu, n, a.T, bos, eos);
}

template <typename T, int W>
__device__ __forceinline__ float state_at(const ConvArgs& a, int n, int c, int k) {
    return a.s0 ? ld_f32(static_cast<const T*>(a.s0), ((long)n * a.C + c) * (W - 1) + k) : 0.f;
}

// DPP lane moves within rows of 16 lanes (every lane has a source)
template <int CTRL>
__device__ __forceinline__ float dpp16(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// sum over each group of G consecutive lanes (G = 2, 4, 8 or 16, aligned), in every lane:
// lane ^ 1, lane ^ 2, then the 8- and 16-lane mirrors
__device__ __forceinline__ float group_sum(float x, int G) {
    x += dpp16<0xB1>(x);
    if (G >= 4) x += dpp16<0x4E>(x);
    if (G >= 8) x += dpp16<0x141>(x);
    if (G >= 16) x += dpp16<0x140>(x);
    return x;
}

template <typename T, int W>
__global__ __launch_bounds__(NTH) void conv_kernel(ConvArgs a) {
    const int g = blockIdx.y * NTH + threadIdx.x;   // channel group; blockIdx.x: token block
    const bool act = g * CG < a.C;                  // lanes past C compute lane 0's channels
    const int c0 = act ? g * CG : 0;                // and store nothing
    const T* x = static_cast<const T*>(a.x);
    T* sT = static_cast<T*>(a.sT);
    float w[W][CG], bb[CG];
#pragma unroll
    for (int e = 0; e < CG; ++e) {
        bb[e] = a.b ? a.b[c0 + e] : 0.f;
#pragma unroll
        for (int j = 0; j < W; ++j) w[j][e] = a.w[(long)(c0 + e) * W + j];
    }
    // this lane's output: q, k (normalised per head when asked) or the rest
    T* ob;
    long ostr;
    bool nrm = false;
    if (c0 < a.qk) {
        ob = static_cast<T*>(a.q) + c0;
        ostr = a.qk;
        nrm = a.qk_norm;
    } else if (c0 < 2 * a.qk) {
        ob = static_cast<T*>(a.k) + (c0 - a.qk);
        ostr = a.qk;
        nrm = a.qk_norm;
    } else {
        ob = static_cast<T*>(a.y) + (c0 - 2 * a.qk);
        ostr = a.y_stride;
    }
    const int G = a.Dk / CG;   // lanes per q/k head
    if (blockIdx.x == 0 && sT && act) {   // empty sequences keep their state
        for (int n = 0; n < a.N; ++n) {
            long bos, eos;
            seq_range(a.cu, n, a.T, bos, eos);
            if (eos != bos) continue;
#pragma unroll
            for (int e = 0; e < CG; ++e)
#pragma unroll
                for (int k = 0; k < W - 1; ++k)
                    st_out(sT, ((long)n * a.C + c0 + e) * (W - 1) + k, state_at<T, W>(a, n, c0 + e, k));
        }
    }
    const long total = (long)a.B * a.T;
    const long t0 = (long)blockIdx.x * TB;
    if (t0 >= total) return;
    int n;
    long bos, eos;
    seq_of(a, t0, n, bos, eos);
    float win[W - 1][CG];   // x_{t-W+1} .. x_{t-1}
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const long s = t0 - (W - 1) + k;
        if (s >= bos) {
            ld8(x + s * a.C + c0, win[k]);
        } else {
#pragma unroll
            for (int e = 0; e < CG; ++e) win[k][e] = state_at<T, W>(a, n, c0 + e, (int)(s - bos + W - 1));
        }
    }
    const long t1 = t0 + TB < total ? t0 + TB : total;
    for (long t = t0; t < t1; ++t) {
        if (t == eos) {   // the next non-empty sequence starts here: its state fills the window
            do {
                ++n;
                seq_range(a.cu, n, a.T, bos, eos);
            } while (eos == bos);
#pragma unroll
            for (int k = 0; k < W - 1; ++k)
#pragma unroll
                for (int e = 0; e < CG; ++e) win[k][e] = state_at<T, W>(a, n, c0 + e, k);
        }
        float xv[CG], out[CG], ss = 0.f;
        ld8(x + t * a.C + c0, xv);
#pragma unroll
        for (int e = 0; e < CG; ++e) {
            float acc = bb[e] + w[W - 1][e] * xv[e];
#pragma unroll
            for (int k = 0; k < W - 1; ++k) acc += w[k][e] * win[k][e];
            out[e] = a.silu ? silu(acc) : acc;
            ss += out[e] * out[e];
        }
        if (a.qk_norm) {   // |head|^2 over its G lanes (every lane of the wave takes part)
            ss = group_sum(ss, G);
            if (nrm) {
                const float r = 1.f / __builtin_sqrtf(ss + a.eps);
#pragma unroll
                for (int e = 0; e < CG; ++e) out[e] *= r;
            }
        }
        if (act) st8(ob + t * ostr, out);
#pragma unroll
        for (int k = 0; k < W - 2; ++k)
#pragma unroll
            for (int e = 0; e < CG; ++e) win[k][e] = win[k + 1][e];
#pragma unroll
        for (int e = 0; e < CG; ++e) win[W - 2][e] = xv[e];
        if (t == eos - 1 && sT && act) {
#pragma unroll
            for (int e = 0; e < CG; ++e)
#pragma unroll
                for (int k = 0; k < W - 1; ++k) st_out(sT, ((long)n * a.C + c0 + e) * (W - 1) + k, win[k][e]);
        }
    }
}

// n consecutive state entries as floats, 16 bytes at a time when `vec` (the host checked
// the alignment), else one by one
template <typename T, int NE>
__device__ __forceinline__ void ld_state(const T* p, float (&v)[NE], bool vec) {
    constexpr int PER = 16 / (int)sizeof(T);
    if (vec && NE % PER == 0) {
#pragma unroll
        for (int i = 0; i < NE / PER; ++i) {
            const uint4 u = *reinterpret_cast<const uint4*>(p + i * PER);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (sizeof(T) == 2) {
                    v[i * PER + 2 * j] = __uint_as_float(w[j] << 16);
                    v[i * PER + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
                } else {
                    v[i * PER + j] = __uint_as_float(w[j]);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NE; ++i) v[i] = ld_f32(p, i);
    }
}

template <typename T, int NE>
__device__ __forceinline__ void st_state(T* p, const float (&v)[NE], bool vec) {
    constexpr int PER = 16 / (int)sizeof(T);
    if (vec && NE % PER == 0) {
#pragma unroll
        for (int i = 0; i < NE / PER; ++i) {
            T h[PER];
#pragma unroll
            for (int e = 0; e < PER; ++e) h[e] = (T)v[i * PER + e];
            *reinterpret_cast<uint4*>(p + i * PER) = __builtin_bit_cast(uint4, h);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NE; ++i) st_out(p, i, v[i]);
    }
}

template <typename T, int W>
__global__ __launch_bounds__(NTH) void conv_step_kernel(ConvArgs a, bool vec) {
    const long idx = (long)blockIdx.x * NTH + threadIdx.x;
    const int groups = a.C / CG;
    const long n = idx / groups;
    if (n >= a.N) return;
    const int c0 = (int)(idx % groups) * CG;
    T* st = static_cast<T*>(a.sT) + (n * a.C + c0) * (W - 1);   // 8 channels x (W - 1), contiguous
    float xv[CG], out[CG], sf[CG * (W - 1)];
    ld8(static_cast<const T*>(a.x) + n * a.C + c0, xv);
    ld_state<T, CG * (W - 1)>(st, sf, vec);
#pragma unroll
    for (int e = 0; e < CG; ++e) {
        const float* we = a.w + (long)(c0 + e) * W;
        float acc = (a.b ? a.b[c0 + e] : 0.f) + we[W - 1] * xv[e];
#pragma unroll
        for (int k = 0; k < W - 1; ++k) acc += we[k] * sf[e * (W - 1) + k];
        out[e] = a.silu ? silu(acc) : acc;
    }
    st8(static_cast<T*>(a.y) + n * a.C + c0, out);
#pragma unroll
    for (int e = 0; e < CG; ++e) {   // shift by one, append x
#pragma unroll
        for (int k = 0; k < W - 2; ++k) sf[e * (W - 1) + k] = sf[e * (W - 1) + k + 1];
        sf[e * (W - 1) + W - 2] = xv[e];
    }
    st_state<T, CG * (W - 1)>(st, sf, vec);
}

template <typename T, int W>
hipError_t launch_w(const ConvArgs& a, hipStream_t s, bool step) {
    const long groups = a.C / CG;
    if (step) {
        const long blocks = ((long)a.N * groups + NTH - 1) / NTH;
        if (blocks == 0) return hipSuccess;
        if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
        const bool vec = (reinterpret_cast<uintptr_t>(a.sT) & 15) == 0;
        hipLaunchKernelGGL((conv_step_kernel<T, W>), dim3((unsigned)blocks), dim3(NTH), 0, s, a, vec);
    } else {
        const long total = (long)a.B * a.T;
        long tblocks = (total + TB - 1) / TB;
        if (tblocks == 0) {
            if (!a.sT || a.N == 0) return hipSuccess;
            tblocks = 1;   // only the empty-sequence states to copy
        }
        const long cblocks = (groups + NTH - 1) / NTH;
        if (tblocks > 0x7fffffffL || cblocks > 65535) return hipErrorInvalidConfiguration;
        const dim3 grid((unsigned)tblocks, (unsigned)cblocks);
        hipLaunchKernelGGL((conv_kernel<T, W>), grid, dim3(NTH), 0, s, a);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const ConvArgs& a, hipStream_t s, bool step) {
    switch (a.W) {
        case 2: return launch_w<T, 2>(a, s, step);
        case 3: return launch_w<T, 3>(a, s, step);
        case 4: return launch_w<T, 4>(a, s, step);
        case 5: return launch_w<T, 5>(a, s, step);
        case 6: return launch_w<T, 6>(a, s, step);
        case 7: return launch_w<T, 7>(a, s, step);
        case 8: return launch_w<T, 8>(a, s, step);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_causal_conv(const ConvArgs& a, hipStream_t s) {
    return a.bf16 ? launch_t<__bf16>(a, s, false) : launch_t<float>(a, s, false);
}

hipError_t launch_causal_conv_step(const ConvArgs& a, hipStream_t s) {
    return a.bf16 ? launch_t<__bf16>(a, s, true) : launch_t<float>(a, s, true);
}

}  // namespace dn
