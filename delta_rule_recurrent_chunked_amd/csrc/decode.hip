// decode.hip -- one token of the gated delta rule against a cached fp32 state,
// updated in place (the nnterp "linear_attention" page: the token-by-token rule on
// a decode step, with the cached state as state_input, overwritten afterwards).
//
// Per (sequence n, value head h), with the state stored key-major, M = S^T [Dk][Dv], and a
// decay a_i for each state row i (nnterp "decays": the log of the fraction kept):
//   M'     = diag(a) M
//   r_k    = M'^T k,  r_q = M'^T q          (column reductions over the key dim)
//   delta  = beta (v - r_k)                 (= -beta (S' k - v); "The Delta Rule" section
//                                            of the mutichung DeltaNet page)
//   o      = scale (r_q + (k.q) delta)      (= scale S_t q with S_t = S' + delta k^T)
//   M     <- M' + k delta^T
// a_i = exp(g[i]) with gates per key channel (the nnterp page's ChannelGates), a_i = exp(g)
// for every row with one gate per head (the same gate read with row stride 0), a_i = 1
// without a gate (a constant zero log decay read the same way).  The per-row form serves
// every step because it measured faster: with the per-row gate loads and exponentials
// ahead of the state stream, the compiler paces the sixteen state loads of a thread (about
// seven in flight per wave, each taken by the reduction as it lands) and spreads the
// sixteen stores through the update, where a single-factor form issued every state load at
// once and stored in a burst (168 us against 191 us for 256 x 32 heads at d = 128).
// With the in-rule normalisation (q, k -> x / sqrt(|x|^2 + eps)) the norms come out of
// the same reductions: r_k, r_q and k.q take the factors 1/|k|, 1/|q|, and the update
// adds k (delta / |k|)^T.
// The readout epilogue (normalisation over the head's d_v entries, silu output gate) can
// run fused: the workgroup holds the head's whole readout.
// The state is read once and written once: this kernel is bound by HBM bandwidth.
//
// Work decomposition: one workgroup per (n, h, slice of CW value columns; CW = Dv).  A
// thread owns a float4 of columns in RPT consecutive rows, so a wave reads whole
// CW*4-byte row segments and every state byte moves through one 128-bit load and one
// 128-bit store, both nontemporal (the state streams through once); the thread's RPT
// elements of k and q arrive in 16-byte loads.  Everything a workgroup reads is requested
// before its first wait.  Column sums over the key dim reduce across lanes (xor shuffles),
// then across the waves of the workgroup through LDS.
#include "internal.h"

namespace dn {
namespace {

// log decay 0 (a factor of 1): the gate an ungated step reads, so that it takes the
// per-row path too
__device__ const float zero_gate[1] = {0.f};

template <int DK, int CW>
struct DecodeShape {
    static constexpr int TPR = CW / 4;                              // threads per state row
    static constexpr int NT = (TPR * DK < 256) ? TPR * DK : 256;    // threads per workgroup
    static constexpr int RPP = NT / TPR;                            // rows per pass
    static constexpr int RPT = DK / RPP;                            // rows per thread
    static constexpr int NW = NT / 64;                              // waves
    static_assert(CW % 4 == 0 && TPR <= 64 && NT % 64 == 0 && DK % RPP == 0, "decode tiling");
};

// N consecutive elements of k or q as floats, from a 16-byte-aligned address
template <typename T, int N>
__device__ __forceinline__ void ld_vec(const T* p, float (&out)[N]) {
    constexpr int PER = 16 / (int)sizeof(T);
    static_assert(N % PER == 0, "ld_vec: whole 16-byte pieces");
#pragma unroll
    for (int i = 0; i < N / PER; ++i) {
        const uint4 u = *reinterpret_cast<const uint4*>(p + i * PER);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if constexpr (sizeof(T) == 2) {   // bf16 pair: low half first
                out[i * PER + 2 * j] = __uint_as_float(w[j] << 16);
                out[i * PER + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            } else {
                out[i * PER + j] = __uint_as_float(w[j]);
            }
        }
    }
}

template <typename T, int DK, int DV, int CW, bool VEC>
__global__ __launch_bounds__((DecodeShape<DK, CW>::NT)) void decode_kernel(DecodeArgs a) {
    using S = DecodeShape<DK, CW>;
    constexpr int TPR = S::TPR, RPT = S::RPT, NW = S::NW, SLICES = DV / CW;
    __shared__ float red[NW][2 * CW + 3];
    __shared__ float dsh[CW];
    __shared__ __align__(16) float osh[CW];   // the readout, for a fused epilogue

    const int tid = threadIdx.x;
    const int ct = tid % TPR;                 // float4 column group
    const int rg = tid / TPR;                 // row group
    const int slice = blockIdx.x % SLICES;
    const int nh = blockIdx.x / SLICES;       // n * Hv + h
    const int h = nh % a.Hv;
    const int n = nh / a.Hv;
    const int hq = h / (a.Hv / a.Hqk);

    const T* qp = static_cast<const T*>(a.q) + ((long)n * a.Hqk + hq) * DK;
    const T* kp = static_cast<const T*>(a.k) + ((long)n * a.Hqk + hq) * DK;
    float* Mp = a.state + (long)nh * DK * DV + slice * CW + ct * 4;

    // the state streams through once: nontemporal loads and stores keep it from
    // displacing q, k, v in the caches
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const int row0 = rg * RPT;                // this thread's rows: row0 .. row0 + RPT - 1
    f32x4v m[RPT];
#pragma unroll
    for (int p = 0; p < RPT; ++p)
        m[p] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(Mp + (long)(row0 + p) * DV));
    float kr[RPT], qr[RPT];
    if constexpr (VEC) {
        ld_vec(kp + row0, kr);
        ld_vec(qp + row0, qr);
    } else {
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            kr[p] = ld_f32(kp, row0 + p);
            qr[p] = ld_f32(qp, row0 + p);
        }
    }
    const long vo = (long)nh * DV + slice * CW + (tid < CW ? tid : 0);
    const float vval = ld_f32(static_cast<const T*>(a.v), vo);
    const float beta = a.beta[nh];
    float ar[RPT];   // decay of each of this thread's rows
    {
        const float* gp = a.g ? a.g : zero_gate;
        const long gs = a.g_per_key ? DK : (a.g ? 1 : 0);   // gates of (n, h) start at nh * gs
        const int gk = a.g_per_key ? 1 : 0;                 // row stride: 0 for one gate per head
#pragma unroll
        for (int p = 0; p < RPT; ++p) ar[p] = expf(gp[(long)nh * gs + (row0 + p) * gk]);
    }

    const bool nrm = a.qk_norm;
    float pk[4] = {0.f, 0.f, 0.f, 0.f}, pq[4] = {0.f, 0.f, 0.f, 0.f}, kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const float kd = ar[p] * kr[p], qd = ar[p] * qr[p];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pk[c] += m[p][c] * kd;
            pq[c] += m[p][c] * qd;
        }
        if (ct == 0) {
            kq += kr[p] * qr[p];
            kk += kr[p] * kr[p];
            qq += qr[p] * qr[p];
        }
    }
    // reduce over the row groups of this wave (lanes that share ct)
#pragma unroll
    for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pk[c] += __shfl_xor(pk[c], off);
            pq[c] += __shfl_xor(pq[c], off);
        }
        kq += __shfl_xor(kq, off);
        if (nrm) {
            kk += __shfl_xor(kk, off);
            qq += __shfl_xor(qq, off);
        }
    }
    const int lane = tid % 64, wave = tid / 64;
    if (lane < TPR) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            red[wave][ct * 4 + c] = pk[c];
            red[wave][CW + ct * 4 + c] = pq[c];
        }
        if (lane == 0) {
            red[wave][2 * CW] = kq;
            red[wave][2 * CW + 1] = kk;
            red[wave][2 * CW + 2] = qq;
        }
    }
    __syncthreads();
    if (tid < CW) {
        float rk = 0.f, rq = 0.f, kqs = 0.f, kks = 0.f, qqs = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            rk += red[w][tid];
            rq += red[w][CW + tid];
            kqs += red[w][2 * CW];
            kks += red[w][2 * CW + 1];
            qqs += red[w][2 * CW + 2];
        }
        float ik = 1.f;   // 1/|k| of the in-rule normalisation
        if (nrm) {
            ik = inv_norm(kks, a.eps);
            const float iq = inv_norm(qqs, a.eps);
            rk *= ik;
            rq *= iq;
            kqs *= ik * iq;
        }
        const float d = beta * (vval - rk);
        dsh[tid] = d * ik;
        const float ov = a.scale * (rq + kqs * d);
        if (a.ep.kind >= 0) osh[tid] = ov;
        else st_out(static_cast<T*>(a.o), vo, ov);
    }
    __syncthreads();

    const float d0 = dsh[ct * 4 + 0], d1 = dsh[ct * 4 + 1], d2 = dsh[ct * 4 + 2], d3 = dsh[ct * 4 + 3];
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        const float am = ar[p];
        f32x4v r;
        r[0] = am * m[p][0] + kr[p] * d0;
        r[1] = am * m[p][1] + kr[p] * d1;
        r[2] = am * m[p][2] + kr[p] * d2;
        r[3] = am * m[p][3] + kr[p] * d3;
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4v*>(Mp + (long)(row0 + p) * DV));
    }
    if (a.ep.kind >= 0 && tid < CW) {
        // readout epilogue over the head's d_v = CW entries (one slice per head), after the
        // state stores: the mean (layer norm) and the mean square around it, from the
        // readout in LDS; the weight, bias and gate of this column are requested first
        const int j = slice * CW + tid;
        const float wj = a.ep.w ? a.ep.w[j] : 1.f;
        const float bj = a.ep.b ? a.ep.b[j] : 0.f;
        const float zj = a.ep.gate ? ld_f32(static_cast<const T*>(a.ep.gate), vo) : 0.f;
        const float4* o4 = reinterpret_cast<const float4*>(osh);
        float sm = 0.f;
#pragma unroll
        for (int i = 0; i < CW / 4; ++i) sm += o4[i].x + o4[i].y + o4[i].z + o4[i].w;
        const float c = a.ep.kind == 1 ? sm * (1.f / CW) : 0.f;
        float sq = 0.f;
#pragma unroll
        for (int i = 0; i < CW / 4; ++i) {
            const float4 t = o4[i];
            sq += (t.x - c) * (t.x - c) + (t.y - c) * (t.y - c) + (t.z - c) * (t.z - c) + (t.w - c) * (t.w - c);
        }
        float y = (osh[tid] - c) * rsqrtf(sq * (1.f / CW) + a.ep.eps) * wj + bj;
        if (a.ep.gate) y *= silu(zj);
        st_out(static_cast<T*>(a.o), vo, y);
    }
}

template <typename T, int DK, int DV>
hipError_t launch_dims(const DecodeArgs& a, hipStream_t s) {
    constexpr int CW = DV;   // one workgroup per (sequence, head): 16 float4 of state per thread at d = 128
    using S = DecodeShape<DK, CW>;
    const long blocks = (long)a.N * a.Hv * (DV / CW);
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    // 16-byte loads of k and q when a thread's rows fill whole pieces and the rows of every
    // (sequence, head) start 16-byte aligned
    constexpr bool kVecShape = (S::RPT * sizeof(T)) % 16 == 0 && (DK * sizeof(T)) % 16 == 0;
    const bool aligned = ((reinterpret_cast<uintptr_t>(a.q) | reinterpret_cast<uintptr_t>(a.k)) & 15) == 0;
    const dim3 grid((unsigned)blocks), block(S::NT);
    if (kVecShape && aligned) hipLaunchKernelGGL((decode_kernel<T, DK, DV, CW, kVecShape>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<T, DK, DV, CW, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_dv(const DecodeArgs& a, hipStream_t s) {
    switch (a.Dv) {
        case 16: return launch_dims<T, DK, 16>(a, s);
        case 32: return launch_dims<T, DK, 32>(a, s);
        case 64: return launch_dims<T, DK, 64>(a, s);
        case 128: return launch_dims<T, DK, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_dk(const DecodeArgs& a, hipStream_t s) {
    switch (a.Dk) {
        case 16: return launch_dv<T, 16>(a, s);
        case 32: return launch_dv<T, 32>(a, s);
        case 64: return launch_dv<T, 64>(a, s);
        case 128: return launch_dv<T, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    if (a.N == 0) return hipSuccess;
    return a.bf16 ? launch_dk<__bf16>(a, s) : launch_dk<float>(a, s);
}

}  // namespace dn
