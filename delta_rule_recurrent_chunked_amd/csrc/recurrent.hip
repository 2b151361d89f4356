// recurrent.hip -- the rule token by token over whole sequences, with the state kept in
// registers, optionally writing the state after every token.  This is the recurrent
// route of the pages: the frankenstein forward processes the sequence token by token,
// and the nnterp page exposes the state after every token through its recurrent
// delta-rule route.  The per-token state trace is for inspection; the chunked form
// (prefill_fused.hip, prefill_generic.hip) is the fast prompt path.
//
// Per token, as in decode.hip (state stored key-major, M = S^T):
//   r_k = M'^T k, r_q = M'^T q with M' = diag(a) M, a the decay of each row
//   delta = beta (v - r_k),  o = scale (r_q + (k.q) delta),  M <- M' + k delta^T
// with the in-rule normalisation folded in as in decode.hip.
//
// One workgroup per (sequence, value head); a thread owns a float4 of columns in RPT
// consecutive rows for the whole sequence.  Two workgroup barriers per token (the column
// sums, then delta).  The trace, when asked for, streams out with nontemporal stores.
#include "internal.h"

namespace dn {
namespace {

template <int DK, int DV>
struct RecShape {
    static constexpr int TPR = DV / 4;                              // threads per state row
    static constexpr int NT = (TPR * DK < 256) ? TPR * DK : 256;    // threads per workgroup
    static constexpr int RPP = NT / TPR;                            // rows per pass
    static constexpr int RPT = DK / RPP;                            // rows per thread
    static constexpr int NW = NT / 64;                              // waves
    static_assert(DV % 4 == 0 && TPR <= 64 && NT % 64 == 0 && DK % RPP == 0, "recurrent tiling");
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__((RecShape<DK, DV>::NT)) void recurrent_kernel(RecurrentArgs a) {
    using S = RecShape<DK, DV>;
    constexpr int TPR = S::TPR, RPT = S::RPT, NW = S::NW;
    __shared__ float red[NW][2 * DV + 3];
    __shared__ float dsh[DV];
    typedef float f32x4v __attribute__((ext_vector_type(4)));

    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int ct = tid % TPR, rg = tid / TPR;
    const int nh = blockIdx.x;                // n * Hv + h
    const int h = nh % a.Hv, n = nh / a.Hv;
    const int hq = h / (a.Hv / a.Hqk);
    const int row0 = rg * RPT;
    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);

    f32x4v m[RPT];
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        m[p] = f32x4v{0.f, 0.f, 0.f, 0.f};
        if (a.h0) m[p] = *reinterpret_cast<const f32x4v*>(a.h0 + ((long)nh * DK + row0 + p) * DV + ct * 4);
    }
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    T* o = static_cast<T*>(a.o);

    for (long t = bos; t < eos; ++t) {
        const long kq0 = (t * a.Hqk + hq) * DK + row0;
        float kr[RPT], qr[RPT], ar[RPT];
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            kr[p] = ld_f32(k, kq0 + p);
            qr[p] = ld_f32(q, kq0 + p);
            ar[p] = 1.f;
        }
        if (a.g) {
            if (a.g_per_key) {
#pragma unroll
                for (int p = 0; p < RPT; ++p) ar[p] = expf(a.g[(t * a.Hv + h) * DK + row0 + p]);
            } else {
                const float al = expf(a.g[t * a.Hv + h]);
#pragma unroll
                for (int p = 0; p < RPT; ++p) ar[p] = al;
            }
        }
        const float vval = tid < DV ? ld_f32(v, (t * a.Hv + h) * DV + tid) : 0.f;
        const float beta = a.beta[t * a.Hv + h];

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
#pragma unroll
        for (int off = TPR; off < 64; off <<= 1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pk[c] += __shfl_xor(pk[c], off);
                pq[c] += __shfl_xor(pq[c], off);
            }
            kq += __shfl_xor(kq, off);
            kk += __shfl_xor(kk, off);
            qq += __shfl_xor(qq, off);
        }
        if (lane < TPR) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                red[wave][ct * 4 + c] = pk[c];
                red[wave][DV + ct * 4 + c] = pq[c];
            }
            if (lane == 0) {
                red[wave][2 * DV] = kq;
                red[wave][2 * DV + 1] = kk;
                red[wave][2 * DV + 2] = qq;
            }
        }
        __syncthreads();
        if (tid < DV) {
            float rk = 0.f, rq = 0.f, kqs = 0.f, kks = 0.f, qqs = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                rk += red[w][tid];
                rq += red[w][DV + tid];
                kqs += red[w][2 * DV];
                kks += red[w][2 * DV + 1];
                qqs += red[w][2 * DV + 2];
            }
            float ik = 1.f;
            if (a.qk_norm) {
                ik = inv_norm(kks, a.eps);
                const float iq = inv_norm(qqs, a.eps);
                rk *= ik;
                rq *= iq;
                kqs *= ik * iq;
            }
            const float d = beta * (vval - rk);
            dsh[tid] = d * ik;
            st_out(o, (t * a.Hv + h) * DV + tid, a.scale * (rq + kqs * d));
        }
        __syncthreads();
        const float d0 = dsh[ct * 4 + 0], d1 = dsh[ct * 4 + 1], d2 = dsh[ct * 4 + 2], d3 = dsh[ct * 4 + 3];
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            m[p][0] = ar[p] * m[p][0] + kr[p] * d0;
            m[p][1] = ar[p] * m[p][1] + kr[p] * d1;
            m[p][2] = ar[p] * m[p][2] + kr[p] * d2;
            m[p][3] = ar[p] * m[p][3] + kr[p] * d3;
        }
        if (a.trace) {
            float* tr = a.trace + ((t * a.Hv + h) * (long)DK + row0) * DV + ct * 4;
#pragma unroll
            for (int p = 0; p < RPT; ++p)
                __builtin_nontemporal_store(m[p], reinterpret_cast<f32x4v*>(tr + (long)p * DV));
        }
    }
    if (a.hT) {
#pragma unroll
        for (int p = 0; p < RPT; ++p)
            *reinterpret_cast<f32x4v*>(a.hT + ((long)nh * DK + row0 + p) * DV + ct * 4) = m[p];
    }
}

// ------------------------------------------------------------------------ reverse pass
// Walks each sequence backwards with the adjoint G = dL/dM_t in registers (the forward
// layout: a thread owns a float4 of columns in RPT consecutive rows).  Per token, with M'
// = a M_{t-1} rebuilt from the forward's state trace (or the initial state):
//   r = M'^T k, delta = beta (v - r), M_t = M' + k delta^T
//   G += scale q do^T,  dq = scale M_t do,  dd = G^T k,  dv = beta dd,
//   dbeta = dd . (v - r),  dk = G delta - beta M' dd,  G' = G - beta k dd^T,
//   dg = <G', M'>,  G <- a G'
// Column sums (r, dd) reduce over row groups like the forward; row sums (dq, dk) over the
// lanes that share rows; dbeta and dg through LDS atomics.  dq and dk come out per value
// head; a second kernel sums the value heads that share a query/key head.
template <typename T, int DK, int DV>
__global__ __launch_bounds__((RecShape<DK, DV>::NT)) void recurrent_bwd_kernel(RecurrentBwdArgs a) {
    using S = RecShape<DK, DV>;
    constexpr int TPR = S::TPR, RPT = S::RPT, NW = S::NW;
    __shared__ float red[NW][DV];
    __shared__ float vec_vr[DV], vec_d[DV], vec_do[DV], vec_dd[DV];
    __shared__ float acc2[2];
    typedef float f32x4v __attribute__((ext_vector_type(4)));

    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int ct = tid % TPR, rg = tid / TPR;
    const int nh = blockIdx.x;
    const int h = nh % a.Hv, n = nh / a.Hv;
    const int hq = h / (a.Hv / a.Hqk);
    const int row0 = rg * RPT;
    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    const T* dout = static_cast<const T*>(a.dout);

    f32x4v G[RPT];
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        G[p] = f32x4v{0.f, 0.f, 0.f, 0.f};
        if (a.dfinal) G[p] = *reinterpret_cast<const f32x4v*>(a.dfinal + ((long)nh * DK + row0 + p) * DV + ct * 4);
    }
    // column sums over the key rows: lanes sharing ct, then the waves through LDS
    auto colsum = [&](float (&c)[4]) {
#pragma unroll
        for (int off = TPR; off < 64; off <<= 1)
#pragma unroll
            for (int e = 0; e < 4; ++e) c[e] += __shfl_xor(c[e], off);
        if (lane < TPR) {
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wave][ct * 4 + e] = c[e];
        }
    };
    // row sums over the value columns: the TPR lanes that share rows
    auto rowsum = [&](float& x) {
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) x += __shfl_xor(x, off);
    };

    for (long t = eos - 1; t >= bos; --t) {
        // M_{t-1}: the trace of the previous token, or the sequence's initial state
        f32x4v Mp[RPT];
        const float* prev = t > bos ? a.trace + ((t - 1) * a.Hv + h) * (long)DK * DV
                                    : (a.h0 ? a.h0 + (long)nh * DK * DV : nullptr);
        const float al = a.g ? expf(a.g[t * a.Hv + h]) : 1.f;
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            Mp[p] = f32x4v{0.f, 0.f, 0.f, 0.f};
            if (prev) Mp[p] = al * *reinterpret_cast<const f32x4v*>(prev + (long)(row0 + p) * DV + ct * 4);
        }
        const long kq0 = (t * a.Hqk + hq) * DK + row0;
        float kr[RPT], qr[RPT];
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            kr[p] = ld_f32(k, kq0 + p);
            qr[p] = ld_f32(q, kq0 + p);
        }
        const float beta = a.beta[t * a.Hv + h];
        // r = M'^T k
        float c[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < RPT; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) c[e] += Mp[p][e] * kr[p];
        colsum(c);
        if (tid < 2) acc2[tid] = 0.f;
        __syncthreads();
        if (tid < DV) {
            float r = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) r += red[w][tid];
            const float vr = ld_f32(v, (t * a.Hv + h) * DV + tid) - r;   // v - r
            vec_vr[tid] = vr;
            vec_d[tid] = beta * vr;
            vec_do[tid] = a.scale * ld_f32(dout, (t * a.Hv + h) * DV + tid);
        }
        __syncthreads();
        float dl[4], dov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dl[e] = vec_d[ct * 4 + e];
            dov[e] = vec_do[ct * 4 + e];
        }
        // G += scale q do^T;  dq = scale M_t do;  dd = G^T k
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] = 0.f;
        float dqp[RPT];
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            dqp[p] = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                G[p][e] += qr[p] * dov[e];
                dqp[p] += (Mp[p][e] + kr[p] * dl[e]) * dov[e];
                c[e] += G[p][e] * kr[p];
            }
        }
#pragma unroll
        for (int p = 0; p < RPT; ++p) rowsum(dqp[p]);
        colsum(c);
        __syncthreads();
        if (tid < DV) {
            float dd = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) dd += red[w][tid];
            a.dv[(t * a.Hv + h) * DV + tid] = beta * dd;
            atomicAdd(&acc2[0], dd * vec_vr[tid]);   // dbeta = dd . (v - r)
            vec_dd[tid] = dd;
        }
        __syncthreads();
        float ddv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ddv[e] = vec_dd[ct * 4 + e];
        // dk = G delta - beta M' dd;  G' = G - beta k dd^T;  dg = <G', M'>;  G <- a G'
        float dkp[RPT], dgp = 0.f;
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            dkp[p] = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dkp[p] += G[p][e] * dl[e] - beta * Mp[p][e] * ddv[e];
                G[p][e] -= beta * kr[p] * ddv[e];
                dgp += G[p][e] * Mp[p][e];
                G[p][e] *= al;
            }
        }
#pragma unroll
        for (int p = 0; p < RPT; ++p) rowsum(dkp[p]);
        if (ct == 0) {
            float* dq = a.dq + (t * a.Hv + h) * (long)DK + row0;
            float* dk = a.dk + (t * a.Hv + h) * (long)DK + row0;
#pragma unroll
            for (int p = 0; p < RPT; ++p) {
                dq[p] = dqp[p];
                dk[p] = dkp[p];
            }
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) dgp += __shfl_xor(dgp, off);
        if (lane == 0) atomicAdd(&acc2[1], dgp);
        __syncthreads();
        if (tid == 0) {
            a.dbeta[t * a.Hv + h] = acc2[0];
            if (a.dg) a.dg[t * a.Hv + h] = acc2[1];
        }
        __syncthreads();   // acc2 and the reduction buffers are reused by the next token
    }
    if (a.dh0) {
#pragma unroll
        for (int p = 0; p < RPT; ++p)
            *reinterpret_cast<f32x4v*>(a.dh0 + ((long)nh * DK + row0 + p) * DV + ct * 4) = G[p];
    }
}

// dq, dk per value head [tokens, Hv, D] -> per query/key head [tokens, Hqk, D]: the sum over
// the Hv / Hqk value heads that read each query/key head
__global__ __launch_bounds__(256) void group_sum_kernel(const float* src, float* dst, long tokens, int Hqk,
                                                       int grp, int D) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    const long total = tokens * Hqk * D;
    if (i >= total) return;
    const int d = (int)(i % D);
    const long th = i / D;          // t * Hqk + hq
    const int hq = (int)(th % Hqk);
    const long t = th / Hqk;
    float s = 0.f;
    for (int r = 0; r < grp; ++r) s += src[((t * Hqk + hq) * grp + r) * (long)D + d];
    dst[i] = s;
}

template <typename T, int DK>
hipError_t launch_dv(const RecurrentArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((long)a.N * a.Hv));
    switch (a.Dv) {
        case 16: hipLaunchKernelGGL((recurrent_kernel<T, DK, 16>), grid, dim3(RecShape<DK, 16>::NT), 0, s, a); break;
        case 32: hipLaunchKernelGGL((recurrent_kernel<T, DK, 32>), grid, dim3(RecShape<DK, 32>::NT), 0, s, a); break;
        case 64: hipLaunchKernelGGL((recurrent_kernel<T, DK, 64>), grid, dim3(RecShape<DK, 64>::NT), 0, s, a); break;
        case 128: hipLaunchKernelGGL((recurrent_kernel<T, DK, 128>), grid, dim3(RecShape<DK, 128>::NT), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dk(const RecurrentArgs& a, hipStream_t s) {
    switch (a.Dk) {
        case 16: return launch_dv<T, 16>(a, s);
        case 32: return launch_dv<T, 32>(a, s);
        case 64: return launch_dv<T, 64>(a, s);
        case 128: return launch_dv<T, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename T, int DK>
hipError_t launch_bwd_dv(const RecurrentBwdArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((long)a.N * a.Hv));
    switch (a.Dv) {
        case 16: hipLaunchKernelGGL((recurrent_bwd_kernel<T, DK, 16>), grid, dim3(RecShape<DK, 16>::NT), 0, s, a); break;
        case 32: hipLaunchKernelGGL((recurrent_bwd_kernel<T, DK, 32>), grid, dim3(RecShape<DK, 32>::NT), 0, s, a); break;
        case 64: hipLaunchKernelGGL((recurrent_bwd_kernel<T, DK, 64>), grid, dim3(RecShape<DK, 64>::NT), 0, s, a); break;
        case 128: hipLaunchKernelGGL((recurrent_bwd_kernel<T, DK, 128>), grid, dim3(RecShape<DK, 128>::NT), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_bwd_dk(const RecurrentBwdArgs& a, hipStream_t s) {
    switch (a.Dk) {
        case 16: return launch_bwd_dv<T, 16>(a, s);
        case 32: return launch_bwd_dv<T, 32>(a, s);
        case 64: return launch_bwd_dv<T, 64>(a, s);
        case 128: return launch_bwd_dv<T, 128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_recurrent_bwd(const RecurrentBwdArgs& a, hipStream_t s) {
    if ((long)a.N * a.Hv == 0) return hipSuccess;
    if ((long)a.N * a.Hv > 0x7fffffffL) return hipErrorInvalidConfiguration;
    const hipError_t e = a.bf16 ? launch_bwd_dk<__bf16>(a, s) : launch_bwd_dk<float>(a, s);
    if (e != hipSuccess) return e;
    const long tokens = (long)a.B * a.T;
    if (a.dq_out && tokens > 0) {   // sum the value heads of each query/key head
        const int grp = a.Hv / a.Hqk;
        const long total = tokens * a.Hqk * a.Dk;
        const long blocks = (total + 255) / 256;
        if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(group_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.dq, a.dq_out, tokens, a.Hqk, grp, a.Dk);
        hipLaunchKernelGGL(group_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a.dk, a.dk_out, tokens, a.Hqk, grp, a.Dk);
    }
    return hipGetLastError();
}

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t s) {
    if ((long)a.N * a.Hv == 0) return hipSuccess;
    if ((long)a.N * a.Hv > 0x7fffffffL) return hipErrorInvalidConfiguration;
    return a.bf16 ? launch_dk<__bf16>(a, s) : launch_dk<float>(a, s);
}

}  // namespace dn
