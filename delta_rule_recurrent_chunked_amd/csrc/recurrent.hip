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

}  // namespace

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t s) {
    if ((long)a.N * a.Hv == 0) return hipSuccess;
    if ((long)a.N * a.Hv > 0x7fffffffL) return hipErrorInvalidConfiguration;
    return a.bf16 ? launch_dk<__bf16>(a, s) : launch_dk<float>(a, s);
}

}  // namespace dn
