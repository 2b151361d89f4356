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
// One workgroup per (sequence, value head, slice of CW = min(Dv, 32) value columns): the
// columns are independent, and every slice forms k.q and the norms itself.  A thread owns a
// float4 of columns in RPT consecutive rows for the whole sequence.  Two workgroup barriers
// per token (the column sums, then delta).  The trace, when asked for, streams out with
// nontemporal stores.
#include "chunk_ops.h"

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

constexpr int bwd_cols(int Dk) { return Dk >= 32 ? 8 : 16; }

template <typename T, int DK, int DV, int CW>
__global__ __launch_bounds__((RecShape<DK, CW>::NT)) void recurrent_kernel(RecurrentArgs a) {
    using S = RecShape<DK, CW>;
    constexpr int TPR = S::TPR, RPT = S::RPT, NW = S::NW, NSL = DV / CW;
    __shared__ float red[NW][2 * CW + 3];
    __shared__ float dsh[CW];
    typedef float f32x4v __attribute__((ext_vector_type(4)));

    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int ct = tid % TPR, rg = tid / TPR;
    const int slice = blockIdx.x % NSL;
    const int nh = blockIdx.x / NSL;          // n * Hv + h
    const int h = nh % a.Hv, n = nh / a.Hv;
    const int hq = h / (a.Hv / a.Hqk);
    const int row0 = rg * RPT, jc = slice * CW + ct * 4;   // this thread's first column
    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);

    f32x4v m[RPT];
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        m[p] = f32x4v{0.f, 0.f, 0.f, 0.f};
        if (a.h0) m[p] = *reinterpret_cast<const f32x4v*>(a.h0 + ((long)nh * DK + row0 + p) * DV + jc);
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
        const float vval = tid < CW ? ld_f32(v, (t * a.Hv + h) * DV + slice * CW + tid) : 0.f;
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
            st_out(o, (t * a.Hv + h) * DV + slice * CW + tid, a.scale * (rq + kqs * d));
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
            float* tr = a.trace + ((t * a.Hv + h) * (long)DK + row0) * DV + jc;
#pragma unroll
            for (int p = 0; p < RPT; ++p)
                __builtin_nontemporal_store(m[p], reinterpret_cast<f32x4v*>(tr + (long)p * DV));
        }
    }
    if (a.hT) {
#pragma unroll
        for (int p = 0; p < RPT; ++p)
            *reinterpret_cast<f32x4v*>(a.hT + ((long)nh * DK + row0 + p) * DV + jc) = m[p];
    }
}

// ------------------------------------------------------------------------ reverse pass
// Walks each sequence backwards with the adjoint G = dL/dM_t in registers.  Per token, with
// M' = a M_{t-1} rebuilt from the forward's state trace (or the initial state):
//   r = M'^T k, delta = beta (v - r), M_t = M' + k delta^T
//   G += scale q do^T,  dq = scale M_t do,  dd = G^T k,  dv = beta dd,
//   dbeta = dd . (v - r),  dk = G delta - beta M' dd,  G' = G - beta k dd^T,
//   dg = <G', M'>,  G <- a G'
// The value columns are independent up to the row sums (dq, dk) and the scalars (dbeta,
// dg), so a workgroup takes one slice of CW columns of one (sequence, value head) and writes
// its share of those; a second kernel adds the slices (and the value heads that share a
// query/key head) in a fixed order.  Column sums (r, dd) reduce over row groups like the
// forward, row sums over the lanes that share rows.  Each token's inputs and trace state are
// requested one token ahead, while the previous one is computed.
template <typename T, int DK, int CW>
struct BwdIn {
    float m[RecShape<DK, CW>::RPT][4];   // M_{t-1} (this thread's block)
    float k[RecShape<DK, CW>::RPT], q[RecShape<DK, CW>::RPT];
    float g[RecShape<DK, CW>::RPT];      // log decay of each of the thread's rows
    float v, dout, beta;
};

template <typename T, int DK, int DV, int CW>
__device__ __forceinline__ void bwd_fetch(const RecurrentBwdArgs& a, long t, long bos, int nh, int h,
                                          int hq, int row0, int ct, int tid, int j0, BwdIn<T, DK, CW>& f) {
    constexpr int RPT = RecShape<DK, CW>::RPT;
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    const float* prev = t > bos ? a.trace + ((t - 1) * a.Hv + h) * (long)DK * DV
                                : (a.h0 ? a.h0 + (long)nh * DK * DV : nullptr);
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        f32x4v x = f32x4v{0.f, 0.f, 0.f, 0.f};
        if (prev) x = *reinterpret_cast<const f32x4v*>(prev + (long)(row0 + p) * DV + j0 + ct * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) f.m[p][e] = x[e];
    }
    const long kq0 = (t * a.Hqk + hq) * DK + row0;
#pragma unroll
    for (int p = 0; p < RPT; ++p) {
        f.k[p] = ld_f32(static_cast<const T*>(a.k), kq0 + p);
        f.q[p] = ld_f32(static_cast<const T*>(a.q), kq0 + p);
    }
    const long vo = (t * a.Hv + h) * DV + j0 + (tid < CW ? tid : 0);
    f.v = ld_f32(static_cast<const T*>(a.v), vo);
    f.dout = ld_f32(static_cast<const T*>(a.dout), vo);
    f.beta = a.beta[t * a.Hv + h];
#pragma unroll
    for (int p = 0; p < RPT; ++p)
        f.g[p] = !a.g ? 0.f : a.g_per_key ? a.g[(t * a.Hv + h) * (long)DK + row0 + p] : a.g[t * a.Hv + h];
}

template <typename T, int DK, int DV, int CW>
__global__ __launch_bounds__((RecShape<DK, CW>::NT)) void recurrent_bwd_kernel(RecurrentBwdArgs a) {
    using S = RecShape<DK, CW>;
    constexpr int TPR = S::TPR, RPT = S::RPT, NW = S::NW, NSL = DV / CW;
    __shared__ float red[NW][CW];
    __shared__ float vec_vr[CW], vec_d[CW], vec_do[CW], vec_dd[CW];
    __shared__ float dbp[CW];      // this slice's dbeta terms, one per value column
    __shared__ float dgw[NW];      // per-wave dg partials (one gate per head)
    __shared__ float nrm[NW][2];   // per-wave |k|^2, |q|^2 partials (in-call normalisation)

    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int ct = tid % TPR, rg = tid / TPR;
    const int slice = blockIdx.x % NSL;
    const int nh = blockIdx.x / NSL;
    const int h = nh % a.Hv, n = nh / a.Hv;
    const int hq = h / (a.Hv / a.Hqk);
    const int row0 = rg * RPT, j0 = slice * CW;
    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);
    const long tokens = (long)a.B * a.T;

    float G[RPT][4];
#pragma unroll
    for (int p = 0; p < RPT; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            G[p][e] = a.dfinal ? a.dfinal[((long)nh * DK + row0 + p) * DV + j0 + ct * 4 + e] : 0.f;
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
    auto rowsum = [&](float& x) {
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) x += __shfl_xor(x, off);
    };

    BwdIn<T, DK, CW> cur, nxt;
    if (eos > bos) bwd_fetch<T, DK, DV, CW>(a, eos - 1, bos, nh, h, hq, row0, ct, tid, j0, cur);
    for (long t = eos - 1; t >= bos; --t) {
        if (t - 1 >= bos) bwd_fetch<T, DK, DV, CW>(a, t - 1, bos, nh, h, hq, row0, ct, tid, j0, nxt);
        float al[RPT];
#pragma unroll
        for (int p = 0; p < RPT; ++p) al[p] = a.g ? expf(cur.g[p]) : 1.f;
        const float beta = cur.beta;
        float Mp[RPT][4];
#pragma unroll
        for (int p = 0; p < RPT; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) Mp[p][e] = al[p] * cur.m[p][e];
        // r = M'^T k (k as loaded; with the in-call normalisation r is scaled once the
        // norms are reduced)
        float c[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < RPT; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) c[e] += Mp[p][e] * cur.k[p];
        colsum(c);
        if (a.qk_norm) {
            float kk = 0.f, qq = 0.f;
            if (ct == 0) {
#pragma unroll
                for (int p = 0; p < RPT; ++p) {
                    kk += cur.k[p] * cur.k[p];
                    qq += cur.q[p] * cur.q[p];
                }
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                kk += __shfl_xor(kk, off);
                qq += __shfl_xor(qq, off);
            }
            if (lane == 0) {
                nrm[wave][0] = kk;
                nrm[wave][1] = qq;
            }
        }
        __syncthreads();
        float ik = 1.f, iq = 1.f;
        if (a.qk_norm) {
            float kk = 0.f, qq = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                kk += nrm[w][0];
                qq += nrm[w][1];
            }
            ik = inv_norm(kk, a.eps);
            iq = inv_norm(qq, a.eps);
        }
        if (tid < CW) {
            float r = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) r += red[w][tid];
            const float vr = cur.v - ik * r;   // v - r
            vec_vr[tid] = vr;
            vec_d[tid] = beta * vr;
            vec_do[tid] = a.scale * cur.dout;
        }
        __syncthreads();
        if (a.qk_norm) {   // from here on the rule's own (normalised) k and q
#pragma unroll
            for (int p = 0; p < RPT; ++p) {
                cur.k[p] *= ik;
                cur.q[p] *= iq;
            }
        }
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
                G[p][e] += cur.q[p] * dov[e];
                dqp[p] += (Mp[p][e] + cur.k[p] * dl[e]) * dov[e];
                c[e] += G[p][e] * cur.k[p];
            }
        }
#pragma unroll
        for (int p = 0; p < RPT; ++p) rowsum(dqp[p]);
        colsum(c);
        __syncthreads();
        if (tid < CW) {
            float dd = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) dd += red[w][tid];
            a.dv[(t * a.Hv + h) * DV + j0 + tid] = beta * dd;
            dbp[tid] = dd * vec_vr[tid];   // summed below in column order
            vec_dd[tid] = dd;
        }
        __syncthreads();
        float ddv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ddv[e] = vec_dd[ct * 4 + e];
        // dk = G delta - beta M' dd;  G' = G - beta k dd^T;  dg = <G', M'> (per row of M' with
        // a decay per key channel);  G <- diag(a) G'
        float dkp[RPT], dgr[RPT];
#pragma unroll
        for (int p = 0; p < RPT; ++p) {
            dkp[p] = 0.f;
            dgr[p] = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dkp[p] += G[p][e] * dl[e] - beta * Mp[p][e] * ddv[e];
                G[p][e] -= beta * cur.k[p] * ddv[e];
                dgr[p] += G[p][e] * Mp[p][e];
                G[p][e] *= al[p];
            }
        }
#pragma unroll
        for (int p = 0; p < RPT; ++p) rowsum(dkp[p]);
        if (ct == 0) {   // this slice's share of dq, dk for the rows of this thread
            float* dq = a.ws_dq + ((slice * tokens + t) * a.Hv + h) * (long)DK + row0;
            float* dk = a.ws_dk + ((slice * tokens + t) * a.Hv + h) * (long)DK + row0;
#pragma unroll
            for (int p = 0; p < RPT; ++p) {
                dq[p] = dqp[p];
                dk[p] = dkp[p];
            }
        }
        if (a.g_per_key) {   // this slice's share of dg for the thread's rows
#pragma unroll
            for (int p = 0; p < RPT; ++p) rowsum(dgr[p]);
            if (ct == 0) {
                float* dg = a.ws_dg + ((slice * tokens + t) * a.Hv + h) * (long)DK + row0;
#pragma unroll
                for (int p = 0; p < RPT; ++p) dg[p] = dgr[p];
            }
        } else {
            float dgp = 0.f;
#pragma unroll
            for (int p = 0; p < RPT; ++p) dgp += dgr[p];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) dgp += __shfl_xor(dgp, off);
            if (lane == 0) dgw[wave] = dgp;   // summed below in wave order
        }
        __syncthreads();
        if (tid == 0) {   // fixed summation orders: the pass is bitwise reproducible
            float db = 0.f;
#pragma unroll
            for (int c2 = 0; c2 < CW; ++c2) db += dbp[c2];
            a.ws_db[(slice * tokens + t) * a.Hv + h] = db;
            if (!a.g_per_key) {
                float dg = 0.f;
#pragma unroll
                for (int w = 0; w < NW; ++w) dg += dgw[w];
                a.ws_dg[(slice * tokens + t) * a.Hv + h] = dg;
            }
        }
        __syncthreads();   // dbp, dgw and the reduction buffers are reused by the next token
        cur = nxt;
    }
    if (a.dh0) {
#pragma unroll
        for (int p = 0; p < RPT; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) a.dh0[((long)nh * DK + row0 + p) * DV + j0 + ct * 4 + e] = G[p][e];
    }
}

// The slices' shares, in a fixed order: dq, dk per query/key head (over the slices and the
// value heads that read the head), dbeta and dg per value head (over the slices); with a
// decay per key channel, dg per value head and key channel (over the slices).
__global__ __launch_bounds__(256) void bwd_sum_kernel(RecurrentBwdArgs a, int nsl) {
    const long tokens = (long)a.B * a.T;
    const int grp = a.Hv / a.Hqk;
    const long nqk = tokens * a.Hqk * a.Dk;
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < nqk) {
        const int d = (int)(i % a.Dk);
        const long th = i / a.Dk;          // t * Hqk + hq
        float sq = 0.f, sk = 0.f;
        for (int sl = 0; sl < nsl; ++sl)
            for (int r = 0; r < grp; ++r) {
                const long o = ((sl * tokens * a.Hqk + th) * grp + r) * (long)a.Dk + d;
                sq += a.ws_dq[o];
                sk += a.ws_dk[o];
            }
        a.dq[i] = sq;
        a.dk[i] = sk;
    } else if (i < nqk + tokens * a.Hv) {
        const long th = i - nqk;           // t * Hv + h
        float sb = 0.f, sg = 0.f;
        for (int sl = 0; sl < nsl; ++sl) {
            sb += a.ws_db[sl * tokens * a.Hv + th];
            sg += a.ws_dg[sl * tokens * a.Hv + th];
        }
        a.dbeta[th] = sb;
        if (a.dg && !a.g_per_key) a.dg[th] = sg;
    } else if (a.g_per_key && a.dg && i < nqk + tokens * a.Hv + tokens * a.Hv * a.Dk) {
        const long th = i - nqk - tokens * a.Hv;   // (t * Hv + h) * Dk + x
        float sg = 0.f;
        for (int sl = 0; sl < nsl; ++sl) sg += a.ws_dg[sl * tokens * a.Hv * a.Dk + th];
        a.dg[th] = sg;
    }
}

// The in-call normalisation as passes of their own: NRW rows (token, query/key head) per
// wave, two consecutive key channels per lane, every row's loads issued before the first
// row's sums (DPP wave sums).
constexpr int NRW = 8;

// dq, dk through the normalisation, in place: with x_hat = x / n, n = sqrt(|x|^2 + eps),
// dx = (dx_hat - x (x . dx_hat) / n^2) / n (zero where n = 0).
template <typename T>
__global__ __launch_bounds__(256) void norm_bwd_kernel(RecurrentBwdArgs a) {
    const long rows = (long)a.B * a.T * a.Hqk;
    const long r0 = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * NRW;
    const int lane = threadIdx.x & 63;
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const bool in = 2 * lane < a.Dk;   // Dk is even
    // dq and dk need only 4-byte alignment: 8-byte accesses where both allow them
    const bool v2 = (((uintptr_t)a.dq | (uintptr_t)a.dk) & 7) == 0;
    float xq[NRW][2], xk[NRW][2], gq[NRW][2], gk[NRW][2];
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
        const bool ok = in && r0 + r < rows;
        const long i0 = (r0 + r) * a.Dk + 2 * lane;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            xq[r][c] = ok ? ld_f32(q, i0 + c) : 0.f;
            xk[r][c] = ok ? ld_f32(k, i0 + c) : 0.f;
        }
        if (ok && v2) {
            const float2 a2 = *reinterpret_cast<const float2*>(a.dq + i0), b2 = *reinterpret_cast<const float2*>(a.dk + i0);
            gq[r][0] = a2.x; gq[r][1] = a2.y; gk[r][0] = b2.x; gk[r][1] = b2.y;
        } else {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                gq[r][c] = ok ? a.dq[i0 + c] : 0.f;
                gk[r][c] = ok ? a.dk[i0 + c] : 0.f;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
        const float nq = ck::wave_sum(xq[r][0] * xq[r][0] + xq[r][1] * xq[r][1]) + a.eps;
        const float nk = ck::wave_sum(xk[r][0] * xk[r][0] + xk[r][1] * xk[r][1]) + a.eps;
        const float sq = ck::wave_sum(xq[r][0] * gq[r][0] + xq[r][1] * gq[r][1]);
        const float sk = ck::wave_sum(xk[r][0] * gk[r][0] + xk[r][1] * gk[r][1]);
        const float rq = nq > 0.f ? rsqrtf(nq) : 0.f, rk = nk > 0.f ? rsqrtf(nk) : 0.f;
        const float cq = nq > 0.f ? sq / nq : 0.f, ck_ = nk > 0.f ? sk / nk : 0.f;
        if (!(in && r0 + r < rows)) continue;
        const long i0 = (r0 + r) * a.Dk + 2 * lane;
        const float q0 = (gq[r][0] - xq[r][0] * cq) * rq, q1 = (gq[r][1] - xq[r][1] * cq) * rq;
        const float k0 = (gk[r][0] - xk[r][0] * ck_) * rk, k1 = (gk[r][1] - xk[r][1] * ck_) * rk;
        if (v2) {
            *reinterpret_cast<float2*>(a.dq + i0) = make_float2(q0, q1);
            *reinterpret_cast<float2*>(a.dk + i0) = make_float2(k0, k1);
        } else {
            a.dq[i0] = q0; a.dq[i0 + 1] = q1;
            a.dk[i0] = k0; a.dk[i0 + 1] = k1;
        }
    }
}

// q, k -> x / sqrt(|x|^2 + eps) as bf16 (zero where the sum is 0)
__global__ __launch_bounds__(256) void norm_rows_kernel(PrefillArgs a, __bf16* qn, __bf16* kn, float* rnorm) {
    const long rows = (long)a.B * a.T * a.Hqk;
    const long r0 = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * NRW;
    const int lane = threadIdx.x & 63;
    const __bf16* q = static_cast<const __bf16*>(a.q);
    const __bf16* k = static_cast<const __bf16*>(a.k);
    const bool in = 2 * lane < a.Dk;   // Dk is even
    uint32_t uq[NRW], uk[NRW];
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
        const bool ok = in && r0 + r < rows;
        const long i0 = (r0 + r) * a.Dk + 2 * lane;
        uq[r] = ok ? *reinterpret_cast<const uint32_t*>(q + i0) : 0u;
        uk[r] = ok ? *reinterpret_cast<const uint32_t*>(k + i0) : 0u;
    }
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
        const float q0 = __uint_as_float(uq[r] << 16), q1 = __uint_as_float(uq[r] & 0xffff0000u);
        const float k0 = __uint_as_float(uk[r] << 16), k1 = __uint_as_float(uk[r] & 0xffff0000u);
        const float rq = inv_norm(ck::wave_sum(q0 * q0 + q1 * q1), a.eps);
        const float rk = inv_norm(ck::wave_sum(k0 * k0 + k1 * k1), a.eps);
        if (rnorm && lane == 0 && r0 + r < rows) {
            rnorm[r0 + r] = rq;
            rnorm[rows + r0 + r] = rk;
        }
        if (!(in && r0 + r < rows)) continue;
        const long i0 = (r0 + r) * a.Dk + 2 * lane;
        *reinterpret_cast<uint32_t*>(qn + i0) = pack_bf16x2(q0 * rq, q1 * rq);
        *reinterpret_cast<uint32_t*>(kn + i0) = pack_bf16x2(k0 * rk, k1 * rk);
    }
}

template <typename T, int DK>
hipError_t launch_dv(const RecurrentArgs& a, hipStream_t s) {
    const long nh = (long)a.N * a.Hv;
    switch (a.Dv) {
        case 16: hipLaunchKernelGGL((recurrent_kernel<T, DK, 16, 16>), dim3((unsigned)nh), dim3(RecShape<DK, 16>::NT), 0, s, a); break;
        case 32: hipLaunchKernelGGL((recurrent_kernel<T, DK, 32, 32>), dim3((unsigned)nh), dim3(RecShape<DK, 32>::NT), 0, s, a); break;
        case 64: hipLaunchKernelGGL((recurrent_kernel<T, DK, 64, 32>), dim3((unsigned)(2 * nh)), dim3(RecShape<DK, 32>::NT), 0, s, a); break;
        case 128: hipLaunchKernelGGL((recurrent_kernel<T, DK, 128, 32>), dim3((unsigned)(4 * nh)), dim3(RecShape<DK, 32>::NT), 0, s, a); break;
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
    // value columns per workgroup: 8 (more workgroups per head, the per-token latency is
    // spread over more CUs) where a workgroup still holds a whole number of waves
    constexpr int CW = bwd_cols(DK);
    const long nh = (long)a.N * a.Hv;
    switch (a.Dv) {
        case 16: hipLaunchKernelGGL((recurrent_bwd_kernel<T, DK, 16, CW>), dim3((unsigned)(16 / CW * nh)), dim3(RecShape<DK, CW>::NT), 0, s, a); break;
        case 32: hipLaunchKernelGGL((recurrent_bwd_kernel<T, DK, 32, CW>), dim3((unsigned)(32 / CW * nh)), dim3(RecShape<DK, CW>::NT), 0, s, a); break;
        case 64: hipLaunchKernelGGL((recurrent_bwd_kernel<T, DK, 64, CW>), dim3((unsigned)(64 / CW * nh)), dim3(RecShape<DK, CW>::NT), 0, s, a); break;
        case 128: hipLaunchKernelGGL((recurrent_bwd_kernel<T, DK, 128, CW>), dim3((unsigned)(128 / CW * nh)), dim3(RecShape<DK, CW>::NT), 0, s, a); break;
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

int recurrent_bwd_slices(int Dk, int Dv) { return Dv / bwd_cols(Dk); }

hipError_t launch_qk_norm_rows(const PrefillArgs& a, void* qn, void* kn, float* rnorm, hipStream_t s) {
    const long rows = (long)a.B * a.T * a.Hqk;
    if (rows == 0) return hipSuccess;
    if (!a.bf16 || a.Dk > 128) return hipErrorInvalidValue;
    const long blocks = (rows + 4 * NRW - 1) / (4 * NRW);
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(norm_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, static_cast<__bf16*>(qn),
                       static_cast<__bf16*>(kn), rnorm);
    return hipGetLastError();
}

hipError_t launch_recurrent_bwd(const RecurrentBwdArgs& a, hipStream_t s) {
    if ((long)a.N * a.Hv == 0) return hipSuccess;
    if ((long)a.N * a.Hv * recurrent_bwd_slices(a.Dk, a.Dv) > 0x7fffffffL) return hipErrorInvalidConfiguration;
    const hipError_t e = a.bf16 ? launch_bwd_dk<__bf16>(a, s) : launch_bwd_dk<float>(a, s);
    if (e != hipSuccess) return e;
    const long tokens = (long)a.B * a.T;
    const long total = tokens * a.Hqk * a.Dk + tokens * a.Hv + (a.g_per_key && a.dg ? tokens * a.Hv * a.Dk : 0);
    if (total > 0) {
        const long blocks = (total + 255) / 256;
        if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(bwd_sum_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a, recurrent_bwd_slices(a.Dk, a.Dv));
    }
    const long rows = tokens * a.Hqk;
    if (a.qk_norm && rows > 0) {
        const long blocks = (rows + 4 * NRW - 1) / (4 * NRW);
        if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
        if (a.bf16) hipLaunchKernelGGL(norm_bwd_kernel<__bf16>, dim3((unsigned)blocks), dim3(256), 0, s, a);
        else hipLaunchKernelGGL(norm_bwd_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t s) {
    if ((long)a.N * a.Hv == 0) return hipSuccess;
    if ((long)a.N * a.Hv * recurrent_bwd_slices(a.Dk, a.Dv) > 0x7fffffffL) return hipErrorInvalidConfiguration;
    return a.bf16 ? launch_dk<__bf16>(a, s) : launch_dk<float>(a, s);
}

}  // namespace dn
