// prefill_generic.hip -- chunked form of the gated delta rule in fp32 on the vector
// ALUs, for every supported size (Dk, Dv <= 128, chunk <= 64) and for fp32 inputs.
// The bf16 Dk = Dv = 128 prompts take the matrix-core path (prefill_fused.hip).
//
// The chunked form follows from the update of the frankenstein "DeltaNet
// Attention" page (module docstring) with the gate order of the nnterp
// "linear_attention" page (decay, then take up the pair, then read).  Inside one
// chunk of n tokens with start state M0 = S0^T and gamma_r = sum_{i<=r} g_i:
//
//   A_ri  = beta_r exp(gamma_r - gamma_i) k_r.k_i         (i < r; strictly lower)
//   P_ri  = exp(gamma_r - gamma_i) q_r.k_i                (i <= r)
//   R     = diag(beta) (V - diag(exp(gamma)) K M0)
//   (I + A) Delta = R                                     (forward substitution)
//   O     = scale (diag(exp(gamma)) Q M0 + P Delta)
//   M1    = exp(gamma_{n-1}) M0 + sum_r exp(gamma_{n-1} - gamma_r) k_r Delta_r^T
//
// Row r of Delta is beta_r times the prediction error of token r against the
// decayed state it sees, so this reproduces the token-by-token rule exactly in exact
// arithmetic.  The decay factors are formed as exp(gamma_r - gamma_i) for i <= r only
// (never as a ratio of two exponentials), so strong decay cannot produce 0/0.
//
// With the in-rule normalisation the chunk's K and Q rows are normalised in LDS first.
// Gates per key channel take a kernel of their own (below).
//
// One workgroup per (sequence, value head, slice of GS value columns); the value
// columns of the state are independent, so slices need no exchange.  K, Q, the V
// slice, the state slice, A and P live in LDS for the whole chunk.
#include "internal.h"

namespace dn {
namespace {

constexpr int GK = 128;      // largest key dim
constexpr int GS = 32;       // value columns per workgroup
constexpr int GC = 64;       // largest chunk
constexpr int NT = 256;      // threads per workgroup
constexpr int KP = GK + 1;   // padded pitches
constexpr int SP = GS + 1;
constexpr int CP = GC + 1;
constexpr int YPT = GC * GS / NT;   // (row, column) output pairs per thread

struct GenericSmem {
    float K[GC][KP];
    float Q[GC][KP];
    float V[GC][SP];
    float M[GK][SP];
    float A[GC][CP];
    float P[GC][CP];
    float D[GC][SP];
    float gam[GC];
    float beta[GC];
};

template <typename T>
__global__ __launch_bounds__(NT) void prefill_generic_kernel(PrefillArgs a) {
    __shared__ GenericSmem sm;
    const int tid = threadIdx.x;
    const int Dk = a.Dk, Dv = a.Dv, C = a.C;
    const int slices = (Dv + GS - 1) / GS;
    const int slice = blockIdx.x % slices;
    const int nh = blockIdx.x / slices;
    const int h = nh % a.Hv;
    const int n = nh / a.Hv;
    const int hq = h / (a.Hv / a.Hqk);
    const int j0 = slice * GS;
    const int sw = min(GS, Dv - j0);
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    T* o = static_cast<T*>(a.o);

    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);

    for (int e = tid; e < GK * GS; e += NT) {
        const int i = e / GS, j = e % GS;
        sm.M[i][j] = (a.h0 && i < Dk && j < sw) ? a.h0[((long)nh * Dk + i) * Dv + j0 + j] : 0.f;
    }

    for (long c0 = bos; c0 < eos; c0 += C) {
        const int len = (int)min((long)C, eos - c0);
        __syncthreads();  // the previous chunk is done with every buffer
        for (int e = tid; e < C * Dk; e += NT) {
            const int r = e / Dk, i = e % Dk;
            float kv = 0.f, qv = 0.f;
            if (r < len) {
                const long off = ((c0 + r) * a.Hqk + hq) * Dk + i;
                kv = ld_f32(k, off);
                qv = ld_f32(q, off);
            }
            sm.K[r][i] = kv;
            sm.Q[r][i] = qv;
        }
        for (int e = tid; e < C * GS; e += NT) {
            const int r = e / GS, j = e % GS;
            sm.V[r][j] = (r < len && j < sw) ? ld_f32(v, ((c0 + r) * a.Hv + h) * Dv + j0 + j) : 0.f;
        }
        if (tid < C) {
            const bool in = tid < len;
            sm.beta[tid] = in ? a.beta[(c0 + tid) * a.Hv + h] : 0.f;
            sm.gam[tid] = (in && a.g) ? a.g[(c0 + tid) * a.Hv + h] : 0.f;
        }
        __syncthreads();
        if (tid == 0) {  // inclusive prefix sum of the log decays over the chunk
            float s = 0.f;
            for (int r = 0; r < C; ++r) {
                s += sm.gam[r];
                sm.gam[r] = s;
            }
        }
        if (a.qk_norm) {  // q, k -> x / sqrt(|x|^2 + eps) in place, four threads per row
            const int r = tid >> 2, part = tid & 3;
            float sk = 0.f, sq = 0.f;
            if (r < C) {
                for (int x = part; x < Dk; x += 4) {
                    sk += sm.K[r][x] * sm.K[r][x];
                    sq += sm.Q[r][x] * sm.Q[r][x];
                }
            }
            sk += __shfl_xor(sk, 1);
            sk += __shfl_xor(sk, 2);
            sq += __shfl_xor(sq, 1);
            sq += __shfl_xor(sq, 2);
            const float ik = inv_norm(sk, a.eps), iq = inv_norm(sq, a.eps);
            if (r < C) {
                for (int x = part; x < Dk; x += 4) {
                    sm.K[r][x] *= ik;
                    sm.Q[r][x] *= iq;
                }
            }
        }
        __syncthreads();

        // masked, decay-weighted Gram matrices
        for (int e = tid; e < C * C; e += NT) {
            const int r = e / C, i = e % C;
            float av = 0.f, pv = 0.f;
            if (r < len && i <= r) {
                const float d = expf(sm.gam[r] - sm.gam[i]);
                float kk = 0.f, qk = 0.f;
                for (int x = 0; x < Dk; ++x) {
                    kk += sm.K[r][x] * sm.K[i][x];
                    qk += sm.Q[r][x] * sm.K[i][x];
                }
                if (i < r) av = sm.beta[r] * d * kk;
                pv = d * qk;
            }
            sm.A[r][i] = av;
            sm.P[r][i] = pv;
        }
        // right-hand side R (into D) and the inter-chunk part of the read (registers)
        float Y[YPT];
#pragma unroll
        for (int t = 0; t < YPT; ++t) {
            const int e = tid + t * NT;
            const int r = e / GS, j = e % GS;
            float xk = 0.f, xq = 0.f;
            for (int x = 0; x < Dk; ++x) {
                xk += sm.K[r][x] * sm.M[x][j];
                xq += sm.Q[r][x] * sm.M[x][j];
            }
            const float G = expf(sm.gam[r]);
            sm.D[r][j] = (r < len) ? sm.beta[r] * (sm.V[r][j] - G * xk) : 0.f;
            Y[t] = G * xq;
        }
        __syncthreads();
        // (I + A) Delta = R by forward substitution, one thread per value column
        if (tid < GS) {
            const int j = tid;
            for (int r = 1; r < len; ++r) {
                float s = sm.D[r][j];
                for (int i = 0; i < r; ++i) s -= sm.A[r][i] * sm.D[i][j];
                sm.D[r][j] = s;
            }
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < YPT; ++t) {
            const int e = tid + t * NT;
            const int r = e / GS, j = e % GS;
            if (r < len && j < sw) {
                float s = Y[t];
                for (int i = 0; i <= r; ++i) s += sm.P[r][i] * sm.D[i][j];
                st_out(o, ((c0 + r) * a.Hv + h) * Dv + j0 + j, a.scale * s);
            }
        }
        __syncthreads();
        const float gl = sm.gam[len - 1];
        for (int e = tid; e < C * GS; e += NT) {
            const int r = e / GS, j = e % GS;
            sm.D[r][j] *= (r < len) ? expf(gl - sm.gam[r]) : 0.f;
        }
        __syncthreads();
        const float Gl = expf(gl);
        for (int e = tid; e < Dk * GS; e += NT) {
            const int x = e / GS, j = e % GS;
            float s = Gl * sm.M[x][j];
            for (int r = 0; r < len; ++r) s += sm.K[r][x] * sm.D[r][j];
            sm.M[x][j] = s;
        }
    }
    __syncthreads();
    if (a.hT) {
        for (int e = tid; e < Dk * GS; e += NT) {
            const int i = e / GS, j = e % GS;
            if (j < sw) a.hT[((long)nh * Dk + i) * Dv + j0 + j] = sm.M[i][j];
        }
    }
}

// ------------------------------------------------------------- gates per key channel
// The nnterp page's ChannelGates (one log decay per key channel, the KDA variant): the
// state's key channel x keeps exp(g_t[x]), S'_t = S_{t-1} diag(exp(g_t)).  With
// G[r][x] = sum_{i<=r} g_i[x] inside the chunk, the chunked form becomes
//
//   A_ri  = beta_r sum_x k_r[x] k_i[x] exp(G[r][x] - G[i][x])        (i < r)
//   P_ri  = sum_x q_r[x] k_i[x] exp(G[r][x] - G[i][x])               (i <= r)
//   R     = diag(beta) (V - (K o exp(G)) M0),   (I + A) Delta = R
//   O     = scale ((Q o exp(G)) M0 + P Delta)
//   M1[x] = exp(G[n-1][x]) M0[x] + sum_r k_r[x] exp(G[n-1][x] - G[r][x]) Delta_r
//
// The pairwise factor exp(G[r][x] - G[i][x]), i <= r, is exp(G[r][x]) exp(-G[i][x]) from two
// per-token tables when the chunk's decay stays above exp(-60) on every channel (then
// exp(-G) <= exp(60) and every product <= 1); a chunk that decays harder forms each factor
// as one exponential of a difference, never as a ratio.
// The per-channel sums take a [chunk][Dk] tile of their own, so this path runs 32-token
// chunks (the chunk size does not change the result in exact arithmetic).
constexpr int HC = 32;                  // chunk of the channel-gate path
constexpr int HCP = HC + 1;
constexpr int HYPT = HC * GS / NT;      // (row, column) output pairs per thread

struct ChannelSmem {
    float K[HC][KP];     // keys; before the state update, k_r[x] exp(G[n-1][x] - G[r][x])
    float Q[HC][KP];
    float G[HC][KP];     // per-channel inclusive sums of g over the chunk
    float E[HC][KP];     // exp(G)
    float En[HC][KP];    // exp(-G), when the chunk's decay allows the factored form
    int hard;            // some channel decays below exp(-60) over the chunk
    float V[HC][SP];
    float M[GK][SP];
    float A[HC][HCP];
    float P[HC][HCP];
    float D[HC][SP];
    float beta[HC];
};

template <typename T>
__global__ __launch_bounds__(NT) void prefill_channel_gate_kernel(PrefillArgs a) {
    __shared__ ChannelSmem sm;
    const int tid = threadIdx.x;
    const int Dk = a.Dk, Dv = a.Dv, C = min(a.C, HC);
    const int slices = (Dv + GS - 1) / GS;
    const int slice = blockIdx.x % slices;
    const int nh = blockIdx.x / slices;
    const int h = nh % a.Hv;
    const int n = nh / a.Hv;
    const int hq = h / (a.Hv / a.Hqk);
    const int j0 = slice * GS;
    const int sw = min(GS, Dv - j0);
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    T* o = static_cast<T*>(a.o);

    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);

    for (int e = tid; e < GK * GS; e += NT) {
        const int i = e / GS, j = e % GS;
        sm.M[i][j] = (a.h0 && i < Dk && j < sw) ? a.h0[((long)nh * Dk + i) * Dv + j0 + j] : 0.f;
    }

    for (long c0 = bos; c0 < eos; c0 += C) {
        const int len = (int)min((long)C, eos - c0);
        __syncthreads();  // the previous chunk is done with every buffer
        for (int e = tid; e < C * Dk; e += NT) {
            const int r = e / Dk, x = e % Dk;
            float kv = 0.f, qv = 0.f, gv = 0.f;
            if (r < len) {
                const long off = ((c0 + r) * a.Hqk + hq) * Dk + x;
                kv = ld_f32(k, off);
                qv = ld_f32(q, off);
                gv = a.g[((c0 + r) * a.Hv + h) * Dk + x];
            }
            sm.K[r][x] = kv;
            sm.Q[r][x] = qv;
            sm.G[r][x] = gv;
        }
        for (int e = tid; e < C * GS; e += NT) {
            const int r = e / GS, j = e % GS;
            sm.V[r][j] = (r < len && j < sw) ? ld_f32(v, ((c0 + r) * a.Hv + h) * Dv + j0 + j) : 0.f;
        }
        if (tid < C) sm.beta[tid] = tid < len ? a.beta[(c0 + tid) * a.Hv + h] : 0.f;
        if (tid == 0) sm.hard = 0;
        __syncthreads();
        if (tid < Dk) {  // inclusive sums of the log decays, one key channel per thread
            float s = 0.f;
            for (int r = 0; r < C; ++r) {
                s += sm.G[r][tid];
                sm.G[r][tid] = s;
            }
        }
        if (a.qk_norm) {  // q, k -> x / sqrt(|x|^2 + eps) in place, four threads per row
            const int r = tid >> 2, part = tid & 3;
            float sk = 0.f, sq = 0.f;
            if (r < C) {
                for (int x = part; x < Dk; x += 4) {
                    sk += sm.K[r][x] * sm.K[r][x];
                    sq += sm.Q[r][x] * sm.Q[r][x];
                }
            }
            sk += __shfl_xor(sk, 1);
            sk += __shfl_xor(sk, 2);
            sq += __shfl_xor(sq, 1);
            sq += __shfl_xor(sq, 2);
            const float ik = inv_norm(sk, a.eps), iq = inv_norm(sq, a.eps);
            if (r < C) {
                for (int x = part; x < Dk; x += 4) {
                    sm.K[r][x] *= ik;
                    sm.Q[r][x] *= iq;
                }
            }
        }
        __syncthreads();
        for (int e = tid; e < C * Dk; e += NT) {
            const int r = e / Dk, x = e % Dk;
            sm.E[r][x] = expf(sm.G[r][x]);
            sm.En[r][x] = expf(-sm.G[r][x]);
        }
        if (tid < Dk && sm.G[len - 1][tid] < -60.f) sm.hard = 1;
        __syncthreads();
        const bool hard = sm.hard != 0;

        // Gram matrices with the per-channel decay inside the sum
        for (int e = tid; e < C * C; e += NT) {
            const int r = e / C, i = e % C;
            float av = 0.f, pv = 0.f;
            if (r < len && i <= r) {
                float kk = 0.f, qk = 0.f;
                if (hard) {
                    for (int x = 0; x < Dk; ++x) {
                        const float d = expf(sm.G[r][x] - sm.G[i][x]);
                        kk += sm.K[r][x] * sm.K[i][x] * d;
                        qk += sm.Q[r][x] * sm.K[i][x] * d;
                    }
                } else {
                    for (int x = 0; x < Dk; ++x) {
                        const float ki = sm.K[i][x] * sm.En[i][x] * sm.E[r][x];
                        kk += sm.K[r][x] * ki;
                        qk += sm.Q[r][x] * ki;
                    }
                }
                if (i < r) av = sm.beta[r] * kk;
                pv = qk;
            }
            sm.A[r][i] = av;
            sm.P[r][i] = pv;
        }
        // right-hand side R (into D) and the inter-chunk part of the read (registers)
        float Y[HYPT];
#pragma unroll
        for (int t = 0; t < HYPT; ++t) {
            const int e = tid + t * NT;
            const int r = e / GS, j = e % GS;
            float xk = 0.f, xq = 0.f;
            if (r < C) {
                for (int x = 0; x < Dk; ++x) {
                    const float m = sm.E[r][x] * sm.M[x][j];
                    xk += sm.K[r][x] * m;
                    xq += sm.Q[r][x] * m;
                }
                sm.D[r][j] = (r < len) ? sm.beta[r] * (sm.V[r][j] - xk) : 0.f;
            }
            Y[t] = xq;
        }
        __syncthreads();
        // (I + A) Delta = R by forward substitution, one thread per value column
        if (tid < GS) {
            const int j = tid;
            for (int r = 1; r < len; ++r) {
                float s = sm.D[r][j];
                for (int i = 0; i < r; ++i) s -= sm.A[r][i] * sm.D[i][j];
                sm.D[r][j] = s;
            }
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < HYPT; ++t) {
            const int e = tid + t * NT;
            const int r = e / GS, j = e % GS;
            if (r < len && j < sw) {
                float s = Y[t];
                for (int i = 0; i <= r; ++i) s += sm.P[r][i] * sm.D[i][j];
                st_out(o, ((c0 + r) * a.Hv + h) * Dv + j0 + j, a.scale * s);
            }
        }
        // keys decayed to the chunk end, for the state update
        for (int e = tid; e < C * Dk; e += NT) {
            const int r = e / Dk, x = e % Dk;
            sm.K[r][x] *= (r < len) ? expf(sm.G[len - 1][x] - sm.G[r][x]) : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < Dk * GS; e += NT) {
            const int x = e / GS, j = e % GS;
            float s = sm.E[len - 1][x] * sm.M[x][j];
            for (int r = 0; r < len; ++r) s += sm.K[r][x] * sm.D[r][j];
            sm.M[x][j] = s;
        }
    }
    __syncthreads();
    if (a.hT) {
        for (int e = tid; e < Dk * GS; e += NT) {
            const int i = e / GS, j = e % GS;
            if (j < sw) a.hT[((long)nh * Dk + i) * Dv + j0 + j] = sm.M[i][j];
        }
    }
}

}  // namespace

hipError_t launch_prefill_generic(const PrefillArgs& a, hipStream_t s) {
    if (a.Dk > GK || a.C > GC || a.C < 1) return hipErrorInvalidValue;
    const long blocks = (long)a.N * a.Hv * ((a.Dv + GS - 1) / GS);
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (a.g_per_key) {
        if (!a.g) return hipErrorInvalidValue;
        if (prefill_chg_supported(a)) return launch_prefill_chg(a, s);
        if (a.bf16)
            hipLaunchKernelGGL(prefill_channel_gate_kernel<__bf16>, dim3((unsigned)blocks), dim3(NT), 0, s, a);
        else
            hipLaunchKernelGGL(prefill_channel_gate_kernel<float>, dim3((unsigned)blocks), dim3(NT), 0, s, a);
    } else if (a.bf16) {
        hipLaunchKernelGGL(prefill_generic_kernel<__bf16>, dim3((unsigned)blocks), dim3(NT), 0, s, a);
    } else {
        hipLaunchKernelGGL(prefill_generic_kernel<float>, dim3((unsigned)blocks), dim3(NT), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace dn
