// prefill_fast.hip -- chunked prefill of the gated delta rule on the gfx950 matrix
// cores (bf16 MFMA, fp32 accumulation), for bf16 inputs with Dk = Dv = 128 and
// 64-token chunks.
//
// The algebra is the chunked form of the update on the frankenstein "DeltaNet
// Attention" page (module docstring), with the gate order of the nnterp
// "linear_attention" page.  Inside a chunk of n <= 64 tokens, with the state slice
// M (key-major, S^T) at the chunk start and gamma_r = sum_{i<=r} g_i:
//
//   A_ri = beta_r exp(gamma_r - gamma_i) k_r.k_i (i < r),  T = (I + A)^{-1}
//   R    = diag(beta) (V - diag(exp(gamma)) K M)
//   Delta = T R                                   (row r: beta_r x prediction error)
//   O    = scale (diag(exp(gamma)) Q M + P Delta),  P_ri = exp(gamma_r - gamma_i) q_r.k_i (i <= r)
//   M   <- exp(gamma_last) M + K^T diag(exp(gamma_last - gamma)) Delta
//
// Three kernels on the caller's stream:
//   chunk_offsets_kernel  (packed batches only) chunk index of each sequence's first
//                         chunk, into the workspace.
//   prep_kernel           one workgroup per (chunk, query/key head), all chunks in
//                         parallel: K K^T on the matrix cores, the decay/beta mask, and
//                         T = (I + A)^{-1} by 16x16 diagonal-block substitution plus
//                         block back-substitution in fp32; T goes to the workspace in
//                         bf16.  The Gram matrix is shared by the value heads that read
//                         the same key head.
//   state_kernel          one workgroup per (sequence, value head, 32-column slice of
//                         the state).  The value columns of the state are independent,
//                         so slices never exchange data; each carries its 128 x 32 fp32
//                         state slice in MFMA accumulators across the sequential chunk
//                         loop, with a bf16 copy in LDS as the next chunk's operand.
//                         The next chunk's K, Q, V and T are fetched into registers
//                         while the current chunk computes.
//
// MFMA lane layouts used here (gfx950, wave64):
//   32x32x16 bf16: lane l supplies A[l%32][8(l/32) + e] and B[8(l/32) + e][l%32],
//                  e < 8; accumulator element e is D[8(e/4) + 4(l/32) + e%4][l%32].
//   16x16x32 bf16: lane l supplies A[l%16][8(l/16) + e] and B[8(l/16) + e][l%16];
//                  accumulator element e is D[4(l/16) + e][l%16].
// Every operand is read from LDS as 8 consecutive bf16 along the contraction index, so
// operands are stored contraction-contiguous (the state copy and the R/Delta tiles
// are stored value-column-major for that reason).
#include "internal.h"

namespace dn {
namespace {

constexpr int FC = 64;             // chunk
constexpr int FD = 128;            // Dk = Dv
constexpr int DVS = 32;            // state columns per state-pass workgroup
constexpr int NSL = FD / DVS;      // slices per (sequence, value head)
constexpr int KPITCH = FD + 8;     // bf16 row pitches (16-byte multiples, skewed banks)
constexpr int CPITCH = FC + 8;
constexpr int VPITCH = DVS + 8;

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

// Chunks each workspace T slot can hold: enough for a batch of rows and for a packed
// batch (sum_n ceil(len_n / 64) <= ceil(total / 64) + N).
__host__ __device__ inline long slot_bound(const PrefillArgs& a) {
    return ((long)a.B * a.T + FC - 1) / FC + a.N;
}
inline size_t offsets_bytes(const PrefillArgs& a) { return ((size_t)(a.N + 1) * 4 + 255) & ~(size_t)255; }

// ------------------------------------------------------------------ chunk offsets
constexpr int OFF_NT = 1024;

__global__ __launch_bounds__(OFF_NT) void chunk_offsets_kernel(const int32_t* cu, int N, int32_t* off) {
    __shared__ int part[OFF_NT];
    const int tid = threadIdx.x;
    const int per = (N + OFF_NT - 1) / OFF_NT;
    const int lo = min(N, tid * per), hi = min(N, lo + per);
    int s = 0;
    for (int n = lo; n < hi; ++n) s += (cu[n + 1] - cu[n] + FC - 1) / FC;
    part[tid] = s;
    __syncthreads();
    if (tid == 0) {  // exclusive scan of the 1024 partial sums
        int acc = 0;
        for (int t = 0; t < OFF_NT; ++t) {
            const int x = part[t];
            part[t] = acc;
            acc += x;
        }
    }
    __syncthreads();
    s = part[tid];
    if (tid == 0) off[0] = 0;
    for (int n = lo; n < hi; ++n) {
        s += (cu[n + 1] - cu[n] + FC - 1) / FC;
        off[n + 1] = s;
    }
}

// Locate chunk slot gc: sequence n, first token t0 and length len (len <= 0: unused).
__device__ __forceinline__ void locate_chunk(const PrefillArgs& a, const int32_t* off, long nct,
                                             long gc, int& n, long& t0, int& len) {
    if (a.cu) {
        len = 0;
        n = 0;
        t0 = 0;
        if (gc >= off[a.N]) return;
        int lo = 0, hi = a.N - 1;  // largest n with off[n] <= gc (never an empty sequence)
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= gc) lo = mid; else hi = mid - 1;
        }
        n = lo;
        t0 = a.cu[n] + (gc - off[n]) * FC;
        len = (int)min((long)FC, (long)a.cu[n + 1] - t0);
    } else {
        n = (int)(gc / nct);
        const long c = gc % nct;
        t0 = (long)n * a.T + c * FC;
        len = (int)min((long)FC, (long)a.T - c * FC);
    }
}

// --------------------------------------------------------------------------- prep
struct PrepSmem {
    __bf16 K[FC][KPITCH];
    float A[FC][FC + 1];
    float Tm[FC][FC + 1];
    float X[3][16][17];
    float gam[FC];
    float beta[FC];
};

__global__ __launch_bounds__(256) void prep_kernel(PrefillArgs a, const int32_t* off, __bf16* Tws, long nct) {
    __shared__ PrepSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hq = blockIdx.x % a.Hqk;
    const long gc = blockIdx.x / a.Hqk;
    int n, len;
    long t0;
    locate_chunk(a, off, nct, gc, n, t0, len);
    if (len <= 0) return;
    const int R = a.Hv / a.Hqk;
    const __bf16* kp = static_cast<const __bf16*>(a.k);

#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int v = tid + 256 * p, row = v >> 4, cg = v & 15;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (row < len) val = *reinterpret_cast<const uint4*>(kp + ((t0 + row) * a.Hqk + hq) * FD + cg * 8);
        *reinterpret_cast<uint4*>(&sm.K[row][cg * 8]) = val;
    }
    __syncthreads();

    // K K^T, lower tiles (0,0), (1,0), (1,1) on waves 0..2
    const int ta = wave == 0 ? 0 : 1, tb = wave == 2 ? 1 : 0;
    f32x16 G = {};
    if (wave < 3) {
        const int ra = 32 * ta + (lane & 31), rb = 32 * tb + (lane & 31), ko = (lane >> 5) * 8;
#pragma unroll
        for (int kk = 0; kk < FD / 16; ++kk)
            G = mma32(ld8(&sm.K[ra][kk * 16 + ko]), ld8(&sm.K[rb][kk * 16 + ko]), G);
    }

    for (int u = 0; u < R; ++u) {
        const int h = hq * R + u;
        if (tid < FC) {
            const bool in = tid < len;
            const long idx = (t0 + tid) * a.Hv + h;
            float gv = (in && a.g) ? a.g[idx] : 0.f;
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(gv, o);
                if (lane >= o) gv += y;
            }
            sm.gam[tid] = gv;
            sm.beta[tid] = in ? a.beta[idx] : 0.f;
        }
        __syncthreads();
        // A = strictly-lower beta/decay-weighted Gram; zero the tile above the diagonal
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int m = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3), c = lane & 31;
            if (wave < 3) {
                const int r = 32 * ta + m, i = 32 * tb + c;
                sm.A[r][i] = (i < r && r < len) ? sm.beta[r] * expf(sm.gam[r] - sm.gam[i]) * G[e] : 0.f;
            } else {
                sm.A[m][32 + c] = 0.f;
            }
        }
        // T's blocks above the block diagonal are zero
        for (int e = tid; e < FC * FC; e += 256) {
            const int r = e >> 6, i = e & 63;
            if ((i >> 4) > (r >> 4)) sm.Tm[r][i] = 0.f;
        }
        __syncthreads();
        // diagonal 16x16 blocks of (I + A)^{-1}: forward substitution, one lane per column
        if (wave == 0) {
            const int base = 16 * (lane >> 4), c = lane & 15;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float s = 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) s += sm.A[base + r][base + m] * x[m];
                x[r] = (r == c) ? 1.f : (r < c ? 0.f : -s);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.Tm[base + r][base + c] = x[r];
        }
        __syncthreads();
        // blocks below the diagonal, one block diagonal at a time:
        // T_ij = -T_ii sum_{j <= m < i} A_im T_mj
        for (int d = 1; d < 4; ++d) {
            const int nb = 4 - d;
            for (int e = tid; e < nb * 256; e += 256) {
                const int j = e >> 8, i = j + d, r = (e >> 4) & 15, c = e & 15;
                float s = 0.f;
                for (int m = j; m < i; ++m)
#pragma unroll
                    for (int x = 0; x < 16; ++x) s += sm.A[16 * i + r][16 * m + x] * sm.Tm[16 * m + x][16 * j + c];
                sm.X[j][r][c] = s;
            }
            __syncthreads();
            for (int e = tid; e < nb * 256; e += 256) {
                const int j = e >> 8, i = j + d, r = (e >> 4) & 15, c = e & 15;
                float s = 0.f;
#pragma unroll
                for (int x = 0; x < 16; ++x) s += sm.Tm[16 * i + r][16 * i + x] * sm.X[j][x][c];
                sm.Tm[16 * i + r][16 * j + c] = -s;
            }
            __syncthreads();
        }
        __bf16* tout = Tws + ((size_t)gc * a.Hv + h) * (FC * FC);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int v = tid + 256 * p, row = v >> 3, cg = v & 7;
            bf16x8 val;
#pragma unroll
            for (int e = 0; e < 8; ++e) val[e] = (__bf16)sm.Tm[row][cg * 8 + e];
            *reinterpret_cast<bf16x8*>(tout + row * FC + cg * 8) = val;
        }
        __syncthreads();
    }
}

// --------------------------------------------------------------------- state pass
struct StateSmem {
    __bf16 K[FC][KPITCH];      // chunk keys, token-major
    __bf16 Q[FC][KPITCH];      // chunk queries, token-major
    __bf16 T[FC][CPITCH];      // (I + A)^{-1}
    __bf16 P[FC][CPITCH];      // masked, decayed Q K^T
    __bf16 V[FC][VPITCH];      // value slice
    __bf16 MbT[DVS][KPITCH];   // bf16 copy of the state slice, value-column-major
    __bf16 RT[DVS][CPITCH];    // R, value-column-major
    __bf16 DT[DVS][CPITCH];    // Delta, value-column-major
    __bf16 DtT[DVS][CPITCH];   // Delta scaled by exp(gamma_last - gamma_r)
    float gam[FC];
    float beta[FC];
    float eg[FC];              // exp(gamma_r)
    float tail[FC];            // exp(gamma_last - gamma_r)
};

struct Prefetch {
    uint4 k[4], q[4], t[2], v;
    float beta, g;
};

__device__ __forceinline__ void fetch_chunk(const PrefillArgs& a, const __bf16* Tchunk, long t0, int len,
                                            int hq, int h, int j0, int tid, Prefetch& f) {
    const __bf16* kp = static_cast<const __bf16*>(a.k);
    const __bf16* qp = static_cast<const __bf16*>(a.q);
    const __bf16* vp = static_cast<const __bf16*>(a.v);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int v = tid + 256 * p, row = v >> 4, cg = v & 15;
        f.k[p] = f.q[p] = make_uint4(0, 0, 0, 0);
        if (row < len) {
            const long off = ((t0 + row) * a.Hqk + hq) * FD + cg * 8;
            f.k[p] = *reinterpret_cast<const uint4*>(kp + off);
            f.q[p] = *reinterpret_cast<const uint4*>(qp + off);
        }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int v = tid + 256 * p;
        f.t[p] = *reinterpret_cast<const uint4*>(Tchunk + v * 8);
    }
    {
        const int row = tid >> 2, cg = tid & 3;
        f.v = make_uint4(0, 0, 0, 0);
        if (row < len) f.v = *reinterpret_cast<const uint4*>(vp + ((t0 + row) * a.Hv + h) * FD + j0 + cg * 8);
    }
    f.beta = 0.f;
    f.g = 0.f;
    if (tid < FC && tid < len) {
        const long idx = (t0 + tid) * a.Hv + h;
        f.beta = a.beta[idx];
        if (a.g) f.g = a.g[idx];
    }
}

__global__ __launch_bounds__(256) void state_kernel(PrefillArgs a, const int32_t* off, const __bf16* Tws,
                                                    long nct) {
    __shared__ StateSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi32 = lane >> 5;

    // Workgroup -> (chain = sequence * Hv + head, slice).  When the chain count is a
    // multiple of 8, the slices of one chain land on one XCD (workgroups are dealt to
    // the 8 XCDs round-robin), so they share K, Q and T through that XCD's L2.
    const int chains = a.N * a.Hv;
    const int b = blockIdx.x;
    int chain, slice;
    if ((chains & 7) == 0) {
        const int y = b >> 3;
        slice = y % NSL;
        chain = (b & 7) + 8 * (y / NSL);
    } else {
        slice = b % NSL;
        chain = b / NSL;
    }
    int n = chain / a.Hv;
    const int h = chain % a.Hv;
    if (a.cu && a.N <= 64) {
        // longest sequences first: rank -> sequence (ties by index)
        const int rank = n;
        for (int m = 0; m < a.N; ++m) {
            const int lm = a.cu[m + 1] - a.cu[m];
            int r = 0;
            for (int x = 0; x < a.N; ++x) {
                const int lx = a.cu[x + 1] - a.cu[x];
                r += (lx > lm) || (lx == lm && x < m);
            }
            if (r == rank) n = m;
        }
    }
    const int nh = n * a.Hv + h;
    const int hq = h / (a.Hv / a.Hqk);
    const int j0 = slice * DVS;
    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);
    const int nchunks = (int)((eos - bos + FC - 1) / FC);
    const long gc0 = a.cu ? (long)off[n] : (long)n * nct;

    // state slice rows 32*wave .. +31 (key index), columns j0 + l32 (value index)
    f32x16 M;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = 32 * wave + 8 * (e >> 2) + 4 * hi32 + (e & 3);
        M[e] = a.h0 ? a.h0[((long)nh * FD + i) * FD + j0 + l32] : 0.f;
    }
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
        st4(&sm.MbT[l32][32 * wave + 8 * g4 + 4 * hi32], M[4 * g4], M[4 * g4 + 1], M[4 * g4 + 2], M[4 * g4 + 3]);

    Prefetch f;
    if (nchunks > 0)
        fetch_chunk(a, Tws + ((size_t)gc0 * a.Hv + h) * (FC * FC), bos, (int)min((long)FC, eos - bos),
                    hq, h, j0, tid, f);

    for (int c = 0; c < nchunks; ++c) {
        const long t0 = bos + (long)c * FC;
        const int len = (int)min((long)FC, eos - t0);
        // ---- stage the fetched chunk in LDS
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int v = tid + 256 * p, row = v >> 4, cg = v & 15;
            *reinterpret_cast<uint4*>(&sm.K[row][cg * 8]) = f.k[p];
            *reinterpret_cast<uint4*>(&sm.Q[row][cg * 8]) = f.q[p];
        }
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int v = tid + 256 * p, row = v >> 3, cg = v & 7;
            *reinterpret_cast<uint4*>(&sm.T[row][cg * 8]) = f.t[p];
        }
        *reinterpret_cast<uint4*>(&sm.V[tid >> 2][(tid & 3) * 8]) = f.v;
        if (tid < FC) {
            float gv = f.g;
            for (int o = 1; o < 64; o <<= 1) {
                const float y = __shfl_up(gv, o);
                if (lane >= o) gv += y;
            }
            const float glast = __shfl(gv, 63);
            sm.gam[tid] = gv;
            sm.beta[tid] = f.beta;
            sm.eg[tid] = expf(gv);
            sm.tail[tid] = expf(glast - gv);
        }
        __syncthreads();
        if (c + 1 < nchunks) {
            const long t1 = t0 + FC;
            fetch_chunk(a, Tws + ((size_t)(gc0 + c + 1) * a.Hv + h) * (FC * FC), t1,
                        (int)min((long)FC, eos - t1), hq, h, j0, tid, f);
        }

        // ---- phase A: X = [K; Q] M (waves 0,1: K rows, waves 2,3: Q rows) and P^T tiles
        const int xr = 32 * (wave & 1) + l32;
        const __bf16* xsrc = wave < 2 ? &sm.K[xr][0] : &sm.Q[xr][0];
        f32x16 X = {};
#pragma unroll
        for (int kk = 0; kk < FD / 16; ++kk)
            X = mma32(ld8(xsrc + kk * 16 + 8 * hi32), ld8(&sm.MbT[l32][kk * 16 + 8 * hi32]), X);
        if (wave < 2) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int r = 32 * wave + 8 * g4 + 4 * hi32;
                float rv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rv[e] = sm.beta[r + e] * ((float)sm.V[r + e][l32] - sm.eg[r + e] * X[4 * g4 + e]);
                st4(&sm.RT[l32][r], rv[0], rv[1], rv[2], rv[3]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = 32 * (wave - 2) + 8 * (e >> 2) + 4 * hi32 + (e & 3);
                X[e] *= sm.eg[r];
            }
        }
        // P^T tile (ti, tr): rows = key token i, columns = query token r; tile (1,0) is zero
        {
            const int ti = wave == 2 ? 1 : 0, tr = wave == 0 ? 0 : 1;
            f32x16 Pt = {};
            if (wave < 3) {
#pragma unroll
                for (int kk = 0; kk < FD / 16; ++kk)
                    Pt = mma32(ld8(&sm.K[32 * ti + l32][kk * 16 + 8 * hi32]),
                               ld8(&sm.Q[32 * tr + l32][kk * 16 + 8 * hi32]), Pt);
            }
            const int r = (wave < 3 ? 32 * tr : 0) + l32;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int i = (wave < 3 ? 32 * ti : 32) + 8 * g4 + 4 * hi32;
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pv[e] = (wave < 3 && i + e <= r) ? expf(sm.gam[r] - sm.gam[i + e]) * Pt[4 * g4 + e] : 0.f;
                st4(&sm.P[r][i], pv[0], pv[1], pv[2], pv[3]);
            }
        }
        __syncthreads();

        // ---- phase B: Delta = T R, rows 16*wave .. +15, two 16-column tiles
        {
            const int l16 = lane & 15, q16 = lane >> 4;
            f32x4 D0 = {}, D1 = {};
#pragma unroll
            for (int kk = 0; kk < FC / 32; ++kk) {
                const bf16x8 ta = ld8(&sm.T[16 * wave + l16][kk * 32 + 8 * q16]);
                D0 = mma16(ta, ld8(&sm.RT[l16][kk * 32 + 8 * q16]), D0);
                D1 = mma16(ta, ld8(&sm.RT[16 + l16][kk * 32 + 8 * q16]), D1);
            }
            const int r = 16 * wave + 4 * q16;
            st4(&sm.DT[l16][r], D0[0], D0[1], D0[2], D0[3]);
            st4(&sm.DT[16 + l16][r], D1[0], D1[1], D1[2], D1[3]);
            st4(&sm.DtT[l16][r], sm.tail[r] * D0[0], sm.tail[r + 1] * D0[1], sm.tail[r + 2] * D0[2],
                sm.tail[r + 3] * D0[3]);
            st4(&sm.DtT[16 + l16][r], sm.tail[r] * D1[0], sm.tail[r + 1] * D1[1], sm.tail[r + 2] * D1[2],
                sm.tail[r + 3] * D1[3]);
        }
        __syncthreads();

        // ---- phase C: carry M <- exp(gamma_last) M + K^T Delta~, and O = X + P Delta
        {
            const float Gl = sm.eg[FC - 1];  // rows past the chunk end add g = 0
#pragma unroll
            for (int e = 0; e < 16; ++e) M[e] *= Gl;
            const int i = 32 * wave + l32;
#pragma unroll
            for (int kk = 0; kk < FC / 16; ++kk) {
                bf16x8 ka;
#pragma unroll
                for (int e = 0; e < 8; ++e) ka[e] = sm.K[kk * 16 + 8 * hi32 + e][i];
                M = mma32(ka, ld8(&sm.DtT[l32][kk * 16 + 8 * hi32]), M);
            }
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                st4(&sm.MbT[l32][32 * wave + 8 * g4 + 4 * hi32], M[4 * g4], M[4 * g4 + 1], M[4 * g4 + 2],
                    M[4 * g4 + 3]);
            if (wave >= 2) {
                const int pr = 32 * (wave - 2) + l32;
#pragma unroll
                for (int kk = 0; kk < FC / 16; ++kk)
                    X = mma32(ld8(&sm.P[pr][kk * 16 + 8 * hi32]), ld8(&sm.DT[l32][kk * 16 + 8 * hi32]), X);
                __bf16* op = static_cast<__bf16*>(a.o);
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int r = 32 * (wave - 2) + 8 * (e >> 2) + 4 * hi32 + (e & 3);
                    if (r < len) op[((t0 + r) * a.Hv + h) * FD + j0 + l32] = (__bf16)(a.scale * X[e]);
                }
            }
        }
        __syncthreads();
    }

    if (a.hT) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = 32 * wave + 8 * (e >> 2) + 4 * hi32 + (e & 3);
            a.hT[((long)nh * FD + i) * FD + j0 + l32] = M[e];
        }
    }
}

}  // namespace

bool prefill_fast_supported(const PrefillArgs& a) {
    return a.bf16 && a.Dk == FD && a.Dv == FD && a.C == FC;
}

size_t prefill_fast_workspace_bytes(const PrefillArgs& a) {
    return offsets_bytes(a) + (size_t)slot_bound(a) * a.Hv * FC * FC * sizeof(__bf16);
}

hipError_t launch_prefill_fast(const PrefillArgs& a, hipStream_t s) {
    if (a.ws_bytes < prefill_fast_workspace_bytes(a)) return hipErrorInvalidValue;
    int32_t* off = static_cast<int32_t*>(a.ws);
    __bf16* Tws = reinterpret_cast<__bf16*>(static_cast<char*>(a.ws) + offsets_bytes(a));
    const long nct = a.cu ? 0 : ((long)a.T + FC - 1) / FC;
    const long slots = a.cu ? slot_bound(a) : (long)a.B * nct;
    if (a.cu) hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(OFF_NT), 0, s, a.cu, a.N, off);
    const long prep_blocks = slots * a.Hqk;
    if (prep_blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (prep_blocks > 0)
        hipLaunchKernelGGL(prep_kernel, dim3((unsigned)prep_blocks), dim3(256), 0, s, a, off, Tws, nct);
    const long state_blocks = (long)a.N * a.Hv * NSL;
    if (state_blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (state_blocks > 0)
        hipLaunchKernelGGL(state_kernel, dim3((unsigned)state_blocks), dim3(256), 0, s, a, off, Tws, nct);
    return hipGetLastError();
}

}  // namespace dn
