// prefill_fast.hip -- chunked prefill of the gated delta rule on the gfx950 matrix
// cores (bf16 MFMA, fp32 accumulation), for bf16 inputs with Dk = Dv = 128 and
// 64-token chunks.
//
// The algebra is the chunked form of the update on the frankenstein "DeltaNet
// Attention" page (module docstring), with the gate order of the nnterp
// "linear_attention" page.  Inside a chunk of n <= 64 tokens, with the state slice
// M (key-major, S^T) at the chunk start and gamma_r = sum_{i<=r} g_i:
//
//   A_ri  = beta_r exp(gamma_r - gamma_i) k_r.k_i (i < r),   T = (I + A)^{-1}
//   R     = diag(beta) (V - diag(exp(gamma)) K M)
//   Delta = T R                                   (row r: beta_r x prediction error)
//   O     = scale (diag(exp(gamma)) Q M + P Delta),  P_ri = exp(gamma_r - gamma_i) q_r.k_i (i <= r)
//   M    <- exp(gamma_last) M + K^T diag(exp(gamma_last - gamma)) Delta
//
// Three kernels on the caller's stream:
//   chunk_offsets_kernel  (packed batches only) index of each sequence's first chunk.
//   prep_kernel           one wave per (chunk, value head), all chunks in parallel:
//                         K K^T on the matrix cores, the decay/beta mask, and
//                         T = (I + A)^{-1}: the four 16x16 diagonal blocks by fp32
//                         forward substitution (one lane per column), then the blocks
//                         below the diagonal in two levels of 2x2 block inversion,
//                         T21 = -T22 A21 T11, one MFMA per 16x16 tile.  T goes to the
//                         workspace in bf16.
//   state_kernel          one workgroup of 8 waves per (sequence, value head, 32-column
//                         slice of the state); the value columns of the state are
//                         independent, so slices never exchange data.
//                           waves 0-3 ("chain"): X = K M, R, Delta = T R and the state
//                             update, holding the 128 x 32 fp32 slice in accumulators;
//                           waves 4-7 ("output"): Q M, the P tiles and O = Y + P Delta,
//                             and they stage the next chunk (fetched into registers one
//                             chunk ahead) into the other half of a double-buffered LDS.
//                         Three workgroup barriers per chunk.
//
// MFMA lane layouts (gfx950, wave64):
//   32x32x16 bf16: lane l supplies A[l%32][8(l/32) + e] and B[8(l/32) + e][l%32],
//                  e < 8; accumulator element e is D[8(e/4) + 4(l/32) + e%4][l%32].
//   16x16x32 bf16: lane l supplies A[l%16][8(l/16) + e] and B[8(l/16) + e][l%16];
//                  accumulator element e is D[4(l/16) + e][l%16].
// Every operand is read from LDS as 8 consecutive bf16 along the contraction index, so
// each operand is stored contraction-contiguous; the matrices produced here (state copy,
// R, Delta, T's transposed copy) are written in the layout their consumer reads.
#include <type_traits>

#include "internal.h"

namespace dn {
namespace {

constexpr int FC = 64;             // chunk
constexpr int FD = 128;            // Dk = Dv
constexpr int DVS = 32;            // state columns per state-pass workgroup
constexpr int NSL = FD / DVS;      // slices per (sequence, value head)
constexpr int KPITCH = FD + 8;     // bf16 row pitches: 16-byte multiples that put the
constexpr int CPITCH = FC + 8;     //   16 rows of one MFMA operand read on distinct banks
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
    if (tid == 0) {  // exclusive scan of the per-thread sums
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
// Per (chunk slot, value head) the workspace holds T^T and P, both 64 x 64 bf16:
//   Tt[c][r] = T[r][c]   (T = (I + A)^{-1}, stored transposed)
//   P[r][i]  = exp(gamma_r - gamma_i) q_r.k_i for i <= r < len, else 0 (rows past len: 0)
constexpr int TP_ELEMS = 2 * FC * FC;

struct alignas(16) PrepSmem {
    __bf16 Ab[FC][CPITCH];     // A in bf16 (only the blocks below the diagonal are read)
    float Ad[4][260];          // A's diagonal 16x16 blocks, fp32, row pitch 16, block pitch 260
    __bf16 Tt[FC][CPITCH];     // T^T
    __bf16 XT[32][40];         // level products' intermediate, transposed
    float gam[FC];
    float beta[FC];
};

// One wave = one (chunk slot, value head).  The Gram operands come straight from global
// memory in MFMA layout (each key/query element is loaded once), so the only LDS traffic
// is the small triangular solve.
__global__ __launch_bounds__(64) void prep_kernel(PrefillArgs a, const int32_t* off, __bf16* Tws, long nct) {
    __shared__ PrepSmem sm;
    const int l = threadIdx.x;
    const int l32 = l & 31, hi32 = l >> 5, l16 = l & 15, q16 = l >> 4;
    const int h = blockIdx.x % a.Hv;
    const long gc = blockIdx.x / a.Hv;
    int n, len;
    long t0;
    locate_chunk(a, off, nct, gc, n, t0, len);
    if (len <= 0) return;
    const int hq = h / (a.Hv / a.Hqk);
    const __bf16* kp = static_cast<const __bf16*>(a.k);
    const __bf16* qp = static_cast<const __bf16*>(a.q);

    // operand fragments: rows 32*rb + l32, columns 16*kk + 8*hi32 .. +7
    bf16x8 kf[2][8], qf[2][8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = 32 * rb + l32;
        const long base = ((t0 + row) * a.Hqk + hq) * FD + 8 * hi32;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            kf[rb][kk] = row < len ? ld8(kp + base + 16 * kk) : zero8();
            qf[rb][kk] = row < len ? ld8(qp + base + 16 * kk) : zero8();
        }
    }
    {
        const bool in = l < len;
        const long idx = (t0 + l) * a.Hv + h;
        float gv = (in && a.g) ? a.g[idx] : 0.f;
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(gv, o);
            if (l >= o) gv += y;
        }
        sm.gam[l] = gv;
        sm.beta[l] = in ? a.beta[idx] : 0.f;
    }
    // T^T is zero where T is (above T's block diagonal): Tt blocks below the diagonal
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int v = l + 64 * p, r = v >> 3, cg = v & 7;
        if (cg * 8 + 8 <= (r >> 4) * 16) *reinterpret_cast<bf16x8*>(&sm.Tt[r][cg * 8]) = zero8();
    }

    // K K^T tiles (0,0), (1,0), (1,1) and K Q^T tiles (key block, query block)
    // (0,0), (0,1), (1,1): element e of tile (x, y) is row 32x + 8(e/4) + 4 hi32 + e%4,
    // column 32y + l32
    f32x16 G00 = {}, G10 = {}, G11 = {}, P00 = {}, P01 = {}, P11 = {};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
        G00 = mma32(kf[0][kk], kf[0][kk], G00);
        G10 = mma32(kf[1][kk], kf[0][kk], G10);
        G11 = mma32(kf[1][kk], kf[1][kk], G11);
        P00 = mma32(kf[0][kk], qf[0][kk], P00);
        P01 = mma32(kf[0][kk], qf[1][kk], P01);
        P11 = mma32(kf[1][kk], qf[1][kk], P11);
    }
    __syncthreads();

    // A_ri = beta_r exp(gamma_r - gamma_i) (k_r . k_i) for i < r < len
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const int ta = t == 0 ? 0 : 1, tb = t == 2 ? 1 : 0;
        const f32x16 G = t == 0 ? G00 : (t == 1 ? G10 : G11);
        const int i = 32 * tb + l32;
        const float gi = sm.gam[i];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int r0 = 32 * ta + 8 * g4 + 4 * hi32;
            const float4 gr = *reinterpret_cast<const float4*>(&sm.gam[r0]);
            const float4 br = *reinterpret_cast<const float4*>(&sm.beta[r0]);
            const float grv[4] = {gr.x, gr.y, gr.z, gr.w}, brv[4] = {br.x, br.y, br.z, br.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = r0 + e;
                const float av = (i < r && r < len) ? brv[e] * __expf(grv[e] - gi) * G[4 * g4 + e] : 0.f;
                if ((r >> 4) == (i >> 4)) sm.Ad[r >> 4][(r & 15) * 16 + (i & 15)] = av;
                sm.Ab[r][i] = (__bf16)av;
            }
        }
    }
    // P_ri = exp(gamma_r - gamma_i) (q_r . k_i) for i <= r < len, written row-major
    {
        __bf16* pout = Tws + ((size_t)gc * a.Hv + h) * TP_ELEMS + FC * FC;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int xa = t == 2 ? 1 : 0, yb = t == 0 ? 0 : 1;  // key block, query block
            const f32x16 Pt = t == 0 ? P00 : (t == 1 ? P01 : P11);
            const int r = 32 * yb + l32;
            const float gr = sm.gam[r];
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int i0 = 32 * xa + 8 * g4 + 4 * hi32;
                const float4 gi = *reinterpret_cast<const float4*>(&sm.gam[i0]);
                const float giv[4] = {gi.x, gi.y, gi.z, gi.w};
                bf16x4 pv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pv[e] = (__bf16)((i0 + e <= r && r < len) ? __expf(gr - giv[e]) * Pt[4 * g4 + e] : 0.f);
                *reinterpret_cast<bf16x4*>(pout + r * FC + i0) = pv;
            }
        }
    }
    __syncthreads();

    // diagonal blocks: lane = 16 * block + column; forward substitution down the column
    {
        const int b = q16, c = l16;
        const float* Ab_ = &sm.Ad[b][0];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int m4 = 0; m4 < (r + 3) / 4; ++m4) {
                const float4 av = *reinterpret_cast<const float4*>(Ab_ + r * 16 + 4 * m4);
                const float avv[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int m = 4 * m4 + u;
                    if (m < r) {
                        if (u & 1) s1 += avv[u] * x[m];
                        else s0 += avv[u] * x[m];
                    }
                }
            }
            x[r] = (r == c) ? 1.f : (r < c ? 0.f : -(s0 + s1));
        }
        bf16x8 lo8, hi8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo8[e] = (__bf16)x[e];
            hi8[e] = (__bf16)x[8 + e];
        }
        *reinterpret_cast<bf16x8*>(&sm.Tt[16 * b + c][16 * b]) = lo8;
        *reinterpret_cast<bf16x8*>(&sm.Tt[16 * b + c][16 * b + 8]) = hi8;
    }
    __syncthreads();

    // level 1: within each 32x32 diagonal block, T21 = -T22 A21 T11 (16x16 blocks; k = 16
    // padded to the instruction's 32 with zero lanes)
    const bool live = q16 < 2;
#pragma unroll
    for (int base = 0; base < FC; base += 32) {
        const bf16x8 af = live ? ld8(&sm.Ab[base + 16 + l16][base + 8 * q16]) : zero8();
        const bf16x8 bf = live ? ld8(&sm.Tt[base + l16][base + 8 * q16]) : zero8();
        const f32x4 X = mma16(af, bf, f32x4{0.f, 0.f, 0.f, 0.f});
        st4(&sm.XT[(base >> 1) + l16][4 * q16], X[0], X[1], X[2], X[3]);
    }
    __syncthreads();
#pragma unroll
    for (int base = 0; base < FC; base += 32) {
        // A operand T22[m][k] = Tt[base+16+k][base+16+m]: transposed read, k = 8 q16 + e
        const int s = l16;   // groups 2,3 only pad k: keep their (unused) reads inside the tile
        const __bf16* src = &sm.Tt[base + 16 + 8 * (q16 & 1) + (s >> 2)][base + 16 + 4 * (s & 3)];
        bf16x8 af = cat(trld(src), trld(src + 4 * CPITCH));
        if (!live) af = zero8();
        const bf16x8 bf = live ? ld8(&sm.XT[(base >> 1) + l16][8 * q16]) : zero8();
        const f32x4 Y = mma16(af, bf, f32x4{0.f, 0.f, 0.f, 0.f});
        st4(&sm.Tt[base + l16][base + 16 + 4 * q16], -Y[0], -Y[1], -Y[2], -Y[3]);
    }
    __syncthreads();
    // level 2: T[32:64, 0:32] = -T[32:64, 32:64] A[32:64, 0:32] T[0:32, 0:32], 16x16 tiles
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tr = tt >> 1, tc = tt & 1;
        const f32x4 X = mma16(ld8(&sm.Ab[32 + 16 * tr + l16][8 * q16]), ld8(&sm.Tt[16 * tc + l16][8 * q16]),
                              f32x4{0.f, 0.f, 0.f, 0.f});
        st4(&sm.XT[16 * tc + l16][16 * tr + 4 * q16], X[0], X[1], X[2], X[3]);
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tr = tt >> 1, tc = tt & 1;
        const int s = l16;
        const __bf16* src = &sm.Tt[32 + 8 * q16 + (s >> 2)][32 + 16 * tr + 4 * (s & 3)];
        const bf16x8 af = cat(trld(src), trld(src + 4 * CPITCH));
        const f32x4 Y = mma16(af, ld8(&sm.XT[16 * tc + l16][8 * q16]), f32x4{0.f, 0.f, 0.f, 0.f});
        st4(&sm.Tt[16 * tc + l16][32 + 16 * tr + 4 * q16], -Y[0], -Y[1], -Y[2], -Y[3]);
    }
    __syncthreads();
    __bf16* tout = Tws + ((size_t)gc * a.Hv + h) * TP_ELEMS;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int v = l + 64 * p, row = v >> 3, cg = v & 7;
        *reinterpret_cast<bf16x8*>(tout + row * FC + cg * 8) = ld8(&sm.Tt[row][cg * 8]);
    }
}

// --------------------------------------------------------------------- state pass
constexpr int CW = 16;              // state columns per chain wave
constexpr int NCW = DVS / CW;       // chain waves per workgroup
constexpr int NLW = 4;              // loader waves per workgroup
constexpr int SNT = 64 * (NCW + NLW);

struct alignas(16) ChunkBuf {
    __bf16 K[FC][KPITCH];      // chunk keys, token-major
    __bf16 Q[FC][KPITCH];      // chunk queries, token-major
    __bf16 Tt[FC][CPITCH];     // T^T
    __bf16 P[FC][CPITCH];      // masked, decayed Q K^T, row r = query token
    __bf16 V[FC][VPITCH];      // value slice, token-major
    float beta[FC];
    float eg[FC];              // exp(gamma_r)
    float tail[FC];            // exp(gamma_last - gamma_r)
};

struct alignas(16) StateSmem {
    ChunkBuf buf[2];              // chunk c in buf[c & 1]; the loader waves stage chunk c + 1
    __bf16 OT[NCW][CW][CPITCH];   // per chain wave: its output tile, column-major
};

struct Prefetch {
    uint4 k[4], q[4], t[2], p[2], v;
    float beta, g;
};

// Loader thread lt (0..255) fetches its share of one chunk into registers.
__device__ __forceinline__ void fetch_chunk(const PrefillArgs& a, const __bf16* TP, long t0, int len, int hq,
                                            int h, int j0, int lt, Prefetch& f) {
    const __bf16* kp = static_cast<const __bf16*>(a.k);
    const __bf16* qp = static_cast<const __bf16*>(a.q);
    const __bf16* vp = static_cast<const __bf16*>(a.v);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int v = lt + 256 * p, row = v >> 4, cg = v & 15;
        f.k[p] = f.q[p] = make_uint4(0, 0, 0, 0);
        if (row < len) {
            const long off = ((t0 + row) * a.Hqk + hq) * FD + cg * 8;
            f.k[p] = *reinterpret_cast<const uint4*>(kp + off);
            f.q[p] = *reinterpret_cast<const uint4*>(qp + off);
        }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        f.t[p] = *reinterpret_cast<const uint4*>(TP + (lt + 256 * p) * 8);
        f.p[p] = *reinterpret_cast<const uint4*>(TP + FC * FC + (lt + 256 * p) * 8);
    }
    {
        const int row = lt >> 2, cg = lt & 3;
        f.v = make_uint4(0, 0, 0, 0);
        if (row < len) f.v = *reinterpret_cast<const uint4*>(vp + ((t0 + row) * a.Hv + h) * FD + j0 + cg * 8);
    }
    f.beta = 0.f;
    f.g = 0.f;
    if (lt < FC && lt < len) {
        const long idx = (t0 + lt) * a.Hv + h;
        f.beta = a.beta[idx];
        if (a.g) f.g = a.g[idx];
    }
}

__device__ __forceinline__ void stage_chunk(ChunkBuf& cb, const Prefetch& f, int lt) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int v = lt + 256 * p, row = v >> 4, cg = v & 15;
        *reinterpret_cast<uint4*>(&cb.K[row][cg * 8]) = f.k[p];
        *reinterpret_cast<uint4*>(&cb.Q[row][cg * 8]) = f.q[p];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int v = lt + 256 * p, row = v >> 3, cg = v & 7;
        *reinterpret_cast<uint4*>(&cb.Tt[row][cg * 8]) = f.t[p];
        *reinterpret_cast<uint4*>(&cb.P[row][cg * 8]) = f.p[p];
    }
    *reinterpret_cast<uint4*>(&cb.V[lt >> 2][(lt & 3) * 8]) = f.v;
    if (lt < FC) {  // one wave: inclusive scan of the log decays over the chunk
        float gv = f.g;
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(gv, o);
            if (lt >= o) gv += y;
        }
        const float glast = __shfl(gv, 63);
        cb.beta[lt] = f.beta;
        cb.eg[lt] = __expf(gv);
        cb.tail[lt] = __expf(glast - gv);
    }
}

// Orders this wave's LDS writes before its later LDS reads of the same data (LDS executes
// one wave's instructions in order; this only stops the compiler from reordering them).
__device__ __forceinline__ void wave_lds_order() { __asm__ volatile("" ::: "memory"); }

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

// One workgroup = (sequence, value head, 32-column slice); six waves, one barrier per chunk.
//   waves 0,1  chain waves: each owns 16 state columns (128 x 16 fp32 in eight 16x16
//              accumulator tiles) and, per chunk, runs X = K M, R, Delta = T R, the state
//              update, Y = Q M and O = exp(gamma) Y + P Delta for its columns.  Results
//              feed the next product as B operands through register lane swaps.
//   waves 2-5  loader waves: stage the next chunk from registers into the other LDS
//              buffer and fetch the chunk three ahead (two chunks in flight).
template <bool GATED>
__global__ __launch_bounds__(SNT, 1) __attribute__((amdgpu_waves_per_eu(1, 2))) void state_kernel(PrefillArgs a, const int32_t* off, const __bf16* Tws,
                                                       long nct) {
    __shared__ StateSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q16 = lane >> 4;
    const bool chainw = wave < NCW;
    const int lt = tid - 64 * NCW;                          // loader thread index
    const int jc = CW * wave;                               // chain wave: first column

    // Workgroup -> (chain = sequence * Hv + head, slice).  When the chain count is a
    // multiple of 8, the slices of one chain land on one XCD (workgroups are dealt to
    // the 8 XCDs round-robin), so they share K, Q, T and P through that XCD's L2.
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
    const __bf16* TPseq = Tws + ((size_t)gc0 * a.Hv + h) * TP_ELEMS;
    const size_t TPstride = (size_t)a.Hv * TP_ELEMS;
    __bf16* const obase = static_cast<__bf16*>(a.o) + (long)h * FD + j0 + jc;

    // Every wave passes one barrier per chunk: the chain waves after consuming chunk c
    // from buf[c & 1], the loader waves after staging chunk c + 1 into buf[(c + 1) & 1].
    // The two roles run separate loops so their registers never overlap.
    if (chainw) {
        // tile mt holds keys 16 mt + 4 q16 + e, column jc + l16 of the slice
        f32x4 M[8];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) M[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.h0) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    M[mt][e] = a.h0[((long)nh * FD + 16 * mt + 4 * q16 + e) * FD + j0 + jc + l16];
        }
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            const ChunkBuf& cb = sm.buf[c & 1];
            const long t0 = bos + (long)c * FC;
            const int len = (int)min((long)FC, eos - t0);
            // the state at the chunk start as B operands: k = key 32 s + 8 q16 + e
            bf16x8 mb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) mb[s] = acc_to_b(M[2 * s], M[2 * s + 1]);
            // X = K M: token tile t holds tokens 16 t + 4 q16 + e, column jc + l16
            f32x4 X[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) X[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int t = 0; t < 4; ++t) X[t] = mma16(ld8(&cb.K[16 * t + l16][32 * s + 8 * q16]), mb[s], X[t]);
            // R = beta (V - exp(gamma) X); V read transposed: lane gets 4 tokens of its column
            f32x4 R[4], egv[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r0 = 16 * t + 4 * q16;
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&cb.beta[r0]);
                const bf16x4 vv = trld(&cb.V[r0 + (l16 >> 2)][jc + 4 * (l16 & 3)]);
                if (GATED) egv[t] = *reinterpret_cast<const f32x4*>(&cb.eg[r0]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    R[t][e] = bt[e] * ((float)vv[e] - (GATED ? egv[t][e] * X[t][e] : X[t][e]));
            }
            const bf16x8 rb[2] = {acc_to_b(R[0], R[1]), acc_to_b(R[2], R[3])};
            // Delta = T R (T lower triangular: token tile t needs k < 16 (t + 1)); A operand
            // T[16 t + m][k] = Tt[k][16 t + m] by transposed reads
            f32x4 D[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) D[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int t = 2 * u; t < 4; ++t) {
                    const __bf16* src = &cb.Tt[32 * u + 8 * q16 + (l16 >> 2)][16 * t + 4 * (l16 & 3)];
                    D[t] = mma16(cat(trld(src), trld(src + 4 * CPITCH)), rb[u], D[t]);
                }
            const bf16x8 dd[2] = {acc_to_b(D[0], D[1]), acc_to_b(D[2], D[3])};
            bf16x8 db[2] = {dd[0], dd[1]};
            if (GATED) {  // Delta~ = diag(exp(gamma_last - gamma)) Delta for the state update
                f32x4 Dt[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const f32x4 tl = *reinterpret_cast<const f32x4*>(&cb.tail[16 * t + 4 * q16]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) Dt[t][e] = tl[e] * D[t][e];
                }
                db[0] = acc_to_b(Dt[0], Dt[1]);
                db[1] = acc_to_b(Dt[2], Dt[3]);
            }
            // Y = Q M (uses the chunk-start state)
            f32x4 Y[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) Y[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int t = 0; t < 4; ++t) Y[t] = mma16(ld8(&cb.Q[16 * t + l16][32 * s + 8 * q16]), mb[s], Y[t]);
            // M <- exp(gamma_last) M + K^T Delta~  (rows past the chunk end add g = 0)
            const float Gl = GATED ? cb.eg[FC - 1] : 1.f;
            if (GATED) {
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) M[mt] *= Gl;
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    // A operand K^T[16 mt + m][k] = K[k][16 mt + m], k = 32 u + 8 q16 + e
                    const __bf16* src = &cb.K[32 * u + 8 * q16 + (l16 >> 2)][16 * mt + 4 * (l16 & 3)];
                    M[mt] = mma16(cat(trld(src), trld(src + 4 * KPITCH)), db[u], M[mt]);
                }
            // O = scale (exp(gamma) Y + P Delta), P lower triangular; staged column-major
            if (GATED) {
#pragma unroll
                for (int t = 0; t < 4; ++t) Y[t] *= egv[t];
            }
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int t = 2 * u; t < 4; ++t) Y[t] = mma16(ld8(&cb.P[16 * t + l16][32 * u + 8 * q16]), dd[u], Y[t]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                st4(&sm.OT[wave][l16][16 * t + 4 * q16], a.scale * Y[t][0], a.scale * Y[t][1], a.scale * Y[t][2],
                    a.scale * Y[t][3]);
            wave_lds_order();
            // rows back by transposed reads: lane gets token 16 k + l16, columns 4 q16 .. +3
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bf16x4 ov = trld(&sm.OT[wave][4 * q16 + (l16 >> 2)][16 * k + 4 * (l16 & 3)]);
                const int r = 16 * k + l16;
                if (r < len) *reinterpret_cast<bf16x4*>(obase + (t0 + r) * a.Hv * FD + 4 * q16) = ov;
            }
            __syncthreads();
        }
        if (a.hT) {
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.hT[((long)nh * FD + 16 * mt + 4 * q16 + e) * FD + j0 + jc + l16] = M[mt][e];
        }
    } else {
        Prefetch f0, f1;   // even chunks in f0, odd chunks in f1
        auto fetch = [&](int c, Prefetch& f) {
            const long tc = bos + (long)c * FC;
            fetch_chunk(a, TPseq + (size_t)c * TPstride, tc, (int)min((long)FC, eos - tc), hq, h, j0, lt, f);
        };
        if (nchunks > 0) fetch(0, f0);
        if (nchunks > 1) fetch(1, f1);
        if (nchunks > 0) stage_chunk(sm.buf[0], f0, lt);
        if (nchunks > 2) fetch(2, f0);
        __syncthreads();
        // phase c: stage chunk c + 1 (held in f[(c + 1) & 1]) and refill that set with c + 3
        for (int c = 0; c < nchunks; c += 2) {
            if (c + 1 < nchunks) {
                stage_chunk(sm.buf[1], f1, lt);
                if (c + 3 < nchunks) fetch(c + 3, f1);
            }
            __syncthreads();
            if (c + 1 < nchunks) {
                if (c + 2 < nchunks) {
                    stage_chunk(sm.buf[0], f0, lt);
                    if (c + 4 < nchunks) fetch(c + 4, f0);
                }
                __syncthreads();
            }
        }
    }
}

}  // namespace

bool prefill_fast_supported(const PrefillArgs& a) {
    return a.bf16 && a.Dk == FD && a.Dv == FD && a.C == FC;
}

size_t prefill_fast_workspace_bytes(const PrefillArgs& a) {
    return offsets_bytes(a) + (size_t)slot_bound(a) * a.Hv * 2 * FC * FC * sizeof(__bf16);
}

hipError_t launch_prefill_fast(const PrefillArgs& a, hipStream_t s) {
    if (a.ws_bytes < prefill_fast_workspace_bytes(a)) return hipErrorInvalidValue;
    int32_t* off = static_cast<int32_t*>(a.ws);
    __bf16* Tws = reinterpret_cast<__bf16*>(static_cast<char*>(a.ws) + offsets_bytes(a));
    const long nct = a.cu ? 0 : ((long)a.T + FC - 1) / FC;
    const long slots = a.cu ? slot_bound(a) : (long)a.B * nct;
    if (a.cu) hipLaunchKernelGGL(chunk_offsets_kernel, dim3(1), dim3(OFF_NT), 0, s, a.cu, a.N, off);
    const long prep_blocks = slots * a.Hv;
    if (prep_blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (prep_blocks > 0)
        hipLaunchKernelGGL(prep_kernel, dim3((unsigned)prep_blocks), dim3(64), 0, s, a, off, Tws, nct);
    const long state_blocks = (long)a.N * a.Hv * NSL;
    if (state_blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (state_blocks > 0) {
        if (a.g)
            hipLaunchKernelGGL(state_kernel<true>, dim3((unsigned)state_blocks), dim3(SNT), 0, s, a, off, Tws, nct);
        else
            hipLaunchKernelGGL(state_kernel<false>, dim3((unsigned)state_blocks), dim3(SNT), 0, s, a, off, Tws, nct);
    }
    return hipGetLastError();
}

}  // namespace dn
