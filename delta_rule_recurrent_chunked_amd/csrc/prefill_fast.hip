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
constexpr int SNT = 512;           // state-pass threads (8 waves)

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
struct PrepSmem {
    union {
        __bf16 K[FC][KPITCH];              // the chunk's keys (until the Gram is formed)
        struct {
            __bf16 Ab[FC][CPITCH];         // A, bf16 (blocks below the diagonal)
            float Ad[4][16][17];           // A's diagonal 16x16 blocks, fp32
        } a;
    } u;
    __bf16 Tb[FC][CPITCH];                 // T row-major
    __bf16 TbT[FC][CPITCH];                // T transposed (column-major)
    __bf16 XT[32][40];                     // level products' intermediate, transposed
    float gam[FC];
    float beta[FC];
};

// One wave = one (chunk slot, value head).
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

#pragma unroll
    for (int p = 0; p < 16; ++p) {
        const int v = l + 64 * p, row = v >> 4, cg = v & 15;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (row < len) val = *reinterpret_cast<const uint4*>(kp + ((t0 + row) * a.Hqk + hq) * FD + cg * 8);
        *reinterpret_cast<uint4*>(&sm.u.K[row][cg * 8]) = val;
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
    // T is zero above its block diagonal: those blocks of Tb, and the mirrored blocks
    // (below the block diagonal) of the transposed copy TbT
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int v = l + 64 * p, r = v >> 3, cg = v & 7;  // 8 bf16 per store
        if (cg * 8 >= ((r >> 4) + 1) * 16) *reinterpret_cast<bf16x8*>(&sm.Tb[r][cg * 8]) = zero8();
        if (cg * 8 + 8 <= (r >> 4) * 16) *reinterpret_cast<bf16x8*>(&sm.TbT[r][cg * 8]) = zero8();
    }
    __syncthreads();

    // Gram K K^T: lower tiles (0,0), (1,0), (1,1) of 32x32
    f32x16 G00 = {}, G10 = {}, G11 = {};
#pragma unroll
    for (int kk = 0; kk < FD / 16; ++kk) {
        const bf16x8 f0 = ld8(&sm.u.K[l32][kk * 16 + 8 * hi32]);
        const bf16x8 f1 = ld8(&sm.u.K[32 + l32][kk * 16 + 8 * hi32]);
        G00 = mma32(f0, f0, G00);
        G10 = mma32(f1, f0, G10);
        G11 = mma32(f1, f1, G11);
    }
    __syncthreads();  // K is overwritten below
    // A_ri = beta_r exp(gamma_r - gamma_i) G_ri for i < r < len
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        const int ta = t == 0 ? 0 : 1, tb = t == 2 ? 1 : 0;
        const f32x16& G = t == 0 ? G00 : (t == 1 ? G10 : G11);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int r = 32 * ta + 8 * (e >> 2) + 4 * hi32 + (e & 3), i = 32 * tb + l32;
            const float av = (i < r && r < len) ? sm.beta[r] * expf(sm.gam[r] - sm.gam[i]) * G[e] : 0.f;
            if ((r >> 4) == (i >> 4)) sm.u.a.Ad[r >> 4][r & 15][i & 15] = av;
            sm.u.a.Ab[r][i] = (__bf16)av;
        }
    }
    __syncthreads();

    // diagonal blocks: lane = 16 * block + column; forward substitution down the column
    {
        const int b = q16, c = l16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) {
                if (m & 1) s1 += sm.u.a.Ad[b][r][m] * x[m];
                else s0 += sm.u.a.Ad[b][r][m] * x[m];
            }
            x[r] = (r == c) ? 1.f : (r < c ? 0.f : -(s0 + s1));
        }
        bf16x8 lo8, hi8;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            lo8[e] = (__bf16)x[e];
            hi8[e] = (__bf16)x[8 + e];
        }
        *reinterpret_cast<bf16x8*>(&sm.TbT[16 * b + c][16 * b]) = lo8;
        *reinterpret_cast<bf16x8*>(&sm.TbT[16 * b + c][16 * b + 8]) = hi8;
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Tb[16 * b + r][16 * b + c] = (__bf16)x[r];
    }
    __syncthreads();

    // level 1: within each 32x32 diagonal block, T21 = -T22 A21 T11 (16x16 blocks, k = 16
    // padded to the instruction's 32 with zero lanes)
#pragma unroll
    for (int base = 0; base < FC; base += 32) {
        const bool live = q16 < 2;
        bf16x8 af = live ? ld8(&sm.u.a.Ab[base + 16 + l16][base + 8 * q16]) : zero8();
        bf16x8 bf = live ? ld8(&sm.TbT[base + l16][base + 8 * q16]) : zero8();
        f32x4 X = mma16(af, bf, f32x4{0.f, 0.f, 0.f, 0.f});
        st4(&sm.XT[(base >> 1) + l16][4 * q16], X[0], X[1], X[2], X[3]);
    }
    __syncthreads();
#pragma unroll
    for (int base = 0; base < FC; base += 32) {
        const bool live = q16 < 2;
        bf16x8 af = live ? ld8(&sm.Tb[base + 16 + l16][base + 16 + 8 * q16]) : zero8();
        bf16x8 bf = live ? ld8(&sm.XT[(base >> 1) + l16][8 * q16]) : zero8();
        f32x4 Y = mma16(af, bf, f32x4{0.f, 0.f, 0.f, 0.f});
        const int r = base + 16 + 4 * q16, i = base + l16;
        st4(&sm.TbT[i][r], -Y[0], -Y[1], -Y[2], -Y[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Tb[r + e][i] = (__bf16)(-Y[e]);
    }
    __syncthreads();
    // level 2: T[32:64, 0:32] = -T[32:64, 32:64] A[32:64, 0:32] T[0:32, 0:32], 16x16 tiles
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tr = tt >> 1, tc = tt & 1;
        f32x4 X = mma16(ld8(&sm.u.a.Ab[32 + 16 * tr + l16][8 * q16]), ld8(&sm.TbT[16 * tc + l16][8 * q16]),
                        f32x4{0.f, 0.f, 0.f, 0.f});
        st4(&sm.XT[16 * tc + l16][16 * tr + 4 * q16], X[0], X[1], X[2], X[3]);
    }
    __syncthreads();
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tr = tt >> 1, tc = tt & 1;
        f32x4 Y = mma16(ld8(&sm.Tb[32 + 16 * tr + l16][32 + 8 * q16]), ld8(&sm.XT[16 * tc + l16][8 * q16]),
                        f32x4{0.f, 0.f, 0.f, 0.f});
        const int r = 32 + 16 * tr + 4 * q16, i = 16 * tc + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Tb[r + e][i] = (__bf16)(-Y[e]);
    }
    __syncthreads();
    __bf16* tout = Tws + ((size_t)gc * a.Hv + h) * (FC * FC);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int v = l + 64 * p, row = v >> 3, cg = v & 7;
        *reinterpret_cast<bf16x8*>(tout + row * FC + cg * 8) = ld8(&sm.Tb[row][cg * 8]);
    }
}

// --------------------------------------------------------------------- state pass
struct ChunkBuf {
    __bf16 K[FC][KPITCH];      // chunk keys, token-major
    __bf16 Q[FC][KPITCH];      // chunk queries, token-major
    __bf16 T[FC][CPITCH];      // (I + A)^{-1}
    __bf16 V[FC][VPITCH];      // value slice
    float gam[FC];
    float beta[FC];
    float eg[FC];              // exp(gamma_r)
    float tail[FC];            // exp(gamma_last - gamma_r)
};

struct StateSmem {
    ChunkBuf buf[2];           // chunk c in buf[c & 1]; the output waves stage chunk c + 1
    __bf16 P[FC][CPITCH];      // masked, decayed Q K^T (row r = query token)
    __bf16 MbT[DVS][KPITCH];   // bf16 copy of the state slice, value-column-major
    __bf16 RT[DVS][CPITCH];    // R, value-column-major
    __bf16 DT[DVS][CPITCH];    // Delta, value-column-major
    __bf16 DtT[DVS][CPITCH];   // Delta scaled by exp(gamma_last - gamma_r)
};

struct Prefetch {
    uint4 k[4], q[4], t[2], v;
    float beta, g;
};

// Output-wave thread pt (0..255) fetches its share of one chunk into registers.
__device__ __forceinline__ void fetch_chunk(const PrefillArgs& a, const __bf16* Tchunk, long t0, int len,
                                            int hq, int h, int j0, int pt, Prefetch& f) {
    const __bf16* kp = static_cast<const __bf16*>(a.k);
    const __bf16* qp = static_cast<const __bf16*>(a.q);
    const __bf16* vp = static_cast<const __bf16*>(a.v);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int v = pt + 256 * p, row = v >> 4, cg = v & 15;
        f.k[p] = f.q[p] = make_uint4(0, 0, 0, 0);
        if (row < len) {
            const long off = ((t0 + row) * a.Hqk + hq) * FD + cg * 8;
            f.k[p] = *reinterpret_cast<const uint4*>(kp + off);
            f.q[p] = *reinterpret_cast<const uint4*>(qp + off);
        }
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) f.t[p] = *reinterpret_cast<const uint4*>(Tchunk + (pt + 256 * p) * 8);
    {
        const int row = pt >> 2, cg = pt & 3;
        f.v = make_uint4(0, 0, 0, 0);
        if (row < len) f.v = *reinterpret_cast<const uint4*>(vp + ((t0 + row) * a.Hv + h) * FD + j0 + cg * 8);
    }
    f.beta = 0.f;
    f.g = 0.f;
    if (pt < FC && pt < len) {
        const long idx = (t0 + pt) * a.Hv + h;
        f.beta = a.beta[idx];
        if (a.g) f.g = a.g[idx];
    }
}

__device__ __forceinline__ void stage_chunk(ChunkBuf& cb, const Prefetch& f, int pt) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int v = pt + 256 * p, row = v >> 4, cg = v & 15;
        *reinterpret_cast<uint4*>(&cb.K[row][cg * 8]) = f.k[p];
        *reinterpret_cast<uint4*>(&cb.Q[row][cg * 8]) = f.q[p];
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int v = pt + 256 * p, row = v >> 3, cg = v & 7;
        *reinterpret_cast<uint4*>(&cb.T[row][cg * 8]) = f.t[p];
    }
    *reinterpret_cast<uint4*>(&cb.V[pt >> 2][(pt & 3) * 8]) = f.v;
    if (pt < FC) {  // one wave: inclusive scan of the log decays over the chunk
        float gv = f.g;
        for (int o = 1; o < 64; o <<= 1) {
            const float y = __shfl_up(gv, o);
            if (pt >= o) gv += y;
        }
        const float glast = __shfl(gv, 63);
        cb.gam[pt] = gv;
        cb.beta[pt] = f.beta;
        cb.eg[pt] = expf(gv);
        cb.tail[pt] = expf(glast - gv);
    }
}

__global__ __launch_bounds__(SNT) void state_kernel(PrefillArgs a, const int32_t* off, const __bf16* Tws,
                                                    long nct) {
    __shared__ StateSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q16 = lane >> 4;
    const bool chain_wave = wave < 4;
    const int w4 = wave & 3;          // index within the chain or the output group
    const int pt = tid - 256;         // output-wave thread index

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
    const __bf16* Tseq = Tws + ((size_t)gc0 * a.Hv + h) * (FC * FC);
    const size_t Tstride = (size_t)a.Hv * FC * FC;

    // Chain waves: state rows 32*w4 + 16*rt + 4*q16 + e, columns 16*ct + l16, as four
    // 16x16 accumulator tiles M[rt][ct].
    f32x4 M[2][2];
    Prefetch f;
    if (chain_wave) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int i = 32 * w4 + 16 * rt + 4 * q16, j = 16 * ct + l16;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    M[rt][ct][e] = a.h0 ? a.h0[((long)nh * FD + i + e) * FD + j0 + j] : 0.f;
                st4(&sm.MbT[j][i], M[rt][ct][0], M[rt][ct][1], M[rt][ct][2], M[rt][ct][3]);
            }
    } else {
        // P above the diagonal stays zero for the whole sequence
        for (int e = pt; e < FC * FC; e += 256) {
            const int r = e >> 6, i = e & 63;
            if (i > r) sm.P[r][i] = (__bf16)0.f;
        }
        if (nchunks > 0) {
            fetch_chunk(a, Tseq, bos, (int)min((long)FC, eos - bos), hq, h, j0, pt, f);
            stage_chunk(sm.buf[0], f, pt);
        }
        if (nchunks > 1) {
            const long t1 = bos + FC;
            fetch_chunk(a, Tseq + Tstride, t1, (int)min((long)FC, eos - t1), hq, h, j0, pt, f);
        }
    }
    __syncthreads();

    for (int c = 0; c < nchunks; ++c) {
        const long t0 = bos + (long)c * FC;
        const int len = (int)min((long)FC, eos - t0);
        ChunkBuf& cb = sm.buf[c & 1];
        bf16x8 kcol[2][2];            // chain waves: K^T operand of the state update
        f32x4 Y[2];                   // output waves: exp(gamma) Q M for rows 16*w4 + ...

        // ================= phase A =================
        {
            // X = (K or Q) M for rows 16*w4 .. +15, both 16-column tiles
            const __bf16* src = chain_wave ? &cb.K[16 * w4 + l16][0] : &cb.Q[16 * w4 + l16][0];
            bf16x8 af[4], bf0[4], bf1[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                af[kk] = ld8(src + 32 * kk + 8 * q16);
                bf0[kk] = ld8(&sm.MbT[l16][32 * kk + 8 * q16]);
                bf1[kk] = ld8(&sm.MbT[16 + l16][32 * kk + 8 * q16]);
            }
            f32x4 X0 = {0.f, 0.f, 0.f, 0.f}, X1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                X0 = mma16(af[kk], bf0[kk], X0);
                X1 = mma16(af[kk], bf1[kk], X1);
            }
            const int r = 16 * w4 + 4 * q16;
            if (chain_wave) {
                // K^T operand for phase C: A[i][k] = K[k][i], i = 32*w4 + 16*rt + l16
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            kcol[rt][kk][e] = cb.K[32 * kk + 8 * q16 + e][32 * w4 + 16 * rt + l16];
                // R = beta (V - exp(gamma) X), stored value-column-major
                float rv0[4], rv1[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float bt = cb.beta[r + e], eg = cb.eg[r + e];
                    rv0[e] = bt * ((float)cb.V[r + e][l16] - eg * X0[e]);
                    rv1[e] = bt * ((float)cb.V[r + e][16 + l16] - eg * X1[e]);
                }
                st4(&sm.RT[l16][r], rv0[0], rv0[1], rv0[2], rv0[3]);
                st4(&sm.RT[16 + l16][r], rv1[0], rv1[1], rv1[2], rv1[3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float eg = cb.eg[r + e];
                    Y[0][e] = eg * X0[e];
                    Y[1][e] = eg * X1[e];
                }
            }
        }
        if (!chain_wave) {
            // P tiles (16x16, key token i below query token r); output wave w4 does
            // tiles (ti, tr): w4=0: (0,0) (0,3) (1,3); 1: (0,1) (1,1) (2,3);
            // 2: (0,2) (1,2) (2,2); 3: (3,3)
            const int ntile = w4 == 3 ? 1 : 3;
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                if (t >= ntile) break;
                int ti, tr;
                if (w4 == 0) { ti = t == 0 ? 0 : t - 1; tr = t == 0 ? 0 : 3; }
                else if (w4 == 1) { ti = t == 2 ? 2 : t; tr = t == 2 ? 3 : 1; }
                else if (w4 == 2) { ti = t; tr = 2; }
                else { ti = 3; tr = 3; }
                bf16x8 ka[4], qb[4];
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    ka[kk] = ld8(&cb.K[16 * ti + l16][32 * kk + 8 * q16]);
                    qb[kk] = ld8(&cb.Q[16 * tr + l16][32 * kk + 8 * q16]);
                }
                f32x4 Pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) Pt = mma16(ka[kk], qb[kk], Pt);
                // element e: key token i = 16 ti + 4 q16 + e, query token r = 16 tr + l16
                const int i = 16 * ti + 4 * q16, r = 16 * tr + l16;
                const float gr = cb.gam[r];
                float pv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) pv[e] = (i + e <= r) ? expf(gr - cb.gam[i + e]) * Pt[e] : 0.f;
                st4(&sm.P[r][i], pv[0], pv[1], pv[2], pv[3]);
            }
        }
        __syncthreads();

        // ================= phase B =================
        if (chain_wave) {
            // Delta = T R for rows 16*w4 .. +15 (T is lower triangular: k < 16 (w4 + 1))
            const int nk = w4 < 2 ? 1 : 2;
            f32x4 D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= nk) break;
                const bf16x8 ta = ld8(&cb.T[16 * w4 + l16][32 * kk + 8 * q16]);
                const bf16x8 r0 = ld8(&sm.RT[l16][32 * kk + 8 * q16]);
                const bf16x8 r1 = ld8(&sm.RT[16 + l16][32 * kk + 8 * q16]);
                D0 = mma16(ta, r0, D0);
                D1 = mma16(ta, r1, D1);
            }
            const int r = 16 * w4 + 4 * q16;
            st4(&sm.DT[l16][r], D0[0], D0[1], D0[2], D0[3]);
            st4(&sm.DT[16 + l16][r], D1[0], D1[1], D1[2], D1[3]);
            const float t0v = cb.tail[r], t1v = cb.tail[r + 1], t2v = cb.tail[r + 2], t3v = cb.tail[r + 3];
            st4(&sm.DtT[l16][r], t0v * D0[0], t1v * D0[1], t2v * D0[2], t3v * D0[3]);
            st4(&sm.DtT[16 + l16][r], t0v * D1[0], t1v * D1[1], t2v * D1[2], t3v * D1[3]);
        } else if (c + 1 < nchunks) {
            // stage chunk c + 1 into the other buffer, then fetch chunk c + 2
            stage_chunk(sm.buf[(c + 1) & 1], f, pt);
            if (c + 2 < nchunks) {
                const long t2 = t0 + 2 * FC;
                fetch_chunk(a, Tseq + (size_t)(c + 2) * Tstride, t2, (int)min((long)FC, eos - t2), hq, h, j0,
                            pt, f);
            }
        }
        __syncthreads();

        // ================= phase C =================
        if (chain_wave) {
            // M <- exp(gamma_last) M + K^T Delta~   (rows past the chunk end add g = 0)
            const float Gl = cb.eg[FC - 1];
            bf16x8 db[2][2];
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) db[ct][kk] = ld8(&sm.DtT[16 * ct + l16][32 * kk + 8 * q16]);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    M[rt][ct] *= Gl;
#pragma unroll
                    for (int kk = 0; kk < 2; ++kk) M[rt][ct] = mma16(kcol[rt][kk], db[ct][kk], M[rt][ct]);
                }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    st4(&sm.MbT[16 * ct + l16][32 * w4 + 16 * rt + 4 * q16], M[rt][ct][0], M[rt][ct][1],
                        M[rt][ct][2], M[rt][ct][3]);
        } else {
            // O = Y + P Delta for query rows 16*w4 .. +15 (P is lower triangular)
            const int nk = w4 < 2 ? 1 : 2;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (kk >= nk) break;
                const bf16x8 pa = ld8(&sm.P[16 * w4 + l16][32 * kk + 8 * q16]);
                const bf16x8 d0 = ld8(&sm.DT[l16][32 * kk + 8 * q16]);
                const bf16x8 d1 = ld8(&sm.DT[16 + l16][32 * kk + 8 * q16]);
                Y[0] = mma16(pa, d0, Y[0]);
                Y[1] = mma16(pa, d1, Y[1]);
            }
            __bf16* op = static_cast<__bf16*>(a.o);
            const int r = 16 * w4 + 4 * q16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (r + e < len) {
                    __bf16* row = op + ((t0 + r + e) * a.Hv + h) * FD + j0;
                    row[l16] = (__bf16)(a.scale * Y[0][e]);
                    row[16 + l16] = (__bf16)(a.scale * Y[1][e]);
                }
            }
        }
        __syncthreads();
    }

    if (chain_wave && a.hT) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const int i = 32 * w4 + 16 * rt + 4 * q16, j = 16 * ct + l16;
#pragma unroll
                for (int e = 0; e < 4; ++e) a.hT[((long)nh * FD + i + e) * FD + j0 + j] = M[rt][ct][e];
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
    const long prep_blocks = slots * a.Hv;
    if (prep_blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (prep_blocks > 0)
        hipLaunchKernelGGL(prep_kernel, dim3((unsigned)prep_blocks), dim3(64), 0, s, a, off, Tws, nct);
    const long state_blocks = (long)a.N * a.Hv * NSL;
    if (state_blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (state_blocks > 0)
        hipLaunchKernelGGL(state_kernel, dim3((unsigned)state_blocks), dim3(SNT), 0, s, a, off, Tws, nct);
    return hipGetLastError();
}

}  // namespace dn
