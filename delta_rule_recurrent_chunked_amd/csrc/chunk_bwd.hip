// chunk_bwd.hip -- reverse pass of the chunked form of the gated delta rule on the gfx950
// matrix cores (bf16 operands, fp32 accumulation), for bf16 inputs with Dk = Dv = 128,
// 64-token chunks and one log decay per head (or none).
//
// The forward rule is the update of the frankenstein "DeltaNet Attention" page (module
// docstring) with the gate order of the nnterp "linear_attention" page (LinearAttention
// class text), in its chunked form: per chunk, with M the state at its start (key-major),
// gamma the in-chunk inclusive sum of g, D_ri = exp(gamma_r - gamma_i) (i <= r),
// tail_r = exp(gamma_L - gamma_r):
//
//   A = strict_lower(diag(beta) (D o K K^T)),  T = (I + A)^-1,  P = lower(D o Q K^T)
//   X = K M,  R = diag(beta) (V - diag(exp(gamma)) X),  Delta = T R
//   O = scale (diag(exp(gamma)) Q M + P Delta),  M' = exp(gamma_L) M + K^T diag(tail) Delta
//
// Given dO and dM' (the gradient of the state after the chunk), the chain rule gives
//
//   dDelta = scale P^T dO + diag(tail) K dM',   dR = T^T dDelta,   dV = diag(beta) dR
//   dX = -diag(beta exp(gamma)) dR
//   dM = exp(gamma_L) dM' + scale Q^T diag(exp(gamma)) dO + K^T dX       (the carry)
//   dA = -strict_lower(dR Delta^T),  dP = scale lower(dO Delta^T),  W = dA o diag(beta) D,
//   Z = dP o D
//   dQ = scale diag(exp(gamma)) dO M^T + Z K
//   dK = dX M^T + diag(tail) Delta dM'^T + (W + W^T) K + Z^T Q
//   dbeta_r = (V - diag(exp(gamma)) X)_r . dR_r + sum_i dA_ri (D o K K^T)_ri
//   dgamma_r = scale exp(gamma_r) (Q M)_r . dO_r - beta_r exp(gamma_r) X_r . dR_r
//              + rowsum_r(dA o A) - colsum_r(dA o A) + rowsum_r(dP o P) - colsum_r(dP o P)
//              - c_r,   c_r = tail_r (K dM')_r . Delta_r,
//   and on the chunk's last row + exp(gamma_L) <M, dM'> + sum_r c_r;
//   dg_i = sum of dgamma_r over the rows r >= i of the chunk.
//
// Every product contracting over the value columns is linear in them, so the pass splits
// the state's columns into 32-column slices like the forward: one workgroup of eight waves
// per (sequence, value head, slice) walks the chunks backwards from the chunk-start states
// the forward kernel saved, carries its columns of dM in MFMA accumulators, writes dV and
// the initial state's gradient directly, and writes its share of dQ, dK, dbeta and dgamma
// per (chunk, row) to the workspace; bwd_chunk_sum_kernel adds the shares over the slices
// (and over the value heads of a q/k head) in a fixed order and sums dgamma into dg.
//
// Each chunk takes ten steps separated by workgroup barriers; a step's output tiles are
// dealt to the waves.  Operands live in LDS as bf16, row-major: a "row" fragment (lane =
// row of the stored matrix) is one 16-byte read, a "column" fragment (lane = column) two
// transposed 8-byte reads (ds_read_b64_tr_b16).  The next chunk's inputs are fetched into
// registers while the current one is worked.
#include "internal.h"
#include "mfma_ops.h"

namespace dn {
namespace {

constexpr int BC = 64;             // chunk
constexpr int BD = 128;            // Dk = Dv
constexpr int BS = 32;             // state columns per workgroup
constexpr int BNS = BD / BS;       // slices
constexpr int NTB = 512;           // threads (8 waves)
constexpr int P128 = BD + 16;      // bf16 pitches (16-byte reads of 16 rows conflict-free)
constexpr int P64 = BC + 16;
constexpr int P32 = BS + 16;
constexpr int ADP = 136;           // A's diagonal 16x16 blocks, 120 packed fp16 entries + spare
constexpr int NDB = 8;             // dbeta partial slots per row
constexpr int NDG = 48;            // dgamma partial slots per row
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct alignas(16) BwdSmem {
    __bf16 K[BC][P128], Q[BC][P128];
    __bf16 V[BC][P32], dO[BC][P32], R[BC][P32], Dl[BC][P32], dDl[BC][P32], dR[BC][P32];
    __bf16 M[BD][P32];             // the slice of the state at the chunk start
    __bf16 dM[BD][P32];            // the slice of dM' (the gradient of the state after the chunk)
    __bf16 Tt[BC][P64];            // T^T, T = (I + A)^-1 lower triangular
    __bf16 P[BC][P64];             // P, then Z = dP o D
    __bf16 G[BC][P64];             // D o K K^T (strictly lower), then W = dA o diag(beta) D
    _Float16 Ad[4][ADP];           // A's diagonal blocks (strictly lower, packed by rows)
    float X[BC][BS];               // X = K M (fp32, for the dbeta and dgamma terms)
    float beta[BC], gam[BC], eg[BC], tail[BC];
    float pb[BC][NDB], pg[BC][NDG];   // per-row partial sums (fixed slots, summed in order)
    float mdm[8];                  // <M, dM'> per wave
};

// --------------------------------------------------------------------- fragments
__device__ __forceinline__ bf16x8 frag_r(const __bf16* S, int pitch, int r0, int k0, int l16, int q16) {
    return ld8(S + (r0 + l16) * pitch + k0 + 8 * q16);
}
__device__ __forceinline__ bf16x8 frag_c(const __bf16* S, int pitch, int c0, int k0, int l16, int q16) {
    const __bf16* p = S + (k0 + 8 * q16 + (l16 >> 2)) * pitch + c0 + 4 * (l16 & 3);
    return cat(trld(p), trld(p + 4 * pitch));
}
__device__ __forceinline__ bf16x8 scale_r(bf16x8 x, float f) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (__bf16)((float)x[e] * f);
    return x;
}
// an accumulator tile C[16 i + 4 q16 + e][16 j + l16] to a bf16 row-major matrix
__device__ __forceinline__ void put_tile(__bf16* S, int pitch, int i, int j, const f32x4& c, int l16, int q16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) S[(16 * i + 4 * q16 + e) * pitch + 16 * j + l16] = (__bf16)c[e];
}
// DPP lane moves within rows of 16 lanes (every lane has a source)
template <int CTRL>
__device__ __forceinline__ float dpp16(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// sum over the 16 lanes of one q16 group (the tile's columns) of each of the lane's 4 rows:
// lane ^ 1, lane ^ 2 (quad permutes), then the 8- and 16-lane mirrors, in every lane
__device__ __forceinline__ f32x4 row_sum16(f32x4 v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float x = v[e];
        x += dpp16<0xB1>(x);
        x += dpp16<0x4E>(x);
        x += dpp16<0x141>(x);
        x += dpp16<0x140>(x);
        v[e] = x;
    }
    return v;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ float ld32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// One chunk's inputs in registers: thread t holds 16-byte pieces t and t + 512 of K and Q
// (row = piece / 16), piece t & 255 of V (t < 256) or dO (t >= 256) (row = piece / 4),
// pieces t and t + 512 of the state slice (128 rows x 8 float4), beta and g of token t (t < 64).
struct BwdIn {
    uint4 k[2], q[2], vo;
    float4 m[2];
    float beta, g;
};

template <bool GATED>
__global__ __launch_bounds__(NTB, 1) void chunk_bwd_kernel(ChunkBwdArgs a) {
    __shared__ BwdSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q16 = lane >> 4;
    const int slice = blockIdx.x % BNS;
    const int nh = blockIdx.x / BNS;
    const int h = nh % a.Hv, n = nh / a.Hv;
    const int hq = h / (a.Hv / a.Hqk);
    const int j0 = slice * BS;
    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);
    const long L = eos - bos;
    const int nc = (int)((L + BC - 1) / BC);
    const long cid0 = chunk_id_base(a, n);
    const float sc = a.scale;

    // streams over this sequence (range-checked: rows past its end read zeros)
    const uint32_t kq_tok = (uint32_t)a.Hqk * BD * 2, v_tok = (uint32_t)a.Hv * BD * 2, s_tok = (uint32_t)a.Hv * 4;
    const long kq0 = (bos * a.Hqk + hq) * BD, v0 = (bos * a.Hv + h) * BD + j0, s0 = bos * a.Hv + h;
    const uint32_t kq_end = L > 0 ? (uint32_t)((L - 1) * kq_tok + BD * 2) : 0;
    const uint32_t v_end = L > 0 ? (uint32_t)((L - 1) * v_tok + BS * 2) : 0;
    const uint32_t s_end = L > 0 ? (uint32_t)((L - 1) * s_tok + 4) : 0;
    const auto k_rs = rsrc(static_cast<const __bf16*>(a.k) + kq0, kq_end);
    const auto q_rs = rsrc(static_cast<const __bf16*>(a.q) + kq0, kq_end);
    const auto v_rs = rsrc(static_cast<const __bf16*>(a.v) + v0, v_end);
    const auto o_rs = rsrc(static_cast<const __bf16*>(a.dout) + v0, v_end);
    const auto b_rs = rsrc(a.beta + s0, s_end);
    const auto g_rs = rsrc(a.g ? a.g + s0 : a.beta + s0, a.g ? s_end : 0);
    uint32_t kq_off[2], m_off[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int pc = tid + NTB * u;
        kq_off[u] = (uint32_t)(pc >> 4) * kq_tok + (pc & 15) * 16;
        m_off[u] = (uint32_t)((pc >> 3) * BD + (pc & 7) * 4);   // floats within the head's state
    }
    const int vp = tid & 255;
    const uint32_t vo_off = (uint32_t)(vp >> 2) * v_tok + (vp & 3) * 16;
    const uint32_t sc_off = (uint32_t)(tid & 63) * s_tok;

    auto fetch = [&](int c, BwdIn& f) {
        const uint32_t ck = (uint32_t)c * BC * kq_tok, cv = (uint32_t)c * BC * v_tok, cs = (uint32_t)c * BC * s_tok;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f.k[u] = ld128(k_rs, kq_off[u], ck);
            f.q[u] = ld128(q_rs, kq_off[u], ck);
        }
        f.vo = ld128(tid < 256 ? v_rs : o_rs, vo_off, cv);
        const float* st = a.states + ((cid0 + c) * a.Hv + h) * (long)BD * BD + j0;
#pragma unroll
        for (int u = 0; u < 2; ++u) f.m[u] = *reinterpret_cast<const float4*>(st + m_off[u]);
        f.beta = ld32(b_rs, sc_off, cs);
        f.g = ld32(g_rs, sc_off, cs);
    };

    // dM' of this slice in MFMA accumulators: wave w holds tiles (key block 2 (w >> 1) + u,
    // column block w & 1), u = 0, 1: keys 16 (2 (w >> 1) + u) + 4 q16 + e, column 16 (w & 1) + l16
    f32x4 dm[2];
    const int dmj = wave & 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int ki = 2 * (wave >> 1) + u;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dm[u][e] = a.dfinal ? a.dfinal[((long)nh * BD + 16 * ki + 4 * q16 + e) * BD + j0 + 16 * dmj + l16] : 0.f;
    }
    auto put_dm = [&]() {
#pragma unroll
        for (int u = 0; u < 2; ++u) put_tile(&sm.dM[0][0], P32, 2 * (wave >> 1) + u, dmj, dm[u], l16, q16);
    };
    put_dm();

    // P and G (later Z and W) are written below their 16-block diagonal only, T^T above
    // it; the products that read them by 32-row blocks also read the other tiles, zero
    for (int i = tid; i < BC * P64; i += NTB) {
        (&sm.P[0][0])[i] = (__bf16)0.f;
        (&sm.G[0][0])[i] = (__bf16)0.f;
        (&sm.Tt[0][0])[i] = (__bf16)0.f;   // T's blocks above the diagonal stay zero
    }

    BwdIn cur, nxt;
    if (nc > 0) fetch(nc - 1, cur);
    for (int c = nc - 1; c >= 0; --c) {
        // -------------------------------------------------------- B0: inputs to LDS
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pc = tid + NTB * u, row = pc >> 4, cg = pc & 15;
            *reinterpret_cast<uint4*>(&sm.K[row][cg * 8]) = cur.k[u];
            *reinterpret_cast<uint4*>(&sm.Q[row][cg * 8]) = cur.q[u];
            const int mr = pc >> 3, mc = (pc & 7) * 4;
            *reinterpret_cast<uint2*>(&sm.M[mr][mc]) =
                make_uint2(pack_bf16x2(cur.m[u].x, cur.m[u].y), pack_bf16x2(cur.m[u].z, cur.m[u].w));
        }
        *reinterpret_cast<uint4*>(tid < 256 ? &sm.V[vp >> 2][(vp & 3) * 8] : &sm.dO[vp >> 2][(vp & 3) * 8]) = cur.vo;
        for (int i = tid; i < BC * NDB; i += NTB) (&sm.pb[0][0])[i] = 0.f;
        for (int i = tid; i < BC * NDG; i += NTB) (&sm.pg[0][0])[i] = 0.f;
        if (wave == 0) {
            // gamma: inclusive scan of g over the chunk (rows past the end carry g = 0)
            float gv = GATED ? cur.g : 0.f;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(gv, off);
                if (lane >= off) gv += o;
            }
            const float gl = __shfl(gv, 63);
            sm.beta[lane] = cur.beta;
            sm.gam[lane] = gv;
            sm.eg[lane] = __expf(gv);
            sm.tail[lane] = __expf(gl - gv);
        }
        if (c > 0) fetch(c - 1, nxt);
        __syncthreads();

        // ------------------------------------------ B1: D o K K^T, P = D o Q K^T, Ad
        // 20 lower tiles (incl. the diagonal): t < 10 of G, t >= 10 of P; tile (ri, ci)
        // of rows 16 ri + 4 q16 + e, columns 16 ci + l16, ci <= ri
        for (int t = wave; t < 20; t += 8) {
            const int u = t % 10;
            const int ri = u < 1 ? 0 : u < 3 ? 1 : u < 6 ? 2 : 3;
            const int ci = u - ri * (ri + 1) / 2;
            const __bf16* A = t < 10 ? &sm.K[0][0] : &sm.Q[0][0];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BD; k0 += 32)
                acc = mma16(frag_r(A, P128, 16 * ri, k0, l16, q16), frag_r(&sm.K[0][0], P128, 16 * ci, k0, l16, q16), acc);
            const int col = 16 * ci + l16;
            const float gc = sm.gam[col];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * ri + 4 * q16 + e;
                const bool keep = t < 10 ? col < row : col <= row;
                const float d = GATED ? __expf(fminf(sm.gam[row] - gc, 0.f)) : 1.f;
                acc[e] = keep ? d * acc[e] : 0.f;
            }
            put_tile(t < 10 ? &sm.G[0][0] : &sm.P[0][0], P64, ri, ci, acc, l16, q16);
            if (t < 10 && ri == ci) {   // A's diagonal block ri in fp16, strictly lower, packed
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int lr = 4 * q16 + e, lc = l16;
                    if (lc < lr) sm.Ad[ri][lr * (lr - 1) / 2 + lc] = (_Float16)(sm.beta[16 * ri + lr] * acc[e]);
                }
            }
        }
        __syncthreads();

        // ------------------------- B2: T (wave 0); X = K M, R (waves 1-4); Y = Q M (5-7)
        if (wave == 0) {
            __bf16 (*Tt)[P64] = sm.Tt;
            {   // the four 16x16 diagonal blocks by forward substitution (lane = block, column):
                // column cc of T_bb is row cc of T^T_bb, written as two 16-byte pieces
                const int b = q16, cc = l16;
                f16x8 ap[15];
#pragma unroll
                for (int g = 0; g < 15; ++g) ap[g] = *reinterpret_cast<const f16x8*>(&sm.Ad[b][8 * g]);
                float x[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = r == cc ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < 15; ++m)
#pragma unroll
                    for (int r = m + 1; r < 16; ++r) {
                        const int idx = r * (r - 1) / 2 + m;
                        x[r] = __builtin_fmaf(-(float)ap[idx >> 3][idx & 7], x[m], x[r]);
                    }
                bf16x8 lo8, hi8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    lo8[e] = (__bf16)x[e];
                    hi8[e] = (__bf16)x[8 + e];
                }
                *reinterpret_cast<bf16x8*>(&Tt[16 * b + cc][16 * b]) = lo8;
                *reinterpret_cast<bf16x8*>(&Tt[16 * b + cc][16 * b + 8]) = hi8;
            }
            wave_lds_order();
            const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
            const bool lo = q16 < 2;   // k = 16 padded to the instruction's 32
            // level 1: T21 = -T22 (A21 T11) within each 32x32 diagonal block (base 0, 32);
            // T's block (b + 1, b) is T^T's block (b, b + 1)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int base = 32 * hb;
                const bf16x8 af = lo ? scale_r(frag_r(&sm.G[0][0], P64, base + 16, base, l16, q16),
                                               sm.beta[base + 16 + l16]) : zero8();
                const bf16x8 bf = lo ? frag_r(&Tt[0][0], P64, base, base, l16, q16) : zero8();
                const f32x4 X1 = mma16(af, bf, z4);
                const bf16x8 tf = lo ? frag_c(&Tt[0][0], P64, base + 16, base + 16, l16, q16) : zero8();
                const f32x4 Y1 = mma16(tf, acc_to_b(X1, z4), z4);
                st4(&Tt[base + l16][base + 16 + 4 * q16], -Y1[0], -Y1[1], -Y1[2], -Y1[3]);
            }
            wave_lds_order();
            // level 2: T_BL = -T_BR (A_BL T_TL), 32 x 32 blocks
            f32x4 X2[2][2];
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj)
                    X2[ti][tj] = mma16(scale_r(frag_r(&sm.G[0][0], P64, 32 + 16 * ti, 0, l16, q16), sm.beta[32 + 16 * ti + l16]),
                                       frag_r(&Tt[0][0], P64, 16 * tj, 0, l16, q16), z4);
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) {
                    const f32x4 Y2 = mma16(frag_c(&Tt[0][0], P64, 32 + 16 * ti, 32, l16, q16),
                                           acc_to_b(X2[0][tj], X2[1][tj]), z4);
                    st4(&Tt[16 * tj + l16][32 + 16 * ti + 4 * q16], -Y2[0], -Y2[1], -Y2[2], -Y2[3]);
                }
        } else {
            // X tiles (i, j) on waves 1-4 (two each), Y tiles on waves 5-7
            const bool isx = wave <= 4;
            const int first = isx ? 2 * (wave - 1) : 3 * (wave - 5);
            const int count = isx ? 2 : (wave == 7 ? 2 : 3);
            for (int t = first; t < first + count && (isx || GATED); ++t) {
                const int i = t >> 1, j = t & 1;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < BD; k0 += 32)
                    acc = mma16(frag_r(isx ? &sm.K[0][0] : &sm.Q[0][0], P128, 16 * i, k0, l16, q16),
                                frag_c(&sm.M[0][0], P32, 16 * j, k0, l16, q16), acc);
                const int col = 16 * j + l16;
                if (isx) {
                    f32x4 r4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = 16 * i + 4 * q16 + e;
                        sm.X[row][col] = acc[e];
                        r4[e] = sm.beta[row] * ((float)sm.V[row][col] - sm.eg[row] * acc[e]);
                    }
                    put_tile(&sm.R[0][0], P32, i, j, r4, l16, q16);
                } else {   // scale exp(gamma_r) (Q M)_r . dO_r, this tile's 16 columns
                    f32x4 p;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int row = 16 * i + 4 * q16 + e;
                        p[e] = acc[e] * (float)sm.dO[row][col];
                    }
                    p = row_sum16(p);
                    if (l16 == 0) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int row = 16 * i + 4 * q16 + e;
                            sm.pg[row][0 + j] = sc * sm.eg[row] * p[e];
                        }
                    }
                }
            }
        }
        __syncthreads();

        // each wave owns one 64 x 32 tile (i, j) in the next steps
        const int ti = wave >> 1, tj = wave & 1;
        // ---------------------------------------------------------- B3: Delta = T R
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32)
                if (k0 <= 16 * ti) acc = mma16(frag_c(&sm.Tt[0][0], P64, 16 * ti, k0, l16, q16),
                                               frag_c(&sm.R[0][0], P32, 16 * tj, k0, l16, q16), acc);
            put_tile(&sm.Dl[0][0], P32, ti, tj, acc, l16, q16);
        }
        __syncthreads();

        // ------------------------------ B4: dDelta = scale P^T dO + diag(tail) K dM'; c_r
        {
            f32x4 pd = {0.f, 0.f, 0.f, 0.f}, kd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32)
                if (k0 + 32 > 16 * ti) pd = mma16(frag_c(&sm.P[0][0], P64, 16 * ti, k0, l16, q16),
                                                  frag_c(&sm.dO[0][0], P32, 16 * tj, k0, l16, q16), pd);
#pragma unroll
            for (int k0 = 0; k0 < BD; k0 += 32)
                kd = mma16(frag_r(&sm.K[0][0], P128, 16 * ti, k0, l16, q16), frag_c(&sm.dM[0][0], P32, 16 * tj, k0, l16, q16), kd);
            f32x4 dd, cr;
            const int col = 16 * tj + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * ti + 4 * q16 + e;
                const float tk = sm.tail[row] * kd[e];
                dd[e] = sc * pd[e] + tk;
                cr[e] = -tk * (float)sm.Dl[row][col];   // -c_r (this tile's columns)
            }
            put_tile(&sm.dDl[0][0], P32, ti, tj, dd, l16, q16);
            if (GATED) {
                cr = row_sum16(cr);
                if (l16 == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sm.pg[16 * ti + 4 * q16 + e][44 + tj] = cr[e];
                }
            }
        }
        __syncthreads();

        // ------------------------------------------- B5: dR = T^T dDelta; dV; row terms
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32)
                if (k0 + 32 > 16 * ti) acc = mma16(frag_r(&sm.Tt[0][0], P64, 16 * ti, k0, l16, q16),
                                                   frag_c(&sm.dDl[0][0], P32, 16 * tj, k0, l16, q16), acc);
            put_tile(&sm.dR[0][0], P32, ti, tj, acc, l16, q16);
            const int col = 16 * tj + l16;
            f32x4 rb, xg;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * ti + 4 * q16 + e;
                const float x = sm.X[row][col];
                rb[e] = ((float)sm.V[row][col] - sm.eg[row] * x) * acc[e];   // (V - e^gamma X) . dR
                xg[e] = x * acc[e];                                            // X . dR
                const long tok = (long)c * BC + row;
                if (tok < L) a.dv[((bos + tok) * a.Hv + h) * BD + j0 + col] = sm.beta[row] * acc[e];
            }
            rb = row_sum16(rb);
            xg = row_sum16(xg);
            if (l16 == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * ti + 4 * q16 + e;
                    sm.pb[row][tj] = rb[e];
                    sm.pg[row][2 + tj] = -sm.beta[row] * sm.eg[row] * xg[e];
                }
            }
        }
        __syncthreads();

        // ------------------------------------------ B6: dA -> W, dP -> Z; <M, dM'>
        // 20 lower tiles (incl. the diagonal): t < 10 of dA = -dR Delta^T, t >= 10 of
        // dP = scale dO Delta^T; k = the 32 slice columns
        for (int t = wave; t < 20; t += 8) {
            const int u = t % 10;
            const int ri = u < 1 ? 0 : u < 3 ? 1 : u < 6 ? 2 : 3;
            const int ci = u - ri * (ri + 1) / 2;
            const bool isa = t < 10;
            f32x4 d = mma16(frag_r(isa ? &sm.dR[0][0] : &sm.dO[0][0], P32, 16 * ri, 0, l16, q16),
                            frag_r(&sm.Dl[0][0], P32, 16 * ci, 0, l16, q16), f32x4{0.f, 0.f, 0.f, 0.f});
            __bf16* S = isa ? &sm.G[0][0] : &sm.P[0][0];
            const int col = 16 * ci + l16;
            const float gc = sm.gam[col];
            f32x4 rs, cs4, bsum;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * ri + 4 * q16 + e;
                const bool keep = isa ? col < row : col <= row;
                const float dv = keep ? (isa ? -d[e] : sc * d[e]) : 0.f;
                const float s = (float)S[row * P64 + col];   // D o K K^T, or P
                const float dec = GATED ? __expf(fminf(sm.gam[row] - gc, 0.f)) : 1.f;
                const float f = isa ? sm.beta[row] : 1.f;
                rs[e] = dv * f * s;          // dA o A (A = beta G) or dP o P
                cs4[e] = rs[e];
                bsum[e] = dv * s;            // dA o G (the dbeta term)
                S[row * P64 + col] = (__bf16)(keep ? dv * f * dec : 0.f);   // W or Z
            }
            const f32x4 r16 = row_sum16(rs);
            const float c4 = cs4[0] + cs4[1] + cs4[2] + cs4[3];   // this lane's 4 rows of the column
            if (isa) {
                const f32x4 b16 = row_sum16(bsum);
                if (l16 == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sm.pb[16 * ri + 4 * q16 + e][2 + ci] = b16[e];
                }
            }
            if (GATED) {
                if (l16 == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sm.pg[16 * ri + 4 * q16 + e][(isa ? 4 : 24) + ci] = r16[e];
                }
                sm.pg[col][(isa ? 8 : 28) + 4 * ri + q16] = -c4;
            }
        }
        if (GATED) {   // <M, dM'> over this wave's two dM' tiles
            float s = 0.f;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ki = 2 * (wave >> 1) + u;
#pragma unroll
                for (int e = 0; e < 4; ++e) s += (float)sm.M[16 * ki + 4 * q16 + e][16 * dmj + l16] * dm[u][e];
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) s += __shfl_xor(s, off);
            if (lane == 0) sm.mdm[wave] = s;
        }
        __syncthreads();

        // --------------------------------------------------- B7: dQ and dK shares
        {
            const long ws_row = ((long)(slice * a.ncid + cid0 + c) * a.Hv + h) * BC;
            float* wq = a.ws_dq + ws_row * BD;
            float* wk = a.ws_dk + ws_row * BD;
#pragma unroll 1
            for (int t4 = 0; t4 < 4; ++t4) {
                const int t = wave + 8 * t4;   // tile (i, j) of the 64 x 128 output
                const int i = t >> 3, j = t & 7;
                // dQ = scale diag(e^gamma) dO M^T + Z K
                f32x4 qa = mma16(frag_r(&sm.dO[0][0], P32, 16 * i, 0, l16, q16), frag_r(&sm.M[0][0], P32, 16 * j, 0, l16, q16),
                                 f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
                for (int e = 0; e < 4; ++e) qa[e] *= sc * sm.eg[16 * i + 4 * q16 + e];
#pragma unroll
                for (int k0 = 0; k0 < BC; k0 += 32)
                    if (k0 <= 16 * i) qa = mma16(frag_r(&sm.P[0][0], P64, 16 * i, k0, l16, q16),
                                                 frag_c(&sm.K[0][0], P128, 16 * j, k0, l16, q16), qa);
                // dK = -diag(beta e^gamma) dR M^T + diag(tail) Delta dM'^T + (W + W^T) K + Z^T Q
                f32x4 k1 = mma16(frag_r(&sm.dR[0][0], P32, 16 * i, 0, l16, q16), frag_r(&sm.M[0][0], P32, 16 * j, 0, l16, q16),
                                 f32x4{0.f, 0.f, 0.f, 0.f});
                f32x4 k2 = mma16(frag_r(&sm.Dl[0][0], P32, 16 * i, 0, l16, q16), frag_r(&sm.dM[0][0], P32, 16 * j, 0, l16, q16),
                                 f32x4{0.f, 0.f, 0.f, 0.f});
                f32x4 ka;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * i + 4 * q16 + e;
                    ka[e] = -sm.beta[row] * sm.eg[row] * k1[e] + sm.tail[row] * k2[e];
                }
#pragma unroll
                for (int k0 = 0; k0 < BC; k0 += 32) {
                    if (k0 <= 16 * i)   // W K (W strictly lower)
                        ka = mma16(frag_r(&sm.G[0][0], P64, 16 * i, k0, l16, q16), frag_c(&sm.K[0][0], P128, 16 * j, k0, l16, q16), ka);
                    if (k0 + 32 > 16 * i) {   // W^T K and Z^T Q (upper triangular factors)
                        ka = mma16(frag_c(&sm.G[0][0], P64, 16 * i, k0, l16, q16), frag_c(&sm.K[0][0], P128, 16 * j, k0, l16, q16), ka);
                        ka = mma16(frag_c(&sm.P[0][0], P64, 16 * i, k0, l16, q16), frag_c(&sm.Q[0][0], P128, 16 * j, k0, l16, q16), ka);
                    }
                }
                // in the accumulator layout: tile t's 64 lanes x 4 entries, 1 KiB per tile
                *reinterpret_cast<f32x4*>(wq + 256 * t + 4 * lane) = qa;
                *reinterpret_cast<f32x4*>(wk + 256 * t + 4 * lane) = ka;
            }
        }
        __syncthreads();   // the dM', M and Delta tiles are read above; dM' is replaced below

        // ------------------- B8: dM' <- e^gamma_L dM' + scale Q^T diag(e^gamma) dO + K^T dX
        {
            const float gl = sm.eg[BC - 1];   // dX is not stored: dR's tokens are scaled as read
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ki = 2 * (wave >> 1) + u;
                f32x4 acc = dm[u] * gl;
#pragma unroll
                for (int k0 = 0; k0 < BC; k0 += 32) {
                    bf16x8 od = frag_c(&sm.dO[0][0], P32, 16 * dmj, k0, l16, q16);
                    bf16x8 rd = frag_c(&sm.dR[0][0], P32, 16 * dmj, k0, l16, q16);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int tok = k0 + 8 * q16 + e;
                        od[e] = (__bf16)((float)od[e] * sc * sm.eg[tok]);
                        rd[e] = (__bf16)(-(float)rd[e] * sm.beta[tok] * sm.eg[tok]);
                    }
                    acc = mma16(frag_c(&sm.Q[0][0], P128, 16 * ki, k0, l16, q16), od, acc);
                    acc = mma16(frag_c(&sm.K[0][0], P128, 16 * ki, k0, l16, q16), rd, acc);
                }
                dm[u] = acc;
            }
            put_dm();
        }
        // this chunk's dbeta and dgamma shares (the partial slots were written before the
        // last two barriers), on wave 7: lane = row
        if (wave == 7) {
            const long ws_row = ((long)(slice * a.ncid + cid0 + c) * a.Hv + h) * BC + lane;
            float b = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < 6; ++s2) b += sm.pb[lane][s2];
            a.ws_db[ws_row] = b;
            if (GATED) {
                float gsum = 0.f;
#pragma unroll
                for (int s2 = 0; s2 < 46; ++s2) gsum += sm.pg[lane][s2];
                // gamma_L, on the last row: e^gamma_L <M, dM'> + sum_r c_r (slots 44, 45 hold -c_r)
                float ct = -(sm.pg[lane][44] + sm.pg[lane][45]);
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) ct += __shfl_xor(ct, off);
                if (lane == BC - 1) {
                    float m = 0.f;
#pragma unroll
                    for (int w = 0; w < 8; ++w) m += sm.mdm[w];
                    gsum += sm.eg[BC - 1] * m + ct;
                }
                a.ws_dg[ws_row] = gsum;
            }
        }
        __syncthreads();
        cur = nxt;
    }
    // the initial state's gradient: dM' after the first chunk
    if (a.dh0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ki = 2 * (wave >> 1) + u;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                a.dh0[((long)nh * BD + 16 * ki + 4 * q16 + e) * BD + j0 + 16 * dmj + l16] = dm[u][e];
        }
    }
}

// The slices' shares added in a fixed order, one workgroup per (chunk number, q/k head):
// dq and dk summed over the slices and over the value heads of the q/k head (the shares sit
// in the accumulator layout: tile t = 8 i + j of 16 x 16, lane l, entry e is row
// 16 i + 4 (l >> 4) + e, key 16 j + (l & 15)); per value head of the group, dbeta summed over
// the slices and dg_t = the sum of dgamma_r over the rows r >= t of the chunk (a suffix scan
// on one wave, lane = row).
__global__ __launch_bounds__(256) void bwd_chunk_sum_kernel(ChunkBwdArgs a) {
    const int hq = (int)(blockIdx.x % a.Hqk);
    const long cid = blockIdx.x / a.Hqk;
    int n;
    if (a.cu) {   // the last sequence whose first chunk number is <= cid (strictly increasing)
        int lo = 0, hi = a.N - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (chunk_id_base(a, mid) <= cid) lo = mid; else hi = mid - 1;
        }
        n = lo;
    } else {
        n = (int)(cid / ((a.T + BC - 1) / BC));
    }
    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);
    const long c = cid - chunk_id_base(a, n);
    if (c * BC >= eos - bos) return;   // a number no chunk uses
    const int rows = (int)min((long)BC, eos - bos - c * BC);
    const long tok0 = bos + c * BC;
    const int grp = a.Hv / a.Hqk;
    const long sstride = a.ncid * a.Hv * BC;   // rows between slices
    const int tid = threadIdx.x;
    for (int p = tid; p < BC * BD / 4; p += 256) {
        const int t = p >> 6, ln = p & 63;
        const int i = t >> 3, j = t & 7, l16 = ln & 15, q16 = ln >> 4;
        f32x4 sq = {0.f, 0.f, 0.f, 0.f}, sk = {0.f, 0.f, 0.f, 0.f};
        for (int sl = 0; sl < BNS; ++sl)
            for (int g = 0; g < grp; ++g) {
                const long r = (sl * sstride + (cid * a.Hv + (long)hq * grp + g) * BC) * BD + 4 * p;
                sq += *reinterpret_cast<const f32x4*>(a.ws_dq + r);
                sk += *reinterpret_cast<const f32x4*>(a.ws_dk + r);
            }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * i + 4 * q16 + e;
            if (row < rows) {
                const long o = ((tok0 + row) * a.Hqk + hq) * BD + 16 * j + l16;
                a.dq[o] = sq[e];
                a.dk[o] = sk[e];
            }
        }
    }
    const int lane = tid & 63;
    for (int g = tid >> 6; g < grp; g += 4) {
        const int h = hq * grp + g;
        float sb = 0.f, sg = 0.f;
        for (int sl = 0; sl < BNS; ++sl) {
            const long r = sl * sstride + (cid * a.Hv + h) * BC + lane;
            sb += a.ws_db[r];
            if (a.dg) sg += a.ws_dg[r];
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float o = __shfl_down(sg, off);
            if (lane + off < 64) sg += o;
        }
        if (lane < rows) {
            a.dbeta[(tok0 + lane) * a.Hv + h] = sb;
            if (a.dg) a.dg[(tok0 + lane) * a.Hv + h] = sg;
        }
    }
}

}  // namespace

bool chunk_bwd_supported(const PrefillArgs& a) {
    const long span = ((long)a.T + 2 * BC) * (a.Hqk > a.Hv ? a.Hqk : a.Hv) * BD * 2;
    return a.bf16 && a.Dk == BD && a.Dv == BD && a.C == BC && !a.g_per_key && !a.qk_norm && span < (1L << 31);
}

size_t chunk_bwd_workspace_bytes(const PrefillArgs& a, long ncid_l) {
    const size_t ncid = (size_t)ncid_l;
    const size_t states = ncid * a.Hv * BD * BD;
    const size_t shares = (size_t)BNS * ncid * a.Hv * BC * (2 * BD + 2);
    return (states + shares) * sizeof(float);
}

hipError_t launch_chunk_bwd(const ChunkBwdArgs& a0, hipStream_t s) {
    ChunkBwdArgs a = a0;
    a.ncid = chunk_id_bound(a);
    const size_t ncid = (size_t)a.ncid;
    float* ws = static_cast<float*>(a.ws);
    a.states = ws;
    a.ws_dq = ws + ncid * a.Hv * BD * BD;
    a.ws_dk = a.ws_dq + (size_t)BNS * ncid * a.Hv * BC * BD;
    a.ws_db = a.ws_dk + (size_t)BNS * ncid * a.Hv * BC * BD;
    a.ws_dg = a.ws_db + (size_t)BNS * ncid * a.Hv * BC;
    // 1. the state at every chunk start (the forward kernel, outputs skipped)
    PrefillArgs f = a;
    f.ws = a.states;
    f.hT = nullptr;
    hipError_t e = launch_prefill_fused_states(f, s);
    if (e != hipSuccess) return e;
    // 2. the reverse pass per (sequence, value head, slice)
    const long blocks = (long)a.N * a.Hv * BNS;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (blocks > 0) {
        if (a.g) hipLaunchKernelGGL(chunk_bwd_kernel<true>, dim3((unsigned)blocks), dim3(NTB), 0, s, a);
        else hipLaunchKernelGGL(chunk_bwd_kernel<false>, dim3((unsigned)blocks), dim3(NTB), 0, s, a);
    }
    // 3. the slices' shares added
    const long sum_blocks = a.ncid * a.Hqk;
    if (sum_blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (sum_blocks > 0) hipLaunchKernelGGL(bwd_chunk_sum_kernel, dim3((unsigned)sum_blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dn
