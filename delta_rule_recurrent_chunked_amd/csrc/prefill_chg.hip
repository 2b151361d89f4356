// prefill_chg.hip -- the chunked form with one log decay per key channel (the nnterp
// "linear_attention" page's ChannelGates, the Kimi Delta Attention variant) on the
// matrix cores, for bf16 q/k/v/o with Dk = 128, Dv a multiple of 32 and 64-token chunks.
//
// Key channel x of the state keeps exp(g_t[x]) at token t.  Inside one chunk, with
// G_r[x] the sum of g over the chunk up to and including token r, the token-by-token
// rule (decay, take up the pair, read) becomes, with M0 the chunk's start state:
//
//   A_ri = beta_r sum_x k_r[x] k_i[x] exp(G_r[x] - G_i[x])         (i < r)
//   P_ri = sum_x q_r[x] k_i[x] exp(G_r[x] - G_i[x])                (i <= r)
//   R    = diag(beta) (V - (K o e^G) M0)
//   (I + A) Delta = R
//   O    = scale ((Q o e^G) M0 + P Delta)
//   M1   = diag(e^{G_last}) M0 + (K o e^{G_last - G})^T Delta
//
// A and P are plain products once the pairwise factor splits in two.  The chunk's tokens
// form four blocks of 16; with Z_b the sum of g over the blocks before b, for r in block b
// and i in block b' <= b,  exp(G_r - G_i) = exp(G_r - Z_b) exp(Z_b - G_i).  The first
// factor is at most 1; so is the second when b' < b, and when b' = b it is at most
// exp of block b's own decay.  The row operands k_r o exp(G_r - Z_b), q_r o exp(G_r - Z_b)
// and the column operands k_i o exp(Z_b - G_i) (one set per row block) therefore stay in
// range.  When some channel decays by more than e^60 within a block, that block's
// diagonal tiles of A and P are formed from one exponential per pair and channel instead.
// Every other operand (K o e^G, Q o e^G, K o e^{G_last - G}) has factors at most 1.
//
// Two forms of the same arithmetic.  With the workspace dn_chunk_fwd_workspace_bytes
// returns, chg_prep_kernel runs steps 1 to 4 below once per (chunk, value head) for all
// chunks at once and chg_chain_kernel runs step 5 over each sequence's chunks (see the
// two-kernel form further down).  Without it, prefill_chg_kernel does everything in its
// chunk loop:  one workgroup of four waves per (sequence, value head, 32 value columns).
// Per chunk:
//   1  every wave takes the g, k, q of one 16-token block (two channels per lane), sums g
//      over the block and stages V and beta; the next chunk's loads are then issued
//   2  operands into LDS (bf16); wave b forms block b's diagonal tiles of A and P from
//      the rows it wrote (exactly, per pair, for blocks that decay too fast) and inverts
//      (I + A_bb)
//   3  A (waves 0, 1) and P (waves 2, 3) below the diagonal on the matrix cores
//   4  K o e^G and Q o e^G over the column operands
//   5  waves 0, 1 hold 16 state columns each in accumulators: X = (K o e^G) M0,
//      R, Delta by block substitution; waves 2, 3 form (Q o e^G) M0 transposed;
//      then waves 2, 3 add Delta^T P^T and store O (8 bytes: four columns of one token
//      per lane), waves 0, 1 update the state.
#include <mutex>

#include "../../include/deltanet.h"
#include "internal.h"
#include "mfma_ops.h"

namespace dn {
namespace {

constexpr int CC = 64;          // tokens per chunk
constexpr int NB = 4;           // 16-token blocks per chunk
constexpr int HK = 128;         // key dim
constexpr int SL = 32;          // value columns per workgroup
constexpr int NTH = 256;
constexpr int OP = 144;         // bf16 pitch of [token][key channel] tiles
constexpr int AP = 80;          // bf16 pitch of A and P
constexpr int TP = 24;          // bf16 pitch of the 16x16 inverses
constexpr int VP = 40;          // bf16 pitch of the V slice
constexpr int DP = 80;          // bf16 pitch of Delta^T
constexpr float HARD = 60.f;    // in-block decay (nats) beyond which the diagonal tiles go exact
constexpr float CLAMP = 80.f;   // cap of a diagonal column factor's exponent (hard blocks only)

// Row offset, in the column-operand buffer, of the operand set of row block b (rows i < 16(b+1)).
__device__ __forceinline__ int kc_off(int b) { return b == 0 ? 0 : b == 1 ? 16 : b == 2 ? 48 : 96; }

struct ChgSmem {
    __bf16 Kr[CC][OP];      // k_r o exp(G_r - Z_b(r))
    __bf16 Qr[CC][OP];      // q_r o exp(G_r - Z_b(r))
    __bf16 Kd[CC][OP];      // k_r o exp(G_last - G_r)
    __bf16 Kc[160][OP];     // column operands of A and P; then K o e^G (0..63), Q o e^G (64..127)
    __bf16 A[CC][AP];
    __bf16 P[CC][AP];
    float Ad[NB][16][20];   // A's diagonal tiles in fp32, transposed ([column][row]), for the inverses
    __bf16 Tb[NB][16][TP];  // (I + A_bb)^-1
    __bf16 V[CC][VP];
    __bf16 Mt[SL][OP];      // the state slice, transposed (B operand of (Q o e^G) M0)
    __bf16 Dt[SL][DP];      // Delta, transposed (B operand of P Delta)
    float beta[CC];
    float tot[NB][HK];      // per-block sums of g
    float eg[HK];           // exp(G_last)
    int hard[NB];
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, long bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float2 bf2_to_f2(uint32_t u) {
    return make_float2(__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u));
}
__device__ __forceinline__ void st2(__bf16* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(a, b);
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
    return x;
}

// tile t of the six 16x16 tiles below the diagonal of a 64x64 matrix -> (row block,
// column block): (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
__device__ __forceinline__ void offdiag_tile(int t, int& b, int& bp) {
    b = t < 1 ? 1 : t < 3 ? 2 : 3;
    bp = t - (b * (b - 1)) / 2;
}

__global__ __launch_bounds__(NTH) void prefill_chg_kernel(PrefillArgs a) {
    __shared__ __align__(16) ChgSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int Hv = a.Hv, Dv = a.Dv;
    const int slices = Dv / SL;

    // workgroup -> (sequence * Hv + head, slice); with a head count that is a multiple
    // of 8 the slices of a head land on one XCD and share its k, q, g through that L2
    const int heads = a.N * Hv;
    int nh, slice;
    if ((heads & 7) == 0) {
        const int y = blockIdx.x >> 3;
        slice = y % slices;
        nh = (blockIdx.x & 7) + 8 * (y / slices);
    } else {
        slice = blockIdx.x % slices;
        nh = blockIdx.x / slices;
    }
    const int h = nh % Hv, n = nh / Hv;
    const int hq = h / (Hv / a.Hqk);
    const int j0 = slice * SL;
    const int u = w & 1;            // 16-column tile of the slice (waves 0, 1 and 2, 3)
    const bool chain = w < 2;
    const __bf16* qp = static_cast<const __bf16*>(a.q);
    const __bf16* kp = static_cast<const __bf16*>(a.k);
    const __bf16* vp = static_cast<const __bf16*>(a.v);
    __bf16* op = static_cast<__bf16*>(a.o);

    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);

    // P's tiles above the diagonal that the output product reads stay zero
    for (int e = tid; e < CC * AP; e += NTH) (&sm.P[0][0])[e] = (__bf16)0.f;

    // state: chain wave u keeps rows 16t + 4 g4 + e, column 16u + l16 of the slice
    f32x4 m[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int x = 16 * t + 4 * g4 + e;
            m[t][e] = (chain && a.h0) ? a.h0[((long)nh * HK + x) * Dv + j0 + 16 * u + l16] : 0.f;
        }
        if (chain) st4(&sm.Mt[16 * u + l16][16 * t + 4 * g4], m[t][0], m[t][1], m[t][2], m[t][3]);
    }

    // raw inputs of one chunk: block w's tokens, key channels 2 lane and 2 lane + 1.  The
    // buffer descriptors cover exactly this sequence's tokens, so loads past its end (the
    // ragged last chunk, the chunk after the last) read zeros and every load is unconditional.
    const long L = eos - bos;
    const uint32_t g_tok = (uint32_t)Hv * HK * 4, kq_tok = (uint32_t)a.Hqk * HK * 2;
    const uint32_t v_tok = (uint32_t)Hv * Dv * 2, b_tok = (uint32_t)Hv * 4;
    const __amdgpu_buffer_rsrc_t gs = rsrc(a.g + (bos * Hv + h) * HK, L > 0 ? (L - 1) * g_tok + HK * 4 : 0);
    const __amdgpu_buffer_rsrc_t ks = rsrc(kp + (bos * a.Hqk + hq) * HK, L > 0 ? (L - 1) * kq_tok + HK * 2 : 0);
    const __amdgpu_buffer_rsrc_t qs = rsrc(qp + (bos * a.Hqk + hq) * HK, L > 0 ? (L - 1) * kq_tok + HK * 2 : 0);
    const __amdgpu_buffer_rsrc_t vs = rsrc(vp + (bos * Hv + h) * Dv + j0, L > 0 ? (L - 1) * v_tok + SL * 2 : 0);
    const __amdgpu_buffer_rsrc_t bs = rsrc(a.beta + bos * Hv + h, L > 0 ? (L - 1) * b_tok + 4 : 0);
    float2 rg[16];
    uint32_t rk[16], rq[16];
    bf16x8 rv;
    float rb;
    auto fetch = [&](uint32_t c) {  // c: the chunk's first token, counted from the sequence start
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t r = c + 16 * w + i;
            const u32x2 gv = __builtin_amdgcn_raw_buffer_load_b64(gs, r * g_tok + 8 * lane, 0, 0);
            rg[i] = make_float2(__uint_as_float(gv[0]), __uint_as_float(gv[1]));
            rk[i] = __builtin_amdgcn_raw_buffer_load_b32(ks, r * kq_tok + 4 * lane, 0, 0);
            rq[i] = __builtin_amdgcn_raw_buffer_load_b32(qs, r * kq_tok + 4 * lane, 0, 0);
        }
        rv = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(vs, (c + (tid >> 2)) * v_tok + 16 * (tid & 3), 0, 0));
        rb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bs, (c + (tid & 63)) * b_tok, 0, 0));
    };
    fetch(0);

    for (long c0 = bos; c0 < eos; c0 += CC) {
        const int len = (int)min((long)CC, eos - c0);

        // ---- 1: block sums of g (each 8-token half summed on its own, then the two added,
        // the order the two-kernel form takes), k and q as floats (normalised if asked), V
        // and beta
        float2 L[16], kf[16], qf[16];
        {
            float2 s = make_float2(0.f, 0.f), h0 = make_float2(0.f, 0.f);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i == 8) {
                    h0 = s;
                    s = make_float2(0.f, 0.f);
                }
                s.x += rg[i].x;
                s.y += rg[i].y;
                L[i] = i < 8 ? s : make_float2(h0.x + s.x, h0.y + s.y);
                kf[i] = bf2_to_f2(rk[i]);
                qf[i] = bf2_to_f2(rq[i]);
            }
            s = L[15];
            if (a.qk_norm) {
                float nk[16], nq[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    nk[i] = kf[i].x * kf[i].x + kf[i].y * kf[i].y;
                    nq[i] = qf[i].x * qf[i].x + qf[i].y * qf[i].y;
                }
#pragma unroll
                for (int mm = 1; mm < 64; mm <<= 1) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        nk[i] += __shfl_xor(nk[i], mm);
                        nq[i] += __shfl_xor(nq[i], mm);
                    }
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float ik = inv_norm(nk[i], a.eps), iq = inv_norm(nq[i], a.eps);
                    kf[i].x *= ik;
                    kf[i].y *= ik;
                    qf[i].x *= iq;
                    qf[i].y *= iq;
                }
            }
            *reinterpret_cast<bf16x8*>(&sm.V[tid >> 2][8 * (tid & 3)]) = rv;
            if (tid < CC) sm.beta[tid] = rb;
            *reinterpret_cast<float2*>(&sm.tot[w][2 * lane]) = s;
            const bool hb = __ballot(fminf(s.x, s.y) < -HARD) != 0;
            if (lane == 0) sm.hard[w] = hb ? 1 : 0;
        }
        __syncthreads();

        // ---- 2: operands
        float2 Z[NB], Zw = make_float2(0.f, 0.f), Gl = make_float2(0.f, 0.f);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            Z[b] = Gl;
            if (b == w) Zw = Gl;
            const float2 tb = *reinterpret_cast<const float2*>(&sm.tot[b][2 * lane]);
            Gl.x += tb.x;
            Gl.y += tb.y;
        }
        uint32_t pke[16], pqe[16];  // K o e^G and Q o e^G, stored once the column operands are read
        const bool hard = sm.hard[w] != 0;
        if (!hard) {
            // every factor from two exponentials per entry, e^{L} and e^{-L} (L the in-block
            // sum, -L at most 60 here), and per-channel factors of at most 1
            const float2 eZ = make_float2(__expf(Zw.x), __expf(Zw.y));
            const float2 eD = make_float2(__expf(Gl.x - Zw.x), __expf(Gl.y - Zw.y));
            float2 eF[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) eF[b] = make_float2(__expf(Z[b].x - Zw.x), __expf(Z[b].y - Zw.y));
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * w + i;
                const float e1x = __expf(L[i].x), e1y = __expf(L[i].y);
                const float e2x = __expf(-L[i].x), e2y = __expf(-L[i].y);
                const float kx = kf[i].x * e1x, ky = kf[i].y * e1y, qx = qf[i].x * e1x, qy = qf[i].y * e1y;
                st2(&sm.Kr[r][2 * lane], kx, ky);
                st2(&sm.Qr[r][2 * lane], qx, qy);
                pke[i] = pack_bf16x2(kx * eZ.x, ky * eZ.y);
                pqe[i] = pack_bf16x2(qx * eZ.x, qy * eZ.y);
                const float cx = kf[i].x * e2x, cy = kf[i].y * e2y;
                st2(&sm.Kd[r][2 * lane], cx * eD.x, cy * eD.y);
                st2(&sm.Kc[kc_off(w) + r][2 * lane], cx, cy);
#pragma unroll
                for (int b = 1; b < NB; ++b)
                    if (b > w) st2(&sm.Kc[kc_off(b) + r][2 * lane], cx * eF[b].x, cy * eF[b].y);
            }
        } else {
            // one exponential per factor, each of a difference that is at most 0 (the
            // diagonal column factor, replaced below, is capped)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int r = 16 * w + i;
                const float ax = __expf(Zw.x + L[i].x), ay = __expf(Zw.y + L[i].y);
                pke[i] = pack_bf16x2(kf[i].x * ax, kf[i].y * ay);
                pqe[i] = pack_bf16x2(qf[i].x * ax, qf[i].y * ay);
                const float ex = __expf(L[i].x), ey = __expf(L[i].y);
                st2(&sm.Kr[r][2 * lane], kf[i].x * ex, kf[i].y * ey);
                st2(&sm.Qr[r][2 * lane], qf[i].x * ex, qf[i].y * ey);
                st2(&sm.Kd[r][2 * lane], kf[i].x * __expf(Gl.x - Zw.x - L[i].x),
                    kf[i].y * __expf(Gl.y - Zw.y - L[i].y));
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < w) continue;
                    float cx = Z[b].x - Zw.x - L[i].x, cy = Z[b].y - Zw.y - L[i].y;
                    if (b == w) {
                        cx = fminf(cx, CLAMP);
                        cy = fminf(cy, CLAMP);
                    }
                    st2(&sm.Kc[kc_off(b) + r][2 * lane], kf[i].x * __expf(cx), kf[i].y * __expf(cy));
                }
            }
        }
        if (w == 0) *reinterpret_cast<float2*>(&sm.eg[2 * lane]) = make_float2(__expf(Gl.x), __expf(Gl.y));
        if (!hard) {
            // block w's diagonal tiles of A and P from the rows this wave has just written
            wave_lds_order();
            f32x4 aa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 kc = ld8(&sm.Kc[kc_off(w) + 16 * w + l16][32 * s + 8 * g4]);
                aa = mma16(ld8(&sm.Kr[16 * w + l16][32 * s + 8 * g4]), kc, aa);
                pa = mma16(ld8(&sm.Qr[16 * w + l16][32 * s + 8 * g4]), kc, pa);
            }
            const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * w + 4 * g4]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                const float av = l16 < r ? bt[e] * aa[e] : 0.f;
                sm.A[16 * w + r][16 * w + l16] = (__bf16)av;
                sm.Ad[w][l16][r] = av;
                sm.P[16 * w + r][16 * w + l16] = (__bf16)(l16 <= r ? pa[e] : 0.f);
            }
        } else {
            // block w decays too fast for the factored diagonal tile: one exponential per
            // (row, column, channel); the wave sums over its 128 channels.  Rare, so it
            // runs over private copies rather than holding registers for the common path.
            float2 hl[16], hk[16], hq[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                hl[i] = L[i];
                hk[i] = kf[i];
                hq[i] = qf[i];
            }
#pragma unroll 1
            for (int r = 0; r < 16; ++r) {
#pragma unroll 1
                for (int i = 0; i < 16; ++i) {
                    float pa = 0.f, pp = 0.f;
                    if (i <= r) {
                        const float dx = __expf(hl[r].x - hl[i].x), dy = __expf(hl[r].y - hl[i].y);
                        pa = wave_sum(hk[r].x * hk[i].x * dx + hk[r].y * hk[i].y * dy);
                        pp = wave_sum(hq[r].x * hk[i].x * dx + hq[r].y * hk[i].y * dy);
                    }
                    if (lane == 0) {
                        const float av = i < r ? sm.beta[16 * w + r] * pa : 0.f;
                        sm.A[16 * w + r][16 * w + i] = (__bf16)av;
                        sm.Ad[w][i][r] = av;
                        sm.P[16 * w + r][16 * w + i] = (__bf16)pp;
                    }
                }
            }
        }
        // (I + A_ww)^-1 by forward substitution, lane c < 16 solving column c in fp32; once
        // row i is final it is taken out of every later row at once (independent updates)
        wave_lds_order();
        if (lane < 16) {
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) t[r] = r == lane ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < 15; ++i) {
#pragma unroll
                for (int r4 = (i + 1) & ~3; r4 < 16; r4 += 4) {
                    const f32x4 av = *reinterpret_cast<const f32x4*>(&sm.Ad[w][i][r4]);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (r4 + j > i) t[r4 + j] -= av[j] * t[i];
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.Tb[w][r][lane] = (__bf16)t[r];
        }
        fetch((uint32_t)(c0 + CC - bos));  // the next chunk's inputs land while this one is worked
        __syncthreads();

        // ---- 3: A (waves 0, 1) and P (waves 2, 3) below the diagonal, three tiles per wave
        {
            const bool isP = w >= 2;
#pragma unroll
            for (int tt = 0; tt < 3; ++tt) {
                int b, bp;
                offdiag_tile(2 * tt + u, b, bp);
                const __bf16* rowp = isP ? &sm.Qr[16 * b + l16][8 * g4] : &sm.Kr[16 * b + l16][8 * g4];
                const __bf16* colp = &sm.Kc[kc_off(b) + 16 * bp + l16][8 * g4];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mma16(ld8(rowp + 32 * s), ld8(colp + 32 * s), acc);
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * b + 4 * g4]);
                const int i = 16 * bp + l16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * b + 4 * g4 + e;
                    if (isP) sm.P[r][i] = (__bf16)acc[e];
                    else sm.A[r][i] = (__bf16)(bt[e] * acc[e]);
                }
            }
        }
        __syncthreads();

        // ---- 4: K o e^G and Q o e^G over the column operands
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            *reinterpret_cast<uint32_t*>(&sm.Kc[16 * w + i][2 * lane]) = pke[i];
            *reinterpret_cast<uint32_t*>(&sm.Kc[CC + 16 * w + i][2 * lane]) = pqe[i];
        }
        __syncthreads();

        // ---- 5a: chain waves: R and Delta; waves 2, 3: (Q o e^G) M0
        const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
        f32x4 Y[NB] = {z4, z4, z4, z4};
        bf16x8 d01 = zero8(), d23 = zero8();
        if (chain) {
            bf16x8 mb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) mb[s] = acc_to_b(m[2 * s], m[2 * s + 1]);
            f32x4 R[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4 x = z4;
#pragma unroll
                for (int s = 0; s < 4; ++s) x = mma16(ld8(&sm.Kc[16 * b + l16][32 * s + 8 * g4]), mb[s], x);
                // V read transposed: the lane's four tokens of its column in one read
                const int r0 = 16 * b + 4 * g4;
                const bf16x4 vv = trld(&sm.V[r0 + (l16 >> 2)][16 * u + 4 * (l16 & 3)]);
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[r0]);
#pragma unroll
                for (int e = 0; e < 4; ++e) R[b][e] = bt[e] * ((float)vv[e] - x[e]);
            }
            bf16x8 ta[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) ta[b] = g4 < 2 ? ld8(&sm.Tb[b][l16][8 * g4]) : zero8();
            // Delta_b = T_bb (R_b - sum_{b'<b} A_bb' Delta_b')
            const f32x4 D0 = mma16(ta[0], acc_to_b(R[0], z4), z4);
            f32x4 c = mma16(ld8(&sm.A[16 + l16][8 * g4]), acc_to_b(D0, z4), z4);
            const f32x4 D1 = mma16(ta[1], acc_to_b(R[1] - c, z4), z4);
            d01 = acc_to_b(D0, D1);
            c = mma16(ld8(&sm.A[32 + l16][8 * g4]), d01, z4);
            const f32x4 D2 = mma16(ta[2], acc_to_b(R[2] - c, z4), z4);
            c = mma16(ld8(&sm.A[48 + l16][8 * g4]), d01, z4);
            c = mma16(ld8(&sm.A[48 + l16][32 + 8 * g4]), acc_to_b(D2, z4), c);
            const f32x4 D3 = mma16(ta[3], acc_to_b(R[3] - c, z4), z4);
            d23 = acc_to_b(D2, D3);
            st4(&sm.Dt[16 * u + l16][4 * g4], D0[0], D0[1], D0[2], D0[3]);
            st4(&sm.Dt[16 * u + l16][16 + 4 * g4], D1[0], D1[1], D1[2], D1[3]);
            st4(&sm.Dt[16 * u + l16][32 + 4 * g4], D2[0], D2[1], D2[2], D2[3]);
            st4(&sm.Dt[16 * u + l16][48 + 4 * g4], D3[0], D3[1], D3[2], D3[3]);
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4 y = z4;
#pragma unroll
                for (int s = 0; s < 4; ++s)   // transposed: lane holds 4 columns of one token
                    y = mma16(ld8(&sm.Mt[16 * u + l16][32 * s + 8 * g4]),
                              ld8(&sm.Kc[CC + 16 * b + l16][32 * s + 8 * g4]), y);
                Y[b] = y;
            }
        }
        __syncthreads();

        // ---- 5b: waves 2, 3: O = scale (Y + P Delta); chain waves: the state update
        if (!chain) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4 acc = Y[b];
#pragma unroll
                for (int s = 0; s <= b / 2; ++s)   // O^T = Delta^T P^T + Y^T
                    acc = mma16(ld8(&sm.Dt[16 * u + l16][32 * s + 8 * g4]),
                                ld8(&sm.P[16 * b + l16][32 * s + 8 * g4]), acc);
                const int r = 16 * b + l16;   // token; columns 16 u + 4 g4 .. + 3
                if (r < len)
                    st4(op + ((c0 + r) * Hv + h) * Dv + j0 + 16 * u + 4 * g4, a.scale * acc[0],
                        a.scale * acc[1], a.scale * acc[2], a.scale * acc[3]);
            }
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                f32x4 acc;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = m[t][e] * sm.eg[16 * t + 4 * g4 + e];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    // A operand (K o e^{G_last - G})^T: rows are key channels, read down columns
                    const __bf16* base = &sm.Kd[32 * s + 8 * g4 + (l16 >> 2)][16 * t + 4 * (l16 & 3)];
                    const bf16x8 ka = cat(trld(base), trld(base + 4 * OP));
                    acc = mma16(ka, s ? d23 : d01, acc);
                }
                m[t] = acc;
                st4(&sm.Mt[16 * u + l16][16 * t + 4 * g4], acc[0], acc[1], acc[2], acc[3]);
            }
        }
        __syncthreads();
    }

    if (chain && a.hT) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                a.hT[((long)nh * HK + 16 * t + 4 * g4 + e) * Dv + j0 + 16 * u + l16] = m[t][e];
    }
}


// ------------------------------------------------------------------ two-kernel form
// With a workspace, the state-independent work of every chunk (steps 1 to 4 above) runs
// once per (chunk, value head) in a kernel over all chunks at once, instead of once per
// 32-column slice inside the sequential loop; the chain kernel then only loads each
// chunk's operands and runs step 5.  Workspace record of one (chunk, value head), bytes:
constexpr long OP_KE = 0;          // K o e^G            [64][128] bf16
constexpr long OP_QE = 16384;      // Q o e^G            [64][128] bf16
constexpr long OP_KD = 32768;      // K o e^{G_last - G} [64][128] bf16
constexpr long OP_A = 49152;       // A                  [64][64] bf16
constexpr long OP_P = 57344;       // P                  [64][64] bf16
constexpr long OP_TB = 65536;      // (I + A_bb)^-1      [4][16][16] bf16
constexpr long OP_EG = 67584;      // exp(G_last)        [128] fp32
constexpr long OP_BETA = 68096;    // beta               [64] fp32
constexpr long OP_BYTES = 68352;

// Record numbers.  A batch of rows numbers its chunks row by row.  Packed sequences give
// chunk c of sequence n the number floor(cu[n] / 64) + n + c: distinct (the next
// sequence's first number is past this one's last) and found without a scan; at most
// T / 64 + N of them.  first_chunk(n) is sequence n's first number; chunk_of inverts the
// numbering (false for a number no chunk takes).
__device__ long first_chunk(const PrefillArgs& a, int n) {
    if (!a.cu) return (long)n * (((long)a.T + CC - 1) / CC);
    return (long)a.cu[n] / CC + n;
}
__device__ bool chunk_of(const PrefillArgs& a, long gid, int& n, long& c) {
    if (!a.cu) {
        const long cps = ((long)a.T + CC - 1) / CC;
        if (cps == 0) return false;
        n = (int)(gid / cps);
        c = gid % cps;
        return n < a.N;
    }
    // the last sequence whose first number is at most gid (first numbers increase with n)
    int lo = 0, hi = a.N - 1;
    if (hi < 0 || first_chunk(a, 0) > gid) return false;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (first_chunk(a, mid) <= gid) lo = mid;
        else hi = mid - 1;
    }
    n = lo;
    c = gid - first_chunk(a, lo);
    return c < ((long)a.cu[lo + 1] - a.cu[lo] + CC - 1) / CC;
}

// LDS of the prep kernel: the operand tiles of one (chunk, value head) item.
struct PrepSmemChg {
    __bf16 Kr[CC][OP];      // k_r o exp(G_r - Z_b(r))
    __bf16 Qr[CC][OP];      // q_r o exp(G_r - Z_b(r))
    __bf16 Kc[160][OP];     // column operands of A and P; then K o e^G (0..63), Q o e^G (64..127)
    __bf16 A[CC][AP];
    __bf16 P[CC][AP];
    float Ad[NB][16][20];   // A's diagonal tiles in fp32, transposed ([column][row]), for the inverses
    __bf16 Tb[NB][16][TP];  // (I + A_bb)^-1
    float beta[CC];
    float toth[2 * NB][HK]; // sums of g over each 8-token half of a block
    float eg[HK];           // exp(G_last)
};

constexpr int NPP = 512;    // threads of the prep kernel: two waves per 16-token block

// One workgroup per CU walks the (chunk, value head) items, item = chunk * Hv + head; the
// next item's inputs are requested as soon as the current one's are consumed.  Wave w
// takes the 8 tokens 8 w .. 8 w + 7 (half of block w / 2), two key channels per lane, for
// the block sums and the operands; then waves 0-3 form block w's diagonal tiles of A and
// P and invert (I + A_ww) while waves 4-7 form the tiles below the diagonal.
__global__ __launch_bounds__(NPP) void chg_prep_kernel(PrefillArgs a, long nitems) {
    __shared__ __align__(16) PrepSmemChg sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int blk = w >> 1, hf = w & 1;   // this wave's rows: 16 blk + 8 hf + i, i < 8
    const int Hv = a.Hv;
    const __bf16* qp = static_cast<const __bf16*>(a.q);
    const __bf16* kp = static_cast<const __bf16*>(a.k);
    const uint32_t g_tok = (uint32_t)Hv * HK * 4, kq_tok = (uint32_t)a.Hqk * HK * 2, b_tok = (uint32_t)Hv * 4;

    // A's and P's tiles above the diagonal stay zero (only the tiles on and below it are written)
    for (int e = tid; e < CC * AP; e += NPP) {
        (&sm.P[0][0])[e] = (__bf16)0.f;
        (&sm.A[0][0])[e] = (__bf16)0.f;
    }

    // the first item from `item` on (in steps of the grid) that a chunk takes; nitems if none
    auto next_item = [&](long item) -> long {
        int n;
        long cix;
        while (item < nitems && !chunk_of(a, item / Hv, n, cix)) item += gridDim.x;
        return item;
    };
    // range-checked streams of an item's sequence (rows past its end read zeros) and the
    // item's first token within it
    struct Streams {
        __amdgpu_buffer_rsrc_t gs, ks, qs, bs;
        uint32_t c;
    };
    auto streams = [&](long item) -> Streams {
        int n;
        long cix;
        chunk_of(a, item / Hv, n, cix);
        const int h = (int)(item % Hv);
        const int hq = h / (Hv / a.Hqk);
        long bos, eos;
        seq_range(a.cu, n, a.T, bos, eos);
        const long L = eos - bos;
        Streams s;
        s.gs = rsrc(a.g + (bos * Hv + h) * HK, L > 0 ? (L - 1) * g_tok + HK * 4 : 0);
        s.ks = rsrc(kp + (bos * a.Hqk + hq) * HK, L > 0 ? (L - 1) * kq_tok + HK * 2 : 0);
        s.qs = rsrc(qp + (bos * a.Hqk + hq) * HK, L > 0 ? (L - 1) * kq_tok + HK * 2 : 0);
        s.bs = rsrc(a.beta + bos * Hv + h, L > 0 ? (L - 1) * b_tok + 4 : 0);
        s.c = (uint32_t)(cix * CC);
        return s;
    };
    float2 rg[8];
    uint32_t rk[8], rq[8];
    float rb = 0.f;
    // requests item `item`'s inputs (a chunk takes it): this wave's 8 tokens, key channels
    // 2 lane and 2 lane + 1; wave 0 also the 64 betas
    auto fetch = [&](long item) {
        const Streams s = streams(item);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t r = s.c + 8 * w + i;
            const u32x2 gv = __builtin_amdgcn_raw_buffer_load_b64(s.gs, r * g_tok + 8 * lane, 0, 0);
            rg[i] = make_float2(__uint_as_float(gv[0]), __uint_as_float(gv[1]));
            rk[i] = __builtin_amdgcn_raw_buffer_load_b32(s.ks, r * kq_tok + 4 * lane, 0, 0);
            rq[i] = __builtin_amdgcn_raw_buffer_load_b32(s.qs, r * kq_tok + 4 * lane, 0, 0);
        }
        if (w == 0) rb = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(s.bs, (s.c + lane) * b_tok, 0, 0));
    };
    // k, q rows (float pairs) normalised in place if asked: one wave reduction per row
    auto normalise = [&](float2* kf, float2* qf, int rows) {
        if (!a.qk_norm) return;
#pragma unroll 1
        for (int i = 0; i < rows; ++i) {
            float nk = kf[i].x * kf[i].x + kf[i].y * kf[i].y, nq = qf[i].x * qf[i].x + qf[i].y * qf[i].y;
#pragma unroll
            for (int mm = 1; mm < 64; mm <<= 1) {
                nk += __shfl_xor(nk, mm);
                nq += __shfl_xor(nq, mm);
            }
            const float ik = inv_norm(nk, a.eps), iq = inv_norm(nq, a.eps);
            kf[i].x *= ik;
            kf[i].y *= ik;
            qf[i].x *= iq;
            qf[i].y *= iq;
        }
    };

    long item = next_item(blockIdx.x);
    if (item < nitems) fetch(item);
    while (item < nitems) {
        // ---- 1: sums of g over this wave's 8 tokens; k and q as floats (normalised if asked)
        float2 L[8], kf[8], qf[8];
        {
            float2 s = make_float2(0.f, 0.f);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                s.x += rg[i].x;
                s.y += rg[i].y;
                L[i] = s;
                kf[i] = bf2_to_f2(rk[i]);
                qf[i] = bf2_to_f2(rq[i]);
            }
            if (a.qk_norm) {
                float nk[8], nq[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    nk[i] = kf[i].x * kf[i].x + kf[i].y * kf[i].y;
                    nq[i] = qf[i].x * qf[i].x + qf[i].y * qf[i].y;
                }
#pragma unroll
                for (int mm = 1; mm < 64; mm <<= 1) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        nk[i] += __shfl_xor(nk[i], mm);
                        nq[i] += __shfl_xor(nq[i], mm);
                    }
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float ik = inv_norm(nk[i], a.eps), iq = inv_norm(nq[i], a.eps);
                    kf[i].x *= ik;
                    kf[i].y *= ik;
                    qf[i].x *= iq;
                    qf[i].y *= iq;
                }
            }
            if (w == 0) sm.beta[lane] = rb;
            *reinterpret_cast<float2*>(&sm.toth[w][2 * lane]) = s;
        }
        __syncthreads();

        const long next = next_item(item + gridDim.x);
        const Streams cur = streams(item);   // kept for a block that decays too fast
        if (next < nitems) fetch(next);   // lands while this item is worked
        // ---- 2: operands.  Z_b = sum of g over the blocks before b; G_r - Z_b for this
        // wave's rows is the first half's sum (second half only) plus the running sum
        float2 Z[NB], Zw = make_float2(0.f, 0.f), Gl = make_float2(0.f, 0.f), off = make_float2(0.f, 0.f);
        int hardm = 0;   // blocks in which some channel decays by more than e^HARD
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            Z[b] = Gl;
            const float2 t0 = *reinterpret_cast<const float2*>(&sm.toth[2 * b][2 * lane]);
            const float2 t1 = *reinterpret_cast<const float2*>(&sm.toth[2 * b + 1][2 * lane]);
            const float2 tb = make_float2(t0.x + t1.x, t0.y + t1.y);
            if (b == blk) {
                Zw = Gl;
                if (hf) off = t0;
            }
            if (__ballot(fminf(tb.x, tb.y) < -HARD) != 0) hardm |= 1 << b;
            Gl.x += tb.x;
            Gl.y += tb.y;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            L[i].x += off.x;
            L[i].y += off.y;
        }
        // this wave's rows of K o e^G, Q o e^G and K o e^{G_last - G} go to the record from
        // registers as they are formed (a row of 128 channels is one 256-byte store a wave),
        // so that only A, P, the inverses, e^{G_last} and beta leave at the item's end
        char* rec = static_cast<char*>(a.ws) + item * OP_BYTES;
        auto put_row = [&](long off, int r, float x, float y) {
            *reinterpret_cast<uint32_t*>(rec + off + r * 256 + 4 * lane) = pack_bf16x2(x, y);
        };
        if (!((hardm >> blk) & 1)) {
            // every factor from two exponentials per entry, e^{L} and e^{-L} (L the in-block
            // sum, -L at most 60 here), and per-channel factors of at most 1
            const float2 eZ = make_float2(__expf(Zw.x), __expf(Zw.y));
            const float2 eD = make_float2(__expf(Gl.x - Zw.x), __expf(Gl.y - Zw.y));
            float2 eF[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) eF[b] = make_float2(__expf(Z[b].x - Zw.x), __expf(Z[b].y - Zw.y));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 16 * blk + 8 * hf + i;
                const float e1x = __expf(L[i].x), e1y = __expf(L[i].y);
                const float e2x = __expf(-L[i].x), e2y = __expf(-L[i].y);
                const float kx = kf[i].x * e1x, ky = kf[i].y * e1y, qx = qf[i].x * e1x, qy = qf[i].y * e1y;
                st2(&sm.Kr[r][2 * lane], kx, ky);
                st2(&sm.Qr[r][2 * lane], qx, qy);
                put_row(OP_KE, r, kx * eZ.x, ky * eZ.y);
                put_row(OP_QE, r, qx * eZ.x, qy * eZ.y);
                const float cx = kf[i].x * e2x, cy = kf[i].y * e2y;
                put_row(OP_KD, r, cx * eD.x, cy * eD.y);
                st2(&sm.Kc[kc_off(blk) + r][2 * lane], cx, cy);
#pragma unroll
                for (int b = 1; b < NB; ++b)
                    if (b > blk) st2(&sm.Kc[kc_off(b) + r][2 * lane], cx * eF[b].x, cy * eF[b].y);
            }
        } else {
            // one exponential per factor, each of a difference that is at most 0 (the
            // diagonal column factor, replaced below, is capped)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 16 * blk + 8 * hf + i;
                const float ax = __expf(Zw.x + L[i].x), ay = __expf(Zw.y + L[i].y);
                put_row(OP_KE, r, kf[i].x * ax, kf[i].y * ay);
                put_row(OP_QE, r, qf[i].x * ax, qf[i].y * ay);
                const float ex = __expf(L[i].x), ey = __expf(L[i].y);
                st2(&sm.Kr[r][2 * lane], kf[i].x * ex, kf[i].y * ey);
                st2(&sm.Qr[r][2 * lane], qf[i].x * ex, qf[i].y * ey);
                put_row(OP_KD, r, kf[i].x * __expf(Gl.x - Zw.x - L[i].x), kf[i].y * __expf(Gl.y - Zw.y - L[i].y));
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (b < blk) continue;
                    float cx = Z[b].x - Zw.x - L[i].x, cy = Z[b].y - Zw.y - L[i].y;
                    if (b == blk) {
                        cx = fminf(cx, CLAMP);
                        cy = fminf(cy, CLAMP);
                    }
                    st2(&sm.Kc[kc_off(b) + r][2 * lane], kf[i].x * __expf(cx), kf[i].y * __expf(cy));
                }
            }
        }
        if (w == 0) *reinterpret_cast<float2*>(&sm.eg[2 * lane]) = make_float2(__expf(Gl.x), __expf(Gl.y));
        __syncthreads();   // every operand row is in LDS

        if (w < NB) {
            // ---- 3a: block w's diagonal tiles of A and P, then (I + A_ww)^-1
            if (!((hardm >> w) & 1)) {
                f32x4 aa = {0.f, 0.f, 0.f, 0.f}, pa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8 kc = ld8(&sm.Kc[kc_off(w) + 16 * w + l16][32 * s + 8 * g4]);
                    aa = mma16(ld8(&sm.Kr[16 * w + l16][32 * s + 8 * g4]), kc, aa);
                    pa = mma16(ld8(&sm.Qr[16 * w + l16][32 * s + 8 * g4]), kc, pa);
                }
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * w + 4 * g4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 4 * g4 + e;
                    const float av = l16 < r ? bt[e] * aa[e] : 0.f;
                    sm.A[16 * w + r][16 * w + l16] = (__bf16)av;
                    sm.Ad[w][l16][r] = av;
                    sm.P[16 * w + r][16 * w + l16] = (__bf16)(l16 <= r ? pa[e] : 0.f);
                }
            } else {
                // block w decays too fast for the factored diagonal tile: one exponential per
                // (row, column, channel), the wave summing over its 128 channels, from the
                // block's g, k and q read again (rare, so it holds no registers elsewhere)
                float2 hl[16], hk[16], hq[16];
                {
                    // the in-block sums as the operands took them: each half on its own
                    float2 s = make_float2(0.f, 0.f), h0 = make_float2(0.f, 0.f);
#pragma unroll 1
                    for (int i = 0; i < 16; ++i) {
                        const uint32_t r = cur.c + 16 * w + i;
                        const u32x2 gv = __builtin_amdgcn_raw_buffer_load_b64(cur.gs, r * g_tok + 8 * lane, 0, 0);
                        if (i == 8) {
                            h0 = s;
                            s = make_float2(0.f, 0.f);
                        }
                        s.x += __uint_as_float(gv[0]);
                        s.y += __uint_as_float(gv[1]);
                        hl[i] = i < 8 ? s : make_float2(h0.x + s.x, h0.y + s.y);
                        hk[i] = bf2_to_f2(__builtin_amdgcn_raw_buffer_load_b32(cur.ks, r * kq_tok + 4 * lane, 0, 0));
                        hq[i] = bf2_to_f2(__builtin_amdgcn_raw_buffer_load_b32(cur.qs, r * kq_tok + 4 * lane, 0, 0));
                    }
                }
                normalise(hk, hq, 16);
#pragma unroll 1
                for (int r = 0; r < 16; ++r) {
#pragma unroll 1
                    for (int i = 0; i < 16; ++i) {
                        float pa = 0.f, pp = 0.f;
                        if (i <= r) {
                            const float dx = __expf(hl[r].x - hl[i].x), dy = __expf(hl[r].y - hl[i].y);
                            pa = wave_sum(hk[r].x * hk[i].x * dx + hk[r].y * hk[i].y * dy);
                            pp = wave_sum(hq[r].x * hk[i].x * dx + hq[r].y * hk[i].y * dy);
                        }
                        if (lane == 0) {
                            const float av = i < r ? sm.beta[16 * w + r] * pa : 0.f;
                            sm.A[16 * w + r][16 * w + i] = (__bf16)av;
                            sm.Ad[w][i][r] = av;
                            sm.P[16 * w + r][16 * w + i] = (__bf16)pp;
                        }
                    }
                }
            }
            // (I + A_ww)^-1 by forward substitution, lane c < 16 solving column c in fp32; once
            // row i is final it is taken out of every later row at once (independent updates)
            wave_lds_order();
            if (lane < 16) {
                float t[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) t[r] = r == lane ? 1.f : 0.f;
#pragma unroll
                for (int i = 0; i < 15; ++i) {
#pragma unroll
                    for (int r4 = (i + 1) & ~3; r4 < 16; r4 += 4) {
                        const f32x4 av = *reinterpret_cast<const f32x4*>(&sm.Ad[w][i][r4]);
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (r4 + j > i) t[r4 + j] -= av[j] * t[i];
                    }
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) sm.Tb[w][r][lane] = (__bf16)t[r];
            }
        } else {
            // ---- 3b: A (waves 4, 5) and P (waves 6, 7) below the diagonal, three tiles a wave
            const bool isP = w >= 6;
#pragma unroll
            for (int tt = 0; tt < 3; ++tt) {
                int b, bp;
                offdiag_tile(2 * tt + hf, b, bp);
                const __bf16* rowp = isP ? &sm.Qr[16 * b + l16][8 * g4] : &sm.Kr[16 * b + l16][8 * g4];
                const __bf16* colp = &sm.Kc[kc_off(b) + 16 * bp + l16][8 * g4];
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mma16(ld8(rowp + 32 * s), ld8(colp + 32 * s), acc);
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[16 * b + 4 * g4]);
                const int i = 16 * bp + l16;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * b + 4 * g4 + e;
                    if (isP) sm.P[r][i] = (__bf16)acc[e];
                    else sm.A[r][i] = (__bf16)(bt[e] * acc[e]);
                }
            }
        }
        __syncthreads();

        // ---- out: the rest of this item's record
        {
            const int r = tid >> 3, p = tid & 7;
            *reinterpret_cast<u32x4v*>(rec + OP_A + r * 128 + p * 16) = *reinterpret_cast<const u32x4v*>(&sm.A[r][8 * p]);
            *reinterpret_cast<u32x4v*>(rec + OP_P + r * 128 + p * 16) = *reinterpret_cast<const u32x4v*>(&sm.P[r][8 * p]);
        }
        if (tid < 128) {
            const int b = tid >> 5, r = (tid >> 1) & 15, p = tid & 1;
            *reinterpret_cast<u32x4v*>(rec + OP_TB + (b * 16 + r) * 32 + p * 16) = *reinterpret_cast<const u32x4v*>(&sm.Tb[b][r][8 * p]);
        } else if (tid < 160) {
            const int e = tid - 128;
            *reinterpret_cast<u32x4v*>(rec + OP_EG + e * 16) = *reinterpret_cast<const u32x4v*>(&sm.eg[4 * e]);
        } else if (tid < 176) {
            const int e = tid - 160;
            *reinterpret_cast<u32x4v*>(rec + OP_BETA + e * 16) = *reinterpret_cast<const u32x4v*>(&sm.beta[4 * e]);
        }
        __syncthreads();   // the next item rewrites LDS
        item = next;
    }
}

// LDS of the chain kernel: the operands step 5a reads are double-buffered so that the
// next chunk's arrive while this one is worked; those of step 5b are single.
struct ChainSmem {
    __bf16 Ke[2][CC][OP];      // K o e^G
    __bf16 Qe[2][CC][OP];      // Q o e^G
    __bf16 A[2][CC][AP];
    __bf16 Tb[2][NB][16][TP];
    __bf16 V[2][CC][VP];
    float beta[2][CC];
    __bf16 Kd[CC][OP];         // K o e^{G_last - G}
    __bf16 P[CC][AP];
    float eg[HK];
    __bf16 Mt[SL][OP];
    __bf16 Dt[SL][DP];
};

// Waves 0, 1 run the chain (16 state columns each in accumulators).  Waves 2, 3 load every
// chunk's record and V slice one chunk ahead into registers and store them to LDS in
// their slack, form (Q o e^G) M0 and store O.  Two barriers per chunk:
//   X  chain: X, R, Delta from A/B buffer c % 2   |  2, 3: K o e^{G_last-G}, P, e^{G_last} of
//      chunk c to LDS, request chunk c + 1, (Q o e^G) M0
//   Y  chain: the state update                    |  2, 3: O; chunk c + 1's step-5a operands
//                                                 |  to buffer (c + 1) % 2
__global__ __launch_bounds__(NTH) void chg_chain_kernel(PrefillArgs a) {
    __shared__ __align__(16) ChainSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int Hv = a.Hv, Dv = a.Dv;
    const int slices = Dv / SL;
    const int heads = a.N * Hv;
    int nh, slice;
    if ((heads & 7) == 0) {
        const int y = blockIdx.x >> 3;
        slice = y % slices;
        nh = (blockIdx.x & 7) + 8 * (y / slices);
    } else {
        slice = blockIdx.x % slices;
        nh = blockIdx.x / slices;
    }
    const int h = nh % Hv, n = nh / Hv;
    const int j0 = slice * SL;
    const int u = w & 1;
    long bos, eos;
    seq_range(a.cu, n, a.T, bos, eos);
    const long nch = (eos - bos + CC - 1) / CC;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

    if (w < 2) {
        // ------------------------------------------------------------ chain waves
        f32x4 m[8];   // rows 16t + 4 g4 + e, column 16u + l16 of the slice
#pragma unroll
        for (int t = 0; t < 8; ++t) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int x = 16 * t + 4 * g4 + e;
                m[t][e] = a.h0 ? a.h0[((long)nh * HK + x) * Dv + j0 + 16 * u + l16] : 0.f;
            }
            st4(&sm.Mt[16 * u + l16][16 * t + 4 * g4], m[t][0], m[t][1], m[t][2], m[t][3]);
        }
        __syncthreads();   // buffer 0 holds chunk 0's step-5a operands
        for (long cix = 0; cix < nch; ++cix) {
            const int cb = (int)(cix & 1);
            // X: R = beta (V - (K o e^G) M0), Delta by block substitution
            bf16x8 mb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) mb[s] = acc_to_b(m[2 * s], m[2 * s + 1]);
            f32x4 R[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4 x = z4;
#pragma unroll
                for (int s = 0; s < 4; ++s) x = mma16(ld8(&sm.Ke[cb][16 * b + l16][32 * s + 8 * g4]), mb[s], x);
                // V read transposed: the lane's four tokens of its column in one read
                const int r0 = 16 * b + 4 * g4;
                const bf16x4 vv = trld(&sm.V[cb][r0 + (l16 >> 2)][16 * u + 4 * (l16 & 3)]);
                const f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.beta[cb][r0]);
#pragma unroll
                for (int e = 0; e < 4; ++e) R[b][e] = bt[e] * ((float)vv[e] - x[e]);
            }
            bf16x8 ta[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) ta[b] = g4 < 2 ? ld8(&sm.Tb[cb][b][l16][8 * g4]) : zero8();
            // Delta_b = T_bb (R_b - sum_{b'<b} A_bb' Delta_b')
            const f32x4 D0 = mma16(ta[0], acc_to_b(R[0], z4), z4);
            f32x4 c = mma16(ld8(&sm.A[cb][16 + l16][8 * g4]), acc_to_b(D0, z4), z4);
            const f32x4 D1 = mma16(ta[1], acc_to_b(R[1] - c, z4), z4);
            const bf16x8 d01 = acc_to_b(D0, D1);
            c = mma16(ld8(&sm.A[cb][32 + l16][8 * g4]), d01, z4);
            const f32x4 D2 = mma16(ta[2], acc_to_b(R[2] - c, z4), z4);
            c = mma16(ld8(&sm.A[cb][48 + l16][8 * g4]), d01, z4);
            c = mma16(ld8(&sm.A[cb][48 + l16][32 + 8 * g4]), acc_to_b(D2, z4), c);
            const f32x4 D3 = mma16(ta[3], acc_to_b(R[3] - c, z4), z4);
            const bf16x8 d23 = acc_to_b(D2, D3);
            st4(&sm.Dt[16 * u + l16][4 * g4], D0[0], D0[1], D0[2], D0[3]);
            st4(&sm.Dt[16 * u + l16][16 + 4 * g4], D1[0], D1[1], D1[2], D1[3]);
            st4(&sm.Dt[16 * u + l16][32 + 4 * g4], D2[0], D2[1], D2[2], D2[3]);
            st4(&sm.Dt[16 * u + l16][48 + 4 * g4], D3[0], D3[1], D3[2], D3[3]);
            __syncthreads();
            // Y: M1 = diag(e^{G_last}) M0 + (K o e^{G_last - G})^T Delta
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                f32x4 acc;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = m[t][e] * sm.eg[16 * t + 4 * g4 + e];
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    // A operand (K o e^{G_last - G})^T: rows are key channels, read down columns
                    const __bf16* base = &sm.Kd[32 * s + 8 * g4 + (l16 >> 2)][16 * t + 4 * (l16 & 3)];
                    const bf16x8 ka = cat(trld(base), trld(base + 4 * OP));
                    acc = mma16(ka, s ? d23 : d01, acc);
                }
                m[t] = acc;
                st4(&sm.Mt[16 * u + l16][16 * t + 4 * g4], acc[0], acc[1], acc[2], acc[3]);
            }
            __syncthreads();
        }
        if (a.hT) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.hT[((long)nh * HK + 16 * t + 4 * g4 + e) * Dv + j0 + 16 * u + l16] = m[t][e];
        }
    } else {
        // ------------------------------------------------ loader and output waves
        const int lt = tid - 128;   // 0 .. 127
        const __bf16* vp = static_cast<const __bf16*>(a.v);
        __bf16* op = static_cast<__bf16*>(a.o);
        const long first = first_chunk(a, n);
        const long L = eos - bos;
        const uint32_t v_tok = (uint32_t)Hv * Dv * 2;
        const __amdgpu_buffer_rsrc_t vs = rsrc(vp + (bos * Hv + h) * Dv + j0, L > 0 ? (L - 1) * v_tok + SL * 2 : 0);
        // pieces (16 bytes) of one chunk: step 5a's K o e^G, Q o e^G (8 each), A (4), an inverse
        // piece, V (2), beta (lt < 16); step 5b's K o e^{G_last - G} (8), P (4), e^{G_last} (lt < 32)
        u32x4v rke[8], rqe[8], ra[4], rtb, rbe = u32x4v{0u, 0u, 0u, 0u};
        u32x4v rkd[8], rp[4], reg = u32x4v{0u, 0u, 0u, 0u};
        bf16x8 rv[2];
        auto fetch = [&](long c) {
            const char* rec = static_cast<const char*>(a.ws) + ((first + c) * Hv + h) * OP_BYTES;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = lt + 128 * i, r = e >> 4, p = e & 15;
                rke[i] = *reinterpret_cast<const u32x4v*>(rec + OP_KE + r * 256 + p * 16);
                rqe[i] = *reinterpret_cast<const u32x4v*>(rec + OP_QE + r * 256 + p * 16);
                rkd[i] = *reinterpret_cast<const u32x4v*>(rec + OP_KD + r * 256 + p * 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = lt + 128 * i, r = e >> 3, p = e & 7;
                ra[i] = *reinterpret_cast<const u32x4v*>(rec + OP_A + r * 128 + p * 16);
                rp[i] = *reinterpret_cast<const u32x4v*>(rec + OP_P + r * 128 + p * 16);
            }
            rtb = *reinterpret_cast<const u32x4v*>(rec + OP_TB + lt * 16);
            if (lt < 16) rbe = *reinterpret_cast<const u32x4v*>(rec + OP_BETA + lt * 16);
            if (lt < 32) reg = *reinterpret_cast<const u32x4v*>(rec + OP_EG + lt * 16);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int e = lt + 128 * i;   // row e >> 2, 16-byte piece e & 3 of the slice
                rv[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                            vs, (uint32_t)(c * CC + (e >> 2)) * v_tok + 16 * (e & 3), 0, 0));
            }
        };
        auto store_a = [&](int cb) {   // step 5a's operands to buffer cb
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = lt + 128 * i, r = e >> 4, p = e & 15;
                *reinterpret_cast<u32x4v*>(&sm.Ke[cb][r][8 * p]) = rke[i];
                *reinterpret_cast<u32x4v*>(&sm.Qe[cb][r][8 * p]) = rqe[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = lt + 128 * i, r = e >> 3, p = e & 7;
                *reinterpret_cast<u32x4v*>(&sm.A[cb][r][8 * p]) = ra[i];
            }
            *reinterpret_cast<u32x4v*>(&sm.Tb[cb][lt >> 5][(lt >> 1) & 15][8 * (lt & 1)]) = rtb;
            if (lt < 16) *reinterpret_cast<u32x4v*>(&sm.beta[cb][4 * lt]) = rbe;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int e = lt + 128 * i;
                *reinterpret_cast<bf16x8*>(&sm.V[cb][e >> 2][8 * (e & 3)]) = rv[i];
            }
        };
        auto store_b = [&]() {   // step 5b's operands
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int e = lt + 128 * i, r = e >> 4, p = e & 15;
                *reinterpret_cast<u32x4v*>(&sm.Kd[r][8 * p]) = rkd[i];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = lt + 128 * i, r = e >> 3, p = e & 7;
                *reinterpret_cast<u32x4v*>(&sm.P[r][8 * p]) = rp[i];
            }
            if (lt < 32) *reinterpret_cast<u32x4v*>(&sm.eg[4 * lt]) = reg;
        };
        if (nch > 0) {
            fetch(0);
            store_a(0);
        }
        __syncthreads();   // buffer 0 holds chunk 0's step-5a operands
        for (long cix = 0; cix < nch; ++cix) {
            const int cb = (int)(cix & 1);
            const long c0 = bos + cix * CC;
            const int len = (int)min((long)CC, eos - c0);
            // X: this chunk's step-5b operands, the next chunk's request, (Q o e^G) M0
            store_b();
            if (cix + 1 < nch) fetch(cix + 1);
            f32x4 Y[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4 y = z4;
#pragma unroll
                for (int s = 0; s < 4; ++s)   // transposed: lane holds 4 columns of one token
                    y = mma16(ld8(&sm.Mt[16 * u + l16][32 * s + 8 * g4]),
                              ld8(&sm.Qe[cb][16 * b + l16][32 * s + 8 * g4]), y);
                Y[b] = y;
            }
            __syncthreads();
            // Y: O^T = Delta^T P^T + Y^T, stored four columns per lane; the next chunk's
            // step-5a operands to the other buffer
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                f32x4 acc = Y[b];
#pragma unroll
                for (int s = 0; s <= b / 2; ++s)
                    acc = mma16(ld8(&sm.Dt[16 * u + l16][32 * s + 8 * g4]),
                                ld8(&sm.P[16 * b + l16][32 * s + 8 * g4]), acc);
                const int r = 16 * b + l16;
                if (r < len)
                    st4(op + ((c0 + r) * Hv + h) * Dv + j0 + 16 * u + 4 * g4, a.scale * acc[0],
                        a.scale * acc[1], a.scale * acc[2], a.scale * acc[3]);
            }
            if (cix + 1 < nch) store_a(cb ^ 1);
            __syncthreads();
        }
    }
}

}  // namespace

// record numbers in use: exact for a batch of rows; for packed sequences (only B = 1
// packs) the numbering above stays below T / 64 + N + 1
static long chg_chunk_bound(const PrefillArgs& a) {
    const long rows = (long)a.B * (((long)a.T + CC - 1) / CC);
    if (a.B != 1) return rows;
    const long packed = (long)a.T / CC + a.N + 1;
    return rows > packed ? rows : packed;
}

static bool chg_shape_ok(const PrefillArgs& a) {
    // buffer offsets are 32-bit: a sequence plus the chunk fetched past its end must span
    // less than 2 GiB of every stream (g, fp32 per key channel, is the widest)
    const int hmax = a.Hqk > a.Hv ? a.Hqk : a.Hv;
    const long span = ((long)a.T + 2 * CC) * hmax * (HK * 4 > a.Dv * 2 ? HK * 4 : a.Dv * 2);
    return a.g_per_key && a.bf16 && a.Dk == HK && a.Dv >= SL && a.Dv % SL == 0 && a.C == CC &&
           span < (1L << 31);
}

bool prefill_chg_shape_ok(const PrefillArgs& a) { return chg_shape_ok(a); }

bool prefill_chg_supported(const PrefillArgs& a) {
    const uintptr_t al = (uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.v | (uintptr_t)a.o;
    return chg_shape_ok(a) && a.g && (al & 15) == 0 && ((uintptr_t)a.g & 7) == 0;
}

size_t prefill_chg_workspace_bytes(const PrefillArgs& a) {
    if (!chg_shape_ok(a)) return 0;
    return (size_t)chg_chunk_bound(a) * a.Hv * OP_BYTES;
}

hipError_t launch_prefill_chg(const PrefillArgs& a, hipStream_t s) {
    const long blocks = (long)a.N * a.Hv * (a.Dv / SL);
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (blocks == 0) return hipGetLastError();
    const size_t need = prefill_chg_workspace_bytes(a);
    if (need > 0 && a.ws && a.ws_bytes >= need && ((uintptr_t)a.ws & 15) == 0) {
        // two kernels: every chunk's operands at once, then the chain over the chunks
        const long items = chg_chunk_bound(a) * a.Hv;
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            cus = 256;
        const long prep = items < cus ? items : cus;   // one workgroup per CU (its LDS allows no more)
        hipLaunchKernelGGL(chg_prep_kernel, dim3((unsigned)prep), dim3(NPP), 0, s, a, items);
        hipLaunchKernelGGL(chg_chain_kernel, dim3((unsigned)blocks), dim3(NTH), 0, s, a);
    } else {
        hipLaunchKernelGGL(prefill_chg_kernel, dim3((unsigned)blocks), dim3(NTH), 0, s, a);
    }
    return hipGetLastError();
}

// ------------------------------------------------------------ allocation-free scratch
// The per-(chunk, value head) records of the two-kernel form, for callers that cannot
// allocate device memory: one static device array per GPU, held from the code object's
// load on that GPU until the process ends.  In host code `scratch` names a host-side
// stand-in, not the device array: its device address comes from hipGetSymbolAddress, once
// per device with that device current, and only that address is ever handed to a kernel.
constexpr size_t NOALLOC_BYTES = (size_t)64 << 20;
static_assert(NOALLOC_BYTES == DN_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
static __device__ __align__(256) unsigned char scratch[NOALLOC_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_dev[MAX_DEVICES];   // device address of `scratch` on each GPU, once known
}  // namespace

size_t noalloc_scratch_bytes() { return NOALLOC_BYTES; }

hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_dev[dev] = p;
    }
    *ptr = scratch_dev[dev];
    return hipSuccess;
}

}  // namespace dn

