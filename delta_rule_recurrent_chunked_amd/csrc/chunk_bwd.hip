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
// Only the carry dM runs across chunks, and it needs just T, P and the chunk's inputs; the
// rest is independent per chunk once M and dM' are known.  Four launches:
//   1. the prompt kernel writes the state at every chunk start (outputs skipped);
//   2. chunk_tp_kernel, one workgroup per (chunk, value head): T^T and P to the workspace
//      (when launch 1 has a workgroup for every CU, nothing could run beside it, and it
//      writes T^T and P itself instead);
//   3. chunk_carry_kernel, one workgroup per (sequence, value head, 32-column slice): the
//      chunks backwards, dM' kept in MFMA accumulators and written out at every chunk (the
//      last one is the initial state's gradient);
//   4. chunk_grad_kernel, one workgroup per (chunk, q/k head): every gradient of the chunk,
//      over the value heads of the q/k head and the four column slices, with dA, dP and the
//      dq, dk terms accumulated in registers, so dq and dk are written once, in a fixed
//      order, without atomics.  Three row dot products come out of accumulators already
//      formed: (Q M)_r . dO_r = Q_r . (dO M^T)_r, X_r . dR_r = K_r . (dR M^T)_r and
//      (K dM')_r . Delta_r = K_r . (Delta dM'^T)_r.
//
// Operands live in LDS as bf16: a "row" fragment (lane = row of the stored matrix) is one
// 16-byte read, a "column" fragment (lane = column) two transposed 8-byte reads
// (ds_read_b64_tr_b16).  Products whose consumer reads them by rows of their transpose are
// stored transposed, four values of a lane in one 8-byte write.
#include <mutex>

#include "chunk_ops.h"

namespace dn {
namespace {
using namespace ck;

constexpr int BD = 128;            // Dk = Dv
constexpr int BNS = BD / BS;       // slices
constexpr int P128 = BD + 16;      // bf16 pitch of [token][key] tiles

// ============================================ 3. the carry dM per (sequence, head, slice)
constexpr int NTB = 512;           // 8 waves (the gradient kernel; the carry's compute waves)
constexpr int NTC = 768;           // the carry: 8 compute waves and 4 loader waves
constexpr int NLC = NTC - NTB;     // loader threads

struct alignas(16) CarrySmem {
    __bf16 K[2][BC][P128], Q[2][BC][P128];    // two chunks: the current one and the next
    __bf16 dO[2][BC][P32];
    __bf16 Tt[2][BC][P64], P[2][BC][P64];
    __bf16 dDt[BS][P64];           // dDelta^T
    __bf16 dXt[BS][P64];           // dX^T
    __bf16 dMt[BS][P128];          // the slice of dM' (the gradient of the state after the chunk), transposed
    float tail[2][BC], sod[2][BC], bx[2][BC], egl[2][4];
};

// one chunk's inputs in a loader thread's registers: loader thread t holds 16-byte pieces
// t + 256 u of K and Q (u < 4, row = piece / 16), piece t of dO's slice (row = piece / 4),
// pieces t + 256 u of T^T and of P (u < 2, row = piece / 8), beta and g of token t (t < 64)
struct CarryIn {
    uint4 k[4], q[4], o, t[2], p[2];
    float beta, g;
};

// Waves 0-7 run the three product steps of each chunk; waves 8-11 move the next chunk's
// inputs into the other half of the double-buffered LDS and request the chunk after it, so
// that neither sits between the products.  Every wave takes the three barriers of a chunk.
__global__ __launch_bounds__(NTC, 1) void chunk_carry_kernel(ChunkBwdArgs a) {
    __shared__ CarrySmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q16 = lane >> 4;
    // workgroup -> (sequence, value head, slice): when the count of (sequence, q/k head)
    // pairs is a multiple of 8, the slices of the value heads of one q/k head run one after
    // another on one XCD (workgroups are dealt to the 8 XCDs round-robin) and share that
    // head's K and Q through the XCD's L2
    const int grp = a.Hv / a.Hqk, qchains = a.N * a.Hqk;
    int slice, nh;
    if ((qchains & 7) == 0) {
        const int y = blockIdx.x >> 3, t = y / BNS;
        const int qc = (blockIdx.x & 7) + 8 * (t / grp);
        slice = y % BNS;
        nh = (qc / a.Hqk) * a.Hv + (qc % a.Hqk) * grp + t % grp;
    } else {
        slice = blockIdx.x % BNS;
        nh = blockIdx.x / BNS;
    }
    const int h = nh % a.Hv, n = nh / a.Hv;
    const int hq = h / grp;
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
    const auto o_rs = rsrc(static_cast<const __bf16*>(a.dout) + v0, v_end);
    const auto b_rs = rsrc(a.beta + s0, s_end);
    const auto g_rs = rsrc(a.g ? a.g + s0 : a.beta + s0, a.g ? s_end : 0);
    const bool loader = wave >= NTB / 64;
    const int lt = tid - NTB;   // loader thread 0 .. 255 (negative on the compute waves)
    uint32_t kq_off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int pc = lt + NLC * u;
        kq_off[u] = (uint32_t)(pc >> 4) * kq_tok + (pc & 15) * 16;
    }
    const uint32_t o_off = (uint32_t)(lt >> 2) * v_tok + (lt & 3) * 16;
    const uint32_t sc_off = (uint32_t)lane * s_tok;
    const uint4* tp_head = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.tp)) + lt;

    auto fetch = [&](int c, CarryIn& f) {   // loader waves only
        const uint32_t ck = (uint32_t)c * BC * kq_tok, cv = (uint32_t)c * BC * v_tok, cs = (uint32_t)c * BC * s_tok;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            f.k[u] = ld128(k_rs, kq_off[u], ck);
            f.q[u] = ld128(q_rs, kq_off[u], ck);
        }
        f.o = ld128(o_rs, o_off, cv);
        const uint4* tp = tp_head + ((cid0 + c) * a.Hv + h) * (2L * BC * BC / 8);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f.t[u] = tp[NLC * u];
            f.p[u] = tp[BC * BC / 8 + NLC * u];
        }
        if (lt < 64) {
            f.beta = ld32(b_rs, sc_off, cs);
            f.g = ld32(g_rs, sc_off, cs);
        }
    };
    auto put_in = [&](const CarryIn& f, int b) {   // loader waves only
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int pc = lt + NLC * u, row = pc >> 4, cg = pc & 15;
            *reinterpret_cast<uint4*>(&sm.K[b][row][cg * 8]) = f.k[u];
            *reinterpret_cast<uint4*>(&sm.Q[b][row][cg * 8]) = f.q[u];
        }
        *reinterpret_cast<uint4*>(&sm.dO[b][lt >> 2][(lt & 3) * 8]) = f.o;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int pc = lt + NLC * u;
            *reinterpret_cast<uint4*>(&sm.Tt[b][pc >> 3][(pc & 7) * 8]) = f.t[u];
            *reinterpret_cast<uint4*>(&sm.P[b][pc >> 3][(pc & 7) * 8]) = f.p[u];
        }
        if (lt < 64) {
            float gl;
            const float gv = gamma_scan(a.g ? f.g : 0.f, gl);
            const float eg = __expf(gv);
            sm.tail[b][lane] = __expf(gl - gv);
            sm.sod[b][lane] = sc * eg;
            sm.bx[b][lane] = -f.beta * eg;
            if (lane == 0) sm.egl[b][0] = __expf(gl);
        }
    };

    // dM' of this slice in MFMA accumulators: wave w holds tiles (key block 2 (w >> 1) + u,
    // column block w & 1), u = 0, 1: keys 16 (2 (w >> 1) + u) + 4 q16 + e, column 16 (w & 1) + l16
    if (loader) {
        // ------------------------------------------------------------ loader waves
        // at the start of chunk c's turn: chunk c - 1's inputs (requested a turn ago) into the
        // buffer chunk c + 1 used, then the request for chunk c - 2
        CarryIn f;
        if (nc > 0) {
            fetch(nc - 1, f);
            put_in(f, (nc - 1) & 1);
            if (nc > 1) fetch(nc - 2, f);
        }
        __syncthreads();
        for (int c = nc - 1; c >= 0; --c) {
            if (c > 0) {
                put_in(f, (c & 1) ^ 1);
                if (c > 1) fetch(c - 2, f);
            }
            __syncthreads();
            __syncthreads();
            __syncthreads();
        }
        return;
    }

    // ---------------------------------------------------------------- compute waves
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
        for (int u = 0; u < 2; ++u) put_tile_t(&sm.dMt[0][0], P128, 2 * (wave >> 1) + u, dmj, dm[u], l16, q16);
    };

    put_dm();
    __syncthreads();
    const int ti = wave >> 1, tj = wave & 1;   // this wave's 16 x 16 tile of a 64 x 32 product
    for (int c = nc - 1; c >= 0; --c) {
        const int b = c & 1;
        {   // dM' of chunk c to the workspace (the gradient kernel's input), in 16 x 16 tiles of
            // the accumulator layout like the chunk-start states: one 16-byte store per tile
            float* dst = a.dstates + ((cid0 + c) * a.Hv + h) * (long)BD * BD + (2 * slice + dmj) * 256 + 4 * lane;
#pragma unroll
            for (int u = 0; u < 2; ++u) *reinterpret_cast<f32x4*>(dst + (2 * (wave >> 1) + u) * 8 * 256) = dm[u];
        }
        // ---------------------------- dDelta = scale P^T dO + diag(tail) K dM', stored transposed
        {
            f32x4 pd = {0.f, 0.f, 0.f, 0.f}, kd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32)
                if (k0 + 32 > 16 * ti) pd = mma16(frag_c(&sm.P[b][0][0], P64, 16 * ti, k0, l16, q16),
                                                  frag_c(&sm.dO[b][0][0], P32, 16 * tj, k0, l16, q16), pd);
#pragma unroll
            for (int k0 = 0; k0 < BD; k0 += 32)
                kd = mma16(frag_r(&sm.K[b][0][0], P128, 16 * ti, k0, l16, q16), frag_r(&sm.dMt[0][0], P128, 16 * tj, k0, l16, q16), kd);
            f32x4 dd;
#pragma unroll
            for (int e = 0; e < 4; ++e) dd[e] = sc * pd[e] + sm.tail[b][16 * ti + 4 * q16 + e] * kd[e];
            put_tile_t(&sm.dDt[0][0], P64, ti, tj, dd, l16, q16);
        }
        __syncthreads();
        // ------------------------------ dX = -diag(beta e^gamma) T^T dDelta, stored transposed;
        // scale Q^T diag(e^gamma) dO of this wave's dM tiles (no carry in it) alongside
        f32x4 qd[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ki = 2 * (wave >> 1) + u;
            qd[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32) {
                bf16x8 od = frag_c(&sm.dO[b][0][0], P32, 16 * dmj, k0, l16, q16);
#pragma unroll
                for (int e = 0; e < 8; ++e) od[e] = (__bf16)((float)od[e] * sm.sod[b][k0 + 8 * q16 + e]);
                qd[u] = mma16(frag_c(&sm.Q[b][0][0], P128, 16 * ki, k0, l16, q16), od, qd[u]);
            }
        }
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32)
                if (k0 + 32 > 16 * ti) acc = mma16(frag_r(&sm.Tt[b][0][0], P64, 16 * ti, k0, l16, q16),
                                                   frag_r(&sm.dDt[0][0], P64, 16 * tj, k0, l16, q16), acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] *= sm.bx[b][16 * ti + 4 * q16 + e];
            put_tile_t(&sm.dXt[0][0], P64, ti, tj, acc, l16, q16);
        }
        __syncthreads();
        // ------------------------- dM' <- e^gamma_L dM' + scale Q^T diag(e^gamma) dO + K^T dX
        {
            const float gl = sm.egl[b][0];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ki = 2 * (wave >> 1) + u;
                f32x4 acc = dm[u] * gl + qd[u];
#pragma unroll
                for (int k0 = 0; k0 < BC; k0 += 32)
                    acc = mma16(frag_c(&sm.K[b][0][0], P128, 16 * ki, k0, l16, q16),
                                frag_r(&sm.dXt[0][0], P64, 16 * dmj, k0, l16, q16), acc);
                dm[u] = acc;
            }
        }
        // the new dM' into LDS (read before the last two barriers)
        put_dm();
        __syncthreads();
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

// ==================================== 4. every gradient of a chunk per (chunk, q/k head)
struct alignas(16) GradSmem {
    __bf16 K[BC][P128], Q[BC][P128];
    __bf16 Tt[BC][P64];            // T^T; W = dA o diag(beta) D (row-major) at a head's end
    __bf16 P[BC][P64];             // P; Z = dP o D at a head's end
    __bf16 V[BC][P32], dO[BC][P32];   // one 32-column slice of V and dO
    __bf16 Dl[BC][P32], dR[BC][P32];  // Delta and dR of the slice
    __bf16 Rt[BS][P64], dDt[BS][P64]; // R^T and dDelta^T of the slice
    __bf16 Mt[BS][P128], dMt[BS][P128];   // the slice of M and of dM', transposed
    float beta[BC], gam[BC], eg[BC], tail[BC];
    // per-row partial sums in fixed slots (summed in order at a head's end)
    float vdr[BC][8];              // V . dR, per (slice, column block)
    float ku[BC][8], qy[BC][8], kc[BC][8];   // K . (dR M^T), Q . (dO M^T), K . (Delta dM'^T), per key block
    float ag[BC][4];               // sum_i dA_ri G_ri, per column block
    float aa_r[BC][4], pp_r[BC][4];   // row sums of dA o A and dP o P, per column block
    float aa_c[BC][16], pp_c[BC][16]; // minus their column sums, per (row block, row group)
    float mdm[8];                  // <M, dM'> per wave
};

// one slice's inputs in registers: piece t & 255 of V (t < 256) or dO (t >= 256) (row =
// piece / 4), pieces t and t + 512 of M's and dM''s slices: the slice's 16 tiles (8 key
// blocks x 2 column blocks) of 64 lanes x float4, piece p = tile (p >> 6), lane p & 63
struct GradIn {
    uint4 vo;
    float4 m[2], d[2];
};

template <bool GATED>
__global__ __launch_bounds__(NTB, 1) void chunk_grad_kernel(ChunkBwdArgs a) {
    __shared__ GradSmem sm;
    // (every phase re-derives its lane offsets l16 = lane & 15, q16 = lane >> 4 with fresh())
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hq = (int)(blockIdx.x % a.Hqk);
    const long cid = blockIdx.x / a.Hqk;
    int n;
    long c, bos, L;
    if (!chunk_of_id(a, cid, n, c, bos, L)) return;
    const int grp = a.Hv / a.Hqk;
    const long t0 = bos + c * BC;
    const int rows = (int)min((long)BC, L - c * BC);
    const float sc = a.scale;
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);

    // K and Q of the chunk (rows past the end read zeros), issued with the first slice's loads
    const uint32_t kq_tok = (uint32_t)a.Hqk * BD * 2;
    const uint32_t kq_bytes = (uint32_t)(rows - 1) * kq_tok + BD * 2;
    const auto k_rs = rsrc(static_cast<const __bf16*>(a.k) + (t0 * a.Hqk + hq) * BD, kq_bytes);
    const auto q_rs = rsrc(static_cast<const __bf16*>(a.q) + (t0 * a.Hqk + hq) * BD, kq_bytes);
    uint4 kin[2], qin[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int pc = tid + NTB * u;
        const uint32_t off = (uint32_t)(pc >> 4) * kq_tok + (pc & 15) * 16;
        kin[u] = ld128(k_rs, off, 0);
        qin[u] = ld128(q_rs, off, 0);
    }

    // buffer resources over this chunk's rows (rows past the end read zeros, stores there are
    // dropped) and this chunk's states; per-thread 32-bit offsets, the head and slice in the
    // scalar offset
    const uint32_t v_tok = (uint32_t)a.Hv * BD;   // elements per token of v, dO, dv
    const auto vo_rs = rsrc(static_cast<const __bf16*>(wave < 4 ? a.v : a.dout) + t0 * v_tok, (uint32_t)rows * v_tok * 2);
    const auto dv_rs = rsrc(a.dv + t0 * v_tok, (uint32_t)rows * v_tok * 4);
    const uint32_t st_bytes = (uint32_t)a.Hv * BD * BD * 4;
    const auto m_rs = rsrc(a.states + cid * a.Hv * (long)BD * BD, st_bytes);
    const auto d_rs = rsrc(a.dstates + cid * a.Hv * (long)BD * BD, st_bytes);
    const int vrow = (tid & 255) >> 2;
    const uint32_t vo_off = ((uint32_t)vrow * v_tok + (tid & 3) * 8) * 2;
    uint32_t m_off[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {   // tile (key block kb, column block 2 sl + cb) at (8 kb + 2 sl + cb) 256 floats
        const int pc = tid + NTB * u, tt = pc >> 6;
        m_off[u] = (uint32_t)(((tt >> 1) * 8 + (tt & 1)) * 256 + 4 * (pc & 63)) * 4;
    }
    auto fetch = [&](int g, int sl, GradIn& f) {
        const int h = hq * grp + g, j0 = sl * BS;
        f.vo = ld128(vo_rs, vo_off, (uint32_t)(h * BD + j0) * 2);
        const uint32_t so = (uint32_t)(h * BD * BD + 2 * sl * 256) * 4;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f.m[u] = __builtin_bit_cast(float4, ld128(m_rs, m_off[u], so));
            f.d[u] = __builtin_bit_cast(float4, ld128(d_rs, m_off[u], so));
        }
    };

    f32x4 dqg[4], dkg[4];   // dq, dk over the group's value heads: tiles (t4, wave) of 64 x 128
#pragma unroll
    for (int t4 = 0; t4 < 4; ++t4) dqg[t4] = dkg[t4] = f32x4{0.f, 0.f, 0.f, 0.f};

    GradIn f;
    fetch(0, 0, f);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int pc = tid + NTB * u, row = pc >> 4, cg = pc & 15;
        *reinterpret_cast<uint4*>(&sm.K[row][cg * 8]) = kin[u];
        *reinterpret_cast<uint4*>(&sm.Q[row][cg * 8]) = qin[u];
    }
    for (int g = 0; g < grp; ++g) {
        const int h = hq * grp + g;
        // ---------------------------------------- head prologue: T^T, P, beta, gamma
        __syncthreads();   // the previous head's last reads of W, Z and the slots are done
        {
            const int tf = fresh(tid);
            const uint4* tp = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(a.tp)) +
                              (cid * a.Hv + h) * (2L * BC * BC / 8) + tf;
            *reinterpret_cast<uint4*>(&sm.Tt[tf >> 3][(tf & 7) * 8]) = tp[0];
            *reinterpret_cast<uint4*>(&sm.P[tf >> 3][(tf & 7) * 8]) = tp[BC * BC / 8];
            for (int i = tf; i < BC * 4; i += NTB) {   // slots not every tile writes
                (&sm.ag[0][0])[i] = 0.f;
                (&sm.aa_r[0][0])[i] = 0.f;
                (&sm.pp_r[0][0])[i] = 0.f;
            }
            for (int i = tf; i < BC * 16; i += NTB) {
                (&sm.aa_c[0][0])[i] = 0.f;
                (&sm.pp_c[0][0])[i] = 0.f;
            }
        }
        if (wave == 0) {
            const bool ok = lane < rows;
            const long s = (t0 + lane) * a.Hv + h;
            float gl = 0.f, gv = 0.f;
            if (GATED) gv = gamma_scan(ok ? a.g[s] : 0.f, gl);
            sm.beta[lane] = ok ? a.beta[s] : 0.f;
            sm.gam[lane] = gv;
            sm.eg[lane] = __expf(gv);
            sm.tail[lane] = __expf(gl - gv);
        }
        f32x4 dap[3];                  // dR Delta^T (t < 10) or dO Delta^T (t >= 10), tile t = wave + 8 m
        f32x4 qa[4], uu[4], k2[4];     // dO M^T, dR M^T, Delta dM'^T: tiles (t4, wave)
#pragma unroll
        for (int m = 0; m < 3; ++m) dap[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) qa[t4] = uu[t4] = k2[t4] = f32x4{0.f, 0.f, 0.f, 0.f};
        float mdm_t = 0.f;
        const int ti = wave >> 1, tj = wave & 1;   // this wave's tile of a 64 x 32 product

#pragma unroll 1
        for (int sl = 0; sl < BNS; ++sl) {
            const int j0 = sl * BS;
            // ------------------------------------------------------ the slice's inputs
            if (sl > 0) __syncthreads();   // the last slice's products are read
            {
            const int tf = fresh(tid), vr = (tf & 255) >> 2;
            *reinterpret_cast<uint4*>(tf < 256 ? &sm.V[vr][(tf & 3) * 8] : &sm.dO[vr][(tf & 3) * 8]) = f.vo;
#pragma unroll
            for (int u = 0; u < 2; ++u) {   // four keys of one column: 8 bytes of the transposed tile
                const int pc = tf + NTB * u, tt = pc >> 6, ln = pc & 63;
                const int col = 16 * (tt & 1) + (ln & 15), key = 16 * (tt >> 1) + 4 * (ln >> 4);
                *reinterpret_cast<uint2*>(&sm.Mt[col][key]) =
                    make_uint2(pack_bf16x2(f.m[u].x, f.m[u].y), pack_bf16x2(f.m[u].z, f.m[u].w));
                *reinterpret_cast<uint2*>(&sm.dMt[col][key]) =
                    make_uint2(pack_bf16x2(f.d[u].x, f.d[u].y), pack_bf16x2(f.d[u].z, f.d[u].w));
                if (GATED)
                    mdm_t += f.m[u].x * f.d[u].x + f.m[u].y * f.d[u].y + f.m[u].z * f.d[u].z + f.m[u].w * f.d[u].w;
            }
            }
            if (sl + 1 < BNS) fetch(g, sl + 1, f);
            else if (g + 1 < grp) fetch(g + 1, 0, f);
            __syncthreads();

            // ------------- R = diag(beta) (V - diag(e^gamma) K M); dDelta = scale P^T dO + diag(tail) K dM'
            {
                const int ln = fresh(lane), l16 = ln & 15, q16 = ln >> 4;   // lane offsets rederived here
                f32x4 x = {0.f, 0.f, 0.f, 0.f}, kd = {0.f, 0.f, 0.f, 0.f}, pd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < BD; k0 += 32) {
                    const bf16x8 kf = frag_r(&sm.K[0][0], P128, 16 * ti, k0, l16, q16);
                    x = mma16(kf, frag_r(&sm.Mt[0][0], P128, 16 * tj, k0, l16, q16), x);
                    kd = mma16(kf, frag_r(&sm.dMt[0][0], P128, 16 * tj, k0, l16, q16), kd);
                }
#pragma unroll
                for (int k0 = 0; k0 < BC; k0 += 32)
                    if (k0 + 32 > 16 * ti) pd = mma16(frag_c(&sm.P[0][0], P64, 16 * ti, k0, l16, q16),
                                                      frag_c(&sm.dO[0][0], P32, 16 * tj, k0, l16, q16), pd);
                const int col = 16 * tj + l16;
                f32x4 r, dd;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * ti + 4 * q16 + e;
                    r[e] = sm.beta[row] * ((float)sm.V[row][col] - sm.eg[row] * x[e]);
                    dd[e] = sc * pd[e] + sm.tail[row] * kd[e];
                }
                put_tile_t(&sm.Rt[0][0], P64, ti, tj, r, l16, q16);
                put_tile_t(&sm.dDt[0][0], P64, ti, tj, dd, l16, q16);
            }
            __syncthreads();

            // ------------------------------ Delta = T R; dR = T^T dDelta; dV; V . dR
            {
                const int ln = fresh(lane), l16 = ln & 15, q16 = ln >> 4;   // lane offsets rederived here
                f32x4 dl = {0.f, 0.f, 0.f, 0.f}, dr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < BC; k0 += 32) {
                    if (k0 <= 16 * ti) dl = mma16(frag_c(&sm.Tt[0][0], P64, 16 * ti, k0, l16, q16),
                                                  frag_r(&sm.Rt[0][0], P64, 16 * tj, k0, l16, q16), dl);
                    if (k0 + 32 > 16 * ti) dr = mma16(frag_r(&sm.Tt[0][0], P64, 16 * ti, k0, l16, q16),
                                                      frag_r(&sm.dDt[0][0], P64, 16 * tj, k0, l16, q16), dr);
                }
                put_tile(&sm.Dl[0][0], P32, ti, tj, dl, l16, q16);
                put_tile(&sm.dR[0][0], P32, ti, tj, dr, l16, q16);
                const int col = 16 * tj + l16;
                f32x4 vd;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * ti + 4 * q16 + e;
                    vd[e] = (float)sm.V[row][col] * dr[e];
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sm.beta[row] * dr[e]), dv_rs,
                                                          ((uint32_t)row * v_tok + col) * 4, (uint32_t)(h * BD + j0) * 4, 0);
                }
                vd = row_sum16(vd);
                if (l16 == 0) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) sm.vdr[16 * ti + 4 * q16 + e][2 * sl + tj] = vd[e];
                }
            }
            __syncthreads();

            // ---------------- dR Delta^T, dO Delta^T (lower tiles); dO M^T, dR M^T, Delta dM'^T
            {
            const int ln = fresh(lane), l16 = ln & 15, q16 = ln >> 4;   // lane offsets rederived here
#pragma unroll
            for (int m = 0; m < 3; ++m) {
                const int t = wave + 8 * m;
                if (t < 20) {
                    int ri, ci;
                    lower_tile(t % 10, ri, ci);
                    dap[m] = mma16(frag_r(t < 10 ? &sm.dR[0][0] : &sm.dO[0][0], P32, 16 * ri, 0, l16, q16),
                                   frag_r(&sm.Dl[0][0], P32, 16 * ci, 0, l16, q16), dap[m]);
                }
            }
            {
                const bf16x8 mf = frag_c(&sm.Mt[0][0], P128, 16 * wave, 0, l16, q16);
                const bf16x8 df = frag_c(&sm.dMt[0][0], P128, 16 * wave, 0, l16, q16);
#pragma unroll
                for (int t4 = 0; t4 < 4; ++t4) {
                    qa[t4] = mma16(frag_r(&sm.dO[0][0], P32, 16 * t4, 0, l16, q16), mf, qa[t4]);
                    uu[t4] = mma16(frag_r(&sm.dR[0][0], P32, 16 * t4, 0, l16, q16), mf, uu[t4]);
                    k2[t4] = mma16(frag_r(&sm.Dl[0][0], P32, 16 * t4, 0, l16, q16), df, k2[t4]);
                    sched_fence();
                }
            }
            }
        }

        // ------------------------------------------------- head end: W, Z, row sums
        // (T^T was last read before the last slice's final barrier; each P tile is read and
        // overwritten by the wave that owns it)
#pragma unroll
        for (int m = 0; m < 3; ++m) {
            const int ln = fresh(lane), l16 = ln & 15, q16 = ln >> 4;   // lane offsets rederived here
            const int t = wave + 8 * m;
            if (t < 20) {
                int ri, ci;
                lower_tile(t % 10, ri, ci);
                const bool isa = t < 10;
                f32x4 gk = {0.f, 0.f, 0.f, 0.f};   // K K^T (the dA tiles)
                if (isa) {
#pragma unroll
                    for (int k0 = 0; k0 < BD; k0 += 32)
                        gk = mma16(frag_r(&sm.K[0][0], P128, 16 * ri, k0, l16, q16),
                                   frag_r(&sm.K[0][0], P128, 16 * ci, k0, l16, q16), gk);
                }
                const int col = 16 * ci + l16;
                const float gc = sm.gam[col];
                f32x4 rs, bs, wz;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * ri + 4 * q16 + e;
                    const bool keep = isa ? col < row : col <= row;
                    const float dv = keep ? (isa ? -dap[m][e] : sc * dap[m][e]) : 0.f;
                    const float dec = GATED ? __expf(fminf(sm.gam[row] - gc, 0.f)) : 1.f;
                    const float s = isa ? dec * gk[e] : (float)sm.P[row][col];   // D o K K^T, or P
                    const float fb = isa ? sm.beta[row] : 1.f;
                    rs[e] = dv * fb * s;     // dA o A (A = beta G) or dP o P
                    bs[e] = dv * s;          // dA o G (the dbeta term)
                    wz[e] = keep ? dv * fb * dec : 0.f;   // W or Z
                }
                put_tile(isa ? &sm.Tt[0][0] : &sm.P[0][0], P64, ri, ci, wz, l16, q16);
                if (isa) {
                    const f32x4 b16 = row_sum16(bs);
                    if (l16 == 0) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) sm.ag[16 * ri + 4 * q16 + e][ci] = b16[e];
                    }
                }
                if (GATED) {
                    const f32x4 r16 = row_sum16(rs);
                    if (l16 == 0) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) (isa ? sm.aa_r : sm.pp_r)[16 * ri + 4 * q16 + e][ci] = r16[e];
                    }
                    (isa ? sm.aa_c : sm.pp_c)[col][4 * ri + q16] = -(rs[0] + rs[1] + rs[2] + rs[3]);
                }
            }
            sched_fence();
        }
        if (tid < 192) {   // W's blocks above the diagonal (T^T's entries are there)
            const int tf = fresh(tid), u = tf >> 5, r = (tf >> 1) & 15, half = tf & 1;
            const int ri = u < 3 ? 0 : u < 5 ? 1 : 2;
            const int ci = u < 3 ? u + 1 : u < 5 ? u - 1 : 3;
            *reinterpret_cast<uint4*>(&sm.Tt[16 * ri + r][16 * ci + 8 * half]) = z4;
        }
        // the three row dot products, and the state terms of this head's dq and dk
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int ln = fresh(lane), l16 = ln & 15, q16 = ln >> 4;   // lane offsets rederived here
            const int key = 16 * wave + l16;
            f32x4 pq, pu, pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * t4 + 4 * q16 + e;
                const float kv = (float)sm.K[row][key];
                pq[e] = (float)sm.Q[row][key] * qa[t4][e];
                pu[e] = kv * uu[t4][e];
                pk[e] = kv * k2[t4][e];
                dqg[t4][e] += sc * sm.eg[row] * qa[t4][e];
                dkg[t4][e] += -sm.beta[row] * sm.eg[row] * uu[t4][e] + sm.tail[row] * k2[t4][e];
            }
            pu = row_sum16(pu);
            if (GATED) {
                pq = row_sum16(pq);
                pk = row_sum16(pk);
            }
            if (l16 == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int row = 16 * t4 + 4 * q16 + e;
                    sm.ku[row][wave] = pu[e];
                    if (GATED) {
                        sm.qy[row][wave] = pq[e];
                        sm.kc[row][wave] = pk[e];
                    }
                }
            }
            sched_fence();
        }
        if (GATED) {
            const float s = wave_sum(mdm_t);
            if (lane == 0) sm.mdm[wave] = s;
        }
        __syncthreads();

        // ------------------- dq += Z K; dk += W K + W^T K + Z^T Q (W in Tt, Z in P)
#pragma unroll
        for (int t4 = 0; t4 < 4; ++t4) {
            const int ln = fresh(lane), l16 = ln & 15, q16 = ln >> 4;   // lane offsets rederived here
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32) {
                if (k0 <= 16 * t4) {   // the lower factors
                    const bf16x8 kc = frag_c(&sm.K[0][0], P128, 16 * wave, k0, l16, q16);
                    dqg[t4] = mma16(frag_r(&sm.P[0][0], P64, 16 * t4, k0, l16, q16), kc, dqg[t4]);
                    dkg[t4] = mma16(frag_r(&sm.Tt[0][0], P64, 16 * t4, k0, l16, q16), kc, dkg[t4]);
                }
                if (k0 + 32 > 16 * t4) {   // the transposed (upper) factors
                    dkg[t4] = mma16(frag_c(&sm.Tt[0][0], P64, 16 * t4, k0, l16, q16),
                                    frag_c(&sm.K[0][0], P128, 16 * wave, k0, l16, q16), dkg[t4]);
                    dkg[t4] = mma16(frag_c(&sm.P[0][0], P64, 16 * t4, k0, l16, q16),
                                    frag_c(&sm.Q[0][0], P128, 16 * wave, k0, l16, q16), dkg[t4]);
                }
            }
            sched_fence();   // one tile's operands in flight at a time (register pressure)
        }
        // this head's dbeta and dg (wave 7, lane = row)
        if (wave == 7) {
            const int r = fresh(lane);
            float xdr = 0.f, db = 0.f;
#pragma unroll
            for (int s = 0; s < 8; ++s) xdr += sm.ku[r][s];
#pragma unroll
            for (int s = 0; s < 8; ++s) db += sm.vdr[r][s];
            db -= sm.eg[r] * xdr;
#pragma unroll
            for (int s = 0; s < 4; ++s) db += sm.ag[r][s];
            const long o = (t0 + r) * a.Hv + h;
            if (r < rows) a.dbeta[o] = db;
            if (GATED) {
                float y = 0.f, cr = 0.f;
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    y += sm.qy[r][s];
                    cr += sm.kc[r][s];
                }
                cr *= sm.tail[r];
                float dgam = sc * sm.eg[r] * y - sm.beta[r] * sm.eg[r] * xdr - cr;
#pragma unroll
                for (int s = 0; s < 4; ++s) dgam += sm.aa_r[r][s] + sm.pp_r[r][s];
#pragma unroll
                for (int s = 0; s < 16; ++s) dgam += sm.aa_c[r][s] + sm.pp_c[r][s];
                // gamma_L, on the last row: e^gamma_L <M, dM'> + sum_r c_r
                const float ct = wave_sum(cr);
                if (r == BC - 1) {
                    float mm = 0.f;
#pragma unroll
                    for (int w = 0; w < 8; ++w) mm += sm.mdm[w];
                    dgam += sm.eg[BC - 1] * mm + ct;
                }
                // dg_i = sum over the rows r >= i
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const float up = __shfl_down(dgam, off);
                    if (r + off < 64) dgam += up;
                }
                if (r < rows) a.dg[o] = dgam;
            }
        }
    }
    // dq and dk of the q/k head, staged through LDS (the slice buffers, free after the last
    // head) so that each lane stores 16 bytes of a row; rows past the end are dropped by the
    // range check
    float (*stage)[BD + 4] = reinterpret_cast<float (*)[BD + 4]>(&sm.V[0][0]);
    static_assert(sizeof(float) * BC * (BD + 4) <= sizeof(sm.V) + sizeof(sm.dO) + sizeof(sm.Dl) + sizeof(sm.dR) +
                  sizeof(sm.Rt) + sizeof(sm.dDt) + sizeof(sm.Mt) + sizeof(sm.dMt), "dq/dk stage");
    const uint32_t kq_tokf = (uint32_t)a.Hqk * BD;
    const uint32_t kq_rec = ((uint32_t)(rows - 1) * kq_tokf + BD) * 4;
    const auto dq_rs = rsrc(a.dq + (t0 * a.Hqk + hq) * BD, kq_rec);
    const auto dk_rs = rsrc(a.dk + (t0 * a.Hqk + hq) * BD, kq_rec);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        if (m) __syncthreads();   // dq's stage is read
        {
            const int ln = fresh(lane), l16 = ln & 15, q16 = ln >> 4;
#pragma unroll
            for (int t4 = 0; t4 < 4; ++t4)
#pragma unroll
                for (int e = 0; e < 4; ++e) stage[16 * t4 + 4 * q16 + e][16 * wave + l16] = (m ? dkg : dqg)[t4][e];
        }
        __syncthreads();
        const int tf = fresh(tid);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int pc = tf + NTB * u, row = pc >> 5, c4 = (pc & 31) * 4;
            typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
            u32x4 v = *reinterpret_cast<const u32x4*>(&stage[row][c4]);
            if (a.rnorm) {
                // the rows are normalised ones, x_hat = x r (r = 1 / sqrt(|x|^2 + eps)):
                // dx = r (dx_hat - x_hat (x_hat . dx_hat)), the dot over the row's 32 lanes
                const bf16x4 xh = *reinterpret_cast<const bf16x4*>(m ? &sm.K[row][c4] : &sm.Q[row][c4]);
                float g4[4], x4[4], dot = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    g4[e] = __uint_as_float(v[e]);
                    x4[e] = (float)xh[e];
                    dot += x4[e] * g4[e];
                }
                dot += dpp16<0xB1>(dot);
                dot += dpp16<0x4E>(dot);
                dot += dpp16<0x141>(dot);
                dot += dpp16<0x140>(dot);
                dot += __shfl_xor(dot, 16);   // the row's other 16 lanes
                const float r = row < rows ? a.rnorm[(m ? (long)a.B * a.T * a.Hqk : 0) + (t0 + row) * a.Hqk + hq] : 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(r * (g4[e] - x4[e] * dot));
            }
            __builtin_amdgcn_raw_buffer_store_b128(v, m ? dk_rs : dq_rs, ((uint32_t)row * kq_tokf + c4) * 4, 0, 0);
        }
    }
}

}  // namespace

bool chunk_bwd_supported(const PrefillArgs& a) {
    const long span = ((long)a.T + 2 * BC) * (a.Hqk > a.Hv ? a.Hqk : a.Hv) * BD * 2;
    return a.bf16 && a.Dk == BD && a.Dv == BD && a.C == BC && !a.g_per_key && span < (1L << 31);
}

size_t chunk_bwd_workspace_bytes(const PrefillArgs& a, long ncid_l) {
    const size_t per = (size_t)ncid_l * a.Hv;
    // with the in-call normalisation, the normalised q and k (bf16) and the inverse norms of
    // their rows (fp32) come first
    const size_t nrows = (size_t)a.B * a.T * a.Hqk;
    const size_t qk = a.qk_norm ? nrows * BD * 2 * 2 + ((nrows * 2 * sizeof(float) + 255) & ~(size_t)255) : 0;
    return qk + per * BD * BD * sizeof(float) * 2 + per * 2 * BC * BC * 2;
}

namespace {
// A second stream per device for the chunk-start states: that launch needs nothing the T/P
// and carry launches produce, so it runs beside them (with few sequences it fills only part
// of the chip); the caller's stream waits for it before the gradient launch.  Fork and join
// are events, so the pattern also records into a graph captured on the caller's stream.
// The record / wait sequence is serialised per process (calls from several host threads).
struct SideStream {
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
SideStream g_side[kMaxDevices];
std::mutex g_side_mu;

// compute units of the current device (queried once per device)
int g_cus[kMaxDevices];

hipError_t cu_count(int& n) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_side_mu);
    if (!g_cus[dev]) {
        int v = 0;
        if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
        g_cus[dev] = v > 0 ? v : 1;
    }
    n = g_cus[dev];
    return hipSuccess;
}

hipError_t side_stream(SideStream*& out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    SideStream& ss = g_side[dev];
    if (!ss.stream) {
        if ((e = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess) return e;
        if ((e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess) return e;
    }
    out = &ss;
    return hipSuccess;
}
}  // namespace

hipError_t launch_chunk_bwd(const ChunkBwdArgs& a0, hipStream_t s) {
    ChunkBwdArgs a = a0;
    a.ncid = chunk_id_bound(a);
    const size_t per = (size_t)a.ncid * a.Hv;
    char* base = static_cast<char*>(a.ws);
    hipError_t e;
    if (a0.qk_norm) {
        // the in-call normalisation as a pass of its own: the whole reverse pass then runs on
        // the normalised rows (and the inverse norms of q's and k's rows), and the gradient
        // kernel takes dq, dk back through the normalisation before it stores them
        const size_t nrows = (size_t)a.B * a.T * a.Hqk, nb = nrows * BD * 2;
        float* rn = reinterpret_cast<float*>(base + 2 * nb);
        if ((e = launch_qk_norm_rows(a0, base, base + nb, rn, s)) != hipSuccess) return e;
        a.q = base;
        a.k = base + nb;
        a.qk_norm = 0;
        a.rnorm = rn;
        base += 2 * nb + ((nrows * 2 * sizeof(float) + 255) & ~(size_t)255);
    }
    float* ws = reinterpret_cast<float*>(base);
    a.states = ws;
    a.dstates = ws + per * BD * BD;
    a.tp = a.dstates + per * BD * BD;
    const long ids = a.ncid * a.Hv, qk_ids = a.ncid * a.Hqk, chains = (long)a.N * a.Hv * BNS;
    if (ids > 0x7fffffffL || chains > 0x7fffffffL) return hipErrorInvalidConfiguration;
    PrefillArgs f = a;
    f.ws = a.states;
    f.hT = nullptr;
    int cus = 0;
    if ((e = cu_count(cus)) != hipSuccess) return e;
    if (chains >= cus) {
        // The states launch alone fills the chip (one workgroup per CU), so no launch could
        // run beside it: it writes the T^T and P records itself, and the four steps run in
        // order on the caller's stream, without the T/P launch.
        f.tp_rec = a.tp;
        if ((e = launch_prefill_fused_states(f, s)) != hipSuccess) return e;
        hipLaunchKernelGGL(chunk_carry_kernel, dim3((unsigned)chains), dim3(NTC), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (qk_ids > 0) {
            if (a.g) hipLaunchKernelGGL(chunk_grad_kernel<true>, dim3((unsigned)qk_ids), dim3(NTB), 0, s, a);
            else hipLaunchKernelGGL(chunk_grad_kernel<false>, dim3((unsigned)qk_ids), dim3(NTB), 0, s, a);
        }
        return hipGetLastError();
    }
    std::lock_guard<std::mutex> lock(g_side_mu);
    SideStream* ss = nullptr;
    e = side_stream(ss);
    if (e != hipSuccess) return e;
    // 1. the state at every chunk start (the prompt kernel, outputs skipped), on the side
    //    stream once the caller's stream has reached this call
    if ((e = hipEventRecord(ss->fork, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss->stream, ss->fork, 0)) != hipSuccess) return e;
    if ((e = launch_prefill_fused_states(f, ss->stream)) != hipSuccess) return e;
    if ((e = hipEventRecord(ss->join, ss->stream)) != hipSuccess) return e;
    // 2. T^T and P per (chunk, value head)
    if ((e = launch_chunk_tp(a, a.ncid, a.tp, false, s)) != hipSuccess) return e;
    // 3. the carry per (sequence, value head, slice)
    if (chains > 0) hipLaunchKernelGGL(chunk_carry_kernel, dim3((unsigned)chains), dim3(NTC), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // 4. the gradients per (chunk, q/k head), after the states
    if ((e = hipStreamWaitEvent(s, ss->join, 0)) != hipSuccess) return e;
    if (qk_ids > 0) {
        if (a.g) hipLaunchKernelGGL(chunk_grad_kernel<true>, dim3((unsigned)qk_ids), dim3(NTB), 0, s, a);
        else hipLaunchKernelGGL(chunk_grad_kernel<false>, dim3((unsigned)qk_ids), dim3(NTB), 0, s, a);
    }
    return hipGetLastError();
}

}  // namespace dn
