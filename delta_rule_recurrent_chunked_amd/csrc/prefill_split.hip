// prefill_split.hip -- the prompt in two launches on the matrix cores (bf16 operands, fp32
// accumulation), for bf16 inputs with d_k = d_v = 64 and 64-token chunks; the fused one-launch
// kernel (prefill_fused.hip) covers d = 128.  The rule is the update of the frankenstein
// "DeltaNet Attention" page (module docstring) with the gate order of the nnterp
// "linear_attention" page (LinearAttention class text), in its chunked form: per chunk, M the
// state at its start (key-major), gamma the in-chunk inclusive sum of g,
// D_ri = exp(gamma_r - gamma_i) (i <= r), tail_r = exp(gamma_L - gamma_r):
//
//   A = strict_lower(diag(beta) (D o K K^T)),  T = (I + A)^-1,  P = lower(D o Q K^T)
//   R = diag(beta) (V - diag(e^gamma) K M),  Delta = T R
//   O = scale (diag(e^gamma) Q M + P Delta),  M' = e^{gamma_L} M + K^T diag(tail) Delta
//
// 1. chunk_tp_kernel, one workgroup per (chunk, value head), every chunk at once: the masked
//    Grams and T (the state-independent part), T^T and P to the workspace in bf16.  The same
//    kernel (d = 128) gives the chunkwise reverse pass its T and P.
// 2. split_chain_kernel, one workgroup of 8 waves per (sequence, value head, 32 value
//    columns) walks the chunks in order with its columns of M in MFMA accumulators.  Per
//    chunk three steps between barriers: X = K M and Y = Q M, then R (stored transposed);
//    Delta = T R (stored transposed, and scaled by tail); O = scale (e^gamma Y + P Delta)
//    (staged in LDS, stored a step later with 16 bytes a lane) and the state update, while
//    the next chunk's K, Q, V, T^T, P go into the other half of double-buffered LDS.
#include "chunk_ops.h"

namespace dn {
namespace {
using namespace ck;

// ============================================ T^T and P per (chunk, value head)
constexpr int NTP = 256;
constexpr int CU_LDS = 111;        // packed batches up to this many sequences look up chunks in LDS
                                   // (at d_k = 64 three workgroups then fit a CU, with LDS taken in 2 KiB units)

template <int DK>
struct alignas(16) PrepSmem {
    __bf16 K[BC][DK + 16], Q[BC][DK + 16];
    __bf16 Tt[BC][P64];            // T^T, T = (I + A)^-1 lower triangular
    __bf16 P[BC][P64];             // P = lower(D o Q K^T)
    __bf16 G[BC][P64];             // D o K K^T, strictly lower
    _Float16 Ad[4][ADP];           // A's diagonal blocks (strictly lower, packed by rows)
    float beta[BC], gam[BC];
    int cu[CU_LDS + 1];            // cu_seqlens of a packed batch of at most CU_LDS sequences
};

// one item's K and Q pieces (16 bytes each: piece tid + NTP u, row = piece / (DK / 8)), and
// beta and g of token lane (wave 0)
template <int DK>
struct PrepIn {
    uint4 k[BC * DK / 8 / NTP], q[BC * DK / 8 / NTP];
    float beta, g;
    int h, cid;
};

// Persistent: workgroup w takes items w, w + grid, ... (item = record number cid * Hv + h),
// skipping numbers no chunk takes, and loads the next item's K, Q, beta and g while it
// works on the current one.
template <int DK>
__global__ __launch_bounds__(NTP, DK == 64 ? 3 : 2) void chunk_tp_kernel(PrefillArgs a, void* tp, long ncid, int head_major) {
    __shared__ PrepSmem<DK> sm;
    constexpr int PK = DK + 16, NPC = BC * DK / 8 / NTP;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q16 = lane >> 4;
    const int ids = (int)(ncid * a.Hv);   // below 2^31 (checked by the launcher)
    const uint32_t kq_tok = (uint32_t)a.Hqk * DK * 2, s_tok = (uint32_t)a.Hv * 4;
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    const bool cu_lds = a.cu && a.N <= CU_LDS;
    if (cu_lds)
        for (int i = tid; i <= a.N; i += NTP) sm.cu[i] = a.cu[i];
    const int cps = (a.T + BC - 1) / BC;   // chunks per row of a batch of rows

    // the blocks above the diagonal of P and G, and below it of T^T, stay zero for every item
    for (int i = tid; i < BC * P64 / 8; i += NTP) {
        reinterpret_cast<uint4*>(&sm.Tt[0][0])[i] = z4;
        reinterpret_cast<uint4*>(&sm.P[0][0])[i] = z4;
        reinterpret_cast<uint4*>(&sm.G[0][0])[i] = z4;
    }
    // This workgroup's items in increasing order: a cursor over (item, chunk number cid, head
    // h) and the sequence n of chunk cid, moved forward without divisions.
    const int sc = gridDim.x / a.Hv, sh = gridDim.x - sc * a.Hv;
    int u_item = blockIdx.x, u_cid = u_item / a.Hv, u_h = u_item - u_cid * a.Hv, u_n = 0;
    int u_c = 0, u_L = 0;
    long u_bos = 0;
    auto cu_at = [&](int i) -> int { return cu_lds ? sm.cu[i] : a.cu[i]; };
    // chunk c of sequence n, its first token and length for u_cid; false for a number no
    // chunk takes
    auto place = [&]() -> bool {
        if (!a.cu) {
            while (u_cid >= (u_n + 1) * cps) ++u_n;
            u_c = u_cid - u_n * cps;
            u_bos = (long)u_n * a.T;
            u_L = a.T;
            return true;
        }
        while (u_n + 1 < a.N && cu_at(u_n + 1) / BC + u_n + 1 <= u_cid) ++u_n;
        u_bos = cu_at(u_n);
        u_L = cu_at(u_n + 1) - (int)u_bos;
        u_c = u_cid - ((int)u_bos / BC + u_n);
        return u_c * BC < u_L;
    };
    auto advance = [&]() {
        u_item += gridDim.x;
        u_h += sh;
        u_cid += sc;
        if (u_h >= a.Hv) {
            u_h -= a.Hv;
            ++u_cid;
        }
    };
    auto seek = [&]() {   // to the next item a chunk takes (or past the last)
        while (u_item < ids && !place()) advance();
    };
    // the cursor's item's inputs, through descriptors that cover exactly the chunk's tokens
    // (rows past the sequence's end read zeros)
    auto fetch = [&](PrepIn<DK>& f) {
        const int hq = u_h / (a.Hv / a.Hqk);
        const long t0 = u_bos + (long)u_c * BC;
        const int rows = min(BC, u_L - u_c * BC);
        const auto k_rs = rsrc(static_cast<const __bf16*>(a.k) + (t0 * a.Hqk + hq) * DK, (uint32_t)(rows - 1) * kq_tok + DK * 2);
        const auto q_rs = rsrc(static_cast<const __bf16*>(a.q) + (t0 * a.Hqk + hq) * DK, (uint32_t)(rows - 1) * kq_tok + DK * 2);
#pragma unroll
        for (int u = 0; u < NPC; ++u) {
            const int pc = tid + NTP * u;
            const uint32_t off = (uint32_t)(pc / (DK / 8)) * kq_tok + (pc % (DK / 8)) * 16;
            f.k[u] = ld128(k_rs, off, 0);
            f.q[u] = ld128(q_rs, off, 0);
        }
        if (wave == 0) {
            const uint32_t nb = (uint32_t)(rows - 1) * s_tok + 4;
            f.beta = ld32(rsrc(a.beta + t0 * a.Hv + u_h, nb), (uint32_t)lane * s_tok, 0);
            f.g = ld32(rsrc(a.g ? a.g + t0 * a.Hv + u_h : a.beta, a.g ? nb : 0), (uint32_t)lane * s_tok, 0);
        }
        f.h = u_h;
        f.cid = u_cid;
    };

    __syncthreads();   // sm.cu is in
    PrepIn<DK> f;
    seek();
    bool have = u_item < ids;
    if (have) fetch(f);
    for (int iter = 0; have; ++iter) {
        const int h = f.h, cid = f.cid;
#pragma unroll
        for (int u = 0; u < NPC; ++u) {
            const int pc = tid + NTP * u, row = pc / (DK / 8), cg = pc % (DK / 8);
            *reinterpret_cast<uint4*>(&sm.K[row][cg * 8]) = f.k[u];
            *reinterpret_cast<uint4*>(&sm.Q[row][cg * 8]) = f.q[u];
        }
        if (wave == 0) {
            float gl;
            sm.gam[lane] = gamma_scan(f.g, gl);
            sm.beta[lane] = f.beta;
        }
        __syncthreads();
        advance();
        seek();
        const bool more = u_item < ids;
        if (more) fetch(f);   // lands while this item is worked

        // 20 lower tiles (incl. the diagonal), five per wave: t < 10 of D o K K^T (strictly
        // lower), t >= 10 of P
        f32x4 acc[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int t = wave + 4 * i;
            int ri, ci;
            lower_tile(t % 10, ri, ci);
            const __bf16* A = t < 10 ? &sm.K[0][0] : &sm.Q[0][0];
            acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32)
                acc[i] = mma16(frag_r(A, PK, 16 * ri, k0, l16, q16), frag_r(&sm.K[0][0], PK, 16 * ci, k0, l16, q16), acc[i]);
        }
        float gc[5];
        f32x4 gr[5], bt[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) {   // the decay sums and write strengths first (one round trip)
            const int t = wave + 4 * i;
            int ri, ci;
            lower_tile(t % 10, ri, ci);
            gc[i] = sm.gam[16 * ci + l16];
            gr[i] = *reinterpret_cast<const f32x4*>(&sm.gam[16 * ri + 4 * q16]);
            bt[i] = *reinterpret_cast<const f32x4*>(&sm.beta[16 * ri + 4 * q16]);
        }
#pragma unroll
        for (int i = 0; i < 5; ++i) {
            const int t = wave + 4 * i;
            int ri, ci;
            lower_tile(t % 10, ri, ci);
            const int col = 16 * ci + l16;
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {   // branch-free: the factor is formed for every entry
                const int row = 16 * ri + 4 * q16 + e;
                const bool keep = t < 10 ? col < row : col <= row;
                const float x = __expf(fminf(gr[i][e] - gc[i], 0.f)) * acc[i][e];
                v[e] = keep ? x : 0.f;
            }
            put_tile(t < 10 ? &sm.G[0][0] : &sm.P[0][0], P64, ri, ci, v, l16, q16);
            if (t < 10 && ri == ci) {   // A's diagonal block ri in fp16, strictly lower, packed
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int lr = 4 * q16 + e, lc = l16;
                    if (lc < lr) sm.Ad[ri][lr * (lr - 1) / 2 + lc] = (_Float16)(bt[i][e] * v[e]);
                }
            }
        }
        __syncthreads();

        // T = (I + A)^-1 on one wave (a different one, so a different SIMD, from item to
        // item), stored transposed
        if (wave == ((iter + (int)blockIdx.x) & 3)) {
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
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const bool lo = q16 < 2;   // k = 16 padded to the instruction's 32
            // level 1: T21 = -T22 (A21 T11) within each 32x32 diagonal block (base 0, 32);
            // T's block (b + 1, b) is T^T's block (b, b + 1)
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int base = 32 * hb;
                const bf16x8 af = lo ? scale_r(frag_r(&sm.G[0][0], P64, base + 16, base, l16, q16),
                                               sm.beta[base + 16 + l16]) : zero8();
                const bf16x8 bf = lo ? frag_r(&Tt[0][0], P64, base, base, l16, q16) : zero8();
                const f32x4 X1 = mma16(af, bf, z);
                const bf16x8 tf = lo ? frag_c(&Tt[0][0], P64, base + 16, base + 16, l16, q16) : zero8();
                const f32x4 Y1 = mma16(tf, acc_to_b(X1, z), z);
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
                                       frag_r(&Tt[0][0], P64, 16 * tj, 0, l16, q16), z);
#pragma unroll
            for (int ti = 0; ti < 2; ++ti)
#pragma unroll
                for (int tj = 0; tj < 2; ++tj) {
                    const f32x4 Y2 = mma16(frag_c(&Tt[0][0], P64, 32 + 16 * ti, 32, l16, q16),
                                           acc_to_b(X2[0][tj], X2[1][tj]), z);
                    st4(&Tt[16 * tj + l16][32 + 16 * ti + 4 * q16], -Y2[0], -Y2[1], -Y2[2], -Y2[3]);
                }
        }
        __syncthreads();

        __bf16* out = static_cast<__bf16*>(tp) + (head_major ? h * ncid + cid : (long)cid * a.Hv + h) * (2L * BC * BC);
#pragma unroll
        for (int u = 0; u < 2 * BC * 8 / NTP; ++u) {
            const int pc = tid + NTP * u;
            const int m = pc >> 9, r = (pc >> 3) & 63, cg = pc & 7;
            const __bf16* src = m ? &sm.P[r][cg * 8] : &sm.Tt[r][cg * 8];
            *reinterpret_cast<uint4*>(out + m * BC * BC + r * BC + cg * 8) = *reinterpret_cast<const uint4*>(src);
        }
        have = more;
    }
}


// ============================================================ the chunk chain
constexpr int NTS = 512;           // 8 waves
constexpr int PF = 3;              // chunks loaded ahead into registers
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int DK>
struct alignas(16) ChainSmem {
    __bf16 K[2][BC][DK + 16], Q[2][BC][DK + 16];   // the current chunk and the next
    __bf16 V[2][BC][P32];                         // the slice of V
    __bf16 Tt[2][BC][P64], P[2][BC][P64];
    __bf16 Rt[BS][P64];            // R^T
    __bf16 Dt[BS][P64];            // Delta^T
    __bf16 Et[BS][P64];            // (diag(tail) Delta)^T
    __bf16 Mt[BS][DK + 16];        // the state slice at the chunk start, transposed
    __bf16 Os[BC][BS + 8];         // O of the chunk, staged for 16-byte stores
    float beta[2][BC], eg[2][BC], tail[2][BC], egl[2][4];
};

// one chunk's inputs in registers: 16-byte pieces t + 512 u of K and Q (row = piece /
// (DK / 8)), 8-byte piece t of V's slice (row = t / 8), 16-byte piece t of T^T and of P
// (row = t / 8), beta and g of token t % 64.  Every lane loads in every step, so that the
// waits for the oldest loads can count the younger ones.
template <int DK>
struct ChainIn {
    uint4 k[DK / 64], q[DK / 64], v, t, p;
    float beta, g;
};

template <int DK, bool GATED>
__global__ __launch_bounds__(NTS, 1) void split_chain_kernel(PrefillArgs a, const void* tp, long ncid) {
    __shared__ ChainSmem<DK> sm;
    constexpr int PK = DK + 16, MT = DK / 64, DV = DK;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, q16 = lane >> 4;
    // workgroup -> (sequence, value head, slice), the slices of the value heads of one q/k
    // head one after another on one XCD when the (sequence, q/k head) count is a multiple of 8
    constexpr int NSL = DV / BS;
    const int grp = a.Hv / a.Hqk, qchains = a.N * a.Hqk;
    int slice, nh;
    if ((qchains & 7) == 0) {
        const int y = blockIdx.x >> 3, t = y / NSL;
        const int qc = (blockIdx.x & 7) + 8 * (t / grp);
        slice = y % NSL;
        nh = (qc / a.Hqk) * a.Hv + (qc % a.Hqk) * grp + t % grp;
    } else {
        slice = blockIdx.x % NSL;
        nh = blockIdx.x / NSL;
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

    // streams over this sequence (range-checked: rows past its end read zeros, stores drop)
    const uint32_t kq_tok = (uint32_t)a.Hqk * DK * 2, v_tok = (uint32_t)a.Hv * DV * 2, s_tok = (uint32_t)a.Hv * 4;
    const long kq0 = (bos * a.Hqk + hq) * DK, v0 = (bos * a.Hv + h) * DV + j0, s0 = bos * a.Hv + h;
    const uint32_t kq_end = L > 0 ? (uint32_t)((L - 1) * kq_tok + DK * 2) : 0;
    const uint32_t v_end = L > 0 ? (uint32_t)((L - 1) * v_tok + BS * 2) : 0;
    const uint32_t s_end = L > 0 ? (uint32_t)((L - 1) * s_tok + 4) : 0;
    const auto k_rs = rsrc(static_cast<const __bf16*>(a.k) + kq0, kq_end);
    const auto q_rs = rsrc(static_cast<const __bf16*>(a.q) + kq0, kq_end);
    const auto v_rs = rsrc(static_cast<const __bf16*>(a.v) + v0, v_end);
    const auto o_rs = rsrc(static_cast<__bf16*>(a.o) + v0, v_end);
    const auto b_rs = rsrc(a.beta + s0, s_end);
    const auto g_rs = rsrc(a.g ? a.g + s0 : a.beta + s0, a.g ? s_end : 0);
    uint32_t kq_off[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u) {
        const int pc = tid + NTS * u;
        kq_off[u] = (uint32_t)(pc / (DK / 8)) * kq_tok + (pc % (DK / 8)) * 16;
    }
    const int vp = tid & 255;
    const uint32_t v_off = (uint32_t)(vp >> 2) * v_tok + (vp & 3) * 16;
    const uint32_t sc_off = (uint32_t)lane * s_tok;
    // T^T and P of this head's chunks, one 16 KiB record a chunk (head-major records)
    constexpr uint32_t REC = 2 * BC * BC * 2;
    const auto tp_rs = rsrc(static_cast<const unsigned char*>(tp) + ((long)h * ncid + cid0) * REC, (uint32_t)nc * REC);

    auto fetch = [&](int c, ChainIn<DK>& f) {
        const uint32_t ck = (uint32_t)c * BC * kq_tok, cv = (uint32_t)c * BC * v_tok, cs = (uint32_t)c * BC * s_tok;
#pragma unroll
        for (int u = 0; u < MT; ++u) {
            f.k[u] = ld128(k_rs, kq_off[u], ck);
            f.q[u] = ld128(q_rs, kq_off[u], ck);
        }
        if (tid < 256) f.v = ld128(v_rs, v_off, cv);
        f.t = ld128(tp_rs, 16 * tid, (uint32_t)c * REC);
        f.p = ld128(tp_rs, 16 * tid + REC / 2, (uint32_t)c * REC);
        if (wave == 0) {
            f.beta = ld32(b_rs, sc_off, cs);
            f.g = ld32(g_rs, sc_off, cs);
        }
    };
    auto put_in = [&](const ChainIn<DK>& f, int b) {
#pragma unroll
        for (int u = 0; u < MT; ++u) {
            const int pc = tid + NTS * u, row = pc / (DK / 8), cg = pc % (DK / 8);
            *reinterpret_cast<uint4*>(&sm.K[b][row][cg * 8]) = f.k[u];
            *reinterpret_cast<uint4*>(&sm.Q[b][row][cg * 8]) = f.q[u];
        }
        if (tid < 256) *reinterpret_cast<uint4*>(&sm.V[b][vp >> 2][(vp & 3) * 8]) = f.v;
        *reinterpret_cast<uint4*>(&sm.Tt[b][tid >> 3][(tid & 7) * 8]) = f.t;
        *reinterpret_cast<uint4*>(&sm.P[b][tid >> 3][(tid & 7) * 8]) = f.p;
        if (wave == 0) {
            float gl = 0.f, gv = 0.f;
            if (GATED) gv = gamma_scan(f.g, gl);
            const float eg = __expf(gv);
            sm.beta[b][lane] = f.beta;
            sm.eg[b][lane] = eg;
            sm.tail[b][lane] = __expf(gl - gv);
            if (lane == 0) sm.egl[b][0] = __expf(gl);
        }
    };

    // this slice of M in MFMA accumulators: wave w holds tiles u of key block 4 u + (w >> 1),
    // column block w & 1 (keys 16 ki + 4 q16 + e, column 16 (w & 1) + l16 of the slice)
    f32x4 M[MT];
    const int cj = wave & 1;
#pragma unroll
    for (int u = 0; u < MT; ++u) {
        const int ki = 4 * u + (wave >> 1);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            M[u][e] = a.h0 ? a.h0[((long)nh * DK + 16 * ki + 4 * q16 + e) * DV + j0 + 16 * cj + l16] : 0.f;
    }
    auto put_mt = [&]() {
#pragma unroll
        for (int u = 0; u < MT; ++u) put_tile_t(&sm.Mt[0][0], PK, 4 * u + (wave >> 1), cj, M[u], l16, q16);
    };
    auto store_o = [&](int c) {   // the staged O of chunk c: 64 rows x eight 8-byte pieces
        if (tid < 256)
            __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(&sm.Os[vp >> 2][(vp & 3) * 8]), o_rs,
                                                   v_off, (uint32_t)c * BC * v_tok, 0);
    };

    // chunk j's inputs wait in register set j % PF from PF chunks ahead (the chain's step
    // is shorter than a load's latency) until they go into LDS a chunk ahead
    ChainIn<DK> f[PF];
    put_mt();
    if (nc > 0) {
        fetch(0, f[0]);
        put_in(f[0], 0);
#pragma unroll
        for (int j = 1; j <= PF; ++j) fetch(min(j, nc - 1), f[j % PF]);   // past the end: unused
    }
    __syncthreads();
    const int ti = wave >> 1, tj = wave & 1;   // this wave's 16 x 16 tile of a 64 x 32 product
    for (int c0 = 0; c0 < nc; c0 += PF)
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int c = c0 + u;
        if (c >= nc) break;
        ChainIn<DK>& fn = f[(u + 1) % PF];   // chunk c + 1
        const int b = c & 1;
        // ------------------------------ X = K M, Y = Q M; R = diag(beta) (V - e^gamma X)
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
        {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += 32) {
                const bf16x8 mf = frag_r(&sm.Mt[0][0], PK, 16 * tj, k0, l16, q16);
                x = mma16(frag_r(&sm.K[b][0][0], PK, 16 * ti, k0, l16, q16), mf, x);
                y = mma16(frag_r(&sm.Q[b][0][0], PK, 16 * ti, k0, l16, q16), mf, y);
            }
            f32x4 r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * ti + 4 * q16 + e;
                r[e] = sm.beta[b][row] * ((float)sm.V[b][row][16 * tj + l16] - sm.eg[b][row] * x[e]);
            }
            put_tile_t(&sm.Rt[0][0], P64, ti, tj, r, l16, q16);
        }
        __syncthreads();
        // ------------------------------------------ Delta = T R (and diag(tail) Delta)
        {
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32)
                if (k0 <= 16 * ti) d = mma16(frag_c(&sm.Tt[b][0][0], P64, 16 * ti, k0, l16, q16),
                                             frag_r(&sm.Rt[0][0], P64, 16 * tj, k0, l16, q16), d);
            put_tile_t(&sm.Dt[0][0], P64, ti, tj, d, l16, q16);
#pragma unroll
            for (int e = 0; e < 4; ++e) d[e] *= sm.tail[b][16 * ti + 4 * q16 + e];
            put_tile_t(&sm.Et[0][0], P64, ti, tj, d, l16, q16);
        }
        __syncthreads();
        // ------------------- O = scale (e^gamma Y + P Delta); M <- e^gamma_L M + K^T diag(tail) Delta
        {
            f32x4 pd = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < BC; k0 += 32)
                if (k0 <= 16 * ti) pd = mma16(frag_r(&sm.P[b][0][0], P64, 16 * ti, k0, l16, q16),
                                              frag_r(&sm.Dt[0][0], P64, 16 * tj, k0, l16, q16), pd);
            f32x4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = sc * (sm.eg[b][16 * ti + 4 * q16 + e] * y[e] + pd[e]);
            put_tile(&sm.Os[0][0], BS + 8, ti, tj, o, l16, q16);
            const float gl = sm.egl[b][0];
#pragma unroll
            for (int u = 0; u < MT; ++u) {
                const int ki = 4 * u + (wave >> 1);
                f32x4 acc = M[u] * gl;
#pragma unroll
                for (int k0 = 0; k0 < BC; k0 += 32)
                    acc = mma16(frag_c(&sm.K[b][0][0], PK, 16 * ki, k0, l16, q16),
                                frag_r(&sm.Et[0][0], P64, 16 * cj, k0, l16, q16), acc);
                M[u] = acc;
            }
        }
        // the next chunk's inputs into the other buffers (read a chunk ago), M into LDS (read
        // before the last two barriers)
        if (c + 1 < nc) put_in(fn, b ^ 1);
        fetch(min(c + 1 + PF, nc - 1), fn);
        put_mt();
        __syncthreads();
        store_o(c);
    }
    if (a.hT) {
#pragma unroll
        for (int u = 0; u < MT; ++u) {
            const int ki = 4 * u + (wave >> 1);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                a.hT[((long)nh * DK + 16 * ki + 4 * q16 + e) * DV + j0 + 16 * cj + l16] = M[u][e];
        }
    }
}

}  // namespace

hipError_t launch_chunk_tp(const PrefillArgs& a, long ncid, void* tp, bool head_major, hipStream_t s) {
    const long ids = ncid * a.Hv;
    if (ids > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (ids == 0) return hipSuccess;
    const int hm = head_major ? 1 : 0;
    // persistent: as many workgroups as fit on the chip at once (LDS bound), at most one per item
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    auto launch = [&](auto kernel) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, NTP, 0) != hipSuccess || per_cu < 1) per_cu = 1;
        const long grid = min(ids, (long)cus * per_cu);
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(NTP), 0, s, a, tp, ncid, hm);
    };
    if (a.Dk == 64) launch(chunk_tp_kernel<64>);
    else if (a.Dk == 128) launch(chunk_tp_kernel<128>);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

bool prefill_split_supported(const PrefillArgs& a) {
    // buffer offsets are 32-bit: a sequence's tokens plus a chunk, and its T / P records
    const long span = ((long)a.T + 2 * BC) * (a.Hqk > a.Hv ? a.Hqk : a.Hv) * a.Dk * 2;
    const long recs = ((long)a.T / BC + 2) * (2 * BC * BC * 2);
    return a.bf16 && a.Dk == 64 && a.Dv == 64 && a.C == BC && !a.g_per_key && !a.qk_norm && span < (1L << 31) &&
           recs < (1L << 31);
}

// chunk numbers in use: exact for a batch of rows; for packed sequences (only B = 1 packs)
// the numbering stays below T / 64 + N + 1 (the bound holds before cu_seqlens is known)
static long split_chunk_bound(const PrefillArgs& a) {
    const long rows = (long)a.B * (((long)a.T + BC - 1) / BC);
    if (a.B != 1) return rows;
    const long packed = (long)a.T / BC + a.N + 1;
    return rows > packed ? rows : packed;
}

size_t prefill_split_workspace_bytes(const PrefillArgs& a) {
    return prefill_split_supported(a) ? (size_t)split_chunk_bound(a) * a.Hv * 2 * BC * BC * 2 : 0;
}

hipError_t launch_prefill_split(const PrefillArgs& a, hipStream_t s) {
    // exact now that cu_seqlens is known (never above the bound the workspace was sized for)
    const long ncid = chunk_id_bound(a);
    hipError_t e = launch_chunk_tp(a, ncid, a.ws, true, s);
    if (e != hipSuccess) return e;
    const long blocks = (long)a.N * a.Hv * (a.Dv / BS);
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (blocks > 0) {
        if (a.g) hipLaunchKernelGGL((split_chain_kernel<64, true>), dim3((unsigned)blocks), dim3(NTS), 0, s, a, a.ws, ncid);
        else hipLaunchKernelGGL((split_chain_kernel<64, false>), dim3((unsigned)blocks), dim3(NTS), 0, s, a, a.ws, ncid);
    }
    return hipGetLastError();
}

}  // namespace dn
