// chunk_tp.hip -- the state-independent part of the chunked form on the matrix cores, for
// every chunk at once: per (chunk, value head) the masked Grams, T = (I + A)^-1 and P, stored
// in bf16 (T transposed) for the chunkwise reverse pass.  The rule is the update of the
// frankenstein "DeltaNet Attention" page (module docstring) with the gate order of the nnterp
// "linear_attention" page (LinearAttention class text), in its chunked form: per chunk,
// gamma the in-chunk inclusive sum of g, D_ri = exp(gamma_r - gamma_i) (i <= r):
//
//   A = strict_lower(diag(beta) (D o K K^T)),  T = (I + A)^-1,  P = lower(D o Q K^T)
//
// One persistent kernel: as many workgroups of 4 waves as fit on the chip walk the (chunk,
// value head) items.
#include "chunk_ops.h"

namespace dn {
namespace {
using namespace ck;

// ============================================ T^T and P per (chunk, value head)
constexpr int NTP = 256;
constexpr int CU_LDS = 111;        // packed batches up to this many sequences look up chunks in LDS
                                   // (LDS is taken in 2 KiB units: at d_k = 64 three workgroups fit a CU)

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
    if (a.Dk != 128) return hipErrorInvalidValue;   // the reverse pass takes d = 128
    launch(chunk_tp_kernel<128>);
    return hipGetLastError();
}

}  // namespace dn
