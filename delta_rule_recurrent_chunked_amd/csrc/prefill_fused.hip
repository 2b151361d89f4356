// prefill_fused.hip -- one-kernel chunked prefill of the gated delta rule on the gfx950
// matrix cores (bf16 operands, fp32 accumulation), for bf16 inputs with Dk = Dv = 128 or
// Dk = Dv = 64 (the head size D is a template parameter) and 64-token chunks.
//
// The algebra is the chunked form of the update on the frankenstein "DeltaNet
// Attention" page (module docstring), with the gate order of the nnterp
// "linear_attention" page.  Inside a chunk of n <= 64 tokens, with the state slice M
// (key-major, S^T) at the chunk start and gamma_r = sum_{i<=r} g_i:
//
//   A_ri  = beta_r exp(gamma_r - gamma_i) k_r.k_i (i < r),   T = (I + A)^{-1}
//   R     = diag(beta) (V - diag(exp(gamma)) K M)
//   Delta = T R                                   (row r: beta_r x prediction error)
//   O     = scale (diag(exp(gamma)) Q M + P Delta),  P_ri = exp(gamma_r - gamma_i) q_r.k_i (i <= r)
//   M    <- exp(gamma_last) M + K^T diag(exp(gamma_last - gamma)) Delta
//
// With the in-rule normalisation (q, k -> x / sqrt(|x|^2 + eps)) the kernel keeps the raw
// q and k as matrix operands and folds the norms into per-token factors.  With
// s_r = 1 / |k_r| and Delta'_r = s_r Delta_r, row r of (I + A) Delta = R times s_r gives
//
//   A'_ri = beta_r s_r^2 exp(gamma_r - gamma_i) k_r.k_i,     (I + A') Delta' = R'
//   R'_r  = beta_r s_r v_r - beta_r s_r^2 exp(gamma_r) (K M)_r
//   O_r   = scale / |q_r| (exp(gamma_r) (Q M)_r + (P Delta')_r)
//   M    <- exp(gamma_last) M + K^T diag(exp(gamma_last - gamma)) Delta'
//
// with P and the state update in raw q and k: only the per-token scalars change.  The
// squared norms come from the matrix cores: |k_r|^2 is the diagonal of the K K^T tiles the
// UT-inverse wave builds for A's diagonal blocks, and |q_r|^2 the diagonal of Q Q^T tiles
// the output waves add to their P products.
//
// One workgroup of eight waves per (sequence, value head, 32-column slice of the state).
// The value columns of the state are independent, so slices never exchange data; the
// chunk-local matrices (A, T, P) are recomputed by each slice's workgroup, which keeps
// every intermediate on chip: HBM sees q, k, v, beta, g once and o once.
//
// Each chunk takes one "phase" of two halves separated by workgroup barriers.  In phase j:
//
//   wave      SIMD  first half (.1)                    second half (.2)
//   0, 1      0, 2  chain, chunk j: X = K M, R         Delta, state update
//   3, 7      3     output: O of chunk j - 1 (to HBM),  P of chunk j
//                   Y = Q M
//                   (each wave: two 16-token row blocks, all 32 columns)
//   4, 5      0, 2  loaders: K, scalars of j + 1       Q, V of j + 1; fetch j + 3
//   6         1     T of chunk j (UT inverse of A)     A of chunk j + 1, diagonal tiles
//   2         1     A of chunk j, rows 32..63 x        A of chunk j + 1, tiles (0,1), (2,3)
//                   columns 0..31 (the chain's A_BL)   (the UT inverse's A21 blocks)
//
// Waves w and w + 4 share a SIMD (the hardware deals waves 0-3 to SIMDs 0, 2, 1, 3; read
// from the HW_ID register).  The UT inverse, the longest serial step, has its SIMD to
// itself in the first half; the
// wave that runs it builds A's diagonal tiles itself and keeps them in registers.  The
// chain waves and that wave raise their wave priority: their instructions issue first.
//
// Chain wave w owns state columns 16w .. 16w+15 of the slice as D / 16 16x16 fp32
// accumulator tiles (one per 16 keys); products that consume its results take them as B operands through
// register lane swaps (acc_to_b).  The output waves get the chain's bf16 state and Delta
// fragments through LDS and use them as the A operands of the transposed products; P stays
// in their registers, and store O to HBM from their registers.  LDS holds K and Q
// double-buffered and one V, T and A tile.
#include <type_traits>

#include "internal.h"
#include "mfma_ops.h"

namespace dn {
namespace {

constexpr int FC = 64;             // chunk
constexpr int DVS = 32;            // state columns per workgroup
constexpr int CW = 16;             // state columns per chain wave
constexpr int NCW = DVS / CW;      // chain waves
// bf16 row pitches.  gfx950's LDS serves a 16-byte-per-lane read 32 lanes at a time
// across 128 four-byte banks (measured: this model predicts which pitches run
// conflict-free).  An operand read takes 16 rows x 2 chunks per 32 lanes, so the 16 row
// offsets (pitch in dwords x row, mod 128) must be distinct multiples of 8: 72 dwords for
// the 128-wide K and Q rows, 40 for the 64-wide T and A rows.  V (read only transposed,
// 16 rows x 8 dwords) takes 24.
constexpr int CPITCH = FC + 16;
constexpr int VPITCH = DVS + 16;
// A's diagonal blocks, 120 packed fp16 entries each (+ a spare slot), 68 dwords apart: the
// four blocks' broadcast reads fall on distinct banks.
constexpr int ADPITCH = 136;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
constexpr int NT = 512;            // threads (8 waves)
constexpr int NLD = 128;           // loader threads (waves 4, 5)

// What depends on the head size D = Dk = Dv (64 or 128): the K and Q rows, the 32-key steps
// of a product over keys, the 16-key tiles of a state slice, the slices of a head, and the
// 16-byte pieces of K (and Q) each loader lane moves per chunk.
template <int D>
struct Dims {
    static_assert(D == 64 || D == 128, "head size");
    static constexpr int KPITCH = D + 16;          // bf16 pitch of K and Q rows (72 or 40 dwords)
    static constexpr int NKS = D / 32;             // 32-key steps
    static constexpr int NKT = D / 16;             // 16-key tiles of the state
    static constexpr int NSL = D / DVS;            // slices per (sequence, value head)
    static constexpr int PPR = D / 8;              // 16-byte pieces per K row (a power of 2)
    static constexpr int PPR_LOG = D == 128 ? 4 : 3;
    static constexpr int NKP = FC * PPR / NLD;     // K pieces per loader lane
};

// Per-token scalars of a chunk.  With e(I) = 16 I + 15 the last token of 16-token block I,
// exp(gamma_r - gamma_i) for i in block I < block of r factors as
// F1[I][r] * F2[i] = exp(gamma_r - gamma_e(I)) * exp(gamma_e(I) - gamma_i), both <= 1 when
// g <= 0, so the masks of the blocks below the diagonal need no exponentials.
// With the in-rule normalisation (s_r = 1 / sqrt(|k_r|^2 + eps)): SC_B1 = beta_r s_r,
// SC_B2 = beta_r s_r^2 exp(gamma_r), SC_S2 = s_r^2.
enum Sc { SC_BETA = 0, SC_GAM = 1, SC_EG = 2, SC_TAIL = 3, SC_F2 = 4, SC_F1 = 5,
          SC_B1 = 8, SC_B2 = 9, SC_S2 = 10, SC_N = 11 };

template <int D>
struct alignas(16) FusedSmem {
    __bf16 K[2][FC][Dims<D>::KPITCH];   // chunk keys, token-major (chunk j in K[j & 1])
    __bf16 Q[2][FC][Dims<D>::KPITCH];   // chunk queries, token-major
    __bf16 V[FC][VPITCH];          // value slice of the next chunk the chain reads
    __bf16 Tt[FC][CPITCH];         // T^T of the chunk being processed
    __bf16 Ab[FC][CPITCH];         // A in bf16 (blocks below the 16x16 block diagonal)
    _Float16 Ad[4][ADPITCH];       // A's diagonal 16x16 blocks, fp16, strictly lower part
                                   //   packed by rows: (r, m), m < r, at r (r - 1) / 2 + m
    bf16x8 mb[2][NCW][Dims<D>::NKS][64];   // chain -> output: bf16 state as B operands (k = key)
    bf16x8 dd[NCW][2][64];         // chain -> output: Delta as B operands (k = token)
    float sc[3][SC_N][FC];         // per chunk (slot j % 3): the Sc scalars
    int seq_len[NT];               // packed batches of up to 512 sequences: their lengths,
    int rank_seq[NT];              //   and the sequence of each length rank
    f32x4 pdec[2][4][64];          // with decay, chunk j's (slot j & 1) factors exp(gamma_r -
                                   //   gamma_i) of the four diagonal 16x16 tiles, lane layout
                                   //   of the Gram tiles: A's wave forms them, P's waves reuse them
};

template <int D>
struct LoadSet {
    uint4 k[Dims<D>::NKP], q[Dims<D>::NKP], v[2];
    float beta, g;
};

struct Geo {  // where this workgroup works
    long bos, eos;
    int n, h, hq, j0, nh, nchunks;
};


// ------------------------------------------------------------------------ loaders
// Raw buffer loads: the descriptor of each stream covers exactly the sequence's own
// tokens, so loads past the sequence end (the ragged last chunk and the chunks the loop
// fetches beyond the last) return zeros by the hardware range check: every load is
// unconditional, and each lane keeps one 32-bit offset per 16-byte piece.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int D>
struct Streams {
    __amdgpu_buffer_rsrc_t k, q, v, beta, g;
    uint32_t kq_chunk, v_chunk, s_chunk;   // bytes per chunk of 64 tokens
    uint32_t off_kq[Dims<D>::NKP], off_v[2], off_s;   // this lane's piece offsets within a chunk
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int D>
__device__ __forceinline__ void make_streams(const PrefillArgs& a, const Geo& w, int lt, Streams<D>& st) {
    const long L = w.eos - w.bos;           // tokens of this sequence
    const uint32_t kq_tok = (uint32_t)a.Hqk * D * 2, v_tok = (uint32_t)a.Hv * D * 2, s_tok = (uint32_t)a.Hv * 4;
    const uint32_t kq_end = L > 0 ? (uint32_t)((L - 1) * kq_tok + D * 2) : 0;
    const uint32_t v_end = L > 0 ? (uint32_t)((L - 1) * v_tok + DVS * 2) : 0;
    const uint32_t s_end = L > 0 ? (uint32_t)((L - 1) * s_tok + 4) : 0;
    const long kq0 = (w.bos * a.Hqk + w.hq) * D, v0 = (w.bos * a.Hv + w.h) * D + w.j0, s0 = w.bos * a.Hv + w.h;
    st.k = rsrc(static_cast<const __bf16*>(a.k) + kq0, kq_end);
    st.q = rsrc(static_cast<const __bf16*>(a.q) + kq0, kq_end);
    st.v = rsrc(static_cast<const __bf16*>(a.v) + v0, v_end);
    st.beta = rsrc(a.beta + s0, s_end);
    st.g = rsrc(a.g ? a.g + s0 : a.beta + s0, a.g ? s_end : 0);
    st.kq_chunk = FC * kq_tok;
    st.v_chunk = FC * v_tok;
    st.s_chunk = FC * s_tok;
#pragma unroll
    for (int p = 0; p < Dims<D>::NKP; ++p) {
        const int v = lt + NLD * p;
        st.off_kq[p] = (uint32_t)(v >> Dims<D>::PPR_LOG) * kq_tok + (v & (Dims<D>::PPR - 1)) * 16;
    }
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int v = lt + NLD * p;
        st.off_v[p] = (uint32_t)(v >> 2) * v_tok + (v & 3) * 16;
    }
    st.off_s = (uint32_t)(lt & 63) * s_tok;  // both loader waves fetch the chunk's scalars
}

__device__ __forceinline__ uint4 u4(u32x4 x) { return make_uint4(x[0], x[1], x[2], x[3]); }

template <int D>
__device__ __forceinline__ void fetch(const Streams<D>& st, int j, LoadSet<D>& f) {
    // the chunk offset goes into the per-lane offset, which the range check covers
    // issued in the order of use (loads complete in order): the scalars and K, which the
    // first half takes, before Q and V
    const uint32_t ckq = (uint32_t)j * st.kq_chunk, cv = (uint32_t)j * st.v_chunk, cs = (uint32_t)j * st.s_chunk;
    f.beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(st.beta, st.off_s + cs, 0, 0));
    f.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(st.g, st.off_s + cs, 0, 0));
#pragma unroll
    for (int p = 0; p < Dims<D>::NKP; ++p) f.k[p] = u4(__builtin_amdgcn_raw_buffer_load_b128(st.k, st.off_kq[p] + ckq, 0, 0));
    sched_fence();
#pragma unroll
    for (int p = 0; p < Dims<D>::NKP; ++p) f.q[p] = u4(__builtin_amdgcn_raw_buffer_load_b128(st.q, st.off_kq[p] + ckq, 0, 0));
#pragma unroll
    for (int p = 0; p < 2; ++p) f.v[p] = u4(__builtin_amdgcn_raw_buffer_load_b128(st.v, st.off_v[p] + cv, 0, 0));
}

// DPP move of a float with bound_ctrl (lanes without a source read 0)
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_f32(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK, 0xf, true));
}
__device__ __forceinline__ float lane_f32(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// K and the per-token scalars of chunk j (rows past the sequence end hold zeros)
template <int D>
__device__ __forceinline__ void put_k(FusedSmem<D>& sm, int j, int lt, const LoadSet<D>& f) {
#pragma unroll
    for (int p = 0; p < Dims<D>::NKP; ++p) {
        const int v = lt + NLD * p, row = v >> Dims<D>::PPR_LOG, cg = v & (Dims<D>::PPR - 1);
        *reinterpret_cast<uint4*>(&sm.K[j & 1][row][cg * 8]) = f.k[p];
    }
    if (lt < FC) {  // one wave: inclusive scan of the log decays over the chunk (DPP)
        float gv = f.g;
        gv += dpp_f32<0x111, 0xf>(gv);   // row_shr:1, 2, 4, 8 within rows of 16 lanes
        gv += dpp_f32<0x112, 0xf>(gv);
        gv += dpp_f32<0x114, 0xf>(gv);
        gv += dpp_f32<0x118, 0xf>(gv);
        gv += dpp_f32<0x142, 0xa>(gv);   // row_bcast:15 into rows 1, 3
        gv += dpp_f32<0x143, 0xc>(gv);   // row_bcast:31 into rows 2, 3
        const float ge[4] = {lane_f32(gv, 15), lane_f32(gv, 31), lane_f32(gv, 47), lane_f32(gv, 63)};
        float* s = &sm.sc[j % 3][0][0];
        s[SC_BETA * FC + lt] = f.beta;
        s[SC_GAM * FC + lt] = gv;
        s[SC_EG * FC + lt] = __expf(gv);
        s[SC_TAIL * FC + lt] = __expf(ge[3] - gv);
        const int blk = lt >> 4;
        s[SC_F2 * FC + lt] = __expf((blk == 0 ? ge[0] : blk == 1 ? ge[1] : blk == 2 ? ge[2] : ge[3]) - gv);
#pragma unroll
        for (int I = 0; I < 3; ++I) s[(SC_F1 + I) * FC + lt] = __expf(fminf(gv - ge[I], 0.f));
    }
}

// Q of chunk j
template <int D>
__device__ __forceinline__ void put_q(FusedSmem<D>& sm, int j, int lt, const LoadSet<D>& f) {
#pragma unroll
    for (int p = 0; p < Dims<D>::NKP; ++p) {
        const int v = lt + NLD * p, row = v >> Dims<D>::PPR_LOG, cg = v & (Dims<D>::PPR - 1);
        *reinterpret_cast<uint4*>(&sm.Q[j & 1][row][cg * 8]) = f.q[p];
    }
}

template <int D>
__device__ __forceinline__ void put_v(FusedSmem<D>& sm, int lt, const LoadSet<D>& f) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int v = lt + NLD * p;
        *reinterpret_cast<uint4*>(&sm.V[v >> 2][(v & 3) * 8]) = f.v[p];
    }
}

// ------------------------------------------------------------------ Gram products
// Key fragments of one chunk as 16x16x32 operands: kf[X][s] = rows 16 X + l16, keys
// 32 s + 8 q16 .. +7.  The same fragment serves as A operand (rows of the tile) and as
// B operand (columns of the tile) of a product contracting over keys.
template <int D>
__device__ __forceinline__ void load_rows(const __bf16 (*src)[Dims<D>::KPITCH], int l16, int q16,
                                          bf16x8 (&f)[4][Dims<D>::NKS]) {
#pragma unroll
    for (int X = 0; X < 4; ++X)
#pragma unroll
        for (int s = 0; s < Dims<D>::NKS; ++s) f[X][s] = ld8(&src[16 * X + l16][32 * s + 8 * q16]);
}

// A and P come from 16x16 tiles (I, R), I <= R, of K K^T and K Q^T: tile (I, R) holds
// k_i . k_r (or k_i . q_r) with i = 16 I + 4 q16 + e, r = 16 R + l16, so each lane owns
// four consecutive columns i of one row r: 8-byte stores.  Rows past the sequence end
// need no mask: their keys, queries and beta are zero.
struct DecayIn {  // what exp(gamma_r - gamma_i), i = i0 .. i0 + 3 <= r, is made from
    float a;       // diagonal tile: gamma_r; below it: F1[I][r]
    f32x4 b;       // diagonal tile: gamma_i; below it: F2[i]
};
__device__ __forceinline__ DecayIn decay_load(const float* s, int R, int I, int r, int i0) {
    DecayIn x;
    x.a = I == R ? s[SC_GAM * FC + r] : s[(SC_F1 + I) * FC + r];
    x.b = *reinterpret_cast<const f32x4*>(&s[(I == R ? SC_GAM : SC_F2) * FC + i0]);
    return x;
}
__device__ __forceinline__ f32x4 decay_eval(const DecayIn& x, bool diag) {
    f32x4 d;
#pragma unroll
    for (int e = 0; e < 4; ++e) d[e] = diag ? __expf(fminf(x.a - x.b[e], 0.f)) : x.a * x.b[e];
    return d;
}

// Diagonal entry of row l16 of a 16x16 Gram tile (entry (4 q16 + e, l16) in lane
// (l16, q16)), in every lane: lane l16 + 16 (l16 >> 2) holds it as entry l16 & 3.
__device__ __forceinline__ float gram_diag(const f32x4& g, int l16) {
    const int e = l16 & 3;
    const float mine = e == 0 ? g[0] : e == 1 ? g[1] : e == 2 ? g[2] : g[3];
    const int src = l16 + 16 * (l16 >> 2);
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, mine)));
}

// A of chunk j, one part of its tiles (I, R).  Part 0, the four diagonal tiles, goes to
// Ad in fp16 (strictly lower part, packed); part 1, the tiles (0,1) and (2,3) right below
// them (the UT inverse's A21 blocks), and part 2, the block rows 32..63 x columns 0..31
// (the chain's A_BL), go to Ab in bf16.
constexpr int a_tiles(int part) { return part == 0 ? 4 : part == 1 ? 2 : 4; }
constexpr int a_tile_i(int part, int n) { return part == 0 ? n : part == 1 ? 2 * n : (n & 1); }
constexpr int a_tile_r(int part, int n) { return part == 0 ? n : part == 1 ? 2 * n + 1 : 2 + (n >> 1); }

//
// With the in-rule normalisation, part 0 takes |k_r|^2 from the diagonal of its own Gram
// tiles, scales A's rows by s_r^2 and publishes the chain's factors (SC_B1, SC_B2, SC_S2)
// for row 16 q16 + l16.  Parts 1 and 2 write their tiles with beta alone; their consumers
// apply s_r^2 to the rows of the products they form from them.
template <int D, bool GATED, bool NORM, int PART>
__device__ __forceinline__ void make_a(FusedSmem<D>& sm, int j, int l16, int q16, float eps) {
    constexpr bool NRM = NORM && PART == 0;
    constexpr int NTL = a_tiles(PART);
    // every LDS read before the first store (a read after a store waits a round trip)
    const float* s = &sm.sc[j % 3][0][0];
    float br[NTL];
    DecayIn din[NTL];
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
        const int I = a_tile_i(PART, n), R = a_tile_r(PART, n), r = 16 * R + l16;
        br[n] = s[SC_BETA * FC + r];
        if (GATED) din[n] = decay_load(s, R, I, r, 16 * I + 4 * q16);
    }
    float egq = 1.f;
    if (NRM) egq = s[SC_EG * FC + 16 * q16 + l16];
    bf16x8 kf[4][Dims<D>::NKS];
    load_rows<D>(sm.K[j & 1], l16, q16, kf);
    sched_fence();  // all fragments in one round trip (the compiler would stage them)
    f32x4 G[NTL];
#pragma unroll
    for (int n = 0; n < NTL; ++n) G[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < Dims<D>::NKS; ++ks)
#pragma unroll
        for (int n = 0; n < NTL; ++n)
            G[n] = mma16(kf[a_tile_i(PART, n)][ks], kf[a_tile_r(PART, n)][ks], G[n]);
    if (NRM) {
        float rs[NTL];   // s_r of row 16 n + l16
#pragma unroll
        for (int n = 0; n < NTL; ++n) rs[n] = inv_norm(gram_diag(G[n], l16), eps);
        const float rq = q16 == 0 ? rs[0] : q16 == 1 ? rs[1] : q16 == 2 ? rs[2] : rs[3];
        const float bq = q16 == 0 ? br[0] : q16 == 1 ? br[1] : q16 == 2 ? br[2] : br[3];
        float* so = &sm.sc[j % 3][0][0];
        so[SC_S2 * FC + 16 * q16 + l16] = rq * rq;
        so[SC_B1 * FC + 16 * q16 + l16] = bq * rq;
        so[SC_B2 * FC + 16 * q16 + l16] = bq * rq * rq * egq;
#pragma unroll
        for (int n = 0; n < NTL; ++n) br[n] *= rs[n] * rs[n];
    }
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
        const int I = a_tile_i(PART, n), R = a_tile_r(PART, n);
        const int r = 16 * R + l16, i0 = 16 * I + 4 * q16;
        f32x4 d = {1.f, 1.f, 1.f, 1.f};
        if (GATED) {
            d = decay_eval(din[n], I == R);
            if (PART == 0) sm.pdec[j & 1][n][16 * q16 + l16] = d;   // the same factors for P
        }
        f32x4 av;
#pragma unroll
        for (int e = 0; e < 4; ++e) av[e] = br[n] * d[e] * G[n][e];
        if (PART >= 1) {
            st4(&sm.Ab[r][i0], av[0], av[1], av[2], av[3]);
        } else {
            // entries on or above the diagonal go to the spare slot 120 of the block
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 4 * q16 + e;
                sm.Ad[R][m < l16 ? l16 * (l16 - 1) / 2 + m : 120] = (_Float16)av[e];
            }
        }
    }
}

// Diagonal block q16 of A (packed, as part 0 of make_a wrote it) into registers, by the
// wave that wrote it: the UT inverse of the next half starts without an LDS round trip.
template <int D>
__device__ __forceinline__ void load_ad(const FusedSmem<D>& sm, int q16, f16x8 (&ap)[15]) {
    wave_lds_order();
#pragma unroll
    for (int g = 0; g < 15; ++g) ap[g] = *reinterpret_cast<const f16x8*>(&sm.Ad[q16][8 * g]);
}

// P of chunk j for the query rows of one output wave's two row blocks R (half 0: 0 and 3,
// half 1: 1 and 2, five tiles each), from the query fragments qf[u] of row block R_u that
// the wave holds.  The tiles come out as P^T (rows i = key token, columns r = query token):
// pt[u][s] is P^T for keys 32 s .. 32 s + 31 and the queries of R_u as a B operand
// (k = key token), the form the output product O^T = Delta^T P^T takes.  P never goes
// through LDS.
constexpr int p_block(int half, int u) { return half == 0 ? (u == 0 ? 0 : 3) : (u == 0 ? 1 : 2); }

//
// With the in-rule normalisation it also returns |q_r|^2 of its query rows (qn[u], row
// 16 R_u + l16), the diagonal of Q Q^T tiles formed from the same fragments.
template <int D, bool GATED, bool NORM, int HALF>
__device__ __forceinline__ void make_p(const FusedSmem<D>& sm, int j, const bf16x8 (&qf)[2][Dims<D>::NKS], int l16,
                                       int q16, bf16x8 (&pt)[2][2], float (&qn)[2]) {
    const float* s = &sm.sc[j % 3][0][0];
    DecayIn din[2][4];
    f32x4 pd[2];   // the diagonal tiles' factors, as A's wave formed them for this chunk
    if (GATED) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int R = p_block(HALF, u), r = 16 * R + l16;
            pd[u] = sm.pdec[j & 1][R][16 * q16 + l16];
#pragma unroll
            for (int I = 0; I < R; ++I) din[u][I] = decay_load(s, R, I, r, 16 * I + 4 * q16);
        }
    }
    bf16x8 kf[4][Dims<D>::NKS];
    load_rows<D>(sm.K[j & 1], l16, q16, kf);
    f32x4 G[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int I = 0; I < 4; ++I) G[u][I] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < Dims<D>::NKS; ++ks)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int R = p_block(HALF, u);
#pragma unroll
            for (int I = 0; I <= R; ++I) G[u][I] = mma16(kf[I][ks], qf[u][ks], G[u][I]);
        }
    if (NORM) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            f32x4 gq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < Dims<D>::NKS; ++ks) gq = mma16(qf[u][ks], qf[u][ks], gq);
            qn[u] = gram_diag(gq, l16);
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int R = p_block(HALF, u);
        const int r = 16 * R + l16;
#pragma unroll
        for (int I = 0; I <= R; ++I) {
            // tile (I, R): lane holds P[r][i] for i = 16 I + 4 q16 + e; zero above the diagonal
            const int i0 = 16 * I + 4 * q16;
            f32x4 d = {1.f, 1.f, 1.f, 1.f};
            if (GATED) d = I == R ? pd[u] : decay_eval(din[u][I], false);
#pragma unroll
            for (int e = 0; e < 4; ++e) G[u][I][e] = (I < R || i0 + e <= r) ? d[e] * G[u][I][e] : 0.f;
        }
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
            if (2 * sb <= R) pt[u][sb] = acc_to_b(G[u][2 * sb], G[u][2 * sb + 1]);  // tiles past R are zero
    }
}

// Wave 6, first half: the two 32x32 diagonal blocks of T = (I + A)^{-1} into Tt (T^T).
// The four 16x16 diagonal blocks by forward substitution in fp32 arithmetic (from A's
// entries stored in fp16), then the blocks below them
// by one level of 2x2 block inversion, T21 = -T22 (A21 T11), the inner product handed to
// the outer one as a B operand in registers.  The rest of T is never formed: the chain
// waves finish Delta by block substitution over the two 32-token halves.  The zero blocks
// of Tt are written once, before the first chunk.
//
// With the in-rule normalisation the stored A21 rows lack s_r^2 (the tiles below the
// block diagonal are written with beta alone): the product A21 T11 takes it per row, from
// s2 = the chunk's SC_S2 scalars.
template <int D, bool NORM>
__device__ __forceinline__ void make_t(FusedSmem<D>& sm, int l16, int q16, const f16x8 (&ap)[15], const float* s2) {
    {
        // lane = 16 * block + column c: solve (I + A_bb) x = e_c in the column order: once
        // x[m] is final, subtract its share from every later row.  ap holds the block's
        // strictly lower entries (120, packed, fp16: mixed-precision FMAs take them as they
        // are, and the arithmetic stays fp32).
        const int b = q16, c = l16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = r == c ? 1.f : 0.f;
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
        *reinterpret_cast<bf16x8*>(&sm.Tt[16 * b + c][16 * b]) = lo8;
        *reinterpret_cast<bf16x8*>(&sm.Tt[16 * b + c][16 * b + 8]) = hi8;
    }
    wave_lds_order();
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    // level 1, both 32x32 diagonal blocks (base 0, 32); k = 16 is padded to the
    // instruction's 32 with zero lanes (q16 >= 2)
    const bool live = q16 < 2;
    f32x4 X[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int base = 32 * h;
        // X = A21 T11: A rows base+16+m; B[k][n] = T11[k][n] = Tt[base+n][base+k]
        const bf16x8 af = live ? ld8(&sm.Ab[base + 16 + l16][base + 8 * q16]) : zero8();
        const bf16x8 bf = live ? ld8(&sm.Tt[base + l16][base + 8 * q16]) : zero8();
        X[h] = mma16(af, bf, z4);
        if (NORM) X[h] *= *reinterpret_cast<const f32x4*>(&s2[base + 16 + 4 * q16]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int base = 32 * h;
        // T21 = -T22 X: A operand T22[m][k] = Tt[base+16+k][base+16+m] (transposed read;
        // k >= 16 meets the zero half of the B operand)
        const __bf16* src = &sm.Tt[base + 16 + 8 * (q16 & 1) + (l16 >> 2)][base + 16 + 4 * (l16 & 3)];
        const f32x4 Y = mma16(cat(trld(src), trld(src + 4 * CPITCH)), acc_to_b(X[h], z4), z4);
        st4(&sm.Tt[base + l16][base + 16 + 4 * q16], -Y[0], -Y[1], -Y[2], -Y[3]);
    }
}

// The reverse pass's record of chunk j (T^T, then P, bf16 64 x 64 each, row-major), written
// in the second half of phase j by the two output waves of a (sequence, head)'s first slice.
// P: each wave's rows, from the P^T fragments make_p formed (lane l16 of q16 holds row
// 16 R + l16, keys 32 s + 8 q16 ..; the tiles above R are zero).  T^T: wave 0 forms the
// block of T below its two 32x32 diagonal blocks, T_BL = -T_BR (A_BL T_TL) (A_BL is the
// chain's block of A, still in Ab), and copies the diagonal blocks from Tt, which the
// UT-inverse wave wrote in the first half and rewrites only in the next phase.
template <int D>
__device__ __forceinline__ void put_tp_record(const FusedSmem<D>& sm, __bf16* rec, int ow, const bf16x8 (&pt)[2][2],
                                              int lane) {
    const int l16 = lane & 15, q16 = lane >> 4;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int R = p_block(ow, u);
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
            *reinterpret_cast<bf16x8*>(rec + FC * FC + (16 * R + l16) * FC + 32 * sb + 8 * q16) =
                2 * sb <= R ? pt[u][sb] : zero8();
    }
    if (ow != 0) return;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    f32x4 X[2][2];   // A_BL T_TL: tile (ti, tj) rows 32 + 16 ti, columns 16 tj
#pragma unroll
    for (int ti = 0; ti < 2; ++ti)
#pragma unroll
        for (int tj = 0; tj < 2; ++tj)
            X[ti][tj] = mma16(ld8(&sm.Ab[32 + 16 * ti + l16][8 * q16]), ld8(&sm.Tt[16 * tj + l16][8 * q16]), z4);
#pragma unroll
    for (int ti = 0; ti < 2; ++ti) {
        // A operand T_BR[16 ti + m][k] = Tt[32 + k][32 + 16 ti + m] (transposed read)
        const __bf16* src = &sm.Tt[32 + 8 * q16 + (l16 >> 2)][32 + 16 * ti + 4 * (l16 & 3)];
        const bf16x8 ta = cat(trld(src), trld(src + 4 * CPITCH));
#pragma unroll
        for (int tj = 0; tj < 2; ++tj) {
            // T[32 + 16 ti + 4 q16 + e][16 tj + l16] = -Y[e]: row 16 tj + l16 of T^T
            const f32x4 Y = mma16(ta, acc_to_b(X[0][tj], X[1][tj]), z4);
            st4(rec + (16 * tj + l16) * FC + 32 + 16 * ti + 4 * q16, -Y[0], -Y[1], -Y[2], -Y[3]);
        }
    }
    // the diagonal blocks (lane = row of T^T) and the zero block left of the lower one
    const int c0 = lane < 32 ? 0 : 32;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        *reinterpret_cast<bf16x8*>(rec + lane * FC + c0 + 8 * p) = ld8(&sm.Tt[lane][c0 + 8 * p]);
        if (lane >= 32) *reinterpret_cast<bf16x8*>(rec + lane * FC + 8 * p) = zero8();
    }
}

// -------------------------------------------------------------------------- kernel
// STATES: the chain waves also write the state at every chunk start (fp32, for chunk number
// chunk_id_base(n) + chunk and value head h at a.ws + (number Hv + h) Dk Dv, as 8 x 8 tiles of
// 16 keys x 16 columns in the accumulator layout: tile (key block kb, column block cb) at
// (8 kb + cb) 256 floats, lane l's four entries (keys 16 kb + 4 (l >> 4) + e, column
// 16 cb + (l & 15)) at 4 l, one 16-byte store each), the input of the chunkwise reverse pass;
// the output waves skip O, and with a.tp_rec those of the first slice write each chunk's
// T^T and P record of the reverse pass instead (put_tp_record).
template <int D, bool GATED, bool NORM, bool STATES = false>
__global__ __launch_bounds__(NT, 1) __attribute__((amdgpu_waves_per_eu(1, 2))) void fused_kernel(PrefillArgs a) {
    constexpr int NKS = Dims<D>::NKS, NKT = Dims<D>::NKT, NSL = Dims<D>::NSL, KPITCH = Dims<D>::KPITCH;
    __shared__ FusedSmem<D> sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q16 = lane >> 4;

    // Workgroup -> (chain = sequence * Hv + head, slice).  When the count of (sequence, q/k
    // head) pairs is a multiple of 8, all the slices of all the value heads of one q/k head
    // land on one XCD (workgroups are dealt to the 8 XCDs round-robin), one after another,
    // so they share that q/k head's K and Q through the XCD's L2.
    const int grp = a.Hv / a.Hqk;
    const int qchains = a.N * a.Hqk;
    const int b = blockIdx.x;
    int chain, slice;
    if ((qchains & 7) == 0) {
        const int y = b >> 3;                      // the workgroup's turn on its XCD
        slice = y % NSL;
        const int t = y / NSL;
        const int qc = (b & 7) + 8 * (t / grp);    // sequence * Hqk + q/k head
        chain = (qc / a.Hqk) * a.Hv + (qc % a.Hqk) * grp + t % grp;
    } else {
        slice = b % NSL;
        chain = b / NSL;
    }
    Geo w;
    w.n = chain / a.Hv;
    w.h = chain % a.Hv;
    if (a.cu && a.N <= NT) {
        // longest sequences first: rank -> sequence (ties by index).  Thread m ranks sequence
        // m against the lengths staged in LDS; the ranks are a permutation of 0 .. N - 1.
        if (tid < a.N) sm.seq_len[tid] = a.cu[tid + 1] - a.cu[tid];
        __syncthreads();
        if (tid < a.N) {
            const int lm = sm.seq_len[tid];
            int r = 0;
            for (int x = 0; x < a.N; ++x) {
                const int lx = sm.seq_len[x];
                r += (lx > lm) || (lx == lm && x < tid);
            }
            sm.rank_seq[r] = tid;
        }
        __syncthreads();
        w.n = sm.rank_seq[w.n];
    }
    w.nh = w.n * a.Hv + w.h;
    w.hq = w.h / (a.Hv / a.Hqk);
    w.j0 = slice * DVS;
    seq_range(a.cu, w.n, a.T, w.bos, w.eos);
    w.nchunks = (int)((w.eos - w.bos + FC - 1) / FC);
    const int nc = w.nchunks;
    const int nph = nc + 1;   // phases 0 .. nc (the last one writes O of the last chunk)

    // Every wave runs phases j = -1 .. nph - 1, two barriers each.
    if (wave < NCW) {
        // ------------------------------------------------------------ chain waves
        const int jc = CW * wave;
        __builtin_amdgcn_s_setprio(2);  // the sequential chain goes first on its SIMD
        f32x4 M[NKT];  // tile mt: keys 16 mt + 4 q16 + e, column jc + l16 of the slice
#pragma unroll
        for (int mt = 0; mt < NKT; ++mt) M[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.h0) {
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    M[mt][e] = a.h0[((long)w.nh * D + 16 * mt + 4 * q16 + e) * D + w.j0 + jc + l16];
        }
        bf16x8 mb[NKS];  // the state at the chunk start as B operands: k = key 32 s + 8 q16 + e
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
            mb[s] = acc_to_b(M[2 * s], M[2 * s + 1]);
            sm.mb[0][wave][s][lane] = mb[s];
        }
        __syncthreads();
        __syncthreads();
        float* st_out = nullptr;   // STATES: this chain wave's columns of chunk 0's start state
        if (STATES) st_out = static_cast<float*>(a.ws) + ((long)chunk_id_base(a, w.n) * a.Hv + w.h) * D * D +
                             ((w.j0 + jc) / 16) * 256 + 4 * lane;
        for (int j = 0; j < nph; ++j) {
            const bool live = j < nc;
            const float* s = &sm.sc[j % 3][0][0];
            bf16x8 rb0;   // R rows 0..31 as B operand (k = token)
            f32x4 R[4];   // R, token tile t: tokens 16 t + 4 q16 + e, column jc + l16
            if (STATES && live) {
                float* dst = st_out + (long)j * a.Hv * D * D;
#pragma unroll
                for (int mt = 0; mt < NKT; ++mt) *reinterpret_cast<f32x4*>(dst + mt * NKT * 256) = M[mt];
            }
            if (live) {
                // X = K M: token tile t holds tokens 16 t + 4 q16 + e, column jc + l16
                f32x4 X[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) X[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        X[t] = mma16(ld8(&sm.K[j & 1][16 * t + l16][32 * ks + 8 * q16]), mb[ks], X[t]);
                // R = beta (V - exp(gamma) X); V read transposed: lane gets 4 tokens of its column
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int r0 = 16 * t + 4 * q16;
                    const bf16x4 vv = trld(&sm.V[r0 + (l16 >> 2)][jc + 4 * (l16 & 3)]);
                    if (NORM) {  // R' = beta s V - beta s^2 exp(gamma) X
                        const f32x4 b1 = *reinterpret_cast<const f32x4*>(&s[SC_B1 * FC + r0]);
                        const f32x4 b2 = *reinterpret_cast<const f32x4*>(&s[SC_B2 * FC + r0]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) R[t][e] = b1[e] * (float)vv[e] - b2[e] * X[t][e];
                    } else {
                        const f32x4 bt = *reinterpret_cast<const f32x4*>(&s[SC_BETA * FC + r0]);
                        f32x4 eg = {1.f, 1.f, 1.f, 1.f};
                        if (GATED) eg = *reinterpret_cast<const f32x4*>(&s[SC_EG * FC + r0]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) R[t][e] = bt[e] * ((float)vv[e] - eg[e] * X[t][e]);
                    }
                }
                rb0 = acc_to_b(R[0], R[1]);
            }
            __syncthreads();
            if (live) {
                // Delta = T R by block substitution over the two 32-token halves:
                //   Delta_top = T_TL R_top;  Delta_bot = T_BR (R_bot - A_BL Delta_top).
                // T operands T[16 t + m][k] = Tt[k][16 t + m] by transposed reads.  With decay,
                // the tail factors are read here, ahead of the Delta store (a read behind a
                // store waits a round trip of its own).
                // A rows 32..63, tokens 0..31 (wave 2 wrote them in the first half)
                bf16x8 abl[2];
                f32x4 s2bl[2];  // in-rule normalisation: s_r^2 of those rows (Ab holds them without)
#pragma unroll
                for (int t = 2; t < 4; ++t) abl[t - 2] = ld8(&sm.Ab[16 * t + l16][8 * q16]);
                if (NORM) {
#pragma unroll
                    for (int t = 2; t < 4; ++t) s2bl[t - 2] = *reinterpret_cast<const f32x4*>(&s[SC_S2 * FC + 16 * t + 4 * q16]);
                }
                f32x4 tl[4];
                float Gl = 1.f;
                if (GATED) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) tl[t] = *reinterpret_cast<const f32x4*>(&s[SC_TAIL * FC + 16 * t + 4 * q16]);
                    Gl = s[SC_EG * FC + FC - 1];
                }
                f32x4 Dl[4];
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const __bf16* src = &sm.Tt[8 * q16 + (l16 >> 2)][16 * t + 4 * (l16 & 3)];
                    Dl[t] = mma16(cat(trld(src), trld(src + 4 * CPITCH)), rb0, f32x4{0.f, 0.f, 0.f, 0.f});
                }
                const bf16x8 dtop = acc_to_b(-Dl[0], -Dl[1]);
#pragma unroll
                for (int t = 2; t < 4; ++t) {
                    if (NORM) R[t] += s2bl[t - 2] * mma16(abl[t - 2], dtop, f32x4{0.f, 0.f, 0.f, 0.f});
                    else R[t] = mma16(abl[t - 2], dtop, R[t]);
                }
                const bf16x8 zb = acc_to_b(R[2], R[3]);
#pragma unroll
                for (int t = 2; t < 4; ++t) {
                    const __bf16* src = &sm.Tt[32 + 8 * q16 + (l16 >> 2)][16 * t + 4 * (l16 & 3)];
                    Dl[t] = mma16(cat(trld(src), trld(src + 4 * CPITCH)), zb, f32x4{0.f, 0.f, 0.f, 0.f});
                }
                bf16x8 db[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    db[u] = acc_to_b(Dl[2 * u], Dl[2 * u + 1]);
                    sm.dd[wave][u][lane] = db[u];
                }
                if (GATED) {  // Delta~ = diag(exp(gamma_last - gamma)) Delta for the state update
#pragma unroll
                    for (int t = 0; t < 4; ++t) Dl[t] *= tl[t];
                    db[0] = acc_to_b(Dl[0], Dl[1]);
                    db[1] = acc_to_b(Dl[2], Dl[3]);
#pragma unroll
                    for (int mt = 0; mt < NKT; ++mt) M[mt] *= Gl;
                }
                // M <- exp(gamma_last) M + K^T Delta~  (rows past the chunk end add g = 0)
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int mt = 0; mt < NKT; ++mt) {
                        // A operand K^T[16 mt + m][k] = K[k][16 mt + m], k = 32 u + 8 q16 + e
                        const __bf16* src = &sm.K[j & 1][32 * u + 8 * q16 + (l16 >> 2)][16 * mt + 4 * (l16 & 3)];
                        M[mt] = mma16(cat(trld(src), trld(src + 4 * KPITCH)), db[u], M[mt]);
                    }
#pragma unroll
                for (int s4 = 0; s4 < NKS; ++s4) {
                    mb[s4] = acc_to_b(M[2 * s4], M[2 * s4 + 1]);
                    sm.mb[(j + 1) & 1][wave][s4][lane] = mb[s4];
                }
            }
            __syncthreads();
        }
        if (a.hT) {
#pragma unroll
            for (int mt = 0; mt < NKT; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.hT[((long)w.nh * D + 16 * mt + 4 * q16 + e) * D + w.j0 + jc + l16] = M[mt][e];
        }
    } else if (wave == 3 || wave == 7) {
        // ----------------------------------------------------------- output waves
        // Output wave ow owns the query rows of row blocks R_0, R_1 (ow 0: blocks 0 and 3,
        // ow 1: blocks 1 and 2) for all 32 columns, and computes in the transposed form,
        // O^T = exp(gamma) Y^T + Delta^T P^T with Y^T = M^T Q^T: the chain's bf16 state and
        // Delta fragments serve unchanged as the A operands M^T and Delta^T, the query rows as
        // B operands, and P^T stays in registers from make_p.
        const int ow = wave == 3 ? 0 : 1;
        // O goes to HBM from registers: a lane stores four consecutive columns of one token
        // (8 bytes), through a buffer descriptor that covers exactly this sequence's tokens
        // of the slice, so rows past the sequence end are dropped by the range check.  The
        // other slices of the row, on the same XCD, fill the rest of its cache lines.
        const long L = w.eos - w.bos;
        const uint32_t o_tok = (uint32_t)a.Hv * D * 2;
        const __amdgpu_buffer_rsrc_t o_rs =
            rsrc(static_cast<__bf16*>(a.o) + (w.bos * a.Hv + w.h) * D + w.j0,
                 L > 0 ? (uint32_t)((L - 1) * o_tok + DVS * 2) : 0);
        f32x4 yt[2][2];      // Y^T tile (u, c): columns 16 c + 4 q16 + e, query 16 R_u + l16
        bf16x8 pt[2][2];     // P^T of the chunk as B operands (make_p)
        bf16x8 qf[2][NKS];   // query rows of R_u: qf[u][ks] = keys 32 ks + 8 q16 ..
        float qn[2] = {0.f, 0.f};   // in-rule normalisation: |q_r|^2 of the rows of P^T
        // STATES with a.tp_rec: the first slice's output waves, which store no O, write every
        // chunk's T^T and P record instead
        __bf16* rec = nullptr;
        if (STATES && !NORM && a.tp_rec && slice == 0)
            rec = static_cast<__bf16*>(a.tp_rec) + (chunk_id_base(a, w.n) * a.Hv + w.h) * (2L * FC * FC);
        const long rec_step = (long)a.Hv * 2 * FC * FC;   // to the next chunk's record
        __syncthreads();
        __syncthreads();
        for (int j = 0; j < nph; ++j) {
            const bool o_live = !STATES && j >= 1 && j <= nc, y_live = !STATES && j < nc;
            const bool r_live = rec && j < nc;
            if (o_live) {
                // O of chunk j - 1 = scale (exp(gamma) Y + P Delta), P lower triangular
                const int jp = j - 1;
                const float* s = &sm.sc[jp % 3][0][0];
                bf16x8 dq[2][2];   // Delta^T: column tile c, key tokens 32 s ..
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int sb = 0; sb < 2; ++sb) dq[c][sb] = sm.dd[c][sb][lane];
                float egr[2] = {1.f, 1.f}, osc[2] = {a.scale, a.scale};
                if (GATED) {
#pragma unroll
                    for (int u = 0; u < 2; ++u) egr[u] = s[SC_EG * FC + 16 * (ow == 0 ? 3 * u : 1 + u) + l16];
                }
                if (NORM) {  // scale / |q_r|
#pragma unroll
                    for (int u = 0; u < 2; ++u) osc[u] *= inv_norm(qn[u], a.eps);
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int R = ow == 0 ? 3 * u : 1 + u;
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        f32x4 o = yt[u][c] * egr[u];
#pragma unroll
                        for (int sb = 0; sb < 2; ++sb)
                            if (2 * sb <= R) o = mma16(dq[c][sb], pt[u][sb], o);
                        const uint32_t off = (uint32_t)(jp * FC + 16 * R + l16) * o_tok + (16 * c + 4 * q16) * 2;
                        const uint32_t lo = pack_bf16x2(osc[u] * o[0], osc[u] * o[1]);
                        const uint32_t hi = pack_bf16x2(osc[u] * o[2], osc[u] * o[3]);
                        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                        __builtin_amdgcn_raw_buffer_store_b64(u32x2{lo, hi}, o_rs, off, 0, 0);
                    }
                }
            }
            if (y_live) {
                // Y^T = M^T Q^T with the chain's bf16 state at the start of chunk j (written at
                // the end of the previous phase)
                bf16x8 m4[2][NKS];
#pragma unroll
                for (int c = 0; c < 2; ++c)
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) m4[c][ks] = sm.mb[j & 1][c][ks][lane];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int R = ow == 0 ? 3 * u : 1 + u;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) qf[u][ks] = ld8(&sm.Q[j & 1][16 * R + l16][32 * ks + 8 * q16]);
                }
#pragma unroll
                for (int u = 0; u < 2; ++u)
#pragma unroll
                    for (int c = 0; c < 2; ++c) yt[u][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int c = 0; c < 2; ++c) yt[u][c] = mma16(m4[c][ks], qf[u][ks], yt[u][c]);
            }
            if (r_live) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int R = ow == 0 ? 3 * u : 1 + u;
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) qf[u][ks] = ld8(&sm.Q[j & 1][16 * R + l16][32 * ks + 8 * q16]);
                }
            }
            __syncthreads();
            if (y_live || r_live) {  // P of chunk j for the same query rows
                if (ow == 0) make_p<D, GATED, NORM, 0>(sm, j, qf, l16, q16, pt, qn);
                else make_p<D, GATED, NORM, 1>(sm, j, qf, l16, q16, pt, qn);
            }
            if (r_live) put_tp_record<D>(sm, rec + j * rec_step, ow, pt, lane);
            __syncthreads();
        }
    } else if (wave == 4 || wave == 5) {
        // ---------------------------------------------------------------- loaders
        const int lt = tid - 256;
        Streams<D> st;
        make_streams<D>(a, w, lt, st);
        LoadSet<D> f0, f1;   // even chunks in f0, odd chunks in f1
        fetch(st, 0, f0);
        fetch(st, 1, f1);
        // phase -1: chunk 0
        put_k(sm, 0, lt, f0);
        __syncthreads();
        put_q(sm, 0, lt, f0);
        put_v(sm, lt, f0);
        fetch(st, 2, f0);
        __syncthreads();
        // phase j: chunk j + 1 (in f[(j + 1) & 1]): K and the scalars in the first half, Q
        // and V in the second; then refill that set with chunk j + 3
        for (int j = 0; j < nph; j += 2) {
            put_k(sm, j + 1, lt, f1);
            __syncthreads();
            put_q(sm, j + 1, lt, f1);
            put_v(sm, lt, f1);
            fetch(st, j + 3, f1);
            __syncthreads();
            if (j + 1 >= nph) break;
            put_k(sm, j + 2, lt, f0);
            __syncthreads();
            put_q(sm, j + 2, lt, f0);
            put_v(sm, lt, f0);
            fetch(st, j + 4, f0);
            __syncthreads();
        }
    } else if (wave == 6) {
        // ------------------------------------------ wave 6: T of j, half of A of j + 1
        // zero blocks of Tt below its block diagonal, written once
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int v = lane + 64 * p, r = v >> 3, cg = v & 7;
            if (cg * 8 + 8 <= (r >> 4) * 16) *reinterpret_cast<bf16x8*>(&sm.Tt[r][cg * 8]) = zero8();
        }
        // phase -1, second half: A's diagonal tiles of chunk 0
        f16x8 ap[15];
        // first on its SIMD: the UT inverse and A's diagonal tiles (with their readback) are
        // the longer steps of both halves; the other A wave has slack
        __builtin_amdgcn_s_setprio(2);
        __syncthreads();
        make_a<D, GATED, NORM, 0>(sm, 0, l16, q16, a.eps);
        load_ad<D>(sm, q16, ap);
        __syncthreads();
        for (int j = 0; j < nph; ++j) {
            if (j < nc) make_t<D, NORM>(sm, l16, q16, ap, &sm.sc[j % 3][SC_S2][0]);
            __syncthreads();
            if (j + 1 < nc) {
                make_a<D, GATED, NORM, 0>(sm, j + 1, l16, q16, a.eps);
                load_ad<D>(sm, q16, ap);
            }
            __syncthreads();
        }
    } else {
        // ------------------ wave 2: A_BL of j in the first half, A21 of j + 1 in the second
        __syncthreads();
        make_a<D, GATED, NORM, 1>(sm, 0, l16, q16, a.eps);
        __syncthreads();
        for (int j = 0; j < nph; ++j) {
            if (j < nc) make_a<D, GATED, NORM, 2>(sm, j, l16, q16, a.eps);
            __syncthreads();
            if (j + 1 < nc) make_a<D, GATED, NORM, 1>(sm, j + 1, l16, q16, a.eps);
            __syncthreads();
        }
    }
}

}  // namespace

bool prefill_fused_supported(const PrefillArgs& a) {
    // buffer offsets are 32-bit: a sequence (plus the two chunks fetched past its end) must
    // span less than 2 GiB of q / k / v / o
    const long span = ((long)a.T + 2 * FC) * (a.Hqk > a.Hv ? a.Hqk : a.Hv) * a.Dk * 2;
    return a.bf16 && a.Dk == a.Dv && (a.Dk == 128 || a.Dk == 64) && a.C == FC && !a.g_per_key &&
           span < (1L << 31);
}

hipError_t launch_prefill_fused_states(const PrefillArgs& a, hipStream_t s) {
    // the chunk-start states of the reverse pass (d = 128 only)
    if (a.Dk != 128 || a.Dv != 128) return hipErrorInvalidValue;
    const long blocks = (long)a.N * a.Hv * Dims<128>::NSL;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (blocks > 0) {
        const dim3 grid((unsigned)blocks), block(NT);
        if (a.g) hipLaunchKernelGGL((fused_kernel<128, true, false, true>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((fused_kernel<128, false, false, true>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

template <int D>
static hipError_t launch_fused_d(const PrefillArgs& a, hipStream_t s) {
    const long blocks = (long)a.N * a.Hv * Dims<D>::NSL;
    if (blocks > 0x7fffffffL) return hipErrorInvalidConfiguration;
    if (blocks > 0) {
        const dim3 grid((unsigned)blocks), block(NT);
        if (a.qk_norm) {
            if (a.g) hipLaunchKernelGGL((fused_kernel<D, true, true>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((fused_kernel<D, false, true>), grid, block, 0, s, a);
        } else {
            if (a.g) hipLaunchKernelGGL((fused_kernel<D, true, false>), grid, block, 0, s, a);
            else hipLaunchKernelGGL((fused_kernel<D, false, false>), grid, block, 0, s, a);
        }
    }
    return hipGetLastError();
}

hipError_t launch_prefill_fused(const PrefillArgs& a, hipStream_t s) {
    return a.Dk == 64 ? launch_fused_d<64>(a, s) : launch_fused_d<128>(a, s);
}

}  // namespace dn
