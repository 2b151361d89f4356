// internal.h -- declarations shared by the HIP sources of libdeltanet (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dn {

// Everything one prefill launch needs, already validated on the host.
struct PrefillArgs {
    int B, T, N, Hqk, Hv, Dk, Dv, C;
    int bf16;                       // 1: q/k/v/o are bfloat16, 0: float
    float scale;
    int qk_norm;                    // 1: q, k -> x / sqrt(|x|^2 + eps) inside the rule
    float eps;
    int g_per_key;                  // 1: g is [.., Hv, Dk], one log decay per key channel
    const void* q;
    const void* k;
    const void* v;
    const float* beta;
    const float* g;                 // may be null (no decay)
    const float* h0;                // may be null (zero initial state)
    float* hT;                      // may be null (no final state); may alias h0
    const int32_t* cu;              // may be null (each batch row is a sequence)
    void* o;
    void* ws;                       // caller's workspace (the two-kernel channel-gate path)
    size_t ws_bytes;
    void* tp_rec;                   // the chunk-start states launch only: may be null, else
                                    //   T^T and P of every chunk (the reverse pass's records)
};

// Readout epilogue, validated on the host (kind < 0: none).
struct EpilogueArgs {
    int kind;                       // -1 none, 0 RMS, 1 layer norm
    float eps;
    const float* w;                 // may be null (ones)
    const float* b;                 // may be null (zeros)
    const void* gate;               // may be null (no output gate)
};

struct DecodeArgs {
    int N, Hqk, Hv, Dk, Dv;
    int bf16;
    float scale;
    int qk_norm;                    // as in PrefillArgs
    float eps;
    int g_per_key;
    EpilogueArgs ep;
    const void* q;
    const void* k;
    const void* v;
    const float* beta;
    const float* g;
    float* state;
    void* o;
};

struct NormGateArgs {
    long rows;                      // tokens x value heads
    int Dv;
    int bf16;
    EpilogueArgs ep;
    const void* o;
    void* y;                        // may alias o
};

// The token-by-token route over whole sequences: the prefill's arguments plus an
// optional per-token state trace [tokens, Hv, Dk, Dv].
struct RecurrentArgs : PrefillArgs {
    float* trace;                   // may be null
};

// Short causal depthwise convolution (+ silu), validated on the host.  The prompt kernel
// can also split its output into q, k and v (the first qk channels to q, the next qk to k,
// the rest to y with a token stride of y_stride) and L2-normalise q and k per head of Dk
// channels; the plain convolution is qk = 0, y_stride = C.
struct ConvArgs {
    int B, T, N, C, W;
    int bf16;
    int silu;
    const void* x;
    const float* w;                 // [C, W]
    const float* b;                 // may be null
    const void* s0;                 // [N, C, W - 1], may be null (zeros)
    void* sT;                       // [N, C, W - 1], may be null; in place for a step
    const int32_t* cu;              // may be null
    void* y;
    int qk;                         // q (and k) channels split off; 0: none
    long y_stride;                  // y elements per token
    int Dk;                         // channels per q/k head (the L2 norm's group)
    int qk_norm;                    // 1: q, k -> x / sqrt(|x|^2 + eps) per head
    float eps;
    void* q;                        // [tokens, qk] when qk > 0
    void* k;                        // [tokens, qk] when qk > 0
};

// The reverse pass of the token-by-token route: the forward's arguments, its state
// trace, dL/do and dL/dM_T in; gradients out (fp32).  Each workgroup takes a slice of the
// value columns (recurrent_bwd_slices(Dk, Dv) of them) and writes its share of dq, dk, dbeta
// and dg to the workspace; a second kernel adds the shares.
struct RecurrentBwdArgs : PrefillArgs {
    const float* trace;             // [tokens, Hv, Dk, Dv] from the forward
    const void* dout;               // [tokens, Hv, Dv] dtype
    const float* dfinal;            // [N, Hv, Dk, Dv] or null
    float* ws_dq;                   // [slices, tokens, Hv, Dk]
    float* ws_dk;                   // [slices, tokens, Hv, Dk]
    float* ws_db;                   // [slices, tokens, Hv]
    float* ws_dg;                   // [slices, tokens, Hv]
    float* dq;                      // [tokens, Hqk, Dk]
    float* dk;                      // [tokens, Hqk, Dk]
    float* dv;                      // [tokens, Hv, Dv]
    float* dbeta;                   // [tokens, Hv]
    float* dg;                      // [tokens, Hv] or null (no gate)
    float* dh0;                     // [N, Hv, Dk, Dv] or null
};
int recurrent_bwd_slices(int Dk, int Dv);

// The chunkwise reverse pass: the forward's arguments, dL/do and dL/dM_T in; gradients out
// (fp32).  The workspace holds, per (chunk number, value head), the state at the chunk's
// start and the gradient of the state after the chunk (fp32, key-major), and T^T and P of
// the chunk (bf16, 64 x 64 each).
struct ChunkBwdArgs : PrefillArgs {
    const void* dout;               // [tokens, Hv, Dv] bf16
    const float* dfinal;            // [N, Hv, Dk, Dv] or null
    long ncid;                      // chunk numbers (chunk_id_bound)
    float* states;                  // [ncid, Hv, 8 x 8 tiles of 16 x 16 in the accumulator layout]
    float* dstates;                 // the same layout
    void* tp;                       // [ncid, Hv, 2, 64, 64] bf16: T^T, then P
    float* dq;                      // [tokens, Hqk, Dk]
    float* dk;                      // [tokens, Hqk, Dk]
    float* dv;                      // [tokens, Hv, Dv]
    float* dbeta;                   // [tokens, Hv]
    float* dg;                      // [tokens, Hv] or null (no gate)
    float* dh0;                     // [N, Hv, Dk, Dv] or null
    const float* rnorm;             // null, or with q, k normalised rows: 1 / sqrt(|x|^2 + eps)
                                    //   of the raw q rows [tokens, Hqk], then of the k rows
};
bool chunk_bwd_supported(const PrefillArgs& a);
size_t chunk_bwd_workspace_bytes(const PrefillArgs& a, long ncid);
hipError_t launch_chunk_bwd(const ChunkBwdArgs& a, hipStream_t s);

// Launchers (host functions); each returns hipGetLastError() after its launches.
hipError_t launch_recurrent_bwd(const RecurrentBwdArgs& a, hipStream_t s);
// the in-call normalisation as a pass of its own: bf16 q, k rows -> x / sqrt(|x|^2 + eps)
// into qn, kn ([tokens, Hqk, Dk] bf16), and 1 / sqrt(|x|^2 + eps) of every q row, then of
// every k row, into rnorm (may be null)
hipError_t launch_qk_norm_rows(const PrefillArgs& a, void* qn, void* kn, float* rnorm, hipStream_t s);
hipError_t launch_causal_conv(const ConvArgs& a, hipStream_t s);
hipError_t launch_causal_conv_step(const ConvArgs& a, hipStream_t s);
hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t s);
hipError_t launch_norm_gate(const NormGateArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_prefill_generic(const PrefillArgs& a, hipStream_t s);
bool prefill_fused_supported(const PrefillArgs& a);
bool prefill_chg_supported(const PrefillArgs& a);
bool prefill_chg_shape_ok(const PrefillArgs& a);
size_t prefill_chg_workspace_bytes(const PrefillArgs& a);
// The allocation-free prompt call's static scratch: its size, and its device address on
// the current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_prefill_chg(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_fused(const PrefillArgs& a, hipStream_t s);
// the same kernel writing the state at every chunk start to a.ws instead of the outputs
hipError_t launch_prefill_fused_states(const PrefillArgs& a, hipStream_t s);
// T^T and P (bf16, 64 x 64 each) of every (chunk number < ncid, value head) to tp, one
// 16 KiB record each: record cid * Hv + h, or h * ncid + cid when head_major
hipError_t launch_chunk_tp(const PrefillArgs& a, long ncid, void* tp, bool head_major, hipStream_t s);

}  // namespace dn

// ------------------------------------------------------------------ device helpers
namespace dn {

__device__ __forceinline__ float ld_f32(const float* p, long i) { return p[i]; }
__device__ __forceinline__ float ld_f32(const __bf16* p, long i) { return (float)p[i]; }

__device__ __forceinline__ void st_out(float* p, long i, float x) { p[i] = x; }
__device__ __forceinline__ void st_out(__bf16* p, long i, float x) { p[i] = (__bf16)x; }

// 1 / sqrt(ss + eps) of the in-rule q/k normalisation (ss = sum of squares); a zero
// vector with eps == 0 normalises to zero.
__device__ __forceinline__ float inv_norm(float ss, float eps) {
    const float x = ss + eps;
    return x > 0.f ? rsqrtf(x) : 0.f;
}

// silu(z) = z / (1 + exp(-z)), the output gate's activation (hardware reciprocal)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// Number of the first 64-token chunk of sequence n in per-chunk workspaces: n * ceil(T / 64)
// for a batch of rows; floor(cu[n] / 64) + n for packed sequences, which gives every chunk
// of every sequence a distinct number below T / 64 + N + 1 without a scan over the
// sequences (chunk c of sequence n is chunk_id_base + c).
__host__ __device__ __forceinline__ long chunk_id_base(const PrefillArgs& a, int n) {
    return a.cu ? (long)(a.cu[n] / 64) + n : (long)n * ((a.T + 63) / 64);
}
__host__ __device__ __forceinline__ long chunk_id_bound(const PrefillArgs& a) {
    return a.cu ? (long)(a.T / 64) + a.N + 1 : (long)a.N * ((a.T + 63) / 64);
}

// Token range [bos, eos) of sequence n.
__device__ __forceinline__ void seq_range(const int32_t* cu, int n, int T, long& bos, long& eos) {
    if (cu) {
        bos = cu[n];
        eos = cu[n + 1];
    } else {
        bos = (long)n * T;
        eos = bos + T;
    }
}

}  // namespace dn
