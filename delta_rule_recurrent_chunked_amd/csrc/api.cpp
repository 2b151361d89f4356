// api.cpp -- the exported C ABI (include/deltanet.h): host-side argument checks,
// then the launch of the right kernels on the caller's stream.  No allocation, no
// global state.
#include <cmath>
#include "../../include/deltanet.h"
#include "internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Checks shared by both entry points.  Returns DN_OK or the error to report.
dn_status check_common(const dn_shape* s) {
    if (!s) return DN_ERR_INVALID_ARG;
    if (s->B < 0 || s->T < 0 || s->num_seqs < 0 || s->Hqk <= 0 || s->Hv <= 0 || s->Dk <= 0 ||
        s->Dv <= 0)
        return DN_ERR_INVALID_ARG;
    if (s->Hv % s->Hqk != 0) return DN_ERR_INVALID_ARG;
    if (s->dtype != DN_F32 && s->dtype != DN_BF16) return DN_ERR_UNSUPPORTED;
    if (!dim_ok(s->Dk) || !dim_ok(s->Dv)) return DN_ERR_UNSUPPORTED;
    if (s->flags & ~(DN_QK_L2NORM | DN_GATE_PER_KEY)) return DN_ERR_INVALID_ARG;
    if ((s->flags & DN_QK_L2NORM) && !(s->l2norm_eps >= 0.f && s->l2norm_eps <= 3.0e38f))
        return DN_ERR_INVALID_ARG;
    return DN_OK;
}

// The epilogue's fields; fills `e` (kind -1 when ep is null and `optional`).
dn_status check_epilogue(const dn_epilogue* ep, bool optional, dn::EpilogueArgs& e) {
    e = dn::EpilogueArgs{-1, 0.f, nullptr, nullptr, nullptr};
    if (!ep) return optional ? DN_OK : DN_ERR_INVALID_ARG;
    if (ep->kind != DN_NORM_RMS && ep->kind != DN_NORM_LAYER) return DN_ERR_INVALID_ARG;
    if (!(ep->eps >= 0.f && ep->eps <= 3.0e38f)) return DN_ERR_INVALID_ARG;
    if (ep->kind == DN_NORM_RMS && ep->bias) return DN_ERR_INVALID_ARG;
    if ((ep->weight && !aligned4(ep->weight)) || (ep->bias && !aligned4(ep->bias)) ||
        (ep->gate && !aligned16(ep->gate)))
        return DN_ERR_INVALID_ARG;
    e.kind = ep->kind;
    e.eps = ep->eps;
    e.w = ep->weight;
    e.b = ep->bias;
    e.gate = ep->gate;
    return DN_OK;
}

}  // namespace

extern "C" {

int32_t dn_version(void) { return 10200; }

const char* dn_status_str(dn_status st) {
    switch (st) {
        case DN_OK: return "ok";
        case DN_ERR_INVALID_ARG: return "invalid argument";
        case DN_ERR_UNSUPPORTED: return "unsupported size or dtype";
        case DN_ERR_HIP: return "HIP runtime error";
        case DN_ERR_WORKSPACE: return "workspace missing or too small";
    }
    return "unknown status";
}

// Sizes of a prefill call.  `packed` tells whether cu_seqlens is given.
static dn_status prefill_shape(const dn_shape* s, bool packed, dn::PrefillArgs& a) {
    dn_status st = check_common(s);
    if (st != DN_OK) return st;
    const int C = s->chunk_size == 0 ? 64 : s->chunk_size;
    if (C != 16 && C != 32 && C != 64) return DN_ERR_UNSUPPORTED;
    if (packed) {
        if (s->B != 1 || s->num_seqs < 1) return DN_ERR_INVALID_ARG;
    } else if (s->num_seqs != s->B) {
        return DN_ERR_INVALID_ARG;
    }
    a = dn::PrefillArgs{};
    a.B = s->B; a.T = s->T; a.N = s->num_seqs; a.Hqk = s->Hqk; a.Hv = s->Hv;
    a.Dk = s->Dk; a.Dv = s->Dv; a.C = C; a.bf16 = s->dtype == DN_BF16; a.scale = s->scale;
    a.qk_norm = (s->flags & DN_QK_L2NORM) != 0;
    a.eps = s->l2norm_eps;
    a.g_per_key = (s->flags & DN_GATE_PER_KEY) != 0;
    return DN_OK;
}

size_t dn_chunk_fwd_workspace_bytes(const dn_shape* s) {
    // The bound covers both a batch of rows and a packed batch of num_seqs sequences.
    dn::PrefillArgs a;
    const bool packed = s && s->B == 1 && s->num_seqs != 1;
    if (prefill_shape(s, packed, a) != DN_OK) return 0;
    // the two-kernel channel-gate path keeps per-chunk operands in HBM
    return dn::prefill_chg_workspace_bytes(a);
}

int32_t dn_chunk_fwd_path(const dn_shape* s, size_t ws_bytes) {
    dn::PrefillArgs a;
    const bool packed = s && s->B == 1 && s->num_seqs != 1;
    if (prefill_shape(s, packed, a) != DN_OK) return DN_PATH_INVALID;
    if (a.g_per_key) {
        if (!dn::prefill_chg_shape_ok(a)) return DN_PATH_VECTOR;
        const size_t need = dn::prefill_chg_workspace_bytes(a);
        return ws_bytes >= need ? DN_PATH_CHANNEL_GATE_TWO_KERNELS : DN_PATH_CHANNEL_GATE_ONE_KERNEL;
    }
    return dn::prefill_fused_supported(a) ? DN_PATH_FUSED : DN_PATH_VECTOR;
}

dn_status dn_chunk_fwd_noalloc(const dn_shape* s, const void* q, const void* k, const void* v,
                               const float* beta, const float* g, const float* h0, float* hT,
                               const int32_t* cu, void* o, hipStream_t stream) {
    // Only the two-kernel channel-gate path needs scratch; it gets the static array (the
    // checks that follow in dn_chunk_fwd see a workspace of exactly the array's size).
    dn::PrefillArgs a;
    dn_status st = prefill_shape(s, cu != nullptr, a);
    if (st != DN_OK) return st;
    void* ws = nullptr;
    size_t ws_bytes = 0;
    const size_t need = dn::prefill_chg_workspace_bytes(a);
    if (need > 0) {
        if (need > dn::noalloc_scratch_bytes()) return DN_ERR_WORKSPACE;
        if (dn::noalloc_scratch(&ws) != hipSuccess) return DN_ERR_HIP;
        ws_bytes = dn::noalloc_scratch_bytes();
    }
    return dn_chunk_fwd(s, q, k, v, beta, g, h0, hT, cu, o, ws, ws_bytes, stream);
}

dn_status dn_chunk_fwd(const dn_shape* s, const void* q, const void* k, const void* v,
                       const float* beta, const float* g, const float* h0, float* hT,
                       const int32_t* cu, void* o, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    dn::PrefillArgs a;
    dn_status st = prefill_shape(s, cu != nullptr, a);
    if (st != DN_OK) return st;
    const long tokens = (long)s->B * s->T;
    if (tokens > 0 && (!q || !k || !v || !beta || !o)) return DN_ERR_INVALID_ARG;
    if (a.g_per_key && !g) return DN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, h0, hT, o, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return DN_ERR_INVALID_ARG;
    const void* scalars[] = {beta, g, cu};
    for (const void* p : scalars)
        if (p && !aligned4(p)) return DN_ERR_INVALID_ARG;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g; a.h0 = h0; a.hT = hT; a.cu = cu; a.o = o;
    a.ws = ws;
    a.ws_bytes = ws_bytes;
    hipError_t e;
    if (dn::prefill_fused_supported(a)) {
        e = dn::launch_prefill_fused(a, stream);
    } else {
        e = dn::launch_prefill_generic(a, stream);
    }
    return e == hipSuccess ? DN_OK : DN_ERR_HIP;
}

dn_status dn_recurrent_fwd(const dn_shape* s, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, const float* h0, float* hT,
                           const int32_t* cu, void* o, float* trace, hipStream_t stream) {
    dn::RecurrentArgs a;
    dn_status st = prefill_shape(s, cu != nullptr, a);
    if (st != DN_OK) return st;
    const long tokens = (long)s->B * s->T;
    if (tokens > 0 && (!q || !k || !v || !beta || !o)) return DN_ERR_INVALID_ARG;
    if (a.g_per_key && !g) return DN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, h0, hT, o, trace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return DN_ERR_INVALID_ARG;
    const void* scalars[] = {beta, g, cu};
    for (const void* p : scalars)
        if (p && !aligned4(p)) return DN_ERR_INVALID_ARG;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g; a.h0 = h0; a.hT = hT; a.cu = cu; a.o = o;
    a.trace = trace;
    return dn::launch_recurrent(a, stream) == hipSuccess ? DN_OK : DN_ERR_HIP;
}

static dn_status conv_shape(const dn_conv_shape* s, dn::ConvArgs& a) {
    if (!s) return DN_ERR_INVALID_ARG;
    if (s->B < 0 || s->T < 0 || s->num_seqs < 0 || s->C <= 0 || s->C % 8) return DN_ERR_INVALID_ARG;
    if (s->dtype != DN_F32 && s->dtype != DN_BF16) return DN_ERR_UNSUPPORTED;
    if (s->width < 2 || s->width > 8) return DN_ERR_UNSUPPORTED;
    if (s->activation != 0 && s->activation != 1) return DN_ERR_INVALID_ARG;
    a = dn::ConvArgs{};
    a.B = s->B; a.T = s->T; a.N = s->num_seqs; a.C = s->C; a.W = s->width;
    a.bf16 = s->dtype == DN_BF16; a.silu = s->activation;
    a.y_stride = s->C;
    return DN_OK;
}

dn_status dn_causal_conv(const dn_conv_shape* s, const void* x, const float* w, const float* b,
                         const void* s0, void* sT, const int32_t* cu, void* y, hipStream_t stream) {
    dn::ConvArgs a;
    dn_status st = conv_shape(s, a);
    if (st != DN_OK) return st;
    if (cu) {
        if (s->B != 1 || s->num_seqs < 1) return DN_ERR_INVALID_ARG;
    } else if (s->num_seqs != s->B) {
        return DN_ERR_INVALID_ARG;
    }
    const long tokens = (long)s->B * s->T;
    if (!w || (tokens > 0 && (!x || !y))) return DN_ERR_INVALID_ARG;
    if ((x && !aligned16(x)) || (y && !aligned16(y)) || !aligned4(w) || (b && !aligned4(b)) ||
        (cu && !aligned4(cu)))
        return DN_ERR_INVALID_ARG;
    const int es = s->dtype == DN_BF16 ? 2 : 4;
    if ((s0 && ((uintptr_t)s0 % es)) || (sT && ((uintptr_t)sT % es))) return DN_ERR_INVALID_ARG;
    if ((x && x == y) || (s0 && s0 == sT)) return DN_ERR_INVALID_ARG;
    a.x = x; a.w = w; a.b = b; a.s0 = s0; a.sT = sT; a.cu = cu; a.y = y;
    return dn::launch_causal_conv(a, stream) == hipSuccess ? DN_OK : DN_ERR_HIP;
}

dn_status dn_conv_qkv(const dn_conv_shape* s, const dn_qkv_split* sp, const void* x,
                      const float* w, const float* b, const void* s0, void* sT, const int32_t* cu,
                      void* q, void* k, void* v, hipStream_t stream) {
    dn::ConvArgs a;
    dn_status st = conv_shape(s, a);
    if (st != DN_OK) return st;
    if (!sp) return DN_ERR_INVALID_ARG;
    if (sp->Hqk < 1 || sp->Hv < 1 || sp->Dv < 8 || sp->Dv % 8) return DN_ERR_INVALID_ARG;
    if (sp->Dk != 16 && sp->Dk != 32 && sp->Dk != 64 && sp->Dk != 128) return DN_ERR_UNSUPPORTED;
    if ((long)s->C != 2L * sp->Hqk * sp->Dk + (long)sp->Hv * sp->Dv) return DN_ERR_INVALID_ARG;
    if (sp->qk_l2norm != 0 && sp->qk_l2norm != 1) return DN_ERR_INVALID_ARG;
    if (!(sp->eps >= 0.f) || !std::isfinite(sp->eps)) return DN_ERR_INVALID_ARG;
    if (cu) {
        if (s->B != 1 || s->num_seqs < 1) return DN_ERR_INVALID_ARG;
    } else if (s->num_seqs != s->B) {
        return DN_ERR_INVALID_ARG;
    }
    const long tokens = (long)s->B * s->T;
    if (!w || (tokens > 0 && (!x || !q || !k || !v))) return DN_ERR_INVALID_ARG;
    const void* p16[] = {x, q, k, v};
    for (const void* p : p16)
        if (p && !aligned16(p)) return DN_ERR_INVALID_ARG;
    if (!aligned4(w) || (b && !aligned4(b)) || (cu && !aligned4(cu))) return DN_ERR_INVALID_ARG;
    const int es = s->dtype == DN_BF16 ? 2 : 4;
    if ((s0 && ((uintptr_t)s0 % es)) || (sT && ((uintptr_t)sT % es))) return DN_ERR_INVALID_ARG;
    if (x && (x == q || x == k || x == v)) return DN_ERR_INVALID_ARG;
    if (tokens > 0 && (q == k || q == v || k == v)) return DN_ERR_INVALID_ARG;
    if (s0 && s0 == sT) return DN_ERR_INVALID_ARG;
    a.x = x; a.w = w; a.b = b; a.s0 = s0; a.sT = sT; a.cu = cu;
    a.qk = sp->Hqk * sp->Dk;
    a.q = q; a.k = k; a.y = v;
    a.y_stride = (long)sp->Hv * sp->Dv;
    a.Dk = sp->Dk;
    a.qk_norm = sp->qk_l2norm;
    a.eps = sp->eps;
    return dn::launch_causal_conv(a, stream) == hipSuccess ? DN_OK : DN_ERR_HIP;
}

dn_status dn_causal_conv_step(const dn_conv_shape* s, const void* x, const float* w, const float* b,
                              void* state, void* y, hipStream_t stream) {
    dn::ConvArgs a;
    dn_status st = conv_shape(s, a);
    if (st != DN_OK) return st;
    if (s->T != 1 || s->num_seqs != s->B) return DN_ERR_INVALID_ARG;
    if (!w || (s->B > 0 && (!x || !y || !state))) return DN_ERR_INVALID_ARG;
    const int es = s->dtype == DN_BF16 ? 2 : 4;
    if ((x && !aligned16(x)) || (y && !aligned16(y)) || !aligned4(w) || (b && !aligned4(b)) ||
        (state && ((uintptr_t)state % es)))
        return DN_ERR_INVALID_ARG;
    a.x = x; a.w = w; a.b = b; a.s0 = state; a.sT = state; a.y = y;
    return dn::launch_causal_conv_step(a, stream) == hipSuccess ? DN_OK : DN_ERR_HIP;
}

size_t dn_recurrent_bwd_workspace_bytes(const dn_shape* s) {
    dn::PrefillArgs a;
    const bool packed = s && s->B == 1 && s->num_seqs != 1;
    if (prefill_shape(s, packed, a) != DN_OK) return 0;
    // dq, dk shares [slices, tokens, Hv, Dk]; dbeta [slices, tokens, Hv]; dg [slices, tokens,
    // Hv] or, with a decay per key channel, [slices, tokens, Hv, Dk]
    const size_t per = (s->flags & DN_GATE_PER_KEY) ? 3 * (size_t)s->Dk + 1 : 2 * (size_t)s->Dk + 2;
    return (size_t)dn::recurrent_bwd_slices(s->Dk, s->Dv) * s->B * s->T * s->Hv * per * sizeof(float);
}

dn_status dn_recurrent_bwd(const dn_shape* s, const void* q, const void* k, const void* v,
                           const float* beta, const float* g, const float* h0,
                           const float* trace, const void* dout, const float* dfinal,
                           const int32_t* cu, float* dq, float* dk, float* dv, float* dbeta,
                           float* dg, float* dh0, void* ws, size_t ws_bytes, hipStream_t stream) {
    dn::RecurrentBwdArgs a{};
    dn_status st = prefill_shape(s, cu != nullptr, a);
    if (st != DN_OK) return st;
    if (a.g_per_key && !g) return DN_ERR_INVALID_ARG;
    const long tokens = (long)s->B * s->T;
    if (tokens > 0 && (!q || !k || !v || !beta || !trace || !dout || !dq || !dk || !dv || !dbeta ||
                       (g && !dg)))
        return DN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, h0, trace, dout, dfinal, dh0, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return DN_ERR_INVALID_ARG;
    const void* scalars[] = {beta, g, cu, dq, dk, dv, dbeta, dg};
    for (const void* p : scalars)
        if (p && !aligned4(p)) return DN_ERR_INVALID_ARG;
    const size_t need = dn_recurrent_bwd_workspace_bytes(s);
    if (need && (!ws || ws_bytes < need)) return DN_ERR_WORKSPACE;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g; a.h0 = h0; a.cu = cu;
    a.trace = trace; a.dout = dout; a.dfinal = dfinal;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dbeta = dbeta; a.dg = g ? dg : nullptr; a.dh0 = dh0;
    // the slices' shares: dq, dk [slices, tokens, Hv, Dk], then dbeta [slices, tokens, Hv],
    // then dg ([slices, tokens, Hv], or [slices, tokens, Hv, Dk] with a decay per key channel)
    const size_t qk = (size_t)dn::recurrent_bwd_slices(s->Dk, s->Dv) * tokens * s->Hv * s->Dk;
    const size_t sc = (size_t)dn::recurrent_bwd_slices(s->Dk, s->Dv) * tokens * s->Hv;
    a.ws_dq = static_cast<float*>(ws);
    a.ws_dk = a.ws_dq + qk;
    a.ws_db = a.ws_dk + qk;
    a.ws_dg = a.ws_db + sc;
    return dn::launch_recurrent_bwd(a, stream) == hipSuccess ? DN_OK : DN_ERR_HIP;
}

// Chunk numbers the chunkwise reverse pass keeps per value head: every batch row's chunks,
// or the packed bound; a query without cu_seqlens at B == 1 may be followed by either call.
static long chunk_bwd_ncid(const dn_shape* s, bool packed) {
    const long rows = (long)s->B * ((s->T + 63) / 64);
    const long pk = (long)(s->T / 64) + s->num_seqs + 1;
    return packed ? pk : (s->B == 1 ? (rows > pk ? rows : pk) : rows);
}

size_t dn_chunk_bwd_workspace_bytes(const dn_shape* s) {
    dn::PrefillArgs a;
    const bool packed = s && s->B == 1 && s->num_seqs != 1;
    if (prefill_shape(s, packed, a) != DN_OK || !dn::chunk_bwd_supported(a)) return 0;
    return dn::chunk_bwd_workspace_bytes(a, chunk_bwd_ncid(s, packed));
}

dn_status dn_chunk_bwd(const dn_shape* s, const void* q, const void* k, const void* v,
                       const float* beta, const float* g, const float* h0, const void* dout,
                       const float* dfinal, const int32_t* cu, float* dq, float* dk, float* dv,
                       float* dbeta, float* dg, float* dh0, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    dn::ChunkBwdArgs a{};
    dn_status st = prefill_shape(s, cu != nullptr, a);
    if (st != DN_OK) return st;
    if (!dn::chunk_bwd_supported(a)) return DN_ERR_UNSUPPORTED;
    const long tokens = (long)s->B * s->T;
    if (tokens > 0 && (!q || !k || !v || !beta || !dout || !dq || !dk || !dv || !dbeta || (g && !dg)))
        return DN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, h0, dout, dfinal, dh0, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return DN_ERR_INVALID_ARG;
    const void* scalars[] = {beta, g, cu, dq, dk, dv, dbeta, dg};
    for (const void* p : scalars)
        if (p && !aligned4(p)) return DN_ERR_INVALID_ARG;
    const size_t need = dn::chunk_bwd_workspace_bytes(a, chunk_bwd_ncid(s, cu != nullptr));
    if (!ws || ws_bytes < need) return DN_ERR_WORKSPACE;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g; a.h0 = h0; a.cu = cu; a.ws = ws;
    a.ws_bytes = ws_bytes;
    a.dout = dout; a.dfinal = dfinal;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dbeta = dbeta; a.dg = g ? dg : nullptr; a.dh0 = dh0;
    return dn::launch_chunk_bwd(a, stream) == hipSuccess ? DN_OK : DN_ERR_HIP;
}

dn_status dn_decode_step(const dn_shape* s, const void* q, const void* k, const void* v,
                         const float* beta, const float* g, float* state, void* o,
                         hipStream_t stream) {
    return dn_decode_step_ex(s, q, k, v, beta, g, state, nullptr, o, stream);
}

dn_status dn_decode_step_ex(const dn_shape* s, const void* q, const void* k, const void* v,
                            const float* beta, const float* g, float* state,
                            const dn_epilogue* ep, void* o, hipStream_t stream) {
    dn_status st = check_common(s);
    if (st != DN_OK) return st;
    dn::EpilogueArgs e;
    st = check_epilogue(ep, true, e);
    if (st != DN_OK) return st;
    if (s->T != 1 || s->num_seqs != s->B) return DN_ERR_INVALID_ARG;
    if (s->B > 0 && (!q || !k || !v || !beta || !state || !o)) return DN_ERR_INVALID_ARG;
    const void* ptrs[] = {q, k, v, state, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return DN_ERR_INVALID_ARG;
    const void* scalars[] = {beta, g};
    for (const void* p : scalars)
        if (p && !aligned4(p)) return DN_ERR_INVALID_ARG;
    dn::DecodeArgs a{};
    a.N = s->B; a.Hqk = s->Hqk; a.Hv = s->Hv; a.Dk = s->Dk; a.Dv = s->Dv;
    a.bf16 = s->dtype == DN_BF16; a.scale = s->scale;
    a.qk_norm = (s->flags & DN_QK_L2NORM) != 0;
    a.eps = s->l2norm_eps;
    a.g_per_key = (s->flags & DN_GATE_PER_KEY) != 0;
    if (a.g_per_key && !g) return DN_ERR_INVALID_ARG;
    a.q = q; a.k = k; a.v = v; a.beta = beta; a.g = g; a.state = state; a.o = o;
    a.ep = e;
    return dn::launch_decode(a, stream) == hipSuccess ? DN_OK : DN_ERR_HIP;
}

dn_status dn_norm_gate(const dn_shape* s, const dn_epilogue* ep, const void* o, void* y,
                       hipStream_t stream) {
    dn_status st = check_common(s);
    if (st != DN_OK) return st;
    dn::EpilogueArgs e;
    st = check_epilogue(ep, false, e);
    if (st != DN_OK) return st;
    const long rows = (long)s->B * s->T * s->Hv;
    if (rows > 0 && (!o || !y)) return DN_ERR_INVALID_ARG;
    if ((o && !aligned16(o)) || (y && !aligned16(y))) return DN_ERR_INVALID_ARG;
    dn::NormGateArgs a{};
    a.rows = rows;
    a.Dv = s->Dv;
    a.bf16 = s->dtype == DN_BF16;
    a.ep = e;
    a.o = o;
    a.y = y;
    return dn::launch_norm_gate(a, stream) == hipSuccess ? DN_OK : DN_ERR_HIP;
}

}  // extern "C"
