// kda_api.cpp -- host side of libkda.so: argument validation, workspace layout and the
// C ABI declared in include/kda.h.  Validation is plain host code that touches no HIP
// API, so every error path can be exercised without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "kda.h"
#include "kda_internal.h"

namespace {

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};
Range range_of(const void *p, size_t bytes)
{
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, lo + bytes};
}
bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

size_t state_elem_bytes(kda_state_dtype d) { return d == KDA_STATE_BF16 ? 2 : 4; }

// Everything kda_fwd checks before touching the device.
kda_status validate(const void *q, const void *k, const void *v, const void *g, const void *beta,
                    float scale, void *out, const float *A_log, const float *dt_bias,
                    float lower_bound, const void *h0, kda_state_dtype h0_dt, void *ht,
                    kda_state_dtype ht_dt, const int64_t *cu, const int64_t *cu_host, int64_t B,
                    int64_t T, int64_t H, int64_t N, int64_t K, int64_t V, void *ws,
                    size_t ws_bytes, uint32_t flags, kda::Layout *lay)
{
    if ((flags & ~KDA_ALL_IN_KERNEL) != 0)
        return KDA_ERR_FLAGS;
    // A_log and dt_bias feed only the in-pass gate
    const bool gate_in = (flags & KDA_GATE_IN_KERNEL) != 0;
    // token tensors may be NULL only when they hold no elements (B * T == 0)
    const bool no_tokens = (T == 0);
    if ((!no_tokens && (!q || !k || !v || !g || !beta || !out)) || (gate_in && (!A_log || !dt_bias)))
        return KDA_ERR_NULL;
    if (B < 1 || T < 0 || H < 1)
        return KDA_ERR_SHAPE;
    if (cu) {
        if (B != 1 || N < 1)
            return KDA_ERR_SHAPE;
    } else if (N != 0 && N != B) {
        return KDA_ERR_SHAPE;
    }
    // overflow guard on element counts (tokens * heads * 128 must fit comfortably); a
    // sequence (at most T tokens) has fewer than 2^31 chunks of 16
    if (T > ((int64_t)1 << 40) / B || (B * T) > ((int64_t)1 << 46) / (H * kda::kD) ||
        T >= ((int64_t)1 << 35))
        return KDA_ERR_SHAPE;
    if (K != kda::kD || V != kda::kD)
        return KDA_ERR_HEAD_DIM;
    auto dt_ok = [](kda_state_dtype d) {
        return d == KDA_STATE_NONE || d == KDA_STATE_BF16 || d == KDA_STATE_FP32;
    };
    if (!dt_ok(h0_dt) || !dt_ok(ht_dt))
        return KDA_ERR_DTYPE;
    if ((h0 == nullptr) != (h0_dt == KDA_STATE_NONE) || (ht == nullptr) != (ht_dt == KDA_STATE_NONE))
        return KDA_ERR_DTYPE;
    if (h0 && ht && h0_dt != ht_dt)
        return KDA_ERR_DTYPE;
    if (!(lower_bound >= -5.0f && lower_bound <= 0.0f))  // also rejects NaN
        return KDA_ERR_LOWER_BOUND;
    if (!isfinite(scale))
        return KDA_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) ||
        !aligned(out, 16) || !aligned(beta, 2) || (gate_in && (!aligned(A_log, 4) || !aligned(dt_bias, 16))) ||
        (h0 && !aligned(h0, 16)) || (ht && !aligned(ht, 16)) || (cu && !aligned(cu, 8)) ||
        (ws && !aligned(ws, kda::kAlign)))
        return KDA_ERR_ALIGN;

    const int64_t n_seq = cu ? N : B;
    const size_t tok_bytes = (size_t)B * (size_t)T * (size_t)H * kda::kD * 2;
    const size_t beta_bytes = (size_t)B * (size_t)T * (size_t)H * 2;
    const Range rq = range_of(q, tok_bytes), rk = range_of(k, tok_bytes), rv = range_of(v, tok_bytes),
                rg = range_of(g, tok_bytes), rb = range_of(beta, beta_bytes), ro = range_of(out, tok_bytes);
    if (overlap(ro, rq) || overlap(ro, rk) || overlap(ro, rv) || overlap(ro, rg) || overlap(ro, rb))
        return KDA_ERR_ALIAS;
    if (ht) {
        const Range rs = range_of(ht, (size_t)n_seq * (size_t)H * kda::kD * kda::kD * state_elem_bytes(ht_dt));
        if (overlap(rs, rq) || overlap(rs, rk) || overlap(rs, rv) || overlap(rs, rg) ||
            overlap(rs, rb) || overlap(rs, ro))
            return KDA_ERR_ALIAS;
        if (h0 && h0 != ht) {
            const Range ri = range_of(h0, (size_t)n_seq * (size_t)H * kda::kD * kda::kD * state_elem_bytes(h0_dt));
            if (overlap(rs, ri))
                return KDA_ERR_ALIAS;
        }
    }
    if (h0) {
        const Range ri = range_of(h0, (size_t)n_seq * (size_t)H * kda::kD * kda::kD * state_elem_bytes(h0_dt));
        if (overlap(ri, ro))
            return KDA_ERR_ALIAS;
    }

    if (!kda::make_layout(B, T, H, cu ? N : 0, cu != nullptr, lay))
        return KDA_ERR_SHAPE;
    if (!ws || ws_bytes < lay->total)
        return KDA_ERR_WORKSPACE;
    if (cu && cu_host) {
        if (cu_host[0] != 0 || cu_host[N] != T)
            return KDA_ERR_CU_SEQLENS;
        for (int64_t i = 0; i < N; ++i)
            if (cu_host[i + 1] < cu_host[i])
                return KDA_ERR_CU_SEQLENS;
    }
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_version(void) { return 100; }

const char *kda_status_string(int s)
{
    switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: invalid B/T/H/N or cu_seqlens with B != 1";
    case KDA_ERR_HEAD_DIM: return "KDA_ERR_HEAD_DIM: K and V must be 128";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: invalid or mismatched state dtypes";
    case KDA_ERR_LOWER_BOUND: return "KDA_ERR_LOWER_BOUND: lower_bound must be in [-5, 0]";
    case KDA_ERR_SCALE: return "KDA_ERR_SCALE: scale must be finite";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: pointer alignment requirement violated";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: workspace missing or too small";
    case KDA_ERR_CU_SEQLENS: return "KDA_ERR_CU_SEQLENS: cu_seqlens content invalid";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: HIP launch or query failed";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input";
    case KDA_ERR_FLAGS: return "KDA_ERR_FLAGS: unknown activation switch bits";
    case KDA_ERR_SCRATCH: return "KDA_ERR_SCRATCH: the call needs more than kda_fwd_noalloc's static scratch";
    default: return "KDA_ERR_UNKNOWN";
    }
}

size_t kda_fwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t N, int has_cu_seqlens)
{
    kda::Layout lay;
    if (!kda::make_layout(B, T, H, has_cu_seqlens ? N : (N == B ? B : 0), has_cu_seqlens != 0, &lay))
        return 0;
    return lay.total;
}

}  // extern "C"

namespace {

kda_status fwd_impl(const void *q, const void *k, const void *v, const void *g, const void *beta,
                    float scale, void *out, const float *A_log, const float *dt_bias,
                    float lower_bound, const void *initial_state, kda_state_dtype initial_state_dtype,
                    void *final_state, kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                    const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H, int64_t N,
                    int64_t K, int64_t V, void *workspace, size_t workspace_bytes, void *stream,
                    uint32_t flags, void *const *events, bool recurrent = false)
{
    kda::Layout lay;
    kda_status st = validate(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound,
                             initial_state, initial_state_dtype, final_state, final_state_dtype,
                             cu_seqlens, cu_seqlens_host, B, T, H, N, K, V, workspace,
                             workspace_bytes, flags, &lay);
    if (st != KDA_OK)
        return st;
    kda::FwdArgs a;
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.g = static_cast<const uint16_t *>(g);
    a.beta = static_cast<const uint16_t *>(beta);
    a.out = static_cast<uint16_t *>(out);
    a.A_log = A_log;
    a.dt_bias = dt_bias;
    a.scale = scale;
    a.lower_bound = lower_bound;
    a.flags = (int)flags;
    a.h0 = initial_state;
    a.ht = final_state;
    a.h0_dtype = (int)initial_state_dtype;
    a.ht_dtype = (int)final_state_dtype;
    a.cu = cu_seqlens;
    a.B = B;
    a.T = T;
    a.H = H;
    a.N = lay.n_seq;
    a.ws = static_cast<unsigned char *>(workspace);
    a.lay = lay;
    hipStream_t s = static_cast<hipStream_t>(stream);
    auto mark = [&](int i) {
        return events == nullptr || hipEventRecord(static_cast<hipEvent_t>(events[i]), s) == hipSuccess;
    };
    if (!mark(0) || kda::launch_chunk_table(a, s, !recurrent) != hipSuccess)
        return KDA_ERR_HIP;
    hipEvent_t marks[3];
    if (events)
        for (int i = 0; i < 3; ++i)
            marks[i] = static_cast<hipEvent_t>(events[2 + i]);
    if (recurrent)
        return mark(1) && kda::launch_recurrent(a, s) == hipSuccess && mark(2) ? KDA_OK : KDA_ERR_HIP;
    if (!mark(1) || kda::launch_forward(a, s, events ? marks : nullptr) != hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}

}  // namespace

extern "C" {

kda_status kda_fwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                   float scale, void *out, const float *A_log, const float *dt_bias,
                   float lower_bound, const void *initial_state, kda_state_dtype initial_state_dtype,
                   void *final_state, kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                   const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H, int64_t N,
                   int64_t K, int64_t V, void *workspace, size_t workspace_bytes, void *stream)
{
    return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                    initial_state_dtype, final_state, final_state_dtype, cu_seqlens, cu_seqlens_host,
                    B, T, H, N, K, V, workspace, workspace_bytes, stream, KDA_ALL_IN_KERNEL, nullptr);
}

kda_status kda_fwd_ex(const void *q, const void *k, const void *v, const void *g, const void *beta,
                      float scale, void *out, const float *A_log, const float *dt_bias,
                      float lower_bound, const void *initial_state, kda_state_dtype initial_state_dtype,
                      void *final_state, kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                      const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H, int64_t N,
                      int64_t K, int64_t V, void *workspace, size_t workspace_bytes, void *stream,
                      uint32_t flags)
{
    return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                    initial_state_dtype, final_state, final_state_dtype, cu_seqlens, cu_seqlens_host,
                    B, T, H, N, K, V, workspace, workspace_bytes, stream, flags, nullptr);
}

kda_status kda_fwd_recurrent(const void *q, const void *k, const void *v, const void *g, const void *beta,
                             float scale, void *out, const float *A_log, const float *dt_bias,
                             float lower_bound, const void *initial_state,
                             kda_state_dtype initial_state_dtype, void *final_state,
                             kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                             const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H, int64_t N,
                             int64_t K, int64_t V, void *workspace, size_t workspace_bytes, void *stream,
                             uint32_t flags)
{
    return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                    initial_state_dtype, final_state, final_state_dtype, cu_seqlens, cu_seqlens_host,
                    B, T, H, N, K, V, workspace, workspace_bytes, stream, flags, nullptr, true);
}

kda_status kda_fwd_recurrent_timed(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, float scale, void *out, const float *A_log,
                                   const float *dt_bias, float lower_bound, const void *initial_state,
                                   kda_state_dtype initial_state_dtype, void *final_state,
                                   kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                                   const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H,
                                   int64_t N, int64_t K, int64_t V, void *workspace,
                                   size_t workspace_bytes, void *stream, uint32_t flags,
                                   void *const *stage_events)
{
    if (!stage_events)
        return KDA_ERR_NULL;
    for (int i = 0; i < 3; ++i)
        if (!stage_events[i])
            return KDA_ERR_NULL;
    return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                    initial_state_dtype, final_state, final_state_dtype, cu_seqlens, cu_seqlens_host,
                    B, T, H, N, K, V, workspace, workspace_bytes, stream, flags, stage_events, true);
}

kda_status kda_fwd_timed(const void *q, const void *k, const void *v, const void *g, const void *beta,
                         float scale, void *out, const float *A_log, const float *dt_bias,
                         float lower_bound, const void *initial_state,
                         kda_state_dtype initial_state_dtype, void *final_state,
                         kda_state_dtype final_state_dtype, const int64_t *cu_seqlens,
                         const int64_t *cu_seqlens_host, int64_t B, int64_t T, int64_t H, int64_t N,
                         int64_t K, int64_t V, void *workspace, size_t workspace_bytes, void *stream,
                         void *const *stage_events)
{
    if (!stage_events)
        return KDA_ERR_NULL;
    for (int i = 0; i < 5; ++i)
        if (!stage_events[i])
            return KDA_ERR_NULL;
    return fwd_impl(q, k, v, g, beta, scale, out, A_log, dt_bias, lower_bound, initial_state,
                    initial_state_dtype, final_state, final_state_dtype, cu_seqlens, cu_seqlens_host,
                    B, T, H, N, K, V, workspace, workspace_bytes, stream, KDA_ALL_IN_KERNEL,
                    stage_events);
}

kda_status kda_fwd_device_status(const void *workspace, int32_t *status_out, void *stream)
{
    if (!workspace || !status_out)
        return KDA_ERR_NULL;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(status_out, workspace, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess)
        return KDA_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}

kda_status kda_chunk_table(const int64_t *cu_seqlens, int64_t B, int64_t T, int64_t H, int64_t N,
                           void *workspace, size_t workspace_bytes, int64_t *seq_off_host,
                           int64_t *n_total_host, int32_t *status_host, void *stream)
{
    kda::Layout lay;
    if (B < 1 || T < 0 || H < 1)
        return KDA_ERR_SHAPE;
    if (!kda::make_layout(B, T, H, cu_seqlens ? N : 0, cu_seqlens != nullptr, &lay))
        return KDA_ERR_SHAPE;
    if (!workspace || workspace_bytes < lay.total)
        return KDA_ERR_WORKSPACE;
    if (!aligned(workspace, kda::kAlign) || (cu_seqlens && !aligned(cu_seqlens, 8)))
        return KDA_ERR_ALIGN;
    kda::FwdArgs a;
    memset(&a, 0, sizeof a);
    a.cu = cu_seqlens;
    a.B = B;
    a.T = T;
    a.H = H;
    a.N = lay.n_seq;
    a.ws = static_cast<unsigned char *>(workspace);
    a.lay = lay;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (kda::launch_chunk_table(a, s) != hipSuccess)
        return KDA_ERR_HIP;
    bool copied = false;
    if (seq_off_host) {
        if (hipMemcpyAsync(seq_off_host, a.ws + lay.off_seq_off, sizeof(int64_t) * (lay.n_seq + 1),
                           hipMemcpyDeviceToHost, s) != hipSuccess)
            return KDA_ERR_HIP;
        copied = true;
    }
    if (n_total_host) {
        if (hipMemcpyAsync(n_total_host, a.ws + lay.off_status + 8, sizeof(int64_t),
                           hipMemcpyDeviceToHost, s) != hipSuccess)
            return KDA_ERR_HIP;
        copied = true;
    }
    if (status_host) {
        if (hipMemcpyAsync(status_host, a.ws + lay.off_status, sizeof(int32_t), hipMemcpyDeviceToHost,
                           s) != hipSuccess)
            return KDA_ERR_HIP;
        copied = true;
    }
    if (copied && hipStreamSynchronize(s) != hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}

}  // extern "C"

namespace {

// Everything kda_bwd checks before touching the device.
kda_status validate_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta,
                        float scale, const float *A_log, const float *dt_bias, float lower_bound,
                        const void *h0, kda_state_dtype h0_dt, const void *dout, const float *dht,
                        const float *dq, const float *dk, const float *dv, const float *dg,
                        const float *dbeta, const float *dA_log, const float *ddt, const float *dh0,
                        const int64_t *cu, const int64_t *cu_host, int64_t B, int64_t T, int64_t H,
                        int64_t N, int64_t K, int64_t V, const void *ws, size_t ws_bytes, uint32_t flags,
                        kda::BwdLayout *bl)
{
    if ((flags & ~KDA_ALL_IN_KERNEL) != 0)
        return KDA_ERR_FLAGS;
    const bool gate_in = (flags & KDA_GATE_IN_KERNEL) != 0;
    const bool tokens = T > 0;
    if ((tokens && (!q || !k || !v || !g || !beta || !dout || !dq || !dk || !dv || !dg || !dbeta)) ||
        (gate_in && (!A_log || !dt_bias)))
        return KDA_ERR_NULL;
    if (B < 1 || T < 0 || H < 1)
        return KDA_ERR_SHAPE;
    if (cu) {
        if (B != 1 || N < 1)
            return KDA_ERR_SHAPE;
    } else if (N != 0 && N != B) {
        return KDA_ERR_SHAPE;
    }
    if (T > ((int64_t)1 << 40) / B || (B * T) > ((int64_t)1 << 46) / (H * kda::kD) || T >= ((int64_t)1 << 35))
        return KDA_ERR_SHAPE;
    if (K != kda::kD || V != kda::kD)
        return KDA_ERR_HEAD_DIM;
    if (!(h0_dt == KDA_STATE_NONE || h0_dt == KDA_STATE_BF16 || h0_dt == KDA_STATE_FP32) ||
        (h0 == nullptr) != (h0_dt == KDA_STATE_NONE))
        return KDA_ERR_DTYPE;
    if (!(lower_bound >= -5.0f && lower_bound <= 0.0f))
        return KDA_ERR_LOWER_BOUND;
    if (!isfinite(scale))
        return KDA_ERR_SCALE;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(g, 16) || !aligned(dout, 16) ||
        !aligned(beta, 2) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(dg, 16) ||
        !aligned(dbeta, 4) || (gate_in && (!aligned(A_log, 4) || !aligned(dt_bias, 16))) ||
        (dA_log && !aligned(dA_log, 4)) || (ddt && !aligned(ddt, 16)) || (h0 && !aligned(h0, 16)) ||
        (dht && !aligned(dht, 16)) || (dh0 && !aligned(dh0, 16)) || (cu && !aligned(cu, 8)) ||
        (ws && !aligned(ws, kda::kAlign)))
        return KDA_ERR_ALIGN;
    const int64_t n_seq = cu ? N : B;
    const size_t tokh = (size_t)B * (size_t)T * (size_t)H;
    const size_t st = (size_t)n_seq * (size_t)H * kda::kD * kda::kD;
    const Range ins[] = {range_of(q, tokh * kda::kD * 2), range_of(k, tokh * kda::kD * 2),
                         range_of(v, tokh * kda::kD * 2), range_of(g, tokh * kda::kD * 2),
                         range_of(beta, tokh * 2), range_of(dout, tokh * kda::kD * 2),
                         range_of(h0, h0 ? st * state_elem_bytes(h0_dt) : 0), range_of(dht, dht ? st * 4 : 0),
                         range_of(A_log, gate_in ? (size_t)H * 4 : 0),
                         range_of(dt_bias, gate_in ? (size_t)H * kda::kD * 4 : 0)};
    const Range outs[] = {range_of(dq, tokh * kda::kD * 4), range_of(dk, tokh * kda::kD * 4),
                          range_of(dv, tokh * kda::kD * 4), range_of(dg, tokh * kda::kD * 4),
                          range_of(dbeta, tokh * 4), range_of(dA_log, dA_log ? (size_t)H * 4 : 0),
                          range_of(ddt, ddt ? (size_t)H * kda::kD * 4 : 0), range_of(dh0, dh0 ? st * 4 : 0)};
    for (const Range &o : outs) {
        for (const Range &i : ins)
            if (overlap(o, i))
                return KDA_ERR_ALIAS;
        for (const Range &o2 : outs)
            if (&o2 != &o && overlap(o, o2))
                return KDA_ERR_ALIAS;
    }
    if (!kda::make_bwd_layout(B, T, H, cu ? N : 0, cu != nullptr, bl))
        return KDA_ERR_SHAPE;
    if (!ws || ws_bytes < bl->total)
        return KDA_ERR_WORKSPACE;
    if (cu && cu_host) {
        if (cu_host[0] != 0 || cu_host[N] != T)
            return KDA_ERR_CU_SEQLENS;
        for (int64_t i = 0; i < N; ++i)
            if (cu_host[i + 1] < cu_host[i])
                return KDA_ERR_CU_SEQLENS;
    }
    return KDA_OK;
}

}  // namespace

extern "C" {

size_t kda_bwd_workspace_size(int64_t B, int64_t T, int64_t H, int64_t N, int has_cu_seqlens)
{
    kda::BwdLayout bl;
    if (!kda::make_bwd_layout(B, T, H, has_cu_seqlens ? N : (N == B ? B : 0), has_cu_seqlens != 0, &bl))
        return 0;
    return bl.total;
}

kda_status kda_bwd(const void *q, const void *k, const void *v, const void *g, const void *beta, float scale,
                   const float *A_log, const float *dt_bias, float lower_bound, const void *initial_state,
                   kda_state_dtype initial_state_dtype, const void *dout, const float *dfinal_state, float *dq,
                   float *dk, float *dv, float *dg, float *dbeta, float *dA_log, float *ddt_bias,
                   float *dinitial_state, const int64_t *cu_seqlens, const int64_t *cu_seqlens_host, int64_t B,
                   int64_t T, int64_t H, int64_t N, int64_t K, int64_t V, void *workspace,
                   size_t workspace_bytes, void *stream, uint32_t flags)
{
    kda::BwdLayout bl;
    kda_status st = validate_bwd(q, k, v, g, beta, scale, A_log, dt_bias, lower_bound, initial_state,
                                 initial_state_dtype, dout, dfinal_state, dq, dk, dv, dg, dbeta, dA_log,
                                 ddt_bias, dinitial_state, cu_seqlens, cu_seqlens_host, B, T, H, N, K, V,
                                 workspace, workspace_bytes, flags, &bl);
    if (st != KDA_OK)
        return st;
    kda::BwdLaunch a;
    memset(&a, 0, sizeof a);
    a.fwd.q = static_cast<const uint16_t *>(q);
    a.fwd.k = static_cast<const uint16_t *>(k);
    a.fwd.v = static_cast<const uint16_t *>(v);
    a.fwd.g = static_cast<const uint16_t *>(g);
    a.fwd.beta = static_cast<const uint16_t *>(beta);
    a.fwd.A_log = A_log;
    a.fwd.dt_bias = dt_bias;
    a.fwd.scale = scale;
    a.fwd.lower_bound = lower_bound;
    a.fwd.flags = (int)flags;
    a.fwd.h0 = initial_state;
    a.fwd.h0_dtype = (int)initial_state_dtype;
    a.fwd.cu = cu_seqlens;
    a.fwd.B = B;
    a.fwd.T = T;
    a.fwd.H = H;
    a.fwd.N = bl.tab.n_seq;
    a.fwd.ws = static_cast<unsigned char *>(workspace);
    a.fwd.lay = bl.tab;
    a.bl = bl;
    a.dout = static_cast<const uint16_t *>(dout);
    a.dht = dfinal_state;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.dg = dg;
    a.dbeta = dbeta;
    a.dA_log = (flags & KDA_GATE_IN_KERNEL) ? dA_log : nullptr;
    a.ddt = (flags & KDA_GATE_IN_KERNEL) ? ddt_bias : nullptr;
    a.dh0 = dinitial_state;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (kda::launch_chunk_table(a.fwd, s, false) != hipSuccess || kda::launch_backward(a, s) != hipSuccess)
        return KDA_ERR_HIP;
    return KDA_OK;
}

}  // extern "C"

