// kda_backward.hip -- gradients of the KDA forward pass (reverse mode of the token
// recurrence).  The pages describe a forward pass only (the news digest "FlashKDA Kernels
// 2.22x Faster for Kimi Attention": no backward yet); this is the chain rule applied to the
// recurrence the forward kernels evaluate (FlashKDA README "Kernel API" table and the
// FLA-backend flags; article index "Delta Attention Algorithm: linear-time recurrence"):
//
//   per token:  S' = S Diag(alpha);  r = v - S' k^;  S = S' + beta r k^T;  o = scale S q^
//
// Given dL/dout and dL/dS_final, with D = dL/dS after token t (V-major, D[v][c]):
//   D += scale do q^^T;   dq^ = scale S^T do;   u = D k^;   dv = beta u;   dbeta = u . r
//   dk^ = beta (D^T r - S'^T u);   da_c = sum_v S'[v][c] D[v][c] - beta k^_c (S'^T u)_c
//   D <- (D - beta u k^^T) Diag(alpha)
// and the activations' chain rules in a last parallel pass.  All arithmetic is fp32.
//
// Kernels, in launch order (the chunk table comes first, as in the forward pass):
//   bwd_prep_kernel    per token-head: k^, q^ (fp32), alpha, and 1/|k|, 1/|q|, beta
//   bwd_chain_kernel   per (sequence, head): a forward pass keeping the state at every
//                      16-token chunk start; then chunk by chunk in reverse: the chunk's
//                      per-token states S_{t-1} recomputed into a per-chain buffer, and the
//                      reverse step per token.  Writes dq^, dk^, da, the beta gradient before
//                      its sigmoid, dv, and dS_0.
//   bwd_finish_kernel  per token-head: l2norm, gate and sigmoid chain rules, in place
//   bwd_head_part_kernel, bwd_head_kernel
//                      per head: dt_bias and A_log gradients summed over all tokens (fixed
//                      token slices, then the slices in order: deterministic)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

constexpr int kBGateIn = 1, kBL2In = 2, kBSigIn = 4;
constexpr int kBThreads = 512;   // chain kernel: thread (c = tid % 128, vq = tid / 128)
constexpr int kBRows = 32;       // value rows per thread: 32 vq .. 32 vq + 31
constexpr int64_t kBState = (int64_t)kD * kD;

__device__ __forceinline__ float bbf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

struct BwdArgs {
    const uint16_t *q, *k, *v, *g, *beta, *dout;
    const float *A_log, *dt_bias;
    float scale, lower_bound;
    int flags;
    const void *h0;
    int h0_dtype;
    const float *dht;
    float *dq, *dk, *dv, *dg, *dbeta, *dA_log, *ddt, *dh0;
    int64_t B, T, H, N;
    const int64_t *seq_start, *seq_len, *seq_off;
    float *kn, *qn, *al;     // [B*T][H][128]
    float *rk, *rq, *bt;     // [B*T][H]
    float *ckpt;             // [n_chunks][H][128][128]: state before chunk (seq_off[n] + j)
    float *buf;              // [chains][16][128][128]: S_{t-1} of the chunk being reversed
    float *hpart;            // [H][kHeadSlices][2][128]: head-gradient partial sums
};

// ---- prep: one wavefront per token-head, two channels per lane ----
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // token * H + head
    if (th >= a.B * a.T * a.H)
        return;
    const int h = (int)(th % a.H);
    const size_t base = (size_t)th * kD;
    float qv[2], kv[2], gv[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int c = lane + 64 * e;
        qv[e] = bbf16(a.q[base + c]);
        kv[e] = bbf16(a.k[base + c]);
        gv[e] = bbf16(a.g[base + c]);
    }
    float qq = qv[0] * qv[0] + qv[1] * qv[1], kk = kv[0] * kv[0] + kv[1] * kv[1];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        qq += __shfl_xor(qq, o);
        kk += __shfl_xor(kk, o);
    }
    const bool l2_in = (a.flags & kBL2In) != 0;
    const float rq = l2_in ? 1.0f / sqrtf(qq + 1e-6f) : 1.0f;
    const float rk = l2_in ? 1.0f / sqrtf(kk + 1e-6f) : 1.0f;
    const float eA = (a.flags & kBGateIn) ? expf(a.A_log[h]) : 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int c = lane + 64 * e;
        float lg;
        if (a.flags & kBGateIn)
            lg = a.lower_bound / (1.0f + expf(-eA * (gv[e] + a.dt_bias[(size_t)h * kD + c])));
        else
            lg = fminf(fmaxf(gv[e], a.lower_bound), 0.f);
        a.kn[base + c] = kv[e] * rk;
        a.qn[base + c] = qv[e] * rq;
        a.al[base + c] = expf(lg);
    }
    if (lane == 0) {
        const float braw = bbf16(a.beta[th]);
        a.rk[th] = rk;
        a.rq[th] = rq;
        a.bt[th] = (a.flags & kBSigIn) ? 1.0f / (1.0f + expf(-braw)) : braw;
    }
}

// ---- chain kernel helpers ----
// Sum over the 128 channels of x[i] (this thread: channel c, rows 32 vq + i), for all 32 i:
// a reduce-scatter over the wavefront's 64 channels (after it lane L holds row L >> 1),
// the two half-sums of a row meet in LDS (part[wave][row]); returns nothing -- the caller
// reads part after a barrier: full(row j of quarter vq) = part[2vq][j] + part[2vq+1][j].
// One reduce-scatter step over lane bit O with N values left: lanes with bit O set keep the
// upper N/2 values (adding their partner's), the others the lower N/2.  The partner is a lane
// of the other side of bit O that holds the same values so far: for O = 32 and 16 the
// lanes 32 (16) apart, exchanged with v_permlane32_swap / v_permlane16_swap (which swap one
// half of one register with the other half of a second, so one swap serves a pair of values
// and every lane's sum is the sum of the two swapped registers); for O = 8 and 4 the mirror
// lane within 16 (8) lanes, for O = 2 and 1 the xor lane within 4, all by DPP.
template <int N>
__device__ __forceinline__ void swap_step32(float *x)
{
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[j]), __float_as_uint(x[j + N / 2]), false,
                                                        false);
        x[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}
template <int N>
__device__ __forceinline__ void swap_step16(float *x)
{
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[j]), __float_as_uint(x[j + N / 2]), false,
                                                        false);
        x[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
}
// DPP controls: row_mirror (lane i <- 15 - i of its row), row_half_mirror (i <- 7 - i of its
// half row), quad_perm [2,3,0,1] (xor 2), quad_perm [1,0,3,2] (xor 1)
template <int O, int N, int kCtrl>
__device__ __forceinline__ void dpp_step(float *x, int lane)
{
    const bool up = (lane & O) != 0;
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
        const float send = up ? x[j] : x[j + N / 2];
        const float keep = up ? x[j + N / 2] : x[j];
        x[j] = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), kCtrl, 0xf, 0xf, false));
    }
}

__device__ __forceinline__ void row_reduce(float *x, float *part, int wave, int lane)
{
    swap_step32<32>(x);
    swap_step16<16>(x);
    dpp_step<8, 8, 0x140>(x, lane);
    dpp_step<4, 4, 0x141>(x, lane);
    dpp_step<2, 2, 0x4e>(x, lane);
    x[0] += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x[0]), 0xb1, 0xf, 0xf, false));
    if ((lane & 1) == 0)
        part[wave * 32 + (lane >> 1)] = x[0];
}

__device__ __forceinline__ void bwd_barrier()
{
    __syncthreads();
}

// 32 bf16 values (a row block of one token-head) widened, all lanes the same addresses
// (here: LDS rows of the staged chunk)
__device__ __forceinline__ void load_rows_bf16(const uint16_t *p, float *x)
{
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const u32x4 w = *reinterpret_cast<const u32x4 *>(p + 8 * m);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[8 * m + 2 * e] = __uint_as_float(w[e] << 16);
            x[8 * m + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
}

// One token forward: S <- S' + beta r k^^T with S' = S Diag(alpha), r = v - S' k^ (vrow:
// this thread's 32 rows of v, bf16).  With r_lds set, the threads of channel 0 also store r
// for their rows there.  Two barriers inside.
__device__ __forceinline__ void fwd_token(float *S, float kc, float ac, float bt, const uint16_t *vrow,
                                         float *r_lds, float *part, int wave, int lane, int vq, int c)
{
    float x[kBRows];
#pragma unroll
    for (int i = 0; i < kBRows; ++i) {
        S[i] *= ac;
        x[i] = S[i] * kc;
    }
    row_reduce(x, part, wave, lane);
    bwd_barrier();
    float vv[kBRows];
    load_rows_bf16(vrow, vv);
#pragma unroll
    for (int i = 0; i < kBRows; ++i) {
        const float r = vv[i] - (part[(2 * vq) * 32 + i] + part[(2 * vq + 1) * 32 + i]);
        S[i] = fmaf(bt * r, kc, S[i]);
        if (r_lds && c == 0)
            r_lds[kBRows * vq + i] = r;
    }
    bwd_barrier();  // part is read by every thread before the next token overwrites it
}

// The per-token vectors of one chunk (up to 16 tokens), staged in LDS once per chunk so that
// the token steps read them there instead of waiting on global memory twice per token:
// k^, alpha, beta, the v row and, for the reverse pass, q^ and the dout row.
struct Stage {
    float kn[kCH][kD], al[kCH][kD], qn[kCH][kD];
    uint16_t v[kCH][kD], dout[kCH][kD];
    float bt[kCH];
};

// Thread tid loads 4 channels (4 (tid % 32) ..) of token tid / 32 of tokens [t0, t1) (its
// token-head rows from th(t)); the caller puts a barrier before (readers of the previous
// chunk) and after (readers of this one).
template <typename TH>
__device__ __forceinline__ void stage_chunk(const BwdArgs &a, Stage &st, int64_t t0, int64_t t1, bool rev,
                                            TH th, int tid)
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const int r = tid >> 5, c4 = 4 * (tid & 31);
    if (t0 + r < t1) {
        const size_t ti = th(t0 + r);
        *reinterpret_cast<f32x4 *>(&st.kn[r][c4]) = *reinterpret_cast<const f32x4 *>(a.kn + ti * kD + c4);
        *reinterpret_cast<f32x4 *>(&st.al[r][c4]) = *reinterpret_cast<const f32x4 *>(a.al + ti * kD + c4);
        *reinterpret_cast<u32x2 *>(&st.v[r][c4]) = *reinterpret_cast<const u32x2 *>(a.v + ti * kD + c4);
        if (rev) {
            *reinterpret_cast<f32x4 *>(&st.qn[r][c4]) = *reinterpret_cast<const f32x4 *>(a.qn + ti * kD + c4);
            *reinterpret_cast<u32x2 *>(&st.dout[r][c4]) = *reinterpret_cast<const u32x2 *>(a.dout + ti * kD + c4);
        }
        if ((tid & 31) == 0)
            st.bt[r] = a.bt[ti];
    }
}

__global__ __launch_bounds__(kBThreads) void bwd_chain_kernel(BwdArgs a)
{
    __shared__ float s_part[8 * 32];           // row-reduction half sums
    __shared__ float s_r[kCH][kD];             // r_t of the chunk being reversed
    __shared__ float s_col[4][5][kD];          // per-quarter column sums: A, B, C, E, (u.r at c = 0)
    __shared__ __attribute__((aligned(16))) Stage s_st;  // the chunk's per-token vectors
    const int64_t chain = blockIdx.x;
    const int64_t H = a.H;
    if (chain >= a.N * H)
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c = tid & (kD - 1), vq = tid >> 7;
    const int64_t n = chain / H;
    const int h = (int)(chain % H);
    const int64_t start = a.seq_start[n], len = a.seq_len[n], off = a.seq_off[n];
    const int64_t nch = (len + kCH - 1) / kCH;
    float *buf = a.buf + (size_t)chain * kCH * kBState;
    auto ck = [&](int64_t j) { return a.ckpt + ((size_t)(off + j) * (size_t)H + (size_t)h) * kBState; };
    auto th = [&](int64_t t) { return (size_t)(start + t) * (size_t)H + (size_t)h; };  // token-head index
    const size_t col = (size_t)(kBRows * vq) * kD + (size_t)c;  // this thread's entry in a 128 x 128 block

    // initial state
    float S[kBRows];
    {
        const size_t sb = (size_t)chain * kBState + col;
#pragma unroll
        for (int i = 0; i < kBRows; ++i) {
            float s0 = 0.f;
            if (a.h0_dtype == 2)
                s0 = reinterpret_cast<const float *>(a.h0)[sb + (size_t)i * kD];
            else if (a.h0_dtype == 1)
                s0 = bbf16(reinterpret_cast<const uint16_t *>(a.h0)[sb + (size_t)i * kD]);
            S[i] = s0;
        }
    }
    // forward pass: the state before every chunk
    for (int64_t j = 0; j < nch; ++j) {
        float *cp = ck(j) + col;
#pragma unroll
        for (int i = 0; i < kBRows; ++i)
            cp[(size_t)i * kD] = S[i];
        const int64_t t0 = j * kCH, t1 = (j + 1) * kCH < len ? (j + 1) * kCH : len;
        bwd_barrier();  // the previous chunk's stage is read
        stage_chunk(a, s_st, t0, t1, false, th, tid);
        bwd_barrier();
        for (int64_t t = t0; t < t1; ++t) {
            const int r = (int)(t - t0);
            fwd_token(S, s_st.kn[r][c], s_st.al[r][c], s_st.bt[r], &s_st.v[r][kBRows * vq], nullptr,
                      s_part, wave, lane, vq, c);
        }
    }
    // reverse pass
    float D[kBRows];
    {
        const size_t sb = (size_t)chain * kBState + col;
#pragma unroll
        for (int i = 0; i < kBRows; ++i)
            D[i] = a.dht ? a.dht[sb + (size_t)i * kD] : 0.f;
    }
    const float scale = a.scale;
    for (int64_t j = nch - 1; j >= 0; --j) {
        const int64_t t0 = j * kCH;
        const int64_t t1 = t0 + kCH < len ? t0 + kCH : len;
        // recompute the chunk: S_{t-1} into the buffer, r_t into LDS
        {
            const float *cp = ck(j) + col;
#pragma unroll
            for (int i = 0; i < kBRows; ++i)
                S[i] = cp[(size_t)i * kD];
        }
        bwd_barrier();  // the previous chunk's stage is read
        stage_chunk(a, s_st, t0, t1, true, th, tid);
        bwd_barrier();
        for (int64_t t = t0; t < t1; ++t) {
            const int r = (int)(t - t0);
            float *bp = buf + (size_t)r * kBState + col;
#pragma unroll
            for (int i = 0; i < kBRows; ++i)
                bp[(size_t)i * kD] = S[i];
            fwd_token(S, s_st.kn[r][c], s_st.al[r][c], s_st.bt[r], &s_st.v[r][kBRows * vq], s_r[r], s_part, wave,
                      lane, vq, c);
        }
        // s_r complete (every thread reads back only the buffer entries it wrote itself)
        bwd_barrier();
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const size_t ti = th(t);
            const int r = (int)(t - t0);
            const float kc = s_st.kn[r][c], qc = s_st.qn[r][c], ac = s_st.al[r][c];
            const float bt = s_st.bt[r];
            const uint16_t *dorow = &s_st.dout[r][kBRows * vq];
            const float *bp = buf + (size_t)(t - t0) * kBState + col;
            float x[kBRows];
            {
                float dov[kBRows];
                load_rows_bf16(dorow, dov);
#pragma unroll
                for (int i = 0; i < kBRows; ++i) {
                    D[i] = fmaf(scale * dov[i], qc, D[i]);
                    x[i] = D[i] * kc;
                }
            }
            row_reduce(x, s_part, wave, lane);
            bwd_barrier();
            // S' and do again (cached), so that neither is live across the reduction
            float A = 0.f, Bs = 0.f, C = 0.f, E = 0.f, ur = 0.f;
            {
                float dov[kBRows];
                load_rows_bf16(dorow, dov);
#pragma unroll
                for (int i = 0; i < kBRows; ++i) {
                    const float u = s_part[(2 * vq) * 32 + i] + s_part[(2 * vq + 1) * 32 + i];
                    const float rr = s_r[t - t0][kBRows * vq + i];
                    const float sp = bp[(size_t)i * kD] * ac;
                    const float st = fmaf(bt * rr, kc, sp);
                    A = fmaf(st, dov[i], A);
                    Bs = fmaf(D[i], rr, Bs);
                    C = fmaf(sp, u, C);
                    E = fmaf(sp, D[i], E);
                    ur = fmaf(u, rr, ur);
                    D[i] = (D[i] - bt * u * kc) * ac;
                }
            }
            if (c < kBRows)  // dv for row 32 vq + c
                a.dv[ti * kD + kBRows * vq + c] = bt * (s_part[(2 * vq) * 32 + c] + s_part[(2 * vq + 1) * 32 + c]);
            s_col[vq][0][c] = A;
            s_col[vq][1][c] = Bs;
            s_col[vq][2][c] = C;
            s_col[vq][3][c] = E;
            if (c == 0)
                s_col[vq][4][0] = ur;
            bwd_barrier();
            if (tid < kD) {
                float sA = 0.f, sB = 0.f, sC = 0.f, sE = 0.f;
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    sA += s_col[p][0][c];
                    sB += s_col[p][1][c];
                    sC += s_col[p][2][c];
                    sE += s_col[p][3][c];
                }
                a.dq[ti * kD + c] = scale * sA;                 // dq^ (chain rule in finish)
                a.dk[ti * kD + c] = bt * (sB - sC);             // dk^
                a.dg[ti * kD + c] = sE - bt * kc * sC;          // d(log-decay) = dalpha * alpha
                if (c == 0)
                    a.dbeta[ti] = s_col[0][4][0] + s_col[1][4][0] + s_col[2][4][0] + s_col[3][4][0];
            }
            // s_part and s_col are rewritten after the next token's first barrier; the
            // readers above are done by then
        }
        bwd_barrier();  // s_r of this chunk is read by everyone before the next chunk rewrites it
    }
    if (a.dh0) {
        float *p = a.dh0 + (size_t)chain * kBState + col;
#pragma unroll
        for (int i = 0; i < kBRows; ++i)
            p[(size_t)i * kD] = D[i];
    }
}

// ---- finish: activations' chain rules, in place, one wavefront per token-head ----
__global__ __launch_bounds__(256) void bwd_finish_kernel(BwdArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t th = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (th >= a.B * a.T * a.H)
        return;
    const int h = (int)(th % a.H);
    const size_t base = (size_t)th * kD;
    float dqn[2], dkn[2], qn[2], kn[2];
    float pq = 0.f, pk = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int c = lane + 64 * e;
        dqn[e] = a.dq[base + c];
        dkn[e] = a.dk[base + c];
        qn[e] = a.qn[base + c];
        kn[e] = a.kn[base + c];
        pq = fmaf(qn[e], dqn[e], pq);
        pk = fmaf(kn[e], dkn[e], pk);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        pq += __shfl_xor(pq, o);
        pk += __shfl_xor(pk, o);
    }
    const bool l2_in = (a.flags & kBL2In) != 0;
    const float rq = a.rq[th], rk = a.rk[th];
    const float eA = (a.flags & kBGateIn) ? expf(a.A_log[h]) : 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int c = lane + 64 * e;
        // l2norm: dq = (dq^ - q^ (q^ . dq^)) / |q|
        a.dq[base + c] = l2_in ? (dqn[e] - qn[e] * pq) * rq : dqn[e];
        a.dk[base + c] = l2_in ? (dkn[e] - kn[e] * pk) * rk : dkn[e];
        const float da = a.dg[base + c];
        const float gc = bbf16(a.g[base + c]);
        float dgv;
        if (a.flags & kBGateIn) {
            const float x = eA * (gc + a.dt_bias[(size_t)h * kD + c]);
            const float s = 1.0f / (1.0f + expf(-x));
            dgv = da * a.lower_bound * s * (1.0f - s) * eA;
        } else {
            dgv = (gc > a.lower_bound && gc < 0.f) ? da : 0.f;
        }
        a.dg[base + c] = dgv;
    }
    if (lane == 0 && (a.flags & kBSigIn)) {
        const float b = a.bt[th];
        a.dbeta[th] = a.dbeta[th] * b * (1.0f - b);
    }
}

// ---- head reduction: ddt_bias[h][c] = sum_t dg, dA_log[h] = sum_{t,c} dg (g + dt_bias) ----
// dt_bias and A_log gradients: per head, sums over every token of dg (d log-decay) and of
// dg * (g + dt_bias) (the gate's pre-activation x = e^{A_log} (g + dt_bias) has dx/dA_log = x
// and the d log-decay / dx factor is already in dg).  Two passes with a fixed partition and a
// fixed order (deterministic): bwd_head_part_kernel sums kHeadSlices contiguous token ranges
// per head (two interleaved halves of each range meet in LDS), bwd_head_kernel adds the
// slices in order.
__global__ __launch_bounds__(256) void bwd_head_part_kernel(BwdArgs a)
{
    __shared__ float s_d[2][kD], s_a[2][kD];
    const int h = blockIdx.x / kHeadSlices, slice = blockIdx.x % kHeadSlices;
    const int c = threadIdx.x & (kD - 1), half = threadIdx.x >> 7;
    const int64_t ntok = a.B * a.T;
    const int64_t t0 = ntok * slice / kHeadSlices, t1 = ntok * (slice + 1) / kHeadSlices;
    const float dt = a.dt_bias[(size_t)h * kD + c];
    float sd = 0.f, sa = 0.f;
    for (int64_t t = t0 + half; t < t1; t += 2) {
        const size_t i = ((size_t)t * (size_t)a.H + (size_t)h) * kD + (size_t)c;
        const float d = a.dg[i];
        sd += d;
        sa = fmaf(d, bbf16(a.g[i]) + dt, sa);
    }
    s_d[half][c] = sd;
    s_a[half][c] = sa;
    __syncthreads();
    if (half == 0) {
        float *part = a.hpart + ((size_t)h * kHeadSlices + (size_t)slice) * 2 * kD;
        part[c] = s_d[0][c] + s_d[1][c];
        part[kD + c] = s_a[0][c] + s_a[1][c];
    }
}

__global__ __launch_bounds__(kD) void bwd_head_kernel(BwdArgs a)
{
    __shared__ float s_a[kD];
    const int h = blockIdx.x, c = threadIdx.x;
    const float *part = a.hpart + (size_t)h * kHeadSlices * 2 * kD;
    float sd = 0.f, sa = 0.f;
    for (int sl = 0; sl < kHeadSlices; ++sl) {
        sd += part[(size_t)sl * 2 * kD + c];
        sa += part[(size_t)sl * 2 * kD + kD + c];
    }
    if (a.ddt)
        a.ddt[(size_t)h * kD + c] = sd;
    s_a[c] = sa;
    __syncthreads();
    if (c == 0 && a.dA_log) {
        float tot = 0.f;  // over the 128 channels in order
        for (int j = 0; j < kD; ++j)
            tot += s_a[j];
        a.dA_log[h] = tot;
    }
}

}  // namespace

hipError_t launch_backward(const BwdLaunch &f, hipStream_t s)
{
    BwdArgs a;
    a.q = f.fwd.q;
    a.k = f.fwd.k;
    a.v = f.fwd.v;
    a.g = f.fwd.g;
    a.beta = f.fwd.beta;
    a.dout = f.dout;
    a.A_log = f.fwd.A_log;
    a.dt_bias = f.fwd.dt_bias;
    a.scale = f.fwd.scale;
    a.lower_bound = f.fwd.lower_bound;
    a.flags = f.fwd.flags;
    a.h0 = f.fwd.h0;
    a.h0_dtype = f.fwd.h0_dtype;
    a.dht = f.dht;
    a.dq = f.dq;
    a.dk = f.dk;
    a.dv = f.dv;
    a.dg = f.dg;
    a.dbeta = f.dbeta;
    a.dA_log = f.dA_log;
    a.ddt = f.ddt;
    a.dh0 = f.dh0;
    a.B = f.fwd.B;
    a.T = f.fwd.T;
    a.H = f.fwd.H;
    a.N = f.fwd.lay.n_seq;
    unsigned char *ws = f.fwd.ws;
    a.seq_start = reinterpret_cast<const int64_t *>(ws + f.fwd.lay.off_seq_start);
    a.seq_len = reinterpret_cast<const int64_t *>(ws + f.fwd.lay.off_seq_len);
    a.seq_off = reinterpret_cast<const int64_t *>(ws + f.fwd.lay.off_seq_off);
    a.kn = reinterpret_cast<float *>(ws + f.bl.off_kn);
    a.qn = reinterpret_cast<float *>(ws + f.bl.off_qn);
    a.al = reinterpret_cast<float *>(ws + f.bl.off_al);
    a.rk = reinterpret_cast<float *>(ws + f.bl.off_rk);
    a.rq = reinterpret_cast<float *>(ws + f.bl.off_rq);
    a.bt = reinterpret_cast<float *>(ws + f.bl.off_bt);
    a.ckpt = reinterpret_cast<float *>(ws + f.bl.off_ckpt);
    a.buf = reinterpret_cast<float *>(ws + f.bl.off_buf);
    a.hpart = reinterpret_cast<float *>(ws + f.bl.off_hpart);
    const int64_t toks = a.B * a.T * a.H;
    const int64_t chains = a.N * a.H;
    if (toks > 0) {
        hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((toks + 3) / 4)), dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (chains > 0) {
        hipLaunchKernelGGL(bwd_chain_kernel, dim3((unsigned)chains), dim3(kBThreads), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (toks > 0) {
        hipLaunchKernelGGL(bwd_finish_kernel, dim3((unsigned)((toks + 3) / 4)), dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    if (a.flags & kBGateIn) {
        hipLaunchKernelGGL(bwd_head_part_kernel, dim3((unsigned)(a.H * kHeadSlices)), dim3(256), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        hipLaunchKernelGGL(bwd_head_kernel, dim3((unsigned)a.H), dim3(kD), 0, s, a);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace kda
