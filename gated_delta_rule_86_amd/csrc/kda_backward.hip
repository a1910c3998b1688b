// kda_backward.hip -- gradients of the KDA forward pass.  The pages describe a forward pass
// only (the news digest "FlashKDA Kernels 2.22x Faster for Kimi Attention": no backward yet);
// this is the reverse mode of the recurrence the forward kernels evaluate (FlashKDA README
// "Kernel API" table and the FLA-backend flags; article index "Delta Attention Algorithm:
// linear-time recurrence"):
//
//   per token:  S' = S Diag(alpha);  r = v - S' k^;  S = S' + beta r k^T;  o = scale S q^
//
// taken in the chunked form of the forward pass (16-token chunks; within a chunk, with
// b the cumulative log-decay, Gamma = e^b per channel, gamma = Gamma of the last token):
//   KG = k^ Gamma, KI = k^ / Gamma, QG = scale q^ Gamma, KD = k^ gamma / Gamma
//   T = (I + strictly_lower(diag(beta) KG KI^T))^-1,  W = T diag(beta) KG,  U = T diag(beta) V
//   V' = U - W S0^T,  O = QG S0^T + lower(QG KI^T) V',  S_end = S0 Diag(gamma) + V'^T KD
// Reverse mode, with D = dL/dS_end and dO = dL/dO of the chunk:
//   dV' = lower(QG KI^T)^T dO + KD D^T            dS0 = D Diag(gamma) + dO^T QG - dV'^T W
// (neither needs S0: dL/dS runs backwards over the chunks on its own, as the state runs
// forwards), and for the chunk's inputs, given S0, D, V' and dV':
//   dKD = V' D,  dQG = dO S0 + dAqk KI,  dW = -dV' S0,  dgamma_c = sum_v S0[v][c] D[v][c]
//   dAqk = lower(dO V'^T),  P = T^T dV',  Q = T^T dW,  dv = beta P
//   dA = -strictly_lower(P U^T + Q W^T),  dbeta = rowdot(P, V) + rowdot(Q, KG) + rowdot(dA, KG KI^T)
//   dKG = diag(beta) (Q + dA KI),  dKI = dA^T diag(beta) KG + dAqk^T QG
//   dk^ = dKG Gamma + (dKI + dKD gamma) / Gamma,  dq^ = scale dQG Gamma
//   db = dKG KG - dKI KI + dQG QG - dKD KD, plus sum_r dKD KD + dgamma gamma on the last row;
//   d(log-decay) = reverse cumulative sum of db over the chunk.
// Then the activations' chain rules.  All arithmetic is fp32 (products on the fp32 MFMA).
//
// Kernels, in launch order (the chunk table comes first, as in the forward pass):
//   bwd_prep_kernel    per token-head: k^, q^, the log-decay a, and 1/|k|, 1/|q|, beta
//   bwd_ops_kernel     per chunk-head: the chunk's operands for the two chains (-W, U, KD,
//                      U~ = lower(QG KI^T)^T dO, QG, gamma, in the layouts they are read in)
//   bwd_chain_kernel   per (sequence, head, role, half of the value rows): role 0 runs the
//                      state forwards over the chunks, writing S0 and V' of every chunk; role 1
//                      runs dL/dS backwards, writing D and dV' of every chunk and dL/dS_0.  The
//                      value rows of a state are independent given the chunk operands, so two
//                      workgroups take 64 rows each.
//   bwd_grad_kernel    per chunk-head: the gradients of the chunk's tokens from S0, D, V', dV'
//                      (dq^, dk^, d log-decay, dbeta before its sigmoid, dv)
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
constexpr int64_t kBState = (int64_t)kD * kD;
constexpr int kP = kD + 4;         // LDS row stride of the [16][128] fp32 tiles
constexpr int kQ = kCH + 1;        // LDS row stride of the 16 x 16 tiles
constexpr int kGradThreads = 512;  // bwd_ops_kernel, bwd_grad_kernel
constexpr int kChainThreads = 256; // bwd_chain_kernel: 4 wavefronts of 16 value rows
// operand block of a chunk-head (kBwdOps floats)
constexpr int kOpNegW = 0, kOpU = 2048, kOpKDt = 4096, kOpKD = 6144, kOpUt = 8192, kOpQGt = 10240,
              kOpNegWt = 12288, kOpGam = 14336;
static_assert(kOpGam + kD == kBwdOps, "operand block layout");

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bbf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st4(float *p, f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }
// four bf16 values widened (8-byte aligned)
__device__ __forceinline__ f32x4 ld4_bf16(const uint16_t *p)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 w = *reinterpret_cast<const u32x2 *>(p);
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                 __uint_as_float(w[1] & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// The four steps of one 16-wide slice of a contraction: lane L holds a = A[L % 16][k0 + 4 (L / 16)
// .. + 3] and b = B[k0 + 4 (L / 16) .. + 3][L % 16] (step j takes element j of both); the
// accumulator is in the D layout (lane L, element i: row 4 (L / 16) + i, column L % 16).
__device__ __forceinline__ f32x4 mm4(f32x4 a, f32x4 b, f32x4 c)
{
    c = mfma4(a[0], b[0], c);
    c = mfma4(a[1], b[1], c);
    c = mfma4(a[2], b[2], c);
    return mfma4(a[3], b[3], c);
}
// acc + A B^T for A, B [16][nk] row-major in LDS (row stride kP), one wavefront
__device__ __forceinline__ f32x4 mm_rows(const float *A, const float *B, int nk, f32x4 acc, int lane)
{
    const int m = lane & 15, g = lane >> 4;
    for (int t = 0; t < nk; t += 16)
        acc = mm4(ld4(A + m * kP + t + 4 * g), ld4(B + m * kP + t + 4 * g), acc);
    return acc;
}

struct BwdArgs {
    const uint16_t *q, *k, *v, *g, *beta, *dout;
    const float *A_log, *dt_bias;
    float scale, lower_bound;
    int flags;
    const void *h0;
    int h0_dtype;
    const float *dht;
    float *dq, *dk, *dv, *dg, *dbeta, *dA_log, *ddt, *dh0;
    int64_t B, T, H, N, chunks;
    const int64_t *seq_start, *seq_len, *seq_off;
    float *kn, *qn, *lg;     // [B*T][H][128]
    float *rk, *rq, *bt;     // [B*T][H]
    float *ops;              // [chunks][H][kBwdOps]
    float *cks, *ckd;        // [chunks][H][128][128]: S before the chunk, dL/dS after it (transposed)
    float *xf, *xb;          // [chunks][H][16][128]: V' and dL/dV'
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
        a.lg[base + c] = lg;
    }
    if (lane == 0) {
        const float braw = bbf16(a.beta[th]);
        a.rk[th] = rk;
        a.rq[th] = rq;
        a.bt[th] = (a.flags & kBSigIn) ? 1.0f / (1.0f + expf(-braw)) : braw;
    }
}

// ---- per-chunk operands (shared by bwd_ops_kernel and bwd_grad_kernel) ----
// Chunk x of a head's chunk list: sequence n (the first with seq_off[n + 1] > x), chunk j of
// it, first token t0 (row index), len tokens (1 .. 16).  False past the last chunk.
struct ChunkLoc {
    int64_t n, t0;
    int len;
};
__device__ bool locate_chunk(const BwdArgs &a, int64_t x, ChunkLoc &c)
{
    if (x >= a.seq_off[a.N])
        return false;
    int64_t lo = 0, hi = a.N - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (a.seq_off[mid + 1] > x)
            hi = mid;
        else
            lo = mid + 1;
    }
    const int64_t j = x - a.seq_off[lo];
    c.n = lo;
    c.t0 = a.seq_start[lo] + kCH * j;
    const int64_t rem = a.seq_len[lo] - kCH * j;
    c.len = rem < kCH ? (int)rem : kCH;
    return true;
}

// Rows past the chunk's tokens are zero (k^, q^, v, dO, beta, log-decay), which leaves every
// quantity of the real rows as it is and gamma the decay up to the last real token.
struct PrepLds {
    float KG[kCH][kP], KI[kCH][kP], QG[kCH][kP], KD[kCH][kP], Gm[kCH][kP], Gi[kCH][kP];
    float W[kCH][kP], U[kCH][kP], V[kCH][kP], dO[kCH][kP];
    float T[kCH][kQ], M[kCH][kQ], Aqk[kCH][kQ];  // T, KG KI^T, lower(QG KI^T)
    float beta[kCH], gam[kD];
};

// kGradThreads threads; ends with a barrier.
__device__ void prep_chunk(const BwdArgs &a, const ChunkLoc &c, int h, PrepLds &p, int tid)
{
    {  // the chunk's rows: thread -> token r = tid / 32, channels 4 (tid % 32) .. + 3
        const int r = tid >> 5, c4 = 4 * (tid & 31);
        f32x4 kk = {0.f, 0.f, 0.f, 0.f}, qq = kk, ll = kk, vv = kk, oo = kk;
        float bt = 0.f;
        if (r < c.len) {
            const size_t ti = (size_t)(c.t0 + r) * (size_t)a.H + (size_t)h;
            kk = ld4(a.kn + ti * kD + c4);
            qq = ld4(a.qn + ti * kD + c4);
            ll = ld4(a.lg + ti * kD + c4);
            vv = ld4_bf16(a.v + ti * kD + c4);
            oo = ld4_bf16(a.dout + ti * kD + c4);
            bt = a.bt[ti];
        }
        st4(&p.KG[r][c4], kk);  // k^ until the next step
        st4(&p.QG[r][c4], qq);  // q^
        st4(&p.Gm[r][c4], ll);  // log-decay
        st4(&p.V[r][c4], vv);
        st4(&p.dO[r][c4], oo);
        if ((tid & 31) == 0)
            p.beta[r] = bt;
    }
    __syncthreads();
    if (tid < kD) {  // per channel: b = cumulative log-decay, Gamma, 1 / Gamma, the gated rows
        const int ch = tid;
        float b[kCH];
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < kCH; ++r) {
            run += p.Gm[r][ch];
            b[r] = run;
        }
        const float gam = expf(run);
        p.gam[ch] = gam;
#pragma unroll
        for (int r = 0; r < kCH; ++r) {
            const float G = expf(b[r]), Gi = expf(-b[r]), k = p.KG[r][ch];
            p.Gm[r][ch] = G;
            p.Gi[r][ch] = Gi;
            p.KG[r][ch] = k * G;
            p.KI[r][ch] = k * Gi;
            p.KD[r][ch] = k * expf(run - b[r]);
            p.QG[r][ch] = a.scale * p.QG[r][ch] * G;
        }
    }
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, m = lane & 15;
    if (wave == 0) {  // KG KI^T
        const f32x4 acc = mm_rows(&p.KG[0][0], &p.KI[0][0], kD, f32x4{0.f, 0.f, 0.f, 0.f}, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            p.M[4 * g + i][m] = acc[i];
    } else if (wave == 1) {  // lower(QG KI^T), diagonal included
        const f32x4 acc = mm_rows(&p.QG[0][0], &p.KI[0][0], kD, f32x4{0.f, 0.f, 0.f, 0.f}, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            p.Aqk[4 * g + i][m] = m <= 4 * g + i ? acc[i] : 0.f;
    }
    __syncthreads();
    if (tid < kCH) {  // T = (I + A)^-1, A = strictly_lower(diag(beta) M): lane s solves column s
        const int s = tid;
        float t[kCH];
#pragma unroll
        for (int r = 0; r < kCH; ++r) {
            float x = r == s ? 1.f : 0.f;
            const float br = p.beta[r];
#pragma unroll
            for (int q = 0; q < r; ++q)
                x = fmaf(-br * p.M[r][q], t[q], x);
            t[r] = x;
        }
#pragma unroll
        for (int r = 0; r < kCH; ++r)
            p.T[r][s] = t[r];
    }
    __syncthreads();
    {  // W = T diag(beta) KG, U = T diag(beta) V: thread -> channel tid % 128, rows 4 (tid / 128) ..
        const int ch = tid & (kD - 1), q4 = 4 * (tid >> 7);
        float w[4] = {0.f, 0.f, 0.f, 0.f}, u[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kCH; ++s) {
            const float bk = p.beta[s] * p.KG[s][ch], bv = p.beta[s] * p.V[s][ch];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                w[i] = fmaf(p.T[q4 + i][s], bk, w[i]);
                u[i] = fmaf(p.T[q4 + i][s], bv, u[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p.W[q4 + i][ch] = w[i];
            p.U[q4 + i][ch] = u[i];
        }
    }
    __syncthreads();
}

// ---- operands of the two chains, one workgroup per chunk-head ----
__global__ __launch_bounds__(kGradThreads) void bwd_ops_kernel(BwdArgs a)
{
    __shared__ __attribute__((aligned(16))) PrepLds p;
    const int64_t x = blockIdx.x / a.H;
    const int h = (int)(blockIdx.x % a.H);
    ChunkLoc c;
    if (!locate_chunk(a, x, c))
        return;
    const int tid = threadIdx.x;
    prep_chunk(a, c, h, p, tid);
    float *o = a.ops + ((size_t)x * (size_t)a.H + (size_t)h) * kBwdOps;
    const int ch = tid & (kD - 1), q4 = 4 * (tid >> 7);
    f32x4 kd, qg, nw;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = q4 + i;
        float ut = 0.f;  // U~ = lower(QG KI^T)^T dO
#pragma unroll
        for (int s = 0; s < kCH; ++s)
            ut = fmaf(p.Aqk[s][r], p.dO[s][ch], ut);
        o[kOpNegW + r * kD + ch] = -p.W[r][ch];
        o[kOpU + r * kD + ch] = p.U[r][ch];
        o[kOpKD + r * kD + ch] = p.KD[r][ch];
        o[kOpUt + r * kD + ch] = ut;
        kd[i] = p.KD[r][ch];
        qg[i] = p.QG[r][ch];
        nw[i] = -p.W[r][ch];
    }
    st4(o + kOpKDt + ch * kCH + q4, kd);
    st4(o + kOpQGt + ch * kCH + q4, qg);
    st4(o + kOpNegWt + ch * kCH + q4, nw);
    if (tid < kD)
        o[kOpGam + tid] = p.gam[tid];
}

// ---- the two chains over the chunks of one (sequence, head) ----
// One chunk's operands for one half (64 value rows) of a chain, staged in LDS.
struct ChainStage {
    float A0[kCH * kD];  // role 0: -W [r][c];  role 1: KD [r][c]
    float A1[kD * kCH];  // role 0: KD^T [c][r]; role 1: QG^T [c][r]
    float A2[kD * kCH];  // role 1: -W^T [c][r]
    float U[kCH][64];    // role 0: U, role 1: U~ (the half's value columns)
    float O[kCH][64];    // role 1: dO (the half's value columns)
    float gam[kD];
};

// Global -> register copies of one chunk's stage (issued a chunk ahead), then register -> LDS.
struct StageRegs {
    f32x4 a0[2], a1[2], a2[2], u, o, gm;
};
__device__ __forceinline__ void stage_load(const BwdArgs &a, int role, int hv, const float *op, int64_t t0, int len,
                                           int h, StageRegs &r, int tid)
{
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int f = 4 * (tid + kChainThreads * e);
        r.a0[e] = ld4(op + (role ? kOpKD : kOpNegW) + f);
        r.a1[e] = ld4(op + (role ? kOpQGt : kOpKDt) + f);
        if (role)
            r.a2[e] = ld4(op + kOpNegWt + f);
    }
    const int row = tid >> 4, c4 = 4 * (tid & 15);
    r.u = ld4(op + (role ? kOpUt : kOpU) + row * kD + 64 * hv + c4);
    if (role) {
        r.o = f32x4{0.f, 0.f, 0.f, 0.f};
        if (row < len)
            r.o = ld4_bf16(a.dout + ((size_t)(t0 + row) * (size_t)a.H + (size_t)h) * kD + 64 * hv + c4);
    }
    if (tid < kD / 4)
        r.gm = ld4(op + kOpGam + 4 * tid);
}
__device__ __forceinline__ void stage_store(int role, const StageRegs &r, ChainStage &st, int tid)
{
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int f = 4 * (tid + kChainThreads * e);
        st4(st.A0 + f, r.a0[e]);
        st4(st.A1 + f, r.a1[e]);
        if (role)
            st4(st.A2 + f, r.a2[e]);
    }
    const int row = tid >> 4, c4 = 4 * (tid & 15);
    st4(&st.U[row][c4], r.u);
    if (role)
        st4(&st.O[row][c4], r.o);
    if (tid < kD / 4)
        st4(st.gam + 4 * tid, r.gm);
}

// Workgroups: XCD-aware pairs (the two halves of a (chain, role) unit land on one XCD and
// share its L2 for the operand reads).  Unit u: chain u / 2, role u % 2.  Wave w of half hv
// owns value rows v0 .. v0 + 15, v0 = 64 hv + 16 w; its state is held transposed in the
// D layout: tile ct (channels 16 ct ..) lane L element i = S[v0 + L % 16][16 ct + 4 (L / 16) + i].
__global__ __launch_bounds__(kChainThreads) void bwd_chain_kernel(BwdArgs a)
{
    __shared__ __attribute__((aligned(16))) ChainStage s_st[2];
    const int64_t bid = blockIdx.x;
    const int xcd = (int)(bid & 7);
    const int64_t slot = bid >> 3;
    const int hv = (int)(slot & 1);
    const int64_t unit = (slot >> 1) * 8 + xcd;
    const int64_t H = a.H;
    if (unit >= 2 * a.N * H)
        return;
    const int role = (int)(unit & 1);
    const int64_t chain = unit >> 1, n = chain / H;
    const int h = (int)(chain % H);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, m = lane & 15;
    const int v0 = 64 * hv + 16 * wave;
    const int64_t start = a.seq_start[n], len = a.seq_len[n], off = a.seq_off[n];
    const int64_t nch = (len + kCH - 1) / kCH;
    auto slot_of = [&](int64_t j) { return (size_t)(off + j) * (size_t)H + (size_t)h; };
    auto op_of = [&](int64_t j) { return a.ops + slot_of(j) * kBwdOps; };
    auto tok_len = [&](int64_t j) { return (int)(len - kCH * j < kCH ? len - kCH * j : kCH); };
    const size_t srow = (size_t)chain * kBState + (size_t)(v0 + m) * kD + 4 * g;  // + 16 ct
    f32x4 S[8];
    if (role == 0) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            if (a.h0_dtype == 2)
                S[ct] = ld4(reinterpret_cast<const float *>(a.h0) + srow + 16 * ct);
            else if (a.h0_dtype == 1)
                S[ct] = ld4_bf16(reinterpret_cast<const uint16_t *>(a.h0) + srow + 16 * ct);
            else
                S[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    } else {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
            S[ct] = a.dht ? ld4(a.dht + srow + 16 * ct) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    StageRegs rg;
    if (nch > 0) {
        const int64_t j0 = role ? nch - 1 : 0;
        stage_load(a, role, hv, op_of(j0), start + kCH * j0, tok_len(j0), h, rg, tid);
        stage_store(role, rg, s_st[0], tid);
    }
    __syncthreads();
    for (int64_t it = 0; it < nch; ++it) {
        const int64_t j = role ? nch - 1 - it : it, jn = role ? j - 1 : j + 1;
        const bool more = it + 1 < nch;
        if (more)
            stage_load(a, role, hv, op_of(jn), start + kCH * jn, tok_len(jn), h, rg, tid);
        const ChainStage &st = s_st[it & 1];
        const size_t sl = slot_of(j);
        // the state before the chunk (role 0) or dL/dS after it (role 1), as [channel][value row]
        float *ck = (role ? a.ckd : a.cks) + sl * kBState + v0 + m;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ck[(size_t)(16 * ct + 4 * g + i) * kD] = S[ct][i];
        // role 0: V' = U - W S^T;  role 1: dV' = U~ + KD D^T   (rows r = 4 g + i, column v0 + m)
        f32x4 X;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            X[i] = st.U[4 * g + i][16 * wave + m];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
            X = mm4(ld4(st.A0 + m * kD + 16 * ct + 4 * g), S[ct], X);
        float *xo = (role ? a.xb : a.xf) + sl * (kCH * kD) + v0 + m;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            xo[(4 * g + i) * kD] = X[i];
        if (role == 0) {
            if (more) {  // S <- S Diag(gamma) + V'^T KD
#pragma unroll
                for (int ct = 0; ct < 8; ++ct)
                    S[ct] = mm4(ld4(st.A1 + (16 * ct + m) * kCH + 4 * g), X, S[ct] * ld4(st.gam + 16 * ct + 4 * g));
            }
        } else {  // D <- D Diag(gamma) + dO^T QG - dV'^T W
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = st.O[4 * g + i][16 * wave + m];
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                f32x4 acc = S[ct] * ld4(st.gam + 16 * ct + 4 * g);
                acc = mm4(ld4(st.A1 + (16 * ct + m) * kCH + 4 * g), o, acc);
                S[ct] = mm4(ld4(st.A2 + (16 * ct + m) * kCH + 4 * g), X, acc);
            }
        }
        if (more)
            stage_store(role, rg, s_st[(it + 1) & 1], tid);
        __syncthreads();
    }
    if (role == 1 && a.dh0) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
            st4(a.dh0 + srow + 16 * ct, S[ct]);
    }
}

// ---- gradients of one chunk-head's tokens ----
struct GradLds {
    PrepLds p;
    float Xf[kCH][kP], Xb[kCH][kP], dKD[kCH][kP], G1[kCH][kP], G2[kCH][kP];
    float dA[kCH][kQ], dAqk[kCH][kQ];
    float dgam[kD];
};

__global__ __launch_bounds__(kGradThreads) void bwd_grad_kernel(BwdArgs a)
{
    __shared__ __attribute__((aligned(16))) GradLds L;
    PrepLds &p = L.p;
    const int64_t x = blockIdx.x / a.H;
    const int h = (int)(blockIdx.x % a.H);
    ChunkLoc c;
    if (!locate_chunk(a, x, c))
        return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, m = lane & 15;
    const size_t sl = (size_t)x * (size_t)a.H + (size_t)h;
    {  // V' and dV' of the chunk
        const int r = tid >> 5, c4 = 4 * (tid & 31);
        st4(&L.Xf[r][c4], ld4(a.xf + sl * (kCH * kD) + r * kD + c4));
        st4(&L.Xb[r][c4], ld4(a.xb + sl * (kCH * kD) + r * kD + c4));
    }
    prep_chunk(a, c, h, p, tid);  // ends with a barrier
    {  // dKD = V' D, G1 = dO S0, G2 = dV' S0, dgamma: wave w takes channels 16 w .. 16 w + 15
        const int c0 = 16 * wave;
        const float *cs = a.cks + sl * kBState + (size_t)(c0 + m) * kD + 4 * g;
        const float *cd = a.ckd + sl * kBState + (size_t)(c0 + m) * kD + 4 * g;
        f32x4 aKD = {0.f, 0.f, 0.f, 0.f}, aG1 = aKD, aG2 = aKD;
        float dgp = 0.f;
#pragma unroll 2
        for (int t = 0; t < kD; t += 16) {
            const f32x4 bs = ld4(cs + t), bd = ld4(cd + t);
            aKD = mm4(ld4(&L.Xf[m][t + 4 * g]), bd, aKD);
            aG1 = mm4(ld4(&p.dO[m][t + 4 * g]), bs, aG1);
            aG2 = mm4(ld4(&L.Xb[m][t + 4 * g]), bs, aG2);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                dgp = fmaf(bs[j], bd[j], dgp);
        }
        dgp += __shfl_xor(dgp, 16);
        dgp += __shfl_xor(dgp, 32);
        if (g == 0)
            L.dgam[c0 + m] = dgp;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            L.dKD[4 * g + i][c0 + m] = aKD[i];
            L.G1[4 * g + i][c0 + m] = aG1[i];
            L.G2[4 * g + i][c0 + m] = aG2[i];
        }
    }
    __syncthreads();
    const int ch = tid & (kD - 1), q4 = 4 * (tid >> 7);
    const size_t tok0 = (size_t)c.t0 * (size_t)a.H + (size_t)h;  // token-head index of row 0
    auto row_at = [&](int r) { return (tok0 + (size_t)r * (size_t)a.H) * kD + (size_t)ch; };
    {
        if (wave == 0) {  // dAqk = lower(dO V'^T)
            const f32x4 acc = mm_rows(&p.dO[0][0], &L.Xf[0][0], kD, f32x4{0.f, 0.f, 0.f, 0.f}, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                L.dAqk[4 * g + i][m] = m <= 4 * g + i ? acc[i] : 0.f;
        }
        // P = T^T dV', Q = T^T dW = -T^T G2 (rows q4 .. q4 + 3, channel / value column ch)
        float P[4] = {0.f, 0.f, 0.f, 0.f}, Q[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kCH; ++s) {
            const float xb = L.Xb[s][ch], g2 = L.G2[s][ch];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                P[i] = fmaf(p.T[s][q4 + i], xb, P[i]);
                Q[i] = fmaf(-p.T[s][q4 + i], g2, Q[i]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = q4 + i;
            L.Xb[r][ch] = P[i];  // P replaces dV'
            L.G2[r][ch] = Q[i];  // Q replaces G2
            if (r < c.len)
                a.dv[row_at(r)] = p.beta[r] * P[i];
        }
    }
    __syncthreads();
    if (wave == 0) {  // dA = -strictly_lower(P U^T + Q W^T)
        f32x4 acc = mm_rows(&L.Xb[0][0], &p.U[0][0], kD, f32x4{0.f, 0.f, 0.f, 0.f}, lane);
        acc = mm_rows(&L.G2[0][0], &p.W[0][0], kD, acc, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            L.dA[4 * g + i][m] = m < 4 * g + i ? -acc[i] : 0.f;
    }
    __syncthreads();
    {  // dbeta_r = P_r . V_r + Q_r . KG_r + dA_r . M_r: 32 lanes per row
        const int r = tid >> 5, part = tid & 31;
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int cc = 4 * part + e;
            s = fmaf(L.Xb[r][cc], p.V[r][cc], s);
            s = fmaf(L.G2[r][cc], p.KG[r][cc], s);
        }
        if (part < kCH)
            s = fmaf(L.dA[r][part], p.M[r][part], s);
#pragma unroll
        for (int o = 16; o > 0; o >>= 1)
            s += __shfl_xor(s, o);
        if (part == 0 && r < c.len)
            a.dbeta[tok0 + (size_t)r * (size_t)a.H] = s;
    }
    {  // dKG, dKI, dQG; dk^, dq^; db into Xf (free now)
        float db[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = q4 + i;
            float sKG = L.G2[r][ch], sQG = L.G1[r][ch], sKI = 0.f;
#pragma unroll
            for (int s = 0; s < kCH; ++s) {
                const float ki = p.KI[s][ch];
                sKG = fmaf(L.dA[r][s], ki, sKG);
                sQG = fmaf(L.dAqk[r][s], ki, sQG);
                sKI = fmaf(L.dA[s][r] * p.beta[s], p.KG[s][ch], sKI);
                sKI = fmaf(L.dAqk[s][r], p.QG[s][ch], sKI);
            }
            const float dKG = p.beta[r] * sKG, dKD = L.dKD[r][ch];
            const float G = p.Gm[r][ch], Gi = p.Gi[r][ch];
            db[i] = dKG * p.KG[r][ch] - sKI * p.KI[r][ch] + sQG * p.QG[r][ch] - dKD * p.KD[r][ch];
            if (r < c.len) {
                a.dk[row_at(r)] = dKG * G + (sKI + dKD * p.gam[ch]) * Gi;
                a.dq[row_at(r)] = a.scale * sQG * G;
            }
        }
        __syncthreads();  // every reader of Xf (dAqk) is long done; the barrier orders the reuse
#pragma unroll
        for (int i = 0; i < 4; ++i)
            L.Xf[q4 + i][ch] = db[i];
    }
    __syncthreads();
    if (tid < kD) {  // the last row takes the decay of the whole chunk; d log-decay by reverse sums
        float e = L.dgam[ch] * p.gam[ch];
#pragma unroll
        for (int r = 0; r < kCH; ++r)
            e = fmaf(L.dKD[r][ch], p.KD[r][ch], e);
        float acc = e;
        for (int r = kCH - 1; r >= 0; --r) {
            acc += L.Xf[r][ch];
            if (r < c.len)
                a.dg[row_at(r)] = acc;
        }
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
    a.chunks = f.bl.chunks;
    unsigned char *ws = f.fwd.ws;
    a.seq_start = reinterpret_cast<const int64_t *>(ws + f.fwd.lay.off_seq_start);
    a.seq_len = reinterpret_cast<const int64_t *>(ws + f.fwd.lay.off_seq_len);
    a.seq_off = reinterpret_cast<const int64_t *>(ws + f.fwd.lay.off_seq_off);
    a.kn = reinterpret_cast<float *>(ws + f.bl.off_kn);
    a.qn = reinterpret_cast<float *>(ws + f.bl.off_qn);
    a.lg = reinterpret_cast<float *>(ws + f.bl.off_lg);
    a.rk = reinterpret_cast<float *>(ws + f.bl.off_rk);
    a.rq = reinterpret_cast<float *>(ws + f.bl.off_rq);
    a.bt = reinterpret_cast<float *>(ws + f.bl.off_bt);
    a.ops = reinterpret_cast<float *>(ws + f.bl.off_ops);
    a.cks = reinterpret_cast<float *>(ws + f.bl.off_cks);
    a.ckd = reinterpret_cast<float *>(ws + f.bl.off_ckd);
    a.xf = reinterpret_cast<float *>(ws + f.bl.off_xf);
    a.xb = reinterpret_cast<float *>(ws + f.bl.off_xb);
    a.hpart = reinterpret_cast<float *>(ws + f.bl.off_hpart);
    const int64_t toks = a.B * a.T * a.H;
    const int64_t units = 2 * a.N * a.H;          // (chain, role)
    const int64_t slots = a.chunks * a.H;         // chunk-heads (a bound)
    auto check = [] { return hipGetLastError(); };
    hipError_t e;
    if (toks > 0) {
        hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((toks + 3) / 4)), dim3(256), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
        hipLaunchKernelGGL(bwd_ops_kernel, dim3((unsigned)slots), dim3(kGradThreads), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
    }
    if (units > 0) {
        // two workgroups (halves) per unit, units in groups of 8 (one per XCD)
        hipLaunchKernelGGL(bwd_chain_kernel, dim3((unsigned)(cdiv(units, 8) * 16)), dim3(kChainThreads), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
    }
    if (toks > 0) {
        hipLaunchKernelGGL(bwd_grad_kernel, dim3((unsigned)slots), dim3(kGradThreads), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
        hipLaunchKernelGGL(bwd_finish_kernel, dim3((unsigned)((toks + 3) / 4)), dim3(256), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
    }
    if (a.flags & kBGateIn) {
        hipLaunchKernelGGL(bwd_head_part_kernel, dim3((unsigned)(a.H * kHeadSlices)), dim3(256), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
        hipLaunchKernelGGL(bwd_head_kernel, dim3((unsigned)a.H), dim3(kD), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace kda
