// kda_recurrent.hip -- token-by-token (recurrent) KDA forward pass for short sequences:
// the decode step (one token per sequence, state in and out) and anything a few tokens
// long.  The mathematics is the delta-rule recurrence the chunked kernels evaluate in
// 16-token chunks (FlashKDA article index, "Delta Attention Algorithm: linear-time
// recurrence"), with the activations of the FlashKDA README "Kernel API" table and the
// FLA-backend flags (gate, q/k l2norm, beta sigmoid in the pass, or pre-activated):
//
//   per token:  S <- S Diag(alpha);  r = v - S k^;  S <- S + beta r k^T;  o = scale S q^
//
// One workgroup of 512 threads per (sequence, head) chain.  The 128 x 128 fp32 state
// (V-major, S[v][c]) lives in registers: thread t holds row v = t / 4, channels
// 32 (t % 4) .. +31.  Per token, threads 0..127 prepare the per-channel vectors alpha,
// k^, scale q^ (channel c = thread t) and the scalars beta, k^.q^ into LDS; every thread
// then decays its 32 state entries, forms its quarters of S k^ and S q^ (summed over the
// row's four lanes), and applies the rank-1 write.  Using S_new q^ = S_dec q^ + beta r (k^.q^)
// the state is read once per token.  Everything is fp32; out is rounded to bf16 (nearest
// even) once, the final state likewise when it is bf16.
//
// Memory: the state moves once each way per chain (64 KiB fp32 / 32 KiB bf16), the token
// rows once.  For one token per chain that is 128 KiB of state traffic per head-token, so
// the kernel is HBM-bound; it keeps many chains in flight (one workgroup per chain).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {
namespace {

typedef float rf32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t ru32x4 __attribute__((ext_vector_type(4)));

constexpr float kRLog2e = 1.4426950408889634f;
constexpr int kRGateIn = 1, kRL2In = 2, kRSigIn = 4;

__device__ __forceinline__ float rbf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t rto_bf16(float f)
{
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)0x7fc0;  // NaN stays NaN
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

struct RecArgs {
    const uint16_t *q, *k, *v, *g, *beta;
    const float *A_log, *dt_bias;
    float scale, lower_bound;
    int flags;
    uint16_t *out;
    const void *h0;
    void *ht;
    int h0_dtype, ht_dtype;
    int64_t H, N;
    const int64_t *seq_start, *seq_len;
};

// Sum over the 64 lanes of a wavefront (every lane gets the total).
__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        x += __shfl_xor(x, o);
    return x;
}

constexpr int kRowThreads = 4;                 // threads per state row
constexpr int kRowCols = kD / kRowThreads;     // channels per thread
constexpr int kRecThreads = kD * kRowThreads;  // 512

// This thread's 32 entries of chain ch's initial state (zeros without one).
__device__ __forceinline__ void load_state(const RecArgs &a, int64_t ch, int row, int c0, float *S)
{
    const size_t sbase = ((size_t)ch * kD + (size_t)row) * kD + (size_t)c0;
    if (a.h0_dtype == 2) {
        const rf32x4 *p = reinterpret_cast<const rf32x4 *>(reinterpret_cast<const float *>(a.h0) + sbase);
#pragma unroll
        for (int i = 0; i < kRowCols / 4; ++i) {
            const rf32x4 x = p[i];
            S[4 * i] = x[0];
            S[4 * i + 1] = x[1];
            S[4 * i + 2] = x[2];
            S[4 * i + 3] = x[3];
        }
    } else if (a.h0_dtype == 1) {
        const ru32x4 *p = reinterpret_cast<const ru32x4 *>(reinterpret_cast<const uint16_t *>(a.h0) + sbase);
#pragma unroll
        for (int i = 0; i < kRowCols / 8; ++i) {
            const ru32x4 x = p[i];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                S[8 * i + 2 * e] = __uint_as_float(x[e] << 16);
                S[8 * i + 2 * e + 1] = __uint_as_float(x[e] & 0xffff0000u);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < kRowCols; ++i)
            S[i] = 0.f;
    }
}

__device__ __forceinline__ void store_state(const RecArgs &a, int64_t ch, int row, int c0, const float *S)
{
    const size_t sbase = ((size_t)ch * kD + (size_t)row) * kD + (size_t)c0;
    if (a.ht_dtype == 2) {
        rf32x4 *p = reinterpret_cast<rf32x4 *>(reinterpret_cast<float *>(a.ht) + sbase);
#pragma unroll
        for (int i = 0; i < kRowCols / 4; ++i)
            p[i] = rf32x4{S[4 * i], S[4 * i + 1], S[4 * i + 2], S[4 * i + 3]};
    } else if (a.ht_dtype == 1) {
        ru32x4 *p = reinterpret_cast<ru32x4 *>(reinterpret_cast<uint16_t *>(a.ht) + sbase);
#pragma unroll
        for (int i = 0; i < kRowCols / 8; ++i) {
            ru32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                x[e] = (uint32_t)rto_bf16(S[8 * i + 2 * e]) | ((uint32_t)rto_bf16(S[8 * i + 2 * e + 1]) << 16);
            p[i] = x;
        }
    }
}

// One workgroup per chain.
__global__ __launch_bounds__(kRecThreads) void recurrent_kernel(RecArgs a)
{
    // per-token vectors, double-buffered so one barrier per token suffices
    __shared__ __attribute__((aligned(16))) float s_alpha[2][kD];
    __shared__ __attribute__((aligned(16))) float s_k[2][kD];
    __shared__ __attribute__((aligned(16))) float s_q[2][kD];
    __shared__ float s_red[2][2][3];  // [buffer][wave 0/1][k.k, q.q, k.q]
    __shared__ float s_beta[2];

    const int64_t H = a.H;
    const int64_t ch = blockIdx.x;
    if (ch >= a.N * H)
        return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int row = tid / kRowThreads;               // value row v
    const int c0 = kRowCols * (tid % kRowThreads);   // first channel of this thread's part
    const bool gate_in = (a.flags & kRGateIn) != 0;
    const bool l2_in = (a.flags & kRL2In) != 0;
    const bool sig_in = (a.flags & kRSigIn) != 0;
    const float lb = a.lower_bound;
    const size_t rowstride = (size_t)H * kD;  // elements between consecutive tokens of a head

    float S[kRowCols];
    load_state(a, ch, row, c0, S);
    {
        const int64_t n = ch / H;
        const int h = (int)(ch % H);
        const int64_t start = a.seq_start[n];
        const int64_t len = a.seq_len[n];
        // gate constants for channel c = tid (threads 0..127): 2^(g m1 + d1) = exp(-e^{A_log}(g + dt))
        float m1 = 0.f, d1 = 0.f;
        if (tid < kD && gate_in) {
            m1 = -kRLog2e * __expf(a.A_log[h]);
            d1 = m1 * a.dt_bias[(size_t)h * kD + tid];
        }
        for (int64_t t = 0; t < len; ++t) {
            const int buf = (int)(t & 1);
            const size_t tok = (size_t)(start + t);
            const size_t base = tok * rowstride + (size_t)h * kD;
            // value of this thread's row (the row's four threads read it)
            const float vv = rbf16(a.v[base + row]);
            if (tid < kD) {
                const float kc = rbf16(a.k[base + tid]);
                const float qc = rbf16(a.q[base + tid]);
                const float gc = rbf16(a.g[base + tid]);
                float al;
                if (gate_in)
                    al = lb / (1.0f + exp2f(fmaf(gc, m1, d1)));  // lb * sigmoid(e^{A_log}(g + dt))
                else
                    al = fminf(fmaxf(gc, lb), 0.f);
                s_alpha[buf][tid] = __expf(al);
                // norms and k.q over the 128 channels: wave sums, combined below
                const float kk = wave_sum(kc * kc), qq = wave_sum(qc * qc), kq = wave_sum(kc * qc);
                if (lane == 0) {
                    s_red[buf][tid >> 6][0] = kk;
                    s_red[buf][tid >> 6][1] = qq;
                    s_red[buf][tid >> 6][2] = kq;
                }
                s_k[buf][tid] = kc;
                s_q[buf][tid] = qc;
                if (tid == 0) {
                    const float b = rbf16(a.beta[tok * (size_t)H + (size_t)h]);
                    s_beta[buf] = sig_in ? 1.0f / (1.0f + __expf(-b)) : b;
                }
            }
            __syncthreads();
            const float kk = s_red[buf][0][0] + s_red[buf][1][0];
            const float qq = s_red[buf][0][1] + s_red[buf][1][1];
            const float kqraw = s_red[buf][0][2] + s_red[buf][1][2];
            const float rk = l2_in ? rsqrtf(kk + 1e-6f) : 1.f;
            const float rq = (l2_in ? rsqrtf(qq + 1e-6f) : 1.f) * a.scale;
            const float beta = s_beta[buf];
            // decay, S k^ and S q^ (this thread's channels)
            float pk = 0.f, pq = 0.f;
#pragma unroll
            for (int i = 0; i < kRowCols / 4; ++i) {
                const rf32x4 al = *reinterpret_cast<const rf32x4 *>(&s_alpha[buf][c0 + 4 * i]);
                const rf32x4 kc = *reinterpret_cast<const rf32x4 *>(&s_k[buf][c0 + 4 * i]);
                const rf32x4 qc = *reinterpret_cast<const rf32x4 *>(&s_q[buf][c0 + 4 * i]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float sv = S[4 * i + e] * al[e];
                    S[4 * i + e] = sv;
                    pk = fmaf(sv, kc[e], pk);
                    pq = fmaf(sv, qc[e], pq);
                }
            }
            pk += __shfl_xor(pk, 1);
            pq += __shfl_xor(pq, 1);
            pk += __shfl_xor(pk, 2);
            pq += __shfl_xor(pq, 2);
            // r = v - S k^;  S += beta r k^T;  o = scale (S_dec q^ + beta r k^.q^)
            const float r = vv - pk * rk;
            const float br = beta * r * rk;  // times the raw k below
#pragma unroll
            for (int i = 0; i < kRowCols / 4; ++i) {
                const rf32x4 kc = *reinterpret_cast<const rf32x4 *>(&s_k[buf][c0 + 4 * i]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[4 * i + e] = fmaf(br, kc[e], S[4 * i + e]);
            }
            if (tid % kRowThreads == 0) {
                const float o = rq * (pq + beta * r * (kqraw * rk));
                a.out[base + row] = rto_bf16(o);
            }
        }
        store_state(a, ch, row, c0, S);
    }
}

}  // namespace

hipError_t launch_recurrent(const FwdArgs &f, hipStream_t s)
{
    const int64_t chains = f.lay.n_seq * f.H;
    if (chains == 0)
        return hipSuccess;
    RecArgs a;
    a.q = f.q;
    a.k = f.k;
    a.v = f.v;
    a.g = f.g;
    a.beta = f.beta;
    a.A_log = f.A_log;
    a.dt_bias = f.dt_bias;
    a.scale = f.scale;
    a.lower_bound = f.lower_bound;
    a.flags = f.flags;
    a.out = f.out;
    a.h0 = f.h0;
    a.ht = f.ht;
    a.h0_dtype = f.h0_dtype;
    a.ht_dtype = f.ht_dtype;
    a.H = f.H;
    a.N = f.lay.n_seq;
    a.seq_start = reinterpret_cast<const int64_t *>(f.ws + f.lay.off_seq_start);
    a.seq_len = reinterpret_cast<const int64_t *>(f.ws + f.lay.off_seq_len);
    hipLaunchKernelGGL(recurrent_kernel, dim3((unsigned)chains), dim3(kRecThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
