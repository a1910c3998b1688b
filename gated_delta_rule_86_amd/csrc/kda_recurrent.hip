// kda_recurrent.hip -- token-by-token (recurrent) KDA forward pass for short sequences:
// the decode step (one token per sequence, state in and out) and anything a few tokens
// long.  The mathematics is the delta-rule recurrence the chunked kernels evaluate in
// 16-token chunks (FlashKDA article index, "Delta Attention Algorithm: linear-time
// recurrence"), with the activations of the FlashKDA README "Kernel API" table and the
// FLA-backend flags (gate, q/k l2norm, beta sigmoid in the pass, or pre-activated):
//
//   per token:  S <- S Diag(alpha);  r = v - S k^;  S <- S + beta r k^T;  o = scale S q^
//
// A workgroup of 512 threads runs one (sequence, head) chain at a time.  The 128 x 128 fp32
// state (V-major, S[v][c]) lives in registers: thread t holds row v = t / 4 and 32 of its
// channels (16m + 4(t % 4) + e).  Per token, threads 0..127 prepare the per-channel vectors alpha,
// k^, scale q^ (channel c = thread t) and the scalars beta, k^.q^ into LDS; every thread
// then decays its 32 state entries, forms its quarters of S k^ and S q^ (summed over the
// row's four lanes), and applies the rank-1 write.  Using S_new q^ = S_dec q^ + beta r (k^.q^)
// the state is read once per token.  Everything is fp32; out is rounded to bf16 (nearest
// even) once, the final state likewise when it is bf16.
//
// Memory: the state moves once each way per chain (64 KiB fp32 / 32 KiB bf16), the token
// rows once.  For one token per chain that is 128 KiB of state traffic per head-token, so
// the kernel is HBM-bound; persistent workgroups stage the next chain's state in LDS while
// they compute and store the current one.
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

// Workgroup barrier for LDS hand-offs only: this wave's LDS traffic is complete, global
// memory operations stay in flight (__syncthreads would also wait for them, which would
// expose the next chain's state copy).
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

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
constexpr int kRecGroupsPerCU = 2;             // resident workgroups per CU (registers, LDS)
constexpr int kRecStateLds = kD * kD * 4;      // one fp32 state (a bf16 one uses half)
constexpr int kRecLds = kRecStateLds + 2 * 3 * kD * 4 + 64;

typedef uint32_t ru32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void rlds_void;

// Thread (row, q) holds channels 16m + 4q + e (m < 8, e < 4): S[4m + e].  Its 16-byte pieces
// of a row are then interleaved with the row's other three threads, so the LDS reads of a
// state (row-major, as in memory) touch distinct banks for the four threads of a row.

// Wave w's share (rows 16w .. 16w+15) of chain ch's state, global -> LDS with direct loads:
// 1 KB per instruction, the instruction offset carrying 1 KB steps within a 4 KB window.
__device__ __forceinline__ void dma_state(const RecArgs &a, int64_t ch, unsigned char *lds_state, int w, int lane)
{
    const size_t bytes = a.h0_dtype == 2 ? (size_t)kD * kD * 4 : (size_t)kD * kD * 2;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<unsigned char *>(reinterpret_cast<const unsigned char *>(a.h0) + (size_t)ch * bytes), 0,
        (int)bytes, 0x00020000);
    const int per_wave = (int)(bytes / 8);  // 8 KB (fp32) or 4 KB (bf16)
    for (int win = 0; win < per_wave; win += 4096) {
        const uint32_t vo = (uint32_t)(w * per_wave + win + lane * 16);
        unsigned char *dst = lds_state + w * per_wave + win;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (rlds_void *)dst, 16, vo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (rlds_void *)dst, 16, vo, 0, 1024, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (rlds_void *)dst, 16, vo, 0, 2048, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (rlds_void *)dst, 16, vo, 0, 3072, 0);
    }
}

// This thread's entries of a state staged in LDS (row-major, fp32 or bf16 as in memory).
__device__ __forceinline__ void lds_to_state(int dtype, const unsigned char *lds_state, int row, int q, float *S)
{
    if (dtype == 2) {
        const float *p = reinterpret_cast<const float *>(lds_state) + row * kD + 4 * q;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const rf32x4 x = *reinterpret_cast<const rf32x4 *>(p + 16 * m);
            S[4 * m] = x[0];
            S[4 * m + 1] = x[1];
            S[4 * m + 2] = x[2];
            S[4 * m + 3] = x[3];
        }
    } else {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(lds_state) + row * kD + 4 * q;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const ru32x2 x = *reinterpret_cast<const ru32x2 *>(p + 16 * m);
            S[4 * m] = __uint_as_float(x[0] << 16);
            S[4 * m + 1] = __uint_as_float(x[0] & 0xffff0000u);
            S[4 * m + 2] = __uint_as_float(x[1] << 16);
            S[4 * m + 3] = __uint_as_float(x[1] & 0xffff0000u);
        }
    }
}

__device__ __forceinline__ void store_state(const RecArgs &a, int64_t ch, int row, int q, const float *S)
{
    const size_t base = ((size_t)ch * kD + (size_t)row) * kD + (size_t)(4 * q);
    if (a.ht_dtype == 2) {
        float *p = reinterpret_cast<float *>(a.ht) + base;
#pragma unroll
        for (int m = 0; m < 8; ++m)
            *reinterpret_cast<rf32x4 *>(p + 16 * m) = rf32x4{S[4 * m], S[4 * m + 1], S[4 * m + 2], S[4 * m + 3]};
    } else if (a.ht_dtype == 1) {
        uint16_t *p = reinterpret_cast<uint16_t *>(a.ht) + base;
#pragma unroll
        for (int m = 0; m < 8; ++m)
            *reinterpret_cast<ru32x2 *>(p + 16 * m) =
                ru32x2{(uint32_t)rto_bf16(S[4 * m]) | ((uint32_t)rto_bf16(S[4 * m + 1]) << 16),
                       (uint32_t)rto_bf16(S[4 * m + 2]) | ((uint32_t)rto_bf16(S[4 * m + 3]) << 16)};
    }
}

// Persistent: workgroup b runs the chains b, b + gridDim.x, ....  The next chain's initial
// state is copied global -> LDS with direct loads while the current chain is computed and
// its final state stored, so the state traffic of consecutive chains overlaps.
__global__ __launch_bounds__(kRecThreads) __attribute__((amdgpu_waves_per_eu(4))) void recurrent_kernel(RecArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char rlds[];
    unsigned char *lds_state = rlds;
    // per-token vectors, double-buffered so one barrier per token suffices (the buffer
    // alternates with the workgroup's running token count, across chains too)
    float (*s_alpha)[kD] = reinterpret_cast<float (*)[kD]>(rlds + kRecStateLds);
    float (*s_k)[kD] = reinterpret_cast<float (*)[kD]>(rlds + kRecStateLds + 2 * kD * 4);
    float (*s_q)[kD] = reinterpret_cast<float (*)[kD]>(rlds + kRecStateLds + 4 * kD * 4);
    float *s_red = reinterpret_cast<float *>(rlds + kRecStateLds + 6 * kD * 4);  // [2][2][3]
    float *s_beta = s_red + 12;                                                   // [2]

    const int64_t H = a.H;
    const int64_t chains = a.N * H;
    int64_t ch = blockIdx.x;
    if (ch >= chains)
        return;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int row = tid / kRowThreads;   // value row v
    const int q = tid % kRowThreads;     // channels 16m + 4q + e
    const bool gate_in = (a.flags & kRGateIn) != 0;
    const bool l2_in = (a.flags & kRL2In) != 0;
    const bool sig_in = (a.flags & kRSigIn) != 0;
    const bool has_h0 = a.h0_dtype != 0;
    const float lb = a.lower_bound;
    const size_t rowstride = (size_t)H * kD;  // elements between consecutive tokens of a head
    uint32_t tcount = 0;

    if (has_h0) {
        dma_state(a, ch, lds_state, w, lane);
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    }
    for (;;) {
        float S[kRowCols];
        lds_barrier();  // the staged state is complete (every wave waited for its part)
        if (has_h0) {
            lds_to_state(a.h0_dtype, lds_state, row, q, S);
        } else {
#pragma unroll
            for (int i = 0; i < kRowCols; ++i)
                S[i] = 0.f;
        }
        const int64_t nx = ch + gridDim.x;
        // everything this chain reads first goes out before the next chain's state is
        // requested (memory operations complete in order, so a later wait for any of them
        // would also wait for that copy)
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
        // token inputs, one token ahead (kept as raw bf16 until used, so that no wait for
        // them is placed before their use): v of this thread's row; k, q, g of channel tid; beta
        uint16_t vv_n = 0, kc_n = 0, qc_n = 0, gc_n = 0, b_n = 0;
        auto load_token = [&](int64_t t) {
            const size_t tok = (size_t)(start + t);
            const size_t base = tok * rowstride + (size_t)h * kD;
            vv_n = a.v[base + row];
            if (tid < kD) {
                kc_n = a.k[base + tid];
                qc_n = a.q[base + tid];
                gc_n = a.g[base + tid];
                b_n = a.beta[tok * (size_t)H + (size_t)h];
            }
        };
        if (len > 0)
            load_token(0);
        if (has_h0 && nx < chains) {
            lds_barrier();  // every thread has read the staged state
            dma_state(a, nx, lds_state, w, lane);
        }
        for (int64_t t = 0; t < len; ++t, ++tcount) {
            const int buf = (int)(tcount & 1);
            const size_t tok = (size_t)(start + t);
            const size_t base = tok * rowstride + (size_t)h * kD;
            const float vv = rbf16(vv_n), kc = rbf16(kc_n), qc = rbf16(qc_n), gc = rbf16(gc_n), braw = rbf16(b_n);
            if (t + 1 < len)
                load_token(t + 1);
            if (tid < kD) {
                float al;
                if (gate_in)
                    al = lb / (1.0f + exp2f(fmaf(gc, m1, d1)));  // lb * sigmoid(e^{A_log}(g + dt))
                else
                    al = fminf(fmaxf(gc, lb), 0.f);
                s_alpha[buf][tid] = __expf(al);
                // norms and k.q over the 128 channels: wave sums, combined below
                const float kk = wave_sum(kc * kc), qq = wave_sum(qc * qc), kq = wave_sum(kc * qc);
                if (lane == 0) {
                    s_red[buf * 6 + (tid >> 6) * 3 + 0] = kk;
                    s_red[buf * 6 + (tid >> 6) * 3 + 1] = qq;
                    s_red[buf * 6 + (tid >> 6) * 3 + 2] = kq;
                }
                s_k[buf][tid] = kc;
                s_q[buf][tid] = qc;
                if (tid == 0)
                    s_beta[buf] = sig_in ? 1.0f / (1.0f + __expf(-braw)) : braw;
            }
            lds_barrier();
            const float kk = s_red[buf * 6 + 0] + s_red[buf * 6 + 3];
            const float qq = s_red[buf * 6 + 1] + s_red[buf * 6 + 4];
            const float kqraw = s_red[buf * 6 + 2] + s_red[buf * 6 + 5];
            const float rk = l2_in ? rsqrtf(kk + 1e-6f) : 1.f;
            const float rq = (l2_in ? rsqrtf(qq + 1e-6f) : 1.f) * a.scale;
            const float beta = s_beta[buf];
            // decay, S k^ and S q^ (this thread's channels)
            float pk = 0.f, pq = 0.f;
#pragma unroll
            for (int m = 0; m < 8; ++m) {
                const rf32x4 al = *reinterpret_cast<const rf32x4 *>(&s_alpha[buf][16 * m + 4 * q]);
                const rf32x4 kc = *reinterpret_cast<const rf32x4 *>(&s_k[buf][16 * m + 4 * q]);
                const rf32x4 qc = *reinterpret_cast<const rf32x4 *>(&s_q[buf][16 * m + 4 * q]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float sv = S[4 * m + e] * al[e];
                    S[4 * m + e] = sv;
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
            for (int m = 0; m < 8; ++m) {
                const rf32x4 kc = *reinterpret_cast<const rf32x4 *>(&s_k[buf][16 * m + 4 * q]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[4 * m + e] = fmaf(br, kc[e], S[4 * m + e]);
            }
            if (q == 0) {
                const float o = rq * (pq + beta * r * (kqraw * rk));
                a.out[base + row] = rto_bf16(o);
            }
        }
        store_state(a, ch, row, q, S);
        if (nx >= chains)
            break;
        ch = nx;
        // the staged next state: every vector-memory operation older than this chain's
        // state stores (8 per thread when a final state is written) is done
        if (has_h0) {
            if (a.ht_dtype != 0)
                __builtin_amdgcn_s_waitcnt(0x0f78);  // vmcnt(8)
            else
                __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
        }
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
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&recurrent_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kRecLds);
    if (e != hipSuccess)
        return e;
    const int64_t grid = chains < kRecGroupsPerCU * kPlanCUs ? chains : kRecGroupsPerCU * kPlanCUs;
    hipLaunchKernelGGL(recurrent_kernel, dim3((unsigned)grid), dim3(kRecThreads), kRecLds, s, a);
    return hipGetLastError();
}

}  // namespace kda
