// kda_kernels.hip -- gfx950 kernels of the KDA chunked forward pass.
//
// Method: "MoonshotAI/FlashKDA" README, "Kernel API" table (arguments, layouts, K = V = 128)
// and "Using FlashKDA as an FLA backend" (in-kernel gate, l2norm and beta sigmoid, V-major
// state).  FlashKDA article index: 16-token chunks, Neumann-series inverse, base-2
// exponentials, lower_bound as the exponent-range guard.
//
// Two kernels:
//   chunk table  (integer)  sequences -> chunk offsets, validity word
//   forward      one workgroup per (sequence, head): four producer wavefronts prepare
//                chunks (gate, cumulative log-decay, l2norm, sigmoid, A_kk / A_qk on MFMA,
//                Neumann inverse on fp32 MFMA) into LDS; four consumer wavefronts hold the
//                128 x 128 fp32 state in registers and run, per chunk, Z = KG S^T,
//                Y = QG S^T, V' = Tb (V - Z), O = Y + Mq (V - Z), S <- S diag(gamma) + KD^T V'
//                on bf16 MFMA.  The products that feed the carried state (Z, V', the update,
//                and A_kk) use a hi/lo bf16 split (three products, two for the update), the
//                output-only ones (Y, Mq X, A_qk) one.
//
// Chunk algebra (per chunk of l <= 16 tokens, b = inclusive cumsum of the log-decay a):
//   Gamma_r = exp(b_r), gamma = Gamma_{l-1}
//   A_kk[r,s] = beta_r sum_c k^_rc k^_sc exp(b_rc - b_sc)  (s < r)
//   T = (I + A_kk)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8)   (A nilpotent, 16 x 16)
//   Tb = T diag(beta);  V' = Tb (V - (k^*Gamma) S^T)
//   A_qk[r,s] = scale sum_c q^_rc k^_sc exp(b_rc - b_sc)   (s <= r)
//   O = scale (q^*Gamma) S^T + A_qk V' = Y + (A_qk Tb)(V - Z)
//   S <- S diag(gamma) + V'^T (k^ * gamma / Gamma)
// lower_bound >= -5 keeps 16 * |a| <= 80 < 126 ln 2, so every factor exp(+-b) stays a
// normal fp32/bf16 number (the article index's "lower_bound ... bf16 limits").

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kda_internal.h"

namespace kda {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to bf16, nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t p;
    p[0] = (__bf16)a;
    p[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint16_t to_bf16(float a) { return __builtin_bit_cast(uint16_t, (__bf16)a); }
// hi = bf16(x), lo = bf16(x - hi) for two values: x ~ hi + lo to about 16 significant bits.
// Returns {hi, lo}, each two packed bf16.
__device__ __forceinline__ u32x2_t split_bf16x2(float a, float b)
{
    const uint32_t hi = pack_bf16x2(a, b);
    const uint32_t lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
    return u32x2_t{hi, lo};
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
// c + a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs, fp32 accumulation
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoidf_fast(float x) { return frcp(1.0f + fexp2(-x * kLog2e)); }

// v_mfma_f32_16x16x32_bf16: A[m][k] in lane m + 16*(k/8), element k%8; B[k][n] in lane
// n + 16*(k/8), element k%8; D[m][n] in lane n + 16*(m/4), element m%4.
__device__ __forceinline__ f32x4_t mfma32(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// A operands that subtract B from C lane by lane: mfma32(negI0, b, c) = c - b[0..3] and
// mfma32(negI1, b, c) = c - b[4..7], element by element in every lane (b's bf16 values
// widened exactly).  negI0 holds -1 at A[m][8(m/4) + m%4], negI1 at A[m][8(m/4) + 4 + m%4]:
// lane m + 16(m/4), element m%4 (resp. 4 + m%4).  With b = bf16(c) the result is the exact
// rounding residue c - bf16(c).
__device__ __forceinline__ void make_neg_identity(int lane, u32x4_t &negI0, u32x4_t &negI1)
{
    negI0 = u32x4_t{0u, 0u, 0u, 0u};
    negI1 = negI0;
    const int m = lane & 15;
    if ((lane >> 4) == (m >> 2)) {
        const int e = m & 3;
        const uint32_t v = (e & 1) ? 0xbf800000u : 0x0000bf80u;
        negI0[e >> 1] = v;
        negI1[2 + (e >> 1)] = v;
    }
}

__device__ __forceinline__ void lds_sync_wave()
{
    // LDS traffic of one wavefront is in order; wait for it and keep the compiler from
    // moving LDS accesses across this point.
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------------------
// Stage 1: chunk table.  One workgroup of 256 threads.
// ---------------------------------------------------------------------------------------
struct TableArgs {
    const int64_t *cu;
    int64_t B, T, N;
    int64_t P;  // whole-chain workgroups per head
    int32_t *status;
    int64_t *n_total;
    int64_t *seq_start, *seq_len, *seq_off;
    int64_t *wg_first;  // [P + 1]: first unit of each whole-chain workgroup of a head
    int32_t *units;     // [2 N]: (sequence << 2) | (0 whole, 1 + column half)
    int whole;          // the forward pass runs whole chains (no cut plan)
    int split;          // whole-chain pass that may split sequences into column halves
    int64_t Pc;         // workgroups per head of the cut plan (0: none)
    int32_t *cut_seq, *cut_off, *cut_first;  // [Pc + 1]: the cut plan's cuts
};

__device__ void chunk_table_body(const TableArgs &a, int tid);

// Whole-chain workgroup split: the P workgroups of a head take contiguous runs of
// sequences with about equal chunk counts.  Sequence i goes to workgroup
// floor(P * mid_i / total) (at most P - 1), mid_i = (seq_off[i] + seq_off[i+1]) / 2 its
// chunk midpoint; wg_first[s] is the first sequence of workgroup s, wg_first[P] = N.
// With no chunks at all every sequence goes to the last workgroup.
__device__ void partition_sequences(const TableArgs &a, int tid)
{
    // seq_off was written by this workgroup: make it visible to every thread's loads
    __threadfence();
    __syncthreads();
    const int64_t tot = a.seq_off[a.N];
    auto group_of = [&](int64_t i) -> int64_t {
        if (tot <= 0)
            return a.P - 1;
        const int64_t g = (a.seq_off[i] + a.seq_off[i + 1]) * a.P / (2 * tot);
        return g < a.P - 1 ? g : a.P - 1;
    };
    for (int64_t i = tid; i < a.N; i += 256) {
        a.units[i] = (int32_t)(i << 2);
        const int64_t lo = i == 0 ? 0 : group_of(i - 1) + 1;
        const int64_t hi = group_of(i);
        for (int64_t g = lo; g <= hi; ++g)
            a.wg_first[g] = i;
    }
    if (tid == 0) {
        const int64_t lo = a.N == 0 ? 0 : group_of(a.N - 1) + 1;
        for (int64_t g = lo; g <= a.P; ++g)
            a.wg_first[g] = a.N;
    }
}

// Whole-chain plan with column halves (varlen launches that split_plan admits): N <=
// kSplitMaxSeq sequences, P <= kSplitMaxP workgroups per head.  Thread k (k = 0 .. min(N, kSplitMaxK)) packs the
// head's units when the k longest sequences run as two column halves each: units are taken
// by weight, heaviest first (whole 100 n, half 82 n for n chunks; a tie takes the half
// first, sequences of equal length go by index), each to the least loaded workgroup (the
// lowest index among equals).  The k with the smallest largest load wins (the smallest k
// among equals); its units replace the contiguous runs, workgroup s taking units
// wg_first[s] .. wg_first[s+1]-1 in packing order.
__device__ void plan_halves(const TableArgs &a, int tid)
{
    constexpr int kU = 2 * (int)kSplitMaxSeq;
    __shared__ int64_t s_w[kSplitMaxSeq];  // chunk count of the sequence of rank r (longest first)
    __shared__ int s_ord[kSplitMaxSeq];    // sequence of rank r
    __shared__ int64_t s_mk[kSplitMaxK + 1];
    __shared__ int s_code[kSplitMaxK + 1][kU];           // unit u of plan k: (seq << 2) | code
    __shared__ unsigned char s_bin[kSplitMaxK + 1][kU];  // its workgroup
    __shared__ int64_t s_n[kSplitMaxSeq];  // chunk count of sequence i
    __shared__ int s_best;
    const int N = (int)a.N, P = (int)a.P;
    __syncthreads();
    if (tid < N)
        s_n[tid] = a.seq_off[tid + 1] - a.seq_off[tid];
    __syncthreads();
    if (tid < N) {
        const int64_t n = s_n[tid];
        int rank = 0;
        for (int j = 0; j < N; ++j)
            rank += s_n[j] > n || (s_n[j] == n && j < tid);
        s_ord[rank] = tid;
        s_w[rank] = n;
    }
    __syncthreads();
    const int K = N < kSplitMaxK ? N : kSplitMaxK;
    if (tid <= K) {
        const int k = tid;
        int64_t load[kSplitMaxP];  // constant indices only: stays in registers
#pragma unroll
        for (int b = 0; b < kSplitMaxP; ++b)
            load[b] = 0;
        int hi = 0, wi = k, u = 0;  // next half (0 .. 2k-1), next whole rank (k .. N-1)
        while (hi < 2 * k || wi < N) {
            const int64_t wh = hi < 2 * k ? kHalfW * s_w[hi >> 1] : -1;
            const int64_t ww = wi < N ? kWholeW * s_w[wi] : -1;
            int code;
            int64_t w;
            if (wh >= ww) {
                code = (s_ord[hi >> 1] << 2) | (1 + (hi & 1));
                w = wh;
                ++hi;
            } else {
                code = s_ord[wi] << 2;
                w = ww;
                ++wi;
            }
            int best = 0;
            int64_t lmin = load[0];
#pragma unroll
            for (int b = 1; b < kSplitMaxP; ++b)
                if (b < P && load[b] < lmin) {
                    lmin = load[b];
                    best = b;
                }
#pragma unroll
            for (int b = 0; b < kSplitMaxP; ++b)
                if (b == best)
                    load[b] += w;
            s_code[k][u] = code;
            s_bin[k][u] = (unsigned char)best;
            ++u;
        }
        int64_t mk = 0;
#pragma unroll
        for (int b = 0; b < kSplitMaxP; ++b)
            mk = b < P && load[b] > mk ? load[b] : mk;
        s_mk[k] = mk;
    }
    __syncthreads();
    if (tid == 0) {
        int best = 0;
        for (int k = 1; k <= K; ++k)
            if (s_mk[k] < s_mk[best])
                best = k;
        s_best = best;
    }
    __syncthreads();
    const int best = s_best, U = N + best;
    if (tid < U) {
        // position: units of lower workgroups, then earlier units of this one
        const int b = s_bin[best][tid];
        int pos = 0;
        for (int v = 0; v < U; ++v)
            pos += s_bin[best][v] < b || (s_bin[best][v] == b && v < tid);
        a.units[pos] = s_code[best][tid];
    }
    if (tid <= P) {
        int first = 0;
        for (int v = 0; v < U; ++v)
            first += s_bin[best][v] < tid;
        a.wg_first[tid] = first;
    }
}

// Snake order for up to kSnakeMaxSeq sequences per head: sequence i of rank r by chunk
// count (longest first, ties by index) goes to workgroup r % P in even rounds r / P and
// to P - 1 - r % P in odd ones, as unit r / P of that workgroup.  Every workgroup then
// holds the same number of sequences (one more for some, in the last round) and about the
// same number of chunks, each sequence's place following from its rank alone.
constexpr int64_t kSnakeMaxSeq = 512;

__device__ void plan_snake(const TableArgs &a, int tid)
{
    // Key of sequence i: its chunk count above, kSnakeMaxSeq - 1 - i below, so that one
    // comparison orders by count and breaks ties by index (N <= 512; a count is held to
    // 2^31 - 1, which no sequence that fits in memory comes near).
    __shared__ int64_t s_key[kSnakeMaxSeq];
    const int N = (int)a.N, P = (int)a.P;
    __syncthreads();
    for (int i = tid; i < N; i += 256) {
        const int64_t c = a.seq_off[i + 1] - a.seq_off[i];
        s_key[i] = ((c < 0x7fffffff ? c : 0x7fffffff) << 10) | (int64_t)(kSnakeMaxSeq - 1 - i);
    }
    __syncthreads();
    const int R = N / P, rem = N % P;  // full rounds; units of the last, partial round
    // first unit of workgroup b: R per lower workgroup, plus the lower workgroups that take
    // a unit in the last round (the first rem in its direction)
    auto first = [&](int b) {
        const int extra = (R & 1) == 0 ? (b < rem ? b : rem) : (b > P - rem ? b - (P - rem) : 0);
        return b * R + extra;
    };
    for (int i = tid; i < N; i += 256) {
        const int64_t key = s_key[i];
        int r = 0;
#pragma unroll 8
        for (int j = 0; j < N; ++j)
            r += s_key[j] > key;
        const int rnd = r / P, pos = r - rnd * P;
        const int b = (rnd & 1) ? P - 1 - pos : pos;
        a.units[first(b) + rnd] = i << 2;
    }
    for (int b = tid; b <= P; b += 256)
        a.wg_first[b] = first(b);
}

// Cut plan (see kda_internal.h): cut j = (sequence cut_seq[j], chunk cut_off[j] of it) at
// chunk x_j = floor(j C / Pc) of the head's chunk list, moved to the nearest sequence
// boundary within min(kSnapChunks, C / (4 Pc)) chunks.  The sequence of chunk x is the first
// one ending after x (empty sequences before it stay with the run before); cut 0 = (0, 0)
// takes leading empty sequences, cut Pc = (N, 0).  cut_first[j]: the first of the cuts
// inside cut j's sequence (j itself for a cut at a sequence boundary).
__device__ void plan_cut_table(const TableArgs &a, int tid)
{
    __shared__ int32_t s_seq[kPlanCUs + 1], s_off[kPlanCUs + 1];
    __threadfence();
    __syncthreads();
    const int64_t C = a.seq_off[a.N], P = a.Pc;
    int64_t snap = C / (4 * P);
    if (snap > kSnapChunks)
        snap = kSnapChunks;
    auto holder = [&](int64_t x) {  // smallest i with seq_off[i + 1] > x, N if none
        int64_t lo = 0, hi = a.N;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (a.seq_off[mid + 1] > x)
                hi = mid;
            else
                lo = mid + 1;
        }
        return lo;
    };
    for (int64_t j = tid; j <= P; j += 256) {
        int64_t x = j * C / P, i;
        if (j == 0) {
            i = 0;
            x = 0;
        } else if (j == P) {
            i = a.N;
            x = C;
        } else {
            i = holder(x);
            if (i < a.N) {
                const int64_t dlo = x - a.seq_off[i], dhi = a.seq_off[i + 1] - x;
                if (dlo > 0 && dlo <= snap)
                    x -= dlo;
                else if (dlo > 0 && dhi <= snap)
                    x += dhi;
                i = holder(x);
            }
        }
        a.cut_seq[j] = s_seq[j] = (int32_t)i;
        a.cut_off[j] = s_off[j] = i < a.N ? (int32_t)(x - a.seq_off[i]) : 0;
    }
    __syncthreads();
    for (int64_t j = tid; j <= P; j += 256) {
        int64_t j0 = j;
        if (s_off[j] > 0)
            while (j0 > 1 && s_seq[j0 - 1] == s_seq[j] && s_off[j0 - 1] > 0)
                --j0;
        a.cut_first[j] = (int32_t)j0;
    }
}

__global__ __launch_bounds__(256) void chunk_table_kernel(TableArgs a)
{
    chunk_table_body(a, threadIdx.x);
    if (a.Pc > 1) {
        plan_cut_table(a, threadIdx.x);
        return;
    }
    partition_sequences(a, threadIdx.x);
    if (a.split && a.N <= kSplitMaxSeq && a.P <= kSplitMaxP)
        plan_halves(a, threadIdx.x);
    else if (a.whole && a.N <= kSnakeMaxSeq && a.P > 1)
        plan_snake(a, threadIdx.x);
}

__device__ void chunk_table_body(const TableArgs &a, int tid)
{
    __shared__ int s_bad;
    __shared__ int64_t s_scan[256];
    __shared__ int64_t s_carry;
    if (a.cu == nullptr) {
        const int64_t per = cdiv(a.T, kCH);
        for (int64_t b = tid; b < a.N; b += 256) {
            a.seq_start[b] = b * a.T;
            a.seq_len[b] = a.T;
            a.seq_off[b] = b * per;
        }
        if (tid == 0) {
            a.seq_off[a.N] = a.N * per;
            *a.n_total = a.N * per;
            *a.status = 0;
        }
        return;
    }
    if (tid == 0) {
        int bad = 0;
        if (a.cu[0] != 0)
            bad |= 1;
        if (a.cu[a.N] != a.T)
            bad |= 4;
        s_bad = bad;
        s_carry = 0;
    }
    __syncthreads();
    int mybad = 0;
    for (int64_t i = tid; i < a.N; i += 256)
        if (a.cu[i + 1] < a.cu[i])
            mybad |= 2;
    if (mybad)
        atomicOr(&s_bad, mybad);
    __syncthreads();
    const int bad = s_bad;
    if (bad) {
        // Invalid content: every sequence becomes empty, nothing downstream reads tokens.
        for (int64_t i = tid; i < a.N; i += 256) {
            a.seq_start[i] = 0;
            a.seq_len[i] = 0;
            a.seq_off[i] = 0;
        }
        if (tid == 0) {
            a.seq_off[a.N] = 0;
            *a.n_total = 0;
            *a.status = bad;
        }
        return;
    }
    for (int64_t base = 0; base < a.N; base += 256) {
        const int64_t i = base + tid;
        int64_t len = 0;
        if (i < a.N) {
            len = a.cu[i + 1] - a.cu[i];
            a.seq_start[i] = a.cu[i];
            a.seq_len[i] = len;
        }
        const int64_t cnt = (len + kCH - 1) / kCH;
        s_scan[tid] = cnt;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            int64_t x = tid >= d ? s_scan[tid - d] : 0;
            __syncthreads();
            s_scan[tid] += x;
            __syncthreads();
        }
        const int64_t incl = s_scan[tid];
        const int64_t carry = s_carry;
        if (i < a.N)
            a.seq_off[i] = carry + incl - cnt;
        __syncthreads();
        if (tid == 255)
            s_carry = carry + incl;
        __syncthreads();
    }
    if (tid == 0) {
        a.seq_off[a.N] = s_carry;
        *a.n_total = s_carry;
        *a.status = 0;
    }
}

// ---------------------------------------------------------------------------------------
// Helpers of the forward kernel: 16x16 fp32 products, DPP scans, direct-to-LDS loads
// ---------------------------------------------------------------------------------------
// 16x16 fp32 product on v_mfma_f32_16x16x4_f32 with both factors held in the D layout
// (lane n + 16*(m/4), element m%4 holds X[m][n]).  xt is X^T in that layout, y is Y.
// Step j contracts over k = 4*(L/16) + j, which is element j of both operands.
__device__ __forceinline__ f32x4_t mm16(f32x4_t xt, f32x4_t y)
{
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[0], y[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[1], y[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[2], y[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xt[3], y[3], acc, 0, 0, 0);
    return acc;
}

// Transpose of a 16x16 matrix held in the D layout, through this wavefront's LDS tile.
__device__ __forceinline__ f32x4_t transpose16(f32x4_t x, float *tile, int lane)
{
    const int g = lane >> 4, c = lane & 15;
    lds_sync_wave();
#pragma unroll
    for (int i = 0; i < 4; ++i)
        tile[(4 * g + i) * 16 + c] = x[i];
    lds_sync_wave();
    f32x4_t y = *reinterpret_cast<const f32x4_t *>(tile + c * 16 + 4 * g);
    return y;
}

__device__ __forceinline__ float dpp_row_shr(float x, int n)
{
    int v = __builtin_bit_cast(int, x);
    int r;
    switch (n) {
    case 1: r = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false); break;
    case 2: r = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false); break;
    case 4: r = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false); break;
    }
    return __builtin_bit_cast(float, r);
}
// Value of lane 15 of this lane's row of 16 (DPP row_newbcast:15).
// Inclusive prefix sum over the 16 lanes of each row.  x is pinned to a register first
// (an empty asm the compiler cannot see through), so the first add is not contracted with
// the multiply that produced x and every step is one v_add_f32 with a DPP source operand.
__device__ __forceinline__ float row_scan16(float x)
{
    __asm__("" : "+v"(x));
    x = __fadd_rn(x, dpp_row_shr(x, 1));
    x = __fadd_rn(x, dpp_row_shr(x, 2));
    x = __fadd_rn(x, dpp_row_shr(x, 4));
    return __fadd_rn(x, dpp_row_shr(x, 8));
}

// Value of lane I of this lane's quad (DPP quad_perm [I, I, I, I]).  With a single use
// the move folds into that instruction's DPP source operand.
template <int I>
__device__ __forceinline__ float quad_bcast(float x)
{
    const int v = __builtin_bit_cast(int, x);
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, I * 0x55, 0xf, 0xf, true));
}

__device__ __forceinline__ float dpp_row_last(float x)
{
    int v = __builtin_bit_cast(int, x);
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0x15f, 0xf, 0xf, false));
}

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(n), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0), other counters untouched
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Buffer descriptor over [base, base + bytes): loads past the end return zeros without
// touching memory.  Word 3 = raw (untyped) buffer access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}


// ---------------------------------------------------------------------------------------
// Fused forward pass: one workgroup of 8 wavefronts per chain (sequence, head).
//
//   waves 0-3  producers.  Producer p prepares chunks p, p+4, p+8, ...: it streams the
//              chunk's q, k, g, beta into LDS with direct global->LDS loads (one chunk
//              ahead), then computes gate, cumulative log-decay, l2norm, sigmoid(beta),
//              A_kk / A_qk, the Neumann inverse, Tb and Mq exactly as the chunk algebra at
//              the top of this file, and writes the chunk's operand block (same layout as
//              kBlk*) into one of kNS LDS slots.
//   waves 4-7  consumers.  Consumer c owns value columns 32c .. 32c+31 of the state, all
//              128 channels, in registers (two 16-column blocks, 8 channel tiles each),
//              runs the chunk recurrence on bf16 MFMA and writes the output.
//
// Slot hand-off through LDS words: ready[s] = index of the chunk that slot s holds;
// taken[s][c] = number of chunks consumer c has read out of slot s.  Each word has a
// single writer (plain LDS stores).  Every wait is a bounded spin: on time-out the wave
// records kStatusSpin in the status word and goes on, so no input can hang the kernel.
// ---------------------------------------------------------------------------------------
// Operand block of one chunk (what a producer hands to the consumers), in the exact
// register layout of the consumers' MFMA operands, so that each lane fetches an operand
// with one 16-byte LDS read.
constexpr int kBlkKG = 0;       // K^*Gamma (hi), bf16, [4 channel pairs][64 lanes][8]
constexpr int kBlkKGL = 4096;   // K^*Gamma (lo), same layout
constexpr int kBlkQG = 8192;    // scale*q^*Gamma, bf16, same layout
constexpr int kBlkKD = 12288;   // K^*gamma/Gamma (hi, lo bf16), [8 channel tiles][4 token groups][16 slots, swizzled][4+4]
constexpr int kBlkGAM = 20480;  // gamma = Gamma at the chunk's last token, fp32 [16][8]: channel 16t + j at 8j + t
constexpr int kBlkTB = 20992;   // T*diag(beta) (hi, lo bf16), [64 lanes][4+4]
constexpr int kBlkMQ = 22016;   // A_qk*T*diag(beta) (hi, lo bf16), [64 lanes][4+4]
constexpr int kBlkBytes = 23040;

constexpr int kNS = 4;                           // operand slots
constexpr int kStageBytes = 3 * 4096 + 256;      // q, k, g tiles (swizzled rows) + beta
constexpr int kNV = 3;                           // value-tile ring depth per consumer
constexpr int kOffStage = kNS * kBlkBytes;
constexpr int kOffVring = kOffStage + 4 * kStageBytes;
constexpr int kOffTile = kOffVring + 4 * kNV * 1024;
constexpr int kOffDt = kOffTile + 4 * 1024;
constexpr int kOffOut = kOffDt + 512;               // per consumer: one output tile (1 KB)
constexpr int kOffFlags = kOffOut + 4 * 1024;   // int words: ready [kNS], taken [kNS][4],
constexpr int kFlagStop = 5 * kNS;               // stop item of a transition run,
constexpr int kFlagVote = kFlagStop + 1;         // consumer votes [2][4]
constexpr int kFusedLds = kOffFlags + 128;
static_assert(4 * (kFlagVote + 8) <= 128, "flag words");
static_assert(kFusedLds <= 160 * 1024, "LDS budget");
static_assert(kBlkBytes % 256 == 0 && kBlkKD % 256 == 0, "slot alignment (the KD swizzle XORs address bits 4-7)");
constexpr int32_t kStatusSpin = 0x100;
constexpr int kGateIn = 1, kL2In = 2, kSigIn = 4;
constexpr int kSpinMax = 1 << 22;

struct FusedArgs {
    const uint16_t *q, *k, *v, *g, *beta;
    const float *A_log, *dt_bias;
    float scale, lower_bound;
    int flags;  // activation switches: kGateIn | kL2In | kSigIn (others: input already activated)
    uint16_t *out;
    const void *h0;
    void *ht;
    int h0_dtype, ht_dtype;
    int64_t H, N;
    const int64_t *seq_start, *seq_len;
    const int64_t *wg_first;  // whole-chain pass: first unit of each workgroup of a head
    const int32_t *units;     // whole-chain units: (sequence << 2) | (0 whole, 1 + column half)
    int32_t *status;
    // pass 0 = whole chains; cut plan (kda_internal.h): 1 = pass A, 2 = pass B,
    // 3 = transition runs
    int pass, Pc;    // Pc: workgroups per head of the cut plan
    const int32_t *cut_seq, *cut_off, *cut_first;  // [Pc + 1]
    float *segS, *segF, *segP;  // [H][Pc][128][128] fp32, V-major, slot (h, cut j)
    int32_t *segZ;   // [H][Pc]: chunks a transition run took before stopping, -1 = all
    int32_t *segD;   // [H][Pc]: 1 where the scan dropped S_j's share of S_{j+1}
    float *segNS, *segNF;  // [H][Pc][4]: squared norms of S_j and F_j, per consumer
    int trunc;       // transition runs may stop early (in-kernel l2norm and beta sigmoid)
};

// One work unit: a chunk range of one chain, where its state comes from and goes to.
enum { kInitZero = 0, kInitBf16 = 1, kInitFp32 = 2, kInitIdentity = 3 };
struct Unit {
    int64_t n;
    int h;
    int64_t start, len;   // the sequence's first token and length
    int64_t c0, c1;       // chunk range [c0, c1) of the sequence
    int init_kind;        // kInit*
    const void *init;     // 128 x 128 block (V-major) for kInitBf16 / kInitFp32
    int fin_kind;         // 0 none, 1 bf16, 2 fp32
    void *fin;            // 128 x 128 block
    bool v_on;            // false: v taken as zero (the P run of a segment)
    bool out_on;          // write out rows of this range
    int half;             // -1: all 128 value columns; 0 / 1: columns 64*half .. 64*half+63
    float *nrm;           // pass A: squared norm of the end state, one float per consumer
    const float *fin_src; // fp32 state written as the final state instead of the run's own
    int32_t *zout;        // transition runs: where the chunk count before the stop goes
    float thr;            // transition runs: stop once every state entry is below this
};

// A workgroup's work: one unit (segment passes), or -- whole-chain pass -- the units
// sub, sub + 1, ... < n_end of the unit list (chains (n, h) of one head h, whole or one
// column half), one after another.  The producers then run ahead into the next unit
// while the consumers finish the current one.
struct WgPlan {
    int pass;
    int h;
    int64_t sub, n_end;   // whole-chain pass: units sub, sub + 1, ... < n_end
    int64_t n;            // (unused by the cut plan)
    int seg;              // cut plan: the run (pass A) or the cut (passes B, 3)
};

// Launch kinds of the fused kernel: whole chains (pass 0), whole chains that may hold column
// halves (pass 0), the cut plan's pass A (1), pass B (2) and transition runs (3).  The unit
// lookups below are instantiated per kind, so each kernel carries only its own pass.
constexpr int kModeWhole = 0, kModeHalves = 1, kModeA = 2, kModeTrans = 3, kModeB = 4;

__device__ __forceinline__ int64_t seq_chunks(const FusedArgs &a, int64_t i) { return (a.seq_len[i] + kCH - 1) / kCH; }

// A piece of the cut plan: chunks [c0, c1) of sequence seq.
struct Piece {
    int64_t seq;
    int c0, c1;
};
// Piece k of run w (pass A); false past the run's end.
__device__ bool run_piece(const FusedArgs &a, int w, int64_t k, Piece &p)
{
    const int64_t i0 = a.cut_seq[w], i1 = a.cut_seq[w + 1], i = i0 + k;
    const int o1 = a.cut_off[w + 1];
    if (i > i1 || (i == i1 && o1 == 0))
        return false;
    const int64_t n = seq_chunks(a, i);
    p.seq = i;
    p.c0 = k == 0 ? a.cut_off[w] : 0;
    p.c1 = i == i1 ? o1 : (int)n;
    return !(p.c0 == p.c1 && n > 0);  // (a run with no chunks)
}
// The piece that starts at cut j (passes B and 3); false for a cut at a sequence boundary.
__device__ bool cut_piece(const FusedArgs &a, int j, Piece &p)
{
    const int o = a.cut_off[j];
    if (o == 0)
        return false;
    const int64_t i = a.cut_seq[j];
    p.seq = i;
    p.c0 = o;
    p.c1 = a.cut_seq[j + 1] == i ? a.cut_off[j + 1] : (int)seq_chunks(a, i);
    return true;
}
// First of the cuts inside the sequence that holds cut j (a cut inside it): j0 <= j.
__device__ __forceinline__ int first_cut(const FusedArgs &a, int j) { return a.cut_first[j]; }

template <int kMode>
__device__ bool unit_at(const FusedArgs &a, const WgPlan &w, int64_t k, Unit &u)
{
    constexpr bool kWholeMode = kMode == kModeWhole || kMode == kModeHalves;
    constexpr int64_t kBlock = (int64_t)kD * kD;
    const size_t elt = a.h0_dtype == 1 ? 2 : 4, elt_t = a.ht_dtype == 1 ? 2 : 4;
    u.half = -1;
    u.h = w.h;
    u.v_on = true;
    u.out_on = true;
    u.nrm = nullptr;
    u.fin_src = nullptr;
    u.zout = nullptr;
    u.thr = 0.f;
    auto states = [&](int64_t n, const void *&h0c, void *&htc) {
        const int64_t chain = n * a.H + w.h;
        h0c = a.h0 ? reinterpret_cast<const unsigned char *>(a.h0) + (size_t)chain * kBlock * elt : nullptr;
        htc = a.ht ? reinterpret_cast<unsigned char *>(a.ht) + (size_t)chain * kBlock * elt_t : nullptr;
    };
    const void *h0c;
    void *htc;
    if constexpr (kWholeMode) {
        if (w.sub + k >= w.n_end)
            return false;
        const int32_t code = a.units[w.sub + k];
        u.n = code >> 2;
        u.half = (code & 3) - 1;
        u.len = a.seq_len[u.n];
        u.start = a.seq_start[u.n];
        states(u.n, h0c, htc);
        u.c0 = 0;
        u.c1 = (u.len + kCH - 1) / kCH;
        u.init_kind = a.h0_dtype;  // 0 none -> zeros, 1 bf16, 2 fp32
        u.init = h0c;
        u.fin_kind = a.ht_dtype;
        u.fin = htc;
        return true;
    }
    Piece p;
    constexpr bool passA = kMode == kModeA;
    if (passA ? !run_piece(a, w.seg, k, p) : (k > 0 || !cut_piece(a, w.seg, p)))
        return false;
    u.n = p.seq;
    u.len = a.seq_len[u.n];
    u.start = a.seq_start[u.n];
    states(u.n, h0c, htc);
    u.c0 = p.c0;
    u.c1 = p.c1;
    const int64_t nch = (u.len + kCH - 1) / kCH;
    const size_t hs = (size_t)w.h * (size_t)a.Pc;  // slot of cut 0 of this head
    auto slot = [&](float *base, int j) { return base + (hs + (size_t)j) * kBlock; };
    if constexpr (passA) {
        // pass A: run w; a piece that starts at cut w runs from zero (F_w), one that starts
        // its sequence from the initial state, ending at cut w + 1 (S_{w+1}) or at the end
        const int wr = w.seg;
        if (p.c0 > 0) {
            u.init_kind = kInitZero;
            u.init = nullptr;
            u.fin_kind = 2;
            u.fin = slot(a.segF, wr);
            u.nrm = a.segNF + 4 * (hs + wr);
        } else {
            u.init_kind = a.h0_dtype;
            u.init = h0c;
            if (p.c1 < nch) {
                u.fin_kind = 2;
                u.fin = slot(a.segS, wr + 1);
                u.nrm = a.segNS + 4 * (hs + wr + 1);
            } else {
                u.fin_kind = a.ht_dtype;
                u.fin = htc;
            }
        }
    } else if constexpr (kMode == kModeTrans) {
        // transition run of the piece at cut j: from I, v = 0, no out; stop bound from the
        // norms of pass A (kda_internal.h)
        const int j = w.seg, j0 = first_cut(a, j);
        u.init_kind = kInitIdentity;
        u.init = nullptr;
        u.v_on = false;
        u.out_on = false;
        u.fin_kind = 2;
        u.fin = slot(a.segP, j);
        u.zout = a.segZ + hs + j;
        if (a.trunc) {
            // |F_j0|_F + ... + |F_{j-1}|_F over the lanes (one cut each), then |S_j0|_F
            auto fro = [&](const float *nr) { return sqrtf(nr[0] + nr[1] + nr[2] + nr[3]); };
            const int lane = (int)(threadIdx.x & 63);
            float part = 0.f;
            for (int base = j0; base < j; base += 64)
                if (base + lane < j)
                    part += fro(a.segNF + 4 * (hs + base + lane));
#pragma unroll
            for (int o = 32; o > 0; o >>= 1)
                part += __shfl_xor(part, o);
            const float bound = fro(a.segNS + 4 * (hs + j0)) + part;
            u.thr = bound == 0.f ? __builtin_inff() : kTruncRel * fro(a.segNF + 4 * (hs + j)) / bound;
        }
    } else {
        // pass B: the piece at cut j from S_j (F_{j-1} where the scan dropped S_{j-1}'s
        // share), the first z chunks where S_j's share was dropped, else all of it
        const int j = w.seg;
        u.init_kind = kInitFp32;
        u.init = first_cut(a, j) < j && a.segD[hs + j - 1] ? slot(a.segF, j - 1) : slot(a.segS, j);
        const bool drop = a.segD[hs + j] != 0;
        if (drop && u.c0 + a.segZ[hs + j] < u.c1)
            u.c1 = u.c0 + a.segZ[hs + j];
        const bool last = p.c1 == nch;
        u.fin_kind = last ? a.ht_dtype : 0;
        u.fin = last ? htc : nullptr;
        if (last && drop)
            u.fin_src = slot(a.segF, j);
    }
    return true;
}

// Token range of unit k of a workgroup (what the producers need of it).  Chunk indices
// fit 32 bits (the host rejects sequences of 2^31 chunks or more).
struct Range {
    int64_t start, len;  // the sequence's first token and length
    int c0, c1;          // chunk range of the unit
};
template <int kMode>
__device__ bool range_at(const FusedArgs &a, const WgPlan &w, int64_t k, Range &r)
{
    int64_t n;
    if constexpr (kMode == kModeWhole || kMode == kModeHalves) {
        if (w.sub + k >= w.n_end)
            return false;
        n = a.units[w.sub + k] >> 2;
        r.len = a.seq_len[n];
        r.start = a.seq_start[n];
        r.c0 = 0;
        r.c1 = (int)((r.len + kCH - 1) / kCH);
        return true;
    }
    Piece p;
    constexpr bool passA = kMode == kModeA;
    if (passA ? !run_piece(a, w.seg, k, p) : (k > 0 || !cut_piece(a, w.seg, p)))
        return false;
    r.len = a.seq_len[p.seq];
    r.start = a.seq_start[p.seq];
    r.c0 = p.c0;
    r.c1 = p.c1;
    if constexpr (kMode == kModeB) {  // the chunks pass B reruns (as unit_at)
        const size_t sl = (size_t)w.h * (size_t)a.Pc + (size_t)w.seg;
        if (a.segD[sl] && r.c0 + a.segZ[sl] < r.c1)
            r.c1 = r.c0 + (int)a.segZ[sl];
    }
    return true;
}

// Walks the workgroup's items (chunks of its units, in order) forward.
template <int kMode>
struct ItemWalk {
    int k = 0, base = 0;  // unit index and its first item
    bool valid = false;
    Range r;
    __device__ void init(const FusedArgs &a, const WgPlan &w) { k = 0; base = 0; valid = range_at<kMode>(a, w, 0, r); }
    // position the walk on the unit holding item it (items only move forward)
    __device__ void seek(const FusedArgs &a, const WgPlan &w, int it)
    {
        while (valid && it >= base + (r.c1 - r.c0)) {
            base += r.c1 - r.c0;
            ++k;
            valid = range_at<kMode>(a, w, k, r);
        }
    }
};

typedef __attribute__((address_space(3))) volatile int lds_flag_t;

// Spin until *p == want (all lanes read the same LDS word).  Returns false on time-out.
__device__ __forceinline__ bool lds_wait_eq(lds_flag_t *p, int want)
{
    for (int it = 0; it < kSpinMax; ++it) {
        const int v = __builtin_amdgcn_readfirstlane(*p);
        if (v == want) {
            __asm__ volatile("" ::: "memory");
            return true;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}
// Spin until the four words p[0..3] all equal want.
__device__ __forceinline__ bool lds_wait_eq4(lds_flag_t *p, int want)
{
    for (int it = 0; it < kSpinMax; ++it) {
        const int v0 = __builtin_amdgcn_readfirstlane(p[0]);
        const int v1 = __builtin_amdgcn_readfirstlane(p[1]);
        const int v2 = __builtin_amdgcn_readfirstlane(p[2]);
        const int v3 = __builtin_amdgcn_readfirstlane(p[3]);
        if (v0 == want && v1 == want && v2 == want && v3 == want) {
            __asm__ volatile("" ::: "memory");
            return true;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// Spin until the four words p[0..3] all equal want (returns 1) or *stop <= item (returns 2);
// 0 on time-out.
__device__ __forceinline__ int lds_wait_eq4_or_stop(lds_flag_t *p, int want, lds_flag_t *stop, int item)
{
    for (int it = 0; it < kSpinMax; ++it) {
        const int v0 = __builtin_amdgcn_readfirstlane(p[0]);
        const int v1 = __builtin_amdgcn_readfirstlane(p[1]);
        const int v2 = __builtin_amdgcn_readfirstlane(p[2]);
        const int v3 = __builtin_amdgcn_readfirstlane(p[3]);
        if (v0 == want && v1 == want && v2 == want && v3 == want) {
            __asm__ volatile("" ::: "memory");
            return 1;
        }
        if (__builtin_amdgcn_readfirstlane(*stop) <= item)
            return 2;
        __builtin_amdgcn_s_sleep(1);
    }
    return 0;
}

// s_waitcnt vmcnt(n) for a run-time n in [0, 5]
__device__ __forceinline__ void wait_vmcnt_rt(int n)
{
    switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    default: wait_vmcnt<5>(); break;
    }
}

// Four 16-byte-per-lane direct-to-LDS loads into dst + 1024*i, i = 0..3, from voffsets
// vo[i] + 1024*i (the instruction offset carries the 1024*i on both sides).
__device__ __forceinline__ void dma_tile16(__amdgpu_buffer_rsrc_t r, unsigned char *dst, const uint32_t *vo)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, vo[0], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, vo[1], 0, 1024, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, vo[2], 0, 2048, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)dst, 16, vo[3], 0, 3072, 0);
}

// kSw: the activation switches are read from a.flags; without it every activation runs in
// the pass (the common case gets code with no switch logic in it).  kMode: the launch kind.
// kQ: the workgroup's units write output rows; without it (the transition runs) q is
// neither loaded nor used, and the output-only operands (QG, Mq) are not formed.  kStop:
// the consumers may stop the run early (transition runs).
template <bool kSw, int kMode>
__device__ void fused_producer(const FusedArgs &a, const WgPlan &w, unsigned char *lds, int p, int lane)
{
    constexpr bool kQ = kMode != kModeTrans, kStop = kMode == kModeTrans;
    const int64_t H = a.H;
    const int h = w.h;
    const int r = lane & 15;   // token within the chunk
    const int qb = lane >> 4;  // channels 32*qb .. 32*qb+31
    unsigned char *stage = lds + kOffStage + p * kStageBytes;
    float *tile = reinterpret_cast<float *>(lds + kOffTile + p * 1024);
    const float *dtc = reinterpret_cast<const float *>(lds + kOffDt);
    lds_flag_t *ready = (lds_flag_t *)(lds + kOffFlags);
    lds_flag_t *taken = ready + kNS;
    lds_flag_t *stop = ready + kFlagStop;  // kStop: items from here on are not wanted
    const uint32_t rowb = (uint32_t)(H * kD * 2);  // bytes between consecutive tokens of a head

    // Direct-to-LDS loads of chunk j of unit u: 4 loads of 16 B per lane per tensor (4
    // token rows each) and one 2-byte load per lane for beta.  Row t, 16-byte segment s
    // of a tensor goes to LDS segment s ^ (t & 7) of row t, so that the reads below (8
    // lanes = 8 rows of one segment) hit distinct banks.  Rows past the chunk's end load
    // zeros.
    auto issue_stage = [&](const Range &u, int64_t j) {
        const int64_t t0 = u.start + j * kCH;
        const int64_t rem = u.len - j * kCH;
        const int tl = rem < kCH ? (int)rem : kCH;
        const size_t elem0 = ((size_t)t0 * (size_t)H + (size_t)h) * kD;
        const uint32_t nb = (uint32_t)(tl - 1) * rowb + 256u;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + elem0, nb);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + elem0, nb);
        const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.g + elem0, nb);
        // The 1 KB quarter i of a tile is addressed by the instruction offset 1024*i, which
        // moves the LDS destination and the global address alike (and takes part in the
        // range check), so the voffset drops it and M0 changes once per tensor.
        uint32_t vo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t row = 4 * i + (lane >> 4);
            const uint32_t seg = (uint32_t)(lane & 15) ^ (row & 7u);
            vo[i] = row * rowb + seg * 16u - 1024u * i;  // row * rowb >= 1024 i: rowb >= 256
        }
        if (kQ)
            dma_tile16(rq, stage, vo);
        dma_tile16(rk, stage + 4096, vo);
        dma_tile16(rg, stage + 8192, vo);
        // (the byte count is wave-uniform; say so, or the descriptor goes through a
        // readfirstlane loop)
        const uint32_t nbb = __builtin_amdgcn_readfirstlane((uint32_t)(tl - 1) * (uint32_t)(H * 2) + 2u);
        const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.beta + (size_t)t0 * (size_t)H + (size_t)h, nbb);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void *)(stage + 12288), 2,
                                                 (uint32_t)lane * (uint32_t)(H * 2), 0, 0, 0);
    };

    const bool gate_in = !kSw || (a.flags & kGateIn) != 0;
    const bool l2_in = !kSw || (a.flags & kL2In) != 0;
    const bool sig_in = !kSw || (a.flags & kSigIn) != 0;
    const float m1 = gate_in ? -kLog2e * fexp2(a.A_log[h] * kLog2e) : 0.f;
    const float lb2 = a.lower_bound * kLog2e;

    bool spun_out = false;
    // this wavefront prepares items p, p+4, p+8, ...; `nxt` stays 4 items ahead of `cur`
    ItemWalk<kMode> cur, nxt;
    cur.init(a, w);
    nxt.init(a, w);
    nxt.seek(a, w, p);
    if (nxt.valid)
        issue_stage(nxt.r, nxt.r.c0 + (p - nxt.base));
    for (int it = p;; it += 4) {
        if (kStop && __builtin_amdgcn_readfirstlane(*stop) <= it)
            break;
        cur.seek(a, w, it);
        if (!cur.valid)
            break;
        const Range &u = cur.r;
        const int64_t j = u.c0 + (it - cur.base);  // chunk of the sequence
        const int64_t rem = u.len - j * kCH;
        const int tlen = rem < kCH ? (int)rem : kCH;
        const bool valid = r < tlen;

        wait_vmcnt<0>();
        float qf[32], kf[32], gf[32];
        float ssq = 0.f, ssk = 0.f;  // squared norms over this lane's 32 channels (bf16 dot2)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t seg = (uint32_t)(4 * qb + w) ^ (uint32_t)(r & 7);
            const uint32_t o = (uint32_t)r * 256u + seg * 16u;
            const u32x4_t uq = *reinterpret_cast<const u32x4_t *>(stage + o);
            const u32x4_t uk = *reinterpret_cast<const u32x4_t *>(stage + 4096 + o);
            const u32x4_t ug = *reinterpret_cast<const u32x4_t *>(stage + 8192 + o);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qf[8 * w + 2 * e] = kQ ? bf_lo(uq[e]) : 0.f;
                qf[8 * w + 2 * e + 1] = kQ ? bf_hi(uq[e]) : 0.f;
                kf[8 * w + 2 * e] = bf_lo(uk[e]);
                kf[8 * w + 2 * e + 1] = bf_hi(uk[e]);
                gf[8 * w + 2 * e] = bf_lo(ug[e]);
                gf[8 * w + 2 * e + 1] = bf_hi(ug[e]);
                if (kQ)
                    ssq = dot2_bf16(uq[e], uq[e], ssq);
                ssk = dot2_bf16(uk[e], uk[e], ssk);
            }
        }
        const uint32_t braw = *reinterpret_cast<const uint32_t *>(stage + 12288 + 4 * r);
        wait_lgkmcnt0();
        // the staging tile is consumed: fetch this wavefront's next item into it
        nxt.seek(a, w, it + 4);
        if (nxt.valid)
            issue_stage(nxt.r, nxt.r.c0 + (it + 4 - nxt.base));

        const float braw_f = bf16f((uint16_t)(braw & 0xffffu));
        const float bt = valid ? (sig_in ? sigmoidf_fast(braw_f) : braw_f) : 0.f;

        ssq += __shfl_xor(ssq, 16);
        ssq += __shfl_xor(ssq, 32);
        ssk += __shfl_xor(ssk, 16);
        ssk += __shfl_xor(ssk, 32);
        const float rq = l2_in ? __builtin_amdgcn_rsqf(ssq + 1e-6f) * a.scale : a.scale;
        const float rk = l2_in ? __builtin_amdgcn_rsqf(ssk + 1e-6f) : 1.f;

        // log2-domain log-decay lb*log2e*sigmoid(x), x = exp(A_log)*(g + dt_bias):
        // sigmoid(x) = 1 / (1 + 2^(g*m1 + d1)), m1 = -log2e*exp(A_log), d1 = m1*dt_bias.
        // A pre-activated gate is the natural-log decay itself, held to [lb, 0].  Tokens
        // past the chunk's end get a zero log-decay.
        const float lbv = valid ? lb2 : 0.f;
        float b2[32];
        if (gate_in) {
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const f32x4_t d4 = *reinterpret_cast<const f32x4_t *>(dtc + 32 * qb + 4 * w);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 4 * w + e;
                    float av = lbv * frcp(1.0f + fexp2(fmaf(gf[c], m1, d4[e])));
                    av = row_scan16(av);
                    b2[c] = av;
                }
            }
        } else {
            const float gk = valid ? kLog2e : 0.f;
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                float av = gk * fminf(fmaxf(gf[c], a.lower_bound), 0.f);
                av = row_scan16(av);
                b2[c] = av;
            }
        }

        // Gamma = 2^b, 1/Gamma = 2^-b; gamma is Gamma at the chunk's last token (lane 15 of
        // the row).  KG = k^ Gamma, QG = scale q^ Gamma, KI = k^ / Gamma, KD = KI gamma.
        // A_kk = KG KI^T and A_qk = QG KI^T (gamma cancels in both).
        float KG[32], QG[32], KD[32], KI[32], GL[32];
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            const float G = fexp2(b2[c]);
            const float Gi = fexp2(-b2[c]);
            const float kn = kf[c] * rk;
            const float qn = qf[c] * rq;
            KG[c] = kn * G;
            QG[c] = qn * G;
            KI[c] = kn * Gi;
            KD[c] = KI[c] * dpp_row_last(G);
            GL[c] = G;
        }
        // bf16 hi/lo pairs.  KG, KI and QG go in the operand-block order: group gg holds
        // channels 4gg .. 4gg+3 and 16+4gg .. 16+4gg+3 of the lane's 32 (the same K order
        // on both MFMA operands, so A_kk and A_qk contract over every channel).  KD keeps
        // the natural order (8s .. 8s+7).  lo = x - hi comes from one MFMA per 4 values:
        // (-I) hi + x, exact in fp32.
        u32x4_t negI0, negI1;
        make_neg_identity(lane, negI0, negI1);
        auto split8 = [&](const float *x0, const float *x1, u32x4_t &hi, u32x4_t &lo) {
            hi = u32x4_t{pack_bf16x2(x0[0], x0[1]), pack_bf16x2(x0[2], x0[3]),
                         pack_bf16x2(x1[0], x1[1]), pack_bf16x2(x1[2], x1[3])};
            const f32x4_t r0 = mfma32(negI0, hi, f32x4_t{x0[0], x0[1], x0[2], x0[3]});
            const f32x4_t r1 = mfma32(negI1, hi, f32x4_t{x1[0], x1[1], x1[2], x1[3]});
            lo = u32x4_t{pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3]),
                         pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
        };
        u32x4_t kgh[4], kgl[4], qgh[4], kih[4], kil[4], kdb[4], kdlo[4];
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            split8(KG + 4 * gg, KG + 16 + 4 * gg, kgh[gg], kgl[gg]);
            split8(KI + 4 * gg, KI + 16 + 4 * gg, kih[gg], kil[gg]);
            qgh[gg] = u32x4_t{pack_bf16x2(QG[4 * gg], QG[4 * gg + 1]), pack_bf16x2(QG[4 * gg + 2], QG[4 * gg + 3]),
                              pack_bf16x2(QG[16 + 4 * gg], QG[16 + 4 * gg + 1]),
                              pack_bf16x2(QG[16 + 4 * gg + 2], QG[16 + 4 * gg + 3])};
            split8(KD + 8 * gg, KD + 8 * gg + 4, kdb[gg], kdlo[gg]);
        }
        f32x4_t akk = {0.f, 0.f, 0.f, 0.f}, aqkT = akk;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            akk = mfma32(kgh[gg], kih[gg], akk);
            akk = mfma32(kgl[gg], kih[gg], akk);
            akk = mfma32(kgh[gg], kil[gg], akk);
            if (kQ)
                aqkT = mfma32(kih[gg], qgh[gg], aqkT);
        }
        const int g4 = (lane >> 4) * 4, col = lane & 15;
        f32x4_t A, AqT, I4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = g4 + i;
            const float brow = __shfl(bt, row);
            A[i] = col < row ? brow * akk[i] : 0.f;
            AqT[i] = row <= col ? aqkT[i] : 0.f;
            I4[i] = row == col ? 1.f : 0.f;
        }
        const f32x4_t AT = transpose16(A, tile, lane);
        const f32x4_t P2 = mm16(AT, A);
        const f32x4_t P2T = transpose16(P2, tile, lane);
        const f32x4_t P4 = mm16(P2T, P2);
        const f32x4_t P4T = transpose16(P4, tile, lane);
        const f32x4_t P8 = mm16(P4T, P4);
        const f32x4_t R1 = mm16(I4 + P4T, I4 + P8);
        const f32x4_t R2 = mm16(I4 + P2T, R1);
        const f32x4_t Tm = mm16(I4 - AT, R2);
        const f32x4_t Tb = Tm * bt;
        const f32x4_t TbT = transpose16(Tb, tile, lane);
        f32x4_t MqT = {0.f, 0.f, 0.f, 0.f};
        if (kQ)
            MqT = transpose16(mm16(AqT, Tb), tile, lane);

        // ---- hand the operand block to the consumers ----
        const int s = it % kNS;
        if (kStop) {
            // a transition run that stops early never frees the slots of the items after
            // its last: wait for the slot or for the stop word
            const int r = spun_out ? 1 : lds_wait_eq4_or_stop(taken + 4 * s, it / kNS, stop, it);
            if (r == 2)
                break;
            if (r == 0) {
                spun_out = true;
                atomicOr(a.status, kStatusSpin);
            }
        } else if (!spun_out && !lds_wait_eq4(taken + 4 * s, it / kNS)) {
            spun_out = true;  // stop waiting from here on; the status word reports it
            atomicOr(a.status, kStatusSpin);
        }
        unsigned char *rec = lds + (size_t)s * kBlkBytes;
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const int o = (qb * 64 + r + 16 * gg) * 16;
            *reinterpret_cast<u32x4_t *>(rec + kBlkKG + o) = kgh[gg];
            *reinterpret_cast<u32x4_t *>(rec + kBlkKGL + o) = kgl[gg];
            if (kQ)
                *reinterpret_cast<u32x4_t *>(rec + kBlkQG + o) = qgh[gg];
        }
        // KD: channel ch = 32qb + c goes to tile ch/16, token group r/4, token r%4 of the
        // hi and lo quarters of a 16-byte fragment.  In tile t and token group gq the
        // fragment of channel position j sits at 16-byte slot j ^ (4gq + t/2) of the
        // group's 256-byte row: the 16 lanes (qb, r/4) that write one channel hit 16
        // different slots, so the 2-byte stores meet no bank conflicts, and a consumer's
        // 16-lane group still reads the 16 slots of one row.  Every term of the address
        // but the slot index is a multiple of 256 or below 16, so the XOR acts on bits 4-7.
        {
            const uint32_t kd0 = (uint32_t)(rec - lds) + (uint32_t)kBlkKD + 2048u * (uint32_t)qb +
                                 256u * (uint32_t)(r >> 2) + 2u * (uint32_t)(r & 3) +
                                 16u * (uint32_t)(4 * (r >> 2) + qb);
#pragma unroll
            for (int c = 0; c < 32; ++c) {
                const uint32_t o = (kd0 ^ (16u * (uint32_t)(c & 15))) + 1024u * (uint32_t)(c >> 4);
                const uint32_t word = (c & 1) ? kdb[c >> 3][(c & 7) >> 1] >> 16 : kdb[c >> 3][(c & 7) >> 1] & 0xffffu;
                const uint32_t wlo = (c & 1) ? kdlo[c >> 3][(c & 7) >> 1] >> 16 : kdlo[c >> 3][(c & 7) >> 1] & 0xffffu;
                *reinterpret_cast<uint16_t *>(lds + o) = (uint16_t)word;
                *reinterpret_cast<uint16_t *>(lds + o + 8) = (uint16_t)wlo;
            }
        }
        if (r == 15) {
            // channels 32qb + j and 32qb + 16 + j are tiles 2qb, 2qb + 1 of position j
            float *gp = reinterpret_cast<float *>(rec + kBlkGAM) + 2 * qb;
#pragma unroll
            for (int j = 0; j < 16; ++j)
                *reinterpret_cast<f32x2_t *>(gp + 8 * j) = f32x2_t{GL[j], GL[16 + j]};
        }
        {
            u32x4_t w;
            const float h0 = bf16f(to_bf16(TbT[0])), h1 = bf16f(to_bf16(TbT[1]));
            const float h2 = bf16f(to_bf16(TbT[2])), h3 = bf16f(to_bf16(TbT[3]));
            w[0] = pack_bf16x2(TbT[0], TbT[1]);
            w[1] = pack_bf16x2(TbT[2], TbT[3]);
            w[2] = pack_bf16x2(TbT[0] - h0, TbT[1] - h1);
            w[3] = pack_bf16x2(TbT[2] - h2, TbT[3] - h3);
            *reinterpret_cast<u32x4_t *>(rec + kBlkTB + (size_t)lane * 16) = w;
        }
        if (kQ) {
            const float m0 = bf16f(to_bf16(MqT[0])), m1 = bf16f(to_bf16(MqT[1]));
            const float m2 = bf16f(to_bf16(MqT[2])), m3 = bf16f(to_bf16(MqT[3]));
            u32x4_t m;
            m[0] = pack_bf16x2(MqT[0], MqT[1]);
            m[1] = pack_bf16x2(MqT[2], MqT[3]);
            m[2] = pack_bf16x2(MqT[0] - m0, MqT[1] - m1);
            m[3] = pack_bf16x2(MqT[2] - m2, MqT[3] - m3);
            *reinterpret_cast<u32x4_t *>(rec + kBlkMQ + (size_t)lane * 16) = m;
        }
        wait_lgkmcnt0();
        __asm__ volatile("" ::: "memory");
        if (lane == 0)
            ready[s] = it;
    }
    // a stopped run may leave the next item's staging loads in flight: they write LDS
    wait_vmcnt<0>();
}

// One unit's items for consumer wavefront cw: state in, chunk recurrence, state out.
// Items of the unit are it0, it0+1, ... in the workgroup's item numbering (slots, flags).
// kOut: the unit writes output rows (u.out_on); without it Y and O are not formed and the
// output-only operands are not read.  NB: 16-column blocks of this wave -- 2 for a whole
// unit (columns 32cw .. 32cw+31), 1 for a column half (64*half + 16cw .. +15).
// kP: a transition run (from I, v = 0) of the piece at cut j that, when a.trunc allows,
// stops after the first chunk at whose end every entry of the state is below u.thr =
// kTruncRel |F_j|_F / B_j (the bound of kda_internal.h: S_j's share of every later state
// of the piece is then at most 2^-30 |F_j|_F in Frobenius norm).  The four consumers vote
// after every chunk, so they stop together, and the producers are told through the stop
// word.  The chunk count goes to *u.zout (-1: ran to the end, state written).
// kSeg: a segment pass unit (pass A end-state norms, pass B final state taken from F).
template <bool kOut, int NB, bool kP, bool kSeg>
__device__ void consume_unit(const FusedArgs &a, const Unit &u, unsigned char *lds, int cw, int lane,
                             int it0, bool &spun_out)
{
    const int cb0 = NB == 2 ? 32 * cw : 64 * u.half + 16 * cw;  // first value column of this wave
    constexpr int kRowB = 32 * NB;   // bytes per token row of this wave's value and output tiles
    constexpr int kLpr = kRowB / 16; // lanes per row of 16 bytes each
    const int64_t H = a.H;
    const int h = u.h;
    const int64_t start = u.start, len = u.len, c0 = u.c0, c1 = u.c1;
    const int g = lane >> 4;
    const int col = lane & 15;
    lds_flag_t *ready = (lds_flag_t *)(lds + kOffFlags);
    lds_flag_t *taken = ready + kNS;
    int stopped = -1;     // kP: chunks run before the stop
    const float thr = u.thr;  // kP: stop once every entry is below this (NaN: never)
    unsigned char *vring = lds + kOffVring + cw * (kNV * 1024);
    const uint32_t rowb = (uint32_t)(H * kD * 2);

    // state: S[b][t] = S[v][16t + 4g + i] (element i) for value column v = cb0 + 16b + col
    f32x4_t S[NB][8];
    {
        const int64_t sb0 = (int64_t)(cb0 + col) * kD + 4 * g;  // column block b adds 16*128
        if (u.init_kind == kInitFp32) {
            const float *p = reinterpret_cast<const float *>(u.init) + sb0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    S[b][t] = *reinterpret_cast<const f32x4_t *>(p + b * 16 * kD + 16 * t);
        } else if (u.init_kind == kInitBf16) {
            const uint16_t *p = reinterpret_cast<const uint16_t *>(u.init) + sb0;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const u32x2_t w = *reinterpret_cast<const u32x2_t *>(p + b * 16 * kD + 16 * t);
                    S[b][t] = f32x4_t{bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1])};
                }
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    S[b][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (u.init_kind == kInitIdentity) {
                // S[v][v] = 1: column v = cb0 + 16b + col sits in channel tile cb0/16 + b,
                // element col - 4g of this lane when that lies in [0, 4)
                const int e = col - 4 * g;
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int t = 0; t < 8; ++t)
                        if (t == cb0 / 16 + b) {
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                S[b][t][i] = e == i ? 1.f : 0.f;
                        }
            }
        }
    }

    // value tile of chunk j (16 tokens x this wave's 16 NB columns, row-major kRowB-byte rows)
    // into ring slot j % kNV: lane L loads row L/kLpr, bytes 16*(L%kLpr); rows past the end
    // (also rows 16 .. 31 when NB = 1) load zeros
    auto issue_v = [&](int64_t j) {
        const int64_t t0 = start + j * kCH;
        const int64_t rem = len - j * kCH;
        const int tl = rem < kCH ? (int)rem : kCH;
        const __amdgpu_buffer_rsrc_t rv =
            make_rsrc(a.v + ((size_t)t0 * (size_t)H + (size_t)h) * kD + cb0, (uint32_t)(tl - 1) * rowb + (uint32_t)kRowB);
        const uint32_t vo = (uint32_t)(lane / kLpr) * rowb + (uint32_t)(lane % kLpr) * 16u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(vring + ((int)(j - c0) % kNV) * 1024), 16, vo, 0, 0, 0);
    };
    if (u.v_on) {
#pragma unroll
        for (int jp = 0; jp < kNV; ++jp)
            if (c0 + jp < c1)
                issue_v(c0 + jp);
    }
    // -I in the MFMA A layout for the k-slot order of a channel pair of tiles (2t, 2t+1):
    // slot 8*(m/4) + m%4 holds channel m of tile 2t, slot 8*(m/4) + 4 + m%4 channel m of
    // tile 2t+1.  Lane m + 16*(m/4) carries the -1 (bf16 0xbf80) at element m%4 or 4+m%4.
    u32x4_t negI0, negI1;
    make_neg_identity(lane, negI0, negI1);
    unsigned char *obuf = lds + kOffOut + cw * 1024;  // output tile of the previous chunk
    // output row this lane stores: 16 rows of kLpr lanes each; with NB = 1 lanes 32-63 map
    // past row 15 and store nothing
    const int orow = lane / kLpr;
    auto store_out = [&](int64_t jo) {
        const int64_t rem = len - jo * kCH;
        const u32x4_t ow = *reinterpret_cast<const u32x4_t *>(obuf + lane * 16);
        if (orow < kCH && orow < rem)
            *reinterpret_cast<u32x4_t *>(a.out + ((size_t)(start + jo * kCH + orow) * (size_t)H + (size_t)h) * kD +
                                         cb0 + 8 * (lane % kLpr)) = ow;
    };
    int gm_off = 0;
    __asm__("" : "+v"(gm_off));
    // KD fragment of channel position col, token group g, tile t: slot col ^ (4g + t/2)
    int kdo[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
        kdo[k] = 256 * g + 16 * (col ^ (4 * g + k));
    for (int64_t j = c0; j < c1; ++j) {
        const int iu = (int)(j - c0);  // item index within the unit (value ring, store count)
        const int it = it0 + iu;       // item index within the workgroup (operand slots)
        const int s = it % kNS;
        const unsigned char *rec = lds + (size_t)s * kBlkBytes;
        u32x4_t kg[4], kgl[4], qg[4], kd[8];
        // gamma of channel 16t + 4g + (lane & 3) is gm[b][t / 4][t % 4]; each column block b
        // has its own copy, so every quad broadcast below has one use and folds into its
        // multiply (gm_off is an opaque zero that keeps the two reads apart)
        f32x4_t gm[NB][2];
        u32x4_t tb, mq;
        // The operand reads go out right behind the read of ready[s]; LDS serves one
        // wavefront's requests in order, so when that read shows chunk j the operands
        // read after it are chunk j's.  Otherwise wait, then read them again.
        auto read_ops = [&]() {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                kg[t] = *reinterpret_cast<const u32x4_t *>(rec + kBlkKG + (t * 64 + lane) * 16);
                kgl[t] = *reinterpret_cast<const u32x4_t *>(rec + kBlkKGL + (t * 64 + lane) * 16);
                if (kOut)
                    qg[t] = *reinterpret_cast<const u32x4_t *>(rec + kBlkQG + (t * 64 + lane) * 16);
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                kd[t] = *reinterpret_cast<const u32x4_t *>(rec + kBlkKD + t * 1024 + kdo[t >> 1]);
                if (t < 2 * NB)
                    gm[t >> 1][t & 1] = *reinterpret_cast<const f32x4_t *>(
                        rec + kBlkGAM + (8 * (4 * g + (col & 3)) + 4 * (t & 1)) * 4 + ((t >> 1) ? gm_off : 0));
            }
            tb = *reinterpret_cast<const u32x4_t *>(rec + kBlkTB + lane * 16);
            if (kOut)
                mq = *reinterpret_cast<const u32x4_t *>(rec + kBlkMQ + lane * 16);
        };
        const int seen = ready[s];
        __asm__ volatile("" ::: "memory");
        read_ops();
        if (__builtin_amdgcn_readfirstlane(seen) != it) {
            if (!spun_out && !lds_wait_eq(ready + s, it)) {
                spun_out = true;  // stop waiting from here on; the status word reports it
                atomicOr(a.status, kStatusSpin);
            }
            read_ops();
        }
        // the previous chunk's output tile (staged in LDS) goes to HBM
        if (kOut && iu > 0)
            store_out(j - 1);

        // value tile of chunk j: vector-memory operations issued after its ring load are
        // the ring loads of chunks j+1, j+2 (those in range) and, when out is written, the
        // output stores of the items max(0, it-3) .. it-1 (one store instruction each; its
        // lanes for row 0 are always active)
        float vv[NB][4];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vv[b][i] = 0.f;
        if (u.v_on) {
            const int64_t later = c1 - 1 - j;
            const int nd = later < 2 ? (int)later : 2;
            const int ns = !kOut ? 0 : iu < 3 ? iu : 3;
            wait_vmcnt_rt(nd + ns);
            unsigned char *vt = vring + (iu % kNV) * 1024;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    vv[b][i] = bf16f(*reinterpret_cast<const uint16_t *>(vt + (4 * g + i) * kRowB + (16 * b + col) * 2));
            // the value slot is read: refill it with chunk j + kNV
            if (j + kNV < c1) {
                wait_lgkmcnt0();
                issue_v(j + kNV);
            }
        }

        // Z = KG S^T (three products) and Y = QG S^T (one), per channel pair t of tiles
        // (2t, 2t+1).  S splits as hi = bf16(S) and lo = S - hi; the difference is exact in
        // fp32 and one MFMA per tile forms it: (-I) hi + S.
        f32x4_t Z[NB], Y[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            Z[b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            Y[b] = Z[b];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f32x4_t s0 = S[b][2 * t], s1 = S[b][2 * t + 1];
                const u32x4_t sb = {pack_bf16x2(s0[0], s0[1]), pack_bf16x2(s0[2], s0[3]),
                                    pack_bf16x2(s1[0], s1[1]), pack_bf16x2(s1[2], s1[3])};
                const f32x4_t r0 = mfma32(negI0, sb, s0);
                const f32x4_t r1 = mfma32(negI1, sb, s1);
                const u32x4_t sl = {pack_bf16x2(r0[0], r0[1]), pack_bf16x2(r0[2], r0[3]),
                                    pack_bf16x2(r1[0], r1[1]), pack_bf16x2(r1[2], r1[3])};
                Z[b] = mfma32(kg[t], sb, Z[b]);
                Z[b] = mfma32(kgl[t], sb, Z[b]);
                Z[b] = mfma32(kg[t], sl, Z[b]);
                if (kOut)
                    Y[b] = mfma32(qg[t], sb, Y[b]);
            }
        }
        f32x4_t O[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            f32x4_t X;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                X[i] = vv[b][i] - Z[b][i];  // value rows past the chunk's end load zeros, Z is zero there
            const u32x2_t x01 = split_bf16x2(X[0], X[1]);
            const u32x2_t x23 = split_bf16x2(X[2], X[3]);
            const u32x4_t xhh = {x01[0], x23[0], x01[0], x23[0]};
            // V' = Tb X: [Tb_hi | Tb_lo] [X_hi ; X_hi] + [Tb_hi | Tb_lo] [X_lo ; 0]
            f32x4_t Vp = {0.f, 0.f, 0.f, 0.f};
            Vp = mfma32(tb, xhh, Vp);
            Vp = mfma32(tb, u32x4_t{x01[1], x23[1], 0u, 0u}, Vp);
            const u32x2_t v01 = split_bf16x2(Vp[0], Vp[1]);
            const u32x2_t v23 = split_bf16x2(Vp[2], Vp[3]);
            const u32x4_t vhh = {v01[0], v23[0], v01[0], v23[0]};
            const u32x4_t vl0 = {v01[1], v23[1], 0u, 0u};
            // S <- S diag(gamma) + KD^T V': [KD_hi | KD_lo] [V'_hi ; V'_hi] + [KD_hi | KD_lo] [V'_lo ; 0]
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                // element i is channel 16t + 4g + i: its gamma sits in lane i of this quad
                const float gt = gm[b][t >> 2][t & 3];
                f32x4_t st = {S[b][t][0] * quad_bcast<0>(gt), S[b][t][1] * quad_bcast<1>(gt),
                              S[b][t][2] * quad_bcast<2>(gt), S[b][t][3] * quad_bcast<3>(gt)};
                st = mfma32(kd[t], vhh, st);
                st = mfma32(kd[t], vl0, st);
                S[b][t] = st;
            }
            if (kOut)
                O[b] = mfma32(mq, xhh, Y[b]);
        }

        // output rows 4g+i, columns 16b+col -> LDS tile; the next iteration (or the end)
        // stores it with one 16-byte write per lane: row L/4, columns 8*(L%4) .. +7
        if (kOut) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    *reinterpret_cast<uint16_t *>(obuf + (4 * g + i) * kRowB + (16 * b + col) * 2) = to_bf16(O[b][i]);
        }
        // every operand of chunk j is in registers (used above): release the slot
        if (lane == 0)
            taken[4 * s + cw] = it / kNS + 1;
        if (kP && a.trunc) {
            // vote: 2 iu + (every entry of this wave's rows below thr); votes of
            // consecutive chunks alternate between two sets of four words, and a wave can
            // be at most one chunk ahead of the others here
            bool big = false;
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        big |= !(__builtin_fabsf(S[b][t][i]) < thr);  // NaN counts as big
            const bool wbig = __builtin_amdgcn_ballot_w64(big) != 0;
            lds_flag_t *vote = ready + kFlagVote + 4 * (iu & 1);
            if (lane == 0)
                vote[cw] = 2 * iu + (wbig ? 0 : 1);
            bool small = true;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                int v = __builtin_amdgcn_readfirstlane(vote[k]);
                for (int spin = 0; (v >> 1) != iu && !spun_out && spin < kSpinMax; ++spin) {
                    __builtin_amdgcn_s_sleep(1);
                    v = __builtin_amdgcn_readfirstlane(vote[k]);
                }
                if ((v >> 1) != iu) {
                    if (!spun_out) {
                        spun_out = true;
                        atomicOr(a.status, kStatusSpin);
                    }
                    v = 0;  // no vote: keep running
                }
                small = small && (v & 1);
            }
            if (small) {
                stopped = iu + 1;
                if (cw == 0 && lane == 0)
                    ready[kFlagStop] = it + 1;
                break;
            }
        }
    }
    if (kP) {
        if (cw == 0 && lane == 0)
            *u.zout = stopped;
        if (stopped >= 0)
            return;  // the state is below thr: the scan drops it, nothing to write
    }
    if (kOut && c1 > c0) {
        wait_lgkmcnt0();
        store_out(c1 - 1);
    }

    const int64_t sb0 = (int64_t)(cb0 + col) * kD + 4 * g;
    if (kSeg && u.nrm != nullptr) {
        float ss = 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ss = fmaf(S[b][t][i], S[b][t][i], ss);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            ss += __shfl_xor(ss, o);
        if (lane == 0)
            u.nrm[cw] = ss;
    }
    if (kSeg && u.fin_src != nullptr) {
        const float *p = u.fin_src + sb0;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int t = 0; t < 8; ++t)
                S[b][t] = *reinterpret_cast<const f32x4_t *>(p + b * 16 * kD + 16 * t);
    }
    if (u.fin_kind == 2) {
        float *p = reinterpret_cast<float *>(u.fin) + sb0;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int t = 0; t < 8; ++t)
                *reinterpret_cast<f32x4_t *>(p + b * 16 * kD + 16 * t) = S[b][t];
    } else if (u.fin_kind == 1) {
        uint16_t *p = reinterpret_cast<uint16_t *>(u.fin) + sb0;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const u32x2_t w = {pack_bf16x2(S[b][t][0], S[b][t][1]), pack_bf16x2(S[b][t][2], S[b][t][3])};
                *reinterpret_cast<u32x2_t *>(p + b * 16 * kD + 16 * t) = w;
            }
    }
}

// kHalves: the unit list may hold column halves (a separate kernel instantiation, so that
// whole-unit launches carry no NB = 1 code)
// kMode: launch kind of the fused kernel (below)

template <int kMode>
__device__ void fused_consumer(const FusedArgs &a, const WgPlan &w, unsigned char *lds, int cw, int lane)
{
    bool spun_out = false;
    int it0 = 0;
    Unit u;
    if constexpr (kMode == kModeWhole || kMode == kModeHalves) {
        // Whole chains, several per workgroup: the next unit's lookups go out before this unit
        // runs and complete meanwhile, and the previous unit's state and output stores may still
        // be in flight when this one starts (vector memory operations complete in issue order,
        // so the value ring's counted waits, with those older stores ahead of them, still mean
        // what they say).
        Unit next;
        bool have = unit_at<kMode>(a, w, 0, u);
        for (int64_t k = 0; have; ++k) {
            const bool have_next = unit_at<kMode>(a, w, k + 1, next);
            if (kMode == kModeWhole || u.half < 0)
                consume_unit<true, 2, false, false>(a, u, lds, cw, lane, it0, spun_out);
            else
                consume_unit<true, 1, false, false>(a, u, lds, cw, lane, it0, spun_out);
            it0 += (int)(u.c1 - u.c0);
            u = next;
            have = have_next;
        }
    } else {
        for (int64_t k = 0; unit_at<kMode>(a, w, k, u); ++k) {
            // the previous unit's stores are done before this unit's value-ring bookkeeping starts
            wait_vmcnt<0>();
            if (kMode == kModeTrans)
                consume_unit<false, 2, true, false>(a, u, lds, cw, lane, it0, spun_out);
            else
                consume_unit<true, 2, false, true>(a, u, lds, cw, lane, it0, spun_out);
            it0 += (int)(u.c1 - u.c0);
        }
    }
}

// kMode: whole chains (pass 0), whole chains that may hold column halves (pass 0), segment
// passes A and B (1, 2), transition runs (pass 3); separate instantiations, so that each
// carries only its own code and registers.
template <bool kSw, int kMode>
__global__ __launch_bounds__(512) void fused_kernel(FusedArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // this workgroup's work (see SegPlan for the passes)
    WgPlan w;
    w.pass = kMode == kModeWhole || kMode == kModeHalves ? 0 : kMode == kModeA ? 1 : kMode == kModeB ? 2 : 3;
    w.seg = 0;
    const uint32_t bid = blockIdx.x, H32 = (uint32_t)a.H;
    if (w.pass == 0) {
        // heads h = block % H; block / H of a head takes the run of sequences the chunk
        // table assigned to it
        w.h = (int)(bid % H32);
        const uint32_t grp = bid / H32;
        w.sub = a.wg_first[grp];
        w.n_end = a.wg_first[grp + 1];
        w.n = 0;
    } else {
        // cut plan, head h = block % H: pass A takes run block / H, pass B and the transition
        // runs take cut 1 + block / H
        w.h = (int)(bid % H32);
        w.seg = (int)(bid / H32) + (w.pass == 1 ? 0 : 1);
        w.n = 0;
        w.sub = 0;
        w.n_end = 0;
    }

    if (threadIdx.x < kFlagVote + 8) {
        int *fl = reinterpret_cast<int *>(lds + kOffFlags);
        const int t = (int)threadIdx.x;
        fl[t] = t < kNS ? -1 : t < kFlagStop ? 0 : t == kFlagStop ? 0x7fffffff : -1;
    }
    if (threadIdx.x < kD && (!kSw || (a.flags & kGateIn))) {
        const float m1 = -kLog2e * fexp2(a.A_log[w.h] * kLog2e);
        reinterpret_cast<float *>(lds + kOffDt)[threadIdx.x] = m1 * a.dt_bias[(int64_t)w.h * kD + threadIdx.x];
    }
    __syncthreads();
    if (wave < 4) {
        fused_producer<kSw, kMode>(a, w, lds, wave, lane);
    } else {
        // The consumers set the pace (producers finish ahead and wait for free slots), so
        // they get issue priority over the producer sharing their SIMD.
        __builtin_amdgcn_s_setprio(1);
        fused_consumer<kMode>(a, w, lds, wave - 4, lane);
    }
}

// Cut scan: S_{j+1} = S_j P_j + F_j for consecutive cuts j, j + 1 inside one sequence, on
// v_mfma_f32_16x16x32_bf16 with a hi/lo bf16 split of both factors (three products: hi hi,
// lo hi, hi lo; fp32 accumulate, about 16 significant bits per factor, as the chunk
// recurrence's state products).  Rows of S are independent: a workgroup takes 16 rows of
// one head's states (8 workgroups per head).  For contraction chunk kc (32 channels) lane
// m + 16kg holds S[m][32kc + 8kg + e], e = 0..7 (the A operand), split from the 16 rows
// kept in LDS between steps.  Wave w forms output column tiles 2w and 2w + 1; lane n + 16kg
// of chunk kc, tile t takes P[32kc + 8kg + e][16t + n] (the B operand) straight from global
// memory (16 lanes read 64 contiguous bytes) and splits it; the loads of the next computed
// step go out before this step's products.  Workgroup b takes head b % H, so the 8
// workgroups of a head share a slot modulo 8 (the XCD the dispatcher gives them, whose L2
// then holds that head's P_j once).
//
// Dropped shares.  Where the transition run of cut j stopped early (z_j >= 0: its state fell
// below the bound that makes S_j's share negligible), S_{j+1} = F_j: nothing is computed or
// written, and pass B and the next step read F_j.  The first workgroup of a head records
// the decisions for pass B.
struct ScanArgs {
    float *segS, *segF, *segP;
    const int32_t *segZ;
    int32_t *segD;
    const int32_t *cut_seq, *cut_off;
    int Pc;
    int64_t H;
};

__global__ __launch_bounds__(256) void seg_scan_kernel(ScanArgs a)
{
    __shared__ __attribute__((aligned(16))) float s_rows[16][kD + 4];
    __shared__ int s_drop[kPlanCUs + 1];
    __shared__ int s_step[kPlanCUs + 1];  // cuts j, j + 1 both inside one sequence
    constexpr int64_t kBlock = (int64_t)kD * kD;
    const int64_t h = blockIdx.x % a.H;
    const int r0 = (int)(blockIdx.x / a.H) * 16;
    if (r0 >= kD)
        return;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int m = lane & 15, kg = lane >> 4;  // A: row m, k-group kg; B and D: column m
    const int P = a.Pc;
    const size_t hs = (size_t)h * (size_t)P;
    for (int j = threadIdx.x; j < P; j += 256) {
        const bool inner = j > 0 && a.cut_off[j] > 0;  // a cut inside a sequence
        s_drop[j] = inner && a.segZ[hs + j] >= 0;
        s_step[j] = inner && a.cut_off[j + 1] > 0 && a.cut_seq[j + 1] == a.cut_seq[j];
        if (r0 == 0 && j > 0)
            a.segD[hs + j] = s_drop[j];
    }
    __syncthreads();
    auto blk = [&](float *base, int j) { return base + (hs + (size_t)j) * kBlock; };
    u32x4_t ahi[4], alo[4];
    auto split_A = [&](const float *row) {  // row = S[r0 + m]
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const f32x4_t x0 = *reinterpret_cast<const f32x4_t *>(row + 32 * kc + 8 * kg);
            const f32x4_t x1 = *reinterpret_cast<const f32x4_t *>(row + 32 * kc + 8 * kg + 4);
            const u32x2_t p0 = split_bf16x2(x0[0], x0[1]), p1 = split_bf16x2(x0[2], x0[3]);
            const u32x2_t p2 = split_bf16x2(x1[0], x1[1]), p3 = split_bf16x2(x1[2], x1[3]);
            ahi[kc] = u32x4_t{p0[0], p1[0], p2[0], p3[0]};
            alo[kc] = u32x4_t{p0[1], p1[1], p2[1], p3[1]};
        }
    };
    float bv[2][4][8];
    f32x4_t fv[2];  // F_j[r0 + 4kg + i][16(2w + t) + m]: the D layout of the output tiles
    auto load_BF = [&](int j) {
        const float *Pm = blk(a.segP, j) + (size_t)(8 * kg) * kD + 32 * w + m;
        const float *F = blk(a.segF, j) + (size_t)(r0 + 4 * kg) * kD + 32 * w + m;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fv[t][i] = F[(size_t)i * kD + 16 * t];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    bv[t][kc][e] = Pm[(size_t)(32 * kc + e) * kD + 16 * t];
        }
    };
    // the next computed step >= j (P if none)
    auto next_step = [&](int j) {
        while (j < P && !(s_step[j] && !s_drop[j]))
            ++j;
        return j;
    };
    int loaded = next_step(1);
    if (loaded < P)
        load_BF(loaded);
    bool have = false;  // ahi / alo hold S_j
    for (int j = 1; j < P; ++j) {
        if (!s_step[j] || s_drop[j]) {
            have = false;  // no step, or S_{j+1} = F_j
            continue;
        }
        // S_j: from pass A at a sequence's first cut, F_{j-1} after a dropped step
        if (!have)
            split_A((s_step[j - 1] ? blk(a.segF, j - 1) : blk(a.segS, j)) + (size_t)(r0 + m) * kD);
        f32x4_t acc[2];
        u32x4_t ch[2][4], cl[2][4];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            acc[t] = fv[t];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const float *x = bv[t][kc];
                const u32x2_t p0 = split_bf16x2(x[0], x[1]), p1 = split_bf16x2(x[2], x[3]);
                const u32x2_t p2 = split_bf16x2(x[4], x[5]), p3 = split_bf16x2(x[6], x[7]);
                ch[t][kc] = u32x4_t{p0[0], p1[0], p2[0], p3[0]};
                cl[t][kc] = u32x4_t{p0[1], p1[1], p2[1], p3[1]};
            }
        }
        loaded = next_step(j + 1);
        if (loaded < P)
            load_BF(loaded);
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                acc[t] = mfma32(ahi[kc], ch[t][kc], acc[t]);
                acc[t] = mfma32(alo[kc], ch[t][kc], acc[t]);
                acc[t] = mfma32(ahi[kc], cl[t][kc], acc[t]);
            }
        // rows 4kg + i, column 32w + 16t + m: to global, and through LDS to the A layout
        float *Sn = blk(a.segS, j + 1) + (size_t)(r0 + 4 * kg) * kD + 32 * w + m;
        __syncthreads();  // the previous step's reads of s_rows are done
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Sn[(size_t)i * kD + 16 * t] = acc[t][i];
                s_rows[4 * kg + i][32 * w + 16 * t + m] = acc[t][i];
            }
        __syncthreads();
        split_A(&s_rows[m][0]);
        have = true;
    }
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
hipError_t launch_chunk_table(const FwdArgs &f, hipStream_t s, bool plan)
{
    TableArgs a;
    a.cu = f.cu;
    a.B = f.B;
    a.T = f.T;
    a.N = f.lay.n_seq;
    a.status = reinterpret_cast<int32_t *>(f.ws + f.lay.off_status);
    a.n_total = reinterpret_cast<int64_t *>(f.ws + f.lay.off_status + 8);
    a.P = whole_chain_groups(f.H, f.lay.n_seq, f.cu != nullptr);
    a.wg_first = reinterpret_cast<int64_t *>(f.ws + f.lay.off_wg);
    a.units = reinterpret_cast<int32_t *>(f.ws + f.lay.off_units);
    a.whole = plan && f.lay.cutP <= 1;
    a.split = plan && split_plan(f.H, f.lay.n_seq, f.lay.cutP, f.cu != nullptr);
    a.Pc = plan ? f.lay.cutP : 0;
    a.cut_seq = reinterpret_cast<int32_t *>(f.ws + f.lay.off_cut);
    a.cut_off = a.cut_seq + (kPlanCUs + 1);
    a.cut_first = a.cut_off + (kPlanCUs + 1);
    a.seq_start = reinterpret_cast<int64_t *>(f.ws + f.lay.off_seq_start);
    a.seq_len = reinterpret_cast<int64_t *>(f.ws + f.lay.off_seq_len);
    a.seq_off = reinterpret_cast<int64_t *>(f.ws + f.lay.off_seq_off);
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
}

// marks[0..3] (optional, may be NULL): recorded after the first forward launch, after the
// scan, after the last forward launch (a single whole-chain launch records all three
// after it), so the caller can time each launch.
hipError_t launch_forward(const FwdArgs &f, hipStream_t s, hipEvent_t const *marks)
{
    auto mark = [&](int i) { return marks == nullptr ? hipSuccess : hipEventRecord(marks[i], s); };
    const int64_t chains = f.lay.n_seq * f.H;
    if (chains == 0) {
        hipError_t e0;
        if ((e0 = mark(0)) != hipSuccess || (e0 = mark(1)) != hipSuccess)
            return e0;
        return mark(2);
    }
    FusedArgs a;
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
    a.wg_first = reinterpret_cast<const int64_t *>(f.ws + f.lay.off_wg);
    a.units = reinterpret_cast<const int32_t *>(f.ws + f.lay.off_units);
    a.status = reinterpret_cast<int32_t *>(f.ws + f.lay.off_status);
    a.Pc = (int)f.lay.cutP;
    a.cut_seq = reinterpret_cast<const int32_t *>(f.ws + f.lay.off_cut);
    a.cut_off = a.cut_seq + (kPlanCUs + 1);
    a.cut_first = a.cut_off + (kPlanCUs + 1);
    const size_t slots = (size_t)f.H * (size_t)a.Pc;
    const size_t seg_floats = slots * kD * kD;
    a.segS = reinterpret_cast<float *>(f.ws + f.lay.off_seg);
    a.segF = a.segS + seg_floats;
    a.segP = a.segF + seg_floats;
    a.segZ = reinterpret_cast<int32_t *>(f.ws + f.lay.off_segaux);
    a.segD = a.segZ + slots;
    a.segNS = reinterpret_cast<float *>(a.segD + slots);
    a.segNF = a.segNS + 4 * slots;
    a.trunc = (f.flags & kL2In) && (f.flags & kSigIn);
    // separate instantiations read the activation switches (when any is off) and run column
    // halves (whole-chain launches where the chunk table may split sequences)
    const bool sw = f.flags != (kGateIn | kL2In | kSigIn);
    const bool halves = split_plan(f.H, f.lay.n_seq, a.Pc, f.cu != nullptr);
    void (*fused)(FusedArgs) =
        a.Pc > 1 ? (sw ? fused_kernel<true, kModeA> : fused_kernel<false, kModeA>)
        : halves ? (sw ? fused_kernel<true, kModeHalves> : fused_kernel<false, kModeHalves>)
                 : (sw ? fused_kernel<true, kModeWhole> : fused_kernel<false, kModeWhole>);
    void (*trans)(FusedArgs) = sw ? fused_kernel<true, kModeTrans> : fused_kernel<false, kModeTrans>;
    void (*passb)(FusedArgs) = sw ? fused_kernel<true, kModeB> : fused_kernel<false, kModeB>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(fused),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kFusedLds);
    if (e != hipSuccess)
        return e;
    if (a.Pc <= 1) {
        // whole chains: H x per_head workgroups, each running a run of sequences of one
        // head back to back (about one workgroup per CU; runs from the chunk table)
        a.pass = 0;
        const int64_t per_head = whole_chain_groups(f.H, f.lay.n_seq, f.cu != nullptr);
        hipLaunchKernelGGL(fused, dim3((unsigned)(f.H * per_head)), dim3(512), kFusedLds, s, a);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        if ((e = mark(0)) != hipSuccess || (e = mark(1)) != hipSuccess)
            return e;
        return mark(2);
    }
    // cut plan: pass A (the P runs of every head, with out, end-state norms), then the
    // transition runs of cuts 1 .. P-1 (their stopping bound reads the norms)
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void *>(trans), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 kFusedLds)) != hipSuccess ||
        (e = hipFuncSetAttribute(reinterpret_cast<const void *>(passb), hipFuncAttributeMaxDynamicSharedMemorySize,
                                 kFusedLds)) != hipSuccess)
        return e;
    a.pass = 1;
    hipLaunchKernelGGL(fused, dim3((unsigned)(f.H * a.Pc)), dim3(512), kFusedLds, s, a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    a.pass = 3;
    hipLaunchKernelGGL(trans, dim3((unsigned)(f.H * (a.Pc - 1))), dim3(512), kFusedLds, s, a);
    if ((e = hipGetLastError()) != hipSuccess || (e = mark(0)) != hipSuccess)
        return e;
    ScanArgs sa;
    sa.segS = a.segS;
    sa.segF = a.segF;
    sa.segP = a.segP;
    sa.segZ = a.segZ;
    sa.segD = a.segD;
    sa.cut_seq = a.cut_seq;
    sa.cut_off = a.cut_off;
    sa.Pc = a.Pc;
    sa.H = f.H;
    hipLaunchKernelGGL(seg_scan_kernel, dim3((unsigned)(f.H * (kD / 16))), dim3(256), 0, s, sa);
    if ((e = hipGetLastError()) != hipSuccess || (e = mark(1)) != hipSuccess)
        return e;
    a.pass = 2;
    hipLaunchKernelGGL(passb, dim3((unsigned)(f.H * (a.Pc - 1))), dim3(512), kFusedLds, s, a);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    return mark(2);
}

}  // namespace kda
