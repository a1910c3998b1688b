// kda_kernels.hip -- gfx950 kernels of the KDA chunked forward pass.
//
// Method: "MoonshotAI/FlashKDA" README, "Kernel API" table (arguments, layouts, K = V = 128)
// and "Using FlashKDA as an FLA backend" (in-kernel gate, l2norm and beta sigmoid, V-major
// state).  FlashKDA article index: 16-token chunks, Neumann-series inverse, base-2
// exponentials, lower_bound as the exponent-range guard.
//
// Three stages, each its own kernel:
//   chunk table  (integer)  sequences -> chunk offsets, validity word
//   prep         one wavefront per (chunk, head), fully parallel: gate, cumulative
//                log-decay, l2norm, sigmoid, A_kk / A_qk on MFMA, Neumann inverse on fp32
//                MFMA, writes MFMA-ready operand blocks for the state stage
//   state        one wavefront per (sequence, head, 16 value columns), serial over the
//                chunks: Z = KG S^T, Y = QG S^T, V' = Tb (V - Z), O = Y + Mq (V - Z),
//                S <- S diag(gamma) + KD^T V', all on bf16 MFMA; the products that feed
//                the carried state (Z, V', the update, and A_kk in prep) use a hi/lo bf16
//                split (three products), the output-only ones (Y, Mq X, A_qk) one.
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
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoidf_fast(float x) { return frcp(1.0f + fexp2(-x * kLog2e)); }

// v_mfma_f32_16x16x32_bf16: A[m][k] in lane m + 16*(k/8), element k%8; B[k][n] in lane
// n + 16*(k/8), element k%8; D[m][n] in lane n + 16*(m/4), element m%4.
__device__ __forceinline__ f32x4_t mfma32(u32x4_t a, u32x4_t b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
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
    int32_t *status;
    int64_t *n_total;
    int64_t *seq_start, *seq_len, *seq_off;
};

__global__ __launch_bounds__(256) void chunk_table_kernel(TableArgs a)
{
    __shared__ int s_bad;
    __shared__ int64_t s_scan[256];
    __shared__ int64_t s_carry;
    const int tid = threadIdx.x;
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
// Stage 2: prep.  One wavefront per (chunk slot, head); 4 wavefronts per workgroup.
// Lane L works on token r = L % 16 of the chunk and channels 32*(L/16) .. +31.
// ---------------------------------------------------------------------------------------
struct PrepArgs {
    const uint16_t *q, *k, *g, *beta;
    const float *A_log, *dt_bias;
    float scale, lower_bound;
    int64_t H, N, n_slots;
    const int64_t *n_total, *seq_start, *seq_len, *seq_off;
    unsigned char *recs;
};

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
__device__ __forceinline__ float dpp_row_last(float x)
{
    int v = __builtin_bit_cast(int, x);
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0x15f, 0xf, 0xf, false));
}

__global__ __launch_bounds__(256) void prep_kernel(PrepArgs a)
{
    __shared__ float s_tile[4][256];
    __shared__ uint16_t s_kd[4][2][kD * kCH];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;
    const int64_t slot = item / a.H;
    const int h = (int)(item % a.H);
    if (slot >= a.n_slots)
        return;
    const int64_t n_total = *a.n_total;
    if (slot >= n_total)
        return;

    // sequence owning this chunk: the largest n with seq_off[n] <= slot
    int64_t lo = 0, hi = a.N;
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (a.seq_off[mid] <= slot)
            lo = mid;
        else
            hi = mid;
    }
    const int64_t n = lo;
    const int64_t j = slot - a.seq_off[n];
    const int64_t t0 = a.seq_start[n] + j * kCH;
    const int64_t rem = a.seq_len[n] - j * kCH;
    const int tlen = rem < kCH ? (int)rem : kCH;

    const int r = lane & 15;   // token within the chunk
    const int qb = lane >> 4;  // channel block: channels 32*qb .. 32*qb+31
    const bool valid = r < tlen;
    const int64_t H = a.H;

    float qf[32], kf[32], gf[32];
    if (valid) {
        const int64_t row = ((t0 + r) * H + h) * kD + 32 * qb;
        const u32x4_t *qp = reinterpret_cast<const u32x4_t *>(a.q + row);
        const u32x4_t *kp = reinterpret_cast<const u32x4_t *>(a.k + row);
        const u32x4_t *gp = reinterpret_cast<const u32x4_t *>(a.g + row);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            u32x4_t uq = qp[w], uk = kp[w], ug = gp[w];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qf[8 * w + 2 * e] = bf_lo(uq[e]);
                qf[8 * w + 2 * e + 1] = bf_hi(uq[e]);
                kf[8 * w + 2 * e] = bf_lo(uk[e]);
                kf[8 * w + 2 * e + 1] = bf_hi(uk[e]);
                gf[8 * w + 2 * e] = bf_lo(ug[e]);
                gf[8 * w + 2 * e + 1] = bf_hi(ug[e]);
            }
        }
    } else {
#pragma unroll
        for (int c = 0; c < 32; ++c) {
            qf[c] = 0.f;
            kf[c] = 0.f;
            gf[c] = 0.f;
        }
    }
    const float bt = valid ? sigmoidf_fast(bf16f(a.beta[(t0 + r) * H + h])) : 0.f;

    // l2 norms over the token's 128 channels (4 lanes share a token)
    float ssq = 0.f, ssk = 0.f;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        ssq = fmaf(qf[c], qf[c], ssq);
        ssk = fmaf(kf[c], kf[c], ssk);
    }
    ssq += __shfl_xor(ssq, 16);
    ssq += __shfl_xor(ssq, 32);
    ssk += __shfl_xor(ssk, 16);
    ssk += __shfl_xor(ssk, 32);
    const float rq = __builtin_amdgcn_rsqf(ssq + 1e-6f) * a.scale;
    const float rk = __builtin_amdgcn_rsqf(ssk + 1e-6f);

    // gate: log2-domain log-decay a2 = lb*log2e * sigmoid(exp(A_log) * (g + dt_bias)),
    // then the inclusive cumulative sum over the chunk's tokens (lanes of a row).
    const float c1 = fexp2(a.A_log[h] * kLog2e);
    const float lb2 = a.lower_bound * kLog2e;
    const f32x4_t *dtp = reinterpret_cast<const f32x4_t *>(a.dt_bias + (int64_t)h * kD + 32 * qb);
    float b2[32];
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        const f32x4_t dt = dtp[w];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = 4 * w + e;
            float x = c1 * (gf[c] + dt[e]);
            float av = valid ? lb2 * sigmoidf_fast(x) : 0.f;
            av += dpp_row_shr(av, 1);
            av += dpp_row_shr(av, 2);
            av += dpp_row_shr(av, 4);
            av += dpp_row_shr(av, 8);
            b2[c] = av;
        }
    }

    // decay-weighted operands (bl = b at the chunk's last token, broadcast along the row)
    //   KG = k^ Gamma, QG = scale q^ Gamma          (state stage, with S at chunk start)
    //   KD = k^ gamma / Gamma                        (state update)
    //   KE = k^ Gamma / gamma, QE = scale q^ Gamma / gamma  (A_kk = KE KD^T, A_qk = QE KD^T)
    float KG[32], QG[32], KD[32], KE[32], QE[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        const float bl = dpp_row_last(b2[c]);
        const float G = fexp2(b2[c]);
        const float E = fexp2(b2[c] - bl);
        const float Dk = fexp2(bl - b2[c]);
        const float kn = kf[c] * rk;
        const float qn = qf[c] * rq;
        KG[c] = kn * G;
        QG[c] = qn * G;
        KD[c] = kn * Dk;
        KE[c] = kn * E;
        QE[c] = qn * E;
    }
    // MFMA operands for the intra-chunk matrices: step s contracts channels
    // 32*qb + 8s .. +7 of this lane's token (the same k-slot mapping for A and B).
    // A_kk feeds the inverse and through it the carried state, so it takes three bf16
    // products (hi*hi + lo*hi + hi*lo); A_qk only feeds the output and takes one.
    u32x4_t keb[4], kel[4], qeb[4], kdb[4], kdlo[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c0 = 8 * s + 2 * e;
            const u32x2_t ke = split_bf16x2(KE[c0], KE[c0 + 1]);
            keb[s][e] = ke[0];
            kel[s][e] = ke[1];
            const u32x2_t kd = split_bf16x2(KD[c0], KD[c0 + 1]);
            kdb[s][e] = kd[0];
            kdlo[s][e] = kd[1];
            qeb[s][e] = pack_bf16x2(QE[c0], QE[c0 + 1]);
        }
    }

    f32x4_t akk = {0.f, 0.f, 0.f, 0.f}, aqkT = akk;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        akk = mfma32(keb[s], kdb[s], akk);
        akk = mfma32(kel[s], kdb[s], akk);
        akk = mfma32(keb[s], kdlo[s], akk);
        aqkT = mfma32(kdb[s], qeb[s], aqkT);
    }

    // masks; D layout: element i of lane L is row 4*(L/16)+i, column L%16
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

    // Neumann product (I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8), fp32
    float *tile = s_tile[wave];
    const f32x4_t AT = transpose16(A, tile, lane);
    const f32x4_t P2 = mm16(AT, A);
    const f32x4_t P2T = transpose16(P2, tile, lane);
    const f32x4_t P4 = mm16(P2T, P2);
    const f32x4_t P4T = transpose16(P4, tile, lane);
    const f32x4_t P8 = mm16(P4T, P4);
    const f32x4_t R1 = mm16(I4 + P4T, I4 + P8);
    const f32x4_t R2 = mm16(I4 + P2T, R1);
    const f32x4_t Tm = mm16(I4 - AT, R2);
    const f32x4_t Tb = Tm * bt;              // column s scaled by beta_s (own token)
    const f32x4_t Mq = mm16(AqT, Tb);        // A_qk T diag(beta)
    const f32x4_t TbT = transpose16(Tb, tile, lane);
    const f32x4_t MqT = transpose16(Mq, tile, lane);

    // ---- write the record ----
    unsigned char *rec = a.recs + ((size_t)slot * (size_t)H + (size_t)h) * kRecBytes;
    // KG (hi, lo) / QG: record [pair qb][lane r + 16*gg] = channels (4gg..+3, 16+4gg..+3)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
        u32x4_t wk, wl, wq;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c0 = (e < 2 ? 4 * gg : 16 + 4 * gg) + 2 * (e & 1);
            const u32x2_t t2 = split_bf16x2(KG[c0], KG[c0 + 1]);
            wk[e] = t2[0];
            wl[e] = t2[1];
        }
        wq[0] = pack_bf16x2(QG[4 * gg], QG[4 * gg + 1]);
        wq[1] = pack_bf16x2(QG[4 * gg + 2], QG[4 * gg + 3]);
        wq[2] = pack_bf16x2(QG[16 + 4 * gg], QG[16 + 4 * gg + 1]);
        wq[3] = pack_bf16x2(QG[16 + 4 * gg + 2], QG[16 + 4 * gg + 3]);
        const size_t o = (size_t)(qb * 64 + r + 16 * gg) * 16;
        *reinterpret_cast<u32x4_t *>(rec + kRecKG + o) = wk;
        *reinterpret_cast<u32x4_t *>(rec + kRecKGL + o) = wl;
        *reinterpret_cast<u32x4_t *>(rec + kRecQG + o) = wq;
    }
    // KD through LDS: [channel][token] hi and lo, then records [tile][lane][hi4, lo4]
    uint16_t *kdh = s_kd[wave][0];
    uint16_t *kdl = s_kd[wave][1];
    lds_sync_wave();
#pragma unroll
    for (int c = 0; c < 32; ++c) {
        const uint16_t hb = to_bf16(KD[c]);
        const float hf = bf16f(hb);
        kdh[(32 * qb + c) * kCH + r] = hb;
        kdl[(32 * qb + c) * kCH + r] = to_bf16(KD[c] - hf);
    }
    lds_sync_wave();
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
        const int ch = 16 * ct + col;
        const u32x2_t h2 = *reinterpret_cast<const u32x2_t *>(kdh + ch * kCH + g4);
        const u32x2_t l2 = *reinterpret_cast<const u32x2_t *>(kdl + ch * kCH + g4);
        u32x4_t w = {h2[0], h2[1], l2[0], l2[1]};
        *reinterpret_cast<u32x4_t *>(rec + kRecKD + (size_t)(ct * 64 + lane) * 16) = w;
    }
    // gamma: Gamma at the last token; the row's lane 15 holds it (padding adds no decay)
    if (r == 15) {
        f32x4_t *gp = reinterpret_cast<f32x4_t *>(rec + kRecGAM + (size_t)(32 * qb) * 4);
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            f32x4_t gv = {fexp2(b2[4 * w]), fexp2(b2[4 * w + 1]), fexp2(b2[4 * w + 2]),
                          fexp2(b2[4 * w + 3])};
            gp[w] = gv;
        }
    }
    // Tb and Mq: lane L holds X[L%16][4g..4g+3] (from the transposes), hi and lo
    {
        u32x4_t w;
        const float h0 = bf16f(to_bf16(TbT[0])), h1 = bf16f(to_bf16(TbT[1]));
        const float h2 = bf16f(to_bf16(TbT[2])), h3 = bf16f(to_bf16(TbT[3]));
        w[0] = pack_bf16x2(TbT[0], TbT[1]);
        w[1] = pack_bf16x2(TbT[2], TbT[3]);
        w[2] = pack_bf16x2(TbT[0] - h0, TbT[1] - h1);
        w[3] = pack_bf16x2(TbT[2] - h2, TbT[3] - h3);
        *reinterpret_cast<u32x4_t *>(rec + kRecTB + (size_t)lane * 16) = w;
        const float m0 = bf16f(to_bf16(MqT[0])), m1 = bf16f(to_bf16(MqT[1]));
        const float m2 = bf16f(to_bf16(MqT[2])), m3 = bf16f(to_bf16(MqT[3]));
        u32x4_t m;
        m[0] = pack_bf16x2(MqT[0], MqT[1]);
        m[1] = pack_bf16x2(MqT[2], MqT[3]);
        m[2] = pack_bf16x2(MqT[0] - m0, MqT[1] - m1);
        m[3] = pack_bf16x2(MqT[2] - m2, MqT[3] - m3);
        *reinterpret_cast<u32x4_t *>(rec + kRecMQ + (size_t)lane * 16) = m;
    }
}

// ---------------------------------------------------------------------------------------
// Stage 3: state propagation and output.  One wavefront per (sequence, head, value block).
// Lane L owns value column v = 16*vb + L%16 and, for each channel tile ct, the state
// entries S[v][16ct + 4*(L/16) + i], i = 0..3 (S^T in the MFMA D layout).
// ---------------------------------------------------------------------------------------
struct StateArgs {
    const uint16_t *v;
    uint16_t *out;
    const void *h0;
    void *ht;
    int h0_dtype, ht_dtype;
    int64_t H, N;
    const int64_t *seq_start, *seq_len, *seq_off;
    const unsigned char *recs;
};

// The state stage splits each (chain, 16-column value block) over 4 wavefronts of one
// workgroup: wavefront w owns channels 32w .. 32w+31 of the state (channel tiles 2w, 2w+1).
// Z = KG S^T and Y = QG S^T are summed over the 4 channel quarters through LDS (one
// barrier per chunk); every wavefront then forms X = V - Z and V' itself and updates its
// own quarter.  Each wavefront streams the slice of the per-chunk record it reads into a
// private LDS ring, kRing chunks ahead, with direct global->LDS loads.
constexpr int kRing = 4;
constexpr int kSlot = 8192;          // bytes of one wavefront's ring slot
constexpr int kSlotKG = 0, kSlotKGL = 1024, kSlotQG = 2048, kSlotKD = 3072;  // KD: 2 tiles
constexpr int kSlotTB = 5120, kSlotMQ = 6144, kSlotGAM = 7168, kSlotV = 7424;  // GAM 256 B, V 512 B
constexpr int kDmaPerChunk = 10;     // direct-to-LDS load instructions issued per chunk per wave

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

// Issue the direct-to-LDS loads of one chunk's operand slice for wavefront w (exactly
// kDmaPerChunk load instructions, all lanes active, every address inside its buffer).
// Buffer descriptor over [base, base + bytes): loads past the end return zeros without
// touching memory.  Word 3 = raw (untyped) buffer access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// lane offsets used by the ring loads, computed once per wavefront
struct DmaLane {
    uint32_t o16;   // lane * 16
    uint32_t ogm;   // (lane % 32) * 4
    uint32_t ov[2]; // value row 8i + lane/8, dword lane % 8
};

__device__ __forceinline__ void dma_chunk(unsigned char *slot, const unsigned char *rec,
                                          const uint16_t *vrow0, uint32_t vrow_bytes, int tlen,
                                          int w, const DmaLane &dl)
{
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, (uint32_t)kRecBytes);
    // Scalar offsets of the blocks this wavefront reads, kept opaque to constant folding:
    // folding several of them into one descriptor's loads crashes instruction selection.
    const int sKG = __builtin_amdgcn_readfirstlane(kRecKG + w * 1024);
    const int sKGL = __builtin_amdgcn_readfirstlane(kRecKGL + w * 1024);
    const int sQG = __builtin_amdgcn_readfirstlane(kRecQG + w * 1024);
    const int sKD0 = __builtin_amdgcn_readfirstlane(kRecKD + 2 * w * 1024);
    const int sKD1 = __builtin_amdgcn_readfirstlane(kRecKD + (2 * w + 1) * 1024);
    const int sTB = __builtin_amdgcn_readfirstlane((int)kRecTB);
    const int sMQ = __builtin_amdgcn_readfirstlane((int)kRecMQ);
    const int sGM = __builtin_amdgcn_readfirstlane(kRecGAM + 128 * w);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(slot + kSlotKG), 16, dl.o16, sKG, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(slot + kSlotKGL), 16, dl.o16, sKGL, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(slot + kSlotQG), 16, dl.o16, sQG, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(slot + kSlotKD), 16, dl.o16, sKD0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(slot + kSlotKD + 1024), 16, dl.o16, sKD1, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(slot + kSlotTB), 16, dl.o16, sTB, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(slot + kSlotMQ), 16, dl.o16, sMQ, 0, 0);
    // gamma of channels 32w .. 32w+31 (lanes 32..63 load a second copy)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void *)(slot + kSlotGAM), 4, dl.ogm, sGM, 0, 0);
    // values: token row t = 8i + L/8 holds 16 bf16 = 8 dwords (direct-to-LDS loads write one
    // dword per lane).  The descriptor ends after the chunk's last token, so rows past the
    // end of a partial chunk load zeros.
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vrow0, (uint32_t)(tlen - 1) * vrow_bytes + 32u);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(slot + kSlotV), 4, dl.ov[0], 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(slot + kSlotV + 256), 4, dl.ov[1], 0, 0, 0);
}

__global__ __launch_bounds__(256) void state_kernel(StateArgs a)
{
    extern __shared__ __attribute__((aligned(16))) unsigned char s_state[];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: keep it scalar
    // Workgroups are dealt round-robin to the 8 XCDs (workgroup i -> XCD i % 8); place the
    // kNVB value blocks of one chain on the same XCD so that they share its L2 copy of the
    // chain's prep records.
    const int64_t item = blockIdx.x;
    const int64_t xcd = item & 7;
    const int64_t jj = item >> 3;
    const int vb = (int)(jj % kNVB);
    const int64_t chain = (jj / kNVB) * 8 + xcd;
    const int64_t n = chain / a.H;
    const int h = (int)(chain % a.H);
    if (n >= a.N)
        return;  // whole workgroup
    const int64_t H = a.H;
    const int g = lane >> 4;
    const int col = lane & 15;
    const int v = vb * kVB + col;

    unsigned char *ring = s_state + (size_t)w * kRing * kSlot;
    float *part = reinterpret_cast<float *>(s_state + 4 * kRing * kSlot);  // [2][4 waves][Z,Y][64][4]

    f32x4_t S[2];
    const int64_t sbase = ((n * H + h) * kD + v) * kD + 4 * g + 32 * w;
    if (a.h0_dtype == 2) {
        const float *p = reinterpret_cast<const float *>(a.h0) + sbase;
        S[0] = *reinterpret_cast<const f32x4_t *>(p);
        S[1] = *reinterpret_cast<const f32x4_t *>(p + 16);
    } else if (a.h0_dtype == 1) {
        const uint16_t *p = reinterpret_cast<const uint16_t *>(a.h0) + sbase;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u32x2_t u = *reinterpret_cast<const u32x2_t *>(p + 16 * t);
            S[t] = f32x4_t{bf_lo(u[0]), bf_hi(u[0]), bf_lo(u[1]), bf_hi(u[1])};
        }
    } else {
        S[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        S[1] = S[0];
    }

    const int64_t len = a.seq_len[n];
    const int64_t start = a.seq_start[n];
    const int64_t off = a.seq_off[n];
    const int64_t nch = (len + kCH - 1) / kCH;
    const int64_t vstride = H * kD;
    auto rec_of = [&](int64_t j) {
        return a.recs + ((size_t)(off + j) * (size_t)H + (size_t)h) * kRecBytes;
    };
    auto tlen_of = [&](int64_t j) {
        const int64_t rem = len - j * kCH;
        return rem < kCH ? (int)rem : kCH;
    };
    auto vrow_of = [&](int64_t j) { return a.v + ((start + j * kCH) * H + h) * kD + vb * kVB; };

    DmaLane dl;
    dl.o16 = (uint32_t)lane * 16u;
    dl.ogm = (uint32_t)(lane & 31) * 4u;
    const uint32_t vrow_bytes = (uint32_t)(vstride * 2);
    dl.ov[0] = (uint32_t)(lane >> 3) * vrow_bytes + (uint32_t)(lane & 7) * 4u;
    dl.ov[1] = dl.ov[0] + 8u * vrow_bytes;

    // prologue: chunks 0 .. kRing-2 in flight
#pragma unroll
    for (int jp = 0; jp < kRing - 1; ++jp)
        if (jp < nch)
            dma_chunk(ring + jp * kSlot, rec_of(jp), vrow_of(jp), vrow_bytes, tlen_of(jp), w, dl);

    // vmcnt bookkeeping.  Per chunk every wavefront issues exactly kDmaPerChunk ring loads
    // and, for every chunk but a partial last one, exactly one store of output.  The ring
    // loads of chunk j are complete once at most N later vector-memory operations are
    // outstanding, N counting only operations certainly issued after them: the ring loads
    // of the (up to kRing-2) later chunks already in flight, plus one output store when
    // waiting from inside the loop.
    auto ahead_of = [&](int64_t j) {
        return (nch - 1 - j) < (kRing - 2) ? (nch - 1 - j) : (int64_t)(kRing - 2);
    };
    auto wait_chunk = [&](int64_t j, bool after_store) {
        const int64_t ahead = ahead_of(j);
        if (ahead >= 2) {
            if (after_store)
                wait_vmcnt<2 * kDmaPerChunk + 1>();
            else
                wait_vmcnt<2 * kDmaPerChunk>();
        } else if (ahead == 1) {
            if (after_store)
                wait_vmcnt<kDmaPerChunk + 1>();
            else
                wait_vmcnt<kDmaPerChunk>();
        } else {
            wait_vmcnt<0>();
        }
    };

    u32x4_t kg = {0u, 0u, 0u, 0u}, kgl = kg, qg = kg;
    if (nch > 0) {
        wait_chunk(0, false);
        kg = *reinterpret_cast<const u32x4_t *>(ring + kSlotKG + lane * 16);
        kgl = *reinterpret_cast<const u32x4_t *>(ring + kSlotKGL + lane * 16);
        qg = *reinterpret_cast<const u32x4_t *>(ring + kSlotQG + lane * 16);
    }
    for (int64_t j = 0; j < nch; ++j) {
        unsigned char *slot = ring + (j % kRing) * kSlot;
        const int tlen = tlen_of(j);

        // partial Z and Y over this wavefront's 32 channels
        u32x4_t sb, sl;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const u32x2_t t0 = split_bf16x2(S[0][2 * e], S[0][2 * e + 1]);
            const u32x2_t t1 = split_bf16x2(S[1][2 * e], S[1][2 * e + 1]);
            sb[e] = t0[0];
            sl[e] = t0[1];
            sb[2 + e] = t1[0];
            sl[2 + e] = t1[1];
        }
        f32x4_t Zp = {0.f, 0.f, 0.f, 0.f}, Yp = Zp;
        Zp = mfma32(kg, sb, Zp);
        Zp = mfma32(kgl, sb, Zp);
        Zp = mfma32(kg, sl, Zp);
        Yp = mfma32(qg, sb, Yp);
        float *pb = part + (size_t)(j & 1) * (4 * 2 * 64 * 4);
        *reinterpret_cast<f32x4_t *>(pb + ((w * 2 + 0) * 64 + lane) * 4) = Zp;
        *reinterpret_cast<f32x4_t *>(pb + ((w * 2 + 1) * 64 + lane) * 4) = Yp;
        // Barrier for the partials only: they are plain LDS stores, complete once
        // lgkmcnt reaches 0.  The ring loads (vmcnt) stay in flight across it.
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();

        // the rest of this chunk's operands, and the partials of all four quarters
        const uint16_t *vs = reinterpret_cast<const uint16_t *>(slot + kSlotV);  // [token][16]
        const u32x4_t tb = *reinterpret_cast<const u32x4_t *>(slot + kSlotTB + lane * 16);
        const float *gs = reinterpret_cast<const float *>(slot + kSlotGAM);
        const f32x4_t gm0 = *reinterpret_cast<const f32x4_t *>(gs + 4 * g);
        const f32x4_t gm1 = *reinterpret_cast<const f32x4_t *>(gs + 16 + 4 * g);
        const u32x4_t kd0 = *reinterpret_cast<const u32x4_t *>(slot + kSlotKD + lane * 16);
        const u32x4_t kd1 = *reinterpret_cast<const u32x4_t *>(slot + kSlotKD + 1024 + lane * 16);
        f32x4_t Z = *reinterpret_cast<const f32x4_t *>(pb + ((0 * 2 + 0) * 64 + lane) * 4);
#pragma unroll
        for (int q = 1; q < 4; ++q)
            Z += *reinterpret_cast<const f32x4_t *>(pb + ((q * 2 + 0) * 64 + lane) * 4);
        // X = V - Z (rows = tokens 4g+i of this lane's column), split hi/lo
        float vv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vv[i] = bf16f(vs[(4 * g + i) * kVB + col]);
        f32x4_t X;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            X[i] = (4 * g + i < tlen ? vv[i] : 0.f) - Z[i];  // rows past the end hold stale data
        const u32x2_t x01 = split_bf16x2(X[0], X[1]);
        const u32x2_t x23 = split_bf16x2(X[2], X[3]);
        const u32x4_t xhh = {x01[0], x23[0], x01[0], x23[0]};
        // V' = Tb X, three bf16 products as two K-concatenated steps:
        //   [Tb_hi | Tb_lo] [X_hi ; X_hi]  +  [Tb_hi | Tb_hi] [X_lo ; 0]
        // Every accumulation chain uses a single MFMA opcode.
        f32x4_t Vp = {0.f, 0.f, 0.f, 0.f};
        Vp = mfma32(tb, xhh, Vp);
        Vp = mfma32(u32x4_t{tb[0], tb[1], tb[0], tb[1]}, u32x4_t{x01[1], x23[1], 0u, 0u}, Vp);
        const u32x2_t v01 = split_bf16x2(Vp[0], Vp[1]);
        const u32x2_t v23 = split_bf16x2(Vp[2], Vp[3]);
        const u32x4_t vhh = {v01[0], v23[0], v01[0], v23[0]};
        const u32x4_t vl0 = {v01[1], v23[1], 0u, 0u};
        // S <- S diag(gamma) + KD^T V':  [KD_hi | KD_lo] [V'_hi ; V'_hi] + [KD_hi | KD_hi] [V'_lo ; 0]
        {
            f32x4_t s0 = S[0] * gm0, s1 = S[1] * gm1;
            s0 = mfma32(kd0, vhh, s0);
            s1 = mfma32(kd1, vhh, s1);
            s0 = mfma32(u32x4_t{kd0[0], kd0[1], kd0[0], kd0[1]}, vl0, s0);
            s1 = mfma32(u32x4_t{kd1[0], kd1[1], kd1[0], kd1[1]}, vl0, s1);
            S[0] = s0;
            S[1] = s1;
        }
        // O = Y + (A_qk Tb) X_hi  with  [Mq_hi | Mq_lo] [X_hi ; X_hi].  Every wavefront forms
        // it (one MFMA) and stores one of the four token rows it holds: row 4g + w.
        {
            f32x4_t Y = *reinterpret_cast<const f32x4_t *>(pb + ((0 * 2 + 1) * 64 + lane) * 4);
#pragma unroll
            for (int q = 1; q < 4; ++q)
                Y += *reinterpret_cast<const f32x4_t *>(pb + ((q * 2 + 1) * 64 + lane) * 4);
            const u32x4_t mq = *reinterpret_cast<const u32x4_t *>(slot + kSlotMQ + lane * 16);
            const f32x4_t O = mfma32(mq, xhh, Y);
            const float ow = w == 0 ? O[0] : w == 1 ? O[1] : w == 2 ? O[2] : O[3];
            const int rr = 4 * g + w;
            if (rr < tlen)
                a.out[((start + j * kCH + rr) * H + h) * kD + v] = to_bf16(ow);
        }

        // every wavefront has finished chunk j-1 (barrier above): refill its ring slot
        if (j + kRing - 1 < nch) {
            const int64_t jn = j + kRing - 1;
            dma_chunk(ring + (jn % kRing) * kSlot, rec_of(jn), vrow_of(jn), vrow_bytes, tlen_of(jn), w, dl);
        }
        // first operands of the next chunk
        if (j + 1 < nch) {
            wait_chunk(j + 1, true);
            unsigned char *ns = ring + ((j + 1) % kRing) * kSlot;
            kg = *reinterpret_cast<const u32x4_t *>(ns + kSlotKG + lane * 16);
            kgl = *reinterpret_cast<const u32x4_t *>(ns + kSlotKGL + lane * 16);
            qg = *reinterpret_cast<const u32x4_t *>(ns + kSlotQG + lane * 16);
        }
    }

    if (a.ht_dtype == 2) {
        float *p = reinterpret_cast<float *>(a.ht) + sbase;
        *reinterpret_cast<f32x4_t *>(p) = S[0];
        *reinterpret_cast<f32x4_t *>(p + 16) = S[1];
    } else if (a.ht_dtype == 1) {
        uint16_t *p = reinterpret_cast<uint16_t *>(a.ht) + sbase;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            u32x2_t u = {pack_bf16x2(S[t][0], S[t][1]), pack_bf16x2(S[t][2], S[t][3])};
            *reinterpret_cast<u32x2_t *>(p + 16 * t) = u;
        }
    }
}

// ---------------------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------------------
hipError_t launch_chunk_table(const FwdArgs &f, hipStream_t s)
{
    TableArgs a;
    a.cu = f.cu;
    a.B = f.B;
    a.T = f.T;
    a.N = f.lay.n_seq;
    a.status = reinterpret_cast<int32_t *>(f.ws + f.lay.off_status);
    a.n_total = reinterpret_cast<int64_t *>(f.ws + f.lay.off_status + 8);
    a.seq_start = reinterpret_cast<int64_t *>(f.ws + f.lay.off_seq_start);
    a.seq_len = reinterpret_cast<int64_t *>(f.ws + f.lay.off_seq_len);
    a.seq_off = reinterpret_cast<int64_t *>(f.ws + f.lay.off_seq_off);
    hipLaunchKernelGGL(chunk_table_kernel, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_prep(const FwdArgs &f, hipStream_t s)
{
    const int64_t waves = f.lay.n_slots * f.H;
    if (waves == 0)
        return hipSuccess;
    PrepArgs a;
    a.q = f.q;
    a.k = f.k;
    a.g = f.g;
    a.beta = f.beta;
    a.A_log = f.A_log;
    a.dt_bias = f.dt_bias;
    a.scale = f.scale;
    a.lower_bound = f.lower_bound;
    a.H = f.H;
    a.N = f.lay.n_seq;
    a.n_slots = f.lay.n_slots;
    a.n_total = reinterpret_cast<const int64_t *>(f.ws + f.lay.off_status + 8);
    a.seq_start = reinterpret_cast<const int64_t *>(f.ws + f.lay.off_seq_start);
    a.seq_len = reinterpret_cast<const int64_t *>(f.ws + f.lay.off_seq_len);
    a.seq_off = reinterpret_cast<const int64_t *>(f.ws + f.lay.off_seq_off);
    a.recs = f.ws + f.lay.off_recs;
    const int64_t blocks = cdiv(waves, 4);
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_state(const FwdArgs &f, hipStream_t s)
{
    StateArgs a;
    a.v = f.v;
    a.out = f.out;
    a.h0 = f.h0;
    a.ht = f.ht;
    a.h0_dtype = f.h0_dtype;
    a.ht_dtype = f.ht_dtype;
    a.H = f.H;
    a.N = f.lay.n_seq;
    a.seq_start = reinterpret_cast<const int64_t *>(f.ws + f.lay.off_seq_start);
    a.seq_len = reinterpret_cast<const int64_t *>(f.ws + f.lay.off_seq_len);
    a.seq_off = reinterpret_cast<const int64_t *>(f.ws + f.lay.off_seq_off);
    a.recs = f.ws + f.lay.off_recs;
    const int64_t chains = f.lay.n_seq * f.H;
    const int64_t blocks = cdiv(chains, 8) * 8 * kNVB;
    const size_t lds = (size_t)4 * kRing * kSlot + 2 * 4 * 2 * 64 * 16;
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&state_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(state_kernel, dim3((unsigned)blocks), dim3(256), lds, s, a);
    return hipGetLastError();
}

}  // namespace kda
