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
// Then the activations' chain rules.  All arithmetic is fp32; products on the fp32 MFMA, except
// the two chains' products and the gradient kernel's products with the states, which are
// three-term bf16 products (hi hi + lo hi + hi lo, about 16 significant bits per factor, fp32
// accumulation), as in the forward chunk recurrence.
//
// Kernels, in launch order (the chunk table comes first, as in the forward pass):
//   bwd_chunk_info_kernel
//                      per chunk: where it lies (first token, sequence, length, which state the
//                      chain does not store), one record read by the ops and gradient kernels
//   bwd_piece_table_kernel (cut plan only)
//                      the first piece of every sequence
//   bwd_ops_kernel     per chunk-head: the chunk's activated rows (l2norm, gate, sigmoid, as
//                      in the forward pass) and its operands for the two chains (-W, U, KD
//                      row-major, QG^T, lower(QG KI^T), gamma; the chain kernel forms KD^T, -W^T
//                      and U~ = lower(QG KI^T)^T dO itself)
//   bwd_chain_kernel   per (sequence, head, role, half of the value rows): role 0 runs the
//                      state forwards over the chunks, writing V' of every chunk and S0 of the
//                      even chunks of the sequence; role 1 runs dL/dS backwards, writing dV' of
//                      every chunk, D of the odd chunks and dL/dS_0.  The value rows of a state
//                      are independent given the chunk operands, so two workgroups take 64
//                      rows each.  Where the sequences are few and long, the cut plan
//                      (kda_internal.h) runs it per piece instead: pass A, transition runs,
//                      bwd_piece_scan_kernel, pass B.
//   bwd_grad_kernel    per chunk-head: the state the chain did not store, rebuilt from the
//                      neighbouring chunk's (D of an even chunk from the next chunk's by the
//                      dS0 step above, S0 of an odd one from the previous chunk's by the state
//                      step), the products with the chunk's states (dKD, dO S0,
//                      dV' S0, dgamma) and dAqk, the gradients of the chunk's tokens (dq^, dk^,
//                      d log-decay, dbeta, dv), then the l2norm, gate and sigmoid chain rules
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
constexpr int kP = kD;             // LDS row stride of the [16][128] fp32 tiles (unpadded: the
                                   // ops kernel then fits three workgroups per CU)
constexpr int kQ = kCH + 1;        // LDS row stride of the 16 x 16 tiles
constexpr int kQ4 = kCH + 4;       // the same, rows 16-byte aligned
constexpr int kGradThreads = 512;  // bwd_ops_kernel, bwd_grad_kernel
constexpr int kChainThreads = 256; // bwd_chain_kernel: 4 wavefronts of 16 value rows
// operand block of a chunk-head (kBwdOps floats)
constexpr int kOpNegW = 0, kOpU = 2048, kOpKD = 4096, kOpQGt = 6144, kOpAqk = 8192, kOpGam = 8448;
static_assert(kOpGam + kD == kBwdOps, "operand block layout");

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bbf16(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st4(float *p, f32x4 x) { *reinterpret_cast<f32x4 *>(p) = x; }
__device__ __forceinline__ void stu4(float *p, __attribute__((ext_vector_type(4))) uint32_t x)
{
    *reinterpret_cast<__attribute__((ext_vector_type(4))) uint32_t *>(p) = x;
}
__device__ __forceinline__ __attribute__((ext_vector_type(4))) uint32_t ldu4(const float *p)
{
    return *reinterpret_cast<const __attribute__((ext_vector_type(4))) uint32_t *>(p);
}
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
// Three-term bf16 products for the chain kernel (about 16 significant bits per factor, fp32
// accumulation; the chunk recurrence of the forward pass uses the same scheme).
// v_mfma_f32_16x16x16_bf16 takes the operands in the layout of mm4 above: lane L holds
// A[L % 16][4 (L / 16) + j] and B[4 (L / 16) + j][L % 16], j = 0..3, as four packed bf16.  A
// split operand is u32x4 {hi (two words), lo (two words)} with x ~ hi + lo.
typedef short bf16x4s __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b)  // round to nearest even
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ f32x4 mfma16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, f32x4 c)
{
    typedef uint32_t u32x2_ __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4s, u32x2_{a0, a1}),
                                                      __builtin_bit_cast(bf16x4s, u32x2_{b0, b1}), c, 0, 0, 0);
}
// c + A B: hi hi + lo hi + hi lo
__device__ __forceinline__ f32x4 mm3(u32x4 a, u32x4 b, f32x4 c)
{
    c = mfma16(a[0], a[1], b[0], b[1], c);
    c = mfma16(a[2], a[3], b[0], b[1], c);
    return mfma16(a[0], a[1], b[2], b[3], c);
}
// c + A B for a B that is exactly bf16 (b: one word pair): hi B + lo B
__device__ __forceinline__ f32x4 mm2(u32x4 a, uint32_t b0, uint32_t b1, f32x4 c)
{
    c = mfma16(a[0], a[1], b0, b1, c);
    return mfma16(a[2], a[3], b0, b1, c);
}
// c + A B for an A that is exactly bf16 (a's hi words only): A hi + A lo
__device__ __forceinline__ f32x4 mm2a(u32x4 a, u32x4 b, f32x4 c)
{
    c = mfma16(a[0], a[1], b[0], b[1], c);
    return mfma16(a[0], a[1], b[2], b[3], c);
}
// {hi, lo} of four values on the VALU
__device__ __forceinline__ u32x4 split4(f32x4 x)
{
    const uint32_t h0 = pk_bf16(x[0], x[1]), h1 = pk_bf16(x[2], x[3]);
    return u32x4{h0, h1, pk_bf16(x[0] - __uint_as_float(h0 << 16), x[1] - __uint_as_float(h0 & 0xffff0000u)),
                 pk_bf16(x[2] - __uint_as_float(h1 << 16), x[3] - __uint_as_float(h1 & 0xffff0000u))};
}
// {hi, lo} of a tile in the D layout (which is also the B operand layout): lo from the MFMA as
// (-I) hi + x, exact in fp32; negI holds -1 (bf16) at A[m][m]: lane m + 16 (m / 4), element m % 4
__device__ __forceinline__ u32x4 split_tile(f32x4 x, uint32_t n0, uint32_t n1)
{
    const uint32_t h0 = pk_bf16(x[0], x[1]), h1 = pk_bf16(x[2], x[3]);
    const f32x4 r = mfma16(n0, n1, h0, h1, x);
    return u32x4{h0, h1, pk_bf16(r[0], r[1]), pk_bf16(r[2], r[3])};
}

// acc + A B^T for A, B [16][nk] row-major in LDS (row stride kP), one wavefront
__device__ __forceinline__ f32x4 mm_rows(const float *A, const float *B, int nk, f32x4 acc, int lane)
{
    const int m = lane & 15, g = lane >> 4;
    for (int t = 0; t < nk; t += 16)
        acc = mm4(ld4(A + m * kP + t + 4 * g), ld4(B + m * kP + t + 4 * g), acc);
    return acc;
}

// Layout of the per-chunk states and rows in the workspace, chosen so that every store of the
// chain kernel (a wave's 16 value rows, four channels per lane) writes 256 contiguous bytes and
// every read of the gradient kernel's state products (four value rows at one channel) is one
// 16-byte load:
//   state_at(v, c) = ((v / 16) 8 + c / 16) 256 + (c % 4) 64 + (c / 4 % 4) 16 + v % 16
//   rows_at(r, v)  = (v / 16) 256 + (r % 4) 64 + (r / 4) 16 + v % 16     (r: row of the chunk)
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
    const int32_t *status;   // the chunk table's status word (nonzero: invalid cu_seqlens)
    float *ops;              // [chunks][H][kBwdOps]
    float *ck;               // [chunks][H][16384]: S before the chunk (even chunks of a sequence)
                             // or dL/dS after it (odd chunks), state_at
    float *xf, *xb;          // [chunks][H][2048]: V' and dL/dV' (rows_at)
    float *hpart;            // [H][kHeadSlices][2][128]: head-gradient partial sums
    int32_t *cinfo;          // [chunks][4]: where each chunk lies (bwd_chunk_info_kernel)
    // cut plan (plen > 0): chunks per piece; per sequence the first piece index (pieces
    // counted over the sequences, the same for every head); per (piece, head, direction) the
    // start state, F and Phi (fp32, row-major [value row][channel]), the squared norms of F and
    // of the start state per part, and the chunks each part's transition run took (-1: all)
    int64_t plen;
    int trunc;               // transition runs may stop (in-kernel l2norm and beta sigmoid)
    int64_t *poff;           // [N + 1]
    float *pst;              // [pieces][H][2][3][16384]
    float *pnrm;             // [pieces][H][2][8]
    int32_t *pz;             // [pieces][H][2][4]
};

// ---- per-chunk operands (shared by bwd_ops_kernel and bwd_grad_kernel) ----
// Chunk x of a head's chunk list: sequence n (the first with seq_off[n + 1] > x), chunk j of
// it, first token t0 (row index), len tokens (1 .. 16); kind: which of its two states the
// chain does not store (1: S0, j odd; 0: D, j even and not the last chunk; 2: the last chunk
// with j even, D = dL/dS_final); next_len: the next chunk's tokens (kind 0).  Written once per
// call by bwd_chunk_info_kernel as four words per chunk, {t0 low, t0 high, n (-1 past the
// last chunk), len | kind << 8 | next_len << 16}, so that a workgroup learns it with one
// 16-byte load instead of a search over the sequences ahead of its first dependent loads.
struct ChunkLoc {
    int64_t n, t0;
    int len, kind, next_len;
};
__global__ __launch_bounds__(256) void bwd_chunk_info_kernel(BwdArgs a)
{
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= a.chunks)
        return;
    int32_t *rec = a.cinfo + 4 * x;
    if (x >= a.seq_off[a.N]) {
        rec[0] = rec[1] = rec[3] = 0;
        rec[2] = -1;
        return;
    }
    int64_t lo = 0, hi = a.N - 1;
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (a.seq_off[mid + 1] > x)
            hi = mid;
        else
            lo = mid + 1;
    }
    const int64_t j = x - a.seq_off[lo], t0 = a.seq_start[lo] + kCH * j, rem = a.seq_len[lo] - kCH * j;
    const int len = rem < kCH ? (int)rem : kCH;
    const int kind = (j & 1) ? 1 : (x + 1 < a.seq_off[lo + 1] ? 0 : 2);
    const int64_t nrem = rem - kCH;
    const int next = kind == 0 ? (nrem < kCH ? (int)nrem : kCH) : 0;
    rec[0] = (int32_t)(uint32_t)(uint64_t)t0;
    rec[1] = (int32_t)(uint32_t)((uint64_t)t0 >> 32);
    rec[2] = (int32_t)lo;
    rec[3] = len | (kind << 8) | (next << 16);
}
__device__ __forceinline__ bool locate_chunk(const BwdArgs &a, int64_t x, ChunkLoc &c)
{
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    const i32x4 r = *reinterpret_cast<const i32x4 *>(a.cinfo + 4 * x);
    if (r[2] < 0)
        return false;
    c.t0 = (int64_t)(((uint64_t)(uint32_t)r[1] << 32) | (uint32_t)r[0]);
    c.n = r[2];
    c.len = r[3] & 0xff;
    c.kind = (r[3] >> 8) & 0xff;
    c.next_len = r[3] >> 16;
    return true;
}

// Rows past the chunk's tokens are zero (k^, q^, v, dO, beta, log-decay), which leaves every
// quantity of the real rows as it is and gamma the decay up to the last real token.  KD is
// not kept: KD = KI gamma.
struct PrepLds {
    float KG[kCH][kP], KI[kCH][kP], QG[kCH][kP], B[kCH][kP];  // B: the log-decay, then Gamma = e^b
    float W[kCH][kP], U[kCH][kP];
    float T[kCH][kQ], M[kCH][kQ], Aqk[kCH][kQ];  // T, KG KI^T, lower(QG KI^T)
    float beta[kCH], rq[kCH], rk[kCH], gam[kD];     // beta; 1/|q|, 1/|k| (1 without the l2norm)
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ f32x4 widen_bf16(u32x2 w)
{
    return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                 __uint_as_float(w[1] & 0xffff0000u)};
}
// The chunk's raw bf16 rows as prep_chunk takes them: thread -> token r = tid / 32, channels
// 4 (tid % 32) .. + 3 of k, q, g, v, and beta of the row (raw bits, so that nothing waits for
// them until they are used; rows past the chunk's tokens zero); with the gate in the pass,
// A_log of the head and dt_bias at the thread's channels.
struct RawRows {
    u32x2 k, q, g, v;
    uint32_t beta;
    float A_log;
    f32x4 dt_bias;
};
__device__ __forceinline__ RawRows load_rows(const BwdArgs &a, const ChunkLoc &c, int h, int tid)
{
    const int r = tid >> 5, c4 = 4 * (tid & 31);
    RawRows w = {u32x2{0u, 0u}, u32x2{0u, 0u}, u32x2{0u, 0u}, u32x2{0u, 0u}, 0u, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
    if (a.flags & kBGateIn) {
        w.A_log = a.A_log[h];
        w.dt_bias = ld4(a.dt_bias + (size_t)h * kD + c4);
    }
    if (r < c.len) {
        const size_t ti = (size_t)(c.t0 + r) * (size_t)a.H + (size_t)h;
        w.k = *reinterpret_cast<const u32x2 *>(a.k + ti * kD + c4);
        w.q = *reinterpret_cast<const u32x2 *>(a.q + ti * kD + c4);
        w.g = *reinterpret_cast<const u32x2 *>(a.g + ti * kD + c4);
        w.v = *reinterpret_cast<const u32x2 *>(a.v + ti * kD + c4);
        w.beta = a.beta[ti];
    }
    return w;
}

// kGradThreads threads; ends with a barrier.
__device__ void prep_chunk(const BwdArgs &a, const ChunkLoc &c, int h, PrepLds &p, int tid, const RawRows &raw)
{
    {  // the chunk's rows, activated: thread -> token r = tid / 32, channels c4 = 4 (tid % 32) .. + 3
        const int r = tid >> 5, c4 = 4 * (tid & 31);
        const f32x4 kk = widen_bf16(raw.k), qq = widen_bf16(raw.q), gg = widen_bf16(raw.g), vv = widen_bf16(raw.v);
        const float braw = bbf16((uint16_t)raw.beta);
        // l2norm over the 128 channels of the row (32 lanes), eps 1e-6
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sk = fmaf(kk[e], kk[e], sk);
            sq = fmaf(qq[e], qq[e], sq);
        }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) {
            sk += __shfl_xor(sk, o);
            sq += __shfl_xor(sq, o);
        }
        const bool l2_in = (a.flags & kBL2In) != 0;
        const float rk = l2_in ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f, rq = l2_in ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f;
        // log-decay: lower_bound * sigmoid(e^A_log (g + dt_bias)), or g clamped to [lower_bound, 0]
        f32x4 ll = {0.f, 0.f, 0.f, 0.f};
        if (r < c.len) {
            if (a.flags & kBGateIn) {
                const float eA = expf(raw.A_log);
                const f32x4 db = raw.dt_bias;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ll[e] = a.lower_bound * __builtin_amdgcn_rcpf(1.0f + expf(-eA * (gg[e] + db[e])));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ll[e] = fminf(fmaxf(gg[e], a.lower_bound), 0.f);
            }
        }
        st4(&p.KG[r][c4], kk * rk);  // k^ until the next step
        st4(&p.QG[r][c4], qq * rq);  // q^
        st4(&p.B[r][c4], ll);        // log-decay
        st4(&p.U[r][c4], vv);        // v until U replaces it
        if ((tid & 31) == 0) {
            p.beta[r] = r < c.len ? ((a.flags & kBSigIn) ? 1.0f / (1.0f + expf(-braw)) : braw) : 0.f;
            p.rq[r] = rq;
            p.rk[r] = rk;
        }
    }
    __syncthreads();
    {  // per channel: b = cumulative log-decay, then the gated rows.  Thread -> channel tid % 128,
       // rows 4 (tid / 128) .. + 3: local prefix sums, block totals through W (free until W
       // is formed), then the offsets of the blocks above.
        const int ch = tid & (kD - 1), blk = tid >> 7, r0 = 4 * blk;
        float *tot = &p.W[0][0];
        float l[4];
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            run += p.B[r0 + i][ch];
            l[i] = run;
        }
        tot[blk * kD + ch] = run;
        __syncthreads();
        float off = 0.f, all = 0.f;
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2) {
            const float t = tot[b2 * kD + ch];
            off += b2 < blk ? t : 0.f;
            all += t;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = r0 + i;
            // (b >= 16 lower_bound >= -80: Gamma and 1/Gamma are normal fp32 numbers)
            const float b = off + l[i], G = expf(b), Gi = __builtin_amdgcn_rcpf(G), k = p.KG[r][ch];
            p.B[r][ch] = G;
            p.KG[r][ch] = k * G;
            p.KI[r][ch] = k * Gi;
            p.QG[r][ch] = a.scale * p.QG[r][ch] * G;
        }
        if (blk == 0)
            p.gam[ch] = expf(all);
    }
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6, g = lane >> 4, m = lane & 15;
    {  // KG KI^T (waves 0 - 3) and QG KI^T (waves 4 - 7), 32 channels per wave; the four partial
       // sums of each through W
        float *part = &p.W[0][0];
        const int k0 = 32 * (wave & 3);
        const f32x4 acc = mm_rows(wave < 4 ? &p.KG[0][k0] : &p.QG[0][k0], &p.KI[0][k0], 32,
                                  f32x4{0.f, 0.f, 0.f, 0.f}, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            part[wave * (kCH * kCH) + (4 * g + i) * kCH + m] = acc[i];
    }
    __syncthreads();
    {
        const float *part = &p.W[0][0];
        const int e = tid & (kCH * kCH - 1), r = e >> 4, s_ = e & 15, q = 4 * (tid >> 8);
        const float v = (part[q * 256 + e] + part[(q + 1) * 256 + e]) + (part[(q + 2) * 256 + e] + part[(q + 3) * 256 + e]);
        if (tid < kCH * kCH)
            p.M[r][s_] = v;
        else
            p.Aqk[r][s_] = s_ <= r ? v : 0.f;  // diagonal included
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
    {  // W = T diag(beta) KG, U = T diag(beta) V on the MFMA: wave w takes columns 16 w + m (D
       // layout, rows 4 g + i)
        const int cc = 16 * wave + m;
        f32x4 tr, bk, bv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int s = 4 * g + j;
            tr[j] = p.T[m][s];  // A operand: T[m][4 g + j]
            bk[j] = p.beta[s] * p.KG[s][cc];
            bv[j] = p.beta[s] * p.U[s][cc];
        }
        const f32x4 w = mm4(tr, bk, f32x4{0.f, 0.f, 0.f, 0.f}), u = mm4(tr, bv, f32x4{0.f, 0.f, 0.f, 0.f});
        __syncthreads();  // every column of v is read before U replaces it
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p.W[4 * g + i][cc] = w[i];
            p.U[4 * g + i][cc] = u[i];
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
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, m = lane & 15;
    prep_chunk(a, c, h, p, tid, load_rows(a, c, h, tid));
    float *o = a.ops + ((size_t)x * (size_t)a.H + (size_t)h) * kBwdOps;
    if (tid < kCH * kCH)
        o[kOpAqk + tid] = p.Aqk[tid >> 4][tid & 15];
    const int ch = tid & (kD - 1), q4 = 4 * (tid >> 7);
    const float gam = p.gam[ch];
    f32x4 kd, qg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = q4 + i;
        kd[i] = p.KI[r][ch] * gam;
        qg[i] = p.QG[r][ch];
        o[kOpNegW + r * kD + ch] = -p.W[r][ch];
        o[kOpU + r * kD + ch] = p.U[r][ch];
        o[kOpKD + r * kD + ch] = kd[i];
    }
    st4(o + kOpQGt + ch * kCH + q4, qg);
    if (tid < kD)
        o[kOpGam + tid] = p.gam[tid];
}

// ---- the two chains over the chunks of one (sequence, head) ----
// Work split (the value rows of a state are independent given the chunk's operands): with
// kCh = 1, a (chain, role) unit takes two workgroups of 64 value rows, wave w owning 16 rows at
// all channels; with kCh = 2 (few units: each workgroup's chunk then takes half the MFMA work
// per wave), four workgroups of 32 rows, wave w owning 16 rows at the channels of half w % 2,
// the first product's two half sums exchanged through LDS.  The workgroups of a unit land on
// one XCD and share its L2 for the operand reads.  kCh = 1 reads each chunk's operands half as
// often, which is what counts when the chains are many and HBM is the limit.
constexpr int kChainUnitsSplit = 128;  // units (chain, role) up to which kCh = 2 is used

// The MFMA A operands A0, A1, A2 are held split: each group of four consecutive values (the
// four k values of one lane) as {hi, lo} (split4), in the same 16 bytes.
template <int kRows>
struct ChainStage {
    float A0[kCH * kD];  // role 0: -W [r][c];  role 1: KD [r][c]
    float A1[kD * kCH];  // role 0: KD^T [c][r]; role 1: QG^T [c][r]
    float A2[kD * kCH];  // role 1: -W^T [c][r]
    float Y[kCH][kRows]; // role 0: U, role 1: dO (the workgroup's value columns)
    float Mx[kCH][kCH];  // role 1: lower(QG KI^T)
    float gam[kD];
};

// Global -> register copies of one chunk's stage (issued a chunk ahead), then register -> LDS.
// Every load is unconditional (a clamped row or column where the data is not needed) and
// keeps its raw bits, so that nothing waits for it before the copy into LDS.
struct StageRegs {
    f32x4 a0[2], a1[2], a2[2], um, gm;  // um: role 0 U at the workgroup's columns, role 1 lower(QG KI^T)
    uint32_t y[2];                      // two bf16 pairs of dO (role 1)
};
template <int kRows>
__device__ __forceinline__ void stage_load(const BwdArgs &a, int role, int part, const float *op, int64_t t0, int len,
                                           int h, StageRegs &r, int tid)
{
    constexpr int kQ4 = kRows / 4;  // float4 columns of Y
    // the transposed operands (role 0: KD^T, role 1: -W^T) from the row-major arrays: thread ->
    // channel tid % 128, rows 4 (tid / 128 + 2 e) .. + 3, four loads that 64 lanes coalesce
    const int tc = tid & (kD - 1), tr = 4 * (tid >> 7);
    auto col4 = [&](const float *m_, int e) {
        const float *q = m_ + (tr + 8 * e) * kD + tc;
        return f32x4{q[0], q[kD], q[2 * kD], q[3 * kD]};
    };
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int f = 4 * (tid + kChainThreads * e);
        r.a0[e] = ld4(op + (role ? kOpKD : kOpNegW) + f);
        r.a1[e] = role ? ld4(op + kOpQGt + f) : col4(op + kOpKD, e);
        if (role)
            r.a2[e] = col4(op + kOpNegW, e);
    }
    const int row = (tid / kQ4) & 15, c4 = 4 * (tid % kQ4);  // (kRows = 32: threads 128 .. repeat)
    r.um = ld4(role ? op + kOpAqk + 4 * (tid & (kCH * kCH / 4 - 1)) : op + kOpU + row * kD + kRows * part + c4);
    {
        const int rr = row < len ? row : 0;  // (role 0 loads a dO row it does not use)
        const u32x2 w = *reinterpret_cast<const u32x2 *>(a.dout + ((size_t)(t0 + rr) * (size_t)a.H + (size_t)h) * kD +
                                                         kRows * part + c4);
        r.y[0] = w[0];
        r.y[1] = w[1];
    }
    r.gm = ld4(op + kOpGam + 4 * (tid & (kD / 4 - 1)));
}
template <int kRows>
__device__ __forceinline__ void stage_store(int role, const StageRegs &r, ChainStage<kRows> &st, int len, int tid)
{
    constexpr int kQ4 = kRows / 4;
    const int tc = tid & (kD - 1), tr = 4 * (tid >> 7);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int f = 4 * (tid + kChainThreads * e);
        stu4(st.A0 + f, split4(r.a0[e]));
        stu4(st.A1 + (role ? f : tc * kCH + tr + 8 * e), split4(r.a1[e]));
        if (role)
            stu4(st.A2 + tc * kCH + tr + 8 * e, split4(r.a2[e]));
    }
    if (tid < kCH * kQ4) {
        const int row = tid / kQ4, c4 = 4 * (tid % kQ4);
        const bool in = row < len;
        st4(&st.Y[row][c4], role ? f32x4{in ? __uint_as_float(r.y[0] << 16) : 0.f, in ? __uint_as_float(r.y[0] & 0xffff0000u) : 0.f,
                                         in ? __uint_as_float(r.y[1] << 16) : 0.f, in ? __uint_as_float(r.y[1] & 0xffff0000u) : 0.f}
                                 : r.um);
    }
    if (role && tid < kCH * kCH / 4)
        st4(&st.Mx[0][0] + 4 * tid, r.um);
    if (tid < kD / 4)
        st4(st.gam + 4 * tid, r.gm);
}

// s_waitcnt vmcnt(0), the other counters untouched
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }

// Launch kinds of the chain kernel: whole chains, and the cut plan's pass A, transition runs
// and pass B (one workgroup per piece, direction and part).
constexpr int kChWhole = 0, kChA = 1, kChT = 2, kChB = 3;
constexpr int kPieceParts = 2;  // the cut plan runs bwd_chain_kernel<1, ...>

// Workgroup b: XCD b % 8, part (b / 8) % (2 kCh) of unit (b / (16 kCh)) 8 + b % 8.  Whole
// chains: unit u is chain u / 2, direction (role) u % 2.  Cut plan: unit u is piece slot
// u / (2 H) (pieces counted over the sequences), head (u / 2) % H, direction u % 2.  A wave's
// state is held transposed in the D layout: its tile e (channels 16 ct .., ct = ct0 + e) has in
// lane L element i S[v0 + L % 16][16 ct + 4 (L / 16) + i].
template <int kCh, int kMode>
__global__ __launch_bounds__(kChainThreads) void bwd_chain_kernel(BwdArgs a)
{
    constexpr int kRows = 64 / kCh, kTiles = 8 / kCh, kParts = 2 * kCh;
    constexpr bool kPiece = kMode != kChWhole;
    static_assert(!kPiece || kParts == kPieceParts, "the cut plan runs kCh = 1: two row parts per piece");
    // stage buffers: one where the chains are many (kCh = 1: 33 KB of LDS, so that three
    // workgroups fit a CU, at the price of a barrier before each refill), two otherwise
    constexpr int kSt = kCh == 1 ? 1 : 2;
    __shared__ __attribute__((aligned(16))) ChainStage<kRows> s_st[kSt];
    __shared__ __attribute__((aligned(16))) float s_x[kCh == 2 ? kChainThreads / 64 : 1][64][4];  // half sums
    __shared__ int s_vote[kMode == kChT ? 2 : 1][kChainThreads / 64];  // transition runs: a wave's entries not all small
    __shared__ float s_nrm[kChainThreads / 64];
    const int64_t bid = blockIdx.x;
    const int xcd = (int)(bid & 7);
    const int64_t slot = bid >> 3;
    const int part = (int)(slot % kParts);
    const int64_t unit = (slot / kParts) * 8 + xcd;
    const int64_t H = a.H;
    if (unit >= 2 * (kPiece ? a.poff[a.N] : a.N) * H)
        return;
    const int role = (int)(unit & 1);
    const int64_t chain = unit >> 1;
    const int h = (int)(chain % H);
    // whole chains: sequence n; cut plan: piece slot q of sequence n, piece k (chunk order) of
    // its P, w in walk order
    int64_t n = chain / H, q = 0, P = 1, w = 0;
    if constexpr (kPiece) {
        q = n;
        int64_t lo = 0, hi = a.N - 1;
        while (lo < hi) {
            const int64_t mid = (lo + hi) >> 1;
            if (a.poff[mid + 1] > q)
                hi = mid;
            else
                lo = mid + 1;
        }
        n = lo;
        P = a.poff[n + 1] - a.poff[n];
        const int64_t k = q - a.poff[n];
        w = role ? P - 1 - k : k;
        if ((kMode == kChT || kMode == kChB) && w == 0)
            return;  // the first piece of a walk starts from the true state in pass A
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, m = lane & 15;
    const int rg = wave / kCh, hc = wave % kCh;                 // row group, channel half
    const int v0 = kRows * part + 16 * rg, ct0 = kTiles * hc;  // value rows v0 .., channel tiles ct0 ..
    const int64_t start = a.seq_start[n], len = a.seq_len[n], off = a.seq_off[n];
    const int64_t nch = (len + kCH - 1) / kCH;
    // the chunks [c0, c1) this workgroup walks
    int64_t c0 = 0, c1 = nch;
    if constexpr (kPiece) {
        c0 = (q - a.poff[n]) * a.plen;
        c1 = c0 + a.plen < nch ? c0 + a.plen : nch;
    }
    auto slot_of = [&](int64_t j) { return (size_t)(off + j) * (size_t)H + (size_t)h; };
    auto op_of = [&](int64_t j) { return a.ops + slot_of(j) * kBwdOps; };
    auto tok_len = [&](int64_t j) { return (int)(len - kCH * j < kCH ? len - kCH * j : kCH); };
    const size_t srow = (size_t)(n * H + h) * kBState + (size_t)(v0 + m) * kD + 16 * ct0 + 4 * g;  // + 16 e
    const size_t prow = (size_t)(v0 + m) * kD + 16 * ct0 + 4 * g;  // + 16 e (piece states)
    // cut plan: the (piece, head, direction) slot of walk piece ww of this sequence
    auto pslot = [&](int64_t ww) {
        const int64_t kk = role ? P - 1 - ww : ww;
        return ((size_t)(a.poff[n] + kk) * (size_t)H + (size_t)h) * 2 + (size_t)role;
    };
    auto pstate = [&](int64_t ww, int which) { return a.pst + (pslot(ww) * 3 + (size_t)which) * kBState; };
    f32x4 S[kTiles];
    if (kMode == kChT) {
        // from I: S[v][c] = (v == c)
#pragma unroll
        for (int e = 0; e < kTiles; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[e][i] = v0 + m == 16 * (ct0 + e) + 4 * g + i ? 1.f : 0.f;
    } else if (kMode == kChB) {
#pragma unroll
        for (int e = 0; e < kTiles; ++e)
            S[e] = ld4(pstate(w, 0) + prow + 16 * e);
    } else if (w > 0) {
#pragma unroll
        for (int e = 0; e < kTiles; ++e)
            S[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    } else if (role == 0) {
#pragma unroll
        for (int e = 0; e < kTiles; ++e) {
            if (a.h0_dtype == 2)
                S[e] = ld4(reinterpret_cast<const float *>(a.h0) + srow + 16 * e);
            else if (a.h0_dtype == 1)
                S[e] = ld4_bf16(reinterpret_cast<const uint16_t *>(a.h0) + srow + 16 * e);
            else
                S[e] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    } else {
#pragma unroll
        for (int e = 0; e < kTiles; ++e)
            S[e] = a.dht ? ld4(a.dht + srow + 16 * e) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // the chunks this walk takes: pass B reruns the first z of a piece whose transition run
    // stopped in every part (z the most any part took), all of it otherwise
    int64_t n_it = c1 - c0;
    bool dropped = false;
    if (kMode == kChB && a.trunc) {
        int zmax = 0;
        dropped = true;
#pragma unroll
        for (int pp = 0; pp < kParts; ++pp) {
            const int z = a.pz[pslot(w) * 4 + pp];
            dropped = dropped && z >= 0;
            zmax = z > zmax ? z : zmax;
        }
        if (dropped && zmax < n_it)
            n_it = zmax;
    }
    // transition runs: the stop threshold kTruncRel |F_w|_F / (|st_1|_F + |F_1|_F + .. + |F_{w-1}|_F)
    float thr = 0.f;
    if (kMode == kChT && a.trunc) {
        auto fro = [&](int64_t ww, int which) {
            const float *p = a.pnrm + pslot(ww) * 8 + 4 * which;
            float t = 0.f;
#pragma unroll
            for (int pp = 0; pp < kParts; ++pp)
                t += p[pp];
            return sqrtf(t);
        };
        float bound = fro(1, 1);
        for (int64_t i = 1; i < w; ++i)
            bound += fro(i, 0);
        thr = bound == 0.f ? __builtin_inff() : kTruncRel * fro(w, 0) / bound;
    }
    // -I (bf16) as the A operand of split_tile: lane m + 16 (m / 4), element m % 4
    uint32_t nI0 = 0u, nI1 = 0u;
    if (g == (m >> 2)) {
        const uint32_t v = (m & 1) ? 0xbf800000u : 0x0000bf80u;
        if ((m & 2) == 0)
            nI0 = v;
        else
            nI1 = v;
    }
    // The operands of chunk it + 1 are requested while chunk it runs.
    wait_vmem();  // the initial state is in (so that no wait inside the loop is for it)
    StageRegs rg_;
    auto chunk_of = [&](int64_t it) { return role ? c1 - 1 - it : c0 + it; };
    auto load = [&](int64_t it) {
        const int64_t j = chunk_of(it);
        stage_load<kRows>(a, role, part, op_of(j), start + kCH * j, tok_len(j), h, rg_, tid);
    };
    if (n_it > 0) {
        load(0);
        stage_store<kRows>(role, rg_, s_st[0], tok_len(chunk_of(0)), tid);
    }
    __syncthreads();
    int64_t z = -1;  // transition runs: chunks run before the stop
    for (int64_t it = 0; it < n_it; ++it) {
        const int64_t j = chunk_of(it);
        const bool more = it + 1 < n_it;
        const bool upd = kPiece ? j + 1 < nch : more;  // role 0: no update after a sequence's last chunk
        if (more)
            load(it + 1);
        const ChainStage<kRows> &st = s_st[kSt == 1 ? 0 : (it & 1)];
        const size_t sl = slot_of(j);
        u32x4 A[kTiles];  // A operands of the first product (this wave's channels), read before its MFMAs
#pragma unroll
        for (int e = 0; e < kTiles; ++e)
            A[e] = ldu4(st.A0 + m * kD + 16 * (ct0 + e) + 4 * g);
        // X starts at U (role 0) or at U~ = lower(QG KI^T)^T dO (role 1, one fp32 product, in an
        // accumulator of its own so that it overlaps the first product) at the wave's value
        // columns, in the first wave of a row group; transition runs take U and dO as zero
        f32x4 X0 = {0.f, 0.f, 0.f, 0.f}, X1 = X0, XU = X0;
        if (hc == 0 && kMode != kChT) {
            if (role) {
                f32x4 ua, ub;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    ua[j] = st.Mx[4 * g + j][m];  // A: (A_qk^T)[m][4 g + j]
                    ub[j] = st.Y[4 * g + j][16 * rg + m];
                }
                XU = mm4(ua, ub, XU);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    XU[i] = st.Y[4 * g + i][16 * rg + m];
            }
        }
        // the state before an even chunk (role 0) or dL/dS after an odd one (role 1), in the
        // tiled layout (state_at): each store of the wave writes 256 contiguous bytes
        if (kMode != kChT && (int)(j & 1) == role) {
            float *ck = a.ck + sl * kBState + (size_t)(v0 >> 4) * (8 * 256) + 256 * ct0 + 16 * g + m;
#pragma unroll
            for (int e = 0; e < kTiles; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ck[256 * e + 64 * i] = S[e][i];
        }
        // role 0: V' = U - W S^T;  role 1: dV' = U~ + KD D^T   (rows r = 4 g + i, column v0 + m);
        // two accumulators (even and odd tiles), then (kCh = 2) the partner wave's half sum
#pragma unroll
        for (int e = 0; e < kTiles; e += 2) {
            X0 = mm3(A[e], split_tile(S[e], nI0, nI1), X0);
            X1 = mm3(A[e + 1], split_tile(S[e + 1], nI0, nI1), X1);
        }
        f32x4 X = (X0 + X1) + XU;
        if constexpr (kCh == 2) {
            st4(&s_x[wave][lane][0], X);
            __syncthreads();
            const f32x4 other = ld4(&s_x[wave ^ 1][lane][0]);
            X = hc == 0 ? X + other : other + X;  // the same sum in both waves
        }
        if (hc == 0 && kMode != kChT) {
            float *xo = (role ? a.xb : a.xf) + sl * (kCH * kD) + (v0 >> 4) * 256 + 16 * g + m;  // (rows_at)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xo[64 * i] = X[i];
        }
        if (role == 0) {
            if (upd) {  // S <- S Diag(gamma) + V'^T KD
                const u32x4 xs = split_tile(X, nI0, nI1);
                u32x4 K[kTiles];
                f32x4 Gm[kTiles];
#pragma unroll
                for (int e = 0; e < kTiles; ++e) {
                    K[e] = ldu4(st.A1 + (16 * (ct0 + e) + m) * kCH + 4 * g);
                    Gm[e] = ld4(st.gam + 16 * (ct0 + e) + 4 * g);
                }
#pragma unroll
                for (int e = 0; e < kTiles; ++e)
                    S[e] = mm3(K[e], xs, S[e] * Gm[e]);
            }
        } else {  // D <- D Diag(gamma) + dO^T QG - dV'^T W
            // dO is bf16: its four rows as one packed word pair, no lo part
            const uint32_t o0 = kMode == kChT ? 0u : pk_bf16(st.Y[4 * g][16 * rg + m], st.Y[4 * g + 1][16 * rg + m]);
            const uint32_t o1 = kMode == kChT ? 0u : pk_bf16(st.Y[4 * g + 2][16 * rg + m], st.Y[4 * g + 3][16 * rg + m]);
            const u32x4 xs = split_tile(X, nI0, nI1);
#pragma unroll
            for (int c4 = 0; c4 < kTiles; c4 += 4) {
                u32x4 Q[4], Wt[4];
                f32x4 Gm[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    Q[e] = ldu4(st.A1 + (16 * (ct0 + c4 + e) + m) * kCH + 4 * g);
                    Wt[e] = ldu4(st.A2 + (16 * (ct0 + c4 + e) + m) * kCH + 4 * g);
                    Gm[e] = ld4(st.gam + 16 * (ct0 + c4 + e) + 4 * g);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[c4 + e] = mm3(Wt[e], xs, mm2(Q[e], o0, o1, S[c4 + e] * Gm[e]));
            }
        }
        if (kMode == kChT && a.trunc) {
            // vote: this wave's entries all below thr (NaN counts as big); two vote sets, used
            // by alternate chunks, so that a wave that runs ahead does not overwrite a vote
            // another wave has still to read
            bool big = false;
#pragma unroll
            for (int e = 0; e < kTiles; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    big |= !(__builtin_fabsf(S[e][i]) < thr);
            const bool wbig = __builtin_amdgcn_ballot_w64(big) != 0;
            if (lane == 0)
                s_vote[kMode == kChT ? (it & 1) : 0][wave] = wbig ? 1 : 0;
        }
        if (kSt == 1)
            __syncthreads();  // every wave has read the stage of chunk it
        if (more)
            stage_store<kRows>(role, rg_, s_st[kSt == 1 ? 0 : ((it + 1) & 1)], tok_len(chunk_of(it + 1)), tid);
        __syncthreads();
        if (kMode == kChT && a.trunc) {
            int any = 0;
#pragma unroll
            for (int wv = 0; wv < kChainThreads / 64; ++wv)
                any |= s_vote[kMode == kChT ? (it & 1) : 0][wv];
            if (!any) {
                z = it + 1;
                break;
            }
        }
    }
    // squared norm of the workgroup's rows of the end state (pass A)
    auto sum_sq = [&]() {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < kTiles; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                t = fmaf(S[e][i], S[e][i], t);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1)
            t += __shfl_xor(t, o);
        if (lane == 0)
            s_nrm[wave] = t;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int wv = 0; wv < kChainThreads / 64; ++wv)
            tot += s_nrm[wv];
        return tot;
    };
    auto store_state = [&](float *base) {
#pragma unroll
        for (int e = 0; e < kTiles; ++e)
            st4(base + prow + 16 * e, S[e]);
    };
    if constexpr (kMode == kChWhole) {
        if (role == 1 && a.dh0) {
#pragma unroll
            for (int e = 0; e < kTiles; ++e)
                st4(a.dh0 + srow + 16 * e, S[e]);
        }
    } else if constexpr (kMode == kChA) {
        if (P == 1) {
            if (role == 1 && a.dh0) {
#pragma unroll
                for (int e = 0; e < kTiles; ++e)
                    st4(a.dh0 + srow + 16 * e, S[e]);
            }
        } else {
            // w = 0: the true start state of walk piece 1; otherwise F_w
            const int which = w == 0 ? 0 : 1;
            store_state(pstate(w == 0 ? 1 : w, which));
            const float t = sum_sq();
            if (tid == 0)
                a.pnrm[pslot(w == 0 ? 1 : w) * 8 + 4 * (1 - which) + part] = t;
        }
    } else if constexpr (kMode == kChT) {
        // Phi_w's rows; a part that stopped stores zero rows: they were below thr and cannot
        // grow, so the scan's error from them stays under the bound of a dropped share
        if (z >= 0) {
#pragma unroll
            for (int e = 0; e < kTiles; ++e)
                S[e] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        store_state(pstate(w, 2));
        if (tid == 0)
            a.pz[pslot(w) * 4 + part] = (int32_t)z;
    } else {
        // pass B: the walk's last piece ends at the sequence's start (role 1: dL/dS_initial),
        // from pass A's F where only the first chunks were rerun
        if (role == 1 && w == P - 1 && a.dh0) {
            const bool from_f = dropped && n_it < c1 - c0;
#pragma unroll
            for (int e = 0; e < kTiles; ++e)
                st4(a.dh0 + srow + 16 * e, from_f ? ld4(pstate(w, 1) + prow + 16 * e) : S[e]);
        }
    }
}

// Cut plan, scan: per (sequence, head, direction) with three or more pieces, in walk order
// st_{w+1} = F_w where the transition run of piece w stopped in every part, else
// st_w Phi_w + F_w (fp32 MFMA; the rows are independent: workgroup b takes rows 16 (b % 8) ..
// of (sequence, head, direction) b / 8 and keeps them in LDS between steps).
__global__ __launch_bounds__(256) void bwd_piece_scan_kernel(BwdArgs a)
{
    __shared__ __attribute__((aligned(16))) float s_rows[kCH][kD + 4];
    const int64_t b = blockIdx.x;
    const int rb = (int)(b & 7);
    const int64_t u = b >> 3;
    const int role = (int)(u & 1);
    const int64_t chain = u >> 1, n = chain / a.H;
    const int h = (int)(chain % a.H);
    if (n >= a.N)
        return;
    const int64_t P = a.poff[n + 1] - a.poff[n];
    if (P < 3)
        return;
    auto pslot = [&](int64_t ww) {
        const int64_t kk = role ? P - 1 - ww : ww;
        return ((size_t)(a.poff[n] + kk) * (size_t)a.H + (size_t)h) * 2 + (size_t)role;
    };
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 4, m = lane & 15;
    const size_t r0 = (size_t)(kCH * rb) * kD;  // first element of the workgroup's rows
    {
        const float *st1 = a.pst + pslot(1) * 3 * kBState + r0;
        for (int i = tid; i < kCH * kD / 4; i += 256)
            st4(&s_rows[i / (kD / 4)][4 * (i % (kD / 4))], ld4(st1 + 4 * i));
    }
    __syncthreads();
    for (int64_t w = 1; w + 1 < P; ++w) {
        const size_t sw = pslot(w);
        const float *F = a.pst + (sw * 3 + 1) * kBState + r0, *Phi = a.pst + (sw * 3 + 2) * kBState;
        bool dropped = a.trunc != 0;
#pragma unroll
        for (int pp = 0; pp < kPieceParts; ++pp)
            dropped = dropped && a.pz[sw * 4 + pp] >= 0;
        float *dst = a.pst + pslot(w + 1) * 3 * kBState + r0;
        // wave wv: output columns 32 wv .. + 31 as two 16-column tiles (D layout)
        f32x4 acc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col0 = 32 * wv + 16 * t;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                acc[t][i] = F[(size_t)(4 * g + i) * kD + col0 + m];
            if (!dropped) {
                for (int k0 = 0; k0 < kD; k0 += 16) {
                    const f32x4 x = ld4(&s_rows[m][k0 + 4 * g]);
                    f32x4 y;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        y[j] = Phi[(size_t)(k0 + 4 * g + j) * kD + col0 + m];
                    acc[t] = mm4(x, y, acc[t]);
                }
            }
        }
        __syncthreads();  // every wave has read the rows
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col0 = 32 * wv + 16 * t;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s_rows[4 * g + i][col0 + m] = acc[t][i];
                dst[(size_t)(4 * g + i) * kD + col0 + m] = acc[t][i];
            }
        }
        __syncthreads();
    }
}

// Cut plan: the first piece of every sequence, poff[n] = sum over i < n of max(1,
// ceil(chunks_i / plen)) (a sequence without chunks keeps one empty piece, which passes dL/dS
// of the final state to dL/dS of the initial one).
__global__ __launch_bounds__(256) void bwd_piece_table_kernel(BwdArgs a)
{
    __shared__ int64_t s_scan[256];
    __shared__ int64_t s_carry;
    const int tid = threadIdx.x;
    if (tid == 0)
        s_carry = 0;
    __syncthreads();
    for (int64_t base = 0; base < a.N; base += 256) {
        const int64_t i = base + tid;
        int64_t cnt = 0;
        if (i < a.N) {
            const int64_t nc = (a.seq_len[i] + kCH - 1) / kCH;
            cnt = nc > a.plen ? (nc + a.plen - 1) / a.plen : 1;
        }
        s_scan[tid] = cnt;
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
            const int64_t x = tid >= d ? s_scan[tid - d] : 0;
            __syncthreads();
            s_scan[tid] += x;
            __syncthreads();
        }
        const int64_t carry = s_carry;
        if (i < a.N)
            a.poff[i + 1] = carry + s_scan[tid];
        __syncthreads();
        if (tid == 255)
            s_carry = carry + s_scan[255];
        __syncthreads();
    }
    if (tid == 0)
        a.poff[0] = 0;
}

// ---- gradients of one chunk-head's tokens ----
struct GradLds {
    PrepLds p;
    float P[kCH][kP], Q[kCH][kP];  // T^T dV' and T^T dW; P then holds db
    float dA[kCH][kQ4], dAqk[kCH][kQ4];  // rows 16-byte aligned (MFMA A operands)
    union {
        float rowdot[kCH][kGradThreads / 64][2];  // per row and wavefront (16 channels): q^ . dq^, k^ . dk^
        float part[4][kCH][kCH];                  // dA: partial sums of four wavefronts
    };
};

__global__ __launch_bounds__(kGradThreads) __attribute__((amdgpu_waves_per_eu(4))) void bwd_grad_kernel(BwdArgs a)
{
    __shared__ __attribute__((aligned(16))) GradLds L;
    PrepLds &p = L.p;
    const int64_t x = blockIdx.x / a.H;
    const int h = (int)(blockIdx.x % a.H);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, m = lane & 15;
    const size_t sl = (size_t)x * (size_t)a.H + (size_t)h;  // (a slot of the workspace for every x)
    const float *xf = a.xf + sl * (kCH * kD), *xb = a.xb + sl * (kCH * kD);
    // The loads that need only the chunk's slot go out before the search for its sequence: its
    // V' and dV' rows (thread -> row tid / 32, columns 4 (tid % 32) .. + 3, rows_at) and the
    // first two tiles of its stored state for the loop below.
    const int so = 256 * wave + 64 * (m & 3) + 16 * (m >> 2) + 4 * g;
    const float *cs = a.ck + sl * kBState + so;  // the stored state
    const int rr = tid >> 5, rc4 = 4 * (tid & 31);
    const int ro = 256 * (rc4 >> 4) + 64 * (rr & 3) + 16 * (rr >> 2) + (rc4 & 15);  // rows_at(rr, rc4)
    const f32x4 own_v = ld4(xf + ro), own_dv = ld4(xb + ro);
    f32x4 x0 = ld4(cs), x1 = ld4(cs + 2048);
    ChunkLoc c;
    if (!locate_chunk(a, x, c))
        return;
    const int c0 = 16 * wave, cc = c0 + m;
    const size_t tok0 = (size_t)c.t0 * (size_t)a.H + (size_t)h;  // token-head index of row 0
    // The tail's per-element inputs (D layout: wave w, channel 16 w + m, rows 4 g + i) and the
    // dbeta rows' v, requested first so that nothing later waits for them.
    f32x4 tq, tk, tg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        const size_t at = (tok0 + (size_t)(r < c.len ? r : 0) * (size_t)a.H) * kD + (size_t)cc;
        tq[i] = bbf16(a.q[at]);
        tk[i] = bbf16(a.k[at]);
        tg[i] = bbf16(a.g[at]);
    }
    const RawRows raw = load_rows(a, c, h, tid);  // prep_chunk's rows; v also for the dbeta rows
    const float dtb = (a.flags & kBGateIn) ? a.dt_bias[(size_t)h * kD + cc] : 0.f;  // the tail's gate
    st4(&L.P[rr][rc4], own_dv);  // dV' into P (P replaces it below)
    // The chain stored one of the chunk's two states: S0 for an even chunk of the sequence, D
    // for an odd one.  The other is rebuilt from the neighbouring chunk's stored state and
    // operands (the steps the chain took between them):
    //   odd chunk:             S0 = S0' Diag(gamma') + V'^T KD'   (' : the previous chunk)
    //   even chunk, not last:  D = D'' Diag(gamma'') + dO''^T QG'' - dV''^T W''   ('' : the next)
    //   even chunk, last:      D = dL/dS_final (zero when not given)
    const int kind = c.kind;
    const size_t sn = kind == 0 ? sl + (size_t)a.H : kind == 1 ? sl - (size_t)a.H : sl;  // the neighbour
    f32x4 nb0 = {0.f, 0.f, 0.f, 0.f}, nb1 = nb0;  // B operands of the rebuild: rows 4 g + j, channel cc
    float ngam = 0.f;                             // the neighbour's gamma at channel cc
    if (kind != 2) {
        const float *opn = a.ops + sn * kBwdOps;
        if (kind == 0) {
            nb0 = ld4(opn + kOpQGt + cc * kCH + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                nb1[j] = opn[kOpNegW + (4 * g + j) * kD + cc];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                nb0[j] = opn[kOpKD + (4 * g + j) * kD + cc];
        }
        ngam = opn[kOpGam + cc];
    }
    // The neighbour's first two state tiles, requested ahead of the staging loads (for the last
    // chunk of a sequence, kind 2, the neighbour is the chunk itself and they go unused).
    const float *cn = a.ck + sn * kBState + so;
    f32x4 n0 = ld4(cn), n1 = ld4(cn + 2048);
    // Rows staged in LDS (the space prep_chunk fills afterwards) as the bf16 {hi, lo} operands of
    // the three-term products below (each group of four values as u32x4 {hi, lo}; dO is exact
    // in bf16, lo zero): the chunk's V', dO, dV' row-major with rows padded to kRS floats (16
    // lanes reading 16 rows hit distinct banks), and the neighbour's rows (V' or dV'', and dO'')
    // transposed, [value column][row] with columns padded to kNT floats, since the rebuild takes
    // them as A operands of four rows at one column.  Only the two state tiles per step are read
    // from global memory in the loop below, requested two steps ahead.
    constexpr int kRS = kD + 4, kNT = kCH + 4;
    float *const sV = &p.KG[0][0], *const sO = sV + kCH * kRS, *const sD = sO + kCH * kRS;
    float *const nX = sD + kCH * kRS, *const nO = nX + kD * kNT;
    static_assert(3 * kCH * kRS + 2 * kD * kNT <= 6 * kCH * kP, "staging fits in KG .. U");
    {
        const int r = rr, c4 = rc4;
        const u32x4 z = {0u, 0u, 0u, 0u};
        stu4(sV + r * kRS + c4, split4(own_v));
        stu4(sD + r * kRS + c4, split4(own_dv));
        u32x4 ow = z;
        if (r < c.len) {
            const u32x2 w = *reinterpret_cast<const u32x2 *>(a.dout + (tok0 + (size_t)r * (size_t)a.H) * kD + c4);
            ow = u32x4{w[0], w[1], 0u, 0u};
        }
        stu4(sO + r * kRS + c4, ow);
        // the neighbour's rows 4 q .. 4 q + 3 at value column v, q = tid / 128
        const int v = tid & (kD - 1), q = tid >> 7;
        const int nro = 256 * (v >> 4) + 16 * q + (v & 15);  // rows_at(4 q, v); row 4 q + i adds 64 i
        if (kind == 0) {
            const float *xn = a.xb + sn * (kCH * kD) + nro;
            stu4(nX + v * kNT + 4 * q, split4(f32x4{xn[0], xn[64], xn[128], xn[192]}));
            const int rem = c.next_len;  // the next chunk's tokens
            uint32_t hw[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                hw[i] = 4 * q + i < rem ? a.dout[((size_t)(c.t0 + kCH + 4 * q + i) * (size_t)a.H + (size_t)h) * kD + v] : 0u;
            stu4(nO + v * kNT + 4 * q, u32x4{hw[0] | (hw[1] << 16), hw[2] | (hw[3] << 16), 0u, 0u});
        } else if (kind == 1) {
            const float *xn = a.xf + sn * (kCH * kD) + nro;
            stu4(nX + v * kNT + 4 * q, split4(f32x4{xn[0], xn[64], xn[128], xn[192]}));
        }
    }
    // -I (bf16) as the A operand of split_tile: lane m + 16 (m / 4), element m % 4
    uint32_t nI0 = 0u, nI1 = 0u;
    if (g == (m >> 2)) {
        const uint32_t vv = (m & 1) ? 0xbf800000u : 0x0000bf80u;
        if ((m & 2) == 0)
            nI0 = vv;
        else
            nI1 = vv;
    }
    const u32x4 nb0s = split4(nb0), nb1s = split4(nb1);
    // The products with the chunk's states, wave w at channels c0 .. c0 + 15 (lane (g, m): rows
    // 4 g + i, channel cc, the D layout):  dKD = V' D and G1 = dO S0 stay in registers for the
    // tail, G2 = dV' S0 goes to Q, dgamma_c = sum_v S0[v][c] D[v][c] is summed over the lanes
    // of a channel; waves 0 - 3 also form dAqk = lower(dO V'^T) over value columns 32 w .. + 31.
    // A operands: rows m of V', dV', dO at value columns 16 t + 4 g .. + 3; B operands: the
    // states at value rows 16 t + 4 g .. + 3, channel cc (state_at).  Three-term bf16 products
    // (two terms where dO, exact in bf16, is the A operand), fp32 accumulation.
    f32x4 tKD = {0.f, 0.f, 0.f, 0.f}, tG1 = tKD, aG2 = tKD, aQK = tKD;
    float tdgam = 0.f;
    {
        // one 16-row step t: the states at value rows 16 t .. + 15 (bs = S0, bd = D)
        auto prod = [&](int t, f32x4 bs, f32x4 bd) {
            const int ra = m * kRS + 16 * t + 4 * g;
            const u32x4 af = ldu4(sV + ra), ab = ldu4(sD + ra), ao = ldu4(sO + ra);
            const u32x4 bss = split_tile(bs, nI0, nI1), bds = split_tile(bd, nI0, nI1);
            tKD = mm3(af, bds, tKD);
            tG1 = mm2a(ao, bss, tG1);
            aG2 = mm3(ab, bss, aG2);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                tdgam = fmaf(bs[j], bd[j], tdgam);
            if ((t >> 1) == wave)
                aQK = mm2a(ao, af, aQK);
        };
        // the neighbour's rows 4 g .. 4 g + 3 at value column 16 t + m
        auto nrow = [&](const float *X, int t) { return ldu4(X + (16 * t + m) * kNT + 4 * g); };
        if (kind == 2) {
            const float *dh =  // dL/dS_final at value row 4 g, channel cc
                a.dht ? a.dht + ((size_t)c.n * (size_t)a.H + (size_t)h) * kBState + (size_t)(4 * g) * kD + cc : nullptr;
            __syncthreads();
#pragma unroll 1
            for (int t = 0; t < 8; ++t) {
                f32x4 bd = {0.f, 0.f, 0.f, 0.f};
                if (dh)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        bd[i] = dh[(size_t)(16 * t + i) * kD];
                prod(t, ld4(cs + 2048 * t), bd);
            }
        } else {
            __syncthreads();  // the staged rows
#pragma unroll 1
            for (int t = 0; t < 8; ++t) {
                const f32x4 sx = x0, sy = n0;
                const int tn = t + 2 < 8 ? t + 2 : 7;  // (the last two steps load tile 7 again)
                x0 = x1;
                n0 = n1;
                x1 = ld4(cs + 2048 * tn);
                n1 = ld4(cn + 2048 * tn);
                if (kind == 1)
                    prod(t, mm3(nrow(nX, t), nb0s, sy * ngam), sx);
                else
                    prod(t, sx, mm3(nrow(nX, t), nb1s, mm2a(nrow(nO, t), nb0s, sy * ngam)));
            }
        }
        tdgam += __shfl_xor(tdgam, 16);
        tdgam += __shfl_xor(tdgam, 32);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            L.Q[4 * g + i][cc] = aG2[i];
        if (wave < 4)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                L.part[wave][4 * g + i][m] = aQK[i];
    }
    __syncthreads();  // the staged rows are read before prep_chunk overwrites them
    prep_chunk(a, c, h, p, tid, raw);  // ends with a barrier
    if (tid < kCH * kCH) {  // dAqk: the four partial sums, lower triangle with the diagonal
        const int r = tid >> 4, s_ = tid & 15;
        const float v = (L.part[0][r][s_] + L.part[1][r][s_]) + (L.part[2][r][s_] + L.part[3][r][s_]);
        L.dAqk[r][s_] = s_ <= r ? v : 0.f;
    }
    {  // P = T^T dV', Q = T^T dW = -T^T G2 on the MFMA: wave w takes columns cc = 16 w + m (D
       // layout, rows 4 g + i); dv = beta P
        f32x4 tt, bp, bq;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            tt[j] = p.T[4 * g + j][m];  // A operand: (T^T)[m][4 g + j]
            bp[j] = L.P[4 * g + j][cc];
            bq[j] = -L.Q[4 * g + j][cc];
        }
        const f32x4 P = mm4(tt, bp, f32x4{0.f, 0.f, 0.f, 0.f}), Q = mm4(tt, bq, f32x4{0.f, 0.f, 0.f, 0.f});
        __syncthreads();  // every column of dV' and G2 is read
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            L.P[r][cc] = P[i];
            L.Q[r][cc] = Q[i];
            if (r < c.len)
                a.dv[(tok0 + (size_t)r * (size_t)a.H) * kD + (size_t)cc] = p.beta[r] * P[i];
        }
    }
    __syncthreads();
    if (wave < 4) {  // dA = -strictly_lower(P U^T + Q W^T): wave w sums columns 32 w .. 32 w + 31
        const int k0 = 32 * wave;
        f32x4 acc = mm_rows(&L.P[0][k0], &p.U[0][k0], 32, f32x4{0.f, 0.f, 0.f, 0.f}, lane);
        acc = mm_rows(&L.Q[0][k0], &p.W[0][k0], 32, acc, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            L.part[wave][4 * g + i][m] = acc[i];
    }
    __syncthreads();
    if (tid < kCH * kCH) {
        const int r = tid >> 4, s_ = tid & 15;
        const float v = (L.part[0][r][s_] + L.part[1][r][s_]) + (L.part[2][r][s_] + L.part[3][r][s_]);
        L.dA[r][s_] = s_ < r ? -v : 0.f;
    }
    __syncthreads();
    {  // dbeta_r = P_r . V_r + Q_r . KG_r + dA_r . M_r: 32 lanes per row
        const int r = tid >> 5, part = tid & 31;
        float s = 0.f;
        if (r < c.len) {
            const f32x4 vv = widen_bf16(raw.v);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int cc = 4 * part + e;
                s = fmaf(L.P[r][cc], vv[e], s);
                s = fmaf(L.Q[r][cc], p.KG[r][cc], s);
            }
            if (part < kCH)
                s = fmaf(L.dA[r][part], p.M[r][part], s);
        }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1)
            s += __shfl_xor(s, o);
        if (part == 0 && r < c.len) {
            const float b = p.beta[r];  // (after the sigmoid where it runs in the pass)
            a.dbeta[tok0 + (size_t)r * (size_t)a.H] = (a.flags & kBSigIn) ? s * b * (1.0f - b) : s;
        }
    }
    // dKG, dKI, dQG on the MFMA: wave w takes channels c0 .. c0 + 15, c0 = 16 w; lane (g, m)
    // holds rows 4 g + i at channel c0 + m (the D layout) from here on.
    f32x4 sKG, sQG = {0.f, 0.f, 0.f, 0.f}, sKI = sQG;
    {
        f32x4 ki, kgb, qg;  // B operands: rows 4 g + j at channel cc
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * g + j;
            ki[j] = p.KI[r][cc];
            kgb[j] = p.beta[r] * p.KG[r][cc];
            qg[j] = p.QG[r][cc];
            sKG[j] = L.Q[r][cc];
        }
        const f32x4 dA_r = ld4(&L.dA[m][4 * g]), dAqk_r = ld4(&L.dAqk[m][4 * g]);  // rows m
        f32x4 dA_c, dAqk_c;                                                          // columns m
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            dA_c[j] = L.dA[4 * g + j][m];
            dAqk_c[j] = L.dAqk[4 * g + j][m];
        }
        sKG = mm4(dA_r, ki, sKG);      // Q + dA KI
        sQG = mm4(dAqk_r, ki, sQG) + tG1;  // G1 + dAqk KI
        sKI = mm4(dA_c, kgb, sKI);     // dA^T diag(beta) KG
        sKI = mm4(dAqk_c, qg, sKI);    //   + dAqk^T QG
    }
    const float gam = p.gam[cc];
    f32x4 db, dqh, dkh, qh, kh;
    float eKD = 0.f;  // sum over this lane's rows of dKD KD
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * g + i;
        const float dKG = p.beta[r] * sKG[i], dKD = tKD[i];
        const float G = p.B[r][cc], Gi = __builtin_amdgcn_rcpf(G);
        const float kd = p.KI[r][cc] * gam;
        db[i] = dKG * p.KG[r][cc] - sKI[i] * p.KI[r][cc] + sQG[i] * p.QG[r][cc] - dKD * kd;
        eKD = fmaf(dKD, kd, eKD);
        dkh[i] = dKG * G + (sKI[i] + dKD * gam) * Gi;
        dqh[i] = a.scale * sQG[i] * G;
        qh[i] = r < c.len ? tq[i] * p.rq[r] : 0.f;
        kh[i] = r < c.len ? tk[i] * p.rk[r] : 0.f;
    }
    // l2norm: dq = (dq^ - q^ (q^ . dq^)) / |q|, likewise dk; row dots over the 16 lanes of a
    // row group, then over the eight wavefronts
    const bool l2_in = (a.flags & kBL2In) != 0;
    if (l2_in) {
        f32x4 pq = qh * dqh, pk = kh * dkh;
#pragma unroll
        for (int o = 8; o > 0; o >>= 1)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pq[i] += __shfl_xor(pq[i], o);
                pk[i] += __shfl_xor(pk[i], o);
            }
        if (m == 0)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                L.rowdot[4 * g + i][wave][0] = pq[i];
                L.rowdot[4 * g + i][wave][1] = pk[i];
            }
        __syncthreads();
    }
    // d log-decay: reverse cumulative sum of db over the chunk's rows (this lane's four, then the
    // row groups above it by lane exchange), plus the decay of the whole chunk
    // (dgamma gamma + sum_r dKD KD) on every row; then the gate's chain rule.
    float e = eKD;
    e += __shfl_xor(e, 16);
    e += __shfl_xor(e, 32);
    e += tdgam * gam;
    const float tot = (db[0] + db[1]) + (db[2] + db[3]);
    float above = 0.f;  // sum of the row groups g' > g
#pragma unroll
    for (int gg = 1; gg < 4; ++gg) {
        const float t = __shfl(tot, m + 16 * gg);
        above += gg > g ? t : 0.f;
    }
    const bool gate_in = (a.flags & kBGateIn) != 0;
    const float eA = gate_in ? expf(raw.A_log) : 0.f;
    float run = e + above;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
        const int r = 4 * g + i;
        run += db[i];
        if (r < c.len) {
            const size_t at = (tok0 + (size_t)r * (size_t)a.H) * kD + (size_t)cc;
            const float gc = tg[i];
            float dgv;
            if (gate_in) {
                const float sgm = __builtin_amdgcn_rcpf(1.0f + expf(-eA * (gc + dtb)));
                dgv = run * a.lower_bound * sgm * (1.0f - sgm) * eA;
            } else {
                dgv = (gc > a.lower_bound && gc < 0.f) ? run : 0.f;
            }
            a.dg[at] = dgv;
            float dq = dqh[i], dk = dkh[i];
            if (l2_in) {
                float dotq = 0.f, dotk = 0.f;
#pragma unroll
                for (int w = 0; w < kGradThreads / 64; w += 2) {
                    const f32x4 d = ld4(&L.rowdot[r][w][0]);  // waves w, w + 1
                    dotq += d[0];
                    dotk += d[1];
                    dotq += d[2];
                    dotk += d[3];
                }
                dq = (dq - qh[i] * dotq) * p.rq[r];
                dk = (dk - kh[i] * dotk) * p.rk[r];
            }
            a.dq[at] = dq;
            a.dk[at] = dk;
        }
    }
}

// ---- head reduction: ddt_bias[h][c] = sum_t dg, dA_log[h] = sum_{t,c} dg (g + dt_bias) ----
// dt_bias and A_log gradients: per head, sums over every token of dg (d log-decay) and of
// dg * (g + dt_bias) (the gate's pre-activation x = e^{A_log} (g + dt_bias) has dx/dA_log = x
// and the d log-decay / dx factor is already in dg).  Two passes with a fixed partition and a
// fixed order (deterministic): bwd_head_part_kernel sums kHeadSlices contiguous token ranges
// per head (thread -> four channels and every eighth token of the range, four tokens' 16-byte
// loads in flight at a time; the eight token lanes meet in LDS in order), bwd_head_kernel adds
// the slices in order.
__global__ __launch_bounds__(256) void bwd_head_part_kernel(BwdArgs a)
{
    __shared__ f32x4 s_d[8][kD / 4], s_a[8][kD / 4];
    const int h = blockIdx.x / kHeadSlices, slice = blockIdx.x % kHeadSlices;
    const int cq = threadIdx.x & (kD / 4 - 1), tl = threadIdx.x / (kD / 4);  // channels 4 cq .., token lane
    // with invalid cu_seqlens no token belongs to a sequence and dg is not written: sum nothing
    const int64_t ntok = *a.status ? 0 : a.B * a.T;
    const int64_t t0 = ntok * slice / kHeadSlices, t1 = ntok * (slice + 1) / kHeadSlices;
    const f32x4 dt = ld4(a.dt_bias + (size_t)h * kD + 4 * cq);
    const size_t rs = (size_t)a.H * kD;  // elements per token row
    const float *dgp = a.dg + (size_t)h * kD + 4 * cq;
    const uint16_t *gp = a.g + (size_t)h * kD + 4 * cq;
    f32x4 sd = {0.f, 0.f, 0.f, 0.f}, sa = sd;
    auto add = [&](f32x4 d, f32x4 gv) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sd[i] += d[i];
            sa[i] = fmaf(d[i], gv[i] + dt[i], sa[i]);
        }
    };
    int64_t t = t0 + tl;
    for (; t + 24 < t1; t += 32) {
        f32x4 d[4], gv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            d[u] = ld4(dgp + (size_t)(t + 8 * u) * rs);
            gv[u] = ld4_bf16(gp + (size_t)(t + 8 * u) * rs);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            add(d[u], gv[u]);
    }
    for (; t < t1; t += 8)
        add(ld4(dgp + (size_t)t * rs), ld4_bf16(gp + (size_t)t * rs));
    s_d[tl][cq] = sd;
    s_a[tl][cq] = sa;
    __syncthreads();
    if (tl == 0) {
        f32x4 td = s_d[0][cq], ta = s_a[0][cq];
#pragma unroll
        for (int k = 1; k < 8; ++k) {
            td += s_d[k][cq];
            ta += s_a[k][cq];
        }
        float *part = a.hpart + ((size_t)h * kHeadSlices + (size_t)slice) * 2 * kD;
        st4(part + 4 * cq, td);
        st4(part + kD + 4 * cq, ta);
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
    a.status = reinterpret_cast<const int32_t *>(ws + f.fwd.lay.off_status);
    a.ops = reinterpret_cast<float *>(ws + f.bl.off_ops);
    a.ck = reinterpret_cast<float *>(ws + f.bl.off_ck);
    a.xf = reinterpret_cast<float *>(ws + f.bl.off_xf);
    a.xb = reinterpret_cast<float *>(ws + f.bl.off_xb);
    a.hpart = reinterpret_cast<float *>(ws + f.bl.off_hpart);
    a.cinfo = reinterpret_cast<int32_t *>(ws + f.bl.off_cinfo);
    a.plen = f.bl.plen;
    a.trunc = (a.flags & kBL2In) && (a.flags & kBSigIn);
    a.poff = reinterpret_cast<int64_t *>(ws + f.bl.off_poff);
    a.pst = reinterpret_cast<float *>(ws + f.bl.off_pst);
    a.pnrm = reinterpret_cast<float *>(ws + f.bl.off_pnrm);
    a.pz = reinterpret_cast<int32_t *>(ws + f.bl.off_pz);
    const int64_t toks = a.B * a.T * a.H;
    const int64_t units = 2 * a.N * a.H;          // (chain, role)
    const int64_t slots = a.chunks * a.H;         // chunk-heads (a bound)
    auto check = [] { return hipGetLastError(); };
    hipError_t e;
    if (toks > 0) {
        hipLaunchKernelGGL(bwd_chunk_info_kernel, dim3((unsigned)cdiv(a.chunks, 256)), dim3(256), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
    }
    if (units > 0 && a.plen > 0) {
        hipLaunchKernelGGL(bwd_piece_table_kernel, dim3(1), dim3(256), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
    }
    if (toks > 0) {
        hipLaunchKernelGGL(bwd_ops_kernel, dim3((unsigned)slots), dim3(kGradThreads), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
    }
    if (units > 0 && a.plen > 0) {
        // cut plan: pass A, transition runs, scan, pass B; 2 workgroups per (piece, head,
        // direction), in groups of 8 (one per XCD)
        const unsigned grid = (unsigned)(cdiv(2 * f.bl.pieces * a.H, 8) * 16);
        hipLaunchKernelGGL((bwd_chain_kernel<1, kChA>), dim3(grid), dim3(kChainThreads), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
        hipLaunchKernelGGL((bwd_chain_kernel<1, kChT>), dim3(grid), dim3(kChainThreads), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
        hipLaunchKernelGGL(bwd_piece_scan_kernel, dim3((unsigned)(units * 8)), dim3(256), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
        hipLaunchKernelGGL((bwd_chain_kernel<1, kChB>), dim3(grid), dim3(kChainThreads), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
    } else if (units > 0) {
        // 2 kCh workgroups per unit, units in groups of 8 (one per XCD)
        if (units <= kChainUnitsSplit)
            hipLaunchKernelGGL((bwd_chain_kernel<2, kChWhole>), dim3((unsigned)(cdiv(units, 8) * 32)), dim3(kChainThreads), 0, s, a);
        else
            hipLaunchKernelGGL((bwd_chain_kernel<1, kChWhole>), dim3((unsigned)(cdiv(units, 8) * 16)), dim3(kChainThreads), 0, s, a);
        if ((e = check()) != hipSuccess)
            return e;
    }
    if (toks > 0) {
        hipLaunchKernelGGL(bwd_grad_kernel, dim3((unsigned)slots), dim3(kGradThreads), 0, s, a);
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
