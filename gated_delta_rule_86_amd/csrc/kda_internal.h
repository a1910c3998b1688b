// kda_internal.h -- workspace layout and launcher declarations shared by the host API
// (kda_api.cpp) and the gfx950 kernels (kda_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kda {

constexpr int kD = 128;   // head dim, K = V
constexpr int kCH = 16;   // tokens per chunk
constexpr size_t kAlign = 256;

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Segment plan for few, long, equal-length chains (no cu_seqlens).  The state after a
// segment is affine in the state before it: S_end = S_begin Phi + F, with F the segment run
// from S = 0 and Phi the segment's transition (the run from S = I with v = 0).  A chain is
// cut into G segments of L chunks (the last one shorter), and the forward pass runs:
//   pass A:   segment 0 from the true initial state and segments 1 .. G-1 from S = 0, all
//             with out; the end states S_1 and F_g and their norms.
//   transition runs, segments 1 .. G-1: from I with v = 0.  With the in-kernel l2norm and
//             beta sigmoid every token's transition diag(alpha)(I - beta k^ k^T) has
//             spectral norm <= 1, so |S_g|_F <= B_g = |S_1|_F + |F_1|_F + ... + |F_{g-1}|_F,
//             and once every entry of the run's state is below kTruncRel |F_g|_F / B_g
//             after z chunks, S_g's share of every later state of the segment is below
//             2^-30 |F_g|_F.  The run stops there and records z; otherwise it runs the whole
//             segment and keeps Phi_g.
//   scan:     S_{g+1} = F_g where the run stopped (that share dropped), else
//             S_{g+1} = S_g Phi_g + F_g.
//   pass B:   segments 1 .. G-1 again from S_g, with out: only the first z chunks where the
//             share was dropped (pass A's out is right from there on), else all of them.
// With a strong gate (the transition falls below 2^-40 within 2 - 4 chunks at lower bounds
// -5 .. -2) that is about one segment run per chunk over chains x G units; with weak or no
// decay every run goes the whole way (three segment runs per chunk).  G fills the CUs with
// one round of pass A units of at least kSegMinChunks chunks each.
constexpr int64_t kPlanCUs = 256;   // MI355X compute units
constexpr int64_t kSegMinChunks = 16;
constexpr float kTruncRel = 0x1p-37f;  // 2^-30 / 128

struct SegPlan {
    int G;        // segments per chain (1 = no segmentation)
    int64_t L;    // chunks per segment (the last may be shorter)
};

inline SegPlan plan_segments(int64_t chains, int64_t nch)
{
    const SegPlan none{1, nch};
    if (chains <= 0 || chains > kPlanCUs / 2)
        return none;
    int64_t G = kPlanCUs / chains;
    if (G > nch / kSegMinChunks)
        G = nch / kSegMinChunks;
    while (G >= 2 && (G - 1) * cdiv(nch, G) >= nch)  // no empty segment
        --G;
    if (G < 2)
        return none;
    return SegPlan{(int)G, cdiv(nch, G)};
}

// Column halves.  When a head has few workgroups and few sequences, the chunk table may run
// a long sequence as two units of 64 value columns each: the producer work per chunk is
// the same, the consumers' halves, and a half unit takes about 0.82 of a whole one.  The
// units of a head then go to its workgroups longest first, each to the least loaded one.
constexpr int64_t kSplitMaxP = 16;     // at most this many workgroups per head
constexpr int64_t kSplitMaxSeq = 32;   // at most this many sequences
constexpr int kSplitMaxK = 8;          // at most this many sequences split
constexpr int64_t kWholeW = 100, kHalfW = 82;

inline bool split_eligible(int64_t H, int64_t n_seq)
{
    return kPlanCUs / H <= kSplitMaxP && n_seq <= kSplitMaxSeq;
}

// The whole-chain launch may run column halves: varlen (equal-length batch rows never gain
// from a split), whole chains (no segment plan), few sequences and workgroups per head.
// The chunk table plans halves and the forward launch picks the kernel instance that runs
// them under this same condition.
inline bool split_plan(int64_t H, int64_t n_seq, int seg_G, bool varlen)
{
    return varlen && seg_G <= 1 && split_eligible(H, n_seq);
}

// Workgroups per head of the whole-chain launch: about one workgroup per CU over all
// heads, never more than the units (the sequences, or twice that where halves may be used).
inline int64_t whole_chain_groups(int64_t H, int64_t n_seq, bool varlen)
{
    int64_t p = kPlanCUs / H;
    if (p < 1)
        p = 1;
    const int64_t units = varlen && split_eligible(H, n_seq) ? 2 * n_seq : n_seq;
    if (p > units)
        p = units;
    return p < 1 ? 1 : p;
}

struct Layout {
    int64_t n_seq;     // N (or B without cu_seqlens)
    size_t off_status; // int32 status word; int64 n_total at +8
    size_t off_seq_start, off_seq_len, off_seq_off;
    size_t off_wg;     // int64 [kPlanCUs + 1]: first unit of each whole-chain workgroup of a head
    size_t off_units;  // int32 [2 N]: whole-chain units, (sequence << 2) | (0 whole, 1 + column half)
    SegPlan seg;       // segment plan (G == 1 without segmentation)
    size_t off_seg;    // fp32 states S, F, P: 3 x [chains][G][128][128] when G > 1
    size_t off_segaux; // when G > 1: int32 z [chains][G], int32 drop [chains][G],
                       // fp32 squared norms [chains][G][4]
    size_t total;
};

// Returns false for invalid sizes.
inline bool make_layout(int64_t B, int64_t T, int64_t H, int64_t N, bool varlen, Layout *L)
{
    if (B < 1 || T < 0 || H < 1)
        return false;
    if (varlen) {
        if (B != 1 || N < 1)
            return false;
    } else {
        if (N != 0 && N != B)
            return false;
        N = B;
    }
    if (N >= ((int64_t)1 << 29))  // unit codes hold the sequence index in 29 bits
        return false;
    L->n_seq = N;
    size_t off = 0;
    L->off_status = off;
    off += kAlign;
    L->off_seq_start = off;
    off = round_up(off + sizeof(int64_t) * (size_t)N, kAlign);
    L->off_seq_len = off;
    off = round_up(off + sizeof(int64_t) * (size_t)N, kAlign);
    L->off_seq_off = off;
    off = round_up(off + sizeof(int64_t) * (size_t)(N + 1), kAlign);
    L->off_wg = off;
    off = round_up(off + sizeof(int64_t) * (size_t)(kPlanCUs + 1), kAlign);
    L->off_units = off;
    off = round_up(off + sizeof(int32_t) * 2 * (size_t)N, kAlign);
    L->seg = varlen ? SegPlan{1, 0} : plan_segments(N * H, cdiv(T, kCH));
    L->off_seg = off;
    L->off_segaux = off;
    if (L->seg.G > 1) {
        const size_t units = (size_t)(N * H) * (size_t)L->seg.G;
        off += 3 * units * kD * kD * sizeof(float);
        L->off_segaux = off;
        off = round_up(off + units * (2 * sizeof(int32_t) + 4 * sizeof(float)), kAlign);
    }
    L->total = off;
    return true;
}

struct FwdArgs {
    const uint16_t *q, *k, *v, *g, *beta;
    uint16_t *out;
    const float *A_log, *dt_bias;
    float scale, lower_bound;
    int flags;               // activation switches (KDA_*_IN_KERNEL bits of include/kda.h)
    const void *h0;
    void *ht;
    int h0_dtype, ht_dtype;  // 0 none, 1 bf16, 2 fp32
    const int64_t *cu;       // device, may be NULL
    int64_t B, T, H, N;
    unsigned char *ws;
    Layout lay;
};

// Workspace of the backward pass: the chunk table (as the forward pass lays it out, up to
// the segment states, which the backward pass does not use), then per token-head the
// activated k^, q^ and alpha (fp32 [tokens][H][128]) and 1/|k|, 1/|q|, beta (fp32
// [tokens][H]), the state before every 16-token chunk of every chain (fp32 128 x 128 each),
// and one 16-state buffer per chain for the chunk being reversed.
struct BwdLayout {
    Layout tab;
    size_t off_kn, off_qn, off_al, off_rk, off_rq, off_bt, off_ckpt, off_buf;
    size_t total;
};

inline bool make_bwd_layout(int64_t B, int64_t T, int64_t H, int64_t N, bool varlen, BwdLayout *L)
{
    if (!make_layout(B, T, H, N, varlen, &L->tab))
        return false;
    const size_t tok = (size_t)B * (size_t)T * (size_t)H;
    const size_t state = (size_t)kD * kD * sizeof(float);
    const size_t chunks = varlen ? (size_t)cdiv(T, kCH) + (size_t)L->tab.n_seq : (size_t)B * (size_t)cdiv(T, kCH);
    size_t off = L->tab.off_seg;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = round_up(off + bytes, kAlign);
        return o;
    };
    L->off_kn = take(tok * kD * sizeof(float));
    L->off_qn = take(tok * kD * sizeof(float));
    L->off_al = take(tok * kD * sizeof(float));
    L->off_rk = take(tok * sizeof(float));
    L->off_rq = take(tok * sizeof(float));
    L->off_bt = take(tok * sizeof(float));
    L->off_ckpt = take(chunks * (size_t)H * state);
    L->off_buf = take((size_t)L->tab.n_seq * (size_t)H * kCH * state);
    L->total = off;
    return true;
}

struct BwdLaunch {
    FwdArgs fwd;  // inputs, activation switches, workspace (fwd.lay = bl.tab)
    BwdLayout bl;
    const uint16_t *dout;  // bf16 [B, T, H, 128]
    const float *dht;      // fp32 [N, H, 128, 128] or NULL
    float *dq, *dk, *dv, *dg, *dbeta, *dA_log, *ddt, *dh0;
};

// plan: also write the whole-chain workgroup plan (the forward pass reads it; the
// token-by-token path does not)
hipError_t launch_chunk_table(const FwdArgs &a, hipStream_t s, bool plan = true);
hipError_t launch_forward(const FwdArgs &a, hipStream_t s, hipEvent_t const *marks);
// token-by-token evaluation, one workgroup per chain (kda_recurrent.hip)
hipError_t launch_recurrent(const FwdArgs &a, hipStream_t s);
// gradients (kda_backward.hip); the chunk table must have been launched first
hipError_t launch_backward(const BwdLaunch &a, hipStream_t s);

}  // namespace kda
