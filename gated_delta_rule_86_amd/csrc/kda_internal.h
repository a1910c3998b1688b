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
// segment is affine in the state before it: S_end = S_begin P + F, with F the segment run
// from S = 0 and P the segment run from S = I with v = 0.  With G segments per chain the
// forward pass becomes: pass A (segment 0 exactly, and F, P of segments 1 .. G-2), an
// fp32 scan S_{g+1} = S_g P_g + F_g, and pass B (segments 1 .. G-1 from S_g, with out).
// That is three segment runs per chunk instead of one, in exchange for chains x G
// independent work units; the plan picks G by a cost count over the CUs.  Pass A's F and
// P units share the CUs that the chains' segment-0 units leave free, in rA rounds, so
// segment 0 can be longer than the others; the segment-0 units come first in pass A's
// launch order so that they start in its first wave.  Units that write out (segment 0,
// pass B) take about 5/4 the time per chunk of the output-free F and P runs (measured on
// the 2^20-token workload: 2.2-2.3 us against 1.8 us), so segment 0 is sized to
// L0 ~ (4/5) rA L.  That is done only with at least kLongSeg0Chains chains: measured with
// 32 chains (B=2 T=4096 H=16) pass A ran 10 % faster, but with 8 chains (B=1 T=2^20 H=8)
// the F and P units that shared the chip with 8 long segment-0 units ran about 30 % slower
// per chunk (pass A 7.3 -> 9.35 ms; segment 0 alone ran at the usual speed), for a cause
// not found; there every segment keeps the same length.
constexpr int64_t kPlanCUs = 256;   // MI355X compute units
constexpr int64_t kCostOut = 5, kCostFP = 4;
constexpr int64_t kLongSeg0Chains = 16;

struct SegPlan {
    int G;        // segments per chain (1 = no segmentation)
    int64_t L;    // chunks per segment 1 .. G-1 (the last may be shorter)
    int64_t L0;   // chunks of segment 0
};

inline SegPlan plan_segments(int64_t chains, int64_t nch)
{
    SegPlan best{1, nch, nch};
    if (chains <= 0 || nch < 32 || chains >= 192)
        return best;
    auto rounds = [](int64_t units, int64_t cus) { return (units + cus - 1) / cus; };
    int64_t best_cost = rounds(chains, kPlanCUs) * nch * kCostOut;
    for (int64_t G = 3; G <= 256 && G <= nch / 8; ++G) {
        const int64_t rA = rounds(2 * chains * (G - 2), kPlanCUs - chains);
        const int64_t rB = rounds(chains * (G - 1), kPlanCUs);
        // kCostOut L0 = kCostFP rA L with L0 + (G - 1) L = nch (or all equal: L0 <= L)
        const int64_t L = chains >= kLongSeg0Chains ? cdiv(nch * kCostOut, (G - 1) * kCostOut + rA * kCostFP)
                                                    : cdiv(nch, G);
        const int64_t L0 = nch - (G - 1) * L;
        if (L0 < 1)
            continue;
        // pass A, pass B, and the scan at about two chunk times per segment step
        const int64_t a0 = L0 * kCostOut, afp = rA * L * kCostFP;
        const int64_t cost = (a0 > afp ? a0 : afp) + rB * L * kCostOut + 2 * G * kCostOut;
        if (cost < best_cost) {
            best_cost = cost;
            best = SegPlan{(int)G, L, L0};
        }
    }
    return best;
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
    L->seg = varlen ? SegPlan{1, 0, 0} : plan_segments(N * H, cdiv(T, kCH));
    L->off_seg = off;
    if (L->seg.G > 1)
        off += 3 * (size_t)(N * H) * (size_t)L->seg.G * kD * kD * sizeof(float);
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
