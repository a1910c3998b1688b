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

// Cut plan (long sequences: batch rows or varlen).  The P workgroups of a head take equal
// runs of the head's chunk list (its sequences one after another, in index order): run w
// covers chunks [x_w, x_{w+1}) with x_j = floor(j C / P), C the head's chunk count, and a
// cut x_j moved to the nearest sequence boundary when one lies within
// min(kSnapChunks, C / (4P)) chunks.  A cut inside a sequence splits it into pieces; the
// state after a piece is affine in the state before it: S_end = S_begin Phi + F, with F
// the piece run from S = 0 and Phi its transition (the run from S = I with v = 0).  The
// forward pass runs:
//   pass A:   the P runs of every head, each piece with out: a piece starting a sequence
//             from the true initial state, one starting at a cut from S = 0; end states go
//             to final_state, to S_j (the exact state at the sequence's first cut) or to F_j,
//             with their norms.
//   transition runs, one per (head, cut inside a sequence): from I with v = 0.  With the
//             in-kernel l2norm and beta sigmoid every token's transition
//             diag(alpha)(I - beta k^ k^T) has spectral norm <= 1, so |S_j|_F <= B_j = |S_j0|_F
//             + |F_j0|_F + ... + |F_{j-1}|_F (j0 the sequence's first cut), and once every
//             entry of the run's state is below kTruncRel |F_j|_F / B_j after z chunks,
//             S_j's share of every later state of the piece is below 2^-30 |F_j|_F.  The
//             run stops there and records z; otherwise it runs the whole piece and keeps
//             Phi_j.
//   scan:     S_{j+1} = F_j where the run stopped (that share dropped), else
//             S_{j+1} = S_j Phi_j + F_j, for consecutive cuts inside one sequence.
//   pass B:   every piece starting at a cut again from S_j, with out: only the first z
//             chunks where the share was dropped (pass A's out is right from there on),
//             else all of them; a piece that ends its sequence writes final_state.
// With a strong gate (the transition falls below 2^-40 within 2 - 5 chunks at lower bounds
// -5 .. -2) that is about one run per chunk, over P runs per head; with weak or no decay
// every run goes the whole way (three runs per chunk of a cut sequence).  The plan is taken
// when the heads leave at least two workgroups each and sequences are long on average
// (many short ones are better balanced whole, see the whole-chain plans below); runs are
// at least kSegMinChunks chunks long.
constexpr int64_t kPlanCUs = 256;   // MI355X compute units
constexpr int64_t kSegMinChunks = 16;
constexpr int64_t kCutMinAvg = 64;  // average chunks per sequence for the cut plan
constexpr int64_t kSnapChunks = 8;
constexpr float kTruncRel = 0x1p-37f;  // 2^-30 / 128

// Workgroups per head of the cut plan (1: whole-chain plans).  C is the head's chunk count
// for batch rows, its lower bound ceil(T / 16) for varlen.
inline int64_t plan_cuts(int64_t B, int64_t T, int64_t H, int64_t N, bool varlen)
{
    if (H < 1 || H > kPlanCUs / 2)
        return 1;
    const int64_t nseq = varlen ? N : B;
    const int64_t C = varlen ? cdiv(T, kCH) : B * cdiv(T, kCH);
    if (nseq < 1 || C < nseq * kCutMinAvg)
        return 1;
    int64_t P = kPlanCUs / H;
    if (P > C / kSegMinChunks)
        P = C / kSegMinChunks;
    return P >= 2 ? P : 1;
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
// from a split), whole chains (no cut plan), few sequences and workgroups per head.
// The chunk table plans halves and the forward launch picks the kernel instance that runs
// them under this same condition.
inline bool split_plan(int64_t H, int64_t n_seq, int64_t cutP, bool varlen)
{
    return varlen && cutP <= 1 && split_eligible(H, n_seq);
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
    size_t off_cut;    // int32 cut_seq, cut_off, cut_first [kPlanCUs + 1] each: the cut plan
    int64_t cutP;      // workgroups per head of the cut plan (1: whole-chain plans)
    size_t off_seg;    // fp32 states S, F, P: 3 x [H][P][128][128] when cutP > 1
    size_t off_segaux; // when cutP > 1: int32 z [H][P], int32 drop [H][P], fp32 squared
                       // norms of S_j and of F_j [H][P][4] each
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
    L->off_cut = off;
    off = round_up(off + sizeof(int32_t) * 3 * (size_t)(kPlanCUs + 1), kAlign);
    L->cutP = plan_cuts(B, T, H, N, varlen);
    L->off_seg = off;
    L->off_segaux = off;
    if (L->cutP > 1) {
        const size_t slots = (size_t)H * (size_t)L->cutP;
        off += 3 * slots * kD * kD * sizeof(float);
        L->off_segaux = off;
        off = round_up(off + slots * (2 * sizeof(int32_t) + 8 * sizeof(float)), kAlign);
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
// the cut-plan states, which the backward pass does not use), then per chunk-head (chunk x of
// the head's chunk list, slot x H + h) the chain kernels' operand block (kBwdOps fp32), one
// state (fp32 128 x 128, in a tiled layout of the backward kernels: the state before the chunk
// for the even chunks of a sequence, dL/dS after it for the odd ones), the chunk's corrected
// values V' and their gradient (fp32 16 x 128 each, tiled likewise); and the per-head gradient
// partial sums (fp32 [H][kHeadSlices][2][128]).
constexpr int kHeadSlices = 64;  // token slices of the backward pass's per-head gradient sums
// operand block of one chunk-head: -W, U, KD, QG^T (2048 fp32 each), lower(QG KI^T) (256),
// gamma (128)
constexpr int kBwdOps = 4 * kCH * kD + kCH * kCH + kD;

// Backward cut plan.  Both chains of the backward pass are affine in their carried matrix:
// the state forwards, S' = S A_j + U_j^T KD_j with A_j = Diag(gamma_j) - W_j^T KD_j, and dL/dS
// backwards, D' = D A_j^T + dO_j^T (QG_j - A_qk,j W_j).  Where the chains are few and long, a
// sequence is cut into pieces of L chunks (the last one shorter) and, per (sequence, head,
// direction), its pieces in walk order w = 0 .. P-1 (chunk order forwards, reversed
// backwards) run as the forward pass's cut plan:
//   pass A:      every piece with its outputs; w = 0 from the true start (initial state, or
//                dL/dS_final), the others from zero; end states and their norms kept;
//   transitions: every piece w >= 1 from I with zero inputs.  A_j^T has the norms of A_j, so
//                the forward plan's bound holds: with the in-kernel l2norm and sigmoid the run
//                stops once every entry is below kTruncRel |F_w|_F / B_w, with B_w = |st_1|_F +
//                |F_1|_F + ... + |F_{w-1}|_F, and records z (the chunks it ran);
//   scan:        st_{w+1} = F_w where the run stopped, else st_w Phi_w + F_w (fp32);
//   pass B:      every piece w >= 1 again from st_w with its outputs: the first z chunks where
//                the run stopped (pass A's outputs are right from there on), else all of it.
// The whole-chain kernel is latency-bound where the chains are few: the plan is taken when
// sequences average kBwdCutMinAvg chunks or more and pass A then has about kBwdTargetWgs
// workgroups (two per piece and direction; 768 = three per CU, one round: pass A is bound by
// HBM either way, and fewer pieces shorten the transition runs, the scan and pass B), pieces
// of at least kBwdPieceMin chunks and two or more pieces per sequence on average.
constexpr int64_t kBwdCutMinAvg = 64;
constexpr int64_t kBwdPieceMin = 8;
constexpr int64_t kBwdTargetWgs = 768;

// Chunks per piece of the backward cut plan, 0 for whole chains (chunks: the chunk-count
// bound of a head; nseq: sequences).
inline int64_t bwd_piece_len(int64_t chunks, int64_t nseq, int64_t H)
{
    if (nseq < 1 || H < 1 || chunks < nseq * kBwdCutMinAvg)
        return 0;
    int64_t L = cdiv(chunks * H * 4, kBwdTargetWgs);
    if (L < kBwdPieceMin)
        L = kBwdPieceMin;
    return chunks >= 2 * L * nseq ? L : 0;
}

struct BwdLayout {
    Layout tab;
    int64_t chunks;  // bound on the chunk count of a head (the slots per head)
    int64_t plen;    // cut plan: chunks per piece (0: whole chains)
    int64_t pieces;  // cut plan: bound on the pieces of a head
    size_t off_ops, off_ck, off_xf, off_xb, off_hpart, off_cinfo;
    size_t off_poff, off_pst, off_pnrm, off_pz;  // cut plan (0 without)
    size_t total;
};

inline bool make_bwd_layout(int64_t B, int64_t T, int64_t H, int64_t N, bool varlen, BwdLayout *L)
{
    if (!make_layout(B, T, H, N, varlen, &L->tab))
        return false;
    const size_t state = (size_t)kD * kD * sizeof(float);
    L->chunks = varlen ? cdiv(T, kCH) + L->tab.n_seq : B * cdiv(T, kCH);
    const size_t ch = (size_t)L->chunks * (size_t)H;  // chunk-head slots
    size_t off = L->tab.off_seg;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = round_up(off + bytes, kAlign);
        return o;
    };
    L->off_ops = take(ch * kBwdOps * sizeof(float));
    L->off_ck = take(ch * state);
    L->off_xf = take(ch * kCH * kD * sizeof(float));
    L->off_xb = take(ch * kCH * kD * sizeof(float));
    L->off_hpart = take((size_t)H * kHeadSlices * 2 * kD * sizeof(float));
    L->off_cinfo = take((size_t)L->chunks * 4 * sizeof(int32_t));  // where each chunk lies
    L->plen = bwd_piece_len(L->chunks, L->tab.n_seq, H);
    L->pieces = 0;
    L->off_poff = L->off_pst = L->off_pnrm = L->off_pz = 0;
    if (L->plen > 0) {
        // per sequence max(1, ceil(chunks / L)) pieces: at most chunks / L + 1 each
        L->pieces = cdiv(L->chunks, L->plen) + L->tab.n_seq;
        const size_t pu = (size_t)L->pieces * (size_t)H * 2;  // (piece, head, direction) slots
        L->off_poff = take((size_t)(L->tab.n_seq + 1) * sizeof(int64_t));
        L->off_pst = take(pu * 3 * state);  // start state, F, Phi
        L->off_pnrm = take(pu * 8 * sizeof(float));
        L->off_pz = take(pu * 4 * sizeof(int32_t));
    }
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
