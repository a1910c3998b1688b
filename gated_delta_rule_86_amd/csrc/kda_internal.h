// kda_internal.h -- workspace layout and launcher declarations shared by the host API
// (kda_api.cpp) and the gfx950 kernels (kda_kernels.hip).  Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace kda {

constexpr int kD = 128;   // head dim, K = V
constexpr int kCH = 16;   // tokens per chunk
constexpr int kVB = 16;   // value columns per state wave
constexpr int kNVB = kD / kVB;

// Per (chunk, head) record written by the prep kernel and read by the state kernel.
// Every block is stored in the exact register layout the state kernel's MFMA operands
// use, so that each lane fetches its operand with one 16-byte (or 8-byte) load.
constexpr size_t kRecKG = 0;       // K^*Gamma (hi), bf16, [4 channel pairs][64 lanes][8]
constexpr size_t kRecKGL = 4096;   // K^*Gamma (lo), same layout
constexpr size_t kRecQG = 8192;    // scale*q^*Gamma, bf16, same layout
constexpr size_t kRecKD = 12288;   // K^*gamma/Gamma (hi, lo bf16), [8 channel tiles][64 lanes][4+4]
constexpr size_t kRecGAM = 20480;  // gamma = Gamma at the chunk's last token, fp32 [128]
constexpr size_t kRecTB = 20992;   // T*diag(beta) (hi, lo bf16), [64 lanes][4+4]
constexpr size_t kRecMQ = 22016;   // A_qk*T*diag(beta) (hi, lo bf16), [64 lanes][4+4]
constexpr size_t kRecBytes = 23040;

constexpr size_t kAlign = 256;

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
    int64_t n_seq;     // N (or B without cu_seqlens)
    int64_t n_slots;   // chunk slots reserved per head (upper bound of the chunk count)
    size_t off_status; // int32 status word; int64 n_total at +8
    size_t off_seq_start, off_seq_len, off_seq_off;
    size_t off_recs;
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
    L->n_seq = N;
    L->n_slots = varlen ? cdiv(T, kCH) + N : B * cdiv(T, kCH);
    size_t off = 0;
    L->off_status = off;
    off += kAlign;
    L->off_seq_start = off;
    off = round_up(off + sizeof(int64_t) * (size_t)N, kAlign);
    L->off_seq_len = off;
    off = round_up(off + sizeof(int64_t) * (size_t)N, kAlign);
    L->off_seq_off = off;
    off = round_up(off + sizeof(int64_t) * (size_t)(N + 1), kAlign);
    L->off_recs = off;
    off += kRecBytes * (size_t)L->n_slots * (size_t)H;
    L->total = off;
    return true;
}

struct FwdArgs {
    const uint16_t *q, *k, *v, *g, *beta;
    uint16_t *out;
    const float *A_log, *dt_bias;
    float scale, lower_bound;
    const void *h0;
    void *ht;
    int h0_dtype, ht_dtype;  // 0 none, 1 bf16, 2 fp32
    const int64_t *cu;       // device, may be NULL
    int64_t B, T, H, N;
    unsigned char *ws;
    Layout lay;
};

hipError_t launch_chunk_table(const FwdArgs &a, hipStream_t s);
hipError_t launch_prep(const FwdArgs &a, hipStream_t s);
hipError_t launch_state(const FwdArgs &a, hipStream_t s);

}  // namespace kda
