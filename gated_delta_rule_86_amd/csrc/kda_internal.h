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

struct Layout {
    int64_t n_seq;     // N (or B without cu_seqlens)
    size_t off_status; // int32 status word; int64 n_total at +8
    size_t off_seq_start, off_seq_len, off_seq_off;
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
    size_t off = 0;
    L->off_status = off;
    off += kAlign;
    L->off_seq_start = off;
    off = round_up(off + sizeof(int64_t) * (size_t)N, kAlign);
    L->off_seq_len = off;
    off = round_up(off + sizeof(int64_t) * (size_t)N, kAlign);
    L->off_seq_off = off;
    off = round_up(off + sizeof(int64_t) * (size_t)(N + 1), kAlign);
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
hipError_t launch_fused(const FwdArgs &a, hipStream_t s);

}  // namespace kda
