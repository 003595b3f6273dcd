// kda_internal.h -- launch descriptors shared by the host API (kda_api.cpp)
// and the kernel translation units.  Arguments are validated by the host
// API before any launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
    int dk, dv, H, num_seqs;
    bool in_bf16, out_bf16;
    const void *q, *k, *v;
    const float *g, *beta;
    float* state;
    const int32_t* slots;
    void* out;
    float scale;
    hipStream_t stream;
};

struct PrefillArgs {
    int dk, dv, H, num_seqs;
    bool in_bf16, out_bf16;
    int64_t total_tokens;
    int64_t total_chunks;         // sum over sequences of ceil(L_b / chunk rows)
    const int32_t* cu_dev;        // [num_seqs + 1] device offsets
    const int32_t* start_dev;     // nullable: absolute position of each first token
    const int32_t* slots;         // nullable: state row of each sequence (init and final)
    const void *q, *k, *v;
    const float *g, *beta;
    const float* init;            // nullable
    bool init_if_started;         // read init only for sequences with start > 0
    void* out;
    float* final_state;
    int32_t interval;             // 0 = no snapshots
    float* snapshots;             // nullable when no snapshot is due
    void* workspace;
    size_t workspace_bytes;
    float scale;
    hipStream_t stream;
};

struct FrontendArgs {
    int H, dk, W, num_seqs;
    bool in_bf16, out_bf16;
    bool unit_lengths;            // cu[b] == b for every b (a decode step)
    int64_t total_tokens;
    const int32_t* cu_dev;        // [num_seqs + 1] device offsets
    const void* x[2];             // q, k inputs [T, H, dk]
    const float* w[2];            // taps [H * dk, W]
    const void* state_in[2];      // nullable, [num_slots, W-1, H, dk]
    void* state_out[2];           // nullable; may equal state_in
    const int32_t* slots;         // nullable (identity)
    void* y[2];                   // outputs [T, H, dk]
    float eps;
    hipStream_t stream;
};

struct DecodeMultiArgs {
    int dk, dv, H, num_seqs, num_tokens;
    int mode;                     // 0 apply, 1 verify, 2 commit, 3 commit then verify
    bool in_bf16, out_bf16;
    const void *q, *k, *v;        // [num_seqs, num_tokens, H, d]
    const float *g, *beta;
    const void *pk, *pv;          // mode 3: the previous step's tokens (same layout)
    const float *pg, *pbeta;
    float* state;
    const int32_t* slots;         // nullable (identity)
    const int32_t* counts;        // commit, step: accepted tokens per sequence
    void* out;                    // [num_seqs, num_tokens, H, dv]; unused in commit
    float scale;
    hipStream_t stream;
};

struct AttnResArgs {
    int hidden, num_sources;
    int64_t num_tokens;
    bool in_bf16, out_bf16;
    const void* sources[16];      // [T, hidden] each
    const void* x;                // [T, hidden] residual, nullable
    const float *w, *gamma;       // [hidden]; gamma nullable
    void *h, *y;                  // [T, hidden]; h nullable
    float scale, eps;
    hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs& a);
hipError_t launch_attnres(const AttnResArgs& a);
int attnres_max_hidden(int num_sources, bool in_bf16);
hipError_t launch_decode_multi(const DecodeMultiArgs& a);
// verify, commit and step with at most 8 tokens per sequence take the
// chunked form (launch_spec); apply and longer drafts walk the tokens
bool spec_chunked(const DecodeMultiArgs& a);
hipError_t launch_spec(const DecodeMultiArgs& a);
hipError_t launch_frontend(const FrontendArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);
size_t prefill_workspace_bytes(int dk, int dv, int H, int num_seqs, int64_t total_tokens,
                               bool any_start = false);
int prefill_chunk_rows();  // tokens per chunk; snapshot intervals are multiples of 64

// Sets the text kda_last_error_detail() returns on this thread (kda_api.cpp).
void set_error_detail(const char* msg);

}  // namespace kda
