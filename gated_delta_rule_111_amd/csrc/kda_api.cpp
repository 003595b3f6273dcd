// kda_api.cpp -- the C ABI of libkda (declared in include/kda.h): argument
// validation, problem planning and kernel launches.  Every check runs before
// anything is enqueued, so an error return has launched and written nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

thread_local char g_detail[512] = "";

kda_status fail(kda_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
    va_end(ap);
    return st;
}

kda_status ok() {
    g_detail[0] = '\0';
    return KDA_OK;
}

bool aligned(const void* p, uintptr_t bytes) {
    return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0;
}

kda_status check_config(const kda_config* cfg) {
    if (!cfg) return fail(KDA_ERR_INVALID_ARG, "cfg is NULL");
    if (cfg->num_heads <= 0) return fail(KDA_ERR_INVALID_ARG, "num_heads must be > 0");
    if (cfg->dk != cfg->dv)
        return fail(KDA_ERR_UNSUPPORTED, "dk (%d) != dv (%d) is not provided", cfg->dk, cfg->dv);
    if (cfg->dk != 16 && cfg->dk != 32 && cfg->dk != 64 && cfg->dk != 128)
        return fail(KDA_ERR_UNSUPPORTED, "head dim %d not in {16, 32, 64, 128}", cfg->dk);
    if (cfg->in_dtype != KDA_BF16 && cfg->in_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype %d unknown", (int)cfg->in_dtype);
    if (cfg->out_dtype != KDA_BF16 && cfg->out_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "out_dtype %d unknown", (int)cfg->out_dtype);
    if (!std::isfinite(cfg->scale) || cfg->scale < 0.f)
        return fail(KDA_ERR_INVALID_ARG, "scale must be finite and >= 0");
    return KDA_OK;
}

float effective_scale(const kda_config* cfg) {
    return cfg->scale > 0.f ? cfg->scale : (float)(1.0 / std::sqrt((double)cfg->dk));
}

struct PtrCheck {
    const char* name;
    const void* p;
    bool required;
    uintptr_t align;  // tensors read with 128-bit accesses need 16; scalar arrays 4
};

kda_status check_ptrs(const PtrCheck* list, int n) {
    for (int i = 0; i < n; ++i) {
        if (!list[i].p) {
            if (list[i].required)
                return fail(KDA_ERR_INVALID_ARG, "%s is NULL", list[i].name);
            continue;
        }
        if (!aligned(list[i].p, list[i].align))
            return fail(KDA_ERR_ALIGNMENT, "%s is not %d-byte aligned", list[i].name,
                        (int)list[i].align);
    }
    return KDA_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const char* pa = static_cast<const char*>(a);
    const char* pb = static_cast<const char*>(b);
    return pa < pb + nb && pb < pa + na;
}

size_t dtype_bytes(kda_dtype d) { return d == KDA_BF16 ? 2 : 4; }

}  // namespace

namespace kda {
void set_error_detail(const char* msg) { snprintf(g_detail, sizeof(g_detail), "%s", msg); }
}  // namespace kda

extern "C" {

int32_t kda_version(void) { return KDA_VERSION; }

const char* kda_status_string(kda_status status) {
    switch (status) {
        case KDA_OK: return "KDA_OK";
        case KDA_ERR_INVALID_ARG: return "KDA_ERR_INVALID_ARG";
        case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
        case KDA_ERR_ALIGNMENT: return "KDA_ERR_ALIGNMENT";
        case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
        case KDA_ERR_HIP: return "KDA_ERR_HIP";
    }
    return "KDA_ERR_UNKNOWN";
}

const char* kda_last_error_detail(void) { return g_detail; }

int64_t kda_snapshot_count(const int32_t* cu, int32_t num_seqs, int32_t interval) {
    if (!cu || num_seqs < 0) return -1;
    if (interval <= 0) return 0;
    int64_t n = 0;
    for (int32_t b = 0; b < num_seqs; ++b) {
        if (cu[b + 1] < cu[b]) return -1;
        n += (int64_t)(cu[b + 1] - cu[b]) / interval;
    }
    return n;
}

size_t kda_prefill_workspace_size(const kda_config* cfg, int32_t num_seqs, int64_t total_tokens) {
    if (check_config(cfg) != KDA_OK || num_seqs < 0 || total_tokens < 0) return 0;
    return kda::prefill_workspace_bytes(cfg->dk, cfg->dv, cfg->num_heads, num_seqs, total_tokens);
}

int64_t kda_snapshot_count_at(const int32_t* cu, const int32_t* start, int32_t num_seqs,
                              int32_t interval) {
    if (!cu || !start || num_seqs < 0) return -1;
    if (interval <= 0) return 0;
    int64_t n = 0;
    for (int32_t b = 0; b < num_seqs; ++b) {
        if (cu[b + 1] < cu[b] || start[b] < 0) return -1;
        const int64_t s0 = start[b], L = cu[b + 1] - cu[b];
        n += (s0 + L) / interval - s0 / interval;
    }
    return n;
}

size_t kda_prefill_pool_workspace_size(const kda_config* cfg, int32_t num_seqs,
                                       int64_t total_tokens) {
    if (check_config(cfg) != KDA_OK || num_seqs < 0 || total_tokens < 0) return 0;
    return kda::prefill_workspace_bytes(cfg->dk, cfg->dv, cfg->num_heads, num_seqs, total_tokens,
                                        true);
}

}  // extern "C"

namespace {

// Both prefill entry points: without start positions (chunks from each
// sequence's first token, snapshots every `interval` tokens of the call, the
// initial and final states in rows b of two arrays), and over a state pool
// (absolute start positions, slots).
struct PrefillCall {
    const int32_t *cu_host, *cu_dev;
    const int32_t *start_host, *start_dev;  // null without start positions
    const void *q, *k, *v;
    const float *g, *beta;
    const float* init;
    bool init_if_started;
    const int32_t* slots;
    int32_t num_slots;                      // rows of init / final (pool), else num_seqs
    void* out;
    float* final_state;
    int32_t interval;
    float* snapshots;
    void* workspace;
    size_t workspace_bytes;
    void* stream;
};

kda_status prefill_impl(const kda_config* cfg, int32_t num_seqs, const PrefillCall& c) {
    kda_status st = check_config(cfg);
    if (st != KDA_OK) return st;
    if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 0");
    if (num_seqs == 0) return ok();
    const int32_t* cu_host = c.cu_host;
    if (!cu_host) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
    if (cu_host[0] != 0) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
    if (cfg->num_heads > 65535)
        return fail(KDA_ERR_UNSUPPORTED, "num_heads %d exceeds 65535", cfg->num_heads);
    const bool pool = c.start_host != nullptr;
    const int64_t crow = kda::prefill_chunk_rows();
    int64_t total_chunks = 0;
    for (int32_t b = 0; b < num_seqs; ++b) {
        if (cu_host[b + 1] < cu_host[b])
            return fail(KDA_ERR_INVALID_ARG, "cu_seqlens decreases at index %d", b + 1);
        const int64_t L = cu_host[b + 1] - cu_host[b];
        const int64_t s0 = pool ? c.start_host[b] : 0;
        if (s0 < 0 || s0 + L > 0x7fffffffLL)
            return fail(KDA_ERR_INVALID_ARG, "start_pos[%d] = %lld out of range", b, (long long)s0);
        total_chunks += L > 0 ? (s0 % crow + L + crow - 1) / crow : 0;
    }
    const int64_t T = cu_host[num_seqs];
    // one prep workgroup per (chunk, head) and one scan workgroup per
    // (sequence, head, 16 value columns): both grids must fit a launch
    if (total_chunks * cfg->num_heads > 0x7fffffffLL)
        return fail(KDA_ERR_UNSUPPORTED, "%lld chunks x %d heads exceed one launch grid",
                    (long long)total_chunks, cfg->num_heads);
    if (((int64_t)num_seqs * cfg->num_heads + 7) / 8 * 8 * (cfg->dv / 16) > 0x7fffffffLL)
        return fail(KDA_ERR_UNSUPPORTED, "%d sequences x %d heads exceed one launch grid",
                    num_seqs, cfg->num_heads);
    if (c.interval < 0 || c.interval % 64 != 0)
        return fail(KDA_ERR_INVALID_ARG, "snapshot_interval %d is not a non-negative multiple of 64",
                    c.interval);
    const int64_t nsnap = pool ? kda_snapshot_count_at(cu_host, c.start_host, num_seqs, c.interval)
                               : kda_snapshot_count(cu_host, num_seqs, c.interval);
    const bool tok = T > 0;
    const PtrCheck ptrs[] = {
        {"cu_seqlens_dev", c.cu_dev, true, 4},
        {"start_pos_dev", c.start_dev, pool, 4},
        {"q", c.q, tok, 16},
        {"k", c.k, tok, 16},
        {"v", c.v, tok, 16},
        {"g", c.g, tok, 16},
        {"beta", c.beta, tok, 4},
        {pool ? "state_pool" : "initial_state", c.init, pool, 16},
        {"state_slots_dev", c.slots, false, 4},
        {"out", c.out, tok, 16},
        {pool ? "state_pool" : "final_state", c.final_state, true, 16},
        {"snapshots", c.snapshots, nsnap > 0, 16},
        {"workspace", c.workspace, false, 16},
    };
    st = check_ptrs(ptrs, (int)(sizeof(ptrs) / sizeof(ptrs[0])));
    if (st != KDA_OK) return st;
    if (pool) {
        if (c.num_slots < 1 || (!c.slots && c.num_slots < num_seqs))
            return fail(KDA_ERR_INVALID_ARG, "num_slots %d too small for %d sequences", c.num_slots,
                        num_seqs);
    } else if (c.init && c.init != c.final_state) {
        // final_state may alias initial_state exactly; partial overlap is not allowed
        const size_t bytes = (size_t)num_seqs * cfg->num_heads * cfg->dk * cfg->dv * sizeof(float);
        const char* a = reinterpret_cast<const char*>(c.init);
        const char* b = reinterpret_cast<const char*>(c.final_state);
        if (a < b + bytes && b < a + bytes)
            return fail(KDA_ERR_INVALID_ARG, "final_state partially overlaps initial_state");
    }
    const size_t need =
        kda::prefill_workspace_bytes(cfg->dk, cfg->dv, cfg->num_heads, num_seqs, T, pool);
    if (c.workspace_bytes < need || (need > 0 && !c.workspace))
        return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu required",
                    c.workspace_bytes, need);

    kda::PrefillArgs a{};
    a.dk = cfg->dk;
    a.dv = cfg->dv;
    a.H = cfg->num_heads;
    a.num_seqs = num_seqs;
    a.in_bf16 = cfg->in_dtype == KDA_BF16;
    a.out_bf16 = cfg->out_dtype == KDA_BF16;
    a.total_tokens = T;
    a.total_chunks = total_chunks;
    a.cu_dev = c.cu_dev;
    a.start_dev = c.start_dev;
    a.slots = c.slots;
    a.q = c.q;
    a.k = c.k;
    a.v = c.v;
    a.g = c.g;
    a.beta = c.beta;
    a.init = c.init;
    a.init_if_started = c.init_if_started;
    a.out = c.out;
    a.final_state = c.final_state;
    a.interval = c.interval;
    a.snapshots = c.snapshots;
    a.workspace = c.workspace;
    a.workspace_bytes = c.workspace_bytes;
    a.scale = effective_scale(cfg);
    a.stream = static_cast<hipStream_t>(c.stream);
    hipError_t e = kda::launch_prefill(a);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

extern "C" {

kda_status kda_prefill(const kda_config* cfg, int32_t num_seqs, const int32_t* cu_host,
                       const int32_t* cu_dev, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, const float* initial_state, void* out,
                       float* final_state, int32_t snapshot_interval, float* snapshots,
                       void* workspace, size_t workspace_bytes, void* stream) {
    PrefillCall c{};
    c.cu_host = cu_host;
    c.cu_dev = cu_dev;
    c.q = q;
    c.k = k;
    c.v = v;
    c.g = g;
    c.beta = beta;
    c.init = initial_state;
    c.num_slots = num_seqs;
    c.out = out;
    c.final_state = final_state;
    c.interval = snapshot_interval;
    c.snapshots = snapshots;
    c.workspace = workspace;
    c.workspace_bytes = workspace_bytes;
    c.stream = stream;
    return prefill_impl(cfg, num_seqs, c);
}

kda_status kda_prefill_pool(const kda_config* cfg, int32_t num_seqs, const int32_t* cu_host,
                            const int32_t* cu_dev, const int32_t* start_host,
                            const int32_t* start_dev, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, float* state_pool,
                            const int32_t* slots, int32_t num_slots, void* out,
                            int32_t snapshot_interval, float* snapshots, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (num_seqs > 0 && !start_host)
        return fail(KDA_ERR_INVALID_ARG, "start_pos_host is NULL");
    PrefillCall c{};
    c.cu_host = cu_host;
    c.cu_dev = cu_dev;
    c.start_host = start_host;
    c.start_dev = start_dev;
    c.q = q;
    c.k = k;
    c.v = v;
    c.g = g;
    c.beta = beta;
    c.init = state_pool;
    c.init_if_started = true;
    c.slots = slots;
    c.num_slots = num_slots;
    c.out = out;
    c.final_state = state_pool;
    c.interval = snapshot_interval;
    c.snapshots = snapshots;
    c.workspace = workspace;
    c.workspace_bytes = workspace_bytes;
    c.stream = stream;
    return prefill_impl(cfg, num_seqs, c);
}

kda_status kda_decode(const kda_config* cfg, int32_t num_seqs, const void* q, const void* k,
                      const void* v, const float* g, const float* beta, float* state,
                      const int32_t* slots, void* out, void* stream) {
    kda_status st = check_config(cfg);
    if (st != KDA_OK) return st;
    if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 0");
    if (num_seqs == 0) return ok();
    if ((int64_t)num_seqs * cfg->num_heads > 0x7fffffffLL)
        return fail(KDA_ERR_UNSUPPORTED, "num_seqs * num_heads exceeds the grid limit");
    const PtrCheck ptrs[] = {
        {"q", q, true, 16},     {"k", k, true, 16},         {"v", v, true, 16},
        {"g", g, true, 16},     {"beta", beta, true, 4},    {"state", state, true, 16},
        {"state_slots_dev", slots, false, 4},               {"out", out, true, 16},
    };
    st = check_ptrs(ptrs, (int)(sizeof(ptrs) / sizeof(ptrs[0])));
    if (st != KDA_OK) return st;

    kda::DecodeArgs a{};
    a.dk = cfg->dk;
    a.dv = cfg->dv;
    a.H = cfg->num_heads;
    a.num_seqs = num_seqs;
    a.in_bf16 = cfg->in_dtype == KDA_BF16;
    a.out_bf16 = cfg->out_dtype == KDA_BF16;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.slots = slots;
    a.out = out;
    a.scale = effective_scale(cfg);
    a.stream = static_cast<hipStream_t>(stream);
    hipError_t e = kda::launch_decode(a);
    if (e != hipSuccess) return fail(KDA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

kda_status kda_decode_multi(const kda_config* cfg, int32_t num_seqs, int32_t num_tokens,
                            kda_multi_mode mode, const void* q, const void* k, const void* v,
                            const float* g, const float* beta, float* state, const int32_t* slots,
                            const int32_t* accepted, void* out, void* stream) {
    kda_status st = check_config(cfg);
    if (st != KDA_OK) return st;
    if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 0");
    if (num_tokens < 1) return fail(KDA_ERR_INVALID_ARG, "num_tokens must be >= 1");
    if (mode != KDA_MULTI_APPLY && mode != KDA_MULTI_VERIFY && mode != KDA_MULTI_COMMIT)
        return fail(KDA_ERR_INVALID_ARG, "mode %d unknown", (int)mode);
    if (num_seqs == 0) return ok();
    if ((int64_t)num_seqs * cfg->num_heads > 0x7fffffffLL)
        return fail(KDA_ERR_UNSUPPORTED, "num_seqs * num_heads exceeds the grid limit");
    const bool outputs = mode != KDA_MULTI_COMMIT;
    const PtrCheck ptrs[] = {
        {"q", q, outputs, 16},  {"k", k, true, 16},         {"v", v, true, 16},
        {"g", g, true, 16},     {"beta", beta, true, 4},    {"state", state, true, 16},
        {"state_slots_dev", slots, false, 4},
        {"accepted_dev", accepted, mode == KDA_MULTI_COMMIT, 4},
        {"out", out, outputs, 16},
    };
    st = check_ptrs(ptrs, (int)(sizeof(ptrs) / sizeof(ptrs[0])));
    if (st != KDA_OK) return st;

    kda::DecodeMultiArgs a{};
    a.dk = cfg->dk;
    a.dv = cfg->dv;
    a.H = cfg->num_heads;
    a.num_seqs = num_seqs;
    a.num_tokens = num_tokens;
    a.mode = (int)mode;
    a.in_bf16 = cfg->in_dtype == KDA_BF16;
    a.out_bf16 = cfg->out_dtype == KDA_BF16;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.state = state;
    a.slots = slots;
    a.counts = mode == KDA_MULTI_COMMIT ? accepted : nullptr;
    a.out = outputs ? out : nullptr;
    a.scale = effective_scale(cfg);
    a.stream = static_cast<hipStream_t>(stream);
    hipError_t e = kda::spec_chunked(a) ? kda::launch_spec(a) : kda::launch_decode_multi(a);
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "multi-token decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

kda_status kda_decode_spec_step(const kda_config* cfg, int32_t num_seqs, int32_t num_tokens,
                                const void* prev_k, const void* prev_v, const float* prev_g,
                                const float* prev_beta, const int32_t* accepted, const void* q,
                                const void* k, const void* v, const float* g, const float* beta,
                                float* state, const int32_t* slots, void* out, void* stream) {
    kda_status st = check_config(cfg);
    if (st != KDA_OK) return st;
    if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 0");
    if (num_tokens < 1) return fail(KDA_ERR_INVALID_ARG, "num_tokens must be >= 1");
    if (num_seqs == 0) return ok();
    if ((int64_t)num_seqs * cfg->num_heads > 0x7fffffffLL)
        return fail(KDA_ERR_UNSUPPORTED, "num_seqs * num_heads exceeds the grid limit");
    const bool commit = accepted != nullptr;
    const PtrCheck ptrs[] = {
        {"prev_k", prev_k, commit, 16},       {"prev_v", prev_v, commit, 16},
        {"prev_g", prev_g, commit, 16},       {"prev_beta", prev_beta, commit, 4},
        {"accepted_dev", accepted, false, 4}, {"q", q, true, 16},
        {"k", k, true, 16},                   {"v", v, true, 16},
        {"g", g, true, 16},                   {"beta", beta, true, 4},
        {"state", state, true, 16},           {"state_slots_dev", slots, false, 4},
        {"out", out, true, 16},
    };
    st = check_ptrs(ptrs, (int)(sizeof(ptrs) / sizeof(ptrs[0])));
    if (st != KDA_OK) return st;

    kda::DecodeMultiArgs a{};
    a.dk = cfg->dk;
    a.dv = cfg->dv;
    a.H = cfg->num_heads;
    a.num_seqs = num_seqs;
    a.num_tokens = num_tokens;
    a.mode = commit ? 3 : 1;
    a.in_bf16 = cfg->in_dtype == KDA_BF16;
    a.out_bf16 = cfg->out_dtype == KDA_BF16;
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.pk = prev_k;
    a.pv = prev_v;
    a.pg = prev_g;
    a.pbeta = prev_beta;
    a.state = state;
    a.slots = slots;
    a.counts = accepted;
    a.out = out;
    a.scale = effective_scale(cfg);
    a.stream = static_cast<hipStream_t>(stream);
    hipError_t e = kda::spec_chunked(a) ? kda::launch_spec(a) : kda::launch_decode_multi(a);
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "speculative step launch failed: %s", hipGetErrorString(e));
    return ok();
}

kda_status kda_qk_frontend(const kda_frontend_config* cfg, int32_t num_seqs,
                           const int32_t* cu_host, const int32_t* cu_dev, const void* xq,
                           const void* xk, const float* wq, const float* wk,
                           const void* state_in_q, const void* state_in_k, void* state_out_q,
                           void* state_out_k, const int32_t* slots, int32_t num_slots,
                           void* q_out, void* k_out, void* stream) {
    if (!cfg) return fail(KDA_ERR_INVALID_ARG, "cfg is NULL");
    if (cfg->num_heads <= 0 || cfg->num_heads > 65535)
        return fail(KDA_ERR_INVALID_ARG, "num_heads %d not in [1, 65535]", cfg->num_heads);
    if (cfg->dk != 16 && cfg->dk != 32 && cfg->dk != 64 && cfg->dk != 128)
        return fail(KDA_ERR_UNSUPPORTED, "head dim %d not in {16, 32, 64, 128}", cfg->dk);
    if (cfg->conv_width < 1 || cfg->conv_width > 8)
        return fail(KDA_ERR_UNSUPPORTED, "conv_width %d not in [1, 8]", cfg->conv_width);
    if (cfg->in_dtype != KDA_BF16 && cfg->in_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype %d unknown", (int)cfg->in_dtype);
    if (cfg->out_dtype != KDA_BF16 && cfg->out_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "out_dtype %d unknown", (int)cfg->out_dtype);
    if (!std::isfinite(cfg->eps) || !(cfg->eps > 0.f))
        return fail(KDA_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "num_seqs must be >= 0");
    if (num_seqs == 0) return ok();
    if (!cu_host) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens_host is NULL");
    if (cu_host[0] != 0) return fail(KDA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
    bool unit = true;  // every sequence has exactly one token (a decode step)
    for (int32_t b = 0; b < num_seqs; ++b) {
        if (cu_host[b + 1] < cu_host[b])
            return fail(KDA_ERR_INVALID_ARG, "cu_seqlens decreases at index %d", b + 1);
        unit = unit && cu_host[b + 1] == b + 1;
    }
    const int64_t T = cu_host[num_seqs];
    const int W = cfg->conv_width;
    const bool tok = T > 0;
    const bool stateful = W > 1 && (state_in_q || state_in_k || state_out_q || state_out_k);
    const PtrCheck ptrs[] = {
        {"cu_seqlens_dev", cu_dev, true, 4},
        {"xq", xq, tok, 16},
        {"xk", xk, tok, 16},
        {"wq", wq, true, 16},
        {"wk", wk, true, 16},
        {"conv_state_in_q", state_in_q, false, 16},
        {"conv_state_in_k", state_in_k, false, 16},
        {"conv_state_out_q", state_out_q, false, 16},
        {"conv_state_out_k", state_out_k, false, 16},
        {"state_slots_dev", slots, false, 4},
        {"q_out", q_out, tok, 16},
        {"k_out", k_out, tok, 16},
    };
    kda_status st = check_ptrs(ptrs, (int)(sizeof(ptrs) / sizeof(ptrs[0])));
    if (st != KDA_OK) return st;
    if (stateful) {
        if (num_slots < 1) return fail(KDA_ERR_INVALID_ARG, "num_slots must be >= 1");
        if (!slots && num_slots < num_seqs)
            return fail(KDA_ERR_INVALID_ARG, "num_slots %d < num_seqs %d without state_slots_dev",
                        num_slots, num_seqs);
    }
    const size_t C = (size_t)cfg->num_heads * cfg->dk;
    const size_t xb = (size_t)T * C * dtype_bytes(cfg->in_dtype);
    const size_t yb = (size_t)T * C * dtype_bytes(cfg->out_dtype);
    const size_t sb = stateful ? (size_t)num_slots * (W - 1) * C * dtype_bytes(cfg->in_dtype) : 0;
    const void* outs[2] = {q_out, k_out};
    const void* ins[2] = {xq, xk};
    const void* sins[2] = {state_in_q, state_in_k};
    void* souts[2] = {state_out_q, state_out_k};
    for (int i = 0; i < 2; ++i) {
        for (int j = 0; j < 2; ++j)
            if (overlap(outs[i], yb, ins[j], xb))
                return fail(KDA_ERR_INVALID_ARG, "an output overlaps an input");
        if (sins[i] != souts[i] && overlap(sins[i], sb, souts[i], sb))
            return fail(KDA_ERR_INVALID_ARG, "a state output partially overlaps its input");
        if (overlap(souts[i], sb, outs[0], yb) || overlap(souts[i], sb, outs[1], yb) ||
            overlap(souts[i], sb, ins[0], xb) || overlap(souts[i], sb, ins[1], xb))
            return fail(KDA_ERR_INVALID_ARG, "a state output overlaps a token tensor");
    }
    if (overlap(q_out, yb, k_out, yb)) return fail(KDA_ERR_INVALID_ARG, "q_out overlaps k_out");
    if (overlap(state_out_q, sb, state_out_k, sb) ||
        overlap(state_out_q, sb, state_in_k, sb) || overlap(state_out_k, sb, state_in_q, sb))
        return fail(KDA_ERR_INVALID_ARG, "the q and k states overlap");

    kda::FrontendArgs a{};
    a.H = cfg->num_heads;
    a.dk = cfg->dk;
    a.W = W;
    a.num_seqs = num_seqs;
    a.in_bf16 = cfg->in_dtype == KDA_BF16;
    a.out_bf16 = cfg->out_dtype == KDA_BF16;
    a.unit_lengths = unit;
    a.total_tokens = T;
    a.cu_dev = cu_dev;
    a.x[0] = xq;
    a.x[1] = xk;
    a.w[0] = wq;
    a.w[1] = wk;
    a.state_in[0] = W > 1 ? state_in_q : nullptr;
    a.state_in[1] = W > 1 ? state_in_k : nullptr;
    a.state_out[0] = W > 1 ? state_out_q : nullptr;
    a.state_out[1] = W > 1 ? state_out_k : nullptr;
    a.slots = slots;
    a.y[0] = q_out;
    a.y[1] = k_out;
    a.eps = cfg->eps;
    a.stream = static_cast<hipStream_t>(stream);
    hipError_t e = kda::launch_frontend(a);
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "front-end launch failed: %s", hipGetErrorString(e));
    return ok();
}

kda_status kda_attnres(const kda_attnres_config* cfg, int64_t num_tokens,
                       const void* const* sources, const void* residual, const float* query,
                       const float* gamma, void* h_out, void* y_out, void* stream) {
    if (!cfg) return fail(KDA_ERR_INVALID_ARG, "cfg is NULL");
    const int M = cfg->num_sources, d = cfg->hidden;
    if (M < 1 || M > 16) return fail(KDA_ERR_UNSUPPORTED, "num_sources %d not in [1, 16]", M);
    if (cfg->in_dtype != KDA_BF16 && cfg->in_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "in_dtype %d unknown", (int)cfg->in_dtype);
    const int dmax = kda::attnres_max_hidden(M, cfg->in_dtype == KDA_BF16);
    if (d < 16 || d % 16 != 0 || d > dmax)
        return fail(KDA_ERR_UNSUPPORTED, "hidden %d not a multiple of 16 in [16, %d]", d, dmax);
    if (cfg->out_dtype != KDA_BF16 && cfg->out_dtype != KDA_F32)
        return fail(KDA_ERR_UNSUPPORTED, "out_dtype %d unknown", (int)cfg->out_dtype);
    if (!std::isfinite(cfg->logit_scale))
        return fail(KDA_ERR_INVALID_ARG, "logit_scale must be finite");
    if (!std::isfinite(cfg->eps) || !(cfg->eps > 0.f))
        return fail(KDA_ERR_INVALID_ARG, "eps must be finite and > 0");
    if (num_tokens < 0 || num_tokens > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "num_tokens %lld out of range", (long long)num_tokens);
    if (num_tokens == 0) return ok();
    if (!sources) return fail(KDA_ERR_INVALID_ARG, "sources_host is NULL");
    const PtrCheck ptrs[] = {
        {"residual", residual, false, 16}, {"query", query, true, 16},
        {"gamma", gamma, false, 16},       {"h_out", h_out, false, 16},
        {"y_out", y_out, true, 16},
    };
    kda_status st = check_ptrs(ptrs, (int)(sizeof(ptrs) / sizeof(ptrs[0])));
    if (st != KDA_OK) return st;
    const size_t ib = (size_t)num_tokens * d * dtype_bytes(cfg->in_dtype);
    const size_t ob = (size_t)num_tokens * d * dtype_bytes(cfg->out_dtype);
    for (int m = 0; m < M; ++m) {
        if (!sources[m]) return fail(KDA_ERR_INVALID_ARG, "sources[%d] is NULL", m);
        if (!aligned(sources[m], 16))
            return fail(KDA_ERR_ALIGNMENT, "sources[%d] is not 16-byte aligned", m);
        if (overlap(y_out, ob, sources[m], ib) || overlap(h_out, ob, sources[m], ib))
            return fail(KDA_ERR_INVALID_ARG, "an output overlaps sources[%d]", m);
    }
    if (overlap(y_out, ob, residual, ib) || overlap(h_out, ob, residual, ib) ||
        overlap(y_out, ob, h_out, ob))
        return fail(KDA_ERR_INVALID_ARG, "outputs overlap the residual or each other");

    kda::AttnResArgs a{};
    a.hidden = d;
    a.num_sources = M;
    a.num_tokens = num_tokens;
    a.in_bf16 = cfg->in_dtype == KDA_BF16;
    a.out_bf16 = cfg->out_dtype == KDA_BF16;
    for (int m = 0; m < M; ++m) a.sources[m] = sources[m];
    a.x = residual;
    a.w = query;
    a.gamma = gamma;
    a.h = h_out;
    a.y = y_out;
    a.scale = cfg->logit_scale;
    a.eps = cfg->eps;
    a.stream = static_cast<hipStream_t>(stream);
    hipError_t e = kda::launch_attnres(a);
    if (e != hipSuccess)
        return fail(KDA_ERR_HIP, "attnres launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // extern "C"
