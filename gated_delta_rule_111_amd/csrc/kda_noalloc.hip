// kda_noalloc.hip -- kda_prefill_noalloc: the chunked prefill with its chunk
// operands in a fixed device array instead of a caller-provided workspace,
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this translation unit's code object, so a GPU holds it
// (KDA_NOALLOC_SCRATCH_BYTES) from the first call on that GPU until the
// process ends.  Its device address is looked up once per device, with that
// device current, and kept; host code uses that address, never the array's
// name (which in host code is only a stand-in for the symbol).  Nothing here
// allocates: the entry point checks the size, then runs kda_prefill on the
// array.  Every call on one GPU shares that GPU's array, so calls that
// overlap on one GPU (two streams, two threads) race on it; nothing in it has
// to start at zero (the plan kernel writes every offset the other kernels
// read, and the prep kernel every operand the scan reads).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/kda.h"
#include "kda_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
void* g_scratch[MAX_DEVICES];
std::mutex g_scratch_mu;

// device address of this device's copy of the array (looked up on first use)
hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

kda_status report(kda_status st, const char* msg) {
    kda::set_error_detail(msg);
    return st;
}

}  // namespace

extern "C" kda_status kda_prefill_noalloc(const kda_config* cfg, int32_t num_seqs,
                                          const int32_t* cu_seqlens_host,
                                          const int32_t* cu_seqlens_dev, const void* q,
                                          const void* k, const void* v, const float* g,
                                          const float* beta, const float* initial_state,
                                          void* out, float* final_state,
                                          int32_t snapshot_interval, float* snapshots,
                                          void* stream) {
    // argument errors are reported by kda_prefill itself (an invalid config
    // or offsets give a size of 0, and a zero-sequence call is a no-op):
    // only a problem whose operands exceed the array is stopped here
    size_t need = 0;
    if (cfg && num_seqs > 0 && cu_seqlens_host)
        need = kda_prefill_workspace_size(cfg, num_seqs, (int64_t)cu_seqlens_host[num_seqs]);
    if (need > (size_t)KDA_NOALLOC_SCRATCH_BYTES) {
        char msg[256];
        snprintf(msg, sizeof(msg),
                 "kda_prefill_noalloc: this problem needs %zu bytes of chunk operands, the "
                 "fixed array holds %zu (KDA_NOALLOC_SCRATCH_BYTES); use kda_prefill with a "
                 "workspace, or split the call",
                 need, (size_t)KDA_NOALLOC_SCRATCH_BYTES);
        return report(KDA_ERR_WORKSPACE, msg);
    }
    void* ws = nullptr;
    if (need > 0) {
        const hipError_t e = scratch_address(&ws);
        if (e != hipSuccess) {
            char msg[256];
            snprintf(msg, sizeof(msg),
                     "kda_prefill_noalloc: no device address for the scratch array: %s",
                     hipGetErrorString(e));
            return report(KDA_ERR_HIP, msg);
        }
    }
    return kda_prefill(cfg, num_seqs, cu_seqlens_host, cu_seqlens_dev, q, k, v, g, beta,
                       initial_state, out, final_state, snapshot_interval, snapshots, ws,
                       ws ? (size_t)KDA_NOALLOC_SCRATCH_BYTES : 0, stream);
}
