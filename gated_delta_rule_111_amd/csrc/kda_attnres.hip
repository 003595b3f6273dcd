// kda_attnres.hip -- Attention Residuals aggregation: a layer's input as a
// softmax-weighted sum of earlier block outputs, plus the residual, then
// RMSNorm, in one launch.  gfx950.
//
// "Kimi K3 technical FAQ" (Runpod guide), question "What does the
// architecture actually look like?": each layer can attend over the
// embedding plus the preceding block outputs through a learned pseudo-query
// (the block variant, blocks of 12 layers, about 8 blocks).  "Day-0 vLLM
// support for Kimi K3" (vLLM blog), section "Kimi K3's architecture, and how
// vLLM serves it": one fused kernel computes the logits, the softmax across
// the previous layers and the aggregation, with the residual add and the
// output RMSNorm folded in.  Per token t, sources s_m (m < M):
//   l_m = scale <w, s_m,t>,  p = softmax(l),  h = sum_m p_m s_m,t + x_t,
//   y = h / sqrt(mean(h^2) + eps) * gamma.
//
// The op is bound by HBM: every source row is read once.  Design: a
// workgroup per token at a time; thread i holds channels 8i .. 8i+7 of every
// source in registers (one 16-byte load per bf16 source), so the logits (M
// dot products over the hidden dimension, reduced across the workgroup) and
// the weighted sum use the same registers without a second read.  Two
// workgroup reductions per token: the M logits, then the sum of squares.
// Only one such workgroup fits a compute unit at d = 7168, so the launch has
// one workgroup per resident slot, each walking tokens with the next token's
// rows requested before the current token's reductions.
#include <algorithm>
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int AR_MAX_SOURCES = 16;
constexpr int AR_MAX_THREADS = 1024;
// bf16 rows of two tokens (the current one and the next one in flight) fit
// 128 VGPRs, so 16-wave workgroups, for up to 9 sources; fp32 rows (one token
// at a time) for up to 10.  More sources take 8-wave workgroups with room
// for 256 VGPRs.
constexpr int ar_max_threads(int M, bool bf16) { return M <= (bf16 ? 9 : 10) ? 1024 : 512; }

struct ArParams {
    const void* src[AR_MAX_SOURCES];  // [T, d] each
    const void* x;                    // [T, d] or null
    const float* w;                   // [d]
    const float* gamma;               // [d] or null
    void* h;                          // [T, d] or null
    void* y;                          // [T, d]
    int d;
    float scale, eps;
};

// EPT consecutive values as fp32
template <int EPT>
__device__ __forceinline__ void widen(const uint4 (&r)[EPT / 8], float (&v)[EPT]) {
#pragma unroll
    for (int q = 0; q < EPT / 8; ++q) {
        const uint32_t u[4] = {r[q].x, r[q].y, r[q].z, r[q].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[8 * q + 2 * i] = bf16_bits_to_f32(u[i] & 0xffffu);
            v[8 * q + 2 * i + 1] = bf16_bits_to_f32(u[i] >> 16);
        }
    }
}

// raw row slices: bf16 keeps EPT/8 uint4, fp32 keeps EPT/4 float4
template <typename T, int EPT> struct Slice;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <int EPT> struct Slice<bf16_t, EPT> {
    uint4 r[EPT / 8];
    __device__ __forceinline__ void load(const bf16_t* p) {
#pragma unroll
        for (int q = 0; q < EPT / 8; ++q) {  // streamed once: kept out of the caches
            const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + q);
            r[q] = make_uint4(t[0], t[1], t[2], t[3]);
        }
    }
    __device__ __forceinline__ void get(float (&v)[EPT]) const { widen<EPT>(r, v); }
    // an empty asm that claims to rewrite the packed registers: the fp32
    // values widened before it cannot be reused after it, so they are not
    // kept alive (8 registers per slice) until their second use
    __device__ __forceinline__ void fence() {
#pragma unroll
        for (int q = 0; q < EPT / 8; ++q)
            asm volatile("" : "+v"(r[q].x), "+v"(r[q].y), "+v"(r[q].z), "+v"(r[q].w));
    }
};
template <int EPT> struct Slice<float, EPT> {
    float4 r[EPT / 4];
    __device__ __forceinline__ void load(const float* p) {
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q) r[q] = reinterpret_cast<const float4*>(p)[q];
    }
    __device__ __forceinline__ void get(float (&v)[EPT]) const {
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q) {
            v[4 * q] = r[q].x; v[4 * q + 1] = r[q].y; v[4 * q + 2] = r[q].z; v[4 * q + 3] = r[q].w;
        }
    }
    __device__ __forceinline__ void fence() {}
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// one row slice.  A workgroup that walks many tokens streams its h and y
// past the caches: nontemporal buffer stores through a resource at the
// token's row (T = 8192, d = 7168, 8 sources: 240 -> 234 us); with one token
// per workgroup ordinary stores are faster (9.6 against 10.4 us at T = 256).
// (Buffer stores, because two plain stores that differ only in the
// nontemporal hint get merged into one without it.)
template <int EPT>
__device__ __forceinline__ void pack_row(const float (&v)[EPT], u32x4_t (&o)[EPT / 8]) {
#pragma unroll
    for (int q = 0; q < EPT / 8; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x2_t pr = {v[8 * q + 2 * i], v[8 * q + 2 * i + 1]};
            o[q][i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2_t));
        }
}
template <int EPT>
__device__ __forceinline__ void store_row(bf16_t* p, const float (&v)[EPT]) {
    u32x4_t o[EPT / 8];
    pack_row<EPT>(v, o);
#pragma unroll
    for (int q = 0; q < EPT / 8; ++q) reinterpret_cast<u32x4_t*>(p)[q] = o[q];
}
template <int EPT>
__device__ __forceinline__ void store_row(float* p, const float (&v)[EPT]) {
#pragma unroll
    for (int q = 0; q < EPT / 4; ++q)
        reinterpret_cast<float4*>(p)[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
}
constexpr int AR_NT = 2;  // cache policy of a buffer store: nontemporal
// row: the token's row (uniform); c: this thread's first channel
template <int EPT>
__device__ __forceinline__ void stream_row(bf16_t* row, int d, int c, const float (&v)[EPT]) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(row, 0, d * 2, 0x00020000);
    u32x4_t o[EPT / 8];
    pack_row<EPT>(v, o);
#pragma unroll
    for (int q = 0; q < EPT / 8; ++q) __builtin_amdgcn_raw_buffer_store_b128(o[q], r, 2 * c + 16 * q, 0, AR_NT);
}
template <int EPT>
__device__ __forceinline__ void stream_row(float* row, int d, int c, const float (&v)[EPT]) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(row, 0, d * 4, 0x00020000);
#pragma unroll
    for (int q = 0; q < EPT / 4; ++q) {
        const u32x4_t o = {__float_as_uint(v[4 * q]), __float_as_uint(v[4 * q + 1]),
                           __float_as_uint(v[4 * q + 2]), __float_as_uint(v[4 * q + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(o, r, 4 * c + 16 * q, 0, AR_NT);
    }
}

template <int M, typename TIn, typename TOut>
__global__ __launch_bounds__(ar_max_threads(M, sizeof(TIn) == 2))
void attnres_kernel(ArParams p, int64_t T) {
    constexpr int EPT = 8;  // channels per thread: one 16-byte load per bf16 source
    __shared__ float red[AR_MAX_THREADS / 64][M + 1];
    __shared__ float res[M + 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nw = blockDim.x >> 6;
    const int d = p.d;
    const int c0 = EPT * tid;
    const bool live = c0 < d;          // threads past the row hold zeros
    const int cc = live ? c0 : 0;

    // The query and gamma slices are copied to LDS once (dynamic LDS of
    // 2 x blockDim.x x EPT floats) and read there at their use in every
    // token: that keeps two tokens' rows within the register budget, and an
    // LDS read does not wait on the vector-memory counter, which the loads of
    // the next token's rows hold (vector-memory operations complete in issue
    // order, so waiting for a load issued after them waits for them too).
    // Each thread reads back only the slices it wrote: no barrier.
    extern __shared__ __align__(16) float qg[];
    auto stage = [&]() {
        const float4* wq = reinterpret_cast<const float4*>(p.w + cc);
        const float4* gq = reinterpret_cast<const float4*>((p.gamma ? p.gamma : p.w) + cc);
        float4* dq = reinterpret_cast<float4*>(&qg[EPT * tid]);
        float4* dg = reinterpret_cast<float4*>(&qg[EPT * (blockDim.x + tid)]);
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q) {
            dq[q] = wq[q];
            dg[q] = gq[q];
        }
    };
    auto slice4 = [&](int which, float (&v)[EPT]) {
        const float* src = &qg[EPT * (which * blockDim.x + tid)];
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q) {
            const float4 t = reinterpret_cast<const float4*>(src)[q];
            v[4 * q] = t.x; v[4 * q + 1] = t.y; v[4 * q + 2] = t.z; v[4 * q + 3] = t.w;
        }
    };

    // one token's rows: every source slice and the residual slice
    struct Rows {
        Slice<TIn, EPT> s[M];
        Slice<TIn, EPT> x;
    };
    // The row loads are unconditional: a token past the end loads the rows
    // of t_else (a token this workgroup has just loaded, so cache hits) and
    // a missing residual reads source 0, unused.  A load under a branch
    // would leave the compiler copying its registers where the paths join,
    // which waits for the load to land and undoes the prefetch.
    const TIn* xs = static_cast<const TIn*>(p.x ? p.x : p.src[0]);
    auto fetch = [&](Rows& r, int64_t t, int64_t t_else) {
        const int64_t row = (t < T ? t : t_else) * d + cc;
#pragma unroll
        for (int m = 0; m < M; ++m) r.s[m].load(static_cast<const TIn*>(p.src[m]) + row);
        r.x.load(xs + row);
    };

    // stream_tag: std::true_type when this workgroup walks several tokens
    auto token = [&](Rows& r, int64_t t, auto stream_tag) {
        constexpr bool stream = decltype(stream_tag)::value;
        // logits: per-thread partial dot products, then across the workgroup
        float w[EPT];
        slice4(0, w);
        float part[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float v[EPT];
            r.s[m].get(v);
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < EPT; ++i) acc = fmaf(w[i], v[i], acc);
            part[m] = live ? acc : 0.f;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) r.s[m].fence();
#pragma unroll
        for (int m = 0; m < M; ++m) part[m] = wave_sum(part[m]);
        if (lane == 0) {
#pragma unroll
            for (int m = 0; m < M; ++m) red[wave][m] = part[m];
        }
        __barrier(__CLK_LOCAL_MEM_FENCE);
        if (tid < M) {
            float s = 0.f;
            for (int i = 0; i < nw; ++i) s += red[i][tid];
            res[tid] = s * p.scale;
        }
        __barrier(__CLK_LOCAL_MEM_FENCE);

        // softmax over the sources (every thread, from the shared logits)
        float pr[M];
        float mx = res[0];
#pragma unroll
        for (int m = 1; m < M; ++m) mx = fmaxf(mx, res[m]);
        float z = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            pr[m] = __expf(res[m] - mx);
            z += pr[m];
        }
        const float iz = 1.f / z;

        // h = sum_m p_m s_m + x
        float h[EPT];
        if (p.x) {
            r.x.get(h);
        } else {
#pragma unroll
            for (int i = 0; i < EPT; ++i) h[i] = 0.f;
        }
#pragma unroll
        for (int m = 0; m < M; ++m) {
            float v[EPT];
            r.s[m].get(v);
            const float pm = pr[m] * iz;
#pragma unroll
            for (int i = 0; i < EPT; ++i) h[i] = fmaf(pm, v[i], h[i]);
        }
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < EPT; ++i) ss = fmaf(h[i], h[i], ss);
        ss = wave_sum(live ? ss : 0.f);
        if (lane == 0) red[wave][M] = ss;
        __barrier(__CLK_LOCAL_MEM_FENCE);
        if (tid == 0) {
            float s = 0.f;
            for (int i = 0; i < nw; ++i) s += red[i][M];
            res[M] = rsqrtf(s / (float)d + p.eps);
        }
        __barrier(__CLK_LOCAL_MEM_FENCE);
        if (live) {
            const float rr = res[M];
            const int64_t orow = t * d + c0;
            if (p.h) {
                if constexpr (stream)
                    stream_row<EPT>(static_cast<TOut*>(p.h) + t * d, d, c0, h);
                else
                    store_row<EPT>(static_cast<TOut*>(p.h) + orow, h);
            }
            float yv[EPT];
            if (p.gamma) {
                float gm[EPT];
                slice4(1, gm);
#pragma unroll
                for (int i = 0; i < EPT; ++i) yv[i] = h[i] * rr * gm[i];
            } else {
#pragma unroll
                for (int i = 0; i < EPT; ++i) yv[i] = h[i] * rr;
            }
            if constexpr (stream)
                stream_row<EPT>(static_cast<TOut*>(p.y) + t * d, d, c0, yv);
            else
                store_row<EPT>(static_cast<TOut*>(p.y) + orow, yv);
        }
    };

    // tokens blockIdx.x, + gridDim.x, ...: with bf16 rows the next token's
    // rows are requested before the current one is reduced (two register
    // sets used in turn, so nothing loaded is copied); fp32 rows, twice the
    // registers, go one token at a time.  The workgroup barriers inside a
    // token leave loads in flight (they order LDS only).
    const int64_t step = gridDim.x;
    int64_t t = blockIdx.x;
    Rows ra;
    if constexpr (sizeof(TIn) == 2) {
        Rows rb;
        fetch(ra, t, t);
        stage();
        if (t + step >= T) {  // one token for this workgroup
            token(ra, t, std::false_type{});
            return;
        }
        for (; t < T; t += 2 * step) {
            fetch(rb, t + step, t);  // past the end: the current rows again (cache hits)
            token(ra, t, std::true_type{});
            if (t + step >= T) break;
            fetch(ra, t + 2 * step, t + step);
            token(rb, t + step, std::true_type{});
        }
    } else {
        stage();
        if (t + step >= T) {
            fetch(ra, t, t);
            token(ra, t, std::false_type{});
            return;
        }
        for (; t < T; t += step) {
            fetch(ra, t, t);
            token(ra, t, std::true_type{});
        }
    }
}

// compute units of the current device (asked on every launch: the library
// keeps no state between calls)
int compute_units() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        n > 0)
        return n;
    return 256;
}

template <int M, typename TIn, typename TOut>
hipError_t launch_m(const ArParams& p, int64_t T, hipStream_t stream) {
    constexpr int EPT = 8;
    const int threads = (p.d / EPT + 63) / 64 * 64;
    // as many workgroups as are resident at once; each walks its tokens
    const size_t lds = 2 * sizeof(float) * EPT * threads;  // query and gamma slices
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attnres_kernel<M, TIn, TOut>,
                                                     threads, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const int64_t grid = std::min<int64_t>(T, (int64_t)per_cu * compute_units());
    hipLaunchKernelGGL((attnres_kernel<M, TIn, TOut>), dim3((unsigned)grid), dim3(threads), lds,
                       stream, p, T);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_t(const ArParams& p, int M, int64_t T, hipStream_t stream) {
    switch (M) {
        case 1: return launch_m<1, TIn, TOut>(p, T, stream);
        case 2: return launch_m<2, TIn, TOut>(p, T, stream);
        case 3: return launch_m<3, TIn, TOut>(p, T, stream);
        case 4: return launch_m<4, TIn, TOut>(p, T, stream);
        case 5: return launch_m<5, TIn, TOut>(p, T, stream);
        case 6: return launch_m<6, TIn, TOut>(p, T, stream);
        case 7: return launch_m<7, TIn, TOut>(p, T, stream);
        case 8: return launch_m<8, TIn, TOut>(p, T, stream);
        case 9: return launch_m<9, TIn, TOut>(p, T, stream);
        case 10: return launch_m<10, TIn, TOut>(p, T, stream);
        case 11: return launch_m<11, TIn, TOut>(p, T, stream);
        case 12: return launch_m<12, TIn, TOut>(p, T, stream);
        case 13: return launch_m<13, TIn, TOut>(p, T, stream);
        case 14: return launch_m<14, TIn, TOut>(p, T, stream);
        case 15: return launch_m<15, TIn, TOut>(p, T, stream);
        case 16: return launch_m<16, TIn, TOut>(p, T, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

int attnres_max_hidden(int num_sources, bool in_bf16) {
    return 8 * ar_max_threads(num_sources, in_bf16);
}

hipError_t launch_attnres(const AttnResArgs& a) {
    ArParams p{};
    for (int m = 0; m < a.num_sources; ++m) p.src[m] = a.sources[m];
    p.x = a.x;
    p.w = a.w;
    p.gamma = a.gamma;
    p.h = a.h;
    p.y = a.y;
    p.d = a.hidden;
    p.scale = a.scale;
    p.eps = a.eps;
    if (a.num_tokens == 0) return hipSuccess;
    if (a.in_bf16)
        return a.out_bf16 ? launch_t<bf16_t, bf16_t>(p, a.num_sources, a.num_tokens, a.stream)
                          : launch_t<bf16_t, float>(p, a.num_sources, a.num_tokens, a.stream);
    return a.out_bf16 ? launch_t<float, bf16_t>(p, a.num_sources, a.num_tokens, a.stream)
                      : launch_t<float, float>(p, a.num_sources, a.num_tokens, a.stream);
}

}  // namespace kda
