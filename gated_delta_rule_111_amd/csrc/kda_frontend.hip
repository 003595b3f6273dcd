// kda_frontend.hip -- the q/k front end of KDA: a short causal convolution
// along each sequence's tokens, Swish, and L2 normalisation per (token, head).
// gfx950.
//
// "Kimi K3 technical FAQ" (Runpod guide), question "What is KDA, and why does
// a serving engineer care?": queries and keys go through a short convolution,
// Swish and L2 normalisation before the recurrence.  Per channel c = h*dk + i:
//   z_t[c] = sum_{j<W} w[c][j] x_{t-(W-1)+j}[c]   depthwise, causal, no bias
//   a      = z * sigmoid(z)                       Swish
//   y_t[h] = a_t[h] / sqrt(|a_t[h]|^2 + eps)      per token and head
// Inputs before a sequence's first token come from its convolution state (the
// W-1 inputs that preceded it, oldest first) or are zero; the call leaves the
// sequence's last W-1 inputs in the state.
//
// The op is bound by HBM: it reads x and writes y once (the taps and states
// are small).  Design:
// - a wave owns a slab of 512 consecutive channels (lane l: channels 8l..8l+7
//   of the slab, one 16-byte bf16 access per token) for a run of R
//   consecutive tokens, so each token moves one contiguous 1 KB segment;
// - the convolution window (the previous W-1 inputs) stays in registers while
//   the wave walks its tokens in groups of 8: the loads of the first group
//   and of the W-1 tokens before it are issued before anything else, and
//   each group's loads are issued while the previous group computes; a group
//   inside one sequence takes an unrolled path with no sequence checks;
// - each head's sum of squares is reduced over its dk/8 lanes with DPP row
//   operations (cross-lane moves inside the VALU, no LDS);
// - runs ignore sequence boundaries: a wave finds the sequence of its first
//   token with a 64-way search of the offsets and then follows them;
// - when every sequence has one token (a decode step) a kernel of its own
//   gives each wave a few sequences and loads all their rows at once;
// - the first W-1 tokens of every sequence, and its convolution state, belong
//   to the run holding the sequence's first token (which may go up to W-2
//   tokens past its own end).  Exactly one wave reads and writes each slice
//   of a sequence's state, and it reads before it writes, so the output state
//   may be the input state itself.
#include <algorithm>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int FE_LANE_CH = 8;             // channels per lane
constexpr int FE_SLAB = 64 * FE_LANE_CH;  // channels per wave
constexpr int FE_WAVES = 4;               // waves (runs) per workgroup
constexpr int FE_TARGET_WAVES = 8192;     // enough waves to cover HBM latency
constexpr int FE_MAX_RUN = 64;

struct FeParams {
    const void* x[2];         // q and k inputs [T, C]
    const float* w[2];        // taps [C, W]
    const void* sin[2];       // [num_slots, W-1, C] or null (zero history)
    void* sout[2];            // [num_slots, W-1, C] or null (not written)
    void* y[2];               // outputs [T, C]
    const int32_t* cu;        // [N + 1]
    const int32_t* slots;     // [N] or null (identity)
    int T, N, C, dk;
    int unit;                 // every sequence has one token (cu[b] == b)
    int nslab, nrun, R, ngroups, nwg;
    float eps2;               // eps * log2(e)^2 (the kernel works in base-2 units)
};

__device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
    const uint4 t = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(u[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_f32(u[i] >> 16);
    }
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two fp32 -> one packed pair of bf16 (round to nearest even), one instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ void store8(bf16_t* p, const float (&v)[8]) {
    uint4 t;
    t.x = pack_bf16x2(v[0], v[1]);
    t.y = pack_bf16x2(v[2], v[3]);
    t.z = pack_bf16x2(v[4], v[5]);
    t.w = pack_bf16x2(v[6], v[7]);
    *reinterpret_cast<uint4*>(p) = t;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// the same with a nontemporal hint, for every output and new state: none is
// read again by the launch, and streaming them past the caches is faster
// (measured at 4096 channels: a decode step of 256 sequences 7.2 -> 6.8 us,
// 8192 tokens 49-51 -> 46.5 us)
typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
typedef float f32x4_v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store8_stream(bf16_t* p, const float (&v)[8]) {
    const u32x4_v t = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                       pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4_v*>(p));
}
__device__ __forceinline__ void store8_stream(float* p, const float (&v)[8]) {
    const f32x4_v a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4_v*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4_v*>(p) + 1);
}

// sum over the `lanes` consecutive lanes of one head (2, 4, 8 or 16), left
// in every one of them: pairs and quads by quad permutations, 8 lanes by
// mirroring the half row, 16 lanes by rotating the row by 4 and then by 8
__device__ __forceinline__ float head_sum(float v, int lanes) {
    v += dpp<0xB1>(v);                       // quad_perm [1,0,3,2]: lane ^ 1
    if (lanes >= 4) v += dpp<0x4E>(v);       // quad_perm [2,3,0,1]: lane ^ 2
    if (lanes == 8) v += dpp<0x141>(v);      // row_half_mirror: the other quad
    if (lanes == 16) {
        v += dpp<0x124>(v);                  // row_ror 4: the next quad
        v += dpp<0x128>(v);                  // row_ror 8: the other two
    }
    return v;
}

// smallest b in [0, N) with cu[b+1] >= t (N if none), 64 probes per step
__device__ __forceinline__ int first_seq_reaching(const int32_t* __restrict__ cu, int N, int t,
                                                  int lane) {
    int lo = 0, hi = N;
    while (lo < hi) {
        const int step = (hi - lo + 63) >> 6;
        const int probe = lo + lane * step + step - 1;
        const int pc = min(probe, hi - 1);
        const bool below = probe < hi && cu[pc + 1] < t;
        const int k = __popcll(__ballot(below));
        lo += k * step;
        hi = min(hi, lo + step - 1);
    }
    return lo;
}

// 8 channels of one token as loaded (converted to fp32 only at use, so the
// registers of loads in flight hold packed bf16)
template <typename T> struct Raw8;
template <> struct Raw8<bf16_t> { uint4 v; };
template <> struct Raw8<float> { float4 a, b; };

__device__ __forceinline__ Raw8<bf16_t> load_raw(const bf16_t* p) {
    return {*reinterpret_cast<const uint4*>(p)};
}
__device__ __forceinline__ Raw8<float> load_raw(const float* p) {
    return {reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
}
__device__ __forceinline__ void widen(const Raw8<bf16_t>& r, float (&v)[8]) {
    const uint32_t u[4] = {r.v.x, r.v.y, r.v.z, r.v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(u[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_f32(u[i] >> 16);
    }
}
__device__ __forceinline__ void widen(const Raw8<float>& r, float (&v)[8]) {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
}

// G: tokens per group of loads (the launch uses 8)
template <int W, int G, typename TIn, typename TOut>
__global__ __launch_bounds__(64 * FE_WAVES) void frontend_kernel(FeParams p) {
    constexpr int NW = W > 1 ? W - 1 : 1;  // window rows (unused when W == 1)
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

    // workgroup -> (tensor, slab, group of 4 runs).  Workgroups are dealt
    // round-robin over the 8 XCDs; the remap gives each XCD a contiguous range
    // of logical ids, so neighbouring runs (which share window tokens) and
    // the slabs of one token range meet in one L2.
    int L = blockIdx.x;
    if ((p.nwg & 7) == 0) L = (blockIdx.x & 7) * (p.nwg >> 3) + (blockIdx.x >> 3);
    const int grp = L % p.ngroups;
    const int rest = L / p.ngroups;
    const int slab = rest % p.nslab;
    const int tsel = rest / p.nslab;
    const int run = grp * FE_WAVES + wv;
    if (run >= p.nrun) return;
    const bool last_run = run == p.nrun - 1;
    const int T = p.T;
    const int t_begin = run * p.R;
    const int t_end = min(T, t_begin + p.R);

    const int ch0 = slab * FE_SLAB + lane * FE_LANE_CH;
    const bool live = ch0 < p.C;       // the last slab may be partly empty
    const int ch = live ? ch0 : 0;     // dead lanes load channel 0 and store nothing
    const int64_t C = p.C;
    const TIn* __restrict__ x = static_cast<const TIn*>(p.x[tsel]) + ch;
    TOut* __restrict__ y = static_cast<TOut*>(p.y[tsel]) + ch;
    const TIn* sin = static_cast<const TIn*>(p.sin[tsel]);   // may alias sout
    TIn* sout = static_cast<TIn*>(p.sout[tsel]);
    const int head_lanes = p.dk / FE_LANE_CH;
    const float eps2 = p.eps2;

    // Loads that depend on nothing else go first: the run's first G tokens
    // (indices past the run repeat its last token) and the W-1 tokens before
    // the run (clamped into [0, T); rows from another sequence are shifted
    // out of the window before they weigh anything, see below).
    Raw8<TIn> cur[G];
    Raw8<TIn> halo[NW];
    if (T > 0) {
#pragma unroll
        for (int u = 0; u < G; ++u) cur[u] = load_raw(x + (int64_t)min(t_begin + u, t_end - 1) * C);
#pragma unroll
        for (int j = 0; j < W - 1; ++j)
            halo[j] = load_raw(x + (int64_t)max(0, min(t_begin - (W - 1) + j, T - 1)) * C);
    }

    // taps of the lane's 8 channels, pre-scaled by -log2(e) so that the
    // convolution yields zz = -z log2(e), the exponent of exp(-z) in base 2:
    // wt[j][i] = -log2(e) w[ch + i][j]
    float wt[W][8];
    {
        const float4* wp = reinterpret_cast<const float4*>(p.w[tsel] + (int64_t)ch * W);
        float buf[8 * W];
#pragma unroll
        for (int i = 0; i < 2 * W; ++i) {
            const float4 t = wp[i];
            buf[4 * i] = t.x; buf[4 * i + 1] = t.y; buf[4 * i + 2] = t.z; buf[4 * i + 3] = t.w;
        }
#pragma unroll
        for (int j = 0; j < W; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) wt[j][i] = buf[i * W + j] * -1.4426950408889634f;
    }

    float win[NW][8];  // the W-1 previous inputs, oldest first

    // y_t from the window and x_t.  With zz = -z log2(e):
    //   a' = zz / (1 + 2^zz) = -log2(e) * z sigmoid(z)
    //   y  = a' * -(|a'|^2 + eps log2(e)^2)^(-1/2) = z sigmoid(z) / sqrt(|.|^2 + eps)
    // 2^zz overflows to +inf for z << 0, where the reciprocal gives 0.
    auto emit = [&](int t, const float (&xv)[8]) {
        float a[8];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float zz = wt[W - 1][i] * xv[i];
#pragma unroll
            for (int j = 0; j < W - 1; ++j) zz = fmaf(wt[j][i], win[j][i], zz);
            a[i] = zz * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(zz));
            ss = fmaf(a[i], a[i], ss);
        }
        ss = head_sum(ss, head_lanes);
        const float inv = -__builtin_amdgcn_rsqf(ss + eps2);
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] *= inv;
        if (live) store8_stream(y + (int64_t)t * C, a);
    };
    auto push = [&](const float (&xv)[8]) {
#pragma unroll
        for (int j = 0; j + 1 < W - 1; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) win[j][i] = win[j + 1][i];
        if constexpr (W > 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) win[W - 2][i] = xv[i];
        }
    };

    // Sequence bookkeeping (uniform across the wave).  b is the sequence of
    // the current token, [s, e) its tokens; `owned` when it starts in this
    // run, in which case this wave reads and writes its state.
    auto cu_at = [&](int i) { return p.cu[i]; };
    int b = first_seq_reaching(p.cu, p.N, t_begin, lane);
    int s = cu_at(b), e = cu_at(b + 1);
    bool owned = s >= t_begin;
    int64_t slot = 0;
    auto enter = [&]() {  // start of an owned sequence: window = its history
        slot = p.slots ? p.slots[b] : b;
        if constexpr (W > 1) {
            if (sin) {
                Raw8<TIn> h[NW];
#pragma unroll
                for (int j = 0; j < W - 1; ++j) h[j] = load_raw(sin + (slot * (W - 1) + j) * C + ch);
#pragma unroll
                for (int j = 0; j < W - 1; ++j) widen(h[j], win[j]);
            } else {
#pragma unroll
                for (int j = 0; j < W - 1; ++j)
#pragma unroll
                    for (int i = 0; i < 8; ++i) win[j][i] = 0.f;
            }
        }
    };
    auto finish = [&]() {  // end of an owned sequence: the window is its new state
        if constexpr (W > 1) {
            if (sout && live) {
#pragma unroll
                for (int j = 0; j < W - 1; ++j) store8_stream(sout + (slot * (W - 1) + j) * C + ch, win[j]);
            }
        }
    };
    // one token in the general case: sequence ends, starts and skipped
    // tokens (the first W-1 of a sequence that started in an earlier run
    // only pass through the window: that run computes them)
    auto step = [&](int t, const float (&xv)[8]) {
        while (t >= e) {  // sequence b ended before t (or is empty)
            if (owned) finish();
            ++b;
            s = cu_at(b);
            e = cu_at(b + 1);
            owned = true;
            enter();
        }
        if (owned || t >= s + W - 1) emit(t, xv);
        push(xv);
    };

    if (owned) {
        enter();
    } else {
#pragma unroll
        for (int j = 0; j < W - 1; ++j) widen(halo[j], win[j]);
    }

    for (int g0 = t_begin; g0 < t_end; g0 += G) {
        const bool more = g0 + G < t_end;
        Raw8<TIn> nxt[G];
        if (more) {
#pragma unroll
            for (int u = 0; u < G; ++u) nxt[u] = load_raw(x + (int64_t)min(g0 + G + u, t_end - 1) * C);
        }
        if (g0 + G <= t_end && g0 + G <= e && (owned || g0 >= s + W - 1)) {
            // the whole group inside one sequence and computed here
#pragma unroll
            for (int u = 0; u < G; ++u) {
                float xv[8];
                widen(cur[u], xv);
                emit(g0 + u, xv);
                push(xv);
            }
        } else {
            // first token from the registers, the rest reloaded (cache hits)
            const int gn = min(g0 + G, t_end);
            {
                float xv[8];
                widen(cur[0], xv);
                step(g0, xv);
            }
            for (int t = g0 + 1; t < gn; ++t) {
                float xv[8];
                widen(load_raw(x + (int64_t)t * C), xv);
                step(t, xv);
            }
        }
        if (more) {
#pragma unroll
            for (int u = 0; u < G; ++u) cur[u] = nxt[u];
        }
    }

    if (owned) {
        if (e > t_end) {
            // the sequence's first W-1 tokens may reach past the run
            const int xe = min(e, s + W - 1);
            for (int t = t_end; t < xe; ++t) {
                float xv[8];
                widen(load_raw(x + (int64_t)t * C), xv);
                emit(t, xv);
                push(xv);
            }
            if (xe == e) {
                finish();
            } else if constexpr (W > 1) {
                if (sout && live) {  // state = the sequence's last W-1 inputs
                    Raw8<TIn> tl[NW];
#pragma unroll
                    for (int j = 0; j < W - 1; ++j) tl[j] = load_raw(x + (int64_t)(e - (W - 1) + j) * C);
#pragma unroll
                    for (int j = 0; j < W - 1; ++j) {
                        float v[8];
                        widen(tl[j], v);
                        store8_stream(sout + (slot * (W - 1) + j) * C + ch, v);
                    }
                }
            }
        } else {
            finish();
        }
    }
    // the last run also owns the empty sequences that start at T
    if (last_run) {
        for (++b; b < p.N; ++b) {
            enter();
            finish();
        }
    }
}

// One-token sequences (a decode step): each sequence is one token whose
// window is its state, so a wave takes FE_UNIT tokens of one slab and issues,
// before any arithmetic, the slot lookups, then every token's input and state
// rows, then the taps (read once for all its tokens).  The new state of a
// sequence is its old state shifted by one row with the token appended; each
// state slice is read and written by the one wave that owns the token, reads
// first, so the state may be updated in place.  (256 sequences x 4096
// channels: 9.5 us with the general kernel, one token per wave; 7.2 us with
// 2 or 4 tokens per wave; 8 tokens per wave leave too few waves; 6.8 us with
// the parameters read at once and the inputs and taps requested before the
// slot lookups.)
constexpr int FE_UNIT = 4;

template <int W, typename TIn, typename TOut>
__global__ __launch_bounds__(64 * FE_WAVES) void frontend_unit_kernel(FeParams p) {
    constexpr int NW = W > 1 ? W - 1 : 1;
    // Every parameter is read up front and there is no branch before the
    // loads (a wave past the last token clamps its rows and stores nothing),
    // so the kernel-argument loads leave together and are waited for once;
    // the pointers of q or k are selected, not loaded by index.
    const int nwg = p.nwg, ngroups = p.ngroups, nslab = p.nslab, T = p.T, dk = p.dk;
    const float eps2 = p.eps2;
    const int64_t C = p.C;
    const int32_t* __restrict__ slots = p.slots;
    const TIn* x0 = static_cast<const TIn*>(p.x[0]); const TIn* x1 = static_cast<const TIn*>(p.x[1]);
    const float* w0 = p.w[0]; const float* w1 = p.w[1];
    const TIn* si0 = static_cast<const TIn*>(p.sin[0]); const TIn* si1 = static_cast<const TIn*>(p.sin[1]);
    TIn* so0 = static_cast<TIn*>(p.sout[0]); TIn* so1 = static_cast<TIn*>(p.sout[1]);
    TOut* y0 = static_cast<TOut*>(p.y[0]); TOut* y1 = static_cast<TOut*>(p.y[1]);
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int L = (nwg & 7) == 0 ? (int)((blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3)) : (int)blockIdx.x;
    const int grp = L % ngroups;
    const int rest = L / ngroups;
    const int slab = rest % nslab;
    const int tsel = rest / nslab;
    const int t0 = (grp * FE_WAVES + wv) * FE_UNIT;
    const int ch0 = slab * FE_SLAB + lane * FE_LANE_CH;
    const bool live = ch0 < C;
    const int ch = live ? ch0 : 0;
    const TIn* __restrict__ x = (tsel ? x1 : x0) + ch;
    TOut* __restrict__ y = (tsel ? y1 : y0) + ch;
    const TIn* sin = tsel ? si1 : si0;   // may alias sout
    TIn* sout = tsel ? so1 : so0;
    const float* wsel = tsel ? w1 : w0;

    // the inputs and the taps are requested before the slot lookups, whose
    // state rows wait for them
    Raw8<TIn> xr[FE_UNIT];
#pragma unroll
    for (int u = 0; u < FE_UNIT; ++u) xr[u] = load_raw(x + (int64_t)min(t0 + u, T - 1) * C);
    float wt[W][8];  // -log2(e) w[ch + i][j], as in frontend_kernel
    {
        const float4* wp = reinterpret_cast<const float4*>(wsel + (int64_t)ch * W);
        float buf[8 * W];
#pragma unroll
        for (int i = 0; i < 2 * W; ++i) {
            const float4 t = wp[i];
            buf[4 * i] = t.x; buf[4 * i + 1] = t.y; buf[4 * i + 2] = t.z; buf[4 * i + 3] = t.w;
        }
#pragma unroll
        for (int j = 0; j < W; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) wt[j][i] = buf[i * W + j] * -1.4426950408889634f;
    }
    int64_t slot[FE_UNIT];
#pragma unroll
    for (int u = 0; u < FE_UNIT; ++u) {
        const int t = min(t0 + u, T - 1);
        slot[u] = slots ? slots[t] : t;
    }
    Raw8<TIn> hr[FE_UNIT][NW];
    if (W > 1 && sin) {
#pragma unroll
        for (int u = 0; u < FE_UNIT; ++u)
#pragma unroll
            for (int j = 0; j < W - 1; ++j) hr[u][j] = load_raw(sin + (slot[u] * (W - 1) + j) * C + ch);
    }
    const int head_lanes = dk / FE_LANE_CH;
#pragma unroll
    for (int u = 0; u < FE_UNIT; ++u) {
        if (t0 + u >= T) break;
        float xv[8], win[NW][8];
        widen(xr[u], xv);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) {
            if (sin) {
                widen(hr[u][j], win[j]);
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) win[j][i] = 0.f;
            }
        }
        float a[8];
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float zz = wt[W - 1][i] * xv[i];
#pragma unroll
            for (int j = 0; j < W - 1; ++j) zz = fmaf(wt[j][i], win[j][i], zz);
            a[i] = zz * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(zz));
            ss = fmaf(a[i], a[i], ss);
        }
        ss = head_sum(ss, head_lanes);
        const float inv = -__builtin_amdgcn_rsqf(ss + eps2);
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] *= inv;
        if (live) {
            store8_stream(y + (int64_t)(t0 + u) * C, a);
            if (W > 1 && sout) {
                // the new history: the old rows 1 .. W-2, then this token
#pragma unroll
                for (int j = 0; j + 1 < W - 1; ++j) store8_stream(sout + (slot[u] * (W - 1) + j) * C + ch, win[j + 1]);
                store8_stream(sout + (slot[u] * (W - 1) + (W - 2)) * C + ch, xv);
            }
        }
    }
}

template <int W, typename TIn, typename TOut>
hipError_t launch_w(const FeParams& p, hipStream_t stream) {
    if (p.unit)
        hipLaunchKernelGGL((frontend_unit_kernel<W, TIn, TOut>), dim3(p.nwg), dim3(64 * FE_WAVES),
                           0, stream, p);
    else
        hipLaunchKernelGGL((frontend_kernel<W, 8, TIn, TOut>), dim3(p.nwg), dim3(64 * FE_WAVES),
                           0, stream, p);
    return hipGetLastError();
}

template <typename TIn, typename TOut>
hipError_t launch_t(const FeParams& p, int W, hipStream_t stream) {
    switch (W) {
        case 1: return launch_w<1, TIn, TOut>(p, stream);
        case 2: return launch_w<2, TIn, TOut>(p, stream);
        case 3: return launch_w<3, TIn, TOut>(p, stream);
        case 4: return launch_w<4, TIn, TOut>(p, stream);
        case 5: return launch_w<5, TIn, TOut>(p, stream);
        case 6: return launch_w<6, TIn, TOut>(p, stream);
        case 7: return launch_w<7, TIn, TOut>(p, stream);
        case 8: return launch_w<8, TIn, TOut>(p, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_frontend(const FrontendArgs& a) {
    FeParams p{};
    for (int i = 0; i < 2; ++i) {
        p.x[i] = a.x[i];
        p.w[i] = a.w[i];
        p.sin[i] = a.state_in[i];
        p.sout[i] = a.state_out[i];
        p.y[i] = a.y[i];
    }
    p.cu = a.cu_dev;
    p.slots = a.slots;
    p.T = (int)a.total_tokens;
    p.N = a.num_seqs;
    p.C = a.H * a.dk;
    p.dk = a.dk;
    p.eps2 = (float)((double)a.eps * 2.0813689810056077);
    p.nslab = (p.C + FE_SLAB - 1) / FE_SLAB;
    const int runs_wanted = std::max(1, FE_TARGET_WAVES / (2 * p.nslab));
    p.unit = a.unit_lengths ? 1 : 0;
    // runs of one-token sequences each read and write a state per token, so
    // they stay short
    p.R = p.unit ? FE_UNIT
                 : std::min(FE_MAX_RUN, std::max(1, (int)(((int64_t)p.T + runs_wanted - 1) / runs_wanted)));
    p.nrun = p.T > 0 ? (p.T + p.R - 1) / p.R : 1;
    p.ngroups = (p.nrun + FE_WAVES - 1) / FE_WAVES;
    p.nwg = 2 * p.nslab * p.ngroups;
    if (a.in_bf16)
        return a.out_bf16 ? launch_t<bf16_t, bf16_t>(p, a.W, a.stream)
                          : launch_t<bf16_t, float>(p, a.W, a.stream);
    return a.out_bf16 ? launch_t<float, bf16_t>(p, a.W, a.stream)
                      : launch_t<float, float>(p, a.W, a.stream);
}

}  // namespace kda
