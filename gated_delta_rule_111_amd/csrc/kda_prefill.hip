// kda_prefill.hip -- chunked KDA prefill on gfx950 (MI355X): packed varlen
// sequences, optional initial states, fp32 state snapshots at block
// boundaries, fp32 state carried between chunks.
//
// What is computed
// ----------------
// "Kimi K3 technical FAQ", question "What is KDA, and why does a serving
// engineer care?": the delta-rule recurrence with a per-channel forget gate,
// a dk x dv state per head, updated per chunk -- parallel within a chunk and
// recurrent across chunks.  Read as
//     S_t = (I - b_t k_t k_t^T) Diag(exp g_t) S_{t-1} + b_t k_t v_t^T,
//     o_t = scale S_t^T q_t.
// "Day-0 vLLM support for Kimi K3", section "Kimi K3's architecture, and how
// vLLM serves it": state snapshots at block boundaries feed a prefix cache.
//
// Chunked form (C = 64 rows per chunk; G = inclusive cumulative sum of g
// inside the chunk, G_C its last row; S = state at the chunk start):
//   A_ts = b_t sum_c k_t[c] k_s[c] e^{G_t[c]-G_s[c]}   (s < t)
//   B_ts =     sum_c q_t[c] k_s[c] e^{G_t[c]-G_s[c]}   (s <= t)
//   T    = (I + A)^-1,   TB = T Diag(b)                 (the UT transform)
//   U    = TB (V - (K . e^G) S)                         (delta-rule targets)
//   O    = scale ((Q . e^G) S + B U)
//   S'   = Diag(e^{G_C}) S + (K . e^{G_C - G})^T U
// Substituting the recurrence into itself inside a chunk gives
// (I + A) U = Diag(b) (V - (K . e^G) S); the rest follows by unrolling.
//
// Three launches on the caller's stream:
//   plan  -- one workgroup: per-sequence offsets of chunks and snapshots;
//   prep  -- one workgroup per (chunk, head), all chunks in parallel: the
//            Gram matrices A and B on MFMA, T by block forward substitution,
//            then TB and B written to the workspace as hi/lo bf16 MFMA
//            operands (everything here is independent of the state);
//   scan  -- one workgroup per (sequence, head, 16 value columns), walking
//            the sequence chunk by chunk with the fp32 state in registers.
//            Wave w owns 32 state rows.  Per chunk each wave builds its
//            decay-scaled operands from the cumulative log-decay, forms its
//            partial (K e^G) S and (Q e^G) S, and the four waves exchange
//            them through LDS with one barrier; then every wave forms U,
//            its rows of O and its rows of the next state.
//
// Precision: v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Operands that
// are not exact bf16 values are split into hi + lo bf16 and multiplied in
// three passes (hi*hi + hi*lo + lo*hi, ~16 bits); the K K^T Gram and the
// (K e^G) S product use one bf16 rounding of the decay-scaled keys.  State,
// snapshots, outputs and every accumulation are fp32.
//
// Determinism: every reduction has a fixed order that depends neither on the
// number of value tiles nor on where a sequence sits in the packed batch,
// and chunks restart at every sequence start, so resuming from a snapshot
// reproduces the uninterrupted run bit for bit.
#include <algorithm>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;                // chunk rows
constexpr int NT = 256;              // threads per workgroup (4 waves)
constexpr int DKP = 128;             // state rows, zero-padded above dk
constexpr int SL = 32;               // state rows per wave
constexpr float SPAN_LIMIT = 80.0f;  // |exponent| bound for the diagonal Gram factors
constexpr int PLANE = 512;           // uint4 per operand plane (4 row tiles x 2 K-steps x 64 lanes)

__device__ __forceinline__ f32x4 mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier that waits only for this wave's LDS traffic.  The
// generic barrier also drains outstanding global loads and stores, which
// would stall every prefetch issued ahead of it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// LDS writes of this wave are complete (and visible to its other lanes).
__device__ __forceinline__ void lds_wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint16_t bfb(float x) { return f32_to_bf16_bits(x); }
__device__ __forceinline__ float bff(uint32_t b) { return bf16_bits_to_f32(b); }
__device__ __forceinline__ float ex(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in fp32)
__device__ __forceinline__ void split(float x, uint16_t& hi, uint16_t& lo) {
    hi = bfb(x);
    lo = bfb(x - bff(hi));
}

__device__ __forceinline__ uint4 pack8(const uint16_t (&x)[8]) {
    uint4 u;
    u.x = x[0] | ((uint32_t)x[1] << 16); u.y = x[2] | ((uint32_t)x[3] << 16);
    u.z = x[4] | ((uint32_t)x[5] << 16); u.w = x[6] | ((uint32_t)x[7] << 16);
    return u;
}
__device__ __forceinline__ bf16x8_t as_op(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// Two accumulator tiles (row blocks 0 and 1 of a 32-row K-step) as one MFMA
// operand: elements 0..3 come from tile 0, 4..7 from tile 1, split hi / lo.
__device__ __forceinline__ void pack_split(const f32x4& x0, const f32x4& x1, bf16x8_t& hi,
                                           bf16x8_t& lo) {
    uint16_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        split(x0[e], h[e], l[e]);
        split(x1[e], h[4 + e], l[4 + e]);
    }
    hi = as_op(pack8(h));
    lo = as_op(pack8(l));
}

// Row orders inside a chunk.  An accumulator tile holds rows 4*(lane/16)+e;
// two tiles packed as one operand give a lane K positions 4*(lane/16)+e of
// each.  Numbering the chunk's tokens and the wave's state rows so that
// those 8 positions are 8 consecutive tokens (channels) lets every operand
// that comes from memory be one contiguous 8-element vector.
//   token of row r in token tile mt (mt = 0..3, r = 0..15):
__device__ __forceinline__ int tok_of(int mt, int r) {
    return ((mt >> 1) << 5) + ((r >> 2) << 3) + ((mt & 1) << 2) + (r & 3);
}
//   state row (within the wave's 32) of row r in row tile m (m = 0, 1):
__device__ __forceinline__ int chan_of(int m, int r) { return ((r >> 2) << 3) + (m << 2) + (r & 3); }

// ---------------------------------------------------------------------------
// Input access (bf16 or fp32 q, k, v)
// ---------------------------------------------------------------------------
template <typename TIn> struct In;
template <> struct In<bf16_t> {
    using V8 = uint4;  // 8 values
    __device__ __forceinline__ static V8 load8(const void* base, int64_t idx) {
        return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    }
    __device__ __forceinline__ static V8 zero8() { return make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ static void f32x8(const V8& u, float (&x)[8]) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = bff(w[j] & 0xffffu);
            x[2 * j + 1] = bff(w[j] >> 16);
        }
    }
    using V1 = uint16_t;
    __device__ __forceinline__ static V1 load1(const void* base, int64_t idx) {
        return static_cast<const uint16_t*>(base)[idx];
    }
    __device__ __forceinline__ static float f32(V1 x) { return bff(x); }
    __device__ __forceinline__ static float f32(bf16_t x) { return bff(x.bits); }
};
template <> struct In<float> {
    struct V8 { float4 a, b; };
    __device__ __forceinline__ static V8 load8(const void* base, int64_t idx) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
        return V8{p[0], p[1]};
    }
    __device__ __forceinline__ static V8 zero8() {
        return V8{make_float4(0.f, 0.f, 0.f, 0.f), make_float4(0.f, 0.f, 0.f, 0.f)};
    }
    __device__ __forceinline__ static void f32x8(const V8& u, float (&x)[8]) {
        x[0] = u.a.x; x[1] = u.a.y; x[2] = u.a.z; x[3] = u.a.w;
        x[4] = u.b.x; x[5] = u.b.y; x[6] = u.b.z; x[7] = u.b.w;
    }
    using V1 = float;
    __device__ __forceinline__ static V1 load1(const void* base, int64_t idx) {
        return static_cast<const float*>(base)[idx];
    }
    __device__ __forceinline__ static float f32(V1 x) { return x; }
};

// ---------------------------------------------------------------------------
// plan: chunk_start[b] = sum_{b' < b} ceil(L_b' / C), snap_base[b] =
// sum_{b' < b} floor(L_b' / interval), for b = 0 .. num_seqs.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void plan_kernel(const int32_t* __restrict__ cu, int num_seqs,
                                                  int interval, int32_t* __restrict__ chunk_start,
                                                  int32_t* __restrict__ snap_base) {
    __shared__ int32_t wtot[2][4];
    __shared__ int32_t carry[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry[0] = carry[1] = 0;
    __syncthreads();
    for (int base = 0; base <= num_seqs; base += NT) {
        const int b = base + tid;
        int vc = 0, vs = 0;
        if (b < num_seqs) {
            const int L = cu[b + 1] - cu[b];
            vc = (L + C - 1) / C;
            vs = interval > 0 ? L / interval : 0;
        }
        int ic = vc, is = vs;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int yc = __shfl_up(ic, off, 64), ys = __shfl_up(is, off, 64);
            if (lane >= off) { ic += yc; is += ys; }
        }
        if (lane == 63) { wtot[0][wave] = ic; wtot[1][wave] = is; }
        __syncthreads();
        int pc = carry[0], ps = carry[1];
        for (int w = 0; w < wave; ++w) { pc += wtot[0][w]; ps += wtot[1][w]; }
        if (b <= num_seqs) {
            chunk_start[b] = pc + ic - vc;
            snap_base[b] = ps + is - vs;
        }
        __syncthreads();
        if (tid == 0) {
            for (int w = 0; w < 4; ++w) { carry[0] += wtot[0][w]; carry[1] += wtot[1][w]; }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// prep: per (chunk, head) every state-independent quantity of the chunk,
// written to the workspace as MFMA operands in the order the scan reads them.
// ---------------------------------------------------------------------------
// Operand block of one (chunk, head), in 16-byte units (8 bf16 = one MFMA
// operand of one lane).  Scan lane (g = lane/16, i = lane%16) of wave w reads
// index [...][lane] of:
//   TB, B   [mt][ks]     row tok_of(mt, i), columns 32ks + 8g .. +7
//   W, Qd   [w][mt]      row tok_of(mt, i), channels 32w + 8g .. +7
//   Kd      [w][m][ks]   channel 32w + chan_of(m, i), tokens 32ks + 8g .. +7
//   dec     128 floats, e^{G_C} per channel
// with W = TB (K . e^G), Qd = Q . e^G, Kd = (K . e^{G_C - G})^T, each as a hi
// plane followed by a lo plane.
constexpr int OP_TB = 0;
constexpr int OP_B = 2 * PLANE;
constexpr int OP_W = 4 * PLANE;
constexpr int OP_Q = 8 * PLANE;
constexpr int OP_K = 12 * PLANE;
constexpr int OP_DEC = 16 * PLANE;
constexpr int CHUNK_OPS = 16 * PLANE + 32;

template <typename TIn>
struct PrepSmem {
    static constexpr int KP = DKP + 16 / (int)sizeof(TIn);  // padded row of staged keys, queries
    union {
        float G[C][DKP + 4];   // cumulative log-decay
        float T[C][C + 4];     // (I + A)^-1, once the decay-scaled operands are out
        float W[C][DKP + 4];   // W, for the transpose into operand order
    } u;
    union {
        float A[C][C + 1];     // strictly lower b_t sum_c k_t k_s e^{G_t - G_s}
        float B[C][C + 1];     // lower sum_c q_t k_s e^{G_t - G_s}, once T is formed
    } ab;
    union {
        TIn kS[C][KP];             // the chunk's keys (zero past n and dk)
        uint16_t KgT[DKP][C + 8];  // (K . e^G)^T in bf16, [channel][token], once kS is read
    } k;
    float Bd[4][16][17];       // diagonal blocks of B from the pairwise path
    float M[3][16][17];
    float beta[C];
};

struct PrepParams {
    const void* q;
    const void* k;
    const float* g;
    const float* beta;
    const int32_t* cu;
    const int32_t* chunk_start;
    uint4* ops;  // [chunks][H][CHUNK_OPS]
    int H, dk, num_seqs;
};

// Location of one (chunk, head) item.
struct PrepItem {
    int h, n;          // head; valid rows of the chunk (1 .. C)
    int64_t gc, row0;  // global chunk index; first packed row
};

__device__ __forceinline__ PrepItem prep_item(const PrepParams& p, int it) {
    PrepItem r;
    const int gc = it / p.H;
    r.h = it - gc * p.H;
    r.gc = gc;
    // sequence of this chunk: the last b with chunk_start[b] <= gc
    int lo = 0, hi = p.num_seqs;  // invariant: chunk_start[lo] <= gc < chunk_start[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.chunk_start[mid] <= gc) lo = mid; else hi = mid;
    }
    const int ci = gc - p.chunk_start[lo];
    r.row0 = (int64_t)p.cu[lo] + (int64_t)ci * C;
    r.n = min(C, p.cu[lo + 1] - p.cu[lo] - ci * C);
    return r;
}

// This thread's share of one item's raw inputs: g rows 8r + tid/32, channels
// 4*(tid%32)..+3; k, q rows 16r + tid/16, channels 8*(tid%16)..+7; beta of
// row tid (tid < 64).  Rows past the chunk end are read from its last row
// and channels past dk from channel 0; the values are masked when staged.
template <typename TIn>
struct PrepRaw {
    float4 g[8];
    typename In<TIn>::V8 k[4];
    typename In<TIn>::V8 qg[4];  // q at (16w + lane%16, 32ks + 8*(lane/16)), ks = 0..3
    typename In<TIn>::V8 qd[4];  // q at (tok_of(mt, lane%16), 32w' + 8*(lane/16)) of unit r
    float beta;
};

template <typename TIn>
__device__ __forceinline__ void prep_load(PrepRaw<TIn>& r, const PrepParams& p, const PrepItem& x,
                                          int tid) {
    using IO = In<TIn>;
    const int dk = p.dk;
    const int64_t rs = (int64_t)p.H * dk;                    // row stride
    const int64_t base = (x.row0 * p.H + x.h) * (int64_t)dk;  // row 0, channel 0
    {
        const int c = 4 * (tid & 31);
        const int cl = c < dk ? c : 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = 8 * i + (tid >> 5);
            r.g[i] = *reinterpret_cast<const float4*>(p.g + base + min(t, x.n - 1) * rs + cl);
        }
    }
    {
        const int c = 8 * (tid & 15);
        const int cl = c < dk ? c : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * i + (tid >> 4);
            r.k[i] = IO::load8(p.k, base + min(t, x.n - 1) * rs + cl);
        }
    }
    {
        const int lane = tid & 63, w = tid >> 6;
        const int t = 16 * w + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int c = 32 * ks + 8 * (lane >> 4);
            r.qg[ks] = IO::load8(p.q, base + min(t, x.n - 1) * rs + (c < dk ? c : 0));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = tid + NT * u;
            const int ws = idx >> 8, mt = (idx >> 6) & 3, ln = idx & 63;
            const int tt = tok_of(mt, ln & 15), c = SL * ws + 8 * (ln >> 4);
            r.qd[u] = IO::load8(p.q, base + min(tt, x.n - 1) * rs + (c < dk ? c : 0));
        }
    }
    r.beta = p.beta[(x.row0 + min(tid & 63, x.n - 1)) * p.H + x.h];
}

// One workgroup per (chunk, head) item; two are resident per compute unit.
// All of the item's global inputs are requested up front.
template <typename TIn>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prep_kernel(PrepParams p) {
    using IO = In<TIn>;
    using SM = PrepSmem<TIn>;
    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g4 = lane >> 4, i16 = lane & 15;
    const int dk = p.dk;

    const PrepItem x = prep_item(p, blockIdx.x);
    PrepRaw<TIn> raw;
    prep_load<TIn>(raw, p, x, tid);
    {
        const int n = x.n;
        uint4* __restrict__ dst = p.ops + (x.gc * p.H + x.h) * CHUNK_OPS;

        // ---- stage this item's inputs (zero past n and dk) ----
        {
            const int c = 4 * (tid & 31);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = 8 * i + (tid >> 5);
                *reinterpret_cast<float4*>(&sm.u.G[t][c]) =
                    (t < n && c < dk) ? raw.g[i] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        {
            const int c = 8 * (tid & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * i + (tid >> 4);
                const typename IO::V8 kz = (t < n && c < dk) ? raw.k[i] : IO::zero8();
                *reinterpret_cast<typename IO::V8*>(&sm.k.kS[t][c]) = kz;
            }
        }
        if (tid < C) sm.beta[tid] = tid < n ? raw.beta : 0.f;
        __syncthreads();

        // ---- cumulative log-decay per channel ----
        {
            const int c = tid & 127, half = tid >> 7;
            float run = 0.f;
#pragma unroll 8
            for (int r = 0; r < 32; ++r) {
                run += sm.u.G[half * 32 + r][c];
                sm.u.G[half * 32 + r][c] = run;
            }
            __syncthreads();
            if (half == 1) {
                const float base = sm.u.G[31][c];
#pragma unroll 8
                for (int r = 32; r < 64; ++r) sm.u.G[r][c] += base;
            }
            __syncthreads();
        }

        // ---- Gram matrices: wave w computes row tile w (rows 16w .. 16w+15) ----
        // Off-diagonal blocks (column tile ts < w) use the reference r = G at
        // row 16w - 1, so both factors e^{G_t - r} and e^{r - G_s} are <= 1.
        // The diagonal block uses r = G at row 16w + 7, keeping both factors
        // within e^{+-span/2} of the block; spans beyond SPAN_LIMIT take the
        // pairwise path.
        int extreme = 0;
        f32x4 accB[4];
        {
            f32x4 accA[4];
#pragma unroll
            for (int ts = 0; ts < 4; ++ts) {
                accA[ts] = f32x4{0.f, 0.f, 0.f, 0.f};
                accB[ts] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            const int t = 16 * w + i16;
#pragma unroll 1
            for (int ks = 0; ks < 4; ++ks) {
                const int c0 = 32 * ks + 8 * g4;
                float kt[8], qt[8];
                IO::f32x8(*reinterpret_cast<const typename IO::V8*>(&sm.k.kS[t][c0]), kt);
                typename IO::V8 qx = raw.qg[0];
#pragma unroll
                for (int q = 1; q < 4; ++q)
                    if (ks == q) qx = raw.qg[q];
                IO::f32x8((t < n && c0 < dk) ? qx : IO::zero8(), qt);
                float Gt[8], rw[8], rm[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    Gt[e] = sm.u.G[t][c0 + e];
                    rw[e] = sm.u.G[w > 0 ? 16 * w - 1 : 0][c0 + e];
                    rm[e] = sm.u.G[16 * w + 7][c0 + e];
                    extreme |= (sm.u.G[16 * w][c0 + e] - rm[e] > SPAN_LIMIT) |
                               (rm[e] - sm.u.G[16 * w + 15][c0 + e] > SPAN_LIMIT);
                }
                // diagonal block
                {
                    uint16_t xk[8], xqh[8], xql[8], yh[8], yl[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float xd = ex(Gt[e] - rm[e]);
                        const float yd = ex(rm[e] - Gt[e]);
                        xk[e] = bfb(kt[e] * xd);
                        split(qt[e] * xd, xqh[e], xql[e]);
                        split(kt[e] * yd, yh[e], yl[e]);
                    }
                    const bf16x8_t XK = as_op(pack8(xk)), XQH = as_op(pack8(xqh)),
                                   XQL = as_op(pack8(xql)), YH = as_op(pack8(yh)),
                                   YL = as_op(pack8(yl));
#pragma unroll
                    for (int ts = 0; ts < 4; ++ts) {
                        if (ts == w) {
                            accA[ts] = mfma(XK, YH, accA[ts]);
                            accB[ts] = mfma(XQH, YH, accB[ts]);
                            accB[ts] = mfma(XQH, YL, accB[ts]);
                            accB[ts] = mfma(XQL, YH, accB[ts]);
                        }
                    }
                }
                // off-diagonal blocks
                if (w > 0) {
                    uint16_t xk[8], xqh[8], xql[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float xo = ex(Gt[e] - rw[e]);
                        xk[e] = bfb(kt[e] * xo);
                        split(qt[e] * xo, xqh[e], xql[e]);
                    }
                    const bf16x8_t XK = as_op(pack8(xk)), XQH = as_op(pack8(xqh)),
                                   XQL = as_op(pack8(xql));
#pragma unroll
                    for (int ts = 0; ts < 3; ++ts) {
                        if (ts < w) {
                            const int s = 16 * ts + i16;
                            float ksv[8];
                            IO::f32x8(*reinterpret_cast<const typename IO::V8*>(&sm.k.kS[s][c0]), ksv);
                            uint16_t yh[8], yl[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                split(ksv[e] * ex(rw[e] - sm.u.G[s][c0 + e]), yh[e], yl[e]);
                            const bf16x8_t YH = as_op(pack8(yh)), YL = as_op(pack8(yl));
                            accA[ts] = mfma(XK, YH, accA[ts]);
                            accB[ts] = mfma(XQH, YH, accB[ts]);
                            accB[ts] = mfma(XQH, YL, accB[ts]);
                            accB[ts] = mfma(XQL, YH, accB[ts]);
                        }
                    }
                }
            }
            // accumulator (row 4*g4+e, column i16) of block (w, ts); masked
            // entries are selected away, never multiplied (they may hold inf)
#pragma unroll
            for (int ts = 0; ts < 4; ++ts)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tr = 16 * w + 4 * g4 + e, sc = 16 * ts + i16;
                    sm.ab.A[tr][sc] = (sc < tr) ? accA[ts][e] * sm.beta[tr] : 0.f;
                }
        }
        const int any_extreme = __syncthreads_or(extreme);

        if (any_extreme) {
            // a diagonal block spans more decay than fp32 factors can carry:
            // evaluate the four diagonal blocks pair by pair
            for (int idx = tid; idx < 4 * 256; idx += NT) {
                const int blk = idx >> 8, tl = (idx >> 4) & 15, sl = idx & 15;
                if (sl > tl) continue;
                const int t = 16 * blk + tl, s = 16 * blk + sl;
                float sa = 0.f, sb = 0.f;
                for (int c = 0; c < dk; ++c) {
                    const float kt = IO::f32(sm.k.kS[t][c]), kv = IO::f32(sm.k.kS[s][c]);
                    const float qt = t < n ? IO::f32(IO::load1(p.q, ((x.row0 + t) * p.H + x.h) * (int64_t)dk + c)) : 0.f;
                    const float e = ex(sm.u.G[t][c] - sm.u.G[s][c]);
                    sa = fmaf(kt * kv, e, sa);
                    sb = fmaf(qt * kv, e, sb);
                }
                sm.ab.A[t][s] = (s < t) ? sa * sm.beta[t] : 0.f;
                sm.Bd[blk][tl][sl] = sb;
            }
            __syncthreads();
        }

        // ---- decay-scaled operands: Kd planes, Qd planes, dec, then (K e^G)^T ----
#pragma unroll 2
        for (int r = 0; r < 4; ++r) {
            const int idx = tid + NT * r;  // (w', m, ks, lane)
            const int ws = idx >> 8, m = (idx >> 7) & 1, ks = (idx >> 6) & 1, ln = idx & 63;
            const int c = SL * ws + chan_of(m, ln & 15), t0 = 32 * ks + 8 * (ln >> 4);
            const float gcc = sm.u.G[C - 1][c];
            uint16_t kh[8], kl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = t0 + e;
                split(IO::f32(sm.k.kS[t][c]) * ex(gcc - sm.u.G[t][c]), kh[e], kl[e]);
            }
            dst[OP_K + idx] = pack8(kh);
            dst[OP_K + 2 * PLANE + idx] = pack8(kl);
        }
        uint16_t kg[4][8];  // (K e^G) of this thread's Qd units, for the transposed copy
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int idx = tid + NT * r;  // (w', mt, lane)
            const int ws = idx >> 8, mt = (idx >> 6) & 3, ln = idx & 63;
            const int t = tok_of(mt, ln & 15), c0 = SL * ws + 8 * (ln >> 4);
            float qv[8], kv[8];
            IO::f32x8((t < n && c0 < dk) ? raw.qd[r] : IO::zero8(), qv);
            IO::f32x8(*reinterpret_cast<const typename IO::V8*>(&sm.k.kS[t][c0]), kv);
            uint16_t qh[8], ql[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float eg = ex(sm.u.G[t][c0 + e]);
                split(qv[e] * eg, qh[e], ql[e]);
                kg[r][e] = bfb(kv[e] * eg);
            }
            dst[OP_Q + idx] = pack8(qh);
            dst[OP_Q + 2 * PLANE + idx] = pack8(ql);
        }
        if (tid < DKP) reinterpret_cast<float*>(dst + OP_DEC)[tid] = ex(sm.u.G[C - 1][tid]);
        __syncthreads();  // keys are read: their storage becomes (K e^G)^T
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int idx = tid + NT * r;
            const int ws = idx >> 8, mt = (idx >> 6) & 3, ln = idx & 63;
            const int t = tok_of(mt, ln & 15), c0 = SL * ws + 8 * (ln >> 4);
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.k.KgT[c0 + e][t] = kg[r][e];
        }
        __syncthreads();

        // ---- T = (I + A)^-1 by block forward substitution (G is dead now) ----
        if (lane < 16) {
            // diagonal block w, column j = lane
            const int bo = 16 * w, j = lane;
            float xs[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) acc = fmaf(sm.ab.A[bo + r][bo + m], xs[m], acc);
                xs[r] = (r == j) ? 1.f : -acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.u.T[bo + r][bo + j] = xs[r];
        }
        __syncthreads();
        {
            const int r = tid >> 4, cc = tid & 15;
#pragma unroll
            for (int d = 1; d < 4; ++d) {
                // blocks (I, J = I - d): M = sum_{K=J}^{I-1} A_IK T_KJ ; T_IJ = -T_II M
                for (int I = d; I < 4; ++I) {
                    const int J = I - d;
                    float acc = 0.f;
                    for (int K = J; K < I; ++K)
#pragma unroll
                        for (int m = 0; m < 16; ++m)
                            acc = fmaf(sm.ab.A[16 * I + r][16 * K + m], sm.u.T[16 * K + m][16 * J + cc], acc);
                    sm.M[I - d][r][cc] = acc;
                }
                __syncthreads();
                for (int I = d; I < 4; ++I) {
                    const int J = I - d;
                    float acc = 0.f;
#pragma unroll
                    for (int m = 0; m < 16; ++m)
                        acc = fmaf(sm.u.T[16 * I + r][16 * I + m], sm.M[I - d][m][cc], acc);
                    sm.u.T[16 * I + r][16 * J + cc] = -acc;
                }
                __syncthreads();
            }
        }

        // ---- B (A is dead now), then TB and B as operand planes ----
#pragma unroll
        for (int ts = 0; ts < 4; ++ts)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tr = 16 * w + 4 * g4 + e, sc = 16 * ts + i16;
                float v = accB[ts][e];
                if (any_extreme && ts == w) v = sm.Bd[w][4 * g4 + e][i16];
                sm.ab.B[tr][sc] = (sc <= tr) ? v : 0.f;
            }
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int idx = tid + NT * rr;  // (mt, ks, lane)
            const int mt = idx >> 7, ks = (idx >> 6) & 1, ln = idx & 63;
            const int t = tok_of(mt, ln & 15);
            const int s0 = 32 * ks + 8 * (ln >> 4);
            uint16_t th[8], tl[8], bh[8], bl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = s0 + e;
                const float tb = (s <= t) ? sm.u.T[t][s] * sm.beta[s] : 0.f;
                split(tb, th[e], tl[e]);
                split(sm.ab.B[t][s], bh[e], bl[e]);
            }
            dst[OP_TB + idx] = pack8(th);
            dst[OP_TB + PLANE + idx] = pack8(tl);
            dst[OP_B + idx] = pack8(bh);
            dst[OP_B + PLANE + idx] = pack8(bl);
        }

        // ---- W = TB (K e^G): wave w forms token tile w for all 128 channels ----
        {
            bf16x8_t TBh[2], TBl[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int t = tok_of(w, i16), s0 = 32 * ks + 8 * g4;
                uint16_t th[8], tl[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = s0 + e;
                    split((s <= t) ? sm.u.T[t][s] * sm.beta[s] : 0.f, th[e], tl[e]);
                }
                TBh[ks] = as_op(pack8(th));
                TBl[ks] = as_op(pack8(tl));
            }
            f32x4 acc[8];
#pragma unroll
            for (int ct = 0; ct < 8; ++ct) {
                acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8_t kg = as_op(*reinterpret_cast<const uint4*>(&sm.k.KgT[16 * ct + i16][32 * ks + 8 * g4]));
                    acc[ct] = mfma(TBh[ks], kg, acc[ct]);
                    acc[ct] = mfma(TBl[ks], kg, acc[ct]);
                }
            }
            __syncthreads();  // every read of T is done: its storage becomes W
#pragma unroll
            for (int ct = 0; ct < 8; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.u.W[tok_of(w, 4 * g4 + e)][16 * ct + i16] = acc[ct][e];
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int idx = tid + NT * r;  // (w', mt, lane)
            const int ws = idx >> 8, mt = (idx >> 6) & 3, ln = idx & 63;
            const int t = tok_of(mt, ln & 15), c0 = SL * ws + 8 * (ln >> 4);
            const float4 a = *reinterpret_cast<const float4*>(&sm.u.W[t][c0]);
            const float4 bq = *reinterpret_cast<const float4*>(&sm.u.W[t][c0 + 4]);
            const float xv[8] = {a.x, a.y, a.z, a.w, bq.x, bq.y, bq.z, bq.w};
            uint16_t wh[8], wl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) split(xv[e], wh[e], wl[e]);
            dst[OP_W + idx] = pack8(wh);
            dst[OP_W + 2 * PLANE + idx] = pack8(wl);
        }
    }
}

// ---------------------------------------------------------------------------
// scan: per (sequence, head, 16 value columns) the recurrence over chunks.
// Wave w owns state rows 32w .. 32w+31.  Per chunk it forms its partial
// W S and (Q e^G) S over those rows (and TB V for its token tile), the four
// waves exchange the partials through LDS with one barrier, then each wave
// forms U = TB V - W S for the whole chunk, its token tile of O and its rows
// of the next state.
// ---------------------------------------------------------------------------
template <typename TIn>
struct ScanSmem {
    struct Ex { f32x4 Y[4][64]; f32x4 P[4][64]; } ex[2][4];  // by chunk parity, wave
    TIn vt[4][C][16 + 16 / sizeof(TIn)];                  // per wave: the v tile, row-major
};

struct ScanParams {
    const void* v;
    const int32_t* cu;
    const int32_t* chunk_start;
    const int32_t* snap_base;
    const uint4* ops;
    const float* init;
    void* out;
    float* final_state;
    float* snapshots;
    int interval;
    int H, dk, dv;
    int ntiles, nwg;
    float scale;
};

// One chunk's operands for one lane, loaded a chunk ahead.
template <typename TIn>
struct ScanOps {
    uint4 w[4][2];        // W       [mt][hi, lo]
    uint4 q[4][2];        // Qd      [mt][hi, lo]
    uint4 kd[2][2][2];    // Kd      [m][ks][hi, lo]
    uint4 tb[2][2];       // TB rows of this wave's token tile [ks][hi, lo]
    uint4 b[2][2];        // B  rows of this wave's token tile [ks][hi, lo]
    float4 dec[2];        // e^{G_C} of the lane's state rows
    typename In<TIn>::V8 v[2];     // v rows 32r + lane/2, columns 8*(lane%2) .. +7 of the tile
};

// The next chunk's operands are loaded in three parts spread over the
// current chunk, so the wave never stalls on a full memory queue.
template <typename TIn>
__device__ __forceinline__ const uint4* scan_block(const ScanParams& p, int64_t gc, int h) {
    return p.ops + (gc * p.H + h) * CHUNK_OPS;
}

template <typename TIn>
__device__ __forceinline__ void scan_load1(ScanOps<TIn>& o, const uint4* __restrict__ blk, int w,
                                           int lane) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int x = (w * 4 + mt) * 64 + lane;
        o.w[mt][0] = blk[OP_W + x];
        o.w[mt][1] = blk[OP_W + 2 * PLANE + x];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int x = (w * 2 + ks) * 64 + lane;
        o.tb[ks][0] = blk[OP_TB + x];
        o.tb[ks][1] = blk[OP_TB + PLANE + x];
    }
}

template <typename TIn>
__device__ __forceinline__ void scan_load2(ScanOps<TIn>& o, const uint4* __restrict__ blk,
                                           const ScanParams& p, int64_t row0, int n, int h, int j16,
                                           int w, int lane) {
    using IO = In<TIn>;
    const int g4 = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int x = (w * 4 + mt) * 64 + lane;
        o.q[mt][0] = blk[OP_Q + x];
        o.q[mt][1] = blk[OP_Q + 2 * PLANE + x];
    }
    (void)g4;
    // the wave's copy of the chunk's v tile (64 rows x 16 columns), row-major:
    // rows past the chunk end are read from its last row; TB has zero columns
    // there, so they never reach U
    const int64_t vrow = (int64_t)p.H * p.dv;
    const int64_t vbase = (row0 * p.H + h) * (int64_t)p.dv + j16 + 8 * (lane & 1);
#pragma unroll
    for (int r = 0; r < 2; ++r)
        o.v[r] = IO::load8(p.v, vbase + (int64_t)min(32 * r + (lane >> 1), n - 1) * vrow);
}

template <typename TIn>
__device__ __forceinline__ void scan_load3(ScanOps<TIn>& o, const uint4* __restrict__ blk, int w,
                                           int lane) {
    const int g4 = lane >> 4;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int x = ((w * 2 + m) * 2 + ks) * 64 + lane;
            o.kd[m][ks][0] = blk[OP_K + x];
            o.kd[m][ks][1] = blk[OP_K + 2 * PLANE + x];
        }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const int x = (w * 2 + ks) * 64 + lane;
        o.b[ks][0] = blk[OP_B + x];
        o.b[ks][1] = blk[OP_B + PLANE + x];
    }
    const float4* dec = reinterpret_cast<const float4*>(blk + OP_DEC);
    o.dec[0] = dec[8 * w + 2 * g4];
    o.dec[1] = dec[8 * w + 2 * g4 + 1];
}

template <typename TIn>
__device__ __forceinline__ void scan_load(ScanOps<TIn>& o, const ScanParams& p, int64_t gc,
                                          int64_t row0, int n, int h, int j16, int w, int lane) {
    const uint4* blk = scan_block<TIn>(p, gc, h);
    scan_load1<TIn>(o, blk, w, lane);
    scan_load2<TIn>(o, blk, p, row0, n, h, j16, w, lane);
    scan_load3<TIn>(o, blk, w, lane);
}

template <typename TIn, bool OUT_BF16>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void scan_kernel(ScanParams p) {
    using IO = In<TIn>;
    __shared__ ScanSmem<TIn> sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g4 = lane >> 4, i16 = lane & 15;
    (void)tid;

    // workgroup -> (sequence, head, value tile).  Workgroups are dealt
    // round-robin over the 8 XCDs; the remap gives each XCD a contiguous
    // range of logical ids, so the tiles of one head share its L2.
    int L = blockIdx.x;
    if ((p.nwg & 7) == 0) L = (blockIdx.x & 7) * (p.nwg >> 3) + (blockIdx.x >> 3);
    const int tile = L % p.ntiles;
    const int chain = L / p.ntiles;
    const int b = chain / p.H, h = chain - b * p.H;
    const int dk = p.dk, dv = p.dv;
    const int j = 16 * tile + i16;
    const int64_t seq0 = p.cu[b];
    const int len = p.cu[b + 1] - p.cu[b];
    const int nch = (len + C - 1) / C;
    const int64_t cbase = p.chunk_start[b];
    const int64_t sbase = p.snap_base[b];

    // state rows of this lane: 32w + chan_of(m, 4*g4 + e) = 32w + 8*g4 + 4m + e
    f32x4 S[2];
    const int64_t srow = ((int64_t)b * p.H + h) * dk;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = SL * w + 8 * g4 + 4 * m + e;
            S[m][e] = 0.f;
            if (p.init) {
                const float x = p.init[(srow + (c < dk ? c : 0)) * dv + j];
                S[m][e] = c < dk ? x : 0.f;
            }
        }

    // Operands are prefetched one chunk ahead into two register sets used in
    // turn (the loop body is instantiated twice with the roles swapped), so
    // no loaded value is copied and nothing waits early for the next chunk.
    ScanOps<TIn> opA, opB;
    if (nch > 0) scan_load<TIn>(opA, p, cbase, seq0, min(C, len), h, 16 * tile, w, lane);

    auto chunk = [&](const int ci, ScanOps<TIn>& o, ScanOps<TIn>& nx) {
        const int par = ci & 1;
        const int64_t row0 = seq0 + (int64_t)ci * C;
        const int n = min(C, len - ci * C);

        // ---- prefetch the next chunk (the last chunk reloads itself, so the
        // same loads are issued on every path; that data is unused) ----
        const int cn = min(ci + 1, nch - 1);
        const uint4* nblk = scan_block<TIn>(p, cbase + cn, h);
        scan_load1<TIn>(nx, nblk, w, lane);

        // ---- partial W S and (Q e^G) S over this wave's rows; TB V ----
        {
            bf16x8_t Sh, Sl;
            pack_split(S[0], S[1], Sh, Sl);
            // v tile through the wave's LDS area: rows in, K-ordered columns out
            TIn (*vt)[16 + 16 / sizeof(TIn)] = sm.vt[w];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                TIn* row = &vt[32 * r + (lane >> 1)][8 * (lane & 1)];
                if constexpr (sizeof(TIn) == 2) {
                    *reinterpret_cast<uint4*>(row) = o.v[r];
                } else {
                    reinterpret_cast<float4*>(row)[0] = o.v[r].a;
                    reinterpret_cast<float4*>(row)[1] = o.v[r].b;
                }
            }
            lds_wave_sync();
            f32x4 ut = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8_t th = as_op(o.tb[ks][0]), tl = as_op(o.tb[ks][1]);
                if constexpr (sizeof(TIn) == 2) {
                    uint16_t vv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        vv[e] = reinterpret_cast<const uint16_t&>(vt[32 * ks + 8 * g4 + e][i16]);
                    const bf16x8_t vb = as_op(pack8(vv));
                    ut = mfma(th, vb, ut);
                    ut = mfma(tl, vb, ut);
                } else {
                    uint16_t vh[8], vl[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        split(reinterpret_cast<const float&>(vt[32 * ks + 8 * g4 + e][i16]), vh[e], vl[e]);
                    const bf16x8_t bh = as_op(pack8(vh)), bl = as_op(pack8(vl));
                    ut = mfma(th, bh, ut);
                    ut = mfma(th, bl, ut);
                    ut = mfma(tl, bh, ut);
                }
            }
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            typename ScanSmem<TIn>::Ex& E = sm.ex[par][w];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8_t wh = as_op(o.w[mt][0]), wl = as_op(o.w[mt][1]);
                f32x4 y = mfma(wh, Sh, z);
                y = mfma(wh, Sl, y);
                y = mfma(wl, Sh, y);
                if (mt == w) y -= ut;   // Y_w[w] = (W S)_w - TB V, so U = -sum_w Y_w
                const bf16x8_t qh = as_op(o.q[mt][0]), ql = as_op(o.q[mt][1]);
                f32x4 pq = mfma(qh, Sh, z);
                pq = mfma(qh, Sl, pq);
                pq = mfma(ql, Sh, pq);
                E.Y[mt][lane] = y;
                E.P[mt][lane] = pq;
            }
        }
        scan_load2<TIn>(nx, nblk, p, seq0 + (int64_t)cn * C, min(C, len - cn * C), h, 16 * tile, w,
                        lane);
        lds_barrier();

        // ---- U = TB V - W S for every token of the chunk ----
        bf16x8_t Uh[2], Ul[2];
        {
            f32x4 U[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 ys = sm.ex[par][0].Y[mt][lane];
                ys += sm.ex[par][1].Y[mt][lane];
                ys += sm.ex[par][2].Y[mt][lane];
                ys += sm.ex[par][3].Y[mt][lane];
                U[mt] = -ys;
            }
            pack_split(U[0], U[1], Uh[0], Ul[0]);
            pack_split(U[2], U[3], Uh[1], Ul[1]);
        }

        scan_load3<TIn>(nx, nblk, w, lane);

        // ---- this wave's token tile of O = scale ((Q e^G) S + B U) ----
        {
            f32x4 po = sm.ex[par][0].P[w][lane];
            po += sm.ex[par][1].P[w][lane];
            po += sm.ex[par][2].P[w][lane];
            po += sm.ex[par][3].P[w][lane];
            f32x4 bu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8_t bh = as_op(o.b[ks][0]), bl = as_op(o.b[ks][1]);
                bu = mfma(bh, Uh[ks], bu);
                bu = mfma(bh, Ul[ks], bu);
                bu = mfma(bl, Uh[ks], bu);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = tok_of(w, 4 * g4 + e);
                if (t < n) {
                    const float ov = p.scale * (po[e] + bu[e]);
                    const int64_t oi = ((row0 + t) * p.H + h) * (int64_t)dv + j;
                    if constexpr (OUT_BF16)
                        static_cast<uint16_t*>(p.out)[oi] = bfb(ov);
                    else
                        static_cast<float*>(p.out)[oi] = ov;
                }
            }
        }

        // ---- S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T U ----
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const float4 d = o.dec[m];
            f32x4 s = S[m] * f32x4{d.x, d.y, d.z, d.w};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8_t kh = as_op(o.kd[m][ks][0]), kl = as_op(o.kd[m][ks][1]);
                s = mfma(kh, Uh[ks], s);
                s = mfma(kh, Ul[ks], s);
                s = mfma(kl, Uh[ks], s);
            }
            S[m] = s;
        }
        const int done = ci * C + n;
        if (p.interval > 0 && done % p.interval == 0) {
            float* __restrict__ dsts =
                p.snapshots + ((sbase + done / p.interval - 1) * p.H + h) * (int64_t)dk * dv;
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = SL * w + 8 * g4 + 4 * m + e;
                    if (c < dk) dsts[(int64_t)c * dv + j] = S[m][e];
                }
        }
    };

    // The loop body always runs both halves, so the back edge is reached
    // only after the second half has consumed what the first half loaded;
    // an odd last chunk runs after the loop.
    int ci = 0;
    for (; ci + 1 < nch; ci += 2) {
        chunk(ci, opA, opB);
        chunk(ci + 1, opB, opA);
    }
    if (ci < nch) chunk(ci, opA, opB);

#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = SL * w + 8 * g4 + 4 * m + e;
            if (c < dk) p.final_state[(srow + c) * dv + j] = S[m][e];
        }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
    size_t chunk_start, snap_base, ops, total;
};

WsLayout ws_layout(int H, int num_seqs, int64_t max_chunks) {
    WsLayout l;
    l.chunk_start = 0;
    l.snap_base = align_up((size_t)(num_seqs + 1) * 4, 256);
    l.ops = l.snap_base + align_up((size_t)(num_seqs + 1) * 4, 256);
    l.total = l.ops + (size_t)max_chunks * H * CHUNK_OPS * sizeof(uint4);
    return l;
}

template <typename TIn>
hipError_t launch_t(const PrefillArgs& a) {
    const WsLayout l = ws_layout(a.H, a.num_seqs, a.total_chunks);
    char* ws = static_cast<char*>(a.workspace);
    int32_t* chunk_start = reinterpret_cast<int32_t*>(ws + l.chunk_start);
    int32_t* snap_base = reinterpret_cast<int32_t*>(ws + l.snap_base);
    uint4* ops = reinterpret_cast<uint4*>(ws + l.ops);

    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(NT), 0, a.stream, a.cu_dev, a.num_seqs, a.interval,
                       chunk_start, snap_base);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    if (a.total_chunks > 0) {
        PrepParams pp{};
        pp.q = a.q;
        pp.k = a.k;
        pp.g = a.g;
        pp.beta = a.beta;
        pp.cu = a.cu_dev;
        pp.chunk_start = chunk_start;
        pp.ops = ops;
        pp.H = a.H;
        pp.dk = a.dk;
        pp.num_seqs = a.num_seqs;
        const int64_t items = a.total_chunks * a.H;
        if (items > 0x7fffffffLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL((prep_kernel<TIn>), dim3((unsigned)items), dim3(NT), 0, a.stream, pp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    ScanParams sp{};
    sp.v = a.v;
    sp.cu = a.cu_dev;
    sp.chunk_start = chunk_start;
    sp.snap_base = snap_base;
    sp.ops = ops;
    sp.init = a.init;
    sp.out = a.out;
    sp.final_state = a.final_state;
    sp.snapshots = a.snapshots;
    sp.interval = a.interval;
    sp.H = a.H;
    sp.dk = a.dk;
    sp.dv = a.dv;
    sp.ntiles = a.dv / 16;
    sp.scale = a.scale;
    const int64_t nwg = (int64_t)a.num_seqs * a.H * sp.ntiles;
    sp.nwg = (int)nwg;
    if (a.out_bf16)
        hipLaunchKernelGGL((scan_kernel<TIn, true>), dim3((unsigned)nwg), dim3(NT), 0, a.stream, sp);
    else
        hipLaunchKernelGGL((scan_kernel<TIn, false>), dim3((unsigned)nwg), dim3(NT), 0, a.stream, sp);
    return hipGetLastError();
}

}  // namespace

int64_t prefill_max_chunks(int num_seqs, int64_t total_tokens) {
    // sum_b ceil(L_b / C) <= floor(T / C) + num_seqs
    return total_tokens / C + num_seqs;
}

int prefill_chunk_rows() { return C; }

size_t prefill_workspace_bytes(int, int, int H, int num_seqs, int64_t total_tokens) {
    return ws_layout(H, num_seqs, prefill_max_chunks(num_seqs, total_tokens)).total;
}

hipError_t launch_prefill(const PrefillArgs& a) {
    if (a.dk > DKP || a.dv % 16 != 0) return hipErrorInvalidValue;
    if ((int64_t)a.num_seqs * a.H * (a.dv / 16) > 0x7fffffffLL) return hipErrorInvalidValue;
    return a.in_bf16 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace kda
