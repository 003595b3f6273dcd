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
constexpr int CHUNK_OPS = 4 * PLANE; // TB hi, TB lo, B hi, B lo

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
    using V1 = uint32_t;
    __device__ __forceinline__ static V1 load1(const void* base, int64_t idx) {
        return static_cast<const uint16_t*>(base)[idx];
    }
    __device__ __forceinline__ static float f32(V1 x) { return bff(x); }
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
// prep: per (chunk, head) the state-independent chunk quantities.
// ---------------------------------------------------------------------------
struct PrepSmem {
    union {
        float G[C][DKP + 4];  // cumulative log-decay (dead after the Gram matrices)
        float T[C][C + 4];    // (I + A)^-1, lower block triangle
    } u;
    float A[C][C + 1];
    float B[C][C + 1];
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

template <typename TIn>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prep_kernel(PrepParams p) {
    using IO = In<TIn>;
    __shared__ PrepSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g4 = lane >> 4, i16 = lane & 15;
    const int gc = blockIdx.x, h = blockIdx.y;

    // sequence of this chunk: the last b with chunk_start[b] <= gc
    int lo = 0, hi = p.num_seqs;  // invariant: chunk_start[lo] <= gc < chunk_start[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.chunk_start[mid] <= gc) lo = mid; else hi = mid;
    }
    const int b = lo;
    const int ci = gc - p.chunk_start[b];
    const int64_t row0 = (int64_t)p.cu[b] + (int64_t)ci * C;
    const int len = p.cu[b + 1] - p.cu[b];
    const int n = min(C, len - ci * C);
    const int dk = p.dk;

    // ---- cumulative log-decay per channel (rows past n count as g = 0) ----
    {
        const int c = tid & 127, half = tid >> 7;
        float run = 0.f;
#pragma unroll 8
        for (int r = 0; r < 32; ++r) {
            const int t = half * 32 + r;
            run += (t < n && c < dk) ? p.g[((row0 + t) * p.H + h) * (int64_t)dk + c] : 0.f;
            sm.u.G[t][c] = run;
        }
        if (tid < C) sm.beta[tid] = tid < n ? p.beta[(row0 + tid) * p.H + h] : 0.f;
        __syncthreads();
        if (half == 1) {
            const float base = sm.u.G[31][c];
#pragma unroll 8
            for (int r = 32; r < 64; ++r) sm.u.G[r][c] += base;
        }
        __syncthreads();
    }

    // ---- Gram matrices: wave w computes row tile w (rows 16w .. 16w+15) ----
    // Off-diagonal blocks (column tile ts < w) use the reference r = G at row
    // 16w - 1, so both factors e^{G_t - r} and e^{r - G_s} are <= 1.  The
    // diagonal block uses r = G at row 16w + 7, keeping both factors within
    // e^{+-span/2} of the block; spans beyond SPAN_LIMIT take the pairwise path.
    int extreme = 0;
    {
        f32x4 accA[4], accB[4];
#pragma unroll
        for (int ts = 0; ts < 4; ++ts) {
            accA[ts] = f32x4{0.f, 0.f, 0.f, 0.f};
            accB[ts] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        const int t = 16 * w + i16;
#pragma unroll 1
        for (int ks = 0; ks < 4; ++ks) {
            const int c0 = 32 * ks + 8 * g4;
            const bool cok = c0 < dk;
            float kt[8], qt[8];
            {
                const int64_t idx = ((row0 + t) * p.H + h) * (int64_t)dk + c0;
                const bool ok = cok && t < n;
                IO::f32x8(ok ? IO::load8(p.k, idx) : IO::zero8(), kt);
                IO::f32x8(ok ? IO::load8(p.q, idx) : IO::zero8(), qt);
            }
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
                        const int64_t idx = ((row0 + s) * p.H + h) * (int64_t)dk + c0;
                        IO::f32x8((cok && s < n) ? IO::load8(p.k, idx) : IO::zero8(), ksv);
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
        // accumulator (row 4*g4+e, column i16) of block (w, ts); masked entries
        // are selected away, never multiplied (they may hold inf)
#pragma unroll
        for (int ts = 0; ts < 4; ++ts)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tr = 16 * w + 4 * g4 + e, sc = 16 * ts + i16;
                sm.A[tr][sc] = (sc < tr) ? accA[ts][e] * sm.beta[tr] : 0.f;
                sm.B[tr][sc] = (sc <= tr) ? accB[ts][e] : 0.f;
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
            if (t < n) {
                const int64_t bt = ((row0 + t) * p.H + h) * (int64_t)dk;
                const int64_t bs = ((row0 + s) * p.H + h) * (int64_t)dk;
                for (int c = 0; c < dk; ++c) {
                    const float kt = IO::f32(IO::load1(p.k, bt + c));
                    const float kv = IO::f32(IO::load1(p.k, bs + c));
                    const float qt = IO::f32(IO::load1(p.q, bt + c));
                    const float e = ex(sm.u.G[t][c] - sm.u.G[s][c]);
                    sa = fmaf(kt * kv, e, sa);
                    sb = fmaf(qt * kv, e, sb);
                }
            }
            sm.A[t][s] = (s < t) ? sa * sm.beta[t] : 0.f;
            sm.B[t][s] = sb;
        }
        __syncthreads();
    }

    // ---- T = (I + A)^-1 by block forward substitution (G is dead now) ----
    if (lane < 16) {
        // diagonal block w, column j = lane
        const int bo = 16 * w, j = lane;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < r; ++m) acc = fmaf(sm.A[bo + r][bo + m], x[m], acc);
            x[r] = (r == j) ? 1.f : -acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.u.T[bo + r][bo + j] = x[r];
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
                        acc = fmaf(sm.A[16 * I + r][16 * K + m], sm.u.T[16 * K + m][16 * J + cc], acc);
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

    // ---- TB = T Diag(beta) and B as hi/lo MFMA operands in scan order ----
    uint4* __restrict__ dst = p.ops + ((int64_t)gc * p.H + h) * CHUNK_OPS;
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int idx = tid + NT * rr;           // 0 .. 511
        const int mt = idx >> 7, ks = (idx >> 6) & 1, ln = idx & 63;
        const int t = tok_of(mt, ln & 15);
        const int s0 = 32 * ks + 8 * (ln >> 4);
        uint16_t th[8], tl[8], bh[8], bl[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int s = s0 + e;
            const float tb = (s <= t) ? sm.u.T[t][s] * sm.beta[s] : 0.f;
            split(tb, th[e], tl[e]);
            split(sm.B[t][s], bh[e], bl[e]);
        }
        dst[0 * PLANE + idx] = pack8(th);
        dst[1 * PLANE + idx] = pack8(tl);
        dst[2 * PLANE + idx] = pack8(bh);
        dst[3 * PLANE + idx] = pack8(bl);
    }
}

// ---------------------------------------------------------------------------
// scan: per (sequence, head, 16 value columns) the recurrence over chunks.
// ---------------------------------------------------------------------------
// LDS of the scan workgroup.  Staging areas are private to a wave and reused
// every chunk; the exchange area and TB alternate between two parities so
// that one barrier per chunk suffices.
template <typename TIn>
struct ScanSmem {
    static constexpr bool KSTAGE = sizeof(TIn) == 2;  // bf16 keys are staged for the transpose
    float G[4][C][SL + 4];                      // per wave: cumulative log-decay of its 32 rows
    uint16_t K[KSTAGE ? 4 : 1][C][SL + 8];      // per wave: its 32 key channels (bf16)
    struct Ex { f32x4 X[4][64]; f32x4 P[4][64]; } ex[2][4];  // partial (K e^G) S, (Q e^G) S
    uint4 tb[2][2 * PLANE];                     // TB hi, lo of the chunk
};

struct ScanParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
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
    int out_bf16;
    float scale;
};

// One chunk's inputs for one lane, loaded a chunk ahead.
template <typename TIn>
struct ScanPrefetch {
    using IO = In<TIn>;
    uint4 bo[2][2];                // B rows of this wave's token tile: [ks][hi, lo]
    float4 g[8];                   // g of tokens 8*(lane/8)+r, channels 4*(lane%8)..+3
    typename IO::V8 ka[4];         // k at (tok_of(mt, lane%16), channels 8*(lane/16)..+7)
    typename IO::V8 qa[4];         // q at the same positions
    typename IO::V1 v[4][4];       // v at (tok_of(mt, 4*(lane/16)+e), column j)
};

template <typename TIn>
__device__ __forceinline__ void scan_load(ScanPrefetch<TIn>& pf, const ScanParams& p, int64_t gc,
                                          int64_t row0, int n, int h, int j, int w, int lane) {
    using IO = In<TIn>;
    const int g4 = lane >> 4, i16 = lane & 15;
    const int dk = p.dk;
    const uint4* __restrict__ blk = p.ops + (gc * p.H + h) * CHUNK_OPS;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int pl = 0; pl < 2; ++pl)
            pf.bo[ks][pl] = blk[(2 + pl) * PLANE + (w * 2 + ks) * 64 + lane];
    {
        const int cg = SL * w + 4 * (lane & 7), tq = 8 * (lane >> 3);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int t = tq + r;
            pf.g[r] = (t < n && cg < dk)
                          ? *reinterpret_cast<const float4*>(p.g + ((row0 + t) * p.H + h) * (int64_t)dk + cg)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    {
        const int c = SL * w + 8 * g4;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int t = tok_of(mt, i16);
            const bool ok = t < n && c < dk;
            const int64_t idx = ((row0 + t) * p.H + h) * (int64_t)dk + c;
            pf.ka[mt] = ok ? IO::load8(p.k, idx) : IO::zero8();
            pf.qa[mt] = ok ? IO::load8(p.q, idx) : IO::zero8();
        }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = tok_of(mt, 4 * g4 + e);
            pf.v[mt][e] = t < n ? IO::load1(p.v, ((row0 + t) * p.H + h) * (int64_t)p.dv + j)
                                : typename IO::V1(0);
        }
}

// This thread's share (4 x 16 bytes) of a chunk's TB hi and lo planes.
struct TbShare {
    uint4 a, b, c, d;
};
__device__ __forceinline__ TbShare load_tb(const ScanParams& p, int64_t gc, int h, int tid) {
    const uint4* __restrict__ blk = p.ops + (gc * p.H + h) * CHUNK_OPS;
    return TbShare{blk[tid], blk[tid + NT], blk[tid + 2 * NT], blk[tid + 3 * NT]};
}
__device__ __forceinline__ void store_tb(uint4* dst, const TbShare& s, int tid) {
    dst[tid] = s.a;
    dst[tid + NT] = s.b;
    dst[tid + 2 * NT] = s.c;
    dst[tid + 3 * NT] = s.d;
}

template <typename TIn>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void scan_kernel(ScanParams p) {
    using IO = In<TIn>;
    using SM = ScanSmem<TIn>;
    __shared__ SM sm;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g4 = lane >> 4, i16 = lane & 15;

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
    float (*Gs)[SL + 4] = sm.G[w];

    // state rows of this lane: 32w + chan_of(m, 4*g4 + e) = 32w + 8*g4 + 4m + e
    f32x4 S[2];
    const int64_t srow = ((int64_t)b * p.H + h) * dk;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int c = SL * w + 8 * g4 + 4 * m + e;
            S[m][e] = (p.init && c < dk) ? p.init[(srow + c) * dv + j] : 0.f;
        }

    ScanPrefetch<TIn> pf;
    if (nch > 0) {
        store_tb(sm.tb[0], load_tb(p, cbase, h, tid), tid);
        scan_load<TIn>(pf, p, cbase, seq0, min(C, len), h, j, w, lane);
        lds_barrier();
    }

    for (int ci = 0; ci < nch; ++ci) {
        const int par = ci & 1;
        const int64_t row0 = seq0 + (int64_t)ci * C;
        const int n = min(C, len - ci * C);

        // ---- (a) stage the cumulative log-decay (and bf16 keys) of this chunk ----
        typename IO::V1 vcur[4][4];
        uint4 bcur[2][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) vcur[mt][e] = pf.v[mt][e];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) { bcur[ks][0] = pf.bo[ks][0]; bcur[ks][1] = pf.bo[ks][1]; }
        {
            // lane scan over its 8 tokens, then an exclusive scan over the 8 token groups
            float4 run = pf.g[0];
            float4 Gl[8];
            Gl[0] = run;
#pragma unroll
            for (int r = 1; r < 8; ++r) {
                run.x += pf.g[r].x; run.y += pf.g[r].y; run.z += pf.g[r].z; run.w += pf.g[r].w;
                Gl[r] = run;
            }
            float4 incl = run;
#pragma unroll
            for (int off = 8; off < 64; off <<= 1) {
                float4 y;
                y.x = __shfl_up(incl.x, off, 64); y.y = __shfl_up(incl.y, off, 64);
                y.z = __shfl_up(incl.z, off, 64); y.w = __shfl_up(incl.w, off, 64);
                if (lane >= off) { incl.x += y.x; incl.y += y.y; incl.z += y.z; incl.w += y.w; }
            }
            const float4 excl = make_float4(incl.x - run.x, incl.y - run.y, incl.z - run.z, incl.w - run.w);
            const int cq = 4 * (lane & 7), tq = 8 * (lane >> 3);
#pragma unroll
            for (int r = 0; r < 8; ++r)
                *reinterpret_cast<float4*>(&Gs[tq + r][cq]) =
                    make_float4(Gl[r].x + excl.x, Gl[r].y + excl.y, Gl[r].z + excl.z, Gl[r].w + excl.w);
        }
        if constexpr (SM::KSTAGE) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                *reinterpret_cast<uint4*>(&sm.K[w][tok_of(mt, i16)][8 * g4]) = pf.ka[mt];
        }
        lds_wave_sync();

        // ---- (b) decay-scaled operands of the products with the old state ----
        bf16x8_t Kg[4], Qh[4], Ql[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int t = tok_of(mt, i16);
            const float4 ga = *reinterpret_cast<const float4*>(&Gs[t][8 * g4]);
            const float4 gb = *reinterpret_cast<const float4*>(&Gs[t][8 * g4 + 4]);
            const float Gv[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
            float kv[8], qv[8];
            IO::f32x8(pf.ka[mt], kv);
            IO::f32x8(pf.qa[mt], qv);
            uint16_t xk[8], xh[8], xl[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float eg = ex(Gv[e]);
                xk[e] = bfb(kv[e] * eg);
                split(qv[e] * eg, xh[e], xl[e]);
            }
            Kg[mt] = as_op(pack8(xk));
            Qh[mt] = as_op(pack8(xh));
            Ql[mt] = as_op(pack8(xl));
        }

        // ---- (c) prefetch the next chunk ----
        TbShare tbn{};
        if (ci + 1 < nch) {
            tbn = load_tb(p, cbase + ci + 1, h, tid);
            scan_load<TIn>(pf, p, cbase + ci + 1, row0 + C, min(C, len - (ci + 1) * C), h, j, w,
                           lane);
        }

        // ---- (d) partial (K e^G) S and (Q e^G) S over this wave's 32 rows ----
        {
            bf16x8_t Sh, Sl;
            pack_split(S[0], S[1], Sh, Sl);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            typename SM::Ex& E = sm.ex[par][w];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 x = mfma(Kg[mt], Sh, z);
                x = mfma(Kg[mt], Sl, x);
                f32x4 pq = mfma(Qh[mt], Sh, z);
                pq = mfma(Qh[mt], Sl, pq);
                pq = mfma(Ql[mt], Sh, pq);
                E.X[mt][lane] = x;
                E.P[mt][lane] = pq;
            }
        }
        lds_barrier();

        // ---- (e) U = TB (V - (K e^G) S) for all tokens of the chunk ----
        bf16x8_t Uh[2], Ul[2];
        {
            f32x4 D[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 xs = sm.ex[par][0].X[mt][lane];
                xs += sm.ex[par][1].X[mt][lane];
                xs += sm.ex[par][2].X[mt][lane];
                xs += sm.ex[par][3].X[mt][lane];
#pragma unroll
                for (int e = 0; e < 4; ++e) D[mt][e] = IO::f32(vcur[mt][e]) - xs[e];
            }
            bf16x8_t Dh[2], Dl[2];
            pack_split(D[0], D[1], Dh[0], Dl[0]);
            pack_split(D[2], D[3], Dh[1], Dl[1]);
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 U[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 u = z;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const bf16x8_t th = as_op(sm.tb[par][(mt * 2 + ks) * 64 + lane]);
                    const bf16x8_t tl = as_op(sm.tb[par][PLANE + (mt * 2 + ks) * 64 + lane]);
                    u = mfma(th, Dh[ks], u);
                    u = mfma(th, Dl[ks], u);
                    u = mfma(tl, Dh[ks], u);
                }
                U[mt] = u;
            }
            pack_split(U[0], U[1], Uh[0], Ul[0]);
            pack_split(U[2], U[3], Uh[1], Ul[1]);
        }

        // ---- (f) this wave's token tile of O = scale ((Q e^G) S + B U) ----
        {
            f32x4 po = sm.ex[par][0].P[w][lane];
            po += sm.ex[par][1].P[w][lane];
            po += sm.ex[par][2].P[w][lane];
            po += sm.ex[par][3].P[w][lane];
            f32x4 bu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const bf16x8_t bh = as_op(bcur[ks][0]), bl = as_op(bcur[ks][1]);
                bu = mfma(bh, Uh[ks], bu);
                bu = mfma(bh, Ul[ks], bu);
                bu = mfma(bl, Uh[ks], bu);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = tok_of(w, 4 * g4 + e);
                if (t < n) {
                    const float o = p.scale * (po[e] + bu[e]);
                    const int64_t oi = ((row0 + t) * p.H + h) * (int64_t)dv + j;
                    if (p.out_bf16)
                        static_cast<uint16_t*>(p.out)[oi] = bfb(o);
                    else
                        static_cast<float*>(p.out)[oi] = o;
                }
            }
        }

        // ---- (g) S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T U ----
        {
            const float4 gca = *reinterpret_cast<const float4*>(&Gs[C - 1][8 * g4]);
            const float4 gcb = *reinterpret_cast<const float4*>(&Gs[C - 1][8 * g4 + 4]);
            const f32x4 dec[2] = {f32x4{ex(gca.x), ex(gca.y), ex(gca.z), ex(gca.w)},
                                  f32x4{ex(gcb.x), ex(gcb.y), ex(gcb.z), ex(gcb.w)}};
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int cl = chan_of(m, i16);
                const float gcl = Gs[C - 1][cl];
                f32x4 s = S[m] * dec[m];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    uint16_t hh[8], ll[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int t = 32 * ks + 8 * g4 + e;
                        float kv;
                        if constexpr (SM::KSTAGE) {
                            kv = bff(sm.K[w][t][cl]);
                        } else {
                            kv = (t < n && SL * w + cl < dk)
                                     ? IO::f32(IO::load1(p.k, ((row0 + t) * p.H + h) * (int64_t)dk + SL * w + cl))
                                     : 0.f;
                        }
                        split(kv * ex(gcl - Gs[t][cl]), hh[e], ll[e]);
                    }
                    const bf16x8_t kh = as_op(pack8(hh)), kl = as_op(pack8(ll));
                    s = mfma(kh, Uh[ks], s);
                    s = mfma(kh, Ul[ks], s);
                    s = mfma(kl, Uh[ks], s);
                }
                S[m] = s;
            }
        }
        const int done = ci * C + n;
        if (p.interval > 0 && done % p.interval == 0) {
            float* __restrict__ dst =
                p.snapshots + ((sbase + done / p.interval - 1) * p.H + h) * (int64_t)dk * dv;
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = SL * w + 8 * g4 + 4 * m + e;
                    if (c < dk) dst[(int64_t)c * dv + j] = S[m][e];
                }
        }

        // ---- (h) TB of the next chunk into the other parity ----
        if (ci + 1 < nch) store_tb(sm.tb[par ^ 1], tbn, tid);
    }

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
        hipLaunchKernelGGL((prep_kernel<TIn>), dim3((unsigned)a.total_chunks, (unsigned)a.H), dim3(NT),
                           0, a.stream, pp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    ScanParams sp{};
    sp.q = a.q;
    sp.k = a.k;
    sp.v = a.v;
    sp.g = a.g;
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
    sp.out_bf16 = a.out_bf16 ? 1 : 0;
    sp.scale = a.scale;
    const int64_t nwg = (int64_t)a.num_seqs * a.H * sp.ntiles;
    sp.nwg = (int)nwg;
    hipLaunchKernelGGL((scan_kernel<TIn>), dim3((unsigned)nwg), dim3(NT), 0, a.stream, sp);
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
