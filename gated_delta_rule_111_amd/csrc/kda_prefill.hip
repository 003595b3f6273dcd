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
// Chunked form (derived from the recurrence; C = 32 rows per chunk, G = the
// inclusive cumulative sum of g inside the chunk, S = state at chunk start):
//   A_ts = b_t sum_c k_t[c] k_s[c] e^{G_t[c]-G_s[c]}   (s < t)
//   B_ts =     sum_c q_t[c] k_s[c] e^{G_t[c]-G_s[c]}   (s <= t)
//   T    = (I + A)^-1                                   (unit lower triangular)
//   W    = T (b . K . e^G),   U~ = T (b . V)           (the UT / WY transform)
//   U    = U~ - W S                                     (delta-rule targets)
//   O    = scale ((Q . e^G) S + B U)
//   S'   = Diag(e^{G_C}) S + (K . e^{G_C - G})^T U
// The Gram matrices A, B are contractions over channels with a per-channel
// decay between rows t and s; they are factorised per 16-row sub-chunk with
// a reference r so that both factors e^{G_t - r}, e^{r - G_s} stay within
// fp32 range (off-diagonal blocks: r = G at the end of the earlier
// sub-chunk, both factors <= 1; diagonal blocks: r = G at the sub-chunk's
// middle row, factors within e^{+-80}).  When a sub-chunk's decay span is
// too large for that, its diagonal blocks are evaluated pairwise instead.
//
// Precision: MFMA v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Operands
// that are not exact bf16 values are split into hi + lo bf16 and multiplied
// in two or three passes (hi*hi + hi*lo + lo*hi), which keeps ~16 bits; the
// KK^T Gram, b.K.e^G and W tolerate a single bf16 pass.  The state S is kept
// and carried in fp32 registers; snapshots are exact copies of it.
//
// Work decomposition: one workgroup (4 wavefronts) per (sequence, head,
// dv-tile of DVT columns).  Value columns evolve independently, so dv-tiles
// need no communication; each recomputes the dv-independent chunk quantities
// (A, B, T, W).  Inside the workgroup the S-dependent products are split over
// waves either by state rows (small DVT; partial sums combined through LDS)
// or by state columns (large DVT).  The contraction over state rows is always
// evaluated as one MFMA chain per 32-row K-step, started from zero, summed in
// K-step order, so results do not depend on DVT or on the wave split; with
// chunks aligned to each sequence start this makes snapshot resumption
// bit-exact.
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 32;                 // chunk rows
constexpr int NT = 256;               // threads per workgroup (4 waves)
constexpr float SPAN_LIMIT = 80.0f;   // |exponent| bound for the diagonal-block factors
constexpr int AP = 33;                // padded row stride of the fp32 32x32 tiles

__device__ __forceinline__ f32x4 mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint16_t bfb(float x) { return f32_to_bf16_bits(x); }
__device__ __forceinline__ float bff(uint16_t b) { return bf16_bits_to_f32(b); }

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in fp32)
__device__ __forceinline__ void split(float x, uint16_t& hi, uint16_t& lo) {
    hi = bfb(x);
    lo = bfb(x - bff(hi));
}

// 8 consecutive bf16 (16 bytes) as an MFMA operand
__device__ __forceinline__ bf16x8_t ld8(const uint16_t* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p));
}
// operand in the permuted K order used by the state products: elements 0..3
// are p[0..3], elements 4..7 are p[16..19]
__device__ __forceinline__ bf16x8_t ld4x2(const uint16_t* p) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    const uint2 b = *reinterpret_cast<const uint2*>(p + 16);
    return __builtin_bit_cast(bf16x8_t, make_uint4(a.x, a.y, b.x, b.y));
}
// two accumulator tiles (rows 4g..4g+3 and 16+4g..16+4g+3 of a 32-row block)
// packed as one operand in the same permuted K order, hi and lo parts
__device__ __forceinline__ void pack_split(const f32x4& x0, const f32x4& x1, bf16x8_t& hi,
                                           bf16x8_t& lo) {
    uint16_t h[8], l[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        split(x0[e], h[e], l[e]);
        split(x1[e], h[4 + e], l[4 + e]);
    }
    uint4 uh, ul;
    uh.x = h[0] | ((uint32_t)h[1] << 16); uh.y = h[2] | ((uint32_t)h[3] << 16);
    uh.z = h[4] | ((uint32_t)h[5] << 16); uh.w = h[6] | ((uint32_t)h[7] << 16);
    ul.x = l[0] | ((uint32_t)l[1] << 16); ul.y = l[2] | ((uint32_t)l[3] << 16);
    ul.z = l[4] | ((uint32_t)l[5] << 16); ul.w = l[6] | ((uint32_t)l[7] << 16);
    hi = __builtin_bit_cast(bf16x8_t, uh);
    lo = __builtin_bit_cast(bf16x8_t, ul);
}

__device__ __forceinline__ uint4 pack8(const uint16_t (&x)[8]) {
    uint4 u;
    u.x = x[0] | ((uint32_t)x[1] << 16); u.y = x[2] | ((uint32_t)x[3] << 16);
    u.z = x[4] | ((uint32_t)x[5] << 16); u.w = x[6] | ((uint32_t)x[7] << 16);
    return u;
}

__device__ __forceinline__ float ex(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

// ---------------------------------------------------------------------------
// Compile-time geometry
// ---------------------------------------------------------------------------
template <int DK, int DVT, typename TIn>
struct Geo {
    static constexpr int DKP = DK < 32 ? 32 : DK;      // channels padded to one K-step
    static constexpr int NKS = DKP / 32;               // K-steps over state rows
    static constexpr int RW = DVT >= 64 ? 1 : NKS;     // waves splitting state rows
    static constexpr int CWr = 4 / RW;
    static constexpr int CW = CWr < DVT / 16 ? CWr : DVT / 16;  // waves splitting columns
    static constexpr int NSW = RW * CW;                // waves holding state
    static constexpr int KSP = NKS / RW;               // K-steps per state wave
    static constexpr int JT = DVT / CW / 16;           // 16-column tiles per state wave
    static constexpr int NJ = DVT / 16;                // 16-column tiles per workgroup
    static constexpr bool F32IN = sizeof(TIn) == 4;
    static constexpr int VPL = F32IN ? 2 : 1;          // V planes (fp32 inputs are split)
    static constexpr int VEC = 16 / sizeof(TIn);       // elements per 16-byte vector
    static_assert(NSW <= 4 && NSW >= 1 && JT >= 1, "wave geometry");
    static_assert(DKP * 2 <= NT, "one prep thread per 8 channels x 2 rows");
};

template <int DK, int DVT, typename TIn>
struct Smem {
    using G_ = Geo<DK, DVT, TIn>;
    static constexpr int DKP = G_::DKP;
    float G[C][DKP];           // cumulative log-decay inside the chunk
    float decay[DKP];          // e^{G_C}
    float beta[C];
    union {
        struct {               // Gram operands (dead after the Gram products)
            uint16_t XKd[C][DKP];        // k_t e^{G_t - r_diag}          hi
            uint16_t XK1[16][DKP];       // k_t e^{G_t - G_15}, t >= 16   hi
            uint16_t XQd[2][C][DKP];     // q_t e^{G_t - r_diag}          hi, lo
            uint16_t XQ1[2][16][DKP];    // q_t e^{G_t - G_15}, t >= 16   hi, lo
            uint16_t YKd[2][C][DKP];     // k_s e^{r_diag - G_s}          hi, lo
            uint16_t YK1[2][16][DKP];    // k_s e^{G_15 - G_s}, s < 16    hi, lo
        } gram;
        struct {               // state-phase buffers
            uint16_t W[C][DKP];                               // W (bf16)
            f32x4 PW[G_::RW > 1 ? G_::NKS : 1][2][G_::NJ][64];  // per-K-step partials of W S
            f32x4 PQ[G_::RW > 1 ? G_::NKS : 1][2][G_::NJ][64];  // ... of (Q e^G) S
        } st;
    } u;
    uint16_t KgT[DKP][C];      // (b_s k_s e^{G_s})^T                       hi
    uint16_t Qg[2][C][DKP];    // q_t e^{G_t}                               hi, lo
    uint16_t KdT[2][DKP][C];   // (k_t e^{G_C - G_t})^T                     hi, lo
    uint16_t VT[G_::VPL][DVT][C];  // V^T                                   (hi, lo)
    float A[C][AP];
    float B[C][AP];
    float Tf[C][AP];
    float M1[16][17];
    uint16_t Bhl[2][C][C];
    uint16_t Thl[2][C][C];
    uint16_t TBhl[2][C][C];
    int extreme;
};

struct Params {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu;
    const float* init;
    void* out;
    float* final_state;
    float* snapshots;
    int32_t interval;
    int H;
    int num_seqs;
    int ntiles;
    int nwg;
    float scale;
    int out_bf16;
};

// Prefetch registers of one chunk for one prep thread: 2 rows x 8 channels of
// g, k, q, the two betas, and this thread's share of V.
template <int DK, int DVT, typename TIn>
struct Prefetch {
    using G_ = Geo<DK, DVT, TIn>;
    static constexpr int VV = C * DVT / G_::VEC;                 // 16-byte V vectors per chunk
    static constexpr int VPT = (VV + NT - 1) / NT;              // per thread
    float4 g[2][2];
    uint4 k[2][sizeof(TIn) / 2];   // 8 elements = 16 B (bf16) or 32 B (fp32)
    uint4 q[2][sizeof(TIn) / 2];
    float b[2];
    uint4 v[VPT];
};

template <int DK, int DVT, typename TIn>
__device__ __forceinline__ void load_chunk(Prefetch<DK, DVT, TIn>& pf, const Params& p, int64_t row0,
                                           int n, int h, int tile, int tid) {
    using G_ = Geo<DK, DVT, TIn>;
    const int cg = tid >> 4, tb = tid & 15;
    const int c0 = cg * 8;
    const bool chan_ok = c0 < DK;
    const TIn* __restrict__ kp = static_cast<const TIn*>(p.k);
    const TIn* __restrict__ qp = static_cast<const TIn*>(p.q);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int t = 2 * tb + r;
        const bool ok = chan_ok && t < n;
        const int64_t base = ((row0 + t) * p.H + h) * (int64_t)DK + c0;
        if (ok) {
            pf.g[r][0] = *reinterpret_cast<const float4*>(p.g + base);
            pf.g[r][1] = *reinterpret_cast<const float4*>(p.g + base + 4);
#pragma unroll
            for (int i = 0; i < (int)(sizeof(TIn) / 2); ++i) {
                pf.k[r][i] = *reinterpret_cast<const uint4*>(kp + base + i * G_::VEC);
                pf.q[r][i] = *reinterpret_cast<const uint4*>(qp + base + i * G_::VEC);
            }
        } else {
            pf.g[r][0] = pf.g[r][1] = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int i = 0; i < (int)(sizeof(TIn) / 2); ++i) {
                pf.k[r][i] = make_uint4(0, 0, 0, 0);
                pf.q[r][i] = make_uint4(0, 0, 0, 0);
            }
        }
        pf.b[r] = (t < n) ? p.beta[(row0 + t) * p.H + h] : 0.f;
    }
    // V: rows t, 16-byte vectors of VEC columns of this dv-tile
    constexpr int VPR = DVT / G_::VEC;  // vectors per row
    const TIn* __restrict__ vp = static_cast<const TIn*>(p.v);
    const int DVfull = p.ntiles * DVT;
#pragma unroll
    for (int i = 0; i < Prefetch<DK, DVT, TIn>::VPT; ++i) {
        const int vi = tid + i * NT;
        const int t = vi / VPR, cv = vi % VPR;
        if (vi < Prefetch<DK, DVT, TIn>::VV && t < n)
            pf.v[i] = *reinterpret_cast<const uint4*>(
                vp + ((row0 + t) * p.H + h) * (int64_t)DVfull + tile * DVT + cv * G_::VEC);
        else
            pf.v[i] = make_uint4(0, 0, 0, 0);
    }
}

template <typename TIn>
__device__ __forceinline__ void decode8(const uint4* src, float (&x)[8]) {
    if constexpr (sizeof(TIn) == 2) {
        const uint4 u = src[0];
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = bff((uint16_t)(w[j] & 0xffffu));
            x[2 * j + 1] = bff((uint16_t)(w[j] >> 16));
        }
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 u = src[i];
            x[4 * i + 0] = __uint_as_float(u.x); x[4 * i + 1] = __uint_as_float(u.y);
            x[4 * i + 2] = __uint_as_float(u.z); x[4 * i + 3] = __uint_as_float(u.w);
        }
    }
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <int DK, int DVT, typename TIn>
__global__ __launch_bounds__(NT) void prefill_kernel(Params p) {
    using G_ = Geo<DK, DVT, TIn>;
    constexpr int DKP = G_::DKP, NKS = G_::NKS, RW = G_::RW, KSP = G_::KSP, JT = G_::JT;
    __shared__ Smem<DK, DVT, TIn> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g4 = lane >> 4, l16 = lane & 15;

    // workgroup -> (sequence, head, dv-tile); dv-tiles of one head are given
    // consecutive logical ids, and consecutive logical ids are placed on one
    // XCD (workgroups are dealt round-robin over the 8 XCDs), so the tiles of
    // a head share K, Q, g through that XCD's L2.
    int L = blockIdx.x;
    if ((p.nwg & 7) == 0) L = (blockIdx.x & 7) * (p.nwg >> 3) + (blockIdx.x >> 3);
    const int tile = L % p.ntiles;
    const int chain = L / p.ntiles;
    const int b = chain / p.H, h = chain % p.H;
    const int DV = p.ntiles * DVT;
    const int64_t seq0 = p.cu[b];
    const int len = p.cu[b + 1] - p.cu[b];
    int64_t snap_base = 0;
    if (p.interval > 0)
        for (int i = 0; i < b; ++i) snap_base += (p.cu[i + 1] - p.cu[i]) / p.interval;

    // ---- state registers (state waves only) ------------------------------
    const bool swave = wave < G_::NSW;
    const int rw = wave % RW, cw = wave / RW;
    f32x4 S[KSP][2][JT];
    const int64_t sbase = ((int64_t)b * p.H + h) * DK;  // state row base
#pragma unroll
    for (int kk = 0; kk < KSP; ++kk)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const int c = 16 * (2 * (rw * KSP + kk) + m) + 4 * g4;
                const int j = tile * DVT + 16 * (cw * JT + jt) + l16;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    S[kk][m][jt][e] = (swave && p.init && c + e < DK)
                                          ? p.init[(sbase + c + e) * DV + j] : 0.f;
            }

    const int nchunks = (len + C - 1) / C;
    Prefetch<DK, DVT, TIn> pf;
    if (nchunks > 0) load_chunk<DK, DVT, TIn>(pf, p, seq0, len < C ? len : C, h, tile, tid);

    for (int ci = 0; ci < nchunks; ++ci) {
        const int64_t row0 = seq0 + (int64_t)ci * C;
        const int n = (len - ci * C) < C ? (len - ci * C) : C;

        // ================= prep: cumulative decay and all operands =================
        {
            const int cg = tid >> 4, tb = tid & 15;
            const int c0 = cg * 8, t0 = 2 * tb;
            const bool active = cg < DKP / 8;
            float gf[2][8], kf[2][8], qf[2][8];
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                gf[r][0] = pf.g[r][0].x; gf[r][1] = pf.g[r][0].y; gf[r][2] = pf.g[r][0].z;
                gf[r][3] = pf.g[r][0].w; gf[r][4] = pf.g[r][1].x; gf[r][5] = pf.g[r][1].y;
                gf[r][6] = pf.g[r][1].z; gf[r][7] = pf.g[r][1].w;
                decode8<TIn>(pf.k[r], kf[r]);
                decode8<TIn>(pf.q[r], qf[r]);
            }
            const float b0 = pf.b[0], b1 = pf.b[1];
            // inclusive scan of the row-pair sums over the 16 lanes of this channel group
            float G0[8], G1[8];
            int ext = 0;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float pair = gf[0][c] + gf[1][c];
                float incl = pair;
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) {
                    const float y = __shfl_up(incl, off, 16);
                    if (tb >= off) incl += y;
                }
                float excl = __shfl_up(incl, 1, 16);
                if (tb == 0) excl = 0.f;
                G0[c] = excl + gf[0][c];
                G1[c] = G0[c] + gf[1][c];
            }
            // references: G_7 (row 7), G_15, G_23, G_31 = G_C; and G_0, G_16
            const int lb = lane & ~15;
            float r0[8], r01[8], r1[8], GC[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                r0[c] = __shfl(G1[c], lb + 3, 64);
                r01[c] = __shfl(G1[c], lb + 7, 64);
                r1[c] = __shfl(G1[c], lb + 11, 64);
                GC[c] = __shfl(G1[c], lb + 15, 64);
                const float Gfirst0 = __shfl(G0[c], lb + 0, 64);
                const float Gfirst1 = __shfl(G0[c], lb + 8, 64);
                ext |= (Gfirst0 - r0[c] > SPAN_LIMIT) | (r0[c] - r01[c] > SPAN_LIMIT) |
                       (Gfirst1 - r1[c] > SPAN_LIMIT) | (r1[c] - GC[c] > SPAN_LIMIT);
            }
            if (active) {
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int t = t0 + r;
                    const float* Gr = r == 0 ? G0 : G1;
                    const float bt = r == 0 ? b0 : b1;
                    uint16_t xk[8], xqh[8], xql[8], ykh[8], ykl[8], x1h[8], x1l[8], x1k[8];
                    uint16_t qgh[8], qgl[8];
                    uint16_t kg[8], kdh[8], kdl[8];
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        const float rd = t < 16 ? r0[c] : r1[c];
                        const float xe = ex(Gr[c] - rd);
                        const float ye = ex(rd - Gr[c]);
                        xk[c] = bfb(kf[r][c] * xe);
                        split(qf[r][c] * xe, xqh[c], xql[c]);
                        split(kf[r][c] * ye, ykh[c], ykl[c]);
                        if (t >= 16) {
                            const float e1 = ex(Gr[c] - r01[c]);
                            x1k[c] = bfb(kf[r][c] * e1);
                            split(qf[r][c] * e1, x1h[c], x1l[c]);
                        } else {
                            const float e1 = ex(r01[c] - Gr[c]);
                            split(kf[r][c] * e1, x1h[c], x1l[c]);
                        }
                        const float eg = ex(Gr[c]);
                        kg[c] = bfb(bt * kf[r][c] * eg);
                        split(qf[r][c] * eg, qgh[c], qgl[c]);
                        split(kf[r][c] * ex(GC[c] - Gr[c]), kdh[c], kdl[c]);
                    }
                    *reinterpret_cast<uint4*>(&sm.u.gram.XKd[t][c0]) = pack8(xk);
                    *reinterpret_cast<uint4*>(&sm.u.gram.XQd[0][t][c0]) = pack8(xqh);
                    *reinterpret_cast<uint4*>(&sm.u.gram.XQd[1][t][c0]) = pack8(xql);
                    *reinterpret_cast<uint4*>(&sm.u.gram.YKd[0][t][c0]) = pack8(ykh);
                    *reinterpret_cast<uint4*>(&sm.u.gram.YKd[1][t][c0]) = pack8(ykl);
                    if (t >= 16) {
                        *reinterpret_cast<uint4*>(&sm.u.gram.XK1[t - 16][c0]) = pack8(x1k);
                        *reinterpret_cast<uint4*>(&sm.u.gram.XQ1[0][t - 16][c0]) = pack8(x1h);
                        *reinterpret_cast<uint4*>(&sm.u.gram.XQ1[1][t - 16][c0]) = pack8(x1l);
                    } else {
                        *reinterpret_cast<uint4*>(&sm.u.gram.YK1[0][t][c0]) = pack8(x1h);
                        *reinterpret_cast<uint4*>(&sm.u.gram.YK1[1][t][c0]) = pack8(x1l);
                    }
                    *reinterpret_cast<uint4*>(&sm.Qg[0][t][c0]) = pack8(qgh);
                    *reinterpret_cast<uint4*>(&sm.Qg[1][t][c0]) = pack8(qgl);
                    *reinterpret_cast<float4*>(&sm.G[t][c0]) =
                        make_float4(Gr[0], Gr[1], Gr[2], Gr[3]);
                    *reinterpret_cast<float4*>(&sm.G[t][c0 + 4]) =
                        make_float4(Gr[4], Gr[5], Gr[6], Gr[7]);
                    // transposed buffers [channel][row]
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        sm.KgT[c0 + c][t] = kg[c];
                        sm.KdT[0][c0 + c][t] = kdh[c];
                        sm.KdT[1][c0 + c][t] = kdl[c];
                    }
                }
                if (tb == 15) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) sm.decay[c0 + c] = ex(GC[c]);
                }
                if (cg == 0) {
                    sm.beta[t0] = b0;
                    sm.beta[t0 + 1] = b1;
                }
            }
            // V^T (split for fp32 inputs)
            constexpr int VPR = DVT / G_::VEC;
#pragma unroll
            for (int i = 0; i < Prefetch<DK, DVT, TIn>::VPT; ++i) {
                const int vi = tid + i * NT;
                if (vi < Prefetch<DK, DVT, TIn>::VV) {
                    const int t = vi / VPR, cv = vi % VPR;
                    if constexpr (!G_::F32IN) {
                        const uint4 u = pf.v[i];
                        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            sm.VT[0][cv * 8 + 2 * jj][t] = (uint16_t)(w[jj] & 0xffffu);
                            sm.VT[0][cv * 8 + 2 * jj + 1][t] = (uint16_t)(w[jj] >> 16);
                        }
                    } else {
                        const uint4 u = pf.v[i];
                        const float x[4] = {__uint_as_float(u.x), __uint_as_float(u.y),
                                            __uint_as_float(u.z), __uint_as_float(u.w)};
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            uint16_t hh, ll;
                            split(x[jj], hh, ll);
                            sm.VT[0][cv * 4 + jj][t] = hh;
                            sm.VT[G_::VPL - 1][cv * 4 + jj][t] = ll;
                        }
                    }
                }
            }
            const int any_ext = __syncthreads_or(ext);
            if (tid == 0) sm.extreme = any_ext;
        }
        // the prefetch registers are free: start loading the next chunk
        if (ci + 1 < nchunks) {
            const int n2 = (len - (ci + 1) * C) < C ? (len - (ci + 1) * C) : C;
            load_chunk<DK, DVT, TIn>(pf, p, row0 + C, n2, h, tile, tid);
        }

        // ================= Gram matrices A (wave 0) and B (waves 1-3) ================
        {
            const int blk = wave == 0 ? 0 : wave - 1;  // 0: (0,0)  1: (1,1)  2: (1,0)
            const int rb = blk == 0 ? 0 : 16;          // row block start
            const int cb = blk == 1 ? 16 : 0;          // column block start
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (wave == 0) {
#pragma unroll
                for (int bb = 0; bb < 3; ++bb) {
                    const uint16_t* X = bb == 2 ? &sm.u.gram.XK1[0][0] : &sm.u.gram.XKd[bb * 16][0];
                    const uint16_t* Y = bb == 2 ? &sm.u.gram.YK1[0][0][0] : &sm.u.gram.YKd[0][bb * 16][0];
                    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        a = mfma(ld8(X + l16 * DKP + 32 * ks + 8 * g4),
                                 ld8(Y + l16 * DKP + 32 * ks + 8 * g4), a);
                    const int rb2 = bb == 0 ? 0 : 16, cb2 = bb == 1 ? 16 : 0;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int t = rb2 + 4 * g4 + e, s = cb2 + l16;
                        sm.A[t][s] = (s < t) ? a[e] * sm.beta[t] : 0.f;
                    }
                }
            } else {
                const uint16_t* X0 = blk == 2 ? &sm.u.gram.XQ1[0][0][0] : &sm.u.gram.XQd[0][rb][0];
                const uint16_t* X1 = blk == 2 ? &sm.u.gram.XQ1[1][0][0] : &sm.u.gram.XQd[1][rb][0];
                const uint16_t* Y0 = blk == 2 ? &sm.u.gram.YK1[0][0][0] : &sm.u.gram.YKd[0][cb][0];
                const uint16_t* Y1 = blk == 2 ? &sm.u.gram.YK1[1][0][0] : &sm.u.gram.YKd[1][cb][0];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const int off = l16 * DKP + 32 * ks + 8 * g4;
                    const bf16x8_t xh = ld8(X0 + off), xl = ld8(X1 + off);
                    const bf16x8_t yh = ld8(Y0 + off), yl = ld8(Y1 + off);
                    acc = mfma(xh, yh, acc);
                    acc = mfma(xh, yl, acc);
                    acc = mfma(xl, yh, acc);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = rb + 4 * g4 + e, s = cb + l16;
                    sm.B[t][s] = (s <= t) ? acc[e] : 0.f;
                }
            }
        }
        __syncthreads();

        // extreme decay inside a sub-chunk: diagonal blocks pairwise in fp32
        if (sm.extreme) {
            const TIn* __restrict__ kp = static_cast<const TIn*>(p.k);
            const TIn* __restrict__ qp = static_cast<const TIn*>(p.q);
            for (int idx = tid; idx < 512; idx += NT) {
                const int blk = idx >> 8, tl = (idx >> 4) & 15, sl = idx & 15;
                if (sl > tl) continue;
                const int t = blk * 16 + tl, s = blk * 16 + sl;
                float sa = 0.f, sb = 0.f;
                if (t < n) {
                    const int64_t bt = ((row0 + t) * p.H + h) * (int64_t)DK;
                    const int64_t bs = ((row0 + s) * p.H + h) * (int64_t)DK;
                    for (int c = 0; c < DK; ++c) {
                        float kt, ks_, qt;
                        if constexpr (G_::F32IN) {
                            kt = kp[bt + c]; ks_ = kp[bs + c]; qt = qp[bt + c];
                        } else {
                            kt = bff(reinterpret_cast<const uint16_t*>(kp)[bt + c]);
                            ks_ = bff(reinterpret_cast<const uint16_t*>(kp)[bs + c]);
                            qt = bff(reinterpret_cast<const uint16_t*>(qp)[bt + c]);
                        }
                        const float e = ex(sm.G[t][c] - sm.G[s][c]);
                        sa = fmaf(kt * ks_, e, sa);
                        sb = fmaf(qt * ks_, e, sb);
                    }
                }
                sm.A[t][s] = (s < t) ? sa * sm.beta[t] : 0.f;
                sm.B[t][s] = sb;
            }
            __syncthreads();
        }

        // ================= T = (I + A)^-1 ===============================================
        if (wave == 0 && lane < 32) {
            // diagonal 16x16 blocks by forward substitution, one column per lane
            const int bo = (lane >> 4) * 16, j = lane & 15;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) acc = fmaf(sm.A[bo + i][bo + m], x[m], acc);
                x[i] = (i == j) ? 1.f : (i > j ? -acc : 0.f);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sm.Tf[bo + i][bo + j] = x[i];
        }
        __syncthreads();
        {
            const int i = tid >> 4, j = tid & 15;
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) acc = fmaf(sm.A[16 + i][m], sm.Tf[m][j], acc);
            sm.M1[i][j] = acc;
        }
        __syncthreads();
        {
            const int i = tid >> 4, j = tid & 15;
            float acc = 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) acc = fmaf(sm.Tf[16 + i][16 + m], sm.M1[m][j], acc);
            sm.Tf[16 + i][j] = -acc;
            sm.Tf[i][16 + j] = 0.f;
        }
        __syncthreads();
        {
            const int t = tid >> 3, s0 = (tid & 7) * 4;
            uint16_t th[4], tl[4], bh[4], bl[4], qh[4], ql[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = s0 + e;
                const float tv = sm.Tf[t][s];
                split(tv, th[e], tl[e]);
                split(tv * sm.beta[s], bh[e], bl[e]);
                split(s <= t ? sm.B[t][s] : 0.f, qh[e], ql[e]);
            }
            auto p4 = [](const uint16_t (&x)[4]) {
                return make_uint2(x[0] | ((uint32_t)x[1] << 16), x[2] | ((uint32_t)x[3] << 16));
            };
            *reinterpret_cast<uint2*>(&sm.Thl[0][t][s0]) = p4(th);
            *reinterpret_cast<uint2*>(&sm.Thl[1][t][s0]) = p4(tl);
            *reinterpret_cast<uint2*>(&sm.TBhl[0][t][s0]) = p4(bh);
            *reinterpret_cast<uint2*>(&sm.TBhl[1][t][s0]) = p4(bl);
            *reinterpret_cast<uint2*>(&sm.Bhl[0][t][s0]) = p4(qh);
            *reinterpret_cast<uint2*>(&sm.Bhl[1][t][s0]) = p4(ql);
        }
        __syncthreads();

        // ================= W = T (b K e^G), computed as W^T = KgT T^T ==================
        {
            constexpr int NTILE = DKP / 8;  // (DKP/16 channel tiles) x (2 row tiles)
            for (int ti = wave; ti < NTILE; ti += 4) {
                const int mc = ti >> 1, nt = ti & 1;
                const bf16x8_t a = ld8(&sm.KgT[mc * 16 + l16][8 * g4]);
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma(a, ld8(&sm.Thl[0][nt * 16 + l16][8 * g4]), acc);
                acc = mfma(a, ld8(&sm.Thl[1][nt * 16 + l16][8 * g4]), acc);
                uint16_t w4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) w4[e] = bfb(acc[e]);
                *reinterpret_cast<uint2*>(&sm.u.st.W[nt * 16 + l16][mc * 16 + 4 * g4]) =
                    make_uint2(w4[0] | ((uint32_t)w4[1] << 16), w4[2] | ((uint32_t)w4[3] << 16));
            }
        }
        __syncthreads();

        // ================= state products ===============================================
        f32x4 sumW[2][JT], sumQ[2][JT];
        if (swave) {
#pragma unroll
            for (int kk = 0; kk < KSP; ++kk) {
                const int ks = rw * KSP + kk;
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) {
                    bf16x8_t sh, sl;
                    pack_split(S[kk][0][jt], S[kk][1][jt], sh, sl);
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const int roff = (mt * 16 + l16) * DKP + 32 * ks + 4 * g4;
                        const bf16x8_t w = ld4x2(&sm.u.st.W[0][0] + roff);
                        const bf16x8_t qh = ld4x2(&sm.Qg[0][0][0] + roff);
                        const bf16x8_t ql = ld4x2(&sm.Qg[1][0][0] + roff);
                        f32x4 pw = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
                        pw = mfma(w, sh, pw);
                        pw = mfma(w, sl, pw);
                        pq = mfma(qh, sh, pq);
                        pq = mfma(qh, sl, pq);
                        pq = mfma(ql, sh, pq);
                        if constexpr (RW > 1) {
                            sm.u.st.PW[ks][mt][cw * JT + jt][lane] = pw;
                            sm.u.st.PQ[ks][mt][cw * JT + jt][lane] = pq;
                        } else {
                            if (kk == 0) {
                                sumW[mt][jt] = pw;
                                sumQ[mt][jt] = pq;
                            } else {
                                sumW[mt][jt] += pw;
                                sumQ[mt][jt] += pq;
                            }
                        }
                    }
                }
            }
        }
        if constexpr (RW > 1) {
            __syncthreads();
            if (swave) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        const int nj = cw * JT + jt;
                        sumW[mt][jt] = sm.u.st.PW[0][mt][nj][lane];
                        sumQ[mt][jt] = sm.u.st.PQ[0][mt][nj][lane];
#pragma unroll
                        for (int ks = 1; ks < NKS; ++ks) {
                            sumW[mt][jt] += sm.u.st.PW[ks][mt][nj][lane];
                            sumQ[mt][jt] += sm.u.st.PQ[ks][mt][nj][lane];
                        }
                    }
            }
        }
        if (swave) {
            // U = T (b V) - W S, in accumulator layout [t][j]
            bf16x8_t uh[JT], ul[JT];
            f32x4 U[2][JT];
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const int nj = cw * JT + jt;
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const bf16x8_t th = ld8(&sm.TBhl[0][mt * 16 + l16][8 * g4]);
                    const bf16x8_t tl = ld8(&sm.TBhl[1][mt * 16 + l16][8 * g4]);
                    const bf16x8_t vh = ld8(&sm.VT[0][nj * 16 + l16][8 * g4]);
                    f32x4 ut = {0.f, 0.f, 0.f, 0.f};
                    ut = mfma(th, vh, ut);
                    if constexpr (G_::F32IN) {
                        const bf16x8_t vl = ld8(&sm.VT[G_::VPL - 1][nj * 16 + l16][8 * g4]);
                        ut = mfma(th, vl, ut);
                    }
                    ut = mfma(tl, vh, ut);
                    U[mt][jt] = ut - sumW[mt][jt];
                }
                pack_split(U[0][jt], U[1][jt], uh[jt], ul[jt]);
            }
            // O = scale ((Q e^G) S + B U), written by the first row-wave of each column group
            if (rw == 0) {
                const bool ob = p.out_bf16 != 0;
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) {
                    const int j = tile * DVT + 16 * (cw * JT + jt) + l16;
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const int roff = (mt * 16 + l16) * C + 4 * g4;
                        const bf16x8_t bh = ld4x2(&sm.Bhl[0][0][0] + roff);
                        const bf16x8_t bl = ld4x2(&sm.Bhl[1][0][0] + roff);
                        f32x4 bu = {0.f, 0.f, 0.f, 0.f};
                        bu = mfma(bh, uh[jt], bu);
                        bu = mfma(bh, ul[jt], bu);
                        bu = mfma(bl, uh[jt], bu);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int t = mt * 16 + 4 * g4 + e;
                            if (t < n) {
                                const float o = p.scale * (sumQ[mt][jt][e] + bu[e]);
                                const int64_t oi = ((row0 + t) * p.H + h) * (int64_t)DV + j;
                                if (ob)
                                    static_cast<uint16_t*>(p.out)[oi] = bfb(o);
                                else
                                    static_cast<float*>(p.out)[oi] = o;
                            }
                        }
                    }
                }
            }
            // S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T U
#pragma unroll
            for (int kk = 0; kk < KSP; ++kk)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int crow = 16 * (2 * (rw * KSP + kk) + m);
                    const bf16x8_t kh = ld4x2(&sm.KdT[0][crow + l16][4 * g4]);
                    const bf16x8_t kl = ld4x2(&sm.KdT[1][crow + l16][4 * g4]);
                    const float d0 = sm.decay[crow + 4 * g4 + 0], d1 = sm.decay[crow + 4 * g4 + 1];
                    const float d2 = sm.decay[crow + 4 * g4 + 2], d3 = sm.decay[crow + 4 * g4 + 3];
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) {
                        f32x4 s = S[kk][m][jt];
                        s[0] *= d0; s[1] *= d1; s[2] *= d2; s[3] *= d3;
                        s = mfma(kh, uh[jt], s);
                        s = mfma(kh, ul[jt], s);
                        s = mfma(kl, uh[jt], s);
                        S[kk][m][jt] = s;
                    }
                }
            // snapshot at block boundaries of this sequence
            const int done = ci * C + n;
            if (p.interval > 0 && done % p.interval == 0) {
                const int64_t jsnap = done / p.interval - 1;
                float* __restrict__ dst = p.snapshots + ((snap_base + jsnap) * p.H + h) * (int64_t)DK * DV;
#pragma unroll
                for (int kk = 0; kk < KSP; ++kk)
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt) {
                            const int c = 16 * (2 * (rw * KSP + kk) + m) + 4 * g4;
                            const int j = tile * DVT + 16 * (cw * JT + jt) + l16;
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (c + e < DK) dst[(int64_t)(c + e) * DV + j] = S[kk][m][jt][e];
                        }
            }
        }
        __syncthreads();
    }

    // final state
    if (swave) {
#pragma unroll
        for (int kk = 0; kk < KSP; ++kk)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int jt = 0; jt < JT; ++jt) {
                    const int c = 16 * (2 * (rw * KSP + kk) + m) + 4 * g4;
                    const int j = tile * DVT + 16 * (cw * JT + jt) + l16;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c + e < DK) p.final_state[(sbase + c + e) * DV + j] = S[kk][m][jt][e];
                }
    }
}

template <int DK, int DVT, typename TIn>
hipError_t launch_t(const PrefillArgs& a, Params p) {
    p.ntiles = a.dv / DVT;
    const int64_t nwg = (int64_t)a.num_seqs * a.H * p.ntiles;
    if (nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    p.nwg = (int)nwg;
    hipLaunchKernelGGL((prefill_kernel<DK, DVT, TIn>), dim3((unsigned)nwg), dim3(NT), 0, a.stream, p);
    return hipGetLastError();
}

// dv-tile width: the widest tile that still gives every CU a workgroup
// (each dv-tile recomputes the dv-independent chunk work, so wider is cheaper
// whenever the chip is already full).
int pick_dvt(int dv, int64_t chains, bool f32in) {
    int dvt = dv;
    const int cap = f32in ? 16 : 128;
    while (dvt > cap) dvt /= 2;
    while (dvt > 16 && chains * (dv / dvt) < 256) dvt /= 2;
    return dvt;
}

template <int DK, typename TIn>
hipError_t launch_dk(const PrefillArgs& a, const Params& p) {
    const int dvt = pick_dvt(a.dv, (int64_t)a.num_seqs * a.H, sizeof(TIn) == 4);
    if constexpr (sizeof(TIn) == 4) {
        return launch_t<DK, 16, TIn>(a, p);
    } else {
        switch (dvt) {
            case 16: return launch_t<DK, 16, TIn>(a, p);
            case 32: if constexpr (DK >= 32) return launch_t<DK, 32, TIn>(a, p); break;
            case 64: if constexpr (DK >= 64) return launch_t<DK, 64, TIn>(a, p); break;
            case 128: if constexpr (DK >= 128) return launch_t<DK, 128, TIn>(a, p); break;
        }
        return hipErrorInvalidValue;
    }
}

}  // namespace

size_t prefill_workspace_bytes(int, int, int, int, int64_t) { return 0; }

hipError_t launch_prefill(const PrefillArgs& a) {
    Params p{};
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.g = a.g;
    p.beta = a.beta;
    p.cu = a.cu_dev;
    p.init = a.init;
    p.out = a.out;
    p.final_state = a.final_state;
    p.snapshots = a.snapshots;
    p.interval = a.interval;
    p.H = a.H;
    p.num_seqs = a.num_seqs;
    p.scale = a.scale;
    p.out_bf16 = a.out_bf16 ? 1 : 0;
    if (a.in_bf16) {
        switch (a.dk) {
            case 16: return launch_dk<16, bf16_t>(a, p);
            case 32: return launch_dk<32, bf16_t>(a, p);
            case 64: return launch_dk<64, bf16_t>(a, p);
            case 128: return launch_dk<128, bf16_t>(a, p);
        }
    } else {
        switch (a.dk) {
            case 16: return launch_dk<16, float>(a, p);
            case 32: return launch_dk<32, float>(a, p);
            case 64: return launch_dk<64, float>(a, p);
            case 128: return launch_dk<128, float>(a, p);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
