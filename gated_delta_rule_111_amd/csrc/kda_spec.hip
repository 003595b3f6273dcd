// kda_spec.hip -- speculative verify, commit and the fused step for drafts of
// at most 8 tokens, in the chunked form of the recurrence.  gfx950.
//
// The recurrence of "Kimi K3 technical FAQ", question "What is KDA, and why
// does a serving engineer care?" (delta rule with a per-channel forget gate,
// read as S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T, o_t = scale S_t^T
// q_t), over a draft of n tokens from the resident state S, with G the
// inclusive cumulative sum of g = log(a) over the draft:
//   A_ts = b_t sum_c k_t k_s e^(G_t - G_s)   (s < t)     T = (I + A)^-1
//   B_ts = sum_c q_t k_s e^(G_t - G_s)       (s <= t)    TB = T Diag(b)
//   W  = TB (K e^G),   M = B TB,   Q' = Q e^G - M (K e^G),
//   U~ = TB V,   O~ = M V
// verify: O = scale (Q' S + O~) for every draft token;
// commit of the first a tokens: U = U~ - W S (rows < a) and
//   S' = Diag(e^(G_{a-1})) S + sum_{t<a} (k_t e^(G_{a-1} - G_t)) u_t^T.
// With alpha in (0, 1] every exponent above is <= 0, so no factor overflows.
// This is the algebra of the chunked prefill, for one short chunk: the
// token-side part (n x n Grams, the triangular solve, W, Q', U~, O~) costs
// O(n^2 dk) per (sequence, head) and the state enters only through Q' S,
// W S and one rank-n update: 2 + 1/n multiply-adds per state element and
// token for a commit, 1 for a verify, against 3 and 4 when walking the
// tokens one at a time.
//
// One workgroup per (sequence, head).  A wave owns 32 columns (128 bytes of
// every state row it touches) of one half of the rows; a lane 4 columns and
// dk/16 rows, the row group the fastest lane index, so the sums over a half's
// rows are DPP moves inside the wave and the two halves meet once per phase
// in LDS.  The draft's tokens are loaded into registers first and the state
// after them: the token-side work in LDS then runs while the state is still
// in flight.  The fused step loads both drafts (the previous one to commit,
// the new one to verify) up front into two LDS buffers.
#include <type_traits>

#include "kda_common.h"
#include "kda_internal.h"

namespace kda {
namespace {

constexpr int SP_MAX = 8;   // draft tokens handled here

// state tile split: columns per wave, row groups in a wave, row halves
template <int DK, int DV>
struct SpecLayout {
    static constexpr int CW = DV < 32 ? DV : 32;
    static constexpr int CG = CW / 4;
    static constexpr int RG = 64 / CG;
    static constexpr int RH = DK / RG >= 2 ? 2 : 1;
    static constexpr int RPL = DK / (RG * RH);
    static constexpr int CB = DV / CW;
    static constexpr int WAVES = CB * RH;
};

// one draft's tokens in fp32; G holds g, then its cumulative sum.  Once the
// Grams are formed, q holds Q' (verify) or W (commit) and, in a commit, k
// holds k_t e^(G_{a-1} - G_t), each written by the thread that owns the
// channel; v holds O~ (verify) or U~ (commit), each written by the thread
// that owns the column.
template <int DK, int DV>
struct SpecTokens {
    float k[SP_MAX][DK];
    float q[SP_MAX][DK];
    float G[SP_MAX][DK];
    float v[SP_MAX][DV];
    float beta[SP_MAX];
    float pad_[4];          // keeps the next buffer 16-byte aligned
};

template <int DK, int DV, int NB, int RH>
struct __align__(16) SpecSmem {
    SpecTokens<DK, DV> tok[NB];
    // each row half's sums of X S; with two drafts (DK = DV) these live in
    // the drafts' G arrays instead, dead by the time the state is multiplied
    float P[NB == 1 ? RH : 1][SP_MAX][DV];
    float dec[DK];             // e^(G_{a-1}) (commit)
    float A[NB][SP_MAX][SP_MAX];    // per draft (commit: 0, verify: NB - 1)
    float B[SP_MAX][SP_MAX];        // verified draft only
    float TB[NB][SP_MAX][SP_MAX];
    float M[SP_MAX][SP_MAX];
};

struct SpecParams {
    const void *q, *k, *v;
    const float *g, *beta;
    const void *pk, *pv;       // step: the previous draft, committed first
    const float *pg, *pbeta;
    float* state;
    const int32_t* slots;
    const int32_t* counts;     // commit, step: accepted tokens per sequence
    void* out;
    int H, K;
    float scale;
};

// 4 consecutive input values as loaded; widened to fp32 only when written to
// LDS, so that nothing waits for the load before the state loads are issued
template <typename T> struct Raw4;
template <> struct Raw4<bf16_t> {
    uint2 w;
    __device__ __forceinline__ void load(const bf16_t* p) {
        w = *reinterpret_cast<const uint2*>(p);
    }
    __device__ __forceinline__ void put(float* d) const {
        *reinterpret_cast<float4*>(d) =
            make_float4(bf16_bits_to_f32(w.x & 0xffffu), bf16_bits_to_f32(w.x >> 16),
                        bf16_bits_to_f32(w.y & 0xffffu), bf16_bits_to_f32(w.y >> 16));
    }
};
template <> struct Raw4<float> {
    float4 a;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
    }
    __device__ __forceinline__ void put(float* d) const { *reinterpret_cast<float4*>(d) = a; }
};

// a thread's share of one draft: 4 channels of k, q, g of one token, 4
// columns of v of one token, one beta
template <typename TIn>
struct Fetched {
    Raw4<TIn> k, q, v;
    Raw4<float> g;
    float beta;
};

// the RPL consecutive values a lane owns in an LDS row (128-bit reads when
// RPL is a multiple of 4)
template <int RPL>
__device__ __forceinline__ void lds_rows(const float* p, float (&x)[RPL]) {
    if constexpr (RPL % 4 == 0) {
#pragma unroll
        for (int m = 0; m < RPL; m += 4) {
            const float4 t = reinterpret_cast<const float4*>(p)[m / 4];
            x[m] = t.x; x[m + 1] = t.y; x[m + 2] = t.z; x[m + 3] = t.w;
        }
    } else {
#pragma unroll
        for (int m = 0; m < RPL; ++m) x[m] = p[m];
    }
}

// MODE 1 verify, 2 commit, 3 step (commit the previous draft, then verify).
// Commit and step are compiled for 64 VGPRs (a few values spill), so four
// 8-wave workgroups fit a compute unit: 256 x 32 at d = 128, commit
// 200 -> 190 us, step 218 -> 211 us; verify keeps its 60 VGPRs.
template <int DK, int DV, typename TIn, typename TOut, int MODE>
__global__ __launch_bounds__((64 * SpecLayout<DK, DV>::WAVES))
__attribute__((amdgpu_waves_per_eu(MODE == 1 ? 6 : 8)))
void spec_kernel(SpecParams p) {
    using L = SpecLayout<DK, DV>;
    constexpr int WAVES = L::WAVES;
    constexpr int NT = 64 * WAVES;
    constexpr int RG = L::RG;
    constexpr int RH = L::RH;
    constexpr int RPL = L::RPL;
    constexpr int NB = MODE == 3 ? 2 : 1;
    static_assert(L::CW % 4 == 0 && DV % L::CW == 0 && 64 % L::CG == 0 && RPL >= 1 &&
                  DK == RPL * RG * RH, "layout");
    static_assert(SP_MAX * (DK / 4) <= NT && SP_MAX * (DV / 4) <= NT && DK % 4 == 0,
                  "one load of 4 values per thread and draft");
    static_assert(NB * DK <= NT && DK + DV <= NT, "one thread per channel and per column");
    __shared__ SpecSmem<DK, DV, NB, RH> sm;

    const int H = p.H, K = p.K;
    const int n = blockIdx.x / H;
    const int h = blockIdx.x - n * H;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int rg = lane % RG;
    const int cg = lane / RG;
    const int rh = wave / L::CB;
    const int col = (wave - rh * L::CB) * L::CW + cg * 4;
    const int row0 = rh * (DK / RH) + rg * RPL;

    const int acc = p.counts ? min(max(p.counts[n], 0), K) : K;
    if (MODE == 2 && acc == 0) return;  // nothing to commit
    const int64_t tok0 = (int64_t)n * K;

    // ---- loads: the draft(s) first, then the state ----
    // thread tid takes token tid / (d/4), values 4 (tid % (d/4)) .. + 3;
    // threads past the draft load the first token again and store nothing;
    // with_q (a std::integral_constant) says whether the draft is verified
    auto fetch = [&](auto with_q, Fetched<TIn>& f, const TIn* kg, const TIn* qg, const TIn* vg,
                     const float* gg, const float* bg, int nt) {
        const int ik = tid < nt * (DK / 4) ? tid : 0;
        const int tk = ik / (DK / 4);
        const int64_t ek = ((tok0 + tk) * H + h) * DK + 4 * (ik - tk * (DK / 4));
        f.k.load(kg + ek);
        f.g.load(gg + ek);
        if constexpr (decltype(with_q)::value) f.q.load(qg + ek);
        const int iv = tid < nt * (DV / 4) ? tid : 0;
        const int tv = iv / (DV / 4);
        f.v.load(vg + ((tok0 + tv) * H + h) * DV + 4 * (iv - tv * (DV / 4)));
        f.beta = bg[(tok0 + min(tid, nt - 1)) * H + h];
    };
    Fetched<TIn> fa, fb;
    int na;  // tokens of the first buffer
    if constexpr (MODE == 1) {
        na = K;
        fetch(std::true_type{}, fa, static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.q),
              static_cast<const TIn*>(p.v), p.g, p.beta, K);
    } else if constexpr (MODE == 2) {
        na = acc;
        fetch(std::false_type{}, fa, static_cast<const TIn*>(p.k), nullptr,
              static_cast<const TIn*>(p.v), p.g, p.beta, acc);
    } else {
        na = max(acc, 1);  // acc = 0 commits nothing; the buffer is then unused
        fetch(std::false_type{}, fa, static_cast<const TIn*>(p.pk), nullptr,
              static_cast<const TIn*>(p.pv), p.pg, p.pbeta, na);
        fetch(std::true_type{}, fb, static_cast<const TIn*>(p.k), static_cast<const TIn*>(p.q),
              static_cast<const TIn*>(p.v), p.g, p.beta, K);
    }

    const int64_t slot = p.slots ? (int64_t)p.slots[n] : (int64_t)n;
    float* __restrict__ S = p.state + ((slot * H + h) * DK + row0) * (int64_t)DV + col;
    float4 s[RPL];
#pragma unroll
    for (int m = 0; m < RPL; ++m) s[m] = load_stream4(S + m * DV);

    // ---- the drafts into LDS, cumulative gates ----
    auto put = [&](auto with_q, SpecTokens<DK, DV>& b, const Fetched<TIn>& f, int nt) {
        if (tid < nt * (DK / 4)) {
            const int t = tid / (DK / 4), c = 4 * (tid - t * (DK / 4));
            f.k.put(&b.k[t][c]);
            f.g.put(&b.G[t][c]);
            if constexpr (decltype(with_q)::value) f.q.put(&b.q[t][c]);
        }
        if (tid < nt * (DV / 4)) {
            const int t = tid / (DV / 4), j = 4 * (tid - t * (DV / 4));
            f.v.put(&b.v[t][j]);
        }
        if (tid < nt) b.beta[tid] = f.beta;
    };
    put(std::integral_constant<bool, MODE == 1>{}, sm.tok[0], fa, na);
    if constexpr (MODE == 3) put(std::true_type{}, sm.tok[NB - 1], fb, K);
    __syncthreads();
    // one thread per channel and buffer
    if (tid < NB * DK) {
        const int bi = tid / DK, c = tid - bi * DK;
        const int nt = bi == 0 ? na : K;
        float acc_g = 0.f;
        for (int t = 0; t < nt; ++t) {
            acc_g += sm.tok[bi].G[t][c];
            sm.tok[bi].G[t][c] = acc_g;
        }
    }

    // The token side of both drafts at once: the committed draft (nc tokens,
    // buffer 0; nc = 0 when there is none) and the verified one (nv tokens,
    // buffer NB - 1; nv = 0 when there is none).  Every quantity is computed
    // by the same arithmetic whichever drafts the launch holds, so the fused
    // step is bit-identical to commit followed by verify.
    // The n x n Grams (B for the verified draft only), then T, TB, and M.
    auto grams = [&](int nc, int nv) {
        __syncthreads();  // the buffers are complete; earlier reads of the work arrays done
        // one pair (t, s), s <= t, per 16-lane group (4 per wave), DK / 16
        // channels per lane, summed over the group by DPP moves; the pairs of
        // the committed draft come first.  A pair's channels start at a
        // rotation fixed by the pair (fewer LDS bank conflicts between the
        // groups of a wave, and the same order in every launch).
        const int pc = nc * (nc + 1) / 2, pairs = pc + nv * (nv + 1) / 2;
        const int grp = lane >> 4, gl = lane & 15;
        for (int pr0 = 4 * wave; pr0 < pairs; pr0 += 4 * WAVES) {
            const int pr = pr0 + grp;
            const bool ver = pr >= pc;
            const SpecTokens<DK, DV>& b = sm.tok[ver ? NB - 1 : 0];
            // pair index -> (t, s), row by row over the lower triangle
            const int pl = pr < pairs ? (ver ? pr - pc : pr) : 0;
            int t = 0;
            while ((t + 1) * (t + 2) / 2 <= pl) ++t;
            const int s2 = pl - t * (t + 1) / 2;
            float ka = 0.f, qb = 0.f;
#pragma unroll 2
            for (int i = 0; i < DK / 16; ++i) {
                const int c = (gl + 16 * (i + pl)) % DK;
                const float ks = b.k[s2][c] * exp_gate(b.G[t][c] - b.G[s2][c]);
                ka = fmaf(b.k[t][c], ks, ka);
                if (ver) qb = fmaf(b.q[t][c], ks, qb);
            }
            ka = group_sum<16>(ka);
            qb = group_sum<16>(qb);
            if (gl == 0 && pr < pairs) {
                sm.A[ver ? NB - 1 : 0][t][s2] = s2 < t ? b.beta[t] * ka : 0.f;
                if (ver) sm.B[t][s2] = qb;
            }
        }
        __syncthreads();
        // T = (I + A)^-1 by forward substitution, one column per thread
        // (threads 0 .. nc - 1 the committed draft, SP_MAX .. SP_MAX + nv - 1
        // the verified one): T_t,sc = [t == sc] - sum_{m<t} A_tm T_m,sc (zero
        // above the diagonal)
        if (tid < nc || (tid >= SP_MAX && tid < SP_MAX + nv)) {
            const bool ver = tid >= SP_MAX;
            const int bi = ver ? NB - 1 : 0, nt = ver ? nv : nc, sc = ver ? tid - SP_MAX : tid;
            float col_t[SP_MAX];
#pragma unroll
            for (int t = 0; t < SP_MAX; ++t) {
                float x = t == sc ? 1.f : 0.f;
                if (t < nt) {
#pragma unroll
                    for (int m = 0; m < t; ++m) x = fmaf(-sm.A[bi][t][m], col_t[m], x);
                }
                col_t[t] = x;
            }
            const float bs = sm.tok[bi].beta[sc];
#pragma unroll
            for (int t = 0; t < SP_MAX; ++t)
                if (t < nt) sm.TB[bi][t][sc] = col_t[t] * bs;
        }
        __syncthreads();
        if (nv > 0) {
            if (tid < nv * nv) {
                const int t = tid / nv, s2 = tid - t * nv;
                float x = 0.f;
                for (int m = s2; m <= t; ++m) x = fmaf(sm.B[t][m], sm.TB[NB - 1][m][s2], x);
                sm.M[t][s2] = s2 <= t ? x : 0.f;
            }
            __syncthreads();
        }
    };

    // the partial sums of row half r
    auto pbuf = [&](int r) -> float (*)[DV] {
        if constexpr (NB == 1) {
            return sm.P[r];
        } else {
            static_assert(DK == DV && RH <= NB, "partial sums in the G arrays");
            return sm.tok[r].G;
        }
    };
    // P[rh][t] = this row half's sums of X_t S over its rows, for t < nt
    auto xs = [&](const float (*X)[DK], int nt) {
        for (int t = 0; t < nt; ++t) {
            float xr[RPL];
            lds_rows<RPL>(&X[t][row0], xr);
            float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
#pragma unroll
            for (int m = 0; m < RPL; ++m) {
                y0 = fmaf(xr[m], s[m].x, y0); y1 = fmaf(xr[m], s[m].y, y1);
                y2 = fmaf(xr[m], s[m].z, y2); y3 = fmaf(xr[m], s[m].w, y3);
            }
            y0 = group_sum<RG>(y0); y1 = group_sum<RG>(y1);
            y2 = group_sum<RG>(y2); y3 = group_sum<RG>(y3);
            if (rg == 0)
                *reinterpret_cast<float4*>(&pbuf(rh)[t][col]) = make_float4(y0, y1, y2, y3);
        }
        __syncthreads();
    };
    // sum of the row halves' partials at (t, columns c .. c+3)
    auto psum = [&](int t, int c) {
        float4 r = *reinterpret_cast<const float4*>(&pbuf(0)[t][c]);
        if constexpr (RH == 2) {
            const float4 r1 = *reinterpret_cast<const float4*>(&pbuf(1)[t][c]);
            r.x += r1.x; r.y += r1.y; r.z += r1.z; r.w += r1.w;
        }
        return r;
    };

    // verify: O = scale (Q' S + O~) for the nt tokens of buffer b; the
    // token-side part first (no state needed), then the outputs
    // threads u = tid - base .. of the verified draft's token side
    auto prep_verify = [&](SpecTokens<DK, DV>& b, int nt, int base) {
        const int u = tid - base;
        if (u >= 0 && u < DK) {  // Q' = Q e^G - M (K e^G) in place of q, one channel per thread
            const int c = u;
            float ek[SP_MAX];
#pragma unroll
            for (int s2 = 0; s2 < SP_MAX; ++s2)
                ek[s2] = s2 < nt ? b.k[s2][c] * exp_gate(b.G[s2][c]) : 0.f;
#pragma unroll
            for (int t = 0; t < SP_MAX; ++t) {
                if (t < nt) {
                    float x = b.q[t][c] * exp_gate(b.G[t][c]);
#pragma unroll
                    for (int s2 = 0; s2 <= t; ++s2) x = fmaf(-sm.M[t][s2], ek[s2], x);
                    b.q[t][c] = x;
                }
            }
        } else if (u >= DK && u < DK + DV) {  // O~ = M V in place of v, one column per thread
            const int j = u - DK;
            float vv[SP_MAX];
#pragma unroll
            for (int s2 = 0; s2 < SP_MAX; ++s2) vv[s2] = s2 < nt ? b.v[s2][j] : 0.f;
#pragma unroll
            for (int t = 0; t < SP_MAX; ++t) {
                if (t < nt) {
                    float x = 0.f;
#pragma unroll
                    for (int s2 = 0; s2 <= t; ++s2) x = fmaf(sm.M[t][s2], vv[s2], x);
                    b.v[t][j] = x;
                }
            }
        }
    };
    auto emit_verify = [&](SpecTokens<DK, DV>& b, int nt) {
        __syncthreads();
        xs(b.q, nt);
        // outputs, 4 consecutive columns of one token per thread
        TOut* __restrict__ og = static_cast<TOut*>(p.out);
        const float sc = p.scale;
        for (int i = tid; i < nt * (DV / 4); i += NT) {
            const int t = i / (DV / 4), c = 4 * (i - t * (DV / 4));
            const float4 o = psum(t, c);
            const float4 y = *reinterpret_cast<const float4*>(&b.v[t][c]);
            io<TOut>::store4(og + ((tok0 + t) * H + h) * DV + c, sc * (o.x + y.x),
                             sc * (o.y + y.y), sc * (o.z + y.z), sc * (o.w + y.w));
        }
    };

    // commit: the state after the first nt tokens of buffer b, stored; the
    // token-side part first, then the state update
    auto prep_commit = [&](SpecTokens<DK, DV>& b, int nt) {
        if (tid < DK) {  // W = TB (K e^G) in q, Kd in k, dec; one channel per thread
            const int c = tid;
            float ek[SP_MAX];
#pragma unroll
            for (int s2 = 0; s2 < SP_MAX; ++s2)
                ek[s2] = s2 < nt ? b.k[s2][c] * exp_gate(b.G[s2][c]) : 0.f;
            const float gl = b.G[nt - 1][c];
#pragma unroll
            for (int t = 0; t < SP_MAX; ++t) {
                if (t < nt) {
                    float x = 0.f;
#pragma unroll
                    for (int s2 = 0; s2 <= t; ++s2) x = fmaf(sm.TB[0][t][s2], ek[s2], x);
                    b.q[t][c] = x;
                    b.k[t][c] *= exp_gate(gl - b.G[t][c]);
                }
            }
            sm.dec[c] = exp_gate(gl);
        } else if (tid < DK + DV) {  // U~ = TB V in place of v, one column per thread (threads DK ..)
            const int j = tid - DK;
            float vv[SP_MAX];
#pragma unroll
            for (int s2 = 0; s2 < SP_MAX; ++s2) vv[s2] = s2 < nt ? b.v[s2][j] : 0.f;
#pragma unroll
            for (int t = 0; t < SP_MAX; ++t) {
                if (t < nt) {
                    float x = 0.f;
#pragma unroll
                    for (int s2 = 0; s2 <= t; ++s2) x = fmaf(sm.TB[0][t][s2], vv[s2], x);
                    b.v[t][j] = x;
                }
            }
        }
    };
    auto apply_commit = [&](SpecTokens<DK, DV>& b, int nt) {
        __syncthreads();
        xs(b.q, nt);  // W S
        // S' = Diag(e^(G_{nt-1})) S + sum_t Kd_t u_t^T with u_t = U~_t - (W S)_t
        {
            float dr[RPL];
            lds_rows<RPL>(&sm.dec[row0], dr);
#pragma unroll
            for (int m = 0; m < RPL; ++m)
                s[m] = make_float4(s[m].x * dr[m], s[m].y * dr[m], s[m].z * dr[m],
                                   s[m].w * dr[m]);
        }
        for (int t = 0; t < nt; ++t) {
            float kr[RPL];
            lds_rows<RPL>(&b.k[t][row0], kr);
            const float4 ws = psum(t, col);
            const float4 ut = *reinterpret_cast<const float4*>(&b.v[t][col]);
            const float4 u = make_float4(ut.x - ws.x, ut.y - ws.y, ut.z - ws.z, ut.w - ws.w);
#pragma unroll
            for (int m = 0; m < RPL; ++m) {
                s[m].x = fmaf(kr[m], u.x, s[m].x); s[m].y = fmaf(kr[m], u.y, s[m].y);
                s[m].z = fmaf(kr[m], u.z, s[m].z); s[m].w = fmaf(kr[m], u.w, s[m].w);
            }
        }
#pragma unroll
        for (int m = 0; m < RPL; ++m) store_stream4(S + m * DV, s[m]);
    };

    if constexpr (MODE == 1) {
        grams(0, K);
        prep_verify(sm.tok[0], K, 0);
        emit_verify(sm.tok[0], K);
    } else if constexpr (MODE == 2) {
        grams(acc, 0);
        prep_commit(sm.tok[0], acc);
        apply_commit(sm.tok[0], acc);
    } else {
        // both drafts' token side, side by side, before the state is needed
        static_assert(2 * (DK + DV) <= NT, "one thread per channel and column of each draft");
        grams(acc, K);
        if (acc > 0) prep_commit(sm.tok[0], acc);
        prep_verify(sm.tok[NB - 1], K, DK + DV);
        if (acc > 0) apply_commit(sm.tok[0], acc);
        emit_verify(sm.tok[NB - 1], K);
    }
}

template <int DK, typename TIn, typename TOut, int MODE>
hipError_t launch_m(const SpecParams& p, int num_seqs, hipStream_t stream) {
    hipLaunchKernelGGL((spec_kernel<DK, DK, TIn, TOut, MODE>),
                       dim3((unsigned)((int64_t)num_seqs * p.H)),
                       dim3(64 * SpecLayout<DK, DK>::WAVES), 0, stream, p);
    return hipGetLastError();
}

template <int DK, typename TIn, typename TOut>
hipError_t launch_mode(const SpecParams& p, int num_seqs, int mode, hipStream_t stream) {
    switch (mode) {
        case 1: return launch_m<DK, TIn, TOut, 1>(p, num_seqs, stream);
        case 2: return launch_m<DK, TIn, TOut, 2>(p, num_seqs, stream);
        case 3: return launch_m<DK, TIn, TOut, 3>(p, num_seqs, stream);
    }
    return hipErrorInvalidValue;
}

template <int DK>
hipError_t launch_dt(const SpecParams& p, const DecodeMultiArgs& a) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_mode<DK, bf16_t, bf16_t>(p, a.num_seqs, a.mode, a.stream)
                          : launch_mode<DK, bf16_t, float>(p, a.num_seqs, a.mode, a.stream);
    return a.out_bf16 ? launch_mode<DK, float, bf16_t>(p, a.num_seqs, a.mode, a.stream)
                      : launch_mode<DK, float, float>(p, a.num_seqs, a.mode, a.stream);
}

}  // namespace

bool spec_chunked(const DecodeMultiArgs& a) {
    return a.mode >= 1 && a.mode <= 3 && a.num_tokens <= SP_MAX;
}

hipError_t launch_spec(const DecodeMultiArgs& a) {
    SpecParams p{};
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.g = a.g;
    p.beta = a.beta;
    p.pk = a.pk;
    p.pv = a.pv;
    p.pg = a.pg;
    p.pbeta = a.pbeta;
    p.state = a.state;
    p.slots = a.slots;
    p.counts = a.counts;
    p.out = a.out;
    p.H = a.H;
    p.K = a.num_tokens;
    p.scale = a.scale;
    switch (a.dk) {
        case 16: return launch_dt<16>(p, a);
        case 32: return launch_dt<32>(p, a);
        case 64: return launch_dt<64>(p, a);
        case 128: return launch_dt<128>(p, a);
    }
    return hipErrorInvalidValue;
}

}  // namespace kda
