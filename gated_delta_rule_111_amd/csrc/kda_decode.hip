// kda_decode.hip -- one KDA decode step (one token per sequence) against
// fp32 states resident in HBM, updated in place.  gfx950.
//
// Per (sequence n, head h), with the state S (dk x dv, row i = key channel):
//   S' = Diag(exp(g)) S                      per-channel forget gate
//   a  = S'^T k,  b = S'^T q                 two reductions over dk
//   u  = beta (v - a)                        delta-rule correction
//   o  = scale (b + (k.q) u)                 = scale S_new^T q
//   S  = S' + k u^T                          written back in place
// This is the recurrence of "Kimi K3 technical FAQ", question "What is KDA,
// and why does a serving engineer care?" (delta rule, per-channel forget
// gate, dk x dv state), read as S_t = (I - b k k^T) Diag(a) S_{t-1} + b k v^T
// and o_t = scale S_t^T q_t, applied to a single token.
//
// The step is bound by HBM: it moves 2*dk*dv*4 bytes of state per
// (sequence, head) and does 7*dk*dv flops on it.  Design:
// - one workgroup of WAVES wavefronts per (sequence, head); value columns
//   evolve independently, so wave w owns a contiguous block of dv/WAVES
//   columns and never talks to the other waves (no LDS, no barrier);
// - in a wave, lane l owns a 4-column group (16-byte accesses) and a block
//   of dk/RG consecutive rows; the dk-reductions are a per-lane partial sum
//   followed by a butterfly over the RG row groups;
// - the state is loaded once into VGPRs, updated there and stored once, with
//   non-temporal 16-byte accesses (each state is touched once per step, and
//   keeping it out of the caches leaves them to the small per-token inputs).
#include "kda_common.h"
#include "kda_internal.h"

namespace kda {

template <int DK, int DV, int WAVES, typename TIn, typename TOut>
__global__ __launch_bounds__(64 * WAVES) void decode_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    const int32_t* __restrict__ slots, TOut* __restrict__ out, int H, float scale) {
    constexpr int CW = DV / WAVES;   // columns per wave
    constexpr int CG = CW / 4;       // 4-column groups per wave
    constexpr int RG = 64 / CG;      // row groups per wave
    constexpr int RPL = DK / RG;     // rows per lane
    static_assert(CW % 4 == 0 && 64 % CG == 0 && DK % RG == 0 && RPL >= 1, "layout");

    const int unit = blockIdx.x;  // n * H + h
    const int n = unit / H;
    const int h = unit - n * H;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int cg = lane % CG;
    const int rg = lane / CG;
    const int col = wave * CW + cg * 4;
    const int row0 = rg * RPL;

    const int64_t slot = slots ? (int64_t)slots[n] : (int64_t)n;
    float* __restrict__ S = state + ((slot * H + h) * DK + row0) * (int64_t)DV + col;
    const int64_t tok = (int64_t)n * H + h;

    // state tile: RPL rows x 4 columns, issued first so HBM latency overlaps the rest
    float4 s[RPL];
#pragma unroll
    for (int m = 0; m < RPL; ++m) s[m] = load_stream4(S + m * DV);

    float kr[RPL], qr[RPL], gr[RPL], vv[4];
    io<TIn>::template load<RPL>(k + tok * DK + row0, kr);
    io<TIn>::template load<RPL>(q + tok * DK + row0, qr);
    io<float>::template load<RPL>(g + tok * DK + row0, gr);
    io<TIn>::template load<4>(v + tok * DV + col, vv);
    const float bt = beta[tok];

    // S' = Diag(alpha) S ; partial reductions over this lane's rows
    float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
    float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        const float al = exp_gate(gr[m]);
        s[m].x *= al; s[m].y *= al; s[m].z *= al; s[m].w *= al;
        a0 = fmaf(kr[m], s[m].x, a0); a1 = fmaf(kr[m], s[m].y, a1);
        a2 = fmaf(kr[m], s[m].z, a2); a3 = fmaf(kr[m], s[m].w, a3);
        b0 = fmaf(qr[m], s[m].x, b0); b1 = fmaf(qr[m], s[m].y, b1);
        b2 = fmaf(qr[m], s[m].z, b2); b3 = fmaf(qr[m], s[m].w, b3);
        kq = fmaf(kr[m], qr[m], kq);
    }
    // butterfly over the row groups (lanes with the same column group)
#pragma unroll
    for (int off = CG; off < 64; off <<= 1) {
        a0 += __shfl_xor(a0, off, 64); a1 += __shfl_xor(a1, off, 64);
        a2 += __shfl_xor(a2, off, 64); a3 += __shfl_xor(a3, off, 64);
        b0 += __shfl_xor(b0, off, 64); b1 += __shfl_xor(b1, off, 64);
        b2 += __shfl_xor(b2, off, 64); b3 += __shfl_xor(b3, off, 64);
        kq += __shfl_xor(kq, off, 64);
    }
    const float u0 = bt * (vv[0] - a0), u1 = bt * (vv[1] - a1);
    const float u2 = bt * (vv[2] - a2), u3 = bt * (vv[3] - a3);

    // S = S' + k u^T, stored in place
#pragma unroll
    for (int m = 0; m < RPL; ++m) {
        float4 t = s[m];
        t.x = fmaf(kr[m], u0, t.x); t.y = fmaf(kr[m], u1, t.y);
        t.z = fmaf(kr[m], u2, t.z); t.w = fmaf(kr[m], u3, t.w);
        store_stream4(S + m * DV, t);
    }
    if (rg == 0) {
        io<TOut>::store4(out + tok * DV + col, scale * fmaf(kq, u0, b0),
                         scale * fmaf(kq, u1, b1), scale * fmaf(kq, u2, b2),
                         scale * fmaf(kq, u3, b3));
    }
}

template <int DK, int WAVES, typename TIn, typename TOut>
static hipError_t launch_decode_t(const DecodeArgs& a) {
    const void* q = a.q;
    hipLaunchKernelGGL((decode_kernel<DK, DK, WAVES, TIn, TOut>),
                       dim3((unsigned)((int64_t)a.num_seqs * a.H)), dim3(64 * WAVES), 0,
                       a.stream, static_cast<const TIn*>(q), static_cast<const TIn*>(a.k),
                       static_cast<const TIn*>(a.v), a.g, a.beta, a.state, a.slots,
                       static_cast<TOut*>(a.out), a.H, a.scale);
    return hipGetLastError();
}

template <int DK, int WAVES>
static hipError_t launch_decode_d(const DecodeArgs& a) {
    if (a.in_bf16)
        return a.out_bf16 ? launch_decode_t<DK, WAVES, bf16_t, bf16_t>(a)
                          : launch_decode_t<DK, WAVES, bf16_t, float>(a);
    return a.out_bf16 ? launch_decode_t<DK, WAVES, float, bf16_t>(a)
                      : launch_decode_t<DK, WAVES, float, float>(a);
}

hipError_t launch_decode(const DecodeArgs& a) {
    switch (a.dk) {
        case 16: return launch_decode_d<16, 1>(a);
        case 32: return launch_decode_d<32, 1>(a);
        case 64: return launch_decode_d<64, 2>(a);
        case 128: return launch_decode_d<128, 4>(a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace kda
