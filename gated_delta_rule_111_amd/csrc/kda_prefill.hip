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
// With W = TB (K . e^G), M = B TB, U~ = TB V, O~ = M V and
// Q' = Q . e^G - M (K . e^G) the step becomes
//   U = U~ - W S,   O = scale (Q' S + O~),   S' = Diag(e^{G_C}) S + Kd U
// (Kd = (K . e^{G_C - G})^T), so everything but three products with S is
// independent of the state.
//
// Three launches on the caller's stream:
//   plan  -- one workgroup: per-sequence offsets of chunks and snapshots;
//   prep  -- one workgroup per (chunk, head), all chunks in parallel: the
//            Gram matrices A and B, T, W, M, Q', U~ and O~ (MFMA wherever
//            the step is a product), written to the workspace as the
//            scan's per-lane operands;
//   scan  -- one workgroup per (sequence, head, 16 value columns), walking
//            the sequence chunk by chunk with the fp32 state in registers.
//            Wave w owns 32 state rows and one 16-token tile of the chunk;
//            state rows and U tiles are exchanged through LDS, two
//            barriers per chunk.
//
// Precision: MFMAs with fp32 accumulation; state, snapshots, outputs and
// every accumulation are fp32.  In prep, operands that are not exact bf16
// values are split into hi + lo bf16 and multiplied in three passes
// (hi*hi + hi*lo + lo*hi, ~16 bits), except single fp16 operands in the
// off-diagonal Gram blocks (both decay factors there are at most 1, and A
// and B share the key factor).  The diagonal blocks of A and B round alike
// and K e^G enters W and Q' as a hi + lo pair: with q = k and beta = 1 the
// output is formed by cancellation (B = I + A, so M = B TB = I), and a
// single bf16 rounding of either leaves ~4e-3 at dk = 16.  The scan's W, Q'
// and Kd are single fp16 values with one power-of-two exponent per tile,
// its S and U fp16 hi + lo pairs (~22 bits) with their own exponents, so
// each scan product is two v_mfma_f32_16x16x32_f16 passes.
//
// Determinism: every reduction has a fixed order that depends neither on the
// number of value tiles nor on where a sequence sits in the packed batch,
// and chunks restart at every sequence start, so resuming from a snapshot
// reproduces the uninterrupted run bit for bit.
#include <algorithm>

#include "kda_common.h"
#include "kda_internal.h"

#include <type_traits>

namespace kda {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int C = 64;                // chunk rows
constexpr int NT = 256;              // threads per workgroup (4 waves)
constexpr int DKP = 128;             // state rows, zero-padded above dk
constexpr int SL = 32;               // state rows per wave
constexpr float SPAN_LIMIT = 115.0f; // |log2 exponent| bound for the diagonal Gram factors (~e^80)
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
// 2^x; the prep kernel keeps its log-decays in log2 units
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float LOG2E = 1.4426950408889634f;

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (x - hi is exact in fp32)
__device__ __forceinline__ void split(float x, uint16_t& hi, uint16_t& lo) {
    hi = bfb(x);
    lo = bfb(x - bff(hi));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// bf16 of two values (round to nearest even, one instruction), a in the low half
__device__ __forceinline__ uint32_t bf2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
// split of two values at once, packed like bf2
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = bf2(a, b);
    lo = bf2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
// eight values as one operand, rounded once
__device__ __forceinline__ uint4 bf8(const float (&x)[8]) {
    return make_uint4(bf2(x[0], x[1]), bf2(x[2], x[3]), bf2(x[4], x[5]), bf2(x[6], x[7]));
}
// eight values as hi and lo operands
__device__ __forceinline__ void split8(const float (&x)[8], uint4& hi, uint4& lo) {
    split2(x[0], x[1], hi.x, lo.x);
    split2(x[2], x[3], hi.y, lo.y);
    split2(x[4], x[5], hi.z, lo.z);
    split2(x[6], x[7], hi.w, lo.w);
}

__device__ __forceinline__ bf16x8_t as_op(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// ---- fp16 operands of the scan.  Each tile is stored times a power of two
// that puts its largest magnitude in [2^14, 2^15); products are scaled back
// in fp32, so the fp16 range never limits the data. ----
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
constexpr int F16_TOP = 15;  // a tile with magnitudes < 2^e is stored times 2^(F16_TOP - e)

__device__ __forceinline__ f32x4 mfma_h(const uint4& a, const uint4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
// fp16 of two values (round to nearest even), a in the low half
__device__ __forceinline__ uint32_t h2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}
// eight values as one fp16 operand, rounded once
__device__ __forceinline__ uint4 h8(const float (&x)[8]) {
    return make_uint4(h2(x[0], x[1]), h2(x[2], x[3]), h2(x[4], x[5]), h2(x[6], x[7]));
}
// x = hi + lo in fp16 (x - hi is exact in fp32), packed like h2
__device__ __forceinline__ void hsplit2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = h2(a, b);
    const f16x2_t v = __builtin_bit_cast(f16x2_t, hi);
    lo = h2(a - (float)v[0], b - (float)v[1]);
}
__device__ __forceinline__ float scl(float x, int s) { return __builtin_amdgcn_ldexpf(x, s); }
__device__ __forceinline__ f32x4 scl4(const f32x4& x, int s) {
    return f32x4{scl(x[0], s), scl(x[1], s), scl(x[2], s), scl(x[3], s)};
}
// Two accumulator tiles (row blocks 0 and 1 of a 32-row K-step) as one fp16
// MFMA operand times 2^s: elements 0..3 come from tile 0, 4..7 from tile 1.
__device__ __forceinline__ uint4 pack_h(const f32x4& x0, const f32x4& x1, int s) {
    return make_uint4(h2(scl(x0[0], s), scl(x0[1], s)), h2(scl(x0[2], s), scl(x0[3], s)),
                      h2(scl(x1[0], s), scl(x1[1], s)), h2(scl(x1[2], s), scl(x1[3], s)));
}
// max(m, |x|) (fabsf folds into v_max3_f32 as a source modifier); the bit
// patterns of non-negative floats order like their values, so the maxima
// are reduced across lanes as integers
__device__ __forceinline__ float amax(float m, float x) { return fmaxf(m, fabsf(x)); }
__device__ __forceinline__ uint32_t bits(float x) { return __float_as_uint(x); }
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
// largest value over the 64 lanes (DPP inside each 16-lane row, then the
// four rows), uniform
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dppu<0xB1>(v));   // quad_perm [1,0,3,2]
    v = max(v, dppu<0x4E>(v));   // quad_perm [2,3,0,1]
    v = max(v, dppu<0x141>(v));  // row_half_mirror
    v = max(v, dppu<0x140>(v));  // row_mirror
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32),
                           (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
}
// e with m < 2^e for the magnitude whose bit pattern is b (frexp's exponent;
// -126 for zero and subnormals), and the same as a byte e + 126
__device__ __forceinline__ int bound_exp(uint32_t b) { return (int)(b >> 23) - 126; }
__device__ __forceinline__ uint8_t exp_byte(uint32_t b) { return (uint8_t)(b >> 23); }
// exponent byte i of a packed word, and the raw byte (exponent + 126)
__device__ __forceinline__ int byte_exp(uint32_t packed, int i) { return (int)((packed >> (8 * i)) & 0xffu) - 126; }
__device__ __forceinline__ int byte_raw(uint32_t packed, int i) { return (int)((packed >> (8 * i)) & 0xffu); }
// 2^e as a float: exact down to 2^-149 (subnormal), 0 below; e is capped at
// 127 so that a zero accumulator never meets an infinite factor (a product
// that needs a larger factor overflows fp32 anyway)
__device__ __forceinline__ float pow2f(int e) { return __builtin_amdgcn_ldexpf(1.0f, min(e, 127)); }

// -x for a bf16 operand (sign flips, exact)
__device__ __forceinline__ bf16x8_t neg(const bf16x8_t& x) {
    const uint4 u = __builtin_bit_cast(uint4, x);
    return __builtin_bit_cast(bf16x8_t, make_uint4(u.x ^ 0x80008000u, u.y ^ 0x80008000u,
                                                   u.z ^ 0x80008000u, u.w ^ 0x80008000u));
}

// Storage slot of 16-byte group g (tokens 8g .. 8g+7) in row j of V^T.  The
// permutation differs between rows 8 apart (the transposing writes of one
// instruction) and between neighbouring rows (the operand reads).
__device__ __forceinline__ int vt_group(int j, int g) { return g ^ ((j ^ (j >> 3)) & 7); }
// Storage slot of token group g in row c of (K e^G)^T: rows 8 channels apart
// (the transposing writes of one instruction) land in different slots.
__device__ __forceinline__ int kg_group(int c, int g) { return g ^ ((c >> 3) & 7); }
// Token order of the prep's token-contracted operands (TB, V^T, (K e^G)^T and
// M): within each 32-token K-step, slot 8g + e holds token 4g + e (e < 4) or
// 16 + 4g + e - 4 (e >= 4), the order in which an MFMA accumulator of M^T
// (two 16-token tiles) leaves a lane's values, so M needs no LDS transpose.
__device__ __forceinline__ int kslot(int t) {
    return (t & ~31) + (((t & 15) >> 2) << 3) + (t & 3) + ((t & 16) ? 4 : 0);
}
__device__ __forceinline__ int kslot_tok(int q) {
    return (q & ~31) + ((q & 4) ? 16 : 0) + (((q & 31) >> 3) << 2) + (q & 3);
}

// eight consecutive fp32 of an LDS row (16-byte aligned) as two 128-bit reads
__device__ __forceinline__ void lds8(const float* p, float (&x)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
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
    // 8 values at byte offset voff of a buffer resource (zero outside it)
    __device__ __forceinline__ static V8 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
    }
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
    __device__ __forceinline__ static V8 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
        return V8{__builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0)),
                  __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 16, 0))};
    }
};

// Rows lo .. n-1 of one head of a [T, H, d] tensor (elements of es bytes) as
// a buffer resource based at row lo: byte offset (t - lo) * H * d * es + c * es
// addresses row t, and every row outside lo .. n-1 falls outside the
// resource (a row below lo wraps past 2^32 - 1), where loads return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t item_rows(const void* base, int64_t row_lo, int H, int h,
                                                            int d, int es, int rows) {
    const char* p = static_cast<const char*>(base) + ((row_lo * H + h) * (int64_t)d) * es;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), 0, rows * H * d * es, 0x00020000);
}

// ---------------------------------------------------------------------------
// plan: chunk_start[b] = sum_{b' < b} nch(b'), snap_base[b] = sum_{b' < b}
// nsnap(b'), for b = 0 .. num_seqs, and order[]: the sequences by decreasing
// chunk count (ties by index) when there are at most LPT_MAX of them, else
// in index order.  The scan deals its chains out in that order, so the
// longest recurrences start first instead of trailing the batch.  A sequence whose first token sits at
// absolute position s (0 without start positions) is cut into chunks at the
// absolute multiples of C, so it has nch = ceil((s mod C + L) / C) chunks
// (none when L = 0), and snapshots at the absolute multiples of the interval
// in (s, s + L]: nsnap = floor((s + L) / interval) - floor(s / interval).
// ---------------------------------------------------------------------------
constexpr int LPT_MAX = 512;


__global__ __launch_bounds__(NT) void plan_kernel(const int32_t* __restrict__ cu,
                                                  const int32_t* __restrict__ start, int num_seqs,
                                                  int interval, int32_t* __restrict__ chunk_start,
                                                  int32_t* __restrict__ snap_base,
                                                  int32_t* __restrict__ order) {
    __shared__ int32_t wtot[2][4];
    __shared__ int32_t carry[2];
    __shared__ int32_t keys[LPT_MAX];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry[0] = carry[1] = 0;
    __syncthreads();
    const int32_t* sp = start ? start : cu;  // read unconditionally, used only with start
    for (int base = 0; base <= num_seqs; base += NT) {
        const int b = base + tid;
        int vc = 0, vs = 0;
        if (b < num_seqs) {
            const int L = cu[b + 1] - cu[b];
            const int s0 = start ? sp[b] : 0;
            vc = L > 0 ? (s0 % C + L + C - 1) / C : 0;
            vs = interval > 0 ? (s0 + L) / interval - s0 / interval : 0;
            if (num_seqs <= LPT_MAX) keys[b] = vc;  // the sort below reuses the counts
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
    if (num_seqs > LPT_MAX) {
        for (int b = tid; b < num_seqs; b += NT) order[b] = b;
        return;
    }
    for (int b = tid; b < num_seqs; b += NT) {
        const int key = keys[b];
        int rank = 0;
        for (int b2 = 0; b2 < num_seqs; ++b2) {
            const int k2 = keys[b2];
            rank += (k2 > key) | ((k2 == key) & (b2 < b));
        }
        order[rank] = b;
    }
}

// ---------------------------------------------------------------------------
// prep: per (chunk, head) every state-independent quantity of the chunk,
// written to the workspace as MFMA operands in the order the scan reads them.
// ---------------------------------------------------------------------------
// Operand block of one (chunk, head), in 16-byte units (8 fp16 = one MFMA
// operand of one lane, or 4 fp32 accumulator values of one lane).  Scan lane
// (g = lane/16, i = lane%16) of wave w reads index [...][lane] of:
//   W, Q'   [r][mt]      fp16 row tok_of(mt, i), channels 32r + 8g .. +7
//   Kd      [w][m][ks]   fp16 channel 32w + chan_of(m, i), tokens 32ks + 8g .. +7
//   U~, O~  [jt][mt]     fp32 rows tok_of(mt, 4g .. 4g+3), column 16jt + i
//   dec     128 floats, e^{G_C} per channel
//   exp     5 x 16 bytes of tile exponents (below)
// with W = TB (K . e^G), M = B TB, Q' = Q . e^G - M (K . e^G),
// Kd = (K . e^{G_C - G})^T, U~ = TB V and O~ = M V.  With these the chunk
// step is
//   U = U~ - W S,   O = scale (Q' S + O~),   S' = Diag(e^{G_C}) S + Kd U,
// since B U = B TB V - B TB (K . e^G) S.  Each fp16 tile (one lane-operand
// plane slice: 16 rows x 32 K positions) with magnitudes below 2^e is stored
// times 2^(F16_TOP - e).  Exponents are kept as bytes e + 126 (0 .. 255
// covers every fp32 magnitude), four to a 32-bit word: row w of exp holds
// EW[w][r], EQ[w][r] (token tile w, K-step r) and EK[w][m][ks] (state rows of
// wave w, byte 2m + ks); row 4 holds EU[mt] (every |U~| of token tile mt is
// below 2^EU) and EWM[mt] = max_r EW[mt][r].
constexpr int OP_W = 0;
constexpr int OP_Q = 2 * PLANE;
constexpr int OP_K = 4 * PLANE;
constexpr int OP_U = 6 * PLANE;
constexpr int OP_O = 10 * PLANE;
constexpr int OP_DEC = 14 * PLANE;
constexpr int OP_EXP = 14 * PLANE + 32;
constexpr int CHUNK_OPS = 14 * PLANE + 32 + 5;
constexpr int DVP = 128;             // value columns the operand block holds

template <typename TIn>
struct PrepSmem {
    static constexpr int KP = DKP + 16 / (int)sizeof(TIn);  // padded row of staged keys, queries
    static constexpr int NV = sizeof(TIn) == 2 ? 1 : 2;     // bf16 planes of a value (hi[, lo])
    union {
        float G[C][DKP + 4];   // cumulative log-decay, log2 units
        struct {
            union {
                float TT[C][C + 4];        // (I + A)^-1 transposed, TT[s][t] = T[t][s]
                uint16_t KgL[DKP][C];      // low bf16 half of (K . e^G)^T, once T is read;
                                           // 16-byte token groups permuted by vt_group
            } t;
            uint16_t VT[NV][DVP][C];       // V^T in bf16 planes, 16-byte groups swizzled by column
        } tv;
    } u;
    union {
        float A[C][C + 4];     // strictly lower b_t sum_c k_t k_s e^{G_t - G_s}
        float B[C][C + 4];     // lower sum_c q_t k_s e^{G_t - G_s}, once T is formed
    } ab;
    union {
        TIn kS[C][KP];             // the chunk's keys (zero past n and dk)
        uint16_t KgT[DKP][C + 8];  // (K . e^G)^T in bf16, [channel][token], once kS is read;
                                   // 16-byte token groups permuted by kg_group
    } k;
    float Bd[4][16][17];       // diagonal blocks of B from the pairwise path
    float Ms[3][16][17];       // block products of the forward substitution
    float beta[C];
};

// Exchange slots of the Gram partial sums, one 64-lane f32x4 tile per
// (row tile R, column tile ts <= R, A or B): row tiles 2 and 3 in the A/B
// area, row tiles 0 and 1 in the pairwise-path scratch that follows it.
template <typename SM>
__device__ __forceinline__ f32x4* gram_xch(SM& sm, int R, int ts, int which) {
    // blocks before row tile R: R (R + 1) / 2
    if (R >= 2) {
        const int blk = (R * (R + 1) / 2 - 3) + ts;  // row 2 -> 0..2, row 3 -> 3..6
        return reinterpret_cast<f32x4*>(&sm.ab.A[0][0]) + (blk * 2 + which) * 64;
    }
    const int blk = R * (R + 1) / 2 + ts;  // row 0 -> 0, row 1 -> 1..2
    return reinterpret_cast<f32x4*>(&sm.Bd[0][0][0]) + (blk * 2 + which) * 64;
}

struct PrepParams {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* cu;
    const int32_t* start;  // absolute position of each sequence's first token, or null
    const int32_t* chunk_start;
    uint4* ops;  // [chunks][H][CHUNK_OPS]
    int H, dk, dv, num_seqs;
};

// Location of one (chunk, head) item.
struct PrepItem {
    int h, lo, n;      // head; valid rows of the chunk are lo .. n-1
    int64_t gc, row0;  // global chunk index; packed row of chunk row 0
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
    // chunks sit at absolute multiples of C: the first chunk of a sequence
    // starting at absolute position s has s mod C leading rows that are not
    // the sequence's (staged as zero tokens, which leave the state alone)
    const int ci = gc - p.chunk_start[lo];
    const int pad = p.start ? p.start[lo] % C : 0;
    r.row0 = (int64_t)p.cu[lo] - pad + (int64_t)ci * C;
    r.n = min(C, pad + p.cu[lo + 1] - p.cu[lo] - ci * C);
    r.lo = ci == 0 ? pad : 0;
    return r;
}

// Gram work split: waves 0 and 3 form row tiles 0 and 3, waves 1 and 2 row
// tiles 1 and 2 (equal work per pair: a row tile w has w + 1 blocks), each
// wave over one half of the channels (K-steps 2 (w / 2), 2 (w / 2) + 1).
__device__ __forceinline__ int gram_row(int w, int slot) {
    const int ra = (w == 0 || w == 3) ? 0 : 1;
    return slot ? 3 - ra : ra;
}

// This thread's share of one item's raw inputs: g rows 8*(tid/32) + r,
// channels 4*(tid%32)..+3; k, q rows 16r + tid/16, channels 8*(tid%16)..+7; beta of
// row tid (tid < 64).  Rows outside lo .. n-1 read as zero (they fall outside
// the item's buffer resources) and channels past dk are read from channel 0;
// the values are masked when staged.
template <typename TIn>
struct PrepRaw {
    float4 g[8];
    typename In<TIn>::V8 k[4];
    typename In<TIn>::V8 qg[4];  // q of the Gram rows: [row slot][K-step of the channel half]
    typename In<TIn>::V8 qd[4];  // q at (tok_of(mt, lane%16), 32w' + 8*(lane/16)) of unit r
    float beta;
};

template <typename TIn>
__device__ __forceinline__ void prep_load(PrepRaw<TIn>& r, const PrepParams& p, const PrepItem& x,
                                          int tid) {
    using IO = In<TIn>;
    constexpr int ES = (int)sizeof(TIn);
    const int dk = p.dk;
    const int rows = x.n - x.lo;
    const int64_t rlo = x.row0 + x.lo;
    const uint32_t rsb = (uint32_t)(p.H * dk);  // row stride in elements
    {
        const __amdgpu_buffer_rsrc_t gb = item_rows(p.g, rlo, p.H, x.h, dk, 4, rows);
        const int c = 4 * (tid & 31);
        const uint32_t cb = 4 * (c < dk ? c : 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int t = 8 * (tid >> 5) + i;
            r.g[i] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    gb, (uint32_t)(t - x.lo) * rsb * 4 + cb, 0, 0));
        }
    }
    const __amdgpu_buffer_rsrc_t kb = item_rows(p.k, rlo, p.H, x.h, dk, ES, rows);
    const __amdgpu_buffer_rsrc_t qb = item_rows(p.q, rlo, p.H, x.h, dk, ES, rows);
    {
        const int c = 8 * (tid & 15);
        const uint32_t cb = ES * (c < dk ? c : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * i + (tid >> 4);
            r.k[i] = IO::bload8(kb, (uint32_t)(t - x.lo) * rsb * ES + cb);
        }
    }
    {
        const int lane = tid & 63, w = tid >> 6;
        const int ra = gram_row(w, 0), rb = gram_row(w, 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = 16 * ((u >> 1) ? rb : ra) + (lane & 15);
            const int c = 32 * (2 * (w >> 1) + (u & 1)) + 8 * (lane >> 4);
            r.qg[u] = IO::bload8(qb, (uint32_t)(t - x.lo) * rsb * ES + ES * (c < dk ? c : 0));
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int idx = tid + NT * u;
            const int ws = idx >> 8, mt = (idx >> 6) & 3, ln = idx & 63;
            const int tt = tok_of(mt, ln & 15), c = SL * ws + 8 * (ln >> 4);
            r.qd[u] = IO::bload8(qb, (uint32_t)(tt - x.lo) * rsb * ES + ES * (c < dk ? c : 0));
        }
    }
    {
        const __amdgpu_buffer_rsrc_t bb = item_rows(p.beta, rlo, p.H, x.h, 1, 4, rows);
        r.beta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               bb, (uint32_t)((tid & 63) - x.lo) * (uint32_t)p.H * 4, 0, 0));
    }
}

// One workgroup per (chunk, head) item; two are resident per compute unit.
// All of the item's global inputs are requested up front.
template <typename TIn>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prep_kernel(PrepParams p) {
    using IO = In<TIn>;
    using SM = PrepSmem<TIn>;
    __shared__ SM sm;
    // the wave index is uniform: kept in a scalar register, so addresses that
    // depend on it are formed on the scalar unit
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, i16 = lane & 15;
    const int dk = p.dk;

    const PrepItem x = prep_item(p, blockIdx.x);
    PrepRaw<TIn> raw;
    prep_load<TIn>(raw, p, x, tid);
    {
        const int n = x.n, lo = x.lo;
        uint4* __restrict__ dst = p.ops + (x.gc * p.H + x.h) * CHUNK_OPS;

        // ---- stage this item's inputs (zero outside rows lo .. n-1 and past
        // dk); log-decays in log2 units, so every factor below is a bare
        // exp2.  The cumulative log-decay: each thread sums its 8 rows of 4
        // channels in registers, the 8-row totals go through LDS, and each
        // thread adds the totals of the row blocks before its own.  The span
        // check of the diagonal Gram blocks (first and last row against the
        // middle row of each 16-row tile) needs only sums inside one 8-row
        // block: G[16R] - G[16R+7] in the block's first half and
        // G[16R+7] - G[16R+15] (minus the second half's total) ----
        int extreme = 0;
        float4 gr[8];
        const int gblk = tid >> 5, gc = 4 * (tid & 31);
        {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int t = 8 * gblk + i;
                // rows outside lo .. n-1 read as zero and channels past dk
                // from valid (finite) entries: a zero factor clears them
                // without a branch
                const float4 gv = raw.g[i];
                const float f = (t >= lo && t < n && gc < dk) ? LOG2E : 0.f;
                gr[i] = make_float4(gv.x * f, gv.y * f, gv.z * f, gv.w * f);
            }
#pragma unroll
            for (int i = 1; i < 8; ++i) {
                gr[i].x += gr[i - 1].x;
                gr[i].y += gr[i - 1].y;
                gr[i].z += gr[i - 1].z;
                gr[i].w += gr[i - 1].w;
            }
            if (gblk & 1) {
                extreme = (-gr[7].x > SPAN_LIMIT) | (-gr[7].y > SPAN_LIMIT) | (-gr[7].z > SPAN_LIMIT) |
                          (-gr[7].w > SPAN_LIMIT);
            } else {
                extreme = (gr[0].x - gr[7].x > SPAN_LIMIT) | (gr[0].y - gr[7].y > SPAN_LIMIT) |
                          (gr[0].z - gr[7].z > SPAN_LIMIT) | (gr[0].w - gr[7].w > SPAN_LIMIT);
            }
            // 8-row totals, in the A/B area (unused until the Gram exchange)
            reinterpret_cast<float4*>(&sm.ab.A[0][0])[gblk * 32 + (tid & 31)] = gr[7];
        }
        {
            const int c = 8 * (tid & 15);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * i + (tid >> 4);
                const typename IO::V8 kz = (t >= lo && t < n && c < dk) ? raw.k[i] : IO::zero8();
                *reinterpret_cast<typename IO::V8*>(&sm.k.kS[t][c]) = kz;
            }
        }
        if (tid < C) sm.beta[tid] = (tid >= lo && tid < n) ? raw.beta : 0.f;
        __syncthreads();
        {
            // every total is read and the earlier blocks' are selected (a
            // read under a condition becomes a branch and a wait)
            float4 base = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int b2 = 0; b2 < 7; ++b2) {
                const float4 tb = reinterpret_cast<const float4*>(&sm.ab.A[0][0])[b2 * 32 + (tid & 31)];
                if (b2 < gblk) {
                    base.x += tb.x;
                    base.y += tb.y;
                    base.z += tb.z;
                    base.w += tb.w;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *reinterpret_cast<float4*>(&sm.u.G[8 * gblk + i][gc]) =
                    make_float4(gr[i].x + base.x, gr[i].y + base.y, gr[i].z + base.z, gr[i].w + base.w);
        }
        __syncthreads();

        // ---- Gram matrices A and B, 16 x 16 blocks (row tile R, column tile ts <= R) ----
        // Off-diagonal blocks use the reference r = G at row 16R - 1, so both
        // factors e^{G_t - r} and e^{r - G_s} are <= 1.  The diagonal block
        // uses r = G at row 16R + 7, keeping both factors within 2^{+-span/2}
        // of the block; half-spans beyond SPAN_LIMIT take the pairwise path.
        // Wave w forms row tiles gram_row(w, 0..1) over its channel half; the
        // partial sums of the row tile it does not own go to its partner
        // through LDS, so that wave w ends with row tile w summed over all
        // channels.
        f32x4 accB[4];
        {
            f32x4 pA[2][4], pB[2][4];  // [row slot][column tile]
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int ts = 0; ts < 4; ++ts) {
                    pA[sl][ts] = f32x4{0.f, 0.f, 0.f, 0.f};
                    pB[sl][ts] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            const int hh = w >> 1;
            // instantiated per pair of row tiles (waves 0 and 3: tiles 0 and 3;
            // waves 1 and 2: tiles 1 and 2), so that every block choice below
            // is known at compile time and no LDS read waits behind a branch
            auto gram_blocks = [&](auto ra_c) {
            constexpr int RA = decltype(ra_c)::value;
#pragma unroll 1
            for (int kk = 0; kk < 2; ++kk) {
                const int c0 = 32 * (2 * hh + kk) + 8 * g4;
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) {
                    const int R = sl ? 3 - RA : RA;
                    const int t = 16 * R + i16;
                    float kt[8], qt[8];
                    IO::f32x8(*reinterpret_cast<const typename IO::V8*>(&sm.k.kS[t][c0]), kt);
                    const typename IO::V8 qx = kk ? raw.qg[2 * sl + 1] : raw.qg[2 * sl];
                    IO::f32x8((t >= lo && t < n && c0 < dk) ? qx : IO::zero8(), qt);
                    float Gt[8], rw[8], rm[8];
                    lds8(&sm.u.G[t][c0], Gt);
                    lds8(&sm.u.G[R > 0 ? 16 * R - 1 : 0][c0], rw);
                    lds8(&sm.u.G[16 * R + 7][c0], rm);
                    // diagonal block: both Grams in three passes (hi*hi + hi*lo
                    // + lo*hi), so that A and B round alike -- with q = k and
                    // beta = 1, B = I + A and M = B TB must come out as I
                    {
                        float xk[8], xq[8], yv[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float xd = ex2(Gt[e] - rm[e]);
                            const float yd = ex2(rm[e] - Gt[e]);
                            xk[e] = kt[e] * xd;
                            xq[e] = qt[e] * xd;
                            yv[e] = kt[e] * yd;
                        }
                        uint4 xkh, xkl, xqh, xql, yh, yl;
                        split8(xk, xkh, xkl);
                        split8(xq, xqh, xql);
                        split8(yv, yh, yl);
                        const bf16x8_t XKH = as_op(xkh), XKL = as_op(xkl), XQH = as_op(xqh),
                                       XQL = as_op(xql), YH = as_op(yh), YL = as_op(yl);
#pragma unroll
                        for (int ts = 0; ts < 4; ++ts) {
                            if (ts == R) {
                                pA[sl][ts] = mfma(XKH, YH, pA[sl][ts]);
                                pA[sl][ts] = mfma(XKH, YL, pA[sl][ts]);
                                pA[sl][ts] = mfma(XKL, YH, pA[sl][ts]);
                                pB[sl][ts] = mfma(XQH, YH, pB[sl][ts]);
                                pB[sl][ts] = mfma(XQH, YL, pB[sl][ts]);
                                pB[sl][ts] = mfma(XQL, YH, pB[sl][ts]);
                            }
                        }
                    }
                    // off-diagonal blocks: both factors are at most 1
                    // (g <= 0), so the operands are fp16, rounded once
                    if (R > 0) {
                        float xk[8], xq[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float xo = ex2(Gt[e] - rw[e]);
                            xk[e] = kt[e] * xo;
                            xq[e] = qt[e] * xo;
                        }
                        const uint4 XK = h8(xk), XQ = h8(xq);
#pragma unroll
                        for (int ts = 0; ts < 3; ++ts) {
                            if (ts < R) {
                                const int s = 16 * ts + i16;
                                float ksv[8];
                                IO::f32x8(*reinterpret_cast<const typename IO::V8*>(&sm.k.kS[s][c0]), ksv);
                                float gs[8], yv[8];
                                lds8(&sm.u.G[s][c0], gs);
#pragma unroll
                                for (int e = 0; e < 8; ++e) yv[e] = ksv[e] * ex2(rw[e] - gs[e]);
                                const uint4 Y = h8(yv);
                                pA[sl][ts] = mfma_h(XK, Y, pA[sl][ts]);
                                pB[sl][ts] = mfma_h(XQ, Y, pB[sl][ts]);
                            }
                        }
                    }
                }
            }
            };
            if (w == 0 || w == 3) gram_blocks(std::integral_constant<int, 0>{});
            else gram_blocks(std::integral_constant<int, 1>{});
            // exchange: the slot this wave does not own goes to its partner
            const int own = (gram_row(w, 0) == w) ? 0 : 1;
            f32x4 accA[4];
            {
                const int R = gram_row(w, 1 - own);
#pragma unroll
                for (int ts = 0; ts < 4; ++ts)
                    if (ts <= R) {
                        gram_xch(sm, R, ts, 0)[lane] = own ? pA[0][ts] : pA[1][ts];
                        gram_xch(sm, R, ts, 1)[lane] = own ? pB[0][ts] : pB[1][ts];
                    }
            }
            __syncthreads();
#pragma unroll
            for (int ts = 0; ts < 4; ++ts) {
                const f32x4 a = own ? pA[1][ts] : pA[0][ts], bb = own ? pB[1][ts] : pB[0][ts];
                if (ts <= w) {
                    accA[ts] = a + gram_xch(sm, w, ts, 0)[lane];
                    accB[ts] = bb + gram_xch(sm, w, ts, 1)[lane];
                } else {
                    accA[ts] = a;
                    accB[ts] = bb;
                }
            }
            __syncthreads();  // the exchange area overlaps A
            // accumulator (row 4*g4+e, column i16) of block (w, ts); masked
            // entries are selected away, never multiplied (they may hold inf)
#pragma unroll
            for (int ts = 0; ts < 4; ++ts)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tr = 16 * w + 4 * g4 + e, sc = 16 * ts + i16;
                    const float a = accA[ts][e] * sm.beta[tr];
                    sm.ab.A[tr][sc] = (sc < tr) ? a : 0.f;
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
                    const float qt = (t >= lo && t < n) ? IO::f32(IO::load1(p.q, ((x.row0 + t) * p.H + x.h) * (int64_t)dk + c)) : 0.f;
                    const float e = ex2(sm.u.G[t][c] - sm.u.G[s][c]);
                    sa = fmaf(kt * kv, e, sa);
                    sb = fmaf(qt * kv, e, sb);
                }
                sm.ab.A[t][s] = (s < t) ? sa * sm.beta[t] : 0.f;
                sm.Bd[blk][tl][sl] = sb;
            }
            __syncthreads();
        }

        // this item's v rows (4 rows x 8 columns per thread: the row pairs
        // 2a, 2a + 1 and 2a + 32, 2a + 33 with a = tid / 16), requested here
        // and staged as V^T after the diagonal blocks of T are solved
        typename IO::V8 vr[4];
        {
            constexpr int ES = (int)sizeof(TIn);
            const int c = 8 * (tid & 15);
            const __amdgpu_buffer_rsrc_t vbuf = item_rows(p.v, x.row0 + lo, p.H, x.h, p.dv, ES, n - lo);
            const uint32_t rsb = (uint32_t)(p.H * p.dv) * ES, cb = ES * (c < p.dv ? c : 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 2 * (tid >> 4) + (i & 1) + 32 * (i >> 1);
                vr[i] = IO::bload8(vbuf, (uint32_t)(t - lo) * rsb + cb);
            }
        }

        // ---- decay-scaled operands: Kd planes, Qd planes, dec, then (K e^G)^T ----
#pragma unroll 2
        for (int r = 0; r < 4; ++r) {
            const int idx = tid + NT * r;  // (w', m, ks, lane)
            const int ws = idx >> 8, m = (idx >> 7) & 1, ks = (idx >> 6) & 1, ln = idx & 63;
            const int c = SL * ws + chan_of(m, ln & 15), t0 = 32 * ks + 8 * (ln >> 4);
            const float gcc = sm.u.G[C - 1][c];
            float kv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int t = t0 + e;
                kv[e] = IO::f32(sm.k.kS[t][c]) * ex2(gcc - sm.u.G[t][c]);
            }
            // this wave's 64 lanes hold exactly tile (w' = r, m, ks) with
            // m * 2 + ks = w: one exponent per tile
            float mb = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) mb = amax(mb, kv[e]);
            const uint32_t kb = wave_max_u32(bits(mb));
            const int s = F16_TOP - bound_exp(kb);
            dst[OP_K + idx] = make_uint4(h2(scl(kv[0], s), scl(kv[1], s)), h2(scl(kv[2], s), scl(kv[3], s)),
                                         h2(scl(kv[4], s), scl(kv[5], s)), h2(scl(kv[6], s), scl(kv[7], s)));
            if (lane == 0) reinterpret_cast<uint8_t*>(dst + OP_EXP + r)[8 + w] = exp_byte(kb);
        }
        // Q e^G of this thread's units (token tok_of(w, i16), channels
        // 32r + 8*g4 .. +7) stay in fp32 until Q' is formed; K e^G of the same
        // units goes to the transposed copy as bf16 hi (now) and lo (held in
        // registers until T is read, then written over it)
        float qd[4][8];
        uint16_t kg[4][8];
        uint32_t kgl[4][4];  // lo halves, channels c0 + 2i (low) and c0 + 2i + 1 (high)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tok_of(w, i16), c0 = SL * r + 8 * g4;
            float qv[8], kv[8];
            IO::f32x8((t >= lo && t < n && c0 < dk) ? raw.qd[r] : IO::zero8(), qv);
            IO::f32x8(*reinterpret_cast<const typename IO::V8*>(&sm.k.kS[t][c0]), kv);
            float gt[8];
            lds8(&sm.u.G[t][c0], gt);
            float kx[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float eg = ex2(gt[e]);
                qd[r][e] = qv[e] * eg;
                kx[e] = kv[e] * eg;
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hi;
                split2(kx[2 * i], kx[2 * i + 1], hi, kgl[r][i]);
                kg[r][2 * i] = (uint16_t)(hi & 0xffffu);
                kg[r][2 * i + 1] = (uint16_t)(hi >> 16);
            }
        }
        if (tid < DKP) reinterpret_cast<float*>(dst + OP_DEC)[tid] = ex2(sm.u.G[C - 1][tid]);
        __syncthreads();  // keys and G are read: their storage becomes (K e^G)^T, T and V^T
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = tok_of(w, i16), c0 = SL * r + 8 * g4;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int q = kslot(t);
                sm.k.KgT[c0 + e][kg_group(c0 + e, q >> 3) * 8 + (q & 7)] = kg[r][e];
            }
        }
        // ---- T = (I + A)^-1 by block forward substitution ----
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
            for (int r = 0; r < 16; ++r) sm.u.tv.t.TT[bo + j][bo + r] = xs[r];
        }
        // V^T: rows outside lo .. n-1 and columns past dv are zero.  V^T rows are 64
        // tokens; its 16-byte groups are permuted by vt_group so that neither
        // the transposing writes nor the operand reads collide in LDS banks.
        {
            const int c = 8 * (tid & 15);
            if constexpr (sizeof(TIn) == 2) {
                // two tokens of a column as one 32-bit word (row t in the low half)
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    const int t = 2 * (tid >> 4) + 32 * pr;
                    const uint32_t keep = ((t >= lo && t < n && c < p.dv) ? 0xffffu : 0u) |
                                          ((t + 1 >= lo && t + 1 < n && c < p.dv) ? 0xffff0000u : 0u);
                    const uint32_t* r0 = &vr[2 * pr].x;
                    const uint32_t* r1 = &vr[2 * pr + 1].x;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = c + e;
                        const uint32_t wd = __builtin_amdgcn_perm(r1[e >> 1], r0[e >> 1],
                                                                  (e & 1) ? 0x07060302u : 0x05040100u);
                        const int q = kslot(t);  // t even: t + 1 sits in slot q + 1
                        *reinterpret_cast<uint32_t*>(&sm.u.tv.VT[0][j][vt_group(j, q >> 3) * 8 + (q & 7)]) =
                            wd & keep;
                    }
                }
            } else {
                // fp32 values as hi and lo bf16 planes
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 2 * (tid >> 4) + (i & 1) + 32 * (i >> 1);
                    const bool live = t >= lo && t < n && c < p.dv;
                    float xv[8];
                    IO::f32x8(vr[i], xv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = c + e;
                        const int q = kslot(t);
                        const int off = vt_group(j, q >> 3) * 8 + (q & 7);
                        uint16_t hi, lo;
                        split(live ? xv[e] : 0.f, hi, lo);
                        sm.u.tv.VT[0][j][off] = hi;
                        sm.u.tv.VT[SM::NV - 1][j][off] = lo;
                    }
                }
            }
        }
        __syncthreads();
        // Off-diagonal blocks band by band; wave I forms block (I, J = I - d):
        //   M = sum_{K=J}^{I-1} A_IK T_KJ,   T_IJ = -T_II M
        // on the fp32 MFMA (16x16x4, one fp32 value per lane and operand), so
        // every product is exact in fp32.
#pragma unroll
        for (int d = 1; d < 4; ++d) {
            if (w >= d) {
                const int I = w, J = w - d;
                const int ar = 16 * I + i16;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                for (int K = J; K < I; ++K)
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        const int k = 16 * K + 4 * kk + g4;
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.ab.A[ar][k], sm.u.tv.t.TT[16 * J + i16][k],
                                                                 acc, 0, 0, 0);
                    }
                float (*Mw)[17] = sm.Ms[w - 1];
#pragma unroll
                for (int e = 0; e < 4; ++e) Mw[4 * g4 + e][i16] = acc[e];
                lds_wave_sync();
                f32x4 tm = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const int k = 4 * kk + g4;
                    tm = __builtin_amdgcn_mfma_f32_16x16x4f32(sm.u.tv.t.TT[16 * I + k][ar], Mw[k][i16], tm, 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.u.tv.t.TT[16 * J + i16][16 * I + 4 * g4 + e] = -tm[e];
            }
            __syncthreads();
        }

        // ---- B (A is dead now) ----
#pragma unroll
        for (int ts = 0; ts < 4; ++ts)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tr = 16 * w + 4 * g4 + e, sc = 16 * ts + i16;
                // the pairwise value is read unconditionally and selected (a
                // load under a condition becomes a branch and a wait)
                const float bd = sm.Bd[w][4 * g4 + e][i16];
                const float v = (any_extreme && ts == w) ? bd : accB[ts][e];
                sm.ab.B[tr][sc] = (sc <= tr) ? v : 0.f;
            }
        __syncthreads();

        // ---- wave w from here on: token tile w.  Rows of TB (in slot order,
        // see kslot) and of B as MFMA operands, then M = B TB formed as M^T
        // (blocks that vanish by triangularity are skipped), whose
        // accumulators hold the wave's rows of M in slot order ----
        bf16x8_t TBh[2], TBl[2], Mh[2], Ml[2];
        {
            const int t = tok_of(w, i16);
            bf16x8_t Bh[2], Bl[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int s0 = 32 * ks + 8 * g4;
                float tv[8], bv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = s0 + e, sq = kslot_tok(s);
                    const float x = sm.u.tv.t.TT[sq][t] * sm.beta[sq];
                    tv[e] = (sq <= t) ? x : 0.f;
                    bv[e] = sm.ab.B[t][s];
                }
                uint4 th, tl, bh, bl;
                split8(tv, th, tl);
                split8(bv, bh, bl);
                TBh[ks] = as_op(th);
                TBl[ks] = as_op(tl);
                Bh[ks] = as_op(bh);
                Bl[ks] = as_op(bl);
            }
            f32x4 acc[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks == 1 && w < 2) continue;  // tokens of tiles 0, 1 are < 32: B[t][s >= 32] = 0
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    if (ks == 0 && nt >= 2) continue;  // TB[s < 32][s' >= 32] = 0
                    // column 16nt + i16 of TB over tokens 32ks + 8*g4 .. +7
                    const int sc = 16 * nt + i16;
                    float cv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int s = 32 * ks + 8 * g4 + e;
                        const float x = sm.u.tv.t.TT[sc][s] * sm.beta[sc];
                        cv[e] = (sc <= s) ? x : 0.f;
                    }
                    uint4 ch, cl;
                    split8(cv, ch, cl);
                    const bf16x8_t CH = as_op(ch), CL = as_op(cl);
                    acc[nt] = mfma(CH, Bh[ks], acc[nt]);
                    acc[nt] = mfma(CL, Bh[ks], acc[nt]);
                    acc[nt] = mfma(CH, Bl[ks], acc[nt]);
                }
            }
            __syncthreads();  // every row of T is read: its storage becomes the low
                              // half of (K e^G)^T
            // M^T tiles 2 ks and 2 ks + 1 are M's K-step ks in slot order
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const float mv[8] = {acc[2 * ks][0], acc[2 * ks][1], acc[2 * ks][2], acc[2 * ks][3],
                                     acc[2 * ks + 1][0], acc[2 * ks + 1][1], acc[2 * ks + 1][2],
                                     acc[2 * ks + 1][3]};
                uint4 mh, ml;
                split8(mv, mh, ml);
                Mh[ks] = as_op(mh);
                Ml[ks] = as_op(ml);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c0 = SL * r + 8 * g4;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t x = kgl[r][e >> 1];
                    const int q = kslot(t);
                    sm.u.tv.t.KgL[c0 + e][vt_group(c0 + e, q >> 3) * 8 + (q & 7)] =
                        (uint16_t)((e & 1) ? (x >> 16) : (x & 0xffffu));
                }
            }
        }
        __syncthreads();

        // ---- W = TB (K e^G) and Q' = Q e^G - M (K e^G) for token tile w,
        // formed transposed: accumulator rows are channels 32r + chan_of(m, .),
        // columns the tile's tokens, so the two row tiles of K-step r pack
        // directly into the scan's operand ----
        uint32_t ewb[4], eqb[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f32x4 aw[2], aq[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                aw[m] = f32x4{0.f, 0.f, 0.f, 0.f};
                aq[m] = f32x4{qd[r][4 * m], qd[r][4 * m + 1], qd[r][4 * m + 2], qd[r][4 * m + 3]};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const int cr = SL * r + chan_of(m, i16);
                    const bf16x8_t kgo = as_op(*reinterpret_cast<const uint4*>(
                        &sm.k.KgT[cr][kg_group(cr, 4 * ks + g4) * 8]));
                    const bf16x8_t kgl = as_op(*reinterpret_cast<const uint4*>(
                        &sm.u.tv.t.KgL[cr][vt_group(cr, 4 * ks + g4) * 8]));
                    aw[m] = mfma(kgo, TBh[ks], aw[m]);
                    aw[m] = mfma(kgo, TBl[ks], aw[m]);
                    aw[m] = mfma(kgl, TBh[ks], aw[m]);
                    aq[m] = mfma(kgo, neg(Mh[ks]), aq[m]);
                    aq[m] = mfma(kgo, neg(Ml[ks]), aq[m]);
                    aq[m] = mfma(kgl, neg(Mh[ks]), aq[m]);
                }
            }
            const int idx = (r * 4 + w) * 64 + lane;
            float mw = 0.f, mq = 0.f;
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    mw = amax(mw, aw[m][e]);
                    mq = amax(mq, aq[m][e]);
                }
            ewb[r] = wave_max_u32(bits(mw));
            eqb[r] = wave_max_u32(bits(mq));
            dst[OP_W + idx] = pack_h(aw[0], aw[1], F16_TOP - bound_exp(ewb[r]));
            dst[OP_Q + idx] = pack_h(aq[0], aq[1], F16_TOP - bound_exp(eqb[r]));
        }
        if (lane == 0) {
            uint32_t* ex = reinterpret_cast<uint32_t*>(dst + OP_EXP + w);
            ex[0] = exp_byte(ewb[0]) | (exp_byte(ewb[1]) << 8) | (exp_byte(ewb[2]) << 16) |
                    ((uint32_t)exp_byte(ewb[3]) << 24);
            ex[1] = exp_byte(eqb[0]) | (exp_byte(eqb[1]) << 8) | (exp_byte(eqb[2]) << 16) |
                    ((uint32_t)exp_byte(eqb[3]) << 24);
            reinterpret_cast<uint8_t*>(dst + OP_EXP + 4)[4 + w] =
                exp_byte(max(max(ewb[0], ewb[1]), max(ewb[2], ewb[3])));
        }

        // ---- U~ = TB V and O~ = M V for token tile w, every value tile ----
        const int ntv = p.dv >> 4;
        float4* __restrict__ du = reinterpret_cast<float4*>(dst + OP_U);
        float4* __restrict__ dov = reinterpret_cast<float4*>(dst + OP_O);
        float mu = 0.f;  // largest |U~| of the token tile over every value column
#pragma unroll
        for (int jt = 0; jt < DVP / 16; ++jt) {
            if (jt >= ntv) break;
            f32x4 au = {0.f, 0.f, 0.f, 0.f}, ao = {0.f, 0.f, 0.f, 0.f};
            const int j = 16 * jt + i16;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int off = vt_group(j, 4 * ks + g4) * 8;
                const bf16x8_t vh = as_op(*reinterpret_cast<const uint4*>(&sm.u.tv.VT[0][j][off]));
                au = mfma(TBh[ks], vh, au);
                au = mfma(TBl[ks], vh, au);
                ao = mfma(Mh[ks], vh, ao);
                ao = mfma(Ml[ks], vh, ao);
                if constexpr (SM::NV == 2) {
                    const bf16x8_t vl =
                        as_op(*reinterpret_cast<const uint4*>(&sm.u.tv.VT[SM::NV - 1][j][off]));
                    au = mfma(TBh[ks], vl, au);
                    ao = mfma(Mh[ks], vl, ao);
                }
            }
            du[(jt * 4 + w) * 64 + lane] = make_float4(au[0], au[1], au[2], au[3]);
            dov[(jt * 4 + w) * 64 + lane] = make_float4(ao[0], ao[1], ao[2], ao[3]);
#pragma unroll
            for (int e = 0; e < 4; ++e) mu = amax(mu, au[e]);
        }
        const uint32_t ub = wave_max_u32(bits(mu));
        if (lane == 0) reinterpret_cast<uint8_t*>(dst + OP_EXP + 4)[w] = exp_byte(ub);
    }
}

// ---------------------------------------------------------------------------
// scan: per (sequence, head, TPW x 16 value columns) the recurrence over
// chunks.  Wave w owns state rows 32w .. 32w+31 and token tile w of the
// chunk.  Per chunk the waves publish their state rows (as hi/lo MFMA
// operands) through LDS; each wave then forms its token tile of W S,
// U = TB V - W S and (Q e^G) S over all 128 state rows and publishes its
// tile of U; after the second barrier each wave updates its state rows from
// the whole U and writes its token tile of O.  Nothing is reduced across
// waves, so the LDS traffic per chunk is the state once and U once.
//
// A wave carries TPW value tiles of 16 columns: the chunk's W, Q' and Kd
// operands (48 KB of the 57 KB a tile reads per chunk) are loaded once for
// all of them.  Each 16-column tile keeps its own exponents and runs the
// same instructions in the same order whatever TPW is, so results do not
// depend on the width a call chose.
// ---------------------------------------------------------------------------
template <int TPW>
struct ScanSmem {
    uint4 sx[TPW][4][64][2];                               // state rows of wave r as K-step r operands [hi, lo]
    struct Ux { uint2 h[2]; uint2 l[2]; } ux[TPW][2][64];  // U operands per K-step, halves by token tile
    uint32_t se[TPW];                                      // exponent bytes of the state-row blocks
};

struct ScanParams {
    const int32_t* cu;
    const int32_t* start;       // absolute start positions, or null (all 0)
    const int32_t* slots;       // state row of each sequence, or null (row b)
    const int32_t* chunk_start;
    const int32_t* snap_base;
    const int32_t* order;       // sequences, longest first (see plan_kernel)
    const uint4* ops;
    const float* init;          // null: zero initial states
    int init_if_started;        // read init only for sequences with start > 0
    void* out;
    float* final_state;
    float* snapshots;
    int interval;
    int H, dk, dv;
    int ngroups, nchains;       // value-tile groups of TPW tiles per chain; chains
    float scale;
};

// One chunk's operands for one lane, loaded ahead.
template <int TPW>
struct ScanOps {
    uint4 w[4];           // W  of this wave's token tile, K-step r = state rows 32((r + rot) & 3) ..
    uint4 q[4];           // Q' of this wave's token tile, likewise
    uint4 kd[2][2];       // Kd of this wave's state rows [m][ks]
    float4 u[TPW], o[TPW];  // U~ and O~ of this wave's token tile, per value tile
    float4 dec[2];        // e^{G_C} of the lane's state rows
    uint4 ex, ex4;        // exponent rows w and 4 (the same in every lane)
};

// The next chunk's operands are loaded in three parts spread over the
// current chunk, so the wave never stalls on a full memory queue.  Loads go
// through a buffer resource of the chunk's block: the lane's offset is one
// register for every load, the rest of each address is a scalar.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t scan_block(const ScanParams& p, int64_t gc, int h) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(p.ops + (gc * p.H + h) * CHUNK_OPS), 0,
                                             CHUNK_OPS * 16, 0x00020000);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int unit) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, unit * 16, 0));
}
__device__ __forceinline__ float4 ld16f(__amdgpu_buffer_rsrc_t r, uint32_t voff, int unit) {
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, unit * 16, 0));
}

// vo = 16 * lane; tile0 = first value tile of the workgroup.  K-step r of
// W and Q' holds the state rows of block (r + rot) & 3: the workgroups of
// one head take the blocks in different orders, so they do not all request
// the same lines at once.
template <int TPW>
__device__ __forceinline__ void scan_load1(ScanOps<TPW>& o, __amdgpu_buffer_rsrc_t blk, int w, int tile0,
                                           uint32_t vo, int rot) {
#pragma unroll
    for (int r = 0; r < 4; ++r) o.w[r] = ld16(blk, vo, OP_W + (((r + rot) & 3) * 4 + w) * 64);
#pragma unroll
    for (int t = 0; t < TPW; ++t) o.u[t] = ld16f(blk, vo, OP_U + ((tile0 + t) * 4 + w) * 64);
    o.ex = ld16(blk, 0, OP_EXP + w);
    o.ex4 = ld16(blk, 0, OP_EXP + 4);
}

template <int TPW>
__device__ __forceinline__ void scan_load2(ScanOps<TPW>& o, __amdgpu_buffer_rsrc_t blk, int w, int tile0,
                                           uint32_t vo, int rot) {
#pragma unroll
    for (int r = 0; r < 4; ++r) o.q[r] = ld16(blk, vo, OP_Q + (((r + rot) & 3) * 4 + w) * 64);
#pragma unroll
    for (int t = 0; t < TPW; ++t) o.o[t] = ld16f(blk, vo, OP_O + ((tile0 + t) * 4 + w) * 64);
}

// vd = 32 * (lane / 16)
template <int TPW>
__device__ __forceinline__ void scan_load3(ScanOps<TPW>& o, __amdgpu_buffer_rsrc_t blk, int w, uint32_t vo,
                                           uint32_t vd) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) o.kd[m][ks] = ld16(blk, vo, OP_K + ((w * 2 + m) * 2 + ks) * 64);
    // e^{G_C} of channels 32w + 8*(lane/16) .. +7
    o.dec[0] = ld16f(blk, vd, OP_DEC + 8 * w);
    o.dec[1] = ld16f(blk, vd, OP_DEC + 8 * w + 1);
}

// fp16 hi and lo of four fp32 values, as two packed 64-bit halves
__device__ __forceinline__ void hsplit4(const f32x4& x, uint2& hi, uint2& lo) {
    hsplit2(x[0], x[1], hi.x, lo.x);
    hsplit2(x[2], x[3], hi.y, lo.y);
}
__device__ __forceinline__ uint32_t uni(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }

// DB: the next chunk's operands go to a second register set while the
// current chunk runs (the deepest prefetch, one workgroup per compute unit:
// for few, long recurrences).  !DB: one register set, each part reloaded
// as soon as the current chunk has consumed it.  The arithmetic is the same
// instruction for instruction, so both give the same bits.
template <bool OUT_BF16, bool DB, int TPW>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void scan_kernel(ScanParams p) {
    __shared__ ScanSmem<TPW> sm;
    // the wave index is uniform: kept in a scalar register, so addresses that
    // depend on it are formed on the scalar unit
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, i16 = lane & 15;
    (void)tid;

    // workgroup -> (chain, group of TPW value tiles); a chain is a
    // (sequence, head) pair with its sequences taken longest first.
    // Workgroups are dealt round-robin over the 8 XCDs: chain rho goes to XCD
    // rho mod 8, where its groups follow each other in dispatch order, so the
    // tiles of one head share an L2 and the chains start in order of length.
    // The start of a workgroup is a chain of dependent loads (arguments, the
    // chain's sequence, its offsets, its initial state): null index arrays
    // are replaced by a valid one whose values are then ignored, so no load
    // waits behind a branch, and the initial state is requested at once.
    const int ngroups = p.ngroups, nchains = p.nchains, H = p.H, dk = p.dk, dv = p.dv;
    const int32_t* const order = p.order;
    const int32_t* const cu = p.cu;
    const int32_t* const start = p.start;
    const int32_t* const slots = p.slots;
    const int pos = blockIdx.x >> 3;
    const int chain = (pos / ngroups) * 8 + (blockIdx.x & 7);
    if (chain >= nchains) return;
    const int tile0 = (pos % ngroups) * TPW;
    const int rk = chain / H, h = chain - rk * H;
    const int b = order[rk];
    const int j0 = 16 * tile0 + i16;  // value column of this lane in tile t: j0 + 16 t
    // the order of the state-row blocks (see scan_load1): a function of the
    // pair of tiles.  The blocks are loaded in the order of the workgroup's
    // first pair; tile t sums its four block products starting at block
    // (t / 2) of that order, which is its own pair's order, so every tile
    // sums in the same order at any width
    const int rot = (tile0 >> 1) & 3;
    const uint32_t rsh = 8 * rot;
    auto rot_bytes = [rsh](uint32_t x) { return (uint32_t)((((uint64_t)x << 32) | x) >> rsh); };
    const int32_t c0v = cu[b], c1v = cu[b + 1];
    const int32_t startv = (start ? start : cu)[b];
    const int32_t slotv = (slots ? slots : cu)[b];
    const int64_t cbase = p.chunk_start[b];
    const int64_t sbase = p.snap_base[b];
    const int64_t seq0 = c0v;
    const int len = c1v - c0v;
    // chunks sit at absolute multiples of C (see plan_kernel): pad leading
    // rows of the first chunk precede the sequence's first token
    const int spos = start ? startv : 0;
    const int pad = spos % C;
    const int nch = len > 0 ? (pad + len + C - 1) / C : 0;

    // state rows of this lane: 32w + chan_of(m, 4*g4 + e) = 32w + 8*g4 + 4m + e
    f32x4 S[TPW][2];
    const int64_t srow = ((slots ? (int64_t)slotv : (int64_t)b) * H + h) * dk;
    const bool has_init = p.init && (!p.init_if_started || spos > 0);
    if (has_init) {
        float xi[TPW][2][4];  // every load first, then the masking
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = SL * w + 8 * g4 + 4 * m + e;
                    xi[t][m][e] = p.init[(srow + (c < dk ? c : 0)) * dv + j0 + 16 * t];
                }
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = SL * w + 8 * g4 + 4 * m + e;
                    S[t][m][e] = c < dk ? xi[t][m][e] : 0.f;
                }
    } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int m = 0; m < 2; ++m) S[t][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Operands are prefetched into two register sets used in turn (DB: the
    // loop body is instantiated twice with the roles swapped, so no loaded
    // value is copied) or into one set reloaded part by part (!DB).
    const uint32_t vo = 16 * lane, vd = 32 * g4;
    ScanOps<TPW> opA, opB;
    if (nch > 0) {
        const __amdgpu_buffer_rsrc_t blk = scan_block(p, cbase, h);
        scan_load1(opA, blk, w, tile0, vo, rot);
        scan_load2(opA, blk, w, tile0, vo, rot);
        scan_load3(opA, blk, w, vo, vd);
    }

    // Output rows of a chunk through a buffer resource that ends at the
    // sequence's last row: stores past it fall outside and are dropped.
    // Tile t's columns sit 16 t elements after tile 0's (a scalar offset).
    constexpr int OB = OUT_BF16 ? 2 : 4;
    const int64_t orow = (int64_t)H * dv;  // elements per token row
    uint32_t ooff[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        ooff[e] = (uint32_t)(((int64_t)tok_of(w, 4 * g4 + e) * orow + (int64_t)h * dv + j0) * OB);

    // Snapshots fall at the absolute multiples of the interval in
    // (spos, spos + len]; each is a chunk end, so the next one is tracked
    // instead of dividing per chunk.  snap_off: element offset of the next
    // snapshot's block for this head.
    int64_t snap_next = p.interval > 0 ? ((int64_t)spos / p.interval + 1) * p.interval : -1;
    int64_t snap_off = (sbase * H + h) * (int64_t)dk * dv;
    const int64_t snap_step = (int64_t)H * dk * dv;
    // operand block of the chunk after the current one (the last chunk
    // reloads itself, so the same loads are issued on every path; that data
    // is unused)
    const int64_t blk_step = (int64_t)H * CHUNK_OPS;
    const uint4* nptr = p.ops + ((cbase + min(1, nch - 1)) * H + h) * CHUNK_OPS;

    // A chunk's output tiles are stored during the next chunk, while that
    // chunk waits for its state rows from LDS (the last ones after the loop).
    // orsrc spans rows lo .. n-1 of the chunk: a row below lo gets an offset
    // that wraps past 2^32 - 1, so it falls outside too.
    f32x4 opend[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) opend[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(p.out, 0, 0, 0x00020000);
    uint32_t oshift = 0;
    auto store_out = [&]() {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (OUT_BF16)
                    __builtin_amdgcn_raw_buffer_store_b16(bfb(opend[t][e]), orsrc, ooff[e] - oshift,
                                                          16 * t * OB, 0);
                else
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(opend[t][e]), orsrc,
                                                          ooff[e] - oshift, 16 * t * OB, 0);
            }
    };
    // One value tile per workgroup (few, long recurrences): each chunk also
    // touches the operand block two chunks ahead, so that the register
    // prefetch one chunk ahead finds it in L2.  The head's 4 * tiles waves
    // each load one dword of every (4 * tiles)-th 128-byte line; the value is
    // consumed (by an empty asm statement) only a chunk later, after the next
    // such load was issued, so no wait is spent on it.  The two unrolled
    // chunk instances keep it in registers of their own (a copy would wait).
    uint32_t pfA = 0, pfB = 0;
    auto chunk = [&](const int ci, ScanOps<TPW>& o, ScanOps<TPW>& nx, uint32_t& pfo, uint32_t& pfn) {
        // chunk rows lo .. n-1 are tokens row0 + lo .. row0 + n - 1
        const int64_t row0 = seq0 - pad + (int64_t)ci * C;
        const int n = min(C, pad + len - ci * C);
        const int lo = ci == 0 ? pad : 0;
        const __amdgpu_buffer_rsrc_t nblk =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(nptr), 0, CHUNK_OPS * 16, 0x00020000);
        if (ci + 2 < nch) nptr += blk_step;

        // ---- publish this wave's state rows, per value tile: fp16 hi + lo
        // times 2^(F16_TOP - eS) with every |S| of the block below 2^eS ----
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            float mb = 0.f;
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e = 0; e < 4; ++e) mb = amax(mb, S[t][m][e]);
            const uint32_t sb = wave_max_u32(bits(mb));
            const int s = F16_TOP - bound_exp(sb);
            const f32x4 x0 = scl4(S[t][0], s), x1 = scl4(S[t][1], s);
            uint4 hh, ll;
            hsplit2(x0[0], x0[1], hh.x, ll.x);
            hsplit2(x0[2], x0[3], hh.y, ll.y);
            hsplit2(x1[0], x1[1], hh.z, ll.z);
            hsplit2(x1[2], x1[3], hh.w, ll.w);
            sm.sx[t][w][lane][0] = hh;
            sm.sx[t][w][lane][1] = ll;
            if (lane == 0) reinterpret_cast<uint8_t*>(&sm.se[t])[w] = exp_byte(sb);
        }
        if constexpr (DB) scan_load1(nx, nblk, w, tile0, vo, rot);
        lds_barrier();

        // the state rows of every block, then the exponent bytes, as one
        // batch of LDS reads (one round trip)
        uint4 Sh[TPW][4], Sl[TPW][4];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Sh[t][r] = sm.sx[t][(r + rot) & 3][lane][0];
                Sl[t][r] = sm.sx[t][(r + rot) & 3][lane][1];
            }

        // exponents of this chunk (scalar): the state-row blocks of each tile,
        // and the bound of U over each pair of token tiles (a K-step of the
        // state update): |U| <= |U~| + 128 max|W| max|S| < 2^bu[t][ks]
        const uint32_t xw = rot_bytes(uni(o.ex.x)), xq = rot_bytes(uni(o.ex.y)), xk = uni(o.ex.z),
                       xu = uni(o.ex4.x), xm = uni(o.ex4.y);
        // (esb and bub: the state-block and U exponents less 2 F16_TOP and the
        // byte bias, so that a factor's exponent is one raw byte plus one of them)
        int esb[TPW][4], bu[TPW][2], bub[TPW][2];
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const uint32_t sp = uni(sm.se[t]), spr = rot_bytes(sp);
#pragma unroll
            for (int r = 0; r < 4; ++r) esb[t][r] = byte_exp(spr, r) - 2 * F16_TOP - 126;
            const int esmax = bound_exp(max(max(sp & 0xffu, (sp >> 8) & 0xffu),
                                            max((sp >> 16) & 0xffu, sp >> 24)) << 23);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bu[t][ks] = 1 + max(max(byte_exp(xu, 2 * ks), byte_exp(xu, 2 * ks + 1)),
                                    7 + max(byte_exp(xm, 2 * ks), byte_exp(xm, 2 * ks + 1)) + esmax);
                bub[t][ks] = bu[t][ks] - 2 * F16_TOP - 126;
            }
        }

        // ---- this wave's token tile: U = U~ - W S, formed and published
        // first; Q' S (this wave's output products) goes on the matrix unit
        // after it -- with one value tile after barrier 2, while the reads of
        // U are in flight ----
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 pq[TPW][4];
        auto qs_products = [&]() {
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
#pragma unroll
                for (int r = 0; r < 4; ++r) pq[t][r] = mfma_h(o.q[r], Sh[t][r], z);
#pragma unroll
                for (int r = 0; r < 4; ++r) pq[t][r] = mfma_h(o.q[r], Sl[t][r], pq[t][r]);
            }
        };
        if (ci > 0) store_out();
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            f32x4 y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = mfma_h(o.w[r], Sh[t][r], z);
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = mfma_h(o.w[r], Sl[t][r], y[r]);
            const int sh = t >> 1;  // this tile's pair: its block order (see rot)
            f32x4 ws = y[sh & 3] * pow2f(byte_raw(xw, sh & 3) + esb[t][sh & 3]);
#pragma unroll
            for (int r0 = 1; r0 < 4; ++r0) {
                const int r = (r0 + sh) & 3;
                const float f = pow2f(byte_raw(xw, r) + esb[t][r]);
#pragma unroll
                for (int e = 0; e < 4; ++e) ws[e] = __builtin_fmaf(y[r][e], f, ws[e]);
            }
            const float4 ut = o.u[t];
            const f32x4 u = scl4(f32x4{ut.x, ut.y, ut.z, ut.w} - ws, F16_TOP - bu[t][w >> 1]);
            uint2 uh, ul;
            hsplit4(u, uh, ul);
            sm.ux[t][w >> 1][lane].h[w & 1] = uh;
            sm.ux[t][w >> 1][lane].l[w & 1] = ul;
        }
        // two value tiles: the state operands of both are not kept across
        // barrier 2 (register budget)
        if constexpr (TPW != 1) qs_products();
        if constexpr (DB) scan_load2(nx, nblk, w, tile0, vo, rot);
        else scan_load1(nx, nblk, w, tile0, vo, rot);  // W, U~ and the exponents are consumed
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);

        // ---- the whole U: this wave's state rows, and this wave's output
        // tiles O = scale (Q' S + O~) while the products run ----
        f32x4 a[TPW][2][2];
        uint4 Uh[TPW][2], Ul[TPW][2];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const typename ScanSmem<TPW>::Ux x = sm.ux[t][ks][lane];
                Uh[t][ks] = make_uint4(x.h[0].x, x.h[0].y, x.h[1].x, x.h[1].y);
                Ul[t][ks] = make_uint4(x.l[0].x, x.l[0].y, x.l[1].x, x.l[1].y);
            }
        if constexpr (TPW == 1) qs_products();
#pragma unroll
        for (int t = 0; t < TPW; ++t) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) a[t][m][ks] = mfma_h(o.kd[m][ks], Uh[t][ks], z);
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) a[t][m][ks] = mfma_h(o.kd[m][ks], Ul[t][ks], a[t][m][ks]);
        }
        if constexpr (DB) scan_load3(nx, nblk, w, vo, vd);
        if constexpr (TPW == 1) {
            const int ns = 4 * ngroups, si = (pos % ngroups) * 4 + w;
            const __amdgpu_buffer_rsrc_t pb = scan_block(p, cbase + min(ci + 2, nch - 1), h);
            const int line = min(si + lane * ns, (CHUNK_OPS * 16 - 1) / 128);
            pfn = __builtin_amdgcn_raw_buffer_load_b32(pb, line * 128, 0, 0);
            asm volatile("" :: "v"(pfo));
        }

#pragma unroll
        for (int t = 0; t < TPW; ++t) {
            const int sh = t >> 1;
            f32x4 po = pq[t][sh & 3] * pow2f(byte_raw(xq, sh & 3) + esb[t][sh & 3]);
#pragma unroll
            for (int r0 = 1; r0 < 4; ++r0) {
                const int r = (r0 + sh) & 3;
                const float f = pow2f(byte_raw(xq, r) + esb[t][r]);
#pragma unroll
                for (int e = 0; e < 4; ++e) po[e] = __builtin_fmaf(pq[t][r][e], f, po[e]);
            }
            const float4 ot = o.o[t];
            const float ob[4] = {ot.x, ot.y, ot.z, ot.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) opend[t][e] = p.scale * (po[e] + ob[e]);
        }
        orsrc = __builtin_amdgcn_make_buffer_rsrc(static_cast<char*>(p.out) + (row0 + lo) * orow * OB, 0,
                                                  (int)((int64_t)(n - lo) * orow * OB), 0x00020000);
        oshift = (uint32_t)((int64_t)lo * orow * OB);

        // S <- Diag(e^{G_C}) S + (K e^{G_C - G})^T U
#pragma unroll
        for (int t = 0; t < TPW; ++t)
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const float4 d = o.dec[m];
                f32x4 sv = S[t][m] * f32x4{d.x, d.y, d.z, d.w};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const float f = pow2f(byte_raw(xk, 2 * m + ks) + bub[t][ks]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) sv[e] = __builtin_fmaf(a[t][m][ks][e], f, sv[e]);
                }
                S[t][m] = sv;
            }
        if constexpr (!DB) {  // Q', O~, Kd and e^{G_C} are consumed
            scan_load2(nx, nblk, w, tile0, vo, rot);
            scan_load3(nx, nblk, w, vo, vd);
        }

        // absolute position reached
        if ((int64_t)spos - pad + (int64_t)ci * C + n == snap_next) {
            float* __restrict__ dsts = p.snapshots + snap_off;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = SL * w + 8 * g4 + 4 * m + e;
                        if (c < dk) dsts[(int64_t)c * dv + j0 + 16 * t] = S[t][m][e];
                    }
            snap_off += snap_step;
            snap_next += p.interval;
        }
    };

    // DB: the loop body always runs both halves, so the back edge is reached
    // only after the second half has consumed what the first half loaded;
    // an odd last chunk runs after the loop.
    int ci = 0;
    if constexpr (DB) {
        for (; ci + 1 < nch; ci += 2) {
            chunk(ci, opA, opB, pfA, pfB);
            chunk(ci + 1, opB, opA, pfB, pfA);
        }
        if (ci < nch) chunk(ci, opA, opB, pfA, pfB);
    } else {
        (void)opB;
        for (; ci < nch; ++ci) chunk(ci, opA, opA, pfA, pfA);
    }
    if constexpr (TPW == 1) asm volatile("" :: "v"(pfA), "v"(pfB));
    if (nch > 0) store_out();

#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = SL * w + 8 * g4 + 4 * m + e;
                if (c < dk) p.final_state[(srow + c) * dv + j0 + 16 * t] = S[t][m][e];
            }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
    size_t chunk_start, snap_base, order, ops, total;
};

WsLayout ws_layout(int H, int num_seqs, int64_t max_chunks) {
    WsLayout l;
    const size_t idx = align_up((size_t)(num_seqs + 1) * 4, 256);
    l.chunk_start = 0;
    l.snap_base = idx;
    l.order = 2 * idx;
    l.ops = 3 * idx;
    l.total = l.ops + (size_t)max_chunks * H * CHUNK_OPS * sizeof(uint4);
    return l;
}

template <typename TIn>
hipError_t launch_t(const PrefillArgs& a) {
    const WsLayout l = ws_layout(a.H, a.num_seqs, a.total_chunks);
    char* ws = static_cast<char*>(a.workspace);
    int32_t* chunk_start = reinterpret_cast<int32_t*>(ws + l.chunk_start);
    int32_t* snap_base = reinterpret_cast<int32_t*>(ws + l.snap_base);
    int32_t* order = reinterpret_cast<int32_t*>(ws + l.order);
    uint4* ops = reinterpret_cast<uint4*>(ws + l.ops);

    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(NT), 0, a.stream, a.cu_dev, a.start_dev,
                       a.num_seqs, a.interval, chunk_start, snap_base, order);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    if (a.total_chunks > 0) {
        PrepParams pp{};
        pp.q = a.q;
        pp.k = a.k;
        pp.v = a.v;
        pp.g = a.g;
        pp.beta = a.beta;
        pp.cu = a.cu_dev;
        pp.start = a.start_dev;
        pp.chunk_start = chunk_start;
        pp.ops = ops;
        pp.H = a.H;
        pp.dk = a.dk;
        pp.dv = a.dv;
        pp.num_seqs = a.num_seqs;
        const int64_t items = a.total_chunks * a.H;
        hipLaunchKernelGGL((prep_kernel<TIn>), dim3((unsigned)items), dim3(NT), 0, a.stream, pp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }

    ScanParams sp{};
    sp.cu = a.cu_dev;
    sp.start = a.start_dev;
    sp.slots = a.slots;
    sp.chunk_start = chunk_start;
    sp.snap_base = snap_base;
    sp.order = order;
    sp.ops = ops;
    sp.init = a.init;
    sp.init_if_started = a.init_if_started ? 1 : 0;
    sp.out = a.out;
    sp.final_state = a.final_state;
    sp.snapshots = a.snapshots;
    sp.interval = a.interval;
    sp.H = a.H;
    sp.dk = a.dk;
    sp.dv = a.dv;
    sp.scale = a.scale;
    sp.nchains = a.num_seqs * a.H;
    // the value-tile width: one 16-column tile per workgroup while that
    // leaves fewer than two workgroups per compute unit (few, long
    // recurrences: every unit runs one latency-bound chain and the
    // double-buffered prefetch hides the loads); with more chains, two tiles
    // per workgroup, and four once that still leaves two workgroups per unit
    // (W, Q' and Kd loaded once for 32 or 64 columns)
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const int tiles = a.dv / 16;
    const int64_t ntile = ((int64_t)sp.nchains + 7) / 8 * 8 * tiles;
    const int tpw = (tiles % 4 == 0 && ntile >= 8 * (int64_t)cus) ? 4
                    : (tiles % 2 == 0 && ntile >= 2 * (int64_t)cus) ? 2 : 1;
    sp.ngroups = tiles / tpw;
    const int64_t nwg = ((int64_t)sp.nchains + 7) / 8 * 8 * sp.ngroups;
    auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3((unsigned)nwg), dim3(NT), 0, a.stream, sp); };
    if (a.out_bf16) {
        if (tpw == 4) go(scan_kernel<true, true, 4>);
        else if (tpw == 2) go(scan_kernel<true, true, 2>);
        else go(scan_kernel<true, true, 1>);
    } else {
        if (tpw == 4) go(scan_kernel<false, true, 4>);
        else if (tpw == 2) go(scan_kernel<false, true, 2>);
        else go(scan_kernel<false, true, 1>);
    }
    return hipGetLastError();
}

}  // namespace

int64_t prefill_max_chunks(int num_seqs, int64_t total_tokens, bool any_start) {
    // sum_b ceil(L_b / C) <= floor(T / C) + num_seqs; a leading partial chunk
    // (a start position off the chunk grid) adds at most one more per sequence
    return total_tokens / C + (int64_t)num_seqs * (any_start ? 2 : 1);
}

int prefill_chunk_rows() { return C; }

size_t prefill_workspace_bytes(int, int, int H, int num_seqs, int64_t total_tokens, bool any_start) {
    return ws_layout(H, num_seqs, prefill_max_chunks(num_seqs, total_tokens, any_start)).total;
}

hipError_t launch_prefill(const PrefillArgs& a) {
    if (a.dk > DKP || a.dv > DVP || a.dv % 16 != 0) return hipErrorInvalidValue;
    // the host API rejects these before calling; nothing has been launched yet
    if (((int64_t)a.num_seqs * a.H + 7) / 8 * 8 * (a.dv / 16) > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.total_chunks * a.H > 0x7fffffffLL) return hipErrorInvalidValue;
    return a.in_bf16 ? launch_t<bf16_t>(a) : launch_t<float>(a);
}

}  // namespace kda
