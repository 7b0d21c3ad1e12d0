// Quantisation of one token-head into the packed cache, shared by the store
// kernel and the fused store + verify kernel.
//
// Method (Context and Part 6 of "Speculative decoding on Intel Arc:
// TurboQuant KV + a fused N_spec kernel"): keys are rotated by a
// Walsh-Hadamard transform and coded with a precomputed Lloyd-Max codebook
// plus a norm correction (k3v4_nc with 8 levels, k4v4_nc with 16: the
// method's 3-4 bits per coordinate, TL;DR), or kept as FP8 E4M3 codes (k8v4);
// values get uniform 4-bit codes with a scale and a zero.
//
// One wavefront quantises one token-head (128 coordinates): lane l holds
// coordinates l and l + 64, so the last WHT stage and the first step of the
// stride-halving sum are in-lane and every other step is an xor-shuffle.
// IEEE add is commutative, so the xor-butterfly reductions reproduce the
// stride-halving tree bit for bit, and the WHT butterflies take the same
// operands in the same stage order h = 1, 2, ..., 64 as the specification.
// All arithmetic is binary32 with explicit round-to-nearest-even intrinsics
// (no contraction), because the codes are integers decided in binary32 and
// must be bit-exact.
#pragma once
#include "codebook.h"
#include "common.h"

namespace tqkv {
namespace quant {

__device__ inline float h2f_q(uint16_t h) { return __half2float(__ushort_as_half(h)); }

// Correctly rounded binary32 square root (llvm.sqrt.f32 is lowered to
// v_sqrt_f32 plus a one-ulp residual correction; HIP's __fsqrt_rn maps to the
// uncorrected native instruction).
__device__ inline float sqrt_rn(float x) { return __builtin_sqrtf(x); }

// binary32 -> binary16 bits, RNE; NaN becomes the canonical 0x7E00.
__device__ inline uint16_t f2h(float f)
{
    if (f != f)
        return 0x7E00;
    return __half_as_ushort(__float2half_rn(f));
}

// Lloyd-Max cells by binary search over the sorted thresholds: the cell is
// #{j : y >= tau_j} either way (a NaN compares false at every step and lands
// in cell 0), in three comparisons for 8 levels and four for 16 instead of
// seven and fifteen.  Thresholds and levels come from lane tables through
// ds_bpermute (lane l holds tau_(l % 16), and level l % 8 or, for 16 levels,
// the magnitude |c16_(8 + l % 8)|); the probe moves by integer steps, so
// there is no select of floating-point constants (the compiler turned
// nested ones into branches) and no register per constant.
template <int NL> __device__ inline uint32_t threshold_lane_table(int lane)
{
    const int k = lane & 15;
    float v = 0.0f;
#pragma unroll
    for (int j = 0; j < NL - 1; ++j)
        if (k == j)
            v = (NL == 8) ? kThreshold[j] : kThreshold16[j];
    return __float_as_uint(v);
}
template <int NL> __device__ inline uint32_t level_lane_table(int lane)
{
    const int k = lane & 7;
    float v = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (k == j)
            v = (NL == 8) ? kCentroid[j] : kCentroid16[8 + j];
    return __float_as_uint(v);
}
// entry byte_idx / 4 of a lane table
__device__ inline float lane_table_at(uint32_t tab, int byte_idx)
{
    return __uint_as_float((uint32_t)__builtin_amdgcn_ds_bpermute(byte_idx, (int)tab));
}
__device__ inline int lloyd_cell8(float y, uint32_t ttab)
{
    const bool b2 = y >= kThreshold[3];
    int i = b2 ? 4 * 5 : 4 * 1; // tau_(4 b2 + 1)
    const bool b1 = y >= lane_table_at(ttab, i);
    i += b1 ? 4 : -4; // tau_(2k), k = 2 b2 + b1: the cell pair {2k, 2k + 1}
    const bool b0 = y >= lane_table_at(ttab, i);
    return (i >> 2) + (b0 ? 1 : 0);
}
// m: the rank of |c16_c| from zero (c - 8 for c >= 8, 7 - c below: the
// three low bits of c, inverted when bit 3 is clear, since the codebook is
// symmetric)
__device__ inline int lloyd_cell16(float y, uint32_t ttab, int &m)
{
    const bool b3 = y >= kThreshold16[7];
    int i = b3 ? 4 * 11 : 4 * 3; // tau_(8 b3 + 3)
    const bool b2 = y >= lane_table_at(ttab, i);
    i += b2 ? 8 : -8; // tau_(8 b3 + 4 b2 + 1)
    const bool b1 = y >= lane_table_at(ttab, i);
    i += b1 ? 4 : -4; // tau_(2k), k = 4 b3 + 2 b2 + b1: the cell pair {2k, 2k + 1}
    const bool b0 = y >= lane_table_at(ttab, i);
    const int c = (i >> 2) + (b0 ? 1 : 0);
    m = (c & 7) ^ (b3 ? 0 : 7);
    return c;
}

// Stored k4v4_nc key nibble of code c: sign-magnitude, bit 3 set for the
// negative levels (c < 8), bits 0-2 the rank of |c16_c| from zero.
__device__ inline uint32_t k4_nibble(int c) { return (uint32_t)((c >= 8) ? c - 8 : 15 - c); }

// x from lane (lane ^ S) of the wavefront, S = 1, 2, ..., 32, without the
// LDS crossbar: DPP moves within rows of 16 lanes (xor 1, 2: quad
// permutations; xor 4: half-row mirror then quad reversal; xor 8: row
// rotation by 8) and lane-swap instructions across rows (xor 16, 32).
template <int S> __device__ inline uint32_t lane_xor(uint32_t x, int lane)
{
    static_assert(S == 1 || S == 2 || S == 4 || S == 8 || S == 16 || S == 32, "xor distance");
    if constexpr (S == 1) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false); // quad_perm [1,0,3,2]
    } else if constexpr (S == 2) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false); // quad_perm [2,3,0,1]
    } else if constexpr (S == 4) {
        const int m = __builtin_amdgcn_mov_dpp((int)x, 0x141, 0xF, 0xF, false); // row_half_mirror: i -> 7 - i
        return (uint32_t)__builtin_amdgcn_mov_dpp(m, 0x1B, 0xF, 0xF, false);     // quad_perm [3,2,1,0]
    } else if constexpr (S == 8) {
        return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xF, 0xF, false); // row_ror:8
    } else if constexpr (S == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return (lane & 16) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return (lane & 32) ? r[0] : r[1];
    }
}
template <int S> __device__ inline float lane_xor(float x, int lane)
{
    return __uint_as_float(lane_xor<S>(__float_as_uint(x), lane));
}
// runtime distance (unrolled loops pass compile-time values; the switch folds)
template <typename T> __device__ inline T lane_xor_n(T x, int s, int lane)
{
    switch (s) {
    case 1: return lane_xor<1>(x, lane);
    case 2: return lane_xor<2>(x, lane);
    case 4: return lane_xor<4>(x, lane);
    case 8: return lane_xor<8>(x, lane);
    case 16: return lane_xor<16>(x, lane);
    default: return lane_xor<32>(x, lane);
    }
}

// Sum over the wavefront of one value per lane by xor-butterflies 32..1.
__device__ inline float wave_tree_sum(float a, int lane)
{
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1)
        a = __fadd_rn(a, lane_xor_n(a, s, lane));
    return a;
}

// OCP E4M3 code of binary32 q (round to nearest even, saturation to +-448,
// NaN -> 0x7F; the encoding of the FP8 keys), without branches: in the
// normal range the bit pattern is rounded at bit 20 (ties to even) and the
// exponent rebiased by 127 - 7; below 2^-6 the code is rint(|q| * 2^9).
__device__ inline uint32_t e4m3_code(float q)
{
    const uint32_t u = __float_as_uint(q), a = u & 0x7FFFFFFFu;
    const uint32_t rn = (a + 0x7FFFFu + ((a >> 20) & 1u) - (120u << 23)) >> 20;
    const uint32_t cn = rn < 0x7Eu ? rn : 0x7Eu;
    const uint32_t cs = (uint32_t)rintf(__fmul_rn(__uint_as_float(a), 512.0f));
    const uint32_t c = (a < 0x3C800000u) ? cs : cn;
    return (a > 0x7F800000u) ? 0x7Fu : (((u >> 24) & 0x80u) | c);
}

// q = x * (1 / s) (two roundings) is within 2^-23 |x / s| of the correctly
// rounded quotient, i.e. two units in its last place: its E4M3 code can
// differ from the quotient's only where q lies that close to a rounding
// boundary: the 20 discarded bits near 0x80000 (normal range), |q| * 2^9
// near a half-integer (below 2^-6; a 2^-20 error there).  The margins are
// 4 units and 2^-16.
__device__ inline bool e4m3_near_boundary(float q)
{
    const uint32_t a = __float_as_uint(q) & 0x7FFFFFFFu;
    const float t = __fmul_rn(__uint_as_float(a), 512.0f);
    const bool sub = fabsf(t - rintf(t)) > 0.5f - 0x1p-16f;
    const bool nrm = ((a & 0xFFFFFu) - 0x7FFFCu) < 9u;
    return (a < 0x3C800000u) ? sub : nrm;
}

// Value codes clamp(rint(a / s), 0, 15) with a / s the correctly rounded
// binary32 quotient (s > 0).  The product a * (1 / s) of two roundings
// differs from that quotient by under 3e-6 for |a / s| <= 16, so where no
// integer + 1/2 lies within 4e-6 of it both round to the same integer;
// near such a point (rarely) the exact division decides, for the whole
// wavefront at once.  The test reuses the rounding: q is within 4e-6 of a
// half-integer exactly when |q - rint(q)| (an exact difference) exceeds
// 1/2 - 4e-6.  Outside [-0.5, 15.5] the clamp decides either way.
__device__ inline bool code_near_tie(float q, float r) { return fabsf(q - r) > 0.5f - 4e-6f; }
// clamp to [0, 15] of an integral value; NaN -> 0 (fmaxf returns the number)
__device__ inline uint32_t code_clamp(float r) { return (uint32_t)fminf(fmaxf(r, 0.0f), 15.0f); }

// One token-head's inputs as this lane holds them: coordinates lane and
// lane + 64 of the key and of the value (fp16 bit patterns).
// (Held as 32-bit words: four 16-bit fields were packed into two registers
// right after the loads, which made the wavefront wait for them there.)
struct TokenHead {
    uint32_t k0, k1, v0, v1;
};

__device__ inline TokenHead load_token_head(const uint16_t *kp, const uint16_t *vp, int lane)
{
    return TokenHead{kp[lane], kp[lane + 64], vp[lane], vp[lane + 64]};
}

// The quantised record of one token-head, as this lane holds it before the
// stores: 3-bit key code words (k3v4_nc), two key nibble dwords (k4v4_nc)
// or this lane's two FP8 codes (k8v4), the key metadata, this lane's value
// byte and the value scale / zero.  Splitting computation from stores lets
// two token-heads' dependent exchange chains run interleaved.
struct Record {
    uint32_t kw[2][3];  // k3v4_nc: the key code words of this lane's triple (both halves);
                        // k4v4_nc: kw[hh][0] = key dword 8hh + lane / 8
    uint32_t c0, c1;    // k8v4: FP8 codes of coordinates lane, lane + 64
    uint16_t m0, m1;    // k3v4_nc, k4v4_nc: n, gamma; k8v4: key scale
    uint16_t sch, zh;   // value scale, zero
    uint32_t vbyte;     // this lane's value nibble byte
    int vpos;           // ... and its byte index p (coordinates 2p, 2p + 1)
};

// Quantise a loaded token-head (registers only).  Called by all 64 lanes of
// one wavefront.
template <int PRESET>
__device__ inline Record quantize_record(const TokenHead &in, int lane)
{
    Record r;
    // ---------------------------------------------------------------- keys
    float x0 = h2f_q((uint16_t)in.k0), x1 = h2f_q((uint16_t)in.k1);
    if constexpr (kLloydMax<PRESET>) {
        const float n = sqrt_rn(wave_tree_sum(__fadd_rn(__fmul_rn(x0, x0), __fmul_rn(x1, x1)), lane));
#pragma unroll
        for (int h = 1; h < 64; h <<= 1) {
            float p0 = lane_xor_n(x0, h, lane), p1 = lane_xor_n(x1, h, lane);
            if (lane & h) {
                x0 = __fsub_rn(p0, x0);
                x1 = __fsub_rn(p1, x1);
            } else {
                x0 = __fadd_rn(x0, p0);
                x1 = __fadd_rn(x1, p1);
            }
        }
        {
            float u = x0, v = x1;
            x0 = __fadd_rn(u, v);
            x1 = __fsub_rn(u, v);
        }
        const float rr = __fdiv_rn(1.0f, __fmul_rn(sqrt_rn(128.0f), n));
        const float y0 = __fmul_rn(x0, rr), y1 = __fmul_rn(x1, rr);
        constexpr int NL = (PRESET == kPresetK3V4) ? 8 : 16;
        const uint32_t ttab = threshold_lane_table<NL>(lane), ltab = level_lane_table<NL>(lane);
        int c0, c1;
        float q0, q1;
        if constexpr (PRESET == kPresetK3V4) {
            c0 = lloyd_cell8(y0, ttab);
            c1 = lloyd_cell8(y1, ttab);
            q0 = lane_table_at(ltab, 4 * c0);
            q1 = lane_table_at(ltab, 4 * c1);
        } else {
            int m0, m1;
            c0 = lloyd_cell16(y0, ttab, m0);
            c1 = lloyd_cell16(y1, ttab, m1);
            q0 = lane_table_at(ltab, 4 * m0);
            q1 = lane_table_at(ltab, 4 * m1);
        }
        const float gam = __fdiv_rn(1.0f, sqrt_rn(wave_tree_sum(__fadd_rn(__fmul_rn(q0, q0), __fmul_rn(q1, q1)), lane)));
        r.m0 = f2h(n);
        r.m1 = f2h(gam);
        r.c0 = r.c1 = 0u;
        if constexpr (PRESET == kPresetK4V4) {
            // coordinate d = 8j + e -> key dword j, byte e % 4, nibble e / 4;
            // lane l carries d = l (dword l / 8) and d = l + 64 (dword 8 +
            // l / 8); the 8 lanes of a dword OR their nibbles together
            const int sh = 8 * (lane & 3) + 4 * ((lane >> 2) & 1);
            uint32_t w0 = k4_nibble(c0) << sh, w1 = k4_nibble(c1) << sh;
#pragma unroll
            for (int s = 1; s < 8; s <<= 1) {
                w0 |= lane_xor_n(w0, s, lane);
                w1 |= lane_xor_n(w1, s, lane);
            }
            r.kw[0][0] = w0;
            r.kw[1][0] = w1;
            r.kw[0][1] = r.kw[0][2] = r.kw[1][1] = r.kw[1][2] = 0u;
        } else {
            // Bit placement: coordinate d = 64h + 32g + 8k + e -> dword triple
            // 6h+3g+{0,1,2}, byte lane e%4, slot 2k + e/4.  Slots 0-5 hold all
            // three bits at word slot/2, offset 3*(slot%2); slots 6 and 7 keep
            // bits 0-1 at offset 6 of word slot-6 and bit 2 at offset slot of
            // word 2.  Lane l carries d = l (h = 0) and d = l + 64 (h = 1), both
            // in triple g = l/32 of their half.
            uint32_t w[2][3] = {{0, 0, 0}, {0, 0, 0}};
            {
                const int k = (lane >> 3) & 3, e = lane & 7;
                const int sl = 2 * k + (e >> 2), sh = 8 * (e & 3);
                const uint32_t cc[2] = {(uint32_t)c0, (uint32_t)c1};
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    if (sl < 6) {
                        w[hh][sl >> 1] |= cc[hh] << (sh + 3 * (sl & 1));
                    } else {
                        w[hh][sl - 6] |= (cc[hh] & 3u) << (sh + 6);
                        w[hh][2] |= (cc[hh] >> 2) << (sh + sl);
                    }
                }
            }
#pragma unroll
            for (int s = 1; s < 32; s <<= 1)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int j = 0; j < 3; ++j)
                        w[hh][j] |= lane_xor_n(w[hh][j], s, lane);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    r.kw[hh][j] = w[hh][j];
        }
    } else {
        float amax = fmaxf(fmaxf(0.0f, fabsf(x0)), fabsf(x1));
#pragma unroll
        for (int s = 32; s >= 1; s >>= 1)
            amax = fmaxf(amax, lane_xor_n(amax, s, lane));
        const uint16_t sh = f2h(__fdiv_rn(amax, 448.0f));
        const float sc = h2f_q(sh);
        // codes of x / s from the product with 1 / s, the exact division
        // where the product lies near a rounding boundary
        const float rsc = __fdiv_rn(1.0f, sc);
        const float p0 = __fmul_rn(x0, rsc), p1 = __fmul_rn(x1, rsc);
        uint32_t k0 = e4m3_code(p0), k1 = e4m3_code(p1);
        if (__builtin_expect(__any(e4m3_near_boundary(p0) || e4m3_near_boundary(p1)), 0)) {
            if (e4m3_near_boundary(p0))
                k0 = e4m3_code(__fdiv_rn(x0, sc));
            if (e4m3_near_boundary(p1))
                k1 = e4m3_code(__fdiv_rn(x1, sc));
        }
        r.c0 = (sc == 0.0f) ? 0u : k0;
        r.c1 = (sc == 0.0f) ? 0u : k1;
        r.m0 = sh;
        r.m1 = 0;
    }

    // -------------------------------------------------------------- values
    const float v0 = h2f_q((uint16_t)in.v0), v1 = h2f_q((uint16_t)in.v1);
    float mn = fminf(fminf(__int_as_float(0x7F800000), v0), v1);
    float mx = fmaxf(fmaxf(__int_as_float(0xFF800000), v0), v1);
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        mn = fminf(mn, lane_xor_n(mn, s, lane));
        mx = fmaxf(mx, lane_xor_n(mx, s, lane));
    }
    const uint16_t zh = f2h(__fadd_rn(mn, 0.0f)); // -0 -> +0
    const float zero = h2f_q(zh);
    const uint16_t sch = f2h(__fdiv_rn(__fsub_rn(mx, mn), 15.0f));
    const float sc = h2f_q(sch);
    // codes clamp(rint((v - zero) / s), 0, 15): the product with 1 / s, the
    // exact division near a tie
    const float rs = __fdiv_rn(1.0f, sc);
    const float g0 = __fmul_rn(__fsub_rn(v0, zero), rs), g1 = __fmul_rn(__fsub_rn(v1, zero), rs);
    float r0 = rintf(g0), r1 = rintf(g1);
    if (__builtin_expect(__any(code_near_tie(g0, r0) || code_near_tie(g1, r1)), 0)) {
        if (code_near_tie(g0, r0))
            r0 = rintf(__fdiv_rn(__fsub_rn(v0, zero), sc));
        if (code_near_tie(g1, r1))
            r1 = rintf(__fdiv_rn(__fsub_rn(v1, zero), sc));
    }
    const uint32_t vc0 = (sc == 0.0f) ? 0u : code_clamp(r0), vc1 = (sc == 0.0f) ? 0u : code_clamp(r1);
    const uint32_t o0 = lane_xor<1>(vc0, lane), o1 = lane_xor<1>(vc1, lane);
    // even lane: byte l/2 = (d=l | d=l+1); odd lane: byte 32 + l/2 = (d=l+63 | d=l+64)
    r.vpos = (lane & 1) ? (32 + (lane >> 1)) : (lane >> 1);
    r.vbyte = (lane & 1) ? (o1 | (vc1 << 4)) : (vc0 | (o0 << 4));
    r.sch = sch;
    r.zh = zh;
    return r;
}

// Write a record into token slot tb of the 16-token cache block blk (all 64
// lanes of the wavefront that computed it).
template <int PRESET>
__device__ inline void store_record(uint8_t *blk, int tb, const Record &r, int lane)
{
    using L = Layout<PRESET>;
    if constexpr (PRESET == kPresetK3V4) {
        if ((lane & 31) == 0) {
            const int g = lane >> 5;
            uint32_t *kd = reinterpret_cast<uint32_t *>(blk + tb * L::kKeyBytesPerToken);
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                kd[3 * g + j] = r.kw[0][j];
                kd[6 + 3 * g + j] = r.kw[1][j];
            }
        }
        if (lane == 0)
            *reinterpret_cast<uint16_t *>(blk + L::kMeta0 + 2 * tb) = r.m0;
        if (lane == 1)
            *reinterpret_cast<uint16_t *>(blk + L::kMeta1 + 2 * tb) = r.m1;
    } else if constexpr (PRESET == kPresetK4V4) {
        if ((lane & 7) == 0) {
            uint32_t *kd = reinterpret_cast<uint32_t *>(blk + tb * L::kKeyBytesPerToken);
            kd[lane >> 3] = r.kw[0][0];
            kd[8 + (lane >> 3)] = r.kw[1][0];
        }
        if (lane == 0)
            *reinterpret_cast<uint16_t *>(blk + L::kMeta0 + 2 * tb) = r.m0;
        if (lane == 1)
            *reinterpret_cast<uint16_t *>(blk + L::kMeta1 + 2 * tb) = r.m1;
    } else {
        uint8_t *kd = blk + tb * L::kKeyBytesPerToken;
        kd[lane] = (uint8_t)r.c0;
        kd[lane + 64] = (uint8_t)r.c1;
        if (lane == 0)
            *reinterpret_cast<uint16_t *>(blk + L::kMeta0 + 2 * tb) = r.m0;
    }
    blk[L::kValOff + val_byte_offset(tb, r.vpos)] = (uint8_t)r.vbyte;
    if (lane == 2)
        *reinterpret_cast<uint16_t *>(blk + L::kVScale + 2 * tb) = r.sch;
    if (lane == 3)
        *reinterpret_cast<uint16_t *>(blk + L::kVZero + 2 * tb) = r.zh;
}

// Quantise a loaded token-head into token slot tb of the 16-token cache
// block blk.  Called by all 64 lanes of one wavefront.
template <int PRESET>
__device__ inline void quantize_token_head(uint8_t *blk, int tb, const TokenHead &in, int lane)
{
    store_record<PRESET>(blk, tb, quantize_record<PRESET>(in, lane), lane);
}

} // namespace quant
} // namespace tqkv
