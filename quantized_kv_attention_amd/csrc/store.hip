// Store kernel: quantise new K/V token-heads into the packed cache.
//
// Method (Context and Part 6 of "Speculative decoding on Intel Arc:
// TurboQuant KV + a fused N_spec kernel"): keys are rotated by a
// Walsh-Hadamard transform and coded with a precomputed Lloyd-Max codebook
// plus a norm correction (k3v4_nc with 8 levels, k4v4_nc with 16), or kept as
// FP8 E4M3 codes with a per-token scale (k8v4); values get uniform 4-bit
// codes with a scale and a zero.  Every code and metadata bit is the one the
// binary32 definition gives (no contraction, correctly rounded square root
// and division, the stride-halving order of the two sums of squares).
//
// Eight lanes quantise one token-head, eight token-heads per wavefront.
// Lane j of a group holds key coordinates j + 8m (m = 0..15): the first four
// steps of each stride-halving sum and the last four butterfly stages of
// the WHT (h = 8..64) stay inside the lane, and the rest are xor-exchanges
// within the 8-lane group (DPP, no LDS).  Values are held contiguously
// (coordinates 16j .. 16j + 15).  With one token-head per wavefront (the
// layout of the fused store inside the verify kernel, quant.h) most of the
// instructions were lane exchanges: about 750 vector instructions per
// token-head against about a hundred here.
#include "quant.h"

namespace tqkv {
namespace {

constexpr int kGroup = 8;   // lanes per token-head
constexpr int kPer = 16;    // key (and value) coordinates per lane
constexpr int kStoreThreads = 256;

// x from lane (lane ^ S) of the same 8-lane group
template <int S> __device__ inline float gxor(float x, int lane) { return quant::lane_xor<S>(x, lane); }
template <int S> __device__ inline uint32_t gxor(uint32_t x, int lane) { return quant::lane_xor<S>(x, lane); }

// Sum of squares of the token-head's 128 values by the stride-halving tree
// (a[i] += a[i + s] for i < s, s = 64 .. 1): the lane holds a[j + 8m], so
// strides 64..8 pair m with m + 8, 4, 2, 1 inside the lane and strides 4, 2,
// 1 pair lane j with j ^ 4, 2, 1 (IEEE addition is commutative, so each
// pair's sum is the same on both lanes).
__device__ inline float group_tree_sumsq(const float (&x)[kPer], int lane)
{
    float a[kPer];
#pragma unroll
    for (int m = 0; m < kPer; ++m)
        a[m] = __fmul_rn(x[m], x[m]);
#pragma unroll
    for (int s = kPer / 2; s >= 1; s >>= 1)
#pragma unroll
        for (int m = 0; m < s; ++m)
            a[m] = __fadd_rn(a[m], a[m + s]);
    float t = a[0];
    t = __fadd_rn(t, gxor<4>(t, lane));
    t = __fadd_rn(t, gxor<2>(t, lane));
    t = __fadd_rn(t, gxor<1>(t, lane));
    return t;
}

// Normalised-order (Sylvester) WHT of the token-head's key, unnormalised,
// stages h = 1, 2, ..., 64 in that order: at stage h the element with bit h
// clear becomes x + y, its partner x - y.  h = 1, 2, 4 pair lanes, h = 8..64
// pair m with m + h / 8 inside the lane.
__device__ inline void group_wht(float (&x)[kPer], int lane)
{
    const int j = lane & 7;
    // lane pairs: own + partner, or partner - own, as fma(+-1, own, partner)
    // (one rounding of an exact sum: the same value as the add or subtract)
    const float s1 = (j & 1) ? -1.0f : 1.0f, s2 = (j & 2) ? -1.0f : 1.0f, s4 = (j & 4) ? -1.0f : 1.0f;
#pragma unroll
    for (int m = 0; m < kPer; ++m)
        x[m] = __builtin_fmaf(s1, x[m], gxor<1>(x[m], lane));
#pragma unroll
    for (int m = 0; m < kPer; ++m)
        x[m] = __builtin_fmaf(s2, x[m], gxor<2>(x[m], lane));
#pragma unroll
    for (int m = 0; m < kPer; ++m)
        x[m] = __builtin_fmaf(s4, x[m], gxor<4>(x[m], lane));
#pragma unroll
    for (int hb = 1; hb < kPer; hb <<= 1)
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            if (!(m & hb)) {
                const float u = x[m], v = x[m + hb];
                x[m] = __fadd_rn(u, v);
                x[m + hb] = __fsub_rn(u, v);
            }
}

// 16 binary16 values (coordinates 16j .. 16j + 15 of a row) as 8 words
__device__ inline void load_run(uint32_t (&w)[kPer / 2], const uint16_t *p, bool aligned)
{
    if (aligned) { // rows are 256 B: every lane's 32 B aligned
        const uint4 *p4 = reinterpret_cast<const uint4 *>(p);
        const uint4 lo = p4[0], hi = p4[1];
        w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
        w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
    } else {
#pragma unroll
        for (int i = 0; i < kPer / 2; ++i)
            w[i] = (uint32_t)p[2 * i] | ((uint32_t)p[2 * i + 1] << 16);
    }
}

template <int PRESET>
__global__ __launch_bounds__(kStoreThreads) void store_kernel(StoreArgs a)
{
    using L = Layout<PRESET>;
    const int lane = threadIdx.x & 63, j = lane & 7;
    // group index -> (16-token chunk, head, token in chunk): the sixteen
    // consecutive tokens of one head (normally one cache block) are
    // quantised by two neighbouring wavefronts, so each block's lines are
    // written in full at about the same time
    // (32-bit index arithmetic: at most 2^31 / 4 * 16 / 16 chunk-heads, the
    // limit the host checks on T * Hk)
    const uint32_t gi = blockIdx.x * (kStoreThreads / kGroup) + (threadIdx.x >> 3);
    const uint32_t rest = gi >> 4;
    const int hk = (int)(rest % (uint32_t)a.Hk);
    const long t_raw = (long)(rest / (uint32_t)a.Hk) * 16 + (gi & 15);
    const bool live = t_raw < a.T;
    const int t = live ? (int)t_raw : 0; // groups past the last token compute on token 0, store nothing
    const long th = (long)t * a.Hk + hk;

    // destination block and token slot (nullptr: skipped)
    uint8_t *blk = nullptr;
    int tb = 0;
    if (live) {
        if (a.step_lens) {
            const int n = t / a.B, b = t - n * a.B;
            const int Lr = a.step_lens[b];
            const int Ls = Lr < 0 ? 0 : (Lr > a.max_seq ? a.max_seq : Lr);
            const int p = Ls - a.N + n;
            if (p >= 0) { // a sequence shorter than the step skips it
                if (a.btab) {
                    const int pg = a.btab[(size_t)b * a.bstride + (p >> 4)];
                    if (pg >= 0 && pg < a.npages)
                        blk = a.base + ((size_t)pg * a.Hk + hk) * L::kBlockBytes;
                } else {
                    blk = a.base + ((size_t)(b * a.Hk + hk) * a.nblk + (p >> 4)) * L::kBlockBytes;
                }
                tb = p & 15;
            }
        } else if (a.slots) {
            // paged: slot = page * 16 + position in the page; head hk's
            // block of page p is block p * Hk + hk of the pool
            const int sl = a.slots[t];
            if (sl >= 0 && (sl >> 4) < a.npages) {
                blk = a.base + ((size_t)(sl >> 4) * a.Hk + hk) * L::kBlockBytes;
                tb = sl & 15;
            }
        } else {
            const int b = a.seq_idx[t], p = a.pos[t];
            if (b >= 0 && b < a.B && p >= 0 && p < a.max_seq) {
                blk = a.base + ((size_t)(b * a.Hk + hk) * a.nblk + (p >> 4)) * L::kBlockBytes;
                tb = p & 15;
            }
        }
    }

    // ---------------------------------------------------------------- loads
    const uint16_t *kp = a.K + (size_t)th * kD;
    const uint16_t *vp = a.V + (size_t)th * kD;
    // Lloyd-Max keys: coordinates j + 8m (the WHT and sum layout above);
    // FP8 keys and values: coordinates 16j .. 16j + 15
    float x[kPer];
    if constexpr (kLloydMax<PRESET>) {
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            x[m] = quant::h2f_q(kp[j + 8 * m]);
    } else {
        uint32_t kw[kPer / 2];
        load_run(kw, kp + kPer * j, (reinterpret_cast<uintptr_t>(a.K) & 15) == 0);
#pragma unroll
        for (int i = 0; i < kPer / 2; ++i) {
            x[2 * i] = quant::h2f_q((uint16_t)(kw[i] & 0xFFFFu));
            x[2 * i + 1] = quant::h2f_q((uint16_t)(kw[i] >> 16));
        }
    }
    uint32_t vw[kPer / 2];
    load_run(vw, vp + kPer * j, (reinterpret_cast<uintptr_t>(a.V) & 15) == 0);

    // ----------------------------------------------------------------- keys
    uint16_t m0 = 0, m1 = 0;
    if constexpr (kLloydMax<PRESET>) {
        const float n = quant::sqrt_rn(group_tree_sumsq(x, lane));
        group_wht(x, lane);
        const float rr = __fdiv_rn(1.0f, __fmul_rn(quant::sqrt_rn(128.0f), n));
        constexpr int NL = (PRESET == kPresetK3V4) ? 8 : 16;
        const uint32_t ttab = quant::threshold_lane_table<NL>(lane), ltab = quant::level_lane_table<NL>(lane);
        int c[kPer];
        float q[kPer];
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const float y = __fmul_rn(x[m], rr);
            if constexpr (PRESET == kPresetK3V4) {
                c[m] = quant::lloyd_cell8(y, ttab);
                q[m] = quant::lane_table_at(ltab, 4 * c[m]);
            } else {
                int r;
                c[m] = quant::lloyd_cell16(y, ttab, r);
                q[m] = quant::lane_table_at(ltab, 4 * r);
            }
        }
        const float gam = __fdiv_rn(1.0f, quant::sqrt_rn(group_tree_sumsq(q, lane)));
        m0 = quant::f2h(n);
        m1 = quant::f2h(gam);
        if constexpr (PRESET == kPresetK3V4) {
            // coordinate d = 64h + 32g + 8k + e -> word 3 (2h + g) + w, byte
            // lane e % 4, slot 2k + e / 4 (slots 0-5: three bits at 3 (s % 2)
            // of word s / 2; slots 6, 7: bits 0-1 at 6 of word s - 6, bit 2 at
            // bit s of word 2).  Lane j: e = j, k = m % 4, 2h + g = m / 4.
            const int sh = 8 * (j & 3), sp = j >> 2;
            uint32_t w[12];
#pragma unroll
            for (int T = 0; T < 4; ++T) {
                uint32_t w0 = 0u, w1 = 0u, w2 = 0u;
#pragma unroll
                for (int k = 0; k < 3; ++k) {
                    const uint32_t v = (uint32_t)c[4 * T + k] << (sh + 3 * sp);
                    if (k == 0)
                        w0 |= v;
                    else if (k == 1)
                        w1 |= v;
                    else
                        w2 |= v;
                }
                const uint32_t c3 = (uint32_t)c[4 * T + 3];
                const uint32_t lo2 = (c3 & 3u) << (sh + 6);
                w0 |= sp ? 0u : lo2;
                w1 |= sp ? lo2 : 0u;
                w2 |= (c3 >> 2) << (sh + 6 + sp);
                w[3 * T] = w0;
                w[3 * T + 1] = w1;
                w[3 * T + 2] = w2;
            }
#pragma unroll
            for (int i = 0; i < 12; ++i) {
                w[i] |= gxor<4>(w[i], lane);
                w[i] |= gxor<2>(w[i], lane);
                w[i] |= gxor<1>(w[i], lane);
            }
            if (blk && j < 3) {
                // lane j writes words 4j .. 4j + 3 (per-word selects: a
                // select of whole vectors went through a stack copy)
                uint32_t o[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    o[q4] = ((j == 0) ? w[q4] : 0u) | ((j == 1) ? w[4 + q4] : 0u) | ((j == 2) ? w[8 + q4] : 0u);
                reinterpret_cast<uint4 *>(blk + tb * L::kKeyBytesPerToken)[j] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        } else {
            // coordinate 8m + e -> key dword m, byte e % 4, nibble e / 4
            // (sign-magnitude nibble: bit 3 for the negative levels)
            const int sh = 8 * (j & 3) + 4 * (j >> 2);
            uint32_t w[kPer];
#pragma unroll
            for (int m = 0; m < kPer; ++m) {
                w[m] = quant::k4_nibble(c[m]) << sh;
                w[m] |= gxor<4>(w[m], lane);
                w[m] |= gxor<2>(w[m], lane);
                w[m] |= gxor<1>(w[m], lane);
            }
            if (blk && j < 4) {
                uint32_t o[4];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    o[q4] = ((j == 0) ? w[q4] : 0u) | ((j == 1) ? w[4 + q4] : 0u) | ((j == 2) ? w[8 + q4] : 0u) |
                            ((j == 3) ? w[12 + q4] : 0u);
                reinterpret_cast<uint4 *>(blk + tb * L::kKeyBytesPerToken)[j] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    } else {
        float amax = 0.0f;
#pragma unroll
        for (int m = 0; m < kPer; ++m)
            amax = fmaxf(amax, fabsf(x[m]));
        amax = fmaxf(amax, gxor<4>(amax, lane));
        amax = fmaxf(amax, gxor<2>(amax, lane));
        amax = fmaxf(amax, gxor<1>(amax, lane));
        const uint16_t sh = quant::f2h(__fdiv_rn(amax, 448.0f));
        const float sc = quant::h2f_q(sh);
        m0 = sh;
        // codes of x / s: from the product with 1 / s, the exact division
        // where the product lies near a rounding boundary
        const float rsc = __fdiv_rn(1.0f, sc);
        uint32_t w[4]; // the lane's 16 codes, byte m % 4 of word m / 4
        bool doubt = false;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[i] = 0u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float q = __fmul_rn(x[4 * i + e], rsc);
                w[i] |= quant::e4m3_code(q) << (8 * e);
                doubt |= quant::e4m3_near_boundary(q);
            }
        }
        if (__builtin_expect(__any(doubt), 0)) {
#pragma unroll
            for (int m = 0; m < kPer; ++m)
                if (quant::e4m3_near_boundary(__fmul_rn(x[m], rsc))) {
                    const uint32_t c = quant::e4m3_code(__fdiv_rn(x[m], sc));
                    w[m / 4] = (w[m / 4] & ~(0xFFu << (8 * (m % 4)))) | (c << (8 * (m % 4)));
                }
        }
        if (blk) {
            if (sc == 0.0f)
                w[0] = w[1] = w[2] = w[3] = 0u;
            reinterpret_cast<uint4 *>(blk + tb * L::kKeyBytesPerToken)[j] = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }

    // --------------------------------------------------------------- values
    float v[kPer];
#pragma unroll
    for (int i = 0; i < kPer / 2; ++i) {
        v[2 * i] = quant::h2f_q((uint16_t)(vw[i] & 0xFFFFu));
        v[2 * i + 1] = quant::h2f_q((uint16_t)(vw[i] >> 16));
    }
    float mn = __int_as_float(0x7F800000), mx = __int_as_float(0xFF800000);
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
        mn = fminf(mn, v[m]);
        mx = fmaxf(mx, v[m]);
    }
    mn = fminf(mn, gxor<4>(mn, lane));
    mx = fmaxf(mx, gxor<4>(mx, lane));
    mn = fminf(mn, gxor<2>(mn, lane));
    mx = fmaxf(mx, gxor<2>(mx, lane));
    mn = fminf(mn, gxor<1>(mn, lane));
    mx = fmaxf(mx, gxor<1>(mx, lane));
    const uint16_t zh = quant::f2h(__fadd_rn(mn, 0.0f)); // -0 -> +0
    const float zero = quant::h2f_q(zh);
    const uint16_t sch = quant::f2h(__fdiv_rn(__fsub_rn(mx, mn), 15.0f));
    const float sc = quant::h2f_q(sch);
    const float rs = __fdiv_rn(1.0f, sc);
    float qr[kPer]; // rint of the quotient
    bool near = false;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
        const float q = __fmul_rn(__fsub_rn(v[m], zero), rs);
        qr[m] = rintf(q);
        near |= quant::code_near_tie(q, qr[m]);
    }
    if (__builtin_expect(__any(near), 0)) {
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
            const float q = __fmul_rn(__fsub_rn(v[m], zero), rs);
            if (quant::code_near_tie(q, qr[m]))
                qr[m] = rintf(__fdiv_rn(__fsub_rn(v[m], zero), sc));
        }
    }
    if (blk) {
        uint8_t *vb = blk + L::kValOff;
#pragma unroll
        for (int i = 0; i < kPer / 2; ++i) {
            uint32_t c0 = 0u, c1 = 0u;
            if (sc != 0.0f) {
                c0 = quant::code_clamp(qr[2 * i]);
                c1 = quant::code_clamp(qr[2 * i + 1]);
            }
            vb[val_byte_offset(tb, 8 * j + i)] = (uint8_t)(c0 | (c1 << 4));
        }
        if (j == 0) {
            *reinterpret_cast<uint16_t *>(blk + L::kMeta0 + 2 * tb) = m0;
            if constexpr (kLloydMax<PRESET>)
                *reinterpret_cast<uint16_t *>(blk + L::kMeta1 + 2 * tb) = m1;
            *reinterpret_cast<uint16_t *>(blk + L::kVScale + 2 * tb) = sch;
            *reinterpret_cast<uint16_t *>(blk + L::kVZero + 2 * tb) = zh;
        }
    }
}

} // namespace

hipError_t launch_store(int preset, const StoreArgs &a, hipStream_t s)
{
    if ((long)a.T * a.Hk == 0)
        return hipSuccess;
    // 16-token chunks of every head, 32 token-heads per block
    constexpr long kPerBlock = kStoreThreads / kGroup;
    const long groups = ((long)a.T + 15) / 16 * 16 * a.Hk;
    const dim3 grid((unsigned)((groups + kPerBlock - 1) / kPerBlock)), block(kStoreThreads);
    if (preset == kPresetK3V4)
        hipLaunchKernelGGL(store_kernel<kPresetK3V4>, grid, block, 0, s, a);
    else if (preset == kPresetK4V4)
        hipLaunchKernelGGL(store_kernel<kPresetK4V4>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(store_kernel<kPresetK8V4>, grid, block, 0, s, a);
    return hipGetLastError();
}

} // namespace tqkv
