// Speculative verification attention over the packed TurboQuant cache.
//
// Method: Part 3 of "Speculative decoding on Intel Arc: TurboQuant KV + a
// fused N_spec kernel" fuses the N_spec queries of one head into one pass
// that dequantises each key tile once and keeps an online softmax per query;
// Part 4 adds the causal window (query n sees cached_len + n + 1 tokens);
// Part 2 splits the sequence across work-groups and merges the partial
// softmax states with a log-sum-exp reduction.
//
// MI355X design (not the pages' Triton/SYCL design):
//  * One work-group = 4 wavefronts = one (b, hk) unit and one key range.  A
//    wavefront owns ALL R = (Hq/Hk) * N_spec query rows of its KV head (up to
//    64) and a contiguous run of 32-token tiles, so every key/value code is
//    fetched from HBM and dequantised exactly once per launch.
//  * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_f16: keys /
//    value codes are the A operand (M = tokens or d), the 64 query rows the B
//    operand (N).  The C layout then gives each lane one query row and 16
//    tokens, so the softmax row max needs a single cross-half swap and the
//    probabilities become the next B operand without any data movement.
//  * The packed layout is chosen so that each lane loads its MFMA operand
//    bytes directly: 24 B of 3-bit codes or 64 B of FP8 per token half, and
//    one 16 B load of value nibbles per 16-token block (8-token runs at a
//    fixed d).  3-bit codes become fp16 centroids with v_perm_b32 table
//    lookups (no LDS); FP8 becomes fp16 with v_cvt_scalef32_pk_f16_fp8.
//  * Per-token factors stay out of the contraction: the key scale multiplies
//    the score column, the value scale multiplies P, the value zero enters
//    through sum_t p_t * zero_t.  Value codes enter the MFMA as the binary16
//    integers c (low nibble) and 16c (high nibble), built with one mask.
//  * The four wavefronts merge their softmax states through LDS; with more
//    than one key range per unit a second kernel merges the ranges.
#include "codebook.h"
#include "common.h"

#include <type_traits>

namespace tqkv {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;        // tokens per inner-loop step
constexpr int kWaves = 4;        // wavefronts per work-group
constexpr int kQStride = kQPadHalfs; // halfs per query row in LDS (128 + pad)
constexpr int kAccStride = 132;  // floats per row of the LDS merge buffer

union H8 {
    half8_t h;
    uint32_t u[4];
};

__device__ inline float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// 4 packed 3-bit codes (one per byte, values 0..7) -> 4 fp16 centroids
__device__ inline void k3_lookup(uint32_t sel, uint32_t &out01, uint32_t &out23)
{
    const uint32_t lo = perm(kLoBytes47, kLoBytes03, sel);
    const uint32_t hi = perm(kHiBytes47, kHiBytes03, sel);
    out01 = perm(hi, lo, 0x05010400u);
    out23 = perm(hi, lo, 0x07030602u);
}

// ---------------------------------------------------------------------------
// Tile staging.  A 32-token tile of one (b, hk) is two consecutive 16-token
// blocks, i.e. one contiguous run of 2 * kBlockBytes in HBM.  Each wavefront
// streams its tiles through a private ring of kRing slots in LDS with direct
// global->LDS loads (global_load_lds_dwordx4: 64 lanes x 16 B = 1 KiB per
// instruction, no VGPRs held while in flight).  The ring is prefilled before
// the query prologue, and slot i is refilled with tile i + kRing as soon as
// tile i has been read into registers, so kRing - 1 tiles stay in flight.
// ---------------------------------------------------------------------------
template <int PRESET> struct Ring;
template <> struct Ring<kPresetK3V4> {
    static constexpr int kLoads = 4; // ceil(2 * 1920 / 1024)
    static constexpr int kDepth = 8;
};
template <> struct Ring<kPresetK8V4> {
    static constexpr int kLoads = 7; // ceil(2 * 3168 / 1024)
    static constexpr int kDepth = 4;
};

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt vmcnt(N) with a compile-time N; the memory clobber keeps the
// compiler from moving LDS reads of the waited-for slot above it.
template <int N> __device__ inline void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ inline void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// wait until at most `tiles` ring tiles (of LPT instructions each) are in
// flight; counts above 8 tiles are never needed (depth <= 8)
template <int LPT> __device__ inline void wait_ring(int tiles)
{
    static_assert(8 * LPT <= 63, "vmcnt range");
    switch (tiles) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<LPT>(); break;
    case 2: wait_vm<2 * LPT>(); break;
    case 3: wait_vm<3 * LPT>(); break;
    case 4: wait_vm<4 * LPT>(); break;
    case 5: wait_vm<5 * LPT>(); break;
    case 6: wait_vm<6 * LPT>(); break;
    case 7: wait_vm<7 * LPT>(); break;
    default: wait_vm<8 * LPT>(); break;
    }
}

// One 16-byte-per-lane global -> LDS load: lane l's 16 bytes at `g` land at
// LDS byte lds_base + 16 * l.  Written as inline assembly so that the
// compiler's wait insertion does not treat it as a pending write to every
// LDS location (it would wait for the whole ring before each LDS read); the
// ring's completion is tracked explicitly with wait_ring().  Inline memory
// operations the compiler cannot see can only make its own waits longer,
// never shorter, because loads complete in order.  M0 is not used by any
// other instruction of this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma16(const void *g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Issue the loads of tile kt (blocks 2kt, 2kt+1 of this unit) into `slot`.
// Lanes past the last valid byte re-read the final 16 B (the unit's last
// block exists; a missing second block is only ever masked).
template <int PRESET>
__device__ inline void issue_tile(const uint8_t *ubase, int kt, int nblk, uint8_t *slot, int lane)
{
    using L = Layout<PRESET>;
    // the tile's bytes [0, valid); loads past the end re-read the final 16 B
    const int valid = min(2, nblk - 2 * kt) * L::kBlockBytes;
    const uint8_t *src = ubase + (size_t)(2 * kt) * L::kBlockBytes;
    const uint32_t lds = (uint32_t)(size_t)(lds_void_t *)slot;
#pragma unroll
    for (int j = 0; j < Ring<PRESET>::kLoads; ++j) {
        dma16(src + min(1024 * j + 16 * lane, valid - 16), lds + 1024 * j);
    }
}

// Registers of one tile, read back from its ring slot: the key half (the A
// operands of S^T = K Q^T) and the value half (value nibbles and per-token
// fields), read at different times by the software pipeline below.
template <int PRESET> struct KeyRegs;
template <> struct KeyRegs<kPresetK3V4> {
    uint2 k[3]; // 24 B: this lane's 64 key codes (two 32-code dword triples)
};
template <> struct KeyRegs<kPresetK8V4> {
    u32x4 k[4]; // 64 B: this lane's 64 e4m3 key codes
};
struct ValRegs {
    u32x4 v[2];  // value nibbles of blocks 0/1 (8-token runs at 4 d's)
    u32x4 kf[2]; // per-token key factor (fp16): n*gamma (k3v4_nc) or kscale (k8v4), tokens 8h..8h+7
    u32x4 vs[2], vz[2];
};

// Token of the 32-token tile that MFMA row m stands for: bits 2 and 3 of m
// swapped.  With this order the C registers 8s..8s+7 of lane half h hold
// tokens 16s + 8h + 0..7, which are the 8 consecutive tokens the value
// operand of k-step s reads at one d.
__device__ inline int tile_token_of_row(int m)
{
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int PRESET>
__device__ inline void read_keys(KeyRegs<PRESET> &t, const uint8_t *slot, int lane)
{
    using L = Layout<PRESET>;
    const int h = lane >> 5, m = lane & 31;
    const int tok = tile_token_of_row(m);
    const uint8_t *kb = slot + (tok >> 4) * L::kBlockBytes + (tok & 15) * L::kKeyBytesPerToken;
    if constexpr (PRESET == kPresetK3V4) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
            t.k[j] = *reinterpret_cast<const uint2 *>(kb + 24 * h + 8 * j);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            t.k[j] = *reinterpret_cast<const u32x4 *>(kb + 64 * h + 16 * j);
    }
}

__device__ inline uint32_t hmul2(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) * __builtin_bit_cast(half2_t, b));
}

template <int PRESET>
__device__ inline void read_values(ValRegs &t, const uint8_t *slot, int lane)
{
    using L = Layout<PRESET>;
    const int h = lane >> 5, m = lane & 31;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const uint8_t *bs = slot + s * L::kBlockBytes;
        t.v[s] = *reinterpret_cast<const u32x4 *>(bs + L::kValOff + (2 * m + h) * 16);
        const u32x4 n = *reinterpret_cast<const u32x4 *>(bs + L::kMeta0 + 16 * h);
        if constexpr (PRESET == kPresetK3V4) {
            // n * gamma per token, as fp16 pairs (one v_pk_mul_f16 per pair).
            // Written component by component: an in-place update of vector
            // elements in a loop (kf[s][j] = f(kf[s][j], g[j])) was
            // miscompiled by this toolchain (only g[0] was loaded).
            const u32x4 g = *reinterpret_cast<const u32x4 *>(bs + L::kMeta1 + 16 * h);
            u32x4 kf;
            kf.x = hmul2(n.x, g.x);
            kf.y = hmul2(n.y, g.y);
            kf.z = hmul2(n.z, g.z);
            kf.w = hmul2(n.w, g.w);
            t.kf[s] = kf;
        } else {
            t.kf[s] = n;
        }
        t.vs[s] = *reinterpret_cast<const u32x4 *>(bs + L::kVScale + 16 * h);
        t.vz[s] = *reinterpret_cast<const u32x4 *>(bs + L::kVZero + 16 * h);
    }
}

// A operand of k-step ks of S^T = K Q^T: coordinates 64h + 8ks + 0..7 of
// this lane's token.
template <int PRESET>
__device__ inline half8_t key_operand(const KeyRegs<PRESET> &t, int ks)
{
    H8 o;
    if constexpr (PRESET == kPresetK3V4) {
        const int g = ks >> 2, kk = ks & 3;
        // dwords 3g..3g+2 of the lane's six key dwords
        const uint32_t d0 = (g == 0) ? t.k[0].x : t.k[1].y;
        const uint32_t d1 = (g == 0) ? t.k[0].y : t.k[2].x;
        const uint32_t d2 = (g == 0) ? t.k[1].x : t.k[2].y;
        uint32_t sa, sb;
        if (kk == 0) {
            sa = d0 & 0x07070707u;
            sb = (d0 >> 3) & 0x07070707u;
        } else if (kk == 1) {
            sa = d1 & 0x07070707u;
            sb = (d1 >> 3) & 0x07070707u;
        } else if (kk == 2) {
            sa = d2 & 0x07070707u;
            sb = (d2 >> 3) & 0x07070707u;
        } else {
            sa = ((d0 >> 6) & 0x03030303u) | ((d2 >> 4) & 0x04040404u);
            sb = ((d1 >> 6) & 0x03030303u) | ((d2 >> 5) & 0x04040404u);
        }
        k3_lookup(sa, o.u[0], o.u[1]);
        k3_lookup(sb, o.u[2], o.u[3]);
    } else {
        const uint32_t a = t.k[ks >> 1][2 * (ks & 1)], b = t.k[ks >> 1][2 * (ks & 1) + 1];
        half2_t x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, false);
        half2_t x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, true);
        half2_t x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false);
        half2_t x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true);
        o.h = half8_t{x0[0], x0[1], x1[0], x1[1], x2[0], x2[1], x3[0], x3[1]};
    }
    return o.h;
}

// S^T = K Q^T for one tile.  The query B operands are re-read from the LDS
// query tile (qrow points at this lane's row and half) instead of being held
// in 8*NQT*4 VGPRs across the whole loop.
template <int PRESET, int NQT>
__device__ inline void qk_tile(const KeyRegs<PRESET> &k, const _Float16 *qrow, floatx16 (&S)[NQT])
{
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
        S[qt] = floatx16{0};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const half8_t A = key_operand<PRESET>(k, ks);
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            const half8_t Bq = *reinterpret_cast<const half8_t *>(qrow + 32 * qt * kQStride + 8 * ks);
            S[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, Bq, S[qt], 0, 0, 0);
        }
    }
}

// A operand of O^T += V^T P^T for d-tile dt (d = 4i + dt) and k-step s
// (tokens 16s + 8h + 0..7).  The nibbles are used as binary16 bit patterns:
// a low nibble c is the subnormal c * 2^-24, a high nibble the subnormal
// 16c * 2^-24 (gfx950's f16 MFMA multiplies subnormal inputs exactly), so
// one mask per half-pair builds the operand; the epilogue rescales even d by
// 2^24 and odd d by 2^20.
__device__ inline half8_t value_operand(const ValRegs &t, int dt, int s)
{
    const int e = dt >> 1;
    const uint32_t mask = (dt & 1) ? 0x00F000F0u : 0x000F000Fu;
    const uint32_t wa = t.v[s][2 * e], wb = t.v[s][2 * e + 1];
    H8 o;
    o.u[0] = wa & mask;
    o.u[1] = (wa >> 8) & mask;
    o.u[2] = wb & mask;
    o.u[3] = (wb >> 8) & mask;
    return o.h;
}

__device__ inline float half_lo(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w)[0]; }
__device__ inline float half_hi(uint32_t w) { return (float)__builtin_bit_cast(half2_t, w)[1]; }

// Lazy rescaling: the running row maximum m only moves when a tile's maximum
// exceeds it by more than kRescaleSlack (log2 units), so probabilities are
// at most 2^kRescaleSlack = 4.  With value scales below 2^14 (every binary16
// min-max scale is), P * vscale <= 4 * 8736 stays inside binary16 range.
constexpr float kRescaleSlack = 2.0f;

// Online-softmax state of the lane's query rows (one per 32-row tile).
template <int NQT> struct SoftState {
    float m[NQT], l[NQT], z[NQT];
};

// softmax of tile i (scores S), overlapped with the QK^T of tile i+1 (keys
// kn, scores Sn) and followed by O^T += V^T P^T of tile i.  MASKED tiles
// exclude tokens at or beyond each row's end (erow) and drop the value
// scale/zero of excluded tokens (their bytes may never have been written).
template <int PRESET, int NQT, bool MASKED>
__device__ inline void tile_step(const floatx16 (&S)[NQT], const ValRegs &vr, const KeyRegs<PRESET> &kn,
                                 bool have_next, const _Float16 *qrow, floatx16 (&Sn)[NQT],
                                 floatx16 (&acc)[4][NQT], SoftState<NQT> &st, const int (&erow)[NQT],
                                 int tok0, int h)
{
    // 1. scores relative to the running max, the tile max, lazy rescale
    float y[NQT][16];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const float msub = (st.m[qt] == -__builtin_inff()) ? 0.0f : st.m[qt];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const uint32_t w = vr.kf[v >> 3][(v & 7) >> 1];
            const float kf = (v & 1) ? half_hi(w) : half_lo(w);
            y[qt][v] = __builtin_fmaf(S[qt][v], kf, -msub);
            if constexpr (MASKED) {
                const int t = tok0 + 16 * (v >> 3) + 8 * h + (v & 7);
                if (t >= erow[qt])
                    y[qt][v] = -__builtin_inff();
            }
        }
        float tmax = fmaxf(fmaxf(y[qt][0], y[qt][1]), y[qt][2]);
#pragma unroll
        for (int v = 3; v < 15; v += 2)
            tmax = fmaxf(fmaxf(tmax, y[qt][v]), y[qt][v + 1]);
        tmax = fmaxf(tmax, y[qt][15]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const bool first = (st.m[qt] == -__builtin_inff());
        const bool grow = first ? (tmax > -__builtin_inff()) : (tmax > kRescaleSlack);
        if (__builtin_expect(__any(grow), 0)) { // rare after the first tile
            // rows that grew (or any row, for uniformity) move their max up
            const float delta = first ? ((tmax > -__builtin_inff()) ? tmax : 0.0f) : fmaxf(tmax, 0.0f);
            if (!first || tmax > -__builtin_inff()) {
                if (!first) {
                    const float alpha = __builtin_amdgcn_exp2f(-delta);
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
                        acc[dt][qt] *= alpha;
                    st.l[qt] *= alpha;
                    st.z[qt] *= alpha;
                }
                st.m[qt] = msub + delta;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    y[qt][v] -= delta;
            }
        }
    }

    // 2. QK^T of the next tile (independent of the rest of this step)
    if (have_next)
        qk_tile<PRESET, NQT>(kn, qrow, Sn);

    // 3. probabilities, their sums and the P operand
    H8 Pb[NQT][2];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int v = 8 * s + 2 * j;
                const float p0 = __builtin_amdgcn_exp2f(y[qt][v]);
                const float p1 = __builtin_amdgcn_exp2f(y[qt][v + 1]);
                const half2_t ph = half2_t{(_Float16)p0, (_Float16)p1};
                uint32_t vs = vr.vs[s][j], vz = vr.vz[s][j];
                if constexpr (MASKED) {
                    const int t = tok0 + 16 * s + 8 * h + 2 * j;
                    const uint32_t keep = ((t < erow[qt]) ? 0x0000FFFFu : 0u) | ((t + 1 < erow[qt]) ? 0xFFFF0000u : 0u);
                    vs &= keep;
                    vz &= keep;
                }
                st.l[qt] = __builtin_amdgcn_fdot2(ph, half2_t{(_Float16)1.0f, (_Float16)1.0f}, st.l[qt], false);
                st.z[qt] = __builtin_amdgcn_fdot2(ph, __builtin_bit_cast(half2_t, vz), st.z[qt], false);
                Pb[qt][s].u[j] = __builtin_bit_cast(uint32_t, ph * __builtin_bit_cast(half2_t, vs));
            }

    // 4. O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const half8_t A = value_operand(vr, dt, s);
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
                acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, Pb[qt][s].h, acc[dt][qt], 0, 0, 0);
        }
}

// Query preparation, once per (b, hk) unit: row r = n * G + g of the unit
// is query head hk * G + g of speculative token n, scaled by sm_scale *
// log2(e) (the softmax runs in base 2) and, for k3v4_nc, rotated by the same
// normalised Walsh-Hadamard transform as the keys (q' = H q / sqrt(128)),
// then rounded to binary16 -- the B operand of the QK^T MFMAs.  One
// wavefront per row; lane l holds coordinates l and l + 64.
__global__ __launch_bounds__(256) void qprep_kernel(QPrepArgs a)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6); // unit * rows_pad + r
    const int unit = row / a.rows_pad, rr = row % a.rows_pad;
    const int b = unit / a.Hk, hk = unit % a.Hk;
    float x0 = 0.0f, x1 = 0.0f;
    if (rr < a.R) {
        const int n = rr / a.G, g = rr % a.G;
        const size_t off = ((size_t)(n * a.B + b) * a.Hq + hk * a.G + g) * kD;
        if (a.q_f16) {
            const _Float16 *q = reinterpret_cast<const _Float16 *>(a.Q) + off;
            x0 = (float)q[lane];
            x1 = (float)q[lane + 64];
        } else {
            const float *q = reinterpret_cast<const float *>(a.Q) + off;
            x0 = q[lane];
            x1 = q[lane + 64];
        }
    }
    float sc = a.qscale;
    if (a.rotate) {
#pragma unroll
        for (int hh = 1; hh < 64; hh <<= 1) {
            const float p0 = __shfl_xor(x0, hh, 64), p1 = __shfl_xor(x1, hh, 64);
            x0 = (lane & hh) ? p0 - x0 : x0 + p0;
            x1 = (lane & hh) ? p1 - x1 : x1 + p1;
        }
        const float u = x0, v = x1;
        x0 = u + v;
        x1 = u - v;
        sc *= 0.08838834764831845f; // 1 / sqrt(128)
    }
    _Float16 *dst = a.qp + (size_t)row * kQPadHalfs;
    dst[lane] = (_Float16)(x0 * sc);
    dst[lane + 64] = (_Float16)(x1 * sc);
    if (lane < kQPadHalfs - kD)
        dst[kD + lane] = (_Float16)0.0f;
}

template <int PRESET, int NQT>
__global__ __launch_bounds__(256, 1) void verify_kernel(VerifyArgs a)
{
    constexpr int RP = 32 * NQT; // padded rows
    constexpr int LPT = Ring<PRESET>::kLoads, DEPTH = Ring<PRESET>::kDepth;
    constexpr int kSlotBytes = LPT * 1024;
    // query region: the unit's prepared fp16 rows (RP x kQPadHalfs), copied
    // in 1 KiB loads into a region rounded up to whole KiB
    constexpr int kQBytes = RP * kQPadHalfs * 2;
    constexpr int kQRegion = (kQBytes + 1023) / 1024 * 1024;
    constexpr int kRingBytes = kWaves * DEPTH * kSlotBytes;
    constexpr int kMergeBytes = (kWaves * RP * kAccStride + kWaves * RP * 4 + RP * 3) * 4;
    constexpr int kLdsBytes = (kQRegion + kRingBytes) > kMergeBytes ? (kQRegion + kRingBytes) : kMergeBytes;
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];

    const int lane = threadIdx.x & 63;
    // wavefront index as a scalar: every quantity derived from it (the tile
    // range, the ring slot, the wait counts) stays in SGPRs and uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, col = lane & 31;
    const int unit = blockIdx.x / a.nsplit, split = blockIdx.x % a.nsplit;
    const int b = unit / a.Hk, hk = unit % a.Hk;
    const int Lr = a.seq_lens[b];
    const int L = Lr < 0 ? 0 : (Lr > a.max_seq ? a.max_seq : Lr);

    // this wavefront's tiles [kt0, kt1): the unit's tiles are cut into
    // nsplit work-group ranges, each range into 4 wavefront runs
    const int tiles = (L + kTile - 1) / kTile;
    const int tpw = (tiles + a.nsplit - 1) / a.nsplit;
    const int wt0 = min(split * tpw, tiles), wt1 = min(wt0 + tpw, tiles);
    const int tpv = (wt1 - wt0 + kWaves - 1) / kWaves;
    const int kt0 = min(wt0 + wave * tpv, wt1), kt1 = min(kt0 + tpv, wt1);
    const int ntile = kt1 - kt0;

    using L_ = Layout<PRESET>;
    const uint8_t *ubase = a.base + (size_t)unit * a.nblk * L_::kBlockBytes;
    _Float16 *qs = reinterpret_cast<_Float16 *>(lds);
    uint8_t *ring = lds + kQRegion + wave * DEPTH * kSlotBytes;

    // ------------------------------------------------------------ prologue
    // The unit's prepared query rows (qprep_kernel) and the first ring tiles
    // arrive by direct global->LDS loads, query first, so that waiting for
    // the query means "all but the ring prefill".
    {
        constexpr int kQLoads = kQRegion / 1024;
        const uint8_t *qsrc = reinterpret_cast<const uint8_t *>(a.qp) + (size_t)unit * kQBytes;
        const uint32_t qlds = (uint32_t)(size_t)(lds_void_t *)lds;
        for (int J = wave; J < kQLoads; J += kWaves)
            dma16(qsrc + min(1024 * J + 16 * lane, kQBytes - 16), qlds + 1024 * J);
    }
    const int npre = min(DEPTH, ntile);
    for (int i = 0; i < npre; ++i)
        issue_tile<PRESET>(ubase, kt0 + i, a.nblk, ring + i * kSlotBytes, lane);
    wait_ring<LPT>(npre);          // this wavefront's query loads are done
    __builtin_amdgcn_s_barrier();  // ... and every other wavefront's
    const _Float16 *qlane = qs + col * kQStride + 64 * h; // this lane's B-operand row

    // Effective end of this lane's query rows (causal window of the pages).
    int erow[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const int rr = 32 * qt + col;
        const int n = rr / a.G;
        erow[qt] = (rr < a.R) ? (a.causal ? min(L - a.N + n + 1, L) : L) : 0;
    }
    const int emin = a.causal ? (L - a.N + 1) : L;

    floatx16 acc[4][NQT];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
            acc[dt][qt] = floatx16{0};
    SoftState<NQT> st;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        st.m[qt] = -__builtin_inff();
        st.l[qt] = 0.0f;
        st.z[qt] = 0.0f;
    }

    // Software pipeline: the scores of tile i+1 are computed while tile i's
    // softmax and P*V run.  Slot i is refilled with tile i + DEPTH once both
    // of its halves have been read (keys one iteration earlier).
    floatx16 S[NQT], Sn[NQT];
    if (ntile > 0) {
        wait_ring<LPT>(min(ntile - 1, DEPTH - 1));
        KeyRegs<PRESET> k0;
        read_keys<PRESET>(k0, ring, lane);
        qk_tile<PRESET, NQT>(k0, qlane, S);
    }
    // tiles [0, nfast) need no masking; the rest (the sequence's last tile
    // and the causal window) run in a separate, identical loop so that the
    // masking code does not share the main loop's registers
    const int nfast = max(0, min(ntile, (emin - kt0 * kTile) / kTile));
    auto step = [&](int i, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int kt = kt0 + i;
        uint8_t *slot = ring + (i % DEPTH) * kSlotBytes;
        ValRegs vr;
        read_values<PRESET>(vr, slot, lane);
        const bool have_next = i + 1 < ntile;
        KeyRegs<PRESET> kn;
        if (have_next) {
            wait_ring<LPT>(min(ntile - i - 2, DEPTH - 2));
            read_keys<PRESET>(kn, ring + ((i + 1) % DEPTH) * kSlotBytes, lane);
        }
        wait_lgkm0();
        if (i + DEPTH < ntile)
            issue_tile<PRESET>(ubase, kt + DEPTH, a.nblk, slot, lane);
        tile_step<PRESET, NQT, MASKED>(S, vr, kn, have_next, qlane, Sn, acc, st, erow, kt * kTile, h);
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
            S[qt] = Sn[qt];
    };
    for (int i = 0; i < nfast; ++i)
        step(i, std::false_type{});
    for (int i = nfast; i < ntile; ++i)
        step(i, std::true_type{});
    float mrow[NQT], lsum[NQT], zsum[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        mrow[qt] = st.m[qt];
        lsum[qt] = st.l[qt];
        zsum[qt] = st.z[qt];
    }

    // ---------------------------------------------------------------- merge
    // softmax sums of the two lane halves (same rows, different tokens)
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        lsum[qt] += __shfl_xor(lsum[qt], 32, 64);
        zsum[qt] += __shfl_xor(zsum[qt], 32, 64);
    }
    __syncthreads(); // every wavefront is done with the ring and the query tile
    float *macc = reinterpret_cast<float *>(lds);               // [4][RP][kAccStride]
    float *mstat = macc + kWaves * RP * kAccStride;             // [4][RP] m, l, z, alpha
    float *rstat = mstat + kWaves * RP * 4;                     // [RP] L, Z, M
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const int rr = 32 * qt + col;
        if (h == 0) {
            mstat[(wave * RP + rr) * 4 + 0] = mrow[qt];
            mstat[(wave * RP + rr) * 4 + 1] = lsum[qt];
            mstat[(wave * RP + rr) * 4 + 2] = zsum[qt];
        }
        float *dst = macc + (wave * RP + rr) * kAccStride;
#pragma unroll
        for (int aa = 0; aa < 4; ++aa)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 8 * aa + 4 * h + j; // d-quad of C registers 4aa + j
                const int v = 4 * aa + j;
                *reinterpret_cast<float4 *>(dst + 4 * i) =
                    make_float4(acc[0][qt][v], acc[1][qt][v], acc[2][qt][v], acc[3][qt][v]);
            }
    }
    __syncthreads();
    if (threadIdx.x < RP) {
        const int rr = threadIdx.x;
        float M = -__builtin_inff();
        for (int w = 0; w < kWaves; ++w)
            M = fmaxf(M, mstat[(w * RP + rr) * 4 + 0]);
        float Ls = 0.0f, Zs = 0.0f;
        for (int w = 0; w < kWaves; ++w) {
            const float mw = mstat[(w * RP + rr) * 4 + 0];
            const float al = (mw == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
            mstat[(w * RP + rr) * 4 + 3] = al;
            Ls += al * mstat[(w * RP + rr) * 4 + 1];
            Zs += al * mstat[(w * RP + rr) * 4 + 2];
        }
        rstat[rr * 3 + 0] = Ls;
        rstat[rr * 3 + 1] = Zs;
        rstat[rr * 3 + 2] = M;
    }
    __syncthreads();
    const size_t pbase = ((size_t)unit * a.nsplit + split) * a.R;
    for (int e4 = threadIdx.x; e4 < a.R * (kD / 4); e4 += 256) {
        const int rr = e4 >> 5, d = (e4 & 31) * 4;
        float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float al = mstat[(w * RP + rr) * 4 + 3];
            const float4 x = *reinterpret_cast<const float4 *>(macc + (w * RP + rr) * kAccStride + d);
            s4.x += al * x.x;
            s4.y += al * x.y;
            s4.z += al * x.z;
            s4.w += al * x.w;
        }
        const float Ls = rstat[rr * 3 + 0], Zs = rstat[rr * 3 + 1];
        // the value operand carried c * 2^-24 (even d) and 16c * 2^-24 (odd d)
        float4 o = make_float4(s4.x * 16777216.0f + Zs, s4.y * 1048576.0f + Zs, s4.z * 16777216.0f + Zs,
                               s4.w * 1048576.0f + Zs);
        // Ls == 0: the row saw no token in this range.  A NaN Ls (a NaN key
        // or scale the row can see) propagates to the output.
        if (a.nsplit == 1) {
            const int n = rr / a.G, g = rr % a.G;
            const float inv = (Ls != 0.0f) ? 1.0f / Ls : __builtin_nanf("");
            o = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
            *reinterpret_cast<float4 *>(a.out + ((size_t)(n * a.B + b) * a.Hq + hk * a.G + g) * kD + d) = o;
        } else {
            const float inv = (Ls != 0.0f) ? 1.0f / Ls : 0.0f;
            o = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
            *reinterpret_cast<float4 *>(a.part_o + (pbase + rr) * kD + d) = o;
            if (d == 0)
                a.part_ml[pbase + rr] = make_float2(rstat[rr * 3 + 2], Ls);
        }
    }
}

// Merge of the key-range partitions of each (b, hk): out = sum_s w_s O_s /
// sum_s w_s with w_s = exp2(m_s - max_s m_s) * l_s.  One 32-lane group per
// (unit, row), one float4 of the row per lane; every lane loads the row's
// (m, l) pairs and its own partial float4s in one batch, so the kernel costs
// a single round trip to memory.  Ranges whose softmax sum is exactly 0 saw
// no token and get weight 0; a NaN sum is kept so that it reaches the output.
constexpr int kCombineChunk = 16;

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a)
{
    const int grp = blockIdx.x * 8 + (threadIdx.x >> 5);
    if (grp >= a.B * a.Hk * a.R)
        return;
    const int unit = grp / a.R, rr = grp % a.R;
    const int d = (threadIdx.x & 31) * 4;
    const size_t base = (size_t)unit * a.nsplit * a.R + rr;
    float M = -__builtin_inff(), den = 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < a.nsplit; s0 += kCombineChunk) {
        float2 ml[kCombineChunk];
        float4 v[kCombineChunk];
#pragma unroll
        for (int j = 0; j < kCombineChunk; ++j) {
            if (s0 + j < a.nsplit) {
                const size_t ix = base + (size_t)(s0 + j) * a.R;
                ml[j] = a.part_ml[ix];
                v[j] = *reinterpret_cast<const float4 *>(a.part_o + ix * kD + d);
            } else {
                ml[j] = make_float2(-__builtin_inff(), 0.0f);
                v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
        float Mc = M;
#pragma unroll
        for (int j = 0; j < kCombineChunk; ++j)
            if (ml[j].y != 0.0f)
                Mc = fmaxf(Mc, ml[j].x);
        // rescale what earlier chunks accumulated to the new maximum
        const float r = (M == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(M - Mc);
        den *= r;
        acc.x *= r;
        acc.y *= r;
        acc.z *= r;
        acc.w *= r;
        M = Mc;
#pragma unroll
        for (int j = 0; j < kCombineChunk; ++j) {
            const float w = (ml[j].y != 0.0f) ? __builtin_amdgcn_exp2f(ml[j].x - M) * ml[j].y : 0.0f;
            den += w;
            acc.x += w * v[j].x;
            acc.y += w * v[j].y;
            acc.z += w * v[j].z;
            acc.w += w * v[j].w;
        }
    }
    const float inv = (den != 0.0f) ? 1.0f / den : __builtin_nanf("");
    const int b = unit / a.Hk, hk = unit % a.Hk;
    const int n = rr / a.G, g = rr % a.G;
    *reinterpret_cast<float4 *>(a.out + ((size_t)(n * a.B + b) * a.Hq + hk * a.G + g) * kD + d) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

} // namespace

hipError_t launch_verify(int preset, int nqt, const VerifyArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(a.B * a.Hk * a.nsplit)), block(256);
    if (preset == kPresetK3V4) {
        if (nqt == 1)
            hipLaunchKernelGGL((verify_kernel<kPresetK3V4, 1>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((verify_kernel<kPresetK3V4, 2>), grid, block, 0, s, a);
    } else {
        if (nqt == 1)
            hipLaunchKernelGGL((verify_kernel<kPresetK8V4, 1>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((verify_kernel<kPresetK8V4, 2>), grid, block, 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_qprep(const QPrepArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(a.B * a.Hk * a.rows_pad / 4)), block(256);
    hipLaunchKernelGGL(qprep_kernel, grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)((a.B * a.Hk * a.R + 7) / 8)), block(256);
    hipLaunchKernelGGL(combine_kernel, grid, block, 0, s, a);
    return hipGetLastError();
}

} // namespace tqkv
