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
//  * One work-group = 4 wavefronts = one (b, hk) unit, one key range and one
//    group of query rows: the R = (Hq/Hk) * N_spec rows of a KV head are cut
//    into 32-row tiles (one MFMA operand height), and a work-group takes one
//    tile (two work-groups per compute unit) or two (64 rows, one per
//    compute unit, each key/value tile dequantised once for all 64 rows).
//    Each wavefront streams a contiguous run of 32-token tiles through its
//    own LDS ring (direct global->LDS loads).
//  * S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_32x32x16_f16: keys /
//    value codes are the A operand (M = tokens or d), the query rows the B
//    operand (N).  The C layout then gives each lane one query row and 16
//    tokens, so the softmax row max needs a single cross-half swap and the
//    probabilities become the next B operand without any data movement.
//    Units of at most 8 rows (plain decode) use the transposed product
//    S = Q K^T instead: one token per lane, 4 exponentials per lane per tile.
//  * The packed layout is chosen so that each lane loads its MFMA operand
//    bytes directly: 24 B of 3-bit codes, 32 B of 4-bit codes or 64 B of FP8
//    per token half, and one 16 B load of value nibbles per 16-token block
//    (8-token runs at a fixed d).  Lloyd-Max codes become fp16 levels with
//    v_perm_b32 table lookups (no LDS); FP8 becomes fp16 with
//    v_cvt_scalef32_pk_f16_fp8.
//  * Per-token factors: the key factor (FP8 scale, or n * gamma) scales the
//    key operand, the value scale multiplies P, the value zero enters through
//    sum_t p_t * zero_t.  Value codes enter the MFMA as the binary16
//    subnormals c and 16c (low / high nibble), built with one mask.
//  * The query operands are prepared inside the kernel (scale, WHT rotation
//    for the Lloyd-Max presets as one small MFMA product with a +-1 matrix,
//    fp16) and held in AGPRs for the whole key loop; the accumulators stay
//    in VGPRs, where the rare online-softmax rescale reaches them.
//  * The four wavefronts merge their softmax states through LDS; with more
//    than one key range per unit a second kernel merges the ranges.
#include "codebook.h"
#include "common.h"
#include "quant.h"

#include <type_traits>

namespace tqkv {

// Phase trace of verify_wide_kernel, compiled only with -DTQKV_PHASE_TRACE
// (a separate library, quantized_kv_attention_amd/phase_trace.py): every
// wavefront keeps the low 32 bits of s_memrealtime stamps (100 MHz; the
// host takes differences modulo 2^32) in registers and stores
// them after its key loop and at its end, so the stamps add no memory
// operation to the loop's vmcnt bookkeeping.  Slots: 0 entry, 1 query rows
// landed, 2 key loop start, 3 + 3i .. 5 + 3i step i < 4 (tile landed, tile
// max done, step issued), 15 loop end, 16 / 17 fused store start / stores
// issued, 18 merge done, 19 end, 20 = 1 when the work-group stores new
// tokens, 22 / 23 s_memtime (shader clock) at loop start / end.
#ifdef TQKV_PHASE_TRACE
constexpr int kTraceWGs = 4096, kTraceSlots = 24;
__device__ uint32_t g_phase_trace[kTraceWGs * 8 * kTraceSlots];
#define TQKV_TRACE_DECL uint32_t trv_[kTraceSlots] = {}
#define TQKV_STAMP(k) (trv_[(k)] = (uint32_t)__builtin_amdgcn_s_memrealtime())
#define TQKV_CLOCK(k) (trv_[(k)] = (uint32_t)__builtin_amdgcn_s_memtime())
#define TQKV_SET(k, v) (trv_[(k)] = (v))
#define TQKV_STEP_STAMP(i, p)                                                                                         \
    do {                                                                                                               \
        _Pragma("unroll") for (int kk_ = 0; kk_ < 4; ++kk_) if ((i) == kk_) TQKV_STAMP(3 + 3 * kk_ + (p));             \
    } while (0)
#define TQKV_TRACE_STORE(lo, hi)                                                                                       \
    do {                                                                                                               \
        if (lane == 0 && blockIdx.x < kTraceWGs) {                                                                     \
            _Pragma("unroll") for (int k_ = (lo); k_ < (hi); ++k_)                                                     \
                g_phase_trace[((size_t)blockIdx.x * 8 + wave) * kTraceSlots + k_] = trv_[k_];                          \
        }                                                                                                              \
    } while (0)
#else
#define TQKV_TRACE_DECL
#define TQKV_STAMP(k) ((void)0)
#define TQKV_CLOCK(k) ((void)0)
#define TQKV_SET(k, v) ((void)0)
#define TQKV_STEP_STAMP(i, p) ((void)0)
#define TQKV_TRACE_STORE(lo, hi) ((void)0)
#endif

namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kTile = 32;        // tokens per inner-loop step
constexpr int kWaves = 4;        // wavefronts per work-group
constexpr int kQStride = 136;    // halfs per fp16 query row in LDS (128 + 8: no bank collisions
                                 // between the 32 rows an MFMA operand read touches)
constexpr int kInitTiles = 2;    // ring tiles issued before the query preparation

union H8 {
    half8_t h;
    uint32_t u[4];
};

__device__ inline float h2f(uint16_t h) { return __half2float(__ushort_as_half(h)); }

__device__ inline uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel)
{
    return __builtin_amdgcn_perm(hi, lo, sel);
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
// The depth is chosen so that a 32-row work-group fits in 80 KiB of LDS
// (two work-groups per compute unit); a 64-row work-group has a compute
// unit to itself and takes twice the depth (with its 32 KiB of query rows).
template <int PRESET, int NQT> struct Ring;
template <int NQT> struct Ring<kPresetK3V4, NQT> {
    static constexpr int kLoads = 4; // ceil(2 * 1920 / 1024)
    static constexpr int kDepth = 4 * NQT;
};
template <int NQT> struct Ring<kPresetK4V4, NQT> {
    static constexpr int kLoads = 5; // ceil(2 * 2176 / 1024)
    static constexpr int kDepth = 3 * NQT;
};
template <int NQT> struct Ring<kPresetK8V4, NQT> {
    static constexpr int kLoads = 7; // ceil(2 * 3168 / 1024)
    static constexpr int kDepth = 2 * NQT;
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(4))) const int32_t const_i32_t;

// s_waitcnt vmcnt(N) with a compile-time N; the memory clobber keeps the
// compiler from moving LDS reads of the waited-for slot above it.
template <int N> __device__ inline void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ inline void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// s_waitcnt vmcnt(0) that the compiler sees (the waits above are opaque to
// it): after it, the compiler takes every memory instruction it issued
// itself as complete.  It counts only its own loads and stores, not the
// ring's DMA (inline asm), so wherever it believes one of its own may still
// be in flight it waits with vmcnt(0), which in hardware also waits for
// every ring tile in flight.
__device__ inline void wait_vm0_known() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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

// 16-byte-per-lane global -> LDS loads: lane l's 16 bytes land at LDS byte
// lds_base + 16 * l.  Written as inline assembly so that the compiler's wait
// insertion does not treat them as pending writes to every LDS location (it
// would wait for the whole ring before each LDS read); their completion is
// tracked explicitly with wait_ring().  Inline memory operations the
// compiler cannot see can only make its own waits longer, never shorter,
// because loads complete in order.  M0 is not used by any other instruction
// of this kernel.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// per-lane 64-bit address
__device__ inline void dma16(const void *g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(g), "s"(lds_base)
                 : "memory", "m0");
}
// wave-uniform base in SGPRs + per-lane 32-bit byte offset
__device__ inline void dma16_s(const void *base, uint32_t off, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(lds_base)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Loads 4g .. 4g + n - 1 of a tile: one M0 write, then immediate offsets
// (global_load_lds adds the instruction offset to the global address and to
// the LDS destination alike); the tile's last load takes voff_last.
template <int N, bool LAST>
__device__ inline void dma_group(const void *base, uint32_t voff, uint32_t voff_last, uint32_t lds_base)
{
    static_assert(N >= 1 && N <= 4, "group size");
    const uint32_t vl = LAST ? voff_last : voff;
    if constexpr (N == 1) {
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, %1"
                     :
                     : "v"(voff), "s"(base), "s"(lds_base), "v"(vl)
                     : "memory", "m0");
    } else if constexpr (N == 2) {
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
                     "global_load_lds_dwordx4 %3, %1 offset:1024"
                     :
                     : "v"(voff), "s"(base), "s"(lds_base), "v"(vl)
                     : "memory", "m0");
    } else if constexpr (N == 3) {
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:1024\n\tglobal_load_lds_dwordx4 %3, %1 offset:2048"
                     :
                     : "v"(voff), "s"(base), "s"(lds_base), "v"(vl)
                     : "memory", "m0");
    } else {
        asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
                     "global_load_lds_dwordx4 %0, %1 offset:1024\n\tglobal_load_lds_dwordx4 %0, %1 offset:2048\n\t"
                     "global_load_lds_dwordx4 %3, %1 offset:3072"
                     :
                     : "v"(voff), "s"(base), "s"(lds_base), "v"(vl)
                     : "memory", "m0");
    }
}

// Issue the loads of tile kt (blocks 2kt, 2kt+1 of this unit) into the
// ring slot at LDS address slot_lds.  Load j covers tile bytes
// [1024 j, 1024 j + 1024); the last load's lanes past the tile end re-read
// its final 16 B (voff_last = min(16 lane, tile bytes - 16 - 1024 j)).  A
// tile whose second block lies past the unit's last block (odd block count)
// clamps every load to the first block; the missing half is only ever
// masked.
template <int PRESET>
__device__ inline void issue_tile(const uint8_t *ubase, int kt, int nblk, uint32_t slot_lds, uint32_t voff,
                                  uint32_t voff_last, int lane)
{
    using L = Layout<PRESET>;
    constexpr int LPT = Ring<PRESET, 1>::kLoads;
    const uint8_t *src = ubase + (size_t)(2 * kt) * L::kBlockBytes;
    if (__builtin_expect(2 * kt + 1 < nblk, 1)) {
        if constexpr (LPT <= 4) {
            dma_group<LPT, true>(src, voff, voff_last, slot_lds);
        } else {
            static_assert(LPT <= 8, "loads per tile");
            dma_group<4, false>(src, voff, voff_last, slot_lds);
            dma_group<LPT - 4, true>(src + 4096, voff, voff_last, slot_lds + 4096);
        }
    } else {
#pragma unroll
        for (int j = 0; j < LPT; ++j)
            dma16_s(src, (uint32_t)min(1024 * j + 16 * lane, L::kBlockBytes - 16), slot_lds + 1024 * j);
    }
}

// The same for a paged cache, where the tile's two blocks sit at unrelated
// addresses src0 and src1 (both = false: the tile has only its first block).
// Loads before the block boundary read src0, loads after it src1; the one
// load that straddles the boundary (block bytes are a multiple of 16, so
// the boundary falls between two lanes) takes a per-lane address.
template <int PRESET>
__device__ inline void issue_tile_paged(const uint8_t *src0, const uint8_t *src1, bool both, uint32_t slot_lds,
                                        uint32_t voff, uint32_t voff_last, int lane)
{
    using L = Layout<PRESET>;
    constexpr int LPT = Ring<PRESET, 1>::kLoads, BB = L::kBlockBytes;
    constexpr int JS = BB / 1024;                      // the straddling load
    constexpr int kSplitLane = (BB - 1024 * JS) / 16; // its first lane in block 1
    static_assert(BB % 16 == 0 && kSplitLane > 0 && JS < LPT - 1, "tile split");
    if (__builtin_expect(both, 1)) {
#pragma unroll
        for (int j = 0; j < JS; ++j)
            dma16_s(src0 + 1024 * j, voff, slot_lds + 1024 * j);
        const uint8_t *ps = (lane < kSplitLane) ? src0 + (1024 * JS + 16 * lane)
                                                : src1 + (16 * (lane - kSplitLane));
        dma16(ps, slot_lds + 1024 * JS);
#pragma unroll
        for (int j = JS + 1; j < LPT - 1; ++j)
            dma16_s(src1 + (1024 * j - BB), voff, slot_lds + 1024 * j);
        dma16_s(src1 + (1024 * (LPT - 1) - BB), voff_last, slot_lds + 1024 * (LPT - 1));
    } else {
#pragma unroll
        for (int j = 0; j < LPT; ++j)
            dma16_s(src0, (uint32_t)min(1024 * j + 16 * lane, BB - 16), slot_lds + 1024 * j);
    }
}

// Maximum / sum of a per-lane value over the two lane halves (lanes l and
// l ^ 32 hold the same query row): one v_permlane32_swap.
__device__ inline void swap_halves(float x, float &a, float &b)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(r[0]);
    b = __uint_as_float(r[1]);
}
__device__ inline float halves_max(float x)
{
    float a, b;
    swap_halves(x, a, b);
    return fmaxf(a, b);
}
__device__ inline float halves_sum(float x)
{
    float a, b;
    swap_halves(x, a, b);
    return a + b;
}

// Registers of one tile, read back from its ring slot: the key half (the A
// operands of S^T = K Q^T, with the token's key factor folded in) and the
// value half (value nibbles and per-token scale/zero), read at different
// times by the software pipeline below.
template <int PRESET> struct KeyRegs;
template <> struct KeyRegs<kPresetK3V4> {
    uint2 k[3];      // 24 B: this lane's 64 key codes (two 32-code dword triples)
    uint32_t tab[4]; // byte tables of the 8 centroids times n*gamma: lo 0-3, lo 4-7, hi 0-3, hi 4-7
};
template <> struct KeyRegs<kPresetK4V4> {
    u32x4 k[2];      // 32 B: this lane's 64 key nibbles (one dword per 8 coordinates)
    uint32_t tab[4]; // byte tables of the 8 level magnitudes times n*gamma: lo 0-3, lo 4-7, hi 0-3, hi 4-7
};
template <> struct KeyRegs<kPresetK8V4> {
    u32x4 k[4];  // 64 B: this lane's 64 e4m3 key codes
    uint32_t kf; // the token's key scale (fp16) in both halves
};
struct ValRegs {
    u32x4 v[2];         // value nibbles of blocks 0/1 (8-token runs at 4 d's)
    u32x4 vs[2], vz[2]; // value scale / zero (fp16) of the lane's tokens 16s + 8h + 0..7
};

// Token of the 32-token tile that MFMA row m stands for: bits 2 and 3 of m
// swapped.  With this order the C registers 8s..8s+7 of lane half h hold
// tokens 16s + 8h + 0..7, which are the 8 consecutive tokens the value
// operand of k-step s reads at one d.
__device__ inline int tile_token_of_row(int m)
{
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

__device__ inline uint32_t hmul2(uint32_t a, uint32_t b)
{
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) * __builtin_bit_cast(half2_t, b));
}

// n * gamma of token tok of a Lloyd-Max block, in binary32 (the product of
// two binary16 values is exact there)
template <typename L> __device__ inline float key_factor(const uint8_t *blk, int tok)
{
    const uint16_t n = *reinterpret_cast<const uint16_t *>(blk + L::kMeta0 + 2 * (tok & 15));
    const uint16_t g = *reinterpret_cast<const uint16_t *>(blk + L::kMeta1 + 2 * (tok & 15));
    return h2f(n) * h2f(g);
}

// Byte tables (lo 0-3, lo 4-7, hi 0-3, hi 4-7) of the 8 binary16 values
// lv[j] * f, each rounded once from binary32, for v_perm_b32 lookups.
__device__ inline void level_table(uint32_t (&tab)[4], const float *lv, float f)
{
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        c[j] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)(lv[2 * j] * f), (_Float16)(lv[2 * j + 1] * f)});
    tab[0] = perm(c[1], c[0], 0x06040200u);
    tab[1] = perm(c[3], c[2], 0x06040200u);
    tab[2] = perm(c[1], c[0], 0x07050301u);
    tab[3] = perm(c[3], c[2], 0x07050301u);
}

// The lane's key codes and key factor.  The factor (the per-token key scale,
// or n * gamma) multiplies the key operand instead of the score column: for
// FP8 with one packed fp16 multiply per code pair (the scale operand of
// v_cvt_scalef32_pk_f16_fp8 only applies a power of two), for the 3- and
// 4-bit codes through a per-lane table of 8 scaled levels (binary32 products
// rounded once to binary16, then 4 byte permutes per tile; the 16-level
// codebook is symmetric, so its table holds the magnitudes and the code's
// sign bit becomes the fp16 sign).
template <int PRESET>
__device__ inline void read_keys(KeyRegs<PRESET> &t, const uint8_t *slot, int lane)
{
    using L = Layout<PRESET>;
    const int h = lane >> 5, m = lane & 31;
    const int tok = tile_token_of_row(m);
    const uint8_t *blk = slot + (tok >> 4) * L::kBlockBytes;
    const uint8_t *kb = blk + (tok & 15) * L::kKeyBytesPerToken;
    if constexpr (PRESET == kPresetK3V4) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
            t.k[j] = *reinterpret_cast<const uint2 *>(kb + 24 * h + 8 * j);
        level_table(t.tab, kCentroid, key_factor<L>(blk, tok));
    } else if constexpr (PRESET == kPresetK4V4) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            t.k[j] = *reinterpret_cast<const u32x4 *>(kb + 32 * h + 16 * j);
        // magnitudes: levels 8..15 of the ascending codebook
        level_table(t.tab, kCentroid16 + 8, key_factor<L>(blk, tok));
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            t.k[j] = *reinterpret_cast<const u32x4 *>(kb + 64 * h + 16 * j);
        const uint32_t f = *reinterpret_cast<const uint16_t *>(blk + L::kMeta0 + 2 * (tok & 15));
        t.kf = f | (f << 16);
    }
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
        t.vs[s] = *reinterpret_cast<const u32x4 *>(bs + L::kVScale + 16 * h);
        t.vz[s] = *reinterpret_cast<const u32x4 *>(bs + L::kVZero + 16 * h);
    }
}

// 4 packed 3-bit codes (one per byte, values 0..7) -> 4 fp16 table entries
__device__ inline void k3_lookup(const uint32_t (&tab)[4], uint32_t sel, uint32_t &out01, uint32_t &out23)
{
    const uint32_t lo = perm(tab[1], tab[0], sel);
    const uint32_t hi = perm(tab[3], tab[2], sel);
    out01 = perm(hi, lo, 0x05010400u);
    out23 = perm(hi, lo, 0x07030602u);
}

// A operand of k-step ks of S^T = K Q^T: coordinates 64h + 8ks + 0..7 of
// this lane's token, times its key factor.
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
        k3_lookup(t.tab, sa, o.u[0], o.u[1]);
        k3_lookup(t.tab, sb, o.u[2], o.u[3]);
    } else if constexpr (PRESET == kPresetK4V4) {
        // dword ks of the lane's eight: byte b holds coordinate b (low
        // nibble) and b + 4 (high nibble); nibble bits 0-2 index the
        // magnitude table, bit 3 is the sign
        const uint32_t d = t.k[ks >> 2][ks & 3];
        const uint32_t ia = d & 0x07070707u, ib = (d >> 4) & 0x07070707u;
        const uint32_t la = perm(t.tab[1], t.tab[0], ia), lb = perm(t.tab[1], t.tab[0], ib);
        const uint32_t ha = perm(t.tab[3], t.tab[2], ia) | ((d << 4) & 0x80808080u);
        const uint32_t hb = perm(t.tab[3], t.tab[2], ib) | (d & 0x80808080u);
        o.u[0] = perm(ha, la, 0x05010400u);
        o.u[1] = perm(ha, la, 0x07030602u);
        o.u[2] = perm(hb, lb, 0x05010400u);
        o.u[3] = perm(hb, lb, 0x07030602u);
    } else {
        const uint32_t a = t.k[ks >> 1][2 * (ks & 1)], b = t.k[ks >> 1][2 * (ks & 1) + 1];
        const half2_t f = __builtin_bit_cast(half2_t, t.kf);
        const half2_t x0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, false) * f;
        const half2_t x1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, true) * f;
        const half2_t x2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false) * f;
        const half2_t x3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true) * f;
        o.u[0] = __builtin_bit_cast(uint32_t, x0);
        o.u[1] = __builtin_bit_cast(uint32_t, x1);
        o.u[2] = __builtin_bit_cast(uint32_t, x2);
        o.u[3] = __builtin_bit_cast(uint32_t, x3);
    }
    return o.h;
}

// S^T = K Q^T for one tile; QB[qt][ks] is the query B operand of k-step ks
// (coordinates 64h + 8ks + 0..7 of this lane's query row 32qt + lane%32).
// TR: the operands swap roles (the register contents are the same), giving
// S = Q K^T: lane l holds token column l%32 and rows 8(v/4) + 4h + v%4.
template <int PRESET, int NQT, bool TR>
__device__ inline void qk_tile(const KeyRegs<PRESET> &k, const half8_t (&QB)[NQT][8], floatx16 (&S)[NQT])
{
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
        S[qt] = floatx16{0};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        const half8_t A = key_operand<PRESET>(k, ks);
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
            S[qt] = TR ? __builtin_amdgcn_mfma_f32_32x32x16_f16(QB[qt][ks], A, S[qt], 0, 0, 0)
                       : __builtin_amdgcn_mfma_f32_32x32x16_f16(A, QB[qt][ks], S[qt], 0, 0, 0);
    }
}

// A operand of O^T += V^T P^T for d-tile dt (d = 4i + dt) and k-step s
// (tokens 16s + 8h + 0..7).  The nibbles are used as binary16 bit patterns:
// a low nibble c is the subnormal c * 2^-24, a high nibble the subnormal
// 16c * 2^-24 (gfx950's f16 MFMA multiplies subnormal inputs exactly), so
// one mask per half-pair builds the operand; the epilogue rescales even d by
// 2^24 and odd d by 2^20.
__device__ inline half8_t value_operand(const u32x4 (&v)[2], int dt, int s)
{
    const int e = dt >> 1;
    const uint32_t mask = (dt & 1) ? 0x00F000F0u : 0x000F000Fu;
    const uint32_t wa = v[s][2 * e], wb = v[s][2 * e + 1];
    H8 o;
    o.u[0] = wa & mask;
    o.u[1] = (wa >> 8) & mask;
    o.u[2] = wb & mask;
    o.u[3] = (wb >> 8) & mask;
    return o.h;
}

// Lazy rescaling: the running row maximum m only moves when a tile's maximum
// exceeds it by more than kRescaleSlack (log2 units), so probabilities are
// below 2^2.9 < 7.47.  The largest binary16 min-max value scale is
// f16((65504 + 65504) / 15) = 8736, and 7.47 * 8736 < 65504: P * vscale
// stays inside binary16 range.
constexpr float kRescaleSlack = 2.9f;

// Online-softmax state of the lane's query rows (one per 32-row tile).
template <int NQT> struct SoftState {
    float m[NQT], l[NQT], z[NQT];
};

// LDS barrier: the wavefront's LDS operations are complete before it
// arrives, and no LDS access moves across it in either direction.  (The
// ring's outstanding global->LDS loads are not waited for.)
__device__ inline void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The binary16 +-1 entries H[o][16ks + 8h + j], j = 0..7, of the Sylvester
// Hadamard matrix (H[i][k] = (-1)^popcount(i & k)) for output coordinate o:
// the A operand of k-step ks of the query rotation.  The sign splits over
// the disjoint bit ranges of 16ks + 8h and j.
__device__ inline half8_t hadamard_operand(int o, int ks, int h)
{
    const uint32_t flip = (__builtin_popcount(o & (16 * ks + 8 * h)) & 1) ? 0x80008000u : 0u;
    H8 r;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const uint32_t lo = (__builtin_popcount(o & (2 * jj)) & 1) ? 0xBC00u : 0x3C00u;
        const uint32_t hi = (__builtin_popcount(o & (2 * jj + 1)) & 1) ? 0xBC00u : 0x3C00u;
        r.u[jj] = (lo | (hi << 16)) ^ flip;
    }
    return r.h;
}

// TR (units of at most 8 query rows, NQT = 1): the scores are computed
// transposed (one token per lane, rows 4h + v in registers v = 0..3), so the
// softmax of a tile touches 4 registers per lane instead of 16; P reaches
// the P V product's B operand layout (one row per lane) through a small LDS
// block.  The accumulators and the merge are those of the plain path.
template <int PRESET, int NQT, bool PAGED, bool TR>
__global__ __launch_bounds__(256, NQT == 1 ? 2 : 1) void verify_kernel(VerifyArgs a)
{
    static_assert(!TR || NQT == 1, "the transposed path is for one row tile");
    constexpr int RP = 32 * NQT; // padded rows
    constexpr int LPT = Ring<PRESET, NQT>::kLoads, DEPTH = Ring<PRESET, NQT>::kDepth;
    constexpr int kSlotBytes = LPT * 1024;
    // query region: the unit's raw rows (fp32: 512 B, fp16: 256 B each),
    // then, in place, the fp16 operand rows (kQStride halfs each)
    constexpr int kQRegion = RP * kD * 4;
    static_assert(RP * kQStride * 2 <= kQRegion, "query region");
    constexpr int kRingBytes = kWaves * DEPTH * kSlotBytes;
    // merge region: every wavefront's accumulator slots + per-row states
    constexpr int kCombos = 4 * NQT; // (row tile, C-register quad) pairs
    constexpr int kXBytes = kWaves * kCombos * 4 * 64 * 16;
    constexpr int kMergeBytes = kXBytes + kWaves * RP * 16;
    constexpr int kLdsBytes = (kQRegion + kRingBytes) > kMergeBytes ? (kQRegion + kRingBytes) : kMergeBytes;
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];

    const int lane = threadIdx.x & 63;
    // wavefront index as a scalar: every quantity derived from it (the tile
    // range, the ring slot, the wait counts) stays in SGPRs and uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, col = lane & 31;
    // work item of this work-group: (unit, key range, row tile).  Work-groups
    // are dealt to the 8 XCDs round-robin by index; consecutive items (the
    // row tiles and neighbouring key ranges of one unit) go to one XCD, so
    // they share its L2 (tiles read twice, partial results)
    int item = blockIdx.x;
    if ((gridDim.x & 7) == 0)
        item = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    // a work-group covers NQT consecutive 32-row tiles of the unit (its
    // partial states keep the per-32-row-tile layout combine_kernel reads)
    const int nwt = (a.nrt + NQT - 1) / NQT;
    const int rt = item % nwt, us = item / nwt;
    const int unit = us / a.nsplit, split = us % a.nsplit;
    const int row0 = RP * rt;  // first query row of this work-group
    const int tile0 = NQT * rt; // its first 32-row tile
    const int b = unit / a.Hk, hk = unit % a.Hk;
    const int Lr = a.seq_lens[b];
    const int L = Lr < 0 ? 0 : (Lr > a.max_seq ? a.max_seq : Lr);
    // this sequence's queries: nq of them, query n in row qt0 + n * qts of Q
    // and out; they are the last nq tokens of the sequence
    int nq = a.N, qt0 = b, qts = a.B;
    if (a.cu_q) {
        qt0 = a.cu_q[b];
        nq = min(max(a.cu_q[b + 1] - qt0, 0), a.N);
        qts = 1;
    }
    const int Rb = a.G * nq; // query rows of this unit
    if (row0 >= Rb)
        return; // a row tile past a short sequence's rows: nothing to do
    // row r of the unit is query head hk * G + r % G of query r / G; the
    // quotient comes from a float reciprocal (exact: with r < 2^20 the
    // rounding error of (r + 0.5) * rcp(G) stays far below the distance
    // 0.5 / G of (r + 0.5) / G to the nearest integer)
    const float rcpG = __builtin_amdgcn_rcpf((float)a.G);
    auto row_token = [&](int r) { return (int)(((float)r + 0.5f) * rcpG); };

    // this wavefront's tiles [kt0, kt1): the unit's tiles are cut into
    // nsplit work-group ranges, each range into 4 wavefront runs
    const int tiles = (L + kTile - 1) / kTile;
    const int tpw = (tiles + a.nsplit - 1) / a.nsplit;
    const int wt0 = min(split * tpw, tiles), wt1 = min(wt0 + tpw, tiles);
    const int tpv = (wt1 - wt0 + kWaves - 1) / kWaves;
    const int kt0 = min(wt0 + wave * tpv, wt1), kt1 = min(kt0 + tpv, wt1);
    const int ntile = kt1 - kt0;

    using L_ = Layout<PRESET>;
    const uint8_t *ubase = a.base + (size_t)unit * a.nblk * L_::kBlockBytes; // contiguous cache
    const uint32_t lds0 = (uint32_t)(size_t)(lds_void_t *)lds;
    const uint32_t ring_lds = lds0 + kQRegion + wave * DEPTH * kSlotBytes;
    const uint8_t *ring = lds + kQRegion + wave * DEPTH * kSlotBytes;
    _Float16 *qs = reinterpret_cast<_Float16 *>(lds);

    // ------------------------------------------------------------ prologue
    // the fused store's new tokens [tn0, L) of this unit that fall in this
    // work-group's key range
    const int tn0 = (a.Knew != nullptr) ? L - nq : L;
    const int wn0 = max(tn0, wt0 * kTile), wn1 = min(L, wt1 * kTile); // this work-group's share
    // paged cache: the page ids of this wavefront's blocks 2 kt0 + [0, 128)
    // (lane l of pidv[c]: block 2 kt0 + 64 c + l; the launch plan keeps a
    // wavefront at no more than 64 tiles).  Ids outside the pool read page
    // 0, so no load leaves the pool whatever the table holds.
    const int nbl = (L + kBlockTokens - 1) / kBlockTokens; // blocks holding tokens
    const int32_t *brow = PAGED ? a.btab + (size_t)b * a.bstride : nullptr;
    int pidv[2] = {0, 0};

    // 2. the first ring tiles.  The ring fills progressively (at most two
    //    tiles per step): a load instruction waits at issue while the memory
    //    pipeline is full, so a deep prefill would hold the wavefront long
    //    before any tile could be processed.
    const uint32_t voff = 16 * lane;
    const uint32_t voff_last = (uint32_t)min(16 * lane, 2 * L_::kBlockBytes - 16 - 1024 * (LPT - 1));
    int issued = 0; // tiles of this wavefront issued so far (wave-uniform)
    // queue the loads of this wavefront's tile t (tile kt0 + t of the unit)
    auto issue = [&](int t, uint32_t slot) {
        if constexpr (!PAGED) {
            issue_tile<PRESET>(ubase, kt0 + t, a.nblk, slot, voff, voff_last, lane);
        } else {
            const int j = 2 * t;
            int p0, p1;
            if (j < 64) {
                p0 = __builtin_amdgcn_readlane(pidv[0], j);
                p1 = __builtin_amdgcn_readlane(pidv[0], j + 1);
            } else {
                p0 = __builtin_amdgcn_readlane(pidv[1], (j - 64) & 63);
                p1 = __builtin_amdgcn_readlane(pidv[1], (j - 63) & 63);
            }
            const uint8_t *src0 = a.base + ((size_t)p0 * a.Hk + hk) * L_::kBlockBytes;
            const uint8_t *src1 = a.base + ((size_t)p1 * a.Hk + hk) * L_::kBlockBytes;
            issue_tile_paged<PRESET>(src0, src1, 2 * (kt0 + t) + 1 < nbl, slot, voff, voff_last, lane);
        }
    };
    // the cache block holding token t, for the fused store (null: a page id
    // outside the pool, nothing is stored)
    auto store_block = [&](int t) -> uint8_t * {
        if constexpr (!PAGED) {
            return a.wbase + ((size_t)unit * a.nblk + (t >> 4)) * L_::kBlockBytes;
        } else {
            const int p = brow[t >> 4];
            return (p >= 0 && p < a.npages) ? a.wbase + ((size_t)p * a.Hk + hk) * L_::kBlockBytes : nullptr;
        }
    };
    // tiles holding new tokens are loaded only after they have been stored
    // (step 3)
    const int pre = min(kInitTiles, max(0, min(ntile, (tn0 - kt0 * kTile) / kTile)));
    // 1. the query rows, the page ids and the first ring tiles
    auto start_loads = [&]() {
        // the unit's raw query rows -> LDS, 1 KiB per load (2 fp32 or 4
        // fp16 rows).  Padding rows re-read row 0 and are zeroed below.
        // Every wavefront queues these loads before any wavefront queues
        // ring loads, so the query does not wait behind the key stream.
        {
            const int esz = a.q_f16 ? 2 : 4;
            const int rshift = a.q_f16 ? 4 : 5; // lanes per row: 16 or 32
            const int rpi = 64 >> rshift;       // rows per load
            const int rsub = lane >> rshift, cb = 16 * (lane & ((1 << rshift) - 1));
            for (int J = wave; J < RP / rpi; J += kWaves) {
                const int r = row0 + J * rpi + rsub;
                const int rs = r < Rb ? r : 0;
                const int n = row_token(rs), g = rs - n * a.G;
                const uint8_t *src = static_cast<const uint8_t *>(a.Q) +
                                     ((size_t)(qt0 + n * qts) * a.Hq + hk * a.G + g) * kD * esz + cb;
                dma16(src, lds0 + 1024 * J);
            }
        }
        if constexpr (PAGED) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const int j = 2 * kt0 + 64 * c + lane;
                const int p = (j < nbl) ? brow[j] : 0;
                pidv[c] = (p >= 0 && p < a.npages) ? p : 0;
            }
        }
        __builtin_amdgcn_s_barrier();
        for (; issued < pre; ++issued)
            issue(issued, ring_lds + issued * kSlotBytes);
    };

    // 3. Fused store: the work-group whose key range holds new tokens of
    //    this unit quantises them into the cache first (the bytes tqkv_store
    //    writes), spread over its four wavefronts, and waits until all of its
    //    stores are complete before any wavefront loads a tile that holds
    //    them.  (Work-groups of the other row tiles store the same tokens
    //    again: identical bytes.)
    //    This wavefront's first two token-heads are loaded before the
    //    query rows, so their memory latency overlaps the query and ring
    //    loads.  The loads and the stores are all in this branch, which
    //    ends in a wait the compiler sees: no path past it leaves one in
    //    its books (it would wait for the query and ring loads too).
    if (wn0 < wn1) {
        quant::TokenHead nx1{0, 0, 0, 0}, nx2{0, 0, 0, 0};
        if (wn0 + wave < wn1) {
            const int t = wn0 + wave, t2 = min(t + kWaves, wn1 - 1);
            const size_t src = ((size_t)(qt0 + (t - tn0) * qts) * a.Hk + hk) * kD;
            const size_t src2 = ((size_t)(qt0 + (t2 - tn0) * qts) * a.Hk + hk) * kD;
            nx1 = quant::load_token_head(a.Knew + src, a.Vnew + src, lane);
            nx2 = quant::load_token_head(a.Knew + src2, a.Vnew + src2, lane);
        }
        start_loads();
        // two token-heads per wavefront at a time, both loaded up front (the
        // first two at the kernel start)
        for (int t = wn0 + wave; t < wn1; t += 2 * kWaves) {
            const int t2 = t + kWaves;
            quant::TokenHead x = nx1, x2 = nx2;
            if (t != wn0 + wave) {
                const size_t src = ((size_t)(qt0 + (t - tn0) * qts) * a.Hk + hk) * kD;
                const size_t src2 = ((size_t)(qt0 + (min(t2, wn1 - 1) - tn0) * qts) * a.Hk + hk) * kD;
                x = quant::load_token_head(a.Knew + src, a.Vnew + src, lane);
                x2 = quant::load_token_head(a.Knew + src2, a.Vnew + src2, lane);
            }
            uint8_t *blk = store_block(t);
            if (t2 < wn1) {
                // both records first (two independent exchange chains the
                // compiler interleaves), then the stores
                const quant::Record r1 = quant::quantize_record<PRESET>(x, lane);
                const quant::Record r2 = quant::quantize_record<PRESET>(x2, lane);
                uint8_t *blk2 = store_block(t2);
                if (blk)
                    quant::store_record<PRESET>(blk, t & 15, r1, lane);
                if (blk2)
                    quant::store_record<PRESET>(blk2, t2 & 15, r2, lane);
            } else {
                // (the second token-head's loads are consumed all the same,
                // so that no path leaves them pending)
                asm volatile("" ::"v"(x2.k0), "v"(x2.k1), "v"(x2.v0), "v"(x2.v1));
                const quant::Record r1 = quant::quantize_record<PRESET>(x, lane);
                if (blk)
                    quant::store_record<PRESET>(blk, t & 15, r1, lane);
            }
        }
        // every store of this work-group complete (and, the wait being one
        // the compiler sees, no input load left pending in its books: it
        // would otherwise wait for the query and the first ring tiles before
        // reusing those registers)
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    } else {
        start_loads();
    }
    for (; issued < min(kInitTiles, ntile); ++issued)
        issue(issued, ring_lds + issued * kSlotBytes);

    // 4. state set-up while the loads are in flight
    int erow[NQT]; // effective end of this lane's query rows (causal window)
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const int rr = row0 + 32 * qt + col;
        const int n = row_token(rr);
        erow[qt] = (rr < Rb) ? (a.causal ? min(L - nq + n + 1, L) : L) : 0;
    }
    // every row sees every token below emin: tiles ending there need no mask
    const int emin = a.causal ? (L - nq + 1) : L;
    floatx16 acc[4][NQT];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            acc[dt][qt] = floatx16{0};
            asm volatile("" : "+v"(acc[dt][qt])); // zeroed here, under the load latency
        }
    SoftState<NQT> st;
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        st.m[qt] = -__builtin_inff();
        st.l[qt] = 0.0f;
        st.z[qt] = 0.0f;
    }
    // TR state: rows 4h + v (v < 4) of this lane half; the running max is
    // the same in every lane of the half, the sums are this lane's token's
    // share (summed over the half at the end); ttok = the lane's token.  The
    // running max starts at kNoMax, a finite stand-in for -inf far below any
    // score (|q.k| * scale < 1e12 for binary16 inputs), so the first tile's
    // rescale and a row that never sees a token need no special case
    // (exp2(kNoMax - m) = 0, exp2(-inf - kNoMax) = 0).
    constexpr float kNoMax = -1e30f;
    float mT[4], lT[4], zT[4];
    int erowT[4];
    const int ttok = tile_token_of_row(col);
    if constexpr (TR) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int rr = row0 + 4 * h + v;
            const int n = row_token(rr);
            erowT[v] = (rr < Rb) ? (a.causal ? min(L - nq + n + 1, L) : L) : 0;
            mT[v] = kNoMax;
            lT[v] = 0.0f;
            zT[v] = 0.0f;
        }
    }
    H8 Pp[NQT][2]; // P_{i-1} * vscale: the B operands of the pending P V
    u32x4 Vp[2];   // value nibbles of tile i-1 (A operands of the pending P V)
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int s = 0; s < 2; ++s)
            Pp[qt][s].h = half8_t{0, 0, 0, 0, 0, 0, 0, 0};
    Vp[0] = u32x4{0, 0, 0, 0};
    Vp[1] = u32x4{0, 0, 0, 0};

    wait_ring<LPT>(issued); // this wavefront's query loads have landed
    lds_barrier();          // ... and every other wavefront's

    // 5. scale (softmax scale * log2 e: the softmax runs in base 2) and round
    //    to binary16; thread t converts CPT coordinates of row t / TPR
    constexpr int CPT = 16 * NQT, TPR = kD / CPT;
    {
        const int rr = threadIdx.x / TPR, c0 = (threadIdx.x % TPR) * CPT;
        uint32_t qh[CPT / 2];
        if (a.q_f16) {
            const _Float16 *src = reinterpret_cast<const _Float16 *>(lds + rr * 256) + c0;
#pragma unroll
            for (int c = 0; c < CPT; c += 8) {
                const half8_t x = *reinterpret_cast<const half8_t *>(src + c);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const half2_t p = half2_t{(_Float16)((float)x[2 * j] * a.qscale),
                                              (_Float16)((float)x[2 * j + 1] * a.qscale)};
                    qh[c / 2 + j] = __builtin_bit_cast(uint32_t, p);
                }
            }
        } else {
            const float *src = reinterpret_cast<const float *>(lds + rr * 512) + c0;
#pragma unroll
            for (int c = 0; c < CPT; c += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(src + c);
                qh[c / 2] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)(x.x * a.qscale), (_Float16)(x.y * a.qscale)});
                qh[c / 2 + 1] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)(x.z * a.qscale), (_Float16)(x.w * a.qscale)});
            }
        }
        if (row0 + rr >= Rb) {
#pragma unroll
            for (int j = 0; j < CPT / 2; ++j)
                qh[j] = 0u;
        }
        lds_barrier(); // every raw row has been read before it is overwritten
        uint32_t *dst = reinterpret_cast<uint32_t *>(qs + rr * kQStride + c0);
#pragma unroll
        for (int j = 0; j < CPT / 2; j += 4)
            *reinterpret_cast<u32x4 *>(dst + j) = u32x4{qh[j], qh[j + 1], qh[j + 2], qh[j + 3]};
        lds_barrier();
    }

    // 6. Lloyd-Max keys: rotate by the normalised WHT, q' = H q / sqrt(128),
    //    as the MFMA product Q'^T = H Q^T; wavefront w computes output
    //    coordinates 32w..32w+31 of every row and writes them back in place
    if constexpr (kLloydMax<PRESET>) {
        half8_t Bq[NQT][8];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
                Bq[qt][ks] = *reinterpret_cast<const half8_t *>(qs + (32 * qt + col) * kQStride + 16 * ks + 8 * h);
        floatx16 C[NQT];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
            C[qt] = floatx16{0};
        const int o = 32 * wave + col;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const half8_t A = hadamard_operand(o, ks, h);
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
                C[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, Bq[qt][ks], C[qt], 0, 0, 0);
        }
        lds_barrier(); // every wavefront has read the unrotated rows
        constexpr float kInvSqrt128 = 0.08838834764831845f;
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // C register 4g + i is output coordinate 32w + 8g + 4h + i of row 32qt + col
                const half2_t p0 = half2_t{(_Float16)(C[qt][4 * g] * kInvSqrt128), (_Float16)(C[qt][4 * g + 1] * kInvSqrt128)};
                const half2_t p1 = half2_t{(_Float16)(C[qt][4 * g + 2] * kInvSqrt128), (_Float16)(C[qt][4 * g + 3] * kInvSqrt128)};
                *reinterpret_cast<uint2 *>(qs + (32 * qt + col) * kQStride + 32 * wave + 8 * g + 4 * h) =
                    make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
            }
        lds_barrier();
    }

    // 7. the QK^T B operands, held in registers for the whole key loop
    half8_t QB[NQT][8];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            QB[qt][ks] = *reinterpret_cast<const half8_t *>(qs + (32 * qt + col) * kQStride + 64 * h + 8 * ks);
    // kept in AGPRs (MFMA reads its A/B operands from either register file),
    // which leaves the VGPRs to the accumulators and the softmax
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks)
            asm volatile("" : "+a"(QB[qt][ks]));
    // TR: each wavefront's two binary16 P blocks (one per tile parity) live
    // in the query region, free from here on (after every wavefront has read
    // its operands).  A block is 9 rows of 32 tokens: rows 0..7 are written
    // every tile, row 8 stays zero and is the B operand of every padding row
    // (lanes of rows 8..31 all read it: one broadcast); both blocks start as
    // zeros (P_{-1} = 0).  Rows are kPRow = 40 halfs (80 B) apart, so the 8
    // live rows' 16-byte reads fall on different banks (at 64 B apart they
    // shared 4 bank groups).
    constexpr int kPRow = 40, kPBlk = 9 * kPRow;
    _Float16 *ptb = reinterpret_cast<_Float16 *>(lds) + wave * 2 * kPBlk;
    const int prow = min(col, 8); // the block row this lane's B operand reads
    if constexpr (TR) {
        static_assert(kWaves * 2 * kPBlk * 2 <= kQRegion && (kPBlk * 2) % 16 == 0, "P blocks");
        lds_barrier();
        for (int j = lane; j < 2 * kPBlk / 8; j += 64)
            reinterpret_cast<u32x4 *>(ptb)[j] = u32x4{0, 0, 0, 0};
    }

    // ------------------------------------------------------------ key loop
    // One step per tile i.  The scores S_i were computed by the step before
    // (the prologue for i = 0).  Step i
    //   1. finds the tile maximum of S_i per row and, when a row maximum grew
    //      (rare after the first tile), rescales the accumulators and the
    //      pending probabilities P_{i-1};
    //   2. adds P_{i-1} V_{i-1} to the accumulators (MFMA) while it turns S_i
    //      into P_i and the sums l, z (VALU), the two interleaved;
    //   3. computes S_{i+1} = K_{i+1} Q^T (MFMA, the key dequantisation
    //      interleaved).
    // The value operands of P V are built from the nibbles right before
    // their MFMAs.  One score buffer suffices: S_i is consumed before
    // S_{i+1} is written.
    floatx16 S[NQT];
    // one more ring tile, if one is pending and its slot has been read
    // (tiles up to i + DEPTH may reuse the slots of tiles <= i)
    auto refill = [&](int i) {
        if (issued < ntile && issued <= i + DEPTH) {
            wait_lgkm0(); // the slot's LDS reads are complete
            issue(issued, ring_lds + (issued % DEPTH) * kSlotBytes);
            ++issued;
        }
    };
    if (ntile > 0) {
        wait_ring<LPT>(issued - 1);
        KeyRegs<PRESET> k0;
        read_keys<PRESET>(k0, ring, lane);
        qk_tile<PRESET, NQT, TR>(k0, QB, S);
    }
    auto step = [&](int i, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int tok0 = (kt0 + i) * kTile;
        // the next tile's keys (the last step re-reads its own; the product is unused)
        int inext = i;
        if (i + 1 < ntile) {
            wait_ring<LPT>(issued - i - 2);
            inext = i + 1;
        }
        ValRegs vr;
        read_values<PRESET>(vr, ring + (i % DEPTH) * kSlotBytes, lane);

        // 1. tile maximum per row; lazy rescale
        // C register v of the lane holds token tok0 + 8h + 16 (v / 8) + v % 8;
        // lim[qt] = how many of the tile's tokens past tok0 + 8h the row sees
        int lim[NQT];
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
            lim[qt] = erow[qt] - tok0 - 8 * h;
        if constexpr (MASKED) {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (16 * (v >> 3) + (v & 7) >= lim[qt])
                        S[qt][v] = -__builtin_inff();
        }
        float tmax[NQT];
        bool grow_any = false;
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            float tm = fmaxf(fmaxf(S[qt][0], S[qt][1]), S[qt][2]);
#pragma unroll
            for (int v = 3; v < 15; v += 2)
                tm = fmaxf(fmaxf(tm, S[qt][v]), S[qt][v + 1]);
            tm = fmaxf(tm, S[qt][15]);
            tmax[qt] = halves_max(tm); // the row's maximum score in this tile
            grow_any |= (st.m[qt] == -__builtin_inff()) ? (tmax[qt] > -__builtin_inff())
                                                          : (tmax[qt] - st.m[qt] > kRescaleSlack);
        }
        if (__builtin_expect(__any(grow_any), 0)) {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                // every row moves its max up to the tile max (if higher); the
                // accumulators and P_{i-1} (both relative to the old max)
                // shrink by alpha; a row that had no max yet holds zeros
                if (tmax[qt] > st.m[qt]) {
                    const float alpha = (st.m[qt] == -__builtin_inff()) ? 0.0f
                                                                         : __builtin_amdgcn_exp2f(st.m[qt] - tmax[qt]);
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
                        acc[dt][qt] *= alpha;
                    const _Float16 ah = (_Float16)alpha;
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        Pp[qt][s].h *= ah;
                    st.l[qt] *= alpha;
                    st.z[qt] *= alpha;
                    st.m[qt] = tmax[qt];
                }
            }
        }

        // 2. O^T += V_{i-1}^T P_{i-1}^T (MFMA, zero operands at i = 0) while
        //    S_i becomes P_i = exp2(S_i - m) (fp16), l += sum P_i,
        //    z += sum P_i * zero and the next B operand P_i * vscale (VALU).
        //    The two are interleaved by hand: after each MFMA one share of
        //    the softmax work (two scores of both lane halves), with the
        //    compiler's scheduler fenced off so the pairing stays.
        {
            float msub[NQT];
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
                msub[qt] = (st.m[qt] == -__builtin_inff()) ? 0.0f : st.m[qt];
            H8 Pn[NQT][2];
            auto softmax_share = [&](int qt, int s, int j) {
                const int v = 8 * s + 2 * j;
                const float p0 = __builtin_amdgcn_exp2f(S[qt][v] - msub[qt]);
                const float p1 = __builtin_amdgcn_exp2f(S[qt][v + 1] - msub[qt]);
                const half2_t ph = half2_t{(_Float16)p0, (_Float16)p1};
                uint32_t vs = vr.vs[s][j], vz = vr.vz[s][j];
                if constexpr (MASKED) {
                    // fields of invisible tokens never enter (they may hold anything)
                    const uint32_t keep = ((16 * s + 2 * j < lim[qt]) ? 0x0000FFFFu : 0u) |
                                          ((16 * s + 2 * j + 1 < lim[qt]) ? 0xFFFF0000u : 0u);
                    vs &= keep;
                    vz &= keep;
                }
                st.l[qt] = __builtin_amdgcn_fdot2(ph, half2_t{(_Float16)1.0f, (_Float16)1.0f}, st.l[qt], false);
                st.z[qt] = __builtin_amdgcn_fdot2(ph, __builtin_bit_cast(half2_t, vz), st.z[qt], false);
                Pn[qt][s].u[j] = __builtin_bit_cast(uint32_t, ph * __builtin_bit_cast(half2_t, vs));
            };
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(value_operand(Vp, dt, s), Pp[qt][s].h,
                                                                             acc[dt][qt], 0, 0, 0);
                        softmax_share(qt, s, dt); // 16 NQT shares: (qt, s, j = dt)
                        if constexpr (!MASKED)
                            __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    Pp[qt][s] = Pn[qt][s];
            // the new P and sums are complete here: their arithmetic must not
            // sink past the ring refill into the next part
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    asm volatile("" : "+v"(Pp[qt][s].h));
                asm volatile("" : "+v"(st.l[qt]), "+v"(st.z[qt]));
            }
        }
        refill(i);

        // 3. S_{i+1} = K_{i+1} Q^T (MFMA; the keys become operands on the way)
        KeyRegs<PRESET> kn;
        read_keys<PRESET>(kn, ring + (inext % DEPTH) * kSlotBytes, lane);
        qk_tile<PRESET, NQT, TR>(kn, QB, S);
        Vp[0] = vr.v[0];
        Vp[1] = vr.v[1];
        refill(i);
    };

    // TR step i (the scores S_i, transposed, were computed by the step
    // before):
    //   1. masks them and checks whether any row's scores exceed its max by
    //      more than the slack (rare after the first tile); if so the row
    //      maxima move (cross-lane max over the lane half) and everything
    //      relative to the old maxima shrinks;
    //   2. adds P_{i-1} V_{i-1} (MFMA; P_{i-1} * vscale read back from its
    //      LDS block as the B operand, one row per lane) while S_i becomes
    //      P_i (4 exponentials per lane), the sums l, z and P_i * vscale,
    //      written to this tile's LDS block;
    //   3. computes S_{i+1} = Q K_{i+1}^T.
    auto read_pblock = [&](int parity, H8 (&Pq)[2]) {
        const _Float16 *pb = ptb + parity * kPBlk + prow * kPRow + 8 * h;
#pragma unroll
        for (int s = 0; s < 2; ++s)
            Pq[s].h = *reinterpret_cast<const half8_t *>(pb + 16 * s);
    };
    auto step_tr = [&](int i, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int tok0 = (kt0 + i) * kTile;
        int inext = i;
        if (i + 1 < ntile) {
            wait_ring<LPT>(issued - i - 2);
            inext = i + 1;
        }
        const uint8_t *slot = ring + (i % DEPTH) * kSlotBytes;
        // value nibbles of tile i (A operands of its P V, next step) and the
        // value scale / zero of this lane's token
        u32x4 vn[2];
#pragma unroll
        for (int s = 0; s < 2; ++s)
            vn[s] = *reinterpret_cast<const u32x4 *>(slot + s * L_::kBlockBytes + L_::kValOff + (2 * col + h) * 16);
        const uint8_t *fb = slot + (ttok >> 4) * L_::kBlockBytes + 2 * (ttok & 15);
        float vsc = h2f(*reinterpret_cast<const uint16_t *>(fb + L_::kVScale));
        float vze = h2f(*reinterpret_cast<const uint16_t *>(fb + L_::kVZero));
        H8 Pq[2];
        read_pblock((i - 1) & 1, Pq);

        // 1. masked scores; lazy rescale
        float sv[4], dv[4]; // scores, and scores relative to the running max
        bool grow = false;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            sv[v] = S[0][v];
            if constexpr (MASKED) {
                if (tok0 + ttok >= erowT[v])
                    sv[v] = -__builtin_inff();
            }
            dv[v] = sv[v] - mT[v];
            grow |= dv[v] > kRescaleSlack;
        }
        if (__builtin_expect(__any(grow), 0)) {
            float alphaT[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float tm = sv[v];
                tm = fmaxf(tm, quant::lane_xor<1>(tm, lane));
                tm = fmaxf(tm, quant::lane_xor<2>(tm, lane));
                tm = fmaxf(tm, quant::lane_xor<4>(tm, lane));
                tm = fmaxf(tm, quant::lane_xor<8>(tm, lane));
                tm = fmaxf(tm, quant::lane_xor<16>(tm, lane));
                alphaT[v] = 1.0f;
                if (tm > mT[v]) {
                    alphaT[v] = __builtin_amdgcn_exp2f(mT[v] - tm); // 0 from kNoMax
                    lT[v] *= alphaT[v];
                    zT[v] *= alphaT[v];
                    mT[v] = tm;
                    dv[v] = sv[v] - tm;
                }
            }
            // the accumulators and P_{i-1} hold row col: that row's factor
            float ar = 1.0f;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const float x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alphaT[r & 3]), 32 * (r >> 2)));
                ar = (col == r) ? x : ar;
            }
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                acc[dt][0] *= ar;
            const _Float16 ah = (_Float16)ar;
#pragma unroll
            for (int s = 0; s < 2; ++s)
                Pq[s].h *= ah;
        }

        // 2. P_{i-1} V_{i-1} with the softmax of tile i in between
        if constexpr (MASKED) {
            // fields of tokens past the sequence end never enter (they may hold anything)
            if (tok0 + ttok >= L) {
                vsc = 0.0f;
                vze = 0.0f;
            }
        }
        _Float16 *pw = ptb + (i & 1) * kPBlk + ttok; // row r of this tile's block: pw[kPRow r]
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                acc[dt][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(value_operand(Vp, dt, s), Pq[s].h, acc[dt][0], 0, 0,
                                                                    0);
                if (s == 0) {
                    const int v = dt;
                    const float pv = __builtin_amdgcn_exp2f(dv[v]);
                    lT[v] += pv;
                    zT[v] = __builtin_fmaf(pv, vze, zT[v]);
                    pw[kPRow * (4 * h + v)] = (_Float16)(pv * vsc);
                }
            }
#pragma unroll
        for (int v = 0; v < 4; ++v)
            asm volatile("" : "+v"(lT[v]), "+v"(zT[v]));
        Vp[0] = vn[0];
        Vp[1] = vn[1];
        refill(i);

        // 3. S_{i+1} = Q K_{i+1}^T
        KeyRegs<PRESET> kn;
        read_keys<PRESET>(kn, ring + (inext % DEPTH) * kSlotBytes, lane);
        qk_tile<PRESET, NQT, TR>(kn, QB, S);
        refill(i);
    };

    // tiles [0, nfast) need no mask; the sequence's last tiles (the causal
    // window and the partial tail) run through the masked variant
    const int nfast = max(0, min(ntile, (emin - kt0 * kTile) / kTile));
    int i = 0;
    if constexpr (TR) {
        for (; i < nfast; ++i)
            step_tr(i, std::false_type{});
        for (; i < ntile; ++i)
            step_tr(i, std::true_type{});
        // P V of the last tile
        if (ntile > 0) {
            H8 Pq[2];
            read_pblock((ntile - 1) & 1, Pq);
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    acc[dt][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(value_operand(Vp, dt, s), Pq[s].h, acc[dt][0], 0,
                                                                        0, 0);
        }
    } else {
        for (; i < nfast; ++i)
            step(i, std::false_type{});
        for (; i < ntile; ++i)
            step(i, std::true_type{});
        // P V of the last tile
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(value_operand(Vp, dt, s), Pp[qt][s].h,
                                                                         acc[dt][qt], 0, 0, 0);
    }

    // ---------------------------------------------------------------- merge
    // The four wavefronts hold softmax states of the same 32 rows over
    // different tokens.  Each stores its accumulators in LDS in register
    // layout (lane-major float4s, no repacking) and its row states; wavefront
    // w then reduces C-register quad aa = w of all four: lane (col, h) ends
    // up with row lrow = col, coordinates d = 4 (8w + 4h + j) + dt
    // (j, dt = 0..3), i.e. four float4s of the output row.
    __syncthreads(); // every wavefront is done with the ring and the query rows
    float4 *xbuf = reinterpret_cast<float4 *>(lds);           // [w][qt][aa][dt][lane]
    float4 *sbuf = reinterpret_cast<float4 *>(lds + kXBytes); // [w][row]: m, l, z
    if constexpr (TR) {
        // rows 4h + v: the sums over the half's 32 lanes (tokens); rows 8..31
        // are padding
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float ls = lT[v], zs = zT[v];
            ls += quant::lane_xor<1>(ls, lane);
            zs += quant::lane_xor<1>(zs, lane);
            ls += quant::lane_xor<2>(ls, lane);
            zs += quant::lane_xor<2>(zs, lane);
            ls += quant::lane_xor<4>(ls, lane);
            zs += quant::lane_xor<4>(zs, lane);
            ls += quant::lane_xor<8>(ls, lane);
            zs += quant::lane_xor<8>(zs, lane);
            ls += quant::lane_xor<16>(ls, lane);
            zs += quant::lane_xor<16>(zs, lane);
            if (col == 0)
                sbuf[wave * RP + 4 * h + v] = make_float4(mT[v], ls, zs, 0.0f);
        }
        if (h == 0 && col >= 8)
            sbuf[wave * RP + col] = make_float4(-__builtin_inff(), 0.0f, 0.0f, 0.0f);
    } else {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            // softmax sums of the two lane halves (same rows, different tokens)
            const float ls = halves_sum(st.l[qt]), zs = halves_sum(st.z[qt]);
            if (h == 0)
                sbuf[wave * RP + 32 * qt + col] = make_float4(st.m[qt], ls, zs, 0.0f);
        }
    }
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int aa = 0; aa < 4; ++aa)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                xbuf[(((wave * NQT + qt) * 4 + aa) * 4 + dt) * 64 + lane] =
                    make_float4(acc[dt][qt][4 * aa], acc[dt][qt][4 * aa + 1], acc[dt][qt][4 * aa + 2],
                                acc[dt][qt][4 * aa + 3]);
    __syncthreads();
    const int lrow = col; // row within each 32-row tile
    float M[NQT], Ls[NQT];
    float O[NQT][4][4]; // [qt][j][dt]: row 32 qt + lrow, coordinate 4 (8 wave + 4h + j) + dt
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        float4 ms[kWaves];
        M[qt] = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            ms[w] = sbuf[w * RP + 32 * qt + lrow];
            M[qt] = fmaxf(M[qt], ms[w].x);
        }
        float al[kWaves], Zs = 0.0f;
        Ls[qt] = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            al[w] = (ms[w].x == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(ms[w].x - M[qt]);
            Ls[qt] = __builtin_fmaf(al[w], ms[w].y, Ls[qt]);
            Zs = __builtin_fmaf(al[w], ms[w].z, Zs);
        }
        // normalised output O = (sum_w al_w acc_w * 2^24 (even d) or 2^20
        // (odd d) + Zs) / Ls: the value operand carried c * 2^-24 (even d)
        // and 16c * 2^-24 (odd d).  Ls == 0: the row saw no token here
        // (weight 0 below, NaN if nothing else contributes); a NaN Ls
        // propagates.
        const float inv = (Ls[qt] != 0.0f) ? 1.0f / Ls[qt] : 0.0f;
        float ke[kWaves], ko[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            ke[w] = al[w] * (16777216.0f * inv);
            ko[w] = al[w] * (1048576.0f * inv);
        }
        const float zo = Zs * inv;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const float *kw = (dt & 1) ? ko : ke;
            float o[4] = {zo, zo, zo, zo};
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float4 x = xbuf[(((w * NQT + qt) * 4 + wave) * 4 + dt) * 64 + lane];
                o[0] = __builtin_fmaf(kw[w], x.x, o[0]);
                o[1] = __builtin_fmaf(kw[w], x.y, o[1]);
                o[2] = __builtin_fmaf(kw[w], x.z, o[2]);
                o[3] = __builtin_fmaf(kw[w], x.w, o[3]);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
                O[qt][j][dt] = o[j];
        }
    }

    // ------------------------------------------- output or partial state
    // One key range: the output rows (NaN where no token was visible).
    // Several: the normalised partial outputs (binary16, saturated to the
    // finite range, NaN kept) and their (max, sum) go to the workspace, where
    // combine_kernel merges the ranges.  A normalised partial output is a
    // convex combination of dequantised values, so binary16 keeps it to
    // 2^-11 relative.  The rows are
    // transposed through LDS so that every store instruction writes whole
    // 512-byte rows (full cache lines) instead of 16-byte pieces of 32 rows.
    constexpr int kOStride = kD + 4; // floats per LDS row (bank spread)
    // partial states of the 32-row tile t of this work-group's unit
    auto part_slot = [&](int t) { return ((size_t)(unit * a.nrt + t) * a.nsplit + split) * 32; };
    // (partial states are written non-temporally: combine_kernel reads them
    // once, from memory, and they need no write-back at the kernel boundary)
    if (a.nsplit > 1 && wave == 0 && h == 0) {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
            if (tile0 + qt < a.nrt) {
                float *pm = reinterpret_cast<float *>(&a.part_ml[part_slot(tile0 + qt) + lrow]);
                __builtin_nontemporal_store(M[qt], pm);
                __builtin_nontemporal_store(Ls[qt], pm + 1);
            }
    }
    if (a.nsplit == 1) {
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
            if (Ls[qt] == 0.0f) {
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        O[qt][j][k] = __builtin_nanf("");
            }
    }
    __syncthreads(); // every wavefront has read the merge buffer
    float *ob = reinterpret_cast<float *>(lds); // [RP rows][kOStride]
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<float4 *>(ob + (32 * qt + lrow) * kOStride + 4 * (8 * wave + 4 * h + j)) =
                make_float4(O[qt][j][0], O[qt][j][1], O[qt][j][2], O[qt][j][3]);
    __syncthreads();
    if (a.nsplit == 1) {
#pragma unroll
        for (int k = 0; k < RP * kD / 4 / 256; ++k) {
            const int f4 = threadIdx.x + 256 * k; // float4 index, row-major
            const int r = f4 >> 5, c = (f4 & 31) * 4;
            const int grow = row0 + r;
            if (grow >= Rb)
                continue;
            const int n = row_token(grow), g = grow - n * a.G;
            float *dst = a.out + ((size_t)(qt0 + n * qts) * a.Hq + hk * a.G + g) * kD;
            *reinterpret_cast<float4 *>(dst + c) = *reinterpret_cast<const float4 *>(ob + r * kOStride + c);
        }
    } else {
#pragma unroll
        for (int k = 0; k < RP * kD / 8 / 256; ++k) {
            const int e8 = threadIdx.x + 256 * k; // 8-element chunk, row-major
            const int r = e8 >> 4, c = (e8 & 15) * 8;
            if (tile0 + (r >> 5) >= a.nrt)
                continue; // the second tile of a unit with an odd tile count
            _Float16 *pbase = a.part_o + (part_slot(tile0 + (r >> 5)) + (r & 31)) * kD;
            const float4 x0 = *reinterpret_cast<const float4 *>(ob + r * kOStride + c);
            const float4 x1 = *reinterpret_cast<const float4 *>(ob + r * kOStride + c + 4);
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float p = fminf(fmaxf(xs[2 * i], -65504.0f), 65504.0f);
                float q = fminf(fmaxf(xs[2 * i + 1], -65504.0f), 65504.0f);
                p = (xs[2 * i] == xs[2 * i]) ? p : xs[2 * i];
                q = (xs[2 * i + 1] == xs[2 * i + 1]) ? q : xs[2 * i + 1];
                w[i] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)p, (_Float16)q});
            }
            __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4 *>(pbase + c));
        }
    }
}

// A operand of k-step ks of S^T = K Q^T from FP8 codes, without the key
// scale (it multiplies the score column instead).
__device__ inline half8_t key_operand_fp8(const KeyRegs<kPresetK8V4> &t, int ks)
{
    const uint32_t a = t.k[ks >> 1][2 * (ks & 1)], b = t.k[ks >> 1][2 * (ks & 1) + 1];
    H8 o;
    o.u[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, false));
    o.u[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(a, 1.0f, true));
    o.u[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false));
    o.u[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, true));
    return o.h;
}

__device__ inline float max16(const floatx16 &x)
{
    float m = fmaxf(fmaxf(x[0], x[1]), x[2]);
#pragma unroll
    for (int v = 3; v < 15; v += 2)
        m = fmaxf(fmaxf(m, x[v]), x[v + 1]);
    return fmaxf(m, x[15]);
}

// ---------------------------------------------------------------------------
// Work-groups of 64 query rows: eight independent wavefronts.
//
// A wavefront on gfx950 issues one VALU instruction at most about every 8
// cycles, while a SIMD accepts one about every 4 to 5 when two wavefronts
// feed it, and the matrix core working for one wavefront overlaps the VALU
// work of the other (measured with probe kernels).  The 64-row work-group
// therefore runs two wavefronts per SIMD, each streaming its own run of
// 32-token tiles through its own LDS ring and computing everything for all
// 64 rows (each key and value tile is dequantised once): S = K Q^T, the
// online softmax, O += P V and the row sums.  The two wavefronts of a SIMD
// never wait for each other, so the stalls of one (LDS latency, matrix-core
// results) are filled by the other's instructions.  To fit two wavefronts'
// registers (256 each) the fp16 query operands stay in LDS and are read per
// k-step; the accumulators (128 registers) stay in registers.
// ---------------------------------------------------------------------------
template <int PRESET> struct WideRing;
template <> struct WideRing<kPresetK3V4> { static constexpr int kDepth = 4; };
template <> struct WideRing<kPresetK4V4> { static constexpr int kDepth = 3; };
template <> struct WideRing<kPresetK8V4> { static constexpr int kDepth = 2; };

template <int PRESET, bool PAGED, int kW>
__global__ __launch_bounds__(64 * kW, 1) void verify_wide_kernel(VerifyArgs a)
{
    static_assert(kW == 4 || kW == 8, "wavefronts per work-group");
    constexpr int NQT = 2, RP = 64;
    constexpr int LPT = Ring<PRESET, 1>::kLoads, DEPTH = WideRing<PRESET>::kDepth;
    constexpr int kSlotBytes = LPT * 1024;
    // query rows: raw, then the fp16 operand rows in place (resident)
    constexpr int kQRegion = RP * kD * 4;
    static_assert(RP * kQStride * 2 <= kQRegion, "query region");
    constexpr int kRingBytes = kW * DEPTH * kSlotBytes;
    // merge: four wavefronts' accumulators at a time (register layout) and
    // the (m, l, z) states of all eight
    constexpr int kXBytes = 4 * NQT * 4 * 4 * 64 * 16;
    constexpr int kMergeBytes = kXBytes + kW * RP * 16;
    constexpr int kLdsBytes = (kQRegion + kRingBytes) > kMergeBytes ? (kQRegion + kRingBytes) : kMergeBytes;
    static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
    static_assert(DEPTH * LPT <= 63 && DEPTH <= 8, "vmcnt range");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, col = lane & 31;
    TQKV_TRACE_DECL;
    TQKV_STAMP(0);
    int item = blockIdx.x;
    if ((gridDim.x & 7) == 0)
        item = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int nwt = (a.nrt + NQT - 1) / NQT;
    const int rt = item % nwt, us = item / nwt;
    const int unit = us / a.nsplit, split = us % a.nsplit;
    const int row0 = RP * rt;
    const int tile0 = NQT * rt;
    const int b = unit / a.Hk, hk = unit % a.Hk;
    const int Lr = a.seq_lens[b];
    const int L = Lr < 0 ? 0 : (Lr > a.max_seq ? a.max_seq : Lr);
    int nq = a.N, qt0 = b, qts = a.B;
    if (a.cu_q) {
        qt0 = a.cu_q[b];
        nq = min(max(a.cu_q[b + 1] - qt0, 0), a.N);
        qts = 1;
    }
    const int Rb = a.G * nq;
    if (row0 >= Rb)
        return;
    const float rcpG = __builtin_amdgcn_rcpf((float)a.G);
    auto row_token = [&](int r) { return (int)(((float)r + 0.5f) * rcpG); };

    // the work-group's tiles [wt0, wt1).  The two wavefronts of a SIMD do
    // not advance at the same rate (the older one is issued first), so the
    // tiles are handed out on demand: wavefront w starts with tiles
    // wt0 + w + kW j (j < DEPTH) and then claims one tile per step from a
    // work-group counter, always in increasing order
    const int tiles = (L + kTile - 1) / kTile;
    const int tpw = (tiles + a.nsplit - 1) / a.nsplit;
    const int wt0 = min(split * tpw, tiles), wt1 = min(wt0 + tpw, tiles);

    using L_ = Layout<PRESET>;
    const uint8_t *ubase = a.base + (size_t)unit * a.nblk * L_::kBlockBytes;
    const uint32_t lds0 = (uint32_t)(size_t)(lds_void_t *)lds;
    const uint32_t ring_lds = lds0 + kQRegion + wave * DEPTH * kSlotBytes;
    const uint8_t *ring = lds + kQRegion + wave * DEPTH * kSlotBytes;
    _Float16 *qs = reinterpret_cast<_Float16 *>(lds);

    // ------------------------------------------------------------ prologue
    const int tn0 = (a.Knew != nullptr) ? L - nq : L;
    const int wn0 = max(tn0, wt0 * kTile), wn1 = min(L, wt1 * kTile);
    const int nbl = (L + kBlockTokens - 1) / kBlockTokens;
    const int32_t *brow = PAGED ? a.btab + (size_t)b * a.bstride : nullptr;
    // the same row for the ring's page ids, read through the scalar cache: a
    // vector load there would make the compiler wait for it with vmcnt(0),
    // i.e. for every ring tile in flight (the table is not written during
    // the launch)
    const const_i32_t *brow_s = (const const_i32_t *)(uintptr_t)brow;
    // 1. raw query rows -> LDS, every wavefront's queued before any ring load
    auto load_query = [&]() {
        const int esz = a.q_f16 ? 2 : 4;
        const int rshift = a.q_f16 ? 4 : 5;
        const int rpi = 64 >> rshift;
        const int rsub = lane >> rshift, cb = 16 * (lane & ((1 << rshift) - 1));
        for (int J = wave; J < RP / rpi; J += kW) {
            const int r = row0 + J * rpi + rsub;
            const int rs = r < Rb ? r : 0;
            const int n = row_token(rs), g = rs - n * a.G;
            const uint8_t *src = static_cast<const uint8_t *>(a.Q) +
                                 ((size_t)(qt0 + n * qts) * a.Hq + hk * a.G + g) * kD * esz + cb;
            dma16(src, lds0 + 1024 * J);
        }
        __builtin_amdgcn_s_barrier();
    };

    // 2. the first ring tiles
    const uint32_t voff = 16 * lane;
    const uint32_t voff_last = (uint32_t)min(16 * lane, 2 * L_::kBlockBytes - 16 - 1024 * (LPT - 1));
    int issued = 0; // tiles this wavefront has put in flight
    // tile t (absolute index) into the ring slot at LDS address slot
    auto issue = [&](int t, uint32_t slot) {
        if constexpr (!PAGED) {
            issue_tile<PRESET>(ubase, t, a.nblk, slot, voff, voff_last, lane);
        } else {
            // the page ids of the tile's two blocks (uniform loads; ids out
            // of range read page 0, whose tokens the mask never admits)
            const int j = 2 * t;
            const bool two = j + 1 < nbl;
            int p0 = brow_s[j], p1 = two ? brow_s[j + 1] : 0;
            p0 = (p0 >= 0 && p0 < a.npages) ? p0 : 0;
            p1 = (p1 >= 0 && p1 < a.npages) ? p1 : 0;
            const uint8_t *src0 = a.base + ((size_t)p0 * a.Hk + hk) * L_::kBlockBytes;
            const uint8_t *src1 = a.base + ((size_t)p1 * a.Hk + hk) * L_::kBlockBytes;
            issue_tile_paged<PRESET>(src0, src1, two, slot, voff, voff_last, lane);
        }
    };
    // the slot window: tq[j] is the tile in the j-th oldest slot in flight
    // (wt1 or more: none)
    int tq[DEPTH];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j)
        tq[j] = min(wt0 + wave + kW * j, wt1);
    auto store_block = [&](int t) -> uint8_t * {
        if constexpr (!PAGED) {
            return a.wbase + ((size_t)unit * a.nblk + (t >> 4)) * L_::kBlockBytes;
        } else {
            const int p = brow[t >> 4];
            return (p >= 0 && p < a.npages) ? a.wbase + ((size_t)p * a.Hk + hk) * L_::kBlockBytes : nullptr;
        }
    };
    // Ring prefill: a plain verify issues one tile per wavefront now, the
    // rest from the first step; loads issued here compete with the query
    // loads for the memory system, and a wavefront whose load issue stalls
    // (the memory pipeline full) holds up the work-group barriers of the
    // query preparation (measured at the PoC shape 0.7 to 1.1 us per call
    // faster than prefilling the whole ring here).  A fused store + verify
    // issues its first tile only once the query rows have landed: the
    // work-groups that store the new tokens end last, and every load the
    // others issue meanwhile competes with their token loads and stores
    // (PoC step 18.6-19.2 against 19.3-20.0 us; the plain verify is 0.1-0.2
    // us slower that way).
    const bool early_tile = a.Knew == nullptr;
    // 3. fused store of this work-group's share of the new tokens, spread
    //    over the wavefronts; complete (the wait for the query rows
    //    below) before any tile holding them is loaded.  Its loads and
    //    stores end in a wait the compiler sees, so that it does not wait
    //    for them (and so for the ring) again in the query preparation
    TQKV_SET(20, wn0 < wn1 ? 1u : 0u);
    if (wn0 < wn1) {
        // this wavefront's first new token-head(s), loaded before the
        // query rows so that their latency overlaps the query loads
        quant::TokenHead nx1{0, 0, 0, 0}, nx2{0, 0, 0, 0};
        if (wn0 + wave < wn1) {
            const int t = wn0 + wave, t2 = min(t + kW, wn1 - 1);
            const size_t src = ((size_t)(qt0 + (t - tn0) * qts) * a.Hk + hk) * kD;
            const size_t src2 = ((size_t)(qt0 + (t2 - tn0) * qts) * a.Hk + hk) * kD;
            nx1 = quant::load_token_head(a.Knew + src, a.Vnew + src, lane);
            nx2 = quant::load_token_head(a.Knew + src2, a.Vnew + src2, lane);
        }
        load_query();
        TQKV_STAMP(16);
        for (int t = wn0 + wave; t < wn1; t += 2 * kW) {
            const int t2 = t + kW;
            quant::TokenHead x = nx1, x2 = nx2;
            if (t != wn0 + wave) {
                const size_t src = ((size_t)(qt0 + (t - tn0) * qts) * a.Hk + hk) * kD;
                const size_t src2 = ((size_t)(qt0 + (min(t2, wn1 - 1) - tn0) * qts) * a.Hk + hk) * kD;
                x = quant::load_token_head(a.Knew + src, a.Vnew + src, lane);
                x2 = quant::load_token_head(a.Knew + src2, a.Vnew + src2, lane);
            }
            uint8_t *blk = store_block(t);
            if (t2 < wn1) {
                const quant::Record r1 = quant::quantize_record<PRESET>(x, lane);
                const quant::Record r2 = quant::quantize_record<PRESET>(x2, lane);
                uint8_t *blk2 = store_block(t2);
                if (blk)
                    quant::store_record<PRESET>(blk, t & 15, r1, lane);
                if (blk2)
                    quant::store_record<PRESET>(blk2, t2 & 15, r2, lane);
            } else {
                asm volatile("" ::"v"(x2.k0), "v"(x2.k1), "v"(x2.v0), "v"(x2.v1));
                const quant::Record r1 = quant::quantize_record<PRESET>(x, lane);
                if (blk)
                    quant::store_record<PRESET>(blk, t & 15, r1, lane);
            }
        }
        TQKV_STAMP(17);
        wait_vm0_known(); // the query rows are waited for next anyway
    } else {
        load_query();
        if (early_tile && tq[0] < wt1 && (tq[0] + 1) * kTile <= tn0) {
            issue(tq[0], ring_lds);
            ++issued;
        }
    }
    // 4. state
    int erow[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const int rr = row0 + 32 * qt + col;
        const int n = row_token(rr);
        erow[qt] = (rr < Rb) ? (a.causal ? min(L - nq + n + 1, L) : L) : 0;
    }
    const int emin = a.causal ? (L - nq + 1) : L;
    const int tmask = emin / kTile; // tiles from here on need the causal / length mask
    // the claim counter lives past the binary16 query rows (written once the
    // raw rows there have been read)
    uint32_t *claim_ctr = reinterpret_cast<uint32_t *>(lds + kQRegion - 16);
    static_assert(RP * kQStride * 2 <= kQRegion - 16, "claim counter");

    // this wavefront's query loads have landed (a wavefront that stored new
    // tokens has waited for its stores too, so after the barrier every new
    // token is in memory; the ring loads of tiles that hold them come later)
    wait_ring<LPT>(issued);
    TQKV_STAMP(1);
    lds_barrier();
    if (!early_tile && issued == 0 && tq[0] < wt1) {
        issue(tq[0], ring_lds);
        ++issued;
    }

    // 5. scale and round to binary16 (thread t: 16 coordinates of row
    //    t / 8, and with four wavefronts of row t / 8 + 32 as well); every
    //    raw row is read before the binary16 rows overwrite them in place
    {
        constexpr int CPT = 16, TPR = kD / CPT, NPASS = 512 / (64 * kW);
        const int c0 = (threadIdx.x % TPR) * CPT;
        uint32_t qh[NPASS][CPT / 2];
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
            const int rr = (int)threadIdx.x / TPR + ps * (64 / NPASS);
            if (a.q_f16) {
                const _Float16 *src = reinterpret_cast<const _Float16 *>(lds + rr * 256) + c0;
#pragma unroll
                for (int c = 0; c < CPT; c += 8) {
                    const half8_t x = *reinterpret_cast<const half8_t *>(src + c);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const half2_t p = half2_t{(_Float16)((float)x[2 * j] * a.qscale),
                                                  (_Float16)((float)x[2 * j + 1] * a.qscale)};
                        qh[ps][c / 2 + j] = __builtin_bit_cast(uint32_t, p);
                    }
                }
            } else {
                const float *src = reinterpret_cast<const float *>(lds + rr * 512) + c0;
#pragma unroll
                for (int c = 0; c < CPT; c += 4) {
                    const float4 x = *reinterpret_cast<const float4 *>(src + c);
                    qh[ps][c / 2] =
                        __builtin_bit_cast(uint32_t, half2_t{(_Float16)(x.x * a.qscale), (_Float16)(x.y * a.qscale)});
                    qh[ps][c / 2 + 1] =
                        __builtin_bit_cast(uint32_t, half2_t{(_Float16)(x.z * a.qscale), (_Float16)(x.w * a.qscale)});
                }
            }
            if (row0 + rr >= Rb) {
#pragma unroll
                for (int j = 0; j < CPT / 2; ++j)
                    qh[ps][j] = 0u;
            }
        }
        lds_barrier();
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
            const int rr = (int)threadIdx.x / TPR + ps * (64 / NPASS);
            uint32_t *dst = reinterpret_cast<uint32_t *>(qs + rr * kQStride + c0);
#pragma unroll
            for (int j = 0; j < CPT / 2; j += 4)
                *reinterpret_cast<u32x4 *>(dst + j) = u32x4{qh[ps][j], qh[ps][j + 1], qh[ps][j + 2], qh[ps][j + 3]};
        }
        if (threadIdx.x == 0)
            *claim_ctr = (uint32_t)(wt0 + kW * DEPTH);
        lds_barrier();
    }

    // 6. Lloyd-Max keys: q' = H q / sqrt(128) as the MFMA product H Q^T;
    //    wavefronts 0..3 compute output coordinates 32w..32w+31
    if constexpr (kLloydMax<PRESET>) {
        floatx16 C[NQT];
        if (wave < 4) {
            half8_t Bq[NQT][8];
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int ks = 0; ks < 8; ++ks)
                    Bq[qt][ks] = *reinterpret_cast<const half8_t *>(qs + (32 * qt + col) * kQStride + 16 * ks + 8 * h);
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
                C[qt] = floatx16{0};
            const int o = 32 * wave + col;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
                const half8_t A = hadamard_operand(o, ks, h);
#pragma unroll
                for (int qt = 0; qt < NQT; ++qt)
                    C[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, Bq[qt][ks], C[qt], 0, 0, 0);
            }
        }
        lds_barrier();
        if (wave < 4) {
            constexpr float kInvSqrt128 = 0.08838834764831845f;
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const half2_t p0 = half2_t{(_Float16)(C[qt][4 * g] * kInvSqrt128), (_Float16)(C[qt][4 * g + 1] * kInvSqrt128)};
                    const half2_t p1 = half2_t{(_Float16)(C[qt][4 * g + 2] * kInvSqrt128), (_Float16)(C[qt][4 * g + 3] * kInvSqrt128)};
                    *reinterpret_cast<uint2 *>(qs + (32 * qt + col) * kQStride + 32 * wave + 8 * g + 4 * h) =
                        make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
                }
        }
        lds_barrier();
    }

    // ------------------------------------------------------------ key loop
    // the rest of the ring prefill (after the fused store: tiles holding new
    // tokens are loaded only once they are stored): the first tile now, if
    // it is not in flight yet, the others from the first step, once its
    // score products are issued (a load instruction waits at issue while the
    // memory pipeline is full, which here it is: the first tiles of every
    // wavefront and the query rows are still in flight)
    auto prefill_rest = [&]() {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j)
            if (issued == j && tq[j] < wt1) {
                issue(tq[j], ring_lds + j * kSlotBytes);
                ++issued;
            }
    };
    if (issued == 0 && tq[0] < wt1) {
        issue(tq[0], ring_lds);
        ++issued;
    }
    TQKV_STAMP(2);
    TQKV_CLOCK(22);
    // the B operand of k-step ks of row tile qt: coordinates 64h + 8ks + 0..7
    // of this lane's query row 32qt + col, read from LDS when needed
    const _Float16 *qrow = qs + col * kQStride + 64 * h;
    auto qop = [&](int qt, int ks) {
        return *reinterpret_cast<const half8_t *>(qrow + 32 * qt * kQStride + 8 * ks);
    };
    floatx16 acc[4][NQT];
    float m[NQT], msub[NQT], thr[NQT];
    // row sums on the matrix core: rows 2qt and 2qt + 1 of `sums` (registers
    // 2qt, 2qt + 1 of the lanes of half 0) are sum_t P_t and sum_t P_t zero_t
    // of row tile qt, accumulated as A P with A's row 2qt all ones and row
    // 2qt + 1 the tokens' zeros
    floatx16 sums = floatx16{0};
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        m[qt] = -__builtin_inff();
        msub[qt] = 0.0f;
        thr[qt] = -__builtin_inff();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            acc[dt][qt] = floatx16{0};
    }
    // Lloyd-Max keys: the subtrahend enters the score MFMA chain as a
    // 32x32x8 product of a ones column pair (k = 0, 1 in lanes 0-31) with the
    // row's -msub split into binary16 hi + lo (exact to 2^-22 relative),
    // instead of 32 subtractions per tile
    const half4_t sub_ones = (h == 0) ? half4_t{(_Float16)1.0f, (_Float16)1.0f, (_Float16)0.0f, (_Float16)0.0f}
                                      : half4_t{(_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f, (_Float16)0.0f};
    uint32_t sub_hl[NQT]; // lanes 0-31: binary16 (-hi, -lo) of the row's subtrahend
    auto split_sub = [&](float x) -> uint32_t {
        const _Float16 hi = (_Float16)x;
        const _Float16 lo = (_Float16)(x - (float)hi);
        return (h == 0) ? __builtin_bit_cast(uint32_t, half2_t{-hi, -lo}) : 0u;
    };
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt)
        sub_hl[qt] = 0u;
    // A operand of the sums of row tile qt: lane column 2qt all ones, lane
    // column 2qt + 1 the zeros of its tokens (one select per dword)
    uint32_t sum_ones[NQT];
    bool sum_zlane[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        sum_ones[qt] = (col == 2 * qt) ? 0x3C003C00u : 0u;
        sum_zlane[qt] = col == 2 * qt + 1;
    }
    // tile i: S = K Q^T, the lazy online-softmax rescale (the running max
    // moves only when a score exceeds it by more than kRescaleSlack; an
    // unset max takes the tile's maximum), P = exp2(S - m) in binary16, the
    // sums l, z, and O += V^T (P vscale)^T
    auto step = [&](int i, int t, auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
        const int tok0 = t * kTile;
        // tile i has landed (in the steady state DEPTH - 1 later tiles are
        // in flight behind it)
        if (issued - i == DEPTH)
            wait_vm<(DEPTH - 1) * LPT>();
        else
            wait_ring<LPT>(issued - i - 1);
        TQKV_STEP_STAMP(i, 0);
        const uint8_t *slot = ring + (i % DEPTH) * kSlotBytes;
        KeyRegs<PRESET> kr;
        read_keys<PRESET>(kr, slot, lane);
        H8 f[2];
        if constexpr (!kLloydMax<PRESET>) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                f[s2].h = *reinterpret_cast<const half8_t *>(slot + s2 * L_::kBlockBytes + L_::kMeta0 + 16 * h);
        }
        floatx16 S[NQT];
        if constexpr (kLloydMax<PRESET>) {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const half4_t bsub = __builtin_bit_cast(half4_t, make_uint2(sub_hl[qt], 0u));
                S[qt] = __builtin_amdgcn_mfma_f32_32x32x8f16(sub_ones, bsub, floatx16{0}, 0, 0, 0);
            }
        }
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            half8_t A;
            if constexpr (kLloydMax<PRESET>)
                A = key_operand<PRESET>(kr, ks);
            else
                A = key_operand_fp8(kr, ks);
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
                S[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                    A, qop(qt, ks), (ks == 0 && !kLloydMax<PRESET>) ? floatx16{0} : S[qt], 0, 0, 0);
        }
        if (i == 0)
            prefill_rest();
        // FP8: each score column times its token's key scale, relative to
        // the subtrahend (Lloyd-Max: already in the MFMA chain); register v
        // holds token tok0 + 8h + 16 (v / 8) + v % 8
        if constexpr (!kLloydMax<PRESET>) {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    S[qt][v] = __builtin_fmaf(S[qt][v], (float)f[v >> 3].h[v & 7], -msub[qt]);
        }
        if constexpr (MASKED) {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const int lim = erow[qt] - tok0 - 8 * h;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (16 * (v >> 3) + (v & 7) >= lim)
                        S[qt][v] = -__builtin_inff();
            }
        }
        float mx[NQT];
        bool grow = false;
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt) {
            mx[qt] = max16(S[qt]);
            grow |= mx[qt] > thr[qt];
        }
        if (__builtin_expect(__any(grow), 0)) {
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                const float tmax = halves_max(mx[qt]) + msub[qt]; // the row's largest score of the tile
                const float mnew = fmaxf(m[qt], tmax);
                const float alpha = (m[qt] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m[qt] - mnew);
                const float snew = (mnew == -__builtin_inff()) ? 0.0f : mnew;
                const float d = snew - msub[qt];
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    S[qt][v] -= d;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    acc[dt][qt] *= alpha;
                sums[2 * qt] *= alpha;
                sums[2 * qt + 1] *= alpha;
                m[qt] = mnew;
                msub[qt] = snew;
                sub_hl[qt] = split_sub(snew);
                thr[qt] = (mnew == -__builtin_inff()) ? -__builtin_inff() : kRescaleSlack;
            }
        }
        TQKV_STEP_STAMP(i, 1);
        ValRegs vr;
        read_values<PRESET>(vr, slot, lane);
        if constexpr (MASKED) {
            // fields of tokens past the sequence end never enter (they may
            // hold anything); the zeros, which the row sums' A operand shares
            // between rows that see a token and rows that do not, are clamped
            // to the finite range (below: P * vscale per row)
            const int lim = L - tok0 - 8 * h;
            const half2_t big = half2_t{(_Float16)65504.0f, (_Float16)65504.0f};
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t keep = ((16 * s2 + 2 * j < lim) ? 0x0000FFFFu : 0u) |
                                          ((16 * s2 + 2 * j + 1 < lim) ? 0xFFFF0000u : 0u);
                    vr.vs[s2][j] &= keep;
                    const uint32_t z = vr.vz[s2][j] & keep;
                    vr.vz[s2][j] = __builtin_bit_cast(
                        uint32_t,
                        __builtin_elementwise_min(__builtin_elementwise_max(__builtin_bit_cast(half2_t, z), -big), big));
                }
        }
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int qt = 0; qt < NQT; ++qt) {
                H8 Bp, Pr, As;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    // (vector elements are copied to scalars first: a bit cast
                    // of an ext_vector_type element reads element 0 in this
                    // compiler)
                    const uint32_t vsj = vr.vs[s2][j], vzj = vr.vz[s2][j];
                    const float p0 = __builtin_amdgcn_exp2f(S[qt][8 * s2 + 2 * j]);
                    const float p1 = __builtin_amdgcn_exp2f(S[qt][8 * s2 + 2 * j + 1]);
                    const half2_t ph = half2_t{(_Float16)p0, (_Float16)p1};
                    Pr.u[j] = __builtin_bit_cast(uint32_t, ph);
                    As.u[j] = sum_zlane[qt] ? vzj : sum_ones[qt];
                    Bp.u[j] = __builtin_bit_cast(uint32_t, ph * __builtin_bit_cast(half2_t, vsj));
                    if constexpr (MASKED) {
                        // masked tiles hold tokens that some rows do not see
                        // (P = 0): P * vscale is kept only where P is not 0,
                        // so that an infinite value scale (values with an
                        // infinity) reaches exactly the rows that see its token
                        // (0 * inf would be NaN); the zeros of the row sums'
                        // A operand, shared by all rows, were clamped above
                        const uint32_t pu = __builtin_bit_cast(uint32_t, ph);
                        Bp.u[j] &= ((pu & 0x00007FFFu) ? 0x0000FFFFu : 0u) | ((pu & 0x7FFF0000u) ? 0xFFFF0000u : 0u);
                    }
                }
                sums = __builtin_amdgcn_mfma_f32_32x32x16_f16(As.h, Pr.h, sums, 0, 0, 0);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    acc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(value_operand(vr.v, dt, s2), Bp.h, acc[dt][qt],
                                                                         0, 0, 0);
            }
    };
    // step i works on tile tq[0] in slot i % DEPTH; the tile claimed during
    // the step refills that slot, and the window moves on
    int i = 0;
    bool more = true; // the counter may still hold tiles for this wavefront
    auto claim = [&]() {
        uint32_t c = 0u;
        if (more && lane == 0)
            c = __hip_atomic_fetch_add(claim_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        return c;
    };
    auto advance = [&](uint32_t c) {
        int nt = wt1;
        if (more) {
            nt = min((int)__builtin_amdgcn_readfirstlane(c), wt1);
            more = nt < wt1;
        }
        if (nt < wt1) {
            wait_lgkm0(); // the slot's LDS reads are complete
            issue(nt, ring_lds + (i % DEPTH) * kSlotBytes);
            ++issued;
        }
#pragma unroll
        for (int j = 0; j + 1 < DEPTH; ++j)
            tq[j] = tq[j + 1];
        tq[DEPTH - 1] = nt;
        ++i;
    };
    while (tq[0] < min(wt1, tmask)) {
        const uint32_t c = claim();
        step(i, tq[0], std::false_type{});
        TQKV_STEP_STAMP(i, 2);
        advance(c);
    }
    while (tq[0] < wt1) {
        const uint32_t c = claim();
        step(i, tq[0], std::true_type{});
        TQKV_STEP_STAMP(i, 2);
        advance(c);
    }

    TQKV_STAMP(15);
    TQKV_CLOCK(23);
    TQKV_TRACE_STORE(0, 18);
    TQKV_TRACE_STORE(20, 24);
    // ---------------------------------------------------------------- merge
    // kW states per row (one per wavefront, over different tokens): first
    // every (m, l, z), then the accumulators in rounds of four wavefronts
    // through the same LDS area (eight wavefronts: 4..7, then 0..3);
    // wavefront w reduces C-register quad aa = w % 4 of row tile w / 4
    // (eight wavefronts) or of both row tiles (four).
    float4 *xbuf = reinterpret_cast<float4 *>(lds); // [w % 4][qt][aa][dt][lane]
    float4 *sbuf = reinterpret_cast<float4 *>(lds + kXBytes); // [w][row]: m, l, z
    __syncthreads(); // every wavefront is done with the ring and the query rows
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
        const float l2 = sums[2 * qt], z2 = sums[2 * qt + 1];
        if (h == 0)
            sbuf[wave * RP + 32 * qt + col] = make_float4(m[qt], l2, z2, 0.0f);
    }
    constexpr int NMQ = 8 / kW; // row tiles this wavefront reduces
    const int aa = wave & 3, lrow = col;
    auto row_tile = [&](int mi) { return (kW == 8) ? (wave >> 2) : mi; };
    auto put_acc = [&]() {
        const int ww = wave & 3;
#pragma unroll
        for (int qt = 0; qt < NQT; ++qt)
#pragma unroll
            for (int a2 = 0; a2 < 4; ++a2)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    xbuf[(((ww * NQT + qt) * 4 + a2) * 4 + dt) * 64 + lane] =
                        make_float4(acc[dt][qt][4 * a2], acc[dt][qt][4 * a2 + 1], acc[dt][qt][4 * a2 + 2],
                                    acc[dt][qt][4 * a2 + 3]);
    };
    if (kW == 4 || wave >= 4)
        put_acc();
    __syncthreads();
    float M[NMQ], Ls[NMQ], al[NMQ][kW], inv[NMQ];
    float O[NMQ][4][4]; // [mi][j][dt]: row 32 mq + lrow, coordinate 4 (8 aa + 4h + j) + dt
#pragma unroll
    for (int mi = 0; mi < NMQ; ++mi) {
        const int mq = row_tile(mi);
        float4 st[kW];
        M[mi] = -__builtin_inff();
#pragma unroll
        for (int w = 0; w < kW; ++w) {
            st[w] = sbuf[w * RP + 32 * mq + lrow];
            M[mi] = fmaxf(M[mi], st[w].x);
        }
        float Zs = 0.0f;
        Ls[mi] = 0.0f;
#pragma unroll
        for (int w = 0; w < kW; ++w) {
            al[mi][w] = (st[w].x == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(st[w].x - M[mi]);
            Ls[mi] = __builtin_fmaf(al[mi][w], st[w].y, Ls[mi]);
            Zs = __builtin_fmaf(al[mi][w], st[w].z, Zs);
        }
        inv[mi] = (Ls[mi] != 0.0f) ? 1.0f / Ls[mi] : 0.0f;
        const float zo = Zs * inv[mi];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                O[mi][j][dt] = zo;
    }
    // normalised output O = (sum_w al_w acc_w * 2^24 (even d) or 2^20 (odd
    // d) + Zs) / Ls: the value operand carried c * 2^-24 (even d) and
    // 16c * 2^-24 (odd d)
    auto gather = [&](int wbase) {
#pragma unroll
        for (int mi = 0; mi < NMQ; ++mi) {
            const int mq = row_tile(mi);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const float k = al[mi][wbase + w] * (((dt & 1) ? 1048576.0f : 16777216.0f) * inv[mi]);
                    const float4 x = xbuf[(((w * NQT + mq) * 4 + aa) * 4 + dt) * 64 + lane];
                    O[mi][0][dt] = __builtin_fmaf(k, x.x, O[mi][0][dt]);
                    O[mi][1][dt] = __builtin_fmaf(k, x.y, O[mi][1][dt]);
                    O[mi][2][dt] = __builtin_fmaf(k, x.z, O[mi][2][dt]);
                    O[mi][3][dt] = __builtin_fmaf(k, x.w, O[mi][3][dt]);
                }
            }
        }
    };
    if constexpr (kW == 8) {
        gather(4);
        __syncthreads();
        if (wave < 4)
            put_acc();
        __syncthreads();
    }
    gather(0);
    TQKV_STAMP(18);

    // ------------------------------------------- output or partial state
    auto part_slot = [&](int t) { return ((size_t)(unit * a.nrt + t) * a.nsplit + split) * 32; };
#pragma unroll
    for (int mi = 0; mi < NMQ; ++mi) {
        const int mq = row_tile(mi);
        if (a.nsplit > 1 && aa == 0 && h == 0 && tile0 + mq < a.nrt) {
            a.part_ml[part_slot(tile0 + mq) + lrow] = make_float2(M[mi], Ls[mi]);
        }
        if (a.nsplit == 1 && Ls[mi] == 0.0f) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    O[mi][j][k] = __builtin_nanf("");
        }
    }
    TQKV_STAMP(19);
    TQKV_TRACE_STORE(18, 20);
    // Outputs straight from the registers (no LDS staging): this thread's
    // row 32 mq + lrow, coordinates 4 (8 aa + 4h + j) + 0..3 for j = 0..3,
    // as four binary32 (the output) or four binary16 (a partial state).
    // (A staging round through LDS for whole-row stores cost 0.2-0.6 us
    // per PoC call more.)
#pragma unroll
    for (int mi = 0; mi < NMQ; ++mi) {
        const int mq = row_tile(mi);
        if (tile0 + mq >= a.nrt)
            continue;
        if (a.nsplit == 1) {
            const int grow = row0 + 32 * mq + lrow;
            if (grow >= Rb)
                continue;
            const int n = row_token(grow), g = grow - n * a.G;
            float *dst = a.out + ((size_t)(qt0 + n * qts) * a.Hq + hk * a.G + g) * kD;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<float4 *>(dst + 4 * (8 * aa + 4 * h + j)) =
                    make_float4(O[mi][j][0], O[mi][j][1], O[mi][j][2], O[mi][j][3]);
            continue;
        }
        // The 16 coordinates are consecutive (32 B): two 16-byte stores,
        // write-back cached so that the halves meet in L2 before memory
        // (8-byte streaming stores wrote 2.3x the partial-state bytes to HBM).
        _Float16 *po = a.part_o + (part_slot(tile0 + mq) + lrow) * kD + 4 * (8 * aa + 4 * h);
        uint32_t w8[8];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                // binary16 range, NaN kept
                const float x0 = O[mi][j][2 * q], x1 = O[mi][j][2 * q + 1];
                float p = fminf(fmaxf(x0, -65504.0f), 65504.0f);
                float r2 = fminf(fmaxf(x1, -65504.0f), 65504.0f);
                p = (x0 == x0) ? p : x0;
                r2 = (x1 == x1) ? r2 : x1;
                w8[2 * j + q] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)p, (_Float16)r2});
            }
        reinterpret_cast<u32x4 *>(po)[0] = u32x4{w8[0], w8[1], w8[2], w8[3]};
        reinterpret_cast<u32x4 *>(po)[1] = u32x4{w8[4], w8[5], w8[6], w8[7]};
    }
}

// Merge of the key ranges of each (b, hk, row tile): out = sum_s w_s O_s /
// sum_s w_s with w_s = exp2(m_s - max_s m_s) * l_s.  A row is merged by GPR
// groups of 32 lanes (one float4 of the row per lane), group j taking the
// j-th contiguous share of the ranges; every lane loads its share's (m, l)
// pairs and partial float4s in one batch (chunks of kCombineChunk), so
// the kernel costs one round trip to memory, and the groups' states are
// then merged through LDS in group order (a fixed order).  Ranges whose
// softmax sum is exactly 0 saw no token and get weight 0; a NaN sum reaches
// the output.  Blocks are dealt to the XCDs like the verify work-groups of
// the same rows, so the partial states are read where they were written.
// GPR grows with the range count (at most 8 ranges per group up to 64
// ranges): with one group per row, 64 ranges took four round trips.
constexpr int kCombineChunk = 8;

template <int GPR> __global__ __launch_bounds__(256) void combine_kernel(VerifyArgs a)
{
    constexpr int RPB = 8 / GPR; // rows per block
    constexpr int kBlocksPerTile = 32 / RPB;
    int blk = blockIdx.x;
    if ((gridDim.x & 7) == 0)
        blk = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
    const int grp = blk / kBlocksPerTile; // (unit, row tile)
    const int gid = threadIdx.x >> 5, part = gid % GPR;
    const int lrow = (blk % kBlocksPerTile) * RPB + gid / GPR; // row within the tile
    const int unit = grp / a.nrt, rt = grp % a.nrt;
    const int row = 32 * rt + lrow;
    const int b = unit / a.Hk, hk = unit % a.Hk;
    int nq = a.N, qt0 = b, qts = a.B;
    if (a.cu_q) {
        qt0 = a.cu_q[b];
        nq = min(max(a.cu_q[b + 1] - qt0, 0), a.N);
        qts = 1;
    }
    const bool valid = unit < a.B * a.Hk && row < a.G * nq;
    const int d = (threadIdx.x & 31) * 4;
    const size_t base = (size_t)grp * a.nsplit * 32 + lrow;
    const int spg = (a.nsplit + GPR - 1) / GPR;
    const int s_begin = min(part * spg, a.nsplit), s_end = valid ? min(s_begin + spg, a.nsplit) : s_begin;
    float M = -__builtin_inff(), den = 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = s_begin; s0 < s_end; s0 += kCombineChunk) {
        float2 ml[kCombineChunk];
        float4 v[kCombineChunk];
        // every load of the chunk is issued before any is used (ranges past
        // the share re-read its last one and get weight 0): a guarded load
        // per range would cost one memory round trip each
#pragma unroll
        for (int j = 0; j < kCombineChunk; ++j) {
            const size_t ix = base + (size_t)min(s0 + j, s_end - 1) * 32;
            ml[j] = a.part_ml[ix];
            const uint2 hv = *reinterpret_cast<const uint2 *>(a.part_o + ix * kD + d);
            const half2_t h0 = __builtin_bit_cast(half2_t, hv.x), h1 = __builtin_bit_cast(half2_t, hv.y);
            v[j] = make_float4((float)h0[0], (float)h0[1], (float)h1[0], (float)h1[1]);
        }
#pragma unroll
        for (int j = 0; j < kCombineChunk; ++j)
            if (s0 + j >= s_end)
                ml[j] = make_float2(-__builtin_inff(), 0.0f);
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
            acc.x = __builtin_fmaf(w, v[j].x, acc.x);
            acc.y = __builtin_fmaf(w, v[j].y, acc.y);
            acc.z = __builtin_fmaf(w, v[j].z, acc.z);
            acc.w = __builtin_fmaf(w, v[j].w, acc.w);
        }
    }
    if constexpr (GPR > 1) {
        // the groups of a row: (M, den, acc) through LDS, merged by group 0
        __shared__ float4 sacc[8][32];
        __shared__ float2 smd[8][32];
        sacc[gid][threadIdx.x & 31] = acc;
        smd[gid][threadIdx.x & 31] = make_float2(M, den);
        __syncthreads();
        if (part != 0)
            return;
        float2 st[GPR];
        float Mt = -__builtin_inff();
#pragma unroll
        for (int j = 0; j < GPR; ++j) {
            st[j] = smd[gid + j][threadIdx.x & 31];
            if (st[j].y != 0.0f)
                Mt = fmaxf(Mt, st[j].x);
        }
        den = 0.0f;
        acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < GPR; ++j) {
            const float w = (st[j].y != 0.0f) ? __builtin_amdgcn_exp2f(st[j].x - Mt) : 0.0f;
            const float4 x = sacc[gid + j][threadIdx.x & 31];
            den = __builtin_fmaf(w, st[j].y, den);
            acc.x = __builtin_fmaf(w, x.x, acc.x);
            acc.y = __builtin_fmaf(w, x.y, acc.y);
            acc.z = __builtin_fmaf(w, x.z, acc.z);
            acc.w = __builtin_fmaf(w, x.w, acc.w);
        }
    }
    if (!valid)
        return;
    const float inv = (den != 0.0f) ? 1.0f / den : __builtin_nanf("");
    const int n = (int)(((float)row + 0.5f) * __builtin_amdgcn_rcpf((float)a.G)), g = row - n * a.G;
    *reinterpret_cast<float4 *>(a.out + ((size_t)(qt0 + n * qts) * a.Hq + hk * a.G + g) * kD + d) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}




template <int KW>
void launch_verify_wide_w(int preset, bool paged, const VerifyArgs &a, hipStream_t s)
{
    const int nwt = (a.nrt + 1) / 2;
    const dim3 grid((unsigned)(a.B * a.Hk * a.nsplit * nwt)), block(64 * KW);
    if (preset == kPresetK3V4) {
        if (paged)
            hipLaunchKernelGGL((verify_wide_kernel<kPresetK3V4, true, KW>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((verify_wide_kernel<kPresetK3V4, false, KW>), grid, block, 0, s, a);
    } else if (preset == kPresetK4V4) {
        if (paged)
            hipLaunchKernelGGL((verify_wide_kernel<kPresetK4V4, true, KW>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((verify_wide_kernel<kPresetK4V4, false, KW>), grid, block, 0, s, a);
    } else {
        if (paged)
            hipLaunchKernelGGL((verify_wide_kernel<kPresetK8V4, true, KW>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((verify_wide_kernel<kPresetK8V4, false, KW>), grid, block, 0, s, a);
    }
}

template <int NQT, bool TR>
void launch_verify_rows(int preset, bool paged, const VerifyArgs &a, hipStream_t s)
{
    const int nwt = (a.nrt + NQT - 1) / NQT;
    const dim3 grid((unsigned)(a.B * a.Hk * a.nsplit * nwt)), block(256);
    if (preset == kPresetK3V4) {
        if (paged)
            hipLaunchKernelGGL((verify_kernel<kPresetK3V4, NQT, true, TR>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((verify_kernel<kPresetK3V4, NQT, false, TR>), grid, block, 0, s, a);
    } else if (preset == kPresetK4V4) {
        if (paged)
            hipLaunchKernelGGL((verify_kernel<kPresetK4V4, NQT, true, TR>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((verify_kernel<kPresetK4V4, NQT, false, TR>), grid, block, 0, s, a);
    } else {
        if (paged)
            hipLaunchKernelGGL((verify_kernel<kPresetK8V4, NQT, true, TR>), grid, block, 0, s, a);
        else
            hipLaunchKernelGGL((verify_kernel<kPresetK8V4, NQT, false, TR>), grid, block, 0, s, a);
    }
}

} // namespace

// nqt: 32-row tiles per work-group (1: two work-groups per compute unit;
// 2: one work-group of 64 rows per compute unit, each tile dequantised once
// for all 64 rows); transposed: the transposed-score path (nqt 1, at most 8
// rows per unit)
hipError_t launch_verify(int preset, bool paged, int nqt, int wide_waves, bool transposed, const VerifyArgs &a,
                         hipStream_t s)
{
    if (nqt == 2 && wide_waves == 4)
        launch_verify_wide_w<4>(preset, paged, a, s);
    else if (nqt == 2)
        launch_verify_wide_w<8>(preset, paged, a, s);
    else if (transposed && a.R <= 8)
        launch_verify_rows<1, true>(preset, paged, a, s);
    else
        launch_verify_rows<1, false>(preset, paged, a, s);
    if (hipGetLastError() != hipSuccess)
        return hipErrorLaunchFailure;
    if (a.nsplit > 1) {
        // 4 GPR blocks of 256 threads per (unit, row tile)
        const int gpr = combine_groups_per_row(a.nsplit);
        const dim3 grid((unsigned)(a.B * a.Hk * a.nrt * 4 * gpr)), block(256);
        if (gpr == 1)
            hipLaunchKernelGGL(combine_kernel<1>, grid, block, 0, s, a);
        else if (gpr == 2)
            hipLaunchKernelGGL(combine_kernel<2>, grid, block, 0, s, a);
        else if (gpr == 4)
            hipLaunchKernelGGL(combine_kernel<4>, grid, block, 0, s, a);
        else
            hipLaunchKernelGGL(combine_kernel<8>, grid, block, 0, s, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

} // namespace tqkv

#ifdef TQKV_PHASE_TRACE
// Copy the phase stamps of the last verify_wide_kernel launch to the host
// (kTraceWGs x 8 wavefronts x kTraceSlots 32-bit words).  Trace builds only.
extern "C" int tqkv_debug_phase_trace(void *host, size_t bytes)
{
    if (bytes > sizeof(tqkv::g_phase_trace))
        return -1;
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(tqkv::g_phase_trace), bytes, 0, hipMemcpyDeviceToHost) == hipSuccess ? 0
                                                                                                                  : -1;
}
#endif
