// Shared definitions of the HIP library: cache layout constants, launch
// descriptors and small device helpers.  Host and device code include it.
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace tqkv {

constexpr int kD = 128;
constexpr int kBlockTokens = 16;
constexpr int kPresetK8V4 = 1;
constexpr int kPresetK3V4 = 2;
constexpr int kPresetK4V4 = 3;
// Lloyd-Max key presets: WHT-rotated keys, codes against the 8- or 16-level
// codebook, fp16 norm and norm-correction fields
template <int P> constexpr bool kLloydMax = (P == kPresetK3V4 || P == kPresetK4V4);

// Byte layout of one 16-token block (see include/tqkv.h for the overview).
//   k3v4_nc: key codes [0,768) 48 B/token | value nibbles [768,1792) |
//            n_h[16] @1792 | gamma_h[16] @1824 | vscale[16] @1856 | vzero[16] @1888
//   k4v4_nc: key nibbles [0,1024) 64 B/token | value nibbles [1024,2048) |
//            n_h[16] @2048 | gamma_h[16] @2080 | vscale[16] @2112 | vzero[16] @2144
//   k8v4:    e4m3 keys [0,2048) 128 B/token | value nibbles [2048,3072) |
//            kscale[16] @3072 | vscale[16] @3104 | vzero[16] @3136
template <int P> struct Layout;
template <> struct Layout<kPresetK3V4> {
    static constexpr int kBlockBytes = 1920;
    static constexpr int kKeyBytesPerToken = 48;
    static constexpr int kValOff = 768;
    static constexpr int kMeta0 = 1792; // n_h
    static constexpr int kMeta1 = 1824; // gamma_h
    static constexpr int kVScale = 1856;
    static constexpr int kVZero = 1888;
};
template <> struct Layout<kPresetK4V4> {
    static constexpr int kBlockBytes = 2176;
    static constexpr int kKeyBytesPerToken = 64;
    static constexpr int kValOff = 1024;
    static constexpr int kMeta0 = 2048; // n_h
    static constexpr int kMeta1 = 2080; // gamma_h
    static constexpr int kVScale = 2112;
    static constexpr int kVZero = 2144;
};
template <> struct Layout<kPresetK8V4> {
    static constexpr int kBlockBytes = 3168;
    static constexpr int kKeyBytesPerToken = 128;
    static constexpr int kValOff = 2048;
    static constexpr int kMeta0 = 3072; // kscale_h
    static constexpr int kMeta1 = -1;
    static constexpr int kVScale = 3104;
    static constexpr int kVZero = 3136;
};

// Value nibble byte p (coordinates 2p | 2p+1) of block token tb lives at this
// offset inside the value region: dword ((i*2+h)*2+e)*2+q with i = p/2,
// e = p%2, h = tb/8, q = (tb/4)%2, byte {0,2,1,3}[tb%4] of that dword.  The
// order lets one 16-byte load per lane of a wavefront fetch, for 32 d-quads
// x 2 token halves, exactly the 8-token runs an MFMA operand needs.
__host__ __device__ inline int val_byte_offset(int tb, int p)
{
    int dw = (((p >> 1) * 2 + (tb >> 3)) * 2 + (p & 1)) * 2 + ((tb >> 2) & 1);
    int pos = ((tb & 1) << 1) | ((tb >> 1) & 1);
    return dw * 4 + pos;
}

// Where token t (row t of K and V [T, Hk, 128]) goes, in this order:
//   step_lens non-null: a speculative step of N tokens per sequence, T = N * B;
//     token t = n * B + b goes to position step_lens[b] - N + n of sequence b
//     (contiguous cache, or paged through the block table btab);
//   slots non-null: paged cache, slot = page * 16 + position in the page;
//   otherwise: contiguous cache, sequence seq_idx[t], position pos[t].
struct StoreArgs {
    uint8_t *base;
    const uint16_t *K;
    const uint16_t *V;
    const int32_t *seq_idx;
    const int32_t *pos;
    const int32_t *slots;
    const int32_t *step_lens;
    const int32_t *btab;
    int B, Hk, max_seq, nblk, T;
    int N, bstride, npages;
};

struct VerifyArgs {
    const uint8_t *base;
    const void *Q;   // [N, B, Hq, 128], fp32 or fp16 (q_f16)
    const int32_t *seq_lens;
    float *out;      // [N, B, Hq, 128]
    // partial states of the key ranges (nsplit > 1), per (unit, row tile) g:
    _Float16 *part_o; // [g][nsplit][32 rows][128] normalised partial outputs (binary16)
    float2 *part_ml; // [g][nsplit][32 rows] (running max in log2 units, softmax sum)
    float qscale;       // softmax scale * log2(e)
    int q_f16;
    int Hk, max_seq, nblk;
    int B, N, Hq, G, R, causal, nsplit;
    int nrt; // row tiles per (b, hk): one work-group each
    // ragged queries (non-null): device [B + 1] prefix sums of the query
    // counts; query n of sequence b is row cu_q[b] + n of Q [*, Hq, 128] and
    // out, and N is the largest count.  Null: Q and out are [N, B, Hq, 128].
    const int32_t *cu_q;
    // paged cache (non-null): device [B, bstride] page ids; block j of
    // sequence b, head hk is at base + (btab[b * bstride + j] * Hk + hk) *
    // block bytes.  Null: block j of unit u = b * Hk + hk is at
    // base + (u * nblk + j) * block bytes.
    const int32_t *btab;
    int bstride, npages;
    // fused store (null for a plain verify): the n_spec new tokens of every
    // sequence, fp16 [N, B, Hk, 128]; token n of sequence b goes to position
    // seq_lens[b] - N + n of the cache before it is attended to
    const uint16_t *Knew, *Vnew;
    uint8_t *wbase; // the cache, writable (== base)
};

// Lane groups of 32 that merge one output row of the key-range merge (at
// most 8 ranges per group up to 64 ranges); the merge launches 4 * that
// many blocks of 256 threads per (unit, 32-row tile).
inline int combine_groups_per_row(int nsplit)
{
    return nsplit <= 8 ? 1 : nsplit <= 16 ? 2 : nsplit <= 32 ? 4 : 8;
}

// Launchers (defined next to their kernels).
hipError_t launch_store(int preset, const StoreArgs &a, hipStream_t s);
hipError_t launch_verify(int preset, bool paged, int nqt, int wide_waves, bool transposed, const VerifyArgs &a,
                         hipStream_t s);

} // namespace tqkv
