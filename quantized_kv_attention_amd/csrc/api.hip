// C ABI of libtqkv.so (declared in include/tqkv.h): argument validation,
// launch planning and status codes.  No device allocation, no host<->device
// copies, no synchronisation.
#include "common.h"
#include "tqkv.h"

#include <atomic>
#include <math.h>
#include <string.h>

namespace {

using namespace tqkv;

// Per-device state, looked up once per device and kept for the process:
// the compute-unit count and the device address of the scratch array of
// tqkv_verify_noalloc.  Both are plain values that any thread may compute
// again; atomics make the concurrent first calls race-free.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices]; // 0 = not probed yet, -1 = not a gfx950 device
std::atomic<void *> g_scratch[kMaxDevices]; // null = not looked up yet

// The workspace of tqkv_verify_noalloc: one array per device, allocated
// when the code object is loaded on that device and held until the process
// ends.  Host code never uses its name as an address (on the host it is a
// stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device.
constexpr size_t kScratchBytes = TQKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Number of compute units of the current device, or a negative status when
// no gfx950 device is current.
int current_device_cus()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TQKV_ERR_DEVICE;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return TQKV_ERR_DEVICE;
        const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        n = ok ? prop.multiProcessorCount : -1;
        g_cu_count[dev].store(n, std::memory_order_relaxed);
    }
    return n > 0 ? n : TQKV_ERR_DEVICE;
}

// Device address of the current device's scratch array (looked up on the
// first call on each device, with that device current), or a negative
// status.
int current_device_scratch(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TQKV_ERR_DEVICE;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return TQKV_ERR_DEVICE;
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return TQKV_OK;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// A cache as the kernels see it: contiguous (btab null: block j of unit
// b * Hk + hk at base + (unit * nblk + j) * block bytes) or paged (block j of
// sequence b in page btab[b * bstride + j] of the pool).
struct View {
    int preset, B, Hk, max_seq; // max_seq: token capacity per sequence
    void *base;
    const int32_t *btab;
    int bstride, npages;
};

int nblocks(int max_seq) { return (max_seq + kBlockTokens - 1) / kBlockTokens; }

bool known_preset(int preset) { return preset == TQKV_K8V4 || preset == TQKV_K3V4_NC || preset == TQKV_K4V4_NC; }
static_assert(TQKV_K8V4 == kPresetK8V4 && TQKV_K3V4_NC == kPresetK3V4 && TQKV_K4V4_NC == kPresetK4V4, "preset ids");
static_assert(Layout<kPresetK8V4>::kBlockBytes == 16 * 198 && Layout<kPresetK3V4>::kBlockBytes == 16 * 120 &&
                  Layout<kPresetK4V4>::kBlockBytes == 16 * 136,
              "block bytes");


int view_of(const tqkv_cache *c, View &v)
{
    if (!c)
        return TQKV_ERR_ARG;
    if (!known_preset(c->preset))
        return TQKV_ERR_ARG;
    if (c->B < 1 || c->Hk < 1 || c->max_seq < 1 || !c->base)
        return TQKV_ERR_ARG;
    if (c->D != TQKV_HEAD_DIM)
        return TQKV_ERR_UNSUPPORTED;
    if (!aligned(c->base, 16))
        return TQKV_ERR_ALIGN;
    v = View{c->preset, c->B, c->Hk, c->max_seq, c->base, nullptr, 0, 0};
    return TQKV_OK;
}

// the pool part of a paged cache (what the store needs)
int check_pool(const tqkv_paged_cache *c)
{
    if (!c)
        return TQKV_ERR_ARG;
    if (!known_preset(c->preset))
        return TQKV_ERR_ARG;
    if (c->Hk < 1 || c->num_pages < 1 || c->num_pages > (INT32_MAX >> 4) || !c->base)
        return TQKV_ERR_ARG;
    if (c->D != TQKV_HEAD_DIM)
        return TQKV_ERR_UNSUPPORTED;
    if (!aligned(c->base, 16))
        return TQKV_ERR_ALIGN;
    return TQKV_OK;
}

int view_of(const tqkv_paged_cache *c, View &v)
{
    int st = check_pool(c);
    if (st != TQKV_OK)
        return st;
    if (!c->block_table || c->B < 1 || c->max_pages < 1)
        return TQKV_ERR_ARG;
    if (c->max_pages > TQKV_MAX_PAGES_PER_SEQ)
        return TQKV_ERR_UNSUPPORTED;
    if (!aligned(c->block_table, 4))
        return TQKV_ERR_ALIGN;
    v = View{c->preset, c->B, c->Hk, c->max_pages * kBlockTokens, c->base, c->block_table, c->max_pages,
             c->num_pages};
    return TQKV_OK;
}

// Longest key range (in 32-token tiles) that the 64-row work-groups run
// with four wavefronts.
constexpr long kWideFourTiles = 32;

// Query rows per work-group: the rows of one KV head are cut into tiles of
// 32 (one MFMA operand height), one work-group each.
int row_tiles(int rows) { return (rows + 31) / 32; }

// A wavefront of a paged verify holds the page ids of at most 64 tiles (two
// VGPRs), so a work-group covers at most 256 tiles of 32 tokens.
constexpr int kPagedTilesPerGroup = 256;

// 32-row tiles per work-group: units with more than one tile of query rows
// take them in pairs (one 64-row work-group per compute unit, every key
// tile dequantised once for all 64 rows); otherwise one (two work-groups
// per compute unit).
int rows_per_group(int rows) { return row_tiles(rows) >= 2 ? 2 : 1; }

// Wavefronts of a 64-row work-group: four (one per SIMD, each taking a
// quarter of the range's tiles; the merge of four 64-row states moves half
// the LDS bytes of eight) when the key ranges are short, eight (two per
// SIMD, which overlap each other's matrix-core and vector work) otherwise.
// Measured at the PoC shape (16 ranges of 16 tiles, same box, graphs over
// cold replicas): k8v4 verify 16.9 us with four against 17.9-18.7 with the
// 32-row work-groups, fused k8v4 step 19.4 against 21.6 with eight, k4v4_nc
// verify 18.0 against 18.5; k3v4_nc, whose key levels are byte-table
// lookups (more vector instructions per tile, which a lone wavefront per
// SIMD issues at half rate), 17.2 with eight against 18.2 with four (16.0-16.2
// against 16.7 once the query preparation no longer waited for the ring),
// and at long context (128-tile ranges) eight wavefronts are faster for every
// preset.
int wide_waves(const View &c, int splits)
{
    if (c.preset == kPresetK3V4)
        return 8;
    const long tiles = (c.max_seq + 31) / 32;
    const long per_range = (tiles + splits - 1) / splits;
    return per_range <= kWideFourTiles ? 4 : 8;
}

// Key-range partitions per (b, hk): one compute unit's worth of work-groups
// per compute unit overall (two 32-row or one 64-row work-group), at least
// one 32-token tile per wavefront.
int plan_splits(const View &c, int num_splits, int cus, int rows)
{
    const int nqt = rows_per_group(rows);
    const long units = (long)c.B * c.Hk * ((row_tiles(rows) + nqt - 1) / nqt);
    const int tiles = (c.max_seq + 31) / 32;
    const int max_useful = (tiles + 3) / 4;
    int s = num_splits;
    if (s <= 0)
        s = (int)((2 / nqt * cus + units - 1) / units);
    if (s > max_useful)
        s = max_useful;
    if (s > 1024)
        s = 1024;
    if (s < 1)
        s = 1;
    if (c.btab) {
        const int need = (tiles + kPagedTilesPerGroup - 1) / kPagedTilesPerGroup;
        if (s < need)
            s = need; // <= 1024 by the page limit per sequence
    }
    return s;
}

// The launches' work-group counts (verify and combine) fit a grid dimension.
bool grid_fits(const View &c, int rows, int splits)
{
    const long rt = row_tiles(rows), nqt = rows_per_group(rows);
    const long verify_groups = (long)c.B * c.Hk * splits * ((rt + nqt - 1) / nqt);
    const long combine_groups = splits > 1 ? (long)c.B * c.Hk * rt * 4 * combine_groups_per_row(splits) : 0;
    return verify_groups <= INT32_MAX && combine_groups <= INT32_MAX;
}

int check_verify_shape(const View &c, int n_spec, int Hq)
{
    if (n_spec < 1 || Hq < 1)
        return TQKV_ERR_ARG;
    if (Hq % c.Hk != 0)
        return TQKV_ERR_UNSUPPORTED;
    if (n_spec > TQKV_MAX_QLEN || (long)(Hq / c.Hk) * n_spec > TQKV_MAX_ROWS)
        return TQKV_ERR_UNSUPPORTED;
    return TQKV_OK;
}

// Workspace: with more than one key range, the partial softmax states of
// every key range (32 rows per row tile); nothing otherwise.
size_t workspace_for(const View &c, int n_spec, int Hq, int splits)
{
    if (splits <= 1)
        return 0;
    const size_t groups = (size_t)c.B * c.Hk * row_tiles((Hq / c.Hk) * n_spec);
    const size_t slots = groups * splits * 32;
    return slots * 2 * sizeof(float) + slots * TQKV_HEAD_DIM * sizeof(uint16_t);
}

int num_splits_impl(const View &v, int n_spec, int Hq, int num_splits)
{
    if (check_verify_shape(v, n_spec, Hq) != TQKV_OK || num_splits < 0)
        return 0;
    int cus = current_device_cus();
    if (cus < 0)
        return 0;
    return plan_splits(v, num_splits, cus, (Hq / v.Hk) * n_spec);
}

int workspace_impl(const View &v, int n_spec, int Hq, int num_splits, size_t *bytes)
{
    int st = check_verify_shape(v, n_spec, Hq);
    if (st != TQKV_OK)
        return st;
    if (num_splits < 0)
        return TQKV_ERR_ARG;
    int cus = current_device_cus();
    if (cus < 0)
        return cus;
    const int rows = (Hq / v.Hk) * n_spec, splits = plan_splits(v, num_splits, cus, rows);
    if (!grid_fits(v, rows, splits))
        return TQKV_ERR_UNSUPPORTED;
    *bytes = workspace_for(v, n_spec, Hq, splits);
    return TQKV_OK;
}

// The new tokens of a fused store + verify are quantised inside the verify
// launch when few work-groups share them (each row tile's work-groups store
// them again); otherwise the store kernel runs first, on the same stream.
bool fuse_store(int n_spec, int rows) { return n_spec * row_tiles(rows) <= 32; }

// store + verify (Knew, Vnew non-null) or verify; dense queries
// [n_spec, B, Hq, 128] (cu_q null) or ragged ones (cu_q [B + 1], n_spec =
// the largest query count)
int verify_impl(const View &v, const void *Knew, const void *Vnew, const void *Q, int q_dtype,
                const int32_t *cu_q, const int32_t *seq_lens, int n_spec, int Hq, int causal, int num_splits,
                float sm_scale, float *out, void *workspace, size_t workspace_bytes, void *stream)
{
    int st = check_verify_shape(v, n_spec, Hq);
    if (st != TQKV_OK)
        return st;
    if (!Q || !seq_lens || !out || num_splits < 0)
        return TQKV_ERR_ARG;
    if ((Knew == nullptr) != (Vnew == nullptr))
        return TQKV_ERR_ARG;
    if (Knew && (!aligned(Knew, 2) || !aligned(Vnew, 2)))
        return TQKV_ERR_ALIGN;
    if (q_dtype != TQKV_Q_F32 && q_dtype != TQKV_Q_F16)
        return TQKV_ERR_ARG;
    if (causal != 0 && causal != 1)
        return TQKV_ERR_ARG;
    if (!(sm_scale >= 0.0f) || isinf(sm_scale))
        return TQKV_ERR_ARG;
    if (!aligned(Q, 16) || !aligned(seq_lens, 4) || !aligned(out, 16) || !aligned(cu_q, 4))
        return TQKV_ERR_ALIGN;
    int cus = current_device_cus();
    if (cus < 0)
        return cus;
    const int G = Hq / v.Hk;
    const int R = G * n_spec;
    const int splits = plan_splits(v, num_splits, cus, R);
    if (!grid_fits(v, R, splits))
        return TQKV_ERR_UNSUPPORTED;
    const size_t need = workspace_for(v, n_spec, Hq, splits);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return TQKV_ERR_WORKSPACE;
        if (!aligned(workspace, 256))
            return TQKV_ERR_ALIGN;
    }
    const float scale = (sm_scale == 0.0f) ? 0.08838834764831845f : sm_scale;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool fused = Knew && fuse_store(n_spec, R);
    if (Knew && !fused) {
        // the store kernel over the n_spec new tokens of every sequence:
        // token n of sequence b is row (n * B + b) of K and V, at position
        // seq_lens[b] - n_spec + n (computed on the device)
        StoreArgs sa;
        sa.base = static_cast<uint8_t *>(v.base);
        sa.K = static_cast<const uint16_t *>(Knew);
        sa.V = static_cast<const uint16_t *>(Vnew);
        sa.seq_idx = nullptr;
        sa.pos = nullptr;
        sa.slots = nullptr;
        sa.step_lens = seq_lens;
        sa.btab = v.btab;
        sa.B = v.B;
        sa.Hk = v.Hk;
        sa.max_seq = v.max_seq;
        sa.nblk = nblocks(v.max_seq);
        sa.T = n_spec * v.B;
        sa.N = n_spec;
        sa.bstride = v.bstride;
        sa.npages = v.npages;
        if (launch_store(v.preset, sa, s) != hipSuccess)
            return TQKV_ERR_LAUNCH;
    }
    VerifyArgs a;
    a.base = static_cast<const uint8_t *>(v.base);
    a.Q = Q;
    a.seq_lens = seq_lens;
    a.out = out;
    const size_t groups = (size_t)v.B * v.Hk * row_tiles(R);
    // workspace: (max, sum) pairs first (8-byte aligned), then the binary16 outputs
    const size_t slots = groups * splits * 32;
    a.part_ml = splits > 1 ? static_cast<float2 *>(workspace) : nullptr;
    a.part_o = splits > 1 ? reinterpret_cast<_Float16 *>(static_cast<uint8_t *>(workspace) + slots * sizeof(float2)) : nullptr;
    a.qscale = scale * 1.4426950408889634f;
    a.q_f16 = (q_dtype == TQKV_Q_F16);
    a.Hk = v.Hk;
    a.max_seq = v.max_seq;
    a.nblk = nblocks(v.max_seq);
    a.B = v.B;
    a.N = n_spec;
    a.Hq = Hq;
    a.G = G;
    a.R = R;
    a.causal = causal;
    a.nsplit = splits;
    a.nrt = row_tiles(R);
    a.Knew = fused ? static_cast<const uint16_t *>(Knew) : nullptr;
    a.Vnew = fused ? static_cast<const uint16_t *>(Vnew) : nullptr;
    a.wbase = static_cast<uint8_t *>(v.base);
    a.cu_q = cu_q;
    a.btab = v.btab;
    a.bstride = v.bstride;
    a.npages = v.npages;
    const int nqt = rows_per_group(R);
    if (launch_verify(v.preset, v.btab != nullptr, nqt, wide_waves(v, splits), R <= 8, a, s) != hipSuccess)
        return TQKV_ERR_LAUNCH;
    return TQKV_OK;
}

int store_impl(int preset, int Hk, void *base, const tqkv_cache *c, const tqkv_paged_cache *pc, const void *K,
               const void *V, const int32_t *seq_idx, const int32_t *pos, const int32_t *slot_mapping, int T,
               void *stream)
{
    if (T < 0)
        return TQKV_ERR_ARG;
    if (T == 0)
        return TQKV_OK;
    if (!K || !V || (pc ? !slot_mapping : (!seq_idx || !pos)))
        return TQKV_ERR_ARG;
    if (!aligned(K, 2) || !aligned(V, 2) || !aligned(seq_idx, 4) || !aligned(pos, 4) || !aligned(slot_mapping, 4))
        return TQKV_ERR_ALIGN;
    // the store kernel indexes (16-token chunk, head) pairs in 32 bits
    if ((long)((T + 15) / 16) * 16 * Hk > (long)INT32_MAX)
        return TQKV_ERR_UNSUPPORTED;
    int cus = current_device_cus();
    if (cus < 0)
        return cus;
    StoreArgs a;
    a.base = static_cast<uint8_t *>(base);
    a.K = static_cast<const uint16_t *>(K);
    a.V = static_cast<const uint16_t *>(V);
    a.seq_idx = pc ? nullptr : seq_idx;
    a.pos = pc ? nullptr : pos;
    a.slots = pc ? slot_mapping : nullptr;
    a.step_lens = nullptr;
    a.btab = nullptr;
    a.B = pc ? 0 : c->B;
    a.Hk = Hk;
    a.max_seq = pc ? 0 : c->max_seq;
    a.nblk = pc ? 0 : nblocks(c->max_seq);
    a.T = T;
    a.N = 0;
    a.bstride = 0;
    a.npages = pc ? pc->num_pages : 0;
    if (launch_store(preset, a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return TQKV_ERR_LAUNCH;
    return TQKV_OK;
}

} // namespace

extern "C" {

size_t tqkv_slot_bytes(int preset)
{
    if (preset == TQKV_K3V4_NC)
        return 120;
    if (preset == TQKV_K4V4_NC)
        return 136;
    if (preset == TQKV_K8V4)
        return 198;
    return 0;
}

size_t tqkv_block_bytes(int preset) { return 16 * tqkv_slot_bytes(preset); }

size_t tqkv_cache_bytes(int preset, int B, int Hk, int D, int max_seq)
{
    if (tqkv_slot_bytes(preset) == 0 || B < 1 || Hk < 1 || D != TQKV_HEAD_DIM || max_seq < 1)
        return 0;
    return (size_t)B * Hk * nblocks(max_seq) * tqkv_block_bytes(preset);
}

size_t tqkv_paged_cache_bytes(int preset, int Hk, int D, int num_pages)
{
    if (tqkv_slot_bytes(preset) == 0 || Hk < 1 || D != TQKV_HEAD_DIM || num_pages < 1 || num_pages > (INT32_MAX >> 4))
        return 0;
    return (size_t)num_pages * Hk * tqkv_block_bytes(preset);
}

int tqkv_store(const tqkv_cache *cache, const void *K, const void *V, const int32_t *seq_idx,
               const int32_t *pos, int T, void *stream)
{
    View v;
    int st = view_of(cache, v);
    if (st != TQKV_OK)
        return st;
    return store_impl(v.preset, v.Hk, v.base, cache, nullptr, K, V, seq_idx, pos, nullptr, T, stream);
}

int tqkv_paged_store(const tqkv_paged_cache *cache, const void *K, const void *V, const int32_t *slot_mapping, int T,
                     void *stream)
{
    int st = check_pool(cache);
    if (st != TQKV_OK)
        return st;
    return store_impl(cache->preset, cache->Hk, cache->base, nullptr, cache, K, V, nullptr, nullptr, slot_mapping, T,
                      stream);
}

int tqkv_verify_num_splits(const tqkv_cache *cache, int n_spec, int Hq, int num_splits)
{
    View v;
    if (view_of(cache, v) != TQKV_OK)
        return 0;
    return num_splits_impl(v, n_spec, Hq, num_splits);
}

int tqkv_paged_verify_num_splits(const tqkv_paged_cache *cache, int n_spec, int Hq, int num_splits)
{
    View v;
    if (view_of(cache, v) != TQKV_OK)
        return 0;
    return num_splits_impl(v, n_spec, Hq, num_splits);
}

int tqkv_verify_workspace_bytes(const tqkv_cache *cache, int n_spec, int Hq, int num_splits, size_t *bytes)
{
    if (!bytes)
        return TQKV_ERR_ARG;
    *bytes = 0;
    View v;
    int st = view_of(cache, v);
    if (st != TQKV_OK)
        return st;
    return workspace_impl(v, n_spec, Hq, num_splits, bytes);
}

int tqkv_paged_verify_workspace_bytes(const tqkv_paged_cache *cache, int n_spec, int Hq, int num_splits,
                                      size_t *bytes)
{
    if (!bytes)
        return TQKV_ERR_ARG;
    *bytes = 0;
    View v;
    int st = view_of(cache, v);
    if (st != TQKV_OK)
        return st;
    return workspace_impl(v, n_spec, Hq, num_splits, bytes);
}

int tqkv_verify(const tqkv_cache *cache, const void *Q, int q_dtype, const int32_t *seq_lens,
                int n_spec, int Hq, int causal, int num_splits, float sm_scale, float *out,
                void *workspace, size_t workspace_bytes, void *stream)
{
    View v;
    int st = view_of(cache, v);
    if (st != TQKV_OK)
        return st;
    return verify_impl(v, nullptr, nullptr, Q, q_dtype, nullptr, seq_lens, n_spec, Hq, causal, num_splits, sm_scale,
                       out, workspace, workspace_bytes, stream);
}

int tqkv_verify_noalloc(const tqkv_cache *cache, const void *Q, int q_dtype, const int32_t *seq_lens, int n_spec,
                        int Hq, int causal, int num_splits, float sm_scale, float *out, void *stream)
{
    View v;
    int st = view_of(cache, v);
    if (st != TQKV_OK)
        return st;
    // the partial states go to the library's scratch array: a shape that
    // needs more than it holds is refused (TQKV_ERR_WORKSPACE, from
    // verify_impl's size check) before anything is launched
    void *ws = nullptr;
    st = current_device_scratch(&ws);
    if (st != TQKV_OK)
        return st;
    return verify_impl(v, nullptr, nullptr, Q, q_dtype, nullptr, seq_lens, n_spec, Hq, causal, num_splits, sm_scale,
                       out, ws, kScratchBytes, stream);
}

int tqkv_verify_varlen(const tqkv_cache *cache, const void *Q, int q_dtype, const int32_t *cu_q, int max_q,
                       const int32_t *seq_lens, int Hq, int causal, int num_splits, float sm_scale, float *out,
                       void *workspace, size_t workspace_bytes, void *stream)
{
    View v;
    int st = view_of(cache, v);
    if (st != TQKV_OK)
        return st;
    if (!cu_q)
        return TQKV_ERR_ARG;
    return verify_impl(v, nullptr, nullptr, Q, q_dtype, cu_q, seq_lens, max_q, Hq, causal, num_splits, sm_scale, out,
                       workspace, workspace_bytes, stream);
}

int tqkv_store_verify(const tqkv_cache *cache, const void *K, const void *V, const void *Q, int q_dtype,
                      const int32_t *seq_lens, int n_spec, int Hq, int causal, int num_splits, float sm_scale,
                      float *out, void *workspace, size_t workspace_bytes, void *stream)
{
    View v;
    int st = view_of(cache, v);
    if (st != TQKV_OK)
        return st;
    if (!K || !V)
        return TQKV_ERR_ARG;
    return verify_impl(v, K, V, Q, q_dtype, nullptr, seq_lens, n_spec, Hq, causal, num_splits, sm_scale, out,
                       workspace, workspace_bytes, stream);
}

int tqkv_paged_verify(const tqkv_paged_cache *cache, const void *Q, int q_dtype, const int32_t *seq_lens,
                      int n_spec, int Hq, int causal, int num_splits, float sm_scale, float *out, void *workspace,
                      size_t workspace_bytes, void *stream)
{
    View v;
    int st = view_of(cache, v);
    if (st != TQKV_OK)
        return st;
    return verify_impl(v, nullptr, nullptr, Q, q_dtype, nullptr, seq_lens, n_spec, Hq, causal, num_splits, sm_scale,
                       out, workspace, workspace_bytes, stream);
}

int tqkv_paged_verify_varlen(const tqkv_paged_cache *cache, const void *Q, int q_dtype, const int32_t *cu_q,
                             int max_q, const int32_t *seq_lens, int Hq, int causal, int num_splits, float sm_scale,
                             float *out, void *workspace, size_t workspace_bytes, void *stream)
{
    View v;
    int st = view_of(cache, v);
    if (st != TQKV_OK)
        return st;
    if (!cu_q)
        return TQKV_ERR_ARG;
    return verify_impl(v, nullptr, nullptr, Q, q_dtype, cu_q, seq_lens, max_q, Hq, causal, num_splits, sm_scale, out,
                       workspace, workspace_bytes, stream);
}

int tqkv_paged_store_verify(const tqkv_paged_cache *cache, const void *K, const void *V, const void *Q, int q_dtype,
                            const int32_t *seq_lens, int n_spec, int Hq, int causal, int num_splits, float sm_scale,
                            float *out, void *workspace, size_t workspace_bytes, void *stream)
{
    View v;
    int st = view_of(cache, v);
    if (st != TQKV_OK)
        return st;
    if (!K || !V)
        return TQKV_ERR_ARG;
    return verify_impl(v, K, V, Q, q_dtype, nullptr, seq_lens, n_spec, Hq, causal, num_splits, sm_scale, out,
                       workspace, workspace_bytes, stream);
}

const char *tqkv_status_string(int status)
{
    switch (status) {
    case TQKV_OK: return "ok";
    case TQKV_ERR_ARG: return "invalid argument";
    case TQKV_ERR_UNSUPPORTED: return "unsupported shape";
    case TQKV_ERR_ALIGN: return "misaligned pointer";
    case TQKV_ERR_WORKSPACE: return "workspace missing or too small";
    case TQKV_ERR_LAUNCH: return "kernel launch failed";
    case TQKV_ERR_DEVICE: return "no gfx950 device is current";
    default: return "unknown status";
    }
}

int tqkv_version(void) { return 200; }

} // extern "C"
