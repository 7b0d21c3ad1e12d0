// C ABI of libtqkv.so (declared in include/tqkv.h): argument validation,
// launch planning and status codes.  No device allocation, no host<->device
// copies, no synchronisation.
#include "common.h"
#include "tqkv.h"

#include <math.h>
#include <string.h>

namespace {

using namespace tqkv;

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];   // 0 = not probed yet, -1 = not a gfx950 device

// Number of compute units of the current device, or a negative status when
// no gfx950 device is current.
int current_device_cus()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return TQKV_ERR_DEVICE;
    if (g_cu_count[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return TQKV_ERR_DEVICE;
        const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        g_cu_count[dev] = ok ? prop.multiProcessorCount : -1;
    }
    return g_cu_count[dev] > 0 ? g_cu_count[dev] : TQKV_ERR_DEVICE;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_cache(const tqkv_cache *c)
{
    if (!c)
        return TQKV_ERR_ARG;
    if (c->preset != TQKV_K8V4 && c->preset != TQKV_K3V4_NC)
        return TQKV_ERR_ARG;
    if (c->B < 1 || c->Hk < 1 || c->max_seq < 1 || !c->base)
        return TQKV_ERR_ARG;
    if (c->D != TQKV_HEAD_DIM)
        return TQKV_ERR_UNSUPPORTED;
    if (!aligned(c->base, 16))
        return TQKV_ERR_ALIGN;
    return TQKV_OK;
}

int nblocks(int max_seq) { return (max_seq + kBlockTokens - 1) / kBlockTokens; }

// Query rows per work-group: the rows of one KV head are cut into tiles of
// 32 (one MFMA operand height), one work-group each.
int row_tiles(int rows) { return (rows + 31) / 32; }

// Key-range partitions per (b, hk): two work-groups of 4 wavefronts per
// compute unit overall, at least one 32-token tile per wavefront.
int plan_splits(const tqkv_cache *c, int num_splits, int cus, int rows)
{
    const int units = c->B * c->Hk * row_tiles(rows);
    const int tiles = (c->max_seq + 31) / 32;
    const int max_useful = (tiles + 3) / 4;
    int s = num_splits;
    if (s <= 0)
        s = (2 * cus + units - 1) / units;
    if (s > max_useful)
        s = max_useful;
    if (s > 1024)
        s = 1024;
    if (s < 1)
        s = 1;
    return s;
}

int check_verify_shape(const tqkv_cache *c, int n_spec, int Hq)
{
    int st = check_cache(c);
    if (st != TQKV_OK)
        return st;
    if (n_spec < 1 || Hq < 1)
        return TQKV_ERR_ARG;
    if (Hq % c->Hk != 0)
        return TQKV_ERR_UNSUPPORTED;
    if ((Hq / c->Hk) * n_spec > TQKV_MAX_ROWS)
        return TQKV_ERR_UNSUPPORTED;
    return TQKV_OK;
}

// Workspace: with more than one key range, the partial softmax states of
// every key range (32 rows per row tile); nothing otherwise.
size_t workspace_for(const tqkv_cache *c, int n_spec, int Hq, int splits)
{
    if (splits <= 1)
        return 0;
    const size_t groups = (size_t)c->B * c->Hk * row_tiles((Hq / c->Hk) * n_spec);
    const size_t slots = groups * splits * 32;
    return slots * 2 * sizeof(float) + slots * TQKV_HEAD_DIM * sizeof(uint16_t);
}

} // namespace

namespace {
int verify_impl(const tqkv_cache *cache, const void *Knew, const void *Vnew, const void *Q, int q_dtype,
                       const int32_t *seq_lens, int n_spec, int Hq, int causal, int num_splits, float sm_scale,
                       float *out, void *workspace, size_t workspace_bytes, void *stream)
{
    int st = check_verify_shape(cache, n_spec, Hq);
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
    if (!aligned(Q, 16) || !aligned(seq_lens, 4) || !aligned(out, 16))
        return TQKV_ERR_ALIGN;
    int cus = current_device_cus();
    if (cus < 0)
        return cus;
    const int splits = plan_splits(cache, num_splits, cus, (Hq / cache->Hk) * n_spec);
    const size_t need = workspace_for(cache, n_spec, Hq, splits);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return TQKV_ERR_WORKSPACE;
        if (!aligned(workspace, 256))
            return TQKV_ERR_ALIGN;
    }
    const int G = Hq / cache->Hk;
    const int R = G * n_spec;
    const float scale = (sm_scale == 0.0f) ? 0.08838834764831845f : sm_scale;
    VerifyArgs a;
    a.base = static_cast<const uint8_t *>(cache->base);
    a.Q = Q;
    a.seq_lens = seq_lens;
    a.out = out;
    const size_t groups = (size_t)cache->B * cache->Hk * row_tiles(R);
    // workspace: (max, sum) pairs first (8-byte aligned), then the binary16 outputs
    const size_t slots = groups * splits * 32;
    a.part_ml = splits > 1 ? static_cast<float2 *>(workspace) : nullptr;
    a.part_o = splits > 1 ? reinterpret_cast<_Float16 *>(static_cast<uint8_t *>(workspace) + slots * sizeof(float2)) : nullptr;
    a.qscale = scale * 1.4426950408889634f;
    a.q_f16 = (q_dtype == TQKV_Q_F16);
    a.Hk = cache->Hk;
    a.max_seq = cache->max_seq;
    a.nblk = nblocks(cache->max_seq);
    a.B = cache->B;
    a.N = n_spec;
    a.Hq = Hq;
    a.G = G;
    a.R = R;
    a.causal = causal;
    a.nsplit = splits;
    a.nrt = row_tiles(R);
    a.Knew = static_cast<const uint16_t *>(Knew);
    a.Vnew = static_cast<const uint16_t *>(Vnew);
    a.wbase = static_cast<uint8_t *>(cache->base);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_verify(cache->preset, 1, a, s) != hipSuccess)
        return TQKV_ERR_LAUNCH;
    return TQKV_OK;
}

} // namespace

extern "C" {

size_t tqkv_slot_bytes(int preset)
{
    if (preset == TQKV_K3V4_NC)
        return 120;
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

int tqkv_store(const tqkv_cache *cache, const void *K, const void *V, const int32_t *seq_idx,
               const int32_t *pos, int T, void *stream)
{
    int st = check_cache(cache);
    if (st != TQKV_OK)
        return st;
    if (T < 0)
        return TQKV_ERR_ARG;
    if (T == 0)
        return TQKV_OK;
    if (!K || !V || !seq_idx || !pos)
        return TQKV_ERR_ARG;
    if (!aligned(K, 2) || !aligned(V, 2) || !aligned(seq_idx, 4) || !aligned(pos, 4))
        return TQKV_ERR_ALIGN;
    int cus = current_device_cus();
    if (cus < 0)
        return cus;
    StoreArgs a;
    a.base = static_cast<uint8_t *>(cache->base);
    a.K = static_cast<const uint16_t *>(K);
    a.V = static_cast<const uint16_t *>(V);
    a.seq_idx = seq_idx;
    a.pos = pos;
    a.B = cache->B;
    a.Hk = cache->Hk;
    a.max_seq = cache->max_seq;
    a.nblk = nblocks(cache->max_seq);
    a.T = T;
    if (launch_store(cache->preset, a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return TQKV_ERR_LAUNCH;
    return TQKV_OK;
}

int tqkv_verify_num_splits(const tqkv_cache *cache, int n_spec, int Hq, int num_splits)
{
    if (check_verify_shape(cache, n_spec, Hq) != TQKV_OK || num_splits < 0)
        return 0;
    int cus = current_device_cus();
    if (cus < 0)
        return 0;
    return plan_splits(cache, num_splits, cus, (Hq / cache->Hk) * n_spec);
}

int tqkv_verify_workspace_bytes(const tqkv_cache *cache, int n_spec, int Hq, int num_splits,
                                size_t *bytes)
{
    if (!bytes)
        return TQKV_ERR_ARG;
    *bytes = 0;
    int st = check_verify_shape(cache, n_spec, Hq);
    if (st != TQKV_OK)
        return st;
    if (num_splits < 0)
        return TQKV_ERR_ARG;
    int cus = current_device_cus();
    if (cus < 0)
        return cus;
    *bytes = workspace_for(cache, n_spec, Hq, plan_splits(cache, num_splits, cus, (Hq / cache->Hk) * n_spec));
    return TQKV_OK;
}

int tqkv_verify(const tqkv_cache *cache, const void *Q, int q_dtype, const int32_t *seq_lens,
                int n_spec, int Hq, int causal, int num_splits, float sm_scale, float *out,
                void *workspace, size_t workspace_bytes, void *stream)
{
    return verify_impl(cache, nullptr, nullptr, Q, q_dtype, seq_lens, n_spec, Hq, causal, num_splits, sm_scale, out,
                       workspace, workspace_bytes, stream);
}

int tqkv_store_verify(const tqkv_cache *cache, const void *K, const void *V, const void *Q, int q_dtype,
                      const int32_t *seq_lens, int n_spec, int Hq, int causal, int num_splits, float sm_scale,
                      float *out, void *workspace, size_t workspace_bytes, void *stream)
{
    if (!K || !V)
        return TQKV_ERR_ARG;
    return verify_impl(cache, K, V, Q, q_dtype, seq_lens, n_spec, Hq, causal, num_splits, sm_scale, out, workspace,
                       workspace_bytes, stream);
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

int tqkv_version(void) { return 100; }

} // extern "C"
