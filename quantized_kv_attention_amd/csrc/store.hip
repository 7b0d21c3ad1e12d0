// Fused store kernel: quantise new K/V token-heads into the packed cache
// (the quantisation itself is in quant.h, shared with the fused store +
// verify kernel).  One wavefront per token-head.
#include "quant.h"

namespace tqkv {
namespace {

template <int PRESET>
__global__ __launch_bounds__(256) void store_kernel(StoreArgs a)
{
    using L = Layout<PRESET>;
    const int lane = threadIdx.x & 63;
    const long th = (long)blockIdx.x * 4 + (threadIdx.x >> 6); // token-head, wave-uniform
    if (th >= (long)a.T * a.Hk)
        return;
    const int t = (int)(th / a.Hk), hk = (int)(th % a.Hk);
    uint8_t *blk;
    int tb;
    if (a.step_lens) {
        const int n = t / a.B, b = t - n * a.B;
        const int Lr = a.step_lens[b];
        const int L = Lr < 0 ? 0 : (Lr > a.max_seq ? a.max_seq : Lr);
        const int p = L - a.N + n;
        if (p < 0)
            return; // a sequence shorter than the step
        if (a.btab) {
            const int pg = a.btab[(size_t)b * a.bstride + (p >> 4)];
            if (pg < 0 || pg >= a.npages)
                return;
            blk = a.base + ((size_t)pg * a.Hk + hk) * L::kBlockBytes;
        } else {
            blk = a.base + ((size_t)(b * a.Hk + hk) * a.nblk + (p >> 4)) * L::kBlockBytes;
        }
        tb = p & 15;
    } else if (a.slots) {
        // paged: slot = page * 16 + position in the page; head hk's block of
        // page p is block p * Hk + hk of the pool
        const int sl = a.slots[t];
        if (sl < 0 || (sl >> 4) >= a.npages)
            return; // padding and out-of-range entries are skipped
        blk = a.base + ((size_t)(sl >> 4) * a.Hk + hk) * L::kBlockBytes;
        tb = sl & 15;
    } else {
        const int b = a.seq_idx[t], p = a.pos[t];
        if (b < 0 || b >= a.B || p < 0 || p >= a.max_seq)
            return; // out-of-range entries are skipped
        blk = a.base + ((size_t)(b * a.Hk + hk) * a.nblk + (p >> 4)) * L::kBlockBytes;
        tb = p & 15;
    }
    const uint16_t *kp = a.K + (size_t)th * kD;
    const uint16_t *vp = a.V + (size_t)th * kD;

    quant::quantize_token_head<PRESET>(blk, tb, quant::load_token_head(kp, vp, lane), lane);
}

} // namespace

hipError_t launch_store(int preset, const StoreArgs &a, hipStream_t s)
{
    const long waves = (long)a.T * a.Hk;
    if (waves == 0)
        return hipSuccess;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    if (preset == kPresetK3V4)
        hipLaunchKernelGGL(store_kernel<kPresetK3V4>, grid, block, 0, s, a);
    else if (preset == kPresetK4V4)
        hipLaunchKernelGGL(store_kernel<kPresetK4V4>, grid, block, 0, s, a);
    else
        hipLaunchKernelGGL(store_kernel<kPresetK8V4>, grid, block, 0, s, a);
    return hipGetLastError();
}

} // namespace tqkv
