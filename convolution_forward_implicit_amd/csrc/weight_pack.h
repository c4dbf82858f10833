// Plan-time weight prepacking for the single-convolution kernels.
//
// The ExecuTorch conv1d issue's conv2d path (section "The conv2d path
// already solves this") prepacks its weights once, ahead of the runs.  Here
// the packed form of a plan's weights is, for every (group, output-channel
// tile, K-step) of that plan, the weight part of the LDS stage exactly as
// the plan's kernel lays it out -- the direct-to-LDS kernel's swizzled
// 128-byte rows, or the fixed-filter patch kernel's (chunk, tap, channel)
// slots -- with zeros wherever the kernel would load nothing (channels past
// K, reduction past C*Z*Y*X, unused slots).  A K-step then fetches its
// weights as whole contiguous kilobytes, one per load instruction, instead
// of 16-byte pieces of up to 64 different weight rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfwd {

struct PackParams {
    const void *w;          // GKZYXC weights
    void *out;              // packed image
    int64_t slots;          // 16-byte slots of the image
    int esz;                // element bytes
    int mode;               // 0: direct-to-LDS image, 1: fixed-filter patch image
    int K, Kred, C, Z, taps;
    int BN, tiles_n;
    int nk, ksub, subk, vec, sw4;     // mode 0
    int ncs, cc, wslots, img_slots;   // mode 1
};

__global__ void __launch_bounds__(256) pack_weights_kernel(PackParams pp)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= pp.slots) return;
    int64_t src = -1;   // element offset of the slot's 16 bytes in w, or none (zeros)
    if (pp.mode == 0) {
        // slot i = ((((g * tiles_n + nt) * nk + step) * ksub + u) * BN/8 + block) * 64 + lane
        const int per_sub = pp.BN * 8;
        int64_t t = i;
        const int r2 = (int)(t % per_sub); t /= per_sub;
        const int u = (int)(t % pp.ksub); t /= pp.ksub;
        const int step = (int)(t % pp.nk); t /= pp.nk;
        const int nt = (int)(t % pp.tiles_n);
        const int64_t g = t / pp.tiles_n;
        const int bb = r2 / 64, lane = r2 % 64;
        const int lrow = lane >> 3;
        const int cht = ((lane & 7) ^ lrow) ^ (pp.sw4 & (bb >> 1));
        const int n = nt * pp.BN + bb * 8 + lrow;
        const int r = (step * pp.ksub + u) * pp.subk + cht * pp.vec;
        if (n < pp.K && r < pp.Kred) src = (g * pp.K + n) * pp.Kred + r;
    } else {
        // slot i = ((((g * tiles_n + nt) * Z + z) * ncs + cs) * img_slots + s), s = (q*taps + tap)*BN + n
        int64_t t = i;
        const int s = (int)(t % pp.img_slots); t /= pp.img_slots;
        const int cs = (int)(t % pp.ncs); t /= pp.ncs;
        const int z = (int)(t % pp.Z); t /= pp.Z;
        const int nt = (int)(t % pp.tiles_n);
        const int64_t g = t / pp.tiles_n;
        if (s < pp.wslots) {
            const int n = s % pp.BN, rest = s / pp.BN;
            const int tap = rest % pp.taps, q = rest / pp.taps;
            const int k = nt * pp.BN + n;
            if (k < pp.K) src = (g * pp.K + k) * pp.Kred + (z * pp.taps + tap) * pp.C + cs * pp.cc + q * 8;
        }
    }
    uint4 v = {0u, 0u, 0u, 0u};
    if (src >= 0) v = *reinterpret_cast<const uint4 *>(reinterpret_cast<const unsigned char *>(pp.w) + src * pp.esz);
    reinterpret_cast<uint4 *>(pp.out)[i] = v;
}

}  // namespace convfwd
