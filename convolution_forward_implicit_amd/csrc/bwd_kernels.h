// Kernels of the backward passes (the grouped bwd_data / bwd_weight
// convolutions the Composable Kernel grouped-conv note names beside the
// forward one, section 6), same layouts as the forward: x N x D x H x W x G x C,
// w G x K x Z x Y x X x C, dy N x Do x Ho x Wo x G x K.
//
// Backward-data runs on the forward implicit-GEMM kernels.  With
// off = d (F - 1) - p per spatial dim,
//
//   dx[i] = sum_{t, k} dy[(i + p - t d) / s, k] w[k, t, c]   (exact divisions only)
//         = sum_{t', k} dyp[i + t' d, k] w'[c, t', k]
//
// where t' = F - 1 - t (the taps flipped), w'[g][c][z'][y'][x'][k] =
// w[g][k][Z-1-z'][Y-1-y'][X-1-x'][c] (channels swapped, so the reduction runs
// over k, innermost), and dyp is dy spread onto a grid of I + d (F - 1)
// positions: dy[o] at position o s + off, zeros elsewhere.  That is a
// forward convolution with stride 1, no padding, the same dilation, K input
// channels and C output channels.  With unit strides and off >= 0 the spread
// copy is dy itself with padding off, and no copy is made.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfwd {

// w'[g][c][z'][y'][x'][k] = w[g][k][Z-1-z'][Y-1-y'][X-1-x'][c], one element per thread
template <typename T>
__global__ void __launch_bounds__(256) bwd_data_weights_kernel(const T *__restrict__ w, T *__restrict__ wt, int K,
                                                               int C, int Z, int Y, int X, int64_t total)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    int64_t t = i;
    const int k = (int)(t % K); t /= K;
    const int xx = (int)(t % X); t /= X;
    const int y = (int)(t % Y); t /= Y;
    const int z = (int)(t % Z); t /= Z;
    const int c = (int)(t % C); t /= C;
    const int64_t g = t;
    wt[i] = w[((((g * K + k) * Z + (Z - 1 - z)) * Y + (Y - 1 - y)) * X + (X - 1 - xx)) * C + c];
}

struct SpreadParams {
    const void *dy;
    void *dyp;
    int N, G;
    int KB;          // bytes of one (pixel, group) row of channels: K * element size
    int O[3];        // dy extents
    int P[3];        // spread extents, I + d (F - 1)
    int s[3];        // strides
    int off[3];      // d (F - 1) - p: position of dy[0] on the spread grid (may be negative)
    int64_t total;   // V-sized chunks of dyp
};

// dyp[n][j][g][:] = dy[n][(j - off) / s][g][:] when every division is exact
// and in range, else 0.  One chunk (V: 16, 4 or 2 bytes of channels, the
// widest that divides a row) per thread.
template <typename V>
__global__ void __launch_bounds__(256) bwd_data_spread_kernel(SpreadParams sp)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= sp.total) return;
    const int KV = sp.KB / (int)sizeof(V);
    int64_t t = i;
    const int kv = (int)(t % KV); t /= KV;
    const int g = (int)(t % sp.G); t /= sp.G;
    int j[3];
    j[2] = (int)(t % sp.P[2]); t /= sp.P[2];
    j[1] = (int)(t % sp.P[1]); t /= sp.P[1];
    j[0] = (int)(t % sp.P[0]); t /= sp.P[0];
    const int64_t n = t;
    bool ok = true;
    int o[3];
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const int num = j[d] - sp.off[d];
        o[d] = num >= 0 ? num / sp.s[d] : 0;
        ok = ok && num >= 0 && num - o[d] * sp.s[d] == 0 && o[d] < sp.O[d];
    }
    V v;
    if (ok) {
        const int64_t row = (((n * sp.O[0] + o[0]) * sp.O[1] + o[1]) * sp.O[2] + o[2]) * sp.G + g;
        v = reinterpret_cast<const V *>(sp.dy)[row * KV + kv];
    } else {
        v = V{};
    }
    reinterpret_cast<V *>(sp.dyp)[i] = v;
}

}  // namespace convfwd
