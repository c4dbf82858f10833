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

#include "igemm_kernel.h"

namespace convfwd {

// ---- Backward-weight (bf16) --------------------------------------------------
//
//   dw[g,k,t,c] = sum over output pixels q = (n, od, oh, ow) of
//                 dy[q, g, k] * x[n, od*sd - pd + z*dd, oh*sh - ph + y*dh, ow*sw - pw + x*dw, g, c]
//
// per group a GEMM with the PIXELS as the reduction: rows k, columns (t, c).
// MFMA fragments need 8 consecutive reduction elements per lane, but both
// operands keep the channels innermost, so every K-step stages PC pixels of
// dy (KT channels) and of x for each of TT taps (CT channels) in LDS
// TRANSPOSED: one 72-byte row per channel holding its PC = 32 pixels (16-bit
// values, pixel pairs in one dword; the 18-dword pitch keeps the 64 lanes of
// a staging store in distinct bank pairs).  Loads are 16 bytes (8 channels of
// one pixel) and coalesced along the channels.
//
// A workgroup owns a KT x CT block of (k, c) for TT taps of one group and a
// contiguous range of pixel steps (split-K over the pixels: a weight
// gradient has few outputs and a long reduction); its fp32 partial tile
// goes to a caller workspace [split][g][k][t][c], and wgrad_reduce_kernel
// sums the splits in index order (deterministic) and rounds to bf16.  The
// 32x32x16 bf16 MFMA takes dy rows as the first operand (k) and x rows as
// the second (c); block b = (t * KB + kb) * CB + cb goes to wave b mod 4, so
// a wave keeps one (kb, cb) over its taps and reads its dy fragment once per
// step.  Channels per group must be multiples of 8 (16-byte rows).
struct WgradParams {
    const void *x, *dy;
    float *ws;                 // partials [split][G][K][taps][C]
    int N, G, C, K;
    int Di, Hi, Wi, Do, Ho, Wo;
    int sd, sh, sw, pd, ph, pw, dd, dh, dw;
    int Y, X, taps;
    int64_t pixels;            // N * Do * Ho * Wo
    int steps_per_split;       // PC-pixel steps per workgroup
    int splits, kt_n, ct_n, tg_n;
    FastDiv fd_Wo, fd_Ho, fd_Do;
};

typedef bf16x8_t bf16x8_a8 __attribute__((aligned(8)));

template <int KT, int CT, int TT>
struct WgradShape {
    static constexpr int PC = 32;                       // pixels per K-step
    static constexpr int QN = CT / 8;                   // 16-byte chunks per pixel row
    static constexpr int RG = TT + 1;                   // row groups: dy, then one per tap
    static constexpr int PITCH = 72;                    // bytes per LDS row
    static constexpr int ROWS = KT + TT * CT;
    static constexpr int LDS_BYTES = ROWS * PITCH;
    static constexpr int NTG = 256 / (QN * PC / 2);     // thread groups over the row groups
    static constexpr int UPT = (RG + NTG - 1) / NTG;    // staging units per thread
    static constexpr int KB = KT / 32, CB = CT / 32;
    static constexpr int NBLK = TT * KB * CB;           // 32x32 output blocks
    static constexpr int NBW = (NBLK + 3) / 4;          // blocks per wave
    static_assert(KT == CT, "one chunk count for both operands");
    static_assert(KT == 32 || KT == 64, "32 or 64 channels per tile");
    static_assert(NBW * 16 <= 160, "accumulators");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

template <int KT, int CT, int TT>
__global__ void __launch_bounds__(256) wgrad_kernel(WgradParams wp)
{
    using S = WgradShape<KT, CT, TT>;
    __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS_BYTES];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // workgroup -> (split, tap group, c tile, k tile, group)
    int b = blockIdx.x;
    const int split = b % wp.splits; b /= wp.splits;
    const int tgi = b % wp.tg_n; b /= wp.tg_n;
    const int cti = b % wp.ct_n; b /= wp.ct_n;
    const int kti = b % wp.kt_n;
    const int g = b / wp.kt_n;
    const int k0 = kti * KT, c0 = cti * CT, t0 = tgi * TT;
    const int64_t step0 = (int64_t)split * wp.steps_per_split;
    const int64_t nsteps_total = (wp.pixels + S::PC - 1) / S::PC;
    int64_t nsteps = nsteps_total - step0;
    if (nsteps > wp.steps_per_split) nsteps = wp.steps_per_split;

    // ---- this thread's staging units: row group r = tg + NTG*u, chunk q, pixel pair pp
    const int q = tid % S::QN;
    const int pp = (tid / S::QN) % (S::PC / 2);
    const int tg = tid / (S::QN * S::PC / 2);
    int tz[S::UPT], ty[S::UPT], tx[S::UPT];     // tap offsets (row groups >= 1)
#pragma unroll
    for (int u = 0; u < S::UPT; ++u) {
        const int r = tg + S::NTG * u;
        const int t = t0 + (r >= 1 ? r - 1 : 0);
        const int xx = t % wp.X, yz = t / wp.X;
        tz[u] = (yz / wp.Y) * wp.dd;
        ty[u] = (yz % wp.Y) * wp.dh;
        tx[u] = xx * wp.dw;
    }
    const uint16_t *xg = reinterpret_cast<const uint16_t *>(wp.x);
    const uint16_t *dyg = reinterpret_cast<const uint16_t *>(wp.dy);
    const int64_t GC = (int64_t)wp.G * wp.C, GK = (int64_t)wp.G * wp.K;

    uint4 v[S::UPT][2];
    auto load = [&](int64_t step) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t P = step * S::PC + 2 * pp + h;
            const bool pok = P < wp.pixels;
            int n = 0, od = 0, oh = 0, ow = 0;
            if (pok) {
                const int pi = (int)P;
                const int a = fdiv(pi, wp.fd_Wo);
                ow = pi - a * wp.Wo;
                const int b2 = fdiv(a, wp.fd_Ho);
                oh = a - b2 * wp.Ho;
                n = fdiv(b2, wp.fd_Do);
                od = b2 - n * wp.Do;
            }
            const int id0 = od * wp.sd - wp.pd, ih0 = oh * wp.sh - wp.ph, iw0 = ow * wp.sw - wp.pw;
#pragma unroll
            for (int u = 0; u < S::UPT; ++u) {
                const int r = tg + S::NTG * u;
                uint4 val = {0u, 0u, 0u, 0u};
                if (r < S::RG && pok) {
                    if (r == 0) {
                        const int k = k0 + 8 * q;
                        if (k < wp.K) val = *reinterpret_cast<const uint4 *>(dyg + P * GK + (int64_t)g * wp.K + k);
                    } else {
                        const int c = c0 + 8 * q;
                        const int id = id0 + tz[u], ih = ih0 + ty[u], iw = iw0 + tx[u];
                        if (c < wp.C && (unsigned)id < (unsigned)wp.Di && (unsigned)ih < (unsigned)wp.Hi &&
                            (unsigned)iw < (unsigned)wp.Wi)
                            val = *reinterpret_cast<const uint4 *>(
                                xg + ((((int64_t)n * wp.Di + id) * wp.Hi + ih) * wp.Wi + iw) * GC + (int64_t)g * wp.C + c);
                    }
                }
                v[u][h] = val;
            }
        }
    };
    // transposed store: row (row group base + 8q + e), dword column pp = pixels (2pp, 2pp+1)
    auto store = [&]() {
#pragma unroll
        for (int u = 0; u < S::UPT; ++u) {
            const int r = tg + S::NTG * u;
            if (r < S::RG) {
                const int row0 = (r == 0 ? 0 : KT + (r - 1) * CT) + 8 * q;
                const uint32_t lo[4] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w};
                const uint32_t hi[4] = {v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t a = (lo[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    const uint32_t bb = (hi[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                    *reinterpret_cast<uint32_t *>(smem + (row0 + e) * S::PITCH + 4 * pp) = a | (bb << 16);
                }
            }
        }
    };

    f32x16_t acc[S::NBW];
#pragma unroll
    for (int i = 0; i < S::NBW; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.f;
    const int frow = lane & 31, kh = lane >> 5;

    if (nsteps > 0) load(step0);
    for (int64_t it = 0; it < nsteps; ++it) {
        __syncthreads();                      // the previous step's fragments are read
        store();
        __syncthreads();                      // this step is in LDS
        if (it + 1 < nsteps) load(step0 + it + 1);   // in flight during the products
#pragma unroll
        for (int s = 0; s < S::PC / 16; ++s) {
            const int co = 32 * s + 16 * kh;  // byte offset of the lane's 8 pixels
#pragma unroll
            for (int i = 0; i < S::NBW; ++i) {
                const int blk = wave + 4 * i;
                if (blk < S::NBLK) {
                    const int cb = blk % S::CB, kb = (blk / S::CB) % S::KB, t = blk / (S::CB * S::KB);
                    // rows are 8-byte aligned (72-byte pitch): two 8-byte LDS reads per fragment
                    const bf16x8_t a = *reinterpret_cast<const bf16x8_a8 *>(smem + (kb * 32 + frow) * S::PITCH + co);
                    const bf16x8_t bv = *reinterpret_cast<const bf16x8_a8 *>(
                        smem + (KT + t * CT + cb * 32 + frow) * S::PITCH + co);
                    acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bv, acc[i], 0, 0, 0);
                }
            }
        }
    }

    // ---- partial tile: lane holds dw[k = kb*32 + 8j + 4kh + e][c = cb*32 + frow] of tap t
    float *wsg = wp.ws + ((int64_t)split * wp.G + g) * (int64_t)wp.K * wp.taps * wp.C;
#pragma unroll
    for (int i = 0; i < S::NBW; ++i) {
        const int blk = wave + 4 * i;
        if (blk < S::NBLK) {
            const int cb = blk % S::CB, kb = (blk / S::CB) % S::KB, t = t0 + blk / (S::CB * S::KB);
            const int c = c0 + cb * 32 + frow;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int k = k0 + kb * 32 + 8 * j + 4 * kh + e;
                    if (k < wp.K && c < wp.C) wsg[((int64_t)k * wp.taps + t) * wp.C + c] = acc[i][j * 4 + e];
                }
        }
    }
}

// dw[i] = bf16(sum over splits s, in order, of ws[s][i]), four elements per
// thread (n4 = elements / 4)
__global__ void __launch_bounds__(256) wgrad_reduce_kernel(const float4 *__restrict__ ws, uint2 *__restrict__ dw,
                                                           int64_t n4, int splits)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    float4 s = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < splits; ++k) {
        const float4 v = ws[(int64_t)k * n4 + i];
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    dw[i] = uint2{f32x2_to_bf16x2(s.x, s.y), f32x2_to_bf16x2(s.z, s.w)};
}

}  // namespace convfwd
