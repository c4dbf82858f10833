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
// copy is dy itself with padding off, and no copy is made.  A 1-D strided
// problem runs as its stride phases instead (below): no spread copy, and
// none of the products with its zeros.
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

// Stride phases of a 1-D input gradient (stride s > 1 along W).  Input
// position i = s j + f takes the taps t with (f + p - t d) divisible by s,
// dy[j + (f + p - t d) / s]: for each phase f a stride-1 forward convolution
// of dy itself, with those taps (largest first, so the dy offset grows by
// d / gcd(s, d) per tap) -- no spread copy and no products with its zeros.
// Phase f's filter is w_f[g][c][u][k] = w[g][k][tmax_f - u dt][c] (dt =
// s / gcd(s, d)); all phases' filters are written back to back, phase f's
// from element base[f].
constexpr int kMaxPhases = 8;
struct PhaseWeightParams {
    int G, K, C, X;                   // groups, channels and taps of w
    int nphase, dt;
    int ntap[kMaxPhases], tmax[kMaxPhases];
    int64_t base[kMaxPhases + 1];     // each phase's filter starts 256-byte aligned; base[nphase] = the total
};

template <typename T>
__global__ void __launch_bounds__(256) bwd_data_phase_weights_kernel(const T *__restrict__ w, T *__restrict__ wt,
                                                                     PhaseWeightParams q)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    // the phase of element i, and its tap count, first tap and base, by
    // unrolled selects (a dynamic index into the argument arrays would copy
    // them to scratch memory)
    int f = 0;
#pragma unroll
    for (int r = 1; r < kMaxPhases; ++r)
        if (r < q.nphase && i >= q.base[r]) f = r;
    int64_t b = q.base[0];
    int F = q.ntap[0], tm = q.tmax[0];
#pragma unroll
    for (int r = 1; r < kMaxPhases; ++r)
        if (r == f) { b = q.base[r]; F = q.ntap[r]; tm = q.tmax[r]; }
    // the alignment gap after a phase's filter, and past the last one
    if (i - b >= (int64_t)q.G * q.C * F * q.K) return;
    int64_t t = i - b;
    const int k = (int)(t % q.K); t /= q.K;
    const int u = (int)(t % F); t /= F;
    const int c = (int)(t % q.C); t /= q.C;
    const int64_t g = t;
    wt[i] = w[((g * q.K + k) * q.X + (tm - u * q.dt)) * q.C + c];
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

#include "igemm_dma.h"

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
// values, pixel pairs in one dword; with the lanes running over pixel pairs
// fastest, the 18-dword pitch puts at most two lanes of a staging store on a
// bank).  Loads are 16 bytes (8 channels of one pixel).
//
// A workgroup owns a KT x CT block of (k, c) for TT taps of one group and a
// contiguous range of pixel steps (split-K over the pixels: a weight
// gradient has few outputs and a long reduction); its fp32 partial tile
// goes to a caller workspace [split][g][k][t][c], and wgrad_reduce_kernel
// sums the splits in index order (deterministic) and rounds to bf16.  The
// 32x32x16 bf16 MFMA takes dy rows as the first operand (k) and x rows as
// the second (c); block b = (t * KB + kb) * CB + cb goes to wave b mod NWV
// (the workgroup's wave count, a multiple of KB * CB), so a wave keeps one
// (kb, cb) over its taps and reads its dy fragment once per step.  Channels
// per group must be multiples of 8 (16-byte rows).
struct WgradParams {
    const void *x, *dy;
    float *ws;                 // partials [split][G][K][taps][C]
    uint32_t x_bytes, dy_bytes;   // both below 2^31: 32-bit buffer offsets
    int N, G, C, K;
    int Di, Hi, Wi, Do, Ho, Wo;
    int sd, sh, sw, pd, ph, pw, dd, dh, dw;
    int Y, X, taps;
    int64_t pixels;            // N * Do * Ho * Wo
    int steps_per_split;       // PC-pixel steps per workgroup
    int splits, kt_n, ct_n, tg_n;
    FastDiv fd_Wo, fd_Ho, fd_Do;
};

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));

template <int KT, int CT, int TT, int NWV>
struct WgradShape {
    static constexpr int NT = NWV * 64;                 // threads of the workgroup
    static constexpr int PC = 32;                       // pixels per K-step
    static constexpr int QN = CT / 8;                   // 16-byte chunks per pixel row
    static constexpr int RG = TT + 1;                   // row groups: dy, then one per tap
    static constexpr int PITCH = 72;                    // bytes per LDS row
    static constexpr int ROWS = KT + TT * CT;
    static constexpr int LDS_BYTES = ROWS * PITCH;
    static constexpr int NTG = NT / (QN * PC / 2);      // thread groups over the row groups
    static constexpr int UPT = (RG + NTG - 1) / NTG;    // staging units per thread
    static constexpr int KB = KT / 32, CB = CT / 32;
    static constexpr int NBLK = TT * KB * CB;           // 32x32 output blocks
    static constexpr int NBW = (NBLK + NWV - 1) / NWV;  // blocks per wave
    static_assert(KT == CT, "one chunk count for both operands");
    static_assert(KT == 32 || KT == 64, "32 or 64 channels per tile");
    static_assert(NBW * 16 <= 160, "accumulators");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

template <int KT, int CT, int TT, int NWV>
__global__ void __launch_bounds__(NWV * 64) wgrad_kernel(WgradParams wp)
{
    using S = WgradShape<KT, CT, TT, NWV>;
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
    if (wp.pixels <= 0) return;
    const int step0 = split * wp.steps_per_split;
    const int nsteps_total = (int)((wp.pixels + S::PC - 1) / S::PC);
    int nsteps = nsteps_total - step0;
    if (nsteps > wp.steps_per_split) nsteps = wp.steps_per_split;
    const int pixels = (int)wp.pixels;

    // ---- this thread's staging units: row group r = tg + NTG*u, chunk q, pixel pair pp
    // pixel pairs fastest: the transposed LDS writes of a wave (rows 8q + e,
    // dword column pp, 18-dword pitch) then fall at most two to a bank
    const int pp = tid % (S::PC / 2);
    const int q = (tid / (S::PC / 2)) % S::QN;
    // a thread group spans whole waves (QN * PC / 2 is 64 or 128 threads)
    const int tg = __builtin_amdgcn_readfirstlane(tid / (S::QN * S::PC / 2));
    const int Di = wp.Di, Hi = wp.Hi, Wi = wp.Wi;
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
    // Raw buffer loads with 32-bit byte offsets: an offset at or past the
    // buffer's size (kOutOfRange) reads zeros, which is how padding, ragged
    // channel tiles and pixels past the end are masked.
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(wp.x), (short)0,
                                                                        (int)wp.x_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rdy = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(wp.dy), (short)0,
                                                                         (int)wp.dy_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t r0 = tg == 0 ? rdy : rx;   // the first unit's tensor
    // this thread's channel chunk of dy (k) and of x (c), as byte offsets
    const int kq = k0 + 8 * q, cq = c0 + 8 * q;
    const bool kin = kq < wp.K, cin = cq < wp.C;
    const uint32_t dyq = (uint32_t)(g * wp.K + kq) * 2u, xq = (uint32_t)(g * wp.C + cq) * 2u;
    const uint32_t gk2 = (uint32_t)(wp.G * wp.K) * 2u, gc2 = (uint32_t)(wp.G * wp.C) * 2u;
    uint32_t toffb[S::UPT];                     // byte offset of each unit's tap
#pragma unroll
    for (int u = 0; u < S::UPT; ++u) toffb[u] = (uint32_t)((tz[u] * Hi + ty[u]) * Wi + tx[u]) * gc2;

    // Staging registers, two steps deep.  Every unit issues its load, masked
    // or not, so the loads of a step are a fixed count and the wait before a
    // store covers the older step only.
    u32x4_t v[2][S::UPT][2];
    // The refill of one buffer in two parts: the pixel arithmetic of the
    // thread's two pixels (prep), then one 16-byte load per (unit, pixel)
    // (unit), so the loads can be spread between products.
    struct Pix {
        int id0, ih0, iw0;
        uint32_t xb, dyoff;   // byte offset of tap (0, 0, 0) of the thread's chunk; dy's, or masked
        bool pok;
    };
    Pix px[2];
    auto prep = [&](int step) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int P = step * S::PC + 2 * pp + h;
            const bool pok = P < pixels;
            // a pixel past the end decomposes as the last one; its units are masked
            const int pi = pok ? P : pixels - 1;
            const int a = fdiv(pi, wp.fd_Wo);
            const int ow = pi - a * wp.Wo;
            const int b2 = fdiv(a, wp.fd_Ho);
            const int oh = a - b2 * wp.Ho;
            const int n = fdiv(b2, wp.fd_Do);
            const int od = b2 - n * wp.Do;
            Pix &x = px[h];
            x.id0 = od * wp.sd - wp.pd;
            x.ih0 = oh * wp.sh - wp.ph;
            x.iw0 = ow * wp.sw - wp.pw;
            // pixel of tap (0, 0, 0), possibly in the padding: in-range taps wrap back
            x.xb = xq + (uint32_t)(((n * Di + x.id0) * Hi + x.ih0) * Wi + x.iw0) * gc2;
            // bitwise ands throughout: short-circuit forms become branches around the loads
            x.dyoff = (pok & kin) ? dyq + (uint32_t)P * gk2 : kOutOfRange;
            x.pok = pok;
        }
    };
    auto unit = [&](int bsel, int u, int h) __attribute__((always_inline)) {
        const Pix &x = px[h];
        const int r = tg + S::NTG * u;
        // a unit past the last row group loads a masked offset too
        const bool live = S::RG % S::NTG == 0 || r < S::RG;
        const bool in = live & x.pok & cin & ((unsigned)(x.id0 + tz[u]) < (unsigned)Di) &
                        ((unsigned)(x.ih0 + ty[u]) < (unsigned)Hi) & ((unsigned)(x.iw0 + tx[u]) < (unsigned)Wi);
        const uint32_t xoff = in ? x.xb + toffb[u] : kOutOfRange;
        // row group 0 is dy (thread group 0, first unit), the rest are taps of x
        if (u == 0)
            v[bsel][u][h] = __builtin_amdgcn_raw_buffer_load_b128(r0, tg == 0 ? x.dyoff : xoff, 0, 0);
        else
            v[bsel][u][h] = __builtin_amdgcn_raw_buffer_load_b128(rx, xoff, 0, 0);
    };
    auto load = [&](int bsel, int step) __attribute__((always_inline)) {
        prep(step);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int u = 0; u < S::UPT; ++u) unit(bsel, u, h);
    };
    // transposed store: row (row group base + 8q + e), dword column pp = pixels (2pp, 2pp+1)
    auto store = [&](int bsel) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < S::UPT; ++u) {
            const int r = tg + S::NTG * u;
            if (r < S::RG) {
                const int row0 = (r == 0 ? 0 : KT + (r - 1) * CT) + 8 * q;
                const u32x4_t lo = v[bsel][u][0], hi = v[bsel][u][1];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // channel e of pixel 2pp in the low half, of pixel 2pp+1 in the high half
                    const uint32_t w = __builtin_amdgcn_perm(hi[e >> 1], lo[e >> 1], (e & 1) ? 0x07060302u : 0x05040100u);
                    *reinterpret_cast<uint32_t *>(smem + (row0 + e) * S::PITCH + 4 * pp) = w;
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
    static_assert(NWV % (S::KB * S::CB) == 0, "a wave keeps one (kb, cb)");
    constexpr int TSTEP = NWV / (S::KB * S::CB);   // taps between a wave's blocks
    const int kbw = (wave / S::CB) % S::KB, cbw = wave % S::CB, tw0 = wave / (S::KB * S::CB);

    // Fragments are read as 32-bit words and reinterpreted as bf16 at the
    // product (as bf16 vectors the compiler repacks them element by element).
    // Every wave runs NBW blocks: a block past the last (when NWV does not
    // divide the count) reads the last tap's rows and its sums are never
    // stored, so no read or product is predicated.
    constexpr int NM = 2 * S::NBW;              // products per wave and step
    constexpr int NL = 2 * S::UPT;              // loads per thread and step
    // One step: the staged registers of buffer bsel go to LDS; the step's
    // fragments are read; then its products run with the refill of buffer
    // bsel two steps ahead interleaved (the refill's address arithmetic is
    // VALU work the matrix unit does not wait for: one wave per SIMD has
    // no other wave to hide it behind).  The refill is unconditional (past
    // the split's last step it reads pixels that are never stored, or
    // masked ones), which keeps the number of loads in flight the same on
    // every path, so each store waits for its own step's loads only.
    auto step = [&](int bsel, int it) __attribute__((always_inline)) {
        __syncthreads();                      // the previous step's fragments are read
        store(bsel);
        __syncthreads();                      // this step is in LDS
        // Block wave + NWV i has tap t = tw0 + TSTEP i and the wave's own
        // (kb, cb) (NWV is a multiple of the KB x CB channel blocks), so the
        // dy fragment is read once per 16-pixel half and serves every tap of
        // the wave; a block past the last reads the last tap's rows.
        u32x4_t fa[2], fb[2][S::NBW];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int co = 32 * s + 16 * kh;  // byte offset of the lane's 8 pixels
            // rows are 8-byte aligned (72-byte pitch): two 8-byte LDS reads per fragment
            fa[s] = *reinterpret_cast<const u32x4_a8 *>(smem + (kbw * 32 + frow) * S::PITCH + co);
#pragma unroll
            for (int i = 0; i < S::NBW; ++i) {
                const int t = min(tw0 + TSTEP * i, TT - 1);
                fb[s][i] = *reinterpret_cast<const u32x4_a8 *>(smem + (KT + t * CT + cbw * 32 + frow) * S::PITCH + co);
            }
        }
        prep(step0 + it + 2);
        __builtin_amdgcn_sched_barrier(0);
        // products, each followed by one load of the refill
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int s = m / S::NBW, i = m % S::NBW;
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[s]),
                                                             __builtin_bit_cast(bf16x8_t, fb[s][i]), acc[i], 0, 0, 0);
            if (m < NL) unit(bsel, m % S::UPT, m / S::UPT);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int m = NM; m < NL; ++m) unit(bsel, m % S::UPT, m / S::UPT);
    };

    load(0, step0);
    load(1, step0 + 1);
    int it = 0;
    for (; it + 1 < nsteps; it += 2) {
        step(0, it);
        step(1, it + 1);
    }
    if (it < nsteps) step(0, it);

    // ---- partial tile: lane holds dw[k = kb*32 + 8j + 4kh + e][c = cb*32 + frow] of tap t
    float *wsg = wp.ws + ((int64_t)split * wp.G + g) * (int64_t)wp.K * wp.taps * wp.C;
#pragma unroll
    for (int i = 0; i < S::NBW; ++i) {
        const int blk = wave + NWV * i;
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
// thread (n4 = elements / 4).  The partials are read eight splits at a time,
// all eight loads issued before the adds, which keep the split order.
__global__ void __launch_bounds__(64) wgrad_reduce_kernel(const float4 *__restrict__ ws, uint2 *__restrict__ dw,
                                                          int64_t n4, int splits)
{
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (i >= n4) return;
    float4 s = {0.f, 0.f, 0.f, 0.f};
    int k = 0;
    for (; k + 8 <= splits; k += 8) {
        float4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = ws[(int64_t)(k + j) * n4 + i];
#pragma unroll
        for (int j = 0; j < 8; ++j) { s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w; }
    }
    for (; k < splits; ++k) {
        const float4 v = ws[(int64_t)k * n4 + i];
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    dw[i] = uint2{f32x2_to_bf16x2(s.x, s.y), f32x2_to_bf16x2(s.z, s.w)};
}

}  // namespace convfwd
