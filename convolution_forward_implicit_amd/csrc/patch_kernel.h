// Forward convolution with the input patch held in LDS (bf16, gfx950).
//
// Same arithmetic as the implicit GEMM (igemm_dma.h): per group, output
// pixels x output channels, reduced over (z, y, x, c) with fp32 MFMA
// accumulators.  What differs is where the A operand comes from.  The
// implicit GEMM gathers one im2col row per output pixel and filter tap, so
// every input pixel travels from L2 once per tap that reads it (9 times for
// a 3x3 filter).  Here a workgroup owns a TH x TW box of output pixels of one
// (image, output depth) plane and one tile of output channels; each K-step
// is one depth tap z and a CC-channel slice of the input, for which it loads
//   * the input patch the box needs, rows (TH-1)*sh + (Y-1)*dh + 1 by columns
//     (TW-1)*sw + (X-1)*dw + 1, zero outside the input, and
//   * the weights of that (z, channel slice) for all Y*X taps,
// into LDS once (buffer loads straight into LDS, like the implicit GEMM).
// All Y*X taps are then multiplied from that one patch: the A fragment of a
// tap is the patch read at a per-lane pixel offset plus a tap offset that is
// the same for every lane.
//
// LDS rows (one patch pixel, or one weight (n, tap)) are CC channels, plus
// one 16-byte pad chunk when PAD = 1; the pad chunk is written by an
// out-of-range (zero) load, which keeps each wave's 1 KB of LDS writes
// contiguous.  Unpadded 32-byte rows (CC = 16, PAD = 0) swap their two
// 16-byte chunks in every other group of 8 patch pixels (pixel bit 3) and,
// for the weights, in every other group of 16 output channels (channel
// bit 4): a fragment read takes one chunk of 32 pixels (or channels), and
// without the swap pixels 8 apart and channels 16 apart fall into the same
// banks (two-way conflicts on gfx950, measured).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "igemm_dma.h"

namespace convfwd {

struct PatchParams {
    KParams k;
    uint32_t x_bytes;
    uint32_t w_bytes;
    int tiles_h, tiles_w;   // boxes per output plane
    int ph, pw;             // patch rows and columns of this problem
    FastDiv fd_pw, fd_taps;
    FastDiv fd_tw, fd_th, fd_N;   // tiles_w, tiles_h, N
};

template <int TH, int TW, int BN, int CC, int NS, int PHMAX, int PWMAX, int TAPMAX, int PAD>
struct PatchShape {
    static constexpr int NW = 4;                  // waves, splitting the box's pixels
    static constexpr int NT = NW * 64;
    static constexpr int BM = TH * TW;
    static constexpr int TM = BM / NW;            // pixels per wave
    static constexpr int MI = TM / 32, NI = BN / 32;
    static constexpr int CPX = CC / 8 + PAD;      // 16-byte chunks per LDS row (incl. pad)
    static constexpr int PITCH = CPX * 16;        // bytes per LDS row
    static constexpr int PATCH_LOADS = (PHMAX * PWMAX * CPX + 64 * NW - 1) / (64 * NW);  // per wave
    static constexpr int W_LOADS = (BN * TAPMAX * CPX + 64 * NW - 1) / (64 * NW);       // per wave
    static constexpr int L = PATCH_LOADS + W_LOADS;
    static constexpr int PATCH_BYTES = PATCH_LOADS * NW * 1024;
    static constexpr int W_BYTES = W_LOADS * NW * 1024;
    static constexpr int STAGE = PATCH_BYTES + W_BYTES;
    static constexpr bool SWZ = (CPX == 2);       // chunk-pair swap of 32-byte rows
    static constexpr int LDC = BN + 8;
    static constexpr int EPI = BM * LDC * 2;
    static constexpr int LDS_BYTES = NS * STAGE > EPI ? NS * STAGE : EPI;

    static_assert(TW >= 16 && TW <= 256 && (TW & (TW - 1)) == 0, "box width: power of two");
    static_assert(TM % 32 == 0 && BN % 32 == 0 && CC % 16 == 0, "32x32x16 blocks");
    static_assert(NS >= 2 && L * (NS - 2) < 64, "vmcnt budget");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
};

template <int TH, int TW, int BN, int CC, int NS, int PHMAX, int PWMAX, int TAPMAX, int PAD, bool BIAS, bool GELU>
__global__ void __launch_bounds__(256)
patch_conv_kernel(PatchParams pp)
{
    using S = PatchShape<TH, TW, BN, CC, NS, PHMAX, PWMAX, TAPMAX, PAD>;
    const KParams &p = pp.k;
    // Fetch every argument the prologue reads in one batch at entry (left to
    // itself the compiler spreads the scalar argument loads over the blocks
    // of their first use, and the prologue waits for each in turn).
    asm volatile("" ::"s"(gridDim.x), "s"(p.x), "s"(p.w), "s"(pp.x_bytes), "s"(pp.w_bytes),
                 "s"(p.tiles_n), "s"(pp.tiles_w), "s"(pp.tiles_h), "s"(p.Do), "s"(p.N), "s"(p.G),
                 "s"(p.C), "s"(p.K), "s"(p.Di), "s"(p.Hi), "s"(p.Wi), "s"(p.Z), "s"(p.Y), "s"(p.X));
    asm volatile("" ::"s"(p.sd), "s"(p.sh), "s"(p.sw), "s"(p.pd), "s"(p.ph), "s"(p.pw), "s"(p.dd),
                 "s"(p.dh), "s"(p.dw), "s"(p.Kred), "s"(pp.ph), "s"(pp.pw), "s"(pp.fd_pw.m),
                 "s"(pp.fd_pw.s), "s"(pp.fd_taps.m), "s"(pp.fd_taps.s));
    asm volatile("" ::"s"(p.fd_tn.m), "s"(p.fd_tn.s), "s"(pp.fd_tw.m), "s"(pp.fd_tw.s),
                 "s"(pp.fd_th.m), "s"(pp.fd_th.s), "s"(p.fd_Do.m), "s"(p.fd_Do.s), "s"(pp.fd_N.m),
                 "s"(pp.fd_N.s));

    __shared__ __attribute__((aligned(1024))) unsigned char smem[S::LDS_BYTES];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // workgroup -> (n tile, box, plane, group); XCD-contiguous, channel tile fastest
    const int nb = gridDim.x;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = nb >> 3, rem = nb & 7;
    int bid = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    int qt = fdiv(bid, p.fd_tn);
    const int n_tile = bid - qt * p.tiles_n; bid = qt;
    qt = fdiv(bid, pp.fd_tw);
    const int bw_ = bid - qt * pp.tiles_w; bid = qt;
    qt = fdiv(bid, pp.fd_th);
    const int bh_ = bid - qt * pp.tiles_h; bid = qt;
    qt = fdiv(bid, p.fd_Do);
    const int od = bid - qt * p.Do; bid = qt;
    const int g = fdiv(bid, pp.fd_N);
    const int nimg = bid - g * p.N;
    const int oh0 = bh_ * TH, ow0 = bw_ * TW;
    const int n0 = n_tile * BN;

    const i32x4_t xr = buffer_rsrc(p.x, pp.x_bytes);
    const i32x4_t wr = buffer_rsrc(p.w, pp.w_bytes);
    const int GC = p.G * p.C;
    const int ih0 = oh0 * p.sh - p.ph, iw0 = ow0 * p.sw - p.pw;   // patch origin in the input
    const int taps = p.Y * p.X;
    const int csteps = p.C / CC;
    const int nk = p.Z * csteps;

    // ---- loads of one K-step (z, channel slice) ---------------------------
    // Chunk index ci = lane + 64*(wave + NW*t): patch chunks first, weights after.
    uint32_t dv[S::L];
    auto prep = [&](int step) {
        const int z = step / csteps;
        const int cc = (step - z * csteps) * CC;
        const int id = od * p.sd - p.pd + z * p.dd;
        const bool plane_ok = (unsigned)id < (unsigned)p.Di;
        const int npatch = pp.ph * pp.pw * S::CPX;
#pragma unroll
        for (int t = 0; t < S::PATCH_LOADS; ++t) {
            const int ci = lane + 64 * (wave + S::NW * t);
            const int pix = ci / S::CPX, q = ci - pix * S::CPX;
            const int r = fdiv(pix, pp.fd_pw), cpos = pix - r * pp.pw;
            const int ih = ih0 + r, iw = iw0 + cpos;
            const bool ok = plane_ok && ci < npatch && q < CC / 8 && (unsigned)ih < (unsigned)p.Hi &&
                            (unsigned)iw < (unsigned)p.Wi;
            const int qg = S::SWZ ? q ^ ((pix >> 3) & 1) : q;   // chunk stored in slot q
            const int off = ((((nimg * p.Di + id) * p.Hi + ih) * p.Wi + iw) * GC) + g * p.C + cc + qg * 8;
            dv[t] = ok ? (uint32_t)(off * 2) : kOutOfRange;
        }
        const int nw = BN * taps * S::CPX;
#pragma unroll
        for (int t = 0; t < S::W_LOADS; ++t) {
            const int ci = lane + 64 * (wave + S::NW * t);
            const int row = ci / S::CPX, q = ci - row * S::CPX;
            const int n = fdiv(row, pp.fd_taps), tap = row - n * taps;
            const bool ok = ci < nw && q < CC / 8 && n0 + n < p.K;
            const int qg = S::SWZ ? q ^ ((n >> 4) & 1) : q;
            const int off = (g * p.K + n0 + n) * p.Kred + (z * taps + tap) * p.C + cc + qg * 8;
            dv[S::PATCH_LOADS + t] = ok ? (uint32_t)(off * 2) : kOutOfRange;
        }
    };
    auto fire = [&](int stage, int t) {
        const uint32_t base = lds0 + stage * S::STAGE;
        if (t < S::PATCH_LOADS)
            dma16(xr, dv[t], 0, base + (wave + S::NW * t) * 1024);
        else
            dma16(wr, dv[t], 0, base + S::PATCH_BYTES + (wave + S::NW * (t - S::PATCH_LOADS)) * 1024);
    };

    // ---- this lane's fragment rows -----------------------------------------
    const int frow = lane & 31;          // pixel row of an A block / channel of a B block
    const int half = lane >> 5;          // which 16-byte chunk of a 32-byte k-slice
    int abase[S::MI];                    // LDS byte offset of the lane's pixel in the patch
#pragma unroll
    for (int i = 0; i < S::MI; ++i) {
        const int m = wave * S::TM + i * 32 + frow;
        const int th = m / TW, tw = m % TW;
        abase[i] = ((th * p.sh) * pp.pw + tw * p.sw) * S::PITCH;
    }
    const int wrow = taps * S::PITCH;    // bytes per output channel in the weight slice

    f32x16_t acc[S::MI][S::NI];
#pragma unroll
    for (int i = 0; i < S::MI; ++i)
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // One K-step: every tap from the same patch, CC/16 k sub-steps per tap,
    // walked as one sequence of (tap, sub-step) pairs.  Fragments are read
    // one pair ahead (two register sets), so each pair's LDS reads are in
    // flight while the previous pair's products run.  The next stage's loads
    // are issued after the first pair's products; the remaining pairs cover
    // their latency.
    constexpr int HS = CC / 16;
    auto load_frags = [&](const unsigned char *P, const unsigned char *Wt, int pr, bf16x8_t (&a)[S::MI],
                          bf16x8_t (&b)[S::NI]) {
        const int tap = pr / HS, h = pr - tap * HS;
        const int y = tap / p.X, x = tap - y * p.X;
        const int toff = ((y * p.dh) * pp.pw + x * p.dw) * S::PITCH;
        const int co = (2 * h + half) * 16;
#pragma unroll
        for (int i = 0; i < S::MI; ++i) {
            const int t = abase[i] + toff;       // byte offset of the lane's pixel
            const int ca = S::SWZ ? (half ^ ((t >> 8) & 1)) * 16 : co;   // pixel bit 3 = byte bit 8
            a[i] = *reinterpret_cast<const bf16x8_t *>(P + t + ca);
        }
        const int cb = S::SWZ ? (half ^ ((frow >> 4) & 1)) * 16 : co;
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
            b[j] = *reinterpret_cast<const bf16x8_t *>(Wt + (j * 32 + frow) * wrow + tap * S::PITCH + cb);
    };
    auto mma = [&](const bf16x8_t (&a)[S::MI], const bf16x8_t (&b)[S::NI]) {
#pragma unroll
        for (int i = 0; i < S::MI; ++i)
#pragma unroll
            for (int j = 0; j < S::NI; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], a[i], acc[i][j], 0, 0, 0);
    };
    auto compute = [&](int stage, int dst) {
        const unsigned char *P = smem + stage * S::STAGE;
        const unsigned char *Wt = P + S::PATCH_BYTES;
        const int npairs = taps * HS;
        bf16x8_t a0[S::MI], b0[S::NI], a1[S::MI], b1[S::NI];
        load_frags(P, Wt, 0, a0, b0);
        int pr = 0;
        for (; pr + 1 < npairs; pr += 2) {
            load_frags(P, Wt, pr + 1, a1, b1);
            mma(a0, b0);
            if (pr == 0 && dst >= 0) {
#pragma unroll
                for (int t = 0; t < S::L; ++t) fire(dst, t);
            }
            if (pr + 2 < npairs) load_frags(P, Wt, pr + 2, a0, b0);
            mma(a1, b1);
        }
        if (pr < npairs) {          // odd number of pairs: the last one is in a0/b0
            mma(a0, b0);
            if (pr == 0 && dst >= 0) {
#pragma unroll
                for (int t = 0; t < S::L; ++t) fire(dst, t);
            }
        }
    };

    // ---- pipeline ----------------------------------------------------------
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nk) {
            prep(s);
#pragma unroll
            for (int t = 0; t < S::L; ++t) fire(s, t);
        }
    for (int it = 0; it < nk - 1; ++it) {
        if (it + NS - 2 < nk) wait_vmcnt<S::L * (NS - 2)>();
        else wait_vmcnt<0>();
        __syncthreads();
        const bool more = it + NS - 1 < nk;
        if (more) prep(it + NS - 1);
        compute(it % NS, more ? (it + NS - 1) % NS : -1);
    }
    // last step: nothing left to load
    wait_vmcnt<0>();
    __syncthreads();
    // Bias of the lane's output channels, loaded here so that the last step's
    // products hide its latency.
    float bias_v[S::NI][4][4];
    if constexpr (BIAS) {
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int hh = 0; hh < 4; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // unconditional (clamped) loads, so they are all in flight at once
                    const int n = n0 + j * 32 + hh * 8 + half * 4 + e;
                    const float v = bf16_to_f32(reinterpret_cast<const uint16_t *>(p.bias)[g * p.K + (n < p.K ? n : p.K - 1)]);
                    bias_v[j][hh][e] = n < p.K ? v : 0.f;
                }
    }
    compute((nk - 1) % NS, -1);
    __syncthreads();

    // ---- epilogue (as the implicit GEMM: transposed 32x32 blocks) ----------
    uint16_t *Cs = reinterpret_cast<uint16_t *>(smem);
#pragma unroll
    for (int j = 0; j < S::NI; ++j)
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
            const int nl = j * 32 + hh * 8 + half * 4;
            float bv[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (BIAS) {
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[e] = bias_v[j][hh][e];
            }
#pragma unroll
            for (int i = 0; i < S::MI; ++i) {
                const int ml = wave * S::TM + i * 32 + frow;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[i][j][hh * 4 + e] + bv[e];
                    if constexpr (GELU) v[e] = gelu_erf_bf16out(v[e]);
                }
                uint2 pk;
                pk.x = f32x2_to_bf16x2(v[0], v[1]);
                pk.y = f32x2_to_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2 *>(Cs + ml * S::LDC + nl) = pk;
            }
        }
    __syncthreads();

    uint16_t *__restrict__ yg = reinterpret_cast<uint16_t *>(p.y) + g * p.K;
    const int GK = p.ldy;   // output row pitch
    constexpr int OVPR = BN / 8;
    if (!p.out_vec) {   // K not a whole number of vectors: element stores
        for (int idx = tid; idx < S::BM * OVPR; idx += S::NT) {
            const int row = idx / OVPR;
            const int cv = idx % OVPR;
            const int oh = oh0 + row / TW, ow = ow0 + row % TW;
            const int n = n0 + cv * 8;
            if (oh >= p.Ho || ow >= p.Wo || n >= p.K) continue;
            const int m = ((nimg * p.Do + od) * p.Ho + oh) * p.Wo + ow;
            const uint16_t *src = Cs + row * S::LDC + cv * 8;
            uint16_t *dst = yg + (size_t)m * GK + n;
            const int lim = (p.K - n) < 8 ? (p.K - n) : 8;
            for (int e = 0; e < lim; ++e) dst[e] = src[e];
        }
        return;
    }
    // Whole 16-byte vectors: every read from LDS is issued before any store
    // (a native vector type, which stays in registers).
    constexpr int NV = S::BM * OVPR;
    constexpr int ITERS = (NV + S::NT - 1) / S::NT;
    i32x4_t val[ITERS];
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int idx0 = tid + it * S::NT;
        const int idx = idx0 < NV ? idx0 : NV - 1;
        val[it] = *reinterpret_cast<const i32x4_t *>(Cs + (idx / OVPR) * S::LDC + (idx % OVPR) * 8);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
        const int idx = tid + it * S::NT;
        const int row = idx / OVPR;
        const int oh = oh0 + row / TW, ow = ow0 + row % TW;
        const int n = n0 + (idx % OVPR) * 8;
        if (idx < NV && oh < p.Ho && ow < p.Wo && n < p.K) {
            const int m = ((nimg * p.Do + od) * p.Ho + oh) * p.Wo + ow;
            __builtin_nontemporal_store(val[it], reinterpret_cast<i32x4_t *>(yg + (size_t)m * GK + n));
        }
    }
}

}  // namespace convfwd
