// Forward convolution with the input patch in LDS and the filter's spatial
// shape fixed at compile time (bf16, gfx950, unit H/W stride).
//
// Same arithmetic as the other kernels (per group: output pixels x output
// channels, reduced over (z, y, x, c) in fp32 MFMA accumulators) and the
// same idea as patch_kernel.h: a workgroup owns a TH x TW box of output
// pixels of one (image, output depth) plane and BN output channels; each
// K-step is one depth tap z and a CC-channel slice, for which it loads the
// input patch the box needs and that slice of the weights for all FY*FX
// taps into LDS once, and every H/W tap is multiplied from the one patch.
//
// What is fixed at compile time here, and what that buys:
//   * FY x FX taps and the H/W dilation DH, DW: a tap is a constant shift of
//     the patch pixel index, so every fragment read is one LDS instruction
//     with a per-lane base address (computed once) and an immediate offset --
//     the K loop does no address arithmetic at all;
//   * the LDS layout is channel-chunk planar: plane q holds 16-byte chunk q
//     (channels 8q .. 8q+7 of the slice) of every patch pixel, pixel-major.
//     A 32x32x16 fragment read takes one chunk of 32 consecutive box pixels,
//     i.e. 512 contiguous bytes of one plane (no bank conflict and no
//     swizzle, whatever the box width; a box row that ends inside a 32-pixel
//     block only shifts the rest of the block);
//   * the box is flattened: pixel m of the box is row m / TW, column m % TW,
//     and 32-pixel MFMA blocks run across row ends, so a box as wide as the
//     output (say 28 or 56) wastes no products on columns past the edge.
// Uniform per-step quantities (the image plane and channel slice of the
// input, the weight slice) ride in the scalar offset of the buffer loads;
// each lane's vector offset is fixed for the whole kernel (the spatial
// position of its patch chunk, or an out-of-range value that reads zeros
// where the patch leaves the input).  Depth taps that fall outside the
// input for the whole plane are skipped (no loads, no products).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "igemm_dma.h"

namespace convfwd {

struct PatchFixedParams {
    KParams k;
    uint32_t x_bytes;
    uint32_t w_bytes;
    int tiles_h, tiles_w;   // boxes per output plane
    // 1: the workgroups of one image's groups are adjacent (group before
    // image in the order).  Set for groups whose channel slice is narrower
    // than a 128-byte line: the groups that share a line then land on one
    // XCD and the line is fetched into one L2, not two (the dilated 3-D
    // workload, 32 channels of bf16 per group: 16.6-17.1 -> 16.0-16.1 us,
    // 15.5-15.7 from prepacked weights, same box)
    int group_fast;
    FastDiv fd_tw, fd_th, fd_N, fd_G;
};

template <int TH, int TW, int BN, int CC, int NS, int FY, int FX, int DH, int DW, int NW, int PM, int RR>
struct PatchFixedShape {
    static constexpr int BM = TH * TW;                 // box pixels
    static constexpr int NBLK = (BM + 31) / 32;        // 32-pixel MFMA blocks of the box
    static constexpr int MI = (NBLK + NW - 1) / NW;    // blocks per wave (the last wave may have fewer)
    static constexpr int NI = BN / 32;
    static constexpr int NT = NW * 64;
    static constexpr int PH = TH + (FY - 1) * DH;      // patch rows and columns
    static constexpr int PW = TW + (FX - 1) * DW;
    static constexpr int NPIX = PH * PW;
    static constexpr int TAPS = FY * FX;
    static constexpr int CPL = CC / 8;                 // 16-byte chunk planes per slice
    static constexpr int HS = CC / 16;                 // 16-element k sub-steps per tap
    // PM = 0: chunk-planar patch (plane q = chunk q of every pixel);
    // PM = 1: pixel-major patch, each pixel's CPL chunks then one pad slot
    // (an odd number of 16-byte slots per pixel, so 16 consecutive pixels of
    // one chunk fall in 16 different bank groups)
    static constexpr int PPITCH = CPL + 1;             // slots per pixel (PM = 1)
    // Pixel-major rows of a flattened box (RR = 0) end with RSK pad slots:
    // a 32-pixel fragment read that crosses a box row end jumps over the
    // row's PW - TW halo pixels, and with RSK = -(PW - TW) * PPITCH mod 16
    // that jump moves the slot index by PPITCH modulo 16 like any other
    // pixel step, so the 16 lanes of a quarter-wave still hit 16 different
    // 16-byte bank groups (without it the reads that straddle a row end
    // were two-way conflicted: 0.33-0.6 conflict cycles per access).
    static constexpr int RSK = (PM && !RR) ? (16 - ((PW - TW) * PPITCH) % 16) % 16 : 0;
    static constexpr int ROWSLOTS = PW * PPITCH + RSK; // slots per patch row (PM = 1)
    static constexpr int PSLOTS = PM ? ROWSLOTS * PH : CPL * NPIX;   // 16-byte patch slots
    static constexpr int PINST = (PSLOTS + 63) / 64;   // 1 KB loads of the patch (workgroup)
    static constexpr int WSLOTS = CPL * TAPS * BN;
    static constexpr int WINST = (WSLOTS + 63) / 64;
    static constexpr int PATCH_LOADS = (PINST + NW - 1) / NW;   // per wave
    static constexpr int W_LOADS = (WINST + NW - 1) / NW;
    static constexpr int L = PATCH_LOADS + W_LOADS;
    static constexpr int PLANE = NPIX * 16;            // bytes of one chunk plane
    static constexpr int PATCH_BYTES = PATCH_LOADS * NW * 1024;
    static constexpr int W_BYTES = W_LOADS * NW * 1024;
    static constexpr int STAGE = PATCH_BYTES + W_BYTES;
    static constexpr int LDC = BN + 8;
    static constexpr int EPI = NBLK * 32 * LDC * 2;
    static constexpr int LDS_BYTES = NS * STAGE > EPI ? NS * STAGE : EPI;

    static_assert(BN % 32 == 0 && CC % 16 == 0, "32x32x16 blocks");
    static_assert(PM == 0 || (PPITCH & 1), "odd pixel pitch");
    static_assert(!RR || (TW == 32 && NBLK == NW * MI), "row reuse: one 32-pixel box row per block, whole rows per wave");
    static_assert(RSK == 0 || !RR, "row reuse addresses rows as PW * PPITCH slots");
    static_assert(NS >= 2 && L * (NS - 2) < 64, "vmcnt budget");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
};

template <int TH, int TW, int BN, int CC, int NS, int FY, int FX, int DH, int DW, int NW, int PM, int RAHEAD,
          int RR, bool BIAS, bool GELU>
__global__ void __launch_bounds__(NW * 64)
patch_fixed_kernel(PatchFixedParams pp)
{
    using S = PatchFixedShape<TH, TW, BN, CC, NS, FY, FX, DH, DW, NW, PM, RR>;
    const KParams &p = pp.k;
    // every argument the prologue reads, fetched in one batch at entry
    asm volatile("" ::"s"(gridDim.x), "s"(p.x), "s"(p.w), "s"(pp.x_bytes), "s"(pp.w_bytes), "s"(p.tiles_n),
                 "s"(pp.tiles_w), "s"(pp.tiles_h), "s"(p.Do), "s"(p.N), "s"(p.G), "s"(p.C), "s"(p.K),
                 "s"(p.Di), "s"(p.Hi), "s"(p.Wi), "s"(p.Z), "s"(p.sd), "s"(p.pd), "s"(p.ph), "s"(p.pw),
                 "s"(p.dd), "s"(p.Kred));
    asm volatile("" ::"s"(p.fd_tn.m), "s"(p.fd_tn.s), "s"(pp.fd_tw.m), "s"(pp.fd_tw.s), "s"(pp.fd_th.m),
                 "s"(pp.fd_th.s), "s"(p.fd_Do.m), "s"(p.fd_Do.s), "s"(pp.fd_N.m), "s"(pp.fd_N.s),
                 "s"(pp.fd_G.m), "s"(pp.fd_G.s), "s"(pp.group_fast));

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
    int g, nimg;
    if (pp.group_fast) {
        nimg = fdiv(bid, pp.fd_G);
        g = bid - nimg * p.G;
    } else {
        g = fdiv(bid, pp.fd_N);
        nimg = bid - g * p.N;
    }
    const int oh0 = bh_ * TH, ow0 = bw_ * TW;
    const int n0 = n_tile * BN;

    const i32x4_t xr = buffer_rsrc(p.x, pp.x_bytes);
    const i32x4_t wr = buffer_rsrc(p.w, pp.w_bytes);
    const int GC = p.G * p.C;
    const int ih0 = oh0 - p.ph, iw0 = ow0 - p.pw;   // patch origin in the input (unit stride)
    const int ncs = p.C / CC;                       // channel slices per depth tap

    // depth taps whose input plane exists (one bit per z)
    uint32_t zmask = 0;
    for (int z = 0; z < p.Z; ++z) {
        const int id = od * p.sd - p.pd + z * p.dd;
        if ((unsigned)id < (unsigned)p.Di) zmask |= 1u << z;
    }
    const int nk = __builtin_popcount(zmask) * ncs;

    // ---- per-lane load offsets, fixed for the whole kernel -----------------
    // patch slot s = (wave + NW*t)*64 + lane: pixel-major, row s / ROWSLOTS
    // and within it pixel-then-chunk (a row's last RSK slots and each
    // pixel's last slot are pads that read zeros), or chunk-planar, chunk
    // plane s / NPIX and patch pixel s % NPIX; weight slot s: (chunk plane,
    // tap, channel) with the channel fastest.
    uint32_t pv[S::PATCH_LOADS], wv[S::W_LOADS];
#pragma unroll
    for (int t = 0; t < S::PATCH_LOADS; ++t) {
        const int s = (wave + NW * t) * 64 + lane;
        int q, r, c;
        if constexpr (PM) {
            r = s / S::ROWSLOTS;
            const int rs = s - r * S::ROWSLOTS;
            c = rs / S::PPITCH;
            q = c < S::PW ? rs - c * S::PPITCH : S::CPL;   // q == CPL: a pad slot (zero)
        } else {
            q = s / S::NPIX;
            const int px = s - q * S::NPIX;
            r = px / S::PW;
            c = px - r * S::PW;
        }
        const int ih = ih0 + r, iw = iw0 + c;
        const bool ok = s < S::PSLOTS && q < S::CPL && (unsigned)ih < (unsigned)p.Hi && (unsigned)iw < (unsigned)p.Wi;
        pv[t] = ok ? (uint32_t)(((ih * p.Wi + iw) * GC + q * 8) * 2) : kOutOfRange;
    }
    // Weights: GKZYXC rows, or (prepacked) the lane's slot of a K-step's
    // image -- the weight part of the LDS stage exactly as laid out here
    // (zeros past K and past the slots), one W_BYTES image per (group,
    // channel tile, depth tap, channel slice), contiguous in that order.
#pragma unroll
    for (int t = 0; t < S::W_LOADS; ++t) {
        const int s = (wave + NW * t) * 64 + lane;
        const int n = s % BN, rest = s / BN;
        const int tap = rest % S::TAPS, q = rest / S::TAPS;
        const bool ok = s < S::WSLOTS && n0 + n < p.K;
        if (p.wpacked)
            wv[t] = (uint32_t)(s * 16);
        else
            wv[t] = ok ? (uint32_t)(((n0 + n) * p.Kred + tap * p.C + q * 8) * 2) : kOutOfRange;
    }
    // scalar (uniform) parts: image and group of the input, group of the weights
    const uint32_t x_plane = (uint32_t)(p.Hi * p.Wi * GC * 2);
    const uint32_t x_img = (uint32_t)(nimg * p.Di) * x_plane + (uint32_t)(g * p.C * 2);
    const uint32_t w_grp = p.wpacked ? (uint32_t)((g * p.tiles_n + n_tile) * p.Z * ncs) * (uint32_t)S::W_BYTES
                                     : (uint32_t)(g * p.K) * (uint32_t)(p.Kred * 2);
    const int id0 = od * p.sd - p.pd;

    // load cursor: (depth tap, channel slice) of the next step to fetch
    int lz = zmask ? __builtin_ctz(zmask) : 0, lcs = 0;
    auto fetch = [&](int stage) __attribute__((always_inline)) {
        const uint32_t xs = x_img + (uint32_t)(id0 + lz * p.dd) * x_plane + (uint32_t)(lcs * CC * 2);
        const uint32_t ws = p.wpacked ? w_grp + (uint32_t)(lz * ncs + lcs) * (uint32_t)S::W_BYTES
                                      : w_grp + (uint32_t)((lz * S::TAPS * p.C + lcs * CC) * 2);
        const uint32_t base = lds0 + stage * S::STAGE;
#pragma unroll
        for (int t = 0; t < S::PATCH_LOADS; ++t) dma16(xr, pv[t], xs, base + (wave + NW * t) * 1024);
#pragma unroll
        for (int t = 0; t < S::W_LOADS; ++t)
            dma16(wr, wv[t], ws, base + S::PATCH_BYTES + (wave + NW * t) * 1024);
        if (++lcs == ncs) {
            lcs = 0;
            const uint32_t rest = zmask & ~((2u << lz) - 1u);
            lz = rest ? __builtin_ctz(rest) : lz;
        }
    };

    // ---- per-lane fragment bases -------------------------------------------
    const int frow = lane & 31;          // pixel of an A block / channel of a B block
    const int half = lane >> 5;          // which 16-byte chunk of a 32-byte k-slice
    int abase[S::MI];
#pragma unroll
    for (int i = 0; i < S::MI; ++i) {
        int m = (wave * S::MI + i) * 32 + frow;
        m = m < S::BM ? m : 0;           // blocks past the box read pixel 0 (never stored)
        const int r = m / TW, c = m - (m / TW) * TW;
        abase[i] = PM ? (r * S::ROWSLOTS + c * S::PPITCH + half) * 16 : half * S::PLANE + (r * S::PW + c) * 16;
    }
    const int bbase = S::PATCH_BYTES + (half * S::TAPS * BN + frow) * 16;

    f32x16_t acc[S::MI][S::NI];
#pragma unroll
    for (int i = 0; i < S::MI; ++i)
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // waves whose block range ends early skip the products of missing blocks
    const int my_blocks = S::NBLK - wave * S::MI;

    // One K-step from LDS stage ST: every (tap, k sub-step) pair, fragments
    // read RA pairs ahead (RA + 1 register sets), so that a wave keeps enough
    // LDS reads in flight to cover their latency (with one pair ahead a
    // wave's reads arrive at about 27 B/clk, less than its products consume);
    // the next stage's loads are issued after the first pair's products (the
    // remaining pairs cover their latency).
    auto step = [&](auto stc, bool fetch_next, int next_stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stc)::value;
        constexpr int NP = S::TAPS * S::HS;
        constexpr int RA = RAHEAD;
        const unsigned char *P = smem + ST * S::STAGE;
        bf16x8_t a[RA + 1][S::MI], b[RA + 1][S::NI];
        auto rd = [&](int pr, int buf) __attribute__((always_inline)) {
            const int tap = pr / S::HS, h = pr - tap * S::HS;
            const int y = tap / FX, x = tap - y * FX;
            const int aoff = PM ? (y * DH * S::ROWSLOTS + x * DW * S::PPITCH + 2 * h) * 16
                                : 2 * h * S::PLANE + (y * DH * S::PW + x * DW) * 16;
            const int boff = ((2 * h * S::TAPS + tap) * BN) * 16;
#pragma unroll
            for (int i = 0; i < S::MI; ++i)
                a[buf][i] = *reinterpret_cast<const bf16x8_t *>(P + abase[i] + aoff);
#pragma unroll
            for (int j = 0; j < S::NI; ++j)
                b[buf][j] = *reinterpret_cast<const bf16x8_t *>(P + bbase + boff + j * 32 * 16);
        };
#pragma unroll
        for (int pr = 0; pr < RA && pr < NP; ++pr) rd(pr, pr);
#pragma unroll
        for (int pr = 0; pr < NP; ++pr) {
            if (pr + RA < NP) rd(pr + RA, (pr + RA) % (RA + 1));
            const int cur = pr % (RA + 1);
#pragma unroll
            for (int i = 0; i < S::MI; ++i) {
                if (S::NBLK % NW != 0 && i >= my_blocks) continue;
#pragma unroll
                for (int j = 0; j < S::NI; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[cur][j], a[cur][i], acc[i][j], 0, 0, 0);
            }
            if (pr == 0 && fetch_next) fetch(next_stage);
        }
    };

    // Row reuse (RR): every block is one 32-pixel box row and a wave owns MI
    // consecutive rows, so tap (y, x) of block i reads patch row i + y*DH
    // (relative to the wave's first row) shifted by x*DW columns.  Walking
    // the patch rows R instead of the (block, tap) pairs, one A fragment
    // read serves every vertical tap y with 0 <= R - y*DH < MI: MI*FY
    // products from MI + (FY-1)*DH reads instead of MI*FY reads (with a
    // group of 32 output channels no fragment is shared across channel
    // blocks, and the fragment reads are what bounds the K loop).
    const int rbase = PM ? ((wave * S::MI * S::PW + frow) * S::PPITCH + half) * 16
                         : half * S::PLANE + (wave * S::MI * S::PW + frow) * 16;
    auto step_rows = [&](auto stc, bool fetch_next, int next_stage) __attribute__((always_inline)) {
        constexpr int ST = decltype(stc)::value;
        constexpr int NR = S::MI + (FY - 1) * DH;     // patch rows a wave reads per (x, k sub-step)
        constexpr int UNIT = PM ? S::PPITCH * 16 : 16; // bytes per patch pixel step
        const unsigned char *P = smem + ST * S::STAGE;
#pragma unroll
        for (int x = 0; x < FX; ++x)
#pragma unroll
            for (int h = 0; h < S::HS; ++h) {
                bf16x8_t bf[FY][S::NI], a[2];
#pragma unroll
                for (int y = 0; y < FY; ++y)
#pragma unroll
                    for (int j = 0; j < S::NI; ++j)
                        bf[y][j] = *reinterpret_cast<const bf16x8_t *>(
                            P + bbase + ((2 * h * S::TAPS + y * FX + x) * BN + j * 32) * 16);
                // chunk step of a k sub-step: two slots (pixel-major) or two planes (chunk-planar)
                const int hoff = PM ? 2 * h * 16 : 2 * h * S::PLANE;
                auto ard = [&](int R) __attribute__((always_inline)) {
                    const int off = (R * S::PW + x * DW) * UNIT + hoff;
                    return *reinterpret_cast<const bf16x8_t *>(P + rbase + off);
                };
                a[0] = ard(0);
#pragma unroll
                for (int R = 0; R < NR; ++R) {
                    if (R + 1 < NR) a[(R + 1) & 1] = ard(R + 1);
#pragma unroll
                    for (int y = 0; y < FY; ++y) {
                        const int i = R - y * DH;
                        if (i < 0 || i >= S::MI) continue;
#pragma unroll
                        for (int j = 0; j < S::NI; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[y][j], a[R & 1], acc[i][j], 0, 0, 0);
                    }
                    if (x == 0 && h == 0 && R == 1 && fetch_next) fetch(next_stage);
                }
            }
    };

    // ---- pipeline: NS stages, the loop unrolled by NS so each stage's LDS
    // base is a constant ------------------------------------------------------
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nk) fetch(s);
    auto one = [&](auto stc, int it) __attribute__((always_inline)) {
        constexpr int ST = decltype(stc)::value;
        if (it + NS - 2 <= nk - 1) wait_vmcnt<S::L * (NS - 2)>();
        else wait_vmcnt<0>();
        __syncthreads();
        const bool more = it + NS - 1 < nk;
        if constexpr (RR) step_rows(stc, more, (ST + NS - 1) % NS);
        else step(stc, more, (ST + NS - 1) % NS);
    };
    for (int it = 0; it < nk; it += NS) {
        one(std::integral_constant<int, 0>{}, it);
        if (it + 1 < nk) one(std::integral_constant<int, 1 % NS>{}, it + 1);
        if constexpr (NS > 2) {
            if (it + 2 < nk) one(std::integral_constant<int, 2 % NS>{}, it + 2);
        }
        if constexpr (NS > 3) {
            if (it + 3 < nk) one(std::integral_constant<int, 3 % NS>{}, it + 3);
        }
    }

    // bias of the lane's output channels (clamped loads, all in flight at once)
    float bias_v[S::NI][4][4];
    if constexpr (BIAS) {
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int hh = 0; hh < 4; ++hh)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int n = n0 + j * 32 + hh * 8 + half * 4 + e;
                    const float v = bf16_to_f32(reinterpret_cast<const uint16_t *>(p.bias)[g * p.K + (n < p.K ? n : p.K - 1)]);
                    bias_v[j][hh][e] = n < p.K ? v : 0.f;
                }
    }
    __syncthreads();

    // ---- epilogue: the tile through LDS, then whole 16-byte stores ---------
    uint16_t *Cs = reinterpret_cast<uint16_t *>(smem);
#pragma unroll
    for (int i = 0; i < S::MI; ++i) {
        if (S::NBLK % NW != 0 && i >= my_blocks) continue;
        const int ml = (wave * S::MI + i) * 32 + frow;
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) {
                const int nl = j * 32 + hh * 8 + half * 4;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[i][j][hh * 4 + e];
                    if constexpr (BIAS) v[e] += bias_v[j][hh][e];
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
    // whole 16-byte vectors: every LDS read issued before any store
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
