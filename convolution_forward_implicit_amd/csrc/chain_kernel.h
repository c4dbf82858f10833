// Fused two-conv 1-D frontend on gfx950 (bf16): y = act(conv2(h) + b2) with
// h = round_bf16(act(conv1(x) + b1)), conv1 k3 s1 p1 (C1 -> 384 channels),
// conv2 k3 s2 p1 (384 -> 384), act = GELU or identity -- the two-conv
// frontend of the ExecuTorch conv1d issue (the table that splits it into
// conv1 + GELU + conv2 + GELU), with the intermediate kept on chip.
//
// Unfused, h makes a full round trip through HBM (73.7 MB written and read
// again at batch 32).  Here a workgroup owns TO = 63 consecutive outputs of
// one sequence and all 384 output channels, and works in two phases in one
// launch:
//
//  1. conv1 for the 2*TO + 1 = 127 positions of h those outputs read
//     (positions 2*o0 - 1 .. 2*o0 + 2*TO - 1), from an input patch of 129
//     positions x C1 channels in LDS.  Bias, activation and the bf16
//     rounding are applied in registers and h is written to LDS (positions
//     outside the sequence are written as zeros: conv2's padding).
//  2. conv2 from h in LDS: output row o, tap t reads h row 2*o + t.
//
// Both phases are GEMMs on 32x32x16 bf16 MFMAs (fp32 accumulation), the
// product transposed as in the implicit GEMM (weights as the first operand,
// so lanes hold runs of 4 consecutive channels).  Four waves each own 96
// output channels (3 blocks); phase 1 covers 128 rows (4 blocks, one unused),
// phase 2 64 rows (2 blocks, one unused).  The weights stream through five
// LDS stages of 16 reduction elements x 384 rows (buffer loads straight into
// LDS, as in the implicit GEMM), w1's 3*C1/16 steps followed by w2's 72
// steps; while a step is multiplied, the next step's fragments are read
// from LDS and three more steps are in flight from L2.
//
// LDS (bytes): h tile 127 x 768 at 0 (the input patch aliases it during
// phase 1, the output staging after phase 2), 5 x 12288 weight stages at
// 97536, and the biases as fp32 at 158976.  Swizzles (each measured
// conflict-free with an LDS read probe):
//  * input patch, 2*C1-byte rows: 16-byte chunk q of position p at slot
//    q ^ ((p >> 3) & 1);
//  * weight stages, 32-byte rows: half h of channel n at slot h ^ ((n >> 3) & 1);
//  * h tile, 768-byte rows: chunk q of row r at slot q ^ ((r >> 1) & 15).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "igemm_dma.h"

namespace convfwd {

struct ChainParams {
    const void *x, *w1, *b1, *w2, *b2;   // b1 and b2 NULL without bias
    void *y;
    int N, L, C1, Lo;                    // batch, input length, conv1 input channels, output length
    int tiles;                           // output tiles per sequence
    uint32_t x_bytes, w1_bytes, w2_bytes;
};

struct ChainShape {
    static constexpr int K = 384;                 // conv1 out = conv2 in = conv2 out channels
    static constexpr int TO = 63;                 // conv2 outputs per workgroup
    static constexpr int HR = 2 * TO + 1;         // h rows
    static constexpr int XR = HR + 2;             // input patch rows
    static constexpr int HP = 2 * K;              // bytes per h row
    static constexpr int H_BYTES = HR * HP;       // 97536
    static constexpr int STAGE = K * 32;          // 16 bf16 of every weight row
    static constexpr int NST = 5;
    static constexpr int STG0 = H_BYTES;
    static constexpr int BIAS0 = STG0 + NST * STAGE;
    static constexpr int LDS_BYTES = BIAS0 + 2 * K * 4;
    static constexpr int C1MAX = 352;             // input patch within the h region
    static constexpr int YP = HP + 16;            // output staging row pitch
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
    static_assert(XR * C1MAX * 2 <= H_BYTES && 64 * YP <= H_BYTES, "aliases of the h region");
};

template <bool BIAS, bool GELU>
__global__ void __launch_bounds__(256) chain_kernel(ChainParams cp)
{
    using S = ChainShape;
    constexpr int K = S::K;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[S::LDS_BYTES];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int frow = lane & 31;           // row of an operand block
    const int kh = lane >> 5;             // which 8 of a block's 16 reduction elements

    // workgroup -> (sequence, output tile); tiles contiguous per XCD
    const int nb = gridDim.x;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = nb >> 3, rem = nb & 7;
    const int bid = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    const int n = bid / cp.tiles;
    const int o0 = (bid - n * cp.tiles) * S::TO;
    const int hp0 = 2 * o0 - 1;           // sequence position of h row 0
    const int xp0 = hp0 - 1;              // sequence position of patch row 0

    const int C1 = cp.C1;
    const int PX = 2 * C1;                // bytes per patch row
    const int K1 = 3 * C1, K2 = 3 * K;    // reduction lengths
    const int NC1 = K1 / 16, NC = NC1 + K2 / 16;

    const i32x4_t xr = buffer_rsrc(cp.x, cp.x_bytes);
    const i32x4_t w1r = buffer_rsrc(cp.w1, cp.w1_bytes);
    const i32x4_t w2r = buffer_rsrc(cp.w2, cp.w2_bytes);

    // ---- loads -----------------------------------------------------------
    // step j < NC1 holds w1[:, 16j .. 16j+16), step j >= NC1 holds
    // w2[:, 16(j-NC1) ..); each lane moves three 16-byte chunks per step
    auto fire_step = [&](int j) {
        const bool first = j < NC1;
        const int k0 = (first ? j : j - NC1) * 16;
        const int kt = first ? K1 : K2;
        const uint32_t base = lds0 + S::STG0 + (j % S::NST) * S::STAGE;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const int ci = lane + 64 * (wave + 4 * t);      // 0 .. 767
            const int ch = ci >> 1, hs = ci & 1;
            const int g = hs ^ ((ch >> 3) & 1);             // half stored in slot hs
            const uint32_t off = (uint32_t)((ch * kt + k0 + g * 8) * 2);
            dma16(first ? w1r : w2r, off, 0, base + (wave + 4 * t) * 1024);
        }
    };
    // input patch: XR positions x C1 channels; chunk ci lands at byte 16*ci
    {
        const int cpx = C1 / 8;
        const int nchunks = S::XR * cpx;
        for (int t = 0; 64 * (wave + 4 * t) < nchunks; ++t) {
            const int ci = lane + 64 * (wave + 4 * t);
            const int p = ci / cpx, q = ci - p * cpx;
            const int xp = xp0 + p;
            const int qg = q ^ ((p >> 3) & 1);
            const bool ok = ci < nchunks && (unsigned)xp < (unsigned)cp.L;
            const uint32_t off = ok ? (uint32_t)(((n * cp.L + xp) * C1 + qg * 8) * 2) : kOutOfRange;
            dma16(xr, off, 0, lds0 + (wave + 4 * t) * 1024);
        }
    }
#pragma unroll
    for (int j = 0; j < S::NST - 1; ++j)
        if (j < NC) fire_step(j);
    // biases to LDS as fp32 (their global loads complete before the first step)
    float *bias_lds = reinterpret_cast<float *>(smem + S::BIAS0);
    if constexpr (BIAS) {
        for (int i = tid; i < 2 * K; i += 256) {
            const uint16_t *b = reinterpret_cast<const uint16_t *>(i < K ? cp.b1 : cp.b2);
            bias_lds[i] = bf16_to_f32(b[i < K ? i : i - K]);
        }
    }

    // ---- fragment reads --------------------------------------------------
    auto wrow_addr = [&](int j, int nch) {         // weight fragment of channel nch, step j
        return smem + S::STG0 + (j % S::NST) * S::STAGE + nch * 32 + ((kh ^ ((nch >> 3) & 1)) << 4);
    };
    auto rd1 = [&](int j, bf16x8_t (&a)[4], bf16x8_t (&b)[3]) {
        const int k0 = j * 16;
        const int tap = k0 / C1, c0 = k0 - tap * C1;
        const int q = (c0 >> 3) + kh;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int p = mb * 32 + frow + tap;        // patch row (p = 128, 129 only feed unused rows)
            a[mb] = *reinterpret_cast<const bf16x8_t *>(smem + p * PX + ((q ^ ((p >> 3) & 1)) << 4));
        }
#pragma unroll
        for (int nb3 = 0; nb3 < 3; ++nb3)
            b[nb3] = *reinterpret_cast<const bf16x8_t *>(wrow_addr(j, wave * 96 + nb3 * 32 + frow));
    };
    auto rd2 = [&](int j, bf16x8_t (&a)[2], bf16x8_t (&b)[3]) {
        const int k0 = (j - NC1) * 16;
        const int tap = k0 / K, c0 = k0 - tap * K;
        const int q = (c0 >> 3) + kh;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int r = 2 * (mb * 32 + frow) + tap;  // r = 127, 128 only feed the unused row 63
            a[mb] = *reinterpret_cast<const bf16x8_t *>(smem + r * S::HP + ((q ^ ((r >> 1) & 15)) << 4));
        }
#pragma unroll
        for (int nb3 = 0; nb3 < 3; ++nb3)
            b[nb3] = *reinterpret_cast<const bf16x8_t *>(wrow_addr(j, wave * 96 + nb3 * 32 + frow));
    };

    // Step j: wait until steps j and j+1 have landed (after the barrier,
    // step j+1's fragments are read while step j is multiplied), then refill
    // the stage of step j-1 (read by every wave before this barrier) with
    // step j+4.  Loads land in issue order, so waiting until at most the
    // loads of steps j+2, j+3 are outstanding suffices.
    auto step_wait = [&](int j) {
        const int later = NC - 2 - j;
        if (later >= 2) wait_vmcnt<6>();
        else if (later == 1) wait_vmcnt<3>();
        else wait_vmcnt<0>();
    };

    // ---- phase 1: conv1 into h ------------------------------------------
    f32x16_t acc1[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc1[i][j][e] = 0.f;
    auto step1 = [&](int j, const bf16x8_t (&a)[4], const bf16x8_t (&b)[3], bf16x8_t (&an)[4],
                     bf16x8_t (&bn)[3]) {
        if (j > 0) {
            step_wait(j);
            __syncthreads();
        }
        if (j + S::NST - 1 < NC) fire_step(j + S::NST - 1);
        if (j + 1 < NC1) rd1(j + 1, an, bn);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb3 = 0; nb3 < 3; ++nb3)
                acc1[mb][nb3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[nb3], a[mb], acc1[mb][nb3], 0, 0, 0);
    };
    {
        bf16x8_t a0[4], b0[3], a1[4], b1[3];
        wait_vmcnt<0>();          // input patch and steps 0..3
        __syncthreads();
        rd1(0, a0, b0);
        for (int j = 0; j < NC1; j += 2) {      // two steps per trip: fixed register roles
            step1(j, a0, b0, a1, b1);
            if (j + 1 < NC1) step1(j + 1, a1, b1, a0, b0);
        }
    }
    __syncthreads();              // every wave is done with the input patch

    // h rows: bias, activation, bf16; zeros outside the sequence (conv2's padding)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int r = mb * 32 + frow;
        const bool keep = r < S::HR;
        const bool inside = (unsigned)(hp0 + r) < (unsigned)cp.L;
#pragma unroll
        for (int nb3 = 0; nb3 < 3; ++nb3)
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) {
                const int ch = wave * 96 + nb3 * 32 + hh * 8 + kh * 4;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float t = acc1[mb][nb3][hh * 4 + e];
                    if constexpr (BIAS) t += bias_lds[ch + e];
                    if constexpr (GELU) t = gelu_erf_bf16out(t);
                    v[e] = inside ? t : 0.f;
                }
                uint2 pk;
                pk.x = f32x2_to_bf16x2(v[0], v[1]);
                pk.y = f32x2_to_bf16x2(v[2], v[3]);
                if (keep)
                    *reinterpret_cast<uint2 *>(smem + r * S::HP + (((ch >> 3) ^ ((r >> 1) & 15)) << 4) +
                                               (ch & 7) * 2) = pk;
            }
    }

    // ---- phase 2: conv2 from h -------------------------------------------
    f32x16_t acc2[2][3];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc2[i][j][e] = 0.f;

    auto step2 = [&](int j, const bf16x8_t (&a)[2], const bf16x8_t (&b)[3], bf16x8_t (&an)[2],
                     bf16x8_t (&bn)[3]) {
        if (j > NC1) {
            step_wait(j);
            __syncthreads();
        }
        if (j + S::NST - 1 < NC) fire_step(j + S::NST - 1);
        if (j + 1 < NC) rd2(j + 1, an, bn);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb3 = 0; nb3 < 3; ++nb3)
                acc2[mb][nb3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[nb3], a[mb], acc2[mb][nb3], 0, 0, 0);
    };
    {
        bf16x8_t a0[2], b0[3], a1[2], b1[3];
        step_wait(NC1);           // steps NC1 and NC1+1 landed
        __syncthreads();          // ... and h is complete
        rd2(NC1, a0, b0);
        for (int j = NC1; j < NC; j += 2) {
            step2(j, a0, b0, a1, b1);
            if (j + 1 < NC) step2(j + 1, a1, b1, a0, b0);
        }
    }
    __syncthreads();              // every wave is done with h

    // ---- epilogue: bias, activation, bf16, staged in LDS, 16-byte stores --
    unsigned char *Ys = smem;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int o = mb * 32 + frow;
#pragma unroll
        for (int nb3 = 0; nb3 < 3; ++nb3)
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) {
                const int ch = wave * 96 + nb3 * 32 + hh * 8 + kh * 4;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float t = acc2[mb][nb3][hh * 4 + e];
                    if constexpr (BIAS) t += bias_lds[K + ch + e];
                    if constexpr (GELU) t = gelu_erf_bf16out(t);
                    v[e] = t;
                }
                uint2 pk;
                pk.x = f32x2_to_bf16x2(v[0], v[1]);
                pk.y = f32x2_to_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2 *>(Ys + o * S::YP + ch * 2) = pk;
            }
    }
    __syncthreads();
    uint16_t *yg = reinterpret_cast<uint16_t *>(cp.y);
    constexpr int VPR = K / 8;    // 16-byte vectors per output row
    for (int idx = tid; idx < S::TO * VPR; idx += 256) {
        const int row = idx / VPR, v = idx - row * VPR;
        const int o = o0 + row;
        if (o >= cp.Lo) continue;
        store_nt16(yg + ((size_t)n * cp.Lo + o) * K + v * 8, *reinterpret_cast<const uint4 *>(Ys + row * S::YP + v * 16));
    }
}

}  // namespace convfwd
