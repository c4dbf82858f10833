// Fused two-conv 1-D frontend, weights prepacked into MFMA fragment order.
//
// Same computation as chain_kernel.h -- y = act(conv2(h) + b2) with
// h = round_bf16(act(conv1(x) + b1)), conv1 k3 s1 p1 (C1 -> 384 channels),
// conv2 k3 s2 p1 (384 -> 384), the frontend of the ExecuTorch conv1d issue
// (its table that splits the frontend into conv1 + GELU + conv2 + GELU) --
// with a different division of labour inside the workgroup:
//
//  * The weights are read straight from L2 into registers.  Each of the
//    four waves owns 96 output channels in both convs, so no two waves need
//    the same weight fragment, and the K loops have no barrier at all: the
//    only shared operand (the input patch in conv1, h in conv2) is written
//    once per phase.
//  * A strided fragment load (32 weight rows x 32 bytes per instruction) ran
//    at ~16 B/clk per CU from L2 on MI355X, a contiguous 1 KB per
//    instruction at ~50.  So the weights are first rearranged
//    (chain_pack_kernel) so that every fragment is one contiguous KB:
//    packed[wave][s][j][lane] = the 16 bytes lane `lane` feeds to the
//    32x32x16 MFMA for reduction step s (16 elements) and channel block
//    cb = 3 wave + j (32 channels), i.e.
//    w[32 cb + (lane & 31)][16 s + 8 (lane >> 5) .. + 8]; conv1's 3*C1/16
//    steps (rounded up to whole groups of 8 with zeros) first, then conv2's
//    72.  Each wave's stream is then one contiguous
//    run of 3 KB per step.  Weights are constant
//    across calls, so this runs once, as the ExecuTorch conv2d path
//    prepacks its weights.
//  * A workgroup owns TO = 95 consecutive conv2 outputs of one sequence:
//    conv1 runs on 192 rows (the 191 positions of h those outputs read, plus
//    one), conv2 on 96 rows (one unused).  Conv1's weights are streamed
//    once per half.  With 1500 outputs per sequence
//    that is 16 tiles, so the batch-32 frontend is 512 workgroups, two per
//    CU, and the 1.07 MB of weights are streamed 512 times (a 63-output tile
//    streamed them 768 times).
//
// LDS (bytes): the biases as fp32 at 0, h (193 rows x 768) at 3072, the
// input patch (194 positions x C1 <= 224) at 76800, over h rows 96 and up,
// so conv1's first 96 rows of h are written while the patch is still in use
// for the second 96; the output staging aliases h at the end.  Conv1 runs
// in two halves of 96 rows: the accumulators of all 192 rows beside the
// weight ring spilled to scratch.  Swizzles as chain_kernel.h (each
// measured conflict-free):
//  * input patch, 2*C1-byte rows: chunk q of position p at slot q ^ ((p >> 3) & 1);
//  * h, 768-byte rows: chunk q of row r at slot q ^ ((r >> 1) & 15).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "igemm_dma.h"

namespace convfwd {

struct ChainPackedParams {
    const void *x, *packed, *b1, *b2;    // b1 and b2 NULL without bias
    void *y;
    int N, L, C1, Lo;                    // batch, input length, conv1 input channels, output length
    int tiles;                           // output tiles per sequence
    uint32_t x_bytes;
};

struct ChainPackedShape {
    static constexpr int K = 384;                 // conv1 out = conv2 in = conv2 out channels
    static constexpr int TO = 95;                 // conv2 outputs per workgroup
    static constexpr int MB1 = 6;                 // conv1 row blocks of 32 (192 rows)
    static constexpr int MBH = MB1 / 2;           // conv1 row blocks per half
    static constexpr int MB2 = 3;                 // conv2 row blocks of 32 (96 rows)
    static constexpr int HROWS = 2 * 32 * MB2 + 1;  // 193: rows conv2's 96 rows read
    static constexpr int HP = 2 * K;              // bytes per h row
    static constexpr int H_BYTES = HROWS * HP;    // 148224
    static constexpr int XP = 32 * MB1 + 2;       // 194 patch positions: conv1's 192 rows, 3 taps
    static constexpr int BIAS0 = 0;               // fp32 biases, conv1's then conv2's
    static constexpr int H0 = 2 * K * 4;          // h rows
    static constexpr int PATCH0 = H0 + 32 * MBH * HP;   // input patch: above h rows 0..95
    static constexpr int LDS_BYTES = 160 * 1024;
    static constexpr int YP = HP + 16;            // output staging row pitch
    static constexpr int FRAG = 1024;             // one packed fragment
    static constexpr int STEP = (K / 32) * FRAG;  // packed bytes per reduction step (all waves)
    static constexpr int WSTEP = 3 * FRAG;        // one wave's bytes per step
    static constexpr int S2 = 3 * K / 16;         // conv2 reduction steps
    static constexpr int D1 = 8;                  // conv1 steps of weights in flight
    static constexpr int D2 = 12;                 // conv2 steps of weights in flight (registers allow more here)
    static constexpr int C1MAX = 224;             // patch (rounded up to 1 KB loads) below the LDS end
    static_assert(2 * TO + 1 <= 2 * 32 * MB2 - 1 && TO < 32 * MB2, "conv2 rows cover the tile");
    static_assert(H0 + H_BYTES <= LDS_BYTES && TO * YP <= H_BYTES, "h and the output staging");
    static_assert(PATCH0 + (XP * C1MAX / 8 + 63) / 64 * 1024 <= LDS_BYTES, "input patch");
    static_assert(S2 % D2 == 0 && (K / 16) % D2 == 0, "whole groups of steps; a conv2 tap never changes inside one");
    static_assert(D1 <= D2 && 3 * D2 < 64, "ring slots; the vmcnt range");
    // conv1's reduction steps padded to whole groups (the padding is zero weights)
    static __host__ __device__ constexpr int s1p(int C1) { return (3 * C1 / 16 + D1 - 1) / D1 * D1; }
    // packed steps per wave: conv1's (padded), then conv2's
    static __host__ __device__ constexpr int steps(int C1) { return s1p(C1) + S2; }
};

// packed[wave][s][j][lane] (16 bytes each) from the natural GKZYXC weights:
// the fragment of channel block cb = 3 wave + j for step s
__global__ void __launch_bounds__(256) chain_pack_kernel(const uint4 *__restrict__ w1, const uint4 *__restrict__ w2,
                                                         uint4 *__restrict__ packed, int C1, int total)
{
    using S = ChainPackedShape;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int lane = i & 63;
    const int f = i >> 6;                       // fragment index
    const int j = f % 3;
    const int s = (f / 3) % S::steps(C1);
    const int cb = 3 * (f / (3 * S::steps(C1))) + j;
    const int S1 = 3 * C1 / 16, S1p = S::s1p(C1);
    const int row = cb * 32 + (lane & 31);
    const int half = lane >> 5;
    uint4 v = {0, 0, 0, 0};
    if (s < S1)
        v = w1[(size_t)row * (3 * C1 / 8) + 2 * s + half];
    else if (s >= S1p && s < S1p + S::S2)
        v = w2[(size_t)row * (3 * S::K / 8) + 2 * (s - S1p) + half];
    packed[i] = v;
}

template <bool BIAS, bool GELU>
__global__ void __launch_bounds__(256, 1) chain_packed_kernel(ChainPackedParams cp)
{
    using S = ChainPackedShape;
    constexpr int K = S::K;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[S::LDS_BYTES];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)smem;
    unsigned char *const hs = smem + S::H0;        // h rows
    const unsigned char *const xs = smem + S::PATCH0;   // input patch

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int frow = lane & 31;           // row of an operand block
    const int kh = lane >> 5;             // which 8 of a step's 16 reduction elements

    const int n = blockIdx.x / cp.tiles;
    const int o0 = (blockIdx.x - n * cp.tiles) * S::TO;
    const int hp0 = 2 * o0 - 1;           // sequence position of h row 0
    const int xp0 = hp0 - 1;              // sequence position of patch row 0
    const int C1 = cp.C1;
    const int PX = 2 * C1;                // bytes per patch row
    const int S1p = S::s1p(C1);           // conv1 reduction steps, padded to whole groups

    // Biases (both convs, 2K values, three per thread) are fetched first:
    // loads complete in issue order, so the wait for the input patch below
    // then covers them too, and the weight ring's loads issued after the
    // patch stay in flight across that wait.
    constexpr int BPT = (2 * K + 255) / 256;      // bias values per thread
    uint16_t braw[BPT];
    if constexpr (BIAS) {
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int i = tid + 256 * u;
            const uint16_t *b = reinterpret_cast<const uint16_t *>(i < K ? cp.b1 : cp.b2);
            braw[u] = i < 2 * K ? b[i < K ? i : (i < 2 * K ? i - K : 0)] : 0;
        }
    }

    // ---- input patch: XP positions x C1 channels, zeros outside the sequence
    {
        const i32x4_t xr = buffer_rsrc(cp.x, cp.x_bytes);
        const int cpx = C1 / 8;
        const int nchunks = S::XP * cpx;
        for (int t = 0; 64 * (wave + 4 * t) < nchunks; ++t) {
            const int ci = lane + 64 * (wave + 4 * t);   // lands at byte 16 * ci
            const int p = ci / cpx, q = ci - p * cpx;
            const int xp = xp0 + p;
            const int qg = q ^ ((p >> 3) & 1);
            const bool ok = ci < nchunks && (unsigned)xp < (unsigned)cp.L;
            const uint32_t off = ok ? (uint32_t)(((n * cp.L + xp) * C1 + qg * 8) * 2) : kOutOfRange;
            dma16(xr, off, 0, lds0 + S::PATCH0 + (wave + 4 * t) * 1024);
        }
    }

    // ---- the weight stream ---------------------------------------------------
    // Stream step t: conv1's step t for t < S1p (first half), again t - S1p
    // for t < 2 S1p (second half), then conv2's steps.  Conv1 keeps D1 steps
    // in flight, conv2 D2; slot t mod D1 (conv1) or (t - 2 S1p) mod D2
    // (conv2) holds step t, every phase being a whole number of groups.
    // This wave's stream (its three channel blocks) is contiguous: 3 KB per step.
    const unsigned char *const P = reinterpret_cast<const unsigned char *>(cp.packed) +
                                   (size_t)wave * S::steps(C1) * S::WSTEP;
    const uint32_t lane_off = (uint32_t)(lane * 16);
    bf16x8_t wb[S::D2][3];
    auto ldw = [&](int t, int slot, int j) {
        const unsigned char *b = P + (size_t)(t < S1p ? t : t - S1p) * S::WSTEP;
        wb[slot][j] = *reinterpret_cast<const bf16x8_t *>(b + lane_off + j * S::FRAG);
    };
#pragma unroll
    for (int d = 0; d < S::D1; ++d)
#pragma unroll
        for (int j = 0; j < 3; ++j) ldw(d, d, j);

    float *bias_lds = reinterpret_cast<float *>(smem + S::BIAS0);
    wait_vmcnt<3 * S::D1>();      // the biases and the patch (loads complete in issue order)
    if constexpr (BIAS) {
#pragma unroll
        for (int u = 0; u < BPT; ++u) {
            const int i = tid + 256 * u;
            if (i < 2 * K) bias_lds[i] = bf16_to_f32(braw[u]);
        }
    }
    __syncthreads();              // input patch and biases in LDS

    // One reduction step: nine products, weight fragment j major, and one
    // wave per SIMD, so the other work of the step is spread between them
    // (issued while a product runs): after product (mb, j = 0) the next
    // step's operand rows mb are read, and after a fragment's third product
    // its slot is refilled D steps ahead.
    auto step = [&](f32x16_t (&acc)[3][3], int slot, const bf16x8_t (&a)[3], auto &&read_next, auto &&refill) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int mb = 0; mb < 3; ++mb) {
                acc[mb][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb[slot][j], a[mb], acc[mb][j], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (j == 0) read_next(mb);
                if (mb == 2) refill(j);
                __builtin_amdgcn_sched_barrier(0);
            }
    };

    // ---- phase 1: conv1, 192 rows in two halves of 96 ------------------------
    // (the accumulators of all 192 rows beside the weight ring spilled to
    // scratch; half 0's h rows lie below the patch, so they are written at once)
    auto conv1_half = [&](int half) {
        f32x16_t acc[S::MBH][3];
#pragma unroll
        for (int i = 0; i < S::MBH; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
        // reduction element 16 s + 8 kh = tap * C1 + c, stepped incrementally;
        // the padding steps (and the read one step past the end) use tap <= 2
        // rows with zero weights
        int tap = 0, c = 8 * kh;
        const unsigned char *xrow = xs + (half * 32 * S::MBH + frow) * PX;
        auto rd1 = [&](bf16x8_t (&a)[S::MBH], int mb) {
            const int tp = tap < 2 ? tap : 2;
            const int p = half * 32 * S::MBH + mb * 32 + frow + tp;
            a[mb] = *reinterpret_cast<const bf16x8_t *>(xrow + (mb * 32 + tp) * PX + (((c >> 3) ^ ((p >> 3) & 1)) << 4));
            if (mb == S::MBH - 1) {
                c += 16;
                if (c >= C1) { c -= C1; ++tap; }
            }
        };
        bf16x8_t a[2][S::MBH];
#pragma unroll
        for (int mb = 0; mb < S::MBH; ++mb) rd1(a[0], mb);
        const int t0 = half * S1p;
        for (int g = 0; g < S1p; g += S::D1) {
#pragma unroll
            for (int d = 0; d < S::D1; ++d)
                step(acc, d, a[d & 1], [&](int mb) { rd1(a[(d + 1) & 1], mb); },
                     // the last group of a half fetches the next phase's first steps
                     [&](int j) { ldw(t0 + g + d + S::D1, d, j); });
        }
        if (half == 1) __syncthreads();   // every wave is done with the input patch
        // h = bf16(act(acc + b1)), zeros outside the sequence (conv2's padding).
        // Channel runs outermost, so each run's four biases are read once for
        // all row blocks; the next run's are read before this run's h stores
        // (which the compiler cannot tell apart from the bias words, so a read
        // placed after them would wait for its whole latency).
        f32x4_t bnext = BIAS ? *reinterpret_cast<const f32x4_t *>(bias_lds + wave * 96 + kh * 4)
                             : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) {
                const int ch = wave * 96 + j * 32 + hh * 8 + kh * 4;
                const f32x4_t bcur = bnext;
                if (BIAS && j * 4 + hh < 11)
                    bnext = *reinterpret_cast<const f32x4_t *>(bias_lds + ch + 8);
#pragma unroll
                for (int mb = 0; mb < S::MBH; ++mb) {
                    const int r = half * 32 * S::MBH + mb * 32 + frow;
                    const bool inside = (unsigned)(hp0 + r) < (unsigned)cp.L;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float t = acc[mb][j][hh * 4 + e];
                        if constexpr (BIAS) t += bcur[e];
                        if constexpr (GELU) t = gelu_erf_bf16out(t);
                        v[e] = inside ? t : 0.f;
                    }
                    uint2 pk;
                    pk.x = f32x2_to_bf16x2(v[0], v[1]);
                    pk.y = f32x2_to_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2 *>(hs + r * S::HP + (((ch >> 3) ^ ((r >> 1) & 15)) << 4) + (ch & 7) * 2) = pk;
                }
            }
    };
    conv1_half(0);
    conv1_half(1);
    // conv2's steps D1 .. D2-1 (steps 0 .. D1-1 were fetched by conv1's last group)
#pragma unroll
    for (int d = S::D1; d < S::D2; ++d)
#pragma unroll
        for (int j = 0; j < 3; ++j) ldw(2 * S1p + d, d, j);
    // row 192 is read only by conv2's unused row 95; keep it finite
    if (tid < S::HP / 16) *reinterpret_cast<uint4 *>(hs + 192 * S::HP + tid * 16) = uint4{0, 0, 0, 0};
    __syncthreads();              // h complete

    // ---- phase 2: conv2 from h -------------------------------------------------
    f32x16_t acc2[S::MB2][3];
#pragma unroll
    for (int i = 0; i < S::MB2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc2[i][j][e] = 0.f;
    {
        // step s = g + d: reduction element 16 s + 8 kh = tap * 384 + c; a
        // group of D2 steps never changes tap (the read one step past the end
        // uses tap 2)
        auto rd2 = [&](int s, bf16x8_t (&a)[S::MB2], int mb) {
            int tap = s / (K / 16);
            const int q = 2 * (s - tap * (K / 16)) + kh;
            tap = tap < 2 ? tap : 2;
            const int r = 2 * (mb * 32 + frow) + tap;
            a[mb] = *reinterpret_cast<const bf16x8_t *>(hs + r * S::HP + ((q ^ ((r >> 1) & 15)) << 4));
        };
        bf16x8_t a[2][S::MB2];
#pragma unroll
        for (int mb = 0; mb < S::MB2; ++mb) rd2(0, a[0], mb);
        const int t0 = 2 * S1p;
        for (int g = 0; g < S::S2; g += S::D2) {
#pragma unroll
            for (int d = 0; d < S::D2; ++d)
                step(acc2, d, a[d & 1], [&](int mb) { rd2(g + d + 1, a[(d + 1) & 1], mb); },
                     [&](int j) {
                         if (g + S::D2 < S::S2) ldw(t0 + g + d + S::D2, d, j);
                     });
        }
    }
    __syncthreads();              // every wave is done with h

    // ---- epilogue: bias, activation, bf16, staged in LDS, 16-byte stores ----
    // (channel runs outermost, biases read one run ahead, as for h)
    unsigned char *Ys = hs;
    f32x4_t bnext = BIAS ? *reinterpret_cast<const f32x4_t *>(bias_lds + K + wave * 96 + kh * 4)
                         : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
            const int ch = wave * 96 + j * 32 + hh * 8 + kh * 4;
            const f32x4_t bcur = bnext;
            if (BIAS && j * 4 + hh < 11) bnext = *reinterpret_cast<const f32x4_t *>(bias_lds + K + ch + 8);
#pragma unroll
            for (int mb = 0; mb < S::MB2; ++mb) {
                const int o = mb * 32 + frow;
                if (o < S::TO) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float t = acc2[mb][j][hh * 4 + e];
                        if constexpr (BIAS) t += bcur[e];
                        if constexpr (GELU) t = gelu_erf_bf16out(t);
                        v[e] = t;
                    }
                    uint2 pk;
                    pk.x = f32x2_to_bf16x2(v[0], v[1]);
                    pk.y = f32x2_to_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2 *>(Ys + o * S::YP + ch * 2) = pk;
                }
            }
        }
    __syncthreads();
    uint16_t *yg = reinterpret_cast<uint16_t *>(cp.y);
    constexpr int VPR = K / 8;    // 16-byte vectors per output row
    const int rows = cp.Lo - o0 < S::TO ? cp.Lo - o0 : S::TO;
    for (int idx = tid; idx < rows * VPR; idx += 256) {
        const int row = idx / VPR, v = idx - row * VPR;
        store_nt16(yg + ((size_t)n * cp.Lo + o0 + row) * K + v * 8,
                   *reinterpret_cast<const uint4 *>(Ys + row * S::YP + v * 16));
    }
}

}  // namespace convfwd
