// Host side of the C ABI declared in include/convfwd.h: descriptor
// validation and canonicalisation to a 3-D problem, output extents, the
// per-shape tile-configuration selector and the launcher.
//
// Canonicalisation follows the ExecuTorch conv1d issue ("Suggested fix": a
// conv1d is a conv2d with a singleton height) one step further: every
// problem becomes a 3-D one with unit leading dims, so one kernel template
// serves 1-D, 2-D and 3-D.  The selector is the analytic counterpart of the
// per-problem kernel choice in the Composable Kernel grouped-conv note
// (section 1: choosing among tile/pipeline variants per dim tuple), and like
// the onnxruntime subgroup-matrix MatMul change it prefers big tiles for big
// problems and smaller ones where big tiles would leave compute units idle.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "../../include/convfwd.h"
#include "igemm_kernel.h"
#include "igemm_dma.h"
#include "patch_kernel.h"
#include "patch_fixed.h"
#include "chain_kernel.h"
#include "chain_packed.h"
#include "bwd_kernels.h"
#include "weight_pack.h"

namespace convfwd {
namespace {

thread_local char g_err[512] = "";

conv_status_t fail(conv_status_t st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

typedef void (*launch_fn)(const KParams &, uint32_t x_bytes, uint32_t w_bytes, int grid, hipStream_t,
                          hipEvent_t start, hipEvent_t stop);

// hipExtLaunchKernelGGL records the optional events when the kernel itself
// starts and ends.
template <int DT, int BM, int BN, int BK, int WM, int WN, int VEC>
void launch_reg(const KParams &kp, uint32_t, uint32_t, int grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1)
{
    hipExtLaunchKernelGGL((igemm_fwd_kernel<DT, BM, BN, BK, WM, WN, VEC>), dim3(grid),
                          dim3(WM * WN * 64), 0, s, e0, e1, 0, kp);
}

// The epilogue (bias, GELU) is compiled into each kernel variant, so a
// variant carries only the code it runs.
template <int DT, int BM, int BN, int WM, int WN, int NS, int MF, int KSUB, int KG, int FL>
void launch_dma(const KParams &kp, uint32_t xb, uint32_t wb, int grid, hipStream_t s, hipEvent_t e0,
                hipEvent_t e1)
{
    DmaParams dp;
    dp.k = kp;
    dp.x_bytes = xb;
    dp.w_bytes = wb;
    const dim3 g(grid), b(WM * WN * 64 * KG);
    const bool bias = kp.bias != nullptr;
    if (bias && kp.gelu)
        hipExtLaunchKernelGGL((igemm_dma_kernel<DT, BM, BN, WM, WN, NS, MF, KSUB, KG, FL, true, true>), g, b, 0, s, e0, e1, 0, dp);
    else if (bias)
        hipExtLaunchKernelGGL((igemm_dma_kernel<DT, BM, BN, WM, WN, NS, MF, KSUB, KG, FL, true, false>), g, b, 0, s, e0, e1, 0, dp);
    else if (kp.gelu)
        hipExtLaunchKernelGGL((igemm_dma_kernel<DT, BM, BN, WM, WN, NS, MF, KSUB, KG, FL, false, true>), g, b, 0, s, e0, e1, 0, dp);
    else
        hipExtLaunchKernelGGL((igemm_dma_kernel<DT, BM, BN, WM, WN, NS, MF, KSUB, KG, FL, false, false>), g, b, 0, s, e0, e1, 0, dp);
}

FastDiv make_fastdiv(int d);

template <int TH, int TW, int BN, int CC, int NS, int PHMAX, int PWMAX, int TAPMAX, int PAD>
void launch_patch(const KParams &kp, uint32_t xb, uint32_t wb, int grid, hipStream_t s, hipEvent_t e0,
                  hipEvent_t e1)
{
    PatchParams pp;
    pp.k = kp;
    pp.x_bytes = xb;
    pp.w_bytes = wb;
    pp.tiles_h = (kp.Ho + TH - 1) / TH;
    pp.tiles_w = (kp.Wo + TW - 1) / TW;
    pp.ph = (TH - 1) * kp.sh + (kp.Y - 1) * kp.dh + 1;
    pp.pw = (TW - 1) * kp.sw + (kp.X - 1) * kp.dw + 1;
    pp.fd_pw = make_fastdiv(pp.pw);
    pp.fd_taps = make_fastdiv(kp.Y * kp.X);
    pp.fd_tw = make_fastdiv(pp.tiles_w);
    pp.fd_th = make_fastdiv(pp.tiles_h);
    pp.fd_N = make_fastdiv(kp.N);
    const dim3 g(grid), b(256);
    const bool bias = kp.bias != nullptr;
    if (bias && kp.gelu)
        hipExtLaunchKernelGGL((patch_conv_kernel<TH, TW, BN, CC, NS, PHMAX, PWMAX, TAPMAX, PAD, true, true>), g, b, 0, s, e0, e1, 0, pp);
    else if (bias)
        hipExtLaunchKernelGGL((patch_conv_kernel<TH, TW, BN, CC, NS, PHMAX, PWMAX, TAPMAX, PAD, true, false>), g, b, 0, s, e0, e1, 0, pp);
    else if (kp.gelu)
        hipExtLaunchKernelGGL((patch_conv_kernel<TH, TW, BN, CC, NS, PHMAX, PWMAX, TAPMAX, PAD, false, true>), g, b, 0, s, e0, e1, 0, pp);
    else
        hipExtLaunchKernelGGL((patch_conv_kernel<TH, TW, BN, CC, NS, PHMAX, PWMAX, TAPMAX, PAD, false, false>), g, b, 0, s, e0, e1, 0, pp);
}

template <int TH, int TW, int BN, int CC, int NS, int FY, int FX, int DH, int DW, int NW, int PM, int RA, int RR>
void launch_patchf(const KParams &kp, uint32_t xb, uint32_t wb, int grid, hipStream_t s, hipEvent_t e0,
                   hipEvent_t e1)
{
    PatchFixedParams pp;
    pp.k = kp;
    pp.x_bytes = xb;
    pp.w_bytes = wb;
    pp.tiles_h = (kp.Ho + TH - 1) / TH;
    pp.tiles_w = (kp.Wo + TW - 1) / TW;
    pp.fd_tw = make_fastdiv(pp.tiles_w);
    pp.fd_th = make_fastdiv(pp.tiles_h);
    pp.fd_N = make_fastdiv(kp.N);
    pp.fd_G = make_fastdiv(kp.G);
    pp.group_fast = kp.C * 2 < 128 ? 1 : 0;
    const dim3 g(grid), b(NW * 64);
    const bool bias = kp.bias != nullptr;
    if (bias && kp.gelu)
        hipExtLaunchKernelGGL((patch_fixed_kernel<TH, TW, BN, CC, NS, FY, FX, DH, DW, NW, PM, RA, RR, true, true>), g, b, 0, s, e0, e1, 0, pp);
    else if (bias)
        hipExtLaunchKernelGGL((patch_fixed_kernel<TH, TW, BN, CC, NS, FY, FX, DH, DW, NW, PM, RA, RR, true, false>), g, b, 0, s, e0, e1, 0, pp);
    else if (kp.gelu)
        hipExtLaunchKernelGGL((patch_fixed_kernel<TH, TW, BN, CC, NS, FY, FX, DH, DW, NW, PM, RA, RR, false, true>), g, b, 0, s, e0, e1, 0, pp);
    else
        hipExtLaunchKernelGGL((patch_fixed_kernel<TH, TW, BN, CC, NS, FY, FX, DH, DW, NW, PM, RA, RR, false, false>), g, b, 0, s, e0, e1, 0, pp);
}

template <int KT, int TT, int NWV>
void launch_wgrad(const WgradParams &wp, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((wgrad_kernel<KT, KT, TT, NWV>), dim3(grid), dim3(NWV * 64), 0, s, wp);
}

// Workgroups of one backward-weight instantiation that a compute unit holds
// at once (its registers and LDS decide); 1 when the runtime cannot tell.
template <int KT, int TT, int NWV>
int wgrad_occupancy()
{
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, wgrad_kernel<KT, KT, TT, NWV>, NWV * 64, 0) !=
        hipSuccess) {
        (void)hipGetLastError();
        return 1;
    }
    return blocks > 0 ? blocks : 1;
}

enum { KIND_REG = 0, KIND_DMA = 1, KIND_PATCH = 2, KIND_PATCHF = 3 };

struct TileCfg {
    int dtype;          // conv_dtype_t
    int kind;           // KIND_REG: register-staged implicit GEMM, KIND_DMA: direct-to-LDS
                        // implicit GEMM, KIND_PATCH: input patch in LDS
    int BM, BN, BK, WM, WN, VEC, NS;
    int lds_bytes;
    launch_fn fn;
    const char *name;
    int TH, TW, CC, PHMAX, PWMAX, TAPMAX;   // KIND_PATCH (TH, TW, CC also KIND_PATCHF)
    int KG;             // KIND_DMA: reduction groups per workgroup (0 means 1)
    int FY, FX, DH, DW; // KIND_PATCHF: the filter's H/W taps and dilation it is compiled for
    int wimg;           // KIND_PATCHF: bytes of one K-step's prepacked weight image
    int MF;             // KIND_DMA: MFMA block edge (16 or 32)
};

#define CFG(DT, BM, BN, BK, WM, WN, VEC)                                                 \
    TileCfg{DT, KIND_REG, BM, BN, BK, WM, WN, VEC, 2,                                    \
            IgemmShape<DT, BM, BN, BK, WM, WN, VEC>::LDS_BYTES,                          \
            &launch_reg<DT, BM, BN, BK, WM, WN, VEC>,                                    \
            (DT ? "bf16_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_v" #VEC                 \
                : "f32_" #BM "x" #BN "x" #BK "_w" #WM "x" #WN "_v" #VEC),                \
            0, 0, 0, 0, 0, 0}

#define DMA(DT, BM, BN, WM, WN, NS, MF, KSUB)                                            \
    TileCfg{DT, KIND_DMA, BM, BN, KSUB * 128 / (DT ? 2 : 4), WM, WN, 16 / (DT ? 2 : 4), NS, \
            DmaShape<DT, BM, BN, WM, WN, NS, MF, KSUB, 1>::LDS_BYTES,                     \
            &launch_dma<DT, BM, BN, WM, WN, NS, MF, KSUB, 1, 0>,                            \
            (DT ? "bf16_dma_" #BM "x" #BN "_w" #WM "x" #WN "_s" #NS "_m" #MF "_k" #KSUB  \
                : "f32_dma_" #BM "x" #BN "_w" #WM "x" #WN "_s" #NS "_m" #MF "_k" #KSUB), \
            0, 0, 0, 0, 0, 0, 1, 0, 0, 0, 0, 0, MF}

// Loads of the next stage issued during the first 1/FL of the products
#define DMAF(DT, BM, BN, WM, WN, NS, MF, KSUB, FL)                                       \
    TileCfg{DT, KIND_DMA, BM, BN, KSUB * 128 / (DT ? 2 : 4), WM, WN, 16 / (DT ? 2 : 4), NS, \
            DmaShape<DT, BM, BN, WM, WN, NS, MF, KSUB, 1>::LDS_BYTES,                     \
            &launch_dma<DT, BM, BN, WM, WN, NS, MF, KSUB, 1, FL>,                        \
            (DT ? "bf16_dma_" #BM "x" #BN "_w" #WM "x" #WN "_s" #NS "_m" #MF "_k" #KSUB "_f" #FL \
                : "f32_dma_" #BM "x" #BN "_w" #WM "x" #WN "_s" #NS "_m" #MF "_k" #KSUB "_f" #FL), \
            0, 0, 0, 0, 0, 0, 1, 0, 0, 0, 0, 0, MF}

// Two reduction groups per workgroup (twice the waves, half the K-steps each)
#define DMA2(DT, BM, BN, WM, WN, NS, MF, KSUB)                                           \
    TileCfg{DT, KIND_DMA, BM, BN, KSUB * 128 / (DT ? 2 : 4), WM, WN, 16 / (DT ? 2 : 4), NS, \
            DmaShape<DT, BM, BN, WM, WN, NS, MF, KSUB, 2>::LDS_BYTES,                     \
            &launch_dma<DT, BM, BN, WM, WN, NS, MF, KSUB, 2, 0>,                            \
            (DT ? "bf16_dma_" #BM "x" #BN "_w" #WM "x" #WN "_s" #NS "_m" #MF "_k" #KSUB "_g2" \
                : "f32_dma_" #BM "x" #BN "_w" #WM "x" #WN "_s" #NS "_m" #MF "_k" #KSUB "_g2"), \
            0, 0, 0, 0, 0, 0, 2, 0, 0, 0, 0, 0, MF}

// Four one-wave reduction groups per workgroup (a quarter of the K-steps each)
#define DMA4(DT, BM, BN, NS, MF, KSUB)                                                   \
    TileCfg{DT, KIND_DMA, BM, BN, KSUB * 128 / (DT ? 2 : 4), 1, 1, 16 / (DT ? 2 : 4), NS,  \
            DmaShape<DT, BM, BN, 1, 1, NS, MF, KSUB, 4>::LDS_BYTES,                       \
            &launch_dma<DT, BM, BN, 1, 1, NS, MF, KSUB, 4, 0>,                           \
            (DT ? "bf16_dma_" #BM "x" #BN "_w1x1_s" #NS "_m" #MF "_k" #KSUB "_g4"        \
                : "f32_dma_" #BM "x" #BN "_w1x1_s" #NS "_m" #MF "_k" #KSUB "_g4"),       \
            0, 0, 0, 0, 0, 0, 4, 0, 0, 0, 0, 0, MF}

#define DMA4F(DT, BM, BN, NS, MF, KSUB, FL)                                              \
    TileCfg{DT, KIND_DMA, BM, BN, KSUB * 128 / (DT ? 2 : 4), 1, 1, 16 / (DT ? 2 : 4), NS,  \
            DmaShape<DT, BM, BN, 1, 1, NS, MF, KSUB, 4>::LDS_BYTES,                       \
            &launch_dma<DT, BM, BN, 1, 1, NS, MF, KSUB, 4, FL>,                          \
            (DT ? "bf16_dma_" #BM "x" #BN "_w1x1_s" #NS "_m" #MF "_k" #KSUB "_g4_f" #FL  \
                : "f32_dma_" #BM "x" #BN "_w1x1_s" #NS "_m" #MF "_k" #KSUB "_g4_f" #FL), \
            0, 0, 0, 0, 0, 0, 4, 0, 0, 0, 0, 0, MF}

// Any wave grid, reduction groups and load spread, with its name spelled out
#define DMAX(DT, BM, BN, WM, WN, NS, MF, KSUB, KG, FL, NAME)                               \
    TileCfg{DT, KIND_DMA, BM, BN, KSUB * 128 / (DT ? 2 : 4), WM, WN, 16 / (DT ? 2 : 4), NS, \
            DmaShape<DT, BM, BN, WM, WN, NS, MF, KSUB, KG>::LDS_BYTES,                    \
            &launch_dma<DT, BM, BN, WM, WN, NS, MF, KSUB, KG, FL>, NAME,                  \
            0, 0, 0, 0, 0, 0, KG, 0, 0, 0, 0, 0, MF}

// Input-patch kernel (bf16): box TH x TW output pixels, BN output channels,
// CC input channels per K-step, patch at most PHMAX x PWMAX, at most TAPMAX
// filter taps per depth tap.
#define PATCH(TH, TW, BN, CC, NS, PHMAX, PWMAX, TAPMAX, PAD)                             \
    TileCfg{1, KIND_PATCH, TH * TW, BN, CC, 4, 1, 8, NS,                                  \
            PatchShape<TH, TW, BN, CC, NS, PHMAX, PWMAX, TAPMAX, PAD>::LDS_BYTES,         \
            &launch_patch<TH, TW, BN, CC, NS, PHMAX, PWMAX, TAPMAX, PAD>,                \
            "bf16_patch_" #TH "x" #TW "x" #BN "_c" #CC "_s" #NS "_p" #PHMAX "x" #PWMAX "_d" #PAD, \
            TH, TW, CC, PHMAX, PWMAX, TAPMAX}

// Input-patch kernel with the filter's H/W shape compiled in (bf16, unit H/W
// stride): box TH x TW (flattened into 32-pixel blocks), BN output channels,
// CC channels per K-step, NS stages, an FY x FX filter with H/W dilation
// DH x DW, NW waves.
#define PFIX(TH, TW, BN, CC, NS, FY, FX, DH, DW, NW, PM, RA, RR)                          \
    TileCfg{1, KIND_PATCHF, TH * TW, BN, CC, NW, 1, 8, NS,                                 \
            PatchFixedShape<TH, TW, BN, CC, NS, FY, FX, DH, DW, NW, PM, RR>::LDS_BYTES,    \
            &launch_patchf<TH, TW, BN, CC, NS, FY, FX, DH, DW, NW, PM, RA, RR>,           \
            "bf16_pfix_" #TH "x" #TW "x" #BN "_c" #CC "_s" #NS "_f" #FY "x" #FX "_d" #DH "x" #DW "_w" #NW \
            "_l" #PM "_r" #RA "_rr" #RR, TH, TW, CC, 0, 0, 0, 1, FY, FX, DH, DW,          \
            PatchFixedShape<TH, TW, BN, CC, NS, FY, FX, DH, DW, NW, PM, RR>::W_BYTES, 32}

// One candidate table, shared by the selector, forced-config creation and
// the sweeps.  VEC = 16 bytes of channels per load; the VEC = 1 entries serve
// channel counts that are not a multiple of the vector.
const TileCfg kCfgs[] = {
    PFIX(28, 32, 32, 16, 2, 3, 3, 2, 2, 4, 1, 1, 1),
    PFIX(16, 32, 32, 16, 2, 3, 3, 2, 2, 4, 0, 1, 1),
    PFIX(16, 28, 32, 16, 2, 3, 3, 2, 2, 2, 1, 1, 0),
    PFIX(14, 32, 32, 16, 2, 3, 3, 2, 2, 2, 0, 1, 1),
    PFIX(14, 32, 32, 16, 2, 3, 3, 2, 2, 7, 0, 1, 1),
    PFIX(14, 32, 32, 16, 2, 3, 3, 2, 2, 14, 0, 1, 1),
    PFIX(28, 32, 32, 16, 2, 3, 3, 2, 2, 7, 1, 1, 1),
    PFIX(28, 32, 32, 16, 2, 3, 3, 2, 2, 14, 1, 1, 1),
    PFIX(28, 28, 32, 16, 2, 3, 3, 2, 2, 13, 1, 1, 0),
    PFIX(8, 56, 64, 16, 2, 3, 3, 1, 1, 4, 1, 1, 0),
    PFIX(16, 32, 32, 16, 2, 3, 3, 1, 1, 4, 0, 1, 1),
    PFIX(8, 32, 64, 16, 2, 3, 3, 1, 1, 4, 1, 1, 0),
    PFIX(4, 56, 64, 16, 2, 3, 3, 1, 1, 4, 1, 1, 0),
    PFIX(4, 56, 64, 16, 2, 3, 3, 1, 1, 2, 1, 1, 0),
    PFIX(4, 56, 64, 16, 2, 3, 3, 1, 1, 7, 0, 1, 0),
    PFIX(8, 56, 64, 16, 2, 3, 3, 1, 1, 7, 1, 1, 0),
    PFIX(8, 56, 64, 16, 2, 3, 3, 1, 1, 14, 1, 1, 0),
    PATCH(8, 32, 64, 16, 2, 10, 34, 9, 1),
    PATCH(4, 32, 64, 16, 2, 6, 34, 9, 1),
    PATCH(8, 32, 32, 16, 2, 12, 36, 9, 1),
    PATCH(8, 16, 64, 16, 2, 10, 18, 9, 1),
    PATCH(8, 32, 64, 16, 2, 10, 34, 9, 0),
    PATCH(8, 32, 64, 16, 3, 10, 34, 9, 0),
    PATCH(8, 32, 32, 16, 2, 12, 36, 9, 0),
    PATCH(16, 32, 32, 16, 2, 20, 36, 9, 0),
    PATCH(16, 32, 32, 16, 2, 20, 36, 9, 1),
    PATCH(8, 32, 32, 16, 3, 12, 36, 9, 0),
    PATCH(8, 32, 64, 32, 2, 10, 34, 9, 0),
    PATCH(16, 16, 64, 16, 2, 18, 18, 9, 0),
    DMA(1, 128, 128, 2, 2, 2, 32, 1),
    DMA(1, 128, 128, 2, 2, 2, 32, 2),
    DMA(1, 256, 64, 4, 1, 2, 32, 1),
    DMA(1, 128, 64, 2, 2, 2, 32, 1),
    DMA(1, 128, 64, 2, 2, 2, 32, 2),
    DMA(1, 128, 32, 4, 1, 2, 32, 1),
    DMA(1, 64, 64, 2, 2, 2, 16, 1),
    DMA(1, 64, 64, 2, 2, 2, 16, 2),
    DMA(1, 128, 64, 2, 2, 2, 16, 1),
    DMA(1, 128, 32, 4, 1, 2, 16, 1),
    DMA(1, 128, 32, 4, 1, 2, 16, 2),
    DMA(1, 64, 32, 2, 2, 2, 16, 2),
    DMA(1, 128, 64, 2, 2, 3, 16, 1),
    DMA(1, 128, 32, 4, 1, 3, 16, 1),
    DMA(1, 64, 64, 2, 2, 3, 16, 1),
    DMA(1, 128, 128, 2, 2, 3, 32, 1),
    DMAF(1, 192, 384, 2, 4, 2, 32, 1, 4),
    DMAF(1, 256, 256, 2, 4, 2, 32, 1, 4),
    DMA(0, 32, 32, 2, 2, 2, 16, 1),
    DMA(0, 32, 32, 2, 2, 2, 16, 2),
    DMA(0, 32, 32, 2, 2, 2, 16, 4),
    DMA(0, 32, 32, 2, 2, 3, 16, 2),
    DMA(0, 32, 32, 2, 2, 4, 16, 2),
    DMA(0, 32, 64, 1, 4, 2, 16, 1),
    DMA(0, 32, 64, 1, 4, 2, 16, 2),
    DMA(0, 64, 32, 4, 1, 2, 16, 2),
    DMA(0, 64, 64, 2, 2, 2, 16, 1),
    DMA(0, 64, 64, 2, 2, 2, 16, 2),
    DMA2(0, 32, 32, 2, 2, 2, 16, 2),
    DMA2(0, 32, 32, 2, 2, 2, 16, 1),
    DMA2(0, 32, 64, 1, 4, 2, 16, 2),
    DMA2(0, 32, 64, 1, 4, 2, 16, 1),
    DMA2(0, 64, 32, 4, 1, 2, 16, 1),
    DMA2(0, 64, 64, 2, 2, 2, 16, 1),
    DMA4(0, 48, 48, 2, 16, 1),
    DMA4F(0, 48, 48, 2, 16, 1, 4),
    DMAX(0, 48, 48, 1, 3, 3, 16, 1, 4, 4, "f32_dma_48x48_w1x3_s3_m16_k1_g4_f4"),
    DMAX(0, 48, 48, 3, 1, 3, 16, 1, 4, 4, "f32_dma_48x48_w3x1_s3_m16_k1_g4_f4"),
    DMAX(0, 48, 48, 3, 1, 2, 16, 1, 4, 4, "f32_dma_48x48_w3x1_s2_m16_k1_g4_f4"),
    DMAX(0, 48, 48, 1, 3, 2, 16, 1, 4, 4, "f32_dma_48x48_w1x3_s2_m16_k1_g4_f4"),
    DMAX(0, 48, 96, 3, 2, 2, 16, 2, 2, 0, "f32_dma_48x96_w3x2_s2_m16_k2_g2"),
    DMAX(0, 48, 96, 3, 2, 2, 16, 2, 2, 4, "f32_dma_48x96_w3x2_s2_m16_k2_g2_f4"),
    DMA4(0, 48, 48, 3, 16, 1),
    DMA2(0, 48, 96, 1, 2, 3, 16, 1),
    DMA2(0, 48, 96, 1, 2, 2, 16, 2),
    DMA4(0, 32, 32, 2, 16, 1),
    DMA2(1, 128, 64, 2, 2, 2, 32, 1),
    DMA2(1, 64, 64, 2, 2, 2, 16, 1),
    DMA2(1, 128, 32, 4, 1, 2, 16, 1),
    CFG(1, 128, 128, 64, 2, 2, 8),
    CFG(1, 128, 64, 64, 2, 2, 8),
    CFG(1, 128, 32, 64, 4, 1, 8),
    CFG(1, 64, 64, 64, 2, 2, 8),
    CFG(1, 64, 32, 64, 2, 2, 8),
    CFG(1, 256, 64, 64, 4, 1, 8),
    CFG(1, 64, 64, 32, 2, 2, 1),
    CFG(0, 64, 64, 32, 2, 2, 4),
    CFG(0, 32, 64, 32, 1, 4, 4),
    CFG(0, 64, 32, 32, 4, 1, 4),
    CFG(0, 32, 32, 32, 2, 2, 4),
    CFG(0, 128, 64, 32, 2, 2, 4),
    CFG(0, 64, 64, 16, 2, 2, 1),
};
constexpr int kNumCfgs = (int)(sizeof(kCfgs) / sizeof(kCfgs[0]));

// Per-configuration cost coefficients fitted to a sweep of every
// configuration over a grid of problems (tuning/fit.py): predicted
// milliseconds t = a + b*r + d*r*nk + e*nk + f*gelu*r, r = workgroups per
// compute unit, nk = K-steps per workgroup, gelu = 1 with the GELU epilogue.
struct CostCoef {
    const char *name;
    double a, b, d, e, f;
};
const CostCoef kCoef[] = {
#include "selector_coef.inc"
};

// Exact-shape tuning records: for every problem of the calibration sweep,
// the configuration measured fastest on MI355X (256 compute units), with and
// without the GELU epilogue, and the one measured fastest from prepacked
// weights (tuning/fit.py writes them from the sweep; "" when no
// configuration with a prepacked form fits the problem).  A plan for one of
// these shapes (the bias flag is ignored) on a device with that many compute
// units takes the record; every other shape is decided by the fitted cost
// model, and its prepacked entry points use the same configuration.
struct TuneRec {
    int32_t dtype, gelu;
    int64_t N, G, C, K, in[3], filt[3], stride[3], pad[3], dil[3];
    const char *config;
    const char *packed_config;
};
const TuneRec kTuneDb[] = {
#include "selector_db.inc"
};
constexpr int kTuneCus = 256;

int config_index(const char *name)
{
    for (int i = 0; i < kNumCfgs; ++i)
        if (strcmp(kCfgs[i].name, name) == 0) return i;
    return -1;
}

// The record for the problem: its configuration (or -1) and, in *packed,
// its prepacked-weight configuration (or -1).
int tuned_config(const conv_fwd_desc_t &d, int *packed)
{
    *packed = -1;
    for (const TuneRec &t : kTuneDb) {
        bool same = t.dtype == d.dtype && t.gelu == d.gelu && t.N == d.N && t.G == d.G && t.C == d.C &&
                    t.K == d.K;
        for (int i = 0; same && i < 3; ++i)
            same = t.in[i] == d.in[i] && t.filt[i] == d.filt[i] && t.stride[i] == d.stride[i] &&
                   t.pad[i] == d.pad[i] && t.dil[i] == d.dilation[i];
        if (!same) continue;
        *packed = config_index(t.packed_config);
        return config_index(t.config);
    }
    return -1;
}

const CostCoef *coef_of(const TileCfg &c)
{
    for (const CostCoef &k : kCoef)
        if (strcmp(k.name, c.name) == 0) return &k;
    return nullptr;
}

// Division by d >= 1 as a multiply-high and shift (exact for 0 <= n < 2^31).
// A zero-sized dimension (an empty batch has no output rows, so no tiles)
// gets the divisor 1: such a plan launches nothing.
FastDiv make_fastdiv(int d)
{
    if (d < 1) d = 1;
    FastDiv f;
    uint32_t s = 0;
    while ((1ull << s) < (uint64_t)d) ++s;
    f.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << s) - (uint64_t)d)) / (uint64_t)d + 1);
    f.s = s;
    f.d = (uint32_t)d;
    return f;
}

int device_cu_count()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) { (void)hipGetLastError(); return 256; }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    return cus > 0 ? cus : 256;
}

}  // namespace
}  // namespace convfwd

using namespace convfwd;

struct conv_chain_plan {
    conv_fwd_desc_t first, second;
    int64_t out1[3], out2[3];   // output extents of the two convs
    int64_t x_elems, w1_elems, w2_elems, b_elems, y_elems;
    ChainParams cp;  // pointers filled per run
    int grid;
    ChainPackedParams pp;  // prepacked-weight kernel; pointers filled per run
    int pgrid;
    int64_t packed_bytes;   // 0: C1 beyond what the prepacked kernel supports
    char text[320];
};

struct conv_bwd_data_plan {
    conv_fwd_desc_t desc;     // the forward problem
    conv_fwd_plan_t *fwd;     // dx = forward conv of (dyp or dy) with w' (no stride phases)
    bool spread;              // build the zero-inserted copy of dy
    SpreadParams sp;          // pointers filled per run
    // > 0: a 1-D strided problem run as nphase stride phases, each a forward
    // conv of dy itself writing every s-th row of dx (no spread copy)
    int nphase;
    conv_fwd_plan_t *phase[kMaxPhases];
    PhaseWeightParams pwp;    // the phases' filters, at pwp.base[f] elements into the workspace
    int64_t dy_elems, w_elems, dx_elems;
    int64_t ws_wt, ws_dyp, ws_bytes;   // workspace: w' at 0, dyp at ws_wt
    char text[1200];
};

struct conv_bwd_weight_plan {
    conv_fwd_desc_t desc;     // the forward problem
    WgradParams wp;           // pointers filled per run
    int KT, TT;               // tile: KT x KT channels, TT taps
    int NWV;                  // waves per workgroup
    int occ;                  // workgroups per CU at once
    int grid;
    int64_t x_elems, dy_elems, dw_elems, ws_bytes;
    char text[320];
};

struct conv_fwd_plan {
    conv_fwd_desc_t desc;
    int64_t out[3];
    int64_t x_elems, w_elems, b_elems, y_elems;
    int esz;
    int cfg;
    bool tuned;      // cfg came from an exact-shape tuning record
    int grid;
    KParams kp;      // pointers filled per run
    PackParams pk;   // prepacked weights: pointers filled per call
    int64_t packed_bytes;   // 0: the plan's kernel reads natural weights only
    // The prepacked entry points' plan when a tuning record names another
    // configuration for them (owned), else null: they use this plan.
    conv_fwd_plan *packed_plan;
    char text[320];
};

namespace {

int64_t extent(int64_t I, int64_t F, int64_t s, int64_t p, int64_t d)
{
    int64_t span = I + 2 * p - d * (F - 1) - 1;
    return span < 0 ? 0 : span / s + 1;
}

conv_status_t validate(const conv_fwd_desc_t *d, int64_t out[3])
{
    if (!d) return fail(CONV_ERR_INVALID_ARG, "descriptor is NULL");
    if (d->ndim < 1 || d->ndim > 3) return fail(CONV_ERR_INVALID_ARG, "ndim must be 1, 2 or 3 (got %d)", d->ndim);
    if (d->dtype != CONV_DT_F32 && d->dtype != CONV_DT_BF16)
        return fail(CONV_ERR_INVALID_ARG, "unknown dtype %d", d->dtype);
    if (d->has_bias != 0 && d->has_bias != 1) return fail(CONV_ERR_INVALID_ARG, "has_bias must be 0 or 1");
    if (d->gelu != 0 && d->gelu != 1) return fail(CONV_ERR_INVALID_ARG, "gelu must be 0 or 1");
    if (d->N < 0) return fail(CONV_ERR_INVALID_ARG, "N must be >= 0 (got %lld)", (long long)d->N);
    if (d->G < 1 || d->C < 1 || d->K < 1)
        return fail(CONV_ERR_INVALID_ARG, "G, C and K must be >= 1 (got %lld, %lld, %lld)",
                    (long long)d->G, (long long)d->C, (long long)d->K);
    static const char *dn[3] = {"D", "H", "W"};
    for (int i = 0; i < 3; ++i) {
        if (d->in[i] < 1 || d->filt[i] < 1 || d->stride[i] < 1 || d->dilation[i] < 1 || d->pad[i] < 0)
            return fail(CONV_ERR_INVALID_ARG, "dim %s: need in, filt, stride, dilation >= 1 and pad >= 0", dn[i]);
        if (i < 3 - d->ndim &&
            (d->in[i] != 1 || d->filt[i] != 1 || d->stride[i] != 1 || d->dilation[i] != 1 || d->pad[i] != 0))
            return fail(CONV_ERR_INVALID_ARG, "dim %s is unused for ndim=%d and must be trivial", dn[i], d->ndim);
        if (d->in[i] > (1 << 30) || d->filt[i] > (1 << 30) || d->stride[i] > (1 << 30) ||
            d->dilation[i] > (1 << 30) || d->pad[i] > (1 << 30))
            return fail(CONV_ERR_UNSUPPORTED, "dim %s: a size above 2^30", dn[i]);
        out[i] = extent(d->in[i], d->filt[i], d->stride[i], d->pad[i], d->dilation[i]);
        if (out[i] < 1)
            return fail(CONV_ERR_INVALID_ARG, "dim %s: the dilated filter (%lld) is larger than the padded input (%lld)",
                        dn[i], (long long)(d->dilation[i] * (d->filt[i] - 1) + 1),
                        (long long)(d->in[i] + 2 * d->pad[i]));
    }
    if (d->G > (1 << 30) || d->C > (1 << 30) || d->K > (1 << 30) || d->N > (1 << 30))
        return fail(CONV_ERR_UNSUPPORTED, "N, G, C or K above 2^30");
    // Every element offset the kernels form must fit in a signed 32-bit
    // integer.  A row base or a tap offset stays within the zero-padded input
    // (a coordinate lies in [-p, I + p): the last window ends inside the
    // padding), so N x prod(I + 2p) x G x C bounds them all; a sum of the
    // two is only formed for a tap inside the input.
    const double lim = 2147483647.0;
    const double gc = (double)d->G * (double)d->C, gk = (double)d->G * (double)d->K;
    const double xpad = (double)std::max<int64_t>(d->N, 1) * (d->in[0] + 2.0 * d->pad[0]) *
                        (d->in[1] + 2.0 * d->pad[1]) * (d->in[2] + 2.0 * d->pad[2]) * gc;
    const double welem = gk * d->C * (double)d->filt[0] * d->filt[1] * d->filt[2];
    const double yelem = (double)d->N * out[0] * out[1] * out[2] * gk;
    if (xpad >= lim || welem >= lim || yelem >= lim)
        return fail(CONV_ERR_UNSUPPORTED, "tensor too large for 32-bit element offsets");
    return CONV_OK;
}

// Analytic cost of one configuration (seconds), used for configurations the
// calibration sweep has no coefficients for: the
// workgroups are spread over the compute units in rounds; each round costs
// the MFMA time of one tile at an efficiency that grows with the wave
// sub-tile (larger sub-tiles read LDS less per flop); the whole run is at
// least the time to move the algorithmic bytes at HBM speed.
double cost(const TileCfg &c, const conv_fwd_plan &pl, int cus)
{
    const conv_fwd_desc_t &d = pl.desc;
    const int64_t M = d.N * pl.out[0] * pl.out[1] * pl.out[2];
    const int64_t Kred = d.C * d.filt[0] * d.filt[1] * d.filt[2];
    const int64_t tm = (M + c.BM - 1) / c.BM, tn = (d.K + c.BN - 1) / c.BN;
    const double tiles = (double)tm * tn * d.G;
    const double kpad = (double)((Kred + c.BK - 1) / c.BK) * c.BK;
    const double flop_tile = 2.0 * c.BM * c.BN * kpad;
    const double cu_rate = (d.dtype == CONV_DT_BF16 ? 4096.0 : 256.0) * 2.4e9;  // flop/s per CU
    const double tmw = (double)c.BM / c.WM, tnw = (double)c.BN / c.WN;
    const double intensity = tmw * tnw / (tmw + tnw);                          // 8 .. 43
    double eff = std::min(1.0, intensity / (d.dtype == CONV_DT_BF16 ? 40.0 : 12.0));
    eff *= (double)(c.WM * c.WN) / 4.0;                                          // waves per CU
    if (c.kind != KIND_REG) eff = std::min(1.0, eff * 2.0);                      // no register staging
    const double rounds = std::ceil(tiles / cus);
    const double t_mfma = rounds * flop_tile / (cu_rate * std::max(eff, 0.05));
    const double bytes = (double)pl.esz * (pl.x_elems + pl.w_elems + pl.b_elems + pl.y_elems);
    const double t_mem = bytes / 8.0e12;
    return std::max(t_mfma, t_mem) + 1e-7 * kpad / c.BK;  // small per-step overhead
}

// Workgroups of a configuration on a problem, and K-steps per workgroup.
double tiles_of(const TileCfg &c, const conv_fwd_desc_t &d, const int64_t out[3])
{
    const double tn = (double)((d.K + c.BN - 1) / c.BN);
    if (c.kind == KIND_PATCH || c.kind == KIND_PATCHF)
        return (double)d.N * out[0] * (double)((out[1] + c.TH - 1) / c.TH) *
               (double)((out[2] + c.TW - 1) / c.TW) * tn * (double)d.G;
    const int64_t M = d.N * out[0] * out[1] * out[2];
    return (double)((M + c.BM - 1) / c.BM) * tn * (double)d.G;
}

double steps_of(const TileCfg &c, const conv_fwd_desc_t &d)
{
    if (c.kind == KIND_PATCH || c.kind == KIND_PATCHF) return (double)d.filt[0] * (double)(d.C / c.CC);
    const int64_t Kred = d.C * d.filt[0] * d.filt[1] * d.filt[2];
    const int64_t kg = c.KG > 1 ? c.KG : 1;
    return (double)(((Kred + c.BK - 1) / c.BK + kg - 1) / kg);   // K-steps of one reduction group
}

// Predicted milliseconds of one configuration on the plan's problem.
double predicted_ms(const TileCfg &c, const conv_fwd_plan &pl, int cus)
{
    const CostCoef *k = coef_of(c);
    if (!k) return 1e3 * cost(c, pl, cus) * 10.0;   // uncalibrated: last resort
    const double r = std::ceil(tiles_of(c, pl.desc, pl.out) / cus);
    const double nk = steps_of(c, pl.desc);
    const double g = pl.desc.gelu ? 1.0 : 0.0;
    return k->a + k->b * r + k->d * r * nk + k->e * nk + k->f * g * r;
}

// The patch kernel's shape limits: channel slices, patch extent, taps.
bool patch_fits(const TileCfg &c, const conv_fwd_desc_t &d)
{
    const int64_t ph = (c.TH - 1) * d.stride[1] + (d.filt[1] - 1) * d.dilation[1] + 1;
    const int64_t pw = (c.TW - 1) * d.stride[2] + (d.filt[2] - 1) * d.dilation[2] + 1;
    return d.C % c.CC == 0 && ph <= c.PHMAX && pw <= c.PWMAX && d.filt[1] * d.filt[2] <= c.TAPMAX;
}

// The fixed-filter patch kernel: unit H/W stride and exactly its filter.
bool patchf_fits(const TileCfg &c, const conv_fwd_desc_t &d)
{
    return d.C % c.CC == 0 && d.filt[0] <= 32 && d.stride[1] == 1 && d.stride[2] == 1 && d.filt[1] == c.FY && d.filt[2] == c.FX &&
           d.dilation[1] == c.DH && d.dilation[2] == c.DW;
}

}  // namespace

// ---- Backward-data without allocation ---------------------------------------
// For callers that cannot allocate (graph capture, serving loops): the
// workspace is this file-scope device array, one copy per GPU, held until the
// process ends.  Host code never passes the array's name to a kernel -- on
// the host it is only a stand-in for the symbol -- but the device address
// hipGetSymbolAddress returns for it, looked up once per device (with that
// device current) and kept here.
static __device__ __align__(256) unsigned char scratch[CONV_BWD_DATA_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void *g_scratch_ptr[kMaxDevices];

conv_status_t scratch_of_current_device(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(CONV_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(CONV_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(CONV_ERR_HIP, "hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return CONV_OK;
}
}  // namespace

extern "C" {

const char *conv_fwd_last_error(void) { return g_err; }

int32_t conv_fwd_num_configs(void) { return kNumCfgs; }

const char *conv_fwd_config_name(int32_t config)
{
    return (config >= 0 && config < kNumCfgs) ? kCfgs[config].name : nullptr;
}

int32_t conv_fwd_config_dtype(int32_t config)
{
    return (config >= 0 && config < kNumCfgs) ? kCfgs[config].dtype : -1;
}

static conv_status_t create_impl(const conv_fwd_desc_t *desc, int32_t forced, conv_fwd_plan_t **plan)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan output pointer is NULL");
    *plan = nullptr;
    int64_t out[3];
    conv_status_t st = validate(desc, out);
    if (st != CONV_OK) return st;

    conv_fwd_plan *pl = new (std::nothrow) conv_fwd_plan();
    if (!pl) return fail(CONV_ERR_NOMEM, "plan allocation failed");
    const conv_fwd_desc_t &d = *desc;
    pl->desc = d;
    for (int i = 0; i < 3; ++i) pl->out[i] = out[i];
    pl->esz = d.dtype == CONV_DT_BF16 ? 2 : 4;
    pl->x_elems = d.N * d.in[0] * d.in[1] * d.in[2] * d.G * d.C;
    pl->w_elems = d.G * d.K * d.filt[0] * d.filt[1] * d.filt[2] * d.C;
    pl->b_elems = d.has_bias ? d.G * d.K : 0;
    pl->y_elems = d.N * out[0] * out[1] * out[2] * d.G * d.K;

    const int vec = 16 / pl->esz;
    const int want_vec = (d.C % vec == 0) ? vec : 1;
    // the direct-to-LDS kernels address x and w with 32-bit byte offsets
    const bool dma_ok = want_vec == vec && pl->x_elems * pl->esz < (int64_t(1) << 31) &&
                        pl->w_elems * pl->esz < (int64_t(1) << 31);
    auto eligible = [&](const TileCfg &c) {
        if (c.dtype != d.dtype) return false;
        if (c.kind == KIND_REG) return c.VEC == want_vec;
        if (c.kind == KIND_DMA) return dma_ok;
        if (c.kind == KIND_PATCHF) return dma_ok && patchf_fits(c, d);
        return dma_ok && patch_fits(c, d);
    };
    if (forced >= 0) {
        if (forced >= kNumCfgs) {
            delete pl;
            return fail(CONV_ERR_INVALID_ARG, "config %d out of range (0..%d)", forced, kNumCfgs - 1);
        }
        const TileCfg &c = kCfgs[forced];
        if (c.dtype != d.dtype) {
            delete pl;
            return fail(CONV_ERR_UNSUPPORTED, "config %s is for the other dtype", c.name);
        }
        if (c.VEC != 1 && !eligible(c)) {
            delete pl;
            return fail(CONV_ERR_UNSUPPORTED, "config %s needs C %% %d == 0 (C = %lld)%s", c.name,
                        c.kind == KIND_PATCH || c.kind == KIND_PATCHF ? c.CC : c.VEC, (long long)d.C,
                        c.kind == KIND_PATCH ? ", x and w below 2 GiB, and a patch / tap count within its limits"
                        : c.kind == KIND_PATCHF ? ", x and w below 2 GiB, unit H/W stride and exactly its H/W filter "
                                                  "and dilation"
                        : c.kind == KIND_DMA ? " and x, w below 2 GiB" : "");
        }
        pl->cfg = forced;
    } else {
        const int cus = device_cu_count();
        int prec = -1;
        const int rec = cus == kTuneCus ? tuned_config(d, &prec) : -1;
        if (rec >= 0 && eligible(kCfgs[rec])) {
            pl->cfg = rec;
            pl->tuned = true;
            if (prec >= 0 && prec != rec && eligible(kCfgs[prec])) {
                conv_fwd_plan *pp = nullptr;
                st = create_impl(desc, prec, &pp);
                if (st != CONV_OK) {
                    delete pl;
                    return st;
                }
                pp->tuned = true;
                pl->packed_plan = pp;
            }
        } else {
            int best = -1;
            double best_cost = 0.0;
            for (int i = 0; i < kNumCfgs; ++i) {
                const TileCfg &c = kCfgs[i];
                if (!eligible(c)) continue;
                const double t = predicted_ms(c, *pl, cus);
                if (best < 0 || t < best_cost) { best = i; best_cost = t; }
            }
            pl->cfg = best;
        }
    }
    const TileCfg &c = kCfgs[pl->cfg];
    KParams &kp = pl->kp;
    kp.N = (int)d.N; kp.G = (int)d.G; kp.C = (int)d.C; kp.K = (int)d.K;
    kp.Di = (int)d.in[0]; kp.Hi = (int)d.in[1]; kp.Wi = (int)d.in[2];
    kp.Z = (int)d.filt[0]; kp.Y = (int)d.filt[1]; kp.X = (int)d.filt[2];
    kp.sd = (int)d.stride[0]; kp.sh = (int)d.stride[1]; kp.sw = (int)d.stride[2];
    kp.pd = (int)d.pad[0]; kp.ph = (int)d.pad[1]; kp.pw = (int)d.pad[2];
    kp.dd = (int)d.dilation[0]; kp.dh = (int)d.dilation[1]; kp.dw = (int)d.dilation[2];
    kp.Do = (int)out[0]; kp.Ho = (int)out[1]; kp.Wo = (int)out[2];
    kp.M = (int)(d.N * out[0] * out[1] * out[2]);
    kp.Kred = (int)(d.C * d.filt[0] * d.filt[1] * d.filt[2]);
    kp.tiles_m = (kp.M + c.BM - 1) / c.BM;
    kp.tiles_n = (kp.K + c.BN - 1) / c.BN;
    kp.gelu = d.gelu;
    kp.out_vec = (d.K % (16 / pl->esz) == 0) ? 1 : 0;
    kp.fd_Wo = make_fastdiv(kp.Wo);
    kp.fd_Ho = make_fastdiv(kp.Ho);
    kp.fd_Do = make_fastdiv(kp.Do);
    kp.fd_C = make_fastdiv(kp.C);
    kp.fd_X = make_fastdiv(kp.X);
    kp.fd_Y = make_fastdiv(kp.Y);
    kp.fd_tn = make_fastdiv(kp.tiles_n);
    kp.fd_tm = make_fastdiv(kp.tiles_m);
    kp.ldy = (int)(d.G * d.K);
    // prepacked weight image of this plan's kernel (none for the register-staged one)
    PackParams &pk = pl->pk;
    pk.esz = pl->esz;
    pk.K = kp.K; pk.Kred = kp.Kred; pk.C = kp.C; pk.Z = kp.Z; pk.taps = kp.Y * kp.X;
    pk.BN = c.BN; pk.tiles_n = kp.tiles_n;
    double img = 0.0;
    if (c.kind == KIND_DMA) {
        pk.mode = 0;
        pk.subk = 128 / pl->esz;
        pk.ksub = c.BK / pk.subk;
        pk.vec = 16 / pl->esz;
        pk.nk = (kp.Kred + c.BK - 1) / c.BK;
        pk.sw4 = (c.MF == 32 && kp.C % (2 * pk.vec) == 0) ? 1 : 0;
        img = (double)d.G * kp.tiles_n * pk.nk * pk.ksub * c.BN * 128.0;
    } else if (c.kind == KIND_PATCHF) {
        pk.mode = 1;
        pk.ncs = kp.C / c.CC;
        pk.cc = c.CC;
        pk.wslots = (c.CC / 8) * pk.taps * c.BN;
        pk.img_slots = c.wimg / 16;
        img = (double)d.G * kp.tiles_n * kp.Z * pk.ncs * (double)c.wimg;
    }
    pl->packed_bytes = img < 2147483647.0 ? (int64_t)img : 0;
    pk.slots = pl->packed_bytes / 16;
    const double grid = tiles_of(c, d, out);
    if (grid >= 2147483647.0) {
        delete pl->packed_plan;
        delete pl;
        return fail(CONV_ERR_UNSUPPORTED, "grid too large");
    }
    pl->grid = (int)grid;
    if (c.kind == KIND_PATCH || c.kind == KIND_PATCHF)
        snprintf(pl->text, sizeof(pl->text),
                 "patch %s M=%d N=%d Kred=%d G=%d grid=%d (%dx%d boxes/plane, %d n-tiles) lds=%dB%s", c.name,
                 kp.M, kp.K, kp.Kred, kp.G, pl->grid, (kp.Ho + c.TH - 1) / c.TH, (kp.Wo + c.TW - 1) / c.TW,
                 kp.tiles_n, c.lds_bytes, forced >= 0 ? " forced" : pl->tuned ? " tuned" : "");
    else
        snprintf(pl->text, sizeof(pl->text),
                 "igemm %s M=%d N=%d Kred=%d G=%d grid=%d (%dx%dx%d tiles) lds=%dB%s",
                 c.name, kp.M, kp.K, kp.Kred, kp.G, pl->grid, kp.tiles_m, kp.tiles_n, kp.G, c.lds_bytes,
                 forced >= 0 ? " forced" : pl->tuned ? " tuned" : "");
    if (pl->packed_plan) {
        const size_t n = strlen(pl->text);
        snprintf(pl->text + n, sizeof(pl->text) - n, "; prepacked: %s grid=%d", kCfgs[pl->packed_plan->cfg].name,
                 pl->packed_plan->grid);
    }
    if (getenv("CONVFWD_LOG")) fprintf(stderr, "convfwd: %s\n", pl->text);
    *plan = pl;
    return CONV_OK;
}

conv_status_t conv_fwd_create(const conv_fwd_desc_t *desc, conv_fwd_plan_t **plan)
{
    return create_impl(desc, -1, plan);
}

conv_status_t conv_fwd_create_with_config(const conv_fwd_desc_t *desc, int32_t config, conv_fwd_plan_t **plan)
{
    if (config < 0) {
        if (plan) *plan = nullptr;
        return fail(CONV_ERR_INVALID_ARG, "config %d out of range", config);
    }
    return create_impl(desc, config, plan);
}

conv_status_t conv_fwd_out_dims(const conv_fwd_plan_t *plan, int64_t out[3])
{
    if (!plan || !out) return fail(CONV_ERR_INVALID_ARG, "NULL argument");
    for (int i = 0; i < 3; ++i) out[i] = plan->out[i];
    return CONV_OK;
}

conv_status_t conv_fwd_useful_flop(const conv_fwd_plan_t *plan, int64_t *flop)
{
    if (!plan || !flop) return fail(CONV_ERR_INVALID_ARG, "NULL argument");
    const conv_fwd_desc_t &d = plan->desc;
    *flop = 2 * d.N * d.G * d.K * d.C * plan->out[0] * plan->out[1] * plan->out[2] * d.filt[0] * d.filt[1] *
            d.filt[2];
    return CONV_OK;
}

static bool overlaps(const void *a, int64_t an, const void *b, int64_t bn)
{
    if (!a || !b || an <= 0 || bn <= 0) return false;
    const char *pa = (const char *)a, *pb = (const char *)b;
    return pa < pb + bn && pb < pa + an;
}

static conv_status_t run_impl(const conv_fwd_plan_t *plan, const void *x, const void *w, const void *bias, void *y,
                              void *stream, void *start_event, void *stop_event, bool packed);

conv_status_t conv_fwd_run_events(const conv_fwd_plan_t *plan, const void *x, const void *w,
                                  const void *bias, void *y, void *stream, void *start_event,
                                  void *stop_event)
{
    return run_impl(plan, x, w, bias, y, stream, start_event, stop_event, false);
}

// The plan the prepacked entry points run.
static const conv_fwd_plan_t *packed_of(const conv_fwd_plan_t *plan)
{
    return plan && plan->packed_plan ? plan->packed_plan : plan;
}

conv_status_t conv_fwd_packed_config(const conv_fwd_plan_t *plan, int32_t *config)
{
    if (!plan || !config) return fail(CONV_ERR_INVALID_ARG, "plan or config is NULL");
    *config = packed_of(plan)->cfg;
    return CONV_OK;
}

conv_status_t conv_fwd_packed_bytes(const conv_fwd_plan_t *plan, int64_t *bytes)
{
    plan = packed_of(plan);
    if (!plan || !bytes) return fail(CONV_ERR_INVALID_ARG, "plan or bytes is NULL");
    if (plan->packed_bytes == 0)
        return fail(CONV_ERR_UNSUPPORTED, "the plan's kernel (%s) reads natural weights only",
                    kCfgs[plan->cfg].name);
    *bytes = plan->packed_bytes;
    return CONV_OK;
}

conv_status_t conv_fwd_pack_weights(const conv_fwd_plan_t *plan, const void *w, void *packed, void *stream)
{
    plan = packed_of(plan);
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    if (plan->packed_bytes == 0)
        return fail(CONV_ERR_UNSUPPORTED, "the plan's kernel (%s) reads natural weights only",
                    kCfgs[plan->cfg].name);
    if (!w || !packed) return fail(CONV_ERR_INVALID_ARG, "w or packed is NULL");
    if (((uintptr_t)w | (uintptr_t)packed) & 15u)
        return fail(CONV_ERR_INVALID_ARG, "w and packed must be 16-byte aligned");
    if (overlaps(packed, plan->packed_bytes, w, plan->w_elems * plan->esz))
        return fail(CONV_ERR_INVALID_ARG, "packed overlaps w");
    PackParams pk = plan->pk;
    pk.w = w;
    pk.out = packed;
    (void)hipGetLastError();
    hipLaunchKernelGGL(pack_weights_kernel, dim3((unsigned)((pk.slots + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, pk);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(CONV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return CONV_OK;
}

conv_status_t conv_fwd_run_packed_events(const conv_fwd_plan_t *plan, const void *x, const void *packed,
                                         const void *bias, void *y, void *stream, void *start_event,
                                         void *stop_event)
{
    plan = packed_of(plan);
    if (plan && plan->packed_bytes == 0)
        return fail(CONV_ERR_UNSUPPORTED, "the plan's kernel (%s) reads natural weights only",
                    kCfgs[plan->cfg].name);
    return run_impl(plan, x, packed, bias, y, stream, start_event, stop_event, true);
}

conv_status_t conv_fwd_run_packed(const conv_fwd_plan_t *plan, const void *x, const void *packed,
                                  const void *bias, void *y, void *stream)
{
    return conv_fwd_run_packed_events(plan, x, packed, bias, y, stream, nullptr, nullptr);
}

static conv_status_t run_impl(const conv_fwd_plan_t *plan, const void *x, const void *w, const void *bias, void *y,
                              void *stream, void *start_event, void *stop_event, bool packed)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    const conv_fwd_desc_t &d = plan->desc;
    if (plan->desc.has_bias && !bias) return fail(CONV_ERR_INVALID_ARG, "plan has a bias but bias is NULL");
    if (!plan->desc.has_bias && bias) return fail(CONV_ERR_INVALID_ARG, "plan has no bias but bias is not NULL");
    if (!w) return fail(CONV_ERR_INVALID_ARG, "w is NULL");
    if (plan->y_elems == 0) return CONV_OK;   // N = 0: nothing to do
    if (!x || !y) return fail(CONV_ERR_INVALID_ARG, "x or y is NULL");
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & 15u)
        return fail(CONV_ERR_INVALID_ARG, "x, w and y must be 16-byte aligned");
    if (bias && ((uintptr_t)bias & (uintptr_t)(plan->esz - 1)))
        return fail(CONV_ERR_INVALID_ARG, "bias is not aligned to its element size");
    const int64_t e = plan->esz;
    const int64_t wbytes = packed ? plan->packed_bytes : plan->w_elems * e;
    if (overlaps(y, plan->y_elems * e, x, plan->x_elems * e) || overlaps(y, plan->y_elems * e, w, wbytes) ||
        overlaps(y, plan->y_elems * e, bias, plan->b_elems * e))
        return fail(CONV_ERR_INVALID_ARG, "y overlaps an input");
    KParams kp = plan->kp;
    kp.x = x; kp.w = w; kp.bias = bias; kp.y = y;
    kp.wpacked = packed ? 1 : 0;
    (void)d;
    (void)hipGetLastError();  // clear a stale error so the check below is ours
    kCfgs[plan->cfg].fn(kp, (uint32_t)(plan->x_elems * e), (uint32_t)wbytes, plan->grid,
                        (hipStream_t)stream, (hipEvent_t)start_event, (hipEvent_t)stop_event);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(CONV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return CONV_OK;
}

conv_status_t conv_fwd_run(const conv_fwd_plan_t *plan, const void *x, const void *w,
                           const void *bias, void *y, void *stream)
{
    return conv_fwd_run_events(plan, x, w, bias, y, stream, nullptr, nullptr);
}

void conv_fwd_destroy(conv_fwd_plan_t *plan)
{
    if (plan) delete plan->packed_plan;
    delete plan;
}

const char *conv_fwd_describe(const conv_fwd_plan_t *plan) { return plan ? plan->text : ""; }

conv_status_t conv_chain_create(const conv_fwd_desc_t *first, const conv_fwd_desc_t *second,
                                conv_chain_plan_t **plan)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    *plan = nullptr;
    int64_t o1[3], o2[3];
    conv_status_t st = validate(first, o1);
    if (st != CONV_OK) return st;
    st = validate(second, o2);
    if (st != CONV_OK) return st;
    const conv_fwd_desc_t &a = *first, &b = *second;
    using S = ChainShape;
    if (a.ndim != 1 || b.ndim != 1 || a.dtype != CONV_DT_BF16 || b.dtype != CONV_DT_BF16 || a.G != 1 || b.G != 1)
        return fail(CONV_ERR_UNSUPPORTED, "fused chain: both convs must be 1-D, bf16, one group");
    if (b.N != a.N || b.C != a.K || b.in[2] != o1[2])
        return fail(CONV_ERR_INVALID_ARG, "fused chain: the second conv must read the first one's output "
                                          "(same N, C2 == K1, input length == first output length)");
    if (a.filt[2] != 3 || a.stride[2] != 1 || a.pad[2] != 1 || a.dilation[2] != 1 || b.filt[2] != 3 ||
        b.stride[2] != 2 || b.pad[2] != 1 || b.dilation[2] != 1)
        return fail(CONV_ERR_UNSUPPORTED, "fused chain: needs conv1 k3 s1 p1 and conv2 k3 s2 p1 (no dilation)");
    if (a.K != S::K || b.K != S::K)
        return fail(CONV_ERR_UNSUPPORTED, "fused chain: needs %d channels after each conv", S::K);
    if (a.C % 16 != 0 || a.C > S::C1MAX)
        return fail(CONV_ERR_UNSUPPORTED, "fused chain: needs C1 a multiple of 16 and at most %d (C1 = %lld)",
                    S::C1MAX, (long long)a.C);
    if (a.has_bias != b.has_bias || a.gelu != b.gelu)
        return fail(CONV_ERR_UNSUPPORTED, "fused chain: both convs must agree on bias and GELU");
    conv_chain_plan *pl = new (std::nothrow) conv_chain_plan();
    if (!pl) return fail(CONV_ERR_NOMEM, "plan allocation failed");
    pl->first = a;
    pl->second = b;
    for (int i = 0; i < 3; ++i) {
        pl->out1[i] = o1[i];
        pl->out2[i] = o2[i];
    }
    pl->x_elems = a.N * a.in[2] * a.C;
    pl->w1_elems = a.K * 3 * a.C;
    pl->w2_elems = b.K * 3 * b.C;
    pl->b_elems = a.has_bias ? S::K : 0;
    pl->y_elems = b.N * o2[2] * b.K;
    if (pl->x_elems * 2 >= (int64_t(1) << 31) || pl->y_elems * 2 >= (int64_t(1) << 31)) {
        delete pl;
        return fail(CONV_ERR_UNSUPPORTED, "fused chain: x and y must be below 2 GiB");
    }
    ChainParams &cp = pl->cp;
    cp.N = (int)a.N;
    cp.L = (int)a.in[2];
    cp.C1 = (int)a.C;
    cp.Lo = (int)o2[2];
    cp.tiles = (cp.Lo + S::TO - 1) / S::TO;
    cp.x_bytes = (uint32_t)(pl->x_elems * 2);
    cp.w1_bytes = (uint32_t)(pl->w1_elems * 2);
    cp.w2_bytes = (uint32_t)(pl->w2_elems * 2);
    pl->grid = (int)(a.N * cp.tiles);
    using P = ChainPackedShape;
    ChainPackedParams &pp = pl->pp;
    pp.N = cp.N;
    pp.L = cp.L;
    pp.C1 = cp.C1;
    pp.Lo = cp.Lo;
    pp.tiles = (cp.Lo + P::TO - 1) / P::TO;
    pp.x_bytes = cp.x_bytes;
    pl->pgrid = (int)(a.N * pp.tiles);
    pl->packed_bytes = a.C <= P::C1MAX ? (int64_t)P::steps((int)a.C) * P::STEP : 0;
    snprintf(pl->text, sizeof(pl->text),
             "chain bf16 N=%d L=%d C1=%d -> %d -> %d Lo=%d grid=%d (%d outputs per workgroup) lds=%dB; "
             "prepacked: grid=%d (%d outputs per workgroup) lds=%dB%s%s",
             cp.N, cp.L, cp.C1, S::K, S::K, cp.Lo, pl->grid, S::TO, S::LDS_BYTES, pl->pgrid, P::TO, P::LDS_BYTES,
             a.has_bias ? " bias" : "", a.gelu ? " gelu" : "");
    if (getenv("CONVFWD_LOG")) fprintf(stderr, "convfwd: %s\n", pl->text);
    *plan = pl;
    return CONV_OK;
}

conv_status_t conv_chain_run_events(const conv_chain_plan_t *plan, const void *x, const void *w1, const void *b1,
                                    const void *w2, const void *b2, void *y, void *stream, void *start_event,
                                    void *stop_event)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    const bool hb = plan->first.has_bias != 0;
    if (hb && (!b1 || !b2)) return fail(CONV_ERR_INVALID_ARG, "plan has biases but b1 or b2 is NULL");
    if (!hb && (b1 || b2)) return fail(CONV_ERR_INVALID_ARG, "plan has no bias but b1 or b2 is not NULL");
    if (!w1 || !w2) return fail(CONV_ERR_INVALID_ARG, "w1 or w2 is NULL");
    if (plan->y_elems == 0) return CONV_OK;
    if (!x || !y) return fail(CONV_ERR_INVALID_ARG, "x or y is NULL");
    if (((uintptr_t)x | (uintptr_t)w1 | (uintptr_t)w2 | (uintptr_t)y) & 15u)
        return fail(CONV_ERR_INVALID_ARG, "x, w1, w2 and y must be 16-byte aligned");
    if (((uintptr_t)b1 | (uintptr_t)b2) & 1u) return fail(CONV_ERR_INVALID_ARG, "b1 and b2 must be 2-byte aligned");
    const int64_t yb = plan->y_elems * 2;
    if (overlaps(y, yb, x, plan->x_elems * 2) || overlaps(y, yb, w1, plan->w1_elems * 2) ||
        overlaps(y, yb, w2, plan->w2_elems * 2) || overlaps(y, yb, b1, plan->b_elems * 2) ||
        overlaps(y, yb, b2, plan->b_elems * 2))
        return fail(CONV_ERR_INVALID_ARG, "y overlaps an input");
    ChainParams cp = plan->cp;
    cp.x = x; cp.w1 = w1; cp.b1 = b1; cp.w2 = w2; cp.b2 = b2; cp.y = y;
    (void)hipGetLastError();
    const dim3 g(plan->grid), blk(256);
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t e0 = (hipEvent_t)start_event, e1 = (hipEvent_t)stop_event;
    if (hb && plan->first.gelu)
        hipExtLaunchKernelGGL((chain_kernel<true, true>), g, blk, 0, s, e0, e1, 0, cp);
    else if (hb)
        hipExtLaunchKernelGGL((chain_kernel<true, false>), g, blk, 0, s, e0, e1, 0, cp);
    else if (plan->first.gelu)
        hipExtLaunchKernelGGL((chain_kernel<false, true>), g, blk, 0, s, e0, e1, 0, cp);
    else
        hipExtLaunchKernelGGL((chain_kernel<false, false>), g, blk, 0, s, e0, e1, 0, cp);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(CONV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return CONV_OK;
}

conv_status_t conv_chain_run(const conv_chain_plan_t *plan, const void *x, const void *w1, const void *b1,
                             const void *w2, const void *b2, void *y, void *stream)
{
    return conv_chain_run_events(plan, x, w1, b1, w2, b2, y, stream, nullptr, nullptr);
}

conv_status_t conv_chain_packed_bytes(const conv_chain_plan_t *plan, int64_t *bytes)
{
    if (!plan || !bytes) return fail(CONV_ERR_INVALID_ARG, "plan or bytes is NULL");
    if (plan->packed_bytes == 0)
        return fail(CONV_ERR_UNSUPPORTED, "prepacked chain: needs C1 at most %d (C1 = %lld)", ChainPackedShape::C1MAX,
                    (long long)plan->first.C);
    *bytes = plan->packed_bytes;
    return CONV_OK;
}

conv_status_t conv_chain_pack_weights(const conv_chain_plan_t *plan, const void *w1, const void *w2, void *packed,
                                      void *stream)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    if (plan->packed_bytes == 0)
        return fail(CONV_ERR_UNSUPPORTED, "prepacked chain: needs C1 at most %d (C1 = %lld)", ChainPackedShape::C1MAX,
                    (long long)plan->first.C);
    if (!w1 || !w2 || !packed) return fail(CONV_ERR_INVALID_ARG, "w1, w2 or packed is NULL");
    if (((uintptr_t)w1 | (uintptr_t)w2 | (uintptr_t)packed) & 15u)
        return fail(CONV_ERR_INVALID_ARG, "w1, w2 and packed must be 16-byte aligned");
    if (overlaps(packed, plan->packed_bytes, w1, plan->w1_elems * 2) ||
        overlaps(packed, plan->packed_bytes, w2, plan->w2_elems * 2))
        return fail(CONV_ERR_INVALID_ARG, "packed overlaps w1 or w2");
    const int total = (int)(plan->packed_bytes / 16);
    (void)hipGetLastError();
    hipLaunchKernelGGL(chain_pack_kernel, dim3((total + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                       (const uint4 *)w1, (const uint4 *)w2, (uint4 *)packed, (int)plan->first.C, total);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(CONV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return CONV_OK;
}

conv_status_t conv_chain_run_packed_events(const conv_chain_plan_t *plan, const void *x, const void *packed,
                                           const void *b1, const void *b2, void *y, void *stream, void *start_event,
                                           void *stop_event)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    const bool hb = plan->first.has_bias != 0;
    if (hb && (!b1 || !b2)) return fail(CONV_ERR_INVALID_ARG, "plan has biases but b1 or b2 is NULL");
    if (!hb && (b1 || b2)) return fail(CONV_ERR_INVALID_ARG, "plan has no bias but b1 or b2 is not NULL");
    if (plan->packed_bytes == 0)
        return fail(CONV_ERR_UNSUPPORTED, "prepacked chain: needs C1 at most %d (C1 = %lld)", ChainPackedShape::C1MAX,
                    (long long)plan->first.C);
    if (!packed) return fail(CONV_ERR_INVALID_ARG, "packed is NULL");
    if (plan->y_elems == 0) return CONV_OK;
    if (!x || !y) return fail(CONV_ERR_INVALID_ARG, "x or y is NULL");
    if (((uintptr_t)x | (uintptr_t)packed | (uintptr_t)y) & 15u)
        return fail(CONV_ERR_INVALID_ARG, "x, packed and y must be 16-byte aligned");
    if (((uintptr_t)b1 | (uintptr_t)b2) & 1u) return fail(CONV_ERR_INVALID_ARG, "b1 and b2 must be 2-byte aligned");
    const int64_t yb = plan->y_elems * 2;
    if (overlaps(y, yb, x, plan->x_elems * 2) || overlaps(y, yb, packed, plan->packed_bytes) ||
        overlaps(y, yb, b1, plan->b_elems * 2) || overlaps(y, yb, b2, plan->b_elems * 2))
        return fail(CONV_ERR_INVALID_ARG, "y overlaps an input");
    ChainPackedParams pp = plan->pp;
    pp.x = x; pp.packed = packed; pp.b1 = b1; pp.b2 = b2; pp.y = y;
    (void)hipGetLastError();
    const dim3 g(plan->pgrid), blk(256);
    hipStream_t s = (hipStream_t)stream;
    hipEvent_t e0 = (hipEvent_t)start_event, e1 = (hipEvent_t)stop_event;
    if (hb && plan->first.gelu)
        hipExtLaunchKernelGGL((chain_packed_kernel<true, true>), g, blk, 0, s, e0, e1, 0, pp);
    else if (hb)
        hipExtLaunchKernelGGL((chain_packed_kernel<true, false>), g, blk, 0, s, e0, e1, 0, pp);
    else if (plan->first.gelu)
        hipExtLaunchKernelGGL((chain_packed_kernel<false, true>), g, blk, 0, s, e0, e1, 0, pp);
    else
        hipExtLaunchKernelGGL((chain_packed_kernel<false, false>), g, blk, 0, s, e0, e1, 0, pp);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(CONV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return CONV_OK;
}

conv_status_t conv_chain_run_packed(const conv_chain_plan_t *plan, const void *x, const void *packed, const void *b1,
                                    const void *b2, void *y, void *stream)
{
    return conv_chain_run_packed_events(plan, x, packed, b1, b2, y, stream, nullptr, nullptr);
}

conv_status_t conv_chain_out_dims(const conv_chain_plan_t *plan, int64_t out[3])
{
    if (!plan || !out) return fail(CONV_ERR_INVALID_ARG, "NULL argument");
    for (int i = 0; i < 3; ++i) out[i] = plan->out2[i];
    return CONV_OK;
}

conv_status_t conv_chain_useful_flop(const conv_chain_plan_t *plan, int64_t *flop)
{
    if (!plan || !flop) return fail(CONV_ERR_INVALID_ARG, "NULL argument");
    const conv_fwd_desc_t &a = plan->first, &b = plan->second;
    *flop = 2 * a.N * a.K * a.C * a.filt[2] * plan->out1[2] + 2 * b.N * b.K * b.C * b.filt[2] * plan->out2[2];
    return CONV_OK;
}

void conv_chain_destroy(conv_chain_plan_t *plan) { delete plan; }

// ---- Backward-data ---------------------------------------------------------
// The stride phases of a 1-D strided input gradient (see bwd_kernels.h):
// builds pl->phase[] and pl->pwp and returns true, or returns false (and
// leaves nothing allocated) where the rewrite does not apply: more than one
// spatial dimension, a stride beyond kMaxPhases, a phase without taps, rows
// of dx that a fixed pitch cannot address (N > 1 with the length not a
// multiple of the stride), a group row of dx that is not a whole number of
// 16-byte vectors, or a phase convolution a plan cannot be made for.
static bool make_phases(const conv_fwd_desc_t &d, const int64_t o[3], conv_bwd_data_plan *pl)
{
    const int64_t esz = d.dtype == CONV_DT_BF16 ? 2 : 4;
    const int64_t s = d.stride[2], F = d.filt[2], dl = d.dilation[2], p = d.pad[2], L = d.in[2], Lo = o[2];
    if (d.in[0] != 1 || d.in[1] != 1 || d.filt[0] != 1 || d.filt[1] != 1 || d.stride[0] != 1 || d.stride[1] != 1 ||
        d.pad[0] != 0 || d.pad[1] != 0 || s < 2 || s > kMaxPhases || L < s)
        return false;
    if (d.N != 1 && L % s != 0) return false;
    if ((d.G * d.C * esz) % 16 != 0) return false;
    int64_t g = s, b = dl;
    while (b) { const int64_t r = g % b; g = b; b = r; }
    const int64_t dt = s / g, dp = dl / g;
    PhaseWeightParams &q = pl->pwp;
    q.G = (int)d.G; q.K = (int)d.K; q.C = (int)d.C; q.X = (int)F;
    q.nphase = (int)s; q.dt = (int)dt;
    int64_t base = 0;
    conv_fwd_plan_t *ph[kMaxPhases] = {};
    auto drop = [&]() {
        for (int f = 0; f < kMaxPhases; ++f) conv_fwd_destroy(ph[f]);
        g_err[0] = 0;   // a phase that could not be planned is not the caller's error
        return false;
    };
    for (int f = 0; f < s; ++f) {
        int64_t tmax = -1;
        for (int64_t t = F - 1; t >= 0 && tmax < 0; --t)
            if (((f + p - t * dl) % s + s) % s == 0) tmax = t;
        if (tmax < 0) return drop();
        const int64_t ntap = tmax / dt + 1;
        const int64_t e0 = (f + p - tmax * dl) / s;   // dy offset of the first (largest) tap; exact
        const int64_t J = (L - f + s - 1) / s;          // dx positions s j + f < L
        conv_fwd_desc_t fd = d;                          // dx_f = conv(dy, w_f): K input, C output channels
        fd.C = d.K;
        fd.K = d.C;
        fd.in[2] = Lo;
        fd.filt[2] = ntap;
        fd.stride[2] = 1;
        fd.pad[2] = 0;
        fd.dilation[2] = dp;
        fd.has_bias = 0;
        fd.gelu = 0;
        if (create_impl(&fd, -1, &ph[f]) != CONV_OK) return drop();
        conv_fwd_plan *pp = ph[f];
        // output row j reads dy[j + e0 + u dp]: left pad -e0 (may be
        // negative), J rows, each pitch s G C elements from the last
        KParams &kp = pp->kp;
        const TileCfg &c = kCfgs[pp->cfg];
        kp.pw = (int)(-e0);
        kp.Wo = (int)J;
        kp.M = (int)(d.N * J);
        kp.tiles_m = (kp.M + c.BM - 1) / c.BM;
        kp.fd_Wo = make_fastdiv(kp.Wo);
        kp.fd_tm = make_fastdiv(kp.tiles_m);
        kp.ldy = (int)(s * d.G * d.C);
        pp->out[2] = J;
        pp->y_elems = (d.N * L - f) * d.G * d.C;   // the span from the phase's first row to the end of dx
        pp->grid = (int)tiles_of(c, fd, pp->out);
        delete pp->packed_plan;                    // the phases run from the natural layout
        pp->packed_plan = nullptr;
        const size_t n = strlen(pp->text);
        snprintf(pp->text + n, sizeof(pp->text) - n, " [phase %d: taps %lld, dy offset %lld, %lld rows]", f,
                 (long long)ntap, (long long)e0, (long long)J);
        q.ntap[f] = (int)ntap;
        q.tmax[f] = (int)tmax;
        q.base[f] = base;
        base += ((d.G * d.C * ntap * d.K * esz + 255) / 256 * 256) / esz;
    }
    q.base[s] = base;
    for (int f = 0; f < kMaxPhases; ++f) pl->phase[f] = ph[f];
    pl->nphase = (int)s;
    return true;
}

conv_status_t conv_bwd_data_create(const conv_fwd_desc_t *desc, conv_bwd_data_plan_t **plan)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    *plan = nullptr;
    int64_t o[3];
    conv_status_t st = validate(desc, o);
    if (st != CONV_OK) return st;
    const conv_fwd_desc_t &d = *desc;
    if (d.has_bias || d.gelu)
        return fail(CONV_ERR_UNSUPPORTED, "backward of the linear convolution only: has_bias and gelu must be 0");
    const int64_t esz = d.dtype == CONV_DT_BF16 ? 2 : 4;
    conv_bwd_data_plan *pl = new (std::nothrow) conv_bwd_data_plan();
    if (!pl) return fail(CONV_ERR_NOMEM, "plan allocation failed");
    pl->desc = d;
    bool unit = true;
    int64_t off[3], P[3];
    for (int i = 0; i < 3; ++i) {
        off[i] = d.dilation[i] * (d.filt[i] - 1) - d.pad[i];
        P[i] = d.in[i] + d.dilation[i] * (d.filt[i] - 1);
        unit = unit && d.stride[i] == 1 && off[i] >= 0;
    }
    pl->spread = !unit;
    if (!unit && make_phases(d, o, pl)) {
        pl->spread = false;
        pl->fwd = nullptr;
        pl->dy_elems = d.N * o[0] * o[1] * o[2] * d.G * d.K;
        pl->w_elems = d.G * d.K * d.filt[0] * d.filt[1] * d.filt[2] * d.C;
        pl->dx_elems = d.N * d.in[0] * d.in[1] * d.in[2] * d.G * d.C;
        pl->ws_wt = pl->pwp.base[pl->nphase] * esz;
        pl->ws_dyp = 0;
        pl->ws_bytes = pl->ws_wt;
        int n = snprintf(pl->text, sizeof(pl->text), "bwd_data %s via %d stride phases of dy:",
                         d.dtype == CONV_DT_BF16 ? "bf16" : "f32", pl->nphase);
        for (int f = 0; f < pl->nphase && n < (int)sizeof(pl->text); ++f)
            n += snprintf(pl->text + n, sizeof(pl->text) - n, " %s;", conv_fwd_describe(pl->phase[f]));
        if (getenv("CONVFWD_LOG")) fprintf(stderr, "convfwd: %s\n", pl->text);
        *plan = pl;
        return CONV_OK;
    }
    conv_fwd_desc_t f = d;   // dx = conv(dyp, w'): K input channels, C output channels
    f.C = d.K;
    f.K = d.C;
    for (int i = 0; i < 3; ++i) {
        f.stride[i] = 1;
        f.in[i] = unit ? o[i] : P[i];
        f.pad[i] = unit ? off[i] : 0;
    }
    st = conv_fwd_create(&f, &pl->fwd);
    if (st != CONV_OK) {
        delete pl;
        return st;
    }
    int64_t fo[3];
    conv_fwd_out_dims(pl->fwd, fo);
    if (fo[0] != d.in[0] || fo[1] != d.in[1] || fo[2] != d.in[2]) {   // cannot happen: extents of the rewrite
        conv_fwd_destroy(pl->fwd);
        delete pl;
        return fail(CONV_ERR_HIP, "internal: backward-data rewrite has the wrong extent");
    }
    pl->dy_elems = d.N * o[0] * o[1] * o[2] * d.G * d.K;
    pl->w_elems = d.G * d.K * d.filt[0] * d.filt[1] * d.filt[2] * d.C;
    pl->dx_elems = d.N * d.in[0] * d.in[1] * d.in[2] * d.G * d.C;
    pl->ws_wt = (pl->w_elems * esz + 255) / 256 * 256;
    pl->ws_dyp = 0;
    if (pl->spread) {
        const double dyp = (double)d.N * P[0] * P[1] * P[2] * d.G * d.K;
        if (dyp * esz >= 2147483647.0) {
            conv_fwd_destroy(pl->fwd);
            delete pl;
            return fail(CONV_ERR_UNSUPPORTED, "backward-data: the spread copy of dy would be 2 GiB or more");
        }
        pl->ws_dyp = (int64_t)dyp * esz;
        SpreadParams &sp = pl->sp;
        sp.N = (int)d.N;
        sp.G = (int)d.G;
        sp.KB = (int)(d.K * esz);
        for (int i = 0; i < 3; ++i) {
            sp.O[i] = (int)o[i];
            sp.P[i] = (int)P[i];
            sp.s[i] = (int)d.stride[i];
            sp.off[i] = (int)off[i];
        }
    }
    pl->ws_bytes = pl->ws_wt + pl->ws_dyp;
    snprintf(pl->text, sizeof(pl->text), "bwd_data %s via %s: %s", d.dtype == CONV_DT_BF16 ? "bf16" : "f32",
             pl->spread ? "spread dy + flipped weights" : "padded dy + flipped weights", conv_fwd_describe(pl->fwd));
    if (getenv("CONVFWD_LOG")) fprintf(stderr, "convfwd: %s\n", pl->text);
    *plan = pl;
    return CONV_OK;
}

conv_status_t conv_bwd_data_workspace_bytes(const conv_bwd_data_plan_t *plan, int64_t *bytes)
{
    if (!plan || !bytes) return fail(CONV_ERR_INVALID_ARG, "plan or bytes is NULL");
    *bytes = plan->ws_bytes;
    return CONV_OK;
}

conv_status_t conv_bwd_data_run(const conv_bwd_data_plan_t *plan, const void *dy, const void *w, void *dx,
                                void *workspace, int64_t workspace_bytes, void *stream)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    if (!w) return fail(CONV_ERR_INVALID_ARG, "w is NULL");
    if (plan->dx_elems == 0) return CONV_OK;
    if (!dy || !dx || !workspace) return fail(CONV_ERR_INVALID_ARG, "dy, dx or workspace is NULL");
    if (workspace_bytes < plan->ws_bytes)
        return fail(CONV_ERR_INVALID_ARG, "workspace has %lld bytes, the plan needs %lld", (long long)workspace_bytes,
                    (long long)plan->ws_bytes);
    if (((uintptr_t)dy | (uintptr_t)w | (uintptr_t)dx | (uintptr_t)workspace) & 15u)
        return fail(CONV_ERR_INVALID_ARG, "dy, w, dx and workspace must be 16-byte aligned");
    const int64_t esz = plan->desc.dtype == CONV_DT_BF16 ? 2 : 4;
    const int64_t dxb = plan->dx_elems * esz;
    if (overlaps(dx, dxb, dy, plan->dy_elems * esz) || overlaps(dx, dxb, w, plan->w_elems * esz) ||
        overlaps(dx, dxb, workspace, plan->ws_bytes))
        return fail(CONV_ERR_INVALID_ARG, "dx overlaps dy, w or the workspace");
    if (overlaps(workspace, plan->ws_bytes, dy, plan->dy_elems * esz) ||
        overlaps(workspace, plan->ws_bytes, w, plan->w_elems * esz))
        return fail(CONV_ERR_INVALID_ARG, "the workspace overlaps dy or w");
    const conv_fwd_desc_t &d = plan->desc;
    hipStream_t s = (hipStream_t)stream;
    unsigned char *ws = reinterpret_cast<unsigned char *>(workspace);
    (void)hipGetLastError();
    if (plan->nphase > 0) {   // the phases' filters, then one forward conv of dy per phase
        const PhaseWeightParams &q = plan->pwp;
        const dim3 pg((unsigned)((q.base[q.nphase] + 255) / 256));
        if (d.dtype == CONV_DT_BF16)
            hipLaunchKernelGGL(bwd_data_phase_weights_kernel<uint16_t>, pg, dim3(256), 0, s, (const uint16_t *)w,
                               (uint16_t *)ws, q);
        else
            hipLaunchKernelGGL(bwd_data_phase_weights_kernel<float>, pg, dim3(256), 0, s, (const float *)w,
                               (float *)ws, q);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return fail(CONV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
        for (int f = 0; f < plan->nphase; ++f) {
            const conv_status_t st = conv_fwd_run(plan->phase[f], dy, ws + q.base[f] * esz, nullptr,
                                                  reinterpret_cast<unsigned char *>(dx) + f * d.G * d.C * esz, stream);
            if (st != CONV_OK) return st;
        }
        return CONV_OK;
    }
    const int64_t wb = (plan->w_elems + 255) / 256;
    if (d.dtype == CONV_DT_BF16)
        hipLaunchKernelGGL(bwd_data_weights_kernel<uint16_t>, dim3((unsigned)wb), dim3(256), 0, s,
                           (const uint16_t *)w, (uint16_t *)ws, (int)d.K, (int)d.C, (int)d.filt[0], (int)d.filt[1],
                           (int)d.filt[2], plan->w_elems);
    else
        hipLaunchKernelGGL(bwd_data_weights_kernel<float>, dim3((unsigned)wb), dim3(256), 0, s, (const float *)w,
                           (float *)ws, (int)d.K, (int)d.C, (int)d.filt[0], (int)d.filt[1], (int)d.filt[2],
                           plan->w_elems);
    const void *src = dy;
    if (plan->spread) {
        SpreadParams sp = plan->sp;
        sp.dy = dy;
        sp.dyp = ws + plan->ws_wt;
        const int vb = sp.KB % 16 == 0 ? 16 : sp.KB % 4 == 0 ? 4 : 2;
        sp.total = plan->ws_dyp / vb;
        const dim3 g((unsigned)((sp.total + 255) / 256));
        if (vb == 16)
            hipLaunchKernelGGL(bwd_data_spread_kernel<uint4>, g, dim3(256), 0, s, sp);
        else if (vb == 4)
            hipLaunchKernelGGL(bwd_data_spread_kernel<uint32_t>, g, dim3(256), 0, s, sp);
        else
            hipLaunchKernelGGL(bwd_data_spread_kernel<uint16_t>, g, dim3(256), 0, s, sp);
        src = sp.dyp;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(CONV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return conv_fwd_run(plan->fwd, src, ws, nullptr, dx, stream);
}

conv_status_t conv_bwd_data_run_noalloc(const conv_bwd_data_plan_t *plan, const void *dy, const void *w, void *dx,
                                        void *stream)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    if (plan->ws_bytes > (int64_t)CONV_BWD_DATA_SCRATCH_BYTES)
        return fail(CONV_ERR_UNSUPPORTED,
                    "backward-data needs %lld bytes of workspace; the allocation-free entry point holds %lld",
                    (long long)plan->ws_bytes, (long long)CONV_BWD_DATA_SCRATCH_BYTES);
    if (plan->dx_elems == 0) return conv_bwd_data_run(plan, dy, w, dx, nullptr, 0, stream);
    void *ws = nullptr;
    conv_status_t st = scratch_of_current_device(&ws);
    if (st != CONV_OK) return st;
    return conv_bwd_data_run(plan, dy, w, dx, ws, (int64_t)CONV_BWD_DATA_SCRATCH_BYTES, stream);
}

void conv_bwd_data_destroy(conv_bwd_data_plan_t *plan)
{
    if (!plan) return;
    conv_fwd_destroy(plan->fwd);
    for (int f = 0; f < kMaxPhases; ++f) conv_fwd_destroy(plan->phase[f]);
    delete plan;
}

const char *conv_bwd_data_describe(const conv_bwd_data_plan_t *plan) { return plan ? plan->text : ""; }

// ---- Backward-weight ---------------------------------------------------------
conv_status_t conv_bwd_weight_create(const conv_fwd_desc_t *desc, conv_bwd_weight_plan_t **plan)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    *plan = nullptr;
    int64_t o[3];
    conv_status_t st = validate(desc, o);
    if (st != CONV_OK) return st;
    const conv_fwd_desc_t &d = *desc;
    if (d.has_bias || d.gelu)
        return fail(CONV_ERR_UNSUPPORTED, "backward of the linear convolution only: has_bias and gelu must be 0");
    if (d.dtype != CONV_DT_BF16) return fail(CONV_ERR_UNSUPPORTED, "backward-weight: bf16 only");
    if (d.C % 8 != 0 || d.K % 8 != 0)
        return fail(CONV_ERR_UNSUPPORTED, "backward-weight: C and K per group must be multiples of 8 (C = %lld, K = %lld)",
                    (long long)d.C, (long long)d.K);
    conv_bwd_weight_plan *pl = new (std::nothrow) conv_bwd_weight_plan();
    if (!pl) return fail(CONV_ERR_NOMEM, "plan allocation failed");
    pl->desc = d;
    const int taps = (int)(d.filt[0] * d.filt[1] * d.filt[2]);
    pl->KT = std::min(d.K, d.C) > 32 ? 64 : 32;
    const int tmax = pl->KT == 64 ? 9 : 27;     // 32x32 blocks per workgroup <= 36
    pl->TT = 1;
    for (int tt : {27, 9, 3})
        if (tt <= tmax && taps % tt == 0) { pl->TT = tt; break; }
    WgradParams &wp = pl->wp;
    wp.N = (int)d.N; wp.G = (int)d.G; wp.C = (int)d.C; wp.K = (int)d.K;
    wp.Di = (int)d.in[0]; wp.Hi = (int)d.in[1]; wp.Wi = (int)d.in[2];
    wp.Do = (int)o[0]; wp.Ho = (int)o[1]; wp.Wo = (int)o[2];
    wp.sd = (int)d.stride[0]; wp.sh = (int)d.stride[1]; wp.sw = (int)d.stride[2];
    wp.pd = (int)d.pad[0]; wp.ph = (int)d.pad[1]; wp.pw = (int)d.pad[2];
    wp.dd = (int)d.dilation[0]; wp.dh = (int)d.dilation[1]; wp.dw = (int)d.dilation[2];
    wp.Y = (int)d.filt[1]; wp.X = (int)d.filt[2]; wp.taps = taps;
    wp.pixels = d.N * o[0] * o[1] * o[2];
    wp.fd_Wo = make_fastdiv(wp.Wo); wp.fd_Ho = make_fastdiv(wp.Ho); wp.fd_Do = make_fastdiv(wp.Do);
    wp.kt_n = (int)((d.K + pl->KT - 1) / pl->KT);
    wp.ct_n = (int)((d.C + pl->KT - 1) / pl->KT);
    wp.tg_n = taps / pl->TT;
    const int64_t tiles = d.G * wp.kt_n * wp.ct_n * wp.tg_n;
    const int64_t steps = (wp.pixels + 31) / 32;
    // Split the pixels so that all workgroups run in one round (as many as
    // the CUs hold at once: one for the large tiles, several for the small
    // ones) and each has at least 8 steps: every split writes a whole fp32
    // partial tile that the reduction reads back, so more splits than the
    // CUs can run at once only add traffic (at 112 splits of the grouped 2-D
    // workload the reduction took a third of the time).
    // Eight waves for the tiles with many 32x32 output blocks (64 channels x
    // 9 taps: 36, 32 x 27: 27): two waves per SIMD overlap each other's
    // staging and products (grouped 2-D workload +11%, 3-D +3%, same box);
    // with fewer blocks (64 x 3 taps: 12) a quarter of eight waves' block
    // slots would idle and four waves are faster (batch-32 frontend: 271 vs
    // 237 TFLOP/s).
    const bool eight = (pl->KT == 64 && pl->TT == 9) || (pl->KT == 32 && pl->TT == 27);
    pl->NWV = eight ? 8 : 4;
    int occ = 1;
    if (eight) {
        occ = pl->KT == 64 ? wgrad_occupancy<64, 9, 8>() : wgrad_occupancy<32, 27, 8>();
    } else {
        if (pl->KT == 64) occ = pl->TT == 9 ? wgrad_occupancy<64, 9, 4>() : pl->TT == 3 ? wgrad_occupancy<64, 3, 4>()
                                                                                         : wgrad_occupancy<64, 1, 4>();
        else occ = pl->TT == 27 ? wgrad_occupancy<32, 27, 4>() : pl->TT == 9 ? wgrad_occupancy<32, 9, 4>()
                                : pl->TT == 3 ? wgrad_occupancy<32, 3, 4>() : wgrad_occupancy<32, 1, 4>();
    }
    pl->occ = occ;
    int64_t splits = std::max<int64_t>(1, (int64_t)device_cu_count() * occ / tiles);
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, steps / 8));
    const int64_t per = std::max<int64_t>(1, (steps + splits - 1) / splits);
    splits = std::max<int64_t>(1, (steps + per - 1) / per);
    wp.splits = (int)splits;
    wp.steps_per_split = (int)per;
    pl->x_elems = d.N * d.in[0] * d.in[1] * d.in[2] * d.G * d.C;
    pl->dy_elems = wp.pixels * d.G * d.K;
    pl->dw_elems = d.G * d.K * taps * d.C;
    const double grid = (double)tiles * splits;
    // x and dy are read through 32-bit byte offsets
    if (grid >= 2147483647.0 || (double)pl->dw_elems * splits >= 2147483647.0 * 4 ||
        pl->x_elems * 2 >= (int64_t(1) << 31) || pl->dy_elems * 2 >= (int64_t(1) << 31)) {
        delete pl;
        return fail(CONV_ERR_UNSUPPORTED, "backward-weight: problem too large");
    }
    pl->grid = (int)grid;
    pl->ws_bytes = pl->dw_elems * splits * 4;
    snprintf(pl->text, sizeof(pl->text),
             "bwd_weight bf16 tile %dx%d ch x %d taps, %d waves, %lld tiles x %d splits of %d x 32 pixels, "
             "grid=%d (%d per CU) lds=%dB",
             pl->KT, pl->KT, pl->TT, pl->NWV, (long long)tiles, wp.splits, wp.steps_per_split, pl->grid, pl->occ,
             pl->KT == 64 ? (64 + pl->TT * 64) * 72 : (32 + pl->TT * 32) * 72);
    if (getenv("CONVFWD_LOG")) fprintf(stderr, "convfwd: %s\n", pl->text);
    *plan = pl;
    return CONV_OK;
}

conv_status_t conv_bwd_weight_workspace_bytes(const conv_bwd_weight_plan_t *plan, int64_t *bytes)
{
    if (!plan || !bytes) return fail(CONV_ERR_INVALID_ARG, "plan or bytes is NULL");
    *bytes = plan->ws_bytes;
    return CONV_OK;
}

conv_status_t conv_bwd_weight_run(const conv_bwd_weight_plan_t *plan, const void *x, const void *dy, void *dw,
                                  void *workspace, int64_t workspace_bytes, void *stream)
{
    if (!plan) return fail(CONV_ERR_INVALID_ARG, "plan is NULL");
    if (!dw || !workspace) return fail(CONV_ERR_INVALID_ARG, "dw or workspace is NULL");
    if (plan->dy_elems > 0 && (!x || !dy)) return fail(CONV_ERR_INVALID_ARG, "x or dy is NULL");
    if (workspace_bytes < plan->ws_bytes)
        return fail(CONV_ERR_INVALID_ARG, "workspace has %lld bytes, the plan needs %lld", (long long)workspace_bytes,
                    (long long)plan->ws_bytes);
    if (((uintptr_t)x | (uintptr_t)dy | (uintptr_t)dw | (uintptr_t)workspace) & 15u)
        return fail(CONV_ERR_INVALID_ARG, "x, dy, dw and workspace must be 16-byte aligned");
    const int64_t dwb = plan->dw_elems * 2;
    if (overlaps(dw, dwb, x, plan->x_elems * 2) || overlaps(dw, dwb, dy, plan->dy_elems * 2) ||
        overlaps(dw, dwb, workspace, plan->ws_bytes))
        return fail(CONV_ERR_INVALID_ARG, "dw overlaps x, dy or the workspace");
    if (overlaps(workspace, plan->ws_bytes, x, plan->x_elems * 2) ||
        overlaps(workspace, plan->ws_bytes, dy, plan->dy_elems * 2))
        return fail(CONV_ERR_INVALID_ARG, "the workspace overlaps x or dy");
    WgradParams wp = plan->wp;
    wp.x = x;
    wp.dy = dy;
    wp.x_bytes = (uint32_t)(plan->x_elems * 2);
    wp.dy_bytes = (uint32_t)(plan->dy_elems * 2);
    wp.ws = reinterpret_cast<float *>(workspace);
    hipStream_t s = (hipStream_t)stream;
    (void)hipGetLastError();
    // No pixels (an empty batch): x and dy may be null, so the products are
    // skipped and the reduction over zero splits writes dw = 0.
    const bool empty = plan->dy_elems == 0;
    if (empty) {
    } else if (plan->NWV == 8) {
        if (plan->KT == 64) launch_wgrad<64, 9, 8>(wp, plan->grid, s);
        else launch_wgrad<32, 27, 8>(wp, plan->grid, s);
    } else if (plan->KT == 64) {
        if (plan->TT == 9) launch_wgrad<64, 9, 4>(wp, plan->grid, s);
        else if (plan->TT == 3) launch_wgrad<64, 3, 4>(wp, plan->grid, s);
        else launch_wgrad<64, 1, 4>(wp, plan->grid, s);
    } else {
        if (plan->TT == 27) launch_wgrad<32, 27, 4>(wp, plan->grid, s);
        else if (plan->TT == 9) launch_wgrad<32, 9, 4>(wp, plan->grid, s);
        else if (plan->TT == 3) launch_wgrad<32, 3, 4>(wp, plan->grid, s);
        else launch_wgrad<32, 1, 4>(wp, plan->grid, s);
    }
    const int64_t n = plan->dw_elems;   // a multiple of 8 (C % 8 == 0)
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)((n / 4 + 63) / 64)), dim3(64), 0, s,
                       (const float4 *)workspace, (uint2 *)dw, n / 4, empty ? 0 : wp.splits);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return fail(CONV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    return CONV_OK;
}

void conv_bwd_weight_destroy(conv_bwd_weight_plan_t *plan) { delete plan; }

const char *conv_bwd_weight_describe(const conv_bwd_weight_plan_t *plan) { return plan ? plan->text : ""; }

const char *conv_chain_describe(const conv_chain_plan_t *plan) { return plan ? plan->text : ""; }

}  // extern "C"
