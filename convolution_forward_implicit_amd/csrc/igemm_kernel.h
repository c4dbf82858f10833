// Implicit-GEMM forward convolution kernel for gfx950 (CDNA4).
//
// Per group g the convolution is the GEMM
//   Y_g[m, n] = sum_r A_g[m, r] * B_g[n, r]
//   m = ((batch*Do + od)*Ho + oh)*Wo + ow          (GEMM rows; the batch is
//                                                  folded into M, so a batch-1
//                                                  problem leaves no lane idle)
//   n = output channel k                            (GEMM columns)
//   r = ((z*Y + y)*X + x)*C + c                     (reduction)
//   A_g[m, r] = x[batch, od*sd-pd+z*dd, oh*sh-ph+y*dh, ow*sw-pw+x*dw, g, c]
//               (0 where that position is padding)
//   B_g[n, r] = w[g, n, z, y, x, c]                 (contiguous in r)
// which is the im2col + GEMM lowering of the ExecuTorch conv1d issue
// ("The conv2d path already solves this": conv2d_im2col + conv2d_gemm),
// except that the im2col matrix is never written: each K-step gathers its
// BM x BK slice of A straight from the channels-innermost input into LDS.
//
// One workgroup computes a BM x BN tile of Y_g with WM x WN waves; each wave
// owns a (BM/WM) x (BN/WN) sub-tile made of 16x16 MFMA blocks held in fp32
// accumulators.  Global loads are 16-byte vectors along the channel axis (a
// vector never crosses a filter tap because the host only picks VEC > 1 when
// C % VEC == 0); the next K-step's loads are in flight while the current one
// is multiplied (register prefetch + two LDS stages, one barrier per step).
// The epilogue adds the bias, applies erf-GELU in fp32, rounds to the output
// type, stages the tile in LDS and writes whole 16-byte vectors along K, so
// every output row segment of a workgroup leaves in full lines.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convfwd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;

// Output stores carry the non-temporal hint.  A kernel writes each output
// once and never reads it back; streamed stores leave the L2 to the input
// rows and weights that the workgroups re-read.  Same-box A/B on MI355X
// (medians of 64 cold launches): batch-32 frontend layers 46 -> 40 and
// 55 -> 50 us, grouped 2-D 17.1 -> 14.2 us, grouped 3-D 18.3 -> 17.1 us;
// the batch-1 layers, whose outputs are a few MB, within noise.
__device__ __forceinline__ void store_nt16(void *dst, uint4 v)
{
    __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t *>(dst));
}

// Division by a divisor fixed at plan time: n / d = (umulhi(n, m) + n) >> s
// for 0 <= n < 2^31, with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994).  The host fills m and s.
struct FastDiv {
    uint32_t m, s, d;
};

__device__ __forceinline__ int fdiv(int n, FastDiv f)
{
    return (int)((__umulhi((uint32_t)n, f.m) + (uint32_t)n) >> f.s);
}

struct KParams {
    const void *x;
    const void *w;
    const void *bias;   // nullptr when there is no bias
    void *y;
    int N, G, C, K;
    int Di, Hi, Wi;
    int Z, Y, X;
    int sd, sh, sw;
    int pd, ph, pw;
    int dd, dh, dw;
    int Do, Ho, Wo;
    int M;              // N*Do*Ho*Wo
    int Kred;           // Z*Y*X*C
    int tiles_m;        // ceil(M / BM)
    int tiles_n;        // ceil(K / BN)
    int gelu;
    int out_vec;        // K % (16 / sizeof(out)) == 0: whole-vector stores
    int wpacked;        // w is the plan's prepacked weight image (direct-to-LDS and
                        // fixed-filter patch kernels), not GKZYXC
    FastDiv fd_Wo, fd_Ho, fd_Do, fd_C, fd_X, fd_Y;
    FastDiv fd_tn, fd_tm;   // tiles_n, tiles_m
    int ldy;            // elements from one output pixel's row to the next: G*K, or more when
                        // the output is every s-th pixel of a larger tensor (a stride phase of
                        // the input gradient)
};

template <int BYTES> struct RawVec;
template <> struct RawVec<16> { using type = uint4; };
template <> struct RawVec<4>  { using type = uint32_t; };
template <> struct RawVec<2>  { using type = uint16_t; };

template <int DT> struct Elem;
template <> struct Elem<0> { using type = float; };      // fp32
template <> struct Elem<1> { using type = uint16_t; };   // bf16 bit pattern

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float(((uint32_t)h) << 16);
}

// IEEE round-to-nearest-even float32 -> bfloat16 (NaN stays NaN).  On
// gfx950 the conversion is the hardware v_cvt_pk_bf16_f32, which rounds to
// nearest-even in the default rounding mode.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two values at once: low half = a, high half = b.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b)
{
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// Exact GELU, t * Phi(t), branch-free and short (the epilogue of a
// thin-reduction conv is bound by it).  With a = |t|: Phi(-a) = 2^R(a), R
// the degree-7 least-squares fit of log2 Phi(-a) on [0, 6] at Chebyshev
// nodes, within 5.7e-6 (so Phi(-a) within 4e-6 relative); one exp2, seven
// FMAs, no reciprocal.  R is not clamped: past 6 it keeps decreasing, below
// the fit's value at 6 (log2 Phi(-6) = -29.9) for every larger a and to
// -inf for huge ones, so Phi(-a) only shrinks towards 0 there (checked
// against its extrapolation on the CPU).  The result is t times Phi(t) =
// 1 - Phi(-|t|) for t >= +0 and Phi(-|t|) for t <= -0, the choice made from
// t's sign bit by a bit-field select (no compare, so no condition-register
// hazard): neither form cancels.  NaN propagates, +inf maps to +inf and
// -inf to NaN (-inf times Phi(-inf) = 0, as t/2 * erfc(-t/sqrt 2) gives).
__device__ __forceinline__ float gelu_erf(float v)
{
    const float a = fabsf(v);
    float r = -1.889570263e-06f;
    r = fmaf(r, a, 6.268018558e-05f);
    r = fmaf(r, a, -9.388573895e-04f);
    r = fmaf(r, a, 8.539414817e-03f);
    r = fmaf(r, a, -5.402057739e-02f);
    r = fmaf(r, a, -4.584099095e-01f);
    r = fmaf(r, a, -1.151269077e+00f);
    r = fmaf(r, a, -9.999943512e-01f);
    const float p = __builtin_amdgcn_exp2f(r);                                   // Phi(-|v|)
    const uint32_t neg = (uint32_t)((int32_t)__float_as_uint(v) >> 31);          // all ones iff sign set
    const uint32_t q = (neg & __float_as_uint(p)) | (~neg & __float_as_uint(1.0f - p));
    return v * __uint_as_float(q);
}

// GELU for results that are then rounded to bfloat16 (8 significant bits).
// Same t * Phi(t), cut to the output's precision: R is the degree-5
// least-squares fit of log2 Phi(-a) on [0, 6] at Chebyshev nodes, within
// 5.9e-4 (Phi(-a) within 4.1e-4 relative, a tenth of the output's rounding
// step), again unclamped (below -29.9 and decreasing past 6), and t * Phi(t)
// is formed as t/2 + |t| (1/2 - Phi(-|t|)), one fused multiply-add with no
// sign test.  Four vector operations fewer per value than gelu_erf.  For
// t < 0 the two terms nearly cancel, so the rounding of 1/2 - Phi(-|t|)
// leaves an absolute error up to 2^-25 |t|: half an fp32 rounding of t
// itself, inside the error that the fp32 sum producing t already carries.
// NaN propagates, +inf maps to +inf, -inf to NaN (as t/2 * erfc(-t/sqrt 2)
// does).
__device__ __forceinline__ float gelu_erf_bf16out(float v)
{
    const float a = fabsf(v);
    float r = -1.975036866e-04f;
    r = fmaf(r, a, 4.405779764e-03f);
    r = fmaf(r, a, -4.251449928e-02f);
    r = fmaf(r, a, -4.734477997e-01f);
    r = fmaf(r, a, -1.143927097e+00f);
    r = fmaf(r, a, -1.000582814e+00f);
    const float h = 0.5f - __builtin_amdgcn_exp2f(r);   // 1/2 - Phi(-|v|)
    return fmaf(fabsf(v), h, 0.5f * v);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float v) { return f32_to_bf16(v); }

template <int DT, int BM, int BN, int BK, int WM, int WN, int VEC>
struct IgemmShape {
    using T = typename Elem<DT>::type;
    static constexpr int NT = WM * WN * 64;
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int PAD = 16 / ESZ;        // 16-byte row pad: conflict-free b128 reads
    static constexpr int LDK = BK + PAD;        // LDS row stride of the A/B stages (elements)
    static constexpr int TM = BM / WM;          // wave sub-tile
    static constexpr int TN = BN / WN;
    static constexpr int MI = TM / 16;          // 16x16 MFMA blocks per wave
    static constexpr int NI = TN / 16;
    static constexpr int KSTEP = DT == 1 ? 32 : 16;  // K consumed per LDS fragment read
    static constexpr int VPR = BK / VEC;        // load vectors per tile row
    static constexpr int RPP = NT / VPR;        // tile rows covered per load pass
    static constexpr int A_PASSES = (BM + RPP - 1) / RPP;
    static constexpr int B_PASSES = (BN + RPP - 1) / RPP;
    static constexpr int OV = 16 / ESZ;         // output elements per 16-byte store
    static constexpr int LDC = BN + OV;         // LDS row stride of the output tile
    static constexpr int STAGE = (BM + BN) * LDK * ESZ;
    static constexpr int EPI = BM * LDC * ESZ;
    static constexpr int LDS_BYTES = (2 * STAGE > EPI) ? 2 * STAGE : EPI;

    static_assert(BM % (WM * 16) == 0 && BN % (WN * 16) == 0, "wave tile must be 16-aligned");
    static_assert(BK % KSTEP == 0, "BK must be a multiple of the MFMA K step");
    static_assert(BK % VEC == 0 && NT % VPR == 0, "load mapping");
    static_assert(BN % OV == 0, "output vector mapping");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one CU");
};

template <int DT, int BM, int BN, int BK, int WM, int WN, int VEC>
__global__ void __launch_bounds__(WM * WN * 64)
igemm_fwd_kernel(KParams p)
{
    using S = IgemmShape<DT, BM, BN, BK, WM, WN, VEC>;
    using T = typename S::T;
    using V = typename RawVec<VEC * S::ESZ>::type;

    __shared__ __attribute__((aligned(16))) unsigned char smem[S::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave % WN;

    // workgroup -> (m tile, n tile, group)
    int bid = blockIdx.x;
    const int m_tile = bid % p.tiles_m;
    bid /= p.tiles_m;
    const int n_tile = bid % p.tiles_n;
    const int g = bid / p.tiles_n;
    const int m0 = m_tile * BM;
    const int n0 = n_tile * BN;

    const int GC = p.G * p.C;
    const T *__restrict__ xg = reinterpret_cast<const T *>(p.x) + g * p.C;
    const T *__restrict__ wg = reinterpret_cast<const T *>(p.w) + (size_t)g * p.K * p.Kred;

    // ---- per-thread load coordinates -------------------------------------
    const int vcol = tid % S::VPR;            // vector column inside the BK slice
    const int row0 = tid / S::VPR;            // first tile row this thread loads

    int a_off[S::A_PASSES];                   // x offset of (batch, bd, bh, bw), channel 0
    int a_bd[S::A_PASSES], a_bh[S::A_PASSES], a_bw[S::A_PASSES];
#pragma unroll
    for (int i = 0; i < S::A_PASSES; ++i) {
        const int m = m0 + row0 + i * S::RPP;
        int bd = -(1 << 28), bh = 0, bw = 0, off = 0;  // rows past M never pass the bounds test
        if (row0 + i * S::RPP < BM && m < p.M) {
            int t = m;
            const int ow = t % p.Wo; t /= p.Wo;
            const int oh = t % p.Ho; t /= p.Ho;
            const int od = t % p.Do;
            const int nb = t / p.Do;
            bd = od * p.sd - p.pd;
            bh = oh * p.sh - p.ph;
            bw = ow * p.sw - p.pw;
            off = (((nb * p.Di + bd) * p.Hi + bh) * p.Wi + bw) * GC;
        }
        a_off[i] = off; a_bd[i] = bd; a_bh[i] = bh; a_bw[i] = bw;
    }

    V areg[S::A_PASSES];
    V breg[S::B_PASSES];

    auto load_tile = [&](int k0) {
        const int r = k0 + vcol * VEC;
        const bool rok = r < p.Kred;
        int tap = r / p.C;
        const int c = r - tap * p.C;
        const int xk = tap % p.X; tap /= p.X;
        const int yk = tap % p.Y;
        const int zk = tap / p.Y;
        const int zd = zk * p.dd, yh = yk * p.dh, xw = xk * p.dw;
        const int tap_off = ((zd * p.Hi + yh) * p.Wi + xw) * GC + c;
#pragma unroll
        for (int i = 0; i < S::A_PASSES; ++i) {
            V v = {};
            const bool ok = rok && (unsigned)(a_bd[i] + zd) < (unsigned)p.Di &&
                            (unsigned)(a_bh[i] + yh) < (unsigned)p.Hi &&
                            (unsigned)(a_bw[i] + xw) < (unsigned)p.Wi;
            if (ok) v = *reinterpret_cast<const V *>(xg + a_off[i] + tap_off);
            areg[i] = v;
        }
#pragma unroll
        for (int j = 0; j < S::B_PASSES; ++j) {
            V v = {};
            const int row = row0 + j * S::RPP;
            const int n = n0 + row;
            if (row < BN && rok && n < p.K)
                v = *reinterpret_cast<const V *>(wg + (size_t)n * p.Kred + r);
            breg[j] = v;
        }
    };

    auto store_tile = [&](int stage) {
        T *As = reinterpret_cast<T *>(smem + stage * S::STAGE);
        T *Bs = As + BM * S::LDK;
#pragma unroll
        for (int i = 0; i < S::A_PASSES; ++i) {
            const int row = row0 + i * S::RPP;
            if (row < BM) *reinterpret_cast<V *>(As + row * S::LDK + vcol * VEC) = areg[i];
        }
#pragma unroll
        for (int j = 0; j < S::B_PASSES; ++j) {
            const int row = row0 + j * S::RPP;
            if (row < BN) *reinterpret_cast<V *>(Bs + row * S::LDK + vcol * VEC) = breg[j];
        }
    };

    f32x4_t acc[S::MI][S::NI];
#pragma unroll
    for (int i = 0; i < S::MI; ++i)
#pragma unroll
        for (int j = 0; j < S::NI; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int frow = lane & 15;     // row of an A block / column of a B block
    const int fk = lane >> 4;       // which K slice of the fragment this lane feeds

    auto compute = [&](int stage) {
        const T *As = reinterpret_cast<const T *>(smem + stage * S::STAGE);
        const T *Bs = As + BM * S::LDK;
#pragma unroll
        for (int kk = 0; kk < BK; kk += S::KSTEP) {
            if constexpr (DT == 1) {
                // bf16: 16x16x32; lane feeds 8 consecutive k of row/col (lane & 15)
                bf16x8_t a[S::MI], b[S::NI];
#pragma unroll
                for (int i = 0; i < S::MI; ++i)
                    a[i] = *reinterpret_cast<const bf16x8_t *>(
                        As + (wm * S::TM + i * 16 + frow) * S::LDK + kk + fk * 8);
#pragma unroll
                for (int j = 0; j < S::NI; ++j)
                    b[j] = *reinterpret_cast<const bf16x8_t *>(
                        Bs + (wn * S::TN + j * 16 + frow) * S::LDK + kk + fk * 8);
#pragma unroll
                for (int i = 0; i < S::MI; ++i)
#pragma unroll
                    for (int j = 0; j < S::NI; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            } else {
                // fp32: four 16x16x4 MFMAs over 16 k.  Lane group fk reads k =
                // kk + 4*fk .. +3 once; MFMA e takes element e.  A and B use the
                // same k assignment, so the four products together cover
                // kk .. kk+15 exactly once.
                f32x4_t a[S::MI], b[S::NI];
#pragma unroll
                for (int i = 0; i < S::MI; ++i)
                    a[i] = *reinterpret_cast<const f32x4_t *>(
                        As + (wm * S::TM + i * 16 + frow) * S::LDK + kk + fk * 4);
#pragma unroll
                for (int j = 0; j < S::NI; ++j)
                    b[j] = *reinterpret_cast<const f32x4_t *>(
                        Bs + (wn * S::TN + j * 16 + frow) * S::LDK + kk + fk * 4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int i = 0; i < S::MI; ++i)
#pragma unroll
                        for (int j = 0; j < S::NI; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
            }
        }
    };

    // ---- main loop: prefetch step kt+1 while multiplying step kt ----------
    const int nk = (p.Kred + BK - 1) / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_tile((kt + 1) * BK);
        compute(cur);
        if (kt + 1 < nk) store_tile(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue: bias, GELU, round, stage in LDS, whole-vector stores ---
    float bias_v[S::NI];
    if (p.bias != nullptr) {
#pragma unroll
        for (int j = 0; j < S::NI; ++j) {
            // unconditional (clamped) loads, so they are all in flight at once
            const int n = n0 + wn * S::TN + j * 16 + frow;
            const float v = to_f32<T>(reinterpret_cast<const T *>(p.bias)[g * p.K + (n < p.K ? n : p.K - 1)]);
            bias_v[j] = n < p.K ? v : 0.f;
        }
    } else {
#pragma unroll
        for (int j = 0; j < S::NI; ++j) bias_v[j] = 0.f;
    }
    T *Cs = reinterpret_cast<T *>(smem);
#pragma unroll
    for (int i = 0; i < S::MI; ++i)
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // MFMA 16x16 result layout: lane holds rows 4*(lane>>4)+e of column lane&15
                const int ml = wm * S::TM + i * 16 + fk * 4 + e;
                const int nl = wn * S::TN + j * 16 + frow;
                float v = acc[i][j][e] + bias_v[j];
                if (p.gelu) v = gelu_erf(v);
                Cs[ml * S::LDC + nl] = from_f32<T>(v);
            }
    __syncthreads();

    T *__restrict__ yg = reinterpret_cast<T *>(p.y) + g * p.K;
    const int GK = p.ldy;
    constexpr int OVPR = BN / S::OV;
    for (int idx = tid; idx < BM * OVPR; idx += S::NT) {
        const int row = idx / OVPR;
        const int cv = idx % OVPR;
        const int m = m0 + row;
        const int n = n0 + cv * S::OV;
        if (m >= p.M || n >= p.K) continue;
        const T *src = Cs + row * S::LDC + cv * S::OV;
        T *dst = yg + (size_t)m * GK + n;
        if (p.out_vec) {
            store_nt16(dst, *reinterpret_cast<const uint4 *>(src));
        } else {
            const int lim = (p.K - n) < S::OV ? (p.K - n) : S::OV;
            for (int e = 0; e < lim; ++e) dst[e] = src[e];
        }
    }
}

}  // namespace convfwd
