// Implicit-GEMM forward convolution for gfx950 with direct global->LDS loads.
//
// Same GEMM view as igemm_kernel.h (rows m = output pixels with the batch
// folded in, columns n = output channels, reduction r = ((z*Y + y)*X + x)*C
// + c), but the gathered im2col slices never pass through registers:
//
//  * every K-step moves one 128-byte slice of the reduction (64 bf16 or 32
//    fp32 values) per tile row with `buffer_load_dwordx4 ... lds`: each lane
//    fetches one 16-byte chunk and the hardware writes the 64 chunks of a
//    wave to 1 KB of LDS in lane order (8 rows x 128 bytes);
//  * padding needs no branch: an out-of-range tap gets a byte offset beyond
//    the buffer's size and the buffer unit returns zeros;
//  * NS LDS stages are in flight: step it+NS-1 is being fetched while step
//    it is multiplied; the wait before a step names exactly how many newer
//    loads may still be outstanding;
//  * chunk q of row r is stored at 16-byte slot q ^ (r & 7), so the 8 lanes
//    that read one 16-byte column of 8 consecutive rows hit 8 different
//    bank groups; for 32x32 blocks, whose fragment reads take one chunk of
//    32 consecutive rows, rows with bit 4 set also swap the chunks of each
//    pair (slot q ^ (r & 7) ^ 1), which the 8-row swizzle alone leaves in
//    two-way bank conflicts on gfx950 (measured);
//  * the filter-tap position of a lane's chunk advances incrementally from
//    step to step (no integer division in the loop).
//
// The loads are issued from inline assembly so that the compiler, which
// cannot see which LDS bytes such a load writes, does not serialise every
// LDS read behind every outstanding load; the waits are placed here by hand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "igemm_kernel.h"

namespace convfwd {

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

struct DmaParams {
    KParams k;
    uint32_t x_bytes;   // buffer sizes: loads at or beyond them return zeros
    uint32_t w_bytes;
};

constexpr uint32_t kOutOfRange = 0x80000000u;   // >= every buffer size accepted

__device__ __forceinline__ i32x4_t buffer_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    i32x4_t r;
    r[0] = (int)(uint32_t)a;
    r[1] = (int)((uint32_t)(a >> 32) & 0xffffu);   // stride 0
    r[2] = (int)bytes;                              // num_records (bytes)
    r[3] = 0x00020000;                              // raw 32-bit data format
    return r;
}

// The buffer descriptor, the scalar offset and the LDS address of a load
// are the same in every lane.  Where the compiler cannot prove that (values
// that pass through code with divergent branches), it keeps them in vector
// registers, which the instruction cannot take: take them from the first
// active lane.
__device__ __forceinline__ i32x4_t uniform_rsrc(i32x4_t r)
{
    i32x4_t o;
    o[0] = __builtin_amdgcn_readfirstlane(r[0]);
    o[1] = __builtin_amdgcn_readfirstlane(r[1]);
    o[2] = __builtin_amdgcn_readfirstlane(r[2]);
    o[3] = __builtin_amdgcn_readfirstlane(r[3]);
    return o;
}

// One 16-byte-per-lane load into LDS at lds_addr + 16 * lane.  M0 carries
// the LDS address and is restored afterwards.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds_addr)
{
    rsrc = uniform_rsrc(rsrc);
    soff = __builtin_amdgcn_readfirstlane(soff);
    lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %4\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_addr)
        : "memory");
}

// s_waitcnt that waits only on vmcnt (expcnt and lgkmcnt left at their max).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int DT, int BM, int BN, int WM, int WN, int NS, int MF, int KSUB, int KG = 1>
struct DmaShape {
    using T = typename Elem<DT>::type;
    static constexpr int ESZ = (int)sizeof(T);
    static constexpr int VEC = 16 / ESZ;          // elements per 16-byte chunk
    static constexpr int SUBK = 128 / ESZ;        // reduction elements per 128-byte sub-slice
    static constexpr int BK = SUBK * KSUB;        // reduction elements per K-step
    static constexpr int NW = WM * WN;            // waves of one reduction group
    static constexpr int NT = NW * 64 * KG;       // threads of the workgroup
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int MI = TM / MF, NI = TN / MF;   // MFMA blocks per wave
    static constexpr int ACC = MF * MF / 64;          // accumulator floats per lane and block
    static constexpr int A_PER_W = BM / 8 / NW;  // 8-row DMA blocks per wave and stage
    static constexpr int B_PER_W = BN / 8 / NW;
    static constexpr int L = (A_PER_W + B_PER_W) * KSUB;  // DMA loads per wave and stage
    static constexpr int SUB = (BM + BN) * 128;   // bytes of one sub-slice (A rows then B rows)
    static constexpr int STAGE = SUB * KSUB;
    static constexpr int LDC = BN + VEC;
    static constexpr int EPI = BM * LDC * ESZ;
    static constexpr int LDF = BN + 4;                      // row stride (floats) of a partial tile
    static constexpr int PART = KG > 1 ? KG * BM * LDF * 4 : 0;   // every group's fp32 partial tile
    static constexpr int PIPE = KG * NS * STAGE;
    static constexpr int BODY = PIPE > EPI ? (PIPE > PART ? PIPE : PART) : (EPI > PART ? EPI : PART);
    // Big wave tiles (six or more MFMA blocks per wave) keep fewer operand
    // registers live: fragments are read one 32-byte quarter of the slice
    // at a time, the next quarter's while the current one is multiplied, and
    // the bias sits in LDS (fp32, after the body) instead of registers.
    static constexpr bool BIG = MI * NI >= 6;
    // the bias in LDS: big tiles, and split reductions (whose epilogue is
    // shared by all waves)
    static constexpr bool BIAS_LDS = BIG || KG > 1;
    static constexpr int BIAS_OFF = BODY;
    static constexpr int LDS_BYTES = BIAS_LDS ? BODY + BN * 4 : BODY;

    static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "whole DMA blocks per wave");
    static_assert(TM % MF == 0 && TN % MF == 0, "whole MFMA blocks per wave");
    static_assert(MF == 16 || (MF == 32 && DT == 1), "32x32 blocks: bf16 only");
    static_assert(NS >= 2 && L * (NS - 2) < 64, "vmcnt budget");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS of one CU");
    static_assert(KG == 1 || KG == 2 || KG == 4, "one, two or four reduction groups");
};

// FL = 0: the loads of the next stage are spread evenly over all products
// of the current one; FL = f > 0: over the first 1/f of them, so that with
// two stages the last load has most of a step to land before it is waited
// for (spread evenly, the last one is issued just before that wait and its
// whole latency is exposed on every step).
template <int DT, int BM, int BN, int WM, int WN, int NS, int MF, int KSUB, int KG, int FL, bool BIAS, bool GELU>
__global__ void __launch_bounds__(WM * WN * 64 * KG)
igemm_dma_kernel(DmaParams dp)
{
    using S = DmaShape<DT, BM, BN, WM, WN, NS, MF, KSUB, KG>;
    using AccT = typename std::conditional<MF == 32, f32x16_t, f32x4_t>::type;
    using T = typename S::T;
    const KParams &p = dp.k;
    // Fetch every argument the prologue reads in one batch at entry.  Left
    // to itself the compiler issues each scalar argument load in the block
    // of its first use, and the prologue then waits for three or four
    // argument fetches one after another.  (fd_Wo.d and out_vec arrive in
    // the same wide loads as used fields; listing them keeps their registers
    // from being reused by another load of the batch, which would need a
    // wait in between.)
    asm volatile("" ::"s"(gridDim.x), "s"(p.x), "s"(p.w), "s"(dp.x_bytes), "s"(dp.w_bytes), "s"(p.G), "s"(p.C),
                 "s"(p.K), "s"(p.Di), "s"(p.Hi), "s"(p.Wi), "s"(p.Y), "s"(p.X), "s"(p.sd), "s"(p.sh),
                 "s"(p.sw), "s"(p.pd), "s"(p.ph), "s"(p.pw), "s"(p.dd), "s"(p.dh));
    asm volatile("" ::"s"(p.dw), "s"(p.Do), "s"(p.Ho), "s"(p.Wo), "s"(p.M), "s"(p.Kred),
                 "s"(p.tiles_m), "s"(p.tiles_n), "s"(p.fd_Wo.m), "s"(p.fd_Wo.s), "s"(p.fd_Ho.m),
                 "s"(p.fd_Ho.s), "s"(p.fd_Do.m), "s"(p.fd_Do.s), "s"(p.fd_C.m), "s"(p.fd_C.s),
                 "s"(p.fd_X.m), "s"(p.fd_X.s), "s"(p.fd_Y.m), "s"(p.fd_Y.s), "s"(p.fd_Wo.d),
                 "s"(p.out_vec), "s"(p.fd_tn.m), "s"(p.fd_tn.s), "s"(p.fd_tm.m), "s"(p.fd_tm.s));

    __shared__ __attribute__((aligned(1024))) unsigned char smem[S::LDS_BYTES];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char *)smem;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // With KG > 1 the workgroup is KG groups of WM x WN waves that split the
    // reduction: group kg runs K-steps kg*nkh .. kg*nkh + nkh - 1 (steps past
    // the end load zeros) through its own LDS stages; at the end every group
    // writes its partial tile to LDS and all waves share the epilogue, which
    // adds the partials in group order (a fixed order, so the sum is
    // deterministic).  KG
    // times the waves per tile, 1/KG of the serial K-steps each: it pays for
    // problems with few output tiles and a long reduction (KG = 2: measured
    // 10-15% on 7x7 and 14x14 maps with 256-512 channels).  KG = 4 with one
    // wave per group lets a small problem be cut into exactly one tile per
    // compute unit (the batch-1 fp32 frontend's 1500 x 384 outputs are 256
    // tiles of 48 x 48) with all four SIMDs busy on it.
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = wave_all / S::NW;
    const int wave = wave_all - kg * S::NW;   // wave within the group
    const int wm = wave / WN;
    const int wn = wave % WN;

    // Workgroups are handed to the 8 XCDs round-robin.  Renumber them so each
    // XCD gets a contiguous run of tiles, and order tiles output-channel
    // fastest: an XCD then covers a slab of output rows with all their
    // channel tiles, so each input row is fetched into one XCD's L2 only and
    // only the (small) weight tensor is replicated across XCDs.
    const int nb = gridDim.x;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = nb >> 3, rem = nb & 7;
    int bid = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    const int q_n = fdiv(bid, p.fd_tn);
    const int n_tile = bid - q_n * p.tiles_n;
    const int g = fdiv(q_n, p.fd_tm);
    const int m_tile = q_n - g * p.tiles_m;
    const int m0 = m_tile * BM;
    const int n0 = n_tile * BN;

    const i32x4_t xr = buffer_rsrc(p.x, dp.x_bytes);
    const i32x4_t wr = buffer_rsrc(p.w, dp.w_bytes);
    const int GC = p.G * p.C;

    // ---- this lane's DMA assignment -------------------------------------
    const int lrow = lane >> 3;                 // row inside an 8-row block
    const int chunk = (lane & 7) ^ lrow;        // which 16-byte chunk of the K slice
    // Pair swap for rows with bit 4 set (32x32 blocks).  The DMA side then
    // fetches the partner chunk of the pair, which lies in the same filter
    // tap when C is a whole number of chunk pairs; otherwise no swap.
    const int sw4 = (MF == 32 && p.C % (2 * S::VEC) == 0) ? 1 : 0;
    const int pair_delta = (chunk & 1) ? -S::VEC : S::VEC;   // elements to the partner chunk

    // Rows of this lane: m_t = m0 + (wave*A_PER_W + t)*8 + lrow.  The first
    // is decoded with divisions, the others by stepping 8 pixels forward.
    int a_off[S::A_PER_W], a_bd[S::A_PER_W], a_bh[S::A_PER_W], a_bw[S::A_PER_W];
    {
        const int mfirst = m0 + wave * S::A_PER_W * 8 + lrow;
        int q = fdiv(mfirst, p.fd_Wo);
        int ow = mfirst - q * p.Wo;
        int q2 = fdiv(q, p.fd_Ho);
        int oh = q - q2 * p.Ho;
        int nb_ = fdiv(q2, p.fd_Do);
        int od = q2 - nb_ * p.Do;
#pragma unroll
        for (int t = 0; t < S::A_PER_W; ++t) {
            const int m = mfirst + t * 8;
            int bd = -(1 << 28), bh = 0, bw = 0, off = 0;
            if (m < p.M) {
                bd = od * p.sd - p.pd;
                bh = oh * p.sh - p.ph;
                bw = ow * p.sw - p.pw;
                off = (((nb_ * p.Di + bd) * p.Hi + bh) * p.Wi + bw) * GC + g * p.C;
            }
            a_off[t] = off; a_bd[t] = bd; a_bh[t] = bh; a_bw[t] = bw;
            ow += 8;
            while (ow >= p.Wo) {
                ow -= p.Wo;
                if (++oh == p.Ho) {
                    oh = 0;
                    if (++od == p.Do) { od = 0; ++nb_; }
                }
            }
        }
    }
    // K-steps of this group: kstart .. kstart + nkh - 1
    const int nk = (p.Kred + S::BK - 1) / S::BK;
    // Weight rows: GKZYXC rows of the tile's channels, or (prepacked) the
    // lane's 16-byte slot of a K-step's image -- the B part of the LDS stage
    // exactly as this kernel lays it out (swizzle included, zeros for
    // channels past K and reduction past Kred), KSUB sub-slices of BN*128
    // bytes per step, steps of one (group, channel tile) contiguous.
    constexpr int STEP_B = KSUB * BN * 128;
    uint32_t b_off[S::B_PER_W];
#pragma unroll
    for (int t = 0; t < S::B_PER_W; ++t) {
        const int n = n0 + (wave * S::B_PER_W + t) * 8 + lrow;
        const int cht = chunk ^ (sw4 & ((wave * S::B_PER_W + t) >> 1));   // row bit 4 = block bit 1
        if (p.wpacked)
            b_off[t] = (uint32_t)(((g * p.tiles_n + n_tile) * nk) * STEP_B + (wave * S::B_PER_W + t) * 1024 + lane * 16);
        else
            b_off[t] = n < p.K ? (uint32_t)(((g * p.K + n) * p.Kred + cht * S::VEC) * S::ESZ) : kOutOfRange;
    }

    const int nkh = (nk + KG - 1) / KG;
    const int kstart = kg * nkh;

    // Filter-tap position of the reduction index r, stepped by one 128-byte
    // sub-slice (SUBK elements) per call of prep, with the tap's element
    // offset from the row base kept in bytes and advanced by precomputed
    // deltas (no multiplication or division in the loop).  When C is a whole
    // number of sub-slices (the 384- and 64-channel workloads) every lane of
    // a sub-slice sits in the same tap: the position is then tracked once
    // for the workgroup (`tu`, uniform, scalar registers) and the lane's
    // chunk offset is part of its row bases; otherwise per lane (`tl`).
    // (Every helper lambda here is forced inline: one left as a call passes
    // its by-reference captures through scratch memory.)
    struct TapPos { int r, c, xk, yk, zd, yh, xw, offb; };
    const bool uni = p.C % S::SUBK == 0;
    const int dXb = (p.dw * GC - p.C) * S::ESZ;                       // x tap -> x tap + 1
    const int dYb = (p.dh * p.Wi - p.X * p.dw) * GC * S::ESZ;         // (X, y) -> (0, y + 1)
    const int dZb = (p.dd * p.Hi * p.Wi - p.Y * p.dh * p.Wi) * GC * S::ESZ;   // (0, Y, z) -> (0, 0, z + 1)
    auto tap_at = [&](int r0) __attribute__((always_inline)) {
        TapPos t;
        const int tap = fdiv(r0, p.fd_C);
        t.r = r0;
        t.c = r0 - tap * p.C;
        const int t2 = fdiv(tap, p.fd_X);
        t.xk = tap - t2 * p.X;
        const int zk = fdiv(t2, p.fd_Y);
        t.yk = t2 - zk * p.Y;
        t.zd = zk * p.dd;
        t.yh = t.yk * p.dh;
        t.xw = t.xk * p.dw;
        t.offb = (((t.zd * p.Hi + t.yh) * p.Wi + t.xw) * GC + t.c) * S::ESZ;
        return t;
    };
    TapPos tu = tap_at(kstart * S::BK);
    TapPos tl = tap_at(kstart * S::BK + chunk * S::VEC);
    // byte offset of each A row's base (with the pair swap, and with the
    // lane's chunk when the tap position is the workgroup's)
    int a_base[S::A_PER_W];
#pragma unroll
    for (int t = 0; t < S::A_PER_W; ++t) {
        const int swap = sw4 & ((wave * S::A_PER_W + t) >> 1);
        a_base[t] = (a_off[t] + (swap ? pair_delta : 0) + (uni ? chunk * S::VEC : 0)) * S::ESZ;
    }

    // DMA offsets of one stage, computed ahead (prep) and issued one at a
    // time between the MFMAs of the previous stage (fire), so the loads'
    // address arithmetic and issue run in the shadow of the matrix core.
    constexpr int LPS = S::A_PER_W + S::B_PER_W;   // loads per wave and sub-slice
    uint32_t dv[KSUB][LPS];
    auto prep_with = [&](TapPos &ts, int k0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < KSUB; ++u) {
            const bool rok = ts.r < p.Kred;
#pragma unroll
            for (int t = 0; t < S::A_PER_W; ++t) {
                const bool ok = rok && (unsigned)(a_bd[t] + ts.zd) < (unsigned)p.Di &&
                                (unsigned)(a_bh[t] + ts.yh) < (unsigned)p.Hi &&
                                (unsigned)(a_bw[t] + ts.xw) < (unsigned)p.Wi;
                dv[u][t] = ok ? (uint32_t)(a_base[t] + ts.offb) : kOutOfRange;
            }
            const uint32_t kb = p.wpacked ? (uint32_t)((k0 / S::BK) * STEP_B + u * BN * 128)
                                          : (uint32_t)((k0 + u * S::SUBK) * S::ESZ);
#pragma unroll
            for (int t = 0; t < S::B_PER_W; ++t)
                dv[u][S::A_PER_W + t] = (rok && b_off[t] != kOutOfRange) ? b_off[t] + kb : kOutOfRange;
            // advance to the next sub-slice
            ts.r += S::SUBK;
            ts.c += S::SUBK;
            ts.offb += S::SUBK * S::ESZ;
            while (ts.c >= p.C) {
                ts.c -= p.C;
                ts.offb += dXb;
                ts.xw += p.dw;
                if (++ts.xk == p.X) {
                    ts.xk = 0;
                    ts.xw = 0;
                    ts.offb += dYb;
                    ts.yh += p.dh;
                    if (++ts.yk == p.Y) {
                        ts.yk = 0;
                        ts.yh = 0;
                        ts.offb += dZb;
                        ts.zd += p.dd;
                    }
                }
            }
        }
    };
    auto prep = [&](int k0) __attribute__((always_inline)) {
        if (uni) prep_with(tu, k0);
        else prep_with(tl, k0);
    };
    // load number q (0 .. L-1) of the prepared stage into LDS stage `stage`
    auto fire = [&](int stage, int q) __attribute__((always_inline)) {
        const int u = q / LPS, t = q % LPS;
        const uint32_t base = lds0 + (kg * NS + stage) * S::STAGE + u * S::SUB;
        if (t < S::A_PER_W)
            dma16(xr, dv[u][t], 0, base + (wave * S::A_PER_W + t) * 1024);
        else
            dma16(wr, dv[u][t], 0, base + BM * 128 + (wave * S::B_PER_W + (t - S::A_PER_W)) * 1024);
    };

    AccT acc[S::MI][S::NI];
#pragma unroll
    for (int i = 0; i < S::MI; ++i)
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int e = 0; e < S::ACC; ++e) acc[i][j][e] = 0.f;

    // Operand rows: a 16x16 block feeds row (lane & 15) with the 16-byte
    // chunk (lane >> 4) of each 64-byte half; a 32x32 block feeds row
    // (lane & 31) with chunk (lane >> 5) of each 32-byte quarter.
    const int frow = lane & (MF - 1);
    const int fk = lane / MF;
    constexpr int RUNS = S::ACC / 4;     // runs of 4 consecutive channels per block

    // One stage: per sub-slice, all fragments are read first (one LDS
    // latency per sub-slice), then the products run; the prepared loads of
    // the stage `dst` (if >= 0) are spread between the products.  The
    // product is transposed (weights as the first operand), so each lane's
    // results are runs of 4 consecutive output channels.
    constexpr int QS = (DT == 1 && MF == 32) ? 4 : 2;              // fragment reads per 128-byte row
    constexpr int EPQ = (DT == 1) ? 1 : 4;                         // products per fragment pair
    constexpr int NMF = KSUB * QS * EPQ * S::MI * S::NI;           // products per stage
    constexpr int SPAN = FL > 0 ? (NMF + FL - 1) / FL : NMF;      // products the loads are spread over
    typedef typename std::conditional<DT == 1, bf16x8_t, f32x4_t>::type Frag;
    auto frag_off = [&](int q) __attribute__((always_inline)) {
        const int ch = (MF == 32 && DT == 1) ? 2 * q + fk : 4 * q + fk;
        return ((ch ^ (frow & 7) ^ (sw4 & (frow >> 4))) << 4);
    };
    auto compute_big = [&](int stage, int dst) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < KSUB; ++u) {
            const unsigned char *As = smem + (kg * NS + stage) * S::STAGE + u * S::SUB;
            const unsigned char *Bs = As + BM * 128;
            Frag a[2][S::MI], b[2][S::NI];
            auto rd = [&](int q) __attribute__((always_inline)) {
                const int sw = frag_off(q);
#pragma unroll
                for (int i = 0; i < S::MI; ++i)
                    a[q & 1][i] = *reinterpret_cast<const Frag *>(As + (wm * S::TM + i * MF + frow) * 128 + sw);
#pragma unroll
                for (int j = 0; j < S::NI; ++j)
                    b[q & 1][j] = *reinterpret_cast<const Frag *>(Bs + (wn * S::TN + j * MF + frow) * 128 + sw);
            };
            rd(0);
#pragma unroll
            for (int q = 0; q < QS; ++q) {
                if (q + 1 < QS) rd(q + 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int e = 0; e < EPQ; ++e)
#pragma unroll
                    for (int i = 0; i < S::MI; ++i)
#pragma unroll
                        for (int j = 0; j < S::NI; ++j) {
                            if constexpr (DT == 1 && MF == 32)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[q & 1][j], a[q & 1][i], acc[i][j], 0, 0, 0);
                            else if constexpr (DT == 1)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[q & 1][j], a[q & 1][i], acc[i][j], 0, 0, 0);
                            else
                                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b[q & 1][j][e], a[q & 1][i][e], acc[i][j], 0, 0, 0);
                            const int m = (((u * QS + q) * EPQ + e) * S::MI + i) * S::NI + j;
                            const int q0 = m < SPAN ? m * S::L / SPAN : S::L;
                            const int q1 = m < SPAN ? (m + 1) * S::L / SPAN : S::L;
                            if (dst >= 0) {
#pragma unroll
                                for (int qq = q0; qq < q1; ++qq) fire(dst, qq);
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
            }
        }
    };
    auto compute_all = [&](int stage, int dst) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < KSUB; ++u) {
            const unsigned char *As = smem + (kg * NS + stage) * S::STAGE + u * S::SUB;
            const unsigned char *Bs = As + BM * 128;
            Frag a[QS][S::MI], b[QS][S::NI];
#pragma unroll
            for (int q = 0; q < QS; ++q) {
                // 32x32 blocks: lane half fk takes chunk 2q+fk; 16x16 blocks:
                // lane quarter fk takes chunk 4q+fk
                const int sw = frag_off(q);
#pragma unroll
                for (int i = 0; i < S::MI; ++i)
                    a[q][i] = *reinterpret_cast<const Frag *>(As + (wm * S::TM + i * MF + frow) * 128 + sw);
#pragma unroll
                for (int j = 0; j < S::NI; ++j)
                    b[q][j] = *reinterpret_cast<const Frag *>(Bs + (wn * S::TN + j * MF + frow) * 128 + sw);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < QS; ++q)
#pragma unroll
                for (int e = 0; e < EPQ; ++e)
#pragma unroll
                    for (int i = 0; i < S::MI; ++i)
#pragma unroll
                        for (int j = 0; j < S::NI; ++j) {
                            if constexpr (DT == 1 && MF == 32)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[q][j], a[q][i], acc[i][j], 0, 0, 0);
                            else if constexpr (DT == 1)
                                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b[q][j], a[q][i], acc[i][j], 0, 0, 0);
                            else
                                // four 16x16x4 products over the 16 k of chunks 4q .. 4q+3: lane
                                // quarter fk holds chunk 4q+fk, product e uses its element e
                                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b[q][j][e], a[q][i][e], acc[i][j], 0, 0, 0);
                            const int m = (((u * QS + q) * EPQ + e) * S::MI + i) * S::NI + j;
                            const int q0 = m < SPAN ? m * S::L / SPAN : S::L;
                            const int q1 = m < SPAN ? (m + 1) * S::L / SPAN : S::L;
                            if (dst >= 0) {
#pragma unroll
                                for (int qq = q0; qq < q1; ++qq) fire(dst, qq);
                            }
                            __builtin_amdgcn_sched_barrier(0);
                        }
        }
    };

    auto compute = [&](int stage, int dst) __attribute__((always_inline)) {
        if constexpr (S::BIG) compute_big(stage, dst);
        else compute_all(stage, dst);
    };

    // ---- pipeline: stage it+NS-1 is loaded while stage it is multiplied ---
    // (both groups run the same nkh steps, so every barrier sees all waves)
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nkh) {
            prep((kstart + s) * S::BK);
#pragma unroll
            for (int q = 0; q < S::L; ++q) fire(s, q);
        }

    // Big tiles and split reductions: the bias of the tile's output channels
    // goes to LDS (fp32) once the first loads are in flight; the first
    // barrier of the loop orders it before the epilogue.
    if constexpr (BIAS && S::BIAS_LDS) {
        float *bs = reinterpret_cast<float *>(smem + S::BIAS_OFF);
        for (int i = tid; i < BN; i += S::NT) {
            const int n = n0 + i;
            bs[i] = n < p.K ? to_f32<T>(reinterpret_cast<const T *>(p.bias)[g * p.K + n]) : 0.f;
        }
    }

    // A reduction group of one wave loads and reads only its own stages: its
    // own vmcnt wait then suffices (the loads' LDS writes are complete when
    // the count drops, and it read the buffer it refills before issuing the
    // loads), so its steps need no workgroup barrier and the groups' SIMDs
    // run out of lockstep.
    constexpr bool STEP_BARRIER = S::NW > 1;
    for (int it = 0; it < nkh - 1; ++it) {
        if (it + NS - 2 < nkh) wait_vmcnt<S::L * (NS - 2)>();
        else wait_vmcnt<0>();
        if constexpr (STEP_BARRIER) __syncthreads();   // step it is in LDS for every wave
        const bool more = it + NS - 1 < nkh;    // the buffer it refills was read in step it-1
        if (more) prep((kstart + it + NS - 1) * S::BK);
        compute(it % NS, more ? (it + NS - 1) % NS : -1);
    }
    // last step: nothing left to load
    wait_vmcnt<0>();
    if constexpr (STEP_BARRIER) __syncthreads();
    // Bias of the lane's output channels (see the epilogue for the layout),
    // loaded here so that the last step's products hide its latency.
    float bias_v[S::BIAS_LDS ? 1 : S::NI][RUNS][4];
    if constexpr (BIAS && !S::BIAS_LDS) {
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int h = 0; h < RUNS; ++h)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // unconditional (clamped) loads, so they are all in flight at once
                    const int n = n0 + wn * S::TN + j * MF + h * 8 + fk * 4 + e;
                    const float v = to_f32<T>(reinterpret_cast<const T *>(p.bias)[g * p.K + (n < p.K ? n : p.K - 1)]);
                    bias_v[j][h][e] = n < p.K ? v : 0.f;
                }
    }
    compute((nkh - 1) % NS, -1);
    __syncthreads();

    T *__restrict__ yg = reinterpret_cast<T *>(p.y) + g * p.K;
    const int GK = p.ldy;   // output row pitch
    constexpr int OVPR = BN / S::VEC;

    // ---- split reduction: all waves share the epilogue ---------------------
    // Every group's fp32 partial tile goes to LDS (row-major, rows of LDF
    // floats); then each thread takes VEC consecutive outputs of a row, adds
    // the KG partials in group order (a fixed order, so the result is
    // deterministic), then bias, GELU, rounding, one 16-byte store.
    if constexpr (KG > 1) {
        float *pt = reinterpret_cast<float *>(smem);
        float *mine = pt + kg * BM * S::LDF;
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int h = 0; h < RUNS; ++h) {
                const int nl = wn * S::TN + j * MF + h * 8 + fk * 4;
#pragma unroll
                for (int i = 0; i < S::MI; ++i) {
                    const int ml = wm * S::TM + i * MF + frow;
                    *reinterpret_cast<f32x4_t *>(mine + ml * S::LDF + nl) =
                        f32x4_t{acc[i][j][h * 4], acc[i][j][h * 4 + 1], acc[i][j][h * 4 + 2], acc[i][j][h * 4 + 3]};
                }
            }
        __syncthreads();
        // A fixed number of vectors per thread, all read and computed before
        // any is stored (indices past the tile are clamped for the reads and
        // skipped for the stores), so the LDS reads of every vector are in
        // flight together and the VALU work runs back to back.
        constexpr int NV = BM * OVPR;
        constexpr int ITERS = (NV + S::NT - 1) / S::NT;
        constexpr int NQ = S::VEC / 4;
        f32x4_t part[ITERS][NQ][KG], bv[ITERS][NQ];
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int idx0 = tid + it * S::NT;
            const int idx = idx0 < NV ? idx0 : NV - 1;
            const int row = idx / OVPR;
            const int cv = idx % OVPR;
#pragma unroll
            for (int q4 = 0; q4 < NQ; ++q4) {
#pragma unroll
                for (int g2 = 0; g2 < KG; ++g2)
                    part[it][q4][g2] = *reinterpret_cast<const f32x4_t *>(pt + (g2 * BM + row) * S::LDF + cv * S::VEC + q4 * 4);
                bv[it][q4] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                if constexpr (BIAS)
                    bv[it][q4] = *reinterpret_cast<const f32x4_t *>(smem + S::BIAS_OFF + (cv * S::VEC + q4 * 4) * 4);
            }
        }
        __builtin_amdgcn_sched_barrier(0);   // every read issued before the arithmetic
        float v[ITERS][S::VEC];
#pragma unroll
        for (int it = 0; it < ITERS; ++it)
#pragma unroll
            for (int q4 = 0; q4 < NQ; ++q4) {
                f32x4_t sum = part[it][q4][0];
#pragma unroll
                for (int g2 = 1; g2 < KG; ++g2) sum += part[it][q4][g2];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float t = sum[e] + bv[it][q4][e];
                    if constexpr (GELU) t = DT == 1 ? gelu_erf_bf16out(t) : gelu_erf(t);
                    v[it][q4 * 4 + e] = t;
                }
            }
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int idx = tid + it * S::NT;
            const int row = idx / OVPR;
            const int cv = idx % OVPR;
            const int m = m0 + row;
            const int n = n0 + cv * S::VEC;
            if (idx >= NV || m >= p.M || n >= p.K) continue;
            T *dst = yg + (size_t)m * GK + n;
            if constexpr (DT == 1) {
                uint4 pk;
                pk.x = f32x2_to_bf16x2(v[it][0], v[it][1]);
                pk.y = f32x2_to_bf16x2(v[it][2], v[it][3]);
                pk.z = f32x2_to_bf16x2(v[it][4], v[it][5]);
                pk.w = f32x2_to_bf16x2(v[it][6], v[it][7]);
                if (p.out_vec) {
                    store_nt16(dst, pk);
                } else {   // the halfwords taken from the packed words (no type punning)
                    const int lim = (p.K - n) < S::VEC ? (p.K - n) : S::VEC;
                    const uint32_t wd[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
                    for (int e = 0; e < S::VEC; ++e)
                        if (e < lim) dst[e] = (uint16_t)(wd[e >> 1] >> ((e & 1) * 16));
                }
            } else {
                if (p.out_vec) {
                    __builtin_nontemporal_store(f32x4_t{v[it][0], v[it][1], v[it][2], v[it][3]},
                                                reinterpret_cast<f32x4_t *>(dst));
                } else {
                    const int lim = (p.K - n) < S::VEC ? (p.K - n) : S::VEC;
                    for (int e = 0; e < lim; ++e) dst[e] = v[it][e];
                }
            }
        }
        return;
    }

    // ---- epilogue: bias, GELU, round, stage in LDS, whole-vector stores ---
    // Transposed product: in a 16x16 block the lane holds channels
    // 4*fk + e (e = 0..3) of pixel frow; in a 32x32 block it holds channels
    // 8*h + 4*fk + e (h = 0..3, e = 0..3) of pixel frow.
    T *Cs = reinterpret_cast<T *>(smem);
    // Biases kept in LDS during the loop come to registers once, all reads
    // issued together, before any output is staged (a read placed after the
    // staging stores, which the compiler cannot tell apart from the bias
    // words, would wait for its whole latency in every row block).
    f32x4_t bias_l[S::BIAS_LDS && BIAS ? S::NI : 1][RUNS];
    if constexpr (BIAS && S::BIAS_LDS) {
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int h = 0; h < RUNS; ++h)
                bias_l[j][h] = *reinterpret_cast<const f32x4_t *>(smem + S::BIAS_OFF +
                                                                  (wn * S::TN + j * MF + h * 8 + fk * 4) * 4);
    }
    // Row block i of every wave: bias, activation and rounding of its
    // accumulators, written to the tile's rows wm*TM + i*MF + frow in LDS.
    auto stage_rows = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < S::NI; ++j)
#pragma unroll
            for (int h = 0; h < RUNS; ++h) {
                const int nl = wn * S::TN + j * MF + h * 8 + fk * 4;
                float bv[4] = {0.f, 0.f, 0.f, 0.f};
                if constexpr (BIAS && S::BIAS_LDS) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) bv[e] = bias_l[j][h][e];
                } else if constexpr (BIAS) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) bv[e] = bias_v[j][h][e];
                }
                const int ml = wm * S::TM + i * MF + frow;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = acc[i][j][h * 4 + e] + bv[e];
                    if constexpr (GELU) v[e] = DT == 1 ? gelu_erf_bf16out(v[e]) : gelu_erf(v[e]);
                }
                if constexpr (DT == 1) {
                    uint2 pk;
                    pk.x = f32x2_to_bf16x2(v[0], v[1]);
                    pk.y = f32x2_to_bf16x2(v[2], v[3]);
                    *reinterpret_cast<uint2 *>(Cs + ml * S::LDC + nl) = pk;
                } else {
                    *reinterpret_cast<f32x4_t *>(Cs + ml * S::LDC + nl) = f32x4_t{v[0], v[1], v[2], v[3]};
                }
            }
    };

    if (!p.out_vec) {   // K not a whole number of vectors: element stores
#pragma unroll
        for (int i = 0; i < S::MI; ++i) stage_rows(i);
        __syncthreads();
        for (int idx = tid; idx < BM * OVPR; idx += S::NT) {
            const int row = idx / OVPR;
            const int cv = idx % OVPR;
            const int m = m0 + row;
            const int n = n0 + cv * S::VEC;
            if (m >= p.M || n >= p.K) continue;
            const T *src = Cs + row * S::LDC + cv * S::VEC;
            T *dst = yg + (size_t)m * GK + n;
            const int lim = (p.K - n) < S::VEC ? (p.K - n) : S::VEC;
            for (int e = 0; e < lim; ++e) dst[e] = src[e];
        }
        return;
    }
    // Whole 16-byte vectors, one row block at a time: block i of every wave
    // is staged, then its rows (MF rows of each of the WM wave rows) are read
    // back and stored while the waves go on to stage block i + 1, so the
    // stores of one block drain during the activation work of the next
    // instead of all of them after all of it.  Blocks occupy disjoint LDS
    // rows, so one barrier per block suffices.  Within a block every read is
    // issued before any store (indices past the block are clamped for the
    // reads and skipped for the stores).
    constexpr int PROWS = WM * MF;                  // tile rows of one block
    constexpr int NVP = PROWS * OVPR;
    constexpr int ITERS = (NVP + S::NT - 1) / S::NT;
#pragma unroll
    for (int i = 0; i < S::MI; ++i) {
        stage_rows(i);
        __syncthreads();
        i32x4_t val[ITERS];   // (a native vector type: an array of uint4 is kept in scratch)
        int row_of[ITERS];
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int idx0 = tid + it * S::NT;
            const int idx = idx0 < NVP ? idx0 : NVP - 1;
            const int pr = idx / OVPR;
            const int row = (pr / MF) * S::TM + i * MF + (pr % MF);
            row_of[it] = row;
            val[it] = *reinterpret_cast<const i32x4_t *>(Cs + row * S::LDC + (idx % OVPR) * S::VEC);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            const int idx = tid + it * S::NT;
            const int m = m0 + row_of[it];
            const int n = n0 + (idx % OVPR) * S::VEC;
            if (idx < NVP && m < p.M && n < p.K)
                __builtin_nontemporal_store(val[it], reinterpret_cast<i32x4_t *>(yg + (size_t)m * GK + n));
        }
    }
}

}  // namespace convfwd
