// Tiled int8 MFMA GEMM with the dequantization fused into its epilogue (gfx950).
//
// Pages: "探秘Transformer系列之（36）--- 大模型量化方案" 1.2.2 (INT8 GEMM accumulating
// in INT32; the accumulation is scaled by the activation and weight scales
// before the FP16 result is written) and 1.1.2 vector-wise (the scaling is
// the outer product of per-row and per-column scales); ZeroQuant reading
// notes, kernel-fusion flowchart ("GeMM + DeQuantize" is one kernel);
// "Integer Quantization: Deep Dive", MAC unit (the bias joins the sum).
//
// Y[m, n] = fp16( s_x[m] * s_w[n / G] * sum_k Xq[m, k] Wq[n, k] + bias[n] ), optional GeLU.
//
// Design for CDNA4:
//  - v_mfma_i32_32x32x32_i8 (32 cycles per SIMD, the full int8 rate; the
//    16x16x64 form issues at half that rate on gfx950).  W is the A operand
//    and X the B operand, so each lane's 16 accumulators hold 4 runs of 4
//    consecutive output columns of one token.
//  - The prefill tiles (256x192 and 256x256) run eight waves, two per SIMD,
//    each owning a 64x96 (or 128x64) output block: five or six 16-byte LDS
//    reads per lane feed six or eight MFMAs per k-step.  128x128 tiles with
//    four waves cover small problems, 128x96 tiles (four waves of 32x96)
//    grids that 128x128 tiles would leave short of a round.  A last round of
//    large tiles at most half full is split off into a second launch of
//    128x192 tiles over the whole device: eight waves, two groups of four
//    64x96 blocks that take alternate halves of every slab's k-steps and add
//    their int32 partial sums through LDS at the end (int8; the FP8 and
//    outlier-part forms keep four waves).
//  - k slabs of BK bytes move HBM -> LDS with global_load_lds_dwordx4 (no
//    VGPR staging, no ds_write): lane l of a wave-wide load lands at
//    LDS[base + 16 l], so the bank swizzle is applied by choosing which
//    16-byte chunk of its row each lane fetches.  NSTAGE slabs are in flight;
//    one barrier per slab.  Lanes past the end of K fetch a 16-byte zero block.
//  - LDS rows are BK bytes; chunk c of row r sits at position c ^ f(r)
//    (f = (r/4)%4 for 64-byte rows, (r/2)%8 for 128-byte rows), which keeps
//    the MFMA operand reads (32 rows, one chunk) free of bank conflicts.
//  - MFMA fragments are double-buffered, and the schedule is spread out: each
//    MFMA of a k-step is followed by one read of the next k-step's fragments
//    and, at the slab boundary, by one refill DMA, so neither the LDS nor the
//    memory queue takes a burst while the matrix pipe waits.
//  - Per-column weight scales and biases of the tile are staged once in LDS;
//    per-row activation scales sit in registers.  The fp16 epilogue stages
//    each wave's rows through LDS and writes whole-row 16-byte pieces with
//    non-temporal stores.
//  - Workgroup b runs on XCD b % 8.  Tiles are ordered in groups of 4
//    M-tiles (N next; all M-tiles when there are at most 8) and each XCD
//    takes a contiguous run, so the ~32 tiles an XCD runs at once share 4 X
//    panels and 8 W panels in its L2 (on BERT FFN-up 1.5-2% faster than 8 X
//    and 4 W panels, which fetch ~9% more).
//  - Modes: int32 accumulators out (test mode), the FP8 variant (OCP E4M3
//    operands on v_mfma_scale_f32_32x32x64_f8f6f4), partial per-row |Y|
//    maxima, one per wave (for a downstream quantizer), and the
//    mixed-precision decomposition's fp16 outlier part in the epilogue.

#include <atomic>
#include "zq_device.h"
#include "zq_kernels.h"

#include <stdlib.h>

#include <type_traits>

namespace zq {

// 16 zero bytes: the DMA source for lanes whose k chunk lies past the end of K.
__device__ __attribute__((aligned(16))) int8_t g_zero16[16];

namespace {

template <int BK>
__device__ __forceinline__ int swz(int row)
{
    return BK == 64 ? ((row >> 2) & 3) : ((row >> 1) & 7);
}

template <int BM, int BN, int WM, int WN, int BK, int NSTAGE, int KW = 1>
struct Cfg {
    static constexpr int NW = WM * WN * KW;           // waves per workgroup
    static constexpr int NT = NW * 64;
    static constexpr int TWM = BM / WM;               // tokens per wave
    static constexpr int TWN = BN / WN;               // output columns per wave
    static constexpr int FM = TWM / 32;               // X fragments per wave
    static constexpr int FN = TWN / 32;               // W fragments per wave
    static constexpr int RPI = 1024 / BK;             // rows filled by one wave-wide DMA
    static constexpr int CPR = BK / 16;               // 16-byte chunks per row
    static constexpr int LX = BM / RPI / NW;          // DMAs per wave per slab, X
    static constexpr int LW = BN / RPI / NW;          // DMAs per wave per slab, W
    static constexpr int STAGE = (BM + BN) * BK;      // bytes per slab
    static constexpr int KS = BK / 32;                // MFMA k-steps per slab
    static_assert(KW == 1 || KW == 2, "one or two wave groups along k");
    static_assert(BK == 64 || BK == 128, "slab depth");
    static_assert(TWM % 32 == 0 && TWN % 32 == 0, "wave tile must be 32-aligned");
    static_assert(BM % (NW * RPI) == 0 && BN % (NW * RPI) == 0, "DMAs must divide evenly");
    static_assert(NW == 4 || NW == 8, "one or two waves per SIMD");
    static_assert(NSTAGE >= 2 && NSTAGE <= 4, "pipeline depth");
    static_assert(BN <= NT, "column parameters are staged one per thread");
    // Waves per SIMD the configuration runs at: eight-wave workgroups take a
    // CU each (two waves per SIMD); four-wave ones two per CU when their slabs
    // leave room for a second workgroup in the 160 KB of LDS, else one.
    static constexpr int WPS = NW == 8 ? 2 : (2 * (NSTAGE * STAGE + 8 * 1024) <= 160 * 1024 ? 2 : 1);
};

__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    const int total = tiles_m * tiles_n;
    int t = bid;
    if ((total & 7) == 0)
        t = (bid & 7) * (total >> 3) + (bid >> 3);
    // Groups of 4 M-tiles; grids of at most 8 M-tiles take them all in one
    // group (GPT QKV's 2048 x 12288 on 256x192 tiles: 99.2 against 100.8 us).
    const int GM = tiles_m <= 8 ? 8 : 4;
    const int per_group = GM * tiles_n;
    const int g = t / per_group;
    const int gm = min(GM, tiles_m - g * GM);
    const int r = t - g * per_group;
    tm = g * GM + r % gm;
    tn = r / gm;
}

// Configurations run two waves per SIMD (eight-wave workgroups, or two
// four-wave workgroups of the 128x128 tile per CU: 256 registers per wave),
// or one where a four-wave tile's slabs fill more than half of the LDS (the
// round split's 128x192 tail, the 128x96 tile: up to 512 registers).

// F8: the operands are OCP E4M3 codes and the product is
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales) accumulating in fp32;
// OUT_I32 then writes the raw fp32 accumulators.
//
// ODEC (fp16 output only): the mixed-precision decomposition's outlier part
// joins the epilogue.  The int32 accumulators are dequantized in place
// (s_x s_w acc, kept as fp32 bits in the same registers), then for every 16
// outlier columns one v_mfma_f32_32x32x16_f16 per fragment adds
// sum_p XO[m, p] W16t[O_p, n] onto them: W16t is the A operand and XO the
// B operand, so the fp16 product has the int8 accumulator layout.
template <int BM, int BN, int WM, int WN, int BK, int NSTAGE, bool OUT_I32, int ACT, bool F8,
          bool ODEC = false, int KW = 1>
__global__ __launch_bounds__(WM *WN *KW * 64)
__attribute__((amdgpu_waves_per_eu(Cfg<BM, BN, WM, WN, BK, NSTAGE, KW>::WPS,
                                    Cfg<BM, BN, WM, WN, BK, NSTAGE, KW>::WPS))) void k_gemm_tiled(
    const int8_t *__restrict__ Xq, const float *__restrict__ sx, const int8_t *__restrict__ Wq,
    const float *__restrict__ sw, int G, const float *__restrict__ bias, int M, int N, int K,
    void *__restrict__ Y, int ldy, int tiles_m, int tiles_n, float *__restrict__ row_part,
    int part_groups, OutlierOperands dec)
{
    using C = Cfg<BM, BN, WM, WN, BK, NSTAGE, KW>;
    static_assert(KW == 1 || (!ODEC && !F8), "k-split tiles: int8 without the outlier part");
    // One LDS object per slab buffer, referenced statically from an unrolled
    // main loop, so the compiler can tell a read of one buffer from the
    // in-flight DMAs into the others and need not wait for all of them.
    __shared__ __attribute__((aligned(1024))) int8_t lds0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) int8_t lds1[C::STAGE];
    __shared__ __attribute__((aligned(1024))) int8_t lds2[NSTAGE > 2 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(1024))) int8_t lds3[NSTAGE > 3 ? C::STAGE : 16];
    __shared__ __attribute__((aligned(16))) float col_scale[BN];
    __shared__ __attribute__((aligned(16))) float col_bias[BN];
    // ODEC: the outlier count and the first kOutCols outlier columns, fetched
    // at the start so that they have arrived by the epilogue.
    constexpr int kOutCols = 64;
    __shared__ int out_cols[ODEC ? kOutCols + 1 : 1];
    // ODEC, interior tiles with at most kPanel outlier columns (and ldy % 8 ==
    // 0, for 16-byte aligned weight rows): the tile's
    // outlier operands are copied HBM -> LDS by DMA during the main loop:
    // the weight panel [kPanel x BN] fp16 (row p = W16t[O_p, n0 .. n0 + BN)) and
    // the activation panel [BM x kPanel] fp16 (row m = XO[m0 + m, 0 .. kPanel)).
    // kPanel = 32 columns (16 for the 128x128 tile, whose two workgroups per CU
    // leave less LDS).
    constexpr int kPanel = BM * BN <= 128 * 128 ? 16 : 32;
    __shared__ __attribute__((aligned(1024))) _Float16 panel_w[ODEC ? kPanel * BN : 8];
    __shared__ __attribute__((aligned(1024))) _Float16 panel_x[ODEC ? BM * kPanel : 8];

    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    // KW = 2: waves wave and wave + WM * WN own the same output block and take
    // the first and the second half of every slab's k-steps (wave group wk).
    const int wk = KW == 1 ? 0 : wave / (WM * WN);
    const int wo = KW == 1 ? wave : wave % (WM * WN);
    const int wm = wo % WM;
    const int wn = wo / WM;

    if (!OUT_I32 && tid < BN) {
        const int n = min(n0 + tid, N - 1);
        col_scale[tid] = sw[n / G];
        col_bias[tid] = bias ? bias[n] : 0.0f;
    }
    if constexpr (ODEC) {
        if (tid <= kOutCols && tid <= K)  // cols holds K + 1 entries
            out_cols[tid] = dec.cols[tid];
    }
    float sxm[C::FM];
#pragma unroll
    for (int b = 0; b < C::FM; b++)
        sxm[b] = OUT_I32 ? 0.0f : sx[min(m0 + wm * C::TWM + b * 32 + (lane & 31), M - 1)];

    // DMA sources: wave-wide load j of this wave fills rows gi*RPI .. gi*RPI + RPI - 1
    // (gi = wave + NW j); lane l writes position l % CPR of row gi*RPI + l / CPR and
    // therefore fetches chunk (l % CPR) ^ f(row) of that row.
    const int8_t *src_x[C::LX];
    const int8_t *src_w[C::LW];
    int kc_x[C::LX], kc_w[C::LW];
#pragma unroll
    for (int j = 0; j < C::LX; j++) {
        const int row = (wave + C::NW * j) * C::RPI + lane / C::CPR;
        const int c = (lane % C::CPR) ^ swz<BK>(row);
        src_x[j] = Xq + (int64_t)min(m0 + row, M - 1) * K + 16 * c;  // ragged M: never stored
        kc_x[j] = 16 * c;
    }
#pragma unroll
    for (int j = 0; j < C::LW; j++) {
        const int row = (wave + C::NW * j) * C::RPI + lane / C::CPR;
        const int c = (lane % C::CPR) ^ swz<BK>(row);
        src_w[j] = Wq + (int64_t)min(n0 + row, N - 1) * K + 16 * c;
        kc_w[j] = 16 * c;
    }
    // One DMA of a slab: j < LX are the X rows, the rest the W rows.
    auto issue_one = [&](int slab, int8_t *bx, int j) {
        const int k0 = slab * BK;
        if (j < C::LX)
            dma16(k0 + kc_x[j] < K ? src_x[j] + k0 : g_zero16, bx + (wave + C::NW * j) * 1024);
        else
            dma16(k0 + kc_w[j - C::LX] < K ? src_w[j - C::LX] + k0 : g_zero16,
                  bx + BM * BK + (wave + C::NW * (j - C::LX)) * 1024);
    };
    // Lanes whose 16-byte chunk lies past K fetch zeros instead (branch-free select).
    auto issue = [&](int slab, int8_t *bx) {
        const int k0 = slab * BK;
        int8_t *bw = bx + BM * BK;
#pragma unroll
        for (int j = 0; j < C::LX; j++)
            dma16(k0 + kc_x[j] < K ? src_x[j] + k0 : g_zero16, bx + (wave + C::NW * j) * 1024);
#pragma unroll
        for (int j = 0; j < C::LW; j++)
            dma16(k0 + kc_w[j] < K ? src_w[j] + k0 : g_zero16, bw + (wave + C::NW * j) * 1024);
    };

    // MFMA operand reads: lane (frow, fhalf) reads row frow of each 32-row
    // fragment at chunk 2*ks + fhalf.  Fragment rows are multiples of 32 apart,
    // so the swizzle depends on frow only.
    const int frow = lane & 31;
    const int fhalf = lane >> 5;
    const int sw_l = swz<BK>(frow);
    const int xbase = (wm * C::TWM + frow) * BK;
    const int wbase = BM * BK + (wn * C::TWN + frow) * BK;

    // int8: a k-step is 32 bytes of K, lane (frow, fhalf) holds bytes 16 fhalf .. +16
    // (one chunk).  FP8: a k-step is 64 bytes, lane holds bytes 32 fhalf .. +32 (two
    // chunks, each at its own swizzled position).
    constexpr int KS = F8 ? BK / 64 : BK / 32;
    constexpr int KSW = KS / KW;   // k-steps per slab of one wave group
    const int kbase = KW == 1 ? 0 : wk * KSW;
    using Acc = std::conditional_t<F8, v16f, v16i>;
    using Frag = std::conditional_t<F8, v8i, v4i>;
    Acc acc[C::FN][C::FM];
#pragma unroll
    for (int a = 0; a < C::FN; a++)
#pragma unroll
        for (int b = 0; b < C::FM; b++)
            acc[a][b] = Acc{};

    auto load_frags = [&](const int8_t *stage, int ks, Frag (&fx)[C::FM], Frag (&fw)[C::FN]) {
        if constexpr (F8) {
            const int c0 = 4 * ks + 2 * fhalf;
            const int off0 = (c0 ^ sw_l) << 4, off1 = ((c0 + 1) ^ sw_l) << 4;
            auto two = [&](const int8_t *row) {
                const v4i lo = *reinterpret_cast<const v4i *>(row + off0);
                const v4i hi = *reinterpret_cast<const v4i *>(row + off1);
                return Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            };
#pragma unroll
            for (int b = 0; b < C::FM; b++)
                fx[b] = two(stage + xbase + b * 32 * BK);
#pragma unroll
            for (int a = 0; a < C::FN; a++)
                fw[a] = two(stage + wbase + a * 32 * BK);
        } else {
            const int off = ((2 * ks + fhalf) ^ sw_l) << 4;
#pragma unroll
            for (int b = 0; b < C::FM; b++)
                fx[b] = *reinterpret_cast<const v4i *>(stage + xbase + b * 32 * BK + off);
#pragma unroll
            for (int a = 0; a < C::FN; a++)
                fw[a] = *reinterpret_cast<const v4i *>(stage + wbase + a * 32 * BK + off);
        }
    };

    // One fragment: idx < FM are the X fragments, the rest the W fragments.
    auto load_frag_one = [&](const int8_t *stage, int ks, int idx, Frag (&fx)[C::FM],
                             Frag (&fw)[C::FN]) {
        const int8_t *row = idx < C::FM ? stage + xbase + idx * 32 * BK
                                        : stage + wbase + (idx - C::FM) * 32 * BK;
        Frag f;
        if constexpr (F8) {
            const int c0 = 4 * ks + 2 * fhalf;
            const v4i lo = *reinterpret_cast<const v4i *>(row + ((c0 ^ sw_l) << 4));
            const v4i hi = *reinterpret_cast<const v4i *>(row + (((c0 + 1) ^ sw_l) << 4));
            f = Frag{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
            f = *reinterpret_cast<const v4i *>(row + (((2 * ks + fhalf) ^ sw_l) << 4));
        }
        if (idx < C::FM)
            fx[idx] = f;
        else
            fw[idx - C::FM] = f;
    };

    int8_t *const bufs[4] = {lds0, lds1, lds2, lds3};
    // The slab count is padded to a multiple of NSTAGE: padding slabs lie past
    // K, every lane of their DMAs fetches the zero block, and their MFMAs add
    // exactly 0.  This keeps the unrolled slab loop free of branches, so the
    // count of in-flight DMAs at every wait is the same constant.
    const int nk = (K + BK - 1) / BK;
    const int nkp = (nk + NSTAGE - 1) / NSTAGE * NSTAGE;
    constexpr int PER_SLAB = C::LX + C::LW;  // DMAs per wave per slab

    // lgkmcnt(0) then s_barrier: this wave's LDS reads have returned and every
    // wave has passed this point.  (A plain s_barrier: __syncthreads would also
    // wait for the slab DMAs still in flight.)
    auto barrier = [] {
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_s_barrier();
    };

    // Slab j lives in buffer j % NSTAGE.  All NSTAGE buffers start filled.
#pragma unroll
    for (int j = 0; j < NSTAGE; j++)
        issue(j, bufs[j]);
    wait_vmcnt<(NSTAGE - 1) * PER_SLAB>();
    barrier();

    Frag fx[2][C::FM], fw[2][C::FN];
    load_frags(bufs[0], kbase, fx[0], fw[0]);

    // One slab: KS MFMA k-steps (with KW = 2, each wave group takes KS / 2 of
    // them).  The LDS reads for the next k-step are issued before the current
    // k-step's MFMAs.  Before the last k-step's MFMAs the slab hands over: wait
    // for slab kt+1, barrier (after which this slab's buffer is free), refill
    // it with slab kt+NSTAGE, read slab kt+1's first fragments.
    // The outlier panels go out with the first slab refill: by then the
    // outlier list is in LDS (the first barrier has passed).  They are the
    // youngest DMAs of that moment, so the slab waits that follow cover them
    // too, and the final drain before the epilogue certainly does.  Lanes past
    // the outlier count (or past K in the activation rows) fetch the zero block.
    const int n_out = ODEC ? out_cols[0] : 0;
    const bool use_panels =
        ODEC && n_out > 0 && n_out <= kPanel && n0 + BN <= N && (ldy & 7) == 0;
    auto issue_panels = [&] {
        if constexpr (ODEC) {
            if (!use_panels)
                return;
            constexpr int WCH = BN / 8;                     // 16-byte pieces per weight-panel row
            constexpr int NWD = kPanel * WCH / 64;          // wave-wide DMAs, weight panel
            constexpr int NXD = BM * (kPanel / 8) / 64;     // wave-wide DMAs, activation panel
            static_assert((kPanel * WCH) % 64 == 0 && (BM * (kPanel / 8)) % 64 == 0, "whole DMAs");
            for (int j = wave; j < NWD; j += C::NW) {
                const int idx = j * 64 + lane;
                const int p = idx / WCH, c = idx % WCH;
                const _Float16 *src = p < n_out ? dec.wt + (int64_t)out_cols[1 + p] * ldy + n0 + 8 * c
                                                : reinterpret_cast<const _Float16 *>(g_zero16);
                dma16(reinterpret_cast<const int8_t *>(src),
                      reinterpret_cast<int8_t *>(panel_w) + j * 1024);
            }
            for (int j = wave; j < NXD; j += C::NW) {
                const int idx = j * 64 + lane;
                const int ml = idx / (kPanel / 8), c = idx % (kPanel / 8);
                const _Float16 *src =
                    8 * c < K ? dec.xo + (int64_t)min(m0 + ml, M - 1) * K + 8 * c
                              : reinterpret_cast<const _Float16 *>(g_zero16);
                dma16(reinterpret_cast<const int8_t *>(src),
                      reinterpret_cast<int8_t *>(panel_x) + j * 1024);
            }
        }
    };

    auto slab = [&](int kt, auto S) {
        constexpr int s = decltype(S)::value;
#pragma unroll
        for (int ks = 0; ks < KSW; ks++) {
            const bool last = ks + 1 == KSW;
            // Fragments for the wave group's next k-step (this slab's, or the
            // next slab's first).
            const int8_t *nstage = last ? bufs[(s + 1) % NSTAGE] : bufs[s];
            const int nks = kbase + (last ? 0 : ks + 1);
            if (!last) {
                // The reads feeding this k-step were issued a k-step ago.
                __builtin_amdgcn_s_waitcnt(0xc07f);
            } else {
                wait_vmcnt<(NSTAGE - 2) * PER_SLAB>();
                barrier();
            }
            __builtin_amdgcn_sched_barrier(0);
            // Each MFMA is followed by one read of the next k-step's fragments and,
            // in the last k-step, one refill DMA, so neither queue fills in a burst.
#pragma unroll
            for (int a = 0; a < C::FN; a++)
#pragma unroll
                for (int b = 0; b < C::FM; b++) {
                    if constexpr (F8)
                        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                            fw[ks & 1][a], fx[ks & 1][b], acc[a][b], 0, 0, 0, 127, 0, 127);
                    else
                        acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                            fw[ks & 1][a], fx[ks & 1][b], acc[a][b], 0, 0, 0);
                    const int i = a * C::FM + b;
                    __builtin_amdgcn_sched_barrier(0);
                    if (i < C::FM + C::FN)
                        load_frag_one(nstage, nks, i, fx[(ks + 1) & 1], fw[(ks + 1) & 1]);
                    if (last && i < PER_SLAB)
                        issue_one(kt + NSTAGE, bufs[s], i);
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
            for (int i = C::FN * C::FM; i < C::FM + C::FN; i++)
                load_frag_one(nstage, nks, i, fx[(ks + 1) & 1], fw[(ks + 1) & 1]);
            if (last) {
#pragma unroll
                for (int j = C::FN * C::FM; j < PER_SLAB; j++)
                    issue_one(kt + NSTAGE, bufs[s], j);
                if constexpr (ODEC) {
                    if (kt == 0)
                        issue_panels();
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    static_assert(KSW % 2 == 0, "fragment buffers alternate within a slab");
    for (int kt = 0; kt < nkp; kt += NSTAGE) {
        slab(kt, std::integral_constant<int, 0>{});
        slab(kt + 1, std::integral_constant<int, 1>{});
        if constexpr (NSTAGE > 2)
            slab(kt + 2, std::integral_constant<int, 2>{});
        if constexpr (NSTAGE > 3)
            slab(kt + 3, std::integral_constant<int, 3>{});
    }
    // The refills issued by the last slabs read past K (zeros) into buffers
    // nobody reads again; drain them, then let every wave finish its last
    // operand reads, before the slab buffers are reused below.
    wait_vmcnt<0>();
    barrier();

    // KW = 2: the two wave groups hold partial sums of the same output block
    // over disjoint k-steps.  Fragment row b is finished by wave group b % 2:
    // each wave hands its other rows to its partner through the (now free)
    // slab buffers, 16 bytes per lane and store, and adds the partner's
    // partials of its own rows (int32: exact in any order).
    if constexpr (KW == 2) {
        static_assert(C::FM % 2 == 0, "fragment rows split evenly between the wave groups");
        constexpr int PART = C::FN * (C::FM / 2) * 16 * kWave * 4;  // bytes per wave
        constexpr int PER_BUF = C::STAGE / PART;
        static_assert(PER_BUF * NSTAGE >= C::NW, "every wave's partials fit the slab buffers");
        auto region = [&](int r) {
            const int bi = r / PER_BUF;
            int8_t *b = bi == 0 ? lds0 : bi == 1 ? lds1 : bi == 2 ? lds2 : lds3;
            return reinterpret_cast<v4i *>(b + (r % PER_BUF) * PART);
        };
        v4i *const give = region(wo + WM * WN * (1 - wk));  // read by the partner
        const v4i *const take = region(wo + WM * WN * wk);  // written by the partner
#pragma unroll
        for (int a = 0; a < C::FN; a++)
#pragma unroll
            for (int b = 0; b < C::FM; b++) {
                if (b % 2 == wk)
                    continue;
#pragma unroll
                for (int q = 0; q < 4; q++)
                    give[((a * (C::FM / 2) + b / 2) * 4 + q) * kWave + lane] =
                        v4i{acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2],
                            acc[a][b][4 * q + 3]};
            }
        barrier();
#pragma unroll
        for (int a = 0; a < C::FN; a++)
#pragma unroll
            for (int b = 0; b < C::FM; b++) {
                if (b % 2 != wk)
                    continue;
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const v4i p = take[((a * (C::FM / 2) + b / 2) * 4 + q) * kWave + lane];
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        acc[a][b][4 * q + i] += p[i];
                }
            }
        barrier();  // the slab buffers stage the outputs below
    }
    // Rows of fragments this wave finishes.
    auto own_row = [&](int b) { return KW == 1 || b % 2 == wk; };

    // Epilogue.  Accumulator register r of fragment (a, b) holds
    // token  m = m0 + wm*TWM + b*32 + lane%32 and
    // column n = n0 + wn*TWN + a*32 + 8*(r/4) + 4*(lane/32) + r%4.
    if constexpr (OUT_I32) {
#pragma unroll
        for (int b = 0; b < C::FM; b++) {
            if (!own_row(b))
                continue;
            const int m = m0 + wm * C::TWM + b * 32 + frow;
#pragma unroll
            for (int a = 0; a < C::FN; a++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int n = n0 + wn * C::TWN + a * 32 + 8 * q + 4 * fhalf;
                    if (m >= M || n >= N)
                        continue;
                    using Raw4 = std::conditional_t<F8, v4f, v4i>;
                    const Raw4 o = {acc[a][b][4 * q + 0], acc[a][b][4 * q + 1],
                                    acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]};
                    *reinterpret_cast<Raw4 *>(static_cast<int32_t *>(Y) + (int64_t)m * ldy + n) = o;
                }
        }
        return;
    }

    // fp16 results go out through a wave-private LDS block, one 32-token
    // fragment row at a time: registers hold 8-byte pieces of 32 different
    // rows, while the stores from LDS write whole runs of TWN columns, 16
    // bytes per lane, so far fewer write requests reach L2.  Rows of the
    // block are padded by 16 bytes to spread the 8-byte writes over the banks.
    constexpr int RS = C::TWN * 2 + 16;          // bytes per staged row
    constexpr int CPR_OUT = C::TWN / 8;          // 16-byte pieces per row
    constexpr int WPB = (C::NW + NSTAGE - 1) / NSTAGE;  // waves sharing one slab buffer
    static_assert(WPB * 32 * RS <= C::STAGE, "staging block fits in the slab buffers");
    static_assert((32 * CPR_OUT) % 64 == 0, "whole waves of 16-byte pieces");
    const int wb = wave % NSTAGE;
    int8_t *const stage_out =
        (wb == 0 ? lds0 : wb == 1 ? lds1 : wb == 2 ? lds2 : lds3) + (wave / NSTAGE) * 32 * RS;
    _Float16 *const Yh = static_cast<_Float16 *>(Y);
    const bool rows16 = (ldy & 7) == 0;          // 16-byte aligned rows of Y

    if constexpr (ODEC) {
        // Dequantize in place: from here on acc holds fp32 bits.
#pragma unroll
        for (int a = 0; a < C::FN; a++)
#pragma unroll
            for (int b = 0; b < C::FM; b++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int nl = wn * C::TWN + a * 32 + 8 * (r / 4) + 4 * fhalf + r % 4;
                    acc[a][b][r] =
                        __float_as_int((float)acc[a][b][r] * (sxm[b] * col_scale[nl]));
                }
        const int P = n_out;
        if (use_panels) {
            // Operands from the LDS panels (positions >= P are zero in the
            // weight panel; activation positions >= P are dropped here).
#pragma unroll
            for (int h = 0; h < kPanel / 16; h++) {
                if (16 * h >= P)
                    break;
                const int pb = 16 * h + 8 * fhalf;
                h8 xo[C::FM], wo[C::FN];
#pragma unroll
                for (int b = 0; b < C::FM; b++) {
                    const int ml = wm * C::TWM + b * 32 + frow;
                    const h8 raw = *reinterpret_cast<const h8 *>(panel_x + ml * kPanel + pb);
                    h8 v;
#pragma unroll
                    for (int i = 0; i < 8; i++)
                        v[i] = pb + i < P ? raw[i] : (_Float16)0.0f;
                    xo[b] = v;
                }
                // The weight panel is [position][column]; the A operand wants 8
                // consecutive positions of one column per lane.  ds_read_b64_tr_b16
                // transposes 4 x 16 blocks: in each 16-lane group, lane j addresses
                // row j / 4, columns 4 (j % 4) .. + 3 of the block, and lane i
                // receives column i of the block's 4 rows (layout checked on the
                // GPU).  Groups 0, 1 take columns 0-15, 16-31 of positions pb0 ..;
                // groups 2, 3 the same 8 positions further on; two reads per lane
                // give its 8 positions.
                const int grp = lane >> 4, gl = lane & 15;
                const int prow = 16 * h + 8 * (grp >> 1) + (gl >> 2);
                const int pcolb = 16 * (grp & 1) + 4 * (gl & 3);
#pragma unroll
                for (int a = 0; a < C::FN; a++) {
                    const _Float16 *src = panel_w + prow * BN + wn * C::TWN + a * 32 + pcolb;
                    const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(src));
                    const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4s *)(src + 4 * BN));
                    wo[a] = __builtin_bit_cast(h8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4,
                                                                           5, 6, 7));
                }
#pragma unroll
                for (int a = 0; a < C::FN; a++)
#pragma unroll
                    for (int b = 0; b < C::FM; b++) {
                        v16f c;
#pragma unroll
                        for (int r = 0; r < 16; r++)
                            c[r] = __int_as_float(acc[a][b][r]);
                        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(wo[a], xo[b], c, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 16; r++)
                            acc[a][b][r] = __float_as_int(c[r]);
                    }
            }
        }
        // Otherwise straight from global memory, two 16-column chunks per
        // round: every load of the round is issued before the first MFMA.
        // Lane (frow, fhalf) holds positions pb .. pb + 7.
        for (int p0 = 0; !use_panels && p0 < P; p0 += 32) {
            h8 xo[2][C::FM], wo[2][C::FN];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int pb = p0 + 16 * h + 8 * fhalf;
#pragma unroll
                for (int b = 0; b < C::FM; b++) {
                    const int m = min(m0 + wm * C::TWM + b * 32 + frow, M - 1);
                    h8 v = {};
                    if (pb < P) {
                        // pb + 8 <= K (K and pb are multiples of 8, pb < P <= K):
                        // the load stays inside row m; positions >= P are dropped.
                        const h8 raw = *reinterpret_cast<const h8 *>(dec.xo + (int64_t)m * K + pb);
#pragma unroll
                        for (int i = 0; i < 8; i++)
                            v[i] = pb + i < P ? raw[i] : (_Float16)0.0f;
                    }
                    xo[h][b] = v;
                }
                int oc[8];
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const int p = pb + i;
                    oc[i] = p >= P ? -1 : p < kOutCols ? out_cols[1 + p] : dec.cols[1 + p];
                }
#pragma unroll
                for (int a = 0; a < C::FN; a++) {
                    const int n = min(n0 + wn * C::TWN + a * 32 + frow, N - 1);
                    h8 v;
#pragma unroll
                    for (int i = 0; i < 8; i++)
                        v[i] = oc[i] >= 0 ? dec.wt[(int64_t)oc[i] * ldy + n] : (_Float16)0.0f;
                    wo[h][a] = v;
                }
            }
#pragma unroll
            for (int h = 0; h < 2; h++) {
                if (p0 + 16 * h >= P)
                    break;
#pragma unroll
                for (int a = 0; a < C::FN; a++)
#pragma unroll
                    for (int b = 0; b < C::FM; b++) {
                        v16f c;
#pragma unroll
                        for (int r = 0; r < 16; r++)
                            c[r] = __int_as_float(acc[a][b][r]);
                        c = __builtin_amdgcn_mfma_f32_32x32x16_f16(wo[h][a], xo[h][b], c, 0, 0, 0);
#pragma unroll
                        for (int r = 0; r < 16; r++)
                            acc[a][b][r] = __float_as_int(c[r]);
                    }
            }
        }
    }
    // With row_part, each wave also writes max |fp16 output| of each of its
    // rows over its TWN columns to row_part[m * part_groups + tn * WN + wn]
    // (after the two lanes that hold a row have combined theirs): partial
    // maxima for a per-token quantizer downstream, plain stores, no atomics.
    auto epilogue = [&](auto checked, auto fold_amax) {
        constexpr bool CHECK = decltype(checked)::value;
        constexpr bool AMAX = decltype(fold_amax)::value;  // row_part given
#pragma unroll
        for (int b = 0; b < C::FM; b++) {
            if (!own_row(b))
                continue;
            float rmax = 0.0f;
#pragma unroll
            for (int a = 0; a < C::FN; a++) {
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int nw = a * 32 + 8 * q + 4 * fhalf;        // column within wave block
                    const int nl = wn * C::TWN + nw;                  // column within tile
                    const float4 cs = *reinterpret_cast<const float4 *>(&col_scale[nl]);
                    const float4 cb = *reinterpret_cast<const float4 *>(&col_bias[nl]);
                    const float csv[4] = {cs.x, cs.y, cs.z, cs.w};
                    const float cbv[4] = {cb.x, cb.y, cb.z, cb.w};
                    h4 o;
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        float v;
                        if constexpr (ODEC)
                            v = __int_as_float(acc[a][b][4 * q + i]) + cbv[i];
                        else
                            v = fmaf((float)acc[a][b][4 * q + i], sxm[b] * csv[i], cbv[i]);
                        if constexpr (ACT == 1)
                            v = gelu_fast(v);
                        o[i] = (_Float16)v;
                    }
                    if (AMAX && (!CHECK || n0 + nl < N)) {
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            rmax = fmaxf(rmax, fabsf((float)o[i]));
                    }
                    *reinterpret_cast<h4 *>(stage_out + frow * RS + 2 * nw) = o;
                }
            }
            if constexpr (AMAX) {
                rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
                const int m = m0 + wm * C::TWM + b * 32 + frow;
                if (fhalf == 0 && (!CHECK || m < M))
                    row_part[(int64_t)m * part_groups + tn * WN + wn] = rmax;
            }
#pragma unroll
            for (int j = 0; j < 32 * CPR_OUT / 64; j++) {
                const int i = lane + 64 * j;
                const int row = i / CPR_OUT;
                const int c = i % CPR_OUT;
                const h8 v = *reinterpret_cast<const h8 *>(stage_out + row * RS + 16 * c);
                const int m = m0 + wm * C::TWM + b * 32 + row;
                const int n = n0 + wn * C::TWN + 8 * c;
                if (CHECK && m >= M)
                    continue;
                _Float16 *dst = Yh + (int64_t)m * ldy + n;
                // Non-temporal stores: nothing in this kernel reads Y again, and
                // the whole tile's output leaves at once at the end of the
                // tile (measured: BERT FFN-up GEMM 25.1 -> 22.3 us, GPT QKV
                // 128.8 -> 122.7 us, outlier 308 -> 296 us).
                if (rows16 && (!CHECK || n + 8 <= N)) {
                    __builtin_nontemporal_store(v, reinterpret_cast<h8 *>(dst));
                } else {
                    // N is a multiple of 4: each half is wholly inside or outside Y.
                    if (!CHECK || n < N)
                        __builtin_nontemporal_store(v.lo, reinterpret_cast<h4 *>(dst));
                    if (!CHECK || n + 4 < N)
                        __builtin_nontemporal_store(v.hi, reinterpret_cast<h4 *>(dst + 4));
                }
            }
        }
    };
    const bool interior = m0 + BM <= M && n0 + BN <= N;
    if (row_part) {
        if (interior)
            epilogue(std::false_type{}, std::true_type{});
        else
            epilogue(std::true_type{}, std::true_type{});
    } else {
        if (interior)
            epilogue(std::false_type{}, std::false_type{});
        else
            epilogue(std::true_type{}, std::false_type{});
    }
}

template <int BM, int BN, int WM, int WN, int BK, int NSTAGE, bool F8 = false, bool ODEC = false,
          int KW = 1>
hipError_t launch_cfg(const int8_t *Xq, const float *sx, const int8_t *Wq, const float *sw,
                      int64_t G, const float *bias, int act, int64_t M, int64_t N, int64_t K,
                      void *Y, bool out_i32, hipStream_t stream, float *row_part,
                      const OutlierOperands *dec = nullptr, int64_t ldy = -1,
                      int part_groups = -1)
{
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    const dim3 block(WM * WN * KW * 64);
    const OutlierOperands od = dec ? *dec : OutlierOperands{nullptr, nullptr, nullptr};
    // ldy: Y's row stride in elements (N unless this launch covers a column
    // range of a wider Y); part_groups: row_part's row stride in groups.
    const int y_stride = (int)(ldy < 0 ? N : ldy);
    const int groups = part_groups < 0 ? tiles_n * WN : part_groups;
#define ZQ_GEMM_LAUNCH(I32, A, D)                                                                 \
    hipLaunchKernelGGL((k_gemm_tiled<BM, BN, WM, WN, BK, NSTAGE, I32, A, F8, D, KW>), grid, block, \
                       0, stream, Xq, sx, Wq, sw, (int)G, bias, (int)M, (int)N, (int)K, Y,          \
                       y_stride, tiles_m, tiles_n, row_part, groups, od)
    if constexpr (ODEC) {
        static_assert(!F8 && KW == 1, "the outlier epilogue follows the int8 GEMM");
        if (act == 1)
            ZQ_GEMM_LAUNCH(false, 1, true);
        else
            ZQ_GEMM_LAUNCH(false, 0, true);
    } else {
        if (out_i32)
            ZQ_GEMM_LAUNCH(true, 0, false);
        else if (act == 1)
            ZQ_GEMM_LAUNCH(false, 1, false);
        else
            ZQ_GEMM_LAUNCH(false, 0, false);
    }
#undef ZQ_GEMM_LAUNCH
    return hipGetLastError();
}

struct Shape {
    int bm, bn;
};
// Tile configurations (waves: WM x WN; slab: BK bytes, NSTAGE deep):
//  0: 256x192, 4x2 waves, 128 B x2    1: 256x256, 4x2 waves, 128 B x2
//  2: 128x128, 2x2 waves, 64 B x4    3: 128x96, 4x1 waves, 128 B x3
constexpr int kNumShapes = 4;
constexpr Shape kShapes[kNumShapes] = {{256, 192}, {256, 256}, {128, 128}, {128, 96}};

// Compute units of the current device, queried once per device (256 on
// MI355X, also the answer when no device can be queried).
int device_cus()
{
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev >= 0 && dev < kMaxDevices) {
        const int c = cached[dev].load(std::memory_order_relaxed);
        if (c > 0)
            return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev >= 0 && dev < kMaxDevices)
        cached[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Bigger tiles move fewer bytes from L2 per MFMA; the choice trades that
// against how evenly the tiles fill the device's CUs.  ZQ_GEMM_TILE=0..3
// forces one (a measurement aid).
int pick_tile(int64_t M, int64_t N)
{
    static const int forced = [] {
        const char *e = getenv("ZQ_GEMM_TILE");
        return e ? atoi(e) : -1;
    }();
    if (forced >= 0 && forced < kNumShapes)
        return forced;
    const double cus = (double)device_cus();
    // Measured on MI355X: 256x256 does ~10% more work per unit of time than
    // 256x192 when both fill their rounds equally (outlier shape 274 vs 284 us),
    // 128x128 ~25% less (it covers small problems), 128x96 ~0.83 of 128x128
    // (4096 x 3072 -> 768: 256 tiles of 128x96 in 16.2-16.7 us against 192
    // tiles of 128x128 in 17.8-18.1 us).  Score = weight x the fraction of the
    // rounds' CU slots that tiles fill.
    const double weight[kNumShapes] = {1.0, 1.1, 0.7, 0.58};
    int best = 2;
    double best_score = -1.0;
    for (int i = 0; i < kNumShapes; i++) {
        const Shape s = kShapes[i];
        const double tiles = (double)((M + s.bm - 1) / s.bm) * (double)((N + s.bn - 1) / s.bn);
        const double rounds = ceil(tiles / cus);
        const double score = weight[i] * tiles / (rounds * cus);
        if (score > best_score + 1e-9) {
            best_score = score;
            best = i;
        }
    }
    return best;
}

// The round split.  A partly filled last round of tiles costs nearly a full
// round, so when bm x bn tiles would leave a last round at most half full, the
// columns up to the last whole round keep those tiles and the rest go to a
// second launch of 128x192 tiles that spreads them over the whole device.
// That launch has at most one workgroup per CU and a three-slab pipeline; its
// waves own 64x96 blocks (six MFMA blocks per five fragment loads).  The int8
// form runs two such waves per block, each over half of every slab's k-steps
// (two waves per SIMD; at the outlier layer's shape 36.6 us per tail launch
// against 37.4 us with four waves, medians of ~1140 traced dispatches each).  Returns the first column of the second launch, or 0 when the
// split does not apply (no whole round, a tail wider than one round of
// 128x192 tiles, or a split inside a weight group).
int64_t round_split_cols(int64_t M, int64_t N, int64_t G, int bm, int bn)
{
    const int64_t cus = device_cus();
    const int64_t tiles_m = (M + bm - 1) / bm;
    const int64_t total = tiles_m * ((N + bn - 1) / bn);
    const int64_t rounds = total / cus;
    const int64_t n_split = rounds * cus / tiles_m * bn;
    const int64_t tail_tiles = (M + 127) / 128 * ((N - n_split + 191) / 192);
    if (rounds >= 1 && 2 * (total - rounds * cus) <= cus && n_split > 0 && n_split < N &&
        n_split % G == 0 && tail_tiles <= cus)
        return n_split;
    return 0;
}

// Weight rows, weight-group scales, bias and output columns from column n0 on.
struct TailOperands {
    const int8_t *w;
    const float *sw;
    const float *bias;
    void *y;
};
TailOperands tail_operands(const int8_t *Wq, const float *w_scales, const float *bias, void *Y,
                           int64_t n0, int64_t K, int64_t G, bool out_4byte)
{
    const size_t el = out_4byte ? 4 : sizeof(_Float16);
    return {Wq + n0 * K, w_scales ? w_scales + n0 / G : nullptr, bias ? bias + n0 : nullptr,
            static_cast<int8_t *>(Y) + n0 * el};
}

}  // namespace

hipError_t launch_gemm_tiled(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                             const float *w_scales, int64_t G, const float *bias, int act,
                             int64_t M, int64_t N, int64_t K, void *Y, bool out_i32,
                             hipStream_t stream, float *row_part)
{
#define ZQ_CFG(BM, BN, WM, WN, BK, NS)                                                           \
    launch_cfg<BM, BN, WM, WN, BK, NS>(Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K, Y,      \
                                       out_i32, stream, row_part)
    const int tile = pick_tile(M, N);
    if (tile == 1 && row_part == nullptr) {
        const int64_t n_split = round_split_cols(M, N, G, 256, 256);
        if (n_split > 0) {
            hipError_t e = launch_cfg<256, 256, 4, 2, 128, 2>(
                Xq, x_scales, Wq, w_scales, G, bias, act, M, n_split, K, Y, out_i32, stream,
                nullptr, nullptr, N);
            if (e != hipSuccess)
                return e;
            const TailOperands t = tail_operands(Wq, w_scales, bias, Y, n_split, K, G, out_i32);
            return launch_cfg<128, 192, 2, 2, 128, 3, false, false, 2>(
                Xq, x_scales, t.w, t.sw, G, t.bias, act, M, N - n_split, K, t.y, out_i32, stream,
                nullptr, nullptr, N);
        }
    }
    switch (tile) {
    case 0: return ZQ_CFG(256, 192, 4, 2, 128, 2);
    case 1: return ZQ_CFG(256, 256, 4, 2, 128, 2);
    case 3: return ZQ_CFG(128, 96, 4, 1, 128, 3);
    default: return ZQ_CFG(128, 128, 2, 2, 64, 4);
    }
#undef ZQ_CFG
}

int64_t gemm_tiled_row_groups(int64_t M, int64_t N)
{
    switch (pick_tile(M, N)) {
    case 0: return (N + 191) / 192 * 2;   // 256x192, two waves across
    case 1: return (N + 255) / 256 * 2;   // 256x256, two waves across
    case 3: return (N + 95) / 96;         // 128x96, one wave across
    default: return (N + 127) / 128 * 2;  // 128x128, two waves across
    }
}

hipError_t launch_gemm_tiled_decomp(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                    const float *w_scales, int64_t G, const float *bias, int act,
                                    int64_t M, int64_t N, int64_t K, const int32_t *cols,
                                    const _Float16 *XO, const _Float16 *W16t, void *Y,
                                    hipStream_t stream)
{
    const OutlierOperands dec{cols, XO, W16t};
#define ZQ_CFGD(BM, BN, WM, WN, BK, NS)                                                          \
    launch_cfg<BM, BN, WM, WN, BK, NS, false, true>(Xq, x_scales, Wq, w_scales, G, bias, act, M, \
                                                    N, K, Y, false, stream, nullptr, &dec)
    // The 256x256 tiles' slabs leave no LDS for the outlier panels: their
    // problems take 256x192, with the round split; 128x128 covers the problems
    // of the small tiles.
    if (pick_tile(M, N) <= 1) {
        const int64_t n_split = round_split_cols(M, N, G, 256, 192);
        if (n_split > 0) {
            hipError_t e = launch_cfg<256, 192, 4, 2, 128, 2, false, true>(
                Xq, x_scales, Wq, w_scales, G, bias, act, M, n_split, K, Y, false, stream,
                nullptr, &dec, N);
            if (e != hipSuccess)
                return e;
            const TailOperands t = tail_operands(Wq, w_scales, bias, Y, n_split, K, G, false);
            const OutlierOperands tail_dec{cols, XO, W16t + n_split};
            return launch_cfg<128, 192, 2, 2, 128, 3, false, true>(
                Xq, x_scales, t.w, t.sw, G, t.bias, act, M, N - n_split, K, t.y, false, stream,
                nullptr, &tail_dec, N);
        }
        return ZQ_CFGD(256, 192, 4, 2, 128, 2);
    }
    return ZQ_CFGD(128, 128, 2, 2, 64, 4);
#undef ZQ_CFGD
}

hipError_t launch_gemm_tiled_fp8(const int8_t *Xq, const float *x_scales, const int8_t *Wq,
                                 const float *w_scales, int64_t G, const float *bias, int act,
                                 int64_t M, int64_t N, int64_t K, void *Y, bool out_raw,
                                 hipStream_t stream)
{
    // FP8 k-steps are 64 bytes: only the 128-byte slab configurations apply
    // (two k-steps per slab).  The FP8 fragments are twice as wide, so the
    // 256x256 tile would not fit the registers of two waves per SIMD: its
    // problems take 256x192 (with the round split); 128x128 covers the
    // problems of the small tiles.
#define ZQ_CFG8(BM, BN, WM, WN)                                                                   \
    launch_cfg<BM, BN, WM, WN, 128, 2, true>(Xq, x_scales, Wq, w_scales, G, bias, act, M, N, K,   \
                                             Y, out_raw, stream, nullptr)
    if (pick_tile(M, N) <= 1) {
        const int64_t n_split = round_split_cols(M, N, G, 256, 192);
        if (n_split > 0) {
            hipError_t e = launch_cfg<256, 192, 4, 2, 128, 2, true>(
                Xq, x_scales, Wq, w_scales, G, bias, act, M, n_split, K, Y, out_raw, stream,
                nullptr, nullptr, N);
            if (e != hipSuccess)
                return e;
            const TailOperands t = tail_operands(Wq, w_scales, bias, Y, n_split, K, G, out_raw);
            return launch_cfg<128, 192, 2, 2, 128, 3, true>(Xq, x_scales, t.w, t.sw, G, t.bias,
                                                            act, M, N - n_split, K, t.y, out_raw,
                                                            stream, nullptr, nullptr, N);
        }
        return ZQ_CFG8(256, 192, 4, 2);
    }
    return ZQ_CFG8(128, 128, 2, 2);
#undef ZQ_CFG8
}

}  // namespace zq
