// Every Newton–Schulz iteration of a bf16 matrix that is a single 256-row
// panel (m_pad = 256) in one workgroup of 8 waves on gfx950.
//
// Such a matrix's Gram and polynomial are one diagonal 256 x 256 tile each,
// and its update one row of tiles with K = 256, so the tiled kernels spend
// most of each launch in prologues and epilogues. Here the workgroup keeps A
// and then B resident in LDS (128 KB, bf16) across the three stages of an
// iteration:
//  * Gram: X streams through four 64-wide K slices (direct-to-LDS loads into
//    the resident region, which is idle until the epilogue); the waves
//    compute the 32 x 32 blocks on or above the diagonal, and the epilogue
//    writes A = R(g X X^T) and its mirror into the resident region.
//  * Polynomial: A A from the resident A (no global loads), all 64 blocks;
//    the epilogue reads each lane's own A entries and writes
//    B = R(b A + c A A) over them.
//  * Update: for each 256-column block of X, the block streams through two
//    32-row slice buffers after the resident region while B is read from
//    LDS; the waves that own a slice's rows add a X from it to their
//    accumulators, and X' = R(h (a X + B X)) leaves through the idle slice
//    buffers in 64-row rounds as full-line stores, for the next iteration's
//    Gram to read.
// g = s^2 and h = s in iteration 0 (s from the momentum kernel's partial
// sums), 1 afterwards; the rounding points are those of the tiled kernels.
// The last iteration also writes A and B to the workspace (debug views) and,
// with NorMuon, the per-row partial sums of O^2.
//
// Source of the iteration: [P4] "modded-nanogpt 50B-token 长时程训练实验解析",
// section "从源码看 Muon 的分布式正交化实现" (quintic Newton–Schulz in bf16).

#include "kernel_common.hpp"
#include "launch.hpp"
#include "ns_mfma_common.hpp"

namespace muon {

namespace {

constexpr int PT = kPanelRows;          // 256
constexpr int PNT = 512;                 // threads: 8 waves in a 2 x 4 grid
constexpr int PNWV = PNT / 64;
constexpr int PWN = 4;
constexpr int PWTM = PT / 2;             // rows per wave
constexpr int PFRI = PWTM / 32;          // 4 row blocks per wave
constexpr int PFRJ = 2;                  // column blocks wj and 2 PWN - 1 - wj
constexpr int RROW = 2 * PT;             // bytes per resident row (and per X slice row)
constexpr int RES = PT * RROW;           // 128 KB: A, then B
// Gram ring: GBK-wide K slices of the panel's rows
constexpr int GBK = 64;
constexpr int GKROWB = 2 * GBK;
constexpr int GSTAGE = PT * GKROWB;      // 32 KB
constexpr int GNBUF = 4;
constexpr int GD = GNBUF - 1;            // slices in flight ahead of the one read
constexpr int GCPR = GKROWB / 16;        // 16-byte chunks per row
constexpr int GRPI = 64 / GCPR;          // rows per load instruction and wave
constexpr int GSH = GCPR == 8 ? 1 : 2;
constexpr int GKROUND = GRPI * PNWV;     // rows per load instruction round
constexpr int GNKI = PT / GKROUND;       // load instructions per wave and slice
// update ring: 32-row slices of a 256-column block of X in two buffers after
// the resident region
constexpr int UBK = 32;
constexpr int USTAGE = UBK * RROW;       // 16 KB
constexpr int UNS = PT / UBK;            // 8 slices cover K = 256
constexpr int RING = RES;                // byte offset of the update ring
constexpr int SMEM = RES + 2 * USTAGE;   // 160 KB
static_assert(GNBUF * GSTAGE <= RES, "the Gram ring lives in the idle resident region");
static_assert(SMEM <= 160 * 1024, "LDS");

// The value itself, opaque to the optimiser: addresses derived from it are
// computed where they are used instead of being hoisted out of the iteration
// loop and kept live in VGPRs across it.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Resident layout: row r of A / B is 512 bytes, its 16-byte chunk c stored at
// chunk c ^ (r & 15), so the 16 rows of a ds_read_b128 phase fall in 16
// distinct 16-byte bank slots.
__device__ __forceinline__ int res_off(int r, int chunk) { return r * RROW + 16 * (chunk ^ (r & 15)); }
// the bf16 of row r, column c (with c % 4 == 0 also the 8 bytes of columns c .. c+3)
__device__ __forceinline__ int res_elem(int r, int c) { return res_off(r, c >> 3) + 2 * (c & 7); }
// Update slices of X (512-byte rows): chunk c of row r at c ^ xsw(r). Bits
// 2-3 (r & 3) put the 4 rows a 16-lane transposing read touches in 4 distinct
// 64-byte bank windows. Bit 0 (row bit 3) permutes chunks inside a window and
// spreads the a X reads (one 8-byte piece from each of 32 consecutive rows)
// over 8 16-byte slots instead of 4. xsw reads only row bits 0, 1 and 3,
// which adding 4 (to a row with bit 2 clear) or 16 leaves alone: the two
// halves of a transposing read and the two 16-row halves of a slice share one
// offset.
__device__ __forceinline__ int xsw(int r) { return 4 * (r & 3) + ((r >> 3) & 1); }

template <bool ROWSTATS>
__global__ __launch_bounds__(PNT) void k_ns_panel(const MatDesc* __restrict__ mats, const int32_t* __restrict__ list,
                                                  const bf16* __restrict__ xt, bf16* __restrict__ x0,
                                                  bf16* __restrict__ x1, bf16* __restrict__ a_out,
                                                  bf16* __restrict__ b_out, NsCoeffs co,
                                                  const float* __restrict__ partials, float* __restrict__ ss_arr,
                                                  float* __restrict__ scale_arr, int32_t* __restrict__ status_arr,
                                                  float* __restrict__ rowpart) {
    __shared__ __attribute__((aligned(16))) char smem[SMEM];

    const int mi = list[blockIdx.x];
    const MatDesc d = mats[mi];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = wave / PWN;
    const int wj = wave % PWN;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int cb1 = 2 * PWN - 1 - wj;
    auto colblk = [&](int fj) __attribute__((always_inline)) { return fj == 0 ? wj : cb1; };
    const int ldx = d.n_pad;
    // the blocks this wave computes on a diagonal tile (bit fi * 2 + fj)
    const unsigned dmask = diag_mask(wi, wj, PWN, PFRI);

    // ---- s from the momentum kernel's per-tile partial sums (iteration 0) ----
    float s;
    {
        float acc_p = 0.f;
        for (int p = tid; p < d.ew_count; p += PNT) acc_p += partials[d.ew_start + p];
        acc_p = wave_sum(acc_p);
        float* red = reinterpret_cast<float*>(smem + RING);
        if (lane == 0) red[wave] = acc_p;
        __syncthreads();
        float total = 0.f;
#pragma unroll
        for (int v = 0; v < PNWV; ++v) total += red[v];
        s = 1.0f / (sqrtf(total) + co.eps);
        if (tid == 0) {
            ss_arr[mi] = total;
            scale_arr[mi] = s;
            status_arr[mi] = isfinite(total) ? 0 : 1;
        }
        __syncthreads();
    }

    f32x16 acc[PFRI][PFRJ];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int a = 0; a < PFRI; ++a)
#pragma unroll
            for (int b = 0; b < PFRJ; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    };
    bf16x8 pfr[PFRI], qfr[PFRJ];
    // Fragment reads from the resident A / B: the rows of a lane's fragments
    // are all l32 (mod 16), so logical chunk 16 kh + 2 kl + hi of any of them
    // sits at byte 256 kh + swz[kl] of the row; row blocks add immediates.
    int swz[8];
#pragma unroll
    for (int kl = 0; kl < 8; ++kl) swz[kl] = 16 * ((2 * kl + hi) ^ (l32 & 15));
    const int prow = (wi * PWTM + l32) * RROW;
    int qrow[PFRJ];
#pragma unroll
    for (int f = 0; f < PFRJ; ++f) qrow[f] = (colblk(f) * 32 + l32) * RROW;
    // k16 step ks (0 .. 15) of the wave's P rows
    auto read_res_p = [&](int ks) __attribute__((always_inline)) {
        const int o = 256 * (ks >> 3) + swz[ks & 7];
#pragma unroll
        for (int f = 0; f < PFRI; ++f) pfr[f] = *reinterpret_cast<const bf16x8*>(smem + prow + f * 32 * RROW + o);
    };
    // ... and of both operands (the polynomial: A A^T = A A)
    auto read_res_frags = [&](int ks) __attribute__((always_inline)) {
        read_res_p(ks);
        const int o = 256 * (ks >> 3) + swz[ks & 7];
#pragma unroll
        for (int f = 0; f < PFRJ; ++f) qfr[f] = *reinterpret_cast<const bf16x8*>(smem + qrow[f] + o);
    };
    // MFMAs over the blocks in MASK (compile-time)
    auto mfma_mask = [&](auto mask_c) __attribute__((always_inline)) {
        constexpr unsigned MASK = decltype(mask_c)::value;
        static_for<0, PFRI * PFRJ>([&](auto f_c) {
            constexpr int f = decltype(f_c)::value;
            if constexpr ((MASK >> f) & 1u)
                acc[f / PFRJ][f % PFRJ] =
                    __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfr[f % PFRJ], pfr[f / PFRJ], acc[f / PFRJ][f % PFRJ], 0, 0, 0);
        });
    };

    // ---- Gram ring geometry (k-contiguous GKROWB-byte rows of GCPR chunks) ----
    // instruction q of wave w fills rows GKROUND q + GRPI w .. +GRPI-1; lane l
    // takes physical chunk l % GCPR of row GRPI w + l / GCPR, i.e. logical chunk
    // (l % GCPR) ^ ((row >> GSH) & (GCPR - 1)), so the 16 rows of a
    // ds_read_b128 phase fall in 16 distinct 16-byte bank slots
    const int gkr = wave * GRPI + lane / GCPR;
    const int gkc = (lane % GCPR) ^ ((gkr >> GSH) & (GCPR - 1));
    const int gvp = gkr * ldx * 2 + gkc * 16;
    int gfo[GBK / 16];
#pragma unroll
    for (int ks = 0; ks < GBK / 16; ++ks)
        gfo[ks] = l32 * GKROWB + 16 * ((2 * ks + hi) ^ ((l32 >> GSH) & (GCPR - 1)));

    // ---- update ring geometry (2T-byte rows of X, chunk c at c ^ xsw(r)) ----
    // instruction q of wave w fills rows 16 q + 2 w .. +1; lane l takes
    // physical chunk l % 32 of row 2 w + l / 32
    const int uxr = wave * 2 + lane / 32;
    const int uxc = (lane % 32) ^ xsw(uxr);
    // transposing reads: lane s of 16-lane group g reads row 8 (g >> 1) + (s >> 2)
    // (+ 16 ks + 4 h), elements 32 f + 16 (g & 1) + 4 (s & 3) .. +3
    const int g16 = lane >> 4;
    const int s16 = lane & 15;
    const int trow = 8 * (g16 >> 1) + (s16 >> 2);
    int tb[PFRJ];
#pragma unroll
    for (int f = 0; f < PFRJ; ++f) {
        const int e = 32 * colblk(f) + 16 * (g16 & 1) + 4 * (s16 & 3);
        tb[f] = trow * RROW + 16 * ((e >> 3) ^ xsw(trow)) + 2 * (e & 7);
    }
    // a X reads: slice row l32, logical chunk 4 colblk(fj) + gq at
    // (4 colblk(fj) + gq) ^ xsw(l32) = 4 (colblk(fj) ^ (l32 & 3)) + (gq ^ xq),
    // lane half hi
    int xrow[PFRJ];
#pragma unroll
    for (int f = 0; f < PFRJ; ++f) xrow[f] = l32 * RROW + 64 * (colblk(f) ^ (l32 & 3)) + 8 * hi;
    const int xq = (l32 >> 3) & 1;

    const int K_g = (d.n + GBK - 1) / GBK * GBK;  // Gram K, trimmed to the valid columns
    const int nkg = K_g / GBK;                    // >= 4 (n >= m = 256)
    const int nb = d.n_pad / PT;                  // 256-column blocks of X

    for (int it = 0; it < co.steps; ++it) {
        const float ca = co.c[it][0], cb = co.c[it][1], cc = co.c[it][2];
        const bf16* xin = it == 0 ? xt : ((it & 1) ? x1 : x0);
        bf16* xout = it == 0 ? x1 : ((it & 1) ? x0 : x1);
        const bool last = it == co.steps - 1;
        const bf16* xbase = xin + d.x_off;
        const u32x4 rx = rsrc(xbase, (uint32_t)(PT * ldx * 2));

        // ================= Gram: A = R(g X X^T) =================
        zero_acc();
        auto gload = [&](int kt) __attribute__((always_inline)) {
            char* S = smem + (kt % GNBUF) * GSTAGE;
#pragma unroll
            for (int q = 0; q < GNKI; ++q)
                dma16(rx, S + (q * GKROUND + wave * GRPI) * GKROWB, gvp, (q * GKROUND * ldx + kt * GBK) * 2);
        };
        // the previous iteration's X' stores have completed (vmcnt) and every
        // wave is past them (barrier) before its rows are loaded
        wait_vm0();
        __syncthreads();
#pragma unroll
        for (int k = 0; k < GD; ++k) gload(k);  // nkg >= 4 > GD
        static_assert(GNKI * (GD - 1) <= 15 && GD == 3, "vmcnt immediates");
        auto gram_loop = [&](auto mask_c) __attribute__((always_inline)) {
            for (int kt = 0; kt < nkg; ++kt) {
                // slice kt has landed once at most min(GD - 1, nkg - 1 - kt)
                // later slices' loads (GNKI per slice) are still in flight
                const int later = nkg - 1 - kt;
                if (later >= 2)
                    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * GNKI));
                else if (later == 1)
                    __builtin_amdgcn_s_waitcnt(0x0F70 | GNKI);
                else
                    wait_vm0();
                __syncthreads();
                if (kt + GD < nkg) gload(kt + GD);  // into the buffer slice kt - 1 used
                const char* S = smem + (kt % GNBUF) * GSTAGE;
#pragma unroll
                for (int ks = 0; ks < GBK / 16; ++ks) {
#pragma unroll
                    for (int f = 0; f < PFRI; ++f)
                        pfr[f] = *reinterpret_cast<const bf16x8*>(S + (wi * PWTM + f * 32) * GKROWB + gfo[ks]);
#pragma unroll
                    for (int f = 0; f < PFRJ; ++f)
                        qfr[f] = *reinterpret_cast<const bf16x8*>(S + colblk(f) * 32 * GKROWB + gfo[ks]);
                    mfma_mask(mask_c);
                    // one k16 step's fragments live at a time
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };
        static_for<0, PNWV>([&](auto w_c) {
            constexpr int W = decltype(w_c)::value;
            if (wave == W) gram_loop(std::integral_constant<unsigned, diag_mask(W / PWN, W % PWN, PWN, PFRI)>{});
        });
        __syncthreads();  // the ring (inside the resident region) is read

        // A and its mirror into the resident region: lane holds C[i][j .. j+3]
        // with i = 128 wi + 32 fi + l32, j = 32 colblk(fj) + 8 g + 4 hi
        {
            const float g = it == 0 ? s * s : 1.0f;
#pragma unroll
            for (int fi = 0; fi < PFRI; ++fi)
#pragma unroll
                for (int fj = 0; fj < PFRJ; ++fj) {
                    if (!((dmask >> (fi * PFRJ + fj)) & 1u)) continue;
                    const int i = wi * PWTM + fi * 32 + opaque(l32);
                    const bool mirror = colblk(fj) > wi * PFRI + fi;  // strictly above the diagonal
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int j = 32 * colblk(fj) + 8 * gq + 4 * opaque(hi);
                        const float v0 = acc[fi][fj][4 * gq + 0] * g, v1 = acc[fi][fj][4 * gq + 1] * g;
                        const float v2 = acc[fi][fj][4 * gq + 2] * g, v3 = acc[fi][fj][4 * gq + 3] * g;
                        uint2 w;
                        w.x = pack_bf16x2(v0, v1);
                        w.y = pack_bf16x2(v2, v3);
                        *reinterpret_cast<uint2*>(smem + res_elem(i, j)) = w;
                        if (mirror) {
                            *reinterpret_cast<uint16_t*>(smem + res_elem(j + 0, i)) = (uint16_t)(w.x & 0xffffu);
                            *reinterpret_cast<uint16_t*>(smem + res_elem(j + 1, i)) = (uint16_t)(w.x >> 16);
                            *reinterpret_cast<uint16_t*>(smem + res_elem(j + 2, i)) = (uint16_t)(w.y & 0xffffu);
                            *reinterpret_cast<uint16_t*>(smem + res_elem(j + 3, i)) = (uint16_t)(w.y >> 16);
                        }
                    }
                }
        }
        __syncthreads();
        // the last iteration's A to the workspace, row-major m_pad x m_pad
        auto copy_out = [&](bf16* dst) __attribute__((always_inline)) {
#pragma unroll 4
            for (int q = 0; q < PT * (PT / 8) / PNT; ++q) {
                const int id = opaque(tid) + PNT * q;
                const int r = id >> 5, c = id & 31;
                const u32x4 v = *reinterpret_cast<const u32x4*>(smem + res_off(r, c));
                *reinterpret_cast<u32x4*>(dst + d.a_off + (int64_t)r * PT + 8 * c) = v;
            }
        };
        if (last) copy_out(a_out);

        // ================= polynomial: B = R(b A + c A A) =================
        zero_acc();
        // all 64 blocks (K = 256 is short): both halves of the product are
        // computed, each from the same products in the same order
        static_for<0, PT / 16>([&](auto ks_c) {
            constexpr int ks = decltype(ks_c)::value;
            read_res_frags(ks);
            mfma_mask(std::integral_constant<unsigned, (1u << (PFRI * PFRJ)) - 1u>{});
        });
        __syncthreads();  // every wave has read A; B replaces it in place
        {
#pragma unroll
            for (int fi = 0; fi < PFRI; ++fi)
#pragma unroll
                for (int fj = 0; fj < PFRJ; ++fj) {
                    const int i = wi * PWTM + fi * 32 + opaque(l32);
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int j = 32 * colblk(fj) + 8 * gq + 4 * opaque(hi);
                        uint2* pv = reinterpret_cast<uint2*>(smem + res_elem(i, j));
                        const uint2 av = *pv;
                        const float v0 = fmaf(cb, bf16_lo(av.x), cc * acc[fi][fj][4 * gq + 0]);
                        const float v1 = fmaf(cb, bf16_hi(av.x), cc * acc[fi][fj][4 * gq + 1]);
                        const float v2 = fmaf(cb, bf16_lo(av.y), cc * acc[fi][fj][4 * gq + 2]);
                        const float v3 = fmaf(cb, bf16_hi(av.y), cc * acc[fi][fj][4 * gq + 3]);
                        uint2 w;
                        w.x = pack_bf16x2(v0, v1);
                        w.y = pack_bf16x2(v2, v3);
                        *pv = w;
                    }
                }
        }
        __syncthreads();
        if (last) copy_out(b_out);

        // ================= update: X' = R(h (a X + B X)) =================
        const float h = it == 0 ? s : 1.0f;
        for (int jb = 0; jb < nb; ++jb) {
            zero_acc();
            const int vqx = uxr * ldx * 2 + jb * PT * 2 + uxc * 16;
            auto uload = [&](int kt) __attribute__((always_inline)) {
                char* S = smem + RING + (kt & 1) * USTAGE;
#pragma unroll
                for (int q = 0; q < UBK / 16; ++q)
                    dma16(rx, S + (q * 16 + wave * 2) * RROW, vqx, (kt * UBK + q * 16) * ldx * 2);
            };
            uload(0);
            float rsq[PFRI] = {0.f, 0.f, 0.f, 0.f};
            static_for<0, UNS>([&](auto kt_c) {
                constexpr int kt = decltype(kt_c)::value;
                wait_vm0();       // slice kt (and any earlier stores) complete
                __syncthreads();  // ... for every wave; slice kt - 1's buffer is free
                if constexpr (kt + 1 < UNS) uload(kt + 1);
                const char* S = smem + RING + (kt & 1) * USTAGE;
#pragma unroll
                for (int ks = 0; ks < UBK / 16; ++ks) {
                    read_res_p(kt * (UBK / 16) + ks);  // rows of B, k16 step 2 kt + ks
#pragma unroll
                    for (int f = 0; f < PFRJ; ++f) {
                        const bf16x4 lo = tr_read(S + tb[f] + (16 * ks) * RROW);
                        const bf16x4 up = tr_read(S + tb[f] + (16 * ks + 4) * RROW);
                        qfr[f] = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
                    }
                    mfma_mask(std::integral_constant<unsigned, (1u << (PFRI * PFRJ)) - 1u>{});
                }
                // a X: the slice's rows 32 kt .. +31 are row block kt % 4 of the
                // waves with wi = kt / 4, which add a X from the slice
                if (wi == kt / PFRI) {
                    constexpr int FO = kt % PFRI;
#pragma unroll
                    for (int fj = 0; fj < PFRJ; ++fj)
#pragma unroll
                        for (int gq = 0; gq < 4; ++gq) {
                            const uint2 xv = *reinterpret_cast<const uint2*>(S + xrow[fj] + 16 * (gq ^ xq));
                            acc[FO][fj][4 * gq + 0] = fmaf(ca, bf16_lo(xv.x), acc[FO][fj][4 * gq + 0]);
                            acc[FO][fj][4 * gq + 1] = fmaf(ca, bf16_hi(xv.x), acc[FO][fj][4 * gq + 1]);
                            acc[FO][fj][4 * gq + 2] = fmaf(ca, bf16_lo(xv.y), acc[FO][fj][4 * gq + 2]);
                            acc[FO][fj][4 * gq + 3] = fmaf(ca, bf16_hi(xv.y), acc[FO][fj][4 * gq + 3]);
                        }
                }
            });
            // X' leaves through the idle ring in four rounds of 64 rows:
            // round R takes row block R of both wave rows (rows 32 R .. +31 and
            // 128 + 32 R .. +31), so all eight waves write their share as bf16
            // (512-byte rows, chunk c at c ^ (r & 15)); then every thread
            // stores whole 16-byte chunks, so each store instruction covers
            // full cache lines
            bf16* obase = xout + d.x_off + jb * PT;
            __syncthreads();  // every wave is done with the ring's last slice
            static_for<0, PFRI>([&](auto r_c) {
                constexpr int R = decltype(r_c)::value;
                const int rl = wi * 32 + opaque(l32);  // row within the round
#pragma unroll
                for (int fj = 0; fj < PFRJ; ++fj)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int j = 32 * colblk(fj) + 8 * gq + 4 * hi;
                        const f32x16& av = acc[R][fj];
                        uint2 w;
                        w.x = pack_bf16x2(av[4 * gq + 0] * h, av[4 * gq + 1] * h);
                        w.y = pack_bf16x2(av[4 * gq + 2] * h, av[4 * gq + 3] * h);
                        *reinterpret_cast<uint2*>(smem + RING + res_elem(rl, j)) = w;
                        if (ROWSTATS && last) {
                            const float r0 = bf16_lo(w.x), r1 = bf16_hi(w.x), r2 = bf16_lo(w.y), r3 = bf16_hi(w.y);
                            rsq[R] = fmaf(r0, r0, rsq[R]);
                            rsq[R] = fmaf(r1, r1, rsq[R]);
                            rsq[R] = fmaf(r2, r2, rsq[R]);
                            rsq[R] = fmaf(r3, r3, rsq[R]);
                        }
                    }
                __syncthreads();
#pragma unroll
                for (int q = 0; q < 64 * (PT / 8) / PNT; ++q) {
                    const int id = opaque(tid) + PNT * q;
                    const int rr = id >> 5, c = id & 31;  // staged row rr: wave row rr / 32, row rr % 32 of block R
                    const u32x4 v = *reinterpret_cast<const u32x4*>(smem + RING + res_off(rr, c));
                    const int grow = (rr >> 5) * PWTM + 32 * R + (rr & 31);
                    *reinterpret_cast<u32x4*>(obase + (int64_t)grow * ldx + 8 * c) = v;
                }
                __syncthreads();  // the staged rows are stored before the next round
            });
            if (ROWSTATS && last) {
                // row sums over this column block: lanes hi = 0/1, then the 4 wj
                // waves through the ring (idle: its last slice has been read)
                __syncthreads();
                float* rl = reinterpret_cast<float*>(smem + RING);  // [2 wi][4 wj][128]: the idle ring
#pragma unroll
                for (int f = 0; f < PFRI; ++f) rsq[f] += __shfl_xor(rsq[f], 32, 64);
                if (hi == 0) {
#pragma unroll
                    for (int f = 0; f < PFRI; ++f) rl[(wi * PWN + wj) * PWTM + f * 32 + l32] = rsq[f];
                }
                __syncthreads();
                if (tid < PT) {
                    const int wr = tid / PWTM, rr = tid % PWTM;
                    float sum = 0.f;
#pragma unroll
                    for (int v = 0; v < PWN; ++v) sum += rl[(wr * PWN + v) * PWTM + rr];
                    rowpart[d.rowpart_off + (int64_t)jb * d.m_pad + tid] = sum;
                }
                __syncthreads();  // the ring is reused by the next block's loads
            }
        }
    }
}

}  // namespace

hipError_t launch_ns_panel(const LaunchCtx& L, const int32_t* list, int n, const NsCoeffs& co, int rowstats) {
    if (n == 0) return hipSuccess;
    if (L.fp32 || co.steps < 1 || co.steps > 16) return hipErrorInvalidValue;
    const bf16* xt = (const bf16*)L.xt;
    bf16* x0 = (bf16*)L.x0;
    bf16* x1 = (bf16*)L.x1;
    if (rowstats)
        k_ns_panel<true><<<n, PNT, 0, L.stream>>>(L.mats, list, xt, x0, x1, (bf16*)L.a, (bf16*)L.b, co, L.partials,
                                                  L.ss, L.scale, L.status, L.rowpart);
    else
        k_ns_panel<false><<<n, PNT, 0, L.stream>>>(L.mats, list, xt, x0, x1, (bf16*)L.a, (bf16*)L.b, co, L.partials,
                                                   L.ss, L.scale, L.status, L.rowpart);
    return hipGetLastError();
}

}  // namespace muon
