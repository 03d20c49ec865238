// bf16 Newton–Schulz stages for the large tiles (T = 128 or 256) on gfx950.
//
// Same three stages as kernels_ns.hip (Gram with mirrored upper tiles,
// polynomial epilogue, update), re-tiled for MI355X:
//  * T x T output per workgroup of 2 x WN waves (T = 256: 8 waves, 2 per
//    SIMD, each 128 x 64 as 4 x 2 blocks of v_mfma_f32_32x32x16_bf16).
//  * K is staged in slices through a ring of LDS buffers that are filled
//    by direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds): 64-wide
//    slices in two buffers for the polynomial and the update, 32-wide slices
//    in four buffers for the Gram (whose K is the long side). A slice's loads
//    are issued right after the barrier that frees its buffer, one (or
//    three) slices ahead of its use, and no VGPRs or ds_write instructions
//    carry them. Each load instruction lands 64 x 16 bytes contiguously in
//    LDS, so the tiles are unpadded and bank conflicts are avoided by
//    swizzling 16-byte chunks on the global side:
//      - operands whose contraction index is contiguous (rows of X for the
//        Gram, rows of A, rows of B) sit as 2 BK-byte rows; chunk c of row r
//        is stored at chunk c ^ ((r >> 1) & 7) (128-byte rows) or
//        c ^ ((r >> 2) & 3) (64-byte rows), so the 16 rows a 16-lane phase
//        of ds_read_b128 touches fall in 16 distinct 16-byte slots;
//      - the update's X tile (contraction over its rows) sits row-major as
//        2T-byte rows; chunk c of row r is stored at c ^ (4 (r & 3)), so the
//        4 rows x 64 bytes a half-wave of ds_read_b64_tr_b16 touches fall in
//        4 distinct 64-byte bank windows.
//  * ds_read_b64_tr_b16 hands each lane four consecutive rows of one column
//    of X: within a 16-lane group, lane s supplies the address of row
//    (s >> 2), columns 4 (s & 3) .. +3 of a 4 x 16 block, and lane i receives
//    column i of that block. Two such reads make one 8-element fragment.
//  * The fragment reads of sub-step k+1 run under the MFMAs of sub-step k.
//  * On diagonal Gram / polynomial tiles both operands are the same rows,
//    which are loaded once.
//  * The polynomial computes B = b A + c A A and the update X' = alpha (a X +
//    B X), each rounded once. Their b A and a X terms need the output tile's
//    own block of the stage's input (A, or X), which is loaded into LDS in
//    three parts under the last two K slices and after the main loop (see
//    dma_own); the epilogue adds it to the fp32 accumulators before the
//    rounding. The update's epilogue writes X' back over that block in LDS
//    and stores from there.
//
// Source of the iteration: [P4] "modded-nanogpt 50B-token 长时程训练实验解析",
// section "从源码看 Muon 的分布式正交化实现" (quintic Newton–Schulz in bf16).

#include <type_traits>

#include "kernel_common.hpp"
#include "launch.hpp"
#include "ns_mfma_common.hpp"

namespace muon {

namespace {

// K pipeline per stage kind: BK-wide K slices through NBUF LDS buffers, the
// loads of slice kt + NBUF - 1 going out while slice kt is read. The Gram
// (long K: 3072 for a 768 x 3072 X) hides L2-miss latency with four 32-wide
// slices; the polynomial and the update (K = m_pad) do better with two
// 64-wide slices (half the barriers, a shorter prologue).
template <int MODE>
struct Pipe {
    static constexpr int BK = MODE == NS_GRAM ? 32 : 64;
    static constexpr int NBUF = MODE == NS_GRAM ? 4 : 2;
};

template <int T, int BK>
struct Layout {
    static constexpr int KROWB = 2 * BK;                // bytes per row of a k-contiguous tile (swizzled)
    static constexpr int XROWB = 2 * T;                 // bytes per row of the X tile (swizzled)
    static constexpr int KTILE = T * KROWB;             // k-contiguous tile, one stage
    static constexpr int STAGE = 2 * KTILE;             // P tile + (k-contiguous Q or X) tile
    static_assert(BK * XROWB == KTILE, "X tile and k-contiguous tile have the same size");
};

// NTOUT (Gram, polynomial): store the output tile and its mirror
// nontemporally (chosen per stream group; see the tile store below)
template <int T, int WN, int MODE, bool ROWSTATS, bool NTOUT>
__global__ __launch_bounds__(128 * WN) void k_ns_big(const MatDesc* __restrict__ mats,
                                                     const TileWork* __restrict__ work, const bf16* __restrict__ xin,
                                                     const bf16* __restrict__ ain, bf16* __restrict__ out, float ca,
                                                     float cb, float cc, int first, const float* __restrict__ partials,
                                                     float* __restrict__ ss_arr, float* __restrict__ scale_arr,
                                                     int32_t* __restrict__ status_arr, float eps,
                                                     float* __restrict__ rowpart) {
    // 2 x WN waves; each wave owns a WTM x WTN block of the tile
    constexpr int NT = 128 * WN;                     // threads per workgroup
    constexpr int NWV = NT / 64;                     // waves
    constexpr int WTM = T / 2;
    constexpr int WTN = T / WN;
    constexpr int FRI = WTM / 32;
    constexpr int FRJ = WTN / 32;
    constexpr int BK = Pipe<MODE>::BK;
    constexpr int NBUF = Pipe<MODE>::NBUF;
    constexpr int D = NBUF - 1;                      // prefetch distance in slices
    using LY = Layout<T, BK>;
    constexpr int KROWB = LY::KROWB;
    constexpr int EROW = 2 * T + 8;                  // epilogue staging row (bytes)
    // the ring, or the epilogue's staged rows plus a small reduction area at
    // the top (the Gram's first-iteration norm; the ring is idle by then)
    constexpr int REDB = 64;
    // POLY / UPDATE add a spare region after the ring for part of the output
    // tile's own block (below); 160 KB is the workgroup's LDS limit
    constexpr int RING = NBUF * LY::STAGE;
    constexpr int SPARE_BYTES = MODE == NS_GRAM ? 0 : (160 * 1024 - RING < T * 2 * T ? 160 * 1024 - RING : T * 2 * T);
    constexpr int SPARE_OFF = RING;
    constexpr int SMEM = RING + SPARE_BYTES > T * EROW + REDB ? RING + SPARE_BYTES : T * EROW + REDB;
    static_assert(FRJ >= 1 && NWV % 2 == 0 && NWV * 4 <= REDB, "tile too small for this wave grid");

    __shared__ __attribute__((aligned(16))) char smem[SMEM];
    float* red = reinterpret_cast<float*>(smem + SMEM - REDB);

    const TileWork w = work[blockIdx.x];
    const MatDesc d = mats[w.mat];
    const int i0 = (int)w.ti * T;
    const int j0 = (int)w.tj * T;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wi = wave / WN;
    const int wj = wave % WN;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    // diagonal Gram / polynomial tile: both operands are the same rows
    const bool same = MODE != NS_UPDATE && w.ti == w.tj;
    // The wave's 32-row fragment blocks are wi FRI + fi; its two 32-column
    // blocks are wj and 2 WN - 1 - wj, so that on a diagonal tile the two
    // waves of every SIMD hold the same number of blocks on or above the
    // diagonal (9 of 16 at T = 256) and skipping the others shortens the tile.
    static_assert(FRJ == 2, "two fragment columns per wave");
    const int cb1 = 2 * WN - 1 - wj;
    auto colblk = [&](int fj) { return fj == 0 ? wj : cb1; };

    const bf16* Psrc;
    const bf16* Qsrc;
    int ldp, ldq, K;
    // K stops at the first BK slice that lies wholly in the zero padding:
    // the padded columns of X (Gram) and of A (polynomial, update) are zero,
    // so the trimmed sum is the full one
    if (MODE == NS_GRAM) {
        Psrc = xin + d.x_off + (int64_t)i0 * d.n_pad;
        Qsrc = xin + d.x_off + (int64_t)j0 * d.n_pad;
        ldp = ldq = d.n_pad;
        K = (d.n + BK - 1) / BK * BK;
    } else if (MODE == NS_POLY) {
        Psrc = ain + d.a_off + (int64_t)i0 * d.m_pad;
        Qsrc = ain + d.a_off + (int64_t)j0 * d.m_pad;
        ldp = ldq = d.m_pad;
        K = (d.m + BK - 1) / BK * BK;
    } else {
        Psrc = ain + d.a_off + (int64_t)i0 * d.m_pad;  // rows of B
        Qsrc = xin + d.x_off + j0;                     // columns j0.. of X; row k = contraction
        ldp = d.m_pad;
        ldq = d.n_pad;
        K = (d.m + BK - 1) / BK * BK;
    }
    const int nk = K / BK;  // >= 3 for the Gram (K >= 96), >= 2 otherwise (K >= 128): m > 64 here
    // buffer ranges: the tile's rows (P, and Q for Gram / poly) or all K rows of X
    const u32x4 rp = rsrc(Psrc, (uint32_t)(T * ldp * 2));
    const u32x4 rq =
        rsrc(Qsrc, (uint32_t)((MODE == NS_UPDATE ? K * ldq : T * ldq) * 2));

    // ---- direct-to-LDS load geometry ----
    // k-contiguous tile (KROWB-byte rows of CPRK 16-byte chunks): instruction
    // q of wave w fills rows q KROUND + RPI w .. +RPI-1; lane l takes physical
    // chunk l % CPRK of row RPI w + l / CPRK, i.e. logical chunk
    // (l % CPRK) ^ ((row >> SH) & (CPRK - 1)); with 2^SH = 16 / CPRK the 16
    // rows of a ds_read_b128 phase land in 16 distinct 16-byte bank slots
    constexpr int CPRK = KROWB / 16;
    constexpr int RPI = 64 / CPRK;
    constexpr int SH = CPRK == 8 ? 1 : 2;
    static_assert(CPRK == 8 || CPRK == 4, "slice width");
    constexpr int KROUND = RPI * NWV;
    constexpr int NKI = T / KROUND;
    const int kr = wave * RPI + lane / CPRK;
    const int kc = (lane % CPRK) ^ ((kr >> SH) & (CPRK - 1));
    const int vp = kr * ldp * 2 + kc * 16;
    const int vqk = kr * ldq * 2 + kc * 16;
    // X tile (update) and the polynomial's A tile (2T-byte rows): XRPI rows of
    // XCH chunks per instruction; lane l takes physical chunk l % XCH of row
    // w XRPI + l / XCH
    constexpr int XCH = T / 8;
    constexpr int XRPI = 64 / XCH;
    constexpr int XROUND = XRPI * NWV;
    constexpr int NXI = BK / XROUND;
    static_assert(NKI >= 1 && NXI >= 1 && XROUND == 16, "load geometry");
    const int xr = wave * XRPI + lane / XCH;
    const int xc = (lane % XCH) ^ (4 * (xr & 3));
    const int vqx = xr * ldq * 2 + xc * 16;

    auto dma_stage = [&](int kt, char* S) {
        const int k0 = kt * BK;
#pragma unroll
        for (int q = 0; q < NKI; ++q) dma16(rp, S + (q * KROUND + wave * RPI) * KROWB, vp, (q * KROUND * ldp + k0) * 2);
        if (MODE == NS_UPDATE) {
#pragma unroll
            for (int q = 0; q < NXI; ++q)
                dma16(rq, S + LY::KTILE + (q * XROUND + wave * XRPI) * LY::XROWB, vqx, (k0 + q * XROUND) * ldq * 2);
        } else if (!same) {
#pragma unroll
            for (int q = 0; q < NKI; ++q)
                dma16(rq, S + LY::KTILE + (q * KROUND + wave * RPI) * KROWB, vqk, (q * KROUND * ldq + k0) * 2);
        }
    };
    // load instructions one stage issues (a diagonal Gram / poly tile loads one operand)
    constexpr int NDMA = NKI + (MODE == NS_UPDATE ? NXI : NKI);
    constexpr int NDMA_SAME = NKI;
    // wait until at most `stages` later stages' loads are still in flight
    auto wait_stage = [&](auto stages_c) {
        constexpr int ST = decltype(stages_c)::value;
        if (MODE != NS_UPDATE && same)
            __builtin_amdgcn_s_waitcnt(0x0F70 | (ST * NDMA_SAME));
        else
            __builtin_amdgcn_s_waitcnt(0x0F70 | (ST * NDMA));
    };
    static_assert((D - 1) * NDMA < 16, "vmcnt immediate");

    f32x16 acc[FRI][FRJ];
#pragma unroll
    for (int a = 0; a < FRI; ++a)
#pragma unroll
        for (int b = 0; b < FRJ; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // ---- fragment read geometry ----
    // k-contiguous: lane reads row l32 of a 32-row block, logical chunk 2 ks + hi
    int fo[BK / 16];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) fo[ks] = l32 * KROWB + 16 * ((2 * ks + hi) ^ ((l32 >> SH) & (CPRK - 1)));
    const int pb = wi * WTM * KROWB;
    const int qb = same ? 0 : LY::KTILE;
    // X (update): lane s of 16-lane group g reads row 8 (g >> 1) + (s >> 2) (+ 16 ks + 4 h),
    // elements wj WTN + 32 f + 16 (g & 1) + 4 (s & 3) .. +3
    const int g16 = lane >> 4;
    const int s16 = lane & 15;
    const int trow = 8 * (g16 >> 1) + (s16 >> 2);
    int tb[FRJ];
#pragma unroll
    for (int f = 0; f < FRJ; ++f) {
        const int e = 32 * colblk(f) + 16 * (g16 & 1) + 4 * (s16 & 3);
        tb[f] = LY::KTILE + trow * LY::XROWB + 16 * ((e >> 3) ^ (4 * (trow & 3))) + 2 * (e & 7);
    }

    // two fragment sets, alternating between k16 sub-steps
    bf16x8 pfr[2][FRI], qfr[2][FRJ];
    auto read_frags = [&](const char* S, int ks, int set) {
#pragma unroll
        for (int f = 0; f < FRI; ++f)
            pfr[set][f] = *reinterpret_cast<const bf16x8*>(S + pb + fo[ks] + f * 32 * KROWB);
#pragma unroll
        for (int f = 0; f < FRJ; ++f) {
            if (MODE != NS_UPDATE) {
                qfr[set][f] = *reinterpret_cast<const bf16x8*>(S + qb + fo[ks] + colblk(f) * 32 * KROWB);
            } else {
                const bf16x4 lo = tr_read(S + tb[f] + (16 * ks) * LY::XROWB);
                const bf16x4 up = tr_read(S + tb[f] + (16 * ks + 4) * LY::XROWB);
                qfr[set][f] = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
    };
    // The output tile's own block of the stage's input, for the epilogue:
    // POLY needs A[i0.., j0..] for its b A term, UPDATE needs X[i0.., j0..]
    // for its a X term (X' = alpha (a X + B X), a X added in fp32 before the
    // single rounding). It comes into LDS as 2T-byte rows, chunk c of row r
    // at c ^ (r & 15), in three regions so that most of it lands under MFMA
    // work: rows 0 .. NSP-1 in the spare region beyond the ring, loaded at
    // the start of the second-to-last K slice; the next ARPB rows in the ring
    // buffer the last slice leaves free, loaded at its start; the rest (T =
    // 256: 64 rows) into the last slice's buffer once that slice is done.
    constexpr bool OWN = MODE != NS_GRAM;
    constexpr int ARPB = LY::STAGE / LY::XROWB;               // rows of one ring buffer
    constexpr int NSP = SPARE_BYTES / LY::XROWB < T ? SPARE_BYTES / LY::XROWB : T;  // spare rows
    constexpr int NRB = T - NSP < ARPB ? T - NSP : ARPB;      // rows in the free ring buffer
    constexpr int NLAST = T - NSP - NRB;                       // rows loaded after the main loop
    static_assert(!OWN || (NSP % XROUND == 0 && NRB % XROUND == 0 && NLAST % XROUND == 0 && NLAST <= ARPB),
                  "own-tile layout");
    using NSP_C = std::integral_constant<int, NSP>;
    const int ldo = MODE == NS_UPDATE ? d.n_pad : d.m_pad;
    const int ar = wave * XRPI + lane / XCH;
    const int va = ar * ldo * 2 + ((lane % XCH) ^ (ar & 15)) * 16;
    // rows row0 .. row0 + N-1 of the own tile -> LDS at dst (N multiple of XROUND)
    auto dma_own = [&](char* dst, int row0, auto n_c) __attribute__((always_inline)) {
        if constexpr (OWN) {
            constexpr int N = decltype(n_c)::value;
            const bf16* src = MODE == NS_UPDATE ? xin + d.x_off + (int64_t)i0 * d.n_pad + j0
                                                : ain + d.a_off + (int64_t)i0 * d.m_pad + j0;
            const u32x4 ra = rsrc(src, (uint32_t)(T * ldo * 2));
#pragma unroll
            for (int q = 0; q < N / XROUND; ++q)
                dma16(ra, dst + (q * XROUND + wave * XRPI) * LY::XROWB, va, (row0 + q * XROUND) * ldo * 2);
        }
    };

    constexpr int NREAD = FRI + (MODE == NS_UPDATE ? 2 : 1) * FRJ;  // LDS read instructions per sub-step

    // MASK: the blocks this wave computes (all of them, or on a diagonal
    // Gram / polynomial tile those on or above the diagonal; the epilogue
    // writes the others from their mirror images). lo .. hi_ index the set
    // bits of MASK, so the instruction stream is fixed at compile time.
    auto mfma_block = [&](int set, auto lo_c, auto hi_c, auto mask_c) {
        constexpr unsigned MASK = decltype(mask_c)::value;
        constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
        static_for<LO, HI>([&](auto k_c) {
            constexpr int f = nth_bit(MASK, decltype(k_c)::value);
            constexpr int fi = f / FRJ, fj = f % FRJ;
            acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfr[set][fj], pfr[set][fi], acc[fi][fj], 0, 0, 0);
        });
    };
    // One K stage (kt) of the NBUF-deep ring. S: its buffer; N1: the next
    // stage's; NL: the buffer the previous stage released, which receives
    // stage kt + D (LOAD). WAIT: stages beyond kt + 1 whose loads may still be
    // in flight at the barrier (D - 1 .. 0), or -1 for the last stage, which
    // has no barrier to the next. The buffers are restrict (and the loads are
    // invisible to the compiler) so that no wait is inserted before the reads
    // of S; the explicit waits and barriers order the ring.
    constexpr int NKS = BK / 16;  // k16 sub-steps per stage
    auto stage = [&](const char* __restrict__ S, const char* __restrict__ N1, char* __restrict__ NL, int kt,
                     auto load_c, auto wait_c, auto mask_c, auto spare_c) __attribute__((always_inline)) {
        constexpr bool LOAD = decltype(load_c)::value;
        constexpr int WAIT = decltype(wait_c)::value;
        constexpr int NF = bit_count(decltype(mask_c)::value);
        using IC0 = std::integral_constant<int, 0>;
        using ICH = std::integral_constant<int, NF / 2>;
        using ICN = std::integral_constant<int, NF>;
        if constexpr (LOAD) dma_stage(kt + D, NL);
        if constexpr (decltype(spare_c)::value) dma_own(smem + SPARE_OFF, 0, NSP_C{});  // own rows 0 .. NSP-1
        // the last slice: own rows NSP .. NSP + NRB - 1 into the ring buffer it
        // leaves free (the previous slice's, which every wave finished
        // reading before that slice's barrier), so that they land under this
        // slice's MFMAs (nk >= 2: the second-to-last slice sent rows 0 .. NSP-1)
        if constexpr (OWN && WAIT < 0)
            dma_own(smem + ((kt + 1) % NBUF) * LY::STAGE, NSP, std::integral_constant<int, NRB>{});
#pragma unroll
        for (int ks = 0; ks < NKS - 1; ++ks) {
            const int set = ks & 1;
            read_frags(S, ks + 1, set ^ 1);
            mfma_block(set, IC0{}, ICN{}, mask_c);
            // interleave: one MFMA, then one LDS read
#pragma unroll
            for (int i = 0; i < NF; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
        }
        // last sub-step: the barrier sits in the middle of its MFMAs, and the
        // next stage's first fragment reads run under the second half
        constexpr int SL = (NKS - 1) & 1;
        if constexpr (WAIT >= 0) {
            mfma_block(SL, IC0{}, ICH{}, mask_c);
            __builtin_amdgcn_sched_barrier(0);  // keep these MFMAs ahead of the wait
            wait_stage(std::integral_constant<int, WAIT>{});
            __syncthreads();
            read_frags(N1, 0, 0);
            mfma_block(SL, ICH{}, ICN{}, mask_c);
#pragma unroll
            for (int i = 0; i < NF / 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if (NREAD > NF / 2) __builtin_amdgcn_sched_group_barrier(0x100, NREAD - NF / 2, 0);
        } else {
            mfma_block(SL, IC0{}, ICN{}, mask_c);
            __syncthreads();
        }
    };

    static_assert(D <= 4, "ring depth");
    auto buf = [&](int k) { return smem + (k % NBUF) * LY::STAGE; };
#pragma unroll
    for (int k = 0; k < D; ++k) dma_stage(k, buf(k));
    wait_stage(std::integral_constant<int, D - 1>{});
    __syncthreads();
    read_frags(buf(0), 0, 0);
    using C0 = std::integral_constant<int, 0>;
    using C1 = std::integral_constant<int, 1>;
    using C2 = std::integral_constant<int, 2>;
    using CD = std::integral_constant<int, D - 1>;
    using CL = std::integral_constant<int, -1>;
    using NO = std::false_type;
    auto main_loop = [&](auto mask_c) __attribute__((always_inline)) {
        if constexpr (OWN) {
            // D = 1; the second-to-last slice also sends own rows to the spare
            static_assert(D == 1, "own-tile schedule");
            for (int kt = 0; kt < nk - 2; ++kt)
                stage(buf(kt), buf(kt + 1), buf(kt + 1), kt, std::true_type{}, CD{}, mask_c, NO{});
            stage(buf(nk - 2), buf(nk - 1), buf(nk - 1), nk - 2, std::true_type{}, CD{}, mask_c, std::true_type{});
            stage(buf(nk - 1), buf(nk), buf(nk + 2), nk - 1, std::false_type{}, CL{}, mask_c, NO{});
        } else {
            for (int kt = 0; kt < nk - D; ++kt)
                stage(buf(kt), buf(kt + 1), buf(kt + D), kt, std::true_type{}, CD{}, mask_c, NO{});
            if constexpr (D >= 4) stage(buf(nk - 4), buf(nk - 3), buf(nk), nk - 4, std::false_type{}, C2{}, mask_c, NO{});
            if constexpr (D >= 3) stage(buf(nk - 3), buf(nk - 2), buf(nk), nk - 3, std::false_type{}, C1{}, mask_c, NO{});
            if constexpr (D >= 2)
                stage(buf(nk - 2), buf(nk - 1), buf(nk + 1), nk - 2, std::false_type{}, C0{}, mask_c, NO{});
            stage(buf(nk - 1), buf(nk), buf(nk + 2), nk - 1, std::false_type{}, CL{}, mask_c, NO{});
        }
    };
    constexpr unsigned FULL = (1u << (FRI * FRJ)) - 1;
    if (MODE == NS_UPDATE || !same) {
        // Edge tiles of padded matrices: output rows >= m and columns >= m
        // (Gram, polynomial) or >= n (update) are zero (so are A, B and X
        // there), so a wave skips its 32 x 32 blocks that lie wholly in the
        // padding. RV: its row blocks below the edge; CM: 2 if
        // both column blocks are inside, 1 if only block wj (the other,
        // 2 WN - 1 - wj, is further right). All waves still run every stage's
        // loads and barriers.
        const int vcol = MODE == NS_UPDATE ? d.n : d.m;
        const int rrem = d.m - (i0 + wi * WTM);
        const int rv = rrem <= 0 ? 0 : rrem >= WTM ? FRI : (rrem + 31) / 32;
        const int cm = j0 + 32 * cb1 < vcol ? 2 : j0 + 32 * wj < vcol ? 1 : 0;
        if (rv == FRI && cm == 2) {
            main_loop(std::integral_constant<unsigned, FULL>{});
        } else {
            static_for<0, FRI + 1>([&](auto r_c) {
                constexpr int RV = decltype(r_c)::value;
                static_for<0, 3>([&](auto c_c) {
                    constexpr int CM = decltype(c_c)::value;
                    if constexpr (!(RV == FRI && CM == 2))
                        if (rv == RV && cm == CM) main_loop(std::integral_constant<unsigned, edge_mask(RV, CM, FRI)>{});
                });
            });
        }
    } else {
        // a diagonal tile: each wave type runs its own fixed block list
        static_for<0, NWV>([&](auto w_c) {
            constexpr int W = decltype(w_c)::value;
            if (wave == W) main_loop(std::integral_constant<unsigned, diag_mask(W / WN, W % WN, WN, FRI)>{});
        });
    }
    if constexpr (OWN) {
        if constexpr (NLAST > 0) dma_own(buf(nk - 1), NSP + NRB, std::integral_constant<int, NLAST>{});
        wait_vm0();
        __syncthreads();
    }

    // ---------------- epilogue (lane holds C[i][j .. j+3]) ----------------
    float alpha = 1.0f;
    if (MODE == NS_GRAM && first) {
        float acc_p = 0.f;
        for (int p = tid; p < d.ew_count; p += NT) acc_p += partials[d.ew_start + p];
        acc_p = wave_sum(acc_p);
        if (lane == 0) red[wave] = acc_p;
        __syncthreads();
        float total = 0.f;
#pragma unroll
        for (int v = 0; v < NWV; ++v) total += red[v];
        const float sc = 1.0f / (sqrtf(total) + eps);
        alpha = sc * sc;
        if (w.ti == 0 && w.tj == 0 && tid == 0) {
            ss_arr[w.mat] = total;
            scale_arr[w.mat] = sc;
            status_arr[w.mat] = (isfinite(total) ? 0 : 1);
        }
    }
    if (MODE == NS_UPDATE && first) alpha = scale_arr[w.mat];

    // Gram / polynomial output tiles are staged in LDS as bf16 rows of EROW
    // bytes (2T + 8: 32 consecutive rows start in distinct 8-byte bank slots)
    // and leave as whole cache lines; the update's tile leaves from its own
    // X tile's layout.
    auto lds64 = [&](int off) -> uint2& { return *reinterpret_cast<uint2*>(smem + off); };

    float rsq[FRI];
#pragma unroll
    for (int f = 0; f < FRI; ++f) rsq[f] = 0.f;

    // POLY / UPDATE: the own tile's row r (r & 15 selects its chunk swizzle)
    // lives in the spare region, the ring buffer the last slice left free, or
    // the last slice's buffer
    auto own_row = [&](int r) -> char* {
        return r < NSP ? smem + SPARE_OFF + r * LY::XROWB
               : r < NSP + NRB ? smem + (nk % NBUF) * LY::STAGE + (r - NSP) * LY::XROWB
                               : smem + ((nk - 1) % NBUF) * LY::STAGE + (r - NSP - NRB) * LY::XROWB;
    };
    const int asw = l32 & 15;
    if constexpr (MODE == NS_UPDATE) {
        // X' = alpha (a X + B X), in place: each lane reads its own 8-byte
        // groups X[il][jl .. jl+3] from the own tile and writes the rounded
        // result back to the same bytes (no other lane touches them); the
        // tile then leaves from this layout. alpha is 1 after the first
        // iteration, where the multiply is left out (exact either way).
        auto own_update = [&](auto scaled) __attribute__((always_inline)) {
#pragma unroll
            for (int fi = 0; fi < FRI; ++fi) {
                char* row = own_row(wi * WTM + fi * 32 + l32) + 8 * hi;
#pragma unroll
                for (int fj = 0; fj < FRJ; ++fj)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        uint2* pv = reinterpret_cast<uint2*>(row + 16 * ((4 * colblk(fj) + g) ^ asw));
                        const uint2 xv = *pv;
                        float v[4];
                        v[0] = fmaf(ca, bf16_lo(xv.x), acc[fi][fj][4 * g + 0]);
                        v[1] = fmaf(ca, bf16_hi(xv.x), acc[fi][fj][4 * g + 1]);
                        v[2] = fmaf(ca, bf16_lo(xv.y), acc[fi][fj][4 * g + 2]);
                        v[3] = fmaf(ca, bf16_hi(xv.y), acc[fi][fj][4 * g + 3]);
                        if constexpr (decltype(scaled)::value) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] *= alpha;
                        }
                        uint2 ow;
                        ow.x = pack_bf16x2(v[0], v[1]);
                        ow.y = pack_bf16x2(v[2], v[3]);
                        *pv = ow;
                        if (ROWSTATS) {
                            const float r0 = bf16_lo(ow.x), r1 = bf16_hi(ow.x), r2 = bf16_lo(ow.y),
                                        r3 = bf16_hi(ow.y);
                            rsq[fi] = fmaf(r0, r0, rsq[fi]);
                            rsq[fi] = fmaf(r1, r1, rsq[fi]);
                            rsq[fi] = fmaf(r2, r2, rsq[fi]);
                            rsq[fi] = fmaf(r3, r3, rsq[fi]);
                        }
                    }
            }
        };
        if (first)
            own_update(std::true_type{});
        else
            own_update(std::false_type{});
        __syncthreads();
    } else {
    uint2 ev[FRI][FRJ][4];
    // the A entries of one 32-row block (8 loads), read a block ahead of their
    // use so the LDS latency is paid once per block, not once per load
    uint2 a_cur[FRJ][4], a_nxt[FRJ][4];
    auto read_a = [&](int fi, uint2 (&dst)[FRJ][4]) {
        if constexpr (OWN) {
            const char* row = own_row(wi * WTM + fi * 32 + l32) + 8 * hi;
#pragma unroll
            for (int fj = 0; fj < FRJ; ++fj)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    dst[fj][g] = *reinterpret_cast<const uint2*>(row + 16 * ((4 * colblk(fj) + g) ^ asw));
        }
    };
    read_a(0, a_nxt);
#pragma unroll
    for (int fi = 0; fi < FRI; ++fi) {
        if constexpr (OWN) {
#pragma unroll
            for (int fj = 0; fj < FRJ; ++fj)
#pragma unroll
                for (int g = 0; g < 4; ++g) a_cur[fj][g] = a_nxt[fj][g];
            if (fi + 1 < FRI) read_a(fi + 1, a_nxt);
            __builtin_amdgcn_sched_barrier(0);  // the next block's loads go out first
        }
#pragma unroll
        for (int fj = 0; fj < FRJ; ++fj) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[fi][fj][4 * g + e];
                if (MODE == NS_POLY) {
                    // B = b A + c A A
                    const uint2 in = a_cur[fj][g];
                    v[0] = fmaf(cb, bf16_lo(in.x), cc * v[0]);
                    v[1] = fmaf(cb, bf16_hi(in.x), cc * v[1]);
                    v[2] = fmaf(cb, bf16_lo(in.y), cc * v[2]);
                    v[3] = fmaf(cb, bf16_hi(in.y), cc * v[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] *= alpha;
                }
                uint2 ow;
                ow.x = pack_bf16x2(v[0], v[1]);
                ow.y = pack_bf16x2(v[2], v[3]);
                ev[fi][fj][g] = ow;
            }
        }
    }
    if (OWN) __syncthreads();  // the A tile is read; LDS is reused below
#pragma unroll
    for (int fi = 0; fi < FRI; ++fi)
#pragma unroll
        for (int fj = 0; fj < FRJ; ++fj)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                lds64((wi * WTM + fi * 32 + l32) * EROW + 2 * (32 * colblk(fj) + 8 * g + 4 * hi)) = ev[fi][fj][g];
    __syncthreads();
    }

    // the tile itself: each thread moves 16-byte row chunks, a wave covers
    // whole rows. The update's output is stored nontemporally: a round of
    // tiles writes about as much as an XCD's L2 holds, and normal stores
    // would push out the B and X panels the next round reads. The Gram's and
    // the polynomial's outputs (and their mirrors) are too in the NTOUT
    // instances, launched when their stream group's A is larger than the
    // MALL, so that the next stage would find little of them in cache. (A
    // runtime choice between the two stores does not survive: the compiler
    // merges the two branches into one store and drops the hint.)
    {
        bf16* obase = MODE == NS_UPDATE ? out + d.x_off + (int64_t)i0 * d.n_pad + j0
                                        : out + d.a_off + (int64_t)i0 * d.m_pad + j0;
        const int ld = MODE == NS_UPDATE ? d.n_pad : d.m_pad;
        constexpr int CPR = T / 8;
#pragma unroll
        for (int q = 0; q < T * CPR / NT; ++q) {
            const int id = tid + NT * q;
            const int r = id / CPR, c = id % CPR;
            // a diagonal tile's blocks below the diagonal come from the mirror below
            if (MODE != NS_UPDATE && same && (c >> 2) < (r >> 5)) continue;
            u32x4 wv;
            if constexpr (MODE == NS_UPDATE) {
                wv = *reinterpret_cast<const u32x4*>(own_row(r) + 16 * (c ^ (r & 15)));
            } else {
                const uint2 lo = lds64(r * EROW + 16 * c);
                const uint2 up = lds64(r * EROW + 16 * c + 8);
                wv = u32x4{lo.x, lo.y, up.x, up.y};
            }
            if constexpr (MODE == NS_UPDATE || NTOUT)
                __builtin_nontemporal_store(wv, reinterpret_cast<u32x4*>(obase + (int64_t)r * ld + 8 * c));
            else
                *reinterpret_cast<u32x4*>(obase + (int64_t)r * ld + 8 * c) = wv;
        }
    }
    if (MODE != NS_UPDATE) {
        // the mirror tile, read column-wise with two ds_read_b64_tr_b16 per
        // lane: in each 16-lane group G, lane s = 4 e + q points at row
        // IB + 32 G + 8 q + e (then + 4) of the 4-column chunk JB, so lane
        // 4 q + c receives rows IB + 32 G + 8 q .. +7 of column JB + c and
        // stores them as 16 bytes of mirror row JB + c; the 16 lanes with the
        // same c cover 128 consecutive entries (two cache lines) of that row.
        // A diagonal tile is its own mirror: only the 32 x 32 blocks below its
        // diagonal are written, from the computed blocks above it.
        bf16* mbase = out + d.a_off + (int64_t)j0 * d.m_pad + i0;
        const int G = lane >> 4, sl = lane & 15;
        const int sup_row = 32 * G + 8 * (sl & 3) + (sl >> 2);
        const int rc = sl & 3, rq = sl >> 2;
        constexpr int NIT = (T / 4) * (T / 128) / NWV;  // instruction pairs per wave
        static_assert(NIT * NWV == (T / 4) * (T / 128), "mirror work split");
#pragma unroll 4
        for (int k = 0; k < NIT; ++k) {
            const int it = wave + NWV * k;
            const int JB = 4 * (it % (T / 4));
            const int IB = 128 * (it / (T / 4));
            const bf16x4 lo = tr_read(smem + (IB + sup_row) * EROW + 2 * JB);
            const bf16x4 up = tr_read(smem + (IB + sup_row + 4) * EROW + 2 * JB);
            const bf16x8 v = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
            if (!same || ((JB + rc) >> 5) > ((IB + 32 * G + 8 * rq) >> 5)) {
                bf16x8* dst = reinterpret_cast<bf16x8*>(mbase + (int64_t)(JB + rc) * d.m_pad + IB + 32 * G + 8 * rq);
                if constexpr (NTOUT)
                    __builtin_nontemporal_store(v, dst);
                else
                    *dst = v;
            }
        }
    }

    if (MODE == NS_UPDATE && ROWSTATS) {
        __syncthreads();  // the staged output tile has been read
        float* rl = reinterpret_cast<float*>(smem);  // [2 wi][WN wj][WTM]
#pragma unroll
        for (int f = 0; f < FRI; ++f) rsq[f] += __shfl_xor(rsq[f], 32, 64);
        if (hi == 0) {
#pragma unroll
            for (int f = 0; f < FRI; ++f) rl[(wi * WN + wj) * WTM + f * 32 + l32] = rsq[f];
        }
        __syncthreads();
        if (tid < T) {
            const int wr = tid / WTM;
            const int rr = tid % WTM;
            float sum = 0.f;
#pragma unroll
            for (int v = 0; v < WN; ++v) sum += rl[(wr * WN + v) * WTM + rr];
            rowpart[d.rowpart_off + (int64_t)w.tj * d.m_pad + i0 + tid] = sum;
        }
    }
}

template <int T, int WN>
hipError_t launch_big_T(const LaunchCtx& L, const GemmList& G, int mode, const void* xin, const void* ain, void* out,
                        float ca, float cb, float cc, int first, float eps, int rowstats) {
    const TileWork* wl = mode == NS_GRAM ? G.gram : mode == NS_POLY ? G.poly : G.update;
    const int n = mode == NS_GRAM ? G.n_gram : mode == NS_POLY ? G.n_poly : G.n_update;
    if (n == 0) return hipSuccess;
    const bf16* x = (const bf16*)xin;
    const bf16* a = (const bf16*)ain;
    bf16* o = (bf16*)out;
    constexpr int NT = 128 * WN;
#define K_NS_BIG_ARGS \
    L.mats, wl, x, a, o, ca, cb, cc, first, L.partials, L.ss, L.scale, L.status, eps, L.rowpart
    // the Gram's and the polynomial's output stores are nontemporal for a
    // stream group whose A exceeds the MALL (the update's are in any case)
    const bool nt = L.ab_nontemporal != 0;
    if (mode == NS_GRAM) {
        if (nt)
            k_ns_big<T, WN, NS_GRAM, false, true><<<n, NT, 0, L.stream>>>(K_NS_BIG_ARGS);
        else
            k_ns_big<T, WN, NS_GRAM, false, false><<<n, NT, 0, L.stream>>>(K_NS_BIG_ARGS);
    } else if (mode == NS_POLY) {
        if (nt)
            k_ns_big<T, WN, NS_POLY, false, true><<<n, NT, 0, L.stream>>>(K_NS_BIG_ARGS);
        else
            k_ns_big<T, WN, NS_POLY, false, false><<<n, NT, 0, L.stream>>>(K_NS_BIG_ARGS);
    } else if (rowstats) {
        k_ns_big<T, WN, NS_UPDATE, true, false><<<n, NT, 0, L.stream>>>(K_NS_BIG_ARGS);
    } else {
        k_ns_big<T, WN, NS_UPDATE, false, false><<<n, NT, 0, L.stream>>>(K_NS_BIG_ARGS);
    }
#undef K_NS_BIG_ARGS
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_stage_big(const LaunchCtx& L, const GemmList& G, int mode, const void* xin, const void* ain,
                               void* out, float ca, float cb, float cc, int first, float eps, int rowstats) {
    if (G.T == 256) return launch_big_T<256, 4>(L, G, mode, xin, ain, out, ca, cb, cc, first, eps, rowstats);
    return launch_big_T<128, 2>(L, G, mode, xin, ain, out, ca, cb, cc, first, eps, rowstats);
}

}  // namespace muon
