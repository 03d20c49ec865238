// bf16 Newton–Schulz stages for the large tiles (T = 128 or 256) on gfx950.
//
// Same three stages as kernels_ns.hip (Gram with mirrored upper tiles,
// polynomial epilogue, update), re-tiled for MI355X:
//  * T x T output per 256-thread workgroup, 2 x 2 waves, each wave T/2 x T/2
//    as (T/64)^2 blocks of v_mfma_f32_32x32x16_bf16 (T = 256: 128 x 128 per
//    wave, 256 fp32 accumulators per lane), which halves LDS read traffic per
//    MFMA against 64 x 64 wave tiles.
//  * K staged in slices of 64 (128 bytes per row) through two LDS buffers;
//    the next slice is fetched into registers while the current one feeds
//    the MFMAs: its global loads are interleaved one per MFMA over the first
//    two k16 sub-steps and written to LDS in the last, and the fragment reads
//    of sub-step k+1 run under the MFMAs of sub-step k.
//  * Operands whose contraction index is contiguous (rows of X for the
//    Gram, rows of A, rows of B) sit in LDS as 128-byte rows padded to 144
//    bytes, so 16 consecutive rows start in 16 distinct 16-byte bank slots.
//  * The update contracts X over its row index. X stays row-major in LDS
//    (rows padded to 2T + 64 bytes) and its fragments are read with
//    ds_read_b64_tr_b16, which hands each lane four consecutive rows of one
//    column: within a 16-lane group, lane s supplies the address of row
//    (s >> 2), columns 4 (s & 3) .. +3 of a 4 x 16 block, and lane i receives
//    column i of that block. Two such reads make one 8-element fragment.
//  * The a X term of the update is folded into the polynomial: the poly
//    kernel writes B' = a I + b A + c A A, so the update is the pure product
//    X' = alpha B' X and reads X once per iteration.
//  * Every LDS address is a lane base plus a compile-time offset and every
//    global load is a buffer load with a lane offset and a scalar offset, so
//    the 256 accumulators leave room for the staged next slice in registers.
//
// Source of the iteration: [P4] "modded-nanogpt 50B-token 长时程训练实验解析",
// section "从源码看 Muon 的分布式正交化实现" (quintic Newton–Schulz in bf16).

#include <type_traits>

#include "kernel_common.hpp"
#include "launch.hpp"

namespace muon {

namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int BK = 64;       // k per LDS stage
constexpr int KROW = 144;    // bytes per padded row of a k-contiguous tile (128 + 16)

template <int T>
struct Layout {
    static constexpr int XROW = 2 * T + 64;            // bytes per padded row of the X tile
    static constexpr int KTILE = T * KROW;              // k-contiguous tile, one stage
    static constexpr int XTILE = BK * XROW;             // X tile, one stage
    static constexpr int QTILE = KTILE > XTILE ? KTILE : XTILE;
    static constexpr int STAGE = KTILE + QTILE;
};

__device__ __forceinline__ bf16x4 tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(LDS_AS char*)p);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

template <int T, int WN, int MODE, bool ROWSTATS>
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
    using LY = Layout<T>;
    constexpr int NCH = T * BK * 2 / 16 / NT;        // 16-byte chunks per thread per operand
    constexpr int PSTEP = NT / 8;                    // rows between a thread's P chunks
    constexpr int XSTEP = NT / (T / 8);              // X rows between a thread's chunks
    static_assert(NCH >= 1 && FRJ >= 1, "tile too small for this wave grid");

    __shared__ __attribute__((aligned(16))) char smem[2 * LY::STAGE];
    __shared__ float red[NWV];

    const TileWork w = work[blockIdx.x];
    const MatDesc d = mats[w.mat];
    const int i0 = (int)w.ti * T;
    const int j0 = (int)w.tj * T;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = wave / WN;
    const int wj = wave % WN;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const bf16* Psrc;
    const bf16* Qsrc;
    int ldp, ldq, K;
    if (MODE == NS_GRAM) {
        Psrc = xin + d.x_off + (int64_t)i0 * d.n_pad;
        Qsrc = xin + d.x_off + (int64_t)j0 * d.n_pad;
        ldp = ldq = d.n_pad;
        K = d.n_pad;
    } else if (MODE == NS_POLY) {
        Psrc = ain + d.a_off + (int64_t)i0 * d.m_pad;
        Qsrc = ain + d.a_off + (int64_t)j0 * d.m_pad;
        ldp = ldq = d.m_pad;
        K = d.m_pad;
    } else {
        Psrc = ain + d.a_off + (int64_t)i0 * d.m_pad;  // rows of B
        Qsrc = xin + d.x_off + j0;                     // columns j0.. of X; row k = contraction
        ldp = d.m_pad;
        ldq = d.n_pad;
        K = d.m_pad;
    }
    // buffer ranges: the tile's rows (P, and Q for Gram / poly) or all K rows of X
    const __amdgpu_buffer_rsrc_t rp = rsrc(Psrc, (uint32_t)(T * ldp * 2));
    const __amdgpu_buffer_rsrc_t rq =
        rsrc(Qsrc, (uint32_t)((MODE == NS_UPDATE ? K * ldq : T * ldq) * 2));
    // lane parts of the global offsets (bytes)
    const int vp = (tid >> 3) * ldp * 2 + (tid & 7) * 16;
    const int vq = MODE == NS_UPDATE ? (tid / (T / 8)) * ldq * 2 + (tid % (T / 8)) * 16
                                     : (tid >> 3) * ldq * 2 + (tid & 7) * 16;
    // lane parts of the LDS store offsets
    const int sp = (tid >> 3) * KROW + (tid & 7) * 16;
    const int sq = MODE == NS_UPDATE ? (tid / (T / 8)) * LY::XROW + (tid % (T / 8)) * 16 : sp;

    uint4 preg[NCH];
    uint4 qreg[NCH];

    // global -> registers for one stage; which = 1: P chunks, 2: Q chunks, 3: both
    auto load_stage = [&](int k0, int which) {
        if (which & 1) {
#pragma unroll
            for (int q = 0; q < NCH; ++q) preg[q] = bload(rp, vp, (q * PSTEP * ldp + k0) * 2);
        }
        if (which & 2) {
#pragma unroll
            for (int q = 0; q < NCH; ++q) {
                if (MODE != NS_UPDATE)
                    qreg[q] = bload(rq, vq, (q * PSTEP * ldq + k0) * 2);
                else
                    qreg[q] = bload(rq, vq, (q * XSTEP + k0) * ldq * 2);
            }
        }
    };

    auto store_stage = [&](int s) {
        char* P = smem + s * LY::STAGE;
        char* Q = P + LY::KTILE;
#pragma unroll
        for (int q = 0; q < NCH; ++q) *reinterpret_cast<uint4*>(P + sp + q * PSTEP * KROW) = preg[q];
#pragma unroll
        for (int q = 0; q < NCH; ++q) {
            if (MODE != NS_UPDATE)
                *reinterpret_cast<uint4*>(Q + sq + q * PSTEP * KROW) = qreg[q];
            else
                *reinterpret_cast<uint4*>(Q + sq + q * XSTEP * LY::XROW) = qreg[q];
        }
    };

    f32x16 acc[FRI][FRJ];
#pragma unroll
    for (int a = 0; a < FRI; ++a)
#pragma unroll
        for (int b = 0; b < FRJ; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // lane bases of the fragment reads
    const int fp = (wi * WTM + l32) * KROW + 16 * hi;         // + f 32 KROW + 32 ks
    const int fq = (wj * WTN + l32) * KROW + 16 * hi;
    const int g16 = lane >> 4;
    const int s16 = lane & 15;
    const int ft = (8 * (g16 >> 1) + (s16 >> 2)) * LY::XROW + 2 * (wj * WTN + 16 * (g16 & 1) + 4 * (s16 & 3));
    // + (16 ks + 4 h) XROW + 64 f

    // two fragment sets, alternating between k16 sub-steps
    bf16x8 pfr[2][FRI], qfr[2][FRJ];
    auto read_frags = [&](const char* P, int ks, int set) {
        const char* Q = P + LY::KTILE;
#pragma unroll
        for (int f = 0; f < FRI; ++f)
            pfr[set][f] = *reinterpret_cast<const bf16x8*>(P + fp + f * 32 * KROW + 32 * ks);
#pragma unroll
        for (int f = 0; f < FRJ; ++f) {
            if (MODE != NS_UPDATE) {
                qfr[set][f] = *reinterpret_cast<const bf16x8*>(Q + fq + f * 32 * KROW + 32 * ks);
            } else {
                const bf16x4 lo = tr_read(Q + ft + (16 * ks) * LY::XROW + 64 * f);
                const bf16x4 up = tr_read(Q + ft + (16 * ks + 4) * LY::XROW + 64 * f);
                qfr[set][f] = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        }
    };
    constexpr int NREAD = FRI + (MODE == NS_UPDATE ? 2 : 1) * FRJ;  // LDS read instructions per sub-step

    // One K stage. MORE: a next stage exists (its loads and LDS writes are
    // interleaved here); the last stage is peeled so the steady-state loop
    // body has no branches for the scheduler to stop at.
    auto mfma_block = [&](int set, int lo, int hi_) {
#pragma unroll
        for (int f = lo; f < hi_; ++f) {
            const int fi = f / FRJ, fj = f % FRJ;
            acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfr[set][fj], pfr[set][fi], acc[fi][fj], 0, 0, 0);
        }
    };
    auto stage = [&](int kt, auto more_c) {
        constexpr bool MORE = decltype(more_c)::value;
        constexpr int NW = 2 * NCH;
        constexpr int NF = FRI * FRJ;
        const char* P = smem + (kt & 1) * LY::STAGE;
#pragma unroll
        for (int ks = 0; ks < BK / 16 - 1; ++ks) {
            const int set = ks & 1;
            read_frags(P, ks + 1, set ^ 1);
            // the next stage's global loads are spread over sub-steps 0 and 1
            if constexpr (MORE) {
                if (ks == 0) load_stage((kt + 1) * BK, 1);
                if (ks == 1) load_stage((kt + 1) * BK, 2);
            }
            mfma_block(set, 0, NF);
            // interleave: one MFMA, then one LDS read / global load
#pragma unroll
            for (int i = 0; i < NF; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                if (MORE && ks < 2 && i < NCH) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
        }
        // last sub-step: half its MFMAs carry the next stage's LDS writes; the
        // barrier comes next, and the next stage's first fragment reads run
        // under the other half
        constexpr int SL = (BK / 16 - 1) & 1;
        if constexpr (MORE) {
            store_stage((kt & 1) ^ 1);
            mfma_block(SL, 0, NF / 2);
#pragma unroll
            for (int i = 0; i < NF / 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < NW) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
            }
            if (NW > NF / 2) __builtin_amdgcn_sched_group_barrier(0x200, NW - NF / 2, 0);
            __syncthreads();
            read_frags(smem + ((kt + 1) & 1) * LY::STAGE, 0, 0);
            mfma_block(SL, NF / 2, NF);
#pragma unroll
            for (int i = 0; i < NF / 2; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (i < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if (NREAD > NF / 2) __builtin_amdgcn_sched_group_barrier(0x100, NREAD - NF / 2, 0);
        } else {
            mfma_block(SL, 0, NF);
            __syncthreads();
        }
    };

    const int nk = K / BK;
    load_stage(0, 3);
    store_stage(0);
    __syncthreads();
    read_frags(smem, 0, 0);
    for (int kt = 0; kt < nk - 1; ++kt) stage(kt, std::true_type{});
    stage(nk - 1, std::false_type{});

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

    // Output tiles are staged in LDS as bf16 rows of EROW bytes (2T + 8: 32
    // consecutive rows start in distinct 8-byte bank slots) and leave as
    // whole cache lines; the polynomial's A tile comes in the same way.
    constexpr int EROW = 2 * T + 8;
    static_assert(T * EROW <= 2 * LY::STAGE, "staged tile must fit in LDS");
    auto lds64 = [&](int off) -> uint2& { return *reinterpret_cast<uint2*>(smem + off); };

    if (MODE == NS_POLY) {
        const bf16* Asrc = ain + d.a_off + (int64_t)i0 * d.m_pad + j0;
        const __amdgpu_buffer_rsrc_t ra = rsrc(Asrc, (uint32_t)(T * d.m_pad * 2));
        constexpr int CPR = T / 8;                   // 16-byte chunks per row
        constexpr int NE = T * CPR / NT;             // chunks per thread
        const int er = tid / CPR, ec = tid % CPR;
        constexpr int RSTEP = NT / CPR;
#pragma unroll
        for (int b0 = 0; b0 < NE; b0 += NCH) {
#pragma unroll
            for (int q = 0; q < NCH; ++q)
                preg[q] = bload(ra, er * d.m_pad * 2 + ec * 16, (b0 + q) * RSTEP * d.m_pad * 2);
#pragma unroll
            for (int q = 0; q < NCH; ++q) {
                const int off = (er + (b0 + q) * RSTEP) * EROW + ec * 16;
                lds64(off) = make_uint2(preg[q].x, preg[q].y);
                lds64(off + 8) = make_uint2(preg[q].z, preg[q].w);
            }
        }
        __syncthreads();
    }

    float rsq[FRI];
#pragma unroll
    for (int f = 0; f < FRI; ++f) rsq[f] = 0.f;

    uint2 ev[FRI][FRJ][4];
#pragma unroll
    for (int fi = 0; fi < FRI; ++fi) {
        const int il = wi * WTM + fi * 32 + l32;
#pragma unroll
        for (int fj = 0; fj < FRJ; ++fj) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int jl = wj * WTN + fj * 32 + 8 * g + 4 * hi;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[fi][fj][4 * g + e];
                if (MODE == NS_POLY) {
                    // P = a I + b A + c A A: the a X term of the update rides on P's diagonal
                    const uint2 in = lds64(il * EROW + 2 * jl);
                    v[0] = fmaf(cb, bf16_lo(in.x), cc * v[0]);
                    v[1] = fmaf(cb, bf16_hi(in.x), cc * v[1]);
                    v[2] = fmaf(cb, bf16_lo(in.y), cc * v[2]);
                    v[3] = fmaf(cb, bf16_hi(in.y), cc * v[3]);
                    if (w.ti == w.tj) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (jl + e == il) v[e] += ca;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] *= alpha;
                }
                uint2 ow;
                ow.x = pack_bf16x2(v[0], v[1]);
                ow.y = pack_bf16x2(v[2], v[3]);
                ev[fi][fj][g] = ow;
                if (MODE == NS_UPDATE && ROWSTATS) {
                    const float r0 = bf16_lo(ow.x), r1 = bf16_hi(ow.x), r2 = bf16_lo(ow.y), r3 = bf16_hi(ow.y);
                    rsq[fi] = fmaf(r0, r0, rsq[fi]);
                    rsq[fi] = fmaf(r1, r1, rsq[fi]);
                    rsq[fi] = fmaf(r2, r2, rsq[fi]);
                    rsq[fi] = fmaf(r3, r3, rsq[fi]);
                }
            }
        }
    }
    if (MODE == NS_POLY) __syncthreads();  // the staged A tile is read; LDS is reused below
#pragma unroll
    for (int fi = 0; fi < FRI; ++fi)
#pragma unroll
        for (int fj = 0; fj < FRJ; ++fj)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                lds64((wi * WTM + fi * 32 + l32) * EROW + 2 * (wj * WTN + fj * 32 + 8 * g + 4 * hi)) = ev[fi][fj][g];
    __syncthreads();

    // the tile itself: each thread moves 16-byte row chunks, a wave covers whole rows
    {
        bf16* obase = MODE == NS_UPDATE ? out + d.x_off + (int64_t)i0 * d.n_pad + j0
                                        : out + d.a_off + (int64_t)i0 * d.m_pad + j0;
        const int ld = MODE == NS_UPDATE ? d.n_pad : d.m_pad;
        constexpr int CPR = T / 8;
#pragma unroll
        for (int q = 0; q < T * CPR / NT; ++q) {
            const int id = tid + NT * q;
            const int r = id / CPR, c = id % CPR;
            const uint2 lo = lds64(r * EROW + 16 * c);
            const uint2 up = lds64(r * EROW + 16 * c + 8);
            *reinterpret_cast<uint4*>(obase + (int64_t)r * ld + 8 * c) = make_uint4(lo.x, lo.y, up.x, up.y);
        }
    }
    if (MODE != NS_UPDATE && w.ti != w.tj) {
        // the mirror tile, read column-wise with ds_read_b64_tr_b16: in each
        // 16-lane group G, lane s = 4e + q points at row IB + 16G + 4q + e of
        // column chunk JB, so lane 4q + c receives rows IB + 16G + 4q .. +3 of
        // column JB + c; the 16 lanes with the same c then hold 64 consecutive
        // entries (one 128-byte line) of mirror row JB + c.
        bf16* mbase = out + d.a_off + (int64_t)j0 * d.m_pad + i0;
        const int G = lane >> 4, sl = lane & 15;
        const int sup_row = 16 * G + 4 * (sl & 3) + (sl >> 2);
        const int rc = sl & 3, rq = sl >> 2;
        constexpr int NIT = (T / 4) * (T / 64) / NWV;  // instructions per wave
#pragma unroll 4
        for (int k = 0; k < NIT; ++k) {
            const int it = wave + NWV * k;
            const int JB = 4 * (it % (T / 4));
            const int IB = 64 * (it / (T / 4));
            const bf16x4 v = tr_read(smem + (IB + sup_row) * EROW + 2 * JB);
            *reinterpret_cast<bf16x4*>(mbase + (int64_t)(JB + rc) * d.m_pad + IB + 16 * G + 4 * rq) = v;
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
    if (mode == NS_GRAM)
        k_ns_big<T, WN, NS_GRAM, false><<<n, NT, 0, L.stream>>>(L.mats, wl, x, a, o, ca, cb, cc, first, L.partials,
                                                                L.ss, L.scale, L.status, eps, L.rowpart);
    else if (mode == NS_POLY)
        k_ns_big<T, WN, NS_POLY, false><<<n, NT, 0, L.stream>>>(L.mats, wl, x, a, o, ca, cb, cc, first, L.partials,
                                                                L.ss, L.scale, L.status, eps, L.rowpart);
    else if (rowstats)
        k_ns_big<T, WN, NS_UPDATE, true><<<n, NT, 0, L.stream>>>(L.mats, wl, x, a, o, ca, cb, cc, first,
                                                                 L.partials, L.ss, L.scale, L.status, eps, L.rowpart);
    else
        k_ns_big<T, WN, NS_UPDATE, false><<<n, NT, 0, L.stream>>>(L.mats, wl, x, a, o, ca, cb, cc, first,
                                                                  L.partials, L.ss, L.scale, L.status, eps,
                                                                  L.rowpart);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_stage_big(const LaunchCtx& L, const GemmList& G, int mode, const void* xin, const void* ain,
                               void* out, float ca, float cb, float cc, int first, float eps, int rowstats) {
    if (G.T == 256) return launch_big_T<256, 4>(L, G, mode, xin, ain, out, ca, cb, cc, first, eps, rowstats);
    return launch_big_T<128, 2>(L, G, mode, xin, ain, out, ca, cb, cc, first, eps, rowstats);
}

}  // namespace muon
