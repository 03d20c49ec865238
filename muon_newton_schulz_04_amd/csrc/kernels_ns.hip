// Newton–Schulz iteration as grouped MFMA GEMMs over a work list of tiles.
//
// Source: [P4] "modded-nanogpt 50B-token 长时程训练实验解析" section
// "从源码看 Muon 的分布式正交化实现": the quintic iteration with
// (a, b, c) = (3.4445, -4.7750, 2.0315) on the normalised, short-side X,
// run in bf16. It is computed here in the algebraically equal factored form
//     A = X X^T,   B = b A + c A A,   X <- a X + B X
// with three kernels per iteration:
//   GRAM    A = alpha X X^T            (only tiles ti <= tj; the mirror tile is
//                                       written from the same registers)
//   POLY    B = b A + c A A^T          (A symmetric; the polynomial is the epilogue)
//   UPDATE  X' = alpha (a X + B X)     (X enters as the column-side operand,
//                                       transposed on its way into LDS; a X is
//                                       added in the epilogue, before rounding)
// bf16 operands with fp32 accumulation (v_mfma_f32_32x32x16_bf16), or fp32
// throughout (v_mfma_f32_32x32x2_f32) in the fp32 mode. Every output is
// rounded once to the storage type.
//
// Tiles: T x T output per 256-thread workgroup, four waves in a 2 x 2 grid,
// each wave T/2 x T/2 as (T/64)^2 32x32 MFMA blocks. K is staged through
// double-buffered LDS in slices of 128 bytes per row. Buffers are padded to
// multiples of T, so there are no bounds checks: the zero padding stays zero
// through every iteration.
//
// The MFMA is fed the column-side tile as its A operand and the row-side tile
// as its B operand, so each lane ends up holding four consecutive columns of
// one output row (8-byte bf16 stores, 8-byte loads of the epilogue inputs).

#include "kernel_common.hpp"
#include "launch.hpp"

namespace muon {

namespace {

template <typename ET>
struct Traits;

template <>
struct Traits<bf16> {
    static constexpr int BK = 64;   // k per LDS stage (128 bytes per row)
    static constexpr int VEC = 8;   // elements per 16-byte chunk
    static constexpr int PAD = 8;   // row pad (16 bytes) against bank conflicts
};

template <>
struct Traits<float> {
    static constexpr int BK = 32;
    static constexpr int VEC = 4;
    static constexpr int PAD = 4;
};

template <typename ET>
__device__ __forceinline__ void store4(ET* dst, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store4<bf16>(bf16* dst, float a, float b, float c, float d) {
    uint2 w;
    w.x = pack_bf16x2(a, b);
    w.y = pack_bf16x2(c, d);
    *reinterpret_cast<uint2*>(dst) = w;
}

template <>
__device__ __forceinline__ void store4<float>(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}

// value after rounding to the storage type
template <typename ET>
__device__ __forceinline__ float rounded(float x);

template <>
__device__ __forceinline__ float rounded<bf16>(float x) {
    return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, (bf16)x) << 16);
}

template <>
__device__ __forceinline__ float rounded<float>(float x) {
    return x;
}

template <typename ET>
__device__ __forceinline__ void load4(const ET* src, float* v);

template <>
__device__ __forceinline__ void load4<bf16>(const bf16* src, float* v) {
    const uint2 w = *reinterpret_cast<const uint2*>(src);
    v[0] = bf16_lo(w.x);
    v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y);
    v[3] = bf16_hi(w.y);
}

template <>
__device__ __forceinline__ void load4<float>(const float* src, float* v) {
    const float4 w = *reinterpret_cast<const float4*>(src);
    v[0] = w.x;
    v[1] = w.y;
    v[2] = w.z;
    v[3] = w.w;
}

template <typename ET>
__device__ __forceinline__ void store_scalar(ET* dst, float v) {
    *dst = (ET)v;
}

template <typename ET, int T, int MODE>
__global__ __launch_bounds__(kThreads) void k_ns(const MatDesc* __restrict__ mats, const TileWork* __restrict__ work,
                                                 const ET* __restrict__ xin, const ET* __restrict__ ain,
                                                 ET* __restrict__ out, float ca, float cb, float cc, int first,
                                                 const float* __restrict__ partials, float* __restrict__ ss_arr,
                                                 float* __restrict__ scale_arr, int32_t* __restrict__ status_arr,
                                                 float eps, float* __restrict__ rowpart, int rowstats) {
    using TR = Traits<ET>;
    constexpr int BK = TR::BK;
    constexpr int VEC = TR::VEC;
    constexpr int LROW = BK + TR::PAD;
    constexpr int WT = T / 2;
    constexpr int FR = WT / 32;
    constexpr int CPR = BK / VEC;                 // 16-byte chunks per row per stage (8)
    constexpr int NP = (T * CPR) / kThreads;      // row-major chunks per thread
    constexpr int JG = T / VEC;                   // column groups of the transposed loader
    constexpr int NSB = (BK / 4) * JG;            // 4 x VEC sub-blocks per stage
    static_assert(NP >= 1 && (T * CPR) % kThreads == 0, "tile / thread mismatch");
    static_assert(NSB <= kThreads, "one transposed sub-block per thread at most");

    __shared__ __attribute__((aligned(16))) ET smem[2][2][T][LROW];
    __shared__ float red[4];

    const TileWork w = work[blockIdx.x];
    const MatDesc d = mats[w.mat];
    const int i0 = (int)w.ti * T;
    const int j0 = (int)w.tj * T;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = wave >> 1;
    const int wj = wave & 1;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const ET* Psrc;
    const ET* Qsrc;
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
        Qsrc = xin + d.x_off + j0;                     // columns j0.. of X, row k = contraction
        ldp = d.m_pad;
        ldq = d.n_pad;
        K = d.m_pad;
    }

    uint4 preg[NP];
    uint4 qreg[MODE == NS_UPDATE ? 4 : NP];

    auto load_stage = [&](int k0) {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int c = tid + kThreads * q;
            const int row = c / CPR;
            const int col = (c % CPR) * VEC;
            preg[q] = *reinterpret_cast<const uint4*>(Psrc + (int64_t)row * ldp + k0 + col);
        }
        if (MODE != NS_UPDATE) {
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                const int c = tid + kThreads * q;
                const int row = c / CPR;
                const int col = (c % CPR) * VEC;
                qreg[q] = *reinterpret_cast<const uint4*>(Qsrc + (int64_t)row * ldq + k0 + col);
            }
        } else if (tid < NSB) {
            const int jg = tid % JG;
            const int kg = tid / JG;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                qreg[r] = *reinterpret_cast<const uint4*>(Qsrc + (int64_t)(k0 + 4 * kg + r) * ldq + VEC * jg);
        }
    };

    auto store_stage = [&](int s) {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
            const int c = tid + kThreads * q;
            const int row = c / CPR;
            const int col = (c % CPR) * VEC;
            *reinterpret_cast<uint4*>(&smem[s][0][row][col]) = preg[q];
        }
        if (MODE != NS_UPDATE) {
#pragma unroll
            for (int q = 0; q < NP; ++q) {
                const int c = tid + kThreads * q;
                const int row = c / CPR;
                const int col = (c % CPR) * VEC;
                *reinterpret_cast<uint4*>(&smem[s][1][row][col]) = qreg[q];
            }
        } else if (tid < NSB) {
            const int jg = tid % JG;
            const int kg = tid / JG;
            if constexpr (sizeof(ET) == 2) {
                // 4 rows (k) x 8 columns (j) of bf16 -> 8 column vectors of 4 k
                const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&qreg[0]);
                const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&qreg[1]);
                const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&qreg[2]);
                const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&qreg[3]);
#pragma unroll
                for (int dw = 0; dw < 4; ++dw) {
                    uint2 lo, hi2;
                    lo.x = (r0[dw] & 0xffffu) | (r1[dw] << 16);
                    lo.y = (r2[dw] & 0xffffu) | (r3[dw] << 16);
                    hi2.x = (r0[dw] >> 16) | (r1[dw] & 0xffff0000u);
                    hi2.y = (r2[dw] >> 16) | (r3[dw] & 0xffff0000u);
                    *reinterpret_cast<uint2*>(&smem[s][1][VEC * jg + 2 * dw][4 * kg]) = lo;
                    *reinterpret_cast<uint2*>(&smem[s][1][VEC * jg + 2 * dw + 1][4 * kg]) = hi2;
                }
            } else {
                const float* r0 = reinterpret_cast<const float*>(&qreg[0]);
                const float* r1 = reinterpret_cast<const float*>(&qreg[1]);
                const float* r2 = reinterpret_cast<const float*>(&qreg[2]);
                const float* r3 = reinterpret_cast<const float*>(&qreg[3]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    *reinterpret_cast<float4*>(&smem[s][1][VEC * jg + jj][4 * kg]) =
                        make_float4(r0[jj], r1[jj], r2[jj], r3[jj]);
            }
        }
    };

    f32x16 acc[FR][FR];
#pragma unroll
    for (int a = 0; a < FR; ++a)
#pragma unroll
        for (int b = 0; b < FR; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    const int nk = K / BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int s = kt & 1;
        if (kt + 1 < nk) load_stage((kt + 1) * BK);
        if constexpr (sizeof(ET) == 2) {
#pragma unroll
            for (int ks = 0; ks < BK / 16; ++ks) {
                bf16x8 qf[FR], pf[FR];
#pragma unroll
                for (int f = 0; f < FR; ++f) {
                    qf[f] = *reinterpret_cast<const bf16x8*>(&smem[s][1][wj * WT + f * 32 + l32][ks * 16 + 8 * hi]);
                    pf[f] = *reinterpret_cast<const bf16x8*>(&smem[s][0][wi * WT + f * 32 + l32][ks * 16 + 8 * hi]);
                }
#pragma unroll
                for (int fi = 0; fi < FR; ++fi)
#pragma unroll
                    for (int fj = 0; fj < FR; ++fj)
                        acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[fj], pf[fi], acc[fi][fj], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < BK / 8; ++ks) {
                f32x4 qf[FR], pf[FR];
#pragma unroll
                for (int f = 0; f < FR; ++f) {
                    qf[f] = *reinterpret_cast<const f32x4*>(&smem[s][1][wj * WT + f * 32 + l32][ks * 8 + 4 * hi]);
                    pf[f] = *reinterpret_cast<const f32x4*>(&smem[s][0][wi * WT + f * 32 + l32][ks * 8 + 4 * hi]);
                }
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int fi = 0; fi < FR; ++fi)
#pragma unroll
                        for (int fj = 0; fj < FR; ++fj)
                            acc[fi][fj] =
                                __builtin_amdgcn_mfma_f32_32x32x2f32(qf[fj][t], pf[fi][t], acc[fi][fj], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) store_stage(s ^ 1);
        __syncthreads();
    }

    // ---------------- epilogue ----------------
    float alpha = 1.0f;
    if (MODE == NS_GRAM && first) {
        float acc_p = 0.f;
        for (int p = tid; p < d.ew_count; p += kThreads) acc_p += partials[d.ew_start + p];
        const float total = block_sum_256(acc_p, red);
        const float s = 1.0f / (sqrtf(total) + eps);
        alpha = s * s;
        if (w.ti == 0 && w.tj == 0 && tid == 0) {
            ss_arr[w.mat] = total;
            scale_arr[w.mat] = s;
            status_arr[w.mat] = (isfinite(total) ? 0 : 1);
        }
    }
    if (MODE == NS_UPDATE && first) alpha = scale_arr[w.mat];

    float rsq[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) rsq[f] = 0.f;

#pragma unroll
    for (int fi = 0; fi < FR; ++fi) {
        const int i = i0 + wi * WT + fi * 32 + l32;
#pragma unroll
        for (int fj = 0; fj < FR; ++fj) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int jb = j0 + wj * WT + fj * 32 + 8 * g + 4 * hi;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[fi][fj][4 * g + e];
                if (MODE == NS_GRAM) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] *= alpha;
                    ET* o = out + d.a_off;
                    store4<ET>(o + (int64_t)i * d.m_pad + jb, v[0], v[1], v[2], v[3]);
                    if (w.ti != w.tj) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) store_scalar<ET>(o + (int64_t)(jb + e) * d.m_pad + i, v[e]);
                    }
                } else if (MODE == NS_POLY) {
                    // B = b A + c A A
                    float av[4];
                    load4<ET>(ain + d.a_off + (int64_t)i * d.m_pad + jb, av);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = fmaf(cb, av[e], cc * v[e]);
                    ET* o = out + d.a_off;
                    store4<ET>(o + (int64_t)i * d.m_pad + jb, v[0], v[1], v[2], v[3]);
                    if (w.ti != w.tj) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) store_scalar<ET>(o + (int64_t)(jb + e) * d.m_pad + i, v[e]);
                    }
                } else {
                    // X' = alpha (a X + B X)
                    float xv[4];
                    load4<ET>(xin + d.x_off + (int64_t)i * d.n_pad + jb, xv);
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = fmaf(ca, xv[e], v[e]) * alpha;
                    store4<ET>(out + d.x_off + (int64_t)i * d.n_pad + jb, v[0], v[1], v[2], v[3]);
                    if (rowstats) {
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const float rv = rounded<ET>(v[e]);
                            rsq[fi] = fmaf(rv, rv, rsq[fi]);
                        }
                    }
                }
            }
        }
    }

    if (MODE == NS_UPDATE && rowstats) {
        // lanes l and l ^ 32 hold the same row; waves (wi, 0) and (wi, 1) split its columns
        float* rl = reinterpret_cast<float*>(&smem[0][0][0][0]);  // [2 wi][2 wj][WT]
#pragma unroll
        for (int f = 0; f < FR; ++f) rsq[f] += __shfl_xor(rsq[f], 32, 64);
        if (hi == 0) {
#pragma unroll
            for (int f = 0; f < FR; ++f) rl[(wi * 2 + wj) * WT + f * 32 + l32] = rsq[f];
        }
        __syncthreads();
        if (tid < T) {
            const int wr = tid / WT;
            const int rr = tid % WT;
            const float sum = rl[(wr * 2 + 0) * WT + rr] + rl[(wr * 2 + 1) * WT + rr];
            rowpart[d.rowpart_off + (int64_t)w.tj * d.m_pad + i0 + tid] = sum;
        }
    }
}

template <typename ET, int T>
hipError_t launch_T(const LaunchCtx& L, const GemmList& G, int mode, const void* xin, const void* ain, void* out,
                    float ca, float cb, float cc, int first, float eps, int rowstats) {
    const TileWork* wl = mode == NS_GRAM ? G.gram : mode == NS_POLY ? G.poly : G.update;
    const int n = mode == NS_GRAM ? G.n_gram : mode == NS_POLY ? G.n_poly : G.n_update;
    if (n == 0) return hipSuccess;
    const ET* x = (const ET*)xin;
    const ET* a = (const ET*)ain;
    ET* o = (ET*)out;
    if (mode == NS_GRAM)
        k_ns<ET, T, NS_GRAM><<<n, kThreads, 0, L.stream>>>(L.mats, wl, x, a, o, ca, cb, cc, first, L.partials, L.ss,
                                                           L.scale, L.status, eps, L.rowpart, rowstats);
    else if (mode == NS_POLY)
        k_ns<ET, T, NS_POLY><<<n, kThreads, 0, L.stream>>>(L.mats, wl, x, a, o, ca, cb, cc, first, L.partials, L.ss,
                                                           L.scale, L.status, eps, L.rowpart, rowstats);
    else
        k_ns<ET, T, NS_UPDATE><<<n, kThreads, 0, L.stream>>>(L.mats, wl, x, a, o, ca, cb, cc, first, L.partials,
                                                             L.ss, L.scale, L.status, eps, L.rowpart, rowstats);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ns_stage(const LaunchCtx& L, const GemmList& G, int mode, const void* xin, const void* ain,
                           void* out, float ca, float cb, float cc, int first, float eps, int rowstats) {
    if (L.fp32) {
        if (G.T == 128) return launch_T<float, 128>(L, G, mode, xin, ain, out, ca, cb, cc, first, eps, rowstats);
        return launch_T<float, 64>(L, G, mode, xin, ain, out, ca, cb, cc, first, eps, rowstats);
    }
    if (G.T == 128) return launch_T<bf16, 128>(L, G, mode, xin, ain, out, ca, cb, cc, first, eps, rowstats);
    return launch_T<bf16, 64>(L, G, mode, xin, ain, out, ca, cb, cc, first, eps, rowstats);
}

}  // namespace muon
