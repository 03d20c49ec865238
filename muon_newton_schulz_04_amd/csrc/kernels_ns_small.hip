// The whole bf16 Newton–Schulz of a small matrix in one workgroup (gfx950).
//
// Matrices whose short side is at most 64 (m_pad = 64) and whose padded long
// side n_pad is at most 512 are too small for the tiled GEMM launches: one
// 64 x 64 output tile per GEMM and 15 launches a step leave the chip idle.
// Here one workgroup of 4 waves takes one such matrix through every
// iteration with X, A and B resident in LDS:
//   load X~ (bf16, canonical, padded) -> LDS
//   per iteration k:  A = R(alpha X X^T)            alpha = s^2 (k = 0) or 1
//                     B = R(b_k A + c_k A A)
//                     X = R(beta (a_k X + B X))      beta = s (k = 0) or 1
//   store X (the Newton–Schulz output) and, for NorMuon, the row sums of X^2
// with R the bf16 rounding and fp32 accumulation, i.e. exactly the rounding
// points of the tiled path, and s = 1 / (||u||_F + eps) from the momentum
// kernel's per-tile partial sums.
//
// GEMMs are v_mfma_f32_32x32x16_bf16 over 32 x 32 blocks: the 64 x 64
// symmetric A and B are computed as three blocks (waves 0, 1, 3) with the
// off-diagonal block mirrored, and X' = a X + B X as 32 x 32 blocks of all
// four waves (a X read from the resident X, added in fp32 before rounding).
// Lane (l32, hi) of a block holds C[l32][8 g + 4 hi + e] in acc[4 g + e], as
// in the tiled kernels.
//
// Source of the iteration: [P4] "modded-nanogpt 50B-token 长时程训练实验解析",
// section "从源码看 Muon 的分布式正交化实现" (quintic Newton–Schulz in bf16).

#include "kernel_common.hpp"
#include "launch.hpp"

namespace muon {

namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int SM = 64;              // m_pad of a small matrix
constexpr int AROW = 2 * SM + 16;   // bytes per padded row of A / B

__device__ __forceinline__ bf16x4 tr_read(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4*)(LDS_AS char*)p);
}

__device__ __forceinline__ bf16x8 ld8(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }

__global__ __launch_bounds__(kThreads) void k_ns_small(const MatDesc* __restrict__ mats,
                                                      const int32_t* __restrict__ list,
                                                      const bf16* __restrict__ xin, bf16* __restrict__ out,
                                                      NsCoeffs co, const float* __restrict__ partials,
                                                      float* __restrict__ ss_arr, float* __restrict__ scale_arr,
                                                      int32_t* __restrict__ status_arr,
                                                      float* __restrict__ rowpart, int rowstats) {
    extern __shared__ __attribute__((aligned(16))) char sm[];
    __shared__ float red[4];

    const int mi = list[blockIdx.x];
    const MatDesc d = mats[mi];
    const int np = d.n_pad;
    const int XR = 2 * np + 16;  // bytes per padded row of X
    char* Xb[2] = {sm, sm + SM * XR};
    char* A = sm + 2 * SM * XR;
    char* P = A + SM * AROW;  // B = b A + c A A

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wi = wave >> 1;
    const int wj = wave & 1;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const bool sym = !(wi == 1 && wj == 0);  // blocks (0,0), (0,1), (1,1) of A and B

    // X~ -> LDS (16-byte chunks, rows padded)
    const int cpr = np / 8;
    for (int id = tid; id < SM * cpr; id += kThreads) {
        const int r = id / cpr, c = id - r * cpr;
        *reinterpret_cast<uint4*>(Xb[0] + r * XR + 16 * c) =
            *reinterpret_cast<const uint4*>(xin + d.x_off + (int64_t)r * np + 8 * c);
    }
    // s = 1 / (||u||_F + eps) from the momentum kernel's per-tile sums of u^2
    float part = 0.f;
    for (int p = tid; p < d.ew_count; p += kThreads) part += partials[d.ew_start + p];
    part = wave_sum(part);
    if (lane == 0) red[wave] = part;
    __syncthreads();
    const float total = ((red[0] + red[1]) + red[2]) + red[3];
    const float s = 1.0f / (sqrtf(total) + co.eps);
    if (tid == 0) {
        ss_arr[mi] = total;
        scale_arr[mi] = s;
        status_arr[mi] = isfinite(total) ? 0 : 1;
    }

    // writes the lane's 32 x 32 block entries (rounded) at row-major base with
    // stride ld; mirror: also at the transposed position
    auto put_block = [&](char* base, int ld, const float (&v)[16], int i, int j0, bool mirror) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int j = j0 + 8 * g + 4 * hi;
            uint2 w;
            w.x = pack_bf16x2(v[4 * g + 0], v[4 * g + 1]);
            w.y = pack_bf16x2(v[4 * g + 2], v[4 * g + 3]);
            *reinterpret_cast<uint2*>(base + i * ld + 2 * j) = w;
            if (mirror) {
                *reinterpret_cast<uint16_t*>(base + (j + 0) * ld + 2 * i) = (uint16_t)(w.x & 0xffffu);
                *reinterpret_cast<uint16_t*>(base + (j + 1) * ld + 2 * i) = (uint16_t)(w.x >> 16);
                *reinterpret_cast<uint16_t*>(base + (j + 2) * ld + 2 * i) = (uint16_t)(w.y & 0xffffu);
                *reinterpret_cast<uint16_t*>(base + (j + 3) * ld + 2 * i) = (uint16_t)(w.y >> 16);
            }
        }
    };

    const int steps = co.steps;
    for (int k = 0; k < steps; ++k) {
        const char* X = Xb[k & 1];
        char* Xn = Xb[(k + 1) & 1];
        const float ca = co.c[k][0], cb = co.c[k][1], cc = co.c[k][2];
        const int i = wi * 32 + l32;  // the lane's row in its block
        // ---- A = alpha X X^T ----
        if (sym) {
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
            for (int k0 = 0; k0 < np; k0 += 16) {
                const bf16x8 pf = ld8(X + (wi * 32 + l32) * XR + 2 * (k0 + 8 * hi));
                const bf16x8 qf = ld8(X + (wj * 32 + l32) * XR + 2 * (k0 + 8 * hi));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, pf, acc, 0, 0, 0);
            }
            const float alpha = k == 0 ? s * s : 1.0f;
            float v[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) v[r] = acc[r] * alpha;
            put_block(A, AROW, v, i, wj * 32, wi != wj);
        }
        __syncthreads();
        // ---- B = b A + c A A (A symmetric: (A A)_ij = sum_k A_ik A_jk) ----
        if (sym) {
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int k0 = 0; k0 < SM; k0 += 16) {
                const bf16x8 pf = ld8(A + (wi * 32 + l32) * AROW + 2 * (k0 + 8 * hi));
                const bf16x8 qf = ld8(A + (wj * 32 + l32) * AROW + 2 * (k0 + 8 * hi));
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, pf, acc, 0, 0, 0);
            }
            float v[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int j = wj * 32 + 8 * g + 4 * hi;
                const uint2 a2 = *reinterpret_cast<const uint2*>(A + i * AROW + 2 * j);
                const float av[4] = {bf16_lo(a2.x), bf16_hi(a2.x), bf16_lo(a2.y), bf16_hi(a2.y)};
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * g + e] = fmaf(cb, av[e], cc * acc[4 * g + e]);
            }
            put_block(P, AROW, v, i, wj * 32, wi != wj);
        }
        __syncthreads();
        // ---- X' = beta (a X + B X), 64-column chunks, wave (wi, wj): rows wi, cols wj of a chunk ----
        {
            const float beta = k == 0 ? s : 1.0f;
            const int g16 = lane >> 4, s16 = lane & 15;
            const int trow = 8 * (g16 >> 1) + (s16 >> 2);
            for (int jc = 0; jc < np; jc += 64) {
                const int cb0 = jc + wj * 32;
                f32x16 acc;
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
                for (int k0 = 0; k0 < SM; k0 += 16) {
                    const bf16x8 pf = ld8(P + (wi * 32 + l32) * AROW + 2 * (k0 + 8 * hi));
                    const char* q = X + (k0 + trow) * XR + 2 * (cb0 + 16 * (g16 & 1) + 4 * (s16 & 3));
                    const bf16x4 lo = tr_read(q);
                    const bf16x4 up = tr_read(q + 4 * XR);
                    const bf16x8 qf = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, pf, acc, 0, 0, 0);
                }
                float v[16];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const uint2 x2 = *reinterpret_cast<const uint2*>(X + i * XR + 2 * (cb0 + 8 * g + 4 * hi));
                    const float xv[4] = {bf16_lo(x2.x), bf16_hi(x2.x), bf16_lo(x2.y), bf16_hi(x2.y)};
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[4 * g + e] = fmaf(ca, xv[e], acc[4 * g + e]) * beta;
                }
                put_block(Xn, XR, v, i, cb0, false);
            }
        }
        __syncthreads();
    }

    // the output, padded canonical layout (padding rows / columns are zero)
    const char* Xf = Xb[steps & 1];
    bf16* o = out + d.x_off;
    for (int id = tid; id < SM * cpr; id += kThreads) {
        const int r = id / cpr, c = id - r * cpr;
        *reinterpret_cast<uint4*>(o + (int64_t)r * np + 8 * c) = *reinterpret_cast<const uint4*>(Xf + r * XR + 16 * c);
    }
    if (rowstats) {
        // NorMuon: sum of X'^2 per row and 64-column tile -> rowpart[tile][row]
        for (int t = tid; t < SM * (np / 64); t += kThreads) {
            const int r = t & (SM - 1), tj = t >> 6;
            float sum = 0.f;
            for (int c = 0; c < 64; c += 2) {
                const uint32_t w = *reinterpret_cast<const uint32_t*>(Xf + r * XR + 2 * (tj * 64 + c));
                const float x0 = bf16_lo(w), x1 = bf16_hi(w);
                sum = fmaf(x0, x0, sum);
                sum = fmaf(x1, x1, sum);
            }
            rowpart[d.rowpart_off + (int64_t)tj * d.m_pad + r] = sum;
        }
    }
}

}  // namespace

size_t ns_small_lds_bytes(int n_pad_max) { return (size_t)2 * SM * (2 * n_pad_max + 16) + (size_t)2 * SM * AROW; }

hipError_t prepare_ns_small(int n_pad_max) {
    if (n_pad_max <= 0) return hipSuccess;
    return hipFuncSetAttribute((const void*)k_ns_small, hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)ns_small_lds_bytes(n_pad_max));
}

hipError_t launch_ns_small(const LaunchCtx& L, const int32_t* list, int n, int n_pad_max, const NsCoeffs& co,
                           void* out, int rowstats) {
    if (n == 0) return hipSuccess;
    k_ns_small<<<n, kThreads, ns_small_lds_bytes(n_pad_max), L.stream>>>(L.mats, list, (const bf16*)L.xt, (bf16*)out,
                                                                         co, L.partials, L.ss, L.scale, L.status,
                                                                         L.rowpart, rowstats);
    return hipGetLastError();
}

}  // namespace muon
