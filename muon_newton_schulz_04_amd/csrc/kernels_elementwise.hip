// HBM-streaming kernels of the Muon step: momentum (+ Nesterov, cast to the
// Newton–Schulz input, per-matrix sum of squares), the NorMuon row factors,
// the parameter update, and the reset fills.
//
// Sources: [P4] "modded-nanogpt 50B-token 长时程训练实验解析" section
// "从源码看 Muon 的分布式正交化实现" (momentum + Nesterov, Frobenius normalisation,
// transpose to the short side, max(1, rows/cols)^0.5, p -= lr * update);
// [P2] "2025-10-27_FixMuonLR" analysis, change 2 (lerp momentum buffer,
// NorMuon per-lane second moment along the longer dimension).
//
// Matrices stored with rows > cols are transposed into their canonical frame
// (rows <= cols) through LDS, in 64 x 64 tiles over the valid block rounded
// up to whole tiles, so that both the stored-frame and the canonical-frame
// accesses stay coalesced; the momentum kernel writes zeros into the padding
// inside those tiles. For the other matrices the two frames coincide and a
// tile is a run of kEwLinear (4096) consecutive stored elements, which the
// kernels stream like a flat copy: every wave instruction covers 1 KB of one
// fp32 stream, and a workgroup 16 KB. The X~ padding that no tile writes is
// zeroed once when the handle is created.

#include "kernel_common.hpp"
#include "launch.hpp"

namespace muon {

namespace {

constexpr int TS = kEwTile;  // 64
// Streams that are touched once per step (gradients, momentum, parameters,
// the Newton–Schulz output) use nontemporal loads / stores, so they do not
// push the Newton–Schulz working set out of L2 and the MALL. X~, which the
// Gram kernel reads next, is stored normally unless the launch writes more of
// it than the MALL holds (then its start is gone before the Gram runs).
typedef float f4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ntld4(const float* p) {
    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void ntst4(float* p, float4 v) {
    f4v w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<f4v*>(p));
}

struct TileCoord {
    int mi, i0, j0;
};

// Tile order of a transposed matrix: stored rows (canonical column blocks
// tj) are taken in bands of two 64-row blocks; inside a band the stored
// column chunk (canonical row block ti) advances, and the band's two row
// blocks come back to back. With a whole stored-row band in flight at once
// (and not a column strip down the whole matrix), the transposed tiles
// stream 8-14% faster.
__device__ __forceinline__ TileCoord decode_tile(const MatDesc& d, int tile, int mi) {
    const int lt = tile - d.ew_start;
    const int nti = (d.m + TS - 1) / TS;  // canonical row blocks
    const int band = lt / (2 * nti);
    const int r = lt - band * 2 * nti;
    int ti, tj;
    if (2 * band + 1 < d.ew_tiles_n) {
        ti = r >> 1;
        tj = 2 * band + (r & 1);
    } else {  // an odd count of row blocks: the last band holds one
        ti = r;
        tj = 2 * band;
    }
    return {mi, ti * TS, tj * TS};
}

struct MomParams {
    float beta;
    int nesterov;
    int heavy;
};

// m <- beta m + (1-beta) g  (lerp)   |  m <- beta m + g   (heavy ball)
// u =  (1-beta) g + beta m_new       |  u =  g + beta m_new   (Nesterov)
__device__ __forceinline__ float mom_update(float g, float& m, const MomParams& P) {
    const float gs = P.heavy ? g : (1.0f - P.beta) * g;
    const float mn = fmaf(P.beta, m, gs);
    m = mn;
    return P.nesterov ? fmaf(P.beta, mn, gs) : mn;
}

// X~ stores: cached (NT = false) when the Gram kernel can still find X~ in
// L2 / the MALL, nontemporal when the group writes more X~ than the MALL holds.
template <typename XT, bool NT>
__device__ __forceinline__ void store_x4(XT* dst, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store_x4<bf16, false>(bf16* dst, float a, float b, float c, float d) {
    uint2 w;
    w.x = pack_bf16x2(a, b);
    w.y = pack_bf16x2(c, d);
    *reinterpret_cast<uint2*>(dst) = w;
}

template <>
__device__ __forceinline__ void store_x4<bf16, true>(bf16* dst, float a, float b, float c, float d) {
    typedef unsigned u2v __attribute__((ext_vector_type(2)));
    const u2v w = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    __builtin_nontemporal_store(w, reinterpret_cast<u2v*>(dst));
}

template <>
__device__ __forceinline__ void store_x4<float, false>(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(dst) = make_float4(a, b, c, d);
}

template <>
__device__ __forceinline__ void store_x4<float, true>(float* dst, float a, float b, float c, float d) {
    ntst4(dst, make_float4(a, b, c, d));
}

template <typename XT>
__device__ __forceinline__ void load_x4(const XT* src, float* v);

template <>
__device__ __forceinline__ void load_x4<bf16>(const bf16* src, float* v) {
    typedef unsigned u2v __attribute__((ext_vector_type(2)));
    const u2v wv = __builtin_nontemporal_load(reinterpret_cast<const u2v*>(src));
    const uint2 w = make_uint2(wv.x, wv.y);
    v[0] = bf16_lo(w.x);
    v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y);
    v[3] = bf16_hi(w.y);
}

template <>
__device__ __forceinline__ void load_x4<float>(const float* src, float* v) {
    const float4 w = *reinterpret_cast<const float4*>(src);
    v[0] = w.x;
    v[1] = w.y;
    v[2] = w.z;
    v[3] = w.w;
}

template <typename XT>
__device__ __forceinline__ void store_x1(XT* dst, float v) {
    *dst = (XT)v;  // bf16: round to nearest even, as pack_bf16x2
}

template <typename XT>
__device__ __forceinline__ float load_x1(const XT* src) {
    return (float)*src;
}

// Element e (0 <= e < R C < 2^30) of an untransposed matrix is canonical
// (e / C, e % C).
__device__ __forceinline__ void split_index(int e, int C, int& i, int& j) {
    i = (int)((unsigned)e / (unsigned)C);
    j = e - i * C;
}

// Momentum over run lt of an untransposed matrix; returns this thread's sum
// of u^2. Thread t owns the float4 groups at 4 t + 1024 p, p = 0 .. 3.
template <typename XT, bool NTX>
__device__ __forceinline__ float momentum_run(const MatDesc& d, int lt, const float* __restrict__ grads,
                                              float* __restrict__ mom, XT* __restrict__ xt, const MomParams& P) {
    const int total = d.R * d.C;
    const int e0 = lt * kEwLinear + 4 * (int)threadIdx.x;
    float ssq = 0.0f;
    if (d.vec_ok) {
        // C % 4 == 0: a float4 group never crosses a row, and total % 4 == 0
        const bool full = (lt + 1) * kEwLinear <= total;
        float4 g4[4], m4[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int e = e0 + p * 4 * kThreads;
            if (full || e < total) {
                g4[p] = ntld4(grads + d.p_off + e);
                m4[p] = ntld4(mom + d.p_off + e);
            }
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int e = e0 + p * 4 * kThreads;
            if (full || e < total) {
                float u[4];
                u[0] = mom_update(g4[p].x, m4[p].x, P);
                u[1] = mom_update(g4[p].y, m4[p].y, P);
                u[2] = mom_update(g4[p].z, m4[p].z, P);
                u[3] = mom_update(g4[p].w, m4[p].w, P);
                ntst4(mom + d.p_off + e, m4[p]);
                ssq = fmaf(u[0], u[0], ssq);
                ssq = fmaf(u[1], u[1], ssq);
                ssq = fmaf(u[2], u[2], ssq);
                ssq = fmaf(u[3], u[3], ssq);
                int i, j;
                split_index(e, d.C, i, j);
                store_x4<XT, NTX>(xt + d.x_off + (int64_t)i * d.n_pad + j, u[0], u[1], u[2], u[3]);
            }
        }
    } else {
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int e = e0 + p * 4 * kThreads + k;
                if (e < total) {
                    float mv = mom[d.p_off + e];
                    const float u = mom_update(grads[d.p_off + e], mv, P);
                    mom[d.p_off + e] = mv;
                    ssq = fmaf(u, u, ssq);
                    int i, j;
                    split_index(e, d.C, i, j);
                    store_x1<XT>(xt + d.x_off + (int64_t)i * d.n_pad + j, u);
                }
            }
    }
    return ssq;
}

// Parameter update over run lt of an untransposed matrix (same thread layout).
template <typename XT>
__device__ __forceinline__ void apply_run(const MatDesc& d, int lt, const XT* __restrict__ xo,
                                          const float* __restrict__ fr, float* __restrict__ params, float decay,
                                          float coef0) {
    const int total = d.R * d.C;
    const int e0 = lt * kEwLinear + 4 * (int)threadIdx.x;
    if (d.vec_ok) {
        const bool full = (lt + 1) * kEwLinear <= total;
        float x[4][4];
        float4 p4[4];
        float coef[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int e = e0 + p * 4 * kThreads;
            if (full || e < total) {
                int i, j;
                split_index(e, d.C, i, j);
                load_x4<XT>(xo + d.x_off + (int64_t)i * d.n_pad + j, x[p]);
                p4[p] = ntld4(params + d.p_off + e);
                coef[p] = fr ? coef0 * fr[d.row_off + i] : coef0;
            }
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int e = e0 + p * 4 * kThreads;
            if (full || e < total) {
                p4[p].x = fmaf(-coef[p], x[p][0], p4[p].x * decay);
                p4[p].y = fmaf(-coef[p], x[p][1], p4[p].y * decay);
                p4[p].z = fmaf(-coef[p], x[p][2], p4[p].z * decay);
                p4[p].w = fmaf(-coef[p], x[p][3], p4[p].w * decay);
                ntst4(params + d.p_off + e, p4[p]);
            }
        }
    } else {
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int e = e0 + p * 4 * kThreads + k;
                if (e < total) {
                    int i, j;
                    split_index(e, d.C, i, j);
                    const float xv = load_x1<XT>(xo + d.x_off + (int64_t)i * d.n_pad + j);
                    const float coef = fr ? coef0 * fr[d.row_off + i] : coef0;
                    params[d.p_off + e] = fmaf(-coef, xv, params[d.p_off + e] * decay);
                }
            }
    }
}

// ---------------------------------------------------------------------------
// K1: momentum + Nesterov + cast into the canonical Newton–Schulz input,
// and one deterministic sum of u^2 per tile.
// Transposed matrices: a 64 x 64 canonical tile is read as stored rows (16
// column groups of 4 x 16 row lanes, four passes of 16 rows) and written to
// X~ through LDS.
// ---------------------------------------------------------------------------
template <typename XT, bool NTX>
__global__ __launch_bounds__(kThreads) void k_momentum(const MatDesc* __restrict__ mats,
                                                       const int32_t* __restrict__ ew_map,
                                                       const float* __restrict__ grads,
                                                       float* __restrict__ mom, XT* __restrict__ xt,
                                                       float* __restrict__ partials, MomParams P, int tile0) {
    __shared__ float lds[TS][TS + 1];
    __shared__ float red[4];
    const int tile = tile0 + blockIdx.x;
    const int mi = ew_map[tile];
    const MatDesc d = mats[mi];
    const int tid = threadIdx.x;
    if (!d.transposed) {
        const float t = block_sum_256(momentum_run<XT, NTX>(d, tile - d.ew_start, grads, mom, xt, P), red);
        if (tid == 0) partials[tile] = t;
        return;
    }
    // canonical (i, j) == stored (j, i): stored rows r = j0 + rl, columns c = i0 + cg .. +3
    const TileCoord tc = decode_tile(d, tile, mi);
    const int cg = (tid & 15) * 4;
    const int rg = tid >> 4;
    float ssq = 0.0f;
    if (d.vec_ok && tc.i0 + TS <= d.m && tc.j0 + TS <= d.n) {
        // interior tile with 16-byte aligned rows: all four passes' loads go
        // out before the first is used
        float4 g4[4], m4[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int64_t base = d.p_off + (int64_t)(tc.j0 + rg + 16 * p) * d.C + tc.i0 + cg;
            g4[p] = ntld4(grads + base);
            m4[p] = ntld4(mom + base);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            float u[4];
            u[0] = mom_update(g4[p].x, m4[p].x, P);
            u[1] = mom_update(g4[p].y, m4[p].y, P);
            u[2] = mom_update(g4[p].z, m4[p].z, P);
            u[3] = mom_update(g4[p].w, m4[p].w, P);
            ntst4(mom + d.p_off + (int64_t)(tc.j0 + rg + 16 * p) * d.C + tc.i0 + cg, m4[p]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ssq = fmaf(u[e], u[e], ssq);
                lds[cg + e][rg + 16 * p] = u[e];
            }
        }
    } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int rl = rg + 16 * p;
            const int r = tc.j0 + rl;
            const int c = tc.i0 + cg;
            float u[4] = {0.f, 0.f, 0.f, 0.f};
            if (r < d.R) {
                const int64_t base = d.p_off + (int64_t)r * d.C + c;
                if (d.vec_ok && c + 3 < d.C) {
                    const float4 g4 = ntld4(grads + base);
                    float4 m4 = ntld4(mom + base);
                    u[0] = mom_update(g4.x, m4.x, P);
                    u[1] = mom_update(g4.y, m4.y, P);
                    u[2] = mom_update(g4.z, m4.z, P);
                    u[3] = mom_update(g4.w, m4.w, P);
                    ntst4(mom + base, m4);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (c + e < d.C) {
                            float mv = mom[base + e];
                            u[e] = mom_update(grads[base + e], mv, P);
                            mom[base + e] = mv;
                        }
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ssq = fmaf(u[e], u[e], ssq);
                lds[cg + e][rl] = u[e];
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int il = rg + 16 * p;
        store_x4<XT, NTX>(xt + d.x_off + (int64_t)(tc.i0 + il) * d.n_pad + tc.j0 + cg, lds[il][cg],
                          lds[il][cg + 1], lds[il][cg + 2], lds[il][cg + 3]);
    }
    const float t = block_sum_256(ssq, red);
    if (tid == 0) partials[tile] = t;
}

// ---------------------------------------------------------------------------
// K6: p <- p (1 - lr lr_mul wd wd_mul) - lr lr_mul shape_scale f_row O
// (f_row = NorMuon factor of the canonical row, 1 without NorMuon).
// Transposed matrices: canonical rows of O are read, turned through LDS, and
// applied to stored rows.
// ---------------------------------------------------------------------------
template <typename XT>
__global__ __launch_bounds__(kThreads) void k_apply(const MatDesc* __restrict__ mats,
                                                    const int32_t* __restrict__ ew_map,
                                                    const XT* __restrict__ xo, const float* __restrict__ fr,
                                                    float* __restrict__ params, float lr, float wd, int tile0) {
    __shared__ float lds[TS][TS + 1];
    const int tile = tile0 + blockIdx.x;
    const int mi = ew_map[tile];
    const MatDesc d = mats[mi];
    const float lrm = lr * d.lr_mul;
    const float decay = 1.0f - lrm * wd * d.wd_mul;
    const float coef0 = lrm * d.shape_scale;
    if (!d.transposed) {
        apply_run<XT>(d, tile - d.ew_start, xo, fr, params, decay, coef0);
        return;
    }
    const TileCoord tc = decode_tile(d, tile, mi);
    if (tc.i0 >= d.m || tc.j0 >= d.n) return;  // tile lies wholly in the padding
    const int tid = threadIdx.x;
    const int cg = (tid & 15) * 4;
    const int rg = tid >> 4;

    if (d.vec_ok && tc.i0 + TS <= d.m && tc.j0 + TS <= d.n) {
        // interior tile with 16-byte aligned rows: every load of the tile
        // goes out before the first is used
        float x[4][4];
        float4 p4[4];
        // NorMuon row factors of the canonical rows i0 + cg + e (this thread's
        // stored columns)
        float coef[4] = {coef0, coef0, coef0, coef0};
        if (fr) {
#pragma unroll
            for (int e = 0; e < 4; ++e) coef[e] = coef0 * fr[d.row_off + tc.i0 + cg + e];
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            load_x4<XT>(xo + d.x_off + (int64_t)(tc.i0 + rg + 16 * p) * d.n_pad + tc.j0 + cg, x[p]);
            p4[p] = ntld4(params + d.p_off + (int64_t)(tc.j0 + rg + 16 * p) * d.C + tc.i0 + cg);
        }
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int e = 0; e < 4; ++e) lds[cg + e][rg + 16 * p] = x[p][e];
        __syncthreads();
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int rl = rg + 16 * p;
            p4[p].x = fmaf(-coef[0], lds[rl][cg], p4[p].x * decay);
            p4[p].y = fmaf(-coef[1], lds[rl][cg + 1], p4[p].y * decay);
            p4[p].z = fmaf(-coef[2], lds[rl][cg + 2], p4[p].z * decay);
            p4[p].w = fmaf(-coef[3], lds[rl][cg + 3], p4[p].w * decay);
            ntst4(params + d.p_off + (int64_t)(tc.j0 + rl) * d.C + tc.i0 + cg, p4[p]);
        }
        return;
    }
    // read canonical rows (i = stored column), write stored rows
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int il = rg + 16 * p;
        const int i = tc.i0 + il;
        const int j = tc.j0 + cg;
        float x[4];
        load_x4<XT>(xo + d.x_off + (int64_t)i * d.n_pad + j, x);
        lds[cg][il] = x[0];
        lds[cg + 1][il] = x[1];
        lds[cg + 2][il] = x[2];
        lds[cg + 3][il] = x[3];
    }
    __syncthreads();
    float coef[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int c = tc.i0 + cg + e;
        coef[e] = (fr && c < d.C) ? coef0 * fr[d.row_off + c] : coef0;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int rl = rg + 16 * p;
        const int r = tc.j0 + rl;
        const int c = tc.i0 + cg;
        if (r >= d.R) continue;
        const int64_t base = d.p_off + (int64_t)r * d.C + c;
        if (d.vec_ok && c + 3 < d.C) {
            float4 p4 = ntld4(params + base);
            p4.x = fmaf(-coef[0], lds[rl][cg], p4.x * decay);
            p4.y = fmaf(-coef[1], lds[rl][cg + 1], p4.y * decay);
            p4.z = fmaf(-coef[2], lds[rl][cg + 2], p4.z * decay);
            p4.w = fmaf(-coef[3], lds[rl][cg + 3], p4.w * decay);
            ntst4(params + base, p4);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (c + e < d.C) params[base + e] = fmaf(-coef[e], lds[rl][cg + e], params[base + e] * decay);
        }
    }
}

// ---------------------------------------------------------------------------
// K5: NorMuon factors, one block of kNormThreads per active matrix.
//   r_i = (1/n) sum_j O_ij^2   (row partials written by the last NS update)
//   v_i <- beta2 v_i + (1 - beta2) r_i
//   d_i = sqrt(v_i) + eps
//   f_i = gamma / d_i, gamma = sqrt(sum_i r_i / sum_i r_i / d_i^2)  (keeps ||O||_F)
// A matrix's rows (m <= 1024 for the bodies here) are spread over 1024
// threads, so each thread's loads of its row partials go out together; the
// two sums are reduced in a fixed order (deterministic).
// ---------------------------------------------------------------------------
constexpr int kNormThreads = 1024;

// block-wide sums of (a, b) over kNormThreads threads, in a fixed order
__device__ __forceinline__ float2 block_sum2_1024(float a, float b, float2* red /* >= 16 */) {
    a = wave_sum(a);
    b = wave_sum(b);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = make_float2(a, b);
    __syncthreads();
    float2 t = make_float2(0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kNormThreads / 64; ++w) {
        t.x += red[w].x;
        t.y += red[w].y;
    }
    return t;
}

__global__ __launch_bounds__(kNormThreads) void k_normuon(const MatDesc* __restrict__ mats,
                                                          const int32_t* __restrict__ active,
                                                          const float* __restrict__ rowpart,
                                                          float* __restrict__ v, float* __restrict__ f,
                                                          float beta2, float eps) {
    __shared__ float2 red[kNormThreads / 64];
    const int mi = active[blockIdx.x];
    const MatDesc d = mats[mi];
    const int ntn = d.n_pad / d.T;
    const float inv_n = 1.0f / (float)d.n;
    const float* rp = rowpart + d.rowpart_off;
    float s1 = 0.f, s2 = 0.f;
    for (int i = threadIdx.x; i < d.m; i += kNormThreads) {
        // four independent chains over the row's partials, summed in a fixed order
        float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
        int t = 0;
        for (; t + 4 <= ntn; t += 4) {
            r0 += rp[(int64_t)t * d.m_pad + i];
            r1 += rp[(int64_t)(t + 1) * d.m_pad + i];
            r2 += rp[(int64_t)(t + 2) * d.m_pad + i];
            r3 += rp[(int64_t)(t + 3) * d.m_pad + i];
        }
        for (; t < ntn; ++t) r0 += rp[(int64_t)t * d.m_pad + i];
        const float r = ((r0 + r1) + (r2 + r3)) * inv_n;
        const float vi = fmaf(beta2, v[d.row_off + i], (1.0f - beta2) * r);
        v[d.row_off + i] = vi;
        const float di = sqrtf(vi) + eps;
        s1 += r;
        s2 += r / (di * di);
        f[d.row_off + i] = di;
    }
    const float2 S = block_sum2_1024(s1, s2, red);
    const float gamma = S.y > 0.f ? sqrtf(S.x / S.y) : 0.f;
    for (int i = threadIdx.x; i < d.m; i += kNormThreads) f[d.row_off + i] = gamma / f[d.row_off + i];
}

// ---------------------------------------------------------------------------
// Reset fills: zero the momentum of active matrices (stored extent, tile by
// tile) and a float range.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_zero_momentum(const MatDesc* __restrict__ mats,
                                                            const int32_t* __restrict__ ew_map,
                                                            float* __restrict__ mom) {
    const int tile = blockIdx.x;
    const int mi = ew_map[tile];
    const MatDesc d = mats[mi];
    const int tid = threadIdx.x;
    if (!d.transposed) {
        const int total = d.R * d.C;
        const int e0 = (tile - d.ew_start) * kEwLinear;
        for (int e = e0 + tid; e < e0 + kEwLinear && e < total; e += kThreads) mom[d.p_off + e] = 0.f;
        return;
    }
    const TileCoord tc = decode_tile(d, tile, mi);
    if (tc.i0 >= d.m || tc.j0 >= d.n) return;
    const int cg = (tid & 15) * 4;
    const int rg = tid >> 4;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        // canonical (i, j) lives at stored (j, i): stored row j0 + rl, columns i0 + cg .. +3
        const int r = tc.j0 + rg + 16 * p;
        const int c = tc.i0 + cg;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (r < d.R && c + e < d.C) mom[d.p_off + (int64_t)r * d.C + c + e] = 0.f;
    }
}

__global__ __launch_bounds__(kThreads) void k_fill_zero(float* __restrict__ x, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) x[i] = 0.f;
}

}  // namespace

hipError_t launch_momentum(const LaunchCtx& L, const float* grads, float* mom, float beta, int nesterov,
                           int heavy) {
    if (L.ew_tiles == 0) return hipSuccess;
    MomParams P{beta, nesterov, heavy};
    const dim3 grid(L.ew_tiles), block(kThreads);
    if (L.fp32) {
        if (L.xt_nontemporal)
            k_momentum<float, true><<<grid, block, 0, L.stream>>>(L.mats, L.ew_map, grads, mom, (float*)L.xt,
                                                                  L.partials, P, L.ew_tile0);
        else
            k_momentum<float, false><<<grid, block, 0, L.stream>>>(L.mats, L.ew_map, grads, mom, (float*)L.xt,
                                                                   L.partials, P, L.ew_tile0);
    } else {
        if (L.xt_nontemporal)
            k_momentum<bf16, true><<<grid, block, 0, L.stream>>>(L.mats, L.ew_map, grads, mom, (bf16*)L.xt,
                                                                 L.partials, P, L.ew_tile0);
        else
            k_momentum<bf16, false><<<grid, block, 0, L.stream>>>(L.mats, L.ew_map, grads, mom, (bf16*)L.xt,
                                                                  L.partials, P, L.ew_tile0);
    }
    return hipGetLastError();
}

hipError_t launch_apply(const LaunchCtx& L, const void* xo, const float* f, float* params, float lr, float wd) {
    if (L.ew_tiles == 0) return hipSuccess;
    if (L.fp32)
        k_apply<float><<<L.ew_tiles, kThreads, 0, L.stream>>>(L.mats, L.ew_map, (const float*)xo, f, params, lr,
                                                              wd, L.ew_tile0);
    else
        k_apply<bf16><<<L.ew_tiles, kThreads, 0, L.stream>>>(L.mats, L.ew_map, (const bf16*)xo, f, params, lr, wd,
                                                             L.ew_tile0);
    return hipGetLastError();
}

hipError_t launch_normuon(const LaunchCtx& L, float beta2, float eps) {
    if (L.n_active == 0) return hipSuccess;
    k_normuon<<<L.n_active, kNormThreads, 0, L.stream>>>(L.mats, L.active, L.rowpart, L.v, L.f, beta2, eps);
    return hipGetLastError();
}

hipError_t launch_reset(const LaunchCtx& L, float* mom) {
    if (mom && L.ew_tiles) k_zero_momentum<<<L.ew_tiles, kThreads, 0, L.stream>>>(L.mats, L.ew_map, mom);
    if (L.rows_total) {
        const int64_t n = L.rows_total;
        const int blocks = (int)((n + kThreads - 1) / kThreads < 1024 ? (n + kThreads - 1) / kThreads : 1024);
        k_fill_zero<<<blocks, kThreads, 0, L.stream>>>(L.v, n);
    }
    return hipGetLastError();
}

}  // namespace muon
