// Descriptor structs shared by the host planner and the HIP kernels.
// Plain data, laid out identically on host and device.
#pragma once

#include <stdint.h>

namespace muon {

// Tile sizes. GEMM tiles are square T x T with T in {64, 128, 256}; every
// canonical buffer is padded to a multiple of its bucket's T in both
// dimensions (zero-filled padding keeps Newton–Schulz exact on the valid
// block, so the GEMM kernels carry no bounds checks). Elementwise kernels
// work on 64 x 64 tiles of the canonical frame for matrices stored with rows
// > cols (transposed through LDS), and on runs of kEwLinear consecutive
// stored elements for the others, whose canonical frame is the stored one.
constexpr int kEwTile = 64;
constexpr int kEwLinear = 4096;
constexpr int kThreads = 256;
// bf16 matrices with m_pad = 64 and n_pad <= kSmallMaxNPad run every
// Newton–Schulz iteration in one workgroup (X, A, P resident in LDS).
constexpr int kSmallMaxNPad = 512;
// bf16 matrices that are one 256-row panel (m_pad = 256 on 256-tiles) with
// n_pad <= kPanelMaxNPad run every iteration in one workgroup of 8 waves
// (A and B resident in LDS).
constexpr int kPanelRows = 256;
constexpr int kPanelMaxNPad = 4096;

// One (sub-)matrix of the table, in both frames.
//   stored frame:    [R, C] row-major at p_off in params / grads / momentum
//   canonical frame: [m, n], m = min(R, C) <= n = max(R, C); X = u^T if R > C
struct MatDesc {
    int64_t p_off;        // element offset in the flat float32 buffers
    int64_t x_off;        // element offset of X in the padded canonical X buffers
    int64_t a_off;        // element offset of the m_pad x m_pad Gram / poly buffers
    int64_t rowpart_off;  // offset of [n_pad / T] x m_pad row partial sums (NorMuon)
    int32_t R, C, m, n;
    int32_t m_pad, n_pad; // canonical padded dims (multiples of T); ld of X = n_pad
    int32_t T;            // GEMM tile of this matrix's bucket
    int32_t transposed;   // R > C
    int32_t row_off;      // offset into the per-row NorMuon arrays (v, f)
    int32_t ew_start;     // first elementwise tile (index into the momentum partials)
    int32_t ew_count;     // number of elementwise tiles
    int32_t ew_tiles_n;   // transposed: 64 x 64 tiles per canonical row band (ceil(n / 64)); else 0
    float lr_mul, wd_mul, shape_scale;
    int32_t vec_ok;       // stored rows start 16-byte aligned (float4 access legal)
};

// One output tile of a grouped GEMM launch.
struct TileWork {
    int32_t mat;  // MatDesc index
    int16_t ti;   // tile row
    int16_t tj;   // tile column
};

}  // namespace muon
