// Host-side launchers of the libmuon kernels (internal interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_types.hpp"

namespace muon {

// Device addresses inside the caller's workspace plus launch geometry.
struct LaunchCtx {
    hipStream_t stream;
    int fp32;                 // Newton–Schulz precision: 0 bf16, 1 fp32
    const MatDesc* mats;
    const int32_t* ew_map;    // elementwise tile -> matrix
    const int32_t* active;    // active matrix indices
    int ew_tile0;             // first elementwise tile of this launch (a stream group's range)
    int ew_tiles;             // elementwise tiles of this launch
    int n_active;             // active matrices from `active` on
    void* xt;                 // momentum output X~ (canonical, padded)
    int xt_nontemporal;       // momentum stores X~ nontemporally (its group writes more X~ than the MALL holds)
    int ab_nontemporal;       // Gram / polynomial store A, B nontemporally (the group's A exceeds the MALL)
    void* x0;                 // ping-pong X buffers
    void* x1;
    void* a;                  // Gram A
    void* b;                  // polynomial B
    float* partials;          // per elementwise tile sum of u^2
    float* ss;                // per matrix sum of u^2
    float* scale;             // per matrix s
    int32_t* status;          // per matrix flags
    float* v;                 // NorMuon second moment (per canonical row)
    float* f;                 // NorMuon row factor
    float* rowpart;           // NorMuon row partial sums
    int64_t rows_total;
};

// One grouped GEMM launch: a work list of output tiles, all with tile size T.
struct GemmList {
    int T;
    const TileWork* gram;
    int n_gram;
    const TileWork* poly;
    int n_poly;
    const TileWork* update;
    int n_update;
};

enum NsMode { NS_GRAM = 0, NS_POLY = 1, NS_UPDATE = 2 };

// Per-iteration Newton–Schulz coefficients (a, b, c) and the normalisation eps.
struct NsCoeffs {
    float c[16][3];
    int steps;
    float eps;
};

hipError_t launch_momentum(const LaunchCtx& L, const float* grads, float* mom, float beta, int nesterov,
                           int heavy);
hipError_t launch_apply(const LaunchCtx& L, const void* xo, const float* f, float* params, float lr, float wd);
hipError_t launch_normuon(const LaunchCtx& L, float beta2, float eps);
hipError_t launch_reset(const LaunchCtx& L, float* mom);

// One Newton–Schulz iteration stage over a work list.
//   GRAM:   out = alpha * X X^T (upper tiles, mirrored); iteration 0: alpha = s^2
//           from the momentum partials (and s, sum u^2, status are recorded)
//   POLY:   out = b A + c A A^T (upper tiles, mirrored)
//   UPDATE: out = alpha (a X + B X); iteration 0: alpha = s, else 1;
//           rowstats: per-row partial sums of out^2 for NorMuon
hipError_t launch_ns_stage(const LaunchCtx& L, const GemmList& G, int mode, const void* xin, const void* ain,
                           void* out, float ca, float cb, float cc, int first, float eps, int rowstats);

// The same stage with the bf16 large-tile kernels (T = 128 or 256).
hipError_t launch_ns_stage_big(const LaunchCtx& L, const GemmList& G, int mode, const void* xin, const void* ain,
                               void* out, float ca, float cb, float cc, int first, float eps, int rowstats);

// Every iteration of the bf16 Newton–Schulz for the small matrices in `list`
// (m_pad = 64, n_pad <= n_pad_max <= 512), one workgroup per matrix, reading
// X~ and writing the output to `out` (same padded canonical layout); with
// rowstats, also the NorMuon row partial sums.
// Every iteration of the bf16 Newton–Schulz for the one-panel matrices in
// `list` (m_pad = 256 on 256-tiles, n_pad <= kPanelMaxNPad), one workgroup per
// matrix, with the iterations' X ping-pong in xt -> x1 -> x0 -> x1 ... (the
// tiled path's buffers), the last iteration's A and B in the workspace and,
// with rowstats, the NorMuon row partial sums.
hipError_t launch_ns_panel(const LaunchCtx& L, const int32_t* list, int n, const NsCoeffs& co, int rowstats);

hipError_t launch_ns_small(const LaunchCtx& L, const int32_t* list, int n, int n_pad_max, const NsCoeffs& co,
                           void* out, int rowstats);
size_t ns_small_lds_bytes(int n_pad_max);
// Allow the one-workgroup kernel its dynamic LDS for n_pad up to n_pad_max on
// the current device (once, at init; launches do not repeat it).
hipError_t prepare_ns_small(int n_pad_max);

// Device address of the library's static workspace on `device` (current).
hipError_t static_scratch_address(int device, void** addr);

}  // namespace muon
