// Host planner of libmuon: validates the matrix table, puts every matrix in
// its short-side frame, groups matrices by GEMM tile size, orders the tile
// work lists for the 8 XCDs, and lays out the workspace. Pure C++ (no HIP).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/libmuon.h"
#include "device_types.hpp"

namespace muon {

// At most kMaxGroups stream groups; a split needs kMinSplit tiled matrices
// per group (fewer gain nothing from the overlap), and the most update tiles
// (in 64 x 64 units) a step may have for the split: beyond that each launch
// runs so many tile rounds that its tail is negligible, and two groups in
// flight only double the working set in L2 / MALL.
constexpr int kMaxGroups = 4;
constexpr int kMinSplit = 2;
constexpr int64_t kMaxSplitTiles64 = (int64_t)64 * 256 * 16;
// stream_groups = 0 (the default) lets the planner choose: kAutoGroups
// groups when the update output covers at least one round of 256 x 256
// tiles on the GPU's 256 CUs (4096 tiles of 64 x 64), one group below that.
// A smaller step's launches are all partial rounds; more streams only add
// launches and waits to its latency (a 4-layer d = 512 body, 3072 such
// tiles: 0.461 ms per step in one group, 0.490 in three; a 4-layer d = 768
// body, 6912 tiles: 0.826 against 0.794).
constexpr int kAutoGroups = 3;
constexpr int64_t kAutoSplitMinTiles64 = (int64_t)256 * 16;
// Compute units per XCD on MI355X (256 CUs in 8 XCDs).
constexpr int kCusPerXcd = 32;
// A group whose momentum writes more X~ than the 256 MB MALL holds stores it
// nontemporally: by the time its Gram runs, the start of X~ has left the
// caches anyway, and the streaming stores run the pass 1.5% (runs) to 9%
// (transposed tiles) faster.
constexpr int64_t kXtCachedMax = (int64_t)256 << 20;
// Likewise for the Gram and polynomial outputs: a group whose A (an m_pad x
// m_pad tile set per tiled matrix) is larger than the MALL stores A and B,
// mirrors included, nontemporally. The next stage finds little of them in
// cache then, and the streaming stores leave the X and B panels there. Groups
// that fit keep cached stores, which the next stage reads from the MALL.
constexpr int64_t kAbCachedMax = (int64_t)256 << 20;

struct TileList {
    int T = 0;
    int group = 0;                      // stream group (see Plan::n_groups)
    std::vector<TileWork> gram, poly, update;
    size_t off_gram = 0, off_poly = 0, off_update = 0;  // workspace byte offsets
};

struct Plan {
    muon_hparams hp{};
    int esize = 2;                      // bytes per Newton–Schulz element (bf16 / fp32)
    std::vector<MatDesc> mats;          // every matrix, counts expanded
    std::vector<uint8_t> active_flag;   // !frozen
    std::vector<int32_t> active;        // active matrix indices
    std::vector<int32_t> ew_map;        // elementwise tile -> matrix
    std::vector<TileList> lists;        // one per (stream group, tile size) in use
    // The tiled matrices are split into n_groups cost-balanced groups whose
    // Newton–Schulz launches go to separate streams, so that one group's
    // kernels fill the other's tails and launch gaps.
    int n_groups = 1;
    // the active matrices are ordered group by group (small matrices in
    // group 0), and so are their elementwise tiles: group g owns active[
    // act_begin[g] .. act_begin[g+1]) and tiles [ew_begin[g], ew_begin[g+1])
    int act_begin[kMaxGroups + 1] = {};
    int ew_begin[kMaxGroups + 1] = {};
    int xt_nontemporal[kMaxGroups] = {};  // per group: momentum stores X~ nontemporally
    int ab_nontemporal[kMaxGroups] = {};  // per group: Gram / polynomial store A, B nontemporally
    std::vector<int32_t> panel;         // one-panel matrices, group by group
    int panel_begin[kMaxGroups + 1] = {};
    size_t off_panel = 0;
    std::vector<int32_t> small;         // active matrices of the one-workgroup Newton–Schulz
    int small_np = 0;                   // their largest n_pad
    size_t off_small = 0;
    int64_t extent = 0;                 // elements the flat buffers must hold
    int64_t x_elems = 0, a_elems = 0, rows_total = 0, rowpart_elems = 0;
    // workspace byte offsets
    size_t off_xt = 0, off_x0 = 0, off_x1 = 0, off_a = 0, off_b = 0;
    size_t off_part = 0, off_ss = 0, off_scale = 0, off_status = 0;
    size_t off_v = 0, off_f = 0, off_rowpart = 0;
    size_t off_mats = 0, off_ewmap = 0, off_active = 0;
    size_t total_bytes = 0;
    // 64-bit sums used by tools and tests
    double ns_alg_flops = 0.0;          // per step, symmetric products counted as m(m+1)k
    bool is_small(const MatDesc& d) const { return esize == 2 && d.T == 64 && d.n_pad <= kSmallMaxNPad; }
    bool is_panel(const MatDesc& d) const {
        return esize == 2 && d.T == kPanelRows && d.m_pad == kPanelRows && d.n_pad <= kPanelMaxNPad;
    }
};

// Validate and build. Returns MUON_OK or an error code with *err set.
muon_status build_plan(const muon_matrix* table, int32_t n, const muon_hparams* hp, Plan* out, std::string* err);

// Validate hyper-parameters only.
muon_status check_hparams(const muon_hparams* hp, std::string* err);

// Order one list of tiles for the XCD round-robin dispatch: matrices are
// assigned to 8 bins by cost (largest first), and workgroup b takes the next
// tile of bin b % 8, so the tiles of one matrix share an XCD's L2.
std::vector<TileWork> order_for_xcds(const std::vector<std::vector<TileWork>>& per_mat,
                                     const std::vector<double>& cost_per_tile, int n_xcd = 8);

}  // namespace muon
