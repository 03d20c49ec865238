// Host planner of libmuon (see plan.hpp).
//
// Source for the planning rules: [P4] "modded-nanogpt 50B-token 长时程训练实验解析"
// section "从源码看 Muon 的分布式正交化实现" (only 2-D weights; transpose so the
// iteration runs on the shorter side; max(1, rows/cols)^0.5 scale) and [P2]
// "2025-10-27_FixMuonLR" analysis, change 2 (stacking same-class matrices
// into one batched orthogonalisation; qkvo handled as four matrices).

#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <numeric>

namespace muon {

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

bool finite(float x) { return std::isfinite(x); }

// GEMM tile for a matrix whose short side is m: 256 (bf16 only, m >= 256)
// unless it pads m by more than m / 8 beyond what 128 would, 128 for medium,
// 64 small. The 256-tile kernel (8 waves, 2 per SIMD) moves half the bytes
// per flop of the 128-tile one (4 waves): for m = 1600 it wins at m_pad 1792
// against 1664 (1.5B body: 57.3 against 63.1 ms per step), and at m = 256
// (256 x 1024 matrices) its one diagonal Gram tile beats three 128-tiles
// (32 against 38 us per launch for 192 matrices). fp32 matrices up to
// m = 256 take 64-tiles: the fp32 MFMA rate per CU is a sixteenth of bf16,
// so spreading a small matrix over more workgroups pays (tiny d = 128 body:
// one 128-tile per Gram took 62 us).
int pick_tile(int64_t m, bool fp32) {
    if (m <= 64 || (fp32 && m <= 256)) return 64;
    if (!fp32 && m >= 256 && round_up(m, 256) <= round_up(m, 128) + m / 8) return 256;
    return 128;
}

}  // namespace

muon_status check_hparams(const muon_hparams* hp, std::string* err) {
    auto bad = [&](const char* what) {
        *err = what;
        return MUON_E_INVALID_ARG;
    };
    if (!finite(hp->momentum) || hp->momentum < 0.f || hp->momentum > 1.f) return bad("momentum must be in [0, 1]");
    if (hp->nesterov != 0 && hp->nesterov != 1) return bad("nesterov must be 0 or 1");
    if (hp->momentum_kind != MUON_MOMENTUM_LERP && hp->momentum_kind != MUON_MOMENTUM_HEAVY_BALL)
        return bad("unknown momentum_kind");
    if (hp->ns_steps < 1 || hp->ns_steps > MUON_MAX_NS_STEPS) return bad("ns_steps must be in [1, 16]");
    for (int k = 0; k < hp->ns_steps; ++k)
        for (int j = 0; j < 3; ++j)
            if (!finite(hp->ns_coeffs[k][j])) return bad("non-finite Newton-Schulz coefficient");
    if (!finite(hp->ns_eps) || hp->ns_eps < 0.f) return bad("ns_eps must be finite and >= 0");
    if (hp->ns_precision != MUON_NS_BF16 && hp->ns_precision != MUON_NS_FP32) return bad("unknown ns_precision");
    if (hp->normuon != 0 && hp->normuon != 1) return bad("normuon must be 0 or 1");
    if (!finite(hp->normuon_beta2) || hp->normuon_beta2 < 0.f || hp->normuon_beta2 > 1.f)
        return bad("normuon_beta2 must be in [0, 1]");
    if (!finite(hp->normuon_eps) || hp->normuon_eps < 0.f) return bad("normuon_eps must be finite and >= 0");
    if (!finite(hp->weight_decay)) return bad("weight_decay must be finite");
    if (hp->stream_groups < 0 || hp->stream_groups > kMaxGroups) return bad("stream_groups must be in [0, 4]");
    return MUON_OK;
}

std::vector<TileWork> order_for_xcds(const std::vector<std::vector<TileWork>>& per_mat,
                                     const std::vector<double>& cost_per_tile, int n_xcd) {
    const size_t nm = per_mat.size();
    std::vector<size_t> order(nm);
    std::iota(order.begin(), order.end(), 0);
    std::vector<double> mcost(nm);
    for (size_t i = 0; i < nm; ++i) mcost[i] = cost_per_tile[i] * (double)per_mat[i].size();
    std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) { return mcost[a] > mcost[b]; });
    std::vector<std::vector<TileWork>> bins(n_xcd);
    std::vector<double> bcost(n_xcd, 0.0);
    for (size_t idx : order) {
        if (per_mat[idx].empty()) continue;
        int b = (int)(std::min_element(bcost.begin(), bcost.end()) - bcost.begin());
        bins[b].insert(bins[b].end(), per_mat[idx].begin(), per_mat[idx].end());
        bcost[b] += mcost[idx];
    }
    std::vector<size_t> head(n_xcd, 0);
    size_t total = 0;
    for (auto& b : bins) total += b.size();
    std::vector<TileWork> out;
    out.reserve(total);
    while (out.size() < total) {
        int x = (int)(out.size() % (size_t)n_xcd);
        if (head[x] >= bins[x].size()) {
            // this XCD's bin is empty: take from the bin with the most tiles left
            size_t best = 0;
            int bx = -1;
            for (int y = 0; y < n_xcd; ++y) {
                size_t left = bins[y].size() - head[y];
                if (left > best) {
                    best = left;
                    bx = y;
                }
            }
            x = bx;
        }
        out.push_back(bins[x][head[x]++]);
    }
    return out;
}

muon_status build_plan(const muon_matrix* table, int32_t n, const muon_hparams* hp_in, Plan* out,
                       std::string* err) {
    Plan P;
    if (hp_in) {
        P.hp = *hp_in;
    } else {
        muon_hparams_default(&P.hp);
    }
    muon_status st = check_hparams(&P.hp, err);
    if (st != MUON_OK) return st;
    if (n < 0) {
        *err = "negative table length";
        return MUON_E_INVALID_ARG;
    }
    if (n > 0 && !table) {
        *err = "null table";
        return MUON_E_INVALID_ARG;
    }
    P.esize = P.hp.ns_precision == MUON_NS_FP32 ? 4 : 2;

    // ---- validate entries ----
    struct Iv {
        int64_t lo, hi;
        int idx;
    };
    std::vector<Iv> iv;
    int64_t nmat = 0;
    for (int e = 0; e < n; ++e) {
        const muon_matrix& t = table[e];
        if (t.reserved != 0) {
            *err = "entry " + std::to_string(e) + ": reserved field must be 0";
            return MUON_E_INVALID_ARG;
        }
        if (t.rows < 1 || t.cols < 1 || t.count < 1) {
            *err = "entry " + std::to_string(e) + ": rows, cols and count must be >= 1";
            return MUON_E_SHAPE;
        }
        if (t.rows > (1 << 20) || t.cols > (1 << 20) || t.count > (1 << 24)) {
            *err = "entry " + std::to_string(e) + ": dimension or count too large";
            return MUON_E_SHAPE;
        }
        if (t.offset < 0) {
            *err = "entry " + std::to_string(e) + ": negative offset";
            return MUON_E_LAYOUT;
        }
        if (!finite(t.lr_mul) || !finite(t.wd_mul)) {
            *err = "entry " + std::to_string(e) + ": non-finite lr_mul / wd_mul";
            return MUON_E_INVALID_ARG;
        }
        // rows, cols <= 2^20 and count <= 2^24: bound rows x cols first, so the
        // extent below stays far from int64 overflow
        if (t.rows * t.cols >= (INT64_C(1) << 30)) {
            *err = "entry " + std::to_string(e) + ": matrix too large for one tile grid";
            return MUON_E_SHAPE;
        }
        const int64_t sz = t.rows * t.cols * t.count;
        if (t.offset > (INT64_C(1) << 62) - sz) {
            *err = "entry " + std::to_string(e) + ": extent overflows";
            return MUON_E_LAYOUT;
        }
        iv.push_back({t.offset, t.offset + sz, e});
        P.extent = std::max(P.extent, t.offset + sz);
        nmat += t.count;
    }
    if (nmat > (1 << 24)) {
        *err = "too many matrices";
        return MUON_E_SHAPE;
    }
    std::sort(iv.begin(), iv.end(), [](const Iv& a, const Iv& b) { return a.lo < b.lo; });
    for (size_t k = 1; k < iv.size(); ++k) {
        if (iv[k].lo < iv[k - 1].hi) {
            *err = "entries " + std::to_string(iv[k - 1].idx) + " and " + std::to_string(iv[k].idx) + " overlap";
            return MUON_E_LAYOUT;
        }
    }

    // ---- expand into matrices, short-side frame ----
    const bool nm = P.hp.normuon != 0;
    int64_t ew_tiles = 0;
    for (int e = 0; e < n; ++e) {
        const muon_matrix& t = table[e];
        for (int64_t k = 0; k < t.count; ++k) {
            MatDesc d;
            std::memset(&d, 0, sizeof(d));
            d.p_off = t.offset + k * t.rows * t.cols;
            d.R = (int32_t)t.rows;
            d.C = (int32_t)t.cols;
            d.transposed = t.rows > t.cols ? 1 : 0;
            d.m = (int32_t)std::min(t.rows, t.cols);
            d.n = (int32_t)std::max(t.rows, t.cols);
            d.T = pick_tile(d.m, P.hp.ns_precision == MUON_NS_FP32);
            d.m_pad = (int32_t)round_up(d.m, d.T);
            d.n_pad = (int32_t)round_up(d.n, d.T);
            if ((int64_t)d.m_pad * d.n_pad >= (INT64_C(1) << 30)) {
                *err = "entry " + std::to_string(e) + ": matrix too large for one tile grid";
                return MUON_E_SHAPE;
            }
            d.lr_mul = t.lr_mul;
            d.wd_mul = t.wd_mul;
            d.shape_scale = (float)std::sqrt(std::max(1.0, (double)t.rows / (double)t.cols));
            d.vec_ok = (d.p_off % 4 == 0) && (d.C % 4 == 0);
            const bool act = t.frozen == 0;
            P.active_flag.push_back(act ? 1 : 0);
            if (act) {
                d.x_off = P.x_elems;
                d.a_off = P.a_elems;
                d.row_off = (int32_t)P.rows_total;
                d.rowpart_off = nm ? P.rowpart_elems : 0;
                // elementwise tiles: 64 x 64 over the valid block rounded up to
                // 64 (transposed), else runs of kEwLinear stored elements; the X~
                // padding outside them is zeroed once at init and never written
                if (d.transposed) {
                    d.ew_tiles_n = (d.n + kEwTile - 1) / kEwTile;
                    d.ew_count = ((d.m + kEwTile - 1) / kEwTile) * d.ew_tiles_n;
                } else {
                    d.ew_tiles_n = 0;
                    d.ew_count = (int32_t)((t.rows * t.cols + kEwLinear - 1) / kEwLinear);
                }
                d.ew_start = (int32_t)ew_tiles;
                P.x_elems += (int64_t)d.m_pad * d.n_pad;
                P.a_elems += (int64_t)d.m_pad * d.m_pad;
                P.rows_total += d.m_pad;
                if (nm) P.rowpart_elems += (int64_t)(d.n_pad / d.T) * d.m_pad;
                ew_tiles += d.ew_count;
                P.active.push_back((int32_t)P.mats.size());
                const double m = d.m, nn = d.n;
                P.ns_alg_flops += P.hp.ns_steps * (m * (m + 1) * nn + m * (m + 1) * m + 2 * m * m * nn);
            }
            P.mats.push_back(d);
        }
    }
    if (ew_tiles >= (INT64_C(1) << 31) || P.rows_total >= (INT64_C(1) << 31)) {
        *err = "table too large";
        return MUON_E_SHAPE;
    }

    // ---- stream groups: longest-processing-time split of the tiled matrices ----
    std::vector<int> group_of(P.mats.size(), 0);
    {
        std::vector<std::pair<double, int32_t>> cost;
        int64_t tiles64 = 0;  // update output in 64 x 64 tiles
        for (int32_t mi : P.active) {
            const MatDesc& d = P.mats[mi];
            if (P.is_small(d)) continue;
            const double m = d.m, nn = d.n;
            cost.push_back({m * (m + 1) * nn + m * (m + 1) * m + 2 * m * m * nn, mi});
            tiles64 += (int64_t)(d.m_pad / 64) * (d.n_pad / 64);
        }
        const int want = P.hp.stream_groups > 0 ? P.hp.stream_groups
                         : (tiles64 >= kAutoSplitMinTiles64 ? kAutoGroups : 1);
        const int ng = std::min<int>(want, (int)(cost.size() / kMinSplit));
        if (ng > 1 && tiles64 <= kMaxSplitTiles64) {
            P.n_groups = ng;
            std::stable_sort(cost.begin(), cost.end(),
                             [](const std::pair<double, int32_t>& a, const std::pair<double, int32_t>& b) {
                                 return a.first > b.first;
                             });
            double load[kMaxGroups] = {};
            for (const auto& c : cost) {
                const int g = (int)(std::min_element(load, load + ng) - load);
                group_of[c.second] = g;
                load[g] += c.first;
            }
        }
    }

    // ---- order the active matrices and their elementwise tiles by group ----
    {
        std::vector<int32_t> ordered;
        for (int grp = 0; grp < P.n_groups; ++grp) {
            P.act_begin[grp] = (int)ordered.size();
            for (int32_t mi : P.active)
                if (group_of[mi] == grp) ordered.push_back(mi);
        }
        P.act_begin[P.n_groups] = (int)ordered.size();
        P.active = ordered;
        // inside a group, the runs of untransposed matrices come before the
        // transposed tiles: mixing the two access patterns in flight costs
        // about 2% of the momentum pass's bandwidth
        P.ew_map.reserve((size_t)ew_tiles);
        for (int grp = 0; grp < P.n_groups; ++grp) {
            P.ew_begin[grp] = (int)P.ew_map.size();
            int64_t xt_bytes = 0;
            for (int pass = 0; pass < 2; ++pass)
                for (int k = P.act_begin[grp]; k < P.act_begin[grp + 1]; ++k) {
                    MatDesc& d = P.mats[P.active[k]];
                    if (d.transposed != pass) continue;
                    d.ew_start = (int32_t)P.ew_map.size();
                    for (int t = 0; t < d.ew_count; ++t) P.ew_map.push_back(P.active[k]);
                    xt_bytes += (int64_t)d.m * d.n * P.esize;
                }
            P.xt_nontemporal[grp] = xt_bytes > kXtCachedMax ? 1 : 0;
        }
        P.ew_begin[P.n_groups] = (int)P.ew_map.size();
    }

    // ---- one-panel matrices, group by group ----
    for (int grp = 0; grp < P.n_groups; ++grp) {
        P.panel_begin[grp] = (int)P.panel.size();
        for (int k = P.act_begin[grp]; k < P.act_begin[grp + 1]; ++k)
            if (P.is_panel(P.mats[P.active[k]])) P.panel.push_back(P.active[k]);
    }
    P.panel_begin[P.n_groups] = (int)P.panel.size();

    // ---- GEMM work lists per (group, tile size) ----
    for (int grp = 0; grp < P.n_groups; ++grp)
    for (int T : {256, 128, 64}) {
        std::vector<std::vector<TileWork>> g, u;
        std::vector<double> cg, cp, cu;
        for (int32_t mi : P.active) {
            const MatDesc& d = P.mats[mi];
            if (d.T != T) continue;
            if (P.is_small(d)) {
                if (grp == 0) {
                    P.small.push_back(mi);
                    P.small_np = std::max(P.small_np, d.n_pad);
                }
                continue;
            }
            if (group_of[mi] != grp || P.is_panel(d)) continue;
            const int tm = d.m_pad / T, tn = d.n_pad / T;
            std::vector<TileWork> gl, ul;
            // the matrix's upper tiles, the diagonal ones last: they compute
            // only their blocks on or above the diagonal, about half a tile
            for (int ti = 0; ti < tm; ++ti)
                for (int tj = ti + 1; tj < tm; ++tj) gl.push_back({mi, (int16_t)ti, (int16_t)tj});
            for (int ti = 0; ti < tm; ++ti) gl.push_back({mi, (int16_t)ti, (int16_t)ti});
            // update tiles in column blocks of at most one XCD's CU count, of
            // near-equal width: the workgroups that run together read every
            // row panel of B but only W column panels of X, not all of them
            const int nb = (tn + std::max(1, kCusPerXcd / tm) - 1) / std::max(1, kCusPerXcd / tm);
            const int W = (tn + nb - 1) / nb;
            for (int tb = 0; tb < tn; tb += W)
                for (int ti = 0; ti < tm; ++ti)
                    for (int tj = tb; tj < std::min(tn, tb + W); ++tj) ul.push_back({mi, (int16_t)ti, (int16_t)tj});
            g.push_back(gl);
            u.push_back(ul);
            cg.push_back(d.n_pad);
            cp.push_back(d.m_pad);
            cu.push_back(d.m_pad);
        }
        if (g.empty()) continue;  // (also when every matrix of this size is small)
        TileList L;
        L.T = T;
        L.group = grp;
        L.gram = order_for_xcds(g, cg);
        L.poly = order_for_xcds(g, cp);
        L.update = order_for_xcds(u, cu);
        P.lists.push_back(std::move(L));
    }

    // ---- Gram / polynomial output stores per group (see kAbCachedMax) ----
    {
        int64_t ab_bytes[kMaxGroups] = {};
        for (int32_t mi : P.active) {
            const MatDesc& d = P.mats[mi];
            if (P.is_small(d) || P.is_panel(d)) continue;
            ab_bytes[group_of[mi]] += (int64_t)d.m_pad * d.m_pad * P.esize;
        }
        for (int grp = 0; grp < P.n_groups; ++grp) P.ab_nontemporal[grp] = ab_bytes[grp] > kAbCachedMax ? 1 : 0;
    }

    // ---- workspace layout ----
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes);
        return o;
    };
    const size_t nmats = P.mats.size();
    P.off_xt = take((size_t)P.x_elems * P.esize);
    P.off_x0 = take((size_t)P.x_elems * P.esize);
    P.off_x1 = take((size_t)P.x_elems * P.esize);
    P.off_a = take((size_t)P.a_elems * P.esize);
    P.off_b = take((size_t)P.a_elems * P.esize);
    P.off_part = take((size_t)ew_tiles * 4);
    P.off_ss = take(nmats * 4);
    P.off_scale = take(nmats * 4);
    P.off_status = take(nmats * 4);
    P.off_v = take((size_t)P.rows_total * 4);
    P.off_f = take((size_t)P.rows_total * 4);
    P.off_rowpart = take((size_t)P.rowpart_elems * 4);
    P.off_mats = take(nmats * sizeof(MatDesc));
    P.off_ewmap = take(P.ew_map.size() * 4);
    P.off_active = take(P.active.size() * 4);
    P.off_small = take(P.small.size() * 4);
    P.off_panel = take(P.panel.size() * 4);
    for (auto& L : P.lists) {
        L.off_gram = take(L.gram.size() * sizeof(TileWork));
        L.off_poly = take(L.poly.size() * sizeof(TileWork));
        L.off_update = take(L.update.size() * sizeof(TileWork));
    }
    P.total_bytes = off;
    *out = std::move(P);
    return MUON_OK;
}

}  // namespace muon

extern "C" void muon_hparams_default(muon_hparams* hp) {
    if (!hp) return;
    std::memset(hp, 0, sizeof(*hp));
    hp->momentum = 0.95f;
    hp->nesterov = 1;
    hp->momentum_kind = MUON_MOMENTUM_LERP;
    hp->ns_steps = 5;
    for (int k = 0; k < MUON_MAX_NS_STEPS; ++k) {
        hp->ns_coeffs[k][0] = 3.4445f;
        hp->ns_coeffs[k][1] = -4.7750f;
        hp->ns_coeffs[k][2] = 2.0315f;
    }
    hp->ns_eps = 1e-7f;
    hp->ns_precision = MUON_NS_BF16;
    hp->normuon = 0;
    hp->normuon_beta2 = 0.95f;
    hp->normuon_eps = 1e-10f;
    hp->weight_decay = 0.0f;
    hp->stream_groups = 0;
}
