// Host-side checks of the planner's decisions (no device): plans built
// straight from plan.cpp for the workloads' tables and a few edge tables.
// Checked for each plan:
//  - every active tiled matrix has each of its upper tiles exactly once in
//    the Gram list and in the polynomial list, and each of its output tiles
//    exactly once in the update list, all in lists of its own stream group
//    and tile size, and never in more than one kernel class (tiled, one-panel
//    or small);
//  - frozen matrices appear nowhere;
//  - the stream-group count and, per group, the cache policies: X~ stored
//    nontemporally when the group's X~ exceeds 256 MB, A and B when its Gram
//    output does.
// Exit status 0 when every expectation holds.
#include <cstdint>
#include <cstdio>
#include <map>
#include <set>
#include <string>
#include <tuple>
#include <vector>

#include "plan.hpp"

using namespace muon;

static int fails = 0;
#define EXPECT(c)                                                      \
    do {                                                               \
        if (!(c)) {                                                    \
            std::fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #c); \
            ++fails;                                                   \
        }                                                              \
    } while (0)

struct Table {
    std::vector<muon_matrix> t;
    int64_t off = 0;
    void add(int64_t r, int64_t c, int64_t count, int32_t frozen = 0) {
        muon_matrix m{};
        m.rows = r;
        m.cols = c;
        m.count = count;
        m.offset = off;
        m.lr_mul = 1.0f;
        m.wd_mul = 1.0f;
        m.frozen = frozen;
        t.push_back(m);
        off += r * c * count;
    }
    // layers x (qkvo [4, d, d] + c_fc [d, 4d] + c_proj [4d, d])
    void body(int layers, int64_t d) {
        for (int l = 0; l < layers; ++l) {
            add(d, d, 4);
            add(d, 4 * d, 1);
            add(4 * d, d, 1);
        }
    }
};

static bool plan(const Table& tb, int groups, int fp32, Plan* P) {
    muon_hparams hp;
    muon_hparams_default(&hp);
    hp.stream_groups = groups;
    if (fp32) hp.ns_precision = MUON_NS_FP32;
    std::string err;
    const muon_status s = build_plan(tb.t.data(), (int32_t)tb.t.size(), &hp, P, &err);
    if (s != MUON_OK) std::fprintf(stderr, "build_plan: %s\n", err.c_str());
    return s == MUON_OK;
}

// The coverage properties of the lists; returns the number of tiled matrices.
static int check_lists(const Plan& P) {
    std::vector<int> group_of(P.mats.size(), -1);
    for (int g = 0; g < P.n_groups; ++g)
        for (int k = P.act_begin[g]; k < P.act_begin[g + 1]; ++k) group_of[P.active[k]] = g;
    std::set<int32_t> active(P.active.begin(), P.active.end());
    std::set<int32_t> small(P.small.begin(), P.small.end());
    std::set<int32_t> panel(P.panel.begin(), P.panel.end());
    EXPECT(small.size() == P.small.size() && panel.size() == P.panel.size());
    std::map<std::tuple<int, int, int>, int> gram, poly, upd;
    std::set<int32_t> tiled;
    for (const TileList& L : P.lists) {
        for (const TileWork& w : L.gram) {
            const MatDesc& d = P.mats[w.mat];
            EXPECT(d.T == L.T && group_of[w.mat] == L.group && w.ti <= w.tj);
            ++gram[{w.mat, w.ti, w.tj}];
            tiled.insert(w.mat);
        }
        for (const TileWork& w : L.poly) {
            const MatDesc& d = P.mats[w.mat];
            EXPECT(d.T == L.T && group_of[w.mat] == L.group && w.ti <= w.tj);
            ++poly[{w.mat, w.ti, w.tj}];
        }
        for (const TileWork& w : L.update) {
            const MatDesc& d = P.mats[w.mat];
            EXPECT(d.T == L.T && group_of[w.mat] == L.group);
            EXPECT(w.ti < d.m_pad / d.T && w.tj < d.n_pad / d.T);
            ++upd[{w.mat, w.ti, w.tj}];
        }
    }
    for (int32_t mi : tiled) {
        const MatDesc& d = P.mats[mi];
        EXPECT(active.count(mi) && !small.count(mi) && !panel.count(mi));
        const int tm = d.m_pad / d.T, tn = d.n_pad / d.T;
        for (int i = 0; i < tm; ++i)
            for (int j = i; j < tm; ++j) {
                EXPECT((gram[{mi, i, j}] == 1));
                EXPECT((poly[{mi, i, j}] == 1));
            }
        for (int i = 0; i < tm; ++i)
            for (int j = 0; j < tn; ++j) EXPECT((upd[{mi, i, j}] == 1));
    }
    EXPECT(gram.size() == poly.size());
    for (const auto& kv : gram) EXPECT(kv.second == 1);
    for (const auto& kv : upd) EXPECT(kv.second == 1);
    // every active matrix runs in exactly one Newton–Schulz kernel class
    for (int32_t mi : active) EXPECT(((int)tiled.count(mi) + (int)small.count(mi) + (int)panel.count(mi)) == 1);
    for (int32_t mi : small) EXPECT(active.count(mi));
    for (int32_t mi : panel) EXPECT(active.count(mi));
    return (int)tiled.size();
}

int main() {
    Plan P;
    {
        // the 124M body: three stream groups, every cache policy normal
        Table tb;
        tb.body(12, 768);
        EXPECT(plan(tb, 3, 0, &P));
        EXPECT(P.n_groups == 3);
        EXPECT(check_lists(P) == 72);
        for (int g = 0; g < P.n_groups; ++g) EXPECT(P.xt_nontemporal[g] == 0 && P.ab_nontemporal[g] == 0);
        for (const MatDesc& d : P.mats) EXPECT(d.T == 256 && d.m_pad == 768);
    }
    {
        // stream_groups = 0: the planner chooses three groups from 4096 update
        // tiles of 64 x 64 on (one round of 256-tiles on the GPU), one below
        Table tiny, mid, big, body124m;
        tiny.body(1, 128);       // 48 tiles
        mid.body(4, 512);        // 3072 tiles
        big.body(4, 768);        // 6912 tiles
        body124m.body(12, 768);  // 20736 tiles
        EXPECT(plan(tiny, 0, 0, &P) && P.n_groups == 1);
        EXPECT(plan(tiny, 0, 1, &P) && P.n_groups == 1);
        EXPECT(plan(mid, 0, 0, &P) && P.n_groups == 1);
        check_lists(P);
        EXPECT(plan(big, 0, 0, &P) && P.n_groups == 3);
        check_lists(P);
        EXPECT(plan(body124m, 0, 0, &P) && P.n_groups == 3);
        // an explicit count is kept for small steps too (at least two tiled
        // matrices per group)
        EXPECT(plan(tiny, 3, 0, &P) && P.n_groups == 3);
        check_lists(P);
        // the stress batch's one-panel matrices count: 192 x 64 tiles
        Table stress;
        stress.add(64, 64, 4096);
        stress.add(256, 1024, 192);
        EXPECT(plan(stress, 0, 0, &P) && P.n_groups == 3);
    }
    {
        // the same body in one group: X~ (170 MB) and A (85 MB) fit the MALL
        Table tb;
        tb.body(12, 768);
        EXPECT(plan(tb, 1, 0, &P));
        EXPECT(P.n_groups == 1 && P.xt_nontemporal[0] == 0 && P.ab_nontemporal[0] == 0);
        EXPECT(check_lists(P) == 72);
    }
    {
        // the 1.5B body: one group (too many tiles to split), X~ (2.9 GB)
        // and A (1.85 GB) both streamed
        Table tb;
        tb.body(48, 1600);
        EXPECT(plan(tb, 3, 0, &P));
        EXPECT(P.n_groups == 1 && P.xt_nontemporal[0] == 1 && P.ab_nontemporal[0] == 1);
        EXPECT(check_lists(P) == 288);
        for (const MatDesc& d : P.mats) EXPECT(d.T == 256 && d.m_pad == 1792);
    }
    {
        // the boundary of the A rule: a 2048^2 bf16 A is 8 MiB, so 32 of
        // them are exactly 256 MiB (kept cached) and 33 exceed it (streamed)
        Table big, small;
        big.add(2048, 2048, 33);
        small.add(2048, 2048, 32);
        EXPECT(plan(big, 1, 0, &P));
        EXPECT(P.ab_nontemporal[0] == 1);
        EXPECT(plan(small, 1, 0, &P));
        EXPECT(P.ab_nontemporal[0] == 0);
    }
    {
        // an fp32 group whose X~ exceeds 256 MB: X~ streamed
        Table tb;
        tb.add(2048, 4352, 4);
        tb.add(4352, 2048, 4);
        EXPECT(plan(tb, 1, 1, &P));
        EXPECT(P.n_groups == 1 && P.xt_nontemporal[0] == 1);
        check_lists(P);
    }
    {
        // the stress batch: 64 x 64 matrices in the small kernel, 256 x 1024
        // ones in the one-panel kernel, nothing tiled; frozen ones nowhere
        Table tb;
        tb.add(64, 64, 4096);
        tb.add(256, 1024, 192);
        tb.add(1024, 256, 64, 1);
        EXPECT(plan(tb, 3, 0, &P));
        EXPECT(check_lists(P) == 0);
        EXPECT(P.small.size() == 4096 && P.panel.size() == 192 && P.active.size() == 4096 + 192);
    }
    {
        // ragged shapes across the tile classes
        Table tb;
        tb.add(200, 200, 2);
        tb.add(520, 136, 1);
        tb.add(40, 100, 1);
        tb.add(1, 7, 1);
        tb.add(96, 160, 1, 1);
        tb.add(1000, 700, 1);
        tb.add(2100, 700, 1);
        tb.add(100, 1200, 1);
        EXPECT(plan(tb, 2, 0, &P));
        check_lists(P);
        EXPECT(plan(tb, 1, 1, &P));  // fp32: no small or panel kernel
        EXPECT(P.small.empty() && P.panel.empty());
        check_lists(P);
    }
    if (fails == 0) std::printf("all expectations hold\n");
    return fails == 0 ? 0 : 1;
}
