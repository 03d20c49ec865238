// C ABI of libmuon (include/libmuon.h): handle lifecycle, argument checks,
// and the launch sequence of one Muon step on the caller's stream.
//
// Step order ([P4] "modded-nanogpt 50B-token 长时程训练实验解析" section
// "从源码看 Muon 的分布式正交化实现"; [P2] "2025-10-27_FixMuonLR" change 2):
//   momentum + Nesterov -> X~ (short-side frame) and sum u^2
//   ns_steps x (Gram, polynomial, update), normalisation folded into step 0
//   NorMuon row factors (optional)
//   parameter update

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <exception>
#include <memory>
#include <new>
#include <string>
#include <vector>

#include "../../include/libmuon.h"
#include "launch.hpp"
#include "plan.hpp"

struct muon_handle {
    muon::Plan plan;
    int device = 0;
    char* ws = nullptr;
    size_t ws_bytes = 0;
    std::string last_error;
    // optional per-launch event timing
    struct Rec {
        int kind;
        hipEvent_t start, stop;
    };
    bool profiling = false;
    std::vector<Rec> recs;          // recorded, not yet read
    std::vector<hipEvent_t> spare;  // events for reuse
    // stream groups 1 .. n_groups - 1: their own streams (default priority,
    // non-blocking), the events that start each one after the previous
    // group's momentum, and the events that join them back
    hipStream_t aux[muon::kMaxGroups - 1] = {};
    hipEvent_t ev_fork[muon::kMaxGroups - 1] = {}, ev_join[muon::kMaxGroups - 1] = {};
    ~muon_handle() {
        for (int g = 0; g < muon::kMaxGroups - 1; ++g) {
            if (ev_fork[g]) (void)hipEventDestroy(ev_fork[g]);
            if (ev_join[g]) (void)hipEventDestroy(ev_join[g]);
            if (aux[g]) (void)hipStreamDestroy(aux[g]);
        }
        for (auto& r : recs) {
            (void)hipEventDestroy(r.start);
            (void)hipEventDestroy(r.stop);
        }
        for (auto e : spare) (void)hipEventDestroy(e);
    }
};

namespace {

thread_local std::string g_last_error;

// Records msg as the handle's (or this thread's) last error. Never throws:
// if the message cannot be stored, the status still reaches the caller.
muon_status fail(muon_handle* h, muon_status s, const std::string& msg) noexcept {
    try {
        if (h)
            h->last_error = msg;
        else
            g_last_error = msg;
    } catch (...) {
    }
    return s;
}

muon_status fail(muon_handle* h, muon_status s, const char* msg) noexcept {
    try {
        if (h)
            h->last_error = msg;
        else
            g_last_error = msg;
    } catch (...) {
    }
    return s;
}

// Runs the body of an extern "C" entry point; no exception crosses the ABI:
// a host allocation failure (or any other exception from the standard
// library) becomes MUON_E_HOST with its description as the last error.
template <typename F>
muon_status guarded(muon_handle* h, const char* where, F&& body) noexcept {
    try {
        return body();
    } catch (const std::bad_alloc&) {
        return fail(h, MUON_E_HOST, std::string(where) + ": out of host memory");
    } catch (const std::exception& ex) {
        return fail(h, MUON_E_HOST, std::string(where) + ": " + ex.what());
    } catch (...) {
        return fail(h, MUON_E_HOST, where);
    }
}

muon_status hip_fail(muon_handle* h, hipError_t e, const char* where) {
    std::string msg = std::string(where) + ": " + hipGetErrorString(e);
    return fail(h, MUON_E_HIP, msg);
}

muon::LaunchCtx make_ctx(const muon_handle* h, hipStream_t stream) {
    const muon::Plan& P = h->plan;
    char* ws = h->ws;
    muon::LaunchCtx L;
    L.stream = stream;
    L.fp32 = P.hp.ns_precision == MUON_NS_FP32;
    L.mats = reinterpret_cast<const muon::MatDesc*>(ws + P.off_mats);
    L.ew_map = reinterpret_cast<const int32_t*>(ws + P.off_ewmap);
    L.active = reinterpret_cast<const int32_t*>(ws + P.off_active);
    L.ew_tile0 = 0;
    L.ew_tiles = (int)P.ew_map.size();
    L.n_active = (int)P.active.size();
    L.xt = ws + P.off_xt;
    // the whole table as one launch (the step sets this per stream group)
    L.xt_nontemporal = P.n_groups == 1 ? P.xt_nontemporal[0] : 0;
    L.ab_nontemporal = P.n_groups == 1 ? P.ab_nontemporal[0] : 0;
    L.x0 = ws + P.off_x0;
    L.x1 = ws + P.off_x1;
    L.a = ws + P.off_a;
    L.b = ws + P.off_b;
    L.partials = reinterpret_cast<float*>(ws + P.off_part);
    L.ss = reinterpret_cast<float*>(ws + P.off_ss);
    L.scale = reinterpret_cast<float*>(ws + P.off_scale);
    L.status = reinterpret_cast<int32_t*>(ws + P.off_status);
    L.v = reinterpret_cast<float*>(ws + P.off_v);
    L.f = reinterpret_cast<float*>(ws + P.off_f);
    L.rowpart = reinterpret_cast<float*>(ws + P.off_rowpart);
    L.rows_total = P.rows_total;
    return L;
}

muon::GemmList make_list(const muon_handle* h, const muon::TileList& T) {
    muon::GemmList G;
    G.T = T.T;
    G.gram = reinterpret_cast<const muon::TileWork*>(h->ws + T.off_gram);
    G.n_gram = (int)T.gram.size();
    G.poly = reinterpret_cast<const muon::TileWork*>(h->ws + T.off_poly);
    G.n_poly = (int)T.poly.size();
    G.update = reinterpret_cast<const muon::TileWork*>(h->ws + T.off_update);
    G.n_update = (int)T.update.size();
    return G;
}

// Final Newton–Schulz output buffer: iteration 0 writes x1, then x0 / x1 alternate.
void* ns_out(const muon_handle* h) {
    const muon::Plan& P = h->plan;
    return h->ws + ((P.hp.ns_steps & 1) ? P.off_x1 : P.off_x0);
}

muon_status check_device(muon_handle* h) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(h, e, "hipGetDevice");
    if (cur != h->device)
        return fail(h, MUON_E_STATE, "device " + std::to_string(h->device) + " is not current (current is " +
                                         std::to_string(cur) + ")");
    return MUON_OK;
}

hipError_t take_event(muon_handle* h, hipEvent_t* ev) {
    if (!h->spare.empty()) {
        *ev = h->spare.back();
        h->spare.pop_back();
        return hipSuccess;
    }
    return hipEventCreate(ev);
}

bool overlap(const void* a, const void* b, int64_t bytes) {
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + bytes && y < x + bytes;
}

}  // namespace

extern "C" {

muon_status muon_workspace_bytes(const muon_matrix* table, int32_t n, const muon_hparams* hp, size_t* out_bytes) {
    return guarded(nullptr, "muon_workspace_bytes", [&]() -> muon_status {
        if (!out_bytes) return fail(nullptr, MUON_E_INVALID_ARG, "null out_bytes");
        muon::Plan P;
        std::string err;
        muon_status s = muon::build_plan(table, n, hp, &P, &err);
        if (s != MUON_OK) return fail(nullptr, s, err);
        *out_bytes = P.total_bytes;
        return MUON_OK;
    });
}

// muon_init (use_static = false: the caller's workspace) and muon_init_static
// (the library's static workspace on `device`, one stream group)
static muon_status init_impl(muon_handle** out, const muon_matrix* table, int32_t n, const muon_hparams* hp,
                             void* workspace, size_t ws_bytes, int32_t device, bool use_static) {
    if (!out) return fail(nullptr, MUON_E_INVALID_ARG, "null handle output");
    *out = nullptr;
    std::unique_ptr<muon_handle> owner(new muon_handle());
    muon_handle* h = owner.get();
    std::string err;
    muon_hparams hp1;
    if (use_static) {
        // no stream or event is created: every launch on the caller's stream
        if (hp)
            hp1 = *hp;
        else
            muon_hparams_default(&hp1);
        hp1.stream_groups = 1;
        hp = &hp1;
    }
    muon_status s = muon::build_plan(table, n, hp, &h->plan, &err);
    if (s != MUON_OK) return fail(nullptr, s, err);
    const muon::Plan& P = h->plan;
    if (use_static) {
        if (P.total_bytes > MUON_STATIC_WORKSPACE_BYTES)
            return fail(nullptr, MUON_E_WORKSPACE,
                        "table needs " + std::to_string(P.total_bytes) + " bytes of workspace; the static workspace "
                        "holds " + std::to_string(MUON_STATIC_WORKSPACE_BYTES));
    } else if (P.total_bytes > 0) {
        if (!workspace) {
            return fail(nullptr, MUON_E_WORKSPACE, "null workspace");
        }
        if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) {
            return fail(nullptr, MUON_E_WORKSPACE, "workspace not 256-byte aligned");
        }
        if (ws_bytes < P.total_bytes) {
            return fail(nullptr, MUON_E_WORKSPACE,
                        "workspace too small: need " + std::to_string(P.total_bytes) + " bytes");
        }
    }
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count < 1) {
        return fail(nullptr, MUON_E_NO_DEVICE, "no HIP device");
    }
    if (device < 0 || device >= count) {
        return fail(nullptr, MUON_E_NO_DEVICE, "device index out of range");
    }
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess) {
        return hip_fail(nullptr, e, "hipGetDeviceProperties");
    }
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
        return fail(nullptr, MUON_E_NO_DEVICE, std::string("device is ") + prop.gcnArchName + ", need gfx950");
    }
    int prev = -1;
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    e = hipSetDevice(device);
    if (e != hipSuccess) {
        return hip_fail(nullptr, e, "hipSetDevice");
    }
    if (use_static) {
        // the device address of the static array on this device (never its host-side name)
        e = muon::static_scratch_address(device, &workspace);
        if (e != hipSuccess) {
            if (prev >= 0) (void)hipSetDevice(prev);
            return hip_fail(nullptr, e, "hipGetSymbolAddress of the static workspace");
        }
        ws_bytes = MUON_STATIC_WORKSPACE_BYTES;
    }
    h->device = device;
    h->ws = static_cast<char*>(workspace);
    h->ws_bytes = ws_bytes;
    auto up = [&](size_t off, const void* src, size_t bytes) -> hipError_t {
        if (bytes == 0) return hipSuccess;
        return hipMemcpy(h->ws + off, src, bytes, hipMemcpyHostToDevice);
    };
    e = up(P.off_mats, P.mats.data(), P.mats.size() * sizeof(muon::MatDesc));
    if (e == hipSuccess) e = up(P.off_ewmap, P.ew_map.data(), P.ew_map.size() * 4);
    if (e == hipSuccess) e = up(P.off_active, P.active.data(), P.active.size() * 4);
    if (e == hipSuccess) e = up(P.off_small, P.small.data(), P.small.size() * 4);
    if (e == hipSuccess) e = up(P.off_panel, P.panel.data(), P.panel.size() * 4);
    for (const auto& L : P.lists) {
        if (e == hipSuccess) e = up(L.off_gram, L.gram.data(), L.gram.size() * sizeof(muon::TileWork));
        if (e == hipSuccess) e = up(L.off_poly, L.poly.data(), L.poly.size() * sizeof(muon::TileWork));
        if (e == hipSuccess) e = up(L.off_update, L.update.data(), L.update.size() * sizeof(muon::TileWork));
    }
    // the one-workgroup kernel's dynamic LDS, once for this device
    if (e == hipSuccess && !P.small.empty()) e = muon::prepare_ns_small(P.small_np);
    for (int g = 0; g + 1 < P.n_groups && e == hipSuccess; ++g) {
        e = hipStreamCreateWithFlags(&h->aux[g], hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_fork[g], hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&h->ev_join[g], hipEventDisableTiming);
    }
    if (e == hipSuccess && P.rows_total) e = hipMemset(h->ws + P.off_v, 0, (size_t)P.rows_total * 4);
    if (e == hipSuccess && P.mats.size()) e = hipMemset(h->ws + P.off_status, 0, P.mats.size() * 4);
    // the momentum kernel writes X~ only over the valid block rounded up to
    // 64 x 64 tiles; the rest of the padding stays as zeroed here
    if (e == hipSuccess && P.x_elems) e = hipMemset(h->ws + P.off_xt, 0, (size_t)P.x_elems * P.esize);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (prev >= 0) (void)hipSetDevice(prev);
    if (e != hipSuccess) {
        return hip_fail(nullptr, e, "uploading descriptors");
    }
    *out = owner.release();
    return MUON_OK;
}

muon_status muon_init(muon_handle** out, const muon_matrix* table, int32_t n, const muon_hparams* hp, void* workspace,
                      size_t ws_bytes, int32_t device) {
    return guarded(nullptr, "muon_init",
                   [&]() { return init_impl(out, table, n, hp, workspace, ws_bytes, device, false); });
}

muon_status muon_init_static(muon_handle** out, const muon_matrix* table, int32_t n, const muon_hparams* hp,
                             int32_t device) {
    return guarded(nullptr, "muon_init_static",
                   [&]() { return init_impl(out, table, n, hp, nullptr, 0, device, true); });
}

static muon_status step_impl(muon_handle* h, float* params, const float* grads, float* momentum, int64_t numel,
                             float lr, float momentum_coef, void* stream) {
    if (!h) return fail(nullptr, MUON_E_INVALID_ARG, "null handle");
    const muon::Plan& P = h->plan;
    if (P.active.empty()) return MUON_OK;
    if (!params || !grads || !momentum) return fail(h, MUON_E_INVALID_ARG, "null params / grads / momentum");
    if (numel < P.extent)
        return fail(h, MUON_E_LAYOUT, "buffers hold " + std::to_string(numel) + " elements, table needs " +
                                          std::to_string(P.extent));
    if ((reinterpret_cast<uintptr_t>(params) | reinterpret_cast<uintptr_t>(grads) |
         reinterpret_cast<uintptr_t>(momentum)) % 16 != 0)
        return fail(h, MUON_E_LAYOUT, "params / grads / momentum must be 16-byte aligned");
    const int64_t bytes = numel * 4;
    if (overlap(params, grads, bytes) || overlap(params, momentum, bytes) || overlap(grads, momentum, bytes))
        return fail(h, MUON_E_INVALID_ARG, "params, grads and momentum must not overlap");
    if (!std::isfinite(lr)) return fail(h, MUON_E_INVALID_ARG, "non-finite lr");
    float beta = P.hp.momentum;
    if (momentum_coef >= 0.f) {
        if (!(momentum_coef <= 1.f)) return fail(h, MUON_E_INVALID_ARG, "momentum_coef must be in [0, 1]");
        beta = momentum_coef;
    } else if (!(momentum_coef < 0.f)) {
        return fail(h, MUON_E_INVALID_ARG, "momentum_coef is NaN");
    }
    muon_status s = check_device(h);
    if (s != MUON_OK) return s;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const muon::LaunchCtx L = make_ctx(h, st);
    hipError_t e = hipSuccess;
    // run one launch on stream `on`, bracketed by events when profiling
    auto run_on = [&](hipStream_t on, int kind, const char* what, auto&& launch) -> muon_status {
        hipEvent_t a = nullptr, b = nullptr;
        if (h->profiling) {
            hipError_t pe = take_event(h, &a);
            if (pe == hipSuccess) pe = take_event(h, &b);
            if (pe == hipSuccess) pe = hipEventRecord(a, on);
            if (pe != hipSuccess) return hip_fail(h, pe, "profiling event");
        }
        hipError_t le = launch();
        if (le != hipSuccess) return hip_fail(h, le, what);
        if (h->profiling) {
            hipError_t pe = hipEventRecord(b, on);
            if (pe != hipSuccess) return hip_fail(h, pe, "profiling event");
            h->recs.push_back({kind, a, b});
        }
        return MUON_OK;
    };
    const int steps = P.hp.ns_steps;
    // Each stream group runs its whole chain: momentum of its matrices, its
    // one-panel Newton–Schulz launch (all iterations; in group 0 followed by
    // the small-matrix one), its tiled Newton–Schulz launches, NorMuon and the
    // parameter update. Group 0 runs on the
    // caller's stream; group g > 0 on the handle's stream g - 1, which starts
    // once group g - 1's momentum is done and joins the caller's stream at
    // the end. The stagger puts each group's momentum under the previous
    // groups' first GEMMs and the parameter updates under the last groups'
    // GEMMs. Launches are issued iteration by iteration, round-robin over the
    // groups, so every stream has work queued early.
    muon::LaunchCtx Lg[muon::kMaxGroups];
    hipStream_t sg[muon::kMaxGroups];
    for (int grp = 0; grp < P.n_groups; ++grp) {
        Lg[grp] = L;
        sg[grp] = grp == 0 ? st : h->aux[grp - 1];
        Lg[grp].stream = sg[grp];
        Lg[grp].ew_tile0 = P.ew_begin[grp];
        Lg[grp].ew_tiles = P.ew_begin[grp + 1] - P.ew_begin[grp];
        Lg[grp].xt_nontemporal = P.xt_nontemporal[grp];
        Lg[grp].ab_nontemporal = P.ab_nontemporal[grp];
        Lg[grp].active = L.active + P.act_begin[grp];
        Lg[grp].n_active = P.act_begin[grp + 1] - P.act_begin[grp];
    }
    for (int grp = 0; grp < P.n_groups; ++grp) {
        s = run_on(sg[grp], MUON_KERNEL_MOMENTUM, "momentum kernel", [&] {
            return muon::launch_momentum(Lg[grp], grads, momentum, beta, P.hp.nesterov,
                                         P.hp.momentum_kind == MUON_MOMENTUM_HEAVY_BALL);
        });
        if (s != MUON_OK) return s;
        if (grp + 1 < P.n_groups) {
            e = hipEventRecord(h->ev_fork[grp], sg[grp]);
            if (e == hipSuccess) e = hipStreamWaitEvent(sg[grp + 1], h->ev_fork[grp], 0);
            if (e != hipSuccess) return hip_fail(h, e, "stream fork");
        }
    }
    muon::NsCoeffs co_all{};
    std::memcpy(co_all.c, P.hp.ns_coeffs, sizeof(co_all.c));
    co_all.steps = steps;
    co_all.eps = P.hp.ns_eps;
    for (int k = 0; k < steps; ++k) {
        void* xin = k == 0 ? L.xt : ((k & 1) ? L.x1 : L.x0);
        void* xout = k == 0 ? L.x1 : ((k & 1) ? L.x0 : L.x1);
        const float ca = P.hp.ns_coeffs[k][0], cb = P.hp.ns_coeffs[k][1], cc = P.hp.ns_coeffs[k][2];
        const int first = k == 0;
        const int rowstats = (k == steps - 1) && P.hp.normuon;
        for (int grp = 0; grp < P.n_groups; ++grp) {
            // the group's one-panel matrices: every iteration in one launch
            const int np = P.panel_begin[grp + 1] - P.panel_begin[grp];
            if (k == 0 && np > 0) {
                const int32_t* pl = reinterpret_cast<const int32_t*>(h->ws + P.off_panel) + P.panel_begin[grp];
                s = run_on(sg[grp], MUON_KERNEL_NS_PANEL, "panel Newton-Schulz kernel",
                           [&] { return muon::launch_ns_panel(Lg[grp], pl, np, co_all, P.hp.normuon); });
                if (s != MUON_OK) return s;
            }
            // the small matrices, every iteration in one launch, after group 0's
            // panel launch on the same stream: the panels start right after the
            // momentum, and the small matrices follow while the other groups'
            // panels still run (a panel workgroup needs a whole CU, so small
            // workgroups running beside the panels' start would delay them)
            if (k == 0 && grp == 0 && !P.small.empty()) {
                s = run_on(sg[0], MUON_KERNEL_NS_SMALL, "small-matrix Newton-Schulz kernel", [&] {
                    return muon::launch_ns_small(Lg[0], reinterpret_cast<const int32_t*>(h->ws + P.off_small),
                                                 (int)P.small.size(), P.small_np, co_all, ns_out(h), P.hp.normuon);
                });
                if (s != MUON_OK) return s;
            }
            for (const auto& T : P.lists) {
                if (T.group != grp) continue;
                const muon::GemmList G = make_list(h, T);
                const bool big = !L.fp32 && G.T >= 128;
                const muon::LaunchCtx& C = Lg[grp];
                auto stage = [&](int mode, const void* x, const void* a, void* o, int rs) {
                    return big ? muon::launch_ns_stage_big(C, G, mode, x, a, o, ca, cb, cc, first, P.hp.ns_eps, rs)
                               : muon::launch_ns_stage(C, G, mode, x, a, o, ca, cb, cc, first, P.hp.ns_eps, rs);
                };
                s = run_on(sg[grp], MUON_KERNEL_GRAM, "Gram kernel",
                           [&] { return stage(muon::NS_GRAM, xin, nullptr, L.a, 0); });
                if (s != MUON_OK) return s;
                s = run_on(sg[grp], MUON_KERNEL_POLY, "polynomial kernel",
                           [&] { return stage(muon::NS_POLY, nullptr, L.a, L.b, 0); });
                if (s != MUON_OK) return s;
                s = run_on(sg[grp], MUON_KERNEL_UPDATE, "update kernel",
                           [&] { return stage(muon::NS_UPDATE, xin, L.b, xout, rowstats); });
                if (s != MUON_OK) return s;
            }
        }
    }
    for (int grp = 0; grp < P.n_groups; ++grp) {
        const float* f = nullptr;
        if (P.hp.normuon) {
            s = run_on(sg[grp], MUON_KERNEL_NORMUON, "NorMuon kernel",
                       [&] { return muon::launch_normuon(Lg[grp], P.hp.normuon_beta2, P.hp.normuon_eps); });
            if (s != MUON_OK) return s;
            f = L.f;
        }
        s = run_on(sg[grp], MUON_KERNEL_APPLY, "apply kernel",
                   [&] { return muon::launch_apply(Lg[grp], ns_out(h), f, params, lr, P.hp.weight_decay); });
        if (s != MUON_OK) return s;
    }
    for (int grp = 1; grp < P.n_groups; ++grp) {
        e = hipEventRecord(h->ev_join[grp - 1], sg[grp]);
        if (e == hipSuccess) e = hipStreamWaitEvent(st, h->ev_join[grp - 1], 0);
        if (e != hipSuccess) return hip_fail(h, e, "stream join");
    }
    return MUON_OK;
}

muon_status muon_step(muon_handle* h, float* params, const float* grads, float* momentum, int64_t numel, float lr,
                      float momentum_coef, void* stream) {
    return guarded(h, "muon_step",
                   [&]() { return step_impl(h, params, grads, momentum, numel, lr, momentum_coef, stream); });
}

muon_status muon_reset(muon_handle* h, float* momentum, int64_t numel, void* stream) {
    if (!h) return fail(nullptr, MUON_E_INVALID_ARG, "null handle");
    const muon::Plan& P = h->plan;
    if (P.active.empty()) return MUON_OK;
    if (momentum) {
        if (numel < P.extent) return fail(h, MUON_E_LAYOUT, "momentum buffer smaller than the table extent");
    }
    muon_status s = check_device(h);
    if (s != MUON_OK) return s;
    const muon::LaunchCtx L = make_ctx(h, static_cast<hipStream_t>(stream));
    hipError_t e = muon::launch_reset(L, momentum);
    if (e != hipSuccess) return hip_fail(h, e, "reset kernels");
    return MUON_OK;
}

void muon_destroy(muon_handle* h) { delete h; }

const char* muon_status_string(muon_status s) {
    switch (s) {
        case MUON_OK: return "ok";
        case MUON_E_INVALID_ARG: return "invalid argument";
        case MUON_E_SHAPE: return "invalid matrix shape";
        case MUON_E_LAYOUT: return "invalid buffer layout";
        case MUON_E_NO_DEVICE: return "no usable gfx950 device";
        case MUON_E_HIP: return "HIP runtime error";
        case MUON_E_STATE: return "invalid handle state";
        case MUON_E_WORKSPACE: return "invalid workspace";
        case MUON_E_HOST: return "host-side failure";
    }
    return "unknown status";
}

const char* muon_last_error(const muon_handle* h) {
    if (!h) return g_last_error.c_str();
    return h->last_error.c_str();
}

int32_t muon_num_matrices(const muon_handle* h) { return h ? (int32_t)h->plan.mats.size() : 0; }

muon_status muon_matrix_layout(const muon_handle* h, int32_t index, muon_layout* out) {
    if (!h || !out) return MUON_E_INVALID_ARG;
    if (index < 0 || index >= (int32_t)h->plan.mats.size()) return MUON_E_INVALID_ARG;
    const muon::MatDesc& d = h->plan.mats[index];
    out->x_offset = d.x_off;
    out->row_offset = d.row_off;
    out->m = d.m;
    out->n = d.n;
    out->ld = d.n_pad;
    out->m_pad = d.m_pad;
    out->transposed = d.transposed;
    out->active = h->plan.active_flag[index];
    out->stored_rows = d.R;
    out->stored_cols = d.C;
    out->param_offset = d.p_off;
    out->gram_offset = h->plan.active_flag[index] ? d.a_off : -1;
    return MUON_OK;
}

muon_status muon_debug_view(const muon_handle* h, int32_t which, void** dev_ptr, size_t* bytes) {
    if (!h || !dev_ptr || !bytes) return MUON_E_INVALID_ARG;
    const muon::Plan& P = h->plan;
    const size_t nm = P.mats.size();
    switch (which) {
        case MUON_VIEW_XTILDE: *dev_ptr = h->ws + P.off_xt; *bytes = (size_t)P.x_elems * P.esize; break;
        case MUON_VIEW_NS_OUT: *dev_ptr = ns_out(h); *bytes = (size_t)P.x_elems * P.esize; break;
        case MUON_VIEW_SUMSQ: *dev_ptr = h->ws + P.off_ss; *bytes = nm * 4; break;
        case MUON_VIEW_SCALE: *dev_ptr = h->ws + P.off_scale; *bytes = nm * 4; break;
        case MUON_VIEW_V: *dev_ptr = h->ws + P.off_v; *bytes = (size_t)P.rows_total * 4; break;
        case MUON_VIEW_F: *dev_ptr = h->ws + P.off_f; *bytes = (size_t)P.rows_total * 4; break;
        case MUON_VIEW_STATUS: *dev_ptr = h->ws + P.off_status; *bytes = nm * 4; break;
        case MUON_VIEW_GRAM: *dev_ptr = h->ws + P.off_a; *bytes = (size_t)P.a_elems * P.esize; break;
        case MUON_VIEW_POLY: *dev_ptr = h->ws + P.off_b; *bytes = (size_t)P.a_elems * P.esize; break;
        default: return MUON_E_INVALID_ARG;
    }
    return MUON_OK;
}

muon_status muon_work_stats(const muon_handle* h, muon_work* out) {
    if (!h || !out) return MUON_E_INVALID_ARG;
    std::memset(out, 0, sizeof(*out));
    const muon::Plan& P = h->plan;
    const int steps = P.hp.ns_steps;
    const double es = P.esize;
    int64_t act = 0;
    double rows = 0, rowpart = 0;
    for (int32_t mi : P.active) {
        const muon::MatDesc& d = P.mats[mi];
        const double m = d.m, n = d.n;
        const double f_gram = steps * m * (m + 1) * n, f_poly = steps * m * (m + 1) * m, f_upd = steps * 2.0 * m * m * n;
        if (P.is_small(d)) {
            out->flops[MUON_KERNEL_NS_SMALL] += f_gram + f_poly + f_upd;
        } else if (P.is_panel(d)) {
            out->flops[MUON_KERNEL_NS_PANEL] += f_gram + f_poly + f_upd;
        } else {
            out->flops[MUON_KERNEL_GRAM] += f_gram;
            out->flops[MUON_KERNEL_POLY] += f_poly;
            out->flops[MUON_KERNEL_UPDATE] += f_upd;
        }
        act += (int64_t)d.m * d.n;
        rows += m;
        rowpart += (double)(d.n_pad / d.T) * m;
    }
    out->active_elements = act;
    out->bytes[MUON_KERNEL_MOMENTUM] = (double)act * (12.0 + es);
    out->bytes[MUON_KERNEL_APPLY] = (double)act * (8.0 + es);
    if (P.hp.normuon) out->bytes[MUON_KERNEL_NORMUON] = 4.0 * (rowpart + 3.0 * rows);
    const int64_t nl = (int64_t)P.lists.size();
    const int64_t any = P.active.empty() ? 0 : 1;
    out->launches[MUON_KERNEL_MOMENTUM] = any * P.n_groups;
    out->launches[MUON_KERNEL_GRAM] = steps * nl;
    out->launches[MUON_KERNEL_POLY] = steps * nl;
    out->launches[MUON_KERNEL_UPDATE] = steps * nl;
    out->launches[MUON_KERNEL_NS_SMALL] = P.small.empty() ? 0 : 1;
    for (int g = 0; g < P.n_groups; ++g)
        out->launches[MUON_KERNEL_NS_PANEL] += P.panel_begin[g + 1] > P.panel_begin[g] ? 1 : 0;
    out->launches[MUON_KERNEL_NORMUON] = P.hp.normuon ? any * P.n_groups : 0;
    out->launches[MUON_KERNEL_APPLY] = any * P.n_groups;
    return MUON_OK;
}

muon_status muon_profile_enable(muon_handle* h, int32_t on) {
    if (!h) return MUON_E_INVALID_ARG;
    h->profiling = on != 0;
    return MUON_OK;
}

static muon_status profile_read_impl(muon_handle* h, int32_t kernel, int32_t clear, int64_t* launches,
                                     double* total_ms) {
    if (!h || !launches || !total_ms) return MUON_E_INVALID_ARG;
    if (kernel < 0 || kernel >= MUON_KERNEL_COUNT) return MUON_E_INVALID_ARG;
    int64_t n = 0;
    double tot = 0.0;
    for (auto& r : h->recs) {
        if (r.kind != kernel) continue;
        hipError_t e = hipEventSynchronize(r.stop);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) return hip_fail(h, e, "reading profiling events");
        ++n;
        tot += ms;
    }
    *launches = n;
    *total_ms = tot;
    if (clear) {
        for (auto& r : h->recs) {
            (void)hipEventSynchronize(r.stop);
            h->spare.push_back(r.start);
            h->spare.push_back(r.stop);
        }
        h->recs.clear();
    }
    return MUON_OK;
}

muon_status muon_profile_read(muon_handle* h, int32_t kernel, int32_t clear, int64_t* launches, double* total_ms) {
    return guarded(h, "muon_profile_read", [&]() { return profile_read_impl(h, kernel, clear, launches, total_ms); });
}

}  // extern "C"
