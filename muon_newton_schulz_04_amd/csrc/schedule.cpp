// Host-side LR and momentum schedules for muon_step's per-call scalars.
//
// Sources: [P4] "modded-nanogpt 50B-token 长时程训练实验解析", section
// "超参配置解析" (the warmup-stable-decay get_lr: warmup, flat, linear
// warmdown to 0); [P3] the FlexAttention 64K-context record (the same
// schedule with warmdown_iters = 562 of 1875, and the Muon momentum warm-up
// from 0.85 to 0.95 over 500 steps); [P2] "2025-10-27_FixMuonLR", change 3
// (cool-down over the last LR_COOLDOWN_FRAC of the main phase to LR_FLOOR,
// flat at the floor through the extension iterations).

#include <cmath>
#include <limits>

#include "../../include/libmuon.h"

namespace {
constexpr float kNaN = std::numeric_limits<float>::quiet_NaN();
}

extern "C" float muon_lr_wsd(int64_t it, int64_t num_iterations, int64_t warmup_iters, int64_t warmdown_iters) {
    // warmup_iters > num_iterations - warmdown_iters is the sum check without
    // an int64 overflow (all three are non-negative here)
    if (it < 0 || num_iterations <= 0 || it >= num_iterations || warmup_iters < 0 || warmdown_iters < 0 ||
        warmdown_iters > num_iterations || warmup_iters > num_iterations - warmdown_iters)
        return kNaN;
    if (it < warmup_iters) return (float)((double)(it + 1) / (double)warmup_iters);
    if (it < num_iterations - warmdown_iters) return 1.0f;
    return (float)((double)(num_iterations - it) / (double)warmdown_iters);
}

extern "C" float muon_lr_cooldown_floor(int64_t step, int64_t main_iterations, float cooldown_frac, float floor) {
    if (step < 0 || main_iterations <= 0 || !(cooldown_frac > 0.0f) || cooldown_frac > 1.0f || !(floor >= 0.0f) ||
        floor > 1.0f)
        return kNaN;
    const double x = std::fmin((double)step / (double)main_iterations, 1.0);
    const double w = std::fmin(1.0, (1.0 - x) / (double)cooldown_frac);
    return (float)((double)floor + (1.0 - (double)floor) * w);
}

extern "C" float muon_momentum_warmup(int64_t step, int64_t warmup_steps, float start, float end) {
    if (step < 0 || warmup_steps <= 0 || !std::isfinite(start) || !std::isfinite(end)) return kNaN;
    const double frac = std::fmin((double)step / (double)warmup_steps, 1.0);
    return (float)((1.0 - frac) * (double)start + frac * (double)end);
}
