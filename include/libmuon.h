/*
 * libmuon — the Muon optimizer step (momentum orthogonalised by quintic
 * Newton–Schulz) for the 2-D weight matrices of a GPT-2-style body, on one
 * AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *  [P4] "modded-nanogpt 50B-token 长时程训练实验解析：Muon vs Adam 与数据复用策略的实证对比",
 *       section "从源码看 Muon 的分布式正交化实现" (Muon's orthogonalisation, from
 *       the source) and section "超参配置解析" (hyper-parameters).
 *  [P2] "2025-10-27_FixMuonLR" record analysis, sections "改动一" (per-matrix
 *       lr_mul / wd_mul, the Muon learning rate) and "改动二" (the vectorised
 *       step, the lerp momentum buffer owned by the group, reset(), the early
 *       qkvo reshape, NorMuon's per-lane second moment).
 *  [P3] "2024-11-19 FlexAttention" record analysis, optimizer section
 *       (Muon on 2-D params, 5 NS steps, momentum warm-up 0.85 -> 0.95).
 *
 * Conventions for every entry point:
 *  - Plain C: pointers and sizes only. Device pointers are HIP device
 *    addresses; `stream` is a hipStream_t passed as void* (NULL = the
 *    default stream of the current device).
 *  - Ownership: the caller owns params, grads, momentum and the workspace.
 *    A handle owns only host memory. The library never allocates device
 *    memory; muon_init uploads its descriptor tables into the caller's
 *    workspace and zeroes its state there, blocking; muon_step and
 *    muon_reset only enqueue work on `stream` and never synchronise.
 *  - Errors: every call returns a muon_status; nothing aborts or throws
 *    across the ABI (a host allocation failure inside the library returns
 *    MUON_E_HOST). Validation happens before any HIP call. A kernel fault
 *    surfaces at the caller's next synchronisation. Handles are not
 *    thread-safe; use one stream per handle per call. muon_step allocates
 *    no memory, host or device (unless muon_profile_enable turned on its
 *    event records).
 */
#ifndef LIBMUON_H
#define LIBMUON_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum muon_status {
    MUON_OK = 0,
    MUON_E_INVALID_ARG = -1, /* null pointer, bad enum, non-finite / out-of-range scalar */
    MUON_E_SHAPE = -2,       /* rows, cols or count < 1 */
    MUON_E_LAYOUT = -3,      /* negative offset, overlap, extent beyond the buffers */
    MUON_E_NO_DEVICE = -4,   /* no HIP device, or the device is not gfx950 */
    MUON_E_HIP = -5,         /* a HIP runtime call failed (see muon_last_error) */
    MUON_E_STATE = -6,       /* misuse of a handle (wrong device current, ...) */
    MUON_E_WORKSPACE = -7,   /* workspace null, misaligned (256 B) or too small */
    MUON_E_HOST = -8         /* host-side failure: out of host memory (the message says what failed) */
} muon_status;

/* One table entry: `count` contiguous row-major [rows, cols] float32 matrices
 * starting at element `offset` of the flat params / grads / momentum buffers
 * (count = 4 expresses the fused qkvo weight as its four [d, d] matrices,
 * [P2] change 2). Only 2-D weights belong here ([P4] Muon source).
 * lr_mul / wd_mul scale lr and weight decay for these matrices ([P2] change 1).
 * frozen != 0: params and momentum of these matrices are never touched. */
typedef struct muon_matrix {
    int64_t rows;
    int64_t cols;
    int64_t count;
    int64_t offset;
    float lr_mul;
    float wd_mul;
    int32_t frozen;
    int32_t reserved; /* must be 0 */
} muon_matrix;

#define MUON_MAX_NS_STEPS 16

enum { MUON_NS_BF16 = 0, MUON_NS_FP32 = 1 };
enum { MUON_MOMENTUM_LERP = 0, MUON_MOMENTUM_HEAVY_BALL = 1 };

/* Hyper-parameters ([P4] hyper-parameter and Muon source sections):
 *  momentum 0.95, nesterov 1, ns_steps 5 with (a, b, c) = (3.4445, -4.7750,
 *  2.0315) per iteration, ns_eps 1e-7, weight_decay 0, NorMuon off
 *  (beta2 0.95, eps 1e-10 when on). ns_coeffs[k] holds (a, b, c) of
 *  iteration k, so a per-iteration schedule can replace the fixed quintic.
 *  momentum_kind LERP: m <- beta m + (1-beta) g, Nesterov u = (1-beta) g + beta m
 *  ([P2] change 2); HEAVY_BALL: m <- beta m + g, Nesterov u = g + beta m
 *  ([P4] Muon source). ns_precision BF16: bf16 MFMA operands with fp32
 *  accumulation; FP32: fp32 throughout (debug / reference mode).
 *  stream_groups (not a method parameter; 0 .. 4, default 0): G > 1 lets
 *  muon_step split the tiled matrices into up to G cost-balanced groups, at
 *  least 2 matrices per group, when their update output is at most 262144
 *  tiles of 64 x 64 (a few tile rounds of the GPU per launch). 0 lets the
 *  library choose: 3 when the update output is at least 4096 such tiles
 *  (one round of 256 x 256 tiles on 256 CUs), 1 for smaller steps, whose
 *  launches are latency-bound. Each group
 *  runs its chain (momentum, Newton–Schulz, NorMuon, update) on its own
 *  stream: group 0 on the caller's stream, group g > 0 on a default-priority
 *  stream the handle owns, started after group g - 1's momentum and joined
 *  back into the caller's stream at the end, so one group's kernels fill
 *  the others' tails and launch gaps. 1 keeps every launch on the caller's
 *  stream. Results are bit-identical for every value. */
typedef struct muon_hparams {
    float momentum;
    int32_t nesterov;
    int32_t momentum_kind;
    int32_t ns_steps;
    float ns_coeffs[MUON_MAX_NS_STEPS][3];
    float ns_eps;
    int32_t ns_precision;
    int32_t normuon;
    float normuon_beta2;
    float normuon_eps;
    float weight_decay;
    int32_t stream_groups;
} muon_hparams;

/* Opaque handle: the host-side plan for one table on one device. */
typedef struct muon_handle muon_handle;

/* Fill *hp with the defaults above. */
void muon_hparams_default(muon_hparams* hp);

/* Bytes of device workspace muon_init needs for this table and hp.
 * Host-only; validates the table (same errors as muon_init).
 * Library plumbing: the pages have no counterpart (their optimizer keeps its
 * buffers in PyTorch tensors). */
muon_status muon_workspace_bytes(const muon_matrix* table, int32_t n, const muon_hparams* hp,
                                 size_t* out_bytes);

/* Validate the host table, build the plan (short-side frame per matrix:
 * matrices with rows > cols run transposed, [P4] Muon source; same-shape
 * matrices batched per launch, [P2] change 2), upload descriptors into
 * `workspace` (device, caller-owned, >= muon_workspace_bytes, 256-B aligned,
 * kept for the handle's lifetime and not written by the caller), and zero
 * the NorMuon state and the Newton–Schulz input buffer (whose padding beyond
 * the matrices' 64 x 64 tiles no step writes again). Blocking: returns after
 * these copies and fills are done. `device` is the HIP device index; it must
 * be current in every later call.
 * n = 0 is allowed (every step is then a no-op). On error *out is NULL. */
muon_status muon_init(muon_handle** out, const muon_matrix* table, int32_t n, const muon_hparams* hp,
                      void* workspace, size_t ws_bytes, int32_t device);

/* Size of the library's own device workspace (64 MiB per GPU). */
#define MUON_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

/* muon_init without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation): the handle's workspace is a file-scope device
 * array of MUON_STATIC_WORKSPACE_BYTES inside the library, one per GPU, held
 * from the library's first use of that GPU until the process ends. Everything
 * else is muon_init's: the same plan, uploads and zeroing (the array keeps
 * the previous handle's contents, so the state that must start at zero is
 * cleared here), blocking, and the returned handle works with muon_step,
 * muon_reset and the views as usual. No device memory is allocated and no
 * stream or event is created: hp->stream_groups is taken as 1.
 * Tables whose muon_workspace_bytes exceed MUON_STATIC_WORKSPACE_BYTES are
 * rejected with MUON_E_WORKSPACE. All handles made this way on one GPU share
 * its array: a later muon_init_static on that GPU takes it over (an earlier
 * handle on the GPU must not be stepped afterwards), and calls on such
 * handles that overlap in time race. */
muon_status muon_init_static(muon_handle** out, const muon_matrix* table, int32_t n, const muon_hparams* hp,
                             int32_t device);

/* One Muon step ([P4] Muon source; [P2] change 2), enqueued on `stream`:
 * momentum + Nesterov, Frobenius normalisation, hp.ns_steps Newton–Schulz
 * iterations, optional NorMuon, and
 *   p <- p (1 - lr lr_mul wd wd_mul) - lr lr_mul max(1, rows/cols)^0.5 O.
 * params, momentum: float32 device buffers of `numel` elements, updated in
 * place; grads: float32 device buffer of `numel` elements, read only. All
 * three share the table's layout and must not alias each other.
 * momentum_coef < 0 uses hp.momentum (a per-call value supports momentum
 * warm-up, [P3]); lr is the per-call learning rate (schedules live with the
 * caller). Errors: MUON_E_LAYOUT if numel < the table's extent,
 * MUON_E_INVALID_ARG for null buffers or non-finite lr. */
muon_status muon_step(muon_handle* h, float* params, const float* grads, float* momentum, int64_t numel,
                      float lr, float momentum_coef, void* stream);

/* Zero the momentum of every non-frozen matrix in `momentum` (numel
 * elements, may be NULL to skip) and the NorMuon second moment, on
 * `stream` ([P2] change 2: reset() after warm-up / capture dirtied them). */
muon_status muon_reset(muon_handle* h, float* momentum, int64_t numel, void* stream);

/* Free the handle (host memory only). NULL is a no-op. Library plumbing,
 * not defined by the pages. */
void muon_destroy(muon_handle* h);

/* Static description of a status code. Library plumbing, not defined by the
 * pages. */
const char* muon_status_string(muon_status s);

/* Detail of the handle's last error ("" if none); NULL handle -> the last
 * error of a failed muon_init / muon_workspace_bytes on this thread. Library
 * plumbing, not defined by the pages. */
const char* muon_last_error(const muon_handle* h);

/* ---- introspection (tests and tools) ------------------------------------
 * Library plumbing, not defined by the pages: these expose the library's own
 * buffers and plan so that tests can compare each stage with an oracle. */

/* Where matrix `index` (0-based over the table with counts expanded) lives
 * in the workspace: short-side shape m <= n, row stride ld (elements) of the
 * padded canonical buffers, element offsets into the X buffers and into the
 * per-row NorMuon arrays, transposed = stored rows > cols, active = !frozen,
 * gram_offset = element offset of its m_pad x m_pad Gram / polynomial
 * buffers (MUON_VIEW_GRAM / MUON_VIEW_POLY; -1 if frozen). */
typedef struct muon_layout {
    int64_t x_offset;
    int64_t row_offset;
    int32_t m, n, ld, m_pad;
    int32_t transposed;
    int32_t active;
    int32_t stored_rows, stored_cols;
    int64_t param_offset;
    int64_t gram_offset;
} muon_layout;

muon_status muon_matrix_layout(const muon_handle* h, int32_t index, muon_layout* out);

/* Number of matrices (counts expanded). */
int32_t muon_num_matrices(const muon_handle* h);

enum {
    MUON_VIEW_XTILDE = 0,  /* momentum kernel output: canonical, padded X~ (bf16 or fp32) */
    MUON_VIEW_NS_OUT = 1,  /* final Newton–Schulz output, same layout */
    MUON_VIEW_SUMSQ = 2,   /* float32 [num_matrices]: sum of u^2 */
    MUON_VIEW_SCALE = 3,   /* float32 [num_matrices]: s = 1/(sqrt(sumsq) + ns_eps) */
    MUON_VIEW_V = 4,       /* float32 per canonical row: NorMuon second moment */
    MUON_VIEW_F = 5,       /* float32 per canonical row: NorMuon row factor */
    MUON_VIEW_STATUS = 6,  /* int32 [num_matrices]: bit 0 = non-finite u seen this step */
    MUON_VIEW_GRAM = 7,    /* the last iteration's A = X X^T: m_pad x m_pad per matrix at its gram_offset
                              (tiled and one-panel matrices; the short-side <= 64 path keeps A in LDS, its
                              region is unspecified) */
    MUON_VIEW_POLY = 8     /* the last iteration's B = b A + c A A, same layout as MUON_VIEW_GRAM */
};

/* Device pointer and byte size of an internal buffer, valid after the
 * stream work of the last muon_step has completed. */
muon_status muon_debug_view(const muon_handle* h, int32_t which, void** dev_ptr, size_t* bytes);

/* ---- host-side schedules (scalars for muon_step's lr and momentum_coef) ---
 * Pure host functions; no handle, no device. Out-of-range arguments give NaN. */

/* Warmup-stable-decay LR multiplier ([P4] hyper-parameter section, and the
 * [P3] FlexAttention record's schedule): for step it in [0, num_iterations),
 * (it + 1) / warmup_iters while it < warmup_iters, then 1, and from
 * num_iterations - warmdown_iters on (num_iterations - it) / warmdown_iters,
 * i.e. linear to 0 at the end. The Muon group uses warmup_iters = 0. */
float muon_lr_wsd(int64_t it, int64_t num_iterations, int64_t warmup_iters, int64_t warmdown_iters);

/* Cool-down-to-floor LR multiplier ([P2] change 3, reading stated in the
 * design notes): with x = min(step / main_iterations, 1), the multiplier is
 * floor + (1 - floor) * min(1, (1 - x) / cooldown_frac): 1 until the last
 * cooldown_frac of the main phase, then linear down to floor, and flat at
 * floor for every extension step past main_iterations ([P2]: 0.80, 0.30). */
float muon_lr_cooldown_floor(int64_t step, int64_t main_iterations, float cooldown_frac, float floor);

/* Momentum warm-up ([P3] training loop): frac = min(step / warmup_steps, 1),
 * momentum = (1 - frac) start + frac end ([P3]: 500 steps, 0.85 -> 0.95). */
float muon_momentum_warmup(int64_t step, int64_t warmup_steps, float start, float end);

/* ---- measurement (benchmarks) -------------------------------------------
 * Library plumbing, not defined by the pages. */

enum {
    MUON_KERNEL_MOMENTUM = 0, /* momentum + Nesterov + cast + sum of squares */
    MUON_KERNEL_GRAM = 1,     /* A = X X^T (upper tiles, mirrored) */
    MUON_KERNEL_POLY = 2,     /* B = b A + c A^2 (upper tiles, mirrored) */
    MUON_KERNEL_UPDATE = 3,   /* X <- a X + B X (a X added in fp32 before rounding) */
    MUON_KERNEL_NORMUON = 4,  /* NorMuon row factors */
    MUON_KERNEL_APPLY = 5,    /* parameter update */
    MUON_KERNEL_NS_SMALL = 6, /* every Newton-Schulz iteration of the bf16 matrices whose
                               * short side is at most 64 (one workgroup per matrix) */
    MUON_KERNEL_NS_PANEL = 7, /* every Newton-Schulz iteration of the bf16 matrices whose
                               * short side is 256 and long side at most 4096 (one
                               * workgroup per matrix, A and B kept in LDS) */
    MUON_KERNEL_COUNT = 8
};

/* Algorithmic work of one muon_step for this plan (frozen matrices excluded).
 * flops[k]: floating-point operations of kernel class k per step, counting a
 * symmetric product (Gram, A^2) as m(m+1)k; bytes[k]: bytes a kernel class
 * must move per step (momentum: g, m read, m, X~ written; apply: O, p read,
 * p written; NorMuon: row partials, v, f); launches[k]: launches per step. */
typedef struct muon_work {
    double flops[MUON_KERNEL_COUNT];
    double bytes[MUON_KERNEL_COUNT];
    int64_t launches[MUON_KERNEL_COUNT];
    int64_t active_elements;
} muon_work;

muon_status muon_work_stats(const muon_handle* h, muon_work* out);

/* on != 0: every later muon_step records a pair of HIP events around each
 * kernel launch on its stream (host-side records only, no device memory).
 * on == 0 stops recording; recorded pairs are kept until read. */
muon_status muon_profile_enable(muon_handle* h, int32_t on);

/* Wait for the recorded events and return, for kernel class `kernel`, the
 * number of recorded launches and their summed duration in milliseconds.
 * clear != 0 drops every record afterwards. */
muon_status muon_profile_read(muon_handle* h, int32_t kernel, int32_t clear, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* LIBMUON_H */
