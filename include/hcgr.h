/*
 * hcgr.h -- C ABI of the MI355X (gfx950) Hyper-Connection Gated Residual op.
 *
 * The op (ROCm/aiter pull request #5913, "Two-stage Hyper-Connection Gated
 * Residual kernel", section "Technical Details") takes, per token, the HC
 * incoming residual streams R (flattened to K = HC*HS values, stream-major:
 * element (s, c) at k = s*HS + c), the block output y [HS] and the incoming
 * injection logits inj [HC], and computes
 *   (COMBINE) iw[s] = 2*sigmoid(inj[s]/HC);  R2[s,c] = R[s,c] + y[c]*iw[s]
 *   (N)       rrms[s] = 1/sqrt(mean_c R2[s,c]^2 + eps);
 *             xn[s,c] = R2[s,c]*rrms[s]*(1 + Wnorm)
 *   (G1)      h = SiLU((xn . Wd^T) / HC)                  Wd: [r, K]
 *   (INJ)     inj_next = xn . Wi^T                          Wi: [HC, K]
 *   (G2)      G = sigmoid(h . Wu^T)                         Wu: [K, r]
 *   (MIX)     x[c] = (1/HC) * sum_s G[s,c]*xn[s,c]
 * and returns R2 (the next residual), rrms, inj_next and x (the next block's
 * input). xn, h and the gate never leave the chip except h, which crosses
 * between kernels through the caller's workspace.
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, dense rows
 *     unless a leading dimension (ld_*) is given.
 *   - All tensor pointers are device pointers on the handle's device,
 *     allocated and owned by the caller. The library never allocates device
 *     memory, never synchronises the host, and enqueues its kernels on the
 *     caller's stream in order, so a call can be captured into a HIP graph.
 *   - Every check runs on the host before the first launch; on any error
 *     nothing is launched and nothing is written. No C++ exception crosses
 *     this boundary.
 *   - hcgr_last_error() gives a human-readable reason for the last non-OK
 *     status returned on the calling thread.
 */
#ifndef HCGR_H
#define HCGR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hcgr_status {
    HCGR_OK = 0,
    HCGR_ERR_INVALID_ARGUMENT = 1,     /* null/misaligned pointer, bad size, bad stride, bad config */
    HCGR_ERR_UNSUPPORTED = 2,          /* device is not gfx950, or a shape the kernels cannot tile */
    HCGR_ERR_ALIASING = 3,             /* an output overlaps another output or an input            */
    HCGR_ERR_WORKSPACE_TOO_SMALL = 4,  /* workspace_bytes < hcgr_workspace_size(M)                 */
    HCGR_ERR_HIP = 5                   /* a HIP runtime call or a kernel launch failed             */
} hcgr_status;

typedef enum hcgr_weight_layout {
    /* Wd [r, K] and Wi [HC, K] passed separately; (1 + Wnorm) applied in-kernel. */
    HCGR_WEIGHTS_SEPARATE = 0,
    /* One merged matrix Wm [n_pad, K]: rows 0..r-1 are Wd, rows r..r+HC-1 are
     * Wi, rows r+HC..n_pad-1 are padding that is never read; the caller has
     * folded (1 + Wnorm) into its columns (Wm[j,k] = W[j,k]*(1 + Wnorm[k mod HS])
     * rounded to bf16). Described in the "Performance" section of the same
     * pull request (336 rows = 320 + 4 + 12 padding, "(1+w) folded in"). */
    HCGR_WEIGHTS_MERGED_FOLDED = 1
} hcgr_weight_layout;

typedef struct hcgr_config {
    int32_t hc;            /* residual streams HC. Supported: 1, 2, 4, 8 (4 is the tuned one). */
    int32_t hs;            /* stream width HS. Supported: multiple of 128, 128..65536.        */
    int32_t r;             /* low-rank width r. Supported: multiple of 32, 32..512.           */
    float eps;             /* RMSNorm epsilon (>= 0, finite), added to the mean square.       */
    int32_t wnorm_len;     /* hs (Wnorm shared by all streams, indexed by c) or hc*hs (by k). */
    int32_t weight_layout; /* hcgr_weight_layout                                              */
    int32_t n_pad;         /* rows of Wm for MERGED_FOLDED (>= r + hc); ignored otherwise.    */
} hcgr_config;

typedef struct hcgr_op* hcgr_handle;

/* Validates cfg and binds a handle to `device` (a HIP device ordinal).
 * Returns HCGR_ERR_UNSUPPORTED when the device is not gfx950 or the shape is
 * outside the supported set above, HCGR_ERR_INVALID_ARGUMENT for a malformed
 * config or a NULL `out`, HCGR_ERR_HIP when the device cannot be queried.
 * On success *out owns only host memory; free it with hcgr_destroy. */
hcgr_status hcgr_create(const hcgr_config* cfg, int device, hcgr_handle* out);

/* Frees a handle (NULL is allowed). Outstanding work on streams is unaffected. */
void hcgr_destroy(hcgr_handle h);

/* Poll budget of the one wait inside a launch: an up-role workgroup of the
 * persistent decode plan (HCGR_PLAN_PERSISTENT) polls its token tile's ready
 * flag, about 0.2 us apart, at most `polls` times before it gives up. A wait
 * that gives up sets the workspace's error counter (the 32-bit word at byte
 * HCGR_WORKSPACE_COUNTER_BYTES - 128) to 1 and goes on without h: that call's
 * x is invalid, and the caller zeroes the counter bytes again before the next
 * call on that workspace. 0 gives up at once (a check of that error path).
 * Affects later calls through h; other plans do not wait. Default
 * HCGR_DEFAULT_WAIT_POLLS (about 0.2 s). Pure host code. Errors:
 * HCGR_ERR_INVALID_ARGUMENT (NULL h, polls < 0 or > HCGR_MAX_WAIT_POLLS). */
#define HCGR_DEFAULT_WAIT_POLLS 1048576
#define HCGR_MAX_WAIT_POLLS 16777216
hcgr_status hcgr_set_wait_polls(hcgr_handle h, int32_t polls);

/* Bytes at the start of every workspace that hold arrival counters (1024
 * 32-bit counters, each at the start of a 128-byte line of its own). */
#define HCGR_WORKSPACE_COUNTER_BYTES 131072

/* Bytes of device workspace that serve hcgr_forward for every token count
 * from 1 to M (0 for M == 0), with the handle's tuned table if it has one
 * (hcgr_set_plan_table: install the table before sizing the workspace);
 * the value never decreases as M grows, so one
 * workspace sized for the largest M serves all smaller calls. The workspace
 * holds the partial sums of the down/inject contraction (per K chunk at
 * decode sizes, per stream or stream segment at mid sizes), their sums of
 * squares, the SiLU output h handed to the up kernel and, in its first
 * HCGR_WORKSPACE_COUNTER_BYTES, the arrival counters of the decode plan.
 * Zero-fill the workspace once after allocating it (hipMemset; at least the
 * counter bytes): every call leaves the counter bytes zero when it completes,
 * and reads nothing else of the workspace before writing it. After a call
 * that returned HCGR_ERR_HIP, or whose persistent-plan wait gave up (the
 * error counter reads 1; hcgr_set_wait_polls), zero the counter bytes again.
 * Calls that may
 * run concurrently (different streams) need separate workspaces. */
hcgr_status hcgr_workspace_size(hcgr_handle h, int64_t M, size_t* bytes);

/* The full op for M tokens, enqueued on `stream` (a hipStream_t; NULL = the
 * device's default stream), which must belong to the handle's device.
 *
 * Inputs (bf16 unless noted):
 *   R        [M, K]            incoming residual streams, k = s*HS + c
 *   y        [M, HS]           block output to inject
 *   inj      [M, ld_inj]       injection logits; columns 0..HC-1 are read,
 *                              ld_inj >= HC (a strided view such as a previous
 *                              call's inj_next is allowed)
 *   wnorm    [wnorm_len]       RMSNorm weight (the op uses 1 + wnorm)
 *   wd       [r, K]            down weight, or Wm [n_pad, K] when MERGED_FOLDED
 *   wi       [HC, K]           inject weight; must be NULL when MERGED_FOLDED
 *   wu       [K, r]            up weight (row k = s*HS + c)
 * Outputs:
 *   R2       [M, K]   bf16     next residual (round-to-nearest-even of the
 *                              fp32 value)
 *   rrms     [M, HC]  float    per-stream reciprocal RMS
 *   inj_next [M, ld_inj_next]  next layer's injection logits, bf16, columns
 *                              0..HC-1 written, others untouched
 *   x        [M, HS]  bf16     gated mean of the normalised streams
 * Pointer alignment: R, y, wnorm, wd, wi, wu, R2, x and workspace 16 bytes;
 * rrms 4; inj, inj_next 2. Any M >= 1 is accepted (tails are handled in the
 * kernels); M == 0 returns HCGR_OK and touches nothing (pointers may be NULL).
 * Errors: HCGR_ERR_INVALID_ARGUMENT (M < 0, NULL, misalignment, ld < HC,
 * stream of another device, wi given with MERGED_FOLDED), HCGR_ERR_ALIASING
 * (the byte range of any output overlaps another output, an input or the
 * workspace), HCGR_ERR_WORKSPACE_TOO_SMALL, HCGR_ERR_HIP (launch failure). */
hcgr_status hcgr_forward(hcgr_handle h,
                         const uint16_t* R, const uint16_t* y,
                         const uint16_t* inj, int64_t ld_inj,
                         const uint16_t* wnorm, const uint16_t* wd,
                         const uint16_t* wi, const uint16_t* wu,
                         int64_t M,
                         uint16_t* R2, float* rrms,
                         uint16_t* inj_next, int64_t ld_inj_next,
                         uint16_t* x,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/* hcgr_forward with per-kernel timing, for measurement: `events` points to 6
 * hipEvent_t handles owned by the caller (created with timing enabled).
 * events[2i] and events[2i+1] take the start and end times of stage i's
 * kernel itself (the launches go through hipExtLaunchKernelGGL, so the gaps
 * between kernels are not counted): stage 0 is the down/inject kernel, stage
 * 1 the reduction kernel when the plan has one (otherwise both events are
 * recorded right after stage 0, an empty interval), stage 2 the up/mix
 * kernel. Same arguments, checks and results as hcgr_forward otherwise; a
 * NULL events array or handle -> HCGR_ERR_INVALID_ARGUMENT. */
hcgr_status hcgr_forward_timed(hcgr_handle h,
                               const uint16_t* R, const uint16_t* y,
                               const uint16_t* inj, int64_t ld_inj,
                               const uint16_t* wnorm, const uint16_t* wd,
                               const uint16_t* wi, const uint16_t* wu,
                               int64_t M,
                               uint16_t* R2, float* rrms,
                               uint16_t* inj_next, int64_t ld_inj_next,
                               uint16_t* x,
                               void* workspace, size_t workspace_bytes,
                               void* stream, void* const* events);

/* hcgr_forward without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). The workspace is the library's own static scratch
 * array of hcgr_noalloc_scratch_bytes() bytes (32 MiB), one copy per GPU,
 * held until the process ends; hcgr_create looks its address up and zeroes its
 * counter bytes once per device. Arguments, checks and results as
 * hcgr_forward; a call whose plan needs more workspace than the scratch holds
 * (HC = 4, HS = 2560, r = 320: above 4096 tokens) returns
 * HCGR_ERR_WORKSPACE_TOO_SMALL and launches nothing. Every call on one GPU
 * shares the scratch, so calls that may overlap on one GPU (different
 * streams, or threads) race: serialise them. Allocates nothing and does not
 * synchronise. */
hcgr_status hcgr_forward_noalloc(hcgr_handle h,
                                 const uint16_t* R, const uint16_t* y,
                                 const uint16_t* inj, int64_t ld_inj,
                                 const uint16_t* wnorm, const uint16_t* wd,
                                 const uint16_t* wi, const uint16_t* wu,
                                 int64_t M,
                                 uint16_t* R2, float* rrms,
                                 uint16_t* inj_next, int64_t ld_inj_next,
                                 uint16_t* x, void* stream);

/* Bytes of the scratch hcgr_forward_noalloc uses on each GPU. */
size_t hcgr_noalloc_scratch_bytes(void);

/* The host-side checks of hcgr_forward for a configuration, without a handle,
 * a device or a launch: returns what hcgr_forward would return before
 * launching (device and stream checks excluded). Pure host code. */
hcgr_status hcgr_validate(const hcgr_config* cfg,
                          const uint16_t* R, const uint16_t* y,
                          const uint16_t* inj, int64_t ld_inj,
                          const uint16_t* wnorm, const uint16_t* wd,
                          const uint16_t* wi, const uint16_t* wu,
                          int64_t M,
                          const uint16_t* R2, const float* rrms,
                          const uint16_t* inj_next, int64_t ld_inj_next,
                          const uint16_t* x,
                          const void* workspace, size_t workspace_bytes);

/* (COMBINE) alone, for M tokens on `stream`:
 *   R2[m, s*HS + c] = R[m, s*HS + c] + y[m, c] * iw[m, s],
 *   iw[m, s] = 2*sigmoid(inj[m*ld_inj + s] / HC)
 * (the "Technical Details" step of the aiter pull request; the page's "PR
 * Self-Review" section lists this combine-only entry point beside the whole
 * op, for a layer whose block output is injected but whose mixed input is
 * not needed). R [M, K] and y [M, HS] as in hcgr_forward; inj is read at row
 * stride ld_inj >= HC (a previous call's strided inj_next view is allowed);
 * R2 [M, K] bf16, round-to-nearest-even of the fp32 value. No workspace.
 * Alignment: R, y, R2 16 bytes; inj 2. M == 0 returns HCGR_OK and touches
 * nothing. Errors: HCGR_ERR_INVALID_ARGUMENT (M < 0, NULL or misaligned
 * pointer, ld_inj < HC, stream of another device), HCGR_ERR_ALIASING (R2
 * overlaps R, y or inj), HCGR_ERR_HIP (launch failure); nothing is launched
 * on error. */
hcgr_status hcgr_combine(hcgr_handle h, const uint16_t* R, const uint16_t* y,
                         const uint16_t* inj, int64_t ld_inj, int64_t M,
                         uint16_t* R2, void* stream);

/* Every step of the op except COMBINE, for M tokens whose residual needs no
 * injection (the "mix" entry point that the same section lists, for the
 * first layer): the residual R [M, K] is taken as R2 unchanged, and
 *   rrms [M, HC], inj_next [M, ld_inj_next] and x [M, HS]
 * are computed exactly as hcgr_forward computes them from its R2 (N, G1,
 * INJ, G2, MIX). There is no y, inj or R2 argument. Weights, workspace
 * (hcgr_workspace_size serves both entry points), alignment, ownership and
 * errors as in hcgr_forward, with R an input only; an output that overlaps
 * R, another output, a weight or the workspace gives HCGR_ERR_ALIASING. */
hcgr_status hcgr_mix(hcgr_handle h, const uint16_t* R,
                     const uint16_t* wnorm, const uint16_t* wd,
                     const uint16_t* wi, const uint16_t* wu, int64_t M,
                     float* rrms, uint16_t* inj_next, int64_t ld_inj_next,
                     uint16_t* x, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Host-side checks of hcgr_combine and hcgr_mix for a configuration, without
 * a handle, a device or a launch (what the entry point would return before
 * launching, device and stream checks excluded). Pure host code. */
hcgr_status hcgr_validate_combine(const hcgr_config* cfg, const uint16_t* R,
                                  const uint16_t* y, const uint16_t* inj,
                                  int64_t ld_inj, int64_t M, const uint16_t* R2);
hcgr_status hcgr_validate_mix(const hcgr_config* cfg, const uint16_t* R,
                              const uint16_t* wnorm, const uint16_t* wd,
                              const uint16_t* wi, const uint16_t* wu, int64_t M,
                              const float* rrms, const uint16_t* inj_next,
                              int64_t ld_inj_next, const uint16_t* x,
                              const void* workspace, size_t workspace_bytes);

/* Workspace bytes for a configuration without a handle (pure host code). */
hcgr_status hcgr_workspace_size_for(const hcgr_config* cfg, int64_t M, size_t* bytes);

/* Writes a one-line description of the kernel plan used for M tokens (tile
 * sizes, split counts, grids) into buf (always NUL-terminated when len > 0). */
hcgr_status hcgr_describe_plan(const hcgr_config* cfg, int64_t M, char* buf, size_t len);

/* ------------------------------------------------------------------------
 * Tuned plans (the "PR Self-Review" section of the same pull request
 * describes its op's tuned table: token counts resolve to the nearest key in
 * log space; below the smallest key, and for entries marked heuristic, the
 * heuristic plan applies; an entry that cannot tile the actual shape falls
 * back to the heuristic). A plan choice names a plan family and its
 * parameters; the library checks every choice before use.
 * ------------------------------------------------------------------------ */
#define HCGR_PLAN_HEURISTIC (-1) /* the library's own choice                          */
#define HCGR_PLAN_SPLIT 0        /* decode plan: K-chunked down kernel, reduction, up */
#define HCGR_PLAN_TILE 3         /* tile plan: 64-token down tiles, (stream sum), up  */
#define HCGR_PLAN_FUSED 4        /* fused decode plan: down kernel with the chunk
                                    reduction done by its last arrivals, then up     */
#define HCGR_PLAN_PERSISTENT 5   /* persistent decode plan: one kernel, the up role
                                    waits (bounded) for the down role's h; a wait
                                    that gives up sets the last counter (the 32-bit
                                    word at byte HCGR_WORKSPACE_COUNTER_BYTES - 128
                                    of the workspace) to 1 and that call's x is
                                    invalid                                          */
#define HCGR_SPLIT_VARIANTS 13   /* down-kernel variants of the decode plan           */

typedef struct hcgr_plan_choice {
    int64_t tokens;         /* table key (token count >= 1); a candidate carries the M it was made for */
    int32_t kind;           /* HCGR_PLAN_HEURISTIC, HCGR_PLAN_SPLIT, HCGR_PLAN_TILE, HCGR_PLAN_FUSED
                               or HCGR_PLAN_PERSISTENT                                              */
    int32_t down_variant;   /* SPLIT: 0 .. HCGR_SPLIT_VARIANTS-1 (token tile, row blocks, k waves,
                               chunk width; hcgr_plan_lookup describes each); serves M <= 256 only,
                               HC = 4 only.
                               TILE: 0 = 64-token down tiles, 1 = 128-token down tiles (needs
                               streams_per_wg = 1).
                               FUSED, PERSISTENT: 0 = 16-token, 1 = 32-token tiles; serve
                               M <= 256 only                                                        */
    int32_t streams_per_wg; /* TILE: 1, or 4 with HC = 4                                            */
    int32_t segments;       /* TILE with 1 stream per workgroup: column segments per stream,
                               a divisor of HS/128 (1 with 4 streams per workgroup)                  */
    int32_t up_variant;     /* TILE: 0 staged (HC = 4), 1 sweep (HC = 4, 96 <= r <= 320),
                               2 stream-generic (HC != 4), 3 stream-generic over 128-token tiles
                               (HC = 2 or 8), 4 sweep over 256-token tiles (HC = 4,
                               96 <= r <= 320)                                                       */
    int32_t ranges;         /* TILE with a sweep: channel ranges per token tile, 1 .. HS/32;
                               1 otherwise                                                           */
} hcgr_plan_choice;

/* Every plan choice that can run cfg's shape at M tokens (the candidates a
 * tuner times). Writes min(*count, capacity) choices (tokens = M) to out and
 * the total number to *count; out may be NULL when capacity is 0. Pure host
 * code. Errors: HCGR_ERR_INVALID_ARGUMENT (M < 1, NULL count, negative
 * capacity), config errors as hcgr_create. */
hcgr_status hcgr_plan_candidates(const hcgr_config* cfg, int64_t M, hcgr_plan_choice* out,
                                 int32_t capacity, int32_t* count);

/* The plan a table gives M tokens: writes the choice it resolves to (kind
 * HCGR_PLAN_HEURISTIC when the heuristic applies; tokens = the entry's key or
 * 0) to *chosen (may be NULL) and a one-line description of the resulting
 * plan, as hcgr_describe_plan, to buf. n = 0 (table may be NULL) describes
 * the heuristic. Pure host code. Errors: as hcgr_set_plan_table for a
 * malformed table; HCGR_ERR_INVALID_ARGUMENT for M < 0. */
hcgr_status hcgr_plan_lookup(const hcgr_config* cfg, const hcgr_plan_choice* table, int32_t n,
                             int64_t M, hcgr_plan_choice* chosen, char* buf, size_t len);

/* Workspace bytes that serve every token count from 1 to M with a table (the
 * table-aware form of hcgr_workspace_size_for). Pure host code. */
hcgr_status hcgr_workspace_size_table(const hcgr_config* cfg, const hcgr_plan_choice* table, int32_t n,
                                      int64_t M, size_t* bytes);

/* Installs a copy of a tuned table in the handle (n = 0 clears it; the
 * caller keeps ownership of `table`). Keys must be >= 1 and strictly
 * increasing; every non-heuristic entry must be able to run the handle's
 * shape at its own key; otherwise HCGR_ERR_INVALID_ARGUMENT and the handle's
 * table is unchanged. Afterwards hcgr_forward, hcgr_forward_timed, hcgr_mix
 * and hcgr_workspace_size use the table. Calls that may run concurrently on
 * one handle must not overlap with this one. */
hcgr_status hcgr_set_plan_table(hcgr_handle h, const hcgr_plan_choice* table, int32_t n);

/* Static name of a status code. */
const char* hcgr_status_string(hcgr_status s);

/* Reason for the last non-OK status returned on this thread ("" if none). */
const char* hcgr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HCGR_H */
