/*
 * uly.h — C ABI of the MI355X (gfx950) Ulysses sequence-parallel exchange.
 *
 * The P ranks of one Ulysses group are P slabs ("rank slabs") of one GPU's
 * HBM, stored rank-major in a single allocation, so the all-to-all of the
 * pages becomes a device-local permutation executed by hand-written HIP
 * kernels.  This header is the whole boundary: plain pointers, sizes and
 * HIP streams, no framework types.
 *
 * Pages cited (by title and section):
 *  [CA] TeleFuser documentation, "Communication Architecture".
 *  [P27] TeleFuser PR #27, "[PERF] Add CUDA IPC Ulysses overlap and
 *        lossless LingBot streaming", sections "Description" and
 *        "Changes Made".
 *  [QN] flashinfer PR #6332 (QkvNormRopeExchangeOverlap), sections
 *        "Description", "Assumptions", "Tests".
 *  [UC] flashinfer UlyssesCommunicator(backend="pcie") PR, sections
 *        "What" (Transforms, Lifecycle, Failure envelope, element type).
 *
 * ------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ------------------------------------------------------------------------
 * Layouts.  P = the context's world size.  A sequence-sharded operand is
 *   per rank [B, S_l, H, D]; a head-sharded one is per rank [B, S, Hl, D]
 *   with S = P*S_l and Hl = H/P.  Rank q's head band is the contiguous
 *   range of heads [q*Hl, (q+1)*Hl) ([QN "Description"]), and local token
 *   s of rank r is global token r*S_l + s ([CA "Ulysses"]).
 *
 * Targets.  Every destination written by the exchange is a "target": P
 *   contiguous rank slabs, rank-major, element order [P][B][S][Hl][D]
 *   (scatter) or [P][B][S_l][H][D] (gather).  Targets are normally taken
 *   from the context's tagged target cache ([P27 "Changes Made"]: up to 12
 *   targets keyed by tag, shape, dtype, mode and device), which the caller
 *   fills once with uly_target_register; the exchange then writes the
 *   final layout straight into them.  An explicit destination pointer
 *   (the `outs` arguments) bypasses the cache for one call.
 *
 * Ownership.  The library never allocates or frees device memory.  Inputs
 *   are borrowed and stream-ordered: they must stay valid until the work
 *   enqueued on the caller's stream has completed.  Registered target
 *   storage stays owned by the caller and must outlive the context (or the
 *   last call that writes it).  A target's contents stay valid until the
 *   next call that writes the same target ([QN "Description": outputs stay
 *   valid until the slot is reused]).
 *
 * Alignment.  Every device pointer and every byte stride of a copied or
 *   normalised row must be a multiple of 16 bytes (rows move as 16-byte
 *   vectors); in particular D * element_size % 16 == 0 (element size 2 for
 *   ULY_F16 / ULY_BF16, 1 for ULY_U8).
 *
 * Errors.  Every argument check of a call (and of every member of a
 *   grouped call) runs before anything is enqueued, so a rejected call
 *   changes nothing and leaves the context usable ([UC "Failure
 *   envelope"]; [P27 "Description": failures are surfaced rather than a
 *   group being half-submitted]).  A HIP runtime or launch failure returns
 *   ULY_E_HIP and poisons the context: every later call returns
 *   ULY_E_BROKEN and only uly_destroy is allowed (fail-stop).
 *   uly_last_error() returns a thread-local message for the last failure.
 *   Extents, strides, table lengths and the sizes formed from them are
 *   bounded by 2^48 (elements or bytes) and checked without wrapping;
 *   larger ones are refused (ULY_E_UNSUPPORTED, or ULY_E_INVAL for the row
 *   maps and host tables), as are launches past the 32-bit index limits
 *   that each entry point states.
 *
 * Streams.  The context owns one extra HIP stream ("comm stream", default
 *   priority) on which the plain Q/K/V scatter runs, so that it overlaps
 *   the fused Q/K norm + RoPE scatter enqueued on the caller's stream
 *   ([P27 "Changes Made": strided V submitted before Q/K norm and RoPE);
 *   uly_set_route can move it onto the caller's stream instead.
 *   Before writing a target the comm stream waits for everything already
 *   enqueued on the caller's stream, so a consumer that read the previous
 *   contents on that stream is ordered before the overwrite.
 *
 * Threads.  A context is not thread-safe; use one per thread or lock.
 */
#ifndef ULY_H
#define ULY_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct uly_ctx uly_ctx;

typedef enum {
    ULY_OK = 0,
    ULY_E_INVAL = -1,        /* bad argument (null, shape, stride, alignment, divisibility) */
    ULY_E_DTYPE = -2,        /* dtype differs between members or from the cached target */
    ULY_E_CACHE_FULL = -3,   /* registering one more target would exceed max_targets */
    ULY_E_NOT_FOUND = -4,    /* no target registered under this key */
    ULY_E_UNSUPPORTED = -5,  /* valid request this build or context cannot run */
    ULY_E_HIP = -6,          /* HIP runtime/launch failure; the context is now broken */
    ULY_E_BROKEN = -7,       /* the context failed earlier; only uly_destroy is allowed */
    ULY_E_OVERLAP = -8       /* an input's memory range overlaps its destination's */
} uly_status;

/* Element types.  The relayouts move opaque bytes, so ULY_U8 carries any
 * 1-byte payload (fp8, int8) in the same byte budget; the dtype matters to
 * the fused norm + RoPE (16-bit floats only) and to the target cache key
 * ([UC "element type"]). */
typedef enum { ULY_F16 = 1, ULY_BF16 = 2, ULY_U8 = 3 } uly_dtype;

/* Direction of a target, part of its cache key. */
typedef enum {
    ULY_MODE_SCATTER = 0,    /* sequence-sharded -> head-sharded (Q, K, V) */
    ULY_MODE_GATHER = 1      /* head-sharded -> sequence-sharded (attention output) */
} uly_mode;

/* A rank-major operand: P slabs of a 4-D tensor with element strides.
 * Element [rank][b][s][h][d] lives at
 *     data + elem_size * (rank*rank_stride + b*stride[0] + s*stride[1]
 *                         + h*stride[2] + d*stride[3]),
 * stride[3] must be 1.  A fused QKV projection [B, S_l, 3, H, D] per rank
 * is described per component c by data offset c*H*D and stride[1] = 3*H*D. */
typedef struct {
    void *data;
    int32_t dtype;           /* uly_dtype */
    int32_t reserved;        /* must be 0 */
    int64_t rank_stride;     /* elements between consecutive rank slabs */
    int64_t shape[4];        /* per rank: B, S, H, D */
    int64_t stride[4];       /* element strides of b, s, h, d */
} uly_tensor;

/* ---- context ---------------------------------------------------------- */

/* Create a context for `world_size` emulated ranks (1..4096) on HIP device
 * `device` with room for `max_targets` cached targets (1..12, [P27 "Changes
 * Made"]).
 * device = -1 creates a host-only context: argument checks and the target
 * cache work, every call that would enqueue GPU work returns
 * ULY_E_UNSUPPORTED after its checks pass. */
uly_status uly_create(uly_ctx **out, int device, int world_size, int max_targets);

/* Wait for the context's streams, then release its streams, events and
 * cache entries (not the registered storage).  NULL is accepted. */
uly_status uly_destroy(uly_ctx *ctx);

/* ---- tagged target cache ---------------------------------------------- */

/* Register caller-owned device storage as the target for key
 * (tag, mode, dtype, per-rank shape, the context's device).  Per-rank shape
 * is [B, S, Hl, D] for ULY_MODE_SCATTER and [B, S_l, H, D] for
 * ULY_MODE_GATHER; the storage must hold P such slabs contiguously
 * (bytes >= P * B*S*Hl*D * element size) and be 16-byte aligned.  Fails with
 * ULY_E_CACHE_FULL when max_targets keys exist (there is no eviction: an
 * evicted target could still be referenced by a caller) and ULY_E_INVAL
 * when the key is already registered.  tag: NUL-terminated, <= 63 bytes. */
uly_status uly_target_register(uly_ctx *ctx, const char *tag, int mode, int dtype,
                               const int64_t shape[4], void *storage, size_t bytes);

/* Look up a registered target; *storage receives its pointer or NULL. */
uly_status uly_target_lookup(uly_ctx *ctx, const char *tag, int mode, int dtype,
                             const int64_t shape[4], void **storage);

/* Number of registered targets. */
uly_status uly_target_count(uly_ctx *ctx, int *count);

/* ---- the exchange ------------------------------------------------------ */

/* Ulysses scatter of up to three sequence-sharded operands ([CA "Ulysses"]:
 * scatter heads / gather sequence):
 *     Y[q][b][r*S_l + s][j][:] = X[r][b][s][q*Hl + j][:]
 * q, k, v: operands (any may be NULL, at least one non-NULL), per rank
 *     [B, S_l, H, D]; members may differ in H (grouped-query attention) but
 *     share B, S_l, D and dtype; H % P == 0 for each.
 * tags[i]: cache tag of member i's target (mode ULY_MODE_SCATTER, shape
 *     [B, P*S_l, H/P, D]); may be NULL when outs[i] is given.
 * outs: NULL, or per member an explicit destination (NULL entry = cached).
 * caller: stream whose prior work the copy waits for.  The copy itself runs
 *     on the context's comm stream, as one launch for all members; pair with
 *     uly_wait before consuming the targets. */
uly_status ulysses_scatter_qkv(uly_ctx *ctx, const uly_tensor *q, const uly_tensor *k,
                               const uly_tensor *v, const char *const tags[3],
                               void *const outs[3], hipStream_t caller);

/* Q/K RMSNorm + interleaved RoPE fused into the Ulysses scatter ([QN
 * "Assumptions"]): for every row x = X[r][b][s][h][:] of D values,
 *     n_i = x_i * rsqrt(mean(x^2) + eps) * w_i               (fp32)
 *     (y_2j, y_2j+1) = (n_2j c - n_2j+1 s, n_2j s + n_2j+1 c),
 *     c = cos_tab[g][j], s = sin_tab[g][j], g = r*S_l + s   (fp32)
 * rounded once to the operand dtype (round to nearest even) and stored at
 * Y[h / Hl][b][g][h % Hl][:] — no intermediate tensor.
 * q, k: operands normalised and rotated (either may be NULL); v: optional
 *     operand scattered unchanged by the same call, as the fused producer
 *     of [QN "Description"] stores every destination's q, k and v band: in
 *     the same launch when the operands are interleaved (views of one fused
 *     tensor), by the relayout kernel right after on `caller` when they are
 *     separate dense tensors (D = 128, S_l even), where that copies faster.
 *     All members share B, S_l, D and dtype; H % P == 0 for each.
 * w_q, w_k: [D] weights in the operand dtype (required for each non-NULL
 *     q / k).  eps: > 0 (1e-6 in [QN]).
 * cos_tab, sin_tab: device fp32 [table_rows][D/2], row g = global position;
 *     table_rows >= P*S_l.  D must be even and D*2 a multiple of 16 with
 *     D*2/16 in {4, 8, 16, 32} lanes per row (D = 32, 64, 128, 256).
 * tags / outs: as in ulysses_scatter_qkv (members 0 = q, 1 = k, 2 = v).
 * caller: the kernels run on this stream (the compute stream). */
uly_status fused_qk_norm_rope_scatter(uly_ctx *ctx, const uly_tensor *q, const uly_tensor *k,
                                      const uly_tensor *v, const void *w_q, const void *w_k,
                                      float eps, const float *cos_tab, const float *sin_tab,
                                      int64_t table_rows, const char *const tags[3],
                                      void *const outs[3], hipStream_t caller);

/* The same fused scatter into the packed receive layout ([QN "Description", Layouts:
 * the "fused" payload): one target [P][B][S][Hl][3D] whose head rows hold
 * q, k and v side by side,
 *     Y[q'][b][g][j][c*D + d] = (normalised and rotated q, k, or v)[...][d]
 * for c = 0 (q), 1 (k), 2 (v).  q, k and v are all required and share H.
 * tag: cache key of the packed target (shape [B, P*S_l, H/P, 3*D]), or NULL
 * with an explicit `out`. */
uly_status fused_qkv_norm_rope_scatter_packed(uly_ctx *ctx, const uly_tensor *q, const uly_tensor *k,
                                              const uly_tensor *v, const void *w_q, const void *w_k,
                                              float eps, const float *cos_tab, const float *sin_tab,
                                              int64_t table_rows, const char *tag, void *out,
                                              hipStream_t caller);

/* The QKV projection ahead of the fused norm + RoPE scatter, in one launch
 * ([QN "Description": the projection, the per-head RMSNorm of Q and K, the
 * interleaved RoPE and the head exchange fused into one call per layer;
 * "Assumptions": every rank holds a token shard and the full QKV weight,
 * order projection -> QK-norm -> RoPE, fp32 math, 16-bit output]):
 *     qkv[m][n] = sum_k x[m][k] * w_qkv[n][k]          (fp32 accumulation)
 * then, per (token, head) row of q and k, the RMSNorm and rotation of
 * fused_qk_norm_rope_scatter at global position r*S_l + s, one rounding,
 * and the store into the head-sharded targets; v is rounded and stored.
 *
 * x:      [P][B][S_l][hidden] token rows, contiguous, rank-major.
 * w_qkv:  [(Hq + 2*Hkv) * D][hidden], contiguous, output-major: rows
 *         [0, Hq*D) project q (head h at rows h*D ...), then k's Hkv*D rows,
 *         then v's.  No bias.
 * dtype:  ULY_BF16 or ULY_F16 for x, w_qkv, w_q, w_k and the targets.
 * D:      128 (the kernel's tile is one 128-wide head).
 * hidden: a positive multiple of 64.  Hq, Hkv >= 1 and divisible by P.
 * tags/outs: as for fused_qk_norm_rope_scatter; all three of q, k, v are
 *         produced, into [B, P*S_l, Hq/P, D], [B, P*S_l, Hkv/P, D] twice.
 * Runs on `caller`; the grouped handshake (uly_wait) covers it. */
uly_status fused_qkv_proj_norm_rope_scatter(uly_ctx *ctx, const void *x, int dtype, int64_t B, int64_t S_l,
                                           int64_t hidden, const void *w_qkv, int64_t Hq, int64_t Hkv, int64_t D,
                                           const void *w_q, const void *w_k, float eps, const float *cos_tab,
                                           const float *sin_tab, int64_t table_rows, const char *const tags[3],
                                           void *const outs[3], hipStream_t caller);

/* Grouped completion handshake ([P27 "Changes Made": one grouped handshake
 * for the tagged Q/K/V transfers]): make `consumer` wait, without any
 * host or device-wide synchronisation, for every scatter submitted since
 * the previous uly_wait, whichever stream it ran on. */
uly_status uly_wait(uly_ctx *ctx, hipStream_t consumer);

/* Inverse exchange for the attention output ([CA "Ulysses"]: gather heads /
 * scatter sequence):
 *     Z[r][b][s][q*Hl + j][:] = O[q][b][r*S_l + s][j][:]
 * o: head-sharded operand, per rank [B, S, Hl, D]; S % P == 0.
 * tag: target key (mode ULY_MODE_GATHER, shape [B, S/P, P*Hl, D]) or NULL
 *     with an explicit `out`.  Runs on `caller`. */
uly_status ulysses_gather_out(uly_ctx *ctx, const uly_tensor *o, const char *tag, void *out,
                              hipStream_t caller);

/* Destination-major chunk exchange ([UC "Transforms": exchange_chunks]):
 * each rank's payload is already packed destination-major as x[r][q][:]
 * (chunk_bytes bytes per destination); the exchange delivers
 *     y[q][r][:] = x[r][q][:]
 * and interleaves nothing.  x and y hold P*P*chunk_bytes bytes each, are
 * 16-byte aligned and do not overlap; chunk_bytes % 16 == 0.  Opaque bytes,
 * any element type.  Runs on `stream`. */
uly_status uly_exchange_chunks(uly_ctx *ctx, const void *x, void *y, int64_t chunk_bytes, hipStream_t stream);

/* ---- sequence padding (parallel_shard.py's role in [CA]'s ownership table) */

/* Pad a global sequence full[B][S][row] (row = row_elems 16-bit values,
 * contiguous) with zero rows to P*S_l and slice it rank-major:
 *     x[r][b][s][:] = full[b][r*S_l + s][:] if r*S_l + s < S, else 0. */
uly_status uly_seq_pad_shard(uly_ctx *ctx, const void *full, int dtype, int64_t B, int64_t S,
                             int64_t row_elems, int64_t S_l, void *x, hipStream_t stream);

/* Concatenate rank slabs x[P][B][S_l][row] along the sequence and keep
 * [0, S):  full[b][g][:] = x[g / S_l][b][g % S_l][:]. */
uly_status uly_seq_unshard_trim(uly_ctx *ctx, const void *x, int dtype, int64_t B, int64_t S,
                                int64_t row_elems, int64_t S_l, void *full, hipStream_t stream);

/* ---- height-sharded spatial tensors ([CA "Spatial VAE Communication",
 *      "Equal-shape gather"]) ------------------------------------------ */
/* A latent [N][Hh][W] (N = B*C*T, W*2 a multiple of 16) is split by height
 * into P shards: the first Hh % P ranks take floor(Hh/P)+1 rows, the rest
 * floor(Hh/P); hmax = ceil(Hh/P).  */

/* shards[P][N][hmax + 2*halo][W]: rank r's rows o_r-halo .. o_r+h_r+halo-1,
 * zero outside the image (missing neighbour) and past h_r + 2*halo. */
uly_status uly_spatial_split_halo(uly_ctx *ctx, const void *full, int dtype, int64_t N,
                                  int64_t Hh, int64_t W, int64_t halo, void *shards,
                                  hipStream_t stream);

/* stacked[P][N][hmax][W]: each rank's core rows (halos dropped), zero-padded
 * to hmax — one rank-major allocation. */
uly_status uly_spatial_gather_stacked(uly_ctx *ctx, const void *shards, int dtype, int64_t N,
                                      int64_t Hh, int64_t W, int64_t halo, void *stacked,
                                      hipStream_t stream);

/* full[N][Hh][W]: trim each rank to its height and concatenate in rank order. */
uly_status uly_spatial_trim_concat(uly_ctx *ctx, const void *stacked, int dtype, int64_t N,
                                   int64_t Hh, int64_t W, void *full, hipStream_t stream);

/* ---- rotary tables (host, built once per session) ---------------------- */

/* 1-D table: angle[g][j] = g * theta^(-2j/D) for g < real_rows, identity
 * rotation (cos 1, sin 0) for padding rows; evaluated in double, stored
 * fp32 in host buffers [rows][D/2]. */
uly_status uly_rope_table_1d(float *cos_out, float *sin_out, int64_t rows, int64_t real_rows,
                             int64_t D, double theta);

/* 3-D table for a row-major (T, grid_h, grid_w) latent grid: pairs
 * [0, n_t) rotate by t, [n_t, n_t+n_h) by h, [n_t+n_h, n_t+n_h+n_w) by w,
 * each band with frequencies theta^(-2k/(2*n_band)); other pairs and
 * padding rows are the identity. */
uly_status uly_rope_table_3d(float *cos_out, float *sin_out, int64_t rows, int64_t real_rows,
                             int64_t D, int64_t grid_h, int64_t grid_w, int64_t n_t,
                             int64_t n_h, int64_t n_w, double theta);

/* ---- measurement -------------------------------------------------------- */

typedef enum {
    ULY_K_SCATTER = 0,       /* plain Q/K/V relayout (comm stream) */
    ULY_K_NORM_ROPE = 1,     /* fused Q/K norm + RoPE scatter (caller stream) */
    ULY_K_GATHER = 2,        /* output relayout */
    ULY_K_PAD = 3,           /* sequence pad / trim */
    ULY_K_SPATIAL = 4,       /* spatial split / gather / concat */
    ULY_K_PROJ = 5,          /* QKV projection with the norm + RoPE + scatter epilogue */
    ULY_K_COUNT = 6
} uly_kernel_kind;

/* kind_mask bit k (1 << uly_kernel_kind) brackets launches of kind k with
 * HIP events on the stream they run on: the first launch of each kind and
 * then one in every `every` (>= 1).  Each pair of events adds a little
 * latency between kernels, so time only what is needed; 0 turns timing
 * off.  uly_profile_read waits for those events and returns the summed
 * kernel time (ms) and the number of timed launches of `kind` since the
 * last reset. */
uly_status uly_profile_enable(uly_ctx *ctx, int kind_mask, int every);
uly_status uly_profile_read(uly_ctx *ctx, int kind, double *total_ms, int64_t *launches);
uly_status uly_profile_reset(uly_ctx *ctx);

/* Counters: registrations, cache hits, launches enqueued. */
typedef struct {
    int64_t registrations;
    int64_t lookups;
    int64_t hits;
    int64_t launches;
} uly_stats;
uly_status uly_get_stats(uly_ctx *ctx, uly_stats *out);

/* The context's comm stream (for callers that want to order against it). */
uly_status uly_comm_stream(uly_ctx *ctx, hipStream_t *out);

/* How ulysses_scatter_qkv moves its operands.  ULY_ROUTE_KERNEL (default):
 * one relayout kernel on the compute units, on the context's comm stream.
 * ULY_ROUTE_COPY_ENGINE: one 2-D copy per (source rank, destination rank,
 * batch) block on the copy engines, straight into the final layout, leaving
 * the compute units to the fused Q/K kernel ([P27 "Description": copy-engine
 * transfers overlapping Q/K preprocessing]).  ULY_ROUTE_CALLER: the same
 * relayout kernel on the caller's stream itself, with no second stream and
 * no fork or join events, for callers that do not overlap the scatter with
 * other work (the copy is then ordered like any kernel on `caller`, and
 * uly_wait has nothing to do for it on that stream).  Head bands of more
 * than one head must be packed (stride[2] == D), as for the kernel route. */
typedef enum { ULY_ROUTE_KERNEL = 0, ULY_ROUTE_COPY_ENGINE = 1, ULY_ROUTE_CALLER = 2 } uly_route;
uly_status uly_set_route(uly_ctx *ctx, int route);

/* Fault injection for tests of the fail-stop rule: the `after`-th next
 * launch (0 = the next one) is not enqueued and reports a HIP failure. */
uly_status uly_debug_fail_launch(uly_ctx *ctx, int after);

/* Test hook: the depth of fused_qkv_proj_norm_rope_scatter's LDS ring for
 * the token rows.  0 (the default) picks three stages when the token
 * operand exceeds the 256 MB Infinity Cache and two otherwise; 2 or 3
 * force that depth, so that both kernels can be checked at any size.
 * Other values: ULY_E_INVAL. */
uly_status uly_debug_proj_ring(uly_ctx *ctx, int depth);

const char *uly_last_error(void);
const char *uly_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* ULY_H */
