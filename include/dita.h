/*
 * dita.h — C ABI of the partitioned video-DiT attention step with selective
 * attention-state reuse, native on MI355X (gfx950).
 *
 * What the library computes (DiTango, gist.science 2607.15650):
 *   - the token sequence is split into P contiguous context partitions ("Problematica":
 *     context parallelism splits the sequence);
 *   - for query partition i and key partition j the attention state is the pair
 *       lse_ij[r] = log sum_{c in j} exp(tau q_r . k_c)
 *       O_ij[r]   = sum_{c in j} exp(tau q_r . k_c - lse_ij[r]) v_c
 *     ("State-Centric Parallel Runtime / Composizione dello Stato": the cached unit is the
 *     composed state of output and log-sum-exp, not raw K/V);
 *   - every block is FRESH (recomputed from this step's Q/K/V and written to its cache
 *     slot), REUSE (the state its slot holds, written at the step where it was last fresh:
 *     "Anchor-Guided Selection Planner") or SKIP (outside the active set, e.g.
 *     Efficient-vDiT's tile-style sparse 3D mask, chatpaper abstract);
 *   - the states of a row are merged by log-sum-exp, which is associative and commutative:
 *       L[r] = log sum_j exp(lse_ij[r]);   out[r] = sum_j exp(lse_ij[r] - L[r]) O_ij[r].
 * tau defaults to 1/sqrt(D) (the pages do not state the scale).
 *
 * Conventions
 *   - Every call returns dita_status; DITA_OK is 0.  Nothing throws or aborts.  On any
 *     failure no state changes and dita_last_error() returns a thread-local message.
 *   - Pointers marked "device" are HIP device addresses on the calling thread's current
 *     device; "host" pointers are ordinary memory.  The library never allocates device
 *     memory: the caller provides one buffer of dita_cache_required_bytes bytes, which
 *     holds the state cache, the per-step work lists, a transposed-V scratch, the partial
 *     merges of split row groups (below) and the device counters.  The caller owns all device memory and the stream and keeps them
 *     alive until the stream has passed the step.  A handle allocates pinned host memory
 *     of its own (plan uploads, the planner's read-back, merge jobs), released by
 *     dita_cache_free.
 *   - Q, K, V and out are contiguous [B, H, N, D] (row-major, D fastest), or [B, N, H, D]
 *     with the geometry's layout BNHD.
 *   - A handle is not thread-safe; different handles are independent.
 */
#ifndef DITA_H
#define DITA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dita_status {
  DITA_OK = 0,
  DITA_ERR_INVALID_ARGUMENT = 1, /* null pointer, value out of range                          */
  DITA_ERR_SHAPE = 2,            /* inconsistent geometry or partition offsets                 */
  DITA_ERR_UNSUPPORTED = 3,      /* head_dim / dtype combination without a kernel              */
  DITA_ERR_POLICY = 4,           /* mask value not in {0,1,2}; diagonal not FRESH; a FRESH or
                                    REUSE block outside the cache's active set                 */
  DITA_ERR_CACHE_MISS = 5,       /* REUSE of a slot not written since alloc / reset            */
  DITA_ERR_BUFFER_TOO_SMALL = 6, /* device buffer smaller than dita_cache_required_bytes       */
  DITA_ERR_NO_POLICY = 7,        /* dita_attn_step without a policy set for this step          */
  DITA_ERR_DEVICE = 8,           /* a HIP call failed (message in dita_last_error)             */
  DITA_ERR_OFFLOADED = 9         /* the cache's state is offloaded to host memory
                                    (dita_cache_offload); restore it first                    */
} dita_status;

/* DITA_FP8_E4M3: cache O only (with bf16 Q/K/V): OCP e4m3fn (1 sign, 4 exponent bits of bias
 * 7, 3 mantissa bits; largest 448, no infinity), rounded to nearest even and saturated at
 * +-448 -- a compressed state cache (DiTango, "Significato e Claim": cache compression named
 * as a way to ease the state cache's memory cost). */
typedef enum dita_dtype { DITA_F32 = 0, DITA_BF16 = 1, DITA_FP8_E4M3 = 2 } dita_dtype;

enum { DITA_SKIP = 0, DITA_FRESH = 1, DITA_REUSE = 2 };

/* Memory layout of Q, K, V and out (lse_out is always [B, H, N]):
 *   BHND  [B, H, N, D], D fastest (a head's tokens contiguous);
 *   BNHD  [B, N, H, D], D fastest (a token's heads contiguous: the layout of a fused QKV
 *         projection's output, usable without a transpose). */
typedef enum dita_layout { DITA_LAYOUT_BHND = 0, DITA_LAYOUT_BNHD = 1 } dita_layout;

typedef enum dita_policy_kind {
  DITA_POLICY_EXPLICIT = 0,           /* mask given by the caller                            */
  DITA_POLICY_FRAME_THRESHOLD = 1,    /* FRESH iff |f_i - f_j| <= max_fresh_frame_dist       */
  DITA_POLICY_FRESH_BUDGET = 2,       /* per row R = min(floor((pct*A_i + 50)/100), A_i - 1) */
  DITA_POLICY_CENTROID_THRESHOLD = 3, /* FRESH iff |C_i - C_j| <= max_fresh_centroid2        */
  DITA_POLICY_PLANNER = 4             /* reuse chosen by predicted error (below)              */
} dita_policy_kind;

/* Token geometry.  Tokens are (t, y, x) flattened frame-major, row-major inside a frame:
 * tokens == frames * grid_h * grid_w.  Partition p holds tokens [o_p, o_{p+1}).  Its
 * doubled centroid is C_p = o_p + o_{p+1} - 1 and its frame is f_p = C_p / (2*grid_h*grid_w)
 * (integer division): the frame of its centre token. */
typedef struct dita_geometry {
  int32_t batch, heads, tokens, head_dim;   /* B, H, N, D.  bf16: D in {64, 72, 128} (72 is
                                               padded to 96 inside); f32: D <= 64          */
  int32_t frames, grid_h, grid_w;
  int32_t num_partitions;                   /* P, 1 <= P <= 1024, P <= N                    */
  const int32_t* partition_offsets;         /* host, P+1 increasing ints from 0 to N, or
                                               NULL for the array_split rule (the first
                                               N mod P partitions get one more token).
                                               Copied; not kept.                           */
  dita_dtype qkv_dtype;                     /* element type of Q, K, V                      */
  dita_dtype cache_o_dtype;                 /* qkv_dtype, or FP8_E4M3 with bf16 Q/K/V;
                                               cache lse is f32                             */
  float softmax_scale;                      /* tau; <= 0 selects 1/sqrt(D)                  */
  int32_t layout;                           /* dita_layout of Q, K, V, out; zero-initialise
                                               the struct for BHND                          */
  dita_dtype out_dtype;                     /* element type of out: F32 (0, the default of a
                                               zero-initialised struct) or, with bf16
                                               Q/K/V, BF16: the f32 result rounded to
                                               nearest even, for a consumer that takes bf16
                                               (half the bytes written)                     */
} dita_geometry;

/* One step's block policy (DiTango, "Anchor-Guided Selection Planner"): which blocks are
 * recomputed and which reuse a cached state.  Candidates for the budget rule are ranked by
 * (|f_i - f_j|, |C_i - C_j|, j).  Whatever the kind, the diagonal block is FRESH (the local
 * partition is always computed) and only blocks of the active set are non-SKIP.
 *
 * PLANNER (DiTango, "Anchor-Guided Selection Planner": error model, anchor steps, online
 * prediction, group strategy).  Partitions p and q share a group iff p / G == q / G.  The
 * decision unit is a block group (I, J); its members are all FRESH or all REUSE (SKIP
 * members stay SKIP).  With E_ij the predicted error of reusing block (i, j) this step:
 *   E_IJ = sum of E_ij over the active members, i ascending then j ascending, in double;
 *   A_I  = active block groups of query group I, R_I = min(floor((pct A_I + 50)/100), A_I-1);
 *   FRESH: the diagonal group, every group with a member whose slot holds no state, every
 *   group with E_IJ > max_error (if max_error > 0), and then the groups of largest E_IJ
 *   (ties: smaller J first) until at least A_I - R_I groups are FRESH; the rest REUSE.
 * On a cache, E_ij = w_ij * (Cum_i(s-1) - Cum_i(f_ij) + delta_i(s-1)) for step s since the
 * last reset, with the block's last fresh step f_ij and quantities the library measures on
 * the device:
 *   w_ij      importance: mean over (b, h, rows r of partition i) of exp(lse_ij[r] - L_i[r]),
 *             L_i[r] = log sum over active j of exp(lse_ij[r]); measured on anchor steps;
 *   delta_i(t) growth: root mean square over (b, h, rows of i, d < D) of the change of the
 *             cached diagonal state O_ii from step t-1 to step t (the local state, always
 *             computed, as the proxy of remote drift); Cum_i(t) = sum of delta_i up to t.
 * Anchor steps (every active block FRESH, w refreshed): step 1 after a reset, then every
 * anchor_period steps (steps 1, 1 + A, 1 + 2A, ...; A = 0: only step 1), a policy with
 * anchor = 1, and a PLANNER step that has no importance measured since the reset. */
typedef struct dita_block_policy {
  int32_t kind;                  /* dita_policy_kind                                         */
  const uint8_t* explicit_mask;  /* host, P*P row-major, kind == EXPLICIT; copied            */
  int32_t max_fresh_frame_dist;  /* FRAME_THRESHOLD                                           */
  int32_t reuse_percent;         /* FRESH_BUDGET and PLANNER, 0..100                          */
  int32_t max_fresh_centroid2;   /* CENTROID_THRESHOLD, in doubled-token units                */
  int32_t tile_sparse;           /* 1: active iff f_j in {f_i, 0, f_i - 1, f_i + 1}
                                    (Efficient-vDiT's tile-style sparse 3D attention)         */
  int32_t anchor;                /* 1: every active block FRESH (anchor step)                 */
  int32_t group_size;            /* PLANNER: G >= 1 (0 is read as 1)                          */
  int32_t anchor_period;         /* PLANNER: A >= 0                                           */
  double max_error;              /* PLANNER: error cap, <= 0 = none                           */
} dita_block_policy;

typedef struct dita_step_stats {
  int64_t steps_done;            /* successful dita_attn_step calls since alloc              */
  int32_t last_counts[3];        /* SKIP, FRESH, REUSE blocks of the last step (P*P total)   */
  int32_t reserved;
  uint64_t device_fresh_blocks;  /* cumulative (b, h, i, j) fresh blocks counted on device   */
  uint64_t device_reuse_blocks;  /* cumulative (b, h, i, j) reused blocks counted on device  */
  uint64_t host_fresh_blocks;    /* the same two sums from the host plans, for comparison
                                    (reused: states read, a merged group counting once)       */
  uint64_t host_reuse_blocks;
  double last_fresh_flops;       /* sum over fresh blocks of 4 n_i n_j D, times B*H          */
  double last_cache_read_bytes;  /* sum over reused blocks of n_i (D*s_c + 4), times B*H     */
  double last_cache_write_bytes; /* sum over fresh blocks of n_i (D*s_c + 4), times B*H      */
  uint64_t device_v_range_errors;/* cumulative count of V elements with |v| > 65504: the bf16
                                    path multiplies P V in fp16, into which every bf16 value of
                                    magnitude 2^-14 to 65504 converts exactly (smaller ones,
                                    fp16 subnormals, keep an absolute error under 2^-25);
                                    steps that saw larger values are not valid               */
  uint64_t profiled_steps;       /* steps timed since profiling was enabled                  */
  double step_kernel_ms;         /* summed duration of the main step kernel over those steps */
  double prep_kernel_ms;         /* summed duration of the V-transpose kernel (bf16 only)    */
  uint64_t device_ref_recomputes;/* cumulative: bf16 steps computed a second time.  When every
                                    fresh block of a step has a state from an earlier step,
                                    the step first runs with each block's cached lse (per row)
                                    as its fixed softmax reference (no running maximum); if a
                                    row's sum over a block then falls outside [2^2, 2^15] (the
                                    block's lse moved by more than about 6 powers of two since
                                    it was cached) the whole step is computed again with the
                                    running maximum.  Results are
                                    the same either way, within rounding.                     */
  uint64_t fixed_ref_steps;      /* profiled bf16 steps that ran the fixed-reference pass      */
  double fixed_ref_kernel_ms;    /* their part of step_kernel_ms: the fixed-reference pass and
                                    the conditional second pass after it (which exits at once
                                    unless a reference was rejected); step_kernel_ms minus
                                    this is the running-maximum steps' time (anchor steps)    */
} dita_step_stats;

typedef struct dita_cache dita_cache;

/* Library version string (static storage). */
const char* dita_version(void);

/* Thread-local message describing the last failed call on this thread ("" if none). */
const char* dita_last_error(void);

/* Evaluate a policy without a cache: host only, integer arithmetic.
 *   valid     host, P*P, nonzero = the slot holds a state from an earlier step; NULL = none
 *   mask_out  host, P*P, receives DITA_SKIP / DITA_FRESH / DITA_REUSE
 * Errors: INVALID_ARGUMENT, SHAPE, POLICY, CACHE_MISS (REUSE where valid is zero). */
dita_status dita_policy_mask(const dita_geometry* geom, const dita_block_policy* policy,
                             const uint8_t* valid, uint8_t* mask_out);

/* The PLANNER decision from given predicted errors (host only, no cache):
 *   error     host, P*P doubles, E_ij (read for active off-diagonal blocks only)
 *   valid     host, P*P or NULL, as for dita_policy_mask
 *   mask_out  host, P*P
 * policy->kind must be PLANNER; policy->anchor = 1 gives the anchor mask.
 * Errors: INVALID_ARGUMENT, SHAPE. */
dita_status dita_planner_mask(const dita_geometry* geom, const dita_block_policy* policy,
                              const double* error, const uint8_t* valid, uint8_t* mask_out);

/* Partition offsets the geometry resolves to: host out[P+1]. */
dita_status dita_partition_offsets(const dita_geometry* geom, int32_t* out);

/* Bytes the device buffer must hold for this geometry.
 *   active_mask  host, P*P, nonzero = the block may ever be FRESH or REUSE (it gets a cache
 *                slot); NULL = every block. */
dita_status dita_cache_required_bytes(const dita_geometry* geom, const uint8_t* active_mask,
                                      size_t* bytes);

/* Create a cache handle bound to a caller-owned device buffer (device, 256-byte aligned,
 * at least dita_cache_required_bytes).  All slots start invalid, so the first step must be
 * an anchor (or use no REUSE).  No device work happens here.
 * Errors: INVALID_ARGUMENT, SHAPE, UNSUPPORTED, BUFFER_TOO_SMALL. */
dita_status dita_cache_alloc(const dita_geometry* geom, const uint8_t* active_mask,
                             void* device_buffer, size_t buffer_bytes, dita_cache** out);

/* Invalidate every slot and drop a pending policy; the next step must reuse nothing. */
dita_status dita_cache_reset(dita_cache* cache);

/* Free the host state; the device buffer stays the caller's.  Waits for steps in flight. */
dita_status dita_cache_free(dita_cache* cache);

/* Set the policy of the NEXT step.  Validates against the current slot validity.
 * Errors: INVALID_ARGUMENT, POLICY, CACHE_MISS.  On error the previous pending policy (if
 * any) is kept. */
dita_status dita_set_block_policy(dita_cache* cache, const dita_block_policy* policy);

/* The plan of the pending step (or, if none is pending, of the last executed step):
 *   mask        host P*P (members of a merged group all show REUSE)
 *   fresh_ptr   host P+1; fresh_cols host >= counts[1] entries (ascending j per row)
 *   reuse_ptr   host P+1; reuse_cols host >= counts[2] entries: the states read (a merged
 *               group appears once, as its first member)
 *   counts      host [3]: SKIP, FRESH, REUSE blocks of the mask
 * Any output pointer may be NULL.  Errors: INVALID_ARGUMENT, NO_POLICY. */
dita_status dita_get_block_plan(const dita_cache* cache, uint8_t* mask, int32_t* fresh_ptr,
                                int32_t* fresh_cols, int32_t* reuse_ptr, int32_t* reuse_cols,
                                int32_t* counts);

/* Run one denoising step's attention on `hip_stream` (a hipStream_t; NULL = default).
 *   q, k, v   device, [B,H,N,D] (or [B,N,H,D] with layout BNHD) of qkv_dtype (bf16: |v| <=
 *             65504, see device_v_range_errors), 16-byte aligned
 *   out       device, the geometry's out_dtype (f32 or bf16) in the same layout: the merged
 *             output; 16-byte aligned, overlapping neither q, k, v nor the cache buffer
 *   lse_out   device, [B,H,N] f32 natural-log L, or NULL; 4-byte aligned
 * Fresh blocks are recomputed and written back to their slots; reused blocks are read from
 * theirs.  Stream-asynchronous: returns after enqueueing.  On success the pending policy is
 * consumed, written slots become valid and the step counter advances.
 * bf16 path: the row groups that run last on each of the GPU's 8 XCDs are split in two
 * workgroups (half of the row's blocks each) whose partial merges a small second kernel
 * combines, so the grid ends on short workgroups; their rows' sums are associated
 * differently, so outputs may differ in the last bits from a run without splits.  By
 * default an eighth of an XCD's concurrent workgroups are split when the step runs two
 * rounds of workgroups or more.  Environment variables read when a geometry is resolved
 * (by dita_cache_required_bytes and dita_cache_alloc) override this: DITA_SPLITS_PER_XCD
 * sets the number of split row groups per XCD (0: none; at most 128), DITA_SPLIT_PARTS the
 * workgroups per split group (2 to 8).
 * Errors: INVALID_ARGUMENT, NO_POLICY, DEVICE. */
dita_status dita_attn_step(dita_cache* cache, const void* q, const void* k, const void* v,
                           void* out, float* lse_out, void* hip_stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): dita_attn_step with the same arguments, kernels and
 * results, which allocates nothing.  Its per-step scratch -- the transposed-V staging of the
 * bf16 path, the step's work lists and the split row groups' partial merges -- lives in a
 * static device array of 128 MiB that each
 * GPU the library runs on holds until the process ends, instead of in the cache's buffer
 * (which still holds the cached states and counters); the work lists are copied from the
 * handle's own pageable host buffer on `hip_stream`.  No hipMalloc, pinned host allocation,
 * event or other allocating call is made.
 *   - Every call on a GPU uses that GPU's one array, so calls that overlap on one GPU race:
 *     order them on one stream (or synchronise between them).  Nothing in the array needs to
 *     start at zero: each call writes all of what it reads.
 *   - Not profiled (dita_set_profiling does not time it).
 * Errors: those of dita_attn_step, and UNSUPPORTED when the step's scratch (B*H*DP*kt_pad*2
 * bytes of transposed V, DP the padded head dim and kt_pad the token count with each
 * partition padded to 64, plus the work lists and parts x 256 x (2 + DP/2) x 4 bytes per
 * split row group) exceeds 128 MiB, or when the pending policy
 * is a PLANNER step (its measurements are read back into host memory of the library's own). */
dita_status dita_attn_step_static(dita_cache* cache, const void* q, const void* k,
                                  const void* v, void* out, float* lse_out, void* hip_stream);

/* Copy one cache slot out in plain layout (for checks and export), on `hip_stream`:
 *   o_out    device, n_i x D f32 row-major: the cached O_ij rows of query partition i
 *   lse_out  device, n_i f32: the cached lse_ij (natural log)
 * Errors: INVALID_ARGUMENT (indices), POLICY (block without a slot), CACHE_MISS. */
dita_status dita_cache_read_slot(dita_cache* cache, int32_t b, int32_t h, int32_t i, int32_t j,
                                 float* o_out, float* lse_out, void* hip_stream);

/* Merge cached states into coarser groups (DiTango, "State-Centric Parallel Runtime /
 * Composizione Dinamica dei Gruppi": stored attention states are merged recursively into
 * coarser groups, with no recomputation; exact because states compose associatively).
 *   group     g >= 2: key partitions j and j' share a group iff j / g == j' / g
 *   select    host, P * ceil(P/g) bytes, row-major (i, J), nonzero = merge group (i, J);
 *             NULL = every eligible group
 *   merged    host, out, or NULL: the number of groups merged
 * Group (i, J) is eligible when it does not contain the diagonal block, every active member
 * holds a state, and it covers at least two states (a member already merged into a smaller
 * group inside J counts once: merging with g = 2 and then g = 4 gives groups of 4).  For
 * each row r of partition i the merged state is L = log sum_s exp(lse_s[r]) and
 * O = sum_s exp(lse_s[r] - L) O_s[r] over the group's states s, computed in f32 from the
 * cached (rounded) states and stored, rounded to the cache precision, in the slot of the
 * group's first active member.  From then on the group is one state: a REUSE of its members
 * reads it once (dita_get_block_plan lists the group's first member only), and a step whose
 * policy makes any member FRESH recomputes every member, which dissolves the group.
 * Stream-ordered on hip_stream.  Must be called between steps (no policy pending).
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (B*H or max partition rows / 32 above 65535), DEVICE. */
dita_status dita_cache_merge_groups(dita_cache* cache, int32_t group, const uint8_t* select,
                                    int32_t* merged, void* hip_stream);

/* Compaction of merged groups (DiTango, "State-Centric Parallel Runtime / Composizione
 * Dinamica dei Gruppi": merging stored states into coarser groups relieves memory pressure).
 * After dita_cache_merge_groups the members of a merged group other than its first hold no
 * state of their own; compaction moves the cache onto a slot table with one slot per stored
 * state, so that the buffer it needs shrinks with the merges (a group of g states frees g - 1
 * slots).
 *
 * dita_cache_compact_bytes: the bytes that table needs (host only; equals
 *   dita_cache_required_bytes when nothing is merged).
 *
 * dita_cache_compact: bind device_buffer (device, 256-byte aligned, at least
 *   dita_cache_compact_bytes, overlapping not the current buffer) and enqueue on hip_stream
 *   the copy of the counters and every stored state into it.  Between steps only (no policy
 *   pending).  The old buffer is the caller's again once hip_stream has passed the copy.
 *   Steps then run as before -- a REUSE of a merged group reads its one state -- with one
 *   restriction: a compacted group cannot be recomputed (a policy making any of its members
 *   FRESH fails with POLICY), since its members have no slots; dita_cache_reset keeps the
 *   groups (their states become invalid).  Merging further and compacting again is allowed.
 *
 * dita_cache_expand: the reverse: bind device_buffer (at least dita_cache_required_bytes)
 *   with every active block's slot back and copy the stored states into it; merged groups
 *   stay merged (their state in the first member's slot) and may be recomputed again.
 * Errors: INVALID_ARGUMENT (NULL, misaligned, overlapping, other device, policy pending, expand
 * of a cache that is not compacted), BUFFER_TOO_SMALL, OFFLOADED, UNSUPPORTED (B*H above
 * 65535), DEVICE. */
dita_status dita_cache_compact_bytes(const dita_cache* cache, size_t* bytes);
dita_status dita_cache_compact(dita_cache* cache, void* device_buffer, size_t buffer_bytes,
                               void* hip_stream);
dita_status dita_cache_expand(dita_cache* cache, void* device_buffer, size_t buffer_bytes,
                              void* hip_stream);

/* Enable (1) or disable (0) kernel timing: the library records HIP events on the launch
 * stream around each of its kernels and sums their durations into dita_step_stats.
 * Enabling resets the sums.  Errors: INVALID_ARGUMENT. */
dita_status dita_set_profiling(dita_cache* cache, int32_t enable);

/* The PLANNER's measured state, after waiting for the measurements of the last step:
 *   w          host P*P f32 or NULL: importance from the last anchor step (zeros if none)
 *   delta      host steps*P doubles or NULL: delta_i(t) for t = 1..steps, row t-1 for step t
 *              (0 where not measured: step 1, and steps run with another policy kind)
 *   fresh_step host P*P int32 or NULL: step since the reset at which each block was last
 *              FRESH (0 = never)
 *   steps      host, out: steps since the last reset
 * Cum_i(t) = delta_i(1) + ... + delta_i(t), summed in that order.  Pass delta = NULL to
 * query `steps` first.  Errors: INVALID_ARGUMENT, DEVICE. */
dita_status dita_get_planner_state(dita_cache* cache, float* w, double* delta,
                                   int32_t* fresh_step, int32_t* steps);

/* Host offload of the state cache (DiTango, "Significato e Claim": the memory the state cache
 * takes stays a constraint in production, and offloading it to the CPU is named as future
 * work).
 * For a caller that keeps several caches on one GPU, e.g. several generations in flight,
 * and wants an idle cache's device memory back.  The offloaded state is the device counters
 * followed by the cached lse and O of every slot; everything else in the buffer (work lists,
 * V^T scratch, planner partials, merge jobs, snapshots) is rebuilt by the step that uses it.
 *
 * dita_cache_offload_bytes: host bytes the offloaded state takes (host only).
 *
 * dita_cache_offload: enqueue on hip_stream the copy of the state into host_dst (host, at
 *   least dita_cache_offload_bytes; pinned memory from hipHostMalloc for the full link
 *   rate) and mark the cache offloaded.  Stream-ordered: pass the stream of the last step or
 *   merge on this cache (or synchronise first).  Once hip_stream has passed the copy, the
 *   device buffer may be freed or reused.  host_dst must stay untouched until the restore.
 *   While offloaded, dita_attn_step, dita_cache_merge_groups and dita_cache_read_slot fail
 *   with OFFLOADED; policies may be set, plans read, the cache reset or freed, and
 *   dita_get_stats reports the counters from host_dst.
 *   Errors: INVALID_ARGUMENT (NULL pointer, too small, already offloaded), DEVICE.
 *
 * dita_cache_restore: bind device_buffer (device, 256-byte aligned, at least
 *   dita_cache_required_bytes, on the device the cache ran on: the original buffer or
 *   another) and enqueue on hip_stream the copy of the state back from host_src (host, as
 *   written by dita_cache_offload; it must stay alive until hip_stream has passed the copy).
 *   The cache then continues exactly where it stopped: slot validity, last-fresh steps,
 *   merged groups and the planner's measurements are unchanged.
 *   Errors: INVALID_ARGUMENT (not offloaded, NULL, misaligned, other device),
 *   BUFFER_TOO_SMALL, DEVICE.  On error the cache stays offloaded. */
dita_status dita_cache_offload_bytes(const dita_cache* cache, size_t* bytes);
dita_status dita_cache_offload(dita_cache* cache, void* host_dst, size_t host_bytes,
                               void* hip_stream);
dita_status dita_cache_restore(dita_cache* cache, void* device_buffer, size_t buffer_bytes,
                               const void* host_src, size_t host_bytes, void* hip_stream);

/* Counters and last-step work.  Synchronises the device to read the device counters. */
dita_status dita_get_stats(const dita_cache* cache, dita_step_stats* stats);

#ifdef __cplusplus
}
#endif

#endif /* DITA_H */
