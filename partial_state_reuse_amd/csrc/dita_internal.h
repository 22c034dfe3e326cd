// Private interface between the host library (dita_host.cpp) and the HIP kernels
// (dita_kernels.hip).  Not part of the C ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace dita {

// Keys per K/V tile staged in LDS by the bf16 kernel.
constexpr int kKeyTile = 64;
// Waves per workgroup of the bf16 kernel.
constexpr int kWaves = 4;
// Query rows per workgroup of the f32 kernel (one row per lane of one wave).
constexpr int kF32Rows = 64;
// Cache slots hold their rows padded to a multiple of this.
constexpr int kSlotRowAlign = 64;
// Number of device plan slots kept per cache (plans are re-uploaded only on a change).
constexpr int kPlanSlots = 4;

// Padded head dimension used by the bf16 kernel for a head_dim D (0 = unsupported).
inline int bf16_padded_dim(int D) {
  if (D <= 0 || D % 8 != 0 || D > 128) return 0;
  return D <= 64 ? 64 : (D <= 96 ? 96 : 128);
}
// Query rows per bf16 workgroup (each wave owns a 32-row sub-tile).
inline int bf16_wg_rows(int /*DP*/) { return kWaves * 32; }

// Layout of one device plan (int32 words), as written by the host and read by the kernels:
//   [0] num_tiles  [1] P  [2] E (entries)  [3] number of tail workgroups (packs)
//   offs   at kPlanHeader                 : P+1 partition offsets o_p
//   poffs  at kPlanHeader + (P+1)         : P+1 padded offsets of the transposed-V scratch
//   tiles  at kPlanHeader + 2(P+1)        : num_tiles words: (i << 16) | group-in-partition
//                                           for a workgroup of 4 waves on consecutive rows,
//                                           or kTailFlag | k for tail workgroup k (pack k)
//   packs  at tiles + num_tiles           : 4 words per pack {first member, members, first
//                                           union entry, union entries}
//   members at packs + 4 * packs          : 4 words per member {i, first row, rows, first
//                                           lane}: a tail sub-tile of partition i, whose rows
//                                           the pack's lanes first lane.. hold
//   rows   at members + 4 * members       : P x 4 words {first entry, #fresh, #reuse, 0}
//   ent    at rows + 4P                   : E x 2 words {j, slot}; per row the fresh blocks
//                                           (ascending j) precede the reused ones (room for P^2)
//   union  at ent + 2 P^2                 : 2 words per entry {j, first pack slot}: per pack
//                                           the union of its members' fresh blocks, ascending j
//                                           (room for P per pack)
//   pslot  at union + 2 P * packs         : per union entry, one word per member of its pack:
//                                           the slot of block (i_m, j), or -1 where j is not
//                                           fresh for member m (room for P per member)
//   items  at pslot + P * members         : bf16 path: 2 words per workgroup {b*H + h, tile
//                                           word}, in the order of the logical workgroup index
//                                           (after the XCD remap); the tile word is a group or
//                                           tail word as above, or kSplitFlag | (s << 3) | part
//                                           for part `part` of split row group s
//   splits at items + 2 * items           : 2 words per split row group {b*H + h, group word}
constexpr int kPlanHeader = 4;
constexpr int32_t kTailFlag = 1 << 30;
// bf16 path: the row groups dispatched last on each XCD run as split_parts workgroups each
// (consecutive shares of the row's fresh blocks and of its reused states), so that the grid
// ends on short workgroups; each part leaves its partial merge of the rows in a workspace and
// merge_splits combines the parts and writes the rows.
constexpr int32_t kSplitFlag = 1 << 29;
// at most this many split row groups per step
constexpr int kMaxSplits = 1024;
// at most this many parts per split row group
constexpr int kMaxSplitParts = 8;
// bf16 path: a partition whose last row group would leave at most this many of its 4 waves
// with rows hands those rows to tail sub-tiles instead; the tail sub-tiles of consecutive
// partitions are packed into 32-row tiles while their rows fit, one workgroup per pack, whose
// 4 waves share the union of the members' blocks.
constexpr int kMaxTailSubtiles = 2;

struct StepArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;                 // f32, or bf16 with out_bf16
  float* lse_out;            // may be null
  void* vt;                  // fp16 transposed-V scratch [B*H][DP][kt_pad]
  void* cache_o;             // bf16 / fp8: [B*H][slots][slot_rows/32][DP/32][64][16] elements
                             //   in fragment order
                             // f32:  [B*H][slots][DP][slot_rows]
  float* cache_lse;          // [B*H][slots][slot_rows], natural log
  unsigned long long* counters;  // [0] fresh blocks, [1] reused blocks, [2] V elements
                                 // outside the fp16 range, [3] steps computed a second time
                                 // (cumulative); [4] this step's fixed-reference rejection
                                 // flag (cleared by transpose_v)
  const int32_t* plan;       // device plan (layout above)
  int32_t off_offs, off_poffs, off_tiles, off_pack, off_member, off_rows, off_ent, off_union,
      off_pslot, off_items, off_splits;
  int32_t B, H, N, D, DP, P;
  // element strides of Q, K, V and out: (b, h, token n, d) at b*sB + h*sH + n*ld + d
  // ([B,H,N,D]: sB = H N D, sH = N D, ld = D; [B,N,H,D]: sB = N H D, sH = D, ld = H D)
  int64_t sB, sH;
  int32_t ld;
  int32_t num_tiles;         // workgroup tiles per (b, h)
  int32_t num_items;         // bf16 path: workgroups of the step (the items list)
  int32_t num_splits;        // bf16 path: split row groups
  int32_t split_parts;       // bf16 path: workgroups per split row group
  // bf16 path: partial merges of the split parts, [split][part][2 + DP / 2][256] floats
  // (m, l, then the accumulator registers, of thread t of the workgroup at [.][t])
  float* split_ws;
  int32_t num_slots;
  int32_t slot_rows;
  int32_t kt_pad;            // padded token count of the transposed-V scratch
  float scale_log2;          // tau * log2(e)
  // Planner measurement (null = off): at the write-back of each diagonal block the kernel
  // stores, per 32-row sub-tile, the sum over its rows (< n_i) and dims (< D) of
  // (new cached O - old cached O)^2 at delta_part[(bh * P + i) * delta_stride + row / 32].
  float* delta_part;
  int32_t delta_stride;      // slot_rows / 32
  // bf16 path, measuring steps: the diagonal slots' cached O as it was before the step
  // ([B*H][P][slot_rows/32][DP/32][64][16], as a slot), which the measurement reads as the old
  // state, so that a second pass over the step measures the same change
  const void* diag_snap;
  int32_t cache_fp8;         // bf16 path: cached O as fp8 e4m3 (1) or bf16 (0)
  // bf16 path: every fresh block's slot holds a state from an earlier step, so the step runs
  // as a fixed-reference pass followed by the running-maximum kernel as a conditional second
  // pass (fixup = 1), which exits at once unless the first pass rejected a reference
  int32_t fixed_ref;
  int32_t fixup;
  int32_t out_bf16;          // bf16 path: out in bf16 (round to nearest even) instead of f32
};

hipError_t launch_zero_counters(unsigned long long* counters, int n, hipStream_t s);
hipError_t launch_transpose_v(const StepArgs& a, hipStream_t s);
// Both passes of the bf16 step, each followed by merge_splits when the plan has split row
// groups.
hipError_t launch_step_bf16(const StepArgs& a, hipStream_t s);
hipError_t launch_step_f32(const StepArgs& a, hipStream_t s);
// Planner reductions, on a plan whose row lists hold every active block of each row:
//   delta[i] = sqrt(sum over (b, h, sub-tiles of i) of delta_part / (B H n_i D))
//   w[i P + j] = mean over (b, h, rows r of i) of exp(lse_ij[r] - L_i[r]), L_i[r] = log sum
//                over the row's blocks of exp(lse_ij[r]) (natural log, from the cached lse)
// Fixed summation order: the results do not depend on scheduling.
// The importance runs as (row chunks x P) workgroups writing per-chunk sums to `part`
// (P * planner_chunks(P) * P floats), then one sum per partition.
inline int planner_chunks(int P) { return P >= 2048 ? 1 : (2048 / P > 64 ? 64 : 2048 / P); }
hipError_t launch_planner_delta(const StepArgs& a, float* delta, hipStream_t s);
hipError_t launch_snapshot_diag(const StepArgs& a, hipStream_t s);
// the diagonal states' change against the snapshot, after a measuring step (bf16 path)
hipError_t launch_diag_change(const StepArgs& a, hipStream_t s);
hipError_t launch_planner_weights(const StepArgs& a, float* w, float* part, hipStream_t s);
// Group composition: job k = jobs[4k..4k+3] = {n_i, dst slot, first source, sources}; the
// sources are slot numbers in srcs.  Grid (njobs, slot_rows / 32 sub-tiles, B*H).
hipError_t launch_merge_slots(const StepArgs& a, const int32_t* jobs, const int32_t* srcs,
                              int njobs, int cache_esz, hipStream_t s);
hipError_t launch_read_slot(const StepArgs& a, int bh, int slot, int i, float* o_out,
                            float* lse_out, int cache_esz, hipStream_t s);

// Cache compaction / expansion: for each of the npairs {new slot, old slot} pairs of `map`
// (device, 2 * npairs int32) and each of the bhs (b, h) pairs, copy the slot's lse row and O
// from the old slot table's buffers to the new one's.  Grid (npairs, bhs); npairs and bhs up
// to 2^31 - 1 and 65535.
hipError_t launch_remap_slots(const float* old_lse, const void* old_o, float* new_lse,
                              void* new_o, const int32_t* map, int npairs, int bhs,
                              int old_slots, int new_slots, int slot_rows,
                              size_t o_slot_bytes, hipStream_t s);

// Device scratch of the allocation-free step (dita_attn_step_static): a file-scope device
// array of this many bytes per GPU, holding the step's transposed-V staging and work lists.
constexpr size_t kStaticScratchBytes = (size_t)128 << 20;
// Its device address on the current device (looked up once per device with that device
// current; the array's host-side name is not a device address).
hipError_t static_scratch_address(void** out);

}  // namespace dita
