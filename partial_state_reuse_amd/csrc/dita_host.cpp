// Host side of the dita library: geometry, block policy, slot table, work lists,
// validation, bookkeeping and the C ABI declared in include/dita.h.
//
// Method (DiTango, gist.science 2607.15650):
//   "Anchor-Guided Selection Planner": per step each partition block is recomputed or
//   reuses a state from an earlier step; anchor steps recompute everything; the local
//   partition is always computed.
//   "State-Centric Parallel Runtime / Composizione dello Stato": the cached unit is the
//   (output, log-sum-exp) state of a block.
// Efficient-vDiT (chatpaper abstract): tile-style sparse 3D attention (own frame, first
// frame, neighbouring frames), linear in the number of frames, used as the active set.
#include "dita.h"

#include <algorithm>
#include <cstdlib>
#include <array>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "dita_internal.h"

namespace {

thread_local std::string g_err;

dita_status fail(dita_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dita_status ok() { return DITA_OK; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Resolved geometry.
struct Geo {
  int B = 0, H = 0, N = 0, D = 0, DP = 0, P = 0;
  int frames = 0, gh = 0, gw = 0, F = 0;
  dita_dtype qkv = DITA_BF16, cache_o = DITA_BF16;
  int layout = DITA_LAYOUT_BHND;
  dita_dtype out = DITA_F32;
  float tau = 0.f;
  std::vector<int32_t> offs;    // P+1
  std::vector<int64_t> c2;      // doubled centroids
  std::vector<int32_t> frame;   // frame of each partition
  std::vector<int32_t> poffs;   // P+1 padded offsets (multiples of the key tile)
  int kt_pad = 0;
  int wg_rows = 0;
  int num_tiles = 0;                 // workgroups per (b, h): tail workgroups, then groups
  int num_tail_wg = 0;               // tail workgroups per (b, h): one per pack
  std::vector<int32_t> groups;       // per partition: row groups run by 4-wave workgroups
  std::vector<int32_t> members;      // {i, first row, rows, first lane} per tail sub-tile
  std::vector<int32_t> packs;        // {first member, members} per pack of tail sub-tiles
  // bf16 path: the step's workgroups in logical order, {b*H + h, tile word} each, and the
  // split row groups {b*H + h, tile word of the group}
  std::vector<int32_t> items;
  std::vector<int32_t> splits;
  int num_items = 0, num_splits = 0, split_parts = 2;
  int slot_rows = 0;
  bool bf16() const { return qkv == DITA_BF16; }
  // bytes per cached O element
  size_t cache_esz() const { return cache_o == DITA_FP8_E4M3 ? 1 : (cache_o == DITA_BF16 ? 2 : 4); }
};

// The bf16 step's workgroups in logical order.  Workgroup ids are dealt round-robin to the 8
// XCDs and the kernel maps XCD x's ids onto the x-th contiguous range of logical indices
// (xcd_remap), so XCD x runs its range front to back.  The (b, h) tiles are laid out head
// after head; in each XCD's range the last K row groups are split in NP parts, which become
// adjacent workgroups of about 1 / NP of the length, so that the grid's end on that XCD is
// made of short workgroups.  K is an eighth of the XCD's concurrent workgroups (32 CUs x 3 at
// DP = 64, x 2 above), and 0 when the range holds fewer than two rounds of them or when some
// range has fewer than K row groups (not tail workgroups) to split.  The environment
// variables DITA_SPLITS_PER_XCD (0 turns the splitting off; at most kMaxSplits / 8) and
// DITA_SPLIT_PARTS (2 to kMaxSplitParts), read when a geometry is resolved, set K and NP.
constexpr int kDefaultSplitParts = 2;
void build_items(Geo* r) {
  const int64_t G0 = (int64_t)r->B * r->H * r->num_tiles;
  std::vector<int32_t> word(r->num_tiles);   // tile words of one (b, h), in order
  {
    int t = 0;
    for (int k = 0; k < r->num_tail_wg; ++k) word[t++] = dita::kTailFlag | k;
    for (int i = 0; i < r->P; ++i)
      for (int g = 0; g < r->groups[i]; ++g) word[t++] = (i << 16) | g;
  }
  const int per_cu = r->DP == 64 ? 3 : 2;
  const int slots = 32 * per_cu;
  int K = G0 / 8 >= 2 * slots ? slots / 8 : 0;
  if (const char* e = std::getenv("DITA_SPLITS_PER_XCD")) K = std::max(0, std::atoi(e));
  K = std::min(K, dita::kMaxSplits / 8);
  int NP = kDefaultSplitParts;
  if (const char* e = std::getenv("DITA_SPLIT_PARTS"))
    NP = std::max(2, std::min(dita::kMaxSplitParts, std::atoi(e)));
  r->split_parts = NP;
  for (;; K = 0) {
    const int64_t G = G0 + 8 * (int64_t)K * (NP - 1);
    r->items.clear();
    r->splits.clear();
    r->items.reserve(2 * G);
    int64_t cursor = 0;               // next tile of the regular (head-major) order
    bool short_of_groups = false;
    for (int x = 0; x < 8 && !short_of_groups; ++x) {
      const int64_t chunk = G / 8 + (x < G % 8 ? 1 : 0);
      const int64_t n = chunk - (int64_t)K * (NP - 1);   // regular tiles of this XCD's range
      std::vector<uint8_t> split_here(n, 0);
      int need = K;
      for (int64_t y = n - 1; y >= 0 && need > 0; --y)
        if (!(word[(cursor + y) % r->num_tiles] & dita::kTailFlag)) {
          split_here[y] = 1;
          --need;
        }
      if (need > 0) {                 // too few row groups to split here: split none at all
        short_of_groups = true;
        break;
      }
      for (int64_t y = 0; y < n; ++y) {
        const int64_t t = cursor + y;
        const int32_t bh = (int32_t)(t / r->num_tiles), w = word[t % r->num_tiles];
        if (!split_here[y]) {
          r->items.push_back(bh);
          r->items.push_back(w);
          continue;
        }
        const int sidx = (int)(r->splits.size() / 2);
        r->splits.push_back(bh);
        r->splits.push_back(w);
        for (int part = 0; part < NP; ++part) {
          r->items.push_back(bh);
          r->items.push_back(dita::kSplitFlag | (sidx << 3) | part);
        }
      }
      cursor += n;
    }
    if (!short_of_groups || K == 0) break;
  }
  r->num_items = (int)(r->items.size() / 2);
  r->num_splits = (int)(r->splits.size() / 2);
}

dita_status resolve_geometry(const dita_geometry* g, Geo* out) {
  if (!g) return fail(DITA_ERR_INVALID_ARGUMENT, "geometry is NULL");
  Geo r;
  r.B = g->batch; r.H = g->heads; r.N = g->tokens; r.D = g->head_dim;
  r.frames = g->frames; r.gh = g->grid_h; r.gw = g->grid_w; r.P = g->num_partitions;
  if (r.B <= 0 || r.H <= 0 || r.N <= 0 || r.D <= 0)
    return fail(DITA_ERR_SHAPE, "batch, heads, tokens and head_dim must be positive");
  if (r.frames <= 0 || r.gh <= 0 || r.gw <= 0)
    return fail(DITA_ERR_SHAPE, "frames, grid_h and grid_w must be positive");
  if ((int64_t)r.frames * r.gh * r.gw != r.N)
    return fail(DITA_ERR_SHAPE, "tokens (%d) != frames*grid_h*grid_w (%lld)", r.N,
                (long long)r.frames * r.gh * r.gw);
  if (r.P < 1 || r.P > 1024 || r.P > r.N)
    return fail(DITA_ERR_SHAPE, "num_partitions must be in 1..min(1024, tokens)");
  if ((int64_t)r.B * r.H * r.N * r.D >= (int64_t)1 << 40)
    return fail(DITA_ERR_SHAPE, "tensor too large");
  r.F = r.gh * r.gw;
  if (g->qkv_dtype != DITA_F32 && g->qkv_dtype != DITA_BF16)
    return fail(DITA_ERR_INVALID_ARGUMENT, "unknown qkv_dtype");
  if (g->cache_o_dtype != g->qkv_dtype &&
      !(g->cache_o_dtype == DITA_FP8_E4M3 && g->qkv_dtype == DITA_BF16))
    return fail(DITA_ERR_UNSUPPORTED, "cache_o_dtype must equal qkv_dtype, or be FP8_E4M3 with "
                "bf16 Q/K/V");
  r.qkv = g->qkv_dtype;
  r.cache_o = g->cache_o_dtype;
  if (g->layout != DITA_LAYOUT_BHND && g->layout != DITA_LAYOUT_BNHD)
    return fail(DITA_ERR_INVALID_ARGUMENT, "unknown layout %d", g->layout);
  r.layout = g->layout;
  if (g->out_dtype != DITA_F32 && g->out_dtype != DITA_BF16)
    return fail(DITA_ERR_INVALID_ARGUMENT, "out_dtype must be F32 or BF16");
  if (g->out_dtype == DITA_BF16 && g->qkv_dtype != DITA_BF16)
    return fail(DITA_ERR_UNSUPPORTED, "a bf16 output needs bf16 Q/K/V");
  r.out = g->out_dtype;
  if ((int64_t)r.H * r.D > INT32_MAX) return fail(DITA_ERR_SHAPE, "heads x head_dim too large");
  if (r.bf16()) {
    r.DP = dita::bf16_padded_dim(r.D);
    if (!r.DP) return fail(DITA_ERR_UNSUPPORTED, "bf16 head_dim must be a multiple of 8 <= 128");
    r.wg_rows = dita::bf16_wg_rows(r.DP);
  } else {
    if (r.D > 64 || r.D % 4 != 0)
      return fail(DITA_ERR_UNSUPPORTED, "f32 head_dim must be a multiple of 4 <= 64");
    r.DP = 64;
    r.wg_rows = dita::kF32Rows;
  }
  r.tau = g->softmax_scale > 0.f ? g->softmax_scale : 1.0f / std::sqrt((float)r.D);
  r.offs.resize(r.P + 1);
  if (g->partition_offsets) {
    for (int p = 0; p <= r.P; ++p) r.offs[p] = g->partition_offsets[p];
    if (r.offs[0] != 0 || r.offs[r.P] != r.N)
      return fail(DITA_ERR_SHAPE, "partition offsets must start at 0 and end at tokens");
    for (int p = 0; p < r.P; ++p)
      if (r.offs[p + 1] <= r.offs[p])
        return fail(DITA_ERR_SHAPE, "partition offsets must increase strictly");
  } else {
    // numpy array_split rule: the first N mod P partitions hold one extra token
    const int base = r.N / r.P, extra = r.N % r.P;
    r.offs[0] = 0;
    for (int p = 0; p < r.P; ++p) r.offs[p + 1] = r.offs[p] + base + (p < extra ? 1 : 0);
  }
  int max_n = 0;
  r.c2.resize(r.P);
  r.frame.resize(r.P);
  r.poffs.resize(r.P + 1);
  r.poffs[0] = 0;
  r.groups.resize(r.P);
  int num_groups = 0;
  for (int p = 0; p < r.P; ++p) {
    const int n = r.offs[p + 1] - r.offs[p];
    if (n >= 65536 * 32) return fail(DITA_ERR_SHAPE, "partition too large");
    max_n = std::max(max_n, n);
    r.c2[p] = (int64_t)r.offs[p] + r.offs[p + 1] - 1;
    r.frame[p] = (int32_t)(r.c2[p] / (2 * (int64_t)r.F));
    r.poffs[p + 1] = r.poffs[p] + (int)align_up(n, dita::kKeyTile);
    // Row groups of wg_rows rows.  On the bf16 path a last group that would keep at most
    // kMaxTailSubtiles of its 4 waves busy becomes tail sub-tiles instead: one workgroup per
    // sub-tile, whose 4 waves share the row's blocks, so no wave slot idles on empty rows.
    int full = n / r.wg_rows;
    const int rem = n - full * r.wg_rows;
    const int sub = (rem + 31) / 32;
    if (rem > 0 && r.bf16() && sub <= dita::kMaxTailSubtiles) {
      for (int s = 0; s < sub; ++s) {
        r.members.push_back(p);
        r.members.push_back(full * r.wg_rows + 32 * s);
        r.members.push_back(std::min(32, rem - 32 * s));
        r.members.push_back(0);
      }
    } else if (rem > 0) {
      ++full;
    }
    r.groups[p] = full;
    num_groups += full;
  }
  // Tail sub-tiles of consecutive partitions share one 32-row tile while their rows fit: a
  // pack's lanes hold the rows of its members one after another.
  {
    const int nm = (int)(r.members.size() / 4);
    int lanes = 32;
    for (int m = 0; m < nm; ++m) {
      const int rows = r.members[4 * m + 2];
      if (lanes + rows > 32) {
        r.packs.push_back(m);
        r.packs.push_back(0);
        lanes = 0;
      }
      r.members[4 * m + 3] = lanes;
      lanes += rows;
      r.packs.back() += 1;
    }
  }
  r.num_tail_wg = (int)(r.packs.size() / 2);
  r.num_tiles = r.num_tail_wg + num_groups;
  r.kt_pad = r.poffs[r.P];
  r.slot_rows = (int)align_up(max_n, dita::kSlotRowAlign);
  if (r.bf16()) {
    // the step kernel's tile loads take 32-bit byte offsets inside a head's V^T and inside a
    // tile of 64 key rows of K
    const int64_t ld = r.layout == DITA_LAYOUT_BNHD ? (int64_t)r.H * r.D : r.D;
    if ((int64_t)r.DP * r.kt_pad * 2 >= ((int64_t)1 << 31) ||
        (int64_t)dita::kKeyTile * ld * 2 >= ((int64_t)1 << 31))
      return fail(DITA_ERR_SHAPE, "a head's padded V^T or a tile of key rows exceeds 2 GiB");
    const int64_t G0 = (int64_t)r.B * r.H * r.num_tiles;
    if (G0 + dita::kMaxSplits >= ((int64_t)1 << 28))
      return fail(DITA_ERR_SHAPE, "too many workgroups (%lld)", (long long)G0);
    build_items(&r);
  }
  *out = std::move(r);
  return ok();
}

bool tile_active(const Geo& g, int i, int j) {
  const int fi = g.frame[i], fj = g.frame[j];
  return fj == fi || fj == 0 || fj == fi - 1 || fj == fi + 1;
}

// Checks shared by every policy: diagonal FRESH, non-SKIP blocks own a slot, REUSE blocks
// hold a state.
dita_status validate_mask(const Geo& g, std::vector<uint8_t> M, const uint8_t* valid,
                          const int32_t* slot_of, std::vector<uint8_t>* out) {
  const int P = g.P;
  for (int i = 0; i < P; ++i)
    if (M[(size_t)i * P + i] != DITA_FRESH)
      return fail(DITA_ERR_POLICY, "diagonal block (%d,%d) must be FRESH", i, i);
  for (size_t b = 0; b < M.size(); ++b) {
    if (M[b] == DITA_SKIP) continue;
    if (slot_of && slot_of[b] < 0)
      return fail(DITA_ERR_POLICY, "block (%d,%d) has no cache slot (not in the active mask)",
                  (int)(b / P), (int)(b % P));
    if (M[b] == DITA_REUSE && (!valid || !valid[b]))
      return fail(DITA_ERR_CACHE_MISS, "block (%d,%d) is REUSE but its slot holds no state",
                  (int)(b / P), (int)(b % P));
  }
  *out = std::move(M);
  return ok();
}

// PLANNER decision (DiTango, "Anchor-Guided Selection Planner": error model and group
// strategy).  E (P*P, may be null when anchor) holds the predicted reuse errors.  Decision
// unit: block group (I, J) of G x G partitions; its active members are all FRESH or all
// REUSE.  Per query group: the diagonal group, groups with a member whose slot holds no
// state, and groups whose summed error exceeds max_error (if > 0) are FRESH; then groups of
// largest summed error (ties: smaller J) until A - R are FRESH, R = min(floor((pct A + 50) /
// 100), A - 1) of the A active groups.  Sums run in double, i ascending then j ascending.
dita_status planner_decide(const Geo& g, const dita_block_policy* pol, const double* E,
                           const uint8_t* valid, const int32_t* slot_of, bool anchor,
                           std::vector<uint8_t>* out) {
  const int P = g.P;
  if (pol->reuse_percent < 0 || pol->reuse_percent > 100)
    return fail(DITA_ERR_INVALID_ARGUMENT, "reuse_percent must be in 0..100");
  if (pol->group_size < 0 || pol->anchor_period < 0)
    return fail(DITA_ERR_INVALID_ARGUMENT, "group_size and anchor_period must be >= 0");
  if (!anchor && !E) return fail(DITA_ERR_INVALID_ARGUMENT, "error is NULL");
  const int G = pol->group_size > 0 ? pol->group_size : 1;
  const int NG = (P + G - 1) / G;
  auto active = [&](int i, int j) { return !pol->tile_sparse || tile_active(g, i, j); };
  std::vector<uint8_t> M((size_t)P * P, DITA_SKIP);
  struct Cand { int J; double e; bool forced; };
  std::vector<Cand> cand;
  for (int I = 0; I < NG; ++I) {
    const int i0 = I * G, i1 = std::min(P, i0 + G);
    cand.clear();
    for (int J = 0; J < NG; ++J) {
      const int j0 = J * G, j1 = std::min(P, j0 + G);
      bool any = false, invalid = false;
      double e = 0.0;
      for (int i = i0; i < i1; ++i)
        for (int j = j0; j < j1; ++j) {
          if (!active(i, j)) continue;
          any = true;
          const size_t b = (size_t)i * P + j;
          if (!valid || !valid[b]) invalid = true;
          if (!anchor && i != j) e += E[b];
        }
      if (any) cand.push_back({J, e, anchor || J == I || invalid ||
                                         (pol->max_error > 0.0 && e > pol->max_error)});
    }
    const int A = (int)cand.size();
    const int n_reuse = std::min((pol->reuse_percent * A + 50) / 100, A - 1);
    int n_fresh = 0;
    for (const Cand& c : cand) n_fresh += c.forced;
    std::vector<const Cand*> rest;
    for (const Cand& c : cand)
      if (!c.forced) rest.push_back(&c);
    std::sort(rest.begin(), rest.end(), [](const Cand* a, const Cand* b) {
      if (a->e != b->e) return a->e > b->e;
      return a->J < b->J;
    });
    std::vector<uint8_t> gfresh(NG, 0);
    for (const Cand& c : cand)
      if (c.forced) gfresh[c.J] = 1;
    for (const Cand* c : rest)
      if (n_fresh < A - n_reuse) {
        gfresh[c->J] = 1;
        ++n_fresh;
      }
    for (const Cand& c : cand) {
      const int j0 = c.J * G, j1 = std::min(P, j0 + G);
      for (int i = i0; i < i1; ++i)
        for (int j = j0; j < j1; ++j)
          if (active(i, j)) M[(size_t)i * P + j] = gfresh[c.J] ? DITA_FRESH : DITA_REUSE;
    }
  }
  return validate_mask(g, std::move(M), valid, slot_of, out);
}

// Mask of one step.  `valid` (P*P, may be null) marks slots holding an earlier state;
// `slot_of` (P*P, may be null) marks blocks that own a cache slot (>= 0).
dita_status eval_policy(const Geo& g, const dita_block_policy* pol, const uint8_t* valid,
                        const int32_t* slot_of, std::vector<uint8_t>* out) {
  if (!pol) return fail(DITA_ERR_INVALID_ARGUMENT, "policy is NULL");
  const int P = g.P;
  std::vector<uint8_t> M((size_t)P * P, DITA_SKIP);
  auto active = [&](int i, int j) { return !pol->tile_sparse || tile_active(g, i, j); };
  if (pol->kind == DITA_POLICY_EXPLICIT) {
    if (!pol->explicit_mask) return fail(DITA_ERR_INVALID_ARGUMENT, "explicit_mask is NULL");
    for (int i = 0; i < P; ++i)
      for (int j = 0; j < P; ++j) {
        const uint8_t m = pol->explicit_mask[(size_t)i * P + j];
        if (m > DITA_REUSE)
          return fail(DITA_ERR_POLICY, "mask value %d at (%d,%d) outside {0,1,2}", m, i, j);
        if (m != DITA_SKIP && !active(i, j))
          return fail(DITA_ERR_POLICY, "block (%d,%d) is outside the tile-sparse set", i, j);
        M[(size_t)i * P + j] = (pol->anchor && m != DITA_SKIP) ? (uint8_t)DITA_FRESH : m;
      }
  } else if (pol->kind == DITA_POLICY_FRAME_THRESHOLD ||
             pol->kind == DITA_POLICY_CENTROID_THRESHOLD ||
             pol->kind == DITA_POLICY_FRESH_BUDGET) {
    if (pol->kind == DITA_POLICY_FRESH_BUDGET &&
        (pol->reuse_percent < 0 || pol->reuse_percent > 100))
      return fail(DITA_ERR_INVALID_ARGUMENT, "reuse_percent must be in 0..100");
    std::vector<int> cand;
    cand.reserve(P);
    for (int i = 0; i < P; ++i) {
      cand.clear();
      for (int j = 0; j < P; ++j)
        if (active(i, j)) cand.push_back(j);
      uint8_t* row = &M[(size_t)i * P];
      if (pol->anchor) {
        for (int j : cand) row[j] = DITA_FRESH;
      } else if (pol->kind == DITA_POLICY_FRAME_THRESHOLD) {
        for (int j : cand)
          row[j] = std::abs(g.frame[i] - g.frame[j]) <= pol->max_fresh_frame_dist
                       ? DITA_FRESH : DITA_REUSE;
      } else if (pol->kind == DITA_POLICY_CENTROID_THRESHOLD) {
        for (int j : cand)
          row[j] = std::llabs(g.c2[i] - g.c2[j]) <= (int64_t)pol->max_fresh_centroid2
                       ? DITA_FRESH : DITA_REUSE;
      } else {
        const int A = (int)cand.size();
        const int n_reuse = std::min((pol->reuse_percent * A + 50) / 100, A - 1);
        std::sort(cand.begin(), cand.end(), [&](int a, int b) {
          const int fa = std::abs(g.frame[i] - g.frame[a]);
          const int fb = std::abs(g.frame[i] - g.frame[b]);
          if (fa != fb) return fa < fb;
          const int64_t ca = std::llabs(g.c2[i] - g.c2[a]);
          const int64_t cb = std::llabs(g.c2[i] - g.c2[b]);
          if (ca != cb) return ca < cb;
          return a < b;
        });
        for (int r = 0; r < A; ++r) row[cand[r]] = r < A - n_reuse ? DITA_FRESH : DITA_REUSE;
      }
      row[i] = DITA_FRESH;   // the local partition is always computed
    }
  } else if (pol->kind == DITA_POLICY_PLANNER) {
    if (!pol->anchor)
      return fail(DITA_ERR_INVALID_ARGUMENT,
                  "a PLANNER step needs predicted errors: use a cache or dita_planner_mask");
    return planner_decide(g, pol, nullptr, valid, slot_of, true, out);
  } else {
    return fail(DITA_ERR_INVALID_ARGUMENT, "unknown policy kind %d", pol->kind);
  }
  return validate_mask(g, std::move(M), valid, slot_of, out);
}

struct Plan {
  bool planner_w = false;        // measure the importance after the step (anchor)
  bool planner_delta = false;    // measure the diagonal states' change during the step
  bool all_prior = false;        // every fresh block's slot holds a state from an earlier step
  std::vector<uint8_t> mask;
  std::vector<uint8_t> key;      // mask with covered members of merged groups marked 3
  std::vector<int32_t> fresh_ptr, fresh_cols, reuse_ptr, reuse_cols;
  std::array<int32_t, 3> counts{};
};

// Row lists of a mask.  `covered` (P*P, may be null) marks members of merged groups whose
// state is held by another slot: a REUSE of them reads that slot once, so they get no entry.
// `valid` (P*P, may be null = none) marks slots holding a state from an earlier step.
void build_lists(int P, const std::vector<uint8_t>& M, const uint8_t* covered,
                 const uint8_t* valid, Plan* p) {
  p->mask = M;
  p->key = M;
  p->fresh_ptr.assign(1, 0);
  p->reuse_ptr.assign(1, 0);
  p->fresh_cols.clear();
  p->reuse_cols.clear();
  p->counts = {0, 0, 0};
  p->all_prior = true;
  for (int i = 0; i < P; ++i) {
    for (int j = 0; j < P; ++j) {
      const size_t b = (size_t)i * P + j;
      const uint8_t m = M[b];
      p->counts[m]++;
      if (m == DITA_FRESH) {
        p->fresh_cols.push_back(j);
        if (!valid || !valid[b]) p->all_prior = false;
      }
      if (m == DITA_REUSE) {
        if (covered && covered[b]) p->key[b] = 3;
        else p->reuse_cols.push_back(j);
      }
    }
    p->fresh_ptr.push_back((int32_t)p->fresh_cols.size());
    p->reuse_ptr.push_back((int32_t)p->reuse_cols.size());
  }
}

struct Layout {
  size_t counters = 0, plans = 0, plan_bytes = 0, vt = 0, lse = 0, o = 0, delta = 0, pout = 0,
         wpart = 0, merge = 0, merge_bytes = 0, snap = 0, split_ws = 0, total = 0;
};

// Bytes of the split parts' partial merges: per part, 256 threads x (m, l, DP / 2 values).
size_t split_ws_bytes(const Geo& g) {
  return (size_t)g.num_splits * g.split_parts * 256 * (2 + g.DP / 2) * 4;
}

// The persistent part of the device buffer, as offloaded to the host: the counters, then
// the cached lse and O of every slot (the [lse, delta) span of the layout).  The rest (work
// lists, V^T, planner partials, merge jobs, snapshots) is rebuilt by the step that uses it.
size_t offload_counter_bytes(const Layout& L) { return L.plans - L.counters; }
size_t offload_state_bytes(const Layout& L) { return L.delta - L.lse; }
size_t offload_total_bytes(const Layout& L) {
  return offload_counter_bytes(L) + offload_state_bytes(L);
}

Layout compute_layout(const Geo& g, int num_slots) {
  Layout L;
  const size_t P = g.P;
  const size_t nmem = g.members.size() / 4;
  const size_t words = dita::kPlanHeader + 2 * (P + 1) + g.num_tiles + 4 * g.num_tail_wg +
                       4 * nmem + 4 * P + 2 * P * P + 2 * g.num_tail_wg * P + nmem * P +
                       g.items.size() + g.splits.size();
  L.counters = 0;
  L.plans = 256;
  L.plan_bytes = align_up(words * 4, 256);
  size_t at = L.plans + dita::kPlanSlots * L.plan_bytes;
  const size_t bh = (size_t)g.B * g.H;
  L.vt = at;
  if (g.bf16()) at = align_up(at + bh * g.DP * (size_t)g.kt_pad * 2, 256);
  L.lse = at;
  at = align_up(at + bh * num_slots * (size_t)g.slot_rows * 4, 256);
  L.o = at;
  const size_t esz = g.cache_esz();
  at = align_up(at + bh * num_slots * (size_t)g.slot_rows * g.DP * esz, 256);
  // planner measurement: per (b, h, i, 32-row sub-tile) squared changes, then the reduced
  // importance (P*P f32) and growth (P f32)
  L.delta = at;
  at = align_up(at + bh * P * (size_t)(g.slot_rows / 32) * 4, 256);
  L.pout = at;
  at = align_up(at + (P * P + P) * 4, 256);
  L.wpart = at;
  at = align_up(at + P * (size_t)dita::planner_chunks((int)P) * P * 4, 256);
  // group composition jobs: at most P * ceil(P/2) jobs of 4 words, and P*P source slots
  L.merge = at;
  L.merge_bytes = align_up((4 * P * ((P + 1) / 2) + P * P) * 4, 256);
  at += L.merge_bytes;
  // bf16: snapshot of the diagonal slots' cached O, taken before each measuring step
  L.snap = at;
  if (g.bf16()) at = align_up(at + bh * P * (size_t)g.slot_rows * g.DP * esz, 256);
  // bf16: partial merges of the split row groups' halves
  L.split_ws = at;
  at = align_up(at + split_ws_bytes(g), 256);
  L.total = at;
  return L;
}

dita_status slot_table(const Geo& g, const uint8_t* active, std::vector<int32_t>* slot_of,
                       int* num_slots) {
  const int P = g.P;
  slot_of->assign((size_t)P * P, -1);
  int n = 0;
  for (int i = 0; i < P; ++i)
    for (int j = 0; j < P; ++j)
      if (!active || active[(size_t)i * P + j]) (*slot_of)[(size_t)i * P + j] = n++;
  for (int i = 0; i < P; ++i)
    if ((*slot_of)[(size_t)i * P + i] < 0)
      return fail(DITA_ERR_POLICY, "active mask must contain the diagonal block (%d,%d)", i, i);
  *num_slots = n;
  return ok();
}

// One profiled step: events before the first kernel, between the two kernels, after.
struct TimedStep {
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  bool pending = false;
  bool two_kernels = false;
  bool fixed_ref = false;            // the step ran the fixed-reference pass
};
constexpr int kTimingRing = 64;

struct PlanSlot {
  bool used = false;
  std::vector<uint8_t> mask;
  uint64_t last_use = 0;
  hipEvent_t event = nullptr;
  bool event_recorded = false;
};

}  // namespace

struct dita_cache {
  Geo g;
  Layout L;
  std::vector<int32_t> slot_of;
  int num_slots = 0;
  uint8_t* dev = nullptr;
  size_t dev_bytes = 0;
  std::vector<uint8_t> valid;        // P*P slot holds a state
  // P*P: a merged member whose own state was dropped by a compaction (its state is its
  // group's); not a fixed softmax reference until the block is computed again
  std::vector<uint8_t> own_lost;
  std::vector<int32_t> last_fresh;   // P*P step at which the slot was written (0 = never)
  bool has_pending = false;
  Plan pending;
  // host offload: the persistent device state lives in offload_host until the restore
  bool offloaded = false;
  const void* offload_host = nullptr;
  bool has_last = false;
  Plan last;
  int64_t steps_done = 0;
  uint64_t host_fresh = 0, host_reuse = 0;
  double last_flops = 0, last_rd = 0, last_wr = 0;
  // device state, created at the first step
  bool dev_init = false;
  bool counters_init = false;        // device counters cleared (first step of either kind)
  int device = -1;
  std::vector<int32_t> host_plan;    // plan words of dita_attn_step_static (pageable memory)
  int32_t* staging = nullptr;        // pinned host, kPlanSlots * plan_bytes
  PlanSlot pslots[dita::kPlanSlots];
  uint64_t use_clock = 0;
  // profiling
  bool profiling = false;
  TimedStep timing[kTimingRing];
  int timing_next = 0;
  uint64_t profiled_steps = 0;
  double step_ms = 0, prep_ms = 0;
  uint64_t fixed_steps = 0;          // profiled steps that ran the fixed-reference pass
  double fixed_ms = 0;               // their step-kernel time
  // planner state since the last reset
  int32_t steps_since_reset = 0;
  std::vector<int32_t> fresh_step;   // P*P step since reset of the last FRESH (0 = never)
  std::vector<float> w;              // P*P importance of the last anchor
  bool have_w = false;
  std::vector<double> delta_hist;    // steps_since_reset * P: delta_i(t) (0: not measured)
  // group composition: head[i*P+j] = the block whose slot holds the state covering (i, j)
  // (j itself unless (i, j) was merged into a group headed by another block)
  std::vector<int32_t> head;
  // compaction: the slot table of the active set as allocated, and whether the cache now
  // runs on a compacted table (merged members share their group's slot)
  std::vector<int32_t> full_slot_of;
  int full_num_slots = 0;
  bool compacted = false;
  std::vector<int32_t> remap_host;   // {new slot, old slot} pairs of the last rebind
  int32_t* merge_host = nullptr;     // pinned staging of the merge jobs (L.merge_bytes)
  hipEvent_t merge_event = nullptr;
  bool merge_event_recorded = false;
  // planner measurement in flight (device -> pinned host)
  float* meas_host = nullptr;        // pinned: P*P importance, then P growth
  hipEvent_t meas_event = nullptr;
  bool meas_pending = false, meas_w = false, meas_delta = false, meas_discard = false;
  int32_t meas_step = 0;
};

namespace {

void plan_work(const dita_cache* c, const Plan& p, double* flops, double* rd, double* wr) {
  const Geo& g = c->g;
  const double bh = (double)g.B * g.H;
  const double sc = (double)g.cache_esz();
  double f = 0, r = 0, w = 0;
  for (int i = 0; i < g.P; ++i) {
    const double ni = g.offs[i + 1] - g.offs[i];
    for (int j = 0; j < g.P; ++j) {
      const uint8_t m = p.mask[(size_t)i * g.P + j];
      const double nj = g.offs[j + 1] - g.offs[j];
      if (m == DITA_FRESH) {
        f += 4.0 * ni * nj * g.D;
        w += ni * (g.D * sc + 4.0);
      }
    }
    r += (p.reuse_ptr[i + 1] - p.reuse_ptr[i]) * ni * (g.D * sc + 4.0);   // states read
  }
  *flops = f * bh;
  *rd = r * bh;
  *wr = w * bh;
}

// Device plan words for a mask.
void encode_plan(const dita_cache* c, const Plan& pl, int32_t* w) {
  const Geo& g = c->g;
  const int P = g.P;
  int at = dita::kPlanHeader;
  w[0] = g.num_tiles;
  w[1] = P;
  w[3] = g.num_tail_wg;
  for (int p = 0; p <= P; ++p) w[at + p] = g.offs[p];
  at += P + 1;
  for (int p = 0; p <= P; ++p) w[at + p] = g.poffs[p];
  at += P + 1;
  for (int k = 0; k < g.num_tail_wg; ++k) w[at++] = dita::kTailFlag | k;
  for (int i = 0; i < P; ++i)
    for (int t = 0; t < g.groups[i]; ++t) w[at++] = (i << 16) | t;
  const int packs_at = at;
  at += 4 * g.num_tail_wg;
  for (int32_t v : g.members) w[at++] = v;
  const int rows_at = at;
  int ent_at = rows_at + 4 * P;
  int e = 0;
  for (int i = 0; i < P; ++i) {
    w[rows_at + 4 * i] = e;
    for (int x = pl.fresh_ptr[i]; x < pl.fresh_ptr[i + 1]; ++x, ++e) {
      w[ent_at + 2 * e] = pl.fresh_cols[x];
      w[ent_at + 2 * e + 1] = c->slot_of[(size_t)i * P + pl.fresh_cols[x]];
    }
    for (int x = pl.reuse_ptr[i]; x < pl.reuse_ptr[i + 1]; ++x, ++e) {
      w[ent_at + 2 * e] = pl.reuse_cols[x];
      w[ent_at + 2 * e + 1] = c->slot_of[(size_t)i * P + pl.reuse_cols[x]];
    }
    w[rows_at + 4 * i + 1] = pl.fresh_ptr[i + 1] - pl.fresh_ptr[i];
    w[rows_at + 4 * i + 2] = pl.reuse_ptr[i + 1] - pl.reuse_ptr[i];
    w[rows_at + 4 * i + 3] = 0;
  }
  w[2] = e;
  // Per pack, the union of its members' fresh blocks (ascending j), each with the slot of
  // every member's block (i_m, j), or -1 where j is not fresh for member m.
  const int union_at = ent_at + 2 * P * P;
  const int slots_at = union_at + 2 * g.num_tail_wg * P;
  int nu = 0, ns = 0;
  std::vector<int32_t> slot_mj;
  for (int k = 0; k < g.num_tail_wg; ++k) {
    const int m0 = g.packs[2 * k], nm = g.packs[2 * k + 1];
    slot_mj.assign((size_t)nm * P, -1);
    std::vector<uint8_t> any(P, 0);
    for (int m = 0; m < nm; ++m) {
      const int i = g.members[4 * (m0 + m)];
      for (int x = pl.fresh_ptr[i]; x < pl.fresh_ptr[i + 1]; ++x) {
        const int j = pl.fresh_cols[x];
        any[j] = 1;
        slot_mj[(size_t)m * P + j] = c->slot_of[(size_t)i * P + j];
      }
    }
    w[packs_at + 4 * k] = m0;
    w[packs_at + 4 * k + 1] = nm;
    w[packs_at + 4 * k + 2] = nu;
    int cnt = 0;
    for (int j = 0; j < P; ++j) {
      if (!any[j]) continue;
      w[union_at + 2 * nu] = j;
      w[union_at + 2 * nu + 1] = ns;
      for (int m = 0; m < nm; ++m) w[slots_at + ns + m] = slot_mj[(size_t)m * P + j];
      ns += nm;
      ++nu;
      ++cnt;
    }
    w[packs_at + 4 * k + 3] = cnt;
  }
  int at2 = slots_at + (int)(g.members.size() / 4) * P;
  for (int32_t v : g.items) w[at2++] = v;
  for (int32_t v : g.splits) w[at2++] = v;
}

void fill_args(const dita_cache* c, int plan_slot, dita::StepArgs* a) {
  const Geo& g = c->g;
  const int P = g.P;
  a->vt = c->dev + c->L.vt;
  a->cache_o = c->dev + c->L.o;
  a->cache_lse = (float*)(c->dev + c->L.lse);
  a->counters = (unsigned long long*)(c->dev + c->L.counters);
  a->plan = (const int32_t*)(c->dev + c->L.plans + (size_t)plan_slot * c->L.plan_bytes);
  a->off_offs = dita::kPlanHeader;
  a->off_poffs = a->off_offs + P + 1;
  a->off_tiles = a->off_poffs + P + 1;
  a->off_pack = a->off_tiles + g.num_tiles;
  a->off_member = a->off_pack + 4 * g.num_tail_wg;
  a->off_rows = a->off_member + (int32_t)g.members.size();
  a->off_ent = a->off_rows + 4 * P;
  a->off_union = a->off_ent + 2 * P * P;
  a->off_pslot = a->off_union + 2 * g.num_tail_wg * P;
  a->off_items = a->off_pslot + (int32_t)(g.members.size() / 4) * P;
  a->off_splits = a->off_items + (int32_t)g.items.size();
  a->num_items = g.num_items;
  a->num_splits = g.num_splits;
  a->split_parts = g.split_parts;
  a->split_ws = (float*)(c->dev + c->L.split_ws);
  a->B = g.B; a->H = g.H; a->N = g.N; a->D = g.D; a->DP = g.DP; a->P = P;
  if (g.layout == DITA_LAYOUT_BNHD) {
    a->sB = (int64_t)g.N * g.H * g.D; a->sH = g.D; a->ld = g.H * g.D;
  } else {
    a->sB = (int64_t)g.H * g.N * g.D; a->sH = (int64_t)g.N * g.D; a->ld = g.D;
  }
  a->num_tiles = g.num_tiles;
  a->num_slots = c->num_slots;
  a->slot_rows = g.slot_rows;
  a->kt_pad = g.kt_pad;
  a->scale_log2 = g.tau * 1.4426950408889634f;
  a->delta_part = nullptr;
  a->delta_stride = g.slot_rows / 32;
  a->cache_fp8 = g.cache_o == DITA_FP8_E4M3 ? 1 : 0;
  a->fixed_ref = 0;
  a->fixup = 0;
  a->out_bf16 = g.out == DITA_BF16 ? 1 : 0;
  a->diag_snap = nullptr;
}

dita_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return DITA_OK;
  return fail(DITA_ERR_DEVICE, "%s failed: %s", what, hipGetErrorString(e));
}

dita_status device_init(dita_cache* c, hipStream_t s) {
  if (c->dev_init) return ok();
  int dev = -1;
  dita_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (st) return st;
  void* p = nullptr;
  st = hip_check(hipHostMalloc(&p, dita::kPlanSlots * c->L.plan_bytes, hipHostMallocDefault),
                 "hipHostMalloc");
  if (st) return st;
  c->staging = (int32_t*)p;
  for (auto& ps : c->pslots) {
    st = hip_check(hipEventCreateWithFlags(&ps.event, hipEventDisableTiming), "hipEventCreate");
    if (st) return st;
  }
  if (!c->counters_init) {
    st = hip_check(dita::launch_zero_counters(
                       (unsigned long long*)(c->dev + c->L.counters), 32, s),
                   "counter clear launch");
    if (st) return st;
    c->counters_init = true;
  }
  c->device = dev;
  c->dev_init = true;
  return ok();
}

// What dita_attn_step_static sets up: the device and the cleared counters, nothing allocated.
dita_status static_init(dita_cache* c, hipStream_t s) {
  if (!c->counters_init) {
    dita_status st = hip_check(dita::launch_zero_counters(
                                   (unsigned long long*)(c->dev + c->L.counters), 32, s),
                               "counter clear launch");
    if (st) return st;
    c->counters_init = true;
  }
  if (c->device < 0) {
    dita_status st = hip_check(hipGetDevice(&c->device), "hipGetDevice");
    if (st) return st;
  }
  return ok();
}

// Fold a finished profiled step into the sums.
dita_status drain_timing(dita_cache* c, TimedStep& t) {
  if (!t.pending) return ok();
  dita_status st = hip_check(hipEventSynchronize(t.ev[2]), "hipEventSynchronize");
  if (st) return st;
  float a = 0.f, b = 0.f;
  st = hip_check(hipEventElapsedTime(&a, t.ev[0], t.ev[1]), "hipEventElapsedTime");
  if (st) return st;
  st = hip_check(hipEventElapsedTime(&b, t.ev[1], t.ev[2]), "hipEventElapsedTime");
  if (st) return st;
  const double step = t.two_kernels ? b : a + b;
  if (t.two_kernels) c->prep_ms += a;
  c->step_ms += step;
  if (t.fixed_ref) {
    c->fixed_ms += step;
    ++c->fixed_steps;
  }
  ++c->profiled_steps;
  t.pending = false;
  return ok();
}

dita_status drain_all_timing(dita_cache* c) {
  for (int k = 0; k < kTimingRing; ++k) {
    dita_status st = drain_timing(c, c->timing[(c->timing_next + k) % kTimingRing]);
    if (st) return st;
  }
  return ok();
}

// Plan slot holding this mask on the device, uploading it if needed.
dita_status acquire_plan(dita_cache* c, const Plan& pl, hipStream_t s, int* slot) {
  ++c->use_clock;
  for (int k = 0; k < dita::kPlanSlots; ++k)
    if (c->pslots[k].used && c->pslots[k].mask == pl.key) {
      c->pslots[k].last_use = c->use_clock;
      *slot = k;
      return ok();
    }
  int victim = 0;
  for (int k = 0; k < dita::kPlanSlots; ++k) {
    if (!c->pslots[k].used) { victim = k; break; }
    if (c->pslots[k].last_use < c->pslots[victim].last_use) victim = k;
  }
  PlanSlot& ps = c->pslots[victim];
  if (ps.event_recorded) {
    dita_status st = hip_check(hipEventSynchronize(ps.event), "hipEventSynchronize");
    if (st) return st;
  }
  int32_t* host = (int32_t*)((uint8_t*)c->staging + (size_t)victim * c->L.plan_bytes);
  encode_plan(c, pl, host);
  uint8_t* devp = c->dev + c->L.plans + (size_t)victim * c->L.plan_bytes;
  dita_status st = hip_check(
      hipMemcpyAsync(devp, host, c->L.plan_bytes, hipMemcpyHostToDevice, s), "plan upload");
  if (st) { ps.used = false; return st; }
  ps.used = true;
  ps.mask = pl.key;
  ps.last_use = c->use_clock;
  *slot = victim;
  return ok();
}

// Fold the planner measurement of an earlier step into the host state (waits for it).
dita_status planner_sync(dita_cache* c) {
  if (!c->meas_pending) return ok();
  dita_status st = hip_check(hipEventSynchronize(c->meas_event), "hipEventSynchronize");
  if (st) return st;
  const int P = c->g.P;
  if (!c->meas_discard) {
    if (c->meas_delta)
      for (int i = 0; i < P; ++i)
        c->delta_hist[(size_t)(c->meas_step - 1) * P + i] = (double)c->meas_host[(size_t)P * P + i];
    if (c->meas_w) {
      c->w.assign(c->meas_host, c->meas_host + (size_t)P * P);
      c->have_w = true;
    }
  }
  c->meas_pending = c->meas_discard = false;
  return ok();
}

// Predicted reuse errors of step s (since the reset): E_ij = w_ij * (Cum_i(s-1) - Cum_i(f_ij)
// + delta_i(s-1)), Cum summed in step order, for blocks with a state; 0 elsewhere.
void planner_errors(const dita_cache* c, int s, std::vector<double>* E) {
  const int P = c->g.P;
  std::vector<double> cum((size_t)s * P, 0.0);   // cum[t * P + i] = Cum_i(t), t = 0..s-1
  for (int t = 1; t < s; ++t)
    for (int i = 0; i < P; ++i)
      cum[(size_t)t * P + i] = cum[(size_t)(t - 1) * P + i] + c->delta_hist[(size_t)(t - 1) * P + i];
  E->assign((size_t)P * P, 0.0);
  for (int i = 0; i < P; ++i) {
    const double last = c->delta_hist[(size_t)(s - 2) * P + i];
    for (int j = 0; j < P; ++j) {
      const size_t b = (size_t)i * P + j;
      const int f = c->fresh_step[b];
      if (!c->valid[b] || f <= 0) continue;
      const double drift = (cum[(size_t)(s - 1) * P + i] - cum[(size_t)f * P + i]) + last;
      (*E)[b] = (double)c->w[b] * drift;
    }
  }
}

}  // namespace

extern "C" {

const char* dita_version(void) { return "dita 0.1 (gfx950)"; }

const char* dita_last_error(void) { return g_err.c_str(); }

dita_status dita_partition_offsets(const dita_geometry* geom, int32_t* out) {
  if (!out) return fail(DITA_ERR_INVALID_ARGUMENT, "out is NULL");
  Geo g;
  dita_status st = resolve_geometry(geom, &g);
  if (st) return st;
  std::copy(g.offs.begin(), g.offs.end(), out);
  return ok();
}

dita_status dita_policy_mask(const dita_geometry* geom, const dita_block_policy* policy,
                             const uint8_t* valid, uint8_t* mask_out) {
  if (!mask_out) return fail(DITA_ERR_INVALID_ARGUMENT, "mask_out is NULL");
  Geo g;
  dita_status st = resolve_geometry(geom, &g);
  if (st) return st;
  std::vector<uint8_t> M;
  st = eval_policy(g, policy, valid, nullptr, &M);
  if (st) return st;
  std::memcpy(mask_out, M.data(), M.size());
  return ok();
}

dita_status dita_cache_required_bytes(const dita_geometry* geom, const uint8_t* active_mask,
                                      size_t* bytes) {
  if (!bytes) return fail(DITA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Geo g;
  dita_status st = resolve_geometry(geom, &g);
  if (st) return st;
  std::vector<int32_t> so;
  int ns = 0;
  st = slot_table(g, active_mask, &so, &ns);
  if (st) return st;
  *bytes = compute_layout(g, ns).total;
  return ok();
}

dita_status dita_cache_alloc(const dita_geometry* geom, const uint8_t* active_mask,
                             void* device_buffer, size_t buffer_bytes, dita_cache** out) {
  if (!out) return fail(DITA_ERR_INVALID_ARGUMENT, "out is NULL");
  if (!device_buffer) return fail(DITA_ERR_INVALID_ARGUMENT, "device_buffer is NULL");
  if ((uintptr_t)device_buffer % 256 != 0)
    return fail(DITA_ERR_INVALID_ARGUMENT, "device_buffer must be 256-byte aligned");
  Geo g;
  dita_status st = resolve_geometry(geom, &g);
  if (st) return st;
  std::vector<int32_t> so;
  int ns = 0;
  st = slot_table(g, active_mask, &so, &ns);
  if (st) return st;
  Layout L = compute_layout(g, ns);
  if (buffer_bytes < L.total)
    return fail(DITA_ERR_BUFFER_TOO_SMALL, "buffer holds %zu bytes, %zu needed", buffer_bytes,
                L.total);
  dita_cache* c = new (std::nothrow) dita_cache();
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "out of host memory");
  c->g = std::move(g);
  c->L = L;
  c->slot_of = std::move(so);
  c->num_slots = ns;
  c->dev = (uint8_t*)device_buffer;
  c->dev_bytes = buffer_bytes;
  c->valid.assign((size_t)c->g.P * c->g.P, 0);
  c->own_lost.assign((size_t)c->g.P * c->g.P, 0);
  c->last_fresh.assign((size_t)c->g.P * c->g.P, 0);
  c->fresh_step.assign((size_t)c->g.P * c->g.P, 0);
  c->w.assign((size_t)c->g.P * c->g.P, 0.f);
  c->head.resize((size_t)c->g.P * c->g.P);
  for (size_t b = 0; b < c->head.size(); ++b) c->head[b] = (int32_t)(b % c->g.P);
  c->host_plan.assign(L.plan_bytes / 4, 0);
  c->full_slot_of = c->slot_of;
  c->full_num_slots = ns;
  *out = c;
  return ok();
}

dita_status dita_cache_reset(dita_cache* c) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  std::fill(c->valid.begin(), c->valid.end(), 0);
  std::fill(c->last_fresh.begin(), c->last_fresh.end(), 0);
  c->has_pending = false;
  c->steps_since_reset = 0;
  std::fill(c->fresh_step.begin(), c->fresh_step.end(), 0);
  std::fill(c->w.begin(), c->w.end(), 0.f);
  c->have_w = false;
  c->delta_hist.clear();
  if (c->meas_pending) c->meas_discard = true;   // its copy may still be in flight
  // merged groups dissolve, except on a compacted table, whose members share a slot until
  // dita_cache_expand
  if (!c->compacted)
    for (size_t b = 0; b < c->head.size(); ++b) c->head[b] = (int32_t)(b % c->g.P);
  return ok();
}

dita_status dita_cache_free(dita_cache* c) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  for (auto& t : c->timing) {
    if (t.pending) (void)hipEventSynchronize(t.ev[2]);
    for (auto& e : t.ev)
      if (e) (void)hipEventDestroy(e);
  }
  if (c->dev_init) {
    for (auto& ps : c->pslots) {
      if (ps.event_recorded) (void)hipEventSynchronize(ps.event);
      if (ps.event) (void)hipEventDestroy(ps.event);
    }
    if (c->staging) (void)hipHostFree(c->staging);
  }
  if (c->meas_event) {
    (void)hipEventSynchronize(c->meas_event);
    (void)hipEventDestroy(c->meas_event);
  }
  if (c->meas_host) (void)hipHostFree(c->meas_host);
  if (c->merge_event) {
    (void)hipEventSynchronize(c->merge_event);
    (void)hipEventDestroy(c->merge_event);
  }
  if (c->merge_host) (void)hipHostFree(c->merge_host);
  delete c;
  return ok();
}

dita_status dita_set_block_policy(dita_cache* c, const dita_block_policy* policy) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!policy) return fail(DITA_ERR_INVALID_ARGUMENT, "policy is NULL");
  std::vector<uint8_t> M;
  bool meas_w = false, meas_delta = false;
  if (policy->kind == DITA_POLICY_PLANNER) {
    // DiTango planner: the previous step's measurements decide this one (waits for them)
    dita_status st = planner_sync(c);
    if (st) return st;
    const int s = c->steps_since_reset + 1;
    const int A = policy->anchor_period;
    const bool anchor = policy->anchor || s == 1 || !c->have_w ||
                        (A > 0 && (s - 1) % A == 0);
    std::vector<double> E;
    if (!anchor) planner_errors(c, s, &E);
    st = planner_decide(c->g, policy, anchor ? nullptr : E.data(), c->valid.data(),
                        c->slot_of.data(), anchor, &M);
    if (st) return st;
    meas_w = anchor;
    meas_delta = s >= 2;
  } else {
    dita_status st = eval_policy(c->g, policy, c->valid.data(), c->slot_of.data(), &M);
    if (st) return st;
  }
  // merged groups are reused or recomputed as a whole
  const int P = c->g.P;
  std::vector<uint8_t> covered((size_t)P * P, 0);
  for (int i = 0; i < P; ++i)
    for (int j = 0; j < P; ++j) {
      const size_t b = (size_t)i * P + j;
      const int h = c->head[b];
      if (h == j) continue;
      covered[b] = 1;
      const size_t hb = (size_t)i * P + h;
      if (M[b] == DITA_FRESH || M[hb] == DITA_FRESH) {
        M[b] = DITA_FRESH;
        M[hb] = DITA_FRESH;
      }
    }
  for (int i = 0; i < P; ++i)            // a second pass spreads FRESH from a head to all
    for (int j = 0; j < P; ++j) {
      const size_t b = (size_t)i * P + j;
      const size_t hb = (size_t)i * P + c->head[b];
      if (covered[b] && M[hb] == DITA_FRESH) M[b] = DITA_FRESH;
      if (covered[b] && M[b] != M[hb])
        return fail(DITA_ERR_POLICY, "block (%d,%d) is merged with (%d,%d): a merged group is "
                    "reused or recomputed as a whole", i, j, i, c->head[b]);
    }
  if (c->compacted)
    for (size_t b = 0; b < M.size(); ++b)
      if (covered[b] && M[b] == DITA_FRESH)
        return fail(DITA_ERR_POLICY, "block (%d,%d) is compacted with its group into one slot; "
                    "recomputing it needs dita_cache_expand first", (int)(b / P), (int)(b % P));
  // a fresh block's cached lse is its fixed softmax reference only while its slot holds its
  // own state
  std::vector<uint8_t> prior(c->valid);
  for (size_t b = 0; b < prior.size(); ++b)
    if (c->own_lost[b]) prior[b] = 0;
  build_lists(c->g.P, M, covered.data(), prior.data(), &c->pending);
  c->pending.planner_w = meas_w;
  c->pending.planner_delta = meas_delta;
  c->has_pending = true;
  return ok();
}

dita_status dita_get_block_plan(const dita_cache* c, uint8_t* mask, int32_t* fresh_ptr,
                                int32_t* fresh_cols, int32_t* reuse_ptr, int32_t* reuse_cols,
                                int32_t* counts) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  const Plan* p = c->has_pending ? &c->pending : (c->has_last ? &c->last : nullptr);
  if (!p) return fail(DITA_ERR_NO_POLICY, "no policy set and no step executed");
  if (mask) std::memcpy(mask, p->mask.data(), p->mask.size());
  if (fresh_ptr) std::copy(p->fresh_ptr.begin(), p->fresh_ptr.end(), fresh_ptr);
  if (fresh_cols) std::copy(p->fresh_cols.begin(), p->fresh_cols.end(), fresh_cols);
  if (reuse_ptr) std::copy(p->reuse_ptr.begin(), p->reuse_ptr.end(), reuse_ptr);
  if (reuse_cols) std::copy(p->reuse_cols.begin(), p->reuse_cols.end(), reuse_cols);
  if (counts) std::copy(p->counts.begin(), p->counts.end(), counts);
  return ok();
}

}  // extern "C"

namespace {

// Device bytes dita_attn_step_static keeps in the static scratch: the transposed-V staging
// (bf16 path), then the step's plan words, then the split halves' partial merges.
size_t static_vt_bytes(const Geo& g) {
  return g.bf16() ? align_up((size_t)g.B * g.H * g.DP * (size_t)g.kt_pad * 2, 256) : 0;
}

dita_status step_impl(dita_cache* c, const void* q, const void* k, const void* v, void* out,
                      float* lse_out, void* hip_stream, bool static_scratch) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!q || !k || !v || !out) return fail(DITA_ERR_INVALID_ARGUMENT, "q, k, v, out required");
  for (const void* p : {q, k, v, (const void*)out})
    if ((uintptr_t)p % 16 != 0)
      return fail(DITA_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
  if (lse_out && (uintptr_t)lse_out % 4 != 0)
    return fail(DITA_ERR_INVALID_ARGUMENT, "lse_out must be 4-byte aligned");
  if (c->offloaded) return fail(DITA_ERR_OFFLOADED, "the cache is offloaded; restore it first");
  if (!c->has_pending) return fail(DITA_ERR_NO_POLICY, "no block policy set for this step");
  const bool measure = c->pending.planner_w || c->pending.planner_delta;
  const size_t vt_bytes = static_vt_bytes(c->g);
  if (static_scratch) {
    if (measure)
      return fail(DITA_ERR_UNSUPPORTED, "dita_attn_step_static: a PLANNER step reads its "
                  "measurements back into host memory of the library's own; use dita_attn_step");
    const size_t ws_bytes = split_ws_bytes(c->g);
    if (vt_bytes + c->L.plan_bytes + ws_bytes > dita::kStaticScratchBytes)
      return fail(DITA_ERR_UNSUPPORTED, "dita_attn_step_static: the step needs %zu bytes of "
                  "scratch (transposed V %zu, work lists %zu, split partial merges %zu), above "
                  "the static maximum of %zu; use dita_attn_step",
                  vt_bytes + c->L.plan_bytes + ws_bytes, vt_bytes, c->L.plan_bytes, ws_bytes,
                  dita::kStaticScratchBytes);
  }
  hipStream_t s = (hipStream_t)hip_stream;
  dita_status st = ok();
  int pslot = 0;
  uint8_t* sbase = nullptr;
  if (static_scratch) {
    st = static_init(c, s);
    if (st) return st;
    void* sp = nullptr;
    st = hip_check(dita::static_scratch_address(&sp), "hipGetSymbolAddress");
    if (st) return st;
    sbase = (uint8_t*)sp;
    // the work lists go into the scratch on every call (another cache may have used it)
    encode_plan(c, c->pending, c->host_plan.data());
    st = hip_check(hipMemcpyAsync(sbase + vt_bytes, c->host_plan.data(), c->L.plan_bytes,
                                  hipMemcpyHostToDevice, s), "plan upload");
    if (st) return st;
  } else {
    st = device_init(c, s);
    if (st) return st;
    st = acquire_plan(c, c->pending, s, &pslot);
    if (st) return st;
  }
  dita::StepArgs a{};
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse_out = lse_out;
  fill_args(c, pslot, &a);
  if (static_scratch) {
    a.vt = sbase;
    a.plan = (const int32_t*)(sbase + vt_bytes);
    a.split_ws = (float*)(sbase + vt_bytes + c->L.plan_bytes);
  }
  if (measure) {
    st = planner_sync(c);   // no-op unless a measurement was never collected
    if (st) return st;
    if (!c->meas_host) {
      void* hp = nullptr;
      st = hip_check(hipHostMalloc(&hp, ((size_t)c->g.P * c->g.P + c->g.P) * 4,
                                   hipHostMallocDefault), "hipHostMalloc");
      if (st) return st;
      c->meas_host = (float*)hp;
    }
    if (!c->meas_event) {
      st = hip_check(hipEventCreateWithFlags(&c->meas_event, hipEventDisableTiming),
                     "hipEventCreate");
      if (st) return st;
    }
  }
  if (c->pending.planner_delta) a.delta_part = (float*)(c->dev + c->L.delta);
  a.fixed_ref = c->pending.all_prior ? 1 : 0;
  // a measuring bf16 step keeps the old diagonal states aside (the snapshot's grid has one
  // row per b*h: beyond 65535 the step keeps the running maximum and measures in place)
  const bool snap = c->g.bf16() && c->pending.planner_delta &&
                    (int64_t)c->g.B * c->g.H <= 65535;
  if (snap) a.diag_snap = c->dev + c->L.snap;
  TimedStep* ts = nullptr;
  if (c->profiling && !static_scratch) {
    ts = &c->timing[c->timing_next];
    st = drain_timing(c, *ts);   // the ring slot's previous step must have finished
    if (st) return st;
    for (auto& e : ts->ev)
      if (!e) {
        st = hip_check(hipEventCreate(&e), "hipEventCreate");
        if (st) return st;
      }
    st = hip_check(hipEventRecord(ts->ev[0], s), "hipEventRecord");
    if (st) return st;
  }
  if (c->g.bf16()) {
    if (snap) {
      st = hip_check(dita::launch_snapshot_diag(a, s), "snapshot launch");
      if (st) return st;
    }
    st = hip_check(dita::launch_transpose_v(a, s), "transpose launch");
    if (st) return st;
    if (ts) {
      st = hip_check(hipEventRecord(ts->ev[1], s), "hipEventRecord");
      if (st) return st;
    }
    if (snap) {
      // the step runs the plain kernels; the diagonal states' change against the snapshot is
      // measured after both of its passes
      dita::StepArgs plain = a;
      plain.delta_part = nullptr;
      st = hip_check(dita::launch_step_bf16(plain, s), "bf16 step launch");
      if (!st) st = hip_check(dita::launch_diag_change(a, s), "diag_change launch");
    } else {
      st = hip_check(dita::launch_step_bf16(a, s), "bf16 step launch");
    }
  } else {
    if (ts) {
      st = hip_check(hipEventRecord(ts->ev[1], s), "hipEventRecord");
      if (st) return st;
    }
    st = hip_check(dita::launch_step_f32(a, s), "f32 step launch");
  }
  if (st) return st;
  if (ts) {
    st = hip_check(hipEventRecord(ts->ev[2], s), "hipEventRecord");
    if (st) return st;
    ts->pending = true;
    ts->two_kernels = c->g.bf16();
    ts->fixed_ref = c->g.bf16() && a.fixed_ref && (!a.delta_part || a.diag_snap);
    c->timing_next = (c->timing_next + 1) % kTimingRing;
  }
  if (measure) {
    // planner reductions and their copy back, collected at the next PLANNER policy
    float* pout = (float*)(c->dev + c->L.pout);
    const size_t PP = (size_t)c->g.P * c->g.P;
    if (c->pending.planner_delta) {
      st = hip_check(dita::launch_planner_delta(a, pout + PP, s), "planner_delta launch");
      if (st) return st;
    }
    if (c->pending.planner_w) {
      st = hip_check(dita::launch_planner_weights(a, pout, (float*)(c->dev + c->L.wpart), s),
                     "planner_weights launch");
      if (st) return st;
    }
    st = hip_check(hipMemcpyAsync(c->meas_host, pout, (PP + c->g.P) * 4, hipMemcpyDeviceToHost,
                                  s), "planner copy");
    if (st) return st;
    st = hip_check(hipEventRecord(c->meas_event, s), "hipEventRecord");
    if (st) return st;
  }
  if (!static_scratch) {
    st = hip_check(hipEventRecord(c->pslots[pslot].event, s), "hipEventRecord");
    if (st) return st;
    c->pslots[pslot].event_recorded = true;
  }
  // bookkeeping (only after every enqueue succeeded)
  ++c->steps_done;
  ++c->steps_since_reset;
  const size_t PP = (size_t)c->g.P * c->g.P;
  for (size_t b = 0; b < PP; ++b)
    if (c->pending.mask[b] == DITA_FRESH) {
      c->valid[b] = 1;
      c->own_lost[b] = 0;
      c->last_fresh[b] = (int32_t)c->steps_done;
      c->fresh_step[b] = c->steps_since_reset;
      c->head[b] = (int32_t)(b % c->g.P);      // recomputed: its own state again
    }
  c->delta_hist.resize((size_t)c->steps_since_reset * c->g.P, 0.0);
  if (measure) {
    c->meas_pending = true;
    c->meas_discard = false;
    c->meas_w = c->pending.planner_w;
    c->meas_delta = c->pending.planner_delta;
    c->meas_step = c->steps_since_reset;
  }
  const uint64_t bh = (uint64_t)c->g.B * c->g.H;
  c->host_fresh += bh * (uint64_t)c->pending.counts[DITA_FRESH];
  c->host_reuse += bh * (uint64_t)c->pending.reuse_cols.size();
  plan_work(c, c->pending, &c->last_flops, &c->last_rd, &c->last_wr);
  c->last = std::move(c->pending);
  c->has_last = true;
  c->has_pending = false;
  return ok();
}

}  // namespace

extern "C" {

dita_status dita_attn_step(dita_cache* c, const void* q, const void* k, const void* v,
                           void* out, float* lse_out, void* hip_stream) {
  return step_impl(c, q, k, v, out, lse_out, hip_stream, false);
}

dita_status dita_attn_step_static(dita_cache* c, const void* q, const void* k, const void* v,
                                  void* out, float* lse_out, void* hip_stream) {
  return step_impl(c, q, k, v, out, lse_out, hip_stream, true);
}

dita_status dita_cache_read_slot(dita_cache* c, int32_t b, int32_t h, int32_t i, int32_t j,
                                 float* o_out, float* lse_out, void* hip_stream) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (c->offloaded) return fail(DITA_ERR_OFFLOADED, "the cache is offloaded; restore it first");
  const Geo& g = c->g;
  if (b < 0 || b >= g.B || h < 0 || h >= g.H || i < 0 || i >= g.P || j < 0 || j >= g.P)
    return fail(DITA_ERR_INVALID_ARGUMENT, "slot index out of range");
  if (!o_out || !lse_out) return fail(DITA_ERR_INVALID_ARGUMENT, "o_out and lse_out required");
  const size_t blk = (size_t)i * g.P + j;
  if (c->slot_of[blk] < 0) return fail(DITA_ERR_POLICY, "block (%d,%d) has no slot", i, j);
  if (!c->valid[blk]) return fail(DITA_ERR_CACHE_MISS, "slot (%d,%d) holds no state", i, j);
  dita::StepArgs a{};
  fill_args(c, 0, &a);
  const size_t hblk = (size_t)i * g.P + c->head[blk];   // a merged group's state
  return hip_check(dita::launch_read_slot(a, b * g.H + h, c->slot_of[hblk],
                                          g.offs[i + 1] - g.offs[i], o_out, lse_out,
                                          (int)g.cache_esz(), (hipStream_t)hip_stream),
                   "read_slot launch");
}

dita_status dita_set_profiling(dita_cache* c, int32_t enable) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (enable) {
    dita_status st = drain_all_timing(c);
    if (st) return st;
    c->profiled_steps = 0;
    c->step_ms = c->prep_ms = 0;
    c->fixed_steps = 0;
    c->fixed_ms = 0;
  }
  c->profiling = enable != 0;
  return ok();
}

dita_status dita_cache_merge_groups(dita_cache* c, int32_t group, const uint8_t* select,
                                    int32_t* merged, void* hip_stream) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (group < 2) return fail(DITA_ERR_INVALID_ARGUMENT, "group must be >= 2");
  if (c->offloaded) return fail(DITA_ERR_OFFLOADED, "the cache is offloaded; restore it first");
  if (c->has_pending)
    return fail(DITA_ERR_INVALID_ARGUMENT, "merge between steps, before the next policy is set");
  if ((int64_t)c->g.B * c->g.H > 65535 || c->g.slot_rows / 32 > 65535)
    return fail(DITA_ERR_UNSUPPORTED, "group composition supports B*H and rows/32 up to 65535");
  const int P = c->g.P;
  const int NG = (P + group - 1) / group;
  std::vector<int32_t> jobs, srcs;
  std::vector<std::pair<size_t, int32_t>> heads_new;   // (block, new head)
  std::vector<int> members, hs;
  for (int i = 0; i < P; ++i) {
    const int n_i = c->g.offs[i + 1] - c->g.offs[i];
    for (int J = 0; J < NG; ++J) {
      const int j0 = J * group, j1 = std::min(P, j0 + group);
      if (i >= j0 && i < j1) continue;                 // holds the always-fresh diagonal
      if (select && !select[(size_t)i * NG + J]) continue;
      members.clear();
      hs.clear();
      bool ok_group = true;
      for (int j = j0; j < j1; ++j) {
        const size_t b = (size_t)i * P + j;
        if (c->slot_of[b] < 0) continue;
        if (!c->valid[b]) { ok_group = false; break; }
        const int h = c->head[b];
        if (h < j0 || h >= j1) { ok_group = false; break; }   // part of a wider group
        members.push_back(j);
        if (std::find(hs.begin(), hs.end(), h) == hs.end()) hs.push_back(h);
      }
      if (!ok_group || hs.size() < 2) continue;
      // a state inside J must not also cover blocks outside J
      for (int j = 0; j < P && ok_group; ++j)
        if ((j < j0 || j >= j1) &&
            std::find(hs.begin(), hs.end(), c->head[(size_t)i * P + j]) != hs.end())
          ok_group = false;
      if (!ok_group) continue;
      std::sort(hs.begin(), hs.end());
      const int dst = members.front();                 // first active member: a head itself
      jobs.push_back(n_i);
      jobs.push_back(c->slot_of[(size_t)i * P + dst]);
      jobs.push_back((int32_t)srcs.size());
      jobs.push_back((int32_t)hs.size());
      for (int h : hs) srcs.push_back(c->slot_of[(size_t)i * P + h]);
      for (int j : members) heads_new.push_back({(size_t)i * P + j, dst});
    }
  }
  const int njobs = (int)(jobs.size() / 4);
  if (merged) *merged = njobs;
  if (njobs == 0) return ok();
  hipStream_t s = (hipStream_t)hip_stream;
  dita_status st = device_init(c, s);
  if (st) return st;
  if (!c->merge_host) {
    void* hp = nullptr;
    st = hip_check(hipHostMalloc(&hp, c->L.merge_bytes, hipHostMallocDefault), "hipHostMalloc");
    if (st) return st;
    c->merge_host = (int32_t*)hp;
    st = hip_check(hipEventCreateWithFlags(&c->merge_event, hipEventDisableTiming),
                   "hipEventCreate");
    if (st) return st;
  }
  if (c->merge_event_recorded) {                        // the staging of the previous merge
    st = hip_check(hipEventSynchronize(c->merge_event), "hipEventSynchronize");
    if (st) return st;
  }
  std::copy(jobs.begin(), jobs.end(), c->merge_host);
  std::copy(srcs.begin(), srcs.end(), c->merge_host + jobs.size());
  int32_t* dev = (int32_t*)(c->dev + c->L.merge);
  st = hip_check(hipMemcpyAsync(dev, c->merge_host, (jobs.size() + srcs.size()) * 4,
                                hipMemcpyHostToDevice, s), "merge job upload");
  if (st) return st;
  dita::StepArgs a{};
  fill_args(c, 0, &a);
  st = hip_check(dita::launch_merge_slots(a, dev, dev + jobs.size(), njobs,
                                          (int)c->g.cache_esz(), s),
                 "merge_slots launch");
  if (st) return st;
  st = hip_check(hipEventRecord(c->merge_event, s), "hipEventRecord");
  if (st) return st;
  c->merge_event_recorded = true;
  for (const auto& hb : heads_new) c->head[hb.first] = hb.second;
  return ok();
}

dita_status dita_planner_mask(const dita_geometry* geom, const dita_block_policy* policy,
                              const double* error, const uint8_t* valid, uint8_t* mask_out) {
  if (!policy || !mask_out) return fail(DITA_ERR_INVALID_ARGUMENT, "policy and mask_out required");
  if (policy->kind != DITA_POLICY_PLANNER)
    return fail(DITA_ERR_INVALID_ARGUMENT, "policy kind must be PLANNER");
  Geo g;
  dita_status st = resolve_geometry(geom, &g);
  if (st) return st;
  std::vector<uint8_t> M;
  st = planner_decide(g, policy, policy->anchor ? nullptr : error, valid, nullptr,
                      policy->anchor != 0, &M);
  if (st) return st;
  std::memcpy(mask_out, M.data(), M.size());
  return ok();
}

dita_status dita_get_planner_state(dita_cache* c, float* w, double* delta, int32_t* fresh_step,
                                   int32_t* steps) {
  if (!c || !steps) return fail(DITA_ERR_INVALID_ARGUMENT, "cache and steps required");
  dita_status st = planner_sync(c);
  if (st) return st;
  *steps = c->steps_since_reset;
  if (w) std::copy(c->w.begin(), c->w.end(), w);
  if (delta) std::copy(c->delta_hist.begin(), c->delta_hist.end(), delta);
  if (fresh_step) std::copy(c->fresh_step.begin(), c->fresh_step.end(), fresh_step);
  return ok();
}

dita_status dita_cache_offload_bytes(const dita_cache* c, size_t* bytes) {
  if (!c || !bytes) return fail(DITA_ERR_INVALID_ARGUMENT, "cache and bytes required");
  *bytes = offload_total_bytes(c->L);
  return ok();
}

dita_status dita_cache_offload(dita_cache* c, void* host_dst, size_t host_bytes,
                               void* hip_stream) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (c->offloaded) return fail(DITA_ERR_INVALID_ARGUMENT, "the cache is already offloaded");
  if (!host_dst) return fail(DITA_ERR_INVALID_ARGUMENT, "host_dst is NULL");
  const size_t need = offload_total_bytes(c->L);
  if (host_bytes < need)
    return fail(DITA_ERR_INVALID_ARGUMENT, "host_dst holds %zu bytes, %zu needed", host_bytes,
                need);
  hipStream_t s = (hipStream_t)hip_stream;
  uint8_t* h = (uint8_t*)host_dst;
  dita_status st = hip_check(hipMemcpyAsync(h, c->dev + c->L.counters,
                                            offload_counter_bytes(c->L),
                                            hipMemcpyDeviceToHost, s), "offload copy");
  if (st) return st;
  st = hip_check(hipMemcpyAsync(h + offload_counter_bytes(c->L), c->dev + c->L.lse,
                                offload_state_bytes(c->L), hipMemcpyDeviceToHost, s),
                 "offload copy");
  if (st) return st;
  c->offloaded = true;
  c->offload_host = host_dst;
  return ok();
}

dita_status dita_cache_restore(dita_cache* c, void* device_buffer, size_t buffer_bytes,
                               const void* host_src, size_t host_bytes, void* hip_stream) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (!c->offloaded) return fail(DITA_ERR_INVALID_ARGUMENT, "the cache is not offloaded");
  if (!device_buffer || !host_src)
    return fail(DITA_ERR_INVALID_ARGUMENT, "device_buffer and host_src required");
  if ((uintptr_t)device_buffer % 256 != 0)
    return fail(DITA_ERR_INVALID_ARGUMENT, "device_buffer must be 256-byte aligned");
  if (buffer_bytes < c->L.total)
    return fail(DITA_ERR_BUFFER_TOO_SMALL, "buffer holds %zu bytes, %zu needed", buffer_bytes,
                c->L.total);
  const size_t need = offload_total_bytes(c->L);
  if (host_bytes < need)
    return fail(DITA_ERR_INVALID_ARGUMENT, "host_src holds %zu bytes, %zu needed", host_bytes,
                need);
  if (c->device >= 0) {
    int dev = -1;
    dita_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (st) return st;
    if (dev != c->device)
      return fail(DITA_ERR_INVALID_ARGUMENT, "restore on device %d, the cache ran on device %d",
                  dev, c->device);
  }
  hipStream_t s = (hipStream_t)hip_stream;
  uint8_t* d = (uint8_t*)device_buffer;
  const uint8_t* h = (const uint8_t*)host_src;
  dita_status st = hip_check(hipMemcpyAsync(d + c->L.counters, h, offload_counter_bytes(c->L),
                                            hipMemcpyHostToDevice, s), "restore copy");
  if (st) return st;
  st = hip_check(hipMemcpyAsync(d + c->L.lse, h + offload_counter_bytes(c->L),
                                offload_state_bytes(c->L), hipMemcpyHostToDevice, s),
                 "restore copy");
  if (st) return st;
  c->dev = d;
  c->dev_bytes = buffer_bytes;
  // the uploaded work lists lived in the old buffer
  for (auto& ps : c->pslots) ps.used = false;
  c->offloaded = false;
  c->offload_host = nullptr;
  return ok();
}

}  // extern "C"

namespace {

// Move the cache onto another slot table in a new device buffer: the counters, and for each
// {new slot, old slot} pair the stored state, copied device to device on the stream.
dita_status rebind_slots(dita_cache* c, std::vector<int32_t> new_slot_of, int new_slots,
                         const std::vector<int32_t>& pairs, void* device_buffer,
                         size_t buffer_bytes, void* hip_stream, bool compacted) {
  if (!device_buffer) return fail(DITA_ERR_INVALID_ARGUMENT, "device_buffer is NULL");
  if ((uintptr_t)device_buffer % 256 != 0)
    return fail(DITA_ERR_INVALID_ARGUMENT, "device_buffer must be 256-byte aligned");
  const Layout NL = compute_layout(c->g, new_slots);
  if (buffer_bytes < NL.total)
    return fail(DITA_ERR_BUFFER_TOO_SMALL, "buffer holds %zu bytes, %zu needed", buffer_bytes,
                NL.total);
  if ((uint8_t*)device_buffer < c->dev + c->dev_bytes &&
      c->dev < (uint8_t*)device_buffer + buffer_bytes)
    return fail(DITA_ERR_INVALID_ARGUMENT, "the new buffer overlaps the cache's buffer");
  if ((int64_t)c->g.B * c->g.H > 65535)
    return fail(DITA_ERR_UNSUPPORTED, "compaction supports B*H up to 65535");
  if (c->device >= 0) {
    int dev = -1;
    dita_status st = hip_check(hipGetDevice(&dev), "hipGetDevice");
    if (st) return st;
    if (dev != c->device)
      return fail(DITA_ERR_INVALID_ARGUMENT, "rebind on device %d, the cache ran on device %d",
                  dev, c->device);
  }
  hipStream_t s = (hipStream_t)hip_stream;
  uint8_t* nd = (uint8_t*)device_buffer;
  dita_status st = hip_check(hipMemcpyAsync(nd + NL.counters, c->dev + c->L.counters,
                                            offload_counter_bytes(c->L),
                                            hipMemcpyDeviceToDevice, s), "counter copy");
  if (st) return st;
  const int npairs = (int)(pairs.size() / 2);
  if (npairs > 0) {
    // the pairs go through the new buffer's work-list area, rebuilt by the next step
    c->remap_host = pairs;
    int32_t* map = (int32_t*)(nd + NL.plans);
    st = hip_check(hipMemcpyAsync(map, c->remap_host.data(), pairs.size() * 4,
                                  hipMemcpyHostToDevice, s), "slot map upload");
    if (st) return st;
    st = hip_check(dita::launch_remap_slots(
                       (const float*)(c->dev + c->L.lse), c->dev + c->L.o,
                       (float*)(nd + NL.lse), nd + NL.o, map, npairs, c->g.B * c->g.H,
                       c->num_slots, new_slots, c->g.slot_rows,
                       (size_t)c->g.slot_rows * c->g.DP * c->g.cache_esz(), s),
                   "remap_slots launch");
    if (st) return st;
  }
  c->slot_of = std::move(new_slot_of);
  c->num_slots = new_slots;
  c->L = NL;
  c->dev = nd;
  c->dev_bytes = buffer_bytes;
  c->compacted = compacted;
  for (auto& ps : c->pslots) ps.used = false;   // work lists held the old slot numbers
  return ok();
}

dita_status rebind_checks(const dita_cache* c) {
  if (!c) return fail(DITA_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (c->offloaded) return fail(DITA_ERR_OFFLOADED, "the cache is offloaded; restore it first");
  if (c->has_pending)
    return fail(DITA_ERR_INVALID_ARGUMENT, "rebind between steps, before the next policy is set");
  return ok();
}

// Slots of the compacted table: the active blocks that hold their own state (each merged
// group once, at its head), in row-major order.
int compact_slots(const dita_cache* c, std::vector<int32_t>* new_slot_of,
                  std::vector<int32_t>* pairs) {
  const int P = c->g.P;
  if (new_slot_of) new_slot_of->assign((size_t)P * P, -1);
  int n = 0;
  for (size_t b = 0; b < (size_t)P * P; ++b) {
    if (c->full_slot_of[b] < 0 || c->head[b] != (int32_t)(b % P)) continue;
    if (new_slot_of) (*new_slot_of)[b] = n;
    if (pairs && c->valid[b]) {
      pairs->push_back(n);
      pairs->push_back(c->slot_of[b]);
    }
    ++n;
  }
  if (new_slot_of)
    for (size_t b = 0; b < (size_t)P * P; ++b)
      if (c->full_slot_of[b] >= 0 && c->head[b] != (int32_t)(b % P))
        (*new_slot_of)[b] = (*new_slot_of)[(b / P) * P + c->head[b]];
  return n;
}

}  // namespace

extern "C" {

dita_status dita_cache_compact_bytes(const dita_cache* c, size_t* bytes) {
  if (!c || !bytes) return fail(DITA_ERR_INVALID_ARGUMENT, "cache and bytes required");
  *bytes = compute_layout(c->g, compact_slots(c, nullptr, nullptr)).total;
  return ok();
}

dita_status dita_cache_compact(dita_cache* c, void* device_buffer, size_t buffer_bytes,
                               void* hip_stream) {
  dita_status st = rebind_checks(c);
  if (st) return st;
  std::vector<int32_t> slot_of, pairs;
  const int n = compact_slots(c, &slot_of, &pairs);
  st = rebind_slots(c, std::move(slot_of), n, pairs, device_buffer, buffer_bytes, hip_stream,
                    true);
  if (st) return st;
  // merged members now share their group's slot: their own states are gone
  const int P = c->g.P;
  for (size_t b = 0; b < c->head.size(); ++b)
    if (c->head[b] != (int32_t)(b % P)) c->own_lost[b] = 1;
  return ok();
}

dita_status dita_cache_expand(dita_cache* c, void* device_buffer, size_t buffer_bytes,
                              void* hip_stream) {
  dita_status st = rebind_checks(c);
  if (st) return st;
  if (!c->compacted) return fail(DITA_ERR_INVALID_ARGUMENT, "the cache is not compacted");
  const int P = c->g.P;
  std::vector<int32_t> pairs;
  for (size_t b = 0; b < (size_t)P * P; ++b)
    if (c->full_slot_of[b] >= 0 && c->head[b] == (int32_t)(b % P) && c->valid[b]) {
      pairs.push_back(c->full_slot_of[b]);
      pairs.push_back(c->slot_of[b]);
    }
  return rebind_slots(c, c->full_slot_of, c->full_num_slots, pairs, device_buffer, buffer_bytes,
                      hip_stream, false);
}

dita_status dita_get_stats(const dita_cache* cc, dita_step_stats* s) {
  if (!cc || !s) return fail(DITA_ERR_INVALID_ARGUMENT, "cache and stats required");
  dita_cache* c = const_cast<dita_cache*>(cc);   // draining timing events updates sums only
  dita_status dst = drain_all_timing(c);
  if (dst) return dst;
  std::memset(s, 0, sizeof *s);
  s->steps_done = c->steps_done;
  if (c->has_last)
    for (int k = 0; k < 3; ++k) s->last_counts[k] = c->last.counts[k];
  s->host_fresh_blocks = c->host_fresh;
  s->host_reuse_blocks = c->host_reuse;
  s->last_fresh_flops = c->last_flops;
  s->last_cache_read_bytes = c->last_rd;
  s->last_cache_write_bytes = c->last_wr;
  s->profiled_steps = c->profiled_steps;
  s->step_kernel_ms = c->step_ms;
  s->prep_kernel_ms = c->prep_ms;
  s->fixed_ref_steps = c->fixed_steps;
  s->fixed_ref_kernel_ms = c->fixed_ms;
  if (c->counters_init) {
    unsigned long long cnt[4] = {0, 0, 0, 0};
    dita_status st = hip_check(hipDeviceSynchronize(), "hipDeviceSynchronize");
    if (st) return st;
    if (c->offloaded) {
      std::memcpy(cnt, c->offload_host, sizeof cnt);   // the offload copy has completed
    } else {
      st = hip_check(hipMemcpy(cnt, c->dev + c->L.counters, sizeof cnt, hipMemcpyDeviceToHost),
                     "counter read");
      if (st) return st;
    }
    s->device_fresh_blocks = cnt[0];
    s->device_reuse_blocks = cnt[1];
    s->device_v_range_errors = cnt[2];
    s->device_ref_recomputes = cnt[3];
  }
  return ok();
}

}  // extern "C"
