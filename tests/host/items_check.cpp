// Host check of the bf16 step's workgroup list (build_items in dita_host.cpp, compiled into
// this translation unit): every (b, h) tile appears exactly once, as one workgroup or as the
// adjacent parts of a split row group inside one XCD range; the kernel's hardware-to-logical
// remap is a bijection on the list; every XCD range holds the same number of split groups;
// and the split count follows its rule (an eighth of an XCD's concurrent workgroups from two
// rounds on, none for smaller grids, DITA_SPLITS_PER_XCD and DITA_SPLIT_PARTS when set).
// Exit status 0 when every case holds.
#include "dita_host.cpp"

#include <cstdio>
#include <cstdlib>
#include <map>

namespace {

int xcd_remap_host(int bid, int G) {            // the kernel's xcd_remap
  const int xcd = bid & 7, idx = bid >> 3, per = G >> 3, rem = G & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

int check(int B, int H, int frames, int gh, int gw, int P, int D, int want_per_xcd,
          int want_parts = 2) {
  dita_geometry g{};
  g.batch = B; g.heads = H; g.tokens = frames * gh * gw; g.head_dim = D;
  g.frames = frames; g.grid_h = gh; g.grid_w = gw; g.num_partitions = P;
  g.qkv_dtype = DITA_BF16; g.cache_o_dtype = DITA_BF16; g.layout = DITA_LAYOUT_BHND;
  g.out_dtype = DITA_F32;
  Geo r;
  if (resolve_geometry(&g, &r)) {
    printf("resolve failed: %s\n", dita_last_error());
    return 1;
  }
  const long G0 = (long)B * H * r.num_tiles;
  const int G = r.num_items;
  int bad = 0;
  const int NP = r.split_parts;
  if (NP != want_parts) bad |= 512;
  if ((long)G != G0 + (long)r.num_splits * (NP - 1)) bad |= 1;
  std::vector<int> seen(G, 0);
  for (int b = 0; b < G; ++b) {
    const int l = xcd_remap_host(b, G);
    if (l < 0 || l >= G || seen[l]++) bad |= 2;
  }
  std::map<std::pair<int, int>, int> cnt;
  std::vector<int> parts(r.num_splits, 0);
  for (int x = 0; x < G; ++x) {
    const int bh = r.items[2 * x], w = r.items[2 * x + 1];
    if (w & dita::kSplitFlag) {
      const int s = (w & ~dita::kSplitFlag) >> 3, h = w & 7;
      if (r.splits[2 * s] != bh) bad |= 4;
      parts[s] |= 1 << h;
      if (h > 0 && (x == 0 || r.items[2 * x - 1] != (dita::kSplitFlag | (s << 3) | (h - 1))))
        bad |= 8;
      if (h == 0) cnt[{bh, r.splits[2 * s + 1]}]++;
    } else {
      cnt[{bh, w}]++;
    }
  }
  for (int s = 0; s < r.num_splits; ++s)
    if (parts[s] != (1 << NP) - 1) bad |= 16;
  for (int bh = 0; bh < B * H; ++bh) {
    for (int k = 0; k < r.num_tail_wg; ++k)
      if (cnt[{bh, dita::kTailFlag | k}] != 1) bad |= 32;
    for (int i = 0; i < r.P; ++i)
      for (int t = 0; t < r.groups[i]; ++t)
        if (cnt[{bh, (i << 16) | t}] != 1) bad |= 32;
  }
  if ((long)cnt.size() != G0) bad |= 64;
  const int per = G >> 3, rem = G & 7;
  auto range_of = [&](int l) {
    for (int x = 0; x < 8; ++x) {
      const int lo = x * per + std::min(x, rem), hi = lo + per + (x < rem ? 1 : 0);
      if (l >= lo && l < hi) return x;
    }
    return -1;
  };
  int per_range[8] = {0};
  for (int x = 0; x < G; ++x) {
    const int w = r.items[2 * x + 1];
    if ((w & dita::kSplitFlag) && (w & 7) == 0) {
      if (range_of(x) != range_of(x + NP - 1)) bad |= 128;
      per_range[range_of(x)]++;
    }
  }
  for (int x = 0; x < 8; ++x)
    if (per_range[x] != want_per_xcd) bad |= 256;
  printf("B%d H%d N%d P%d D%d: tiles/bh %d tails %d G0 %ld splits %d x %d parts (%d per XCD, "
         "want %d) -> %s (%d)\n", B, H, g.tokens, P, D, r.num_tiles, r.num_tail_wg, G0,
         r.num_splits, NP, per_range[0], want_per_xcd, bad ? "BAD" : "ok", bad);
  return bad ? 1 : 0;
}

}  // namespace

int main() {
  int bad = 0;
  unsetenv("DITA_SPLITS_PER_XCD");
  unsetenv("DITA_SPLIT_PARTS");
  bad += check(1, 24, 8, 45, 80, 32, 64, 12);    // 29 frames of 720p: 5472 workgroups
  bad += check(2, 40, 17, 26, 60, 16, 128, 8);   // CFG long video, D = 128
  bad += check(1, 24, 24, 45, 80, 24, 64, 12);   // 93 frames
  bad += check(3, 11, 13, 30, 40, 29, 96, 8);    // D = 96, tails in every partition
  bad += check(1, 16, 4, 32, 32, 8, 72, 0);      // 512 workgroups: one round, no splits
  bad += check(1, 3, 8, 10, 6, 5, 128, 0);
  bad += check(1, 7, 9, 33, 17, 37, 64, 0);
  bad += check(1, 1, 4, 16, 16, 64, 64, 0);      // tails only
  bad += check(1, 2, 4, 4, 4, 64, 64, 0);
  setenv("DITA_SPLITS_PER_XCD", "2", 1);
  bad += check(1, 3, 4, 20, 26, 8, 64, 2);       // 51 workgroups, 2 split per range
  bad += check(1, 1, 4, 4, 4, 64, 64, 0);        // tails only: nothing to split
  bad += check(1, 24, 8, 45, 80, 32, 64, 2);
  setenv("DITA_SPLITS_PER_XCD", "0", 1);
  bad += check(1, 24, 8, 45, 80, 32, 64, 0);
  setenv("DITA_SPLITS_PER_XCD", "1000", 1);
  bad += check(1, 24, 8, 45, 80, 32, 64, dita::kMaxSplits / 8);
  unsetenv("DITA_SPLITS_PER_XCD");
  setenv("DITA_SPLIT_PARTS", "4", 1);
  bad += check(1, 24, 8, 45, 80, 32, 64, 12, 4);
  bad += check(2, 40, 17, 26, 60, 16, 128, 8, 4);
  setenv("DITA_SPLITS_PER_XCD", "2", 1);
  setenv("DITA_SPLIT_PARTS", "3", 1);
  bad += check(1, 3, 4, 20, 26, 8, 64, 2, 3);
  setenv("DITA_SPLIT_PARTS", "99", 1);
  bad += check(1, 3, 4, 20, 26, 8, 64, 2, dita::kMaxSplitParts);
  return bad ? 1 : 0;
}
