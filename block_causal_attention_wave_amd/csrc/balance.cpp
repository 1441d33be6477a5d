// Tail balancing of one attention round: choice of the items to cut.
#include "balance.hpp"

#include <algorithm>
#include <functional>
#include <queue>
#include <vector>

#include "wave.h"

namespace wave {
namespace {

// Cost model, in units of one 64-key tile of one workgroup.
constexpr double kStartTiles = 3.0;    // Q load, gather-list staging, first tile's latency
constexpr double kPieceTiles = 1.0;    // writing a piece's fp32 partial rows
constexpr double kTileSeconds = 1.7e-6;  // one tile of a head_dim-128 workgroup on one compute unit
constexpr double kMergeBytesPerSecond = 4.0e12;
constexpr double kLaunchSeconds = 5.0e-6;

// Key tiles of each work item of the round, in dispatch order.
std::vector<int64_t> item_tiles(const Plan& p, int32_t round) {
  std::vector<int64_t> out;
  for (int32_t i = p.round_work_begin[round]; i < p.round_work_begin[round + 1]; ++i) {
    const wave_node& n = p.nodes[p.work[i].node];
    int64_t t = 0;
    for (int32_t e = 0; e < n.ctx_count; ++e) t += (p.ctx[n.ctx_begin + e].len + WAVE_KEY_TILE - 1) / WAVE_KEY_TILE;
    out.push_back(t);
  }
  return out;
}

double simulate(const std::vector<int64_t>& tiles, int32_t heads, int32_t cus, const TailSplit& t) {
  std::priority_queue<double, std::vector<double>, std::greater<double>> free_at;
  for (int32_t c = 0; c < cus; ++c) free_at.push(0.0);
  double end = 0.0;
  auto run = [&](double cost) {
    const double s = free_at.top();
    free_at.pop();
    free_at.push(s + cost);
    end = std::max(end, s + cost);
  };
  const size_t n = tiles.size(), direct = n - static_cast<size_t>(t.items);
  for (size_t i = 0; i < direct; ++i)
    for (int32_t h = 0; h < heads; ++h) run(kStartTiles + static_cast<double>(tiles[i]));
  for (size_t i = direct; i < n; ++i) {
    const int64_t per = (tiles[i] + t.splits - 1) / t.splits;
    for (int32_t h = 0; h < heads; ++h)
      for (int32_t s = 0; s < t.splits; ++s) {
        const int64_t first = std::min<int64_t>(tiles[i], s * per);
        const int64_t len = std::min<int64_t>(tiles[i], first + per) - first;
        run(kStartTiles + kPieceTiles + static_cast<double>(len));
      }
  }
  return end;
}

}  // namespace

double simulate_round(const Plan& p, int32_t round, int32_t heads, int32_t cus, const TailSplit& t) {
  return simulate(item_tiles(p, round), heads, std::max(cus, 1), t);
}

int32_t choose_splits(const Plan& p, int32_t round, int32_t heads, int32_t head_dim, int32_t cus) {
  (void)head_dim;
  const std::vector<int64_t> tiles = item_tiles(p, round);
  const int64_t n = static_cast<int64_t>(tiles.size());
  if (n == 0 || heads < 1 || cus < 1) return 1;
  // Split-KV items are short query blocks: a workgroup does little arithmetic
  // per key tile and streams its range from HBM, so the round costs its bytes
  // at the chip's streaming rate, plus one workgroup start-up (gather list,
  // then the first tile's latency) per dispatch wave, plus the merge.  A
  // second wave pays that start-up again and a partly filled one leaves units
  // idle, so the count that fills the compute units exactly once wins.
  const int64_t longest = *std::max_element(tiles.begin(), tiles.end());
  const int64_t s = std::min<int64_t>({static_cast<int64_t>(cus) / (n * heads), longest, 64});
  return static_cast<int32_t>(std::max<int64_t>(s, 1));
}

TailSplit choose_tail_split(const Plan& p, int32_t round, int32_t heads, int32_t head_dim, int32_t cus) {
  const std::vector<int64_t> tiles = item_tiles(p, round);
  const int32_t n = static_cast<int32_t>(tiles.size());
  TailSplit best;
  if (n == 0 || heads < 1 || cus < 1) return best;
  double best_t = simulate(tiles, heads, cus, best);
  // Tile time scales with head_dim; the merge reads every piece's fp32 rows.
  const double tile_s = kTileSeconds * head_dim / 128.0;
  std::vector<int32_t> cands;
  for (int32_t m : {1, 2, 3, 4, 5, 6, 8, 10, 12, 14, 16, 20, 24, 28, 32, 40, 48, 64})
    if (m < n) cands.push_back(m);
  cands.push_back(n);
  for (int32_t m : cands)
    for (int32_t s = 2; s <= 4; ++s) {
      const TailSplit t{m, s};
      const double merge_bytes = static_cast<double>(s) * m * WAVE_Q_TILE * heads * head_dim * 4.0;
      const double merge = (merge_bytes / kMergeBytesPerSecond + kLaunchSeconds) / tile_s;
      const double v = simulate(tiles, heads, cus, t) + merge;
      if (v < best_t) {
        best_t = v;
        best = t;
      }
    }
  return best;
}

}  // namespace wave
