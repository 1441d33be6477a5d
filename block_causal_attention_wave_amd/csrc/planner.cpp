// Host-side wave planner.
//
// Context policies phi(j, r) and the two schedules follow the streaming video
// diffusion design-space paper (thelatestinai.com listing of arXiv
// 2609.22283): Table 1 defines clean / same-level / progressive history,
// Figure 2 contrasts serial rounds (B*K) with pipelined rounds at staggered
// levels (B+K-1).  Refresh passes that make a finished chunk's clean K/V are
// separate forward passes (Wave Forcing summary on aiany.app, opening
// paragraph and Key Findings).
//
// Algorithm (all linear passes over chunk-major node order):
//   1. which chunks need a refresh node: a descending sweep over chunks, since
//      only later chunks (or their refreshes) read a chunk's clean slot;
//   2. pipelined rounds as a longest-path recurrence over the dependency DAG:
//      round(n) = max(admission i, previous node of the chunk + 1,
//                     writer round of each read slot, + 1 if the writer is
//                     not a lower chunk);
//      serial rounds in closed form, then checked against the same rules;
//   3. physical slots: a slot is released after its last reading round; a
//      min-heap hands out the lowest released id, else a new one.
#include "planner.hpp"

#include <algorithm>
#include <cstdio>
#include <functional>
#include <queue>

namespace wave {
namespace {

struct SlotKey {
  int32_t chunk, level;
};

struct NodeI {
  int32_t chunk, level, kind, round;
  std::vector<SlotKey> reads;
  std::vector<SlotKey> writes;
};

int32_t phi(int32_t policy, int32_t j, int32_t r) {
  switch (policy) {
    case WAVE_CLEAN: return 0;
    case WAVE_SAME_LEVEL: return j;
    default: return j - r > 0 ? j - r : 0;  // progressive
  }
}

bool fail(std::string* err, const char* msg) {
  if (err) *err = msg;
  return false;
}

}  // namespace

int32_t build_plan(const wave_plan_params& pin, Plan& out, std::string* err) {
  wave_plan_params p = pin;
  if (p.q_tile == 0) p.q_tile = WAVE_Q_TILE;
  if (p.query_len == 0) p.query_len = p.chunk_len;
  if (p.B < 1 || p.K < 1 || p.B > (1 << 16) || p.K > (1 << 12)) {
    fail(err, "wave_plan: need 1 <= B <= 65536 and 1 <= K <= 4096");
    return WAVE_ERR_INVALID_ARG;
  }
  if (p.policy < WAVE_CLEAN || p.policy > WAVE_PROGRESSIVE) {
    fail(err, "wave_plan: unknown policy");
    return WAVE_ERR_INVALID_ARG;
  }
  if (p.sched != WAVE_SCHED_SERIAL && p.sched != WAVE_SCHED_WAVE) {
    fail(err, "wave_plan: unknown schedule");
    return WAVE_ERR_INVALID_ARG;
  }
  if (p.history_cap < -1 || p.chunk_len < 1 || p.cond_len < 0 || p.q_tile < 1 || p.query_len < 1) {
    fail(err, "wave_plan: need history_cap >= -1, chunk_len >= 1, cond_len >= 0, q_tile >= 0, query_len >= 0");
    return WAVE_ERR_INVALID_ARG;
  }
  if (static_cast<int64_t>(p.B) * (p.K + 1) > (1 << 24)) {
    fail(err, "wave_plan: too many nodes");
    return WAVE_ERR_INVALID_ARG;
  }
  const int32_t B = p.B, K = p.K;
  const bool cond = p.cond_len > 0;
  auto window = [&](int32_t i) { return p.history_cap < 0 ? i : std::min(i, p.history_cap); };
  auto slot_index = [&](SlotKey s) { return static_cast<int64_t>(s.chunk) * (K + 2) + (s.level + 1); };
  const int64_t num_slot_keys = static_cast<int64_t>(B) * (K + 2);

  // 1. Refresh need, from the last chunk down.
  std::vector<char> need(B, 0);
  for (int32_t c = B - 1; c >= 0; --c) {
    for (int32_t i = c + 1; i < B && !need[c]; ++i) {
      const int32_t r = i - c;
      if (r > window(i)) break;  // window(i) - r only shrinks as i grows past the cap
      if (need[i]) need[c] = 1;
      for (int32_t j = 1; j <= K && !need[c]; ++j)
        if (phi(p.policy, j, r) == 0) need[c] = 1;
    }
  }

  // Nodes in chunk-major order.
  std::vector<NodeI> nodes;
  nodes.reserve(static_cast<size_t>(B) * (K + 1));
  auto make_reads = [&](int32_t i, int32_t level) {
    std::vector<SlotKey> v;
    for (int32_t r = window(i); r >= 1; --r) {
      if (cond) v.push_back({i - r, WAVE_LEVEL_COND});
      v.push_back({i - r, phi(p.policy, level, r)});  // phi(0, r) == 0 for refresh
    }
    if (cond) v.push_back({i, WAVE_LEVEL_COND});
    v.push_back({i, level});
    return v;
  };
  for (int32_t i = 0; i < B; ++i) {
    for (int32_t j = K; j >= 1; --j) {
      NodeI n{i, j, WAVE_NODE_UPDATE, -1, make_reads(i, j), {}};
      if (j == K && cond) n.writes.push_back({i, WAVE_LEVEL_COND});
      n.writes.push_back({i, j});
      nodes.push_back(std::move(n));
    }
    if (need[i]) nodes.push_back(NodeI{i, 0, WAVE_NODE_REFRESH, -1, make_reads(i, 0), {{i, 0}}});
  }

  // 2. Rounds.
  std::vector<int32_t> w_round(num_slot_keys, -1), w_chunk(num_slot_keys, -1);
  auto is_own = [](const NodeI& n, SlotKey s) {
    for (auto& w : n.writes)
      if (w.chunk == s.chunk && w.level == s.level) return true;
    return false;
  };
  int32_t prev_chunk = -1, prev_round = -1;
  for (auto& n : nodes) {
    if (n.chunk != prev_chunk) prev_round = -1;
    int32_t t;
    if (p.sched == WAVE_SCHED_WAVE) {
      t = std::max(n.chunk, prev_round + 1);
      for (auto& s : n.reads) {
        if (is_own(n, s)) continue;
        const int64_t k = slot_index(s);
        if (w_round[k] < 0) {
          fail(err, "wave_plan: internal error, read of an unwritten slot");
          return WAVE_ERR_INVALID_ARG;
        }
        t = std::max(t, w_chunk[k] < n.chunk ? w_round[k] : w_round[k] + 1);
      }
    } else {
      t = n.kind == WAVE_NODE_UPDATE ? n.chunk * K + (K - n.level) : (n.chunk + 1) * K;
      if (t <= prev_round) {
        fail(err, "wave_plan: internal error, serial order");
        return WAVE_ERR_INVALID_ARG;
      }
      for (auto& s : n.reads) {
        if (is_own(n, s)) continue;
        const int64_t k = slot_index(s);
        if (w_round[k] < 0 || !(w_round[k] < t || (w_round[k] == t && w_chunk[k] < n.chunk))) {
          fail(err, "wave_plan: internal error, serial schedule reads too early");
          return WAVE_ERR_INVALID_ARG;
        }
      }
    }
    n.round = t;
    for (auto& s : n.writes) {
      w_round[slot_index(s)] = t;
      w_chunk[slot_index(s)] = n.chunk;
    }
    prev_chunk = n.chunk;
    prev_round = t;
  }
  int32_t num_rounds = 0;
  for (auto& n : nodes) num_rounds = std::max(num_rounds, n.round + 1);

  // Group by round; inside a round, ascending chunk (chunk-major order is
  // already ascending, a stable sort by round keeps it).
  std::vector<int32_t> order(nodes.size());
  for (size_t k = 0; k < order.size(); ++k) order[k] = static_cast<int32_t>(k);
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return nodes[a].round < nodes[b].round; });

  // 3. Physical slots.
  std::vector<int32_t> last_read(num_slot_keys, -1);
  for (auto& n : nodes)
    for (auto& s : n.reads) last_read[slot_index(s)] = std::max(last_read[slot_index(s)], n.round);
  std::vector<std::vector<int64_t>> release_at(num_rounds + 1);
  std::vector<int32_t> phys(num_slot_keys, -1);
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_ids;
  int32_t next_id = 0;
  size_t pos = 0;
  for (int32_t t = 0; t < num_rounds; ++t) {
    for (int64_t k : release_at[t]) free_ids.push(phys[k]);
    for (; pos < order.size() && nodes[order[pos]].round == t; ++pos) {
      for (auto& s : nodes[order[pos]].writes) {
        const int64_t k = slot_index(s);
        int32_t id;
        if (!free_ids.empty()) {
          id = free_ids.top();
          free_ids.pop();
        } else {
          id = next_id++;
        }
        phys[k] = id;
        release_at[last_read[k] + 1].push_back(k);
      }
    }
  }

  // Flat arrays.
  Plan pl;
  pl.params = p;
  pl.num_phys_slots = next_id;
  pl.max_slot_len = std::max(p.chunk_len, p.cond_len);
  auto len_of = [&](SlotKey s) { return s.level == WAVE_LEVEL_COND ? p.cond_len : p.chunk_len; };
  pl.round_node_begin.assign(num_rounds + 1, 0);
  pl.round_write_begin.assign(num_rounds + 1, 0);
  pl.round_work_begin.assign(num_rounds + 1, 0);
  pl.round_q_rows.assign(num_rounds, 0);
  pl.round_src_rows.assign(num_rounds, 0);
  pos = 0;
  for (int32_t t = 0; t < num_rounds; ++t) {
    pl.round_node_begin[t] = static_cast<int32_t>(pl.nodes.size());
    pl.round_write_begin[t] = static_cast<int32_t>(pl.writes.size());
    int64_t q_off = 0, src_off = 0;
    const size_t first_node = pl.nodes.size();
    for (; pos < order.size() && nodes[order[pos]].round == t; ++pos) {
      const NodeI& n = nodes[order[pos]];
      wave_node v{};
      v.chunk = n.chunk;
      v.level = n.level;
      v.kind = n.kind;
      v.round = t;
      v.q_offset = static_cast<int32_t>(q_off);
      v.q_len = p.query_len;
      v.ctx_begin = static_cast<int32_t>(pl.ctx.size());
      v.ctx_count = static_cast<int32_t>(n.reads.size());
      v.write_begin = static_cast<int32_t>(pl.writes.size());
      v.write_count = static_cast<int32_t>(n.writes.size());
      for (auto& s : n.reads) pl.ctx.push_back({s.chunk, s.level, phys[slot_index(s)], len_of(s)});
      for (auto& s : n.writes) {
        pl.writes.push_back({s.chunk, s.level, phys[slot_index(s)], len_of(s)});
        src_off += len_of(s);
      }
      q_off += p.query_len;
      pl.max_ctx = std::max(pl.max_ctx, v.ctx_count);
      pl.nodes.push_back(v);
    }
    if (q_off > INT32_MAX || src_off > INT32_MAX) {
      fail(err, "wave_plan: a round's packed rows exceed int32");
      return WAVE_ERR_INVALID_ARG;
    }
    pl.round_q_rows[t] = static_cast<int32_t>(q_off);
    pl.round_src_rows[t] = static_cast<int32_t>(src_off);
    // Work items, most expensive first.
    const size_t w0 = pl.work.size();
    for (size_t ni = first_node; ni < pl.nodes.size(); ++ni) {
      const wave_node& v = pl.nodes[ni];
      int64_t keys = 0;
      for (int32_t c = 0; c < v.ctx_count; ++c) keys += pl.ctx[v.ctx_begin + c].len;
      if (keys > INT32_MAX) {
        fail(err, "wave_plan: context longer than int32");
        return WAVE_ERR_INVALID_ARG;
      }
      for (int32_t q0 = 0; q0 < v.q_len; q0 += p.q_tile)
        pl.work.push_back({static_cast<int32_t>(ni), q0, std::min(p.q_tile, v.q_len - q0),
                           static_cast<int32_t>(keys)});
    }
    auto key_tiles = [&](const wave_work& w) {
      const wave_node& v = pl.nodes[w.node];
      int64_t tiles = 0;
      for (int32_t c = 0; c < v.ctx_count; ++c)
        tiles += (pl.ctx[v.ctx_begin + c].len + WAVE_KEY_TILE - 1) / WAVE_KEY_TILE;
      return tiles;
    };
    std::stable_sort(pl.work.begin() + w0, pl.work.end(), [&](const wave_work& a, const wave_work& b) {
      const int64_t ta = key_tiles(a), tb = key_tiles(b);
      if (ta != tb) return ta > tb;
      return a.q_rows > b.q_rows;
    });
  }
  pl.round_node_begin[num_rounds] = static_cast<int32_t>(pl.nodes.size());
  pl.round_write_begin[num_rounds] = static_cast<int32_t>(pl.writes.size());
  // round_work_begin from the per-round work ranges
  {
    size_t k = 0;
    for (int32_t t = 0; t < num_rounds; ++t) {
      pl.round_work_begin[t] = static_cast<int32_t>(k);
      while (k < pl.work.size() && pl.nodes[pl.work[k].node].round == t) ++k;
    }
    pl.round_work_begin[num_rounds] = static_cast<int32_t>(pl.work.size());
  }
  for (int32_t t = 0; t < num_rounds; ++t) {
    if (pl.round_node_begin[t] == pl.round_node_begin[t + 1]) {
      fail(err, "wave_plan: internal error, empty round");
      return WAVE_ERR_INVALID_ARG;
    }
  }

  // Descriptor.
  const int32_t nr = num_rounds, nn = static_cast<int32_t>(pl.nodes.size());
  const int32_t nc = static_cast<int32_t>(pl.ctx.size()), nw = static_cast<int32_t>(pl.writes.size());
  const int32_t nk = static_cast<int32_t>(pl.work.size());
  const int64_t off_round = kDescHeader;
  const int64_t off_node = off_round + static_cast<int64_t>(nr) * kRoundStride;
  const int64_t off_ctx = off_node + static_cast<int64_t>(nn) * kNodeStride;
  const int64_t off_write = off_ctx + static_cast<int64_t>(nc) * kCtxStride;
  const int64_t off_work = off_write + static_cast<int64_t>(nw) * kWriteStride;
  const int64_t total = off_work + static_cast<int64_t>(nk) * kWorkStride;
  if (total > INT32_MAX) {
    fail(err, "wave_plan: descriptor too large");
    return WAVE_ERR_INVALID_ARG;
  }
  pl.desc.assign(static_cast<size_t>(total), 0);
  int32_t* d = pl.desc.data();
  d[0] = kDescMagic;
  d[1] = kDescVersion;
  d[2] = nr;
  d[3] = nn;
  d[4] = nc;
  d[5] = nw;
  d[6] = nk;
  d[7] = static_cast<int32_t>(off_round);
  d[8] = static_cast<int32_t>(off_node);
  d[9] = static_cast<int32_t>(off_ctx);
  d[10] = static_cast<int32_t>(off_write);
  d[11] = static_cast<int32_t>(off_work);
  for (int32_t t = 0; t < nr; ++t) {
    int32_t* r = d + off_round + static_cast<int64_t>(t) * kRoundStride;
    r[0] = pl.round_node_begin[t];
    r[1] = pl.round_node_begin[t + 1];
    r[2] = pl.round_write_begin[t];
    r[3] = pl.round_write_begin[t + 1];
    r[4] = pl.round_work_begin[t];
    r[5] = pl.round_work_begin[t + 1];
    r[6] = pl.round_q_rows[t];
    r[7] = pl.round_src_rows[t];
  }
  for (int32_t k = 0; k < nn; ++k) {
    int32_t* r = d + off_node + static_cast<int64_t>(k) * kNodeStride;
    r[0] = pl.nodes[k].q_offset;
    r[1] = pl.nodes[k].q_len;
    r[2] = pl.nodes[k].ctx_begin;
    r[3] = pl.nodes[k].ctx_count;
    r[4] = pl.nodes[k].chunk;
    r[5] = pl.nodes[k].level;
  }
  for (int32_t k = 0; k < nc; ++k) {
    int32_t* r = d + off_ctx + static_cast<int64_t>(k) * kCtxStride;
    r[0] = pl.ctx[k].phys_slot;
    r[1] = pl.ctx[k].len;
  }
  for (int32_t t = 0; t < nr; ++t) {
    int32_t src = 0;
    for (int32_t k = pl.round_write_begin[t]; k < pl.round_write_begin[t + 1]; ++k) {
      int32_t* r = d + off_write + static_cast<int64_t>(k) * kWriteStride;
      r[0] = pl.writes[k].phys_slot;
      r[1] = pl.writes[k].len;
      r[2] = src;
      src += pl.writes[k].len;
    }
  }
  for (int32_t k = 0; k < nk; ++k) {
    int32_t* r = d + off_work + static_cast<int64_t>(k) * kWorkStride;
    r[0] = pl.work[k].node;
    r[1] = pl.work[k].q_start;
    r[2] = pl.work[k].q_rows;
  }
  out = std::move(pl);
  return WAVE_OK;
}

}  // namespace wave
