// planner.cpp -- host min-call planner and packed-round layout.
//
// Call model (HARTS, thelatestinai.com Figure 2 and Figure C.1(b); devfeed.tech
// abstract on the linear-time minimum-call planner):
//   * One round = one packed call of independent sequences.  A sequence starts
//     at a B-aligned trajectory position from a state that already exists, then
//     runs contiguous tokens down one root-to-leaf path, so each of its chunks is
//     a chunk of that trajectory's own B-aligned grid.
//   * Each internal segment continues exactly one child in its own sequence.
//     Every other child c (fork position p = start of c) is side-started at
//     b = B*floor(p/B): it replays r = p - b < B rows of its ancestors without
//     writing outputs.  It may run in the round of its parent's sequence when b
//     equals the position that sequence started at (the state it needs is that
//     sequence's own initial state); otherwise the state at b is produced by the
//     parent's sequence and the child waits for the next round.
//   * Two-mode dynamic program over the tree, children before parents: mode A
//     means the sequence holding v is still inside its head chunk at v's end, so
//     side children cost no extra round; mode B costs one.  The continuation is
//     the child with the largest side cost; ties go to the larger subtree token
//     count, then to the smaller segment id.  Linear in the number of segments.
//   * Sequences of a round are ordered by their head segment id; handoff buffers
//     by (producer sequence, position).
#include <algorithm>
#include <climits>
#include <map>
#include <utility>

#include "plan.h"

namespace kda {

namespace {

struct Chain {
  int32_t head = -1;
  int32_t round = 0;
  int64_t b_head = 0;
  int32_t init_kind = 0;   // 0 = root h0, 1 = buffer
  int32_t init_a = 0;      // root index, or producer chain (pre-order id)
  int64_t init_b = 0;      // buffer position
  std::vector<int32_t> members;
};

inline int64_t floor_div(int64_t a, int64_t b) { return a / b; }  // a >= 0

}  // namespace

int build_plan(int32_t n_seg, const int32_t* parent, const int32_t* seg_len,
               const int64_t* seg_row, int32_t B, int32_t mode, Plan& P, std::string& err) {
  if (n_seg <= 0 || parent == nullptr || seg_len == nullptr) {
    err = "n_seg must be positive and parent/seg_len non-null";
    return -4;
  }
  if (B <= 0) {
    err = "chunk size must be positive";
    return -4;
  }
  if (mode < 0 || mode > 4) {
    err = "unknown mode";
    return -4;
  }
  const bool exact = mode == 2 || mode == 3;   // side branches start from exact fork states
  const bool mincall = mode == 0 || mode == 4; // replay side starts, minimum rounds
  const bool shortc = mode == 4;               // drop continuations that cost no round
  const int32_t n = n_seg;
  P = Plan();
  P.mode = mode;
  P.B = B;
  P.n_seg = n;

  // ---- validate and build children lists (ascending ids) ----
  std::vector<int32_t> child_ptr(n + 1, 0), child_list;
  std::vector<int32_t> roots;
  int64_t n_rows = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (seg_len[i] <= 0) {
      err = "segment " + std::to_string(i) + " has non-positive length";
      return -1;
    }
    int32_t p = parent[i];
    if (p < -1 || p >= n || p == i) {
      err = "segment " + std::to_string(i) + " has an invalid parent";
      return -1;
    }
    if (p < 0) roots.push_back(i); else child_ptr[p + 1]++;
    n_rows += seg_len[i];
  }
  if (roots.empty()) {
    err = "tree has no root";
    return -1;
  }
  if (n_rows >= (int64_t)INT32_MAX) {
    err = "too many rows";
    return -1;
  }
  for (int32_t i = 0; i < n; ++i) child_ptr[i + 1] += child_ptr[i];
  child_list.assign(child_ptr[n], 0);
  {
    std::vector<int32_t> fill(child_ptr.begin(), child_ptr.end() - 1);
    for (int32_t i = 0; i < n; ++i)
      if (parent[i] >= 0) child_list[fill[parent[i]]++] = i;
  }
  auto nchild = [&](int32_t v) { return child_ptr[v + 1] - child_ptr[v]; };

  // pre-order: roots ascending, children ascending
  std::vector<int32_t> order;
  order.reserve(n);
  {
    std::vector<char> seen(n, 0);
    std::vector<int32_t> stack(roots.rbegin(), roots.rend());
    while (!stack.empty()) {
      int32_t v = stack.back();
      stack.pop_back();
      if (seen[v]) {
        err = "segment reached twice";
        return -1;
      }
      seen[v] = 1;
      order.push_back(v);
      for (int32_t j = child_ptr[v + 1] - 1; j >= child_ptr[v]; --j) stack.push_back(child_list[j]);
    }
    if ((int32_t)order.size() != n) {
      err = "parent links contain a cycle";
      return -1;
    }
  }

  // rows: default is id order; otherwise the ranges must tile [0, N)
  std::vector<int64_t> row0(n);
  if (seg_row == nullptr) {
    int64_t acc = 0;
    for (int32_t i = 0; i < n; ++i) { row0[i] = acc; acc += seg_len[i]; }
  } else {
    std::vector<std::pair<int64_t, int32_t>> rs(n);
    for (int32_t i = 0; i < n; ++i) rs[i] = {seg_row[i], i};
    std::sort(rs.begin(), rs.end());
    int64_t acc = 0;
    for (auto& pr : rs) {
      if (pr.first != acc) {
        err = "seg_row ranges do not tile the row space";
        return -1;
      }
      acc += seg_len[pr.second];
    }
    for (int32_t i = 0; i < n; ++i) row0[i] = seg_row[i];
  }

  std::vector<int64_t> s(n), e(n);
  for (int32_t v : order) {
    s[v] = parent[v] < 0 ? 0 : e[parent[v]];
    e[v] = s[v] + seg_len[v];
  }
  std::vector<int32_t> root_index(n, -1);
  for (size_t i = 0; i < roots.size(); ++i) root_index[roots[i]] = (int32_t)i;
  std::vector<int32_t> root_of(n);
  for (int32_t v : order) root_of[v] = parent[v] < 0 ? v : root_of[parent[v]];
  std::vector<int32_t> leaf_index(n, -1);
  for (int32_t i = 0; i < n; ++i)
    if (nchild(i) == 0) { leaf_index[i] = (int32_t)P.leaf_seg.size(); P.leaf_seg.push_back(i); }
  P.root_seg = roots;
  P.n_root = (int32_t)roots.size();
  P.n_leaf = (int32_t)P.leaf_seg.size();
  P.n_rows = n_rows;
  P.seg_start = s;
  P.seg_end = e;
  // occurrence count of every compact row: the trajectories through it, i.e.
  // the leaves below its segment (children follow parents in pre-order)
  {
    std::vector<int32_t> below(n, 0);
    for (auto it = order.rbegin(); it != order.rend(); ++it) {
      const int32_t v = *it;
      if (nchild(v) == 0) below[v] = 1;
      if (parent[v] >= 0) below[parent[v]] += below[v];
    }
    P.row_mult.assign(n_rows, 0);
    for (int32_t v = 0; v < n; ++v)
      for (int64_t t = 0; t < seg_len[v]; ++t) P.row_mult[row0[v] + t] = below[v];
  }

  // compact row of trajectory position `pos` on the root path of segment v
  auto row_at = [&](int32_t v, int64_t pos) -> int32_t {
    while (s[v] > pos) v = parent[v];
    return (int32_t)(row0[v] + (pos - s[v]));
  };

  std::vector<Chain> chains;
  std::vector<int32_t> chain_of(n, -1);
  int64_t R = 0;

  if (mincall) {
    // ---- two-mode DP (children before parents) ----
    std::vector<int64_t> sub(n);
    for (int32_t i = 0; i < n; ++i) sub[i] = seg_len[i];
    for (int32_t i = n - 1; i >= 0; --i) {
      int32_t v = order[i];
      if (parent[v] >= 0) sub[parent[v]] += sub[v];
    }
    std::vector<int32_t> gA(n, 0), gB(n, 0), cont(n, -1);
    auto head_mode_is_A = [&](int32_t c) { return floor_div(e[c], B) == floor_div(s[c], B); };
    for (int32_t i = n - 1; i >= 0; --i) {
      int32_t v = order[i];
      if (nchild(v) == 0) continue;
      int32_t best = -1, best_side = -1;
      int32_t top1 = INT_MIN, top2 = INT_MIN;  // two largest side bases
      for (int32_t j = child_ptr[v]; j < child_ptr[v + 1]; ++j) {
        int32_t c = child_list[j];
        int32_t base = head_mode_is_A(c) ? gA[c] : gB[c];
        if (base > top1) { top2 = top1; top1 = base; } else if (base > top2) { top2 = base; }
        bool better = best < 0 || base > best_side || (base == best_side && sub[c] > sub[best]) ||
                      (base == best_side && sub[c] == sub[best] && c < best);
        if (better) { best = c; best_side = base; }
      }
      cont[v] = best;
      // the largest side base among the other children
      int32_t other = (nchild(v) >= 2) ? (best_side == top1 ? top2 : top1) : INT_MIN;
      bool same_chunk = head_mode_is_A(best);
      int32_t cA = same_chunk ? gA[best] : gB[best];
      int32_t cB = gB[best];
      gA[v] = std::max(cA, other == INT_MIN ? 0 : other);
      gB[v] = std::max(cB, other == INT_MIN ? 0 : other + 1);
      // short-chain variant: side-starting every child costs no round in
      // either mode -> continue none (G unchanged, sequences end sooner)
      if (shortc && top1 == gA[v] && top1 + 1 == gB[v]) cont[v] = -1;
    }
    int32_t rounds = 0;
    for (int32_t r : roots) {
      int32_t g = (e[r] < B) ? gA[r] : gB[r];
      rounds = std::max(rounds, 1 + g);
    }

    // ---- chains with as-soon-as-possible rounds ----
    for (int32_t v : order) {
      int32_t p = parent[v];
      if (p < 0) {
        Chain c;
        c.head = v; c.round = 0; c.b_head = 0; c.init_kind = 0; c.init_a = root_index[v];
        chain_of[v] = (int32_t)chains.size();
        chains.push_back(c);
      } else if (cont[p] == v) {
        chain_of[v] = chain_of[p];
      } else {
        const Chain& S = chains[chain_of[p]];
        int64_t b = B * floor_div(s[v], B);
        R += s[v] - b;
        Chain c;
        c.head = v; c.b_head = b;
        if (b == S.b_head) {
          c.round = S.round; c.init_kind = S.init_kind; c.init_a = S.init_a; c.init_b = S.init_b;
        } else {
          c.round = S.round + 1; c.init_kind = 1; c.init_a = chain_of[p]; c.init_b = b;
        }
        chain_of[v] = (int32_t)chains.size();
        chains.push_back(c);
      }
      chains[chain_of[v]].members.push_back(v);
    }
    int32_t maxr = 0;
    for (auto& c : chains) maxr = std::max(maxr, c.round);
    if (maxr + 1 != rounds) {
      err = "internal: planner round count mismatch";
      return -1;
    }
    P.n_rounds = rounds;
  } else if (exact) {
    // ---- exact-state starts: no replay ----
    // A side branch starts at its own first position from the state that the
    // sequence holding its parent emits there, one round after that
    // sequence's round.  No-replay mode keeps the continuation structure,
    // chosen by a one-mode DP (every side start costs one round):
    // G(v) = max(G(cont), max over the other children of 1 + G(c)), the
    // continuation being the child of largest G (ties: larger subtree, then
    // smaller id).  Node-wise mode has no continuations: one sequence per
    // segment, rounds by depth.
    std::vector<int32_t> cont(n, -1);
    if (mode == 2) {
      std::vector<int64_t> sub(n);
      for (int32_t i = 0; i < n; ++i) sub[i] = seg_len[i];
      for (int32_t i = n - 1; i >= 0; --i) {
        int32_t v = order[i];
        if (parent[v] >= 0) sub[parent[v]] += sub[v];
      }
      std::vector<int32_t> G(n, 0);
      for (int32_t i = n - 1; i >= 0; --i) {
        int32_t v = order[i];
        if (nchild(v) == 0) continue;
        int32_t best = -1;
        for (int32_t j = child_ptr[v]; j < child_ptr[v + 1]; ++j) {
          int32_t c = child_list[j];
          bool better = best < 0 || G[c] > G[best] || (G[c] == G[best] && sub[c] > sub[best]) ||
                        (G[c] == G[best] && sub[c] == sub[best] && c < best);
          if (better) best = c;
        }
        cont[v] = best;
        int32_t gv = G[best];
        for (int32_t j = child_ptr[v]; j < child_ptr[v + 1]; ++j)
          if (child_list[j] != best) gv = std::max(gv, 1 + G[child_list[j]]);
        G[v] = gv;
      }
    }
    for (int32_t v : order) {
      int32_t p = parent[v];
      if (p >= 0 && cont[p] == v) {
        chain_of[v] = chain_of[p];
      } else {
        Chain c;
        c.head = v;
        if (p < 0) {
          c.round = 0; c.b_head = 0; c.init_kind = 0; c.init_a = root_index[v];
        } else {
          c.round = chains[chain_of[p]].round + 1;
          c.b_head = s[v];
          c.init_kind = 1; c.init_a = chain_of[p]; c.init_b = s[v];
        }
        chain_of[v] = (int32_t)chains.size();
        chains.push_back(c);
      }
      chains[chain_of[v]].members.push_back(v);
    }
    int32_t maxr = 0;
    for (auto& c : chains) maxr = std::max(maxr, c.round);
    P.n_rounds = maxr + 1;
  } else {
    // ---- expanded: one sequence per trajectory ----
    for (int32_t li = 0; li < P.n_leaf; ++li) {
      Chain c;
      int32_t l = P.leaf_seg[li];
      c.head = root_of[l]; c.round = 0; c.b_head = 0; c.init_kind = 0; c.init_a = root_index[root_of[l]];
      std::vector<int32_t> path;
      for (int32_t v = l; v >= 0; v = parent[v]) path.push_back(v);
      c.members.assign(path.rbegin(), path.rend());
      chains.push_back(c);
    }
    P.n_rounds = 1;
  }
  P.R = R;

  // ---- sequence order: (round, head id); expanded keeps leaf order ----
  const int32_t nc = (int32_t)chains.size();
  std::vector<int32_t> seq_order(nc);
  for (int32_t i = 0; i < nc; ++i) seq_order[i] = i;
  if (mode != 1)
    std::sort(seq_order.begin(), seq_order.end(), [&](int32_t a, int32_t b) {
      if (chains[a].round != chains[b].round) return chains[a].round < chains[b].round;
      return chains[a].head < chains[b].head;
    });
  std::vector<int32_t> seq_of_chain(nc);
  for (int32_t i = 0; i < nc; ++i) seq_of_chain[seq_order[i]] = i;

  // handoff buffers keyed by (producer sequence, position)
  std::map<std::pair<int32_t, int64_t>, int32_t> buf_id;
  for (int32_t ci = 0; ci < nc; ++ci)
    if (chains[ci].init_kind == 1) buf_id[{seq_of_chain[chains[ci].init_a], chains[ci].init_b}] = 0;
  {
    int32_t k = 0;
    for (auto& kv : buf_id) kv.second = k++;
  }
  const int32_t nbuf = (int32_t)buf_id.size();

  // ---- per-segment exports ----
  P.seg_round.assign(n, 0); P.seg_seq.assign(n, -1); P.seg_is_cont.assign(n, 0);
  P.seg_b.assign(n, -1); P.seg_replay.assign(n, 0);
  if (mode != 1) {
    for (int32_t v = 0; v < n; ++v) {
      const Chain& c = chains[chain_of[v]];
      P.seg_round[v] = c.round;
      P.seg_seq[v] = seq_of_chain[chain_of[v]];
      bool is_head = c.head == v;
      P.seg_is_cont[v] = (!is_head) ? 1 : 0;
      if (is_head) {
        P.seg_b[v] = (int32_t)c.b_head;
        P.seg_replay[v] = (int32_t)(s[v] - c.b_head);
      }
    }
  }

  // ---- sequences, packed rows, chunks ----
  P.round_seq_ptr.assign(P.n_rounds + 1, 0);
  P.seq_row_ptr.push_back(0);
  P.seq_chunk_ptr.push_back(0);
  int64_t packed = 0;
  int32_t rep_slots = 0;
  for (int32_t si = 0; si < nc; ++si) {
    const Chain& c = chains[seq_order[si]];
    P.round_seq_ptr[c.round + 1]++;
    int32_t leaf = c.members.back();
    int64_t r = (mode != 1) ? (s[c.head] - c.b_head) : 0;
    P.seq_round.push_back(c.round);
    P.seq_head.push_back(c.head);
    P.seq_leaf.push_back(leaf_index[leaf]);   // -1: a node-wise sequence ending at an inner segment
    P.seq_b_head.push_back((int32_t)c.b_head);
    P.seq_replay.push_back((int32_t)r);
    P.seq_init_kind.push_back(c.init_kind);
    P.seq_init_idx.push_back(c.init_kind == 0 ? c.init_a
                                              : buf_id.at({seq_of_chain[c.init_a], c.init_b}));
    int64_t base = packed;
    // replay rows: positions [b_head, s_head) on the head's root path
    for (int64_t pos = c.b_head; pos < c.b_head + r; ++pos) {
      P.row_index.push_back(row_at(parent[c.head], pos));
      P.out_row.push_back(-1);
    }
    for (int32_t v : c.members)
      for (int32_t t = 0; t < seg_len[v]; ++t) {
        int32_t crow = (int32_t)(row0[v] + t);
        P.row_index.push_back(crow);
        P.out_row.push_back(-2);  // filled below
      }
    int64_t len = (int64_t)P.row_index.size() - base;
    packed += len;
    if (packed >= (int64_t)INT32_MAX) {
      err = "too many packed rows";
      return -1;
    }
    for (int64_t j = r; j < len; ++j)
      P.out_row[base + j] = (mode != 1) ? P.row_index[base + j] : (int32_t)(base + j);
    P.seq_row_ptr.push_back((int32_t)packed);
    // chunks: the sequence's own B-grid from its start; with exact-state
    // starts the grid is also cut at every position a side branch starts from
    std::vector<int64_t> cuts;
    if (exact)
      for (auto it = buf_id.lower_bound({si, INT64_MIN}); it != buf_id.end() && it->first.first == si; ++it)
        cuts.push_back(it->first.second - c.b_head);
    for (int64_t c0 = 0, ci = 0; c0 < len;) {
      int64_t nxt = std::min<int64_t>(len, (c0 / B + 1) * B);
      while (ci < (int64_t)cuts.size() && cuts[ci] <= c0) ++ci;
      if (ci < (int64_t)cuts.size() && cuts[ci] < nxt) nxt = cuts[ci];
      int32_t L = (int32_t)(nxt - c0);
      P.chunk_seq.push_back(si);
      P.chunk_row0.push_back((int32_t)(base + c0));
      P.chunk_len.push_back(L);
      int64_t endpos = c.b_head + c0 + L;
      int32_t save = -1;
      if (exact || L == B) {
        auto it = buf_id.find({si, endpos});
        if (it != buf_id.end()) save = it->second;
      }
      P.chunk_save.push_back(save);
      int32_t nrep = (int32_t)std::max<int64_t>(0, std::min<int64_t>(r - c0, L));
      P.chunk_nrep.push_back(nrep);
      P.chunk_rep0.push_back(rep_slots);
      rep_slots += nrep;
      c0 = nxt;
    }
    P.seq_chunk_ptr.push_back((int32_t)P.chunk_seq.size());
  }
  for (int32_t r = 0; r < P.n_rounds; ++r) {
    P.max_seq_per_round = std::max(P.max_seq_per_round, P.round_seq_ptr[r + 1]);
    P.round_seq_ptr[r + 1] += P.round_seq_ptr[r];
  }
  // launch order of each round's sequences: most chunks first (ties by id), so
  // that when a round has more blocks than compute units the long chains start
  // first; it changes no result (every block is independent)
  P.seq_lpt.resize(P.seq_round.size());
  for (int32_t r = 0; r < P.n_rounds; ++r) {
    const int32_t b = P.round_seq_ptr[r], e = P.round_seq_ptr[r + 1];
    for (int32_t si = b; si < e; ++si) P.seq_lpt[si] = si;
    std::stable_sort(P.seq_lpt.begin() + b, P.seq_lpt.begin() + e, [&](int32_t x, int32_t y) {
      return P.seq_chunk_ptr[x + 1] - P.seq_chunk_ptr[x] > P.seq_chunk_ptr[y + 1] - P.seq_chunk_ptr[y];
    });
  }
  P.n_packed = packed;
  P.n_out_rows = (mode != 1) ? n_rows : packed;

  // ---- handoff buffers and their consumers ----
  P.buf_seq.assign(nbuf, 0); P.buf_pos.assign(nbuf, 0); P.buf_chunk.assign(nbuf, -1);
  for (auto& kv : buf_id) {
    int32_t bi = kv.second, si = kv.first.first;
    int64_t b = kv.first.second;
    P.buf_seq[bi] = si;
    P.buf_pos[bi] = b;
    int32_t ch = -1, hits = 0;
    for (int32_t cc = P.seq_chunk_ptr[si]; cc < P.seq_chunk_ptr[si + 1]; ++cc)
      if (P.chunk_save[cc] == bi) { ch = cc; ++hits; }
    if (hits != 1 || P.buf_pos[bi] != b) {
      err = "internal: handoff buffer not at exactly one chunk end";
      return -1;
    }
    P.buf_chunk[bi] = ch;
  }
  {
    std::vector<std::vector<int32_t>> cons(nbuf);
    for (int32_t si = 0; si < nc; ++si)
      if (P.seq_init_kind[si] == 1) cons[P.seq_init_idx[si]].push_back(si);
    P.buf_cons_ptr.push_back(0);
    for (auto& cl : cons) {
      for (int32_t x : cl) P.buf_cons.push_back(x);
      P.buf_cons_ptr.push_back((int32_t)P.buf_cons.size());
    }
  }

  // ---- replay-gradient reduction (compact rows ascending, slots ascending) ----
  {
    std::vector<std::pair<int32_t, int32_t>> rr;  // (compact row, slot)
    for (int32_t c = 0; c < P.n_chunks(); ++c)
      for (int32_t i = 0; i < P.chunk_nrep[c]; ++i)
        rr.push_back({P.row_index[P.chunk_row0[c] + i], P.chunk_rep0[c] + i});
    std::sort(rr.begin(), rr.end());
    P.rep_ptr.push_back(0);
    for (size_t i = 0; i < rr.size(); ++i) {
      if (i == 0 || rr[i].first != rr[i - 1].first) {
        if (i > 0) P.rep_ptr.push_back((int32_t)i);
        P.rep_row.push_back(rr[i].first);
      }
      P.rep_slot.push_back(rr[i].second);
    }
    if (!rr.empty()) P.rep_ptr.push_back((int32_t)rr.size());
  }

  // ---- sequences started from each root's h0 ----
  {
    std::vector<std::vector<int32_t>> rs(P.n_root);
    for (int32_t si = 0; si < nc; ++si)
      if (P.seq_init_kind[si] == 0) rs[P.seq_init_idx[si]].push_back(si);
    P.root_seq_ptr.push_back(0);
    for (auto& l : rs) {
      for (int32_t x : l) P.root_seq.push_back(x);
      P.root_seq_ptr.push_back((int32_t)P.root_seq.size());
    }
  }

  // ---- gather map (trajectories by leaf id, positions 0..L-2) ----
  {
    int64_t nexp = 0;
    for (int32_t l : P.leaf_seg) {
      std::vector<int32_t> path;
      for (int32_t v = l; v >= 0; v = parent[v]) path.push_back(v);
      std::vector<int32_t> rows;
      for (auto it = path.rbegin(); it != path.rend(); ++it)
        for (int32_t t = 0; t < seg_len[*it]; ++t) rows.push_back((int32_t)(row0[*it] + t));
      nexp += (int64_t)rows.size();
      for (size_t t = 0; t + 1 < rows.size(); ++t) {
        P.pos_row.push_back(rows[t]);
        P.pos_next_row.push_back(rows[t + 1]);
      }
    }
    if ((int64_t)P.pos_row.size() >= (int64_t)INT32_MAX) {
      err = "too many positions";
      return -1;
    }
    P.n_expanded = nexp;
    P.row_pos_ptr.assign(n_rows + 1, 0);
    for (int32_t r : P.pos_row) P.row_pos_ptr[r + 1]++;
    for (int64_t i = 0; i < n_rows; ++i) P.row_pos_ptr[i + 1] += P.row_pos_ptr[i];
    P.row_pos_idx.assign(P.pos_row.size(), 0);
    std::vector<int32_t> fill(P.row_pos_ptr.begin(), P.row_pos_ptr.end() - 1);
    for (size_t pi = 0; pi < P.pos_row.size(); ++pi) P.row_pos_idx[fill[P.pos_row[pi]]++] = (int32_t)pi;
  }

  // ---- tree-ancestor attention tables ----
  {
    P.att_seg_row.resize(n);
    P.att_seg_len.resize(n);
    for (int32_t i = 0; i < n; ++i) {
      P.att_seg_row[i] = (int32_t)row0[i];
      P.att_seg_len[i] = seg_len[i];
    }
    std::vector<int64_t> anc_rows(n, 0);
    P.att_anc_ptr.push_back(0);
    for (int32_t v = 0; v < n; ++v) {
      std::vector<int32_t> path;
      for (int32_t a = parent[v]; a >= 0; a = parent[a]) path.push_back(a);
      for (auto it = path.rbegin(); it != path.rend(); ++it) {
        P.att_anc.push_back(*it);
        anc_rows[v] += seg_len[*it];
      }
      P.att_anc_ptr.push_back((int32_t)P.att_anc.size());
    }
    P.att_seg_tile0.push_back(0);
    for (int32_t v = 0; v < n; ++v) {
      for (int32_t off = 0; off < seg_len[v]; off += ATT_TILE) {
        P.att_tile_seg.push_back(v);
        P.att_tile_off.push_back(off);
      }
      P.att_seg_tile0.push_back((int32_t)P.att_tile_seg.size());
    }
    const int32_t nt = (int32_t)P.att_tile_seg.size();
    // forward order: most keys first
    {
      std::vector<std::pair<int64_t, int32_t>> w(nt);
      for (int32_t t = 0; t < nt; ++t) {
        const int32_t v = P.att_tile_seg[t], off = P.att_tile_off[t];
        w[t] = {-(anc_rows[v] + off + std::min(ATT_TILE, seg_len[v] - off)), t};
      }
      std::sort(w.begin(), w.end());
      for (auto& x : w) P.att_qorder.push_back(x.second);
    }
    // query tiles seeing each key tile: own segment from the tile on, then the
    // descendants (pre-order positions after v up to the end of its subtree)
    std::vector<int32_t> pos(n), sub_end(n);
    for (int32_t i = 0; i < n; ++i) pos[order[i]] = i;
    for (int32_t i = n - 1; i >= 0; --i) {
      const int32_t v = order[i];
      int32_t end = i + 1;
      for (int32_t j = child_ptr[v]; j < child_ptr[v + 1]; ++j) end = std::max(end, sub_end[child_list[j]]);
      sub_end[v] = end;
    }
    P.att_kq_ptr.push_back(0);
    for (int32_t t = 0; t < nt; ++t) {
      const int32_t v = P.att_tile_seg[t];
      for (int32_t u = t; u < P.att_seg_tile0[v + 1]; ++u) P.att_kq.push_back(u);
      for (int32_t i = pos[v] + 1; i < sub_end[v]; ++i) {
        const int32_t d = order[i];
        for (int32_t u = P.att_seg_tile0[d]; u < P.att_seg_tile0[d + 1]; ++u) P.att_kq.push_back(u);
      }
      if ((int64_t)P.att_kq.size() >= (int64_t)INT32_MAX) {
        err = "attention work lists too large";
        return -1;
      }
      P.att_kq_ptr.push_back((int32_t)P.att_kq.size());
    }
    // work items of at most kw query tiles (at least ATT_KW_MIN, and about
    // ATT_KW_TARGET items in all), most query tiles first; split tiles get
    // consecutive slots
    const int64_t total_kq = (int64_t)P.att_kq.size();
    const int32_t kw = (int32_t)std::max<int64_t>(ATT_KW_MIN, (total_kq + ATT_KW_TARGET - 1) / ATT_KW_TARGET);
    P.att_kw_max = kw;
    struct Item { int32_t nq, tile, q0; };
    std::vector<Item> items;
    int32_t slot = 0;
    std::vector<int32_t> tile_slot0(nt, -1);
    for (int32_t t = 0; t < nt; ++t) {
      const int32_t nq = P.att_kq_ptr[t + 1] - P.att_kq_ptr[t];
      const int32_t nitem = (nq + kw - 1) / kw;
      if (nitem > 1) {
        tile_slot0[t] = slot;
        P.att_ks_tile.push_back(t);
        P.att_ks_slot0.push_back(slot);
        P.att_ks_n.push_back(nitem);
        slot += nitem;
      }
      for (int32_t i = 0; i < nitem; ++i)
        items.push_back({std::min(kw, nq - i * kw), t, i * kw});
    }
    std::stable_sort(items.begin(), items.end(),
                     [](const Item& x, const Item& y) { return x.nq > y.nq; });
    for (auto& it : items) {
      P.att_kw_tile.push_back(it.tile);
      P.att_kw_q0.push_back(it.q0);
      P.att_kw_nq.push_back(it.nq);
      P.att_kw_slot.push_back(tile_slot0[it.tile] < 0 ? -1 : tile_slot0[it.tile] + it.q0 / kw);
    }
    P.att_n_slots = slot;
  }

  P.chunk_round.resize(P.chunk_seq.size());
  for (size_t c = 0; c < P.chunk_seq.size(); ++c) P.chunk_round[c] = P.seq_round[P.chunk_seq[c]];

  // ---- device block: int32 tables, each 64-element (256 B) aligned ----
  {
    DevLayout& d = P.dev;
    int64_t off = 0;
    std::vector<std::pair<int64_t*, const std::vector<int32_t>*>> tabs = {
        {&d.round_seq_ptr, &P.round_seq_ptr}, {&d.seq_chunk_ptr, &P.seq_chunk_ptr},
        {&d.seq_row_ptr, &P.seq_row_ptr},     {&d.seq_init_kind, &P.seq_init_kind},
        {&d.seq_init_idx, &P.seq_init_idx},   {&d.seq_leaf, &P.seq_leaf},
        {&d.seq_lpt, &P.seq_lpt},
        {&d.chunk_seq, &P.chunk_seq},         {&d.chunk_row0, &P.chunk_row0},
        {&d.chunk_len, &P.chunk_len},         {&d.chunk_save, &P.chunk_save},
        {&d.chunk_nrep, &P.chunk_nrep},       {&d.chunk_rep0, &P.chunk_rep0},
        {&d.chunk_round, &P.chunk_round},
        {&d.row_index, &P.row_index},         {&d.out_row, &P.out_row},
        {&d.buf_cons_ptr, &P.buf_cons_ptr},   {&d.buf_cons, &P.buf_cons},
        {&d.buf_chunk, &P.buf_chunk},         {&d.rep_row, &P.rep_row},
        {&d.rep_ptr, &P.rep_ptr},             {&d.rep_slot, &P.rep_slot},
        {&d.root_seq_ptr, &P.root_seq_ptr},   {&d.root_seq, &P.root_seq},
        {&d.pos_row, &P.pos_row},             {&d.pos_next_row, &P.pos_next_row},
        {&d.row_pos_ptr, &P.row_pos_ptr},     {&d.row_pos_idx, &P.row_pos_idx},
        {&d.row_mult, &P.row_mult},
        {&d.att_seg_row, &P.att_seg_row},     {&d.att_seg_len, &P.att_seg_len},
        {&d.att_anc_ptr, &P.att_anc_ptr},     {&d.att_anc, &P.att_anc},
        {&d.att_seg_tile0, &P.att_seg_tile0}, {&d.att_tile_seg, &P.att_tile_seg},
        {&d.att_tile_off, &P.att_tile_off},   {&d.att_qorder, &P.att_qorder},
        {&d.att_kq_ptr, &P.att_kq_ptr},       {&d.att_kq, &P.att_kq},
        {&d.att_kw_tile, &P.att_kw_tile},     {&d.att_kw_q0, &P.att_kw_q0},
        {&d.att_kw_nq, &P.att_kw_nq},         {&d.att_kw_slot, &P.att_kw_slot},
        {&d.att_ks_tile, &P.att_ks_tile},     {&d.att_ks_slot0, &P.att_ks_slot0},
        {&d.att_ks_n, &P.att_ks_n},
    };
    for (auto& t : tabs) {
      *t.first = off;
      off += ((int64_t)t.second->size() + 63) / 64 * 64;
    }
    d.total = std::max<int64_t>(off, 64);
    P.dev_blob.assign(d.total, 0);
    for (auto& t : tabs) std::copy(t.second->begin(), t.second->end(), P.dev_blob.begin() + *t.first);
  }
  return 0;
}

}  // namespace kda
