// l1plan.cpp -- compression-oriented microbatches of whole trajectories (host).
//
// HARTS abstract and thelatestinai.com Figure 1(c): the first planner level
// builds compression-oriented microbatches; Table 4 compares planners by
// compression and balance.  The pages give no algorithm; this one:
//   * a microbatch holds whole trajectories (root-to-leaf paths); its load is
//     its unique token count, the union of their rows, within the budget;
//   * a tree that fits the budget stays whole (all its sharing kept);
//   * a larger tree is cut into groups of leaves taken in depth-first order
//     (neighbouring leaves share the longest prefixes): a leaf joins the open
//     group if the group's unique tokens plus the leaf's segments not yet in
//     it stay within the budget, else it opens a new group with its whole
//     path (a path longer than the budget goes alone);
//   * the items (whole trees and groups) are packed first-fit decreasing into
//     microbatches, which fixes their number M; they are then placed again,
//     largest first, each on the least-loaded of the M microbatches it fits
//     in, and that placement is kept when every item fits (it evens the
//     loads: balance = mean load / largest load).
// Deterministic: ties by the lower id.  O(n_seg log n_seg + sum of depths).
#include <algorithm>
#include <cstdint>
#include <string>
#include <vector>

namespace kda {

int l1_plan(int32_t n, const int32_t* parent, const int32_t* seg_len, int64_t budget,
            std::vector<int32_t>& leaf_mb, std::vector<int64_t>& mb_unique,
            std::vector<int64_t>& mb_expanded, std::string& err) {
  if (n <= 0) { err = "empty tree"; return -1; }
  if (budget <= 0) { err = "budget must be positive"; return -1; }
  std::vector<int32_t> cptr(n + 1, 0), clist(n);
  std::vector<int32_t> roots;
  for (int32_t v = 0; v < n; ++v) {
    if (parent[v] < -1 || parent[v] >= n) { err = "parent id out of range"; return -1; }
    if (seg_len[v] <= 0) { err = "segment length must be positive"; return -1; }
    if (parent[v] < 0) roots.push_back(v); else cptr[parent[v] + 1]++;
  }
  for (int32_t v = 0; v < n; ++v) cptr[v + 1] += cptr[v];
  {
    std::vector<int32_t> fill(cptr.begin(), cptr.end() - 1);
    for (int32_t v = 0; v < n; ++v)
      if (parent[v] >= 0) clist[fill[parent[v]]++] = v;
  }
  // depth-first order per tree (children ascending), path ends, tree sizes
  std::vector<int64_t> endp(n, 0);
  std::vector<int32_t> order;
  order.reserve(n);
  std::vector<std::pair<int32_t, int32_t>> tree_span;   // [begin, end) in `order`
  {
    std::vector<char> seen(n, 0);
    for (int32_t r : roots) {
      const int32_t b = (int32_t)order.size();
      std::vector<int32_t> st{r};
      while (!st.empty()) {
        const int32_t v = st.back();
        st.pop_back();
        if (seen[v]) { err = "segment reached twice"; return -1; }
        seen[v] = 1;
        order.push_back(v);
        endp[v] = (parent[v] < 0 ? 0 : endp[parent[v]]) + seg_len[v];
        for (int32_t j = cptr[v + 1] - 1; j >= cptr[v]; --j) st.push_back(clist[j]);
      }
      tree_span.push_back({b, (int32_t)order.size()});
    }
    if ((int32_t)order.size() != n) { err = "parent links contain a cycle"; return -1; }
  }
  std::vector<int32_t> leaf_id(n, -1);
  int32_t n_leaf = 0;
  for (int32_t v = 0; v < n; ++v)
    if (cptr[v + 1] == cptr[v]) leaf_id[v] = n_leaf++;

  // items: sets of leaves with their unique and expanded tokens
  struct Item { int64_t unique = 0, expanded = 0; std::vector<int32_t> leaves; };
  std::vector<Item> items;
  std::vector<int32_t> mark(n, -1);   // group that holds the segment
  int32_t gid = 0;
  for (auto [b, e] : tree_span) {
    int64_t tree_u = 0, tree_x = 0;
    std::vector<int32_t> leaves;
    for (int32_t i = b; i < e; ++i) {
      const int32_t v = order[i];
      tree_u += seg_len[v];
      if (leaf_id[v] >= 0) { leaves.push_back(v); tree_x += endp[v]; }
    }
    if (tree_u <= budget) {
      Item it;
      it.unique = tree_u;
      it.expanded = tree_x;
      it.leaves = leaves;
      items.push_back(std::move(it));
      continue;
    }
    Item cur;
    int32_t cur_g = -1;
    for (int32_t l : leaves) {
      int64_t add = 0;   // this leaf's segments not yet in the open group
      for (int32_t u = l; u >= 0 && mark[u] != cur_g; u = parent[u]) add += seg_len[u];
      if (cur_g >= 0 && cur.unique + add > budget) {
        items.push_back(std::move(cur));
        cur = Item();
        cur_g = -1;
      }
      if (cur_g < 0) {
        cur_g = gid++;
        add = endp[l];
      }
      for (int32_t u = l; u >= 0 && mark[u] != cur_g; u = parent[u]) mark[u] = cur_g;
      cur.unique += add;
      cur.expanded += endp[l];
      cur.leaves.push_back(l);
    }
    if (cur_g >= 0) items.push_back(std::move(cur));
  }

  // first-fit decreasing into microbatches of the budget
  std::vector<int32_t> idx(items.size());
  for (size_t i = 0; i < idx.size(); ++i) idx[i] = (int32_t)i;
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int32_t a, int32_t b) { return items[a].unique > items[b].unique; });
  std::vector<int64_t> load;
  std::vector<int32_t> bin(items.size(), -1);
  for (int32_t i : idx) {
    int32_t m = -1;
    for (size_t j = 0; j < load.size(); ++j)
      if (load[j] + items[i].unique <= budget) { m = (int32_t)j; break; }
    if (m < 0) { m = (int32_t)load.size(); load.push_back(0); }
    load[m] += items[i].unique;
    bin[i] = m;
  }
  // the same number of microbatches, least-loaded placement
  {
    const size_t M = load.size();
    std::vector<int64_t> l2(M, 0);
    std::vector<int32_t> b2(items.size(), -1);
    bool ok = true;
    for (int32_t i : idx) {
      int32_t m = -1;
      for (size_t j = 0; j < M; ++j)
        if ((l2[j] + items[i].unique <= budget || l2[j] == 0) && (m < 0 || l2[j] < l2[m]))
          m = (int32_t)j;
      if (m < 0) { ok = false; break; }
      l2[m] += items[i].unique;
      b2[i] = m;
    }
    if (ok) { load = l2; bin = b2; }
  }
  leaf_mb.assign(n_leaf, -1);
  mb_unique.assign(load.size(), 0);
  mb_expanded.assign(load.size(), 0);
  for (size_t i = 0; i < items.size(); ++i) {
    for (int32_t l : items[i].leaves) leaf_mb[leaf_id[l]] = bin[i];
    mb_unique[bin[i]] += items[i].unique;
    mb_expanded[bin[i]] += items[i].expanded;
  }
  return 0;
}

}  // namespace kda
