// Cache-aware ordering of a waiting queue against the radix tree.
//
// Follows "SGLang: the tree, and the language nobody remembers" (ai.thesatyajit.com),
// section "The scheduler is where the cache is won or lost":
//  * longest prefix match: requests with more of their prompt already cached go
//    first, so the tree stays warm for their siblings;
//  * in-queue prefix dedup: a request whose cached match is thin (<= 32 tokens)
//    is checked against a radix tree of the queue itself (the earlier thin
//    requests); if it shares >= 32 tokens with one of them it goes to the very back,
//    so that its sibling runs first and it returns as a cache hit; otherwise it
//    joins that queue tree;
//  * the longest-prefix order turns itself off above 128 queued requests
//    (arrival order then);
//  * depth-first weighting: each node weighs the waiting requests that hang off its
//    subtree, and the queue is emitted in a depth-first order, heavier subtrees
//    first, so a subtree is drained before it can be evicted.
// "How does SGLang work" (modernaiengineering.com), "Practice: try it yourself",
// serves a toy queue both in arrival order and longest-prefix-first; its printed
// result is reproduced through this call in the tests.
//
// Readings where the page is silent: matching for scheduling only reads the tree (no
// split, no clock tick); ties keep arrival order; a request hangs off the deepest node
// whose whole root path its tokens match; a node's own requests come after its
// subtrees (the deeper matches first, cold requests last), children of equal weight
// in ascending order of their first page (first token at page size 1).  With pages a
// match is rounded down to a page, as the tree's own match is.

#include <algorithm>
#include <unordered_map>
#include <vector>

#include "internal.h"

namespace {

using rs::Node;

// Longest cached prefix of tok[0..n), read-only; *deepest = the deepest node whose
// whole root path is a prefix of tok.
int64_t peek(const rs_tree* t, const int32_t* tok, int64_t n, const Node** deepest) {
  const Node* node = &t->root;
  int64_t pos = 0;
  const int32_t ps = t->ps;
  while (pos + ps <= n) {                 // whole pages only
    const Node* c = t->child_at(node, tok + pos);
    if (!c) break;
    const int64_t len = int64_t(c->key.size());
    const int64_t k = rs::diverge(c->key.data(), tok + pos, std::min(len, n - pos)) / ps * ps;
    pos += k;
    if (k < len) break;
    node = c;
  }
  *deepest = node;
  return pos;
}

uint64_t hash_tokens(const int32_t* p, int64_t n) {
  uint64_t h = 0xcbf29ce484222325ull;           // FNV-1a over the token bytes
  for (int64_t i = 0; i < n; ++i) {
    uint32_t v = uint32_t(p[i]);
    for (int b = 0; b < 4; ++b) {
      h ^= (v >> (8 * b)) & 0xffu;
      h *= 0x100000001b3ull;
    }
  }
  return h;
}

void lpm(const int32_t* tokens, const int64_t* offsets, int32_t n, const std::vector<int64_t>& matched,
         int32_t* order) {
  constexpr int64_t kThin = RS_SCHED_IN_QUEUE_THRESHOLD;
  // The queue's own tree, as far as the decision needs it: a thin request is put back
  // when an earlier thin request (one not put back) has the same first kThin tokens.
  std::unordered_map<uint64_t, std::vector<int32_t>> queue_tree;
  std::vector<char> back(n, 0);
  for (int32_t i = 0; i < n; ++i) {
    if (matched[i] > kThin) continue;
    const int32_t* tok = tokens + offsets[i];
    const int64_t len = offsets[i + 1] - offsets[i];
    if (len < kThin) continue;                 // shares < kThin with anything; cannot be matched to kThin
    auto& bucket = queue_tree[hash_tokens(tok, kThin)];
    bool shared = false;
    for (int32_t j : bucket)
      if (rs::diverge(tokens + offsets[j], tok, kThin) == kThin) { shared = true; break; }
    if (shared) back[i] = 1;
    else bucket.push_back(i);
  }
  for (int32_t i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order, order + n, [&](int32_t a, int32_t b) {
    if (back[a] != back[b]) return back[a] < back[b];
    return !back[a] && matched[a] > matched[b];
  });
}

void dfs_weight(const rs_tree* t, const std::vector<const Node*>& at, int32_t n, int32_t* order) {
  // weight of a node: the requests at it or below it
  std::unordered_map<const Node*, int64_t> weight;
  std::unordered_map<const Node*, std::vector<int32_t>> own;
  for (int32_t i = 0; i < n; ++i) {
    own[at[i]].push_back(i);
    for (const Node* v = at[i]; v; v = v->parent) ++weight[v];
  }
  // weighted children of each weighted node
  std::unordered_map<const Node*, std::vector<const Node*>> kids;
  for (auto& kv : weight)
    if (kv.first->parent) kids[kv.first->parent].push_back(kv.first);
  for (auto& kv : kids)
    std::sort(kv.second.begin(), kv.second.end(), [&](const Node* a, const Node* b) {
      const int64_t wa = weight[a], wb = weight[b];
      if (wa != wb) return wa > wb;
      return std::lexicographical_compare(a->key.begin(), a->key.begin() + t->ps, b->key.begin(),
                                          b->key.begin() + t->ps);
    });
  // post-order walk with an explicit stack: (node, next child index)
  int32_t k = 0;
  std::vector<std::pair<const Node*, size_t>> st;
  st.emplace_back(&t->root, 0);
  while (!st.empty()) {
    auto& top = st.back();
    auto it = kids.find(top.first);
    if (it != kids.end() && top.second < it->second.size()) {
      const Node* c = it->second[top.second++];
      st.emplace_back(c, 0);
      continue;
    }
    auto o = own.find(top.first);
    if (o != own.end())
      for (int32_t i : o->second) order[k++] = i;
    st.pop_back();
  }
}

}  // namespace

extern "C" {

int rs_schedule(const rs_tree* t, const int32_t* tokens, const int64_t* offsets, int32_t n, int32_t policy,
                int32_t* out_order, int64_t* out_matched) {
  if (!t || n < 0 || (n > 0 && (!offsets || !out_order)))
    return rs::fail(RS_E_INVAL, "rs_schedule: bad arguments");
  if (policy != RS_SCHED_FCFS && policy != RS_SCHED_LPM && policy != RS_SCHED_DFS_WEIGHT)
    return rs::fail(RS_E_INVAL, "rs_schedule: unknown policy " + std::to_string(policy));
  if (n == 0) return RS_OK;
  if (offsets[0] < 0) return rs::fail(RS_E_INVAL, "rs_schedule: offsets[0] < 0");
  for (int32_t i = 0; i < n; ++i)
    if (offsets[i + 1] < offsets[i]) return rs::fail(RS_E_INVAL, "rs_schedule: offsets decrease");
  if (offsets[n] > offsets[0] && !tokens) return rs::fail(RS_E_INVAL, "rs_schedule: null tokens");
  std::vector<int64_t> matched(n);
  std::vector<const Node*> at(n);
  for (int32_t i = 0; i < n; ++i)
    matched[i] = peek(t, tokens + offsets[i], offsets[i + 1] - offsets[i], &at[i]);
  if (out_matched) std::copy(matched.begin(), matched.end(), out_matched);
  if (policy == RS_SCHED_LPM && n > RS_SCHED_LPM_MAX_QUEUE) policy = RS_SCHED_FCFS;
  if (policy == RS_SCHED_FCFS) {
    for (int32_t i = 0; i < n; ++i) out_order[i] = i;
  } else if (policy == RS_SCHED_LPM) {
    lpm(tokens, offsets, n, matched, out_order);
  } else {
    dfs_weight(t, at, n, out_order);
  }
  return RS_OK;
}

}  // extern "C"
