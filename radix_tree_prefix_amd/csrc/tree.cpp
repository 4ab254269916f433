// Host radix tree over token prefixes, slot allocator and eviction.
//
// Follows "SGLang: the tree, and the language nobody remembers"
// (ai.thesatyajit.com), section "A tree, not a map": nodes hold a token run,
// one KV slot per token, children keyed on the first token (page size 1) or on the
// first page (larger pages: keys truncated to whole pages, matches rounded down to a
// page, slots allocated and freed in whole pages, from the same section's details of
// the source),
// lock_ref, last access and priority; a node splits at the divergence point;
// lock_ref changes move a node's tokens between the evictable and protected
// totals on its 0<->1 edge; eviction pops unlocked leaves off a heap and
// pushes a parent that the pop left childless and unlocked.  The edge compare
// is a galloping search (doubling windows, then a binary search inside the
// window that holds the divergence), which is what the same section describes
// for long shared prefixes.  Request admission follows "How does SGLang work"
// (modernaiengineering.com), "What happens when a request arrives".
//
// Where the pages leave a rule open the tree takes: a logical clock that ticks
// once per match or insert call and stamps every node the call visits; heap
// key (priority, last_access, id), priority 0 (pure least-recently-used, the
// recency order the other pages describe); splits in match and in insert, the
// upper part getting a fresh id and the lower part's lock_ref and last access;
// lowest-free-first slots; on insert over present tokens the tree's slots win.

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <queue>
#include <tuple>

#include "internal.h"

namespace rs {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

// Index of the first position where a and b differ (n if none).  Galloping:
// windows [0,1), [1,3), [3,7), ... are compared whole; the first window that
// differs is bisected with whole-span compares.
int64_t diverge(const int32_t* a, const int32_t* b, int64_t n) {
  int64_t lo = 0, w = 1;
  while (lo < n) {
    int64_t len = std::min(w, n - lo);
    if (std::memcmp(a + lo, b + lo, size_t(len) * 4) != 0) {
      int64_t l = lo, r = lo + len;       // a[0..l) == b[0..l); they differ in [l, r)
      while (r - l > 1) {
        int64_t mid = l + (r - l) / 2;
        if (std::memcmp(a + l, b + l, size_t(mid - l) * 4) == 0) l = mid;
        else r = mid;
      }
      return l;
    }
    lo += len;
    w *= 2;
  }
  return n;
}

SlotAllocator::SlotAllocator(int64_t n, int32_t ps)
    : n_(n), nfree_(n), hint_(0), ps_(ps), bits_((n + 63) / 64, ~0ull) {
  if (n & 63) bits_.back() = (1ull << (n & 63)) - 1;
}

void SlotAllocator::set_page(int64_t p0, bool free_) {
  for (int64_t x = p0; x < p0 + ps_; ++x) {
    if (free_) bits_[x >> 6] |= 1ull << (x & 63);
    else bits_[x >> 6] &= ~(1ull << (x & 63));
  }
}

void SlotAllocator::take(int64_t k, int32_t* out) {
  int64_t got = 0, w = hint_;
  if (ps_ == 1) {
    while (got < k) {
      uint64_t b = bits_[w];
      while (b && got < k) {
        int tz = __builtin_ctzll(b);
        out[got++] = int32_t(w * 64 + tz);
        b &= b - 1;
      }
      bits_[w] = b;
      if (!b) ++w;
    }
    hint_ = w;
    nfree_ -= k;
    return;
  }
  const int64_t pages = (k + ps_ - 1) / ps_;
  for (int64_t taken = 0; taken < pages;) {
    uint64_t b = bits_[w];
    if (!b) { ++w; continue; }
    const int64_t p0 = w * 64 + __builtin_ctzll(b);   // the lowest free slot starts a free page
    set_page(p0, false);
    for (int64_t i = 0; i < ps_ && got < k; ++i) out[got++] = int32_t(p0 + i);
    ++taken;
  }
  hint_ = w;
  nfree_ -= pages * ps_;
}

bool SlotAllocator::give_back(const int32_t* s, int64_t k) {
  std::vector<int64_t> freed;          // page starts freed by this call
  for (int64_t i = 0; i < k; ++i) {
    const int32_t x = s[i];
    const int64_t p0 = x < 0 ? -1 : int64_t(x) - int64_t(x) % ps_;
    bool bad = x < 0 || x >= n_;
    if (!bad && is_free(int32_t(p0))) {
      bad = std::find(freed.begin(), freed.end(), p0) == freed.end();   // free before this call
      if (!bad) continue;
    }
    if (bad) {
      for (int64_t q : freed) set_page(q, false);
      return false;
    }
    set_page(p0, true);
    freed.push_back(p0);
  }
  for (int64_t q : freed) hint_ = std::min<int64_t>(hint_, q >> 6);
  nfree_ += int64_t(freed.size()) * ps_;
  return true;
}

}  // namespace rs

using rs::Node;

rs_tree::rs_tree(int64_t pool_slots, int32_t page_size) : alloc(pool_slots, page_size), ps(page_size) { root.id = 0; }

Node* rs_tree::child_at(const Node* n, const int32_t* page) const {
  auto r = n->children.equal_range(page[0]);
  for (auto it = r.first; it != r.second; ++it)
    if (ps == 1 || std::memcmp(it->second->key.data(), page, size_t(ps) * 4) == 0) return it->second;
  return nullptr;
}

void rs_tree::link(Node* parent, Node* c) { parent->children.emplace(c->key[0], c); }

void rs_tree::unlink(Node* parent, Node* c) {
  auto r = parent->children.equal_range(c->key[0]);
  for (auto it = r.first; it != r.second; ++it)
    if (it->second == c) {
      parent->children.erase(it);
      return;
    }
}

Node* rs_tree::find(int64_t id) {
  if (id == 0) return &root;
  auto it = nodes.find(id);
  return it == nodes.end() ? nullptr : it->second.get();
}
const Node* rs_tree::find(int64_t id) const {
  if (id == 0) return &root;
  auto it = nodes.find(id);
  return it == nodes.end() ? nullptr : it->second.get();
}

Node* rs_tree::split(Node* child, int64_t k) {
  auto up = std::make_unique<Node>();
  Node* u = up.get();
  u->id = next_id++;
  u->key.assign(child->key.begin(), child->key.begin() + k);
  if (!child->value.empty()) {            // empty: on the host only
    u->value.assign(child->value.begin(), child->value.begin() + k);
    child->value.erase(child->value.begin(), child->value.begin() + k);
  }
  u->parent = child->parent;
  u->lock_ref = child->lock_ref;
  u->last_access = child->last_access;
  u->priority = child->priority;
  u->pend = child->pend;
  if (!child->host.empty()) {
    u->host.assign(child->host.begin(), child->host.begin() + k);
    child->host.erase(child->host.begin(), child->host.begin() + k);
  }
  unlink(u->parent, child);
  link(u->parent, u);
  child->key.erase(child->key.begin(), child->key.begin() + k);
  child->parent = u;
  link(u, child);
  nodes.emplace(u->id, std::move(up));
  return u;
}

int64_t rs_tree::match(const int32_t* tok, int64_t n, int32_t* out, Node** end) {
  ++clock;
  ++match_calls;
  Node* node = &root;
  int64_t pos = 0;
  while (pos + ps <= n) {                 // whole pages only
    Node* c = child_at(node, tok + pos);
    if (!c || c->value.empty()) break;   // absent, or on the host only: not a device match
    c->last_access = clock;
    int64_t len = int64_t(c->key.size());
    int64_t k = rs::diverge(c->key.data(), tok + pos, std::min(len, n - pos)) / ps * ps;
    if (k < len) c = split(c, k);
    if (out) std::memcpy(out + pos, c->value.data(), size_t(k) * 4);
    pos += k;
    node = c;
  }
  matched_total += pos;
  *end = node;
  return pos;
}

int rs_tree::insert(const int32_t* tok, int32_t* slots, int64_t n, int64_t* prefix, Node** end) {
  n = n / ps * ps;                        // whole pages only; the caller keeps the rest
  for (int64_t i = 0; i < n; ++i) {
    if (slots[i] < 0 || slots[i] >= alloc.capacity() || alloc.is_free(slots[i]))
      return rs::fail(RS_E_INVAL, "rs_insert: slot " + std::to_string(slots[i]) + " at position " +
                                      std::to_string(i) + " is out of range or not allocated");
    // with pages: position i's slot is page * ps + i % ps, one page per ps positions
    if (ps > 1 && (i % ps == 0 ? slots[i] % ps != 0 : slots[i] != slots[i - 1] + 1))
      return rs::fail(RS_E_INVAL, "rs_insert: slots are not whole pages aligned with the positions (position " +
                                      std::to_string(i) + ")");
  }
  ++clock;
  ++insert_calls;
  Node* node = &root;
  int64_t pos = 0;
  int rc = RS_OK;
  std::vector<int32_t> differ;
  while (pos + ps <= n) {
    Node* c = child_at(node, tok + pos);
    if (!c) break;
    c->last_access = clock;
    int64_t len = int64_t(c->key.size());
    int64_t k = rs::diverge(c->key.data(), tok + pos, std::min(len, n - pos)) / ps * ps;
    if (k < len) c = split(c, k);
    if (c->value.empty()) {               // on the host only: it takes the caller's device slots
      c->value.assign(slots + pos, slots + pos + k);
      if (c->lock_ref > 0) protected_ += k;
      else evictable += k;
      tree_tokens += k;
    }
    differ.clear();
    for (int64_t i = 0; i < k; ++i)
      if (slots[pos + i] != c->value[i]) differ.push_back(slots[pos + i]);
    if (!differ.empty() && !alloc.give_back(differ.data(), int64_t(differ.size())))
      rc = rs::fail(RS_E_INVAL, "rs_insert: duplicate caller slot");
    for (int64_t i = 0; i < k; ++i) slots[pos + i] = c->value[i];
    pos += k;
    node = c;
  }
  *prefix = pos;
  if (pos < n) {
    auto leaf = std::make_unique<Node>();
    Node* l = leaf.get();
    l->id = next_id++;
    l->key.assign(tok + pos, tok + n);
    l->value.assign(slots + pos, slots + n);
    l->parent = node;
    l->last_access = clock;
    link(node, l);
    nodes.emplace(l->id, std::move(leaf));
    evictable += n - pos;
    tree_tokens += n - pos;
    node = l;
  }
  *end = node;
  return rc;
}

void rs_tree::lock(Node* nd) {
  for (; nd != &root; nd = nd->parent) {
    if (nd->lock_ref == 0) {
      evictable -= int64_t(nd->value.size());
      protected_ += int64_t(nd->value.size());
    }
    ++nd->lock_ref;
  }
}

int rs_tree::unlock(Node* nd) {
  if (nd != &root && nd->lock_ref <= 0)
    return rs::fail(RS_E_INVAL, "rs_dec_lock_ref: node " + std::to_string(nd->id) + " is not locked");
  for (; nd != &root; nd = nd->parent) {
    if (nd->lock_ref == 1) {
      evictable += int64_t(nd->value.size());
      protected_ -= int64_t(nd->value.size());
    }
    --nd->lock_ref;
  }
  return RS_OK;
}

bool rs_tree::device_leaf(const Node* n) const {
  if (n->value.empty() || n->lock_ref != 0) return false;
  for (auto& kv : n->children)
    if (!kv.second->value.empty()) return false;
  return true;
}

int64_t rs_tree::evict(int64_t need) {
  typedef std::tuple<int64_t, uint64_t, int64_t> Key;   // (priority, last_access, id)
  std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
  for (auto& kv : nodes) {
    Node* n = kv.second.get();
    if (device_leaf(n)) heap.emplace(n->priority, n->last_access, n->id);
  }
  int64_t freed = 0;
  while (freed < need && !heap.empty()) {
    int64_t id = std::get<2>(heap.top());
    heap.pop();
    Node* x = nodes[id].get();
    int64_t len = int64_t(x->value.size());
    alloc.give_back(x->value.data(), len);
    freed += len;
    evictable -= len;
    tree_tokens -= len;
    Node* p = x->parent;
    if (!x->host.empty() && x->pend == 0) {
      x->value.clear();                   // a finished host copy: the node stays, on the host
    } else {
      drop_host_subtree(x);               // children left are on the host only; they go too
      unlink(p, x);
      nodes.erase(id);
    }
    if (p != &root && device_leaf(p)) heap.emplace(p->priority, p->last_access, p->id);
  }
  evicted_total += freed;
  return freed;
}

void rs_tree::drop_host_subtree(Node* x) {
  std::vector<Node*> kids;
  for (auto& kv : x->children) kids.push_back(kv.second);
  for (Node* c : kids) {
    drop_host_subtree(c);
    if (host) host->give_back(c->host.data(), int64_t(c->host.size()));
    unlink(x, c);
    nodes.erase(c->id);
  }
}

int64_t rs_tree::evict_host(int64_t need) {
  typedef std::tuple<int64_t, uint64_t, int64_t> Key;
  std::priority_queue<Key, std::vector<Key>, std::greater<Key>> heap;
  auto host_leaf = [&](const Node* n) {
    return n->value.empty() && n->children.empty() && n->lock_ref == 0 && n->pend == 0;
  };
  for (auto& kv : nodes)
    if (host_leaf(kv.second.get())) heap.emplace(kv.second->priority, kv.second->last_access, kv.second->id);
  int64_t freed = 0;
  while (freed < need && !heap.empty()) {
    int64_t id = std::get<2>(heap.top());
    heap.pop();
    Node* x = nodes[id].get();
    host->give_back(x->host.data(), int64_t(x->host.size()));
    freed += int64_t(x->host.size());
    Node* p = x->parent;
    unlink(p, x);
    nodes.erase(id);
    if (p != &root && host_leaf(p)) heap.emplace(p->priority, p->last_access, p->id);
  }
  return freed;
}

int rs_tree::alloc_host(int64_t n, int32_t* out) {
  if (host->num_free() < n) {
    evict_host(n - host->num_free());
    if (host->num_free() < n)
      return rs::fail(RS_E_NOSPACE, "host tier: " + std::to_string(n) + " slots wanted, " +
                                        std::to_string(host->num_free()) + " free after evicting every host leaf");
  }
  host->take(n, out);
  return RS_OK;
}

std::vector<Node*> rs_tree::path(Node* nd) {
  std::vector<Node*> p;
  for (; nd != &root; nd = nd->parent) p.push_back(nd);
  std::reverse(p.begin(), p.end());
  return p;
}

int rs_tree::alloc_slots(int64_t n, int32_t* out) {
  if (n < 0) return rs::fail(RS_E_INVAL, "rs_alloc_slots: negative count");
  const int64_t need = (n + ps - 1) / ps * ps;       // whole pages
  if (alloc.num_free() < need) {
    evict(need - alloc.num_free());
    if (alloc.num_free() < need)
      return rs::fail(RS_E_NOSPACE, "rs_alloc_slots: " + std::to_string(n) + " slots wanted, " +
                                        std::to_string(alloc.num_free()) +
                                        " free after evicting every unlocked leaf");
  }
  alloc.take(n, out);
  return RS_OK;
}

int64_t rs_tree::depth_tokens(const Node* nd) const {
  int64_t d = 0;
  for (; nd != &root; nd = nd->parent) d += int64_t(nd->key.size());
  return d;
}

// ------------------------------------------------------------------ C ABI (tree)

#define RS_GUARD_BEGIN try {
#define RS_GUARD_END                                                    \
  }                                                                     \
  catch (const std::bad_alloc&) {                                       \
    return rs::fail(RS_E_INVAL, "out of host memory");                  \
  }                                                                     \
  catch (const std::exception& e) {                                     \
    return rs::fail(RS_E_INVAL, e.what());                              \
  }

extern "C" {

const char* rs_last_error(void) { return rs::g_last_error.c_str(); }
const char* rs_version(void) { return "librs 0.1 (gfx950)"; }

rs_tree* rs_tree_create(int64_t pool_slots, int32_t page_size) {
  if (pool_slots <= 0 || pool_slots > (int64_t(1) << 31) - 1) {
    rs::set_error("rs_tree_create: pool_slots must be in [1, 2^31)");
    return nullptr;
  }
  if (page_size < 1 || pool_slots % page_size != 0) {
    rs::set_error("rs_tree_create: page_size must be >= 1 and divide pool_slots");
    return nullptr;
  }
  try {
    return new rs_tree(pool_slots, page_size);
  } catch (...) {
    rs::set_error("rs_tree_create: out of host memory");
    return nullptr;
  }
}

void rs_tree_destroy(rs_tree* t) { delete t; }

int rs_match_prefix(rs_tree* t, const int32_t* tokens, int64_t n, int32_t* out_slots,
                    int64_t* out_len, int64_t* out_node) {
  if (!t || n < 0 || (n && (!tokens || !out_slots)) || !out_len || !out_node)
    return rs::fail(RS_E_INVAL, "rs_match_prefix: bad arguments");
  RS_GUARD_BEGIN
  Node* end = nullptr;
  *out_len = t->match(tokens, n, out_slots, &end);
  *out_node = end->id;
  return RS_OK;
  RS_GUARD_END
}

int rs_inc_lock_ref(rs_tree* t, int64_t node) {
  if (!t) return rs::fail(RS_E_INVAL, "rs_inc_lock_ref: null tree");
  Node* n = t->find(node);
  if (!n) return rs::fail(RS_E_STALE, "rs_inc_lock_ref: node " + std::to_string(node) + " is gone");
  t->lock(n);
  return RS_OK;
}

int rs_dec_lock_ref(rs_tree* t, int64_t node) {
  if (!t) return rs::fail(RS_E_INVAL, "rs_dec_lock_ref: null tree");
  Node* n = t->find(node);
  if (!n) return rs::fail(RS_E_STALE, "rs_dec_lock_ref: node " + std::to_string(node) + " is gone");
  return t->unlock(n);
}

int rs_alloc_slots(rs_tree* t, int64_t n, int32_t* out_slots) {
  if (!t || n < 0 || (n && !out_slots)) return rs::fail(RS_E_INVAL, "rs_alloc_slots: bad arguments");
  RS_GUARD_BEGIN
  return t->alloc_slots(n, out_slots);
  RS_GUARD_END
}

int rs_free_slots(rs_tree* t, const int32_t* slots, int64_t n) {
  if (!t || n < 0 || (n && !slots)) return rs::fail(RS_E_INVAL, "rs_free_slots: bad arguments");
  if (!t->alloc.give_back(slots, n))
    return rs::fail(RS_E_INVAL, "rs_free_slots: a slot is out of range or already free");
  return RS_OK;
}

int rs_insert(rs_tree* t, const int32_t* tokens, int32_t* slots, int64_t n, int64_t* out_prefix_len,
              int64_t* out_node) {
  if (!t || n < 0 || (n && (!tokens || !slots)) || !out_prefix_len || !out_node)
    return rs::fail(RS_E_INVAL, "rs_insert: bad arguments");
  RS_GUARD_BEGIN
  Node* end = nullptr;
  int64_t prefix = 0;
  int rc = t->insert(tokens, slots, n, &prefix, &end);
  if (end) {
    *out_prefix_len = prefix;
    *out_node = end->id;
  }
  return rc;
  RS_GUARD_END
}

int64_t rs_evict(rs_tree* t, int64_t num_tokens) {
  if (!t || num_tokens < 0) return rs::fail(RS_E_INVAL, "rs_evict: bad arguments");
  RS_GUARD_BEGIN
  return t->evict(num_tokens);
  RS_GUARD_END
}

int rs_admit(rs_tree* t, const int32_t* tokens, int64_t cached, int64_t n_new, int32_t* out_row,
             int64_t* out_node, int64_t* out_matched) {
  if (!t || cached < 0 || n_new < 0 || (cached + n_new && (!tokens || !out_row)) || !out_node ||
      !out_matched)
    return rs::fail(RS_E_INVAL, "rs_admit: bad arguments");
  RS_GUARD_BEGIN
  Node* node = nullptr;
  int64_t m = t->match(tokens, cached, out_row, &node);
  t->lock(node);
  const int32_t ps = t->ps;
  int64_t tail = 0;                 // slots left in the request's own last page after `cached`
  if (cached > m) {
    int rc = t->alloc_slots(cached - m, out_row + m);
    if (rc != RS_OK) {
      t->unlock(node);
      return rc;
    }
    if (cached % ps) tail = ps - cached % ps;
    int64_t prefix = 0;
    Node* node2 = nullptr;
    rc = t->insert(tokens, out_row, cached, &prefix, &node2);
    if (rc != RS_OK) {
      t->unlock(node);
      return rc;
    }
    t->lock(node2);
    t->unlock(node);
    node = node2;
  }
  if (n_new) {
    // the new tokens continue the request's last page, then take fresh pages
    const int64_t k = std::min(n_new, tail);
    for (int64_t i = 0; i < k; ++i) out_row[cached + i] = out_row[cached - 1] + 1 + int32_t(i);
    if (n_new > k) {
      int rc = t->alloc_slots(n_new - k, out_row + cached + k);
      if (rc != RS_OK) {
        if (tail) t->alloc.give_back(out_row + cached - 1, 1);   // the request's own last page
        t->unlock(node);
        return rc;
      }
    }
  }
  *out_node = node->id;
  *out_matched = m;
  return RS_OK;
  RS_GUARD_END
}

int rs_host_tier_enable(rs_tree* t, int64_t host_slots) {
  if (!t || host_slots <= 0 || host_slots > (int64_t(1) << 31) - 1)
    return rs::fail(RS_E_INVAL, "rs_host_tier_enable: bad arguments");
  if (t->ps != 1) return rs::fail(RS_E_UNSUPPORTED, "rs_host_tier_enable: page size 1 only");
  if (t->host) return rs::fail(RS_E_INVAL, "rs_host_tier_enable: the host tier is already on");
  RS_GUARD_BEGIN
  t->host = std::make_unique<rs::SlotAllocator>(host_slots, 1);
  return RS_OK;
  RS_GUARD_END
}

int rs_match_prefix2(rs_tree* t, const int32_t* tokens, int64_t n, int32_t* out_dev_slots, int32_t* out_host_slots,
                     int64_t* out_dev_len, int64_t* out_len, int64_t* out_dev_node, int64_t* out_node) {
  if (!t || n < 0 || (n && (!tokens || !out_dev_slots || !out_host_slots)) || !out_dev_len || !out_len ||
      !out_dev_node || !out_node)
    return rs::fail(RS_E_INVAL, "rs_match_prefix2: bad arguments");
  // the two-tier walk compares and splits one token at a time: page size 1 only, which is
  // also the only size the host tier is enabled at
  if (t->ps != 1) return rs::fail(RS_E_UNSUPPORTED, "rs_match_prefix2: page size 1 only");
  if (!t->host) return rs::fail(RS_E_INVAL, "rs_match_prefix2: the host tier is off");
  RS_GUARD_BEGIN
  ++t->clock;
  ++t->match_calls;
  Node* node = &t->root;
  Node* dev_node = &t->root;
  int64_t pos = 0, dev_len = 0;
  while (pos < n) {
    Node* c = t->child_at(node, tokens + pos);
    if (!c) break;
    c->last_access = t->clock;
    const int64_t len = int64_t(c->key.size());
    const int64_t k = rs::diverge(c->key.data(), tokens + pos, std::min(len, n - pos));
    if (k < len) c = t->split(c, k);
    if (!c->value.empty() && dev_len == pos) {
      std::memcpy(out_dev_slots + pos, c->value.data(), size_t(k) * 4);
      dev_node = c;
      dev_len = pos + k;
    } else {
      std::memcpy(out_host_slots + (pos - dev_len), c->host.data(), size_t(k) * 4);
    }
    pos += k;
    node = c;
  }
  t->matched_total += dev_len;
  *out_dev_len = dev_len;
  *out_len = pos;
  *out_dev_node = dev_node->id;
  *out_node = node->id;
  return RS_OK;
  RS_GUARD_END
}

int rs_write_through(rs_tree* t, int64_t node, int64_t cap, int32_t* out_dev_slots, int32_t* out_host_slots,
                     int64_t* out_n, int64_t* out_ticket) {
  if (!t || cap < 0 || (cap && (!out_dev_slots || !out_host_slots)) || !out_n || !out_ticket)
    return rs::fail(RS_E_INVAL, "rs_write_through: bad arguments");
  if (!t->host) return rs::fail(RS_E_INVAL, "rs_write_through: the host tier is off");
  Node* nd = t->find(node);
  if (!nd) return rs::fail(RS_E_STALE, "rs_write_through: node " + std::to_string(node) + " is gone");
  RS_GUARD_BEGIN
  std::vector<Node*> todo;
  int64_t need = 0;
  for (Node* x : t->path(nd)) {
    if (x->value.empty()) return rs::fail(RS_E_INVAL, "rs_write_through: the path is not on the device");
    if (x->host.empty() && x->pend == 0) {
      todo.push_back(x);
      need += int64_t(x->key.size());
    }
  }
  if (need > t->host->capacity())
    return rs::fail(RS_E_NOSPACE, "rs_write_through: " + std::to_string(need) + " tokens, host tier of " +
                                      std::to_string(t->host->capacity()) + " slots");
  if (need > cap) return rs::fail(RS_E_INVAL, "rs_write_through: " + std::to_string(need) + " pairs, capacity " +
                                                  std::to_string(cap));
  std::vector<int32_t> got(size_t(need) + 1);
  int rc = t->alloc_host(need, got.data());
  if (rc != RS_OK) return rc;
  const int64_t tk = t->next_ticket++;
  int64_t o = 0;
  for (Node* x : todo) {
    const int64_t len = int64_t(x->key.size());
    x->host.assign(got.begin() + o, got.begin() + o + len);
    x->pend = tk;
    std::memcpy(out_dev_slots + o, x->value.data(), size_t(len) * 4);
    std::memcpy(out_host_slots + o, x->host.data(), size_t(len) * 4);
    o += len;
  }
  t->lock(nd);
  t->tickets[tk] = {0, node};
  *out_n = need;
  *out_ticket = tk;
  return RS_OK;
  RS_GUARD_END
}

int rs_load_back(rs_tree* t, int64_t node, int64_t cap, int32_t* out_host_slots, int32_t* out_dev_slots,
                 int64_t* out_n, int64_t* out_ticket) {
  if (!t || cap < 0 || (cap && (!out_dev_slots || !out_host_slots)) || !out_n || !out_ticket)
    return rs::fail(RS_E_INVAL, "rs_load_back: bad arguments");
  if (!t->host) return rs::fail(RS_E_INVAL, "rs_load_back: the host tier is off");
  Node* nd = t->find(node);
  if (!nd) return rs::fail(RS_E_STALE, "rs_load_back: node " + std::to_string(node) + " is gone");
  RS_GUARD_BEGIN
  std::vector<Node*> todo;
  int64_t need = 0;
  for (Node* x : t->path(nd))
    if (x->value.empty()) {
      todo.push_back(x);
      need += int64_t(x->key.size());
    }
  if (need > t->alloc.capacity())
    return rs::fail(RS_E_NOSPACE, "rs_load_back: " + std::to_string(need) + " tokens, pool of " +
                                      std::to_string(t->alloc.capacity()) + " slots");
  if (need > cap) return rs::fail(RS_E_INVAL, "rs_load_back: " + std::to_string(need) + " pairs, capacity " +
                                                  std::to_string(cap));
  t->lock(nd);
  std::vector<int32_t> got(size_t(need) + 1);
  int rc = t->alloc_slots(need, got.data());
  if (rc != RS_OK) {
    t->unlock(nd);
    return rc;
  }
  const int64_t tk = t->next_ticket++;
  int64_t o = 0;
  for (Node* x : todo) {
    const int64_t len = int64_t(x->key.size());
    x->value.assign(got.begin() + o, got.begin() + o + len);
    x->pend = tk;
    t->protected_ += len;                 // the path is locked
    t->tree_tokens += len;
    std::memcpy(out_host_slots + o, x->host.data(), size_t(len) * 4);
    std::memcpy(out_dev_slots + o, x->value.data(), size_t(len) * 4);
    o += len;
  }
  t->tickets[tk] = {1, node};
  *out_n = need;
  *out_ticket = tk;
  return RS_OK;
  RS_GUARD_END
}

int rs_commit(rs_tree* t, int64_t ticket, int32_t success) {
  if (!t) return rs::fail(RS_E_INVAL, "rs_commit: null tree");
  auto it = t->tickets.find(ticket);
  if (it == t->tickets.end()) return rs::fail(RS_E_INVAL, "rs_commit: unknown ticket " + std::to_string(ticket));
  if (it->second.first == 1 && !success)
    return rs::fail(RS_E_INVAL, "rs_commit: a load back is committed after its copy has run");
  RS_GUARD_BEGIN
  const int64_t node = it->second.second;
  Node* nd = t->find(node);               // locked since the transaction began, so still there
  if (!nd) return rs::fail(RS_E_STALE, "rs_commit: node " + std::to_string(node) + " is gone");
  t->tickets.erase(it);
  for (auto& kv : t->nodes) {
    Node* x = kv.second.get();
    if (x->pend != ticket) continue;
    x->pend = 0;
    if (!success) {                       // a write-through that failed: no host copy
      t->host->give_back(x->host.data(), int64_t(x->host.size()));
      x->host.clear();
    }
  }
  return t->unlock(nd);
  RS_GUARD_END
}

int64_t rs_evict_host(rs_tree* t, int64_t num_tokens) {
  if (!t || num_tokens < 0) return rs::fail(RS_E_INVAL, "rs_evict_host: bad arguments");
  if (!t->host) return rs::fail(RS_E_INVAL, "rs_evict_host: the host tier is off");
  RS_GUARD_BEGIN
  return t->evict_host(num_tokens);
  RS_GUARD_END
}

int rs_stats(const rs_tree* t, rs_stats_t* out) {
  if (!t || !out) return rs::fail(RS_E_INVAL, "rs_stats: bad arguments");
  std::memset(out, 0, sizeof(*out));
  out->pool_slots = t->alloc.capacity();
  out->nodes = int64_t(t->nodes.size());
  out->tree_tokens = t->tree_tokens;
  out->evictable = t->evictable;
  out->protected_ = t->protected_;
  out->free_slots = t->alloc.num_free();
  out->evicted_total = t->evicted_total;
  out->clock = int64_t(t->clock);
  out->matched_total = t->matched_total;
  out->match_calls = t->match_calls;
  out->insert_calls = t->insert_calls;
  if (t->host) {
    out->host_slots = t->host->capacity();
    out->host_free = t->host->num_free();
    for (auto& kv : t->nodes) out->host_tokens += int64_t(kv.second->host.size());
  }
  return RS_OK;
}

int rs_tree_dump(const rs_tree* t, char* buf, int64_t cap, int64_t* need) {
  if (!t || !need || cap < 0 || (cap && !buf)) return rs::fail(RS_E_INVAL, "rs_tree_dump: bad arguments");
  RS_GUARD_BEGIN
  std::string s;
  char tmp[96];
  // explicit stack: (node, depth); children pushed in descending first-page order
  std::vector<std::pair<const Node*, int>> st;
  const int32_t ps = t->ps;
  auto push_children = [&](const Node* n, int depth) {
    std::vector<const Node*> kids;
    kids.reserve(n->children.size());
    for (auto& kv : n->children) kids.push_back(kv.second);
    std::sort(kids.begin(), kids.end(), [&](const Node* a, const Node* b) {
      return std::lexicographical_compare(a->key.begin(), a->key.begin() + ps, b->key.begin(), b->key.begin() + ps);
    });
    for (auto it = kids.rbegin(); it != kids.rend(); ++it) st.emplace_back(*it, depth);
  };
  auto field = [&](const std::vector<int32_t>& v) {     // " | " then the numbers, space-separated
    s += " | ";
    for (size_t i = 0; i < v.size(); ++i) {
      if (i) s += ' ';
      s += std::to_string(v[i]);
    }
  };
  push_children(&t->root, 0);
  while (!st.empty()) {
    const Node* c = st.back().first;
    int depth = st.back().second;
    st.pop_back();
    std::snprintf(tmp, sizeof tmp, "%d %lld %d %llu %zu", depth, (long long)c->id, c->lock_ref,
                  (unsigned long long)c->last_access, c->key.size());
    s += tmp;
    field(c->key);
    field(c->value);
    if (t->host) {
      field(c->host);
      s += " | " + std::to_string(c->pend);
    }
    s += '\n';
    push_children(c, depth + 1);
  }
  *need = int64_t(s.size());
  if (cap > 0) {
    int64_t k = std::min<int64_t>(cap - 1, int64_t(s.size()));
    std::memcpy(buf, s.data(), size_t(k));
    buf[k] = 0;
  }
  return RS_OK;
  RS_GUARD_END
}

}  // extern "C"
