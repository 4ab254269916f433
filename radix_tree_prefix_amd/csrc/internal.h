// Internal declarations shared by the host core and the device ops of librs.
#pragma once

#include <cstdint>
#include <map>
#include <memory>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "rs.h"

namespace rs {

// Thread-local last error; every ABI entry point stores its failure message here.
void set_error(const std::string& msg);
void clear_error();
int fail(int code, const std::string& msg);

// Index of the first position where a[0..n) and b[0..n) differ (n if none).
int64_t diverge(const int32_t* a, const int32_t* b, int64_t n);

// ---------------------------------------------------------------- radix tree

struct Node {
  int64_t id = 0;
  std::vector<int32_t> key;     // token run on the edge into this node
  std::vector<int32_t> value;   // one pool slot per key token; empty: the node is on the host only
  std::vector<int32_t> host;    // host-tier slots; empty: no host copy
  int64_t pend = 0;             // ticket of a copy in flight (0: none)
  Node* parent = nullptr;
  // keyed on the child's first token; with pages > 1 token, siblings may share it and
  // differ later in their first page (the page is the key)
  std::unordered_multimap<int32_t, Node*> children;
  int32_t lock_ref = 0;
  uint64_t last_access = 0;
  int64_t priority = 0;
};

// Lowest-free-first allocator of pages of ps slots (page p = slots p*ps .. p*ps+ps-1)
// over a slot bitmap (1 = free; a page's bits always agree) with a word hint.
class SlotAllocator {
 public:
  SlotAllocator(int64_t n, int32_t ps);
  int64_t capacity() const { return n_; }
  int64_t num_free() const { return nfree_; }     // slots (whole free pages)
  int32_t page() const { return ps_; }
  // Takes the ceil(k/ps) lowest free pages and writes their first k slots, page-major;
  // caller checked ceil(k/ps)*ps <= num_free().
  void take(int64_t k, int32_t* out);
  // Frees the pages that hold these slots (a page named twice is freed once).  Returns
  // false (and changes nothing) if a slot is out of range or its page is already free.
  bool give_back(const int32_t* s, int64_t k);
  bool is_free(int32_t s) const { return (bits_[s >> 6] >> (s & 63)) & 1ull; }

 private:
  void set_page(int64_t p0, bool free_);
  int64_t n_, nfree_, hint_;
  int32_t ps_;
  std::vector<uint64_t> bits_;
};

}  // namespace rs

struct rs_tree {
  rs_tree(int64_t pool_slots, int32_t page_size);

  rs::Node root;
  std::unordered_map<int64_t, std::unique_ptr<rs::Node>> nodes;   // id -> node (root excluded)
  rs::SlotAllocator alloc;
  std::unique_ptr<rs::SlotAllocator> host;          // host tier (null until enabled)
  std::map<int64_t, std::pair<int, int64_t>> tickets;  // ticket -> (0 write / 1 load, locked node)
  int64_t next_ticket = 1;
  int64_t next_id = 1;
  uint64_t clock = 0;
  int64_t evictable = 0, protected_ = 0, evicted_total = 0, tree_tokens = 0;
  int64_t matched_total = 0, match_calls = 0, insert_calls = 0;

  rs::Node* find(int64_t id);                      // nullptr if stale; root for 0
  const rs::Node* find(int64_t id) const;
  int32_t ps;                                       // page size (tokens per child key and slot page)
  // the child of n whose first page is page[0..ps) (nullptr if none)
  rs::Node* child_at(const rs::Node* n, const int32_t* page) const;
  void link(rs::Node* parent, rs::Node* c);
  void unlink(rs::Node* parent, rs::Node* c);
  rs::Node* split(rs::Node* child, int64_t k);      // returns the new upper node
  int64_t match(const int32_t* tok, int64_t n, int32_t* out, rs::Node** end);
  // returns prefix length; slots in/out; frees differing caller slots
  int insert(const int32_t* tok, int32_t* slots, int64_t n, int64_t* prefix, rs::Node** end);
  void lock(rs::Node* nd);
  int unlock(rs::Node* nd);
  int64_t evict(int64_t need);
  int64_t evict_host(int64_t need);
  void drop_host_subtree(rs::Node* x);            // frees and unlinks x's (host-only) descendants
  int alloc_host(int64_t n, int32_t* out);
  bool device_leaf(const rs::Node* n) const;
  std::vector<rs::Node*> path(rs::Node* nd);        // root's child .. nd
  int alloc_slots(int64_t n, int32_t* out);
  int64_t depth_tokens(const rs::Node* nd) const;
};
