// Internal declarations shared by the host core and the device ops of librs.
#pragma once

#include <cstdint>
#include <memory>
#include <string>
#include <unordered_map>
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
  std::vector<int32_t> value;   // one pool slot per key token
  Node* parent = nullptr;
  std::unordered_map<int32_t, Node*> children;  // keyed on the child's first token
  int32_t lock_ref = 0;
  uint64_t last_access = 0;
  int64_t priority = 0;
};

// Lowest-free-first slot allocator over a bitmap (1 = free) with a word hint.
class SlotAllocator {
 public:
  explicit SlotAllocator(int64_t n);
  int64_t capacity() const { return n_; }
  int64_t num_free() const { return nfree_; }
  // Takes the k lowest free slots; caller checked k <= num_free().
  void take(int64_t k, int32_t* out);
  // Returns false (and changes nothing) if any slot is out of range or already free.
  bool give_back(const int32_t* s, int64_t k);
  bool is_free(int32_t s) const { return (bits_[s >> 6] >> (s & 63)) & 1ull; }

 private:
  int64_t n_, nfree_, hint_;
  std::vector<uint64_t> bits_;
};

}  // namespace rs

struct rs_tree {
  explicit rs_tree(int64_t pool_slots);

  rs::Node root;
  std::unordered_map<int64_t, std::unique_ptr<rs::Node>> nodes;   // id -> node (root excluded)
  rs::SlotAllocator alloc;
  int64_t next_id = 1;
  uint64_t clock = 0;
  int64_t evictable = 0, protected_ = 0, evicted_total = 0, tree_tokens = 0;
  int64_t matched_total = 0, match_calls = 0, insert_calls = 0;

  rs::Node* find(int64_t id);                      // nullptr if stale; root for 0
  const rs::Node* find(int64_t id) const;
  rs::Node* split(rs::Node* child, int64_t k);      // returns the new upper node
  int64_t match(const int32_t* tok, int64_t n, int32_t* out, rs::Node** end);
  // returns prefix length; slots in/out; frees differing caller slots
  int insert(const int32_t* tok, int32_t* slots, int64_t n, int64_t* prefix, rs::Node** end);
  void lock(rs::Node* nd);
  int unlock(rs::Node* nd);
  int64_t evict(int64_t need);
  int alloc_slots(int64_t n, int32_t* out);
  int64_t depth_tokens(const rs::Node* nd) const;
};
