// Draft tree of a speculative verify step.
//
// Follows "SGLang: the tree, and the language nobody remembers" (ai.thesatyajit.com),
// section "Speculative decoding puts a tree inside the tree": the verify tokens form a
// tree; the attention of one target pass needs, per token, a mask of its own ancestors
// (each draft token attends only to its ancestors, so every branch is an independent
// continuation), a position equal to the prompt length plus its depth, and the tree in
// first-child / next-sibling form.
//
// Readings where the page is silent: token 0 is the root (the last verified token,
// depth 0) and every other token's parent has a smaller index; a token's mask holds
// itself and its ancestors; children are listed in index order.

#include <string>

#include "internal.h"

extern "C" int rs_draft_tree_build(const int32_t* parents, const int32_t* prefix_lens, int32_t B, int32_t n,
                                   uint64_t* tree_mask, int32_t* positions, int32_t* next_token,
                                   int32_t* next_sibling) {
  if (B < 0 || n < 0 || n > 64) return rs::fail(RS_E_INVAL, "rs_draft_tree_build: bad sizes");
  if (B == 0 || n == 0) return RS_OK;
  if (!parents || !prefix_lens || !tree_mask || !positions || !next_token || !next_sibling)
    return rs::fail(RS_E_INVAL, "rs_draft_tree_build: null pointer");
  for (int32_t b = 0; b < B; ++b) {
    const int32_t* par = parents + int64_t(b) * n;
    if (par[0] != -1) return rs::fail(RS_E_INVAL, "rs_draft_tree_build: token 0 must be the root (parent -1)");
    for (int32_t i = 1; i < n; ++i)
      if (par[i] < 0 || par[i] >= i)
        return rs::fail(RS_E_INVAL, "rs_draft_tree_build: request " + std::to_string(b) + " token " +
                                        std::to_string(i) + " has parent " + std::to_string(par[i]) +
                                        " (must be in 0.." + std::to_string(i - 1) + ")");
    if (prefix_lens[b] < 0) return rs::fail(RS_E_INVAL, "rs_draft_tree_build: negative prefix length");
  }
  for (int32_t b = 0; b < B; ++b) {
    const int64_t o = int64_t(b) * n;
    const int32_t* par = parents + o;
    int32_t last_child[64];
    for (int32_t i = 0; i < n; ++i) {
      next_token[o + i] = -1;
      next_sibling[o + i] = -1;
      last_child[i] = -1;
    }
    for (int32_t i = 0; i < n; ++i) {
      const int32_t p = par[i];
      // parents precede children, so the parent's mask and depth are final
      tree_mask[o + i] = (p < 0 ? 0ull : tree_mask[o + p]) | (1ull << i);
      positions[o + i] = p < 0 ? prefix_lens[b] : positions[o + p] + 1;
      if (p >= 0) {
        if (last_child[p] < 0) next_token[o + p] = i;
        else next_sibling[o + last_child[p]] = i;
        last_child[p] = i;
      }
    }
  }
  return RS_OK;
}
