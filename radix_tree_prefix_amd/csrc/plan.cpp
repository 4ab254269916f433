// Decode plan: the tree's shared prefixes of a decode batch as work items.
//
// "How does SGLang work" (modernaiengineering.com), section "How the runtime
// and frontend work together": forked requests reach the runtime as
// near-identical requests and their common part is computed once; the
// bibekananda.in page ("One tree for everybody") has every request walk one
// shared tree.  For decode this means the shared prefix KV can be *read* once
// for all requests that share it: a tree node on the root paths of >= 2
// requests of the batch is a shared segment read by one work item for all of
// its requests' query rows; what is left of each request is its unique tail.
//
// Work items (per KV head): a segment's key range is cut into chunks of at
// most `chunk` keys and its requests into row tiles of at most 128 query rows
// (requests x Hq/Hkv heads); each (chunk, row tile) is one item that writes
// one partial (o, lse) per (request, head) of its tile.  A request's partials
// are merged by log-sum-exp.  Items are launched with the KV head fastest so
// that, with 8 KV heads on 8 XCDs, every XCD streams one head's KV and the row
// tiles of one chunk meet in the same L2.

#include <algorithm>
#include <cstring>
#include <map>

#include <hip/hip_runtime.h>

#include "internal.h"
#include "plan.h"

struct rs_plan {
  rs_plan_info_t info{};
  std::vector<int32_t> image;
};

namespace {

struct Seg {
  int32_t start, end, rep;
  std::vector<int32_t> reqs;
};

inline int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

}  // namespace

namespace rs {

WsLayout ws_layout(int64_t n_partials, int32_t B, int32_t Hq, int32_t Hkv, int32_t D) {
  WsLayout w;
  int32_t G = Hq / Hkv;
  w.o_off = 0;
  w.lse_off = align256(w.o_off + int64_t(Hkv) * n_partials * G * D * 4);
  w.bytes = align256(w.lse_off + int64_t(Hkv) * n_partials * G * 4);
  (void)B;
  return w;
}

const rs_plan_info_t* plan_info(const rs_plan* p) { return &p->info; }

PlanOffsets plan_offsets(const rs_plan* p) { return PlanOffsets{p->image[5], p->image[6], p->image[7]}; }

}  // namespace rs

extern "C" {

int rs_decode_plan_build(const rs_tree* t, const int64_t* nodes, const int32_t* cached_lens,
                         const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                         rs_plan** out) {
  if (!t || !nodes || !cached_lens || !seq_lens || !out || B <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 ||
      Hq % Hkv)
    return rs::fail(RS_E_INVAL, "rs_decode_plan_build: bad arguments");
  const int32_t G = Hq / Hkv;
  if (G > rs::kMaxRowsPerItem) return rs::fail(RS_E_UNSUPPORTED, "rs_decode_plan_build: Hq/Hkv > 128");
  try {
    // 1. every request's root path and the requests through each node
    std::vector<std::vector<const rs::Node*>> paths(B);
    std::map<const rs::Node*, std::vector<int32_t>> through;
    std::map<const rs::Node*, int32_t> start_of;
    int64_t flat = 0;
    for (int32_t b = 0; b < B; ++b) {
      const rs::Node* n = t->find(nodes[b]);
      if (!n) return rs::fail(RS_E_STALE, "rs_decode_plan_build: node of request " + std::to_string(b) + " is gone");
      if (seq_lens[b] < 1 || seq_lens[b] < cached_lens[b] || cached_lens[b] < 0)
        return rs::fail(RS_E_INVAL, "rs_decode_plan_build: request " + std::to_string(b) + " has bad lengths");
      for (const rs::Node* x = n; x != &t->root; x = x->parent) paths[b].push_back(x);
      std::reverse(paths[b].begin(), paths[b].end());
      int32_t pos = 0;
      for (const rs::Node* x : paths[b]) {
        start_of[x] = pos;
        pos += int32_t(x->key.size());
        through[x].push_back(b);
      }
      if (pos != cached_lens[b])
        return rs::fail(RS_E_INVAL, "rs_decode_plan_build: node of request " + std::to_string(b) +
                                        " covers " + std::to_string(pos) + " tokens, cached_lens says " +
                                        std::to_string(cached_lens[b]));
      flat += seq_lens[b];
    }
    // 2. shared segments (a parent-child chain with one request set is one segment)
    std::vector<Seg> segs;
    std::map<const rs::Node*, int32_t> seg_of;
    std::vector<int32_t> uniq_from(B, 0);
    for (int32_t b = 0; b < B; ++b) {
      for (const rs::Node* x : paths[b]) {
        const auto& rq = through[x];
        if (rq.size() < 2) break;
        int32_t end = start_of[x] + int32_t(x->key.size());
        uniq_from[b] = end;
        if (seg_of.count(x)) continue;
        const rs::Node* p = x->parent;
        if (p != &t->root && through[p].size() == rq.size()) {
          int32_t s = seg_of[p];
          segs[s].end = end;
          seg_of[x] = s;
        } else {
          seg_of[x] = int32_t(segs.size());
          segs.push_back(Seg{start_of[x], end, rq[0], rq});
        }
      }
    }
    const int32_t n_shared = int32_t(segs.size());
    for (int32_t b = 0; b < B; ++b)
      if (seq_lens[b] > uniq_from[b]) segs.push_back(Seg{uniq_from[b], seq_lens[b], b, {b}});

    // 3. chunk size: spread the (keys x row tiles) work over enough items to fill the chip
    const int32_t rpt = std::max(1, rs::kMaxRowsPerItem / G);         // requests per row tile
    int64_t work = 0, uniq = 0;
    for (auto& s : segs) {
      int64_t tiles = (int64_t(s.reqs.size()) + rpt - 1) / rpt;
      work += int64_t(s.end - s.start) * tiles;
      uniq += s.end - s.start;
    }
    const int64_t target = std::max<int64_t>(1, rs::kDecodeItemsTarget / Hkv);
    int64_t chunk = (work + target - 1) / target;
    chunk = std::min<int64_t>(std::max<int64_t>((chunk + 63) / 64 * 64, rs::kMinChunk), rs::kMaxChunk);

    // 4. items; item_req entries {request, partial index, partials of the request, 0}.  A
    // request's partials are numbered consecutively (part_ptr[b] .. part_ptr[b+1]-1), so the
    // merge finds them without a list.
    std::vector<int32_t> items, item_req;
    std::vector<int32_t> n_parts(B, 0);
    int32_t n_items = 0;
    for (auto& s : segs) {
      int32_t len = s.end - s.start;
      int32_t nch = int32_t((len + chunk - 1) / chunk);
      int32_t per = ((len + nch - 1) / nch + rs::kChunkAlign - 1) / rs::kChunkAlign * rs::kChunkAlign;
      int32_t nreq = int32_t(s.reqs.size());
      for (int32_t k0 = s.start; k0 < s.end; k0 += per) {
        int32_t k1 = std::min(s.end, k0 + per);
        for (int32_t r0 = 0; r0 < nreq; r0 += rpt) {
          int32_t nr = std::min(rpt, nreq - r0);
          int32_t req_off = int32_t(item_req.size() / rs::kItemReqWords);
          for (int32_t j = 0; j < nr; ++j) {
            int32_t b = s.reqs[r0 + j];
            int32_t e[rs::kItemReqWords] = {b, n_parts[b]++, 0, 0};   // local index for now
            item_req.insert(item_req.end(), e, e + rs::kItemReqWords);
          }
          int32_t it[rs::kItemWords] = {k0, k1, s.rep, nr, req_off, 0, 0, 0};
          items.insert(items.end(), it, it + rs::kItemWords);
          ++n_items;
        }
      }
    }
    std::vector<int32_t> part_ptr(B + 1, 0);
    for (int32_t b = 0; b < B; ++b) part_ptr[b + 1] = part_ptr[b] + n_parts[b];
    const int64_t P = part_ptr[B];
    for (size_t e = 0; e < item_req.size(); e += rs::kItemReqWords) {
      const int32_t b = item_req[e];
      item_req[e + 1] += part_ptr[b];
      item_req[e + 2] = n_parts[b];
    }
    if (P >= (int64_t(1) << 31) / (int64_t(G) * D * Hkv))
      return rs::fail(RS_E_UNSUPPORTED, "rs_decode_plan_build: batch too large for one plan");

    // the longest items first (their keys are the memory traffic), so that no long item
    // starts late and runs on an otherwise idle chip; items are independent
    {
      std::vector<int32_t> ord(n_items);
      for (int32_t i = 0; i < n_items; ++i) ord[i] = i;
      auto keys_of = [&](int32_t i) { return items[size_t(i) * rs::kItemWords + 1] - items[size_t(i) * rs::kItemWords]; };
      std::stable_sort(ord.begin(), ord.end(), [&](int32_t x, int32_t y) { return keys_of(x) > keys_of(y); });
      std::vector<int32_t> sorted(items.size());
      for (int32_t i = 0; i < n_items; ++i)
        std::copy_n(items.begin() + size_t(ord[i]) * rs::kItemWords, rs::kItemWords,
                    sorted.begin() + size_t(i) * rs::kItemWords);
      items.swap(sorted);
    }

    // 5. device image
    auto p = std::make_unique<rs_plan>();
    std::vector<int32_t>& img = p->image;
    img.assign(rs::kPlanHeaderWords, 0);
    img[0] = rs::kPlanMagic;
    img[1] = n_items;
    img[2] = B;
    img[3] = G;
    img[4] = int32_t(P);
    img[5] = int32_t(img.size());
    img.insert(img.end(), items.begin(), items.end());
    img[6] = int32_t(img.size());                    // 16-byte aligned: header and items are whole vectors
    img.insert(img.end(), item_req.begin(), item_req.end());
    img[7] = int32_t(img.size());
    img.insert(img.end(), part_ptr.begin(), part_ptr.end());
    while (img.size() % 4) img.push_back(0);

    rs_plan_info_t& in = p->info;
    in.B = B; in.Hq = Hq; in.Hkv = Hkv; in.D = D;
    in.n_items = n_items;
    in.n_segments = int32_t(segs.size());
    in.n_shared = n_shared;
    in.chunk = int32_t(chunk);
    in.n_partials = P;
    in.unique_kv_tokens = uniq;
    in.flat_kv_tokens = flat;
    in.bytes = int64_t(img.size()) * 4;
    *out = p.release();
    return RS_OK;
  } catch (const std::exception& e) {
    return rs::fail(RS_E_INVAL, std::string("rs_decode_plan_build: ") + e.what());
  }
}

int rs_plan_info(const rs_plan* p, rs_plan_info_t* out) {
  if (!p || !out) return rs::fail(RS_E_INVAL, "rs_plan_info: bad arguments");
  *out = p->info;
  return RS_OK;
}

int64_t rs_decode_plan_bytes(const rs_plan* p) {
  if (!p) return rs::fail(RS_E_INVAL, "rs_decode_plan_bytes: null plan");
  return p->info.bytes;
}

int rs_decode_plan_upload(const rs_plan* p, void* dev, void* stream) {
  if (!p || !dev || (reinterpret_cast<uintptr_t>(dev) & 15))
    return rs::fail(RS_E_INVAL, "rs_decode_plan_upload: bad arguments (device buffer must be 16-byte aligned)");
  hipError_t e = hipMemcpyAsync(dev, p->image.data(), size_t(p->info.bytes), hipMemcpyHostToDevice,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return rs::fail(RS_E_HIP, std::string("rs_decode_plan_upload: ") + hipGetErrorString(e));
  return RS_OK;
}

int rs_decode_plan_read(const rs_plan* p, void* host, int64_t bytes) {
  if (!p || !host || bytes < p->info.bytes) return rs::fail(RS_E_INVAL, "rs_decode_plan_read: bad arguments");
  std::memcpy(host, p->image.data(), size_t(p->info.bytes));
  return RS_OK;
}

void rs_plan_destroy(rs_plan* p) { delete p; }

int rs_extend_order(const int32_t* prefix_lens, const int32_t* extend_lens, int32_t B, int32_t* order) {
  if (B < 0 || (B && (!prefix_lens || !extend_lens || !order))) return rs::fail(RS_E_INVAL, "rs_extend_order: bad arguments");
  std::vector<std::pair<int64_t, int32_t>> w(B);
  for (int32_t b = 0; b < B; ++b) {
    const int64_t e = extend_lens[b];
    w[b] = {-(e * (int64_t(prefix_lens[b]) + (e + 1) / 2)), b};
  }
  std::sort(w.begin(), w.end());
  for (int32_t b = 0; b < B; ++b) order[b] = w[b].second;
  return RS_OK;
}

int64_t rs_decode_workspace_bytes(const rs_plan* p, int32_t B, int32_t max_seq_len, int32_t Hq,
                                  int32_t Hkv, int32_t D) {
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv) return rs::fail(RS_E_INVAL, "rs_decode_workspace_bytes: bad heads");
  if (p) {
    if (p->info.Hq != Hq || p->info.Hkv != Hkv || p->info.D != D)
      return rs::fail(RS_E_INVAL, "rs_decode_workspace_bytes: heads differ from the plan's");
    return rs::ws_layout(p->info.n_partials, p->info.B, Hq, Hkv, D).bytes;
  }
  if (B <= 0 || max_seq_len <= 0) return rs::fail(RS_E_INVAL, "rs_decode_workspace_bytes: bad sizes");
  int64_t nch = (int64_t(max_seq_len) + rs::kFlatChunk - 1) / rs::kFlatChunk;
  return rs::ws_layout(int64_t(B) * nch, B, Hq, Hkv, D).bytes;
}

}  // extern "C"
