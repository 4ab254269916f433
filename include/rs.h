/*
 * rs.h -- C ABI of librs: RadixAttention's data-parallel hot path on one MI355X.
 *
 * A host radix tree over token prefixes indexes one token-granular KV pool, so
 * requests that share a prefix point at the same pool slots and the shared KV
 * is computed once.  Index tables built from the tree drive hand-written HIP
 * kernels for gfx950: extend attention (prefill of only the unmatched suffix)
 * and prefix-aware decode attention.
 *
 * Sources (pages, with section):
 *  [T]  "SGLang: the tree, and the language nobody remembers" (ai.thesatyajit.com),
 *       "A tree, not a map": node fields, split at divergence, lock_ref accounting,
 *       heap eviction with cascade, page-1 child keys, galloping match.
 *  [B]  "SGLang" (bibekananda.in), "One tree for everybody", "Eviction on a tree".
 *  [L]  "How does SGLang work" (modernaiengineering.com): "A quick recap ..."
 *       (prefill/decode, KV depends only on the prefix), "What happens when a
 *       request arrives" (match, lock, prefill the rest, insert, unlock),
 *       "Worked example, step by step" (LRU among unlocked leaves, whole nodes,
 *       wait when nothing is evictable).
 *  [P]  "SGLang" (llmdeepdive.com, lesson 8.5), "Conceito": the pool of blocks as
 *       a radix tree keyed by token ids; allocate only for the divergent suffix.
 *
 * Conventions for every call:
 *  - Return value: RS_OK (0) or a negative RS_E_* code; calls returning a count
 *    return it (>= 0) or a negative code.  rs_last_error() gives a message for
 *    the calling thread's last failure.  Nothing throws across the ABI.
 *  - Ownership: the library owns only rs_tree and rs_plan objects (and hands out
 *    pinned host blocks from rs_host_alloc, which the caller then owns).  Every array
 *    argument is owned by the caller and only read or written during the call,
 *    except device arrays of asynchronous calls (see below).
 *  - Host vs device: "host" arrays are ordinary CPU memory; "device" arrays are
 *    device memory of the current HIP device.  `stream` is a hipStream_t (NULL =
 *    the default stream).  Device calls enqueue work and return without waiting;
 *    their device arrays must stay valid until the stream reaches that point.
 *  - A tree or plan handle must not be used by two threads at once.
 *  - Node ids are int64, never reused; the root is 0.  A node id whose node has
 *    been evicted is stale (RS_E_STALE).
 *  - Layouts: K and V pools are [pool_slots][Hkv][D] row-major (one slot's row is
 *    Hkv*D contiguous elements).  Index tables are int32 [B][ld] row-major; entry
 *    (b, j) is the pool slot of position j of request b.  Query head h reads KV
 *    head h / (Hq/Hkv).
 *  - dtype: RS_DTYPE_F32 or RS_DTYPE_BF16 (bfloat16 bits).  Supported head dims:
 *    64 and 128; Hq % Hkv == 0; Hq/Hkv <= 128.
 */
#ifndef RS_H_
#define RS_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  RS_OK = 0,
  RS_E_INVAL = -1,        /* bad argument or call sequence */
  RS_E_NOSPACE = -2,      /* slots cannot be found even after eviction: the request waits [L] */
  RS_E_STALE = -3,        /* node id no longer in the tree */
  RS_E_HIP = -4,          /* a HIP runtime call failed */
  RS_E_UNSUPPORTED = -5   /* shape or dtype outside what the kernels implement */
};

enum { RS_DTYPE_F32 = 0, RS_DTYPE_BF16 = 1 };

typedef struct rs_tree rs_tree;
typedef struct rs_plan rs_plan;

typedef struct rs_stats_t {
  int64_t pool_slots;
  int64_t nodes;          /* excluding the root */
  int64_t tree_tokens;    /* sum of key lengths */
  int64_t evictable;      /* tokens in nodes with lock_ref == 0 [T] */
  int64_t protected_;     /* tokens in nodes with lock_ref > 0 [T] */
  int64_t free_slots;
  int64_t evicted_total;  /* tokens freed by eviction since creation */
  int64_t clock;          /* logical clock: +1 per match or insert call */
  int64_t matched_total;  /* tokens returned by rs_match_prefix since creation */
  int64_t match_calls;
  int64_t insert_calls;
  int64_t host_slots;     /* host tier size (0: off) */
  int64_t host_tokens;    /* tokens with a host copy */
  int64_t host_free;      /* free host slots */
  int64_t reserved[2];
} rs_stats_t;

typedef struct rs_plan_info_t {
  int32_t B, Hq, Hkv, D;
  int32_t n_items;          /* work items per KV head (grid x of the decode launch) */
  int32_t n_segments;       /* segments: shared ones first, then one unique tail per request */
  int32_t n_shared;         /* segments read by >= 2 requests */
  int32_t chunk;            /* keys per work item (last chunk of a segment may be shorter) */
  int64_t n_partials;       /* partial (o, lse) records per KV head per query head of a group */
  int64_t unique_kv_tokens; /* distinct positions read: sum of segment lengths */
  int64_t flat_kv_tokens;   /* sum of seq_lens: what a per-request read would touch */
  int64_t bytes;            /* size of the device image rs_decode_plan_upload writes */
  int64_t reserved[4];
} rs_plan_info_t;

/* Message for the calling thread's last failure ("" if none). */
const char* rs_last_error(void);
const char* rs_version(void);

/* ------------------------------------------------------------------ tree [T][B][L] */

/* New empty tree over pool slots 0..pool_slots-1, all free.  page_size >= 1 must divide
 * pool_slots.  page_size 1: token-granular, children keyed on their first token [T].
 * page_size ps > 1 [T "A tree, not a map", the details from the source]: keys are
 * truncated to whole pages, a match is rounded down to a page, children are keyed on
 * their first page (siblings may share a first token), and slots come in whole pages
 * (page p = slots p*ps .. p*ps+ps-1; position j of a sequence sits at offset j % ps of
 * its page).  NULL on failure. */
rs_tree* rs_tree_create(int64_t pool_slots, int32_t page_size);
void rs_tree_destroy(rs_tree* t);

/* Longest cached prefix of tokens[0..n) [B "One tree for everybody"].  Walks from the
 * root comparing edges with a galloping search [T]; if the match ends inside an edge the
 * node is split there (the upper part gets a fresh id and the lower part's lock_ref and
 * last_access; the lower part keeps its id) [T].  Every node visited gets the current
 * clock tick.  Writes the matched slots to out_slots (host, capacity >= n), their count
 * to *out_len and the node the match ends at to *out_node (0 = root, empty match). */
/* With pages the match is a whole number of pages. */
int rs_match_prefix(rs_tree* t, const int32_t* tokens, int64_t n,
                    int32_t* out_slots, int64_t* out_len, int64_t* out_node);

/* lock_ref +1 / -1 on node and every ancestor up to the root.  On the 0->1 edge a
 * node's key length moves from evictable to protected, and back on 1->0 [T].
 * rs_dec_lock_ref on a node whose lock_ref is 0 is RS_E_INVAL (nothing changes). */
int rs_inc_lock_ref(rs_tree* t, int64_t node);
int rs_dec_lock_ref(rs_tree* t, int64_t node);

/* n free slots, lowest ids first, ascending, into out_slots (host).  When fewer than
 * n are free, first evicts (n - free) tokens; if still short, RS_E_NOSPACE: nothing is
 * allocated, and what was evicted stays evicted [L "Worked example"].  With pages: the
 * ceil(n/ps) lowest free pages are taken (the end of the last one belongs to the caller
 * too) and the first n of their slots written, page by page; eviction counts pages. */
int rs_alloc_slots(rs_tree* t, int64_t n, int32_t* out_slots);

/* Return slots that were allocated and never inserted.  Freeing a free slot is RS_E_INVAL.
 * With pages the pages holding the slots are freed (a page named twice, once). */
int rs_free_slots(rs_tree* t, const int32_t* slots, int64_t n);

/* Insert tokens[0..n) with slots[0..n) (host, in/out) [L step 4].  Splits at the
 * divergence point like match.  Positions already in the tree keep the tree's slots:
 * a caller slot that differs is freed and overwritten with the tree's.  The rest,
 * slots[prefix..n), is adopted by one new leaf.  Returns the count already present
 * in *out_prefix_len and the node the sequence ends at in *out_node.  With pages only
 * the whole pages of tokens[0..n) are inserted (the caller keeps the rest), and their
 * slots must be whole pages aligned with the positions (RS_E_INVAL otherwise). */
int rs_insert(rs_tree* t, const int32_t* tokens, int32_t* slots, int64_t n,
              int64_t* out_prefix_len, int64_t* out_node);

/* Evict whole unlocked leaves, least (priority, last_access, node id) first, pushing a
 * parent that becomes childless and unlocked, until num_tokens are freed or nothing is
 * evictable [T][B "Eviction on a tree"][L].  Returns tokens freed (may exceed num_tokens). */
int64_t rs_evict(rs_tree* t, int64_t num_tokens);

/* One request's admission [L "What happens when a request arrives"]: match
 * tokens[0..cached) and lock that node; allocate slots for the unmatched part of the
 * cached tokens (to be re-prefilled), insert them and move the lock to the node the
 * cached tokens end at; allocate n_new slots for the tokens this step computes.
 * out_row (host, capacity cached + n_new) receives the request's index-table row.
 * *out_node = the locked node; *out_matched = tokens matched (positions
 * matched..cached+n_new-1 need their KV written).  On RS_E_NOSPACE the request holds
 * no lock and no slots; tokens it already inserted stay cached.  With pages the locked
 * node covers the whole pages of the cached tokens; the request keeps its last page when
 * the cached tokens end inside it (their slots are in out_row), the new tokens continue
 * that page before taking fresh pages, and the caller frees the last page with
 * rs_free_slots when the request ends. */
int rs_admit(rs_tree* t, const int32_t* tokens, int64_t cached, int64_t n_new,
             int32_t* out_row, int64_t* out_node, int64_t* out_matched);

/* Counters of the tree [T "A tree, not a map": the tree keeps the tokens of unlocked nodes as
 * evictable and those of locked nodes as protected, moving a node's length between the two
 * when its lock_ref goes 0 <-> 1]: evictable and protected tokens, nodes, free slots, tokens
 * evicted so far, the logical clock and match statistics (rs_stats_t).  RS_E_INVAL on NULL. */
int rs_stats(const rs_tree* t, rs_stats_t* out);

/* Canonical text of the tree, an inspection aid for tests (no passage defines a format; the
 * fields printed are the pages' node fields [T "A tree, not a map"]): depth-first from the root, children in
 * ascending first-token order, one line per node
 * "depth id lock_ref last_access len | key tokens | slots\n".
 * Writes at most cap bytes (NUL-terminated if room) and the full size (excluding
 * the NUL) to *need. */
int rs_tree_dump(const rs_tree* t, char* buf, int64_t cap, int64_t* need);

/* ------------------------------------------------------------------ host tier */

/* A second tier of host_slots slots in host memory [T "What the C++ tree is actually
 * for": a two-tier cache with asynchronous copies resolved by a later commit; nodes on the
 * GPU, on the CPU or both].  The library keeps the host slot ids; the caller owns the host
 * K/V pools ([host_slots][Hkv][D] each, pinned so that rs_copy_kv can reach them) and moves
 * the rows.  Page size 1 only (RS_E_UNSUPPORTED otherwise); at most once per tree.
 * With the tier on, device eviction keeps a node that has a finished host copy, on the host
 * only; rs_match_prefix stops at such nodes; rs_insert over them gives them the caller's
 * device slots again.  A node is on the host only after its device slots were evicted, and
 * every node below it is then on the host only too. */
int rs_host_tier_enable(rs_tree* t, int64_t host_slots);

/* Like rs_match_prefix, continued through nodes that are on the host only (split and
 * touched the same way): *out_dev_len tokens are on the device (slots in out_dev_slots,
 * node *out_dev_node), *out_len in total; out_host_slots receives the host slots of
 * positions *out_dev_len .. *out_len-1, *out_node is the node the match ends at.
 * Needs the host tier (RS_E_INVAL if it is off) and page size 1 (RS_E_UNSUPPORTED
 * otherwise); a refused call leaves the tree unchanged. */
int rs_match_prefix2(rs_tree* t, const int32_t* tokens, int64_t n, int32_t* out_dev_slots,
                     int32_t* out_host_slots, int64_t* out_dev_len, int64_t* out_len,
                     int64_t* out_dev_node, int64_t* out_node);

/* Write-through: host slots for every node on node's root path that has no host copy (the
 * path must be on the device), evicting host-only leaves, least recently used first, to
 * fit (RS_E_NOSPACE if it cannot: what was evicted stays evicted, nothing else changes; a path
 * longer than the whole tier fails before anything is evicted).  Writes the (device slot, host slot)
 * pairs to copy, *out_n of them (host arrays of capacity cap), and a ticket; the path stays
 * locked and the copies count as in flight until rs_commit(ticket). */
int rs_write_through(rs_tree* t, int64_t node, int64_t cap, int32_t* out_dev_slots,
                     int32_t* out_host_slots, int64_t* out_n, int64_t* out_ticket);

/* Load back: device slots (rs_alloc_slots rules, evicting to fit; RS_E_NOSPACE: what was
 * evicted stays evicted, nothing else changes; more than the whole pool fails before evicting) for every node on node's root path that is on the host only; writes the (host slot,
 * device slot) pairs to copy and a ticket; the path stays locked until rs_commit(ticket). */
int rs_load_back(rs_tree* t, int64_t node, int64_t cap, int32_t* out_host_slots,
                 int32_t* out_dev_slots, int64_t* out_n, int64_t* out_ticket);

/* Resolve a ticket.  A write-through is committed once its copies are done (success != 0)
 * or abandoned (success == 0: its host slots are freed).  A load back is committed with
 * success != 0 once its copies have run (RS_E_INVAL otherwise; nothing changes): only the
 * write-through's commit carries an outcome in the interface the page prints.  Until then its
 * nodes already hold their device slots, so a match may return them: kernels that read those
 * rows must be ordered after the copy (same stream, or an event).  The path is unlocked. */
int rs_commit(rs_tree* t, int64_t ticket, int32_t success);

/* Drop host-only leaves, least (priority, last_access, id) first, until num_tokens host
 * slots are free; returns the number freed. */
int64_t rs_evict_host(rs_tree* t, int64_t num_tokens);

/* ------------------------------------------------------------------ scheduling */

/* Order of a waiting queue [T "The scheduler is where the cache is won or lost"].
 * Request i's tokens are tokens[offsets[i] .. offsets[i+1]) (host; offsets has n+1
 * non-decreasing entries).  Each request's longest cached prefix is found without
 * changing the tree (no split, no clock tick) and written to out_matched[i] (host,
 * nullable).  out_order (host, n) receives a permutation of 0..n-1, first to run first:
 *  RS_SCHED_FCFS        arrival order;
 *  RS_SCHED_LPM         longest cached prefix first, ties in arrival order.  A request
 *                       whose cached prefix is <= RS_SCHED_IN_QUEUE_THRESHOLD tokens and
 *                       which shares that many leading tokens with an earlier such request
 *                       (not itself put back) goes to the back, in arrival order, so that
 *                       the earlier one fills the cache first.  Above
 *                       RS_SCHED_LPM_MAX_QUEUE requests: arrival order;
 *  RS_SCHED_DFS_WEIGHT  depth-first over the tree: a request hangs off the deepest node
 *                       whose whole root path it matches; a node weighs the requests in
 *                       its subtree; children of larger weight first (equal: ascending
 *                       first token), a node's own requests after its subtrees, in
 *                       arrival order.
 * The tree is only read.  RS_E_INVAL for bad arguments or an unknown policy. */
enum { RS_SCHED_FCFS = 0, RS_SCHED_LPM = 1, RS_SCHED_DFS_WEIGHT = 2 };
#define RS_SCHED_LPM_MAX_QUEUE 128
#define RS_SCHED_IN_QUEUE_THRESHOLD 32
int rs_schedule(const rs_tree* t, const int32_t* tokens, const int64_t* offsets, int32_t n,
                int32_t policy, int32_t* out_order, int64_t* out_matched);

/* ------------------------------------------------------------------ decode plan */

/* Segments of a decode batch from the tree [L "How the runtime and frontend work
 * together": forked requests reach the runtime as near-identical requests and their
 * common part is computed once].  Request b (table row b) holds a lock on nodes[b],
 * whose root path covers positions 0..cached_lens[b]-1 (with pages: the whole pages of
 * its cached tokens, which is what rs_admit locks); seq_lens[b] >= cached_lens[b]
 * is its context including the new token(s).  A tree node on the paths of >= 2
 * requests becomes a shared segment (a parent-child chain with one request set is one
 * segment); the rest of each request, up to seq_lens[b], is its unique tail.  Segments
 * are cut into key chunks and row tiles (<= 128 query rows = requests x Hq/Hkv) that
 * form the work items of rs_decode_attention.  The plan only reads the tree. */
int rs_decode_plan_build(const rs_tree* t, const int64_t* nodes, const int32_t* cached_lens,
                         const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D,
                         rs_plan** out);
int rs_plan_info(const rs_plan* p, rs_plan_info_t* out);
/* Size of the plan's device image; rs_decode_plan_upload copies it to dev (device,
 * >= that many bytes, 16-byte aligned) on stream.  The plan must stay alive until
 * the copy is done. */
int64_t rs_decode_plan_bytes(const rs_plan* p);
int rs_decode_plan_upload(const rs_plan* p, void* dev, void* stream);
/* Copy the device image into host memory (bytes >= rs_decode_plan_bytes), for inspection.
 * int32 words: header[16] = {magic, n_items, B, G, n_partials, off_items, off_item_req,
 * off_part_ptr, 0...}; items[n_items][8] = {k0, k1, rep_row, n_req, req_off, 0, 0, 0}
 * (keys k0..k1-1 of table row rep_row for the requests of item_req[req_off..+n_req));
 * item_req[][4] = {request b, partial index, partials of b, 0}; part_ptr[B+1]: request b's
 * partials are part_ptr[b] .. part_ptr[b+1]-1, one per item that covers it. */
int rs_decode_plan_read(const rs_plan* p, void* host, int64_t bytes);
void rs_plan_destroy(rs_plan* p);

/* Workspace bytes rs_decode_attention needs: one partial (o, lse) per (work item,
 * request, query head) in fp32.  plan = NULL sizes the flat (one segment per request)
 * mode for B requests of up to max_seq_len tokens.  The pages define no workspace: it holds
 * the per-chunk results that the log-sum-exp combine (written out at rs_decode_attention)
 * joins, the structure that lets a shared segment be read once [L "How the runtime and
 * frontend work together"]. */
int64_t rs_decode_workspace_bytes(const rs_plan* p, int32_t B, int32_t max_seq_len,
                                  int32_t Hq, int32_t Hkv, int32_t D);
/* Zero a workspace (a fill kernel on stream; no passage defines it).  Optional: every partial
 * the merge reads is written first by the same rs_decode_attention call. */
int rs_decode_workspace_init(void* ws, int64_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ device ops */

/* Write the K/V rows of n new tokens into their pool slots [L "A quick recap": the new
 * token's keys and values are appended].  k_new, v_new: device [n][Hkv][D]; slots:
 * device int32 [n], each in [0, pool_slots).  Pools: device [pool_slots][Hkv][D]. */
int rs_store_kv(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                const int32_t* slots, int64_t n, int32_t Hkv, int32_t D, int32_t dtype,
                void* stream);

/* Extend attention [L step 3: prefill only the unmatched suffix, attending to the
 * reused KV as if just computed]: for request b, query i (0 <= i < extend_lens[b]) sits
 * at position p = prefix_lens[b] + i and attends causally to positions 0..p, whose K/V
 * rows are k_pool/v_pool[req_to_token[b*ld + j]]:
 *   out[q, h] = softmax_j(sm_scale * q[q, h] . K[j, h/G]) V[j, h/G].
 * q, out: device [sum(extend_lens)][Hq][D], requests packed in order (qo_indptr, device
 * int32 [B+1], gives each request's first query row).  prefix_lens, extend_lens: device
 * int32 [B]; req_to_token: device int32 [B][ld] with prefix+extend <= ld.
 * max_extend_len (host) bounds extend_lens and sizes the grid.  order: device int32 [B],
 * a permutation of 0..B-1 giving the order in which requests' work is started (longest
 * first evens out the finish; rs_extend_order computes it), or NULL for 0..B-1; it changes
 * no result.  bf16: MFMA with fp32 accumulation; fp32: fp32 throughout. */
int rs_extend_attention(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* req_to_token, int64_t ld, const int32_t* qo_indptr,
                        const int32_t* prefix_lens, const int32_t* extend_lens, int32_t B,
                        int32_t max_extend_len, int32_t Hq, int32_t Hkv, int32_t D, float sm_scale,
                        int32_t dtype, const int32_t* order, void* out, void* stream);

/* Host: the request order for rs_extend_attention, longest causal work first
 * (work = extend_len * (prefix_len + (extend_len + 1) / 2); ties by index).  prefix_lens,
 * extend_lens: host int32 [B]; order: host int32 [B] out.  A launch-order aid of this
 * library, not an operation of the pages: it changes when work starts, never a result. */
int rs_extend_order(const int32_t* prefix_lens, const int32_t* extend_lens, int32_t B, int32_t* order);

/* ------------------------------------------------------------------ draft-tree verify */

/* Host: the draft tree of a verify step [T "Speculative decoding puts a tree inside the
 * tree"].  Each of the B requests verifies n <= 64 tokens; parents (host int32 [B][n])
 * gives token i's parent, with token 0 the root (parent -1: the last verified token) and
 * every other parent in 0..i-1.  Outputs (host, [B][n]): tree_mask, bit j set iff token j
 * is token i or one of its ancestors; positions = prefix_lens[b] + depth (root depth 0;
 * depths [0,1,1,2] after a 7-token prompt give [7,8,8,9]); next_token = first child,
 * next_sibling = the next child of the same parent in index order (-1: none).
 * RS_E_INVAL if a parent is out of range. */
int rs_draft_tree_build(const int32_t* parents, const int32_t* prefix_lens, int32_t B, int32_t n,
                        uint64_t* tree_mask, int32_t* positions, int32_t* next_token,
                        int32_t* next_sibling);

/* Verify attention: request b's n tokens (q rows b*n .. b*n+n-1, device [B*n][Hq][D])
 * attend to cached positions 0..prefix_lens[b]-1 and, among the verify tokens (table
 * positions prefix + j, their K/V stored first), to token i itself and its ancestors:
 * token i sees verify token j iff bit j of tree_mask[b*n + i] is set and j <= i
 * [T "Speculative decoding ..."]: one target pass checks every branch.  prefix_lens
 * (device int32 [B]), tree_mask (device uint64 [B*n], from rs_draft_tree_build), out
 * (device [B*n][Hq][D]).  bf16 only (RS_E_UNSUPPORTED otherwise); n <= 64. */
int rs_tree_verify_attention(const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* req_to_token, int64_t ld, const int32_t* prefix_lens,
                             const uint64_t* tree_mask, int32_t B, int32_t n, int32_t Hq,
                             int32_t Hkv, int32_t D, float sm_scale, int32_t dtype, void* out,
                             void* stream);

/* Copy pool rows src_slots[r] -> dst_slots[r] in both pools (device int32 [n] each): the
 * accepted path of a draft tree is scattered over the draft's slots, and the radix tree
 * adopts a token run only with its own run of slots, so the accepted KV is compacted
 * first [T "Speculative decoding ..."].  Every dst slot must differ from every other dst
 * slot and from every src slot at another index; otherwise the result is undefined. */
int rs_move_kv(void* k_pool, void* v_pool, const int32_t* src_slots, const int32_t* dst_slots,
               int64_t n, int32_t Hkv, int32_t D, int32_t dtype, void* stream);

/* Pinned host memory for the host tier's K/V pools [T "What the C++ tree is actually for"],
 * mapped for the GPU at its host address (RS_E_UNSUPPORTED if the runtime maps it elsewhere,
 * RS_E_NOSPACE if it cannot be had).  The caller owns it until rs_host_free, which must come
 * after every copy that reads or writes it has completed (RS_E_INVAL for a pointer that is not
 * the start of such a block). */
int rs_host_alloc(int64_t bytes, void** out);
int rs_host_free(void* p);

/* Copy rows between two pools: dst_k[dst_slots[r]] = src_k[src_slots[r]] and the same for V
 * (r < n; slot arrays device int32; pools [rows][Hkv][D], dst_rows and src_rows rows, 16-byte
 * aligned).  A pool is device memory, or lies wholly inside a block from rs_host_alloc (the
 * host tier's copies of rs_write_through / rs_load_back, which the kernel reads or writes over
 * the bus); any other pointer is refused with RS_E_INVAL before anything runs.  A row whose slot
 * lies outside its pool is skipped.  Destinations must be distinct. */
int rs_copy_kv(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int32_t* dst_slots,
               const int32_t* src_slots, int64_t n, int64_t dst_rows, int64_t src_rows, int32_t Hkv,
               int32_t D, int32_t dtype, void* stream);

/* Decode attention: one query per request at position seq_lens[b]-1 over positions
 * 0..seq_lens[b]-1 (its own KV stored first) [L "A quick recap"].  q, out: device
 * [B][Hq][D]; lse_out: device float [B][Hq] natural-log log-sum-exp, or NULL.
 * With a plan (host handle `plan` and its uploaded image `plan_dev`), a shared segment
 * is read once for all its requests as one multi-query tile.  Every work item writes a
 * partial (o, lse) to the workspace (or the final output when it alone covers a
 * request) and a second kernel on the same stream merges each request's partials:
 *   lse = log sum_i exp(lse_i),  o = sum_i exp(lse_i - lse) o_i.
 * plan = NULL: each request is one segment (flat).  ws: device workspace of at least
 * rs_decode_workspace_bytes.  Launches that share a workspace must not overlap.
 * fp32 runs the flat path (plan ignored).  max_seq_len must be >= every seq_lens[b] and
 * <= ld (RS_E_INVAL if ld is smaller); the device cannot check seq_lens, so without a plan
 * a request longer than max_seq_len is cut to its first max_seq_len keys rather than read
 * out of bounds (a plan carries the key ranges it was built with). */
int rs_decode_attention(const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens,
                        int32_t B, int32_t max_seq_len, int32_t Hq, int32_t Hkv, int32_t D,
                        float sm_scale, int32_t dtype, const rs_plan* plan, const void* plan_dev,
                        void* ws, int64_t ws_bytes, void* out, float* lse_out, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): rs_decode_attention with the workspace
 * taken from a static device array of the library (128 MiB per GPU, held from the library's
 * first use on that GPU until the process ends; its device address is looked up once per
 * device with hipGetSymbolAddress).  Same arguments and results as rs_decode_attention
 * without ws / ws_bytes; the caller still passes every input and output.  A batch whose
 * workspace (rs_decode_workspace_bytes) exceeds 128 MiB is refused with RS_E_UNSUPPORTED
 * before anything runs.  No memory is allocated or freed, and nothing in the array needs
 * clearing: every partial is written before it is read within a call.  All calls on one
 * GPU share the array, so calls that overlap in time on one GPU (other streams, other host
 * threads) race and must be serialized by the caller. */
int rs_decode_attention_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* req_to_token, int64_t ld, const int32_t* seq_lens,
                                int32_t B, int32_t max_seq_len, int32_t Hq, int32_t Hkv, int32_t D,
                                float sm_scale, int32_t dtype, const rs_plan* plan,
                                const void* plan_dev, void* out, float* lse_out, void* stream);

/* Merge two attention states over disjoint key sets (the combine step above), rows x D:
 * o_a, o_b, o: device [rows][D] of dtype; lse_*: device float [rows].  The pages state no
 * formula: this is the log-sum-exp identity that makes attention over a union of key sets
 * from attention over its parts, exposed so that tests can check the combine on its own. */
int rs_merge_states(const void* o_a, const float* lse_a, const void* o_b, const float* lse_b,
                    int64_t rows, int32_t D, int32_t dtype, void* o, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RS_H_ */
