/*
 * tree_attn.h — C ABI of the MI355X (gfx950) tree-attention library.
 *
 * Four device operations sit behind this header:
 *
 *   ta_tree_attn    tree-masked attention of a token tree against a KV cache
 *                   laid out as [verified prefix | tree tokens];
 *   ta_tree_expand  maximum-likelihood expansion of the draft tree: the k
 *                   best children of its frontier leaves;
 *   ta_tree_verify  greedy verification of the tree against the target's
 *                   logits: the accepted path and the bonus token;
 *   ta_kv_reroot    re-root of that cache after verification: the accepted
 *                   path joins the prefix and the surviving subtree is packed
 *                   contiguously right after it.
 *
 * Source: SwiftSpec (arXiv 2506.11309), Pith review page, sections
 * "What carries the argument" (prefix/tree cache invariant, re-root at the
 * last verified token, mask attention kernel without explicit barriers) and
 * "Core claim" (verified tokens move into the prefix cache; surviving tree
 * states are reorganised contiguously after it).
 *
 * Conventions shared by every entry point:
 *  - Plain C types only. No exception crosses this boundary.
 *  - Device buffers are owned by the caller. The library never allocates,
 *    frees or retains device memory (the one exception is the static scratch
 *    of ta_tree_attn_rows_noalloc, a device array of the library's own code
 *    object), and never synchronises a stream.
 *  - Host arrays are read only during the call.
 *  - Every argument is validated before anything is enqueued. On error the
 *    call enqueues nothing, leaves every output untouched, returns a status
 *    and records a message readable through ta_last_error() (per thread).
 *  - Launch failures return TA_ERR_DEVICE. A fault inside a kernel surfaces,
 *    as usual for HIP, at the caller's next synchronisation.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TA_ABI_VERSION 1
#define TA_MAX_TREE 128 /* nodes per call: two 64-bit ancestor words per node */

typedef enum {
  TA_OK = 0,
  TA_ERR_ARG = 1,         /* null pointer, negative size, misalignment, bad workspace */
  TA_ERR_UNSUPPORTED = 2, /* dtype/head_dim/head ratio/tree size outside the built kernels */
  TA_ERR_CAPACITY = 3,    /* prefix_len + n_tree exceeds the cache capacity */
  TA_ERR_TREE = 4,        /* malformed parent array, path or survivor list */
  TA_ERR_DEVICE = 5       /* a HIP runtime call failed */
} ta_status;

typedef enum { TA_F32 = 0, TA_BF16 = 1 } ta_dtype;

/*
 * One model's KV cache (caller-owned device memory).
 * k and v are each dense [n_layers][n_kv_heads][capacity][head_dim] arrays of
 * `dtype`, 16-byte aligned. Slot t < prefix_len holds verified token t; slot
 * prefix_len + j holds tree node j.
 */
typedef struct {
  void* k;
  void* v;
  int32_t n_layers;
  int32_t n_kv_heads;
  int32_t capacity;
  int32_t head_dim; /* 64 or 128 */
  int32_t dtype;    /* ta_dtype */
} ta_kv_cache;

/*
 * Bytes of device workspace ta_tree_attn needs for this shape (0 if none).
 * The workspace carries split-softmax partial results and the hand-off
 * counters of the cross-workgroup combine. The counters always occupy the
 * first 64 KiB, whatever the shape; that region must be zero-filled once
 * before the first use, and every completed call leaves it ready for the next
 * (its arrival counts back at zero), so one workspace can serve calls of any
 * shapes in sequence with no clearing. One workspace must not be used by two
 * calls that can run at the same time (two streams, or graph replays that
 * overlap). Returns 0 and records an error message if the shape is invalid.
 */
size_t ta_tree_attn_workspace_bytes(const ta_kv_cache* cache, int32_t n_q_heads,
                                    int32_t prefix_len, int32_t n_tree);

/*
 * Tree-masked attention of one layer.
 *
 * For tree node i and query head h (KV head g = h / (n_q_heads/n_kv_heads)):
 *   s_t = <q[i][h], K[layer][g][t]> / sqrt(head_dim)
 * over the visible slots t: every prefix slot 0..prefix_len-1 and the slots
 * prefix_len + j of every tree node j that is i itself or an ancestor of i
 * (parent[j] = -1 hangs j off the last prefix token). out[i][h] is the
 * softmax(s)-weighted sum of V[layer][g][t], accumulated in fp32. Slots at or
 * beyond prefix_len + n_tree are never read.
 *
 *  q       device, [n_tree][n_q_heads][head_dim] of cache->dtype, 16-B aligned
 *  parent  host, n_tree entries, parent[i] in {-1} U [0, i)
 *  out     device, like q (bf16 results are rounded to nearest even)
 *  workspace / workspace_bytes: device, >= ta_tree_attn_workspace_bytes(..)
 *          (may be NULL when that is 0); see above for its contract.
 * Limits: 1 <= n_tree <= TA_MAX_TREE (n_tree == 0 is a no-op returning TA_OK),
 * head_dim in {64, 128}, n_q_heads a multiple of n_kv_heads with ratio <= 16,
 * prefix_len >= 0, prefix_len + n_tree <= capacity.
 */
ta_status ta_tree_attn(const void* q, const ta_kv_cache* cache, int32_t layer,
                       int32_t prefix_len, const int32_t* parent, int32_t n_tree,
                       int32_t n_q_heads, void* out, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Tree-masked attention of one layer for the tree nodes q_first .. n_tree-1
 * only: the draft-expansion step, where the queries are the newest leaves and
 * the keys are the whole [prefix | tree]. Node i (i >= q_first) sees exactly
 * what it sees in ta_tree_attn; ta_tree_attn is this call with q_first = 0.
 *
 * Source: the same passages as ta_tree_attn; the Pith review page,
 * "Assumptions & free parameters", fixes the expansion width w (the newest
 * w nodes of the tree are the ones expanded next).
 *
 *  q, out   device, [n_tree - q_first][n_q_heads][head_dim]: row r is tree
 *           node q_first + r
 *  q_first  0 <= q_first <= n_tree (q_first == n_tree is a no-op returning
 *           TA_OK); any other value is TA_ERR_ARG
 * Every other argument, limit and error as ta_tree_attn. The workspace size
 * and split count of this call are ta_tree_attn_rows_workspace_bytes and
 * ta_tree_attn_rows_num_splits (0 on an invalid shape).
 */
ta_status ta_tree_attn_rows(const void* q, const ta_kv_cache* cache, int32_t layer,
                            int32_t prefix_len, const int32_t* parent, int32_t n_tree,
                            int32_t q_first, int32_t n_q_heads, void* out, void* workspace,
                            size_t workspace_bytes, void* stream);
size_t ta_tree_attn_rows_workspace_bytes(const ta_kv_cache* cache, int32_t n_q_heads,
                                         int32_t prefix_len, int32_t n_tree, int32_t q_first);
int32_t ta_tree_attn_rows_num_splits(const ta_kv_cache* cache, int32_t n_q_heads,
                                     int32_t prefix_len, int32_t n_tree, int32_t q_first);
/*
 * Query rows per row block of this call's launch (host only, no device
 * access): 128, or 64 for bf16 heads of at most 64 query rows and for bf16
 * launches whose 128-row blocks would leave CUs idle. A row block is the
 * G * (n_tree - q_first) rows of one KV head cut into pieces of this size;
 * the launch has n_kv_heads * ceil(rows / block) * splits workgroups.
 * 0 on an invalid shape (ta_last_error says why).
 */
int32_t ta_tree_attn_rows_block_rows(const ta_kv_cache* cache, int32_t n_q_heads,
                                     int32_t prefix_len, int32_t n_tree, int32_t q_first);

/*
 * For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): ta_tree_attn_rows with the split workspace taken from a static
 * device array of this library, TA_NOALLOC_SCRATCH_BYTES per GPU, which each
 * GPU the library runs on holds until the process ends. The call itself
 * allocates nothing (no hipMalloc, no allocating library routine); on its
 * first use on a device it looks up that device's copy of the array.
 *
 *  stream  must belong to the current device (TA_ERR_ARG otherwise).
 * Every other argument, limit and error as ta_tree_attn_rows. A shape whose
 * workspace (ta_tree_attn_rows_workspace_bytes) exceeds the scratch is
 * TA_ERR_UNSUPPORTED, with nothing enqueued.
 *
 * All no-alloc calls on one GPU share that GPU's scratch, whose hand-off
 * counters every completed call leaves at zero: calls that can overlap on
 * one GPU (two streams, overlapping graph replays, two threads) race and
 * must be ordered by the caller.
 */
#define TA_NOALLOC_SCRATCH_BYTES (20u << 20)
ta_status ta_tree_attn_rows_noalloc(const void* q, const ta_kv_cache* cache, int32_t layer,
                                    int32_t prefix_len, const int32_t* parent, int32_t n_tree,
                                    int32_t q_first, int32_t n_q_heads, void* out, void* stream);

/*
 * Re-root every layer of the cache after a verification step.
 *
 *  accepted_path    host, n_accepted >= 0 nodes from a first-level node
 *                   (parent -1) downward: parent[a_k] = a_{k-1}
 *  surviving_nodes  host, n_surviving >= 0 nodes, strictly ascending, disjoint
 *                   from the path, closed under parent, with tops hanging off
 *                   the last accepted node (off -1 when n_accepted == 0)
 *  new_parent       host out, n_surviving entries: the survivors' tree in its
 *                   new numbering (-1 under the new last prefix token)
 *  new_prefix_len   host out: prefix_len + n_accepted
 *
 * Row prefix_len + k of every layer, KV head, K and V receives old row
 * prefix_len + order[k], order = accepted_path ++ surviving_nodes; all other
 * rows keep their bytes. The host outputs are final on return; the row moves
 * are enqueued on `stream` and are bit-exact.
 */
ta_status ta_kv_reroot(const ta_kv_cache* cache, int32_t prefix_len,
                       const int32_t* parent, int32_t n_tree,
                       const int32_t* accepted_path, int32_t n_accepted,
                       const int32_t* surviving_nodes, int32_t n_surviving,
                       int32_t* new_parent, int32_t* new_prefix_len, void* stream);

/*
 * Greedy verification of a draft tree (temperature-0 acceptance). Source:
 * SwiftSpec, Pith review page, "What carries the argument" and the referee
 * report's summary (the target checks the draft tree, the verified tokens
 * join the prefix, the tree re-roots at the last verified token), with
 * tree-based verification as in SpecInfer (the page's reference list): the
 * target scores the virtual root and every tree node in one pass.
 *
 *   choice[r] = arg-max of logits row r (the lowest token id among equal
 *               maxima; -0.0 and +0.0 are equal). Row 0 is the target at the
 *               last verified token, row 1 + i at tree node i.
 *   node i matches when tokens[i] == choice[parent[i] + 1]; it is accepted
 *   when it and every ancestor match. The accepted path a_0 .. a_{m-1} is the
 *   root path of the deepest accepted node (the lowest index among equally
 *   deep ones); m = 0 when no first-level node matches. The bonus token is
 *   choice[a_{m-1} + 1] (choice[0] when m = 0).
 *
 *  logits      device, n_tree + 1 rows of `vocab` values of `dtype` (TA_F32 or
 *              TA_BF16), row r at logits + r * row_stride elements; 16-byte
 *              aligned, row_stride >= vocab, row_stride * element size a
 *              multiple of 16; 1 <= vocab < 2^31. NaN values are undefined.
 *  tokens      device, n_tree int32: the drafted token of each node (may be
 *              NULL when n_tree == 0). Any values; they are only compared.
 *  parent      host, as for ta_tree_attn; 0 <= n_tree <= TA_MAX_TREE.
 *  choice_out  device, n_tree + 1 int32.
 *  result_out  device, n_tree + 2 int32: [m, bonus, a_0 .. a_{m-1}, then -1
 *              up to the end].
 *  workspace   device, >= ta_tree_verify_workspace_bytes(n_tree) bytes,
 *              256-byte aligned; zero-filled once before its first use, and
 *              every completed call leaves it zero again. Not shared with a
 *              call that can run at the same time (nor with ta_tree_attn).
 * One launch on `stream`; nothing is synchronised: the outputs are valid
 * once the stream reaches that point.
 */
size_t ta_tree_verify_workspace_bytes(int32_t n_tree);
ta_status ta_tree_verify(const void* logits, int32_t dtype, int64_t vocab, int64_t row_stride,
                         const int32_t* tokens, const int32_t* parent, int32_t n_tree,
                         int32_t* choice_out, int32_t* result_out, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * One maximum-likelihood expansion step of the draft tree. Source: SwiftSpec,
 * Pith review page, "Assumptions & free parameters" (a path scores the sum of
 * its tokens' log-softmax probabilities; expansion width w = 8).
 *
 * Frontier leaf i (row i of `logits`, the draft model's logits for the token
 * after it) has path score path_scores[i]. Every (leaf, token) pair is a
 * candidate child scored path_scores[i] + logits[i][t] - logsumexp(logits[i]);
 * the k best become the new nodes. Within a leaf the candidates rank by logit
 * (the lower token id first among equal logits): that rank is the child's
 * slot. Equal scores go to the lower leaf, then the lower slot. Output entry
 * j (j < k), in (leaf, slot) order: leaf_out[j] (row index), token_out[j],
 * score_out[j] (fp32: log-sum-exp accumulated in fp32).
 *
 *  logits       device, w rows of `vocab` values of `dtype` (TA_F32, TA_BF16),
 *               row i at logits + i * row_stride elements; 16-byte aligned,
 *               row_stride >= vocab, row_stride * element size a multiple
 *               of 16. 1 <= vocab <= 262144. Every row needs a finite value;
 *               -inf entries are allowed (probability 0); NaN is undefined.
 *  path_scores  device, w floats.
 *  1 <= w <= 64, 1 <= k <= 16, k <= w * vocab.
 *  leaf_out, token_out, score_out: device, k entries each.
 *  workspace    device, >= ta_tree_expand_workspace_bytes(w) bytes, 256-byte
 *               aligned; zero-filled once before its first use, and every
 *               completed call leaves its counters at zero again. Not shared
 *               with a call that can run at the same time.
 * One launch on `stream`; nothing is synchronised.
 */
size_t ta_tree_expand_workspace_bytes(int32_t w);
ta_status ta_tree_expand(const void* logits, int32_t dtype, int64_t vocab, int64_t row_stride,
                         const float* path_scores, int32_t w, int32_t k, int32_t* leaf_out,
                         int32_t* token_out, float* score_out, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Host-only planning steps of ta_tree_attn and ta_kv_reroot (no device work; usable
 * without a GPU).
 *
 * ta_tree_ancestor_bitset: words_out[2 i + w] has bit b set iff node 64 w + b
 * is i itself or an ancestor of i (two words per node, 2 n_tree words).
 * Validates parent like ta_tree_attn.
 *
 * ta_tree_ancestor_bits: the same for trees of at most 64 nodes, one word per
 * node (bits_out[i]); TA_ERR_UNSUPPORTED for larger trees.
 *
 * ta_kv_reroot_plan: validates a re-root request exactly like ta_kv_reroot and
 * writes src_rows_out[k] = prefix_len + order[k] for k < n_accepted +
 * n_surviving (the source slot of destination slot prefix_len + k), plus
 * new_parent and new_prefix_len as ta_kv_reroot would.
 */
ta_status ta_tree_ancestor_bitset(const int32_t* parent, int32_t n_tree, uint64_t* words_out);
ta_status ta_tree_ancestor_bits(const int32_t* parent, int32_t n_tree, uint64_t* bits_out);
ta_status ta_kv_reroot_plan(int32_t prefix_len, int32_t capacity, const int32_t* parent,
                            int32_t n_tree, const int32_t* accepted_path, int32_t n_accepted,
                            const int32_t* surviving_nodes, int32_t n_surviving,
                            int32_t* src_rows_out, int32_t* new_parent, int32_t* new_prefix_len);

/*
 * How long a prefix split of ta_tree_attn waits for the other splits of its
 * row block before leaving its share of the merge to the last split to
 * arrive: `polls` polls about 2048 GPU cycles apart (default 1000, about
 * 1 ms). Results do not depend on it: when every split of a row block runs at
 * once (the normal case on an otherwise idle GPU) each merges 1/splits of the
 * rows; a split that stops waiting leaves its rows to the last arrival, which
 * never waits. 0 disables waiting. Process-wide; applies to later calls.
 */
void ta_set_split_wait_limit(int32_t polls);

/* Number of prefix splits ta_tree_attn uses for this shape (>= 1); 0 on invalid shape. */
int32_t ta_tree_attn_num_splits(const ta_kv_cache* cache, int32_t n_q_heads,
                                int32_t prefix_len, int32_t n_tree);

const char* ta_status_string(ta_status status);
const char* ta_last_error(void);
int32_t ta_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
