/*
 * forkattn.h -- C ABI of libforkattn.so: attention over a shared, paged KV-state DAG
 * on AMD Instinct MI355X (gfx950).
 *
 * Many branches / threads read ONE physical copy of a common prefix:
 *   - a host-side page table with reference counts and copy-on-write of shared pages
 *     (zero-copy forks, read-only mounts, drop / repos compaction, rewind, release);
 *   - fork_attn_decode: split-K decode that streams each shared KV page from HBM once
 *     for every query row that reads it, followed by a log-sum-exp merge;
 *   - dag_attn_prefill: block-sparse prefill over a packed DAG block mask.
 *
 * Sources (page title and section):
 *   Octopus (zicq.com): "Zero-Copy Radix Forking", "Attention-Only KV Mounting",
 *     "Packed DAG-GRPO", the core-idea section (fork / read_thread / wait_threads /
 *     rewind / commit) and the developer-advice section (refcounts, snapshot
 *     consistency, OOM fallback, thread-level cancellation).
 *   Agentrix README (gitlink.org.cn): "前缀复用与 ForkAttention" and the CUDA
 *     ForkAttention item (public / private segments by actual cache pages, merge),
 *     the cache-lifecycle item (reclaim only at refcount zero), tool-data snapshots.
 *   AKV (news.farwalk.ai): "AKV 如何工作" (Append / Drop / Repos; drop and reposition
 *     nodes; free dropped KV only when no live request needs it).
 *   AgentKV (rit.work): physical compaction returning freed pages to the allocator.
 *
 * Conventions
 *   - Every call returns a kv_status (0 = OK, negative = error).  No exception crosses
 *     the ABI.  A failing call leaves host metadata and device memory unchanged.
 *   - Device memory (page pools, workspaces, Q / O / LSE, prefill tensors) is owned by
 *     the caller and passed as raw device pointers; it must stay alive while the pool
 *     or the launched work uses it.  The library owns host metadata and a pinned host
 *     staging buffer only; it never allocates device memory.
 *   - Device work is enqueued on the caller's hipStream_t (NULL = default stream) and
 *     returns asynchronously; metadata changes are immediate.  Pages released by an
 *     operation may be handed out again to later operations; their old contents are
 *     read only by work already enqueued, so callers must keep all pool work on ONE
 *     stream (or order streams themselves).
 *   - A pool is not thread-safe: the caller serialises calls on one pool.
 */
#ifndef FORKATTN_H
#define FORKATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kv_pool kv_pool_t; /* opaque; host metadata only */
typedef int32_t kv_seq_t;         /* sequence = branch / thread handle, assigned 0, 1, 2, ... */

typedef enum {
  KV_OK = 0,
  KV_ERR_INVALID = -1,     /* bad argument, handle or range */
  KV_ERR_OOM = -2,         /* not enough free pages; nothing was changed */
  KV_ERR_NOT_FOUND = -3,   /* released or unknown sequence handle */
  KV_ERR_HIP = -4,         /* a HIP runtime call failed */
  KV_ERR_UNSUPPORTED = -5, /* shape / dtype / page size without a kernel */
  KV_ERR_WORKSPACE = -6    /* workspace too small (query the *_workspace_size call) */
} kv_status;

typedef enum { KV_BF16 = 0, KV_F32 = 1 } kv_dtype;
typedef enum { KV_ROPE_NONE = 0, KV_ROPE_NEOX = 1 } kv_rope_style;
enum { KV_DROP_REPOS = 1 }; /* kv_drop flag: re-rotate kept keys to positions 0..r-1 */

typedef struct {
  int32_t n_kv_heads; /* Hkv */
  int32_t head_dim;   /* d: 64 or 128 for device pools */
  int32_t page_size;  /* tokens per page: 16 for device pools; any >= 1 for metadata-only pools */
  int32_t n_pages;    /* pool capacity in pages */
  int32_t dtype;      /* kv_dtype of K, V, Q and O */
  int32_t rope_style; /* kv_rope_style used by Repos (keys are stored already rotated) */
  double rope_theta;  /* rotary base, e.g. 1e6 */
} kv_pool_config;

/* ---------------------------------------------------------------------------------
 * Device page layout (one page = page_size tokens of every KV head).
 *
 * k_pages and v_pages each hold Hkv * n_pages blocks, head-major: block (page p, head h)
 * starts at element (h * n_pages + p) * 16 * d, so the pages one decode work item
 * streams for one head are contiguous whenever their ids are.  Inside a block:
 *   K is stored in matrix-core operand order: the block is a sequence of 16-byte slots
 *     indexed (f, g, t) with slot number (f * 4 + g) * 16 + t, and slot (f, g, t) holds
 *       bf16: K[t][32 f + 8 g + e],      e = 0..7   (f < d/32)
 *       fp32: K[t][16 f + 4 e + g],      e = 0..3   (f < d/16)
 *     so that lane (t + 16 g) of a wave loads, with one contiguous 1 KiB access per f,
 *     exactly the operand fragment it feeds to the matrix instruction.
 *   V is stored transposed, with the 16 slots of a row in the order 0-3, 8-11, 4-7,
 *     12-15: element d * 16 + v(t) holds V[t][d], v(t) = t with bits 2 and 3 swapped, so
 *     the slot pairs of 4-runs {0-3, 8-11} and {4-7, 12-15} are 16 contiguous bytes each.
 * Use kv_pool_read_page() to read a page back in plain [t][d] order.
 * ------------------------------------------------------------------------------- */

/* Bytes of ONE of the two pools (K or V) for cfg->n_pages pages. */
int kv_pool_bytes(const kv_pool_config* cfg, size_t* bytes);

/* Device workspace the pool needs for its own staging (append / write / drop plans). */
int kv_pool_workspace_size(const kv_pool_config* cfg, size_t* bytes);

/* Create a pool (Octopus, "Zero-Copy Radix Forking": every thread's KV lives in one pool
 * of fixed-size pages that forks share by reference; Agentrix README, cache-lifecycle
 * item: a page is reclaimed only when its reference count reaches zero).
 * k_pages / v_pages: device buffers of kv_pool_bytes() each;
 * workspace: device buffer of kv_pool_workspace_size() bytes.
 * Passing k_pages = v_pages = workspace = NULL creates a METADATA-ONLY pool: every
 * page-table operation works and is bit-identical, no device work is issued and the
 * attention calls return KV_ERR_INVALID (capacity planning and host-side tests). */
int kv_pool_create(const kv_pool_config* cfg, void* k_pages, void* v_pages, void* workspace,
                   size_t ws_bytes, kv_pool_t** out);
int kv_pool_destroy(kv_pool_t* pool);

/* New empty root sequence (Octopus: a thread with no parent). */
int kv_seq_create(kv_pool_t* pool, kv_seq_t* out);

/* Append n tokens (AKV "Append").  k, v: DEVICE arrays [n][Hkv][d] in the pool dtype,
 * keys already rotated for their positions.  positions: HOST int64[n] or NULL for
 * next_pos, next_pos + 1, ...  A partially filled tail page shared with another
 * sequence or mount (refcount > 1) is copied first (copy-on-write, lowest free page
 * id); new pages are then taken lowest-id-first in logical order.  KV_ERR_OOM if the
 * pool cannot hold the result (nothing changes). */
int kv_append(kv_pool_t* pool, kv_seq_t seq, int64_t n, const void* k, const void* v,
              const int64_t* positions, hipStream_t stream);

/* Append one token to each of n distinct live sequences in one call (the decode step's
 * append: Octopus forks keep decoding side by side; AKV "Append").  k, v: DEVICE arrays
 * [n][Hkv][d] in the pool dtype, row i for seqs[i], keys already rotated; each token
 * takes its sequence's next_pos.  The page table ends exactly as after n single-token
 * kv_append calls in list order (a shared partial tail page is copied first; a full
 * tail takes a new page; lowest free id first), with one upload and at most two kernel
 * launches (the tail copies first, so a page copied for one sequence and then written in
 * place by a later one in the list is copied as it was before the call).
 * KV_ERR_INVALID for a sequence listed twice or n > n_pages, KV_ERR_NOT_FOUND for a
 * dead handle, KV_ERR_OOM if the pool cannot hold the result (nothing changes). */
int kv_append_batch(kv_pool_t* pool, const kv_seq_t* seqs, int32_t n, const void* k, const void* v,
                    hipStream_t stream);

/* Overwrite tokens [start, start + n) of the sequence's own context in place
 * (positions unchanged).  Every touched page whose refcount > 1 is copied first, so a
 * shared snapshot is never written (Agentrix: local edits create new versions while
 * unchanged pages stay shared).  k, v as in kv_append. */
int kv_write(kv_pool_t* pool, kv_seq_t seq, int64_t start, int64_t n, const void* k,
             const void* v, hipStream_t stream);

/* Fork (Octopus "Zero-Copy Radix Forking"): the child shares every page and mount of
 * the parent (refcount + 1 each); no page is allocated and no KV byte moves. */
int kv_fork(kv_pool_t* pool, kv_seq_t parent, kv_seq_t* child);

/* Mount (Octopus "Attention-Only KV Mounting", read_thread): dst additionally attends
 * to tokens [src_begin, src_begin + len) of src's own context as they are now; the
 * touched pages gain one reference each, nothing is copied, and later writes by src
 * copy away from the snapshot.  Mounted keys keep src's positions. */
int kv_mount(kv_pool_t* pool, kv_seq_t dst, kv_seq_t src, int64_t src_begin, int64_t len);

/* Drop (AKV "Drop", AgentKV physical compaction).  begin / len: HOST int64[n_spans],
 * half-open token ranges of the own context (overlaps are unioned).  Kept tokens are
 * packed in order into slots 0..r-1: logical pages before the first changed slot keep
 * their ids, affected pages are rewritten in place when exclusive (refcount 1) or
 * copied when shared, and pages from ceil(r / page_size) on are released.  Positions
 * and next_pos are unchanged unless flags has KV_DROP_REPOS (AKV "Repos"): then kept
 * token j gets position j, next_pos = r, and its key is re-rotated by
 * (j - old position) in the same kernel; values are moved bit-exactly, never changed.
 * kept_src_idx: optional HOST int64 buffer of at least the current token count;
 * receives the old index of every kept token. */
int kv_drop(kv_pool_t* pool, kv_seq_t seq, const int64_t* begin, const int64_t* len,
            int32_t n_spans, int32_t flags, int64_t* kept_src_idx, hipStream_t stream);

/* Drops of n distinct sequences in one call, ending exactly as n kv_drop calls in list
 * order (same page tables, positions, compaction indices and page contents), with one
 * plan upload and one kernel launch for all of them -- split into a few launches only
 * where a later drop would write a page an earlier one still reads (sequences sharing
 * pages) or the plans outgrow the pool workspace.  Sequence i's spans are
 * begin / len[span_off[i] .. span_off[i + 1]) (HOST int64, span_off has n + 1 entries);
 * flags as for kv_drop, for every listed sequence.  kept_src_idx: optional HOST int64,
 * sequence i's compaction index at offset = the sum of the token counts (before the call)
 * of the sequences listed before it.  Checks everything before changing anything:
 * KV_ERR_INVALID for a sequence listed twice or a bad span, KV_ERR_NOT_FOUND for a dead
 * handle, KV_ERR_OOM when the copies of all listed drops together (counted as if no
 * earlier drop released a page) exceed the free pages. */
int kv_drop_batch(kv_pool_t* pool, const kv_seq_t* seqs, int32_t n, const int64_t* span_off,
                  const int64_t* begin, const int64_t* len, int32_t flags, int64_t* kept_src_idx,
                  hipStream_t stream);

/* Repos alone: kv_drop with no spans and KV_DROP_REPOS. */
int kv_repos(kv_pool_t* pool, kv_seq_t seq, hipStream_t stream);

/* Rewind (Octopus primitive): truncate to new_len tokens, releasing pages past
 * ceil(new_len / page_size); next_pos becomes position[new_len - 1] + 1 (0 if empty).
 * Rewinding to the current length changes nothing. */
int kv_rewind(kv_pool_t* pool, kv_seq_t seq, int64_t new_len);

/* Commit (Octopus primitive): validates the handle; sequences are mountable at any
 * time, so there is nothing else to do. */
int kv_commit(kv_pool_t* pool, kv_seq_t seq);

/* Release (thread-level cancellation / finish): drops every page and mount reference;
 * pages still referenced by other sequences or mounts survive.  The handle dies. */
int kv_release(kv_pool_t* pool, kv_seq_t seq);

/* ---- introspection (exact integers, for tests and capacity planning) ---- */
int kv_seq_info(kv_pool_t* pool, kv_seq_t seq, int64_t* n_tokens, int64_t* next_pos,
                int32_t* n_pages, int32_t* n_mounts);
/* Own-context block table (logical page -> page id).  cap: capacity of `pages`. */
int kv_block_table(kv_pool_t* pool, kv_seq_t seq, int32_t* pages, int32_t cap);
int kv_positions(kv_pool_t* pool, kv_seq_t seq, int64_t* pos, int64_t cap);
int kv_page_refcount(kv_pool_t* pool, int32_t page, int32_t* rc);
int kv_free_pages(kv_pool_t* pool, int32_t* n_free);
/* Copy one page of one head back in plain [16][d] order for K and V (HOST buffers),
 * synchronising the stream. */
int kv_pool_read_page(kv_pool_t* pool, int32_t page, int32_t head, void* k_out, void* v_out,
                      hipStream_t stream);

/* Synchronise the stream and report how many in-place compaction waits gave up
 * (a safety valve of the drop kernel's ordering; 0 unless the device misbehaved). */
int kv_pool_sync_status(kv_pool_t* pool, hipStream_t stream, int32_t* n_wait_timeouts);

/* ---- decode (Agentrix ForkAttention) ----
 * For each i < n_seqs and query head h < n_q_heads (h reads KV head h / (Hq/Hkv)):
 *   O[i][h] = softmax(sm_scale * K_i q[i][h]) V_i,  LSE[i][h] = ln sum exp(sm_scale K_i q)
 * over sequence seqs[i]'s whole visible context (own tokens, then mounts).
 * Pages are grouped by the exact set of query rows that read them (public / private
 * segments by real cache pages); each group's pages are streamed from HBM once for all
 * its rows; partial (max, sum, out) results are merged by log-sum-exp.
 * q: DEVICE [n_seqs][Hq][d] (pool dtype); out: DEVICE [n_seqs][Hq][d] (pool dtype);
 * lse: DEVICE fp32 [n_seqs][Hq] or NULL.
 * workspace: DEVICE buffer of fork_attn_workspace_size() bytes for the same arguments.
 * The plan is cached in the workspace: a later call with the same pool state, seqs,
 * n_q_heads and workspace reuses it without host work or uploads, so the workspace
 * must not be modified between such calls. */
int fork_attn_workspace_size(kv_pool_t* pool, const kv_seq_t* seqs, int32_t n_seqs,
                             int32_t n_q_heads, size_t* bytes);
int fork_attn_decode(kv_pool_t* pool, const kv_seq_t* seqs, int32_t n_seqs, int32_t n_q_heads,
                     const void* q, void* out, float* lse, float sm_scale, void* workspace,
                     size_t ws_bytes, hipStream_t stream);

/* fork_attn_decode in two launches, for callers that overlap the merge with other work
 * (or time the kernels apart): fork_attn_partials streams the KV pages and writes one
 * partial (max, sum, output) per (work item, row) into the workspace;
 * fork_attn_merge combines each row's partials into out / lse.  Same arguments and
 * workspace as fork_attn_decode; the merge must follow the partials on the stream. */
int fork_attn_partials(kv_pool_t* pool, const kv_seq_t* seqs, int32_t n_seqs, int32_t n_q_heads,
                       const void* q, float sm_scale, void* workspace, size_t ws_bytes,
                       hipStream_t stream);
int fork_attn_merge(kv_pool_t* pool, const kv_seq_t* seqs, int32_t n_seqs, int32_t n_q_heads,
                    void* out, float* lse, void* workspace, size_t ws_bytes, hipStream_t stream);

/* Decode plans cut the chunk lists into work items so that one launch holds about two
 * items per compute unit (up to 128 chunks each); the count is the device's at
 * kv_pool_create (256 on MI355X) or 256 for a metadata-only pool.  Set another count for
 * a decode that shares the device with other work, or to plan long items over short
 * contexts.  Invalidates the cached decode plan (the next call plans again).
 * KV_ERR_INVALID for n_cu < 1. */
int kv_pool_set_compute_units(kv_pool_t* pool, int32_t n_cu);

/* fork_attn_decode without a workspace, for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, hosts that forbid allocation).  The
 * plan and the partials live in a device array the library holds for the process
 * lifetime, one per device (FORKATTN_STATIC_WORKSPACE_BYTES = 32 MiB each); the call
 * itself allocates nothing (the plan is copied from host memory the pool already holds).
 * Same arguments, results and errors as fork_attn_decode, plus KV_ERR_WORKSPACE when the
 * decode needs more than that many bytes of workspace (fork_attn_workspace_size tells).
 * Call with the pool's device current.  Every call on a device shares its array and
 * leaves its contents behind: calls that overlap on one device (other host threads,
 * other streams) race and must be serialised by the caller; the plan is uploaded again
 * whenever the array holds another pool's or an older plan. */
#define FORKATTN_STATIC_WORKSPACE_BYTES ((size_t)32 << 20)
int fork_attn_decode_static(kv_pool_t* pool, const kv_seq_t* seqs, int32_t n_seqs, int32_t n_q_heads,
                            const void* q, void* out, float* lse, float sm_scale, hipStream_t stream);

/* Plan statistics of the last fork_attn_decode / fork_attn_workspace_size call:
 * out[0] segments, out[1] work items, out[2] chunks, out[3] partial rows,
 * out[4] unique KV bytes streamed (algorithmic), out[5] query rows, out[6] the largest
 * chunk count of one work item, out[7] how many times the plan was patched since it was
 * last built (instead of replanning after page-table changes that were all appends into
 * pages their sequence owns alone:
 * the tail page's chunk grows and new pages join the last work item of the sequence's
 * private segment, so a decode step after one kv_append_batch re-uploads a few ints
 * instead of the plan). */
int fork_attn_plan_stats(kv_pool_t* pool, int64_t* out, int32_t n);

/* ---- packed DAG prefill (Octopus Packed DAG-GRPO, forward) ----
 * segments: HOST int32 [n_seg][3] = (start, length, parent); segment 0 has parent -1,
 *   parents precede children, segments tile [0, T) in order.  A query of segment S at
 *   packed index i sees every token of S's ancestors, the tokens of S at index <= i,
 *   and every edge range targeting S.
 * edges: HOST int32 [n_edges][4] = (src_segment, src_offset, length, dst_segment).
 * Segment starts and edge ranges must be multiples of `block`, except that the last
 * segment and an edge ending at its source segment's end may end anywhere.
 * Output: CSR over block rows: row_ptr[nb + 1], col[nnz] (ascending), kind[nnz]
 * (0 = every token pair visible, 1 = diagonal block, key <= query), nb = ceil(T/block).
 * Call with col = kind = NULL to get nnz only. */
int dag_mask_build(const int32_t* segments, int32_t n_seg, const int32_t* edges,
                   int32_t n_edges, int32_t T, int32_t block, int32_t* row_ptr, int32_t* col,
                   uint8_t* kind, int64_t* nnz);

/* Block-sparse forward over the CSR (DEVICE arrays row_ptr / col / kind from
 * dag_mask_build, block = 64, nnz = row_ptr[nb]).  Octopus "Packed DAG-GRPO": only
 * the block pairs listed are computed; kind 1 blocks mask key > query (global token
 * indices), keys >= T are always masked.
 *   q: DEVICE bf16 [T][Hq][d], k / v: DEVICE bf16 [T][Hkv][d], out: DEVICE bf16
 *   [T][Hq][d], lse: DEVICE fp32 [Hq][T] (natural log of the softmax denominator of
 *   sm_scale * q.k) or NULL.  d = 128; Hq a multiple of Hkv (query head h reads KV
 *   head h / (Hq / Hkv)).  A row with no visible key yields zeros and lse = -inf.
 *   workspace: DEVICE buffer of at least dag_attn_workspace_size() bytes for the same
 *   T, heads, block and nnz; it receives operand-order images of K and V and the
 *   packed column list.  Column indices outside [0, nb) are clamped, never followed.
 * Errors: KV_ERR_INVALID (shapes, null pointers, scale <= 0), KV_ERR_UNSUPPORTED
 * (d != 128 or block != 64), KV_ERR_WORKSPACE (workspace too small), KV_ERR_HIP
 * (launch failure).  T = 0 returns KV_OK and does nothing. */
int dag_attn_workspace_size(int32_t T, int32_t n_q_heads, int32_t n_kv_heads, int32_t block,
                            int64_t nnz, size_t* bytes);
int dag_attn_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                     int32_t T, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                     const int32_t* row_ptr, const int32_t* col, const uint8_t* kind,
                     int64_t nnz, int32_t block, float sm_scale, void* workspace,
                     size_t ws_bytes, hipStream_t stream);

/* dag_attn_prefill in two steps, for callers that reuse K / V and the mask across
 * several query sets, or time the attention kernel alone:
 *   dag_attn_prepare: copies K / V into the workspace's operand-order images and packs
 *     the column list and the row order (reads k, v, row_ptr, col, kind);
 *   dag_attn_run: the attention itself from a workspace prepared for the same T,
 *     heads, row_ptr, nnz and block (reads q, row_ptr and the workspace).
 * Same arguments, errors and workspace size as dag_attn_prefill. */
int dag_attn_prepare(const void* k, const void* v, int32_t T, int32_t n_q_heads,
                     int32_t n_kv_heads, int32_t head_dim, const int32_t* row_ptr,
                     const int32_t* col, const uint8_t* kind, int64_t nnz, int32_t block,
                     void* workspace, size_t ws_bytes, hipStream_t stream);
int dag_attn_run(const void* q, void* out, float* lse, int32_t T, int32_t n_q_heads,
                 int32_t n_kv_heads, int32_t head_dim, const int32_t* row_ptr, int64_t nnz,
                 int32_t block, float sm_scale, const void* workspace, size_t ws_bytes,
                 hipStream_t stream);

/* Steady-state decode window (Agentrix, "ForkAttention": the fork kernels run inside the
 * captured decode loop; AgentKV runs compaction and fork attention in graph-captured
 * decode).  Every step appends one token to each of n sequences and decodes all of them:
 *   kv_window_plan: reserves each sequence's next n_steps slots now -- the page table
 *     changes as if n_steps rounds of one kv_append per sequence (in list order) had
 *     run: a shared partial tail is copied, new pages are taken lowest-first, positions
 *     continue from next_pos -- and plans the decode of every step (contexts through
 *     that step's token) on the host; *ws_need = workspace bytes.  Works on
 *     metadata-only pools too (page table only).  Sequences must be distinct; n_q_heads
 *     as for fork_attn_decode.  KV_ERR_OOM leaves everything unchanged.
 *   kv_window_upload: uploads the plan (one image shared by every step, plus each
 *     step's slot ends of the reserved pages) into `workspace` (DEVICE, >= ws_need
 *     bytes, caller-owned, used by every step) and enqueues the tail copies.
 *   kv_window_step(step): writes k, v (DEVICE [n][Hkv][d], pool dtype, keys rotated for
 *     their reserved positions) into the step's slots and decodes q (DEVICE
 *     [n][Hq][d]) into out / lse as fork_attn_decode would over the contexts through
 *     this step; three kernels with fixed arguments, so steps 0 .. n_steps - 1 can be
 *     captured in a HIP graph once and replayed.  Steps run in order on one stream.
 * Any other page-table change ends the window (its calls then return KV_ERR_INVALID;
 * replays of a captured graph are not checked). */
int kv_window_plan(kv_pool_t* pool, const kv_seq_t* seqs, int32_t n, int32_t n_q_heads,
                   int32_t n_steps, size_t* ws_need);
int kv_window_upload(kv_pool_t* pool, void* workspace, size_t ws_bytes, hipStream_t stream);
int kv_window_step(kv_pool_t* pool, int32_t step, const void* k, const void* v, const void* q,
                   void* out, float* lse, float sm_scale, hipStream_t stream);

/* Causal attention of a sequence's last n tokens (AKV page, section "AKV 如何工作":
 * segmented batch attention restores an evicted state with one prefill in which each
 * segment keeps its own positions: append the
 * segments' K / V with kv_append and their positions, then call this).  Token j of the
 * n (0-based, query q[j]) attends to the sequence's own tokens up to and including
 * itself, then to the mounts, exactly as fork_attn_decode would for a sequence that
 * ended at that token.  q: DEVICE [n][Hq][d] (pool dtype, rotated by the caller); out:
 * DEVICE [n][Hq][d]; lse: DEVICE fp32 [n][Hq] or NULL.  workspace: DEVICE, at least
 * kv_causal_attend_workspace_size bytes for the same sequence state, n and n_q_heads.
 * bf16 pools with d = 128 run it as one tiled prefill, 64 of the n tokens and one piece of
 * the key range per workgroup, then the pieces are merged by log-sum-exp: when the visible
 * keys fill whole pages in order (own tokens always; mounts when page-aligned) K and V are
 * copied straight from the pages, else they are first relaid into matrix-core operand
 * images in the workspace.  Other pools run n rows of one split-K decode.
 * 1 <= n <= the sequence's length.  Stream-ordered. */
int kv_causal_attend_workspace_size(kv_pool_t* pool, kv_seq_t seq, int64_t n, int32_t n_q_heads,
                                    size_t* bytes);
int kv_causal_attend(kv_pool_t* pool, kv_seq_t seq, int64_t n, int32_t n_q_heads, const void* q,
                     void* out, float* lse, float sm_scale, void* workspace, size_t ws_bytes,
                     hipStream_t stream);

/* Gradients of dag_attn_prefill over the same CSR (Octopus "Packed DAG-GRPO": the packed
 * episode is trained through the same block-sparse attention, so only DAG-visible pairs
 * carry gradient).  For query head h (KV head g = h / (Hq / Hkv)) and a visible pair
 * (i, j): P_ij = exp(sm_scale q_i.k_j - lse_i), D_i = dout_i.out_i,
 * dS_ij = P_ij (dout_i.v_j - D_i); dq_i = sm_scale sum_j dS_ij k_j,
 * dk_j = sm_scale sum over the group's heads and i of dS_ij q_i,
 * dv_j = sum over the group's heads and i of P_ij dout_i.
 *   q, out, dout: DEVICE bf16 [T][Hq][d]; k, v: DEVICE bf16 [T][Hkv][d]; lse: DEVICE fp32
 *   [Hq][T], natural log, as written by the forward (out and lse must be the forward's
 *   outputs for these q, k, v and mask).  dq: DEVICE fp32 [T][Hq][d]; dk, dv: DEVICE
 *   fp32 [T][Hkv][d]; every element is written (keys no query sees get 0).
 *   row_ptr / col / kind: DEVICE CSR as for the forward (entries whose column is
 *   outside [0, nb) are skipped).  workspace: DEVICE, at least
 *   dag_attn_backward_workspace_size() bytes (per 64-token block and query head a 33,280 B
 *   record of Q / dout images, per block and KV head a 32,768 B record of K / V images,
 *   the mask's transpose, its rows' in-range entries and their order).
 * Errors as for dag_attn_prefill (d = 128, block = 64).  Stream-ordered. */
int dag_attn_backward_workspace_size(int32_t T, int32_t n_q_heads, int32_t n_kv_heads,
                                     int32_t block, int64_t nnz, size_t* bytes);
int dag_attn_backward(const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, float* dq, float* dk, float* dv,
                      int32_t T, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                      const int32_t* row_ptr, const int32_t* col, const uint8_t* kind,
                      int64_t nnz, int32_t block, float sm_scale, void* workspace,
                      size_t ws_bytes, hipStream_t stream);

/* ---- measurement probes (ceilings to price the kernels against, besides the vendor
 * peaks; not part of the attention path) ----
 * kv_probe_stream_read: one launch that reads every 16-byte word of `buf` (DEVICE,
 *   16-byte aligned, `bytes` long, multiple of 16 read) once with non-temporal loads;
 *   time it with events on `stream` for the achievable HBM read rate.  sink: DEVICE, at
 *   least 1 KiB, written only in a practically impossible case (keeps the loads live).
 * kv_probe_mfma_loop: n_workgroups workgroups of 4 waves, each wave issuing n_iter x 8
 *   independent v_mfma_f32_32x32x16_bf16 with register operands: 4 * 8 * n_iter * 32768
 *   FLOPs per workgroup; time it for the achievable dense bf16 matrix-core rate at the
 *   clock the chip holds under that load.  sink: DEVICE, at least 1 KiB of floats.
 * Both: KV_ERR_INVALID for bad arguments, KV_ERR_HIP for launch failures. */
int kv_probe_stream_read(const void* buf, size_t bytes, void* sink, hipStream_t stream);
int kv_probe_mfma_loop(int32_t n_iter, int32_t n_workgroups, void* sink, hipStream_t stream);

/* ---- errors ---- */
/* ---- key scoring and keep selection in front of Drop ----
 * AgentKV (rit.work), section "Как AgentKV выбирает и освобождает записи кэша": before a
 * compression the per-phase queues of recent queries are merged, every key is scored
 * against the merged set and the entries with the highest mean attention are kept; the
 * rest is dropped and the freed pages returned.
 *
 * kv_score: scores[t] for each own token t of `seq` (t < n_tokens of kv_seq_info) = the
 * mean over the n_rep x n_q_heads (representative query, head) pairs of t's softmax
 * probability in that query's attention over the sequence's whole visible context (own
 * tokens, then mounts; query head h reads KV head h / (n_q_heads / Hkv); logits =
 * sm_scale * q.k).  q_rep: device, pool dtype, [n_rep][n_q_heads][head_dim], rotated by
 * the caller.  scores: device float [n_tokens].  Needs a device bf16 pool (head_dim 64 or
 * 128; KV_ERR_UNSUPPORTED otherwise) and n_rep * n_q_heads / Hkv <= 256.  The workspace
 * (kv_score_workspace_size bytes, caller-owned device memory) holds the visible chunk
 * list, the per-row normalisers and per-KV-head partial sums; the chunk list stays in
 * it between calls and is uploaded again only after a page-table change, for another
 * sequence or another workspace (so do not write the workspace between calls); the
 * pool's cached decode plan is left alone.  Stream-ordered; scores are valid once the
 * stream has run the call. */
int kv_score_workspace_size(kv_pool_t* pool, kv_seq_t seq, int32_t n_rep, int32_t n_q_heads, size_t* bytes);
int kv_score(kv_pool_t* pool, kv_seq_t seq, const void* q_rep, int32_t n_rep, int32_t n_q_heads, float sm_scale,
             float* scores, void* workspace, size_t ws_bytes, hipStream_t stream);

/* keep[t] = 1 for the `budget` highest scores (ties to the lower index), 0 for the rest;
 * budget <= 0 keeps nothing, budget >= n keeps everything.  scores: device float [n],
 * n <= 2^31 - 1 (KV_ERR_UNSUPPORTED above); keep: device uint8 [n].  workspace:
 * caller-owned device memory of kv_select_workspace_size(n) bytes (at most 1 MiB + 256), used
 * by the calls on `stream` only: two calls in flight on different streams need two
 * workspaces.  A NaN score ranks below every number.  Stream-ordered. */
int kv_select_workspace_size(int64_t n, size_t* bytes);
int kv_select_keep(const float* scores, int64_t n, int64_t budget, uint8_t* keep, void* workspace, size_t ws_bytes,
                   hipStream_t stream);

/* Drop the tokens whose keep entry is 0: kv_drop with the maximal spans of zeros.  keep:
 * HOST uint8 [n], n = the sequence's n_tokens (copy the device mask back first: the page
 * table lives on the host).  flags as for kv_drop. */
int kv_drop_keep(kv_pool_t* pool, kv_seq_t seq, const uint8_t* keep, int64_t n, int32_t flags, hipStream_t stream);

const char* kv_status_str(int status);
const char* kv_last_error(kv_pool_t* pool); /* pool = NULL: last error of pool-less calls */

#ifdef __cplusplus
}
#endif
#endif /* FORKATTN_H */
