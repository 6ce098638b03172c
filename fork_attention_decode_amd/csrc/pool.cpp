// Page pool, block tables and the C ABI of the page-table operations.
//
// Octopus (zicq.com), "Zero-Copy Radix Forking": a fork only adds a cursor and a little
// metadata, KV capacity grows only with new tokens, branches read the same physical
// pages and write new ones, and a shared page is never written in place.
// Agentrix README (gitlink.org.cn): pages are reclaimed only at reference count zero;
// a local edit creates a new version while unchanged pages stay shared.
// AKV (news.farwalk.ai), "AKV 如何工作": Append / Drop / Repos.
//
// Allocation policy (the pages fix none; these rules make block tables canonical):
// the lowest free page id is taken first; within one operation copy-on-write
// destinations are allocated first, then new pages in logical order, and every
// allocation precedes every release of that operation.
#include "pool.hpp"

#include <algorithm>
#include <unordered_map>
#include <cmath>
#include <cstring>
#include <new>

using namespace fa;

static thread_local std::string g_err;

int fa_set_err(kv_pool* P, int code, const std::string& m) {
  if (P) P->err = m;
  else g_err = m;
  return code;
}
#define FAIL(P, code, msg) return fa_set_err((P), (code), (msg))

// ------------------------------------------------------------------ FreeSet
void FreeSet::init(int32_t n) {
  n_ = n;
  count_ = n;
  bits_.assign((size_t)(n + 63) / 64, ~0ull);
  if (n % 64) bits_.back() = (1ull << (n % 64)) - 1;
  hint_ = 0;
}
void FreeSet::peek_lowest(int32_t k, std::vector<int32_t>& out) const {
  out.clear();
  for (size_t w = (size_t)hint_; w < bits_.size() && (int32_t)out.size() < k; ++w) {
    uint64_t b = bits_[w];
    while (b && (int32_t)out.size() < k) {
      out.push_back((int32_t)(w * 64 + __builtin_ctzll(b)));
      b &= b - 1;
    }
  }
}
void FreeSet::take(int32_t id) {
  bits_[id >> 6] &= ~(1ull << (id & 63));
  --count_;
  while (hint_ < (int32_t)bits_.size() && bits_[hint_] == 0) ++hint_;
}
void FreeSet::give(int32_t id) {
  bits_[id >> 6] |= 1ull << (id & 63);
  ++count_;
  if ((id >> 6) < hint_) hint_ = id >> 6;
}

// ------------------------------------------------------------------ helpers
static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

static size_t dtype_size(int dt) { return dt == KV_F32 ? 4 : 2; }

Seq* fa_seq(kv_pool* P, kv_seq_t s) {
  if (s < 0 || s >= (kv_seq_t)P->seqs.size() || !P->seqs[s].live) return nullptr;
  return &P->seqs[s];
}

static void ref_page(kv_pool* P, int32_t p) { P->rc[p]++; }
static void unref_page(kv_pool* P, int32_t p) {
  if (--P->rc[p] == 0) P->free.give(p);
}
static void take_page(kv_pool* P, int32_t p) {
  P->free.take(p);
  P->rc[p] = 1;
}
void fa_take_page(kv_pool* P, int32_t p) { take_page(P, p); }

// One page-table change: a new version, logged for patching the cached decode plan.
void fa_changed(kv_pool* P, int32_t kind, kv_seq_t seq, int64_t n0, int64_t n1) {
  P->version++;
  ChangeJournal& J = P->journal;
  if (J.broken) return;
  if (kind == ChangeJournal::kOther || J.ev.size() >= 65536) {
    J.broken = true;
    J.ev.clear();
    return;
  }
  J.ev.push_back({seq, kind, n0, n1});
}
void fa_unref_page(kv_pool* P, int32_t p) { unref_page(P, p); }

void fa_pos_append(std::vector<PosRun>& v, int64_t p0, int64_t n) {
  if (n <= 0) return;
  if (!v.empty() && v.back().p0 + v.back().len == p0) v.back().len += n;
  else v.push_back({p0, n});
}
void fa_pos_expand(const std::vector<PosRun>& v, std::vector<int64_t>& out) {
  out.clear();
  for (const PosRun& r : v)
    for (int64_t i = 0; i < r.len; ++i) out.push_back(r.p0 + i);
}
static std::vector<PosRun> pos_compress(const int64_t* p, int64_t n) {
  std::vector<PosRun> v;
  for (int64_t i = 0; i < n; ++i) fa_pos_append(v, p[i], 1);
  return v;
}
static std::vector<PosRun> pos_slice(const std::vector<PosRun>& v, int64_t b, int64_t n) {
  std::vector<PosRun> out;
  int64_t at = 0;
  for (const PosRun& r : v) {
    const int64_t lo = std::max(b, at), hi = std::min(b + n, at + r.len);
    if (lo < hi) fa_pos_append(out, r.p0 + (lo - at), hi - lo);
    at += r.len;
  }
  return out;
}
static void pos_truncate(std::vector<PosRun>& v, int64_t n) { v = pos_slice(v, 0, n); }
static int64_t pos_last(const std::vector<PosRun>& v) { return v.back().p0 + v.back().len - 1; }

// Upload a host blob to device memory on `s` through the next slot of the pinned staging
// ring (waiting only if that slot's previous copy has not run yet).
hipError_t fa_upload(kv_pool* P, void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  kv_pool::StageSlot& slot = P->stage[P->stage_next];
  hipError_t e;
  if (!slot.ev && (e = hipEventCreateWithFlags(&slot.ev, hipEventDisableTiming)) != hipSuccess) return e;
  if (slot.pending) {
    if ((e = hipEventSynchronize(slot.ev)) != hipSuccess) return e;
    slot.pending = false;
  }
  if (bytes > slot.bytes) {  // grow (at least double); the old buffer is freed with the pool
    const size_t sz = std::max({bytes, 2 * slot.bytes, (size_t)1 << 20});
    void* fresh = nullptr;
    if ((e = hipHostMalloc(&fresh, sz, hipHostMallocDefault)) != hipSuccess) return e;
    if (slot.ptr) P->retired.push_back(slot.ptr);
    slot.ptr = fresh;
    slot.bytes = sz;
  }
  std::memcpy(slot.ptr, src, bytes);
  if ((e = hipMemcpyAsync(dst, slot.ptr, bytes, hipMemcpyHostToDevice, s)) != hipSuccess) return e;
  if ((e = hipEventRecord(slot.ev, s)) != hipSuccess) return e;
  slot.pending = true;
  P->stage_next = (P->stage_next + 1) % kv_pool::kStageSlots;
  return hipSuccess;
}

// Pool workspace: [0, 4096) counters (compaction wait time-outs at int 1), then one
// read-done flag per page (zeroed at creation), then the plan area of append / write /
// drop (overwritten by every such call, in stream order).
static constexpr size_t kWsHeader = 4096;
static constexpr int kMaxRotations = 4096;  // distinct repos offsets per kv_drop call

size_t fa_ws_plan_offset(const kv_pool_config* c) {
  return kWsHeader + (((size_t)c->n_pages * 4 + 255) & ~(size_t)255);
}

size_t fa_pool_ws_need(const kv_pool_config* c) {
  const size_t tokens = (size_t)c->n_pages * c->page_size;
  return fa_ws_plan_offset(c) + tokens * 16 +
         (size_t)c->n_pages * std::max(sizeof(CompactPage), sizeof(PageWrite)) +
         (size_t)kMaxRotations * (size_t)c->head_dim * 4 + 4 * 4096;
}

extern "C" {

const char* kv_status_str(int s) {
  switch (s) {
    case KV_OK: return "ok";
    case KV_ERR_INVALID: return "invalid argument";
    case KV_ERR_OOM: return "out of pages";
    case KV_ERR_NOT_FOUND: return "no such sequence";
    case KV_ERR_HIP: return "HIP runtime error";
    case KV_ERR_UNSUPPORTED: return "unsupported configuration";
    case KV_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* kv_last_error(kv_pool_t* P) { return P ? P->err.c_str() : g_err.c_str(); }

static int check_cfg(const kv_pool_config* c, bool device) {
  if (!c || c->n_kv_heads < 1 || c->head_dim < 2 || c->page_size < 1 || c->n_pages < 1 ||
      (c->dtype != KV_BF16 && c->dtype != KV_F32) ||
      (c->rope_style != KV_ROPE_NONE && c->rope_style != KV_ROPE_NEOX) || c->head_dim % 2)
    FAIL(nullptr, KV_ERR_INVALID, "invalid kv_pool_config");
  if (c->rope_style == KV_ROPE_NEOX && !(c->rope_theta > 0))
    FAIL(nullptr, KV_ERR_INVALID, "rope_theta must be positive");
  if (device && (c->page_size != kPage || (c->head_dim != 64 && c->head_dim != 128)))
    FAIL(nullptr, KV_ERR_UNSUPPORTED, "device pools need page_size 16 and head_dim 64 or 128");
  return KV_OK;
}

int kv_pool_bytes(const kv_pool_config* c, size_t* bytes) {
  int st = check_cfg(c, false);
  if (st) return st;
  if (!bytes) FAIL(nullptr, KV_ERR_INVALID, "null output");
  *bytes = (size_t)c->n_pages * c->n_kv_heads * c->page_size * c->head_dim * dtype_size(c->dtype);
  return KV_OK;
}

int kv_pool_workspace_size(const kv_pool_config* c, size_t* bytes) {
  int st = check_cfg(c, false);
  if (st) return st;
  if (!bytes) FAIL(nullptr, KV_ERR_INVALID, "null output");
  *bytes = fa_pool_ws_need(c);
  return KV_OK;
}

int kv_pool_create(const kv_pool_config* c, void* k, void* v, void* ws, size_t ws_bytes,
                   kv_pool_t** out) {
  if (!out) FAIL(nullptr, KV_ERR_INVALID, "null output");
  const bool any = k || v || ws, all = k && v && ws;
  if (any && !all) FAIL(nullptr, KV_ERR_INVALID, "give all of k_pages, v_pages, workspace or none");
  int st = check_cfg(c, all);
  if (st) return st;
  if (all && ws_bytes < fa_pool_ws_need(c)) FAIL(nullptr, KV_ERR_WORKSPACE, "pool workspace too small");
  kv_pool* P = new (std::nothrow) kv_pool();
  if (!P) FAIL(nullptr, KV_ERR_OOM, "host allocation failed");
  P->cfg = *c;
  P->device = all;
  P->k = k;
  P->v = v;
  P->ws = (char*)ws;
  P->ws_bytes = ws_bytes;
  P->rc.assign(c->n_pages, 0);
  P->free.init(c->n_pages);
  if (all) {
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    const char* what = "hipGetDevice";
    if (e == hipSuccess) {
      what = "hipDeviceGetAttribute";
      e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    }
    if (e == hipSuccess) {
      what = "hipMemset";
      e = hipMemset(ws, 0, fa_ws_plan_offset(c));
    }
    if (e != hipSuccess) {
      delete P;
      FAIL(nullptr, KV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
    }
    P->n_cu = ncu > 0 ? ncu : 256;
  }
  *out = P;
  return KV_OK;
}

int kv_pool_set_compute_units(kv_pool_t* P, int32_t n_cu) {
  if (!P) FAIL(nullptr, KV_ERR_INVALID, "null pool");
  if (n_cu < 1) FAIL(P, KV_ERR_INVALID, "compute unit count must be >= 1");
  P->n_cu = n_cu;
  P->plan.valid = false;  // the cached decode plan was cut for the old count
  return KV_OK;
}

int kv_pool_destroy(kv_pool_t* P) {
  if (!P) FAIL(nullptr, KV_ERR_INVALID, "null pool");
  for (auto& slot : P->stage) {
    if (slot.pending) (void)hipEventSynchronize(slot.ev);
    if (slot.ptr) (void)hipHostFree(slot.ptr);
    if (slot.ev) (void)hipEventDestroy(slot.ev);
  }
  for (void* p : P->retired) (void)hipHostFree(p);
  delete P;
  return KV_OK;
}

int kv_seq_create(kv_pool_t* P, kv_seq_t* out) {
  if (!P || !out) FAIL(P, KV_ERR_INVALID, "null argument");
  P->seqs.emplace_back();
  *out = (kv_seq_t)P->seqs.size() - 1;
  fa_changed(P, ChangeJournal::kTouch, *out, 0, 0);
  return KV_OK;
}

int kv_fork(kv_pool_t* P, kv_seq_t parent, kv_seq_t* child) {
  if (!P || !child) FAIL(P, KV_ERR_INVALID, "null argument");
  Seq* s = fa_seq(P, parent);
  if (!s) FAIL(P, KV_ERR_NOT_FOUND, "no live parent sequence");
  Seq c = *s;  // pages and mounts by reference: ids only, no KV bytes
  for (int32_t p : c.pages) ref_page(P, p);
  for (const Mount& m : c.mounts)
    for (int32_t p : m.pages) ref_page(P, p);
  P->seqs.push_back(std::move(c));
  *child = (kv_seq_t)P->seqs.size() - 1;
  fa_changed(P, ChangeJournal::kTouch, *child, 0, 0);  // the parent's pages gain references only
  return KV_OK;
}

int kv_mount(kv_pool_t* P, kv_seq_t dst, kv_seq_t src, int64_t b, int64_t n) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* d = fa_seq(P, dst);
  Seq* s = fa_seq(P, src);
  if (!d || !s) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (n <= 0 || b < 0 || b + n > s->n) FAIL(P, KV_ERR_INVALID, "mount range outside the source");
  const int32_t PS = P->cfg.page_size;
  Mount m;
  m.pages.assign(s->pages.begin() + b / PS, s->pages.begin() + (b + n - 1) / PS + 1);
  m.off = (int32_t)(b % PS);
  m.n = n;
  m.pos = pos_slice(s->pos, b, n);
  for (int32_t p : m.pages) ref_page(P, p);
  P->seqs[dst].mounts.push_back(std::move(m));
  fa_changed(P, ChangeJournal::kTouch, dst, 0, 0);
  return KV_OK;
}

// Shared implementation of append (start == n) and in-place write (start + n <= n).
static int write_tokens(kv_pool* P, kv_seq_t seq, int64_t start, int64_t n, const void* k,
                        const void* v, const int64_t* positions, bool append, hipStream_t s) {
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (n < 0 || start < 0 || (append ? start != S->n : start + n > S->n))
    FAIL(P, KV_ERR_INVALID, "token range outside the sequence");
  if (n == 0) return KV_OK;
  if (P->device && (!k || !v)) FAIL(P, KV_ERR_INVALID, "null k / v");
  const int32_t PS = P->cfg.page_size;
  const int64_t end = start + n;
  const int64_t first = start / PS, last = (end - 1) / PS;
  const int64_t have = (int64_t)S->pages.size();
  std::vector<int64_t> cow;
  for (int64_t L = first; L <= last && L < have; ++L)
    if (P->rc[S->pages[L]] > 1) cow.push_back(L);
  const int64_t n_new = std::max<int64_t>(0, last + 1 - have);
  if ((int64_t)cow.size() + n_new > P->free.count())
    FAIL(P, KV_ERR_OOM, "not enough free pages");
  std::vector<int32_t> ids;
  P->free.peek_lowest((int32_t)(cow.size() + n_new), ids);
  // logical page -> (dst id, src id for copy-on-write)
  std::vector<PageWrite> writes;
  if (P->device) {
    size_t ci = 0;
    for (int64_t L = first; L <= last; ++L) {
      PageWrite w;
      if (L < have) {
        const bool c = ci < cow.size() && cow[ci] == L;
        w.dst_page = c ? ids[ci] : S->pages[L];
        w.src_page = c ? S->pages[L] : -1;
        if (c) ++ci;
      } else {
        w.dst_page = ids[cow.size() + (L - have)];
        w.src_page = -1;
      }
      w.lo = (int32_t)(L == first ? start % PS : 0);
      w.hi = (int32_t)std::min<int64_t>(PS, end - L * PS);
      w.tok_base = L * PS + w.lo - start;
      writes.push_back(w);
    }
    char* area = P->ws + fa_ws_plan_offset(&P->cfg);
    hipError_t e = fa_upload(P, area, writes.data(), writes.size() * sizeof(PageWrite), s);
    if (e == hipSuccess)
      e = launch_page_write(P->cfg.dtype, P->cfg.head_dim, P->cfg.n_kv_heads, P->cfg.n_pages, P->k, P->v, k, v,
                            reinterpret_cast<const PageWrite*>(area), (int)writes.size(), s);
    if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("page write: ") + hipGetErrorString(e));
  }
  // metadata (after the device work was enqueued successfully)
  for (size_t i = 0; i < cow.size(); ++i) {
    const int32_t old = S->pages[cow[i]];
    take_page(P, ids[i]);
    S->pages[cow[i]] = ids[i];
    unref_page(P, old);
  }
  for (int64_t j = 0; j < n_new; ++j) {
    take_page(P, ids[cow.size() + j]);
    S->pages.push_back(ids[cow.size() + j]);
  }
  if (append) {
    if (positions) {
      for (int64_t i = 0; i < n; ++i) fa_pos_append(S->pos, positions[i], 1);
      S->next_pos = positions[n - 1] + 1;
    } else {
      fa_pos_append(S->pos, S->next_pos, n);
      S->next_pos += n;
    }
    S->n += n;
  }
  if (append && cow.empty())
    fa_changed(P, ChangeJournal::kAppend, seq, S->n - n, S->n);
  else
    fa_changed(P, cow.empty() ? ChangeJournal::kContent : ChangeJournal::kOther, seq, 0, 0);
  return KV_OK;
}

int kv_append(kv_pool_t* P, kv_seq_t seq, int64_t n, const void* k, const void* v,
              const int64_t* positions, hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  return write_tokens(P, seq, S->n, n, k, v, positions, true, s);
}

// One token onto each of n distinct sequences, exactly as n single-token appends in list
// order would do it (a shared partial tail page is copied, a full tail takes a new page,
// both lowest free id first), with one upload and at most two page-write launches.  The page
// decisions run first on a copy of the refcounts (two forks sharing a tail page: the
// first copies it, the second then owns it alone and writes in place), so a failure
// leaves the pool unchanged.  Copies are written in a launch of their own before the
// in-place and new-page writes.
int kv_append_batch(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, const void* k, const void* v, hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  if (n < 0 || (n > 0 && !seqs)) FAIL(P, KV_ERR_INVALID, "bad sequence list");
  if (n == 0) return KV_OK;
  if (n > P->cfg.n_pages) FAIL(P, KV_ERR_INVALID, "more sequences than pool pages");
  if (P->device && (!k || !v)) FAIL(P, KV_ERR_INVALID, "null k / v");
  std::vector<Seq*> S((size_t)n);
  for (int32_t i = 0; i < n; ++i)
    if (!(S[(size_t)i] = fa_seq(P, seqs[i]))) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence in the list");
  {
    std::vector<kv_seq_t> sorted(seqs, seqs + n);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
      FAIL(P, KV_ERR_INVALID, "a sequence appears twice in the list");
  }
  const int32_t PS = P->cfg.page_size;
  enum { kInPlace = 0, kCopy = 1, kNew = 2 };
  std::vector<uint8_t> how((size_t)n);
  std::unordered_map<int32_t, int32_t> rc_delta;  // refcount changes of earlier copies in the list
  int32_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* q = S[(size_t)i];
    const int64_t L = q->n / PS;
    if (L < (int64_t)q->pages.size()) {
      const int32_t pg = q->pages[(size_t)L];
      const bool shared = P->rc[pg] + rc_delta[pg] > 1;
      if (shared) --rc_delta[pg];
      how[(size_t)i] = shared ? kCopy : kInPlace;
    } else {
      how[(size_t)i] = kNew;
    }
    need += how[(size_t)i] != kInPlace;
  }
  if (need > P->free.count()) FAIL(P, KV_ERR_OOM, "not enough free pages");
  std::vector<int32_t> ids;
  P->free.peek_lowest(need, ids);
  if (P->device) {
    // A page can be the source of one sequence's copy and, once that copy has dropped its
    // reference, the in-place target of a later sequence in the list (a fork rewound into
    // the shared tail).  The copies therefore run in a first launch and every other write
    // in a second, so a copy reads the page as it was before this call.
    std::vector<PageWrite> writes((size_t)n);
    int32_t j = 0, n_copy = 0;
    for (int32_t i = 0; i < n; ++i) n_copy += how[(size_t)i] == kCopy;
    int32_t at_copy = 0, at_rest = n_copy;
    for (int32_t i = 0; i < n; ++i) {
      const Seq* q = S[(size_t)i];
      const int64_t L = q->n / PS;
      const int32_t slot = (int32_t)(q->n % PS);
      PageWrite& w = writes[(size_t)(how[(size_t)i] == kCopy ? at_copy++ : at_rest++)];
      w.dst_page = how[(size_t)i] == kInPlace ? q->pages[(size_t)L] : ids[(size_t)j++];
      w.src_page = how[(size_t)i] == kCopy ? q->pages[(size_t)L] : -1;
      w.lo = slot;
      w.hi = slot + 1;
      w.tok_base = i;  // row i of k / v
    }
    char* area = P->ws + fa_ws_plan_offset(&P->cfg);
    hipError_t e = fa_upload(P, area, writes.data(), writes.size() * sizeof(PageWrite), s);
    const PageWrite* dw = reinterpret_cast<const PageWrite*>(area);
    if (e == hipSuccess && n_copy > 0)
      e = launch_page_write(P->cfg.dtype, P->cfg.head_dim, P->cfg.n_kv_heads, P->cfg.n_pages, P->k, P->v, k, v, dw,
                            n_copy, s);
    if (e == hipSuccess && n > n_copy)
      e = launch_page_write(P->cfg.dtype, P->cfg.head_dim, P->cfg.n_kv_heads, P->cfg.n_pages, P->k, P->v, k, v,
                            dw + n_copy, n - n_copy, s);
    if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("page write: ") + hipGetErrorString(e));
  }
  int32_t j = 0;
  for (int32_t i = 0; i < n; ++i) {
    Seq* q = S[(size_t)i];
    const size_t L = (size_t)(q->n / PS);
    if (how[(size_t)i] == kCopy) {
      const int32_t old = q->pages[L];
      take_page(P, ids[(size_t)j]);
      q->pages[L] = ids[(size_t)j++];
      unref_page(P, old);
    } else if (how[(size_t)i] == kNew) {
      take_page(P, ids[(size_t)j]);
      q->pages.push_back(ids[(size_t)j++]);
    }
    fa_pos_append(q->pos, q->next_pos, 1);
    q->next_pos += 1;
    q->n += 1;
  }
  bool any_copy = false;
  for (int32_t i = 0; i < n; ++i) any_copy |= how[(size_t)i] == kCopy;
  if (any_copy) {
    fa_changed(P, ChangeJournal::kOther, -1, 0, 0);
  } else {  // one version step per appended sequence, as n single appends would take
    for (int32_t i = 0; i < n; ++i) fa_changed(P, ChangeJournal::kAppend, seqs[i], S[(size_t)i]->n - 1, S[(size_t)i]->n);
  }
  return KV_OK;
}

int kv_write(kv_pool_t* P, kv_seq_t seq, int64_t start, int64_t n, const void* k, const void* v,
             hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  return write_tokens(P, seq, start, n, k, v, nullptr, false, s);
}

int kv_rewind(kv_pool_t* P, kv_seq_t seq, int64_t n) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (n < 0 || n > S->n) FAIL(P, KV_ERR_INVALID, "rewind beyond the sequence");
  if (n == S->n) return KV_OK;
  const int64_t keep = ceil_div(n, P->cfg.page_size);
  for (size_t L = (size_t)keep; L < S->pages.size(); ++L) unref_page(P, S->pages[L]);
  S->pages.resize((size_t)keep);
  pos_truncate(S->pos, n);
  S->n = n;
  S->next_pos = n ? pos_last(S->pos) + 1 : 0;
  fa_changed(P, ChangeJournal::kOther, seq, 0, 0);
  return KV_OK;
}

int kv_commit(kv_pool_t* P, kv_seq_t seq) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  if (!fa_seq(P, seq)) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  return KV_OK;
}

int kv_release(kv_pool_t* P, kv_seq_t seq) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  for (int32_t p : S->pages) unref_page(P, p);
  for (const Mount& m : S->mounts)
    for (int32_t p : m.pages) unref_page(P, p);
  S->pages.clear();
  S->pages.shrink_to_fit();
  S->mounts.clear();
  S->pos.clear();
  S->live = false;
  fa_changed(P, ChangeJournal::kOther, seq, 0, 0);
  return KV_OK;
}

int kv_seq_info(kv_pool_t* P, kv_seq_t seq, int64_t* n_tokens, int64_t* next_pos, int32_t* n_pages,
                int32_t* n_mounts) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (n_tokens) *n_tokens = S->n;
  if (next_pos) *next_pos = S->next_pos;
  if (n_pages) *n_pages = (int32_t)S->pages.size();
  if (n_mounts) *n_mounts = (int32_t)S->mounts.size();
  return KV_OK;
}

int kv_block_table(kv_pool_t* P, kv_seq_t seq, int32_t* pages, int32_t cap) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (cap < (int32_t)S->pages.size() || (!pages && !S->pages.empty()))
    FAIL(P, KV_ERR_INVALID, "block table buffer too small");
  std::copy(S->pages.begin(), S->pages.end(), pages);
  return KV_OK;
}

int kv_positions(kv_pool_t* P, kv_seq_t seq, int64_t* pos, int64_t cap) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (cap < S->n || (!pos && S->n)) FAIL(P, KV_ERR_INVALID, "position buffer too small");
  int64_t i = 0;
  for (const PosRun& r : S->pos)
    for (int64_t j = 0; j < r.len; ++j) pos[i++] = r.p0 + j;
  return KV_OK;
}

int kv_page_refcount(kv_pool_t* P, int32_t page, int32_t* rc) {
  if (!P || !rc) FAIL(P, KV_ERR_INVALID, "null argument");
  if (page < 0 || page >= P->cfg.n_pages) FAIL(P, KV_ERR_INVALID, "page id out of range");
  *rc = P->rc[page];
  return KV_OK;
}

int kv_free_pages(kv_pool_t* P, int32_t* n) {
  if (!P || !n) FAIL(P, KV_ERR_INVALID, "null argument");
  *n = P->free.count();
  return KV_OK;
}

int kv_pool_read_page(kv_pool_t* P, int32_t page, int32_t head, void* k_out, void* v_out,
                      hipStream_t s) {
  if (!P || !k_out || !v_out) FAIL(P, KV_ERR_INVALID, "null argument");
  if (!P->device) FAIL(P, KV_ERR_INVALID, "metadata-only pool");
  if (page < 0 || page >= P->cfg.n_pages || head < 0 || head >= P->cfg.n_kv_heads)
    FAIL(P, KV_ERR_INVALID, "page or head out of range");
  const int D = P->cfg.head_dim;
  const size_t es = dtype_size(P->cfg.dtype);
  const size_t blk = (size_t)kPage * D * es;
  const size_t off = ((size_t)head * P->cfg.n_pages + page) * blk;
  std::vector<char> kr(blk), vr(blk);
  hipError_t e = hipMemcpyAsync(kr.data(), (char*)P->k + off, blk, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(vr.data(), (char*)P->v + off, blk, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, hipGetErrorString(e));
  char* ko = (char*)k_out;
  char* vo = (char*)v_out;
  const int E = (int)(16 / es);
  const int NF = (int)(D * es / 16 / 4);  // 16-byte slots per token row / 4 lane groups
  for (int f = 0; f < NF; ++f)
    for (int g = 0; g < 4; ++g)
      for (int t = 0; t < kPage; ++t)
        for (int e2 = 0; e2 < E; ++e2) {
          const int d = es == 2 ? 32 * f + 8 * g + e2 : 16 * f + 4 * e2 + g;
          std::memcpy(ko + ((size_t)t * D + d) * es, kr.data() + ((((size_t)f * 4 + g) * 16 + t) * E + e2) * es, es);
        }
  for (int d = 0; d < D; ++d)
    for (int t = 0; t < kPage; ++t)
      std::memcpy(vo + ((size_t)t * D + d) * es, vr.data() + ((size_t)d * kPage + v_pos(t)) * es, es);
  return KV_OK;
}

}  // extern "C"
