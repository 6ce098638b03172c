// kv_drop / kv_repos / kv_drop_batch: exact integer plan for compaction, then the fused
// kernel.
//
// AKV (news.farwalk.ai), "AKV 如何工作": Drop removes selected entries from future
// attention without changing positions; Repos rotates the kept keys to positions
// 0..r-1 and leaves the values unchanged; dropped KV is freed only when no live
// request needs it.  AgentKV (rit.work): without physical compaction and freeing
// pages, masking keeps paying HBM reads, so kept entries are packed and freed pages
// return to the allocator.
//
// Plan of one drop (integer, exact):
//   kept = complement of the union of the spans, in order; new slot j <- kept[j];
//   c = first slot whose token or position changes; logical pages [c/P, ceil(r/P))
//   are rewritten -- in place when the page is exclusive (refcount 1), else into the
//   lowest free page (copy-on-write, allocated before anything is released); pages
//   from ceil(r/P) on are released.  Repos: offset_j = j - old position of kept[j];
//   cos/sin rows are computed per distinct offset in fp64.
// The device plan describes the kept tokens as runs (consecutive destination slots whose
// sources are consecutive tokens with one rotation offset) plus the sequence's block
// table before the drop, so its size follows the number of runs and pages, not tokens.
// Several drops (kv_drop_batch) share one upload and one launch unless a later drop
// would write a page an earlier one in the launch still reads.
#include "pool.hpp"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>

using namespace fa;

int fa_set_err(kv_pool* P, int code, const std::string& m);
Seq* fa_seq(kv_pool* P, kv_seq_t s);
hipError_t fa_upload(kv_pool* P, void* dst, const void* src, size_t bytes, hipStream_t s);
void fa_pos_expand(const std::vector<PosRun>& v, std::vector<int64_t>& out);
void fa_pos_append(std::vector<PosRun>& v, int64_t p0, int64_t n);
size_t fa_ws_plan_offset(const kv_pool_config* c);
size_t fa_pool_ws_need(const kv_pool_config* c);
void fa_changed(kv_pool* P, int32_t kind, kv_seq_t seq, int64_t n0, int64_t n1);
#define FAIL(P, code, msg) return fa_set_err((P), (code), (msg))

static constexpr int kMaxRot = 4096;  // distinct repos offsets in one launch

namespace {

// Integer plan of one drop against the current page table (nothing changed yet).
struct DropPlan {
  kv_seq_t seq = -1;
  Seq* S = nullptr;
  bool repos = false;
  std::vector<int64_t> kept, oldpos, newpos;
  int64_t r = 0, c = 0, first = 0, n_new = 0;
  std::vector<int64_t> cow;  // logical pages rewritten into copies
};

int plan_drop(kv_pool* P, kv_seq_t seq, const int64_t* begin, const int64_t* len, int32_t n_spans, bool repos,
              DropPlan& d) {
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (n_spans < 0 || (n_spans > 0 && (!begin || !len))) FAIL(P, KV_ERR_INVALID, "bad spans");
  const int64_t N = S->n;
  const int32_t PS = P->cfg.page_size;
  std::vector<char> gone((size_t)N, 0);
  for (int32_t i = 0; i < n_spans; ++i) {
    if (begin[i] < 0 || len[i] < 0 || begin[i] + len[i] > N) FAIL(P, KV_ERR_INVALID, "span outside the sequence");
    std::fill(gone.begin() + begin[i], gone.begin() + begin[i] + len[i], 1);
  }
  d.seq = seq;
  d.S = S;
  d.repos = repos;
  d.kept.clear();
  d.kept.reserve((size_t)N);
  for (int64_t t = 0; t < N; ++t)
    if (!gone[t]) d.kept.push_back(t);
  d.r = (int64_t)d.kept.size();
  fa_pos_expand(S->pos, d.oldpos);
  d.newpos.resize((size_t)d.r);
  d.c = d.r;
  for (int64_t j = 0; j < d.r; ++j) {
    d.newpos[j] = repos ? j : d.oldpos[d.kept[j]];
    if (d.c == d.r && (d.kept[j] != j || d.newpos[j] != d.oldpos[d.kept[j]])) d.c = j;
  }
  d.first = d.c / PS;
  d.n_new = (d.r + PS - 1) / PS;
  d.cow.clear();
  if (d.c < d.r)
    for (int64_t L = d.first; L < d.n_new; ++L)
      if (P->rc[S->pages[L]] > 1) d.cow.push_back(L);
  return KV_OK;
}

// Page-table update of a planned drop; ids = the copies' pages (lowest free first).
void commit_drop(kv_pool* P, const DropPlan& d, const std::vector<int32_t>& ids, int64_t* kept_src_idx) {
  Seq* S = d.S;
  for (size_t i = 0; i < d.cow.size(); ++i) {
    const int32_t old = S->pages[d.cow[i]];
    P->free.take(ids[i]);
    P->rc[ids[i]] = 1;
    S->pages[d.cow[i]] = ids[i];
    if (--P->rc[old] == 0) P->free.give(old);
  }
  for (size_t L = (size_t)d.n_new; L < S->pages.size(); ++L)
    if (--P->rc[S->pages[L]] == 0) P->free.give(S->pages[L]);
  S->pages.resize((size_t)d.n_new);
  S->n = d.r;
  S->pos.clear();
  for (int64_t j = 0; j < d.r; ++j) fa_pos_append(S->pos, d.newpos[j], 1);
  if (d.repos) S->next_pos = d.r;
  if (kept_src_idx) std::copy(d.kept.begin(), d.kept.end(), kept_src_idx);
  fa_changed(P, ChangeJournal::kOther, d.seq, 0, 0);
}

// Device plan of the drops of one launch.
struct LaunchPlan {
  std::vector<CompactJob> jobs;
  std::vector<CompactPage> pages;
  std::vector<CompactRun> runs;
  std::vector<int32_t> tab;
  std::map<int64_t, int32_t> rot_of;  // repos offset -> cos / sin row
  std::vector<char> reads;            // pool pages the launch's drops read (bitmap over page ids)
  bool empty() const { return pages.empty(); }
  size_t bytes(int D) const {
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return al(jobs.size() * sizeof(CompactJob)) + al(pages.size() * sizeof(CompactPage)) +
           al(runs.size() * sizeof(CompactRun)) + al(tab.size() * 4) + al(rot_of.size() * (size_t)D * 4);
  }
};

// Distinct repos offsets a planned drop needs.
int64_t n_offsets(const DropPlan& d, std::map<int64_t, int32_t>* into) {
  std::map<int64_t, int32_t> own;
  std::map<int64_t, int32_t>& m = into ? *into : own;
  const int64_t PS = kPage;
  int64_t added = 0;
  if (!d.repos || d.c >= d.r) return 0;
  for (int64_t j = d.first * PS; j < d.r; ++j) {
    const int64_t delta = d.newpos[j] - d.oldpos[d.kept[j]];
    if (delta != 0 && m.emplace(delta, (int32_t)m.size()).second) ++added;
  }
  return added;
}

// Would the drop write a page the launch already reads?
bool conflicts(const LaunchPlan& L, const DropPlan& d, const std::vector<int32_t>& ids) {
  if (L.empty()) return false;
  size_t ci = 0;
  for (int64_t Lg = d.first; Lg < d.n_new; ++Lg) {
    const bool is_cow = ci < d.cow.size() && d.cow[ci] == Lg;
    const int32_t dst = is_cow ? ids[ci++] : d.S->pages[Lg];
    if (L.reads[(size_t)dst]) return true;
  }
  return false;
}

// Append a planned drop (before its page-table update) to the launch plan.
void add_drop(LaunchPlan& L, const DropPlan& d, const std::vector<int32_t>& ids) {
  const int64_t PS = kPage;
  const Seq* S = d.S;
  const int32_t list_base = (int32_t)L.pages.size();
  const int64_t n_list = d.n_new - d.first;
  CompactJob job;
  job.list_base = list_base;
  job.n_list = (int32_t)n_list;
  job.first = (int32_t)d.first;
  job.tab_base = (int32_t)L.tab.size();
  L.jobs.push_back(job);
  for (size_t q = (size_t)d.first; q < S->pages.size(); ++q) {
    L.tab.push_back(S->pages[q]);
    L.reads[(size_t)S->pages[q]] = 1;
  }
  // runs over destination slots [first * P, r)
  const int32_t run_base = (int32_t)L.runs.size();
  int64_t prev_src = -2, prev_delta = 0;
  for (int64_t j = d.first * PS; j < d.r; ++j) {
    const int64_t src = d.kept[j];
    const int64_t delta = d.newpos[j] - d.oldpos[src];
    if (j == d.first * PS || src != prev_src + 1 || delta != prev_delta) {
      int32_t rot = -1;
      if (d.repos && delta != 0) rot = L.rot_of.emplace(delta, (int32_t)L.rot_of.size()).first->second;
      L.runs.push_back({(int32_t)j, (int32_t)src, 0, rot});
    }
    L.runs.back().len++;
    prev_src = src;
    prev_delta = delta;
  }
  // destination pages; an in-place page waits for the lower entries that read it
  std::vector<int64_t> min_reader(S->pages.size(), -1), max_reader(S->pages.size(), -1);
  size_t ci = 0;
  int32_t run = run_base;
  for (int64_t Lg = d.first; Lg < d.n_new; ++Lg) {
    const bool is_cow = ci < d.cow.size() && d.cow[ci] == Lg;
    CompactPage cp;
    cp.dst_page = is_cow ? ids[ci] : S->pages[Lg];
    const int32_t first_slot = (!is_cow && Lg == d.first) ? (int32_t)(d.c % PS) : 0;
    const int32_t n_slots = (int32_t)std::min<int64_t>(PS, d.r - Lg * PS);
    cp.slots = first_slot | (n_slots << 8) | (is_cow ? 1 << 16 : 0);
    const int64_t j0 = Lg * PS + first_slot;
    while (L.runs[run].j0 + L.runs[run].len <= j0) ++run;
    cp.run0 = run;
    cp.wait = 0;
    if (is_cow) ++ci;
    for (int64_t j = j0; j < Lg * PS + n_slots; ++j) {
      const int64_t Lo = d.kept[j] / PS;
      if (min_reader[Lo] < 0) min_reader[Lo] = Lg;
      max_reader[Lo] = Lg;
    }
    L.pages.push_back(cp);
  }
  for (int64_t Lg = d.first; Lg < d.n_new; ++Lg) {
    CompactPage& cp = L.pages[(size_t)(list_base + Lg - d.first)];
    if (!(cp.slots >> 16 & 1) && min_reader[Lg] >= 0) {  // in place, read by lower entries
      const int64_t hi = std::min<int64_t>(max_reader[Lg], Lg - 1);
      if (hi >= min_reader[Lg])  // at most two readers: a source page's kept tokens are consecutive
        cp.wait = (int32_t)(list_base + min_reader[Lg] - d.first) | (int32_t)((hi - min_reader[Lg] + 1) << 30);
    }
    cp.slots = (cp.slots & 0xffff) | (int32_t)((L.jobs.size() - 1) << 16);
  }
}

hipError_t launch_plan(kv_pool* P, LaunchPlan& L, hipStream_t s) {
  if (L.empty()) return hipSuccess;
  const int D = P->cfg.head_dim;
  std::vector<float> cs(L.rot_of.size() * (size_t)D, 0.f);
  for (const auto& kv : L.rot_of)
    for (int i = 0; i < D / 2; ++i) {
      const double ang = (double)kv.first * std::pow(P->cfg.rope_theta, -2.0 * i / D);
      cs[(size_t)kv.second * D + 2 * i] = (float)std::cos(ang);
      cs[(size_t)kv.second * D + 2 * i + 1] = (float)std::sin(ang);
    }
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t o_jobs = 0;
  const size_t o_pages = al(o_jobs + L.jobs.size() * sizeof(CompactJob));
  const size_t o_runs = al(o_pages + L.pages.size() * sizeof(CompactPage));
  const size_t o_tab = al(o_runs + L.runs.size() * sizeof(CompactRun));
  const size_t o_cs = al(o_tab + L.tab.size() * 4);
  const size_t total = al(o_cs + cs.size() * 4);
  std::vector<char> blob(total, 0);
  std::memcpy(blob.data() + o_jobs, L.jobs.data(), L.jobs.size() * sizeof(CompactJob));
  std::memcpy(blob.data() + o_pages, L.pages.data(), L.pages.size() * sizeof(CompactPage));
  std::memcpy(blob.data() + o_runs, L.runs.data(), L.runs.size() * sizeof(CompactRun));
  std::memcpy(blob.data() + o_tab, L.tab.data(), L.tab.size() * 4);
  if (!cs.empty()) std::memcpy(blob.data() + o_cs, cs.data(), cs.size() * 4);
  char* area = P->ws + fa_ws_plan_offset(&P->cfg);
  hipError_t e = fa_upload(P, area, blob.data(), total, s);
  if (e != hipSuccess) return e;
  CompactParams cp;
  cp.k_pages = P->k;
  cp.v_pages = P->v;
  cp.jobs = reinterpret_cast<const CompactJob*>(area + o_jobs);
  cp.pages = reinterpret_cast<const CompactPage*>(area + o_pages);
  cp.runs = reinterpret_cast<const CompactRun*>(area + o_runs);
  cp.tab = reinterpret_cast<const int32_t*>(area + o_tab);
  cp.cos_sin = reinterpret_cast<const float*>(area + o_cs);
  cp.errors = reinterpret_cast<int32_t*>(P->ws) + 1;
  cp.done = reinterpret_cast<int32_t*>(P->ws + 4096);
  cp.epoch = P->epoch + 1;
  cp.n_jobs = (int32_t)L.jobs.size();
  cp.n_pages = (int32_t)L.pages.size();
  cp.n_kv_heads = P->cfg.n_kv_heads;
  cp.pool_pages = P->cfg.n_pages;
  e = launch_compact(P->cfg.dtype, D, cp, s);
  if (e == hipSuccess) P->epoch += 1;
  return e;
}

void reset(LaunchPlan& L, int32_t n_pages) {
  L.jobs.clear();
  L.pages.clear();
  L.runs.clear();
  L.tab.clear();
  L.rot_of.clear();
  L.reads.assign((size_t)n_pages, 0);
}

}  // namespace

// Drops of n distinct sequences, exactly as n kv_drop calls in list order; the device
// work of consecutive drops shares one plan upload and one launch.
static int drop_many(kv_pool_t* P, int32_t n, const kv_seq_t* seqs, const int64_t* span_off, const int64_t* begin,
                     const int64_t* len, int32_t flags, int64_t* kept_src_idx, hipStream_t s) {
  if (n < 0 || (n > 0 && (!seqs || !span_off)) || (flags & ~KV_DROP_REPOS)) FAIL(P, KV_ERR_INVALID, "bad arguments");
  const bool repos = flags & KV_DROP_REPOS;
  if (repos && P->device && P->cfg.rope_style != KV_ROPE_NEOX) FAIL(P, KV_ERR_UNSUPPORTED, "repos needs a rotary pool");
  if (P->device && !compact_supported(P->cfg.dtype, P->cfg.head_dim, P->cfg.n_kv_heads))
    FAIL(P, KV_ERR_UNSUPPORTED, "drop supports up to 16 KV heads (bf16, d = 128) on device pools");
  // validate everything first, so a failure changes nothing: live distinct sequences,
  // spans inside them, offsets per drop within the table, and copies that fit even if no
  // earlier drop of the list released a page (refcounts only fall during the list)
  {
    std::vector<kv_seq_t> sorted(seqs, seqs + n);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
      FAIL(P, KV_ERR_INVALID, "a sequence appears twice in the list");
  }
  int64_t cow_bound = 0;
  DropPlan d;
  for (int32_t i = 0; i < n; ++i) {
    if (span_off[i] < 0 || span_off[i + 1] < span_off[i] || span_off[i + 1] - span_off[i] > INT32_MAX)
      FAIL(P, KV_ERR_INVALID, "bad span offsets");
    const int32_t ns = (int32_t)(span_off[i + 1] - span_off[i]);
    if (int st = plan_drop(P, seqs[i], ns ? begin + span_off[i] : nullptr, ns ? len + span_off[i] : nullptr, ns,
                           repos, d))
      return st;
    cow_bound += (int64_t)d.cow.size();
    if (P->device && n_offsets(d, nullptr) > kMaxRot)
      FAIL(P, KV_ERR_WORKSPACE, "too many distinct repos offsets in one drop");
  }
  if (cow_bound > P->free.count()) FAIL(P, KV_ERR_OOM, "not enough free pages for copies");
  const size_t area = P->device ? fa_pool_ws_need(&P->cfg) - fa_ws_plan_offset(&P->cfg) : 0;
  LaunchPlan L;
  reset(L, P->cfg.n_pages);
  int64_t out_at = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t ns = (int32_t)(span_off[i + 1] - span_off[i]);
    plan_drop(P, seqs[i], ns ? begin + span_off[i] : nullptr, ns ? len + span_off[i] : nullptr, ns, repos, d);
    std::vector<int32_t> ids;
    P->free.peek_lowest((int32_t)d.cow.size(), ids);
    if (P->device && d.c < d.r) {
      std::map<int64_t, int32_t> rot = L.rot_of;
      const bool rot_full = n_offsets(d, &rot) + (int64_t)L.rot_of.size() > kMaxRot;
      const size_t add = (size_t)(d.n_new - d.first) * sizeof(CompactPage) +
                         (size_t)(d.S->pages.size() - d.first) * 4 + (size_t)(d.r - d.first * kPage) * sizeof(CompactRun);
      if (!L.empty() && (rot_full || L.jobs.size() >= 0xffff || conflicts(L, d, ids) ||
                         L.bytes(P->cfg.head_dim) + add + 4096 > area)) {
        hipError_t e = launch_plan(P, L, s);
        if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("compaction: ") + hipGetErrorString(e));
        reset(L, P->cfg.n_pages);
      }
      add_drop(L, d, ids);
    }
    commit_drop(P, d, ids, kept_src_idx ? kept_src_idx + out_at : nullptr);
    out_at += (int64_t)d.oldpos.size();
  }
  if (P->device) {
    hipError_t e = launch_plan(P, L, s);
    if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("compaction: ") + hipGetErrorString(e));
  }
  return KV_OK;
}

extern "C" {

int kv_drop(kv_pool_t* P, kv_seq_t seq, const int64_t* begin, const int64_t* len, int32_t n_spans,
            int32_t flags, int64_t* kept_src_idx, hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  if (n_spans < 0) FAIL(P, KV_ERR_INVALID, "bad spans or flags");
  const int64_t off[2] = {0, n_spans};
  return drop_many(P, 1, &seq, off, begin, len, flags, kept_src_idx, s);
}

int kv_drop_batch(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, const int64_t* span_off, const int64_t* begin,
                  const int64_t* len, int32_t flags, int64_t* kept_src_idx, hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  return drop_many(P, n, seqs, span_off, begin, len, flags, kept_src_idx, s);
}

int kv_repos(kv_pool_t* P, kv_seq_t seq, hipStream_t s) {
  return kv_drop(P, seq, nullptr, nullptr, 0, KV_DROP_REPOS, nullptr, s);
}

int kv_pool_sync_status(kv_pool_t* P, hipStream_t s, int32_t* n_wait_timeouts) {
  if (!P || !n_wait_timeouts) FAIL(P, KV_ERR_INVALID, "null argument");
  *n_wait_timeouts = 0;
  if (!P->device) return KV_OK;
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, P->ws + 4, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, hipGetErrorString(e));
  *n_wait_timeouts = v;
  return KV_OK;
}

}  // extern "C"
