// kv_drop / kv_repos: exact integer plan for compaction, then the fused kernel.
//
// AKV (news.farwalk.ai), "AKV 如何工作": Drop removes selected entries from future
// attention without changing positions; Repos rotates the kept keys to positions
// 0..r-1 and leaves the values unchanged; dropped KV is freed only when no live
// request needs it.  AgentKV (rit.work): without physical compaction and freeing
// pages, masking keeps paying HBM reads, so kept entries are packed and freed pages
// return to the allocator.
//
// Plan (integer, exact):
//   kept = complement of the union of the spans, in order; new slot j <- kept[j];
//   c = first slot whose token or position changes; logical pages [c/P, ceil(r/P))
//   are rewritten -- in place when the page is exclusive (refcount 1), else into the
//   lowest free page (copy-on-write, allocated before anything is released); pages
//   from ceil(r/P) on are released.  Repos: offset_j = j - old position of kept[j];
//   cos/sin rows are computed per distinct offset in fp64.
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
#define FAIL(P, code, msg) return fa_set_err((P), (code), (msg))

static constexpr int kMaxRot = 4096;

extern "C" {

int kv_drop(kv_pool_t* P, kv_seq_t seq, const int64_t* begin, const int64_t* len, int32_t n_spans,
            int32_t flags, int64_t* kept_src_idx, hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (n_spans < 0 || (n_spans > 0 && (!begin || !len)) || (flags & ~KV_DROP_REPOS))
    FAIL(P, KV_ERR_INVALID, "bad spans or flags");
  const bool repos = flags & KV_DROP_REPOS;
  if (repos && P->device && P->cfg.rope_style != KV_ROPE_NEOX)
    FAIL(P, KV_ERR_UNSUPPORTED, "repos needs a rotary pool");
  if (P->device && !compact_supported(P->cfg.dtype, P->cfg.head_dim, P->cfg.n_kv_heads))
    FAIL(P, KV_ERR_UNSUPPORTED, "drop supports up to 16 KV heads (bf16, d = 128) on device pools");
  const int64_t N = S->n;
  const int32_t PS = P->cfg.page_size;
  std::vector<char> gone((size_t)N, 0);
  for (int32_t i = 0; i < n_spans; ++i) {
    if (begin[i] < 0 || len[i] < 0 || begin[i] + len[i] > N) FAIL(P, KV_ERR_INVALID, "span outside the sequence");
    std::fill(gone.begin() + begin[i], gone.begin() + begin[i] + len[i], 1);
  }
  std::vector<int64_t> kept;
  kept.reserve((size_t)N);
  for (int64_t t = 0; t < N; ++t)
    if (!gone[t]) kept.push_back(t);
  const int64_t r = (int64_t)kept.size();
  std::vector<int64_t> oldpos;
  fa_pos_expand(S->pos, oldpos);
  std::vector<int64_t> newpos((size_t)r);
  int64_t c = r;
  for (int64_t j = 0; j < r; ++j) {
    newpos[j] = repos ? j : oldpos[kept[j]];
    if (c == r && (kept[j] != j || newpos[j] != oldpos[kept[j]])) c = j;
  }
  const int64_t first = c / PS, n_new = (r + PS - 1) / PS;
  std::vector<int64_t> cow;
  if (c < r)
    for (int64_t L = first; L < n_new; ++L)
      if (P->rc[S->pages[L]] > 1) cow.push_back(L);
  if ((int64_t)cow.size() > P->free.count()) FAIL(P, KV_ERR_OOM, "not enough free pages for copies");
  std::vector<int32_t> ids;
  P->free.peek_lowest((int32_t)cow.size(), ids);

  if (P->device && c < r) {
    const int D = P->cfg.head_dim;
    const int64_t n_list = n_new - first;
    const int64_t tok0 = first * PS;
    std::vector<CompactPage> pages((size_t)n_list);
    std::vector<int32_t> src_loc((size_t)(r - tok0)), rot((size_t)(r - tok0), -1);
    std::map<int64_t, int32_t> rot_of;
    std::vector<int64_t> min_reader((size_t)S->pages.size(), -1), max_reader((size_t)S->pages.size(), -1);
    size_t ci = 0;
    for (int64_t L = first; L < n_new; ++L) {
      const bool is_cow = ci < cow.size() && cow[ci] == L;
      CompactPage& cp = pages[(size_t)(L - first)];
      cp.dst_page = is_cow ? ids[ci] : S->pages[L];
      cp.first_slot = (!is_cow && L == first) ? (int32_t)(c % PS) : 0;
      cp.n_slots = (int32_t)std::min<int64_t>(PS, r - L * PS);
      cp.tok_base = (int32_t)(L * PS - tok0);
      cp.wait_lo = cp.wait_hi = (int32_t)(L - first);  // set below for pages rewritten in place
      cp.pad[0] = is_cow ? 1 : 0;                        // host bookkeeping only
      cp.pad[1] = 0;
      if (is_cow) ++ci;
      for (int64_t j = L * PS + cp.first_slot; j < L * PS + cp.n_slots; ++j) {
        const int64_t src = kept[j];
        const int64_t Lo = src / PS;
        src_loc[(size_t)(j - tok0)] = S->pages[Lo] * 16 + (int32_t)(src % PS);
        if (min_reader[Lo] < 0) min_reader[Lo] = L;
        max_reader[Lo] = L;
        const int64_t delta = newpos[j] - oldpos[src];
        if (repos && delta != 0) {
          auto it = rot_of.find(delta);
          if (it == rot_of.end()) {
            if ((int)rot_of.size() >= kMaxRot) FAIL(P, KV_ERR_WORKSPACE, "too many distinct repos offsets in one call");
            it = rot_of.emplace(delta, (int32_t)rot_of.size()).first;
          }
          rot[(size_t)(j - tok0)] = it->second;
        }
      }
    }
    for (int64_t L = first; L < n_new; ++L) {
      CompactPage& cp = pages[(size_t)(L - first)];
      if (!cp.pad[0] && min_reader[L] >= 0) {  // in place: wait for the lower entries that read it
        cp.wait_lo = (int32_t)(min_reader[L] - first);
        cp.wait_hi = (int32_t)(std::min<int64_t>(max_reader[L], L - 1) - first + 1);
      }
      cp.pad[0] = 0;
    }
    std::vector<float> cs((size_t)rot_of.size() * D, 0.f);
    for (const auto& kv : rot_of)
      for (int i = 0; i < D / 2; ++i) {
        const double ang = (double)kv.first * std::pow(P->cfg.rope_theta, -2.0 * i / D);
        cs[(size_t)kv.second * D + 2 * i] = (float)std::cos(ang);
        cs[(size_t)kv.second * D + 2 * i + 1] = (float)std::sin(ang);
      }
    // blob: pages | src_loc | rot | cos_sin
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t o_pages = 0;
    const size_t o_src = al(o_pages + pages.size() * sizeof(CompactPage));
    const size_t o_rot = al(o_src + src_loc.size() * 4);
    const size_t o_cs = al(o_rot + rot.size() * 4);
    const size_t total = al(o_cs + cs.size() * 4);
    const size_t base = fa_ws_plan_offset(&P->cfg);
    if (base + total > P->ws_bytes) FAIL(P, KV_ERR_WORKSPACE, "pool workspace too small for this drop");
    std::vector<char> blob(total, 0);
    std::memcpy(blob.data() + o_pages, pages.data(), pages.size() * sizeof(CompactPage));
    std::memcpy(blob.data() + o_src, src_loc.data(), src_loc.size() * 4);
    std::memcpy(blob.data() + o_rot, rot.data(), rot.size() * 4);
    if (!cs.empty()) std::memcpy(blob.data() + o_cs, cs.data(), cs.size() * 4);
    char* area = P->ws + base;
    hipError_t e = fa_upload(P, area, blob.data(), total, s);
    if (e == hipSuccess) {
      CompactParams cp;
      cp.k_pages = P->k;
      cp.v_pages = P->v;
      cp.pages = reinterpret_cast<const CompactPage*>(area + o_pages);
      cp.src_loc = reinterpret_cast<const int32_t*>(area + o_src);
      cp.rot = reinterpret_cast<const int32_t*>(area + o_rot);
      cp.cos_sin = reinterpret_cast<const float*>(area + o_cs);
      cp.ticket = reinterpret_cast<int32_t*>(P->ws);
      cp.errors = reinterpret_cast<int32_t*>(P->ws) + 1;
      cp.done = reinterpret_cast<int32_t*>(P->ws + 4096);
      cp.ticket_base = P->ticket;
      cp.epoch = P->epoch + 1;
      cp.n_pages = (int32_t)n_list;
      cp.n_kv_heads = P->cfg.n_kv_heads;
      cp.pool_pages = P->cfg.n_pages;
      e = launch_compact(P->cfg.dtype, D, cp, s);
      if (e == hipSuccess) {
        P->ticket = (int32_t)((uint32_t)P->ticket + (uint32_t)((n_list + kCompactBatch - 1) / kCompactBatch));
        P->epoch += 1;
      }
    }
    if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("compaction: ") + hipGetErrorString(e));
  }

  // metadata
  for (size_t i = 0; i < cow.size(); ++i) {
    const int32_t old = S->pages[cow[i]];
    P->free.take(ids[i]);
    P->rc[ids[i]] = 1;
    S->pages[cow[i]] = ids[i];
    if (--P->rc[old] == 0) P->free.give(old);
  }
  for (size_t L = (size_t)n_new; L < S->pages.size(); ++L)
    if (--P->rc[S->pages[L]] == 0) P->free.give(S->pages[L]);
  S->pages.resize((size_t)n_new);
  S->n = r;
  S->pos.clear();
  for (int64_t j = 0; j < r; ++j) fa_pos_append(S->pos, newpos[j], 1);
  if (repos) S->next_pos = r;
  if (kept_src_idx) std::copy(kept.begin(), kept.end(), kept_src_idx);
  P->version++;
  return KV_OK;
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
