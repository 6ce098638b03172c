// Segment planner and fork_attn_decode.
//
// Agentrix README (gitlink.org.cn), "前缀复用与 ForkAttention" and the CUDA ForkAttention
// item: the context of branches decoding together is split into public and private
// segments by the actual cache pages; several queries reuse the loaded public K/V and
// each branch's results are merged.  Octopus (zicq.com), "Attention-Only KV Mounting":
// a thread also attends to mounted sibling blocks, so reader sets differ page by page.
//
// Plan:
//   1. every query row's visible token runs (own pages, then mounts) as
//      (page, lo, hi, reader) entries;
//   2. per physical page, split the slot range at every run boundary and collect the
//      reader multiset of each piece -> chunks; equal reader multisets form one segment
//      (public = many readers, private = one);
//   3. per segment, reader groups of at most 64 / G readers (64 MFMA rows), per KV head,
//      the chunk list is cut into work items of about equal bytes sized so the whole
//      decode is about two workgroups per compute unit;
//   4. every (item, row) owns one partial slot; slots are ordered by output row, so a
//      row's partials are contiguous; the same launch merges them.
#include "pool.hpp"

#include <algorithm>
#include <atomic>
#include <cstring>
#include <map>
#include <climits>
#include <unordered_map>

using namespace fa;

int fa_set_err(kv_pool* P, int code, const std::string& m);
Seq* fa_seq(kv_pool* P, kv_seq_t s);
hipError_t fa_upload(kv_pool* P, void* dst, const void* src, size_t bytes, hipStream_t s);
void fa_take_page(kv_pool* P, int32_t p);
void fa_unref_page(kv_pool* P, int32_t p);
void fa_pos_append(std::vector<PosRun>& v, int64_t p0, int64_t n);
void fa_changed(kv_pool* P, int32_t kind, kv_seq_t seq, int64_t n0, int64_t n1);
hipError_t fa_upload(kv_pool* P, void* dst, const void* src, size_t bytes, hipStream_t s);
size_t fa_ws_plan_offset(const kv_pool_config* c);
size_t fa_pool_ws_need(const kv_pool_config* c);
#define FAIL(P, code, msg) return fa_set_err((P), (code), (msg))

namespace {

// one visible run: slots [lo, hi) of a page read by query `reader` (12 bytes: the sort
// moves tens of thousands of these per plan)
struct Entry {
  int32_t page;
  int32_t rd;
  uint16_t l, h;
  Entry() = default;
  Entry(int32_t p, int32_t lo, int32_t hi, int32_t reader) : page(p), rd(reader), l((uint16_t)lo), h((uint16_t)hi) {}
  int32_t lo() const { return l; }
  int32_t hi() const { return h; }
  int32_t reader() const { return rd; }
};

struct Segment {
  std::vector<int32_t> readers;  // sorted multiset of query indices
  std::vector<Chunk> chunks;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr size_t kMaxCutRanges = 4;  // slot ranges of one page cut into shared chunks

template <typename T>
void put(std::vector<char>& blob, size_t off, const std::vector<T>& v) {
  if (!v.empty()) std::memcpy(blob.data() + off, v.data(), v.size() * sizeof(T));
}

}  // namespace

static std::atomic<uint64_t> g_plan_serial{0};

// Bring the cached decode plan up to date with the journal's changes without replanning:
// possible when every change to a listed sequence is an append that wrote only into pages
// the sequence owns alone -- its tail page (already its query's private chunk) grows, and
// new pages join the last work item of the query's private segment for every KV head.
// Records are patched in the host image; the changed ints are queued for the device.
// false: replan (the image may be half patched; the replan rewrites all of it).
static bool patch_plan(kv_pool* P) {
  DecodePlanCache& pc = P->plan;
  const ChangeJournal& J = P->journal;
  const kv_pool_config& C = P->cfg;
  const int32_t PS = C.page_size, H = C.n_kv_heads;
  if (!pc.patchable || J.broken || J.base != pc.version || J.base + J.ev.size() != P->version) return false;
  int32_t* recs = reinterpret_cast<int32_t*>(pc.blob.data() + pc.off_items);
  const int32_t base_int = (int32_t)(pc.off_items / sizeof(int32_t));
  auto set = [&](int32_t rec, int32_t at, int32_t val) {
    recs[(size_t)rec * kRecInts + at] = val;
    pc.pending.push_back(base_int + rec * kRecInts + at);
    pc.pending.push_back(val);
  };
  const size_t es = C.dtype == KV_F32 ? 4 : 2;
  for (const ChangeJournal::Event& e : J.ev) {
    if (e.kind == ChangeJournal::kContent) continue;
    int32_t i = -1;
    for (size_t q = 0; q < pc.seqs.size(); ++q)
      if (pc.seqs[q] == e.seq) i = pc.q_seq[q] >= 0 ? (int32_t)q : -2;
    if (i == -1) continue;  // a sequence no query reads
    if (i < 0 || e.kind != ChangeJournal::kAppend || e.n0 != pc.q_own_n[i]) return false;
    const Seq* S = fa_seq(P, e.seq);
    if (!S || (int64_t)S->pages.size() * PS < e.n1) return false;
    int64_t L = e.n0 / PS;
    if (e.n0 % PS) {  // the tail page grows
      if (S->pages[(size_t)L] != pc.q_tail_page[i]) return false;
      for (int32_t h = 0; h < H; ++h) {
        const int32_t r = pc.tail_rec[(size_t)i * H + h], sl = pc.tail_slot[(size_t)i * H + h];
        if (r < 0) return false;
        const int32_t at = kRecChunk + 2 * sl + 1;
        const int32_t lo = recs[(size_t)r * kRecInts + at] & 0xff;
        set(r, at, lo | (int32_t)std::min<int64_t>(PS, e.n1 - L * PS) << 8);
      }
      ++L;
    }
    for (; L * PS < e.n1; ++L) {  // new pages
      const int32_t page = S->pages[(size_t)L];
      const int32_t lohi = (int32_t)std::min<int64_t>(PS, e.n1 - L * PS) << 8;
      for (int32_t h = 0; h < H; ++h) {
        const int32_t r = pc.last_rec[(size_t)i * H + h];
        if (r < 0) return false;
        const int32_t nc = recs[(size_t)r * kRecInts];
        if (nc >= kMaxItemChunks) return false;
        set(r, kRecChunk + 2 * nc, page);
        set(r, kRecChunk + 2 * nc + 1, lohi);
        set(r, 0, nc + 1);
        pc.tail_rec[(size_t)i * H + h] = r;
        pc.tail_slot[(size_t)i * H + h] = nc;
        pc.stats[6] = std::max<int64_t>(pc.stats[6], nc + 1);
      }
      pc.q_tail_page[i] = page;
      pc.stats[2] += 1;
    }
    pc.q_own_n[i] = (int32_t)e.n1;
    pc.stats[4] += (e.n1 - e.n0) * H * 2 * C.head_dim * (int64_t)es;
  }
  pc.version = P->version;
  pc.serial = ++g_plan_serial;
  pc.stats[7] += 1;
  P->journal.reset(P->version);
  return true;
}

// len_cap (optional): per query, the number of its sequence's own tokens to attend to
// (a prefix of the own context); the cached plan is bypassed and left invalid.
static int build_plan(kv_pool* P, const kv_seq_t* seqs, int32_t n, int32_t hq, const int64_t* len_cap = nullptr) {
  const kv_pool_config& C = P->cfg;
  if (n < 0 || (n > 0 && !seqs)) FAIL(P, KV_ERR_INVALID, "bad sequence list");
  if (hq < C.n_kv_heads || hq % C.n_kv_heads) FAIL(P, KV_ERR_INVALID, "n_q_heads must be a multiple of n_kv_heads");
  const int32_t G = hq / C.n_kv_heads;
  if (G > kMaxRows) FAIL(P, KV_ERR_UNSUPPORTED, "more than 64 query heads per KV head");
  const int32_t PS = C.page_size;
  DecodePlanCache& pc = P->plan;
  if (!len_cap && pc.valid && pc.causal_n == 0 && pc.n_q_heads == hq && (int32_t)pc.seqs.size() == n &&
      std::equal(pc.seqs.begin(), pc.seqs.end(), seqs) && (pc.version == P->version || patch_plan(P)))
    return KV_OK;
  pc.pending.clear();

  // 1. visible runs
  std::vector<Seq*> qs((size_t)n);
  size_t n_ent = 0;
  for (int32_t i = 0; i < n; ++i) {
    qs[i] = fa_seq(P, seqs[i]);
    if (!qs[i]) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence in the query list");
    const int64_t n_own = len_cap ? std::min<int64_t>(len_cap[i], qs[i]->n) : qs[i]->n;
    n_ent += (size_t)((n_own + PS - 1) / PS);
    for (const Mount& m : qs[i]->mounts) n_ent += m.pages.size();
  }
  // the entry buffers persist per thread: fresh ones of this size cost page faults
  static thread_local std::vector<Entry> ent, sorted;
  ent.clear();
  ent.reserve(n_ent);
  int32_t max_page = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Seq* S = qs[i];
    const int64_t n_own = len_cap ? std::min<int64_t>(len_cap[i], S->n) : S->n;
    for (size_t L = 0; (int64_t)L * PS < n_own; ++L) {
      ent.push_back({S->pages[L], 0, (int32_t)std::min<int64_t>(PS, n_own - (int64_t)L * PS), i});
      max_page = std::max(max_page, S->pages[L]);
    }
    for (const Mount& m : S->mounts) {
      for (size_t j = 0; j < m.pages.size(); ++j) {
        const int64_t a = std::max<int64_t>(0, m.off - (int64_t)j * PS);
        const int64_t b = std::min<int64_t>(PS, m.off + m.n - (int64_t)j * PS);
        if (a < b) {
          ent.push_back({m.pages[j], (int32_t)a, (int32_t)b, i});
          max_page = std::max(max_page, m.pages[j]);
        }
      }
    }
  }
  {  // stable counting sort by page id (readers of a page keep query order): one pass when
     // the page ids are dense enough for a histogram over all of them, else LSD radix
     // passes of at most 11 bits
    sorted.resize(ent.size());
    if ((size_t)max_page + 1 <= std::max<size_t>(4096, 2 * ent.size())) {
      std::vector<int32_t> h((size_t)max_page + 2, 0);
      for (const Entry& e : ent) h[(size_t)e.page + 1]++;
      for (size_t d = 1; d < h.size(); ++d) h[d] += h[d - 1];
      for (const Entry& e : ent) sorted[(size_t)h[(size_t)e.page]++] = e;
      ent.swap(sorted);
    } else {
      int bits = 0;
      while (bits < 31 && ((int64_t)1 << bits) <= max_page) ++bits;
      const int n_pass = (bits + 10) / 11;
      const int db = (bits + n_pass - 1) / n_pass;
      const uint32_t mask = (1u << db) - 1;
      std::vector<int32_t> hist((size_t)n_pass << db, 0);
      for (const Entry& e : ent)
        for (int k = 0; k < n_pass; ++k) hist[((size_t)k << db) + ((uint32_t)e.page >> (k * db) & mask)]++;
      for (int k = 0; k < n_pass; ++k) {
        int32_t* h = hist.data() + ((size_t)k << db);
        int32_t run = 0;
        for (uint32_t d = 0; d <= mask; ++d) {
          const int32_t c = h[d];
          h[d] = run;
          run += c;
        }
        for (const Entry& e : ent) sorted[(size_t)h[(uint32_t)e.page >> (k * db) & mask]++] = e;
        ent.swap(sorted);
      }
    }
  }

  // 2. chunks grouped into segments by reader multiset
  std::vector<Segment> segs;
  std::map<std::vector<int32_t>, int32_t> seg_of;
  std::vector<int32_t> key, last_key;
  int32_t last_seg = -1;
  auto emit = [&](int32_t page, int32_t lo, int32_t hi, std::vector<int32_t>& readers) {
    std::sort(readers.begin(), readers.end());
    int32_t sid;
    if (last_seg >= 0 && readers == last_key) {
      sid = last_seg;
    } else {
      auto it = seg_of.find(readers);
      if (it == seg_of.end()) {
        sid = (int32_t)segs.size();
        seg_of.emplace(readers, sid);
        segs.push_back({readers, {}});
      } else {
        sid = it->second;
      }
      last_key = readers;
      last_seg = sid;
    }
    segs[sid].chunks.push_back({page, lo | (hi << 8)});
  };
  for (size_t a = 0; a < ent.size();) {
    size_t b = a;
    bool uniform = true;
    while (b < ent.size() && ent[b].page == ent[a].page) {
      uniform = uniform && ent[b].lo() == ent[a].lo() && ent[b].hi() == ent[a].hi();
      ++b;
    }
    if (uniform) {
      key.clear();
      for (size_t e = a; e < b; ++e) key.push_back(ent[e].reader());
      emit(ent[a].page, ent[a].lo(), ent[a].hi(), key);
    } else {
      std::vector<int32_t> cuts;
      for (size_t e = a; e < b; ++e) {
        cuts.push_back(ent[e].lo());
        cuts.push_back(ent[e].hi());
      }
      std::sort(cuts.begin(), cuts.end());
      cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
      if (cuts.size() <= kMaxCutRanges + 1) {
        // a few slot ranges: one chunk per range, read by every reader that covers it
        for (size_t c = 0; c + 1 < cuts.size(); ++c) {
          key.clear();
          for (size_t e = a; e < b; ++e)
            if (ent[e].lo() <= cuts[c] && ent[e].hi() >= cuts[c + 1]) key.push_back(ent[e].reader());
          if (!key.empty()) emit(ent[a].page, cuts[c], cuts[c + 1], key);
        }
      } else {
        // many ranges (a causal diagonal page: each of its own tokens reads up to itself):
        // the readers of the most common range share one chunk, every other reader reads
        // its own range alone, instead of one reader set per distinct range
        std::map<std::pair<int32_t, int32_t>, int32_t> freq;
        for (size_t e = a; e < b; ++e) ++freq[{ent[e].lo(), ent[e].hi()}];
        std::pair<int32_t, int32_t> top = freq.begin()->first;
        for (const auto& f : freq)
          if (f.second > freq[top]) top = f.first;
        key.clear();
        for (size_t e = a; e < b; ++e)
          if (ent[e].lo() == top.first && ent[e].hi() == top.second) key.push_back(ent[e].reader());
        emit(ent[a].page, top.first, top.second, key);
        for (size_t e = a; e < b; ++e)
          if (!(ent[e].lo() == top.first && ent[e].hi() == top.second)) {
            key.assign(1, ent[e].reader());
            emit(ent[a].page, ent[e].lo(), ent[e].hi(), key);
          }
      }
    }
    a = b;
  }

  // 3. work items of <= 64 rows and <= kMaxItemChunks chunks, sized so the decode is
  // about two workgroups per compute unit.
  const int32_t per_group = std::max(1, kMaxRows / G);
  int64_t total = 0;
  for (const Segment& s : segs) {
    const int64_t groups = ((int64_t)s.readers.size() + per_group - 1) / per_group;
    total += (int64_t)s.chunks.size() * C.n_kv_heads * groups;
  }
  const int64_t target_items = std::max<int64_t>(1, 2 * (int64_t)P->n_cu);
  const int64_t cpi = std::min<int64_t>(kMaxItemChunks,
                                        std::max<int64_t>(8, (total + target_items - 1) / target_items));

  struct Item {
    int32_t chunk_begin, n_chunks, kv_head, rows;
    const Segment* seg;
    int32_t g0;
  };
  auto orow_of = [&](const Item& it, int32_t r) { return it.seg->readers[(size_t)it.g0 + r / G] * hq + it.kv_head * G + r % G; };
  std::vector<Item> items;
  int64_t unique_tokens = 0, n_chunks_total = 0;
  const int32_t n_out = n * hq;
  std::vector<int32_t> row_count((size_t)n_out, 0);
  for (const Segment& s : segs) {
    for (const Chunk& c : s.chunks) unique_tokens += (c.lohi >> 8) - (c.lohi & 0xff);
    n_chunks_total += (int64_t)s.chunks.size();
    const int32_t nc = (int32_t)s.chunks.size();
    const int32_t n_it = (int32_t)((nc + cpi - 1) / cpi);
    for (size_t g0 = 0; g0 < s.readers.size(); g0 += per_group) {
      const int32_t ng = (int32_t)std::min<size_t>(per_group, s.readers.size() - g0);
      const int32_t rows = ng * G;
      for (int32_t h = 0; h < C.n_kv_heads; ++h) {
        for (int32_t t = 0; t < n_it; ++t) {
          const int32_t c0 = (int32_t)((int64_t)nc * t / n_it), c1 = (int32_t)((int64_t)nc * (t + 1) / n_it);
          items.push_back(Item{c0, c1 - c0, h, rows, &s, (int32_t)g0});
          for (int32_t r = 0; r < rows; ++r) row_count[(size_t)orow_of(items.back(), r)]++;
        }
      }
    }
  }
  // heaviest items first
  std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) { return a.n_chunks > b.n_chunks; });
  // partial slots: output row r owns the block [r * max_parts, (r + 1) * max_parts)
  int32_t max_parts = 1;
  for (int32_t r = 0; r < n_out; ++r) max_parts = std::max(max_parts, row_count[r]);
  const int64_t n_part_slots = (int64_t)n_out * max_parts;
  int64_t n_part = 0;
  std::vector<int32_t> fill((size_t)n_out, 0);
  std::vector<int32_t>& mptr = row_count;  // uploaded as the per-row partial count

  // 4. workspace image: [item records | per-row partial counts] is uploaded, then the
  // partials.  Records are written straight into the host image (chunk slots past a
  // record's count are never read, so they are not cleared)
  const int D = C.head_dim;
  size_t off = 0;
  pc.off_items = off; off = align256(off + items.size() * kRecInts * sizeof(int32_t));
  pc.off_mptr = off; off = align256(off + mptr.size() * sizeof(int32_t));
  const size_t plan_bytes = off;
  pc.off_plse = off; off = align256(off + (size_t)n_part_slots * sizeof(float));
  pc.off_po = off; off = align256(off + (size_t)n_part_slots * D * sizeof(float));
  pc.max_parts = max_parts;
  pc.ws_need = std::max<size_t>(off, 256);
  pc.blob.resize(plan_bytes);
  int32_t* recs = reinterpret_cast<int32_t*>(pc.blob.data() + pc.off_items);
  for (size_t i = 0; i < items.size(); ++i) {
    const Item& it = items[i];
    int32_t* rec = recs + i * kRecInts;
    rec[0] = it.n_chunks;
    rec[1] = it.kv_head;
    rec[2] = it.rows;
    rec[3] = 0;
    for (int32_t r = 0; r < it.rows; ++r) {
      const int32_t o = orow_of(it, r);
      rec[kRecRow + r] = o;
      rec[kRecSlot + r] = o * max_parts + fill[(size_t)o]++;
    }
    for (int32_t r = it.rows; r < kMaxRows; ++r) {
      rec[kRecRow + r] = -1;
      rec[kRecSlot + r] = 0;
    }
    n_part += it.rows;
    static_assert(sizeof(Chunk) == 2 * sizeof(int32_t), "chunk records are (page, lohi) int pairs");
    std::memcpy(rec + kRecChunk, it.seg->chunks.data() + it.chunk_begin, (size_t)it.n_chunks * sizeof(Chunk));
  }
  put(pc.blob, pc.off_mptr, mptr);
  // what a later patch needs (decode plans): each query's tail page chunk and the last
  // item of its private segment, per KV head
  pc.patchable = !len_cap;
  pc.pending.clear();
  if (pc.patchable) {
    const int32_t H = C.n_kv_heads;
    pc.q_seq.assign(seqs, seqs + n);
    for (int32_t i = 0; i < n; ++i)
      for (int32_t j = 0; j < i; ++j)
        if (seqs[j] == seqs[i]) pc.q_seq[i] = pc.q_seq[j] = -1;
    pc.q_own_n.assign((size_t)n, 0);
    pc.q_tail_page.assign((size_t)n, -1);
    for (int32_t i = 0; i < n; ++i) {
      const Seq* S = fa_seq(P, seqs[i]);
      pc.q_own_n[i] = (int32_t)S->n;
      if (S->n % PS) pc.q_tail_page[i] = S->pages[(size_t)(S->n / PS)];
    }
    pc.tail_rec.assign((size_t)n * H, -1);
    pc.tail_slot.assign((size_t)n * H, -1);
    pc.last_rec.assign((size_t)n * H, -1);
    std::vector<int32_t> last_begin((size_t)n * H, -1);
    for (size_t r = 0; r < items.size(); ++r) {
      const Item& it = items[r];
      if (it.seg->readers.size() != 1) continue;
      const int32_t q = it.seg->readers[0];
      const size_t at = (size_t)q * H + it.kv_head;
      if (it.chunk_begin > last_begin[at]) {
        last_begin[at] = it.chunk_begin;
        pc.last_rec[at] = (int32_t)r;
      }
      if (pc.q_tail_page[q] >= 0)
        for (int32_t c = 0; c < it.n_chunks; ++c)
          if (it.seg->chunks[it.chunk_begin + c].page == pc.q_tail_page[q]) {
            pc.tail_rec[at] = (int32_t)r;
            pc.tail_slot[at] = c;
          }
    }
  }
  pc.n_items = (int32_t)items.size();
  pc.n_out_rows = n_out;
  const size_t es = C.dtype == KV_F32 ? 4 : 2;
  pc.stats[0] = (int64_t)segs.size();
  pc.stats[1] = (int64_t)items.size();
  pc.stats[2] = n_chunks_total;
  pc.stats[3] = n_part;
  pc.stats[4] = unique_tokens * C.n_kv_heads * 2 * D * (int64_t)es;
  pc.stats[5] = n_out;
  int64_t longest = 0;
  for (const Item& it : items) longest = std::max<int64_t>(longest, it.n_chunks);
  pc.stats[6] = longest;
  pc.stats[7] = 0;
  pc.valid = true;
  pc.serial = ++g_plan_serial;
  pc.causal_n = len_cap ? -1 : 0;
  pc.version = P->version;
  pc.seqs.assign(seqs, seqs + n);
  pc.n_q_heads = hq;
  pc.ws = nullptr;  // not uploaded yet
  if (!len_cap) P->journal.reset(P->version);
  return KV_OK;
}

extern "C" {

int fork_attn_workspace_size(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t hq, size_t* bytes) {
  if (!P || !bytes) FAIL(P, KV_ERR_INVALID, "null argument");
  int st = build_plan(P, seqs, n, hq);
  if (st) return st;
  *bytes = P->plan.ws_need;
  return KV_OK;
}

int fork_attn_plan_stats(kv_pool_t* P, int64_t* out, int32_t n) {
  if (!P || !out || n < 0) FAIL(P, KV_ERR_INVALID, "null argument");
  if (!P->plan.valid) FAIL(P, KV_ERR_INVALID, "no plan yet");
  for (int32_t i = 0; i < n && i < 8; ++i) out[i] = P->plan.stats[i];
  return KV_OK;
}

// Plan (cached) and upload it into the workspace if needed.
static int prepare(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t hq, void* ws, size_t ws_bytes,
                   hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  if (!P->device) FAIL(P, KV_ERR_INVALID, "metadata-only pool has no KV data");
  if (!ws) FAIL(P, KV_ERR_INVALID, "null workspace");
  int st = build_plan(P, seqs, n, hq);
  if (st) return st;
  DecodePlanCache& pc = P->plan;
  if (ws_bytes < pc.ws_need) FAIL(P, KV_ERR_WORKSPACE, "decode workspace too small");
  hipError_t e = hipSuccess;
  if (pc.ws == ws && !pc.pending.empty()) {
    // the workspace holds this plan before its latest patches: send only the changed ints
    // (the last value of each), scattered by a small kernel, through the pool's plan area
    std::unordered_map<int32_t, size_t> last;
    for (size_t k = 0; k < pc.pending.size(); k += 2) last[pc.pending[k]] = k;
    std::vector<int32_t> list;
    list.reserve(last.size() * 2);
    for (size_t k = 0; k < pc.pending.size(); k += 2)
      if (last[pc.pending[k]] == k) {
        list.push_back(pc.pending[k]);
        list.push_back(pc.pending[k + 1]);
      }
    pc.pending.clear();
    const size_t area = fa_pool_ws_need(&P->cfg) - fa_ws_plan_offset(&P->cfg);
    if (list.size() * sizeof(int32_t) <= area) {
      char* at = P->ws + fa_ws_plan_offset(&P->cfg);
      e = fa_upload(P, at, list.data(), list.size() * sizeof(int32_t), s);
      if (e == hipSuccess)
        e = launch_plan_patch(ws, reinterpret_cast<const int32_t*>(at), (int)(list.size() / 2), s);
      if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("plan patch: ") + hipGetErrorString(e));
    } else {
      pc.ws = nullptr;  // too many changes for the plan area: upload the whole plan
    }
  }
  if (pc.ws != ws) {
    e = fa_upload(P, ws, pc.blob.data(), pc.blob.size(), s);
    if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("plan upload: ") + hipGetErrorString(e));
    pc.ws = ws;
    pc.pending.clear();
  }
  return KV_OK;
}

// The two launches of a planned decode whose plan sits in the device buffer w.
static hipError_t launch_partials(kv_pool_t* P, const void* q, float sm_scale, char* w, hipStream_t s) {
  const DecodePlanCache& pc = P->plan;
  DecodeParams dp;
  dp.q = q;
  dp.k_pages = P->k;
  dp.v_pages = P->v;
  dp.items = reinterpret_cast<const int32_t*>(w + pc.off_items);
  dp.cut_hi = nullptr;
  dp.cached = 0;
  dp.part_lse2 = reinterpret_cast<float*>(w + pc.off_plse);
  dp.part_o = reinterpret_cast<float*>(w + pc.off_po);
  dp.n_items = pc.n_items;
  dp.n_pages = P->cfg.n_pages;
  dp.scale_log2 = sm_scale * 1.4426950408889634f;
  return launch_decode(P->cfg.dtype, P->cfg.head_dim, dp, s);
}

static hipError_t launch_merge_of(kv_pool_t* P, void* out, float* lse, char* w, hipStream_t s) {
  const DecodePlanCache& pc = P->plan;
  MergeParams mp;
  mp.count = reinterpret_cast<const int32_t*>(w + pc.off_mptr);
  mp.max_parts = pc.max_parts;
  mp.part_lse2 = reinterpret_cast<const float*>(w + pc.off_plse);
  mp.part_o = reinterpret_cast<const float*>(w + pc.off_po);
  mp.out = out;
  mp.lse = lse;
  mp.n_rows = pc.n_out_rows;
  return launch_merge(P->cfg.dtype, P->cfg.head_dim, mp, s);
}

int fork_attn_partials(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t hq, const void* q, float sm_scale,
                       void* ws, size_t ws_bytes, hipStream_t s) {
  if (P && n == 0) return KV_OK;
  if (!q) FAIL(P, KV_ERR_INVALID, "null q");
  int st = prepare(P, seqs, n, hq, ws, ws_bytes, s);
  if (st) return st;
  hipError_t e = launch_partials(P, q, sm_scale, (char*)ws, s);
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("decode launch: ") + hipGetErrorString(e));
  return KV_OK;
}

int fork_attn_merge(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t hq, void* out, float* lse, void* ws,
                    size_t ws_bytes, hipStream_t s) {
  if (P && n == 0) return KV_OK;
  if (!out) FAIL(P, KV_ERR_INVALID, "null out");
  int st = prepare(P, seqs, n, hq, ws, ws_bytes, s);
  if (st) return st;
  hipError_t e = launch_merge_of(P, out, lse, (char*)ws, s);
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
  return KV_OK;
}

}  // extern "C"

// fork_attn_decode into a library-held device buffer `w` of cap bytes that every call on
// the device shares: *held names the plan the buffer holds (0 = none); the plan is
// uploaded again unless it is this pool's current one.  The upload copies from pageable
// host memory (no staging buffer to allocate).  Used by the no-allocation entry point.
int fa_decode_shared_buffer(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t hq, const void* q, void* out,
                            float* lse, float sm_scale, char* w, size_t cap, uint64_t* held, hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  if (n == 0) return KV_OK;
  if (!P->device) FAIL(P, KV_ERR_INVALID, "metadata-only pool has no KV data");
  if (!q || !out) FAIL(P, KV_ERR_INVALID, "null device pointer");
  int st = build_plan(P, seqs, n, hq);
  if (st) return st;
  DecodePlanCache& pc = P->plan;
  if (pc.ws_need > cap)
    FAIL(P, KV_ERR_WORKSPACE, "decode needs " + std::to_string(pc.ws_need) + " bytes of workspace, more than the " +
                                  std::to_string(cap) + "-byte static buffer");
  hipError_t e = hipSuccess;
  if (*held != pc.serial) {
    *held = 0;
    e = hipMemcpyAsync(w, pc.blob.data(), pc.blob.size(), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) *held = pc.serial;
  }
  if (e == hipSuccess) e = launch_partials(P, q, sm_scale, w, s);
  if (e == hipSuccess) e = launch_merge_of(P, out, lse, w, s);
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("decode (static buffer): ") + hipGetErrorString(e));
  return KV_OK;
}

extern "C" {

int fork_attn_decode(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t hq, const void* q, void* out,
                     float* lse, float sm_scale, void* ws, size_t ws_bytes, hipStream_t s) {
  if (P && n == 0) return KV_OK;
  if (!q || !out) FAIL(P, KV_ERR_INVALID, "null device pointer");
  int st = fork_attn_partials(P, seqs, n, hq, q, sm_scale, ws, ws_bytes, s);
  if (st) return st;
  return fork_attn_merge(P, seqs, n, hq, out, lse, ws, ws_bytes, s);
}

// ------------------------------------------------------------------ steady-state decode window
// Agentrix (the ForkAttention section) and AgentKV run fork attention inside a captured
// decode loop; a window reserves the slots of the next n_steps tokens of every sequence
// (tail copy-on-write and new pages, in exactly the order n_steps rounds of one append
// per sequence would take them) and plans the decode once over the contexts through the
// window's last token; a chunk of a reserved page carries a cut id, and each step has a
// small table giving every id the page's slot end after that step.  A step is three
// launches with fixed arguments: the new K / V into their reserved slots, the split-K
// partials (every item shared by all steps, reserved chunks cut by the step's table),
// the merge.

int kv_window_plan(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t hq, int32_t n_steps, size_t* ws_need) {
  if (!P || !ws_need) FAIL(P, KV_ERR_INVALID, "null argument");
  if (n < 1 || !seqs || n_steps < 1) FAIL(P, KV_ERR_INVALID, "bad window shape");
  const int32_t PS = P->cfg.page_size;
  for (int32_t i = 0; i < n; ++i) {
    if (!fa_seq(P, seqs[i])) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence in the window");
    for (int32_t j = 0; j < i; ++j)
      if (seqs[j] == seqs[i]) FAIL(P, KV_ERR_INVALID, "a sequence appears twice in the window");
  }
  if (hq < P->cfg.n_kv_heads || hq % P->cfg.n_kv_heads) FAIL(P, KV_ERR_INVALID, "n_q_heads must be a multiple of n_kv_heads");
  // capacity: copies of shared partial tails + pages the new tokens start
  int64_t need = 0;
  std::vector<int64_t> base((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    Seq* S = fa_seq(P, seqs[i]);
    base[i] = S->n;
    const int64_t have = (int64_t)S->pages.size();
    if (S->n % PS && P->rc[S->pages[(size_t)(S->n / PS)]] > 1) ++need;
    need += std::max<int64_t>(0, (S->n + n_steps + PS - 1) / PS - have);
  }
  if (need > P->free.count()) FAIL(P, KV_ERR_OOM, "not enough free pages for the window");
  DecodeWindow& W = P->window;
  std::vector<char> keep = std::move(W.blob);  // reuse the host buffer of the previous window
  W = DecodeWindow();
  W.blob = std::move(keep);
  // 1. reservation, round by round (the page order of n_steps rounds of single appends)
  std::vector<PageWrite> cow;
  std::vector<std::vector<PageWrite>> writes((size_t)n_steps, std::vector<PageWrite>((size_t)n));
  for (int32_t st = 0; st < n_steps; ++st)
    for (int32_t i = 0; i < n; ++i) {
      Seq* S = fa_seq(P, seqs[i]);
      const int64_t L = S->n / PS, slot = S->n % PS;
      if (L < (int64_t)S->pages.size()) {
        if (P->rc[S->pages[(size_t)L]] > 1) {  // shared partial tail: copy before the first write
          std::vector<int32_t> id;
          P->free.peek_lowest(1, id);
          const int32_t old = S->pages[(size_t)L];
          fa_take_page(P, id[0]);
          S->pages[(size_t)L] = id[0];
          fa_unref_page(P, old);
          cow.push_back({id[0], old, 0, 0, 0});
        }
      } else {
        std::vector<int32_t> id;
        P->free.peek_lowest(1, id);
        fa_take_page(P, id[0]);
        S->pages.push_back(id[0]);
      }
      writes[st][i] = {S->pages[(size_t)L], -1, (int32_t)slot, (int32_t)slot + 1, (int64_t)i};  // row i of k / v
      fa_pos_append(S->pos, S->next_pos, 1);
      S->next_pos += 1;
      S->n += 1;
    }
  fa_changed(P, ChangeJournal::kOther, -1, 0, 0);
  // 2. one plan over the contexts through the window's last token; step s is that plan
  // with each reserved page's slot range cut at the sequence's length after step s (the
  // same items, partial slots and merge counts; a chunk past the cut is empty)
  std::vector<int64_t> cap((size_t)n);
  for (int32_t i = 0; i < n; ++i) cap[i] = base[i] + n_steps;
  if (int e = build_plan(P, seqs, n, hq, cap.data())) {
    P->plan.valid = false;
    W = DecodeWindow();
    return e;  // the page table keeps the reservation; the window is unusable
  }
  DecodePlanCache& pc = P->plan;
  // chunks of reserved pages carry a cut id (bits 16..31 of their slot range, id + 1):
  // one per (query, reserved logical page), shared by the KV heads; step st's table gives
  // each id the slot end of its page after st + 1 window tokens
  std::unordered_map<int32_t, int32_t> cut_of;  // reserved page -> cut id
  std::vector<std::pair<int32_t, int64_t>> cuts;  // cut id -> (query, first token of the page)
  for (int32_t i = 0; i < n; ++i) {
    Seq* S = fa_seq(P, seqs[i]);
    for (int64_t L = base[i] / PS; L < (int64_t)S->pages.size(); ++L) {
      cut_of[S->pages[(size_t)L]] = (int32_t)cuts.size();
      cuts.push_back({i, L * PS});
    }
  }
  if (cuts.size() >= ((size_t)1 << 15) - 1) {
    P->plan.valid = false;
    W = DecodeWindow();
    FAIL(P, KV_ERR_UNSUPPORTED, "too many reserved pages in one window");
  }
  // items that read a reserved page go last (measured: the window's steps are slower with
  // them first, in plain heaviest-first order)
  int32_t* recs0 = reinterpret_cast<int32_t*>(pc.blob.data() + pc.off_items);
  std::vector<int32_t> plain, with_cut;
  for (int32_t it = 0; it < pc.n_items; ++it) {
    int32_t* rec = recs0 + (size_t)it * kRecInts;
    bool any = false;
    for (int32_t c = 0; c < rec[0]; ++c) {
      const auto f = cut_of.find(rec[kRecChunk + 2 * c]);
      if (f != cut_of.end()) {
        rec[kRecChunk + 2 * c + 1] |= (f->second + 1) << 16;
        any = true;
      }
    }
    (any ? with_cut : plain).push_back(it);
  }
  if (!with_cut.empty()) {
    std::vector<int32_t> moved((size_t)pc.n_items * kRecInts);
    size_t at = 0;
    for (const std::vector<int32_t>* list : {&plain, &with_cut})
      for (int32_t it : *list) std::memcpy(moved.data() + kRecInts * at++, recs0 + (size_t)it * kRecInts, kRecInts * sizeof(int32_t));
    std::memcpy(recs0, moved.data(), moved.size() * sizeof(int32_t));
  }
  size_t off = 0;
  W.off_cow = off;
  off = align256(off + cow.size() * sizeof(PageWrite));
  const size_t plan_at = off;  // the plan image (items, merge counts), shared by every step
  off = align256(off + pc.blob.size());
  W.steps.resize((size_t)n_steps);
  for (int32_t st = 0; st < n_steps; ++st) {
    DecodeWindow::Step& ws = W.steps[st];
    ws.off_items = plan_at + pc.off_items;
    ws.off_mptr = plan_at + pc.off_mptr;
    ws.n_items = pc.n_items;
    ws.n_out_rows = pc.n_out_rows;
    ws.max_parts = pc.max_parts;
    ws.off_cut = off;
    off = align256(off + std::max<size_t>(1, cuts.size()) * sizeof(int32_t));
    ws.off_writes = off;
    off = align256(off + (size_t)n * sizeof(PageWrite));
  }
  const int64_t part_slots = (int64_t)pc.n_out_rows * pc.max_parts;
  W.off_plse = off;
  off = align256(off + (size_t)part_slots * sizeof(float));
  W.off_po = off;
  off = align256(off + (size_t)part_slots * P->cfg.head_dim * sizeof(float));
  W.ws_need = std::max<size_t>(off, 256);
  W.blob.resize(W.off_plse);  // alignment gaps are never read
  if (!cow.empty()) std::memcpy(W.blob.data() + W.off_cow, cow.data(), cow.size() * sizeof(PageWrite));
  std::memcpy(W.blob.data() + plan_at, pc.blob.data(), pc.blob.size());
  for (int32_t st = 0; st < n_steps; ++st) {
    const DecodeWindow::Step& ws = W.steps[st];
    int32_t* cut = reinterpret_cast<int32_t*>(W.blob.data() + ws.off_cut);
    cut[0] = 0;
    for (size_t c = 0; c < cuts.size(); ++c)
      cut[c] = (int32_t)std::max<int64_t>(0, std::min<int64_t>(PS, base[cuts[c].first] + st + 1 - cuts[c].second));
    std::memcpy(W.blob.data() + ws.off_writes, writes[st].data(), (size_t)n * sizeof(PageWrite));
  }
  P->plan.valid = false;  // the cached plan now describes the window's last step only
  W.seqs.assign(seqs, seqs + n);
  W.n_q_heads = hq;
  W.n_steps = n_steps;
  W.n_cow = (int32_t)cow.size();
  W.version = P->version;
  W.valid = true;
  *ws_need = W.ws_need;
  return KV_OK;
}

int kv_window_upload(kv_pool_t* P, void* workspace, size_t ws_bytes, hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  if (!P->device) FAIL(P, KV_ERR_INVALID, "metadata-only pool has no KV data");
  DecodeWindow& W = P->window;
  if (!W.valid || W.version != P->version) FAIL(P, KV_ERR_INVALID, "no window planned since the last page-table change");
  if (!workspace) FAIL(P, KV_ERR_INVALID, "null workspace");
  if (ws_bytes < W.ws_need) FAIL(P, KV_ERR_WORKSPACE, "window workspace too small");
  char* w = static_cast<char*>(workspace);
  hipError_t e = fa_upload(P, w, W.blob.data(), W.blob.size(), s);
  if (e == hipSuccess && W.n_cow > 0)
    e = launch_page_write(P->cfg.dtype, P->cfg.head_dim, P->cfg.n_kv_heads, P->cfg.n_pages, P->k, P->v, P->k, P->v,
                          reinterpret_cast<const PageWrite*>(w + W.off_cow), W.n_cow, s);
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("window upload: ") + hipGetErrorString(e));
  W.ws = workspace;
  return KV_OK;
}

int kv_window_step(kv_pool_t* P, int32_t step, const void* k, const void* v, const void* q, void* out, float* lse,
                   float sm_scale, hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  DecodeWindow& W = P->window;
  if (!W.valid || W.version != P->version || !W.ws)
    FAIL(P, KV_ERR_INVALID, "no uploaded window since the last page-table change");
  if (step < 0 || step >= W.n_steps) FAIL(P, KV_ERR_INVALID, "step outside the window");
  if (!k || !v || !q || !out) FAIL(P, KV_ERR_INVALID, "null device pointer");
  const DecodeWindow::Step& ws = W.steps[step];
  char* w = static_cast<char*>(W.ws);
  hipError_t e = launch_page_write(P->cfg.dtype, P->cfg.head_dim, P->cfg.n_kv_heads, P->cfg.n_pages, P->k, P->v, k,
                                   v, reinterpret_cast<const PageWrite*>(w + ws.off_writes), (int)W.seqs.size(), s);
  if (e == hipSuccess) {
    DecodeParams dp;
    dp.q = q;
    dp.k_pages = P->k;
    dp.v_pages = P->v;
    dp.items = reinterpret_cast<const int32_t*>(w + ws.off_items);
    dp.cut_hi = reinterpret_cast<const int32_t*>(w + ws.off_cut);
    dp.cached = 0;
    dp.part_lse2 = reinterpret_cast<float*>(w + W.off_plse);
    dp.part_o = reinterpret_cast<float*>(w + W.off_po);
    dp.n_items = ws.n_items;
    dp.n_pages = P->cfg.n_pages;
    dp.scale_log2 = sm_scale * 1.4426950408889634f;
    e = launch_decode(P->cfg.dtype, P->cfg.head_dim, dp, s);
  }
  if (e == hipSuccess) {
    MergeParams mp;
    mp.count = reinterpret_cast<const int32_t*>(w + ws.off_mptr);
    mp.max_parts = ws.max_parts;
    mp.part_lse2 = reinterpret_cast<const float*>(w + W.off_plse);
    mp.part_o = reinterpret_cast<const float*>(w + W.off_po);
    mp.out = out;
    mp.lse = lse;
    mp.n_rows = ws.n_out_rows;
    e = launch_merge(P->cfg.dtype, P->cfg.head_dim, mp, s);
  }
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("window step: ") + hipGetErrorString(e));
  return KV_OK;
}

// ------------------------------------------------------------------ causal attention of a sequence's last tokens
// AKV page, section "AKV 如何工作": segmented batch attention restores an evicted state
// with one prefill, each segment keeping its own positions: the caller appends the segments' K / V (kv_append with
// their positions) and then attends the last n tokens, token j over the context through
// itself (every earlier own token, then the mounts), as n rows of one split-K decode.

static int causal_plan(kv_pool_t* P, kv_seq_t seq, int64_t n, int32_t hq) {
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (n < 1 || n > S->n) FAIL(P, KV_ERR_INVALID, "the attended tokens must be the sequence's last n (n >= 1)");
  if (n * hq > (int64_t)1 << 30) FAIL(P, KV_ERR_UNSUPPORTED, "too many query rows");
  DecodePlanCache& pc = P->plan;
  if (pc.valid && pc.causal_n == n && pc.version == P->version && pc.n_q_heads == hq && !pc.seqs.empty() &&
      pc.seqs[0] == seq)
    return KV_OK;  // planned for the same sequence state
  std::vector<kv_seq_t> seqs((size_t)n, seq);
  std::vector<int64_t> cap((size_t)n);
  for (int64_t j = 0; j < n; ++j) cap[(size_t)j] = S->n - n + j + 1;
  const int st = build_plan(P, seqs.data(), (int32_t)n, hq, cap.data());
  if (st == KV_OK) pc.causal_n = n;
  return st;
}

}  // extern "C"

// bf16 pools with d = 128 restore through the tiled prefill; other pools through rows of
// the split-K decode.
static bool restore_by_prefill(const kv_pool* P) { return P->cfg.dtype == KV_BF16 && P->cfg.head_dim == 128; }

// Plan of the tiled-prefill restore (cached per sequence state, n and head count).
static int restore_plan(kv_pool_t* P, kv_seq_t seq, int64_t n, int32_t hq) {
  const kv_pool_config& C = P->cfg;
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (n < 1 || n > S->n) FAIL(P, KV_ERR_INVALID, "the attended tokens must be the sequence's last n (n >= 1)");
  if (hq < C.n_kv_heads || hq % C.n_kv_heads) FAIL(P, KV_ERR_INVALID, "n_q_heads must be a multiple of n_kv_heads");
  RestorePlan& R = P->restore;
  if (R.valid && R.version == P->version && R.seq == seq && R.n == n && R.hq == hq) return KV_OK;
  const int32_t PS = C.page_size, H = C.n_kv_heads;
  const int64_t N = S->n;
  int64_t T = N;
  for (const Mount& m : S->mounts) T += m.n;
  if (T > INT32_MAX / 2 || n * hq > ((int64_t)1 << 30)) FAIL(P, KV_ERR_UNSUPPORTED, "context too long");
  // visible keys: own tokens, then each mount's range
  std::vector<int32_t> locs;
  locs.reserve((size_t)T);
  for (int64_t t = 0; t < N; ++t) locs.push_back(S->pages[(size_t)(t / PS)] * 16 + (int32_t)(t % PS));
  for (const Mount& m : S->mounts)
    for (int64_t j = 0; j < m.n; ++j) {
      const int64_t tok = m.off + j;
      locs.push_back(m.pages[(size_t)(tok / PS)] * 16 + (int32_t)(tok % PS));
    }
  // rows: query block qb (restored tokens 64 qb ..) x key piece; the visible key blocks of
  // a query block are the own blocks through its last query's and every block from the
  // first mounted key on; a block is masked inside when some own key in it can follow
  // some query of the block
  const int64_t q_off = N - n;
  const int32_t nb = (int32_t)((T + 63) / 64), nqb = (int32_t)((n + 63) / 64);
  const int32_t G = hq / H, n_hg = (G + 3) / 4;
  std::vector<std::vector<int32_t>> cols((size_t)nqb);
  size_t shortest = SIZE_MAX;
  for (int32_t qb = 0; qb < nqb; ++qb) {
    const int64_t i_min = q_off + 64 * qb, i_max = q_off + std::min<int64_t>(64 * qb + 63, n - 1);
    for (int32_t kb = 0; kb < nb; ++kb) {
      const int64_t k0 = 64 * (int64_t)kb;
      if (k0 > i_max && k0 + 63 < N) continue;  // own keys after every query of the block
      const bool diag = k0 + 63 > i_min && k0 < N;
      cols[qb].push_back(kb | (diag ? (int32_t)0x80000000u : 0));
    }
    shortest = std::min(shortest, cols[qb].size());
  }
  // pieces: one workgroup per compute unit (the kernel's LDS ring holds one per unit),
  // so the launch is one wave of workgroups of nearly equal length
  const int64_t base_rows = (int64_t)nqb * H * n_hg;
  int32_t n_split = (int32_t)std::min<int64_t>(32, std::max<int64_t>(1, (P->n_cu + base_rows - 1) / base_rows));
  n_split = (int32_t)std::max<size_t>(1, std::min<size_t>((size_t)n_split, shortest));
  const int32_t n_rows = nqb * n_split;
  std::vector<int32_t> row_ptr((size_t)n_rows + 1, 0), ent;
  for (int32_t qb = 0; qb < nqb; ++qb) {
    const size_t L = cols[qb].size();
    for (int32_t pc = 0; pc < n_split; ++pc) {
      const size_t a = L * pc / n_split, b = L * (pc + 1) / n_split;
      ent.insert(ent.end(), cols[qb].begin() + a, cols[qb].begin() + b);
      row_ptr[(size_t)qb * n_split + pc + 1] = (int32_t)ent.size();
    }
  }
  std::vector<int32_t> order((size_t)n_rows);
  for (int32_t r = 0; r < n_rows; ++r) order[r] = r;
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return row_ptr[a + 1] - row_ptr[a] > row_ptr[b + 1] - row_ptr[b];
  });
  std::vector<int32_t> count((size_t)(n * hq), n_split);
  // K is read straight from the pool when the visible keys fill whole pages in order (own
  // tokens always do; mounts when they start on a page boundary) and one KV head's blocks
  // fit a 2 GiB buffer range; else it is relaid into images like V.  gpages[g] = the page
  // of keys 16 g .. 16 g + 15 (4 per 64-key block; padding and a partial last page point
  // at valid pages, their keys are masked)
  std::vector<int32_t> gpages((size_t)nb * 4, 0);
  bool aligned = PS == 16;
  for (int64_t t = 0; t < T && aligned; ++t) {
    const int32_t loc = locs[(size_t)t];
    if (t % 16 == 0) gpages[(size_t)(t / 16)] = loc >> 4;
    aligned = loc == gpages[(size_t)(t / 16)] * 16 + (int32_t)(t % 16);
  }
  for (size_t g = (size_t)((T + 15) / 16); g < gpages.size() && g > 0; ++g) gpages[g] = gpages[g - 1];
  R.kgather = aligned && (int64_t)C.n_pages * 16 * C.head_dim * 2 <= INT32_MAX;
  size_t off = 0;
  R.off_locs = off; off = align256(off + locs.size() * 4);
  R.off_rowptr = off; off = align256(off + row_ptr.size() * 4);
  R.off_ent = off; off = align256(off + std::max<size_t>(1, ent.size()) * 4);
  R.off_order = off; off = align256(off + order.size() * 4);
  R.off_count = off; off = align256(off + count.size() * 4);
  R.off_gpages = off; off = align256(off + gpages.size() * 4);
  const size_t blob_bytes = off;
  R.off_kimg = off; off += R.kgather ? 0 : (size_t)H * nb * kRestoreImgBytes;
  R.off_vimg = off; off += (size_t)H * nb * kRestoreImgBytes;
  off = align256(off);
  R.off_plse = off; off = align256(off + (size_t)n * hq * n_split * 4);
  R.off_po = off; off = align256(off + (size_t)n * hq * n_split * C.head_dim * 4);
  R.ws_need = off;
  R.blob.assign(blob_bytes, 0);
  std::memcpy(R.blob.data() + R.off_locs, locs.data(), locs.size() * 4);
  std::memcpy(R.blob.data() + R.off_rowptr, row_ptr.data(), row_ptr.size() * 4);
  if (!ent.empty()) std::memcpy(R.blob.data() + R.off_ent, ent.data(), ent.size() * 4);
  std::memcpy(R.blob.data() + R.off_order, order.data(), order.size() * 4);
  std::memcpy(R.blob.data() + R.off_count, count.data(), count.size() * 4);
  std::memcpy(R.blob.data() + R.off_gpages, gpages.data(), gpages.size() * 4);
  R.T = (int32_t)T;
  R.n_own = (int32_t)N;
  R.n_rows = n_rows;
  R.n_split = n_split;
  R.valid = true;
  R.version = P->version;
  R.seq = seq;
  R.n = n;
  R.hq = hq;
  R.ws = nullptr;
  return KV_OK;
}

extern "C" {

int kv_causal_attend_workspace_size(kv_pool_t* P, kv_seq_t seq, int64_t n, int32_t n_q_heads, size_t* bytes) {
  if (!P || !bytes) FAIL(P, KV_ERR_INVALID, "null argument");
  if (restore_by_prefill(P)) {
    if (int st = restore_plan(P, seq, n, n_q_heads)) return st;
    *bytes = P->restore.ws_need;
    return KV_OK;
  }
  if (int st = causal_plan(P, seq, n, n_q_heads)) return st;
  *bytes = P->plan.ws_need;
  return KV_OK;
}

int kv_causal_attend(kv_pool_t* P, kv_seq_t seq, int64_t n, int32_t n_q_heads, const void* q, void* out, float* lse,
                     float sm_scale, void* workspace, size_t ws_bytes, hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  if (!P->device) FAIL(P, KV_ERR_INVALID, "metadata-only pool has no KV data");
  if (!q || !out || !workspace) FAIL(P, KV_ERR_INVALID, "null device pointer");
  if (restore_by_prefill(P)) {
    if (!(sm_scale > 0.f)) FAIL(P, KV_ERR_INVALID, "softmax scale must be positive");
    if (int st = restore_plan(P, seq, n, n_q_heads)) return st;
    RestorePlan& R = P->restore;
    if (ws_bytes < R.ws_need) FAIL(P, KV_ERR_WORKSPACE, "causal attention workspace too small");
    char* w = static_cast<char*>(workspace);
    hipError_t e = hipSuccess;
    if (R.ws != workspace) {
      e = fa_upload(P, w, R.blob.data(), R.blob.size(), s);
      if (e == hipSuccess) R.ws = workspace;
    }
    if (e == hipSuccess) {
      RestoreLaunch rl;
      rl.q = q;
      rl.k_pages = P->k;
      rl.v_pages = P->v;
      rl.pool_pages = P->cfg.n_pages;
      rl.locs = reinterpret_cast<const int32_t*>(w + R.off_locs);
      rl.row_ptr = reinterpret_cast<const int32_t*>(w + R.off_rowptr);
      rl.ent = reinterpret_cast<const int32_t*>(w + R.off_ent);
      rl.order = reinterpret_cast<const int32_t*>(w + R.off_order);
      rl.kimg = w + R.off_kimg;
      rl.vimg = w + R.off_vimg;
      rl.part_lse2 = reinterpret_cast<float*>(w + R.off_plse);
      rl.part_o = reinterpret_cast<float*>(w + R.off_po);
      rl.T = R.T;
      rl.n_own = R.n_own;
      rl.q_off = (int32_t)(R.n_own - n);
      rl.nq = (int32_t)n;
      rl.hq = n_q_heads;
      rl.hkv = P->cfg.n_kv_heads;
      rl.n_rows = R.n_rows;
      rl.n_split = R.n_split;
      rl.sm_scale = sm_scale;
      rl.kgather = R.kgather;
      rl.gpages = reinterpret_cast<const int32_t*>(w + R.off_gpages);
      e = fa_launch_restore(rl, s);
    }
    if (e == hipSuccess) {
      MergeParams mp;
      mp.count = reinterpret_cast<const int32_t*>(w + R.off_count);
      mp.max_parts = R.n_split;
      mp.part_lse2 = reinterpret_cast<const float*>(w + R.off_plse);
      mp.part_o = reinterpret_cast<const float*>(w + R.off_po);
      mp.out = out;
      mp.lse = lse;
      mp.n_rows = (int32_t)(n * n_q_heads);
      e = launch_merge_few(P->cfg.dtype, P->cfg.head_dim, mp, s);
    }
    if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("causal attention: ") + hipGetErrorString(e));
    return KV_OK;
  }
  if (int st = causal_plan(P, seq, n, n_q_heads)) return st;
  DecodePlanCache& pc = P->plan;  // cached for the same sequence state (never a decode plan)
  if (ws_bytes < pc.ws_need) FAIL(P, KV_ERR_WORKSPACE, "causal attention workspace too small");
  char* w = static_cast<char*>(workspace);
  hipError_t e = hipSuccess;
  if (pc.ws != workspace) {
    e = fa_upload(P, w, pc.blob.data(), pc.blob.size(), s);
    if (e == hipSuccess) pc.ws = workspace;
  }
  if (e == hipSuccess) {
    DecodeParams dp;
    dp.q = q;
    dp.k_pages = P->k;
    dp.v_pages = P->v;
    dp.items = reinterpret_cast<const int32_t*>(w + pc.off_items);
    dp.cut_hi = nullptr;
    dp.cached = 1;  // every context page is streamed once per group of 64 / G restored tokens
    dp.part_lse2 = reinterpret_cast<float*>(w + pc.off_plse);
    dp.part_o = reinterpret_cast<float*>(w + pc.off_po);
    dp.n_items = pc.n_items;
    dp.n_pages = P->cfg.n_pages;
    dp.scale_log2 = sm_scale * 1.4426950408889634f;
    e = launch_decode(P->cfg.dtype, P->cfg.head_dim, dp, s);
  }
  if (e == hipSuccess) {
    MergeParams mp;
    mp.count = reinterpret_cast<const int32_t*>(w + pc.off_mptr);
    mp.max_parts = pc.max_parts;
    mp.part_lse2 = reinterpret_cast<const float*>(w + pc.off_plse);
    mp.part_o = reinterpret_cast<const float*>(w + pc.off_po);
    mp.out = out;
    mp.lse = lse;
    mp.n_rows = pc.n_out_rows;
    e = launch_merge(P->cfg.dtype, P->cfg.head_dim, mp, s);
  }
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("causal attention: ") + hipGetErrorString(e));
  return KV_OK;
}

}  // extern "C"
