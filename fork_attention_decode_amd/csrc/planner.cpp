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
#include <cstring>
#include <map>
#include <unordered_map>

using namespace fa;

int fa_set_err(kv_pool* P, int code, const std::string& m);
Seq* fa_seq(kv_pool* P, kv_seq_t s);
hipError_t fa_upload(kv_pool* P, void* dst, const void* src, size_t bytes, hipStream_t s);
void fa_take_page(kv_pool* P, int32_t p);
void fa_unref_page(kv_pool* P, int32_t p);
void fa_pos_append(std::vector<PosRun>& v, int64_t p0, int64_t n);
#define FAIL(P, code, msg) return fa_set_err((P), (code), (msg))

namespace {

struct Entry {
  int32_t page;
  int32_t lo, hi;
  int32_t reader;
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
  if (!len_cap && pc.valid && pc.causal_n == 0 && pc.version == P->version && pc.n_q_heads == hq &&
      (int32_t)pc.seqs.size() == n && std::equal(pc.seqs.begin(), pc.seqs.end(), seqs))
    return KV_OK;

  // 1. visible runs
  std::vector<Entry> ent;
  for (int32_t i = 0; i < n; ++i) {
    Seq* S = fa_seq(P, seqs[i]);
    if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence in the query list");
    const int64_t n_own = len_cap ? std::min<int64_t>(len_cap[i], S->n) : S->n;
    for (size_t L = 0; (int64_t)L * PS < n_own; ++L)
      ent.push_back({S->pages[L], 0, (int32_t)std::min<int64_t>(PS, n_own - (int64_t)L * PS), i});
    for (const Mount& m : S->mounts) {
      for (size_t j = 0; j < m.pages.size(); ++j) {
        const int64_t a = std::max<int64_t>(0, m.off - (int64_t)j * PS);
        const int64_t b = std::min<int64_t>(PS, m.off + m.n - (int64_t)j * PS);
        if (a < b) ent.push_back({m.pages[j], (int32_t)a, (int32_t)b, i});
      }
    }
  }
  {  // stable radix sort by page id, 16 bits a pass (readers of a page keep query order);
     // the cost follows the entries, not the pool's page count
    std::vector<Entry> sorted(ent.size());
    std::vector<int32_t> at((size_t)1 << 16 | 1);
    for (int shift = 0; shift < 32 && (shift == 0 || (C.n_pages - 1) >> shift); shift += 16) {
      std::fill(at.begin(), at.end(), 0);
      for (const Entry& e : ent) at[((uint32_t)e.page >> shift & 0xffffu) + 1]++;
      for (size_t d = 1; d < at.size(); ++d) at[d] += at[d - 1];
      for (const Entry& e : ent) sorted[(size_t)at[(uint32_t)e.page >> shift & 0xffffu]++] = e;
      ent.swap(sorted);
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
      uniform = uniform && ent[b].lo == ent[a].lo && ent[b].hi == ent[a].hi;
      ++b;
    }
    if (uniform) {
      key.clear();
      for (size_t e = a; e < b; ++e) key.push_back(ent[e].reader);
      emit(ent[a].page, ent[a].lo, ent[a].hi, key);
    } else {
      std::vector<int32_t> cuts;
      for (size_t e = a; e < b; ++e) {
        cuts.push_back(ent[e].lo);
        cuts.push_back(ent[e].hi);
      }
      std::sort(cuts.begin(), cuts.end());
      cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
      if (cuts.size() <= kMaxCutRanges + 1) {
        // a few slot ranges: one chunk per range, read by every reader that covers it
        for (size_t c = 0; c + 1 < cuts.size(); ++c) {
          key.clear();
          for (size_t e = a; e < b; ++e)
            if (ent[e].lo <= cuts[c] && ent[e].hi >= cuts[c + 1]) key.push_back(ent[e].reader);
          if (!key.empty()) emit(ent[a].page, cuts[c], cuts[c + 1], key);
        }
      } else {
        // many ranges (a causal diagonal page: each of its own tokens reads up to itself):
        // the readers of the most common range share one chunk, every other reader reads
        // its own range alone, instead of one reader set per distinct range
        std::map<std::pair<int32_t, int32_t>, int32_t> freq;
        for (size_t e = a; e < b; ++e) ++freq[{ent[e].lo, ent[e].hi}];
        std::pair<int32_t, int32_t> top = freq.begin()->first;
        for (const auto& f : freq)
          if (f.second > freq[top]) top = f.first;
        key.clear();
        for (size_t e = a; e < b; ++e)
          if (ent[e].lo == top.first && ent[e].hi == top.second) key.push_back(ent[e].reader);
        emit(ent[a].page, top.first, top.second, key);
        for (size_t e = a; e < b; ++e)
          if (!(ent[e].lo == top.first && ent[e].hi == top.second)) {
            key.assign(1, ent[e].reader);
            emit(ent[a].page, ent[e].lo, ent[e].hi, key);
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
    size_t g0;
    std::vector<int32_t> orow;
  };
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
          Item it{c0, c1 - c0, h, rows, &s, g0, {}};
          for (int32_t r = 0; r < rows; ++r) {
            const int32_t orow = s.readers[g0 + r / G] * hq + h * G + r % G;
            it.orow.push_back(orow);
            row_count[orow]++;
          }
          items.push_back(std::move(it));
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
  std::vector<int32_t> recs(items.size() * kRecInts, 0);
  for (size_t i = 0; i < items.size(); ++i) {
    const Item& it = items[i];
    int32_t* rec = recs.data() + i * kRecInts;
    rec[0] = it.n_chunks;
    rec[1] = it.kv_head;
    rec[2] = it.rows;
    for (int32_t r = 0; r < kMaxRows; ++r) {
      rec[kRecRow + r] = r < it.rows ? it.orow[r] : -1;
      rec[kRecSlot + r] = r < it.rows ? it.orow[r] * max_parts + fill[it.orow[r]]++ : 0;
    }
    n_part += it.rows;
    for (int32_t c = 0; c < it.n_chunks; ++c) {
      const Chunk& ch = it.seg->chunks[it.chunk_begin + c];
      rec[kRecChunk + 2 * c] = ch.page;
      rec[kRecChunk + 2 * c + 1] = ch.lohi;
    }
  }
  std::vector<int32_t>& mptr = row_count;  // uploaded as the per-row partial count

  // 4. workspace image: [item records | per-row partial counts] is uploaded, then the
  // partials
  const int D = C.head_dim;
  size_t off = 0;
  pc.off_items = off; off = align256(off + recs.size() * sizeof(int32_t));
  pc.off_mptr = off; off = align256(off + mptr.size() * sizeof(int32_t));
  const size_t plan_bytes = off;
  pc.off_plse = off; off = align256(off + (size_t)n_part_slots * sizeof(float));
  pc.off_po = off; off = align256(off + (size_t)n_part_slots * D * sizeof(float));
  pc.max_parts = max_parts;
  pc.ws_need = std::max<size_t>(off, 256);
  pc.blob.assign(plan_bytes, 0);
  put(pc.blob, pc.off_items, recs);
  put(pc.blob, pc.off_mptr, mptr);
  pc.n_items = (int32_t)items.size();
  pc.n_out_rows = n_out;
  const size_t es = C.dtype == KV_F32 ? 4 : 2;
  pc.stats[0] = (int64_t)segs.size();
  pc.stats[1] = (int64_t)items.size();
  pc.stats[2] = n_chunks_total;
  pc.stats[3] = n_part;
  pc.stats[4] = unique_tokens * C.n_kv_heads * 2 * D * (int64_t)es;
  pc.stats[5] = n_out;
  pc.valid = true;
  pc.causal_n = len_cap ? -1 : 0;
  pc.version = P->version;
  pc.seqs.assign(seqs, seqs + n);
  pc.n_q_heads = hq;
  pc.ws = nullptr;  // not uploaded yet
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
  for (int32_t i = 0; i < n && i < 6; ++i) out[i] = P->plan.stats[i];
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
  if (pc.ws != ws) {
    hipError_t e = fa_upload(P, ws, pc.blob.data(), pc.blob.size(), s);
    if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("plan upload: ") + hipGetErrorString(e));
    pc.ws = ws;
  }
  return KV_OK;
}

int fork_attn_partials(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t hq, const void* q, float sm_scale,
                       void* ws, size_t ws_bytes, hipStream_t s) {
  if (P && n == 0) return KV_OK;
  if (!q) FAIL(P, KV_ERR_INVALID, "null q");
  int st = prepare(P, seqs, n, hq, ws, ws_bytes, s);
  if (st) return st;
  DecodePlanCache& pc = P->plan;
  char* w = (char*)ws;
  DecodeParams dp;
  dp.q = q;
  dp.k_pages = P->k;
  dp.v_pages = P->v;
  dp.items = reinterpret_cast<const int32_t*>(w + pc.off_items);
  dp.tail = dp.items;
  dp.n_head = pc.n_items;
  dp.cached = 0;
  dp.part_lse2 = reinterpret_cast<float*>(w + pc.off_plse);
  dp.part_o = reinterpret_cast<float*>(w + pc.off_po);
  dp.n_items = pc.n_items;
  dp.n_pages = P->cfg.n_pages;
  dp.scale_log2 = sm_scale * 1.4426950408889634f;
  hipError_t e = launch_decode(P->cfg.dtype, P->cfg.head_dim, dp, s);
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("decode launch: ") + hipGetErrorString(e));
  return KV_OK;
}

int fork_attn_merge(kv_pool_t* P, const kv_seq_t* seqs, int32_t n, int32_t hq, void* out, float* lse, void* ws,
                    size_t ws_bytes, hipStream_t s) {
  if (P && n == 0) return KV_OK;
  if (!out) FAIL(P, KV_ERR_INVALID, "null out");
  int st = prepare(P, seqs, n, hq, ws, ws_bytes, s);
  if (st) return st;
  DecodePlanCache& pc = P->plan;
  char* w = (char*)ws;
  MergeParams mp;
  mp.count = reinterpret_cast<const int32_t*>(w + pc.off_mptr);
  mp.max_parts = pc.max_parts;
  mp.part_lse2 = reinterpret_cast<const float*>(w + pc.off_plse);
  mp.part_o = reinterpret_cast<const float*>(w + pc.off_po);
  mp.out = out;
  mp.lse = lse;
  mp.n_rows = pc.n_out_rows;
  hipError_t e = launch_merge(P->cfg.dtype, P->cfg.head_dim, mp, s);
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
  return KV_OK;
}

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
// per sequence would take them) and plans each step's decode once, so a step is three
// launches with fixed arguments: the new K / V into their reserved slots, the split-K
// partials, the merge.

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
  P->version++;
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
  // the chunk records of reserved pages: (record int, query index, logical page)
  std::unordered_map<int32_t, int64_t> owner;  // reserved page -> i * 2^32 + logical page
  for (int32_t i = 0; i < n; ++i) {
    Seq* S = fa_seq(P, seqs[i]);
    for (int64_t L = base[i] / PS; L < (int64_t)S->pages.size(); ++L)
      owner[S->pages[(size_t)L]] = ((int64_t)i << 32) | L;
  }
  // items that read a reserved page form the per-step tail (their slot ranges change
  // with the step); the rest, and the merge counts, are shared by every step
  const int32_t* recs0 = reinterpret_cast<const int32_t*>(pc.blob.data() + pc.off_items);
  std::vector<int32_t> head, tail;
  for (int32_t it = 0; it < pc.n_items; ++it) {
    const int32_t* rec = recs0 + (size_t)it * kRecInts;
    bool mine = false;
    for (int32_t c = 0; c < rec[0] && !mine; ++c) mine = owner.count(rec[kRecChunk + 2 * c]) != 0;
    (mine ? tail : head).push_back(it);
  }
  struct Patch {
    size_t at;  // int offset in the tail records
    int32_t i;
    int64_t L;
  };
  std::vector<Patch> patches;
  for (size_t t = 0; t < tail.size(); ++t) {
    const int32_t* rec = recs0 + (size_t)tail[t] * kRecInts;
    for (int32_t c = 0; c < rec[0]; ++c) {
      const auto f = owner.find(rec[kRecChunk + 2 * c]);
      if (f == owner.end()) continue;
      const int64_t o = f->second;
      patches.push_back({t * kRecInts + kRecChunk + 2 * c + 1, (int32_t)(o >> 32), o & 0xffffffff});
    }
  }
  const size_t rec_bytes = (size_t)kRecInts * sizeof(int32_t);
  size_t off = 0;
  W.off_cow = off;
  off = align256(off + cow.size() * sizeof(PageWrite));
  const size_t off_head = off;
  off = align256(off + head.size() * rec_bytes);
  const size_t off_mptr = off;
  const size_t mptr_bytes = (size_t)pc.n_out_rows * sizeof(int32_t);
  off = align256(off + mptr_bytes);
  W.steps.resize((size_t)n_steps);
  for (int32_t st = 0; st < n_steps; ++st) {
    DecodeWindow::Step& ws = W.steps[st];
    ws.off_items = off_head;
    ws.off_mptr = off_mptr;
    ws.n_head = (int32_t)head.size();
    ws.n_items = pc.n_items;
    ws.n_out_rows = pc.n_out_rows;
    ws.max_parts = pc.max_parts;
    ws.off_plan = off;  // this step's tail records
    off = align256(off + tail.size() * rec_bytes);
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
  for (size_t h = 0; h < head.size(); ++h)
    std::memcpy(W.blob.data() + off_head + h * rec_bytes, recs0 + (size_t)head[h] * kRecInts, rec_bytes);
  std::memcpy(W.blob.data() + off_mptr, pc.blob.data() + pc.off_mptr, mptr_bytes);
  for (int32_t st = 0; st < n_steps; ++st) {
    const DecodeWindow::Step& ws = W.steps[st];
    int32_t* recs = reinterpret_cast<int32_t*>(W.blob.data() + ws.off_plan);
    for (size_t t = 0; t < tail.size(); ++t)
      std::memcpy(recs + t * kRecInts, recs0 + (size_t)tail[t] * kRecInts, rec_bytes);
    for (const Patch& q : patches) {
      const int64_t len = base[q.i] + st + 1 - q.L * PS;  // valid slots of the page after step st
      const int32_t lohi = recs[q.at], lo = lohi & 0xff, hi = lohi >> 8;
      const int32_t nh = (int32_t)std::min<int64_t>(hi, std::max<int64_t>(lo, len));
      recs[q.at] = nh > lo ? (lo | nh << 8) : 0;
    }
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
    dp.tail = reinterpret_cast<const int32_t*>(w + ws.off_plan);
    dp.n_head = ws.n_head;
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
// AgentKV restores an evicted or edited span of a sequence with one prefill in which each
// segment keeps its own positions: the caller appends the segments' K / V (kv_append with
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

int kv_causal_attend_workspace_size(kv_pool_t* P, kv_seq_t seq, int64_t n, int32_t n_q_heads, size_t* bytes) {
  if (!P || !bytes) FAIL(P, KV_ERR_INVALID, "null argument");
  if (int st = causal_plan(P, seq, n, n_q_heads)) return st;
  *bytes = P->plan.ws_need;
  return KV_OK;
}

int kv_causal_attend(kv_pool_t* P, kv_seq_t seq, int64_t n, int32_t n_q_heads, const void* q, void* out, float* lse,
                     float sm_scale, void* workspace, size_t ws_bytes, hipStream_t s) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  if (!P->device) FAIL(P, KV_ERR_INVALID, "metadata-only pool has no KV data");
  if (!q || !out || !workspace) FAIL(P, KV_ERR_INVALID, "null device pointer");
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
    dp.tail = dp.items;
    dp.n_head = pc.n_items;
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
