// Host runtime of libforkattn: page pool, block tables, plans.  Single-threaded per pool.
#pragma once
#include <stdint.h>
#include <string>
#include <vector>
#include <map>
#include <hip/hip_runtime_api.h>
#include "../../include/forkattn.h"
#include "plan.hpp"

namespace fa {

struct Status {
  int code;
  std::string msg;
};

// Positions of consecutive tokens as runs p0, p0 + 1, ..., p0 + len - 1.
struct PosRun {
  int64_t p0;
  int64_t len;
};

struct Mount {
  std::vector<int32_t> pages;
  int32_t off;  // token offset of the first mounted token in pages[0]
  int64_t n;
  std::vector<PosRun> pos;
};

struct Seq {
  bool live = true;
  std::vector<int32_t> pages;  // own context, logical page -> page id
  int64_t n = 0;
  std::vector<PosRun> pos;
  int64_t next_pos = 0;
  std::vector<Mount> mounts;
};

// Lowest-id-first free set over a bitmap.
class FreeSet {
 public:
  void init(int32_t n);
  int32_t count() const { return count_; }
  // the k lowest free ids, without taking them
  void peek_lowest(int32_t k, std::vector<int32_t>& out) const;
  void take(int32_t id);
  void give(int32_t id);
  bool is_free(int32_t id) const { return (bits_[id >> 6] >> (id & 63)) & 1ull; }

 private:
  std::vector<uint64_t> bits_;  // 1 = free
  int32_t n_ = 0, count_ = 0;
  int32_t hint_ = 0;  // no free id below word hint_
};

// Page-table changes since the cached decode plan, one per version step, so that a plan
// can be patched instead of rebuilt when the only changes are appends that wrote into
// pages their sequence owns alone (a decode step's one token per branch).
struct ChangeJournal {
  // kAppend: tokens appended with no page copied; kTouch: the sequence changed in another
  // way; kContent: only token contents changed; kOther: anything the journal cannot follow
  enum Kind : int32_t { kAppend = 0, kTouch = 1, kOther = 2, kContent = 3 };
  struct Event {
    int32_t seq, kind;
    int64_t n0, n1;  // kAppend: token count before / after
  };
  uint64_t base = 0;  // pool version the journal starts at
  bool broken = true;
  std::vector<Event> ev;
  void reset(uint64_t version) {
    base = version;
    broken = false;
    ev.clear();
  }
};

struct DecodePlanCache {
  bool valid = false;
  uint64_t version = 0;
  std::vector<int32_t> seqs;
  int32_t n_q_heads = 0;
  void* ws = nullptr;
  size_t ws_need = 0;
  // device offsets
  size_t off_items = 0, off_mptr = 0, off_plse = 0, off_po = 0;
  int32_t n_items = 0, n_out_rows = 0, max_parts = 1;
  std::vector<char> blob;  // host image of the plan part of the workspace
  int64_t stats[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int64_t causal_n = 0;  // 0: a decode plan; n > 0: causal rows of the last n tokens; -1: other caps
  uint64_t serial = 0;   // unique across pools and rebuilds: names this plan's contents
  // patching (decode plans only): query of each listed sequence (-1 listed twice), per
  // query its own token count and tail page, per (query, KV head) the record and chunk
  // slot of the tail page's chunk and the record of the private segment's last item
  bool patchable = false;
  std::vector<int32_t> q_seq, q_own_n, q_tail_page;  // by query
  std::vector<int32_t> tail_rec, tail_slot, last_rec;  // by query * Hkv + head
  std::vector<int32_t> pending;                        // (int offset, value) pairs not yet on the device
};

// A steady-state decode window: every sequence's next n_steps slots reserved up front and
// one decode plan per step, so each step is a fixed set of kernel launches.
struct DecodeWindow {
  struct Step {
    size_t off_cut = 0;    // this step's slot end per cut id (reserved pages)
    size_t off_items = 0;  // the item records (shared by every step)
    size_t off_mptr = 0, off_writes = 0;
    int32_t n_items = 0, n_out_rows = 0, max_parts = 1;
  };
  bool valid = false;
  uint64_t version = 0;
  std::vector<int32_t> seqs;
  int32_t n_q_heads = 0, n_steps = 0, n_cow = 0;
  size_t off_cow = 0, off_plse = 0, off_po = 0, ws_need = 0;
  std::vector<Step> steps;
  std::vector<char> blob;  // plan, per-step cut tables and writes, at their workspace offsets
  void* ws = nullptr;
};

// Causal attention of a sequence's last n tokens as a split-K tiled prefill (bf16 pools,
// d = 128): the visible keys' locations, the CSR of (query block, key piece) rows and the
// merge counts, uploaded once per sequence state into the caller's workspace.
struct RestorePlan {
  bool valid = false;
  uint64_t version = 0;
  kv_seq_t seq = -1;
  int64_t n = 0;
  int32_t hq = 0;
  std::vector<char> blob;  // [locs | row_ptr | ent | order | counts | page per 16 keys], uploaded
  size_t off_locs = 0, off_rowptr = 0, off_ent = 0, off_order = 0, off_count = 0, off_gpages = 0;
  size_t off_kimg = 0, off_vimg = 0, off_plse = 0, off_po = 0, ws_need = 0;
  int32_t T = 0, n_own = 0, n_rows = 0, n_split = 1;
  bool kgather = false;  // K read straight from the pool by the prefill kernel (no K images)
  void* ws = nullptr;  // workspace the blob was last uploaded to
};

}  // namespace fa

struct kv_pool {
  kv_pool_config cfg;
  bool device = false;
  void* k = nullptr;
  void* v = nullptr;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  std::vector<int32_t> rc;
  fa::FreeSet free;
  std::vector<fa::Seq> seqs;
  uint64_t version = 1;
  std::string err;
  int32_t n_cu = 256;
  // pinned staging ring for plan uploads: a slot is reused once the copy that read it
  // has run, so the host can plan several operations ahead of the device
  struct StageSlot {
    void* ptr = nullptr;
    size_t bytes = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
  };
  static constexpr int kStageSlots = 8;
  StageSlot stage[kStageSlots];
  // staging buffers outgrown by larger uploads, freed with the pool (freeing pinned
  // memory waits for the whole device, so it never happens between operations)
  std::vector<void*> retired;
  int stage_next = 0;
  // drop-kernel ordering state (see CompactParams)
  int32_t epoch = 0;
  fa::DecodePlanCache plan;
  fa::ChangeJournal journal;
  fa::RestorePlan restore;
  fa::DecodeWindow window;
  // key scoring: the chunk list last uploaded (sequence, page-table version, workspace)
  struct ScoreChunks {
    uint64_t version = 0;
    kv_seq_t seq = -1;
    void* ws = nullptr;
    int32_t n_ch = 0;
  } score_chunks;
};
