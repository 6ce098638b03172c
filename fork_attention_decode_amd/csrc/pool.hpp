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
  int64_t stats[6] = {0, 0, 0, 0, 0, 0};
  int64_t causal_n = 0;  // 0: a decode plan; n > 0: causal rows of the last n tokens; -1: other caps
};

// A steady-state decode window: every sequence's next n_steps slots reserved up front and
// one decode plan per step, so each step is a fixed set of kernel launches.
struct DecodeWindow {
  struct Step {
    size_t off_plan = 0;   // this step's tail item records
    size_t off_items = 0;  // the head item records (shared by every step)
    size_t off_mptr = 0, off_writes = 0;
    int32_t n_head = 0, n_items = 0, n_out_rows = 0, max_parts = 1;
  };
  bool valid = false;
  uint64_t version = 0;
  std::vector<int32_t> seqs;
  int32_t n_q_heads = 0, n_steps = 0, n_cow = 0;
  size_t off_cow = 0, off_plse = 0, off_po = 0, ws_need = 0;
  std::vector<Step> steps;
  std::vector<char> blob;  // plans, step writes and tail copies, at their workspace offsets
  void* ws = nullptr;
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
  int stage_next = 0;
  // drop-kernel ordering state (see CompactParams)
  int32_t ticket = 0;
  int32_t epoch = 0;
  fa::DecodePlanCache plan;
  fa::DecodeWindow window;
  // key scoring: the chunk list last uploaded (sequence, page-table version, workspace)
  struct ScoreChunks {
    uint64_t version = 0;
    kv_seq_t seq = -1;
    void* ws = nullptr;
    int32_t n_ch = 0;
  } score_chunks;
};
