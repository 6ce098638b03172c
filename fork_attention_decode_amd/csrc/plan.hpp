// Plan records shared by the host runtime (C++) and the gfx950 kernels (HIP).
// Plain structs of fixed layout: the host fills them, copies them into a device
// workspace, and the kernels read them.
#pragma once
#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace fa {

constexpr int kPage = 16;        // tokens per page on device pools
constexpr int kMaxRows = 64;     // query rows per decode work item (4 MFMA row blocks of 16)
constexpr int kWaves = 4;        // waves per decode workgroup
constexpr int kMaxItemChunks = 128;     // chunk metadata in two registers per lane
constexpr int kRingBytes = 65536;       // LDS ring of a wide item

// One page write of kv_append / kv_write: slots [lo, hi) of dst_page receive new tokens
// tok_base, tok_base + 1, ...; when src_page >= 0 (copy-on-write) every other slot is
// copied from src_page, otherwise the other slots are left untouched.
struct PageWrite {
  int32_t dst_page;
  int32_t src_page;
  int32_t lo, hi;
  int64_t tok_base;
};

// A run of token slots inside one physical page, read by one segment's rows.
struct Chunk {
  int32_t page;
  int32_t lohi;  // lo | hi << 8, 0 <= lo < hi <= 16
};

// One decode work item: up to kMaxItemChunks chunks of one segment, for KV head kv_head
// and up to 64 of the segment's rows (n_readers * G).  The workgroup streams every chunk
// once into an LDS ring and wave w computes rows [16 w, 16 w + 16).
// Items are self-contained fixed-stride records, so a workgroup finds everything it
// needs with one round of independent loads (no pointer chasing before its first
// K / V load):
//   int32 [0, 4)          n_chunks, kv_head, n_rows, 0
//   int32 [4, 68)         output row (query * Hq + head) of item row r, -1 past n_rows
//   int32 [68, 132)       partial slot of item row r
//   int32 [132, 388)      chunks: (page, lo | hi << 8) pairs
constexpr int kRecRow = 4;
constexpr int kRecSlot = 68;
constexpr int kRecChunk = 132;
constexpr int kRecInts = 416;  // 1664-byte stride

// Decode launch: one workgroup per item record.
struct DecodeParams {
  const void* q;            // [n_seqs][Hq][d]
  const void* k_pages;
  const void* v_pages;
  const int32_t* items;     // [n_head][kRecInts]: items 0 .. n_head - 1
  const int32_t* tail;      // [n_items - n_head][kRecInts]: the rest (a decode window's per-step items)
  float* part_lse2;         // [n_partials] log2-domain log-sum-exp of the partial
  float* part_o;            // [n_partials][d] normalised partial output
  int32_t n_items;
  int32_t n_head;
  int32_t cached;           // 1: cached loads (the launch streams the same pages several times)
  int32_t n_pages;          // pool capacity: head h's blocks start at h * n_pages
  float scale_log2;         // sm_scale * log2(e)
};

// Merge launch: output row r (= query * Hq + head) owns the partial slots
// [r * max_parts, r * max_parts + count[r]); the rest of its block is never read
// into the result (masked by selects).
struct MergeParams {
  const int32_t* count;     // [n_rows] partials of each output row
  const float* part_lse2;
  const float* part_o;
  void* out;                // [n_rows][d]
  float* lse;               // [n_rows] natural log, or null
  int32_t n_rows;
  int32_t max_parts;
};

// Drop / repos compaction: one record per destination page to (re)write.  Slots
// [first_slot, n_slots) of dst_page receive the kept tokens tok_base + slot; when the
// page is rewritten in place its old tokens may be sources of lower destination pages
// (kept tokens only move down), so the page is written only after the list entries
// [wait_lo, wait_hi) that read it have read their sources (an empty range: nothing to
// wait for).  A source page's kept tokens are consecutive in the kept order, so at most
// two destination pages read it.
struct CompactPage {
  int32_t dst_page;
  int32_t first_slot;
  int32_t n_slots;
  int32_t tok_base;
  int32_t wait_lo;
  int32_t wait_hi;
  int32_t pad[2];
};

// Destination pages per compaction workgroup (one start-order ticket per batch).  One:
// with more, a reader page's gather waits behind the earlier pages of its batch, which
// chains the in-place waits (measured 1.2x / 1.8x / 2.7x slower at 2 / 4 / 8).
constexpr int kCompactBatch = 1;

struct CompactParams {
  void* k_pages;
  void* v_pages;
  const CompactPage* pages;
  const int32_t* src_loc;    // [token] old page * 16 + old slot of the kept token
  const int32_t* rot;        // [token] row of cos_sin, -1 = no rotation
  const float* cos_sin;      // [n_rot][d/2][2] cos, sin of (offset * theta^(-2i/d))
  int32_t* ticket;           // monotone counter: order in which workgroups start
  int32_t* done;             // [list entry] = epoch once that entry has read its sources
  int32_t* errors;           // incremented if a wait gives up (never expected)
  int32_t ticket_base;
  int32_t epoch;
  int32_t n_pages;           // destination pages in this launch
  int32_t n_kv_heads;
  int32_t pool_pages;        // pool capacity: head h's blocks start at h * pool_pages
};

hipError_t launch_page_write(int dtype, int d, int hkv, int pool_pages, void* k_pages, void* v_pages,
                             const void* k_new, const void* v_new, const PageWrite* writes,
                             int n_writes, hipStream_t s);
hipError_t launch_decode(int dtype, int d, const DecodeParams& p, hipStream_t s);
hipError_t launch_merge(int dtype, int d, const MergeParams& p, hipStream_t s);
hipError_t launch_compact(int dtype, int d, const CompactParams& p, hipStream_t s);
bool compact_supported(int dtype, int d, int hkv);  // the kernel's register budget

}  // namespace fa
