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
// V^T rows of a page block keep the page's 16 slots in the order 0-3, 8-11, 4-7, 12-15
// (bits 2 and 3 of the slot swapped): slot t of row d is element d * 16 + v_pos(t).  The
// decode reads 4-slot runs (contiguous either way); the tiled prefill's V operand unit, the
// slots {0-3, 8-11} or {4-7, 12-15} of a row, is then 16 contiguous bytes it can copy
// straight from the page.  v_pos is its own inverse.
__host__ __device__ constexpr int v_pos(int t) { return ((t & 4) << 1) | ((t & 8) >> 1) | (t & 3); }

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
  const int32_t* items;     // [n_items][kRecInts]
  const int32_t* cut_hi;    // decode windows: per cut id, the slot end of that reserved page after this
                            // step (a chunk whose lohi carries id + 1 in bits 16..31); null otherwise
  float* part_lse2;         // [n_partials] log2-domain log-sum-exp of the partial
  float* part_o;            // [n_partials][d] normalised partial output
  int32_t n_items;
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

// Drop / repos compaction.  A launch holds the drops of one or more sequences ("jobs");
// every destination page of every job is one list entry, jobs in order, pages in
// ascending logical order within a job.
//   CompactJob: entries [list_base, list_base + n_list) rewrite logical pages first,
//     first + 1, ... of one sequence; tab[tab_base + q - first] is that sequence's page
//     id of logical page q before the drop (q >= first), where the kept tokens are read.
//   CompactRun: destination slots [j0, j0 + len) of the job's sequence receive its old
//     tokens s0, s0 + 1, ... with rotation row rot of cos_sin (-1: no rotation).
//   CompactPage: slots [first_slot, n_slots) of dst_page are (re)written (slots = first_slot
//     | n_slots << 8 | job << 16, job = index of its CompactJob); run0 = the run holding the
//     first of them.  A page rewritten in place
//     may still be a source of lower entries of its job (kept tokens only move down, and a
//     page's kept tokens reach at most two destination pages), so it is written only after
//     entries [wait & 0x3fffffff, + (wait >> 30)) have read their sources.
struct CompactJob {
  int32_t list_base;
  int32_t n_list;
  int32_t first;
  int32_t tab_base;
};
struct CompactRun {
  int32_t j0, s0, len, rot;
};
struct CompactPage {
  int32_t dst_page;
  int32_t run0;
  int32_t slots;
  int32_t wait;
};

struct CompactParams {
  void* k_pages;
  void* v_pages;
  const CompactJob* jobs;
  const CompactPage* pages;
  const CompactRun* runs;
  const int32_t* tab;
  const float* cos_sin;      // [n_rot][d/2][2] cos, sin of (offset * theta^(-2i/d))
  int32_t* done;             // [list entry] = epoch once that entry has read its sources
  int32_t* errors;           // incremented if a wait gives up (never expected)
  int32_t epoch;
  int32_t n_jobs;
  int32_t n_pages;           // list entries (destination pages) in this launch
  int32_t n_kv_heads;
  int32_t pool_pages;        // pool capacity: head h's blocks start at h * pool_pages
};

// Causal attention of a sequence's last nq tokens as a split-K tiled prefill over its
// pages (bf16, d = 128): keys 0 .. T-1 are the visible tokens (own, then mounts) at
// locs[t] = page * 16 + slot; query row r (q row r, key index q_off + r) sees key t
// unless q_off + r < t < n_own.  CSR rows (row_ptr, ent = col | diag bit << 31, order
// by descending length) are (query block r / n_split, key piece r % n_split); each
// writes partials (lse2, normalised o) at slot (row * hq + head) * n_split + piece.
struct RestoreLaunch {
  const void* q;
  const void* k_pages;
  const void* v_pages;
  int32_t pool_pages;
  const int32_t* locs;
  const int32_t* row_ptr;
  const int32_t* ent;
  const int32_t* order;
  char* kimg;  // [hkv][ceil(T / 64)][16 KiB]
  char* vimg;
  float* part_lse2;
  float* part_o;
  int32_t T, n_own, q_off, nq, hq, hkv, n_rows, n_split;
  float sm_scale;
  bool kgather;  // K read straight from the pool (kimg unused): the visible keys in whole pages,
  const int32_t* gpages;  // gpages[g] = the page of keys 16 g .. 16 g + 15 (padded to 4 per 64-key block)
};
constexpr int kRestoreImgBytes = 16384;  // one 64-key image block of one KV head (K or V)

hipError_t launch_page_write(int dtype, int d, int hkv, int pool_pages, void* k_pages, void* v_pages,
                             const void* k_new, const void* v_new, const PageWrite* writes,
                             int n_writes, hipStream_t s);
hipError_t launch_decode(int dtype, int d, const DecodeParams& p, hipStream_t s);
hipError_t launch_merge(int dtype, int d, const MergeParams& p, hipStream_t s);
// the same merge for rows with few partials each (one thread per row and 4 dims)
hipError_t launch_merge_few(int dtype, int d, const MergeParams& p, hipStream_t s);
// ws[patches[2 i]] = patches[2 i + 1] for i < n (int offsets into a decode workspace;
// distinct offsets)
hipError_t launch_plan_patch(void* ws, const int32_t* patches, int n, hipStream_t s);
hipError_t launch_compact(int dtype, int d, const CompactParams& p, hipStream_t s);
bool compact_supported(int dtype, int d, int hkv);  // the kernel's register budget
hipError_t fa_launch_restore(const RestoreLaunch& r, hipStream_t s);

}  // namespace fa
