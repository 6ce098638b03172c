// Fused Drop compaction + Repos re-rotation for gfx950.
//
// AKV (news.farwalk.ai), "AKV 如何工作": Drop removes entries from future attention;
// Repos rewrites the kept keys to positions 0..r-1 by a rotary rotation and leaves the
// values unchanged.  AgentKV (rit.work): kept entries are compacted physically and the
// freed pages go back to the allocator.
//
// One workgroup per destination page (all KV heads); the launch holds the pages of one
// or more drops, each drop's pages in ascending order.  The page's slots find their
// sources through the drop's runs (consecutive kept tokens with one rotation offset) and
// the sequence's block table before the drop.
// Phase 1 gathers the page's kept tokens from their old slots into registers: each
// thread holds a few 16-byte K slot pairs (i, i + d/2) -- rotated by the token's offset
// with fp32 cos/sin rows computed on the host in fp64 (an fp32 angle at 131K positions
// would be off by ~1e-2 rad) -- and a few 16-slot V^T rows, copied bit-exactly: the
// page's kept tokens form a few runs of consecutive source slots, and each run's part of
// a row is its whole source row shifted by the run's slot offset.  Phase 2 stores them
// into the destination page with 16-byte stores.  No LDS image, so many workgroups share
// a CU and hide each other's latency.
//
// In-place hazard: kept tokens only move to lower slots, so a page rewritten in place
// may still be a source of lower destination pages of its drop (at most two: a source
// page's kept tokens are consecutive).  After phase 1 a workgroup publishes "sources
// read" (its loads have returned), and a page rewritten in place waits for exactly the
// lower entries that read it.  The hazard is write-after-read, so relaxed device-scope
// flags order it (acquire / release would write back or invalidate the die's L2 on every
// poll).  Workgroups are dispatched in launch order on each die, and on each die the
// entries rise with the launch order, so the lowest unfinished entry is always resident
// and waits only for finished ones: every wait ends (a bounded spin counts a time-out
// instead of hanging if that order ever failed).
#include <hip/hip_runtime.h>
#include "plan.hpp"

namespace fa {
// 32-bit word q of a stored V^T row holds the slots of word v_word(q) of the row in slot
// order (SPW slots per word; the slot permutation moves whole 4-slot runs)
template <int SPW>
__device__ constexpr int v_word(int q) { return v_pos(SPW * q) / SPW; }
}  // namespace fa

namespace fa {

typedef __bf16 bf16_t;

constexpr int kDies = 8;     // dies (XCDs) of MI355X that workgroups are dealt to in turn
constexpr int kDieRun = 8;   // consecutive list entries per die

template <typename T> __device__ inline float to_f(T x) { return (float)x; }
template <typename T> __device__ inline T from_f(float x) { return (T)x; }

// UK: K slot pairs per thread, UV: V^T rows per thread (upper bounds for this launch)
template <typename T, int D, int UK, int UV>
__global__ __launch_bounds__(256) void compact_kernel(CompactParams p) {
  constexpr int E = 16 / sizeof(T);            // elements per 16-byte slot
  constexpr int NF = D * (int)sizeof(T) / 64;  // K slots per token row and lane group
  constexpr int HALF = NF / 2;                 // slot f pairs with f + HALF (d, d + D/2)
  constexpr int BLK = 16 * D;                  // elements per (page, head) block
  typedef T vec_t __attribute__((__vector_size__(16)));
  const int hkv = p.n_kv_heads;
  __shared__ int s_loc[16], s_rot[16];
  __shared__ int s_run[16][3], s_nrun;  // runs of the page: first slot, length, source location of the first
  // die-aware order: workgroups are handed to the chip's dies round robin, so runs of
  // kDieRun consecutive list entries go to one die; neighbouring destination pages read
  // the same source pages (a source page's kept tokens reach at most two), and the second
  // read then hits that die's L2 instead of HBM.  On each die entries still start in
  // ascending order.
  const int die = blockIdx.x % kDies, on_die = blockIdx.x / kDies;
  const int k = (die + kDies * (on_die / kDieRun)) * kDieRun + on_die % kDieRun;
  if (k >= p.n_pages) return;
  T* kp = reinterpret_cast<T*>(p.k_pages);
  T* vp = reinterpret_cast<T*>(p.v_pages);
  const size_t np = (size_t)p.pool_pages;  // head-major pool: block (page, h) at h * np + page
  const CompactPage cp = p.pages[k];
  const int first_slot = cp.slots & 0xff, n_slots = (cp.slots >> 8) & 0xff;
  const CompactJob jb = p.jobs[(unsigned)cp.slots >> 16];  // the drop this entry belongs to
  const size_t dst = (size_t)cp.dst_page * BLK;
  const bool keep_rest = first_slot > 0 || n_slots < 16;
  // the page's 16 source locations and rotation rows, once, so that every gather below
  // issues its loads independently instead of behind a dependent index load
  if (threadIdx.x < 16) {
    const int t = threadIdx.x;
    int loc = -1, rot = -1;
    if (t >= first_slot && t < n_slots) {
      const int j = (jb.first + (k - jb.list_base)) * 16 + t;  // destination slot in the sequence
      int q = cp.run0;
      CompactRun run = p.runs[q];
      while (j >= run.j0 + run.len) run = p.runs[++q];
      const int src = run.s0 + (j - run.j0);
      loc = p.tab[jb.tab_base + (src >> 4) - jb.first] * 16 + (src & 15);
      rot = run.rot;
    }
    s_loc[t] = loc;
    s_rot[t] = rot;
  }
  __syncthreads();
  // runs: maximal slot ranges whose sources are consecutive slots of one source page
  // (kept tokens are consecutive between dropped spans, so a page has one to three)
  if (threadIdx.x == 0) {
    int nr = 0;
    for (int t = 0; t < 16; ++t) {
      const int loc = s_loc[t];
      if (loc < 0) continue;
      if (nr > 0 && s_run[nr - 1][0] + s_run[nr - 1][1] == t && s_run[nr - 1][2] + s_run[nr - 1][1] == loc &&
          (loc >> 4) == (s_run[nr - 1][2] >> 4)) {
        ++s_run[nr - 1][1];
        continue;
      }
      s_run[nr][0] = t;
      s_run[nr][1] = 1;
      s_run[nr][2] = loc;
      ++nr;
    }
    s_nrun = nr;
  }
  __syncthreads();

  // ---- phase 1a: K slot pairs (with rotation); unit u = ((h * HALF + fp) * 4 + g) * 16 + t
  const int n_ku = hkv * HALF * 64;
  vec_t ka[UK], kb[UK];
#pragma unroll
  for (int i = 0; i < UK; ++i) {
    const int u = threadIdx.x + i * 256;
    const int t = u & 15, g = (u >> 4) & 3, fp = (u >> 6) % HALF, h = (u >> 6) / HALF;
    const int loc = u < n_ku ? s_loc[t] : -1;
    if (loc >= 0) {
      const size_t sb = ((size_t)h * np + (loc >> 4)) * BLK;
      const int st = loc & 15;
      ka[i] = *reinterpret_cast<const vec_t*>(kp + sb + ((fp * 4 + g) * 16 + st) * E);
      kb[i] = *reinterpret_cast<const vec_t*>(kp + sb + (((fp + HALF) * 4 + g) * 16 + st) * E);
      const int run = s_rot[t];
      if (run >= 0) {
        const float* cs = p.cos_sin + (size_t)run * D;  // [D/2][2]
        if constexpr (sizeof(T) == 2) {
          // the slot's 8 dims are consecutive: their (cos, sin) pairs are 64 contiguous bytes
          typedef float f32x4 __attribute__((ext_vector_type(4)));
          const f32x4* c4 = reinterpret_cast<const f32x4*>(cs + 2 * (32 * fp + 8 * g));
          f32x4 w[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) w[q] = c4[q];
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const float c = w[e >> 1][2 * (e & 1)], sn = w[e >> 1][2 * (e & 1) + 1];
            const float x = to_f(ka[i][e]), y = to_f(kb[i][e]);
            ka[i][e] = from_f<T>(x * c - y * sn);
            kb[i][e] = from_f<T>(y * c + x * sn);
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const int d = 16 * fp + 4 * e + g;
            const float c = cs[2 * d], sn = cs[2 * d + 1];
            const float x = to_f(ka[i][e]), y = to_f(kb[i][e]);
            ka[i][e] = from_f<T>(x * c - y * sn);
            kb[i][e] = from_f<T>(y * c + x * sn);
          }
        }
      }
    }
  }
  // ---- phase 1b: V^T rows (bit-exact); row r = h * D + d holds slots 0..15 as WPR 32-bit
  // words.  Per run, the whole source row is loaded (two 16-byte loads) and shifted by the
  // run's slot offset: word moves with a wave-uniform index, alignbyte for half-word
  // shifts of bf16; the run's slots are then merged into the row.
  constexpr int WPR = 16 * (int)sizeof(T) / 4;  // 32-bit words per V^T row
  constexpr int SPW = 4 / (int)sizeof(T);       // slots per word
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const int n_vr = hkv * D;
  const int nrun = s_nrun;
  unsigned vr[UV][WPR];
#pragma unroll
  for (int i = 0; i < UV; ++i) {
    const int r = threadIdx.x + i * 256;
    if (r < n_vr) {
      const int h = r / D, d = r % D;
      const u32x4* old = reinterpret_cast<const u32x4*>(vp + dst + (size_t)h * np * BLK + d * 16);
      // rows are held in slot order: stored word q holds the slots of word v_word(q)
#pragma unroll
      for (int w4 = 0; w4 < WPR / 4; ++w4) {
        const u32x4 x = keep_rest ? old[w4] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[i][v_word<SPW>(4 * w4 + e)] = x[e];
      }
      for (int k = 0; k < nrun; ++k) {  // wave-uniform
        const int t0 = s_run[k][0], len = s_run[k][1], loc = s_run[k][2];
        const int delta = (loc & 15) - t0;  // source slot of destination slot t: t + delta
        const u32x4* srow = reinterpret_cast<const u32x4*>(vp + ((size_t)h * np + (loc >> 4)) * BLK + d * 16);
        unsigned src[WPR + 2];  // the source row with a zero word on either side
        src[0] = 0u;
        src[WPR + 1] = 0u;
#pragma unroll
        for (int w4 = 0; w4 < WPR / 4; ++w4) {
          const u32x4 x = srow[w4];
#pragma unroll
          for (int e = 0; e < 4; ++e) src[1 + v_word<SPW>(4 * w4 + e)] = x[e];
        }
#pragma unroll
        for (int w = 0; w < WPR; ++w) {
          const int a = SPW * w + delta;            // source slot of this word's first slot
          int kw = SPW == 2 ? (a >> 1) : a;         // source word holding it (floor)
          kw = kw < -1 ? -1 : (kw > WPR - 1 ? WPR - 1 : kw);
          unsigned val = src[kw + 1];
          if (SPW == 2 && (a & 1)) val = __builtin_amdgcn_alignbyte(src[kw + 2], src[kw + 1], 2);
          const int lo_slot = SPW * w, hi_slot = SPW * w + SPW - 1;
          const bool lo_in = lo_slot >= t0 && lo_slot < t0 + len;
          const bool hi_in = hi_slot >= t0 && hi_slot < t0 + len;
          if (SPW == 1) {
            vr[i][w] = lo_in ? val : vr[i][w];
          } else {
            const unsigned keep = (lo_in ? 0u : 0x0000ffffu) | (hi_in ? 0u : 0xffff0000u);
            vr[i][w] = (vr[i][w] & keep) | (val & ~keep);
          }
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // every source load of this thread has returned ...
  __syncthreads();                // ... and of every thread

  // ---- publish "sources read", then wait for the lower entries that read this page
  if (threadIdx.x == 0) {
    __hip_atomic_store(&p.done[k], p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int wait_lo = cp.wait & 0x3fffffff, wait_hi = wait_lo + ((unsigned)cp.wait >> 30);
    for (int i = wait_lo; i < wait_hi && i < k; ++i) {
      int spins = 0;
      while (__hip_atomic_load(&p.done[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != p.epoch) {
        __builtin_amdgcn_s_sleep(4);
        if (++spins > (1 << 26)) {  // ~seconds: never expected; counted, never hangs
          atomicAdd(p.errors, 1);
          break;
        }
      }
    }
  }
  __syncthreads();

  // ---- phase 2: stores into the destination page (slots without a source keep their
  // old K; V rows are written whole, old slots included)
#pragma unroll
  for (int i = 0; i < UK; ++i) {
    const int u = threadIdx.x + i * 256;
    const int t = u & 15, g = (u >> 4) & 3, fp = (u >> 6) % HALF, h = (u >> 6) / HALF;
    if (u < n_ku && s_loc[t] >= 0) {
      T* blk = kp + dst + (size_t)h * np * BLK;
      *reinterpret_cast<vec_t*>(blk + ((fp * 4 + g) * 16 + t) * E) = ka[i];
      *reinterpret_cast<vec_t*>(blk + (((fp + HALF) * 4 + g) * 16 + t) * E) = kb[i];
    }
  }
#pragma unroll
  for (int i = 0; i < UV; ++i) {
    const int r = threadIdx.x + i * 256;
    if (r < n_vr) {
      const int h = r / D, d = r % D;
      u32x4* row = reinterpret_cast<u32x4*>(vp + dst + (size_t)h * np * BLK + d * 16);
#pragma unroll
      for (int w4 = 0; w4 < WPR / 4; ++w4)
        row[w4] = u32x4{vr[i][v_word<SPW>(4 * w4)], vr[i][v_word<SPW>(4 * w4 + 1)], vr[i][v_word<SPW>(4 * w4 + 2)],
                        vr[i][v_word<SPW>(4 * w4 + 3)]};
    }
  }
}

template <typename T, int D, int UK, int UV>
static hipError_t compact_t(const CompactParams& p, hipStream_t s) {
  constexpr int per_round = kDies * kDieRun;  // grid rounded up; the surplus workgroups exit at once
  compact_kernel<T, D, UK, UV><<<(p.n_pages + per_round - 1) / per_round * per_round, 256, 0, s>>>(p);
  return hipGetLastError();
}

// per-thread counts: K slot pairs = Hkv * (D * sizeof(T) / 128) * 64 / 256, V^T rows =
// Hkv * D / 256; instantiated for up to 8 of each (Hkv <= 16 at bf16, d = 128)
template <typename T, int D>
static hipError_t compact_dispatch(const CompactParams& p, hipStream_t s) {
  if (p.n_pages == 0) return hipSuccess;
  const int half = D * (int)sizeof(T) / 128;
  const int uk = (p.n_kv_heads * half * 64 + 255) / 256;
  const int uv = (p.n_kv_heads * D + 255) / 256;
  const int u = uk > uv ? uk : uv;
  if (u <= 1) return compact_t<T, D, 1, 1>(p, s);
  if (u <= 2) return compact_t<T, D, 2, 2>(p, s);
  if (u <= 4) return compact_t<T, D, 4, 4>(p, s);
  if (u <= 8) return compact_t<T, D, 8, 8>(p, s);
  return hipErrorInvalidValue;
}

bool compact_supported(int dtype, int d, int hkv) {
  const int half = d * (dtype == 1 ? 4 : 2) / 128;
  return (d == 64 || d == 128) && (hkv * half * 64 + 255) / 256 <= 8 && (hkv * d + 255) / 256 <= 8;
}

hipError_t launch_compact(int dtype, int d, const CompactParams& p, hipStream_t s) {
  if (dtype == 0 && d == 128) return compact_dispatch<bf16_t, 128>(p, s);
  if (dtype == 0 && d == 64) return compact_dispatch<bf16_t, 64>(p, s);
  if (dtype == 1 && d == 128) return compact_dispatch<float, 128>(p, s);
  if (dtype == 1 && d == 64) return compact_dispatch<float, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
