// Key scoring and keep selection in front of Drop, for gfx950.
//
// AgentKV (rit.work), section "Как AgentKV выбирает и освобождает записи кэша": before a
// compression the per-phase queues of recent attention queries are merged, every key is
// scored against the merged set and the entries with the highest mean attention are
// kept (32 representative queries in the main experiments); the rest is dropped, the
// kept entries compacted and the freed pages returned (kv_drop).
//
// score(t) = mean over the n_rep x Hq (representative query, head) pairs of the softmax
// probability of own token t in that query's attention over the sequence's visible
// context.  Two passes over the keys, each streaming a page's K block once per KV head
// through a ring in LDS (buffer loads that write LDS, several slots ahead) and computing
// S = Q K^T for all of the head's rows (query x head-of-group) on
// v_mfma_f32_16x16x32_bf16, each wave taking a share of the row tiles over every page of
// a slot (its query fragments in registers):
//   1. norm_kernel (keys as the A operand, so a lane holds 4 keys of one row): every lane
//      keeps an online (max, sum) per row tile over the visible chunks (own pages, then
//      mounts), rescaled lazily, reduced over the lanes into one partial per row and
//      workgroup; norm_merge_kernel folds the workgroups' partials into each row's log2
//      normaliser;
//   2. score_kernel (keys as B, so a lane holds one key of 4 rows): over the own pages,
//      the sum over a wave's rows of exp2(S c2 - lse2) stays in the lane plus two
//      shuffles, and the waves' sums meet in LDS.
// Keep selection: radix select of the budget-th largest score on an order-preserving
// integer image of the floats (4 passes of 8 bits over many workgroups), then ties kept
// in index order (a slice's ties start after the earlier slices' count of the last
// digit).
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <cstddef>
#include <string>
#include <vector>

#include "pool.hpp"

using namespace fa;

int fa_set_err(kv_pool* P, int code, const std::string& m);
Seq* fa_seq(kv_pool* P, kv_seq_t s);
hipError_t fa_upload(kv_pool* P, void* dst, const void* src, size_t bytes, hipStream_t s);
#define FAIL(P, code, msg) return fa_set_err((P), (code), (msg))

namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((__vector_size__(8 * sizeof(bf16_t))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxScoreRows = 256;  // representative queries x query heads per KV head
constexpr int kWaves = 4;           // waves per scoring workgroup = pages per ring slot
constexpr int kSlots = 4;           // ring slots (3 in flight while one computes)
constexpr int kChunksPerWg = 128;
constexpr float kEmpty = -1e30f;    // running max of an empty (max, sum) state

struct ScoreParams {
  const bf16_t* q;        // [n_rep][hq][D] representative queries (rotated)
  const bf16_t* k_pages;  // pool K, head-major blocks
  const int32_t* chunks;  // [n_ch][2]: page id, lo | hi << 8 (valid slots); own pages first
  float* part;            // normaliser partials [hkv][RP][2][nx]: log2-domain max, sum
  float* lse2;            // [hkv][RP] log2 normaliser of each row (+inf for padding rows)
  float* partial;         // [hkv][n_tok] per-KV-head score sums over that head's rows
  int32_t n_rep, hq, hkv, G, pool_pages, n_ch, n_lp, RP, nx;
  int64_t n_tok;
  float c2;  // sm_scale * log2(e)
};

// (m, l) <- the log-sum-exp union of (m, l) and (mo, lo); empty states are (kEmpty, 0)
__device__ __forceinline__ void lse_combine(float& m, float& l, float mo, float lo) {
  const float mn = fmaxf(m, mo);
  l = l * __builtin_amdgcn_exp2f(m - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
  m = mn;
}

// s_waitcnt vmcnt(N), the other counters left free (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int D>
constexpr int kPageBytes = 16 * D * 2;  // one page's K block

// A workgroup barrier without the fence of __syncthreads (which would also wait for the
// ring copies in flight); the LDS writes before it (the key sums) are waited for here.
__device__ __forceinline__ void ring_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// the workgroup's chunks C0 .. C1 - 1 into LDS
__device__ __forceinline__ void stage_chunks(const ScoreParams& p, int C0, int C1, int* ch) {
  for (int i = threadIdx.x; i < 2 * (C1 - C0); i += blockDim.x) ch[i] = p.chunks[2 * C0 + i];
}

// The K blocks stream through a ring of kSlots slots in LDS, kWaves pages per slot (wave w
// copies page w of each slot with buffer loads that write LDS, issued kSlots - 1 slots
// ahead; a slot past the end reloads the last chunk into a slot nobody reads, so every
// wave always has the same number of loads in flight).  Every wave then computes on all
// the slot's pages for its own row tiles: each K fragment read from LDS feeds TW MFMAs.
template <int D>
__device__ __forceinline__ void ring_issue(const ScoreParams& p, const int* ch, int h, int j, int n, int wave,
                                           int lane, char* ring) {
  constexpr int LPW = kPageBytes<D> / 1024;
  const int c = min(kWaves * j + wave, n - 1);
  const int page = __builtin_amdgcn_readfirstlane(ch[2 * c]);
  const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.k_pages + ((size_t)h * p.pool_pages + page) * 16 * D), 0, kPageBytes<D>, 0x00020000);
  char* dst = ring + ((j % kSlots) * kWaves + wave) * kPageBytes<D>;
#pragma unroll
  for (int i = 0; i < LPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16,
                                             lane * 16, i * 1024, 0, 0);
}

// K fragments of the kWaves pages of ring slot j (lane t + 16 g holds K[t][32 f + 8 g .. + 8])
template <int D>
__device__ __forceinline__ void ring_frags(const char* ring, int j, int lane, bf16x8 (&kf)[kWaves][D / 32]) {
#pragma unroll
  for (int pp = 0; pp < kWaves; ++pp)
#pragma unroll
    for (int f = 0; f < D / 32; ++f)
      kf[pp][f] = *reinterpret_cast<const bf16x8*>(ring + ((j % kSlots) * kWaves + pp) * kPageBytes<D> +
                                                   (f * 64 + lane) * 16);
}

// this wave's query fragments: row tile T, lane r % 16 + 16 g holds Q[row 16 T + r][32 f +
// 8 g .. + 8] (the A and B operand orders agree); rows past R are zero
template <int D, int TW>
__device__ __forceinline__ void load_q(const ScoreParams& p, int h, int row0, int T0, int lane,
                                       bf16x8 (&qf)[TW][D / 32]) {
  const int R = p.n_rep * p.G;
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    const int row = row0 + 16 * (T0 + t) + (lane & 15);
    const int rep = row / p.G, qh = h * p.G + row % p.G;
#pragma unroll
    for (int f = 0; f < D / 32; ++f) {
      i32x4 v = {0, 0, 0, 0};
      if (row < R) v = *reinterpret_cast<const i32x4*>(p.q + ((size_t)rep * p.hq + qh) * D + 32 * f + 8 * (lane >> 4));
      qf[t][f] = __builtin_bit_cast(bf16x8, v);
    }
  }
}

// pass 1: grid (nx, hkv), kWaves waves; RT 16-row tiles cover the head's rows row0 ..
// row0 + 16 RT, TW per wave (waves past RT / TW only copy).  The keys are the MFMA's A
// operand here (the pool's K block is laid out for either side), so each lane holds 4 keys
// of one row per tile and keeps one (max, sum) per tile, rescaled lazily.
template <int D, int RT>
__global__ __launch_bounds__(kWaves * 64) void norm_kernel(ScoreParams p, int row0) {
  constexpr int NF = D / 32, TW = RT >= kWaves ? RT / kWaves : 1, LPW = kPageBytes<D> / 1024;
  static_assert(RT <= 8, "row tiles per launch");
  // one LDS array: with several, the compiler tells their accesses apart and then waits
  // for every copy in flight before each read of the ring
  __shared__ __attribute__((aligned(1024))) char lds[kSlots * kWaves * kPageBytes<D> + 8 * kChunksPerWg];
  char* const ring = lds;
  int* const ch = reinterpret_cast<int*>(lds + kSlots * kWaves * kPageBytes<D>);
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int C0 = blockIdx.x * kChunksPerWg;
  const int n = min(C0 + kChunksPerWg, p.n_ch) - C0;
  const int n_slots = (n + kWaves - 1) / kWaves;
  const bool act = wave * TW < RT;
  stage_chunks(p, C0, C0 + n, ch);
  bf16x8 qf[TW][NF];
  load_q<D, TW>(p, h, row0, act ? wave * TW : 0, lane, qf);
  float m[TW], l[TW];
#pragma unroll
  for (int t = 0; t < TW; ++t) m[t] = kEmpty, l[t] = 0.f;
  const int key0 = 4 * (lane >> 4);
  const float c2 = p.c2;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSlots - 1; ++j) ring_issue<D>(p, ch, h, j, n, wave, lane, ring);
  for (int j = 0; j < n_slots; ++j) {
    wait_vmcnt<(kSlots - 2) * LPW>();  // this wave's page of slot j landed ...
    ring_barrier();                    // ... and every wave's; slot j - 1 is consumed
    ring_issue<D>(p, ch, h, j + kSlots - 1, n, wave, lane, ring);
    if (!act) continue;
    bf16x8 kf[kWaves][NF];
    ring_frags<D>(ring, j, lane, kf);
    int lohi[kWaves];
    bool full = true;
#pragma unroll
    for (int pp = 0; pp < kWaves; ++pp) {
      const int c = kWaves * j + pp;
      lohi[pp] = c < n ? ch[2 * c + 1] : 0;  // past the end: an empty slot range
      full = full && lohi[pp] == (16 << 8);
    }
#pragma unroll
    for (int t = 0; t < TW; ++t) {
      f32x4 acc[kWaves];
#pragma unroll
      for (int pp = 0; pp < kWaves; ++pp) {
        acc[pp] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[pp] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[pp][f], qf[t][f], acc[pp], 0, 0, 0);
      }
      // acc[pp][i]: key 4 (lane / 16) + i of page pp of the slot, row 16 T + lane % 16
      if (!full) {
#pragma unroll
        for (int pp = 0; pp < kWaves; ++pp)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool valid = key0 + i >= (lohi[pp] & 0xff) && key0 + i < (lohi[pp] >> 8);
            acc[pp][i] = valid ? acc[pp][i] : -INFINITY;
          }
      }
      // lazy rescale: the sum is taken against the running max as it stands, and only a
      // lane whose keys reach 2^64 times that (the first keys, against an empty state)
      // takes the max of the slot and rescales
      float sum = 0.f;
#pragma unroll
      for (int pp = 0; pp < kWaves; ++pp)
#pragma unroll
        for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[pp][i], c2, -m[t]));
      if (sum <= 0x1p64f) {
        l[t] += sum;
      } else {
        float mx = acc[0][0];
#pragma unroll
        for (int pp = 0; pp < kWaves; ++pp)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, acc[pp][i]);
        const float mn = fmaxf(m[t], mx * c2);
        sum = 0.f;
#pragma unroll
        for (int pp = 0; pp < kWaves; ++pp)
#pragma unroll
          for (int i = 0; i < 4; ++i) sum += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[pp][i], c2, -mn));
        l[t] = __builtin_fmaf(l[t], __builtin_amdgcn_exp2f(m[t] - mn), sum);
        m[t] = mn;
      }
    }
  }
  wait_vmcnt<0>();  // no load may land in LDS after the workgroup ends
  if (!act) return;
  // row 16 T + lane % 16 is held by the 4 lanes lane % 16 + 16 k, and by no other wave
#pragma unroll
  for (int t = 0; t < TW; ++t) {
    lse_combine(m[t], l[t], __shfl_xor(m[t], 16), __shfl_xor(l[t], 16));
    lse_combine(m[t], l[t], __shfl_xor(m[t], 32), __shfl_xor(l[t], 32));
    if (lane < 16) {
      const int r = 16 * (wave * TW + t) + lane;
      float* dst = p.part + ((size_t)(h * p.RP + row0 + r) * 2) * p.nx + blockIdx.x;
      dst[0] = m[t];
      dst[p.nx] = l[t];
    }
  }
}

// one wave per (KV head, row): lanes stride over the nx workgroup partials
__global__ __launch_bounds__(256) void norm_merge_kernel(ScoreParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // h * RP + r
  if (row >= p.hkv * p.RP) return;
  const float* src = p.part + (size_t)row * 2 * p.nx;
  float M = kEmpty, L = 0.f;
  for (int x = lane; x < p.nx; x += 64) lse_combine(M, L, src[x], src[p.nx + x]);
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) lse_combine(M, L, __shfl_xor(M, off), __shfl_xor(L, off));
  if (lane == 0) {
    const bool pad = row % p.RP >= p.n_rep * p.G;
    p.lse2[row] = (pad || L <= 0.f) ? INFINITY : M + __log2f(L);  // no visible key: adds nothing
  }
}

// pass 2: grid (ceil(n_lp / kChunksPerWg), hkv), kWaves waves, over the own pages (the
// first n_lp chunks); rows of KV head h: r = rep * G + g (query head h * G + g), padded
// with zero queries and +inf normalisers to RT whole 16-row tiles, TW per wave.  Keys are
// the B operand (a lane holds one key of 4 rows): the sum over a wave's rows stays in the
// lane plus two shuffles, and the waves' sums meet in LDS, added one slot later.
template <int D, int RT>
__global__ __launch_bounds__(kWaves * 64) void score_kernel(ScoreParams p) {
  constexpr int NF = D / 32, TW = RT >= kWaves ? RT / kWaves : 1, LPW = kPageBytes<D> / 1024;
  constexpr int NA = RT >= kWaves ? kWaves : RT;  // waves with row tiles
  // one LDS array (as in norm_kernel): ring, chunk list, the waves' key sums [2][kWaves][64]
  __shared__ __attribute__((aligned(1024))) char lds[kSlots * kWaves * kPageBytes<D> + 8 * kChunksPerWg +
                                                     2 * kWaves * kWaves * 16 * 4];
  char* const ring = lds;
  int* const ch = reinterpret_cast<int*>(lds + kSlots * kWaves * kPageBytes<D>);
  float* const red = reinterpret_cast<float*>(lds + kSlots * kWaves * kPageBytes<D> + 8 * kChunksPerWg);
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int C0 = blockIdx.x * kChunksPerWg;
  const int n = min(C0 + kChunksPerWg, p.n_lp) - C0;
  const int n_slots = (n + kWaves - 1) / kWaves;
  const bool act = wave < NA;
  stage_chunks(p, C0, C0 + n, ch);
  bf16x8 qf[TW][NF];
  load_q<D, TW>(p, h, 0, act ? wave * TW : 0, lane, qf);
  f32x4 l4[TW];  // log2 normalisers of rows 16 T + 4 (lane / 16) + i
#pragma unroll
  for (int t = 0; t < TW; ++t)
    l4[t] = *reinterpret_cast<const f32x4*>(p.lse2 + h * p.RP + 16 * ((act ? wave * TW : 0) + t) + 4 * (lane >> 4));
  const float c2 = p.c2;
  // slot j's key sums (one lane per key of the slot's pages) to the partials
  auto flush = [&](int j) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NA; ++w) v += red[((j & 1) * kWaves + w) * 64 + lane];
    const int c = kWaves * j + (lane >> 4);
    const int64_t t = (int64_t)(C0 + c) * 16 + (lane & 15);
    if (c < n && t < p.n_tok) p.partial[(size_t)h * p.n_tok + t] = v;
  };
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSlots - 1; ++j) ring_issue<D>(p, ch, h, j, n, wave, lane, ring);
  for (int j = 0; j < n_slots; ++j) {
    wait_vmcnt<(kSlots - 2) * LPW>();  // this wave's page of slot j landed ...
    ring_barrier();                    // ... and every wave's; slot j - 1 is consumed
    ring_issue<D>(p, ch, h, j + kSlots - 1, n, wave, lane, ring);
    if (wave == 0 && j > 0) flush(j - 1);
    if (!act) continue;
    bf16x8 kf[kWaves][NF];
    ring_frags<D>(ring, j, lane, kf);
    float s[kWaves];
#pragma unroll
    for (int pp = 0; pp < kWaves; ++pp) s[pp] = 0.f;
#pragma unroll
    for (int t = 0; t < TW; ++t) {
#pragma unroll
      for (int pp = 0; pp < kWaves; ++pp) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int f = 0; f < NF; ++f) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[t][f], kf[pp][f], acc, 0, 0, 0);
        // acc[i]: row 16 T + 4 (lane / 16) + i, key lane % 16 of page pp
#pragma unroll
        for (int i = 0; i < 4; ++i) s[pp] += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], c2, -l4[t][i]));
      }
    }
#pragma unroll
    for (int pp = 0; pp < kWaves; ++pp) {
      float v = s[pp] + __shfl_xor(s[pp], 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) red[((j & 1) * kWaves + wave) * 64 + pp * 16 + lane] = v;
    }
  }
  wait_vmcnt<0>();  // no load may land in LDS after the workgroup ends
  __syncthreads();
  if (wave == 0 && n_slots > 0) flush(n_slots - 1);
}

__global__ __launch_bounds__(256) void score_sum_kernel(const float* __restrict__ partial, float* __restrict__ scores,
                                                        int64_t n_tok, int hkv, float inv) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_tok) return;
  float s = 0.f;
  for (int h = 0; h < hkv; ++h) s += partial[(size_t)h * n_tok + t];
  scores[t] = s * inv;
}

// order-preserving image of a float (NaN lowest; -0 and +0 equal)
__device__ __forceinline__ uint32_t key_of(float x) {
  if (x != x) return 0u;
  const uint32_t b = __float_as_uint(x == 0.f ? 0.f : x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Radix select over many workgroups with no atomics or fences between them: digit pass
// k (one launch) writes every workgroup's 256-bin histogram of its slice as plain
// stores, and each workgroup of the next launch first sums those histograms itself to
// find digit k (all of them get the same answer; workgroup 0 also records it).
struct SelState {
  uint32_t prefix, remaining;  // after a digit: the key prefix and how many keys still to take
};
constexpr int kSelThreads = 1024;
constexpr int kSelMaxWg = 256;
constexpr int kSelPerWg = 4096;
constexpr int kSelUnroll = 4;  // keys a thread loads before it histograms them

struct SelWs {
  uint32_t* hist;  // [4][n_wg][256]
  SelState* st;    // [5]: st[k] after digit k - 1 (st[0] unused: the budget is an argument)
};

// digit k from the n_wg histograms of pass k under state `in`; returns the new state
__device__ SelState sel_digit(const uint32_t* __restrict__ hist, int n_wg, SelState in, int shift,
                              uint32_t* lds) {
  __shared__ SelState s_out;
  __shared__ uint32_t part[kSelThreads / 256][256];
  const int tid = threadIdx.x, lane = tid & 63, bin = tid & 255, q = tid >> 8;
  uint32_t c = 0;
  for (int w = q; w < n_wg; w += kSelThreads / 256) c += hist[(size_t)w * 256 + bin];
  part[q][bin] = c;
  __syncthreads();
  if (tid < 256) {
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kSelThreads / 256; ++j) sum += part[j][tid];
    lds[tid] = sum;
  }
  __syncthreads();
  if (tid < 64) {
    // lane l takes bins 255 - 4 l .. 252 - 4 l, so lanes run from the top bin down
    uint32_t v[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) local += (v[j] = lds[255 - 4 * lane - j]);
    uint32_t incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    const uint32_t excl = incl - local;
    if (excl < in.remaining && incl >= in.remaining) {
      uint32_t above = excl;
      int digit = 255 - 4 * lane;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above + v[j] >= in.remaining) {
          digit = 255 - 4 * lane - j;
          break;
        }
        above += v[j];
      }
      s_out = SelState{in.prefix | ((uint32_t)digit << shift), in.remaining - above};
    }
  }
  __syncthreads();
  return s_out;
}

// pass k (shift 24 - 8 k): histogram of digit k over the slice's keys matching the prefix
__global__ __launch_bounds__(kSelThreads) void sel_hist_kernel(const float* __restrict__ scores, int64_t n,
                                                              int64_t slice, SelWs ws, int n_wg, int k,
                                                              uint32_t budget) {
  __shared__ uint32_t hist[256];
  const int shift = 24 - 8 * k;
  SelState st{0u, budget};
  if (k > 0) {
    const SelState in = k == 1 ? st : ws.st[k - 1];
    st = sel_digit(ws.hist + (size_t)(k - 1) * n_wg * 256, n_wg, in, shift + 8, hist);
    if (blockIdx.x == 0 && threadIdx.x == 0) ws.st[k] = st;
  }
  const uint32_t mask = k == 0 ? 0u : ~0u << (shift + 8);
  __syncthreads();
  if (threadIdx.x < 256) hist[threadIdx.x] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.x * slice, t1 = min(t0 + slice, n);
  for (int64_t base = t0 + threadIdx.x; base < t1; base += kSelUnroll * kSelThreads) {
    float v[kSelUnroll];
#pragma unroll
    for (int j = 0; j < kSelUnroll; ++j) {
      const int64_t t = base + (int64_t)j * kSelThreads;
      v[j] = t < t1 ? scores[t] : __builtin_nanf("");
    }
#pragma unroll
    for (int j = 0; j < kSelUnroll; ++j) {
      const uint32_t u = key_of(v[j]);
      if (base + (int64_t)j * kSelThreads < t1 && (u & mask) == st.prefix) atomicAdd(&hist[(u >> shift) & 255], 1u);
    }
  }
  __syncthreads();
  if (threadIdx.x < 256) ws.hist[((size_t)k * n_wg + blockIdx.x) * 256 + threadIdx.x] = hist[threadIdx.x];
}

// the last digit, then: keep every key above the prefix and the first `remaining` keys
// equal to it in index order (a slice's ties start after those of the slices before
// it: its count of the last digit in the last pass)
__global__ __launch_bounds__(kSelThreads) void sel_write_kernel(const float* __restrict__ scores, int64_t n,
                                                               int64_t slice, SelWs ws, int n_wg,
                                                               uint8_t* __restrict__ keep) {
  __shared__ uint32_t lds[256];
  __shared__ uint32_t s_wave[kSelThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t* h3 = ws.hist + (size_t)3 * n_wg * 256;
  const SelState st = sel_digit(h3, n_wg, ws.st[3], 0, lds);
  if (blockIdx.x == 0 && tid == 0) ws.st[4] = st;
  const uint32_t prefix = st.prefix, remaining = st.remaining;
  uint32_t b = 0;
  for (int w = tid; w < (int)blockIdx.x; w += kSelThreads) b += h3[(size_t)w * 256 + (prefix & 255)];
  for (int off = 32; off > 0; off >>= 1) b += __shfl_xor(b, off);
  if (lane == 0) s_wave[wave] = b;
  __syncthreads();
  uint32_t carry = 0;
  for (int w = 0; w < kSelThreads / 64; ++w) carry += s_wave[w];
  const int64_t t0 = (int64_t)blockIdx.x * slice, t1 = min(t0 + slice, n);
  for (int64_t base = t0; base < t1; base += kSelThreads) {
    const int64_t t = base + tid;
    const uint32_t u = t < t1 ? key_of(scores[t]) : 0u;
    const bool tie = t < t1 && u == prefix;
    const uint64_t bal = __ballot(tie);
    const uint32_t before = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();  // every read of s_wave from the step before is done
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    uint32_t wave_base = carry;
    for (int w = 0; w < wave; ++w) wave_base += s_wave[w];
    if (t < t1) keep[t] = (u > prefix || (tie && wave_base + before < remaining)) ? 1 : 0;
    for (int w = 0; w < kSelThreads / 64; ++w) carry += s_wave[w];
  }
}

__global__ __launch_bounds__(256) void fill_kernel(uint8_t* __restrict__ keep, int64_t n, uint8_t v) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n) keep[t] = v;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct ScoreLayout {
  size_t chunks, part, lse2, partial, total;
};


// visible chunks of the sequence: own pages (lo 0, hi the page's fill), then mounted runs
static std::vector<int32_t> score_chunks(const Seq* S, int64_t PS) {
  std::vector<int32_t> c;
  c.reserve(2 * S->pages.size());
  for (size_t L = 0; L < S->pages.size(); ++L) {
    c.push_back(S->pages[L]);
    c.push_back((int32_t)std::min<int64_t>(PS, S->n - (int64_t)L * PS) << 8);
  }
  for (const Mount& m : S->mounts)
    for (size_t j = 0; j < m.pages.size(); ++j) {
      const int64_t a = std::max<int64_t>(0, m.off - (int64_t)j * PS);
      const int64_t b = std::min<int64_t>(PS, m.off + m.n - (int64_t)j * PS);
      if (a < b) {
        c.push_back(m.pages[j]);
        c.push_back((int32_t)(a | b << 8));
      }
    }
  return c;
}

// rows per KV head padded to 16 x a power of two (the normaliser's tile count)
static int32_t score_tiles(int32_t rows) {
  int32_t t = 1;
  while (16 * t < rows) t *= 2;
  return t;
}

static int score_layout(kv_pool_t* P, kv_seq_t seq, int32_t n_rep, int32_t hq, ScoreLayout* w, int64_t* n_tok,
                        int32_t* n_ch) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  const int32_t hkv = P->cfg.n_kv_heads;
  if (n_rep < 1 || hq < hkv || hq % hkv) FAIL(P, KV_ERR_INVALID, "bad representative query shape");
  if ((int64_t)n_rep * (hq / hkv) > kMaxScoreRows)
    FAIL(P, KV_ERR_UNSUPPORTED, "at most 256 representative rows (queries x query heads) per KV head");
  int64_t ch = (int64_t)S->pages.size();
  for (const Mount& m : S->mounts) ch += (int64_t)m.pages.size();
  if (ch > INT32_MAX / 2) FAIL(P, KV_ERR_INVALID, "too many visible pages");
  const int64_t RP = 16 * score_tiles(n_rep * (hq / hkv));
  const int64_t nx = (ch + kChunksPerWg - 1) / kChunksPerWg;
  w->chunks = 0;
  w->part = align256((size_t)ch * 8);
  w->lse2 = align256(w->part + (size_t)hkv * RP * 2 * std::max<int64_t>(nx, 1) * 4);
  w->partial = align256(w->lse2 + (size_t)hkv * RP * 4);
  w->total = w->partial + (size_t)hkv * S->n * 4;
  *n_tok = S->n;
  *n_ch = (int32_t)ch;  // an upper bound: mount pages outside the mounted run add no chunk
  return KV_OK;
}

template <int D>
static void launch_score(const ScoreParams& p, int RT, hipStream_t stream) {
  const dim3 ngrid(p.nx, p.hkv);
  switch (RT) {  // more than 8 tiles (128 rows) would spill: one launch per 128 rows
    case 1: norm_kernel<D, 1><<<ngrid, 256, 0, stream>>>(p, 0); break;
    case 2: norm_kernel<D, 2><<<ngrid, 256, 0, stream>>>(p, 0); break;
    case 4: norm_kernel<D, 4><<<ngrid, 256, 0, stream>>>(p, 0); break;
    default:
      for (int r0 = 0; r0 < 16 * RT; r0 += 128) norm_kernel<D, 8><<<ngrid, 256, 0, stream>>>(p, r0);
  }
  norm_merge_kernel<<<(p.hkv * p.RP + 3) / 4, 256, 0, stream>>>(p);
  const dim3 sgrid((p.n_lp + kChunksPerWg - 1) / kChunksPerWg, p.hkv);
  switch (RT) {
    case 1: score_kernel<D, 1><<<sgrid, 256, 0, stream>>>(p); break;
    case 2: score_kernel<D, 2><<<sgrid, 256, 0, stream>>>(p); break;
    case 4: score_kernel<D, 4><<<sgrid, 256, 0, stream>>>(p); break;
    case 8: score_kernel<D, 8><<<sgrid, 256, 0, stream>>>(p); break;
    default: score_kernel<D, 16><<<sgrid, 256, 0, stream>>>(p); break;
  }
}

}  // namespace

extern "C" {

int kv_score_workspace_size(kv_pool_t* P, kv_seq_t seq, int32_t n_rep, int32_t n_q_heads, size_t* bytes) {
  if (!bytes) FAIL(P, KV_ERR_INVALID, "null bytes");
  ScoreLayout w;
  int64_t n_tok;
  int32_t n_ch;
  if (int st = score_layout(P, seq, n_rep, n_q_heads, &w, &n_tok, &n_ch)) return st;
  *bytes = w.total;
  return KV_OK;
}

int kv_score(kv_pool_t* P, kv_seq_t seq, const void* q_rep, int32_t n_rep, int32_t n_q_heads, float sm_scale,
             float* scores, void* workspace, size_t ws_bytes, hipStream_t stream) {
  ScoreLayout w;
  int64_t n_tok;
  int32_t n_ch_max;
  if (int st = score_layout(P, seq, n_rep, n_q_heads, &w, &n_tok, &n_ch_max)) return st;
  if (!P->device) FAIL(P, KV_ERR_INVALID, "metadata-only pool has no KV data");
  if (P->cfg.dtype != KV_BF16 || (P->cfg.head_dim != 64 && P->cfg.head_dim != 128))
    FAIL(P, KV_ERR_UNSUPPORTED, "key scoring needs a bf16 pool with head_dim 64 or 128");
  if (!(sm_scale > 0.f)) FAIL(P, KV_ERR_INVALID, "softmax scale must be positive");
  if (!q_rep || !workspace || (n_tok > 0 && !scores)) FAIL(P, KV_ERR_INVALID, "null pointer");
  if (ws_bytes < w.total) FAIL(P, KV_ERR_WORKSPACE, "score workspace too small");
  if (n_tok == 0) return KV_OK;
  char* ws = static_cast<char*>(workspace);
  Seq* S = fa_seq(P, seq);
  auto& sc = P->score_chunks;  // the list is uploaded again only when the page table or workspace changed
  if (sc.version != P->version || sc.seq != seq || sc.ws != workspace) {
    const std::vector<int32_t> chunks = score_chunks(S, P->cfg.page_size);
    hipError_t e = fa_upload(P, ws + w.chunks, chunks.data(), chunks.size() * 4, stream);
    if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("score chunk upload: ") + hipGetErrorString(e));
    sc.version = P->version;
    sc.seq = seq;
    sc.ws = workspace;
    sc.n_ch = (int32_t)(chunks.size() / 2);
  }
  hipError_t e = hipSuccess;
  ScoreParams p;
  p.q = static_cast<const bf16_t*>(q_rep);
  p.k_pages = static_cast<const bf16_t*>(P->k);
  p.chunks = reinterpret_cast<const int32_t*>(ws + w.chunks);
  p.part = reinterpret_cast<float*>(ws + w.part);
  p.lse2 = reinterpret_cast<float*>(ws + w.lse2);
  p.partial = reinterpret_cast<float*>(ws + w.partial);
  p.n_rep = n_rep;
  p.hq = n_q_heads;
  p.hkv = P->cfg.n_kv_heads;
  p.G = n_q_heads / p.hkv;
  p.pool_pages = P->cfg.n_pages;
  p.n_ch = sc.n_ch;
  p.n_lp = (int32_t)S->pages.size();
  const int RT = score_tiles(n_rep * p.G);
  p.RP = 16 * RT;
  p.nx = (p.n_ch + kChunksPerWg - 1) / kChunksPerWg;
  p.n_tok = n_tok;
  p.c2 = sm_scale * 1.4426950408889634f;
  if (P->cfg.head_dim == 128)
    launch_score<128>(p, RT, stream);
  else
    launch_score<64>(p, RT, stream);
  score_sum_kernel<<<(unsigned)((n_tok + 255) / 256), 256, 0, stream>>>(p.partial, scores, n_tok, p.hkv,
                                                                         1.f / (float)(n_rep * n_q_heads));
  e = hipGetLastError();
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("score launch: ") + hipGetErrorString(e));
  return KV_OK;
}

static int64_t sel_slice(int64_t n, int32_t* n_wg) {
  const int64_t wg = std::max<int64_t>(1, std::min<int64_t>(kSelMaxWg, (n + kSelPerWg - 1) / kSelPerWg));
  const int64_t slice = ((n + wg - 1) / wg + kSelThreads - 1) / kSelThreads * kSelThreads;
  *n_wg = (int32_t)((n + slice - 1) / slice);
  return slice;
}

static size_t sel_ws_bytes(int32_t n_wg) { return 256 + (size_t)4 * n_wg * 256 * 4; }

int kv_select_workspace_size(int64_t n, size_t* bytes) {
  if (!bytes || n < 0) return fa_set_err(nullptr, KV_ERR_INVALID, "bad select size query");
  int32_t n_wg = 1;
  if (n > 0) sel_slice(n, &n_wg);
  *bytes = sel_ws_bytes(n_wg);
  return KV_OK;
}

int kv_select_keep(const float* scores, int64_t n, int64_t budget, uint8_t* keep, void* workspace, size_t ws_bytes,
                   hipStream_t stream) {
  if (n < 0) return fa_set_err(nullptr, KV_ERR_INVALID, "negative count");
  if (n > INT32_MAX) return fa_set_err(nullptr, KV_ERR_UNSUPPORTED, "at most 2^31 - 1 scores");
  if (n == 0) return KV_OK;
  if (!scores || !keep) return fa_set_err(nullptr, KV_ERR_INVALID, "null pointer");
  if (budget <= 0 || budget >= n) {
    fill_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(keep, n, budget <= 0 ? 0 : 1);
  } else {
    int32_t n_wg;
    const int64_t slice = sel_slice(n, &n_wg);
    if (!workspace) return fa_set_err(nullptr, KV_ERR_INVALID, "null workspace");
    if (ws_bytes < sel_ws_bytes(n_wg)) return fa_set_err(nullptr, KV_ERR_WORKSPACE, "select workspace too small");
    SelWs w;
    w.st = static_cast<SelState*>(workspace);
    w.hist = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + 256);
    for (int k = 0; k < 4; ++k)
      sel_hist_kernel<<<n_wg, kSelThreads, 0, stream>>>(scores, n, slice, w, n_wg, k, (uint32_t)budget);
    sel_write_kernel<<<n_wg, kSelThreads, 0, stream>>>(scores, n, slice, w, n_wg, keep);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_err(nullptr, KV_ERR_HIP, std::string("select launch: ") + hipGetErrorString(e));
  return KV_OK;
}

int kv_drop_keep(kv_pool_t* P, kv_seq_t seq, const uint8_t* keep, int64_t n, int32_t flags, hipStream_t stream) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  if (n != S->n || (n > 0 && !keep)) FAIL(P, KV_ERR_INVALID, "keep mask must cover every own token");
  std::vector<int64_t> begin, len;
  for (int64_t t = 0; t < n;) {
    if (keep[t]) {
      ++t;
      continue;
    }
    const int64_t a = t;
    while (t < n && !keep[t]) ++t;
    begin.push_back(a);
    len.push_back(t - a);
  }
  if (begin.size() > (size_t)INT32_MAX) FAIL(P, KV_ERR_INVALID, "too many spans");
  return kv_drop(P, seq, begin.data(), len.data(), (int32_t)begin.size(), flags, nullptr, stream);
}

}  // extern "C"
