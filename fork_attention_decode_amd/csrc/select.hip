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
// context.  Two passes over the keys:
//   1. the normalisers: the decode path (fork_attn_decode) over the representative
//      queries gives each (query, head) its log-sum-exp over the whole visible context;
//   2. score_kernel streams each own page's K block once per KV head and computes
//      S = Q K^T for all of the head's rows (query x head-of-group) on
//      v_mfma_f32_16x16x32_bf16 with the keys as N: each lane then holds one key, so the
//      sum over rows of exp2(S c2 - lse2) stays in the lane plus two shuffles.
// select_kernel: one workgroup, radix select of the budget-th largest score on an
// order-preserving integer image of the floats (4 passes of 8 bits), then ties kept in
// index order through a block-wide scan.
#include <hip/hip_runtime.h>
#include <math.h>
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
constexpr int kPagesPerWg = 16;

struct ScoreParams {
  const bf16_t* q;        // [n_rep][hq][D] representative queries (rotated)
  const float* lse;       // [n_rep][hq] natural-log normalisers over the visible context
  const bf16_t* k_pages;  // pool K, head-major blocks
  const int32_t* pages;   // own logical page -> page id [n_lp]
  float* partial;         // [hkv][n_tok] per-KV-head sums over that head's rows
  int32_t n_rep, hq, hkv, G, pool_pages, n_lp;
  int64_t n_tok;
  float c2;  // sm_scale * log2(e)
};

// grid (ceil(n_lp / kPagesPerWg), hkv); rows of KV head h: r = rep * G + g (query head
// h * G + g), padded with zero queries and +inf normalisers to whole 16-row tiles
template <int D>
__global__ __launch_bounds__(256) void score_kernel(ScoreParams p) {
  constexpr int NF = D / 32;  // 32-dim k-steps
  __shared__ __attribute__((aligned(16))) char qa[kMaxScoreRows * D * 2];  // A fragments [tile][f][lane]
  __shared__ __attribute__((aligned(16))) float lse2[kMaxScoreRows];
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int R = p.n_rep * p.G;
  const int RT = (R + 15) / 16;
  // stage Q in operand order: unit (row r, f, g) = Q[r][32 f + 8 g .. + 8] at lane r % 16 + 16 g
  for (int u = threadIdx.x; u < RT * 16 * NF * 4; u += 256) {
    const int g = u & 3, f = (u >> 2) % NF, r = (u >> 2) / NF;
    i32x4 val = {0, 0, 0, 0};
    if (r < R) {
      const int rep = r / p.G, qh = h * p.G + r % p.G;
      val = *reinterpret_cast<const i32x4*>(p.q + ((size_t)rep * p.hq + qh) * D + 32 * f + 8 * g);
    }
    *reinterpret_cast<i32x4*>(qa + (((r >> 4) * NF + f) * 64 + (r & 15) + 16 * g) * 16) = val;
  }
  for (int r = threadIdx.x; r < RT * 16; r += 256) {
    float v = INFINITY;  // padding rows and rows without visible keys add nothing
    if (r < R) {
      const float l = p.lse[(size_t)(r / p.G) * p.hq + h * p.G + r % p.G];
      if (l > -INFINITY) v = l * 1.4426950408889634f;
    }
    lse2[r] = v;
  }
  __syncthreads();

  const int L0 = blockIdx.x * kPagesPerWg;
  const int L1 = min(L0 + kPagesPerWg, p.n_lp);
  for (int L = L0 + wave; L < L1; L += 4) {
    const bf16_t* blk = p.k_pages + ((size_t)h * p.pool_pages + p.pages[L]) * 16 * D;
    bf16x8 kf[NF];  // B operand: lane t + 16 g holds K[t][32 f + 8 g .. + 8]
#pragma unroll
    for (int f = 0; f < NF; ++f)
      kf[f] = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(blk + (f * 64 + lane) * 8)));
    float s = 0.f;
    for (int T = 0; T < RT; ++T) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(qa + ((T * NF + f) * 64 + lane) * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, kf[f], acc, 0, 0, 0);
      }
      // acc[i]: row 16 T + 4 (lane / 16) + i, key lane % 16
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + 16 * T + 4 * (lane >> 4));
#pragma unroll
      for (int i = 0; i < 4; ++i) s += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[i], p.c2, -l4[i]));
    }
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    const int64_t t = (int64_t)L * 16 + lane;
    if (lane < 16 && t < p.n_tok) p.partial[(size_t)h * p.n_tok + t] = s;
  }
}

__global__ __launch_bounds__(256) void score_sum_kernel(const float* __restrict__ partial, float* __restrict__ scores,
                                                        int64_t n_tok, int hkv, float inv) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n_tok) return;
  float s = 0.f;
  for (int h = 0; h < hkv; ++h) s += partial[(size_t)h * n_tok + t];
  scores[t] = s * inv;
}

// order-preserving image of a float (NaN lowest)
__device__ __forceinline__ uint32_t key_of(float x) {
  if (x != x) return 0u;
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// one workgroup of 1024 threads; 1 <= budget < n
__global__ __launch_bounds__(1024) void select_kernel(const float* __restrict__ scores, int64_t n, int64_t budget,
                                                      uint8_t* __restrict__ keep) {
  __shared__ int64_t hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int64_t s_remaining;
  __shared__ int64_t s_wave[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0, mask = 0;
  int64_t remaining = budget;  // still to take among the keys that match prefix under mask
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += 1024) hist[b] = 0;
    __syncthreads();
    for (int64_t t = tid; t < n; t += 1024) {
      const uint32_t u = key_of(scores[t]);
      if ((u & mask) == prefix) atomicAdd((unsigned long long*)&hist[(u >> shift) & 255], 1ull);
    }
    __syncthreads();
    if (tid == 0) {
      int64_t above = 0;
      int digit = 0;
      for (int b = 255; b >= 0; --b) {
        if (above + hist[b] >= remaining) {
          digit = b;
          break;
        }
        above += hist[b];
      }
      s_prefix = prefix | ((uint32_t)digit << shift);
      s_remaining = remaining - above;
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= 255u << shift;
  }
  // prefix is the budget-th largest key; keep every larger key and the first `remaining`
  // keys equal to it in index order
  int64_t carry = 0;
  for (int64_t base = 0; base < n; base += 1024) {
    const int64_t t = base + tid;
    const uint32_t u = t < n ? key_of(scores[t]) : 0u;
    const bool tie = t < n && u == prefix;
    const uint64_t bal = __ballot(tie);
    const int64_t before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    int64_t wave_base = carry;
    for (int w = 0; w < wave; ++w) wave_base += s_wave[w];
    if (t < n) keep[t] = (u > prefix || (tie && wave_base + before < remaining)) ? 1 : 0;
    int64_t total = 0;
    for (int w = 0; w < 16; ++w) total += s_wave[w];
    carry += total;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void fill_kernel(uint8_t* __restrict__ keep, int64_t n, uint8_t v) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < n) keep[t] = v;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct ScoreLayout {
  size_t dec, out, lse, pages, partial, total;
};

}  // namespace

extern "C" {

static int score_layout(kv_pool_t* P, kv_seq_t seq, int32_t n_rep, int32_t hq, ScoreLayout* w, int64_t* n_tok,
                        int32_t* n_lp) {
  if (!P) FAIL(P, KV_ERR_INVALID, "null pool");
  Seq* S = fa_seq(P, seq);
  if (!S) FAIL(P, KV_ERR_NOT_FOUND, "no live sequence");
  const int32_t hkv = P->cfg.n_kv_heads;
  if (n_rep < 1 || hq < hkv || hq % hkv) FAIL(P, KV_ERR_INVALID, "bad representative query shape");
  if (n_rep * (hq / hkv) > kMaxScoreRows)
    FAIL(P, KV_ERR_UNSUPPORTED, "at most 256 representative rows (queries x query heads) per KV head");
  std::vector<kv_seq_t> seqs((size_t)n_rep, seq);
  size_t dec = 0;
  if (int st = fork_attn_workspace_size(P, seqs.data(), n_rep, hq, &dec)) return st;
  const size_t es = P->cfg.dtype == KV_F32 ? 4 : 2;
  w->dec = 0;
  w->out = align256(dec);
  w->lse = align256(w->out + (size_t)n_rep * hq * P->cfg.head_dim * es);
  w->pages = align256(w->lse + (size_t)n_rep * hq * 4);
  w->partial = align256(w->pages + S->pages.size() * 4);
  w->total = w->partial + (size_t)hkv * S->n * 4;
  *n_tok = S->n;
  *n_lp = (int32_t)S->pages.size();
  return KV_OK;
}

int kv_score_workspace_size(kv_pool_t* P, kv_seq_t seq, int32_t n_rep, int32_t n_q_heads, size_t* bytes) {
  if (!bytes) FAIL(P, KV_ERR_INVALID, "null bytes");
  ScoreLayout w;
  int64_t n_tok;
  int32_t n_lp;
  if (int st = score_layout(P, seq, n_rep, n_q_heads, &w, &n_tok, &n_lp)) return st;
  *bytes = w.total;
  return KV_OK;
}

int kv_score(kv_pool_t* P, kv_seq_t seq, const void* q_rep, int32_t n_rep, int32_t n_q_heads, float sm_scale,
             float* scores, void* workspace, size_t ws_bytes, hipStream_t stream) {
  ScoreLayout w;
  int64_t n_tok;
  int32_t n_lp;
  if (int st = score_layout(P, seq, n_rep, n_q_heads, &w, &n_tok, &n_lp)) return st;
  if (!P->device) FAIL(P, KV_ERR_INVALID, "metadata-only pool has no KV data");
  if (P->cfg.dtype != KV_BF16 || (P->cfg.head_dim != 64 && P->cfg.head_dim != 128))
    FAIL(P, KV_ERR_UNSUPPORTED, "key scoring needs a bf16 pool with head_dim 64 or 128");
  if (!(sm_scale > 0.f)) FAIL(P, KV_ERR_INVALID, "softmax scale must be positive");
  if (!q_rep || !workspace || (n_tok > 0 && !scores)) FAIL(P, KV_ERR_INVALID, "null pointer");
  if (ws_bytes < w.total) FAIL(P, KV_ERR_WORKSPACE, "score workspace too small");
  if (n_tok == 0) return KV_OK;
  char* ws = static_cast<char*>(workspace);
  float* lse = reinterpret_cast<float*>(ws + w.lse);
  std::vector<kv_seq_t> seqs((size_t)n_rep, seq);
  if (int st = fork_attn_decode(P, seqs.data(), n_rep, n_q_heads, q_rep, ws + w.out, lse, sm_scale, ws + w.dec,
                                w.out - w.dec, stream))
    return st;
  Seq* S = fa_seq(P, seq);
  hipError_t e = fa_upload(P, ws + w.pages, S->pages.data(), (size_t)n_lp * 4, stream);
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("score page upload: ") + hipGetErrorString(e));
  ScoreParams p;
  p.q = static_cast<const bf16_t*>(q_rep);
  p.lse = lse;
  p.k_pages = static_cast<const bf16_t*>(P->k);
  p.pages = reinterpret_cast<const int32_t*>(ws + w.pages);
  p.partial = reinterpret_cast<float*>(ws + w.partial);
  p.n_rep = n_rep;
  p.hq = n_q_heads;
  p.hkv = P->cfg.n_kv_heads;
  p.G = n_q_heads / p.hkv;
  p.pool_pages = P->cfg.n_pages;
  p.n_lp = n_lp;
  p.n_tok = n_tok;
  p.c2 = sm_scale * 1.4426950408889634f;
  const dim3 grid((n_lp + kPagesPerWg - 1) / kPagesPerWg, p.hkv);
  if (P->cfg.head_dim == 128)
    score_kernel<128><<<grid, 256, 0, stream>>>(p);
  else
    score_kernel<64><<<grid, 256, 0, stream>>>(p);
  score_sum_kernel<<<(unsigned)((n_tok + 255) / 256), 256, 0, stream>>>(p.partial, scores, n_tok, p.hkv,
                                                                         1.f / (float)(n_rep * n_q_heads));
  e = hipGetLastError();
  if (e != hipSuccess) FAIL(P, KV_ERR_HIP, std::string("score launch: ") + hipGetErrorString(e));
  return KV_OK;
}

int kv_select_keep(const float* scores, int64_t n, int64_t budget, uint8_t* keep, hipStream_t stream) {
  if (n < 0) return fa_set_err(nullptr, KV_ERR_INVALID, "negative count");
  if (n == 0) return KV_OK;
  if (!scores || !keep) return fa_set_err(nullptr, KV_ERR_INVALID, "null pointer");
  if (budget <= 0 || budget >= n)
    fill_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(keep, n, budget <= 0 ? 0 : 1);
  else
    select_kernel<<<1, 1024, 0, stream>>>(scores, n, budget, keep);
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
