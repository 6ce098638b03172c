// Split-K shared-prefix decode with a fused log-sum-exp merge, for gfx950 (CDNA4).
//
// Agentrix ForkAttention (gitlink.org.cn README, section "前缀复用与 ForkAttention"
// and the CUDA ForkAttention item): the pages a group of branches share are read once
// and reused by all of their queries; each branch's partial results are merged.
//
// Mapping onto CDNA4:
//   * a work item = (segment of pages with one reader set, KV head, chunk range); its
//     rows are every (reader, query head of this KV head) pair, up to 64;
//   * one workgroup of 4 waves per item streams every chunk (a 4 KiB K block and a
//     4 KiB V^T block of one page and head) from HBM exactly once, with buffer loads
//     straight into an LDS ring (each wave loads a quarter, non-temporal), six
//     chunks in flight; wave w computes rows [16 w, 16 w + 16) from LDS, so a shared
//     page feeds all 64 rows with one HBM read;
//   * chunks are consumed in pairs (32 keys): S^T = K Q^T on v_mfma_f32_16x16x32_bf16
//     (keys = M, query rows = N, d = K) lands exactly in the B-operand layout of
//     O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 with the two chunks' keys interleaved
//     along K: no transposes; row statistics live with the lane's query row;
//   * online softmax in fp32 (exp2 domain) with a lazy, wave-uniform rescale;
//   * each item writes one normalised partial (lse2, o) per row into slots ordered by
//     output row, so a row's partials are contiguous; a second launch merges them (a
//     kernel boundary is the cheapest device-wide synchronisation across the chip's
//     separately cached dies).
// fp32 pools use v_mfma_f32_16x16x4_f32 with the same structure.
#include <hip/hip_runtime.h>
#include <math.h>
#include "plan.hpp"

namespace fa {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((__vector_size__(8 * sizeof(bf16_t))));
typedef bf16_t bf16x4 __attribute__((__vector_size__(4 * sizeof(bf16_t))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

template <typename T, int D> struct Tr;

template <int D> struct Tr<bf16_t, D> {
  static constexpr int NF = D / 32;   // 16-byte K slots per lane per page block
  static constexpr int NDB = D / 16;  // 16-wide d blocks of V^T / O^T
  using KF = bf16x8;
  using VF = bf16x4;
  using PF = bf16x4;
  __device__ static KF load_q(const bf16_t* row, int f, int lane) {
    return *reinterpret_cast<const KF*>(row + 32 * f + 8 * (lane >> 4));
  }
  __device__ static KF zero_q() { KF z; for (int i = 0; i < 8; ++i) z[i] = (bf16_t)0.0f; return z; }
  __device__ static f32x4 qk(f32x4 c, KF k, KF q) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(k, q, c, 0, 0, 0);
  }
  __device__ static PF pack(f32x4 p) {
    PF r;
    r[0] = (bf16_t)p[0]; r[1] = (bf16_t)p[1]; r[2] = (bf16_t)p[2]; r[3] = (bf16_t)p[3];
    return r;
  }
  __device__ static VF mask_v(VF v, int g, int lo, int hi) {
    for (int e = 0; e < 4; ++e) {
      int t = 4 * g + e;
      if (t < lo || t >= hi) v[e] = (bf16_t)0.0f;
    }
    return v;
  }
  // two chunks at once: K index 8 g + e is key 4 g + e of chunk e / 4
  __device__ static f32x4 pv2(f32x4 c, VF v0, VF v1, PF p0, PF p1) {
    const KF a = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    const KF b = __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <int D> struct Tr<float, D> {
  static constexpr int NF = D / 16;
  static constexpr int NDB = D / 16;
  using KF = f32x4;
  using VF = f32x4;
  using PF = f32x4;
  __device__ static KF load_q(const float* row, int f, int lane) {
    const int g = lane >> 4;
    KF r;
    for (int e = 0; e < 4; ++e) r[e] = row[16 * f + 4 * e + g];
    return r;
  }
  __device__ static KF zero_q() { KF z = {0.f, 0.f, 0.f, 0.f}; return z; }
  __device__ static f32x4 qk(f32x4 c, KF k, KF q) {
    for (int e = 0; e < 4; ++e) c = __builtin_amdgcn_mfma_f32_16x16x4f32(k[e], q[e], c, 0, 0, 0);
    return c;
  }
  __device__ static PF pack(f32x4 p) { return p; }
  __device__ static VF mask_v(VF v, int g, int lo, int hi) {
    for (int e = 0; e < 4; ++e) {
      int t = 4 * g + e;
      if (t < lo || t >= hi) v[e] = 0.f;
    }
    return v;
  }
  __device__ static f32x4 pv(f32x4 c, VF v, PF p) {
    for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_16x16x4f32(v[i], p[i], c, 0, 0, 0);
    return c;
  }
  __device__ static f32x4 pv2(f32x4 c, VF v0, VF v1, PF p0, PF p1) { return pv(pv(c, v0, p0), v1, p1); }
};

// max / sum over the four lanes {l, l^16, l^32, l^48} that hold one query row
__device__ inline float row_max4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float row_sum4(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kCachePolicyNT = 2;  // non-temporal cache policy bit of the ring loads
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units): p <= 256

// Q fragments of this lane's query row (B operand of S^T = K Q^T); zero past n_rows.
template <typename T, int D>
__device__ __forceinline__ void load_q_row(const DecodeParams& p, int orow, int lane,
                                           typename Tr<T, D>::KF (&qf)[Tr<T, D>::NF]) {
  using TR = Tr<T, D>;
  if (orow >= 0) {
    const T* row = reinterpret_cast<const T*>(p.q) + (size_t)orow * D;
#pragma unroll
    for (int f = 0; f < TR::NF; ++f) qf[f] = TR::load_q(row, f, lane);
  } else {
#pragma unroll
    for (int f = 0; f < TR::NF; ++f) qf[f] = TR::zero_q();
  }
}

// Scores of one chunk for one 16-row block, scaled to log2 units, slots outside
// [lo, hi) masked to -inf (their values zeroed so 0 * garbage cannot appear).
template <typename T, int D>
__device__ __forceinline__ f32x4 chunk_scores(const typename Tr<T, D>::KF (&kf)[Tr<T, D>::NF],
                                              typename Tr<T, D>::VF (&vf)[Tr<T, D>::NDB],
                                              const typename Tr<T, D>::KF (&qf)[Tr<T, D>::NF], int lohi, int g,
                                              float scale_log2) {
  using TR = Tr<T, D>;
  f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int f = 0; f < TR::NF; ++f) sc = TR::qk(sc, kf[f], qf[f]);
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] *= scale_log2;
  if (lohi != (16 << 8)) {  // wave-uniform
    const int lo = lohi & 0xff, hi = lohi >> 8;
#pragma unroll
    for (int db = 0; db < TR::NDB; ++db) vf[db] = TR::mask_v(vf[db], g, lo, hi);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 4 * g + i;
      if (t < lo || t >= hi) sc[i] = -INFINITY;
    }
  }
  return sc;
}

// Online-softmax update of one 16-row block with two chunks (32 keys).
template <typename T, int D>
__device__ __forceinline__ void softmax_pair(const typename Tr<T, D>::KF (&k0)[Tr<T, D>::NF],
                                             typename Tr<T, D>::VF (&v0)[Tr<T, D>::NDB],
                                             const typename Tr<T, D>::KF (&k1)[Tr<T, D>::NF],
                                             typename Tr<T, D>::VF (&v1)[Tr<T, D>::NDB],
                                             const typename Tr<T, D>::KF (&qf)[Tr<T, D>::NF],
                                             f32x4 (&o)[Tr<T, D>::NDB], float& m, float& l, int lohi0, int lohi1,
                                             int g, float scale_log2) {
  using TR = Tr<T, D>;
  const f32x4 s0 = chunk_scores<T, D>(k0, v0, qf, lohi0, g, scale_log2);
  const f32x4 s1 = chunk_scores<T, D>(k1, v1, qf, lohi1, g, scale_log2);
  // Lazy rescale: the running max m only moves when some row's max exceeds it by
  // more than kTau (log2 units), so p = 2^(s - m) stays below 2^kTau and the O
  // rescale (a multiply of every accumulator) is skipped for most pairs.  The branch
  // is wave-uniform (ballot).
  const float lmx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                          fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
  if (__builtin_amdgcn_ballot_w64(lmx > m + kTau)) {
    const float mn = fmaxf(m, row_max4(lmx));
    const float alpha = fast_exp2(m - mn);
    l *= alpha;
    m = mn;
#pragma unroll
    for (int db = 0; db < TR::NDB; ++db) o[db] *= alpha;
  }
  f32x4 p0, p1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p0[i] = fast_exp2(s0[i] - m);
    p1[i] = fast_exp2(s1[i] - m);
  }
  l += ((p0[0] + p0[1]) + (p0[2] + p0[3])) + ((p1[0] + p1[1]) + (p1[2] + p1[3]));
  const typename TR::PF q0 = TR::pack(p0), q1 = TR::pack(p1);
#pragma unroll
  for (int db = 0; db < TR::NDB; ++db) o[db] = TR::pv2(o[db], v0[db], v1[db], q0, q1);
}

// LDS ring slots of one chunk each (K block + V^T block): about kRingBytes, even, >= 4.
template <typename T, int D>
constexpr int ring_slots() {
  constexpr int cb = 2 * kPage * D * (int)sizeof(T);
  constexpr int nb = (kRingBytes / cb) & ~1;
  return nb < 4 ? 4 : nb;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---- one work item: every chunk streamed from HBM once per workgroup into an LDS ring
// with buffer loads straight into LDS (each wave loads a quarter of every chunk); wave w
// computes rows [16 w, 16 w + 16) from LDS, two chunks per step; NB - 2 chunks stay in
// flight; one workgroup barrier per step.
template <typename T, int D, int kPolicy>
__device__ __forceinline__ void decode_item(const DecodeParams& p, const int32_t* __restrict__ rec, int wave,
                                            int lane, char* ring) {
  using TR = Tr<T, D>;
  constexpr int NF = TR::NF;
  constexpr int NDB = TR::NDB;
  constexpr int HALF = kPage * D * (int)sizeof(T);  // bytes of one K (or V^T) block
  constexpr int CB = 2 * HALF;                        // bytes of one chunk in the ring
  constexpr int NB = ring_slots<T, D>();              // ring slots (even)
  constexpr int LPW = CB / 1024 / kWaves;             // 1 KiB loads per wave per chunk
  static_assert(LPW >= 1 && NB >= 4 && NB % 2 == 0, "ring shape");
  const int c16 = lane & 15, g = lane >> 4;
  // one round of independent loads: header (scalar), chunk metadata (lane j holds
  // chunks j and 64 + j) and this lane's row; the record is fixed size, so every
  // address is in bounds and entries past the counts are simply never used
  const int n = rec[0];
  const int kv_head = rec[1];
  const bool active = wave * 16 < rec[2];
  const int2 c0 = reinterpret_cast<const int2*>(rec + kRecChunk)[lane];
  const int2 c1 = reinterpret_cast<const int2*>(rec + kRecChunk)[64 + lane];
  const int mp0 = c0.x, mp1 = c1.x;
  int ml0 = c0.y, ml1 = c1.y;
  // a decode window: a reserved page's range ends at this step's length.  The table loads
  // are issued before the ring's and applied after them, so they land during its fill
  // (entries past the count are stale and never read)
  // Both paths issue the same two loads (outside a window, of the record's first int), so
  // the ring's first loads never wait for them.
  const bool cut0 = p.cut_hi && lane < n && (ml0 >> 16), cut1 = p.cut_hi && 64 + lane < n && (ml1 >> 16);
  const int32_t* tab = p.cut_hi ? p.cut_hi : rec;  // a window's table holds at least one entry
  const int cv0 = tab[cut0 ? (ml0 >> 16) - 1 : 0];
  const int cv1 = tab[cut1 ? (ml1 >> 16) - 1 : 0];
  const int orow = rec[kRecRow + wave * 16 + c16];
  const int slot = rec[kRecSlot + wave * 16 + c16];

  // head-major pool: head h's blocks are contiguous, page q at h * n_pages + q
  const char* kbase = reinterpret_cast<const char*>(p.k_pages) + (size_t)kv_head * p.n_pages * HALF;
  const char* vbase = reinterpret_cast<const char*>(p.v_pages) + (size_t)kv_head * p.n_pages * HALF;
  const int my_off = wave * (CB / kWaves);  // this wave's byte range of every chunk
  const char* my_base = my_off < HALF ? kbase + my_off : vbase + (my_off - HALF);

  auto issue = [&](int j) {
    const int jj = j < n ? j : n - 1;  // past the end: reload the last chunk into an unread slot
    const int page = jj < 64 ? __builtin_amdgcn_readlane(mp0, jj) : __builtin_amdgcn_readlane(mp1, jj - 64);
    // a buffer descriptor over this wave's share of the page: the hardware drops any
    // load outside it, and unlike the flat-encoded global form, buffer loads leave the
    // compiler's LDS wait counts exact (it has to assume a flat load may touch LDS out
    // of order and would wait for every outstanding LDS read)
    const __amdgpu_buffer_rsrc_t src =
        __builtin_amdgcn_make_buffer_rsrc((void*)(my_base + (size_t)page * HALF), 0, LPW * 1024, 0x00020000);
    char* dst = ring + (j % NB) * CB + my_off;
#pragma unroll
    for (int i = 0; i < LPW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16,
                                               lane * 16 + i * 1024, 0, 0, kPolicy);
  };
  auto lohi_of = [&](int j) {
    if (j >= n) return 0;  // empty slot range: every key masked
    return j < 64 ? __builtin_amdgcn_readlane(ml0, j) : __builtin_amdgcn_readlane(ml1, j - 64);
  };
  auto frags = [&](int j, typename TR::KF (&kf)[NF], typename TR::VF (&vf)[NDB]) {
    const char* slot = ring + (j % NB) * CB;
#pragma unroll
    for (int f = 0; f < NF; ++f) kf[f] = *reinterpret_cast<const typename TR::KF*>(slot + f * 1024 + lane * 16);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vf[db] = *reinterpret_cast<const typename TR::VF*>(slot + HALF + ((db * 16 + c16) * 16 + v_pos(4 * g)) * (int)sizeof(T));
  };

  f32x4 o[NDB];
  float m = -1e30f, l = 0.f;  // finite: an item whose slot ranges are all empty stays (m, 0)
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int j = 0; j < NB - 2; ++j) issue(j);
  typename TR::KF qf[NF];  // queries load while the ring fills
  load_q_row<T, D>(p, orow, lane, qf);
  auto cut = [](int lh, int e) {
    const int lo = lh & 0xff, hi = (lh >> 8) & 0xff;
    e = min(hi, max(lo, e));
    return e > lo ? (lo | e << 8) : 0;
  };
  if (cut0) ml0 = cut(ml0, cv0);
  if (cut1) ml1 = cut(ml1, cv1);

  const int n_pairs = (n + 1) / 2;
  for (int i = 0; i < n_pairs; ++i) {
    wait_vmcnt<(NB - 4) * LPW>();            // this wave's quarters of chunks 2i, 2i+1 landed
    asm volatile("s_barrier" ::: "memory");  // ... and every other wave's; the previous pair's slots are free
    issue(2 * i + NB - 2);
    issue(2 * i + NB - 1);
    if (active) {
      typename TR::KF k0[NF], k1[NF];
      typename TR::VF v0[NDB], v1[NDB];
      frags(2 * i, k0, v0);
      frags(2 * i + 1, k1, v1);
      softmax_pair<T, D>(k0, v0, k1, v1, qf, o, m, l, lohi_of(2 * i), lohi_of(2 * i + 1), g, p.scale_log2);
    }
  }
  wait_vmcnt<0>();  // no load may land in LDS after the workgroup ends
  if (active) {
    l = row_sum4(l);
    if (orow >= 0) {
      const float inv = l > 0.f ? 1.f / l : 0.f;  // an item with no visible key leaves (0, -inf)
      float* dst = p.part_o + (size_t)slot * D + 4 * g;
#pragma unroll
      for (int db = 0; db < NDB; ++db) *reinterpret_cast<f32x4*>(dst + 16 * db) = o[db] * inv;
      if (g == 0) p.part_lse2[slot] = m + __log2f(l);
    }
  }
}

template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }
template <> __device__ inline float from_f32<float>(float x) { return x; }

__device__ inline float wave_max(float x) {
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ inline float wave_sum(float x) {
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// ---- merge: two waves per output row, one per half of the head dimension (so a
// decode's few hundred rows still cover every compute unit).  The row's partials sit at
// the fixed-stride block [row * max_parts, ...), so the count, the lse values (one per
// lane) and the partial half-rows (16-byte loads, 512 / d partials per load instruction)
// are all fetched in one round trip; slots past the count are masked with selects,
// never multiplied in.  Both waves of a row compute the same weights.
constexpr int kMergeSplit = 2;
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int DW = D / kMergeSplit;  // dims per wave
  constexpr int LPR = DW / 4;          // lanes per partial half-row
  constexpr int PPI = 64 / LPR;        // partials per load instruction
  constexpr int NL = 64 / PPI;         // load instructions per 64 partials
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWaves + wave;
  const int row = gw / kMergeSplit, half = gw % kMergeSplit;
  if (row >= p.n_rows) return;
  const int sub = lane / LPR, col = lane % LPR;
  const int d0 = half * DW;  // this wave's dims [d0, d0 + DW)
  const int maxp = p.max_parts;
  const size_t base = (size_t)row * maxp;
  const int cnt = p.count[row];
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY, S = 0.f;
  if (maxp <= 64) {
    const float my_lse = lane < maxp ? p.part_lse2[base + lane] : -INFINITY;
    f4 v[NL];
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      const int j = k * PPI + sub;
      v[k] = j < maxp ? *reinterpret_cast<const f4*>(p.part_o + (base + j) * D + d0 + 4 * col) : f4{0.f, 0.f, 0.f, 0.f};
    }
    M = wave_max(lane < cnt ? my_lse : -INFINITY);
    const float my_w = lane < cnt ? fast_exp2(my_lse - M) : 0.f;
    S = wave_sum(my_w);
#pragma unroll
    for (int k = 0; k < NL; ++k) {
      float w = 0.f;
#pragma unroll
      for (int q = 0; q < PPI; ++q) {
        const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), k * PPI + q));
        w = sub == q ? wq : w;
      }
      const int j = k * PPI + sub;
      acc = j < cnt ? acc + w * v[k] : acc;
    }
  } else {
    for (int j0 = 0; j0 < cnt; j0 += 64)
      M = fmaxf(M, j0 + lane < cnt ? p.part_lse2[base + j0 + lane] : -INFINITY);
    M = wave_max(M);
    for (int j0 = 0; j0 < cnt; j0 += 64) {
      const float my_w = j0 + lane < cnt ? fast_exp2(p.part_lse2[base + j0 + lane] - M) : 0.f;
      S += wave_sum(my_w);
      for (int k = 0; k < NL; ++k) {
        float w = 0.f;
        for (int q = 0; q < PPI; ++q) {
          const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), k * PPI + q));
          w = sub == q ? wq : w;
        }
        const int j = j0 + k * PPI + sub;
        if (j < cnt) acc += w * *reinterpret_cast<const f4*>(p.part_o + (base + j) * D + d0 + 4 * col);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= LPR; off >>= 1)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[c] += __shfl_xor(acc[c], off);
  const float inv = S > 0.f ? 1.f / S : 0.f;
  if (sub == 0) {
    T* out = reinterpret_cast<T*>(p.out) + (size_t)row * D + d0 + 4 * col;
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = from_f32<T>(acc[c] * inv);
  }
  if (p.lse && half == 0 && lane == 0) p.lse[row] = S > 0.f ? (M + __log2f(S)) * 0.69314718055994531f : -INFINITY;
}

// ---- merge of few partials per row (a split-K prefill's key pieces): one thread per
// (row, 4 dims), so a launch over tens of thousands of rows issues a few instructions per
// partial instead of a wave-wide reduction per row.  The row's lse values are read by each
// of its threads (the same addresses, served once per wave).
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_few_kernel(MergeParams p) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int TPR = D / 4;  // threads per row
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int row = (int)(gid / TPR), c = (int)(gid % TPR);
  if (row >= p.n_rows) return;
  const int cnt = p.count[row];
  const size_t base = (size_t)row * p.max_parts;
  float M = -INFINITY;
  for (int j = 0; j < cnt; ++j) M = fmaxf(M, p.part_lse2[base + j]);
  f4 acc = {0.f, 0.f, 0.f, 0.f};
  float S = 0.f;
  if (M > -INFINITY) {
    for (int j = 0; j < cnt; ++j) {
      const float w = fast_exp2(p.part_lse2[base + j] - M);
      S += w;
      acc += w * *reinterpret_cast<const f4*>(p.part_o + (base + j) * D + 4 * c);
    }
  }
  const float inv = S > 0.f ? 1.f / S : 0.f;
  T* out = reinterpret_cast<T*>(p.out) + (size_t)row * D + 4 * c;
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = from_f32<T>(acc[k] * inv);
  if (p.lse && c == 0) p.lse[row] = S > 0.f ? (M + __log2f(S)) * 0.69314718055994531f : -INFINITY;
}

// kPolicy: kCachePolicyNT for a single pass over the pages; 0 (cached) where the same
// pages are streamed again by other items of the launch
template <typename T, int D, int kPolicy>
__global__ __launch_bounds__(256, 2) void decode_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(16))) char lds[ring_slots<T, D>() * 2 * kPage * D * sizeof(T)];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int it = blockIdx.x;
  decode_item<T, D, kPolicy>(p, p.items + (size_t)it * kRecInts, wave, lane, lds);
}

// ---------------------------------------------------------------- page writes (append)
// Block (page, head): K slot (f, g, t) -> 16 bytes; V^T row d -> 16 tokens.
template <typename T, int D>
__global__ __launch_bounds__(256) void page_write_kernel(T* __restrict__ kp, T* __restrict__ vp,
                                                         const T* __restrict__ kn,
                                                         const T* __restrict__ vn,
                                                         const PageWrite* __restrict__ writes,
                                                         int hkv, int pool_pages) {
  constexpr int E = 16 / sizeof(T);           // elements per 16-byte slot
  constexpr int NSLOT = kPage * D / E;        // 16-byte slots per block
  const PageWrite w = writes[blockIdx.x];
  const int h = blockIdx.y;
  const size_t blk = ((size_t)h * pool_pages + w.dst_page) * kPage * D;
  const size_t sblk = w.src_page >= 0 ? ((size_t)h * pool_pages + w.src_page) * kPage * D : 0;
  typedef T vec_t __attribute__((__vector_size__(16)));
  for (int sn = threadIdx.x; sn < NSLOT; sn += blockDim.x) {
    const int t = sn & 15, fg = sn >> 4, f = fg >> 2, g = fg & 3;
    vec_t val;
    if (t >= w.lo && t < w.hi) {
      const T* src = kn + ((size_t)(w.tok_base + (t - w.lo)) * hkv + h) * D;
      for (int e = 0; e < E; ++e) {
        const int d = (sizeof(T) == 2) ? 32 * f + 8 * g + e : 16 * f + 4 * e + g;
        val[e] = src[d];
      }
    } else if (w.src_page >= 0) {
      val = *reinterpret_cast<const vec_t*>(kp + sblk + (size_t)sn * E);
    } else {
      continue;
    }
    *reinterpret_cast<vec_t*>(kp + blk + (size_t)sn * E) = val;
  }
  // V^T: row d holds 16 tokens = 16 * sizeof(T) bytes = sizeof(T) pieces of E positions;
  // position q holds slot v_pos(q)
  constexpr int PPR = sizeof(T);
  for (int pc = threadIdx.x; pc < D * PPR; pc += blockDim.x) {
    const int d = pc / PPR, q0 = (pc % PPR) * E;
    bool any = w.src_page >= 0;
    for (int e = 0; e < E; ++e) any = any || (v_pos(q0 + e) >= w.lo && v_pos(q0 + e) < w.hi);
    if (!any) continue;
    vec_t val = *reinterpret_cast<const vec_t*>((w.src_page >= 0 ? vp + sblk : vp + blk) + (size_t)d * 16 + q0);
    for (int e = 0; e < E; ++e) {
      const int t = v_pos(q0 + e);
      if (t >= w.lo && t < w.hi) val[e] = vn[((size_t)(w.tok_base + (t - w.lo)) * hkv + h) * D + d];
    }
    *reinterpret_cast<vec_t*>(vp + blk + (size_t)d * 16 + q0) = val;
  }
}

// ---------------------------------------------------------------- plan patches
__global__ __launch_bounds__(256) void plan_patch_kernel(int32_t* __restrict__ ws, const int32_t* __restrict__ patches,
                                                         int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) ws[patches[2 * i]] = patches[2 * i + 1];
}

hipError_t launch_plan_patch(void* ws, const int32_t* patches, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  plan_patch_kernel<<<(n + 255) / 256, 256, 0, s>>>(static_cast<int32_t*>(ws), patches, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers
template <typename T, int D>
static hipError_t decode_t(const DecodeParams& p, hipStream_t s) {
  if (p.n_items == 0) return hipSuccess;
  if (p.cached)
    decode_kernel<T, D, 0><<<p.n_items, 256, 0, s>>>(p);
  else
    decode_kernel<T, D, kCachePolicyNT><<<p.n_items, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_decode(int dtype, int d, const DecodeParams& p, hipStream_t s) {
  if (dtype == 0 && d == 128) return decode_t<bf16_t, 128>(p, s);
  if (dtype == 0 && d == 64) return decode_t<bf16_t, 64>(p, s);
  if (dtype == 1 && d == 128) return decode_t<float, 128>(p, s);
  if (dtype == 1 && d == 64) return decode_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t merge_t(const MergeParams& p, hipStream_t s) {
  if (p.n_rows == 0) return hipSuccess;
  merge_kernel<T, D><<<(p.n_rows * kMergeSplit + kWaves - 1) / kWaves, 256, 0, s>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t merge_few_t(const MergeParams& p, hipStream_t s) {
  if (p.n_rows == 0) return hipSuccess;
  const int64_t threads = (int64_t)p.n_rows * (D / 4);
  merge_few_kernel<T, D><<<(unsigned)((threads + 255) / 256), 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_merge_few(int dtype, int d, const MergeParams& p, hipStream_t s) {
  if (dtype == 0 && d == 128) return merge_few_t<bf16_t, 128>(p, s);
  if (dtype == 0 && d == 64) return merge_few_t<bf16_t, 64>(p, s);
  if (dtype == 1 && d == 128) return merge_few_t<float, 128>(p, s);
  if (dtype == 1 && d == 64) return merge_few_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

hipError_t launch_merge(int dtype, int d, const MergeParams& p, hipStream_t s) {
  if (dtype == 0 && d == 128) return merge_t<bf16_t, 128>(p, s);
  if (dtype == 0 && d == 64) return merge_t<bf16_t, 64>(p, s);
  if (dtype == 1 && d == 128) return merge_t<float, 128>(p, s);
  if (dtype == 1 && d == 64) return merge_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t page_write_t(int hkv, int pool_pages, void* kp, void* vp, const void* kn, const void* vn,
                               const PageWrite* w, int n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  dim3 grid(n, hkv);
  page_write_kernel<T, D><<<grid, 256, 0, s>>>((T*)kp, (T*)vp, (const T*)kn, (const T*)vn, w, hkv, pool_pages);
  return hipGetLastError();
}

hipError_t launch_page_write(int dtype, int d, int hkv, int pool_pages, void* kp, void* vp, const void* kn,
                             const void* vn, const PageWrite* w, int n, hipStream_t s) {
  if (dtype == 0 && d == 128) return page_write_t<bf16_t, 128>(hkv, pool_pages, kp, vp, kn, vn, w, n, s);
  if (dtype == 0 && d == 64) return page_write_t<bf16_t, 64>(hkv, pool_pages, kp, vp, kn, vn, w, n, s);
  if (dtype == 1 && d == 128) return page_write_t<float, 128>(hkv, pool_pages, kp, vp, kn, vn, w, n, s);
  if (dtype == 1 && d == 64) return page_write_t<float, 64>(hkv, pool_pages, kp, vp, kn, vn, w, n, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
