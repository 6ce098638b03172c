// Split-K shared-prefix decode and log-sum-exp merge for gfx950 (CDNA4).
//
// Agentrix ForkAttention (gitlink.org.cn README, section "前缀复用与 ForkAttention"
// and the CUDA ForkAttention item): the pages a group of branches share are read once
// and reused by all of their queries; each branch's partial results are merged.
//
// Mapping onto CDNA4:
//   * a work item = (segment of pages with one reader set, KV head, chunk range);
//     its rows are every (reader, query head of this KV head) pair, up to 64;
//   * one workgroup of 4 waves per item; the waves take the item's chunks round robin,
//     each streaming whole 4 KiB K and V^T page blocks with contiguous 16 B / 8 B
//     per-lane loads straight into matrix-core operand registers (the pool layout is
//     operand-ordered, so no LDS staging is needed), PF chunks in flight per wave;
//   * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (keys = M, query rows = N, d = K), whose
//     accumulator layout is exactly the B-operand layout of O^T = V^T P^T on
//     v_mfma_f32_16x16x16_bf16: no transposes; row statistics live with the lane's
//     query row (lane % 16), the row max over a page needs two permlane swaps;
//   * online softmax in fp32 (exp2 domain); the 4 waves merge their states through
//     LDS and write one normalised partial (lse2, o) per row;
//   * the merge kernel combines a row's partials by log-sum-exp.
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
  __device__ static KF load_k(const bf16_t* blk, int f, int lane) {
    return *reinterpret_cast<const KF*>(blk + (f * 64 + lane) * 8);
  }
  __device__ static VF load_v(const bf16_t* blk, int db, int lane) {
    return *reinterpret_cast<const VF*>(blk + (db * 16 + (lane & 15)) * 16 + 4 * (lane >> 4));
  }
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
  __device__ static f32x4 pv(f32x4 c, VF v, PF p) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v, p, c, 0, 0, 0);
  }
};

template <int D> struct Tr<float, D> {
  static constexpr int NF = D / 16;
  static constexpr int NDB = D / 16;
  using KF = f32x4;
  using VF = f32x4;
  using PF = f32x4;
  __device__ static KF load_k(const float* blk, int f, int lane) {
    return *reinterpret_cast<const KF*>(blk + (f * 64 + lane) * 4);
  }
  __device__ static VF load_v(const float* blk, int db, int lane) {
    return *reinterpret_cast<const VF*>(blk + (db * 16 + (lane & 15)) * 16 + 4 * (lane >> 4));
  }
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

template <typename T, int D, int RB, int PFD>
__device__ __forceinline__ void decode_item(const DecodeParams& p, const DecodeItem& it, int wave,
                                            int lane, float* lds) {
  using TR = Tr<T, D>;
  constexpr int NF = TR::NF;
  constexpr int NDB = TR::NDB;
  const int c16 = lane & 15;
  const int g = lane >> 4;
  const int G = p.group;

  // ---- query fragments (B operand of S^T = K Q^T), one per row block and d slot
  typename TR::KF qf[RB][NF];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + c16;
    if (r < it.n_rows) {
      const int reader = p.readers[it.reader_begin + r / G];
      const int head = it.kv_head * G + r % G;
      const T* row = reinterpret_cast<const T*>(p.q) + ((size_t)reader * p.n_q_heads + head) * D;
#pragma unroll
      for (int f = 0; f < NF; ++f) qf[rb][f] = TR::load_q(row, f, lane);
    } else {
#pragma unroll
      for (int f = 0; f < NF; ++f) qf[rb][f] = TR::zero_q();
    }
  }

  // ---- this wave's chunks: item chunks wave, wave + 4, ...; lane j holds chunk j's metadata
  const int n_my = it.n_chunks > wave ? (it.n_chunks - wave + kWaves - 1) / kWaves : 0;
  int meta_page = 0, meta_lohi = 16 << 8;
  if (lane < n_my) {
    const Chunk c = p.chunks[it.chunk_begin + wave + kWaves * lane];
    meta_page = c.page;
    meta_lohi = c.lohi;
  }

  f32x4 o[RB][NDB];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = -INFINITY;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t page_elems = (size_t)p.n_kv_heads * kPage * D;
  const T* kbase = reinterpret_cast<const T*>(p.k_pages) + (size_t)it.kv_head * kPage * D;
  const T* vbase = reinterpret_cast<const T*>(p.v_pages) + (size_t)it.kv_head * kPage * D;

  typename TR::KF kb[PFD][NF];
  typename TR::VF vb[PFD][NDB];

  auto issue = [&](int s, int j) {
    const int jj = j < n_my ? j : n_my - 1;  // past the end: reload the last chunk (cache hit)
    const int page = __builtin_amdgcn_readlane(meta_page, jj);
    const T* kblk = kbase + (size_t)page * page_elems;
    const T* vblk = vbase + (size_t)page * page_elems;
#pragma unroll
    for (int f = 0; f < NF; ++f) kb[s][f] = TR::load_k(kblk, f, lane);
#pragma unroll
    for (int db = 0; db < NDB; ++db) vb[s][db] = TR::load_v(vblk, db, lane);
  };

  if (n_my > 0) {
#pragma unroll
    for (int s = 0; s < PFD; ++s) issue(s, s);
  }

  for (int base = 0; base < n_my; base += PFD) {
#pragma unroll
    for (int s = 0; s < PFD; ++s) {
      const int j = base + s;
      if (j < n_my) {
        const int lohi = __builtin_amdgcn_readlane(meta_lohi, j);
        const bool full = lohi == (16 << 8);
        const int lo = lohi & 0xff, hi = lohi >> 8;
        typename TR::VF vv[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) vv[db] = full ? vb[s][db] : TR::mask_v(vb[s][db], g, lo, hi);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int f = 0; f < NF; ++f) sc = TR::qk(sc, kb[s][f], qf[rb][f]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sc[i] *= p.scale_log2;
            if (!full) {
              const int t = 4 * g + i;
              if (t < lo || t >= hi) sc[i] = -INFINITY;
            }
          }
          const float mx = row_max4(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
          const float mn = fmaxf(m[rb], mx);
          const float alpha = fast_exp2(m[rb] - mn);
          f32x4 pr;
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(sc[i] - mn);
          l[rb] = l[rb] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
          m[rb] = mn;
          const typename TR::PF pp = TR::pack(pr);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            o[rb][db] *= alpha;
            o[rb][db] = TR::pv(o[rb][db], vv[db], pp);
          }
        }
        issue(s, j + PFD);
      }
    }
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) l[rb] = row_sum4(l[rb]);

  // ---- merge the 4 waves' states in LDS (deterministic order 1, 2, 3 into wave 0)
  float* lm = lds;                 // [RB * 16] row max (log2 domain)
  float* ll = lds + RB * 16;       // [RB * 16] row sum
  float* lo_ = lds + RB * 32;      // [RB * NDB * 4][64] accumulators in register order
  for (int w = 1; w < kWaves; ++w) {
    __syncthreads();
    if (wave == w) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (g == 0) {
          lm[rb * 16 + c16] = m[rb];
          ll[rb * 16 + c16] = l[rb];
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) lo_[((rb * NDB + db) * 4 + i) * 64 + lane] = o[rb][db][i];
      }
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float mw = lm[rb * 16 + c16];
        const float lw = ll[rb * 16 + c16];
        const float mn = fmaxf(m[rb], mw);
        const float a = mn == -INFINITY ? 0.f : fast_exp2(m[rb] - mn);
        const float b = mn == -INFINITY ? 0.f : fast_exp2(mw - mn);
        l[rb] = l[rb] * a + lw * b;
        m[rb] = mn;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            o[rb][db][i] = o[rb][db][i] * a + lo_[((rb * NDB + db) * 4 + i) * 64 + lane] * b;
      }
    }
  }

  if (wave == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = rb * 16 + c16;
      if (r < it.n_rows) {
        const int slot = it.partial_base + r;
        const float inv = 1.f / l[rb];
        float* dst = p.part_o + (size_t)slot * D + 4 * g;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          f32x4 v = o[rb][db] * inv;
          *reinterpret_cast<f32x4*>(dst + 16 * db) = v;
        }
        if (g == 0) p.part_lse2[slot] = m[rb] + __log2f(l[rb]);
      }
    }
  }
}

template <typename T, int D>
constexpr int lds_floats() { return 4 * 32 + 4 * Tr<T, D>::NDB * 4 * 64; }

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void decode_kernel(DecodeParams p) {
  __shared__ float lds[lds_floats<T, D>()];
  const DecodeItem it = p.items[blockIdx.x];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (it.row_blocks == 1) decode_item<T, D, 1, 4>(p, it, wave, lane, lds);
  else if (it.row_blocks == 2) decode_item<T, D, 2, 4>(p, it, wave, lane, lds);
  else decode_item<T, D, 4, 3>(p, it, wave, lane, lds);
}

template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }
template <> __device__ inline float from_f32<float>(float x) { return x; }

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= p.n_rows) return;
  constexpr int V = D / 64;
  const int b = p.row_ptr[row], e = p.row_ptr[row + 1];
  float M = -INFINITY;
  for (int j = b; j < e; ++j) M = fmaxf(M, p.part_lse2[p.part_idx[j]]);
  float acc[V];
#pragma unroll
  for (int v = 0; v < V; ++v) acc[v] = 0.f;
  float S = 0.f;
  for (int j = b; j < e; ++j) {
    const int idx = p.part_idx[j];
    const float w = fast_exp2(p.part_lse2[idx] - M);
    S += w;
    const float* src = p.part_o + (size_t)idx * D + lane * V;
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] += w * src[v];
  }
  T* out = reinterpret_cast<T*>(p.out) + (size_t)row * D + lane * V;
  const float inv = S > 0.f ? 1.f / S : 0.f;
#pragma unroll
  for (int v = 0; v < V; ++v) out[v] = from_f32<T>(acc[v] * inv);
  if (p.lse && lane == 0) p.lse[row] = S > 0.f ? (M + __log2f(S)) * 0.69314718055994531f : -INFINITY;
}

// ---------------------------------------------------------------- page writes (append)
// Block (page, head): K slot (f, g, t) -> 16 bytes; V^T row d -> 16 tokens.
template <typename T, int D>
__global__ __launch_bounds__(256) void page_write_kernel(T* __restrict__ kp, T* __restrict__ vp,
                                                         const T* __restrict__ kn,
                                                         const T* __restrict__ vn,
                                                         const PageWrite* __restrict__ writes,
                                                         int hkv) {
  constexpr int E = 16 / sizeof(T);           // elements per 16-byte slot
  constexpr int NSLOT = kPage * D / E;        // 16-byte slots per block
  const PageWrite w = writes[blockIdx.x];
  const int h = blockIdx.y;
  const size_t blk = ((size_t)w.dst_page * hkv + h) * kPage * D;
  const size_t sblk = w.src_page >= 0 ? ((size_t)w.src_page * hkv + h) * kPage * D : 0;
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
  // V^T: row d holds 16 tokens = 16 * sizeof(T) bytes = sizeof(T) slots of E tokens
  constexpr int PPR = sizeof(T);
  for (int pc = threadIdx.x; pc < D * PPR; pc += blockDim.x) {
    const int d = pc / PPR, t0 = (pc % PPR) * E;
    if (w.src_page < 0 && (t0 + E <= w.lo || t0 >= w.hi)) continue;
    vec_t val = *reinterpret_cast<const vec_t*>((w.src_page >= 0 ? vp + sblk : vp + blk) + (size_t)d * 16 + t0);
    for (int e = 0; e < E; ++e) {
      const int t = t0 + e;
      if (t >= w.lo && t < w.hi) val[e] = vn[((size_t)(w.tok_base + (t - w.lo)) * hkv + h) * D + d];
    }
    *reinterpret_cast<vec_t*>(vp + blk + (size_t)d * 16 + t0) = val;
  }
}

// ---------------------------------------------------------------- launchers
template <typename T, int D>
static hipError_t decode_t(const DecodeParams& p, hipStream_t s) {
  if (p.n_items == 0) return hipSuccess;
  decode_kernel<T, D><<<p.n_items, 256, 0, s>>>(p);
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
  merge_kernel<T, D><<<(p.n_rows + 3) / 4, 256, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, int d, const MergeParams& p, hipStream_t s) {
  if (dtype == 0 && d == 128) return merge_t<bf16_t, 128>(p, s);
  if (dtype == 0 && d == 64) return merge_t<bf16_t, 64>(p, s);
  if (dtype == 1 && d == 128) return merge_t<float, 128>(p, s);
  if (dtype == 1 && d == 64) return merge_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

template <typename T, int D>
static hipError_t page_write_t(int hkv, void* kp, void* vp, const void* kn, const void* vn,
                               const PageWrite* w, int n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  dim3 grid(n, hkv);
  page_write_kernel<T, D><<<grid, 256, 0, s>>>((T*)kp, (T*)vp, (const T*)kn, (const T*)vn, w, hkv);
  return hipGetLastError();
}

hipError_t launch_page_write(int dtype, int d, int hkv, void* kp, void* vp, const void* kn,
                             const void* vn, const PageWrite* w, int n, hipStream_t s) {
  if (dtype == 0 && d == 128) return page_write_t<bf16_t, 128>(hkv, kp, vp, kn, vn, w, n, s);
  if (dtype == 0 && d == 64) return page_write_t<bf16_t, 64>(hkv, kp, vp, kn, vn, w, n, s);
  if (dtype == 1 && d == 128) return page_write_t<float, 128>(hkv, kp, vp, kn, vn, w, n, s);
  if (dtype == 1 && d == 64) return page_write_t<float, 64>(hkv, kp, vp, kn, vn, w, n, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
