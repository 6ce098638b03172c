// Fused Drop compaction + Repos re-rotation for gfx950.
//
// AKV (news.farwalk.ai), "AKV 如何工作": Drop removes entries from future attention;
// Repos rewrites the kept keys to positions 0..r-1 by a rotary rotation and leaves the
// values unchanged.  AgentKV (rit.work): kept entries are compacted physically and the
// freed pages go back to the allocator.
//
// One workgroup per batch of kCompactBatch consecutive destination pages (all KV heads),
// taken in order.  Phase 1 gathers the page's kept
// tokens from their old slots into an LDS image of the destination page, rotating each
// key pair (i, i + d/2) by the token's offset with fp32 cos/sin rows computed on the
// host in fp64 (an fp32 angle at 131K positions would be off by ~1e-2 rad); values are
// copied bit-exactly.  Phase 2 writes the image back with contiguous 16-byte stores.
//
// In-place hazard: kept tokens only move to lower slots, so a page rewritten in place
// may still be a source of lower destination pages (at most two: a source page's kept
// tokens are consecutive).  Workgroups take list entries in start order (an atomic
// ticket), publish "sources read" with a release store after phase 1, and a page
// rewritten in place waits (acquire) for exactly the lower entries that read it.  A
// workgroup only ever waits for entries started before it, all of which are resident
// and never wait for it, so every wait ends.
#include <hip/hip_runtime.h>
#include "plan.hpp"

namespace fa {

typedef __bf16 bf16_t;

template <typename T> __device__ inline float to_f(T x) { return (float)x; }
template <typename T> __device__ inline T from_f(float x) { return (T)x; }

template <typename T, int D>
__global__ __launch_bounds__(256) void compact_kernel(CompactParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  constexpr int E = 16 / sizeof(T);                 // elements per 16-byte slot
  constexpr int NF = D * (int)sizeof(T) / 64;       // K slots per token row and lane group
  constexpr int HALF = NF / 2;                      // slot f pairs with f + HALF (d, d + D/2)
  constexpr int BLK = 16 * D;                       // elements per (page, head) block
  typedef T vec_t __attribute__((__vector_size__(16)));
  const int hkv = p.n_kv_heads;
  T* lk = reinterpret_cast<T*>(lds_raw);
  T* lv = lk + (size_t)hkv * BLK;
  __shared__ int s_b;
  __shared__ int s_loc[16], s_rot[16];
  if (threadIdx.x == 0) s_b = (int)((unsigned)atomicAdd(p.ticket, 1) - (unsigned)p.ticket_base);
  __syncthreads();
  const int b = s_b;
  if (b < 0 || b * kCompactBatch >= p.n_pages) {  // ticket out of step with the host: count it, touch nothing
    if (threadIdx.x == 0) atomicAdd(p.errors, 1);
    return;
  }
  T* kp = reinterpret_cast<T*>(p.k_pages);
  T* vp = reinterpret_cast<T*>(p.v_pages);
  const size_t np = (size_t)p.pool_pages;  // head-major pool: block (page, h) at h * np + page
  const int k_end = min((b + 1) * kCompactBatch, p.n_pages);
  for (int k = b * kCompactBatch; k < k_end; ++k) {  // this batch's list entries, in order
    const CompactPage cp = p.pages[k];
    const size_t dst = (size_t)cp.dst_page * BLK;
    const bool keep_rest = cp.first_slot > 0 || cp.n_slots < 16;
    // the page's 16 source locations and rotation rows, once, so that every gather below
    // issues its loads independently instead of behind a dependent index load
    if (threadIdx.x < 16) {
      const int t = threadIdx.x;
      const bool mine = t >= cp.first_slot && t < cp.n_slots;
      s_loc[t] = mine ? p.src_loc[cp.tok_base + t] : -1;
      s_rot[t] = mine ? p.rot[cp.tok_base + t] : -1;
    }
    __syncthreads();

    // ---- phase 1: gather K (with rotation) into the LDS image
    const int n_ku = hkv * HALF * 64;
    for (int u = threadIdx.x; u < n_ku; u += blockDim.x) {
      const int t = u & 15, g = (u >> 4) & 3, fp = (u >> 6) % HALF, h = (u >> 6) / HALF;
      const int s0 = ((fp * 4 + g) * 16 + t) * E, s1 = (((fp + HALF) * 4 + g) * 16 + t) * E;
      vec_t a, bb;
      const int loc = s_loc[t];
      if (loc >= 0) {
        const size_t sb = ((size_t)h * np + (loc >> 4)) * BLK;
        const int st = loc & 15;
        a = *reinterpret_cast<const vec_t*>(kp + sb + ((fp * 4 + g) * 16 + st) * E);
        bb = *reinterpret_cast<const vec_t*>(kp + sb + (((fp + HALF) * 4 + g) * 16 + st) * E);
        const int run = s_rot[t];
        if (run >= 0) {
          const float* cs = p.cos_sin + (size_t)run * D;  // [D/2][2]
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const int d = sizeof(T) == 2 ? 32 * fp + 8 * g + e : 16 * fp + 4 * e + g;
            const float c = cs[2 * d], sn = cs[2 * d + 1];
            const float x = to_f(a[e]), y = to_f(bb[e]);
            a[e] = from_f<T>(x * c - y * sn);
            bb[e] = from_f<T>(y * c + x * sn);
          }
        }
      } else if (keep_rest) {
        a = *reinterpret_cast<const vec_t*>(kp + dst + (size_t)h * np * BLK + s0);
        bb = *reinterpret_cast<const vec_t*>(kp + dst + (size_t)h * np * BLK + s1);
      } else {
        continue;
      }
      *reinterpret_cast<vec_t*>(lk + h * BLK + s0) = a;
      *reinterpret_cast<vec_t*>(lk + h * BLK + s1) = bb;
    }
    // ---- phase 1: gather V^T rows (bit-exact copies)
    for (int r = threadIdx.x; r < hkv * D; r += blockDim.x) {
      const int h = r / D, d = r % D;
      vec_t row[16 / E];
      if (keep_rest) {
#pragma unroll
        for (int i = 0; i < 16 / E; ++i)
          row[i] = *reinterpret_cast<const vec_t*>(vp + dst + (size_t)h * np * BLK + d * 16 + i * E);
      }
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int loc = s_loc[t];
        if (loc >= 0) row[t / E][t % E] = vp[((size_t)h * np + (loc >> 4)) * BLK + d * 16 + (loc & 15)];
      }
#pragma unroll
      for (int i = 0; i < 16 / E; ++i) *reinterpret_cast<vec_t*>(lv + h * BLK + d * 16 + i * E) = row[i];
    }
    __syncthreads();

    // ---- publish "sources read", then wait for the lower entries that read this page
    // (earlier entries of this batch published theirs already).  The hazard is
    // write-after-read only: a reader publishes after its loads have returned (their
    // values are in LDS behind the barrier above) and a writer's stores issue only after
    // its poll has seen the flag, so relaxed device-scope atomics order it; acquire /
    // release would write back or invalidate this die's L2 on every poll.
    if (threadIdx.x == 0) {
      __hip_atomic_store(&p.done[k], p.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int i = cp.wait_lo; i < cp.wait_hi && i < k; ++i) {
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

    // ---- phase 2: write the image back, one contiguous block per head
    constexpr int VPB = BLK / E;  // 16-byte vectors per block
    const int n_vec = hkv * VPB;
    const vec_t* ik = reinterpret_cast<const vec_t*>(lk);
    const vec_t* iv = reinterpret_cast<const vec_t*>(lv);
    for (int i = threadIdx.x; i < n_vec; i += blockDim.x) {
      const size_t at = ((size_t)(i / VPB) * np + cp.dst_page) * BLK + (size_t)(i % VPB) * E;
      *reinterpret_cast<vec_t*>(kp + at) = ik[i];
      *reinterpret_cast<vec_t*>(vp + at) = iv[i];
    }
    __syncthreads();  // the image is rebuilt for the next entry
  }
}

size_t compact_lds_bytes(int dtype, int d, int hkv) {
  return (size_t)2 * hkv * 16 * d * (dtype == 1 ? 4 : 2);
}

template <typename T, int D>
static hipError_t compact_t(const CompactParams& p, hipStream_t s) {
  if (p.n_pages == 0) return hipSuccess;
  const size_t lds = compact_lds_bytes(sizeof(T) == 4 ? 1 : 0, D, p.n_kv_heads);
  hipError_t e = hipFuncSetAttribute((const void*)compact_kernel<T, D>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  compact_kernel<T, D><<<(p.n_pages + kCompactBatch - 1) / kCompactBatch, 256, lds, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_compact(int dtype, int d, const CompactParams& p, hipStream_t s) {
  if (dtype == 0 && d == 128) return compact_t<bf16_t, 128>(p, s);
  if (dtype == 0 && d == 64) return compact_t<bf16_t, 64>(p, s);
  if (dtype == 1 && d == 128) return compact_t<float, 128>(p, s);
  if (dtype == 1 && d == 64) return compact_t<float, 64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace fa
