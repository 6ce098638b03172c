// Packed DAG prefill: block-sparse attention forward over a DAG block mask, for gfx950.
//
// Octopus (zicq.com), "Packed DAG-GRPO": the branches of a rollout are packed into one
// sequence and one block-sparse matrix encodes causality inside a thread, cross-thread
// read edges and synchronisation dependencies, so only the block pairs the DAG allows
// are computed.  The CSR over 64 x 64 blocks comes from dag_mask_build; kind 1 marks a
// diagonal block (key <= query inside it), kind 0 a fully visible block.
//
// Mapping onto CDNA4:
//   * relayout pass: K and V of every (KV head, 64-key block) are copied once into a
//     16 KiB image in matrix-core operand order (zero past T), so each operand read in
//     the main kernel is one contiguous 1 KiB wave read from LDS (no bank conflicts)
//     and each block moves into LDS as two contiguous 16 KiB copies;
//   * one workgroup per (64-token query block, KV head, group of 4 query heads): 8
//     waves, two per query head with 32 queries each (GQA packing), so every K / V
//     block staged in LDS feeds 256 query rows;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (keys = M, queries = N, d = K): each lane
//     holds one query column, so row max / sum stay in the lane plus one permlane32
//     swap; its accumulator layout is the B operand of O^T = V^T P^T once the key
//     order of the V image matches it (done in the relayout), so P needs no shuffles;
//   * online softmax in fp32 in the exp2 domain with a lazy, wave-uniform rescale;
//   * K / V blocks stream through a 4-stage LDS ring with buffer loads straight into
//     LDS (each wave copies an eighth), one workgroup barrier per block;
//   * on MI355X the kernel runs at the chip's power limit (the shader clock settles
//     near 1.9 GHz), so its time follows energy: LDS bytes and vector instructions per
//     FLOP count for more than the issue schedule.  32 query rows per wave with two
//     waves per SIMD is the register budget's best point; 64 rows per wave halves LDS
//     reads but leaves one wave per SIMD, which cannot hide its own softmax latency;
//   * workgroups are ordered by descending row cost (a rank pass over row_ptr) so the
//     longest rows start first, and consecutive workgroups take consecutive KV heads,
//     so with 8 KV heads each die (and its L2) serves one head.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string>
#include "../../include/forkattn.h"
#include "plan.hpp"

int fa_set_err(struct kv_pool* P, int code, const std::string& m);

namespace fa {
namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((__vector_size__(8 * sizeof(bf16_t))));
typedef bf16_t bf16x4 __attribute__((__vector_size__(4 * sizeof(bf16_t))));
typedef bf16_t bf16x2 __attribute__((__vector_size__(2 * sizeof(bf16_t))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kB = 64;               // block edge (tokens)
constexpr int kD = 128;              // head dim
constexpr int kImg = kB * kD * 2;    // bytes of one K (or V) block image
constexpr int kStage = 2 * kImg;     // K image + V image
constexpr int kStages = 4;           // LDS ring depth: blocks j (V), j + 1 (K), j + 2 and j + 3 in flight
constexpr int kWaves = 8;            // waves per workgroup (two per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kLoadsPerWave = kStage / kWaves / 1024;  // 1 KiB wave loads per stage per wave
constexpr float kTau = 8.f;          // lazy rescale threshold (log2 units)

struct Params {
  const bf16_t* q;
  const char* kimg;
  const char* vimg;
  bf16_t* out;
  float* lse;
  int32_t T, hq, hkv, G, n_hg, nb;
  float scale_log2, sm_scale;
  // query rows: row r of q / out is the query at key index q_off + r, r < nq; a query
  // at index i sees key t unless i < t < n_own (causal inside [0, n_own); keys from
  // n_own on are visible to every query).  The packed prefill: q_off = 0, nq = n_own = T.
  int32_t q_off, nq, n_own;
  // split mode: CSR row r covers query block r / n_split, key range piece r % n_split;
  // partial (lse2, normalised o) of (query row, head, piece) at slot
  // (row * hq + head) * n_split + piece
  int32_t n_split;
  float* part_lse2;
  float* part_o;
  // K gathered from the pool (restore of a pool sequence): head h's K blocks at
  // kpool + (h * pool_pages + page) * 4 KiB; keys 16 g .. 16 g + 15 of the context are
  // slots 0..15 of page gpages[g] (the kernel's gpages argument)
  const char* kpool;
  const char* vpool;
  int32_t pool_pages;
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---- relayout: one workgroup per (64-key block, KV head)
//   K image slot (kt, ks, lane) = K[32 kt + lane % 32][16 ks + 8 (lane / 32) + 0..7]
//   V image slot (dt, kt, hf, lane) = V[key(e)][32 dt + lane % 32] for e = 0..7 with
//     key(e) = 32 kt + 16 hf + 8 (e / 4) + 4 (lane / 32) + e % 4
// (16-byte slots, slot index = ((..) * 64 + lane)), keys >= T read as zero.
__global__ __launch_bounds__(256) void relayout_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                       char* __restrict__ kimg, char* __restrict__ vimg, int T,
                                                       int hkv, int nb) {
  const int c = blockIdx.x, h = blockIdx.y;
  const size_t img = ((size_t)h * nb + c) * kImg;
  const size_t row = (size_t)hkv * kD;  // elements between consecutive tokens
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = i * 256 + threadIdx.x;
    const int lane = s & 63;
    {  // K slot
      const int ks = (s >> 6) & 7, kt = s >> 9;
      const int key = c * kB + 32 * kt + (lane & 31);
      i32x4 val = {0, 0, 0, 0};
      if (key < T)
        val = *reinterpret_cast<const i32x4*>(k + key * row + (size_t)h * kD + 16 * ks + 8 * (lane >> 5));
      *reinterpret_cast<i32x4*>(kimg + img + (size_t)s * 16) = val;
    }
    {  // V slot
      const int hf = (s >> 6) & 1, kt = (s >> 7) & 1, dt = s >> 8;
      const int d = 32 * dt + (lane & 31);
      bf16x8 val;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = c * kB + 32 * kt + 16 * hf + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        val[e] = key < T ? v[key * row + (size_t)h * kD + d] : (bf16_t)0.f;
      }
      *reinterpret_cast<bf16x8*>(vimg + img + (size_t)s * 16) = val;
    }
  }
}

// ---- column list for the main kernel: col clamped to [0, nb), kind in the sign bit
constexpr int32_t kDiagBit = (int32_t)0x80000000u;
__global__ __launch_bounds__(256) void pack_kernel(const int32_t* __restrict__ col, const uint8_t* __restrict__ kind,
                                                   int32_t* __restrict__ ent, int64_t nnz, int nb) {
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < nnz; j += (int64_t)gridDim.x * 256) {
    int c = col[j];
    c = c < 0 ? 0 : (c >= nb ? nb - 1 : c);
    ent[j] = c | (kind[j] ? kDiagBit : 0);
  }
}

// ---- rows by descending cost (ties by index): order[rank] = row
__global__ __launch_bounds__(256) void rank_kernel(const int32_t* __restrict__ row_ptr, int32_t* __restrict__ order,
                                                   int nb) {
  __shared__ int tile[256];
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int cr = r < nb ? row_ptr[r + 1] - row_ptr[r] : 0;
  int rank = 0;
  for (int base = 0; base < nb; base += 256) {
    const int t = base + threadIdx.x;
    __syncthreads();
    tile[threadIdx.x] = t < nb ? row_ptr[t + 1] - row_ptr[t] : -1;
    __syncthreads();
    const int m = nb - base < 256 ? nb - base : 256;
    for (int i = 0; i < m; ++i) {
      const int ci = tile[i];
      rank += (ci > cr) || (ci == cr && base + i < r);
    }
  }
  if (r < nb) order[rank] = r;
}

// max / sum with lane ^ 32: the swap returns {x[l], x[l ^ 32]} in some order per lane
__device__ __forceinline__ float xhalf_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// row_ptr / ent / order are read-only here and never alias the outputs, so their
// wave-uniform reads become scalar loads (a vector load would have to wait for every
// copy into LDS in flight before it).
//
// 8 waves, two per SIMD (waves w and w + 4 share one): wave w takes query head slot
// w / 2 and tokens [q0 + 32 (w % 2), +32) of the block.
// kMode 0: the packed prefill; 1: split-K pieces over K / V images; 2: split-K pieces with
// K gathered straight from the page pool (V from its image).
template <int kMode>
__global__ __launch_bounds__(kThreads) void prefill_kernel(Params p, const int32_t* __restrict__ row_ptr,
                                                          const int32_t* __restrict__ ent,
                                                          const int32_t* __restrict__ order,
                                                          const int32_t* __restrict__ gpages) {
  constexpr bool kSplit = kMode != 0, kGather = kMode == 2;
  constexpr int kLPW = kLoadsPerWave;  // vector-memory operations per stage per wave
  __shared__ __attribute__((aligned(1024))) char ring[kStages * kStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in a scalar register
  const int b = blockIdx.x;
  const int h = b % p.hkv;
  const int rest = b / p.hkv;
  const int hg = rest % p.n_hg;
  const int row = order[rest / p.n_hg];
  const int qblock = kSplit ? row / p.n_split : row;
  const int hslot = hg * 4 + (wave >> 1);
  const bool active = hslot < p.G;
  const int qhead = h * p.G + (active ? hslot : 0);  // an idle wave computes head 0 and stores nothing
  const int r0 = qblock * kB + 32 * (wave & 1);      // this wave's 32 query rows
  const int q0 = p.q_off + r0;                       // ... at key indices q0 ..
  const int j0 = row_ptr[row];
  const int n = row_ptr[row + 1] - j0;
  const int hi = lane >> 5, lo = lane & 31;

  // this wave's eighth of every stage: waves 0-3 copy the K image, waves 4-7 the V image.
  // The copies are buffer loads into LDS over a descriptor for this wave's part of the
  // block: the hardware drops any load outside it, and unlike the flat-encoded global
  // form they leave the compiler's LDS wait counts exact (it has to assume a flat load
  // may touch LDS out of order and would wait for every outstanding LDS read).
  const int my_off = wave * (kStage / kWaves);
  const char* my_img = (my_off < kImg ? p.kimg + my_off : p.vimg + (my_off - kImg)) + (size_t)h * p.nb * kImg;
  auto ent_of = [&](int j) { return ent[j0 + (j < n ? j : n - 1)]; };
  auto col_of = [&](int j) { return ent_of(j) & ~kDiagBit; };
  auto issue = [&](int j) {  // past the end: reload the last block into a slot nobody reads
    char* dst = ring + (j % kStages) * kStage + my_off;
    if constexpr (kGather) {
      if (wave < 4) {
        // K unit (kt, ks, lane) = K[32 kt + lane % 32][16 ks + 8 (lane / 32) ..], kt = wave / 2:
        // slot (f, g, t) of its page block, f = ks / 2, g = 2 (ks % 2) + lane / 32, t = lane % 16
        // (the block's page ids are scalar loads)
        const int kt = wave >> 1;
        const int g0 = 4 * col_of(j) + 2 * kt;
        const int pg0 = gpages[g0], pg1 = gpages[g0 + 1];  // wave-uniform: scalar loads
        const int pg = lo < 16 ? pg0 : pg1, slot = lo & 15;
        const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.kpool + (size_t)h * p.pool_pages * 4096), 0, p.pool_pages * 4096, 0x00020000);
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) {
          const int ks = 4 * (wave & 1) + i, f = ks >> 1, g = 2 * (ks & 1) + hi;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(dst + i * 1024),
                                                   16, pg * 4096 + ((f * 4 + g) * 16 + slot) * 16, 0, 0, 0);
        }
        return;
      }
      const int c = col_of(j);
      if (c != p.nb - 1 || !(p.T & (kB - 1))) {
        // V unit (dt, kt, hf, lane) = V[t][32 dt + lane % 32] for slots t0 .. t0 + 3 and
        // t0 + 8 .. t0 + 11 of page 2 kt + hf, t0 = 4 (lane / 32): in the pool's V^T slot
        // order these are the 16 bytes at row d, byte 16 (lane / 32).  Waves 4-7: dt =
        // wave - 4, copy i = (kt, hf).  (A last block that the context ends inside takes V
        // from its image: the page's slots past the context hold no data of it.)
        const int dt = wave - 4, d = 32 * dt + lo;
        const int pg_0 = gpages[4 * c], pg_1 = gpages[4 * c + 1], pg_2 = gpages[4 * c + 2], pg_3 = gpages[4 * c + 3];
        const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(p.vpool + (size_t)h * p.pool_pages * 4096), 0, p.pool_pages * 4096, 0x00020000);
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) {
          const int pg = i == 0 ? pg_0 : (i == 1 ? pg_1 : (i == 2 ? pg_2 : pg_3));
          __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(dst + i * 1024),
                                                   16, pg * 4096 + d * 32 + 16 * hi, 0, 0, 0);
        }
        return;
      }
    }
    const __amdgpu_buffer_rsrc_t src = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(my_img + (size_t)col_of(j) * kImg), 0, kLoadsPerWave * 1024, 0x00020000);
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void*)(dst + i * 1024), 16,
                                               lane * 16 + i * 1024, 0, 0, 0);
  };

  // queries: B operand of S^T = K Q^T, lane holds Q[q0 + lo][16 ks + 8 hi + 0..7]
  bf16x8 qf[8];
  {
    const int tr = r0 + lo;
    const bf16_t* src = p.q + ((size_t)(tr < p.nq ? tr : 0) * p.hq + qhead) * kD + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
      if (tr >= p.nq) qf[ks] = bf16x8{};
    }
  }
  f32x16 o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) o[dt] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float c2 = p.scale_log2;
  const bool ragged = (p.T & (kB - 1)) != 0;

  // K fragment (kt, ks) of ring slot j: A operand, keys 32 kt + lane % 32, dims 16 ks + 8 (lane / 32) + 0..7
  auto kfrag = [&](int j, int kt, int ks) {
    return *reinterpret_cast<const bf16x8*>(ring + (j % kStages) * kStage + ((kt * 8 + ks) * 64 + lane) * 16);
  };
  // V fragment (kt, hf, dt) of ring slot j: A operand of O^T += V^T P^T
  auto vfrag = [&](int j, int kt, int hf, int dt) {
    return *reinterpret_cast<const bf16x8*>(ring + (j % kStages) * kStage + kImg +
                                            (((dt * 2 + kt) * 2 + hf) * 64 + lane) * 16);
  };
  // S^T of block j into s, all at once (the prologue only)
  auto scores = [&](int j, f32x16 (&s)[2]) {
    bf16x8 kf[2][8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) kf[kt][ks] = kfrag(j, kt, ks);
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s[kt] = mfma32(kf[kt][ks], qf[ks], s[kt]);
  };
  // diagonal block (query < key < n_own) and keys past T -> -inf; rare, so behind a branch
  auto mask = [&](int e, f32x16 (&s)[2]) {
    const int c = e & ~kDiagBit;
    if (e < 0 || (ragged && c == p.nb - 1)) {
      const int kb = c * kB + 4 * hi;  // key of register r in tile kt: kb + 32 kt + 8 (r / 4) + r % 4
      const int lim = e < 0 ? q0 + lo : 0x7fffffff;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 32 * kt + 8 * (r >> 2) + (r & 3);
          s[kt][r] = ((key > lim && key < p.n_own) || key >= p.T) ? -INFINITY : s[kt][r];
        }
    }
  };
  // new running maximum for a block: this lane's 32 keys in 3-input steps, then the
  // other half-wave's 32
  auto block_max = [&](const f32x16 (&s)[2]) {
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      const float a = r == 1 ? s[1][1] : s[0][r];
      mx = r == 1 ? fmaxf(mx, a) : fmaxf(fmaxf(mx, a), s[1][r]);
    }
    return fmaxf(m, xhalf_max(mx));
  };

  // Software pipeline inside each wave.  Step j: (1) S of block j + 1 on the matrix core
  // while the vector unit turns S of block j into P = exp2(S c2 - m c2) (bf16) and its
  // row sum; (2) O += P V of block j while it takes the maximum of block j + 1.  The code
  // is cut into chunks fenced by scheduling barriers, each one or two matrix
  // instructions plus the vector work that fits under them, with LDS reads issued
  // three chunks ahead.  Ring: step j reads slots j (V) and j + 1 (K) and fills slot
  // j + 3 (block j - 1's, read by every wave before the barrier).  Past the last block
  // issue() reloads the last block, so the S computed for block n is harmless.
  f32x16 sa[2], sb[2];
  bf16x8 pk[2][2];
  float mn = -INFINITY;
  bool resc = false;
  auto step = [&](int j, f32x16 (&sc)[2], f32x16 (&sn)[2]) {
    const int e1 = ent_of(j + 1);
    wait_vmcnt<kLPW>();                      // this wave's part of block j + 1 landed (j + 2 in flight)
    asm volatile("s_barrier" ::: "memory");  // ... every wave's; slot j - 1 is consumed by all
    issue(j + 3);
    if (resc) {  // wave-uniform, rare: the new maximum outgrew the stale one by more than tau
      const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m - mn) * c2);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) o[dt] *= alpha;
    }
    const float mc = m == -INFINITY ? 0.f : m * c2;
    __builtin_amdgcn_sched_barrier(0);

    // (1) chunk ks: S instructions (0, ks) and (1, ks); P for 4 of this lane's 32 keys
    bf16x8 kf[2][8];
#pragma unroll
    for (int ks = 0; ks < 3; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) kf[kt][ks] = kfrag(j + 1, kt, ks);
    sn[0] = f32x16{};
    sn[1] = f32x16{};
    float ls = 0.f;
    const bf16x2 one = {(bf16_t)1.f, (bf16_t)1.f};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + 3 < 8) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) kf[kt][ks + 3] = kfrag(j + 1, kt, ks + 3);
      }
      // P of chunk ks: registers 8 hf + q .. + 3 of S tile t (t = ks / 4, hf = ks / 2 % 2, q = 4 (ks % 2))
      sn[0] = mfma32(kf[0][ks], qf[ks], sn[0]);
      {
        const int t = ks >> 2, hf = (ks >> 1) & 1, q = 4 * (ks & 1);
        pk[t][hf][q + 0] = (bf16_t)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * hf + q + 0], c2, -mc));
        pk[t][hf][q + 1] = (bf16_t)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * hf + q + 1], c2, -mc));
      }
      sn[1] = mfma32(kf[1][ks], qf[ks], sn[1]);
      {
        const int t = ks >> 2, hf = (ks >> 1) & 1, q = 4 * (ks & 1);
        pk[t][hf][q + 2] = (bf16_t)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * hf + q + 2], c2, -mc));
        pk[t][hf][q + 3] = (bf16_t)__builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][8 * hf + q + 3], c2, -mc));
        const bf16x2 p01 = {pk[t][hf][q + 0], pk[t][hf][q + 1]};
        const bf16x2 p23 = {pk[t][hf][q + 2], pk[t][hf][q + 3]};
        ls = __builtin_amdgcn_fdot2_f32_bf16(p01, one, ls, false);
        ls = __builtin_amdgcn_fdot2_f32_bf16(p23, one, ls, false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    l += ls;
    // P and the row sum stay here, ahead of the mask branch (the compiler would sink them
    // next to their use otherwise, away from the S instructions they overlap)
    asm volatile("" ::"v"(pk[0][0]), "v"(pk[0][1]), "v"(pk[1][0]), "v"(pk[1][1]), "v"(l));
    mask(e1, sn);

    // (2) chunk c = (kt, hf): four P V instructions (one per 32-dim tile) + part of the max
    bf16x8 vf[4][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) vf[c][dt] = vfrag(j, c >> 1, c & 1, dt);
    float mx = fmaxf(fmaxf(sn[0][0], sn[0][1]), sn[1][0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c + 2 < 4) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) vf[c + 2][dt] = vfrag(j, (c + 2) >> 1, (c + 2) & 1, dt);
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        o[dt] = mfma32(vf[c][dt], pk[c >> 1][c & 1], o[dt]);
        // registers 4 c + dt of both tiles (register 0, 1 of tile 0 and 0 of tile 1 are in mx)
        const int r = 4 * c + dt;
        if (r == 1) mx = fmaxf(mx, sn[1][1]);
        else if (r > 1) mx = fmaxf(fmaxf(mx, sn[0][r]), sn[1][r]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    mn = fmaxf(m, xhalf_max(mx));
    resc = __builtin_amdgcn_ballot_w64((mn - m) * c2 > kTau) != 0;  // false while both are -inf
  };

  if (n > 0) {
    issue(0);
    issue(1);
    issue(2);
    wait_vmcnt<2 * kLPW>();                  // block 0 landed for this wave ...
    asm volatile("s_barrier" ::: "memory");  // ... and for every wave
    scores(0, sa);
    mask(ent_of(0), sa);
    mn = block_max(sa);
    resc = __builtin_amdgcn_ballot_w64((mn - m) * c2 > kTau) != 0;
    int j = 0;
    for (; j + 1 < n; j += 2) {
      step(j, sa, sb);
      step(j + 1, sb, sa);
    }
    if (j < n) step(j, sa, sb);
  }
  wait_vmcnt<0>();  // no load may land in LDS after the workgroup ends
  if (!active) return;

  const float lt = xhalf_sum(l);
  const int tr = r0 + lo;
  if (tr >= p.nq) return;
  const float inv = lt > 0.f ? 1.f / lt : 0.f;  // a row with no visible key: zeros, lse -inf
  if constexpr (kSplit) {  // this piece's normalised partial, fp32
    const size_t slot = ((size_t)tr * p.hq + qhead) * p.n_split + row % p.n_split;
    float* dst = p.part_o + slot * kD + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef float f32x4v __attribute__((ext_vector_type(4)));
        f32x4v w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = o[dt][4 * g + q] * inv;
        *reinterpret_cast<f32x4v*>(dst + 32 * dt + 8 * g) = w;
      }
    if (hi == 0) p.part_lse2[slot] = lt > 0.f ? m * c2 + __log2f(lt) : -INFINITY;
  } else {
    bf16_t* dst = p.out + ((size_t)tr * p.hq + qhead) * kD + 4 * hi;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int q = 0; q < 4; ++q) w[q] = (bf16_t)(o[dt][4 * g + q] * inv);
        *reinterpret_cast<bf16x4*>(dst + 32 * dt + 8 * g) = w;
      }
    if (p.lse && hi == 0)
      p.lse[(size_t)qhead * p.nq + tr] = lt > 0.f ? (m * c2 + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
}

// ---- relayout of a sequence's visible keys out of the page pool: image block c of KV
// head h holds visible keys 64 c .. 64 c + 63, key t read from locs[t] = page * 16 + slot
// (pool block (page, h) at (h * pool_pages + page) * 16 * 128: K slot (f, g, slot) =
// K[slot][32 f + 8 g .. + 8], V^T element d * 16 + slot); keys >= T read as zero.
__global__ __launch_bounds__(256) void page_relayout_kernel(const bf16_t* __restrict__ kp, const bf16_t* __restrict__ vp,
                                                            const int32_t* __restrict__ locs, char* __restrict__ kimg,
                                                            char* __restrict__ vimg, int T, int nb, int pool_pages,
                                                            bool with_k, int c_first) {
  const int c = c_first + blockIdx.x, h = blockIdx.y;
  const size_t img = ((size_t)h * nb + c) * kImg;
  const size_t head = (size_t)h * pool_pages;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int s = i * 256 + threadIdx.x;
    const int lane = s & 63;
    if (with_k) {  // K slot (kt, ks, lane): K[32 kt + lane % 32][16 ks + 8 (lane / 32) + 0..7]
      const int ks = (s >> 6) & 7, kt = s >> 9;
      const int key = c * kB + 32 * kt + (lane & 31);
      i32x4 val = {0, 0, 0, 0};
      if (key < T) {
        const int loc = locs[key];
        const int d0 = 16 * ks + 8 * (lane >> 5);
        const bf16_t* blk = kp + (head + (loc >> 4)) * 16 * kD;
        val = *reinterpret_cast<const i32x4*>(blk + (((d0 >> 5) * 4 + ((d0 & 31) >> 3)) * 16 + (loc & 15)) * 8);
      }
      *reinterpret_cast<i32x4*>(kimg + img + (size_t)s * 16) = val;
    }
    {  // V slot (dt, kt, hf, lane): V[key(e)][32 dt + lane % 32], keys in two runs of four
      const int hf = (s >> 6) & 1, kt = (s >> 7) & 1, dt = s >> 8;
      const int d = 32 * dt + (lane & 31);
      bf16x8 val;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int key0 = c * kB + 32 * kt + 16 * hf + 8 * half + 4 * (lane >> 5);
        const int loc0 = key0 + 3 < T ? locs[key0] : -1;
        const int loc3 = key0 + 3 < T ? locs[key0 + 3] : -1;
        if (loc0 >= 0 && (loc0 & 3) == 0 && loc3 == loc0 + 3) {
          // four consecutive slots of one page: 8 contiguous bytes of the V^T row
          typedef bf16_t bf16x4v __attribute__((__vector_size__(4 * sizeof(bf16_t))));
          const bf16x4v x = *reinterpret_cast<const bf16x4v*>(vp + (head + (loc0 >> 4)) * 16 * kD + d * 16 + v_pos(loc0 & 15));
#pragma unroll
          for (int e = 0; e < 4; ++e) val[4 * half + e] = x[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = key0 + e;
            bf16_t x = (bf16_t)0.f;
            if (key < T) {
              const int loc = locs[key];
              x = vp[(head + (loc >> 4)) * 16 * kD + d * 16 + v_pos(loc & 15)];
            }
            val[4 * half + e] = x;
          }
        }
      }
      *reinterpret_cast<bf16x8*>(vimg + img + (size_t)s * 16) = val;
    }
  }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t order, ent, kimg, vimg, total;
};
WsLayout ws_layout(int32_t T, int32_t hkv, int64_t nnz) {
  const size_t nb = (size_t)(T + kB - 1) / kB;
  WsLayout w;
  w.order = 0;
  w.ent = align256(nb * 4);
  w.kimg = align256(w.ent + (size_t)nnz * 4);
  w.vimg = w.kimg + (size_t)hkv * nb * kImg;
  w.total = w.vimg + (size_t)hkv * nb * kImg;
  return w;
}

}  // namespace
}  // namespace fa

using namespace fa;

extern "C" int dag_attn_workspace_size(int32_t T, int32_t n_q_heads, int32_t n_kv_heads, int32_t block,
                                       int64_t nnz, size_t* bytes) {
  if (!bytes || T < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || nnz < 0)
    return fa_set_err(nullptr, KV_ERR_INVALID, "bad prefill shape");
  if (block != kB) return fa_set_err(nullptr, KV_ERR_UNSUPPORTED, "prefill block must be 64");
  *bytes = ws_layout(T, n_kv_heads, nnz).total;
  return KV_OK;
}

namespace {
int check_shape(int32_t T, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int64_t nnz, int32_t block) {
  if (T < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || nnz < 0)
    return fa_set_err(nullptr, KV_ERR_INVALID, "bad prefill shape or nnz");
  if (head_dim != kD || block != kB)
    return fa_set_err(nullptr, KV_ERR_UNSUPPORTED, "prefill needs head_dim 128 and block 64");
  return KV_OK;
}
}  // namespace

extern "C" int dag_attn_prepare(const void* k, const void* v, int32_t T, int32_t n_q_heads, int32_t n_kv_heads,
                                int32_t head_dim, const int32_t* row_ptr, const int32_t* col, const uint8_t* kind,
                                int64_t nnz, int32_t block, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (int st = check_shape(T, n_q_heads, n_kv_heads, head_dim, nnz, block)) return st;
  if (T == 0) return KV_OK;
  if (!k || !v || !row_ptr || !workspace || (nnz > 0 && (!col || !kind)))
    return fa_set_err(nullptr, KV_ERR_INVALID, "null pointer");
  const WsLayout w = ws_layout(T, n_kv_heads, nnz);
  if (ws_bytes < w.total) return fa_set_err(nullptr, KV_ERR_WORKSPACE, "prefill workspace too small");
  const int nb = (T + kB - 1) / kB;
  char* ws = static_cast<char*>(workspace);
  relayout_kernel<<<dim3(nb, n_kv_heads), 256, 0, stream>>>(static_cast<const bf16_t*>(k),
                                                           static_cast<const bf16_t*>(v), ws + w.kimg, ws + w.vimg,
                                                           T, n_kv_heads, nb);
  if (nnz > 0) {
    const int64_t blocks = (nnz + 255) / 256;
    pack_kernel<<<(unsigned)(blocks < 4096 ? blocks : 4096), 256, 0, stream>>>(
        col, kind, reinterpret_cast<int32_t*>(ws + w.ent), nnz, nb);
  }
  rank_kernel<<<(nb + 255) / 256, 256, 0, stream>>>(row_ptr, reinterpret_cast<int32_t*>(ws + w.order), nb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_err(nullptr, KV_ERR_HIP, std::string("prefill prepare: ") + hipGetErrorString(e));
  return KV_OK;
}

extern "C" int dag_attn_run(const void* q, void* out, float* lse, int32_t T, int32_t n_q_heads, int32_t n_kv_heads,
                            int32_t head_dim, const int32_t* row_ptr, int64_t nnz, int32_t block, float sm_scale,
                            const void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (int st = check_shape(T, n_q_heads, n_kv_heads, head_dim, nnz, block)) return st;
  if (!(sm_scale > 0.f)) return fa_set_err(nullptr, KV_ERR_INVALID, "softmax scale must be positive");
  if (T == 0) return KV_OK;
  if (!q || !out || !row_ptr || !workspace) return fa_set_err(nullptr, KV_ERR_INVALID, "null pointer");
  const WsLayout w = ws_layout(T, n_kv_heads, nnz);
  if (ws_bytes < w.total) return fa_set_err(nullptr, KV_ERR_WORKSPACE, "prefill workspace too small");
  const char* ws = static_cast<const char*>(workspace);
  Params p;
  p.q = static_cast<const bf16_t*>(q);
  p.kimg = ws + w.kimg;
  p.vimg = ws + w.vimg;
  p.out = static_cast<bf16_t*>(out);
  p.lse = lse;
  p.T = T;
  p.hq = n_q_heads;
  p.hkv = n_kv_heads;
  p.G = n_q_heads / n_kv_heads;
  p.n_hg = (p.G + 3) / 4;
  p.nb = (T + kB - 1) / kB;
  p.sm_scale = sm_scale;
  p.scale_log2 = sm_scale * 1.4426950408889634f;
  p.q_off = 0;
  p.nq = T;
  p.n_own = T;
  p.n_split = 1;
  p.part_lse2 = p.part_o = nullptr;
  p.kpool = nullptr;
  p.vpool = nullptr;
  p.pool_pages = 0;
  prefill_kernel<0><<<(size_t)p.nb * n_kv_heads * p.n_hg, kThreads, 0, stream>>>(
      p, row_ptr, reinterpret_cast<const int32_t*>(ws + w.ent), reinterpret_cast<const int32_t*>(ws + w.order),
      nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_err(nullptr, KV_ERR_HIP, std::string("prefill: ") + hipGetErrorString(e));
  return KV_OK;
}

extern "C" int dag_attn_prefill(const void* q, const void* k, const void* v, void* out, float* lse, int32_t T,
                                int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, const int32_t* row_ptr,
                                const int32_t* col, const uint8_t* kind, int64_t nnz, int32_t block,
                                float sm_scale, void* workspace, size_t ws_bytes, hipStream_t stream) {
  if (int st = check_shape(T, n_q_heads, n_kv_heads, head_dim, nnz, block)) return st;
  if (!(sm_scale > 0.f)) return fa_set_err(nullptr, KV_ERR_INVALID, "softmax scale must be positive");
  if (T == 0) return KV_OK;
  if (!q || !out) return fa_set_err(nullptr, KV_ERR_INVALID, "null pointer");
  if (int st = dag_attn_prepare(k, v, T, n_q_heads, n_kv_heads, head_dim, row_ptr, col, kind, nnz, block, workspace,
                                ws_bytes, stream))
    return st;
  return dag_attn_run(q, out, lse, T, n_q_heads, n_kv_heads, head_dim, row_ptr, nnz, block, sm_scale, workspace,
                      ws_bytes, stream);
}

// Restore of a sequence's last tokens as a split-K tiled prefill over its pages.  When the
// visible keys fill whole pages in order, the prefill kernel copies K and V straight from
// the page blocks into its LDS ring (a page block's 16-byte K slots and 16-byte runs of
// its V^T rows are the operand images' units, so the copies only need per-lane offsets);
// only the V of a last block that the context ends inside is relaid into an image.  Else
// K and V are relaid into operand-order images first.  The kernel runs the CSR rows
// (query block, key-range piece) and writes one partial per (query row, head, piece),
// merged afterwards.
hipError_t fa::fa_launch_restore(const RestoreLaunch& r, hipStream_t stream) {
  const int nb = (r.T + kB - 1) / kB;
  // gather mode: only the V image of a last block that the context ends inside
  const int c_first = r.kgather ? nb - 1 : 0;
  if (!r.kgather || (r.T & (kB - 1)))
    page_relayout_kernel<<<dim3(nb - c_first, r.hkv), 256, 0, stream>>>(
        static_cast<const bf16_t*>(r.k_pages), static_cast<const bf16_t*>(r.v_pages), r.locs, r.kimg, r.vimg, r.T, nb,
        r.pool_pages, !r.kgather, c_first);
  Params p;
  p.q = static_cast<const bf16_t*>(r.q);
  p.kimg = r.kimg;
  p.vimg = r.vimg;
  p.out = nullptr;
  p.lse = nullptr;
  p.T = r.T;
  p.hq = r.hq;
  p.hkv = r.hkv;
  p.G = r.hq / r.hkv;
  p.n_hg = (p.G + 3) / 4;
  p.nb = nb;
  p.sm_scale = r.sm_scale;
  p.scale_log2 = r.sm_scale * 1.4426950408889634f;
  p.q_off = r.q_off;
  p.nq = r.nq;
  p.n_own = r.n_own;
  p.n_split = r.n_split;
  p.part_lse2 = r.part_lse2;
  p.part_o = r.part_o;
  p.kpool = static_cast<const char*>(r.k_pages);
  p.vpool = static_cast<const char*>(r.v_pages);
  p.pool_pages = r.pool_pages;
  const size_t grid = (size_t)r.n_rows * r.hkv * p.n_hg;
  if (r.kgather)
    prefill_kernel<2><<<grid, kThreads, 0, stream>>>(p, r.row_ptr, r.ent, r.order, r.gpages);
  else
    prefill_kernel<1><<<grid, kThreads, 0, stream>>>(p, r.row_ptr, r.ent, r.order, nullptr);
  return hipGetLastError();
}
