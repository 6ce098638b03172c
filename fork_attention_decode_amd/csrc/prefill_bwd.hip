// Packed DAG prefill backward: gradients of the block-sparse attention over a DAG block
// mask, for gfx950.
//
// Octopus (zicq.com), "Packed DAG-GRPO": the packed episode is trained through one
// block-sparse attention whose mask encodes the DAG, so the backward pass visits the same
// (query block, key block) pairs as the forward.  Per visible pair, query head h (KV head
// g = h / G), scale c, the forward's lse_i and o_i:
//   P_ij = exp(c q_i.k_j - lse_i),  D_i = do_i.o_i,  dS_ij = P_ij (do_i.v_j - D_i),
//   dq_i = c sum_j dS_ij k_j,  dk_j = c sum_{h in g, i} dS_ij q_i,  dv_j = sum_{h in g, i} P_ij do_i.
//
// Mapping onto CDNA4 (v_mfma_f32_16x16x32_bf16 throughout):
//   * prep passes write, per (64-query block, query head), the Q and dO blocks in operand
//     order (OPO: 16 rows x 8 dims per lane, one 1 KiB wave read per fragment), the log2
//     normalisers and D; and per (64-key block, KV head) K and V in OPO.  Where a block is
//     the B operand of a product that sums over its rows (Q, dO for dK, dV; K for dQ) the
//     kernels read it from the same image with the LDS transpose load, in an order (TP)
//     that pairs row 4 k + r of two 16-row tiles with the lanes and registers where an
//     accumulator tile holds them, so P and dS feed the next products straight from the
//     accumulators, with no shuffles;
//   * dkdv_kernel: one workgroup per (two 64-key blocks, KV head), 8 waves, wave = 32 keys
//     (K and V fragments held in registers) x one 32-row half of every query block; it
//     walks the union of the two blocks' columns of the mask (a CSC over column pairs
//     built on the device, highest query block first) and, for each listed query block and each of
//     the G query heads, brings that block's record into LDS with buffer loads that write
//     LDS directly (double-buffered: the next record's loads are in flight while the
//     current one computes) and computes S = Q K^T, P, dP = dO V^T, dS, then dV += P^T dO
//     and dK += dS^T Q: each Q / dO fragment read from LDS feeds two MFMAs; dK and dV of
//     the G heads accumulate in registers, with no atomics, and the two query halves
//     meet in LDS at the end;
//   * dq_kernel: one workgroup per (64-query block, 4 query heads of a KV head), 8 waves
//     of 32 queries (two 16-query tiles, so each K / V fragment read from LDS feeds two
//     MFMAs), Q and dO fragments in registers; it walks the block's CSR row (its entries
//     with an in-range column packed on the device, read as scalar loads), brings each
//     key block's K / V / K^T into LDS the same way (double-buffered) once for the 4
//     heads and computes S^T = K Q^T, P^T, dP^T = V dO^T, dS^T and dQ += dS K;
//   * the mask kinds are those of the forward: kind 1 (the diagonal block) hides key >
//     query, keys >= T are hidden, a row with lse = -inf contributes nothing.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string>
#include "../../include/forkattn.h"

int fa_set_err(struct kv_pool* P, int code, const std::string& m);

namespace fa {
namespace {

typedef __bf16 bf16_t;
typedef bf16_t bf16x8 __attribute__((__vector_size__(8 * sizeof(bf16_t))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kB = 64;                     // block edge (tokens)
constexpr int kD = 128;                    // head dim
constexpr int kImg = kB * kD * 2;          // bytes of one 64 x 128 bf16 image (1024 units of 16 B)
constexpr int kQRec = 2 * kImg + 2 * kB * 4;  // Q OPO, dO OPO, lse2[64], D[64]
constexpr int kKRec = 2 * kImg;            // K OPO, V OPO
constexpr int kThreads = 256;
constexpr int kQRecL = (kQRec + 1023) / 1024 * 1024;  // an LDS record buffer: whole 1 KiB units
constexpr unsigned kRowMask = 0xffffffu;   // CSC entry: query block | listed bits << 24 | diagonal bits << 26

// OPO unit of element (r, 8 c8 .. 8 c8 + 7) of a 64 x 128 block: fragment (r / 16, c8 / 4),
// lane r % 16 + 16 (c8 % 4)
__device__ __forceinline__ int opo_unit(int r, int c8) { return ((r >> 4) * 4 + (c8 >> 2)) * 64 + (r & 15) + 16 * (c8 & 3); }

// The B operand of a product over the rows r of a 64 x 128 OPO image (two 32-row steps s,
// eight 16-column tiles n), in TP order: lane c % 16 + 16 k holds, in order, rows
// 32 s + 4 k + (0..3) and 32 s + 16 + 4 k + (0..3) of column 16 n + c % 16 -- the rows where
// two 16-row accumulator tiles hold the other operand, so P and dS feed the product
// straight from the accumulators.  Read with the LDS transpose load (ds_read_b64_tr_b16):
// within each 16-lane group, lane j receives element j % 4 of what lanes 4 e + j / 4 of the
// group loaded (e = 0..3), so lane 4 e + c of group k loads 8 bytes of row 32 s + 4 k + e,
// columns 16 n + 4 c .. + 3; every instruction reads 512 contiguous bytes of the image.
__device__ __forceinline__ int tp_lane_off(int lane) {
  const int k = lane >> 4, e = (lane & 15) >> 2, c = lane & 3;
  return ((4 * k + e) + 16 * (c >> 1)) * 16 + 8 * (c & 1);
}
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 tp_frag(const char* img, int s, int n, int lane_off) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  const char* a = img + (8 * s + (n >> 1)) * 1024 + 512 * (n & 1) + lane_off;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(a + 4 * 1024));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

struct QPrep {
  const bf16_t* q;
  const bf16_t* o;
  const bf16_t* dout;
  const float* lse;
  char* qrec;
  int32_t T, hq;
};

// grid (Hq, n_blocks): the record of (query block, head)
__global__ __launch_bounds__(kThreads) void q_prep_kernel(QPrep p) {
  const int h = blockIdx.x, qb = blockIdx.y, tid = threadIdx.x;
  char* rec = p.qrec + ((size_t)qb * p.hq + h) * kQRec;
  i32x4* q_opo = reinterpret_cast<i32x4*>(rec);
  i32x4* do_opo = reinterpret_cast<i32x4*>(rec + kImg);
  float* lse2 = reinterpret_cast<float*>(rec + 2 * kImg);
  float* dd = lse2 + kB;
  for (int u = tid; u < kB * 16; u += kThreads) {  // 16 units per row; 16 consecutive threads share a row
    const int r = u >> 4, c8 = u & 15;
    const int64_t i = (int64_t)qb * kB + r;
    i32x4 qv = {0, 0, 0, 0}, dv = {0, 0, 0, 0}, ov = {0, 0, 0, 0};
    if (i < p.T) {
      const size_t off = ((size_t)i * p.hq + h) * kD + 8 * c8;
      qv = *reinterpret_cast<const i32x4*>(p.q + off);
      dv = *reinterpret_cast<const i32x4*>(p.dout + off);
      ov = *reinterpret_cast<const i32x4*>(p.o + off);
    }
    q_opo[opo_unit(r, c8)] = qv;
    do_opo[opo_unit(r, c8)] = dv;
    const bf16x8 qe = __builtin_bit_cast(bf16x8, qv), de = __builtin_bit_cast(bf16x8, dv),
                 oe = __builtin_bit_cast(bf16x8, ov);
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot = __builtin_fmaf((float)de[e], (float)oe[e], dot);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) dot += __shfl_xor(dot, off);
    if (c8 == 0) {
      dd[r] = dot;
      float l2 = INFINITY;  // padding rows and rows with no visible key take no part
      if (i < p.T) {
        const float l = p.lse[(size_t)h * p.T + i];
        if (l > -INFINITY) l2 = l * 1.4426950408889634f;
      }
      lse2[r] = l2;
    }
  }
}

// grid (Hkv, n_blocks): K OPO, V OPO of (key block, KV head)
__global__ __launch_bounds__(kThreads) void k_prep_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                          char* __restrict__ krec, int32_t T, int32_t hkv) {
  const int g = blockIdx.x, kb = blockIdx.y, tid = threadIdx.x;
  char* rec = krec + ((size_t)kb * hkv + g) * kKRec;
  i32x4* k_opo = reinterpret_cast<i32x4*>(rec);
  i32x4* v_opo = reinterpret_cast<i32x4*>(rec + kImg);
  for (int u = tid; u < kB * 16; u += kThreads) {
    const int r = u >> 4, c8 = u & 15;
    const int64_t j = (int64_t)kb * kB + r;
    i32x4 kv = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
    if (j < T) {
      const size_t off = ((size_t)j * hkv + g) * kD + 8 * c8;
      kv = *reinterpret_cast<const i32x4*>(k + off);
      vv = *reinterpret_cast<const i32x4*>(v + off);
    }
    k_opo[opo_unit(r, c8)] = kv;
    v_opo[opo_unit(r, c8)] = vv;
  }
}

// The mask's transpose over pairs of key-block columns, query blocks ascending within a
// pair (count, scan, fill), found by a binary search of each column in every CSR row.

// index of column c in the ascending col[a..b), or -1
__device__ __forceinline__ int find_in_row(const int32_t* col, int a, int b, int c) {
  int lo = a, hi = b;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (col[mid] < c) lo = mid + 1;
    else hi = mid;
  }
  return lo < b && col[lo] == c ? lo : -1;
}

// one workgroup per pair of key-block columns (2 c, 2 c + 1): query blocks in either
__global__ __launch_bounds__(kThreads) void csc_count_kernel(const int32_t* __restrict__ row_ptr,
                                                             const int32_t* __restrict__ col, int32_t nb,
                                                             int32_t* __restrict__ count) {
  __shared__ int s_n;
  const int c0 = 2 * blockIdx.x;
  if (threadIdx.x == 0) s_n = 0;
  __syncthreads();
  int n = 0;
  for (int r = threadIdx.x; r < nb; r += kThreads)
    n += find_in_row(col, row_ptr[r], row_ptr[r + 1], c0) >= 0 || find_in_row(col, row_ptr[r], row_ptr[r + 1], c0 + 1) >= 0;
  for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off);
  if ((threadIdx.x & 63) == 0) atomicAdd(&s_n, n);
  __syncthreads();
  if (threadIdx.x == 0) count[blockIdx.x] = s_n;
}

// exclusive scan of nb counts into col_ptr[0..nb] (one workgroup)
__global__ __launch_bounds__(1024) void csc_scan_kernel(const int32_t* __restrict__ count, int32_t nb,
                                                        int32_t* __restrict__ col_ptr) {
  __shared__ int s_wave[16];
  __shared__ int s_carry;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_carry = 0;
  __syncthreads();
  for (int base = 0; base < nb; base += 1024) {
    const int i = base + tid;
    const int x = i < nb ? count[i] : 0;
    int incl = x;
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int before = s_carry;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    if (i < nb) col_ptr[i] = before + incl - x;
    __syncthreads();
    if (tid == 1023) s_carry = before + incl;
    __syncthreads();
  }
  if (tid == 0) col_ptr[nb] = s_carry;
}

// entries of column pair c in ascending query block: qb | present bits << 24 (bit i: column
// 2 c + i lists qb) | diagonal bits << 26
__global__ __launch_bounds__(kThreads) void csc_fill_kernel(const int32_t* __restrict__ row_ptr,
                                                            const int32_t* __restrict__ col,
                                                            const uint8_t* __restrict__ kind, int32_t nb,
                                                            const int32_t* __restrict__ col_ptr,
                                                            uint32_t* __restrict__ crow) {
  __shared__ int s_wave[kThreads / 64];
  const int c0 = 2 * blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = col_ptr[blockIdx.x];
  for (int base = 0; base < nb; base += kThreads) {  // uniform trip count
    const int r = base + tid;
    int e0 = -1, e1 = -1;
    if (r < nb) {
      e0 = find_in_row(col, row_ptr[r], row_ptr[r + 1], c0);
      e1 = find_in_row(col, row_ptr[r], row_ptr[r + 1], c0 + 1);
    }
    const bool any = e0 >= 0 || e1 >= 0;
    const uint64_t bal = __ballot(any);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    __syncthreads();
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    int wb = carry;
    for (int w = 0; w < wave; ++w) wb += s_wave[w];
    if (any) {
      uint32_t ent = (uint32_t)r | (e0 >= 0 ? 1u << 24 : 0u) | (e1 >= 0 ? 2u << 24 : 0u);
      if (e0 >= 0 && kind[e0]) ent |= 1u << 26;
      if (e1 >= 0 && kind[e1]) ent |= 2u << 26;
      crow[wb + before] = ent;
    }
    for (int w = 0; w < kThreads / 64; ++w) carry += s_wave[w];
  }
}

// the CSR rows without their skipped entries, for the dQ pass: rent[row_ptr[r] + i] =
// column | diagonal << 31 of the row's i-th entry whose column is in [0, nb), rcnt[r] = how
// many; one wave per row
__global__ __launch_bounds__(64) void row_pack_kernel(const int32_t* __restrict__ row_ptr,
                                                      const int32_t* __restrict__ col,
                                                      const uint8_t* __restrict__ kind, int32_t nb,
                                                      int32_t* __restrict__ rent, int32_t* __restrict__ rcnt) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const int a = row_ptr[r], b = row_ptr[r + 1];
  int n = 0;
  for (int base = a; base < b; base += 64) {
    const int e = base + lane;
    const int c = e < b ? col[e] : -1;
    const bool ok = c >= 0 && c < nb;
    const uint64_t bal = __ballot(ok);
    if (ok) rent[a + n + __popcll(bal & ((1ull << lane) - 1ull))] = c | (kind[e] ? (int32_t)0x80000000u : 0);
    n += __popcll(bal);
  }
  if (lane == 0) rcnt[r] = n;
}

// s_waitcnt vmcnt(0), the other counters left free (gfx9 encoding)
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }

// query blocks by descending count of packed entries (ties by index): order[rank] = block,
// so the dQ pass starts its longest rows first and ends on short ones (the dK/dV pass
// keeps the natural column order: its first columns, the prefix's, are its longest)
__global__ __launch_bounds__(256) void rank_kernel(const int32_t* __restrict__ cost, int32_t* __restrict__ order,
                                                   int nb) {
  __shared__ int tile[256];
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int cr = r < nb ? cost[r] : 0;
  int rank = 0;
  for (int base = 0; base < nb; base += 256) {
    const int t = base + threadIdx.x;
    __syncthreads();
    tile[threadIdx.x] = t < nb ? cost[t] : -1;
    __syncthreads();
    const int m = nb - base < 256 ? nb - base : 256;
    for (int i = 0; i < m; ++i) {
      const int ci = tile[i];
      rank += (ci > cr) || (ci == cr && base + i < r);
    }
  }
  if (r < nb) order[rank] = r;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// two accumulator tiles (rows 4 k + 0..3 of each) as the A operand of a product over them
__device__ __forceinline__ bf16x8 pack_pair(f32x4 a, f32x4 b) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = (bf16_t)a[e], r[e + 4] = (bf16_t)b[e];
  return r;
}

struct BwdParams {
  const char* qrec;
  const char* krec;
  const int32_t* row_ptr;
  const int32_t* col;
  const uint8_t* kind;
  const int32_t* col_ptr;
  const uint32_t* crow;
  float* dq;
  float* dk;
  float* dv;
  int32_t T, hq, hkv, G, nb;
  float c2, scale;
};

constexpr int kKeyBlocksPerWg = 2;                 // dK / dV workgroup: 2 key blocks, 8 waves
constexpr int kDkdvThreads = 256 * kKeyBlocksPerWg;
constexpr int kHeadsPerWg = 4;                     // dQ workgroup: up to 4 query heads, 8 waves of 32 queries
constexpr int kDqThreads = 512;

// grid (Hkv, ceil(n_blocks / 2)): dK, dV of two 64-key blocks for one KV head.  Wave w takes
// keys 32 (w % 4) .. + 31 of the two blocks (two 16-key tiles, K and V fragments held in
// registers) over query rows 32 (w / 4) .. + 31 of every staged record, so each Q / dO
// fragment read from LDS feeds both key tiles; waves w and w + 4 add their dK, dV at the
// end through LDS.  The workgroup walks the union of the two columns; a wave whose column
// lacks the query block skips it.
__global__ __launch_bounds__(kDkdvThreads) void dkdv_kernel(BwdParams p, const uint32_t* __restrict__ crow) {
  // two record buffers; at the end the same LDS holds the dK, dV halves being added
  constexpr int kLds = 2 * kQRecL > 4 * 2 * 2 * 8 * 4 * 64 * 4 ? 2 * kQRecL : 4 * 2 * 2 * 8 * 4 * 64 * 4;
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  auto rec = [&](int i) { return lds + i * kQRecL; };
  const int g = blockIdx.x, lane = threadIdx.x & 63;
  const int tpo = tp_lane_off(lane);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kq = w & 3, qh = w >> 2;              // 32-key group of the 128, query half
  const int kbi = kq >> 1;                        // key block within the workgroup
  const int kb = kKeyBlocksPerWg * blockIdx.y + kbi;
  const bool live = kb < p.nb;
  bf16x8 kf[2][4], vf[2][4];  // key tiles kt = 0, 1 (16 keys each) as the B operand
  if (live) {
    const char* krec = p.krec + ((size_t)kb * p.hkv + g) * kKRec;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int t16 = 2 * (kq & 1) + kt;  // 16-key tile of the block
        kf[kt][f] = *reinterpret_cast<const bf16x8*>(krec + ((t16 * 4 + f) * 64 + lane) * 16);
        vf[kt][f] = *reinterpret_cast<const bf16x8*>(krec + kImg + ((t16 * 4 + f) * 64 + lane) * 16);
      }
  }
  f32x4 dk[2][8], dv[2][8];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int n = 0; n < 8; ++n) dk[kt][n] = dv[kt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int key0 = kb * kB + 32 * (kq & 1) + (lane & 15);  // + 16 kt
  const int e0 = p.col_ptr[blockIdx.y], e1 = p.col_ptr[blockIdx.y + 1];
  // stages: (entry, head of the group), entries from the highest query block down, so
  // workgroups whose lists share a tail (every prefix column reaches the last branch
  // blocks) start on the same records and read them while they sit in the die's L2
  const int n_st = (e1 - e0) * p.G;
  // (crow is a separate restrict argument so that its reads are scalar loads, which
  // leave the vector-memory count of the records in flight alone)
  auto ent_of = [&](int st) { return crow[e1 - 1 - st / p.G]; };
  // a record goes from memory straight into LDS (no registers): 1 KiB per wave
  // instruction, wave w issuing units w, w + 8, ...; the descriptor ends at the record,
  // so the last unit's second half reads as zero
  auto issue = [&](int st, char* dst) {
    const int qb = (int)(ent_of(st) & kRowMask);
    const char* src = p.qrec + ((size_t)qb * p.hq + g * p.G + st % p.G) * kQRec;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, kQRec, 0x00020000);
#pragma unroll
    for (int i = 0; i < (kQRecL / 1024 + 7) / 8; ++i) {
      const int j = w + 8 * i;
      if (j < kQRecL / 1024)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + j * 1024), 16,
                                                 lane * 16, j * 1024, 0, 0);
    }
  };
  if (n_st > 0) issue(0, rec(0));
  wait_vmcnt0();
  __syncthreads();
  for (int st = 0; st < n_st; ++st) {
    const int cur = st & 1;
    if (st + 1 < n_st) issue(st + 1, rec(cur ^ 1));
    const uint32_t ent = ent_of(st);
    const int qb = (int)(ent & kRowMask);
    if (live && ((ent >> (24 + kbi)) & 1u)) {
      const bool diag = (ent >> (26 + kbi)) & 1u;
      const char* r = rec(cur);
      const float* lse2 = reinterpret_cast<const float*>(r + 2 * kImg);
      const float* dd = lse2 + kB;
      f32x4 s[2][2], dp[2][2];  // [kt][query tile of this half]
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) s[kt][tt] = dp[kt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int u = (((2 * qh + tt) * 4 + f) * 64 + lane) * 16;
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(r + u);
          const bf16x8 da = *reinterpret_cast<const bf16x8*>(r + kImg + u);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            s[kt][tt] = mfma(qa, kf[kt][f], s[kt][tt]);
            dp[kt][tt] = mfma(da, vf[kt][f], dp[kt][tt]);
          }
        }
      // s[kt][tt][i]: query 16 (2 qh + tt) + 4 (lane / 16) + i, key key0 + 16 kt.  Hidden
      // scores become -inf (P = 0) behind a wave-uniform branch: only a diagonal block and
      // the last block (keys >= T) hide any.  A row that takes no part has lse2 = +inf, so
      // its P is 0 as well.
      if (diag || kb == p.nb - 1) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key_tok = key0 + 16 * kt, q_tok = qb * kB + 16 * (2 * qh + tt) + 4 * (lane >> 4) + i;
              if (key_tok >= p.T || (diag && key_tok > q_tok)) s[kt][tt][i] = -INFINITY;
            }
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const int q0 = 16 * (2 * qh + tt) + 4 * (lane >> 4);
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse2 + q0);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dd + q0);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][tt][i], p.c2, -l4[i]));
            s[kt][tt][i] = pr;
            dp[kt][tt][i] = pr * (dp[kt][tt][i] - d4[i]);
          }
      }
      bf16x8 ap[2], ads[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        ap[kt] = pack_pair(s[kt][0], s[kt][1]);
        ads[kt] = pack_pair(dp[kt][0], dp[kt][1]);
      }
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const bf16x8 dot = tp_frag(r + kImg, qh, n, tpo);
        const bf16x8 qt = tp_frag(r, qh, n, tpo);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          dv[kt][n] = mfma(ap[kt], dot, dv[kt][n]);
          dk[kt][n] = mfma(ads[kt], qt, dk[kt][n]);
        }
      }
    }
    wait_vmcnt0();
    __syncthreads();  // stage st + 1 is in place; every wave is done with stage st
  }
  // waves 4-7 hand their query half's sums to waves 0-3 through the (now free) records
  float* xr = reinterpret_cast<float*>(lds) + (size_t)kq * (2 * 2 * 8 * 4 * 64);
  if (qh == 1) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xr[(((0 * 2 + kt) * 8 + n) * 4 + i) * 64 + lane] = dk[kt][n][i];
          xr[(((1 * 2 + kt) * 8 + n) * 4 + i) * 64 + lane] = dv[kt][n][i];
        }
  }
  __syncthreads();
  if (qh == 1 || !live) return;
  // dk[kt][n][i]: key key0 - lane % 16 + 16 kt + 4 (lane / 16) + i, dim 16 n + lane % 16
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = kb * kB + 32 * (kq & 1) + 16 * kt + 4 * (lane >> 4) + i;
      if (j < p.T) {
        float* dkr = p.dk + ((size_t)j * p.hkv + g) * kD + (lane & 15);
        float* dvr = p.dv + ((size_t)j * p.hkv + g) * kD + (lane & 15);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
          dkr[16 * n] = (dk[kt][n][i] + xr[(((0 * 2 + kt) * 8 + n) * 4 + i) * 64 + lane]) * p.scale;
          dvr[16 * n] = dv[kt][n][i] + xr[(((1 * 2 + kt) * 8 + n) * 4 + i) * 64 + lane];
        }
      }
    }
}

// grid (Hq / hw, n_blocks), hw = 4, 2 or 1 query heads of one KV head per workgroup (the
// largest that divides G): dQ of query block order[blockIdx.y] (longest rows first); wave w takes queries 32 (w % 2) .. + 31
// (two 16-query tiles) of head blockIdx.x hw + w / 2 (waves past the hw heads only help
// stage).  Each key block's record staged in LDS serves the workgroup's heads, and each
// K / V fragment read from LDS feeds the products of both tiles.
__global__ __launch_bounds__(kDqThreads) void dq_kernel(BwdParams p, int hw, const int32_t* __restrict__ rent,
                                                        const int32_t* __restrict__ rcnt,
                                                        const int32_t* __restrict__ order) {
  __shared__ __attribute__((aligned(16))) char rec[2][kKRec];
  const int qb = order[blockIdx.y], lane = threadIdx.x & 63;
  const int tpo = tp_lane_off(lane);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool active = (w >> 1) < hw;
  const int h = blockIdx.x * hw + (active ? w >> 1 : 0), qt0 = 2 * (w & 1);
  const int g = blockIdx.x * hw / p.G;
  const char* qrec = p.qrec + ((size_t)qb * p.hq + h) * kQRec;
  bf16x8 qf[2][4], df[2][4];  // tile u's 16 queries as the B operand (query = lane % 16)
  float lq[2], dq_d[2];
  int q_tok[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int qt = qt0 + u;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      qf[u][f] = *reinterpret_cast<const bf16x8*>(qrec + ((qt * 4 + f) * 64 + lane) * 16);
      df[u][f] = *reinterpret_cast<const bf16x8*>(qrec + kImg + ((qt * 4 + f) * 64 + lane) * 16);
    }
    lq[u] = reinterpret_cast<const float*>(qrec + 2 * kImg)[qt * 16 + (lane & 15)];
    dq_d[u] = reinterpret_cast<const float*>(qrec + 2 * kImg)[kB + qt * 16 + (lane & 15)];
    q_tok[u] = qb * kB + qt * 16 + (lane & 15);
  }
  f32x4 dq[2][8];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int n = 0; n < 8; ++n) dq[u][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // stages: the row's entries with a column in [0, nb), as packed by row_pack_kernel
  // (rent and rcnt are separate restrict arguments, so their reads are scalar loads,
  // which leave the vector-memory count of the records in flight alone; the entry after
  // next is read while the current one computes)
  const int e0 = p.row_ptr[qb], n_e = rcnt[qb];
  // a key block's record goes from memory straight into LDS: 48 units of 1 KiB, wave w
  // issuing units w, w + 8, ...
  auto issue = [&](int ent, char* dst) {
    const char* src = p.krec + ((size_t)(ent & 0x7fffffff) * p.hkv + g) * kKRec;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, kKRec, 0x00020000);
#pragma unroll
    for (int i = 0; i < kKRec / 1024 / 8; ++i) {
      const int j = w + 8 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + j * 1024), 16,
                                               lane * 16, j * 1024, 0, 0);
    }
  };
  static_assert(kKRec % (8 * 1024) == 0 && kDqThreads == 512, "record units per wave");
  int ent = n_e > 0 ? rent[e0] : 0;
  if (n_e > 0) issue(ent, rec[0]);
  int ent_n = n_e > 1 ? rent[e0 + 1] : 0;
  wait_vmcnt0();
  __syncthreads();
  for (int i = 0, cur = 0; i < n_e; ++i, cur ^= 1) {
    if (i + 1 < n_e) issue(ent_n, rec[cur ^ 1]);
    const int ent_nn = i + 2 < n_e ? rent[e0 + i + 2] : 0;
    const int kb = ent & 0x7fffffff;
    const bool diag = ent < 0;
    const char* r = rec[cur];
    if (active) {
    f32x4 s[2][4], dp[2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int u = 0; u < 2; ++u) s[u][t] = dp[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int o = ((t * 4 + f) * 64 + lane) * 16;
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(r + o);
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(r + kImg + o);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          s[u][t] = mfma(kf, qf[u][f], s[u][t]);
          dp[u][t] = mfma(vf, df[u][f], dp[u][t]);
        }
      }
    }
    // s[u][t][i]: key 16 t + 4 (lane / 16) + i, query lane % 16 of tile u.  Hidden scores
    // become -inf (P = 0) behind a wave-uniform branch, as in dkdv_kernel.
    if (diag || kb == p.nb - 1) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kb * kB + 16 * t + 4 * (lane >> 4) + i;
            if (key >= p.T || (diag && key > q_tok[u])) s[u][t][i] = -INFINITY;
          }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(s[u][t][i], p.c2, -lq[u]));
          dp[u][t][i] = pr * (dp[u][t][i] - dq_d[u]);
        }
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      bf16x8 ads[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) ads[u] = pack_pair(dp[u][2 * h2], dp[u][2 * h2 + 1]);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const bf16x8 kt = tp_frag(r, h2, n, tpo);
#pragma unroll
        for (int u = 0; u < 2; ++u) dq[u][n] = mfma(ads[u], kt, dq[u][n]);
      }
    }
    }
    wait_vmcnt0();
    __syncthreads();  // the next key block is in place; every wave is done with this one
    ent = ent_n;
    ent_n = ent_nn;
  }
  // dq[u][n][i]: query 4 (lane / 16) + i of tile u, dim 16 n + lane % 16
  if (!active) return;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qi = qb * kB + (qt0 + u) * 16 + 4 * (lane >> 4) + i;
      if (qi < p.T) {
        float* dqr = p.dq + ((size_t)qi * p.hq + h) * kD + (lane & 15);
#pragma unroll
        for (int n = 0; n < 8; ++n) dqr[16 * n] = dq[u][n][i] * p.scale;
      }
    }
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct BwdLayout {
  size_t qrec, krec, count, col_ptr, crow, rcnt, rent, order, total;
};
BwdLayout bwd_layout(int32_t T, int32_t hq, int32_t hkv, int64_t nnz) {
  const size_t nb = (size_t)(T + kB - 1) / kB;
  BwdLayout w;
  w.qrec = 0;
  w.krec = align256(nb * hq * kQRec);
  w.count = align256(w.krec + nb * hkv * kKRec);
  w.col_ptr = align256(w.count + nb * 4);
  w.crow = align256(w.col_ptr + (nb + 1) * 4);
  w.rcnt = align256(w.crow + (size_t)nnz * 4);
  w.rent = align256(w.rcnt + nb * 4);
  w.order = align256(w.rent + (size_t)nnz * 4);
  w.total = w.order + nb * 4;
  return w;
}

}  // namespace
}  // namespace fa

using namespace fa;

extern "C" int dag_attn_backward_workspace_size(int32_t T, int32_t n_q_heads, int32_t n_kv_heads, int32_t block,
                                                int64_t nnz, size_t* bytes) {
  if (!bytes || T < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || nnz < 0)
    return fa_set_err(nullptr, KV_ERR_INVALID, "bad prefill backward shape");
  if (block != kB) return fa_set_err(nullptr, KV_ERR_UNSUPPORTED, "prefill backward block must be 64");
  *bytes = bwd_layout(T, n_q_heads, n_kv_heads, nnz).total;
  return KV_OK;
}

extern "C" int dag_attn_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                 const float* lse, float* dq, float* dk, float* dv, int32_t T, int32_t n_q_heads,
                                 int32_t n_kv_heads, int32_t head_dim, const int32_t* row_ptr, const int32_t* col,
                                 const uint8_t* kind, int64_t nnz, int32_t block, float sm_scale, void* workspace,
                                 size_t ws_bytes, hipStream_t stream) {
  if (T < 0 || n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || nnz < 0)
    return fa_set_err(nullptr, KV_ERR_INVALID, "bad prefill backward shape or nnz");
  if (head_dim != kD || block != kB)
    return fa_set_err(nullptr, KV_ERR_UNSUPPORTED, "prefill backward needs head_dim 128 and block 64");
  if (!(sm_scale > 0.f)) return fa_set_err(nullptr, KV_ERR_INVALID, "softmax scale must be positive");
  if (T == 0) return KV_OK;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !row_ptr || !workspace ||
      (nnz > 0 && (!col || !kind)))
    return fa_set_err(nullptr, KV_ERR_INVALID, "null pointer");
  const int64_t nb = (T + kB - 1) / kB;
  if (nb > 65535) return fa_set_err(nullptr, KV_ERR_UNSUPPORTED, "at most 65,535 blocks of 64 tokens");
  const BwdLayout w = bwd_layout(T, n_q_heads, n_kv_heads, nnz);
  if (ws_bytes < w.total) return fa_set_err(nullptr, KV_ERR_WORKSPACE, "prefill backward workspace too small");
  char* ws = static_cast<char*>(workspace);
  QPrep qp;
  qp.q = static_cast<const bf16_t*>(q);
  qp.o = static_cast<const bf16_t*>(out);
  qp.dout = static_cast<const bf16_t*>(dout);
  qp.lse = lse;
  qp.qrec = ws + w.qrec;
  qp.T = T;
  qp.hq = n_q_heads;
  q_prep_kernel<<<dim3(n_q_heads, (unsigned)nb), kThreads, 0, stream>>>(qp);
  k_prep_kernel<<<dim3(n_kv_heads, (unsigned)nb), kThreads, 0, stream>>>(
      static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), ws + w.krec, T, n_kv_heads);
  int32_t* count = reinterpret_cast<int32_t*>(ws + w.count);
  int32_t* col_ptr = reinterpret_cast<int32_t*>(ws + w.col_ptr);
  uint32_t* crow = reinterpret_cast<uint32_t*>(ws + w.crow);
  const int32_t n_pair = (int32_t)((nb + 1) / 2);
  csc_count_kernel<<<(unsigned)n_pair, kThreads, 0, stream>>>(row_ptr, col, (int32_t)nb, count);
  csc_scan_kernel<<<1, 1024, 0, stream>>>(count, n_pair, col_ptr);
  csc_fill_kernel<<<(unsigned)n_pair, kThreads, 0, stream>>>(row_ptr, col, kind, (int32_t)nb, col_ptr, crow);
  int32_t* rcnt = reinterpret_cast<int32_t*>(ws + w.rcnt);
  int32_t* rent = reinterpret_cast<int32_t*>(ws + w.rent);
  row_pack_kernel<<<(unsigned)nb, 64, 0, stream>>>(row_ptr, col, kind, (int32_t)nb, rent, rcnt);
  int32_t* order = reinterpret_cast<int32_t*>(ws + w.order);
  rank_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, stream>>>(rcnt, order, (int32_t)nb);
  BwdParams p;
  p.qrec = ws + w.qrec;
  p.krec = ws + w.krec;
  p.row_ptr = row_ptr;
  p.col = col;
  p.kind = kind;
  p.col_ptr = col_ptr;
  p.crow = crow;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.T = T;
  p.hq = n_q_heads;
  p.hkv = n_kv_heads;
  p.G = n_q_heads / n_kv_heads;
  p.nb = (int32_t)nb;
  p.scale = sm_scale;
  p.c2 = sm_scale * 1.4426950408889634f;
  dkdv_kernel<<<dim3(n_kv_heads, (unsigned)n_pair), kDkdvThreads, 0, stream>>>(p, p.crow);
  const int hw = p.G % kHeadsPerWg == 0 ? kHeadsPerWg : (p.G % 2 == 0 ? 2 : 1);
  dq_kernel<<<dim3(n_q_heads / hw, (unsigned)nb), kDqThreads, 0, stream>>>(p, hw, rent, rcnt, order);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fa_set_err(nullptr, KV_ERR_HIP, std::string("prefill backward: ") + hipGetErrorString(e));
  return KV_OK;
}
