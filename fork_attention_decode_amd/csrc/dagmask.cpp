// DAG block mask for packed prefill.
//
// Octopus (zicq.com), "Packed DAG-GRPO": the branches of an episode are packed into one
// block-sparse attention whose mask encodes causality inside a thread, the allowed
// cross-thread read edges and the synchronisation dependencies; only block pairs the
// DAG allows are computed, with cost near O(B L^2 + E_DAG L_b^2) (same section).
//
// Rule: a query of segment S at packed index i sees every token of S's ancestors,
// the tokens of S with index <= i, and every edge range whose target is S.  With
// block-aligned segments and edges a block pair is either fully visible (FULL), the
// diagonal block of the query's own segment (CAUSAL: key <= query), or not needed.
#include <algorithm>
#include <string>
#include <vector>

#include "../../include/forkattn.h"

int fa_set_err(struct kv_pool* P, int code, const std::string& m);
#define FAIL(code, msg) return fa_set_err(nullptr, (code), (msg))

extern "C" int dag_mask_build(const int32_t* seg, int32_t n_seg, const int32_t* edges, int32_t n_edges,
                              int32_t T, int32_t block, int32_t* row_ptr, int32_t* col, uint8_t* kind,
                              int64_t* nnz) {
  if (!seg || n_seg < 1 || n_edges < 0 || (n_edges > 0 && !edges) || T < 1 || block < 1 || !nnz)
    FAIL(KV_ERR_INVALID, "bad dag_mask_build arguments");
  // segments tile [0, T) in order, parents precede children, starts block aligned
  int64_t at = 0;
  for (int32_t s = 0; s < n_seg; ++s) {
    const int32_t st = seg[3 * s], ln = seg[3 * s + 1], par = seg[3 * s + 2];
    if (st != at || ln < 1 || (s == 0 ? par != -1 : (par < 0 || par >= s)) || st % block)
      FAIL(KV_ERR_INVALID, "segments must tile [0, T) in order with block-aligned starts");
    at += ln;
  }
  if (at != T) FAIL(KV_ERR_INVALID, "segments do not end at T");
  for (int32_t e = 0; e < n_edges; ++e) {
    const int32_t src = edges[4 * e], off = edges[4 * e + 1], ln = edges[4 * e + 2], dst = edges[4 * e + 3];
    if (src < 0 || src >= n_seg || dst < 0 || dst >= n_seg || src == dst || off < 0 || ln < 1 ||
        off + ln > seg[3 * src + 1])
      FAIL(KV_ERR_INVALID, "edge outside its source segment");
    const int64_t a = (int64_t)seg[3 * src] + off, b = a + ln;
    if (a % block || (b % block && b != T)) FAIL(KV_ERR_INVALID, "edge ranges must be block aligned");
  }
  const int32_t nb = (T + block - 1) / block;
  // key-block intervals visible to every query of each segment (ancestors + edges)
  std::vector<std::vector<std::pair<int32_t, int32_t>>> vis((size_t)n_seg);
  for (int32_t s = 0; s < n_seg; ++s) {
    for (int32_t a = seg[3 * s + 2]; a >= 0; a = seg[3 * a + 2]) {
      const int64_t lo = seg[3 * a], hi = lo + seg[3 * a + 1];
      vis[s].push_back({(int32_t)(lo / block), (int32_t)((hi + block - 1) / block)});
    }
  }
  for (int32_t e = 0; e < n_edges; ++e) {
    const int64_t lo = (int64_t)seg[3 * edges[4 * e]] + edges[4 * e + 1], hi = lo + edges[4 * e + 2];
    vis[edges[4 * e + 3]].push_back({(int32_t)(lo / block), (int32_t)((hi + block - 1) / block)});
  }
  if ((col == nullptr) != (kind == nullptr)) FAIL(KV_ERR_INVALID, "give both col and kind or neither");
  int64_t count = 0;
  if (row_ptr) row_ptr[0] = 0;
  std::vector<std::pair<int32_t, int32_t>> iv;
  int32_t s = 0;
  for (int32_t qb = 0; qb < nb; ++qb) {
    while (s + 1 < n_seg && seg[3 * (s + 1)] <= qb * block) ++s;
    iv = vis[s];
    iv.push_back({seg[3 * s] / block, qb});  // own segment before the diagonal block
    iv.push_back({qb, qb + 1});              // the diagonal block itself
    std::sort(iv.begin(), iv.end());
    int32_t cur_hi = -1;
    for (auto [lo, hi] : iv) {
      lo = std::max(lo, cur_hi);
      for (int32_t kb = lo; kb < hi; ++kb) {
        if (col) {
          col[count] = kb;
          kind[count] = kb == qb ? 1 : 0;
        }
        ++count;
      }
      cur_hi = std::max(cur_hi, hi);
    }
    if (row_ptr) row_ptr[qb + 1] = (int32_t)count;
  }
  *nnz = count;
  return KV_OK;
}
