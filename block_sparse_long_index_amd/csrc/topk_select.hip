// Index Branch, step 3: top-k block selection with the forced local block.
//
// Per (query, group): the query's own block beta(p) is always selected
// (MSA guide, ai-tool-zukan.com/minimax-msa-guide, section
// "クエリを含むローカルブロックの強制取り込み"; zhaixingw.cn ai-news/10, section
// "这套注意力到底怎么省的") and counts toward top_k, so the other top_k - 1
// are the best earlier blocks by block score (section "2段階構造の中身"; the
// budget of top_k * 128 tokens in the table of section
// "ブロック単位選択の数値設計").  Equal scores: the lower block id wins.  The
// output is ascending, -1 padded; one selection per group, shared by the
// group's heads (section "GQAグループ単位の選択共有とは").
//
// This kernel selects from a materialised block-score buffer (the decode
// path); the prefill path fuses the same selection into its scoring kernel.
// Each lane keeps a descending list of the KCAP best (score, block) keys of
// its candidate stream in registers (KCAP = next power of two >= top_k - 1).
// With W lanes per row the lanes split the row's blocks and merge their lists
// in top_k - 1 max-reduction rounds.
#include "msa_common.h"
#include "topk_common.h"

namespace msa {

// grid.x covers the chunk's rows (chunk row = (query - r0) * G + g), 256 / W rows per workgroup.
template <int KCAP, int W>
__global__ __launch_bounds__(256) void topk_select_kernel(
    const float* __restrict__ S, long long ld, int r0, int r1, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int batch, int G, int top_k, int32_t* __restrict__ sel,
    float* __restrict__ sel_score) {
  const int rows_per_wg = 256 / W;
  const long long crow = (long long)blockIdx.x * rows_per_wg + threadIdx.x / W;
  const int w = threadIdx.x % W;
  const long long nrows = (long long)(r1 - r0) * G;
  const bool active = crow < nrows;
  const int km = top_k - 1;

  int r = r0, g = 0, beta_p = 0;
  if (active) {
    r = r0 + (int)(crow / G);
    g = (int)(crow % G);
    RowPos rp = locate_row(r, cu_q, cu_k, batch);
    beta_p = rp.p / kBlock;
  }

  uint64_t list[KCAP];
#pragma unroll
  for (int i = 0; i < KCAP; ++i) list[i] = 0;

  if (active && km > 0) {
    const float* col = S + crow;
    // eight candidates per step: their loads are all in flight before the inserts
    constexpr int kBatch = 8;
    for (int base = w; base < beta_p; base += kBatch * W) {
      float sc[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int beta = base + i * W;
        sc[i] = col[(size_t)min(beta, beta_p - 1) * ld];
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int beta = base + i * W;
        if (beta < beta_p && sc[i] == sc[i]) list_insert(list, make_key(sc[i], beta));
      }
    }
  }

  uint64_t res[KCAP];
  if constexpr (W == 1) {
#pragma unroll
    for (int i = 0; i < KCAP; ++i) res[i] = list[i];
  } else {
#pragma unroll
    for (int i = 0; i < KCAP; ++i) {
      res[i] = 0;
      if (i < km) {
        uint64_t head = list[0];
        uint64_t best = head;
#pragma unroll
        for (int off = W / 2; off >= 1; off >>= 1) {
          uint64_t o = shfl_xor_u64(best, off);
          best = o > best ? o : best;
        }
        if (best != 0 && head == best) {
#pragma unroll
          for (int j = 0; j < KCAP - 1; ++j) list[j] = list[j + 1];
          list[KCAP - 1] = 0;
        }
        res[i] = best;
      }
    }
  }
  if (!active || w != 0) return;

  write_selection(res, km, beta_p, top_k, sel + ((size_t)r * G + g) * top_k,
                  sel_score ? sel_score + ((size_t)r * G + g) * top_k : nullptr);
}

template <int KCAP>
static hipError_t launch_topk_kcap(const float* S, long long ld, int r0, int r1, const int32_t* cu_q,
                                   const int32_t* cu_k, int batch, int G, int top_k, bool wide,
                                   int32_t* sel, float* sel_score, hipStream_t st) {
  long long nrows = (long long)(r1 - r0) * G;
  if (wide) {
    dim3 grid((unsigned)((nrows + 3) / 4));
    hipLaunchKernelGGL((topk_select_kernel<KCAP, 64>), grid, dim3(256), 0, st, S, ld, r0, r1, cu_q,
                       cu_k, batch, G, top_k, sel, sel_score);
  } else {
    dim3 grid((unsigned)((nrows + 255) / 256));
    hipLaunchKernelGGL((topk_select_kernel<KCAP, 1>), grid, dim3(256), 0, st, S, ld, r0, r1, cu_q,
                       cu_k, batch, G, top_k, sel, sel_score);
  }
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* S, long long ld, int r0, int r1, const int32_t* cu_q,
                              const int32_t* cu_k, int batch, int G, int top_k, bool wide,
                              int32_t* sel, float* sel_score, hipStream_t st) {
  int km = top_k - 1;
  if (km <= 1) return launch_topk_kcap<1>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
  if (km <= 2) return launch_topk_kcap<2>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
  if (km <= 4) return launch_topk_kcap<4>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
  if (km <= 8) return launch_topk_kcap<8>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
  if (km <= 16) return launch_topk_kcap<16>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
  return launch_topk_kcap<32>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, wide, sel, sel_score, st);
}

}  // namespace msa
