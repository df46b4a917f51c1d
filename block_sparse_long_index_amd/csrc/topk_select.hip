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
//
// One wave per row.  Candidates are (score, block) 64-bit keys, unique per
// row, so the km = top_k - 1 best form one well-defined set.  Each lane loads
// its share of the row's blocks (lane w takes blocks w, w + 64, ...; the first
// 32 per lane all in flight at once) and keeps its largest key.  The km-th
// largest of the 64 lane maxima is a threshold t: at least km candidates reach
// it (one per lane among the km best lanes), so the km best candidates are all
// >= t, and usually only a few dozen others reach it.  Those survivors are
// gathered in LDS; each one's rank among them (how many survivors are larger)
// decides whether it is selected, and the selected blocks' rank by id gives
// their output slot.  If more survivors than LDS holds reach t (many equal
// scores), the wave falls back to per-lane sorted lists merged by km rounds of
// wave-wide maxima.
#include "msa_common.h"
#include "topk_common.h"

namespace msa {

constexpr int kTopkPerLane = 32;     // candidates per lane held in registers
constexpr int kTopkSurvMax = 256;    // survivors gathered in LDS

// grid.x = rows of the pass (chunk row = (query - r0) * G + g), one wave each.
template <int KCAP>
__global__ __launch_bounds__(64) void topk_select_kernel(
    const float* __restrict__ S, long long ld, int r0, int r1, const int32_t* __restrict__ cu_q,
    const int32_t* __restrict__ cu_k, int batch, int G, int top_k, int32_t* __restrict__ sel,
    float* __restrict__ sel_score) {
  __shared__ uint64_t lane_max[kWave];
  __shared__ uint64_t surv[kTopkSurvMax];
  __shared__ uint64_t chosen[KCAP];
  __shared__ uint64_t thresh;
  __shared__ int n_surv;

  const long long crow = blockIdx.x;
  const int lane = threadIdx.x;
  const int km = top_k - 1;
  const int r = r0 + (int)(crow / G);
  const int g = (int)(crow % G);
  const RowPos rp = locate_row(r, cu_q, cu_k, batch);
  const int beta_p = rp.p / kBlock;
  const float* col = S + crow;
  int32_t* so = sel + ((size_t)r * G + g) * top_k;
  float* sco = sel_score ? sel_score + ((size_t)r * G + g) * top_k : nullptr;

  // key of block beta (0 = no candidate: past the end, or a NaN score)
  auto key_of = [&](int beta) -> uint64_t {
    if (beta >= beta_p) return 0;
    const float s = col[(size_t)beta * ld];
    return s == s ? make_key(s, beta) : 0;
  };

  // 1. the first kTopkPerLane candidates of the lane in registers; the lane's max
  uint64_t first[kTopkPerLane];
  {
    float s[kTopkPerLane];
#pragma unroll
    for (int i = 0; i < kTopkPerLane; ++i) {
      const int beta = lane + i * kWave;
      s[i] = col[(size_t)min(beta, max(beta_p - 1, 0)) * ld];
    }
#pragma unroll
    for (int i = 0; i < kTopkPerLane; ++i) {
      const int beta = lane + i * kWave;
      first[i] = (beta < beta_p && s[i] == s[i]) ? make_key(s[i], beta) : 0;
    }
  }
  uint64_t mx = 0;
#pragma unroll
  for (int i = 0; i < kTopkPerLane; ++i) mx = first[i] > mx ? first[i] : mx;
  for (int beta = lane + kTopkPerLane * kWave; beta < beta_p; beta += kWave) {
    const uint64_t k = key_of(beta);
    mx = k > mx ? k : mx;
  }

  // 2. threshold: the km-th largest lane maximum (0 if fewer than km lanes hold one)
  lane_max[lane] = mx;
  if (lane == 0) {
    thresh = 0;
    n_surv = 0;
  }
  __syncthreads();
  if (km > 0 && mx != 0) {
    int rank = 0;
    for (int j = 0; j < kWave; ++j) rank += lane_max[j] > mx ? 1 : 0;
    if (rank == km - 1) thresh = mx;
  }
  __syncthreads();
  const uint64_t t = thresh;

  // 3. gather the survivors (keys >= t)
  int mine = 0;
  if (km > 0) {
#pragma unroll
    for (int i = 0; i < kTopkPerLane; ++i) mine += (first[i] != 0 && first[i] >= t) ? 1 : 0;
    for (int beta = lane + kTopkPerLane * kWave; beta < beta_p; beta += kWave) {
      const uint64_t k = key_of(beta);
      mine += (k != 0 && k >= t) ? 1 : 0;
    }
  }
  int base = mine ? atomicAdd(&n_surv, mine) : 0;
  __syncthreads();
  const int n = n_surv;
  if (n <= kTopkSurvMax) {
    if (mine) {
#pragma unroll
      for (int i = 0; i < kTopkPerLane; ++i)
        if (first[i] != 0 && first[i] >= t) surv[base++] = first[i];
      for (int beta = lane + kTopkPerLane * kWave; beta < beta_p; beta += kWave) {
        const uint64_t k = key_of(beta);
        if (k != 0 && k >= t) surv[base++] = k;
      }
    }
    __syncthreads();
    // 4. rank among the survivors: the km largest are selected
    for (int i = lane; i < n; i += kWave) {
      const uint64_t k = surv[i];
      int rank = 0;
      for (int j = 0; j < n; ++j) rank += surv[j] > k ? 1 : 0;
      if (rank < km) chosen[rank] = k;
    }
  } else {
    // many equal scores: per-lane sorted lists of the keys >= t, merged by
    // km rounds of wave-wide maxima
    uint64_t list[KCAP];
#pragma unroll
    for (int i = 0; i < KCAP; ++i) list[i] = 0;
#pragma unroll
    for (int i = 0; i < kTopkPerLane; ++i)
      if (first[i] != 0 && first[i] >= t) list_insert(list, first[i]);
    for (int beta = lane + kTopkPerLane * kWave; beta < beta_p; beta += kWave) {
      const uint64_t k = key_of(beta);
      if (k != 0 && k >= t) list_insert(list, k);
    }
    for (int i = 0; i < km; ++i) {
      const uint64_t head = list[0];
      uint64_t best = head;
#pragma unroll
      for (int off = kWave / 2; off >= 1; off >>= 1) {
        const uint64_t o = shfl_xor_u64(best, off);
        best = o > best ? o : best;
      }
      if (best != 0 && head == best) {
#pragma unroll
        for (int j = 0; j < KCAP - 1; ++j) list[j] = list[j + 1];
        list[KCAP - 1] = 0;
      }
      if (lane == 0) chosen[i] = best;
    }
  }
  __syncthreads();

  // 5. output: the selected blocks in ascending id, then the local block, then padding
  const int cnt = min(km, n);   // every survivor is a real candidate; the fallback has n > km
  if (lane < cnt) {
    const uint64_t k = chosen[lane];
    const int id = key_block(k);
    int pos = 0;
    for (int j = 0; j < cnt; ++j) pos += key_block(chosen[j]) < id ? 1 : 0;
    so[pos] = id;
    if (sco) sco[pos] = key_score(k);
  } else if (lane < top_k) {
    so[lane] = lane == cnt ? beta_p : -1;
    if (sco) sco[lane] = lane == cnt ? INFINITY : __uint_as_float(0x7fc00000u);
  }
}

template <int KCAP>
static hipError_t launch_topk_kcap(const float* S, long long ld, int r0, int r1, const int32_t* cu_q,
                                   const int32_t* cu_k, int batch, int G, int top_k, int32_t* sel,
                                   float* sel_score, hipStream_t st) {
  const long long nrows = (long long)(r1 - r0) * G;
  if (nrows <= 0) return hipSuccess;
  hipLaunchKernelGGL((topk_select_kernel<KCAP>), dim3((unsigned)nrows), dim3(kWave), 0, st, S, ld, r0,
                     r1, cu_q, cu_k, batch, G, top_k, sel, sel_score);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* S, long long ld, int r0, int r1, const int32_t* cu_q,
                              const int32_t* cu_k, int batch, int G, int top_k, int32_t* sel,
                              float* sel_score, hipStream_t st) {
  const int km = top_k - 1;
  if (km <= 1) return launch_topk_kcap<1>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
  if (km <= 2) return launch_topk_kcap<2>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
  if (km <= 4) return launch_topk_kcap<4>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
  if (km <= 8) return launch_topk_kcap<8>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
  if (km <= 16) return launch_topk_kcap<16>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
  return launch_topk_kcap<32>(S, ld, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
}

}  // namespace msa
