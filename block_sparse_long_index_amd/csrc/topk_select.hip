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
// Four waves per row.  Candidates are (score, block) 64-bit keys, unique per
// row, so the km = top_k - 1 best form one well-defined set.  Each thread
// loads its share of the row's blocks (thread i takes blocks i, i + 256, ...;
// the first 8 per thread all in flight at once) and keeps its largest key.
// In each wave the km-th largest of the 64 lane maxima is a threshold t_w
// that at least km of that wave's candidates reach; the row's threshold t is
// the largest t_w, so at least km candidates reach t and the km best are all
// >= t, while usually only a few dozen others reach it.  Those survivors are
// gathered in LDS; each one's rank among them (how many survivors are larger)
// decides whether it is selected, and the selected blocks' rank by id gives
// their output slot.  If more survivors than LDS holds reach t (many equal
// scores), the threads fall back to per-thread sorted lists merged by km
// rounds of workgroup-wide maxima.  (One wave per row left three quarters of
// the SIMDs idle at decode sizes, where the rows' latency is the kernel's time.)
#include "msa_common.h"
#include "topk_common.h"

namespace msa {

constexpr int kTopkWaves = 4;
constexpr int kTopkThreads = kTopkWaves * kWave;
constexpr int kTopkPerThread = 8;    // candidates per thread held in registers
constexpr int kTopkSurvMax = 256;    // survivors gathered in LDS

// grid.x = rows of the pass (chunk row = (query - r0) * G + g), one workgroup each.
template <int KCAP>
__global__ __launch_bounds__(kTopkThreads) void topk_select_kernel(
    const float* __restrict__ S, long long ld, int nb_rows, int r0, int r1,
    const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k, int batch, int G, int top_k,
    int32_t* __restrict__ sel, float* __restrict__ sel_score) {
  __shared__ uint64_t lane_max[kTopkWaves][kWave];
  __shared__ uint64_t wave_t[kTopkWaves];
  __shared__ uint64_t wave_best[kTopkWaves];
  __shared__ uint64_t surv[kTopkSurvMax];
  __shared__ uint64_t chosen[KCAP];
  __shared__ int n_surv;

  const long long crow = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int km = top_k - 1;
  const int r = r0 + (int)(crow / G);
  const int g = (int)(crow % G);
  const float* col = S + crow;
  // the first kTopkPerThread scores of the thread are loaded before the row's
  // own block is known (clamped to the buffer's nb_rows block rows; scores of
  // blocks at or after the row's own block are dropped below), so the loads
  // overlap the row lookup
  float s_first[kTopkPerThread];
#pragma unroll
  for (int i = 0; i < kTopkPerThread; ++i)
    s_first[i] = col[(size_t)min(tid + i * kTopkThreads, max(nb_rows - 1, 0)) * ld];
  const RowPos rp = locate_row(r, cu_q, cu_k, batch);
  const int beta_p = rp.p / kBlock;
  int32_t* so = sel + ((size_t)r * G + g) * top_k;
  float* sco = sel_score ? sel_score + ((size_t)r * G + g) * top_k : nullptr;

  // key of block beta (0 = no candidate: past the end, or a NaN score)
  auto key_of = [&](int beta) -> uint64_t {
    if (beta >= beta_p) return 0;
    const float s = col[(size_t)beta * ld];
    return s == s ? make_key(s, beta) : 0;
  };

  // 1. the first kTopkPerThread candidates of the thread in registers; its max
  uint64_t first[kTopkPerThread];
#pragma unroll
  for (int i = 0; i < kTopkPerThread; ++i) {
    const int beta = tid + i * kTopkThreads;
    first[i] = (beta < beta_p && s_first[i] == s_first[i]) ? make_key(s_first[i], beta) : 0;
  }
  uint64_t mx = 0;
#pragma unroll
  for (int i = 0; i < kTopkPerThread; ++i) mx = first[i] > mx ? first[i] : mx;
  for (int beta = tid + kTopkPerThread * kTopkThreads; beta < beta_p; beta += kTopkThreads) {
    const uint64_t k = key_of(beta);
    mx = k > mx ? k : mx;
  }

  // 2. threshold: per wave the km-th largest lane maximum (0 if fewer than km
  // of its lanes hold one), then the largest of the waves'
  lane_max[wave][lane] = mx;
  if (lane == 0) wave_t[wave] = 0;
  if (tid == 0) n_surv = 0;
  __syncthreads();
  if (km > 0 && mx != 0) {
    int rank = 0;
    for (int j = 0; j < kWave; ++j) rank += lane_max[wave][j] > mx ? 1 : 0;
    if (rank == km - 1) wave_t[wave] = mx;
  }
  __syncthreads();
  uint64_t t = wave_t[0];
#pragma unroll
  for (int w = 1; w < kTopkWaves; ++w) t = wave_t[w] > t ? wave_t[w] : t;

  // 3. gather the survivors (keys >= t)
  int mine = 0;
  if (km > 0) {
#pragma unroll
    for (int i = 0; i < kTopkPerThread; ++i) mine += (first[i] != 0 && first[i] >= t) ? 1 : 0;
    for (int beta = tid + kTopkPerThread * kTopkThreads; beta < beta_p; beta += kTopkThreads) {
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
      for (int i = 0; i < kTopkPerThread; ++i)
        if (first[i] != 0 && first[i] >= t) surv[base++] = first[i];
      for (int beta = tid + kTopkPerThread * kTopkThreads; beta < beta_p; beta += kTopkThreads) {
        const uint64_t k = key_of(beta);
        if (k != 0 && k >= t) surv[base++] = k;
      }
    }
    __syncthreads();
    // 4. rank among the survivors: the km largest are selected
    for (int i = tid; i < n; i += kTopkThreads) {
      const uint64_t k = surv[i];
      int rank = 0;
      for (int j = 0; j < n; ++j) rank += surv[j] > k ? 1 : 0;
      if (rank < km) chosen[rank] = k;
    }
  } else {
    // many equal scores: per-thread sorted lists of the keys >= t, merged by
    // km rounds of workgroup-wide maxima
    uint64_t list[KCAP];
#pragma unroll
    for (int i = 0; i < KCAP; ++i) list[i] = 0;
#pragma unroll
    for (int i = 0; i < kTopkPerThread; ++i)
      if (first[i] != 0 && first[i] >= t) list_insert(list, first[i]);
    for (int beta = tid + kTopkPerThread * kTopkThreads; beta < beta_p; beta += kTopkThreads) {
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
      if (lane == 0) wave_best[wave] = best;
      __syncthreads();
      best = wave_best[0];
#pragma unroll
      for (int w = 1; w < kTopkWaves; ++w) best = wave_best[w] > best ? wave_best[w] : best;
      // keys are unique: exactly one thread holds the best at its head
      if (best != 0 && head == best) {
#pragma unroll
        for (int j = 0; j < KCAP - 1; ++j) list[j] = list[j + 1];
        list[KCAP - 1] = 0;
      }
      if (tid == 0) chosen[i] = best;
      __syncthreads();   // wave_best is rewritten by the next round
    }
  }
  __syncthreads();

  // 5. output: the selected blocks in ascending id, then the local block, then padding
  const int cnt = min(km, n);   // every survivor is a real candidate; the fallback has n > km
  if (tid < cnt) {
    const uint64_t k = chosen[tid];
    const int id = key_block(k);
    int pos = 0;
    for (int j = 0; j < cnt; ++j) pos += key_block(chosen[j]) < id ? 1 : 0;
    so[pos] = id;
    if (sco) sco[pos] = key_score(k);
  } else if (tid < top_k) {
    so[tid] = tid == cnt ? beta_p : -1;
    if (sco) sco[tid] = tid == cnt ? INFINITY : __uint_as_float(0x7fc00000u);
  }
}

template <int KCAP>
static hipError_t launch_topk_kcap(const float* S, long long ld, int nb_rows, int r0, int r1, const int32_t* cu_q,
                                   const int32_t* cu_k, int batch, int G, int top_k, int32_t* sel,
                                   float* sel_score, hipStream_t st) {
  const long long nrows = (long long)(r1 - r0) * G;
  if (nrows <= 0) return hipSuccess;
  hipLaunchKernelGGL((topk_select_kernel<KCAP>), dim3((unsigned)nrows), dim3(kTopkThreads), 0, st, S, ld,
                     nb_rows, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* S, long long ld, int nb_rows, int r0, int r1, const int32_t* cu_q,
                              const int32_t* cu_k, int batch, int G, int top_k, int32_t* sel,
                              float* sel_score, hipStream_t st) {
  const int km = top_k - 1;
  if (km <= 1) return launch_topk_kcap<1>(S, ld, nb_rows, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
  if (km <= 2) return launch_topk_kcap<2>(S, ld, nb_rows, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
  if (km <= 4) return launch_topk_kcap<4>(S, ld, nb_rows, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
  if (km <= 8) return launch_topk_kcap<8>(S, ld, nb_rows, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
  if (km <= 16) return launch_topk_kcap<16>(S, ld, nb_rows, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
  return launch_topk_kcap<32>(S, ld, nb_rows, r0, r1, cu_q, cu_k, batch, G, top_k, sel, sel_score, st);
}

}  // namespace msa
