// Attention output: exact softmax terms over the kept blocks' BF16 tokens plus
// Mean compensation of every other block, under one shared normaliser.
//
// CompKV page (onedev.kr/papers/157), "How it works" / "What differs": an
// unselected block b stands in for its |b| tokens with the block-mean logit
// z̄_b = q.k̄_b/sqrt(d) and the mean value v̄_b, contributing |b| e^{z̄_b} to
// the normaliser and |b| e^{z̄_b} v̄_b to the value sum; kept blocks use
// their tokens' exact terms, and both parts are normalised together.
//
// The score kernel already summed the compensation of ALL blocks, per
// chunk (one score workgroup: 32 or 64 blocks). Here workgroup p of a unit
//   * adds the exact terms of its slice of the kept list (each wave one
//     block: 16 tokens x d BF16 keys and values, 4 tokens per load),
//   * subtracts those blocks' own compensation terms |b| e^{z̄_b}(1, v̄_b),
//   * folds in up to 8 of the score kernel's chunk records,
// and writes one record; merge_kernel then combines a unit's P records into
// out and lse.
// Subtracting is safe in FP32: a kept block's exact mass sum_i e^{z_i} is at
// least its compensation mass |b| e^{z̄_b} (Jensen), so the final normaliser
// is at least the sum of all compensation masses and the rounding error of
// the subtraction stays relative to the result.
//
// dense_kernel is the full-attention baseline: every block exact, no
// compensation, a contiguous block range per workgroup.
#include "attend_core.h"

namespace cknv {

namespace {

constexpr int kBlocksPerAttendWave = 1;

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(kThreads) void attend_kernel(AttendArgs a) {
  constexpr int W = rec_words(D);
  constexpr int CAP = stage_cap<G>();
  static_assert(CAP >= kWaves + kMaxChunksPerAttendWG, "record staging too small");
  __shared__ __align__(16) float q_l[G * D];
  __shared__ __align__(16) float recs[CAP * G * W];
  __shared__ float scl[CAP * G + 3 * G];

  int unit, p;
  map_wg(blockIdx.x, a.S * a.H, a.P, a.xcd, unit, p);
  const int s = unit / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- round 1: context length, kept count, this wave's kept indices, the
  // query, this workgroup's share of the score kernel's chunk records
  const int T = a.seq_len[s];
  const int nk = a.n_sel[unit];
  int bidx[kBlocksPerAttendWave];
#pragma unroll
  for (int i = 0; i < kBlocksPerAttendWave; ++i) {
    const int it = (p * kWaves + wave) * kBlocksPerAttendWave + i;
    bidx[i] = it < a.Kb ? a.sel[(size_t)unit * a.Kb + it] : -1;
    bidx[i] = it < nk ? bidx[i] : -1;
  }
  static_assert(G * D / 4 <= kThreads, "one float4 of q per thread");
  const float4 qv = reinterpret_cast<const float4*>(a.q + (size_t)unit * G * D)[tid < G * D / 4 ? tid : G * D / 4 - 1];
  const int c0 = (int)((long)p * a.C / a.P), c1 = (int)((long)(p + 1) * a.C / a.P);
  // The no-compensation ablation has no chunk records and subtracts nothing.
  const bool nc = (a.flags & CKNV_FLAG_NO_COMPENSATION) != 0;
  const int nrec = nc ? 0 : c1 - c0;
  stage_records<D, G>(a.comp + ((size_t)unit * a.C + c0) * G * W, nrec, recs + kWaves * G * W);
  if (tid < G * D / 4) reinterpret_cast<float4*>(q_l)[tid] = qv;
  lds_barrier();

  // ---- round 2: the kept blocks' tokens, mean key and value
  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < a.max_blocks ? NB : a.max_blocks;
  const long cap_tok = (long)a.cap_blocks * kBlock;
  const size_t ubase = (size_t)unit * a.cap_blocks;
  const uint16_t* kc = a.k + (size_t)unit * cap_tok * D;
  const uint16_t* vc = a.v + (size_t)unit * cap_tok * D;
  Tile<D> tile[kBlocksPerAttendWave];
  BlockMean<D> bm[kBlocksPerAttendWave];
  bool use[kBlocksPerAttendWave];
#pragma unroll
  for (int i = 0; i < kBlocksPerAttendWave; ++i) {
    use[i] = bidx[i] >= 0 && bidx[i] < NB;
    const int b = use[i] ? bidx[i] : 0;
    tile[i].load(kc, vc, (long)b * kBlock, use[i] ? (long)T : 0, lane);
    if (use[i]) bm[i].load(a.kbar + (ubase + b) * D, a.vbar + (ubase + b) * D, a.cnt + ubase + b, lane);
  }
  WaveState<D, G> st;
  st.init();
#pragma unroll
  for (int i = 0; i < kBlocksPerAttendWave; ++i)
    if (use[i]) {
      if (nc)
        absorb<D, G, false>(st, tile[i], bm[i], q_l, lane, a.isd);
      else
        absorb<D, G, true>(st, tile[i], bm[i], q_l, lane, a.isd);
    }
  store_wave_record<D, G>(st, recs + wave * G * W, lane);
  lds_barrier();

  float* po = a.part + ((size_t)unit * a.P + p) * G * W;
  merge_records<D, G>(recs, kWaves + nrec, po, scl);
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) void dense_kernel(AttendArgs a) {
  constexpr int W = rec_words(D);
  constexpr int CAP = stage_cap<G>();
  __shared__ __align__(16) float q_l[G * D];
  __shared__ __align__(16) float recs[CAP * G * W];
  __shared__ float scl[CAP * G + 3 * G];

  int unit, p;
  map_wg(blockIdx.x, a.S * a.H, a.P, a.xcd, unit, p);
  const int s = unit / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.seq_len[s];
  const float4 qv = reinterpret_cast<const float4*>(a.q + (size_t)unit * G * D)[tid < G * D / 4 ? tid : G * D / 4 - 1];
  if (tid < G * D / 4) reinterpret_cast<float4*>(q_l)[tid] = qv;
  lds_barrier();
  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < a.max_blocks ? NB : a.max_blocks;
  const long cap_tok = (long)a.cap_blocks * kBlock;
  const uint16_t* kc = a.k + (size_t)unit * cap_tok * D;
  const uint16_t* vc = a.v + (size_t)unit * cap_tok * D;
  const int lo = p * a.BPW, hi = min(lo + a.BPW, NB);
  WaveState<D, G> st;
  st.init();
  BlockMean<D> none;
  for (int b = lo + 2 * wave; b < hi; b += 2 * kWaves) {
    Tile<D> t0, t1;
    const bool u1 = b + 1 < hi;
    t0.template load<true>(kc, vc, (long)b * kBlock, T, lane);
    t1.template load<true>(kc, vc, (long)(u1 ? b + 1 : b) * kBlock, u1 ? (long)T : 0, lane);  // a valid block even when unused
    absorb<D, G, false>(st, t0, none, q_l, lane, a.isd);
    if (u1) absorb<D, G, false>(st, t1, none, q_l, lane, a.isd);
  }
  store_wave_record<D, G>(st, recs + wave * G * W, lane);
  lds_barrier();
  merge_records<D, G>(recs, kWaves, a.part + ((size_t)unit * a.P + p) * G * W, scl);
}

// One workgroup per unit: merge the unit's P part records into out and lse.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttendArgs a) {
  constexpr int W = rec_words(D);
  constexpr int CAP = stage_cap<G>();
  __shared__ __align__(16) float recs[CAP * G * W];
  __shared__ float scl[CAP * G + 3 * G];
  const int unit = blockIdx.x;
  finish_unit<D, G>(a.part + (size_t)unit * a.P * G * W, a.P, a.out + (size_t)unit * G * D,
                    a.lse ? a.lse + (size_t)unit * G : nullptr, recs, CAP, scl);
}

hipError_t launch_attend(int d, int G, bool dense, const AttendArgs& a, int U, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* f = nullptr;
  const void* m = nullptr;
#define CKNV_ATT_CASE(DD, GG)                                                                  \
  if (d == DD && G == GG) {                                                                    \
    f = dense ? (const void*)dense_kernel<DD, GG> : (const void*)attend_kernel<DD, GG>;        \
    m = (const void*)merge_kernel<DD, GG>;                                                     \
  }
  CKNV_ATT_CASE(64, 1) CKNV_ATT_CASE(64, 2) CKNV_ATT_CASE(64, 4) CKNV_ATT_CASE(64, 8)
  CKNV_ATT_CASE(128, 1) CKNV_ATT_CASE(128, 2) CKNV_ATT_CASE(128, 4) CKNV_ATT_CASE(128, 8)
#undef CKNV_ATT_CASE
  if (!f || !m) return hipErrorInvalidValue;
  hipError_t e = hipLaunchKernel(f, dim3(U * a.P), dim3(kThreads), args, 0, st);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(m, dim3(U), dim3(kThreads), args, 0, st);
}

}  // namespace cknv
