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
// compensation, the unit's blocks dealt round-robin over the waves of its
// workgroups.
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

// Full attention, every block exact, no compensation: P workgroups of
// kDenseThreads threads per unit, the unit's blocks dealt round-robin over
// all their waves, each wave keeping several tiles of non-temporal loads in
// flight, logits on MFMA; the waves' records merge into the workgroup's part
// record, and merge_kernel merges the P part records.
template <int D, int G>
__global__ __launch_bounds__(kDenseThreads) void dense_kernel(AttendArgs a) {
  constexpr int W = rec_words(D);
  constexpr int NWV = kDenseThreads / 64;
  __shared__ __align__(16) float q_l[G * D];
  __shared__ __align__(16) float recs[NWV * G * W];
  __shared__ float scl[NWV * G + 3 * G];
  __shared__ __align__(16) float pbuf[NWV * 16 * G];

  int unit, p;
  map_wg(blockIdx.x, a.S * a.H, a.P, a.xcd, unit, p);
  const int s = unit / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  static_assert(G * D / 4 <= kDenseThreads, "one float4 of q per thread");
  const float4 qv = reinterpret_cast<const float4*>(a.q + (size_t)unit * G * D)[tid < G * D / 4 ? tid : G * D / 4 - 1];
  const int T = a.seq_len[s];
  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < a.max_blocks ? NB : a.max_blocks;
  const long cap_tok = (long)a.cap_blocks * kBlock;
  const uint16_t* kc = a.k + (size_t)unit * cap_tok * D;
  const uint16_t* vc = a.v + (size_t)unit * cap_tok * D;
  // The unit's blocks are dealt round-robin over all its workgroups' waves
  // (wave w of part p takes blocks p*NWV + w + k*P*NWV): at any moment the
  // unit's waves read one contiguous stretch of the cache, spread over every
  // memory channel, rather than P far-apart streams in lockstep.
  const int stride = a.P * NWV;
  // This wave's tiles are blocks b0, b0 + stride, ... below NB (n_w of
  // them). Up to 4 query heads the wave keeps two tiles in flight: tile j+1's
  // loads are issued before tile j is absorbed. The loop body is straight
  // line and every load unconditional, so each wait counts only the older
  // tile's loads; past the wave's last tile a slot is empty (no valid
  // token, its loads re-read the last tile from the cache). The first tile's
  // loads go out before the query is staged.
  const int b0 = p * NWV + wave;
  const int n_w = b0 < NB ? (NB - 1 - b0) / stride + 1 : 0;
  const int blast = n_w > 0 ? b0 + (n_w - 1) * stride : 0;
  auto tile_at = [&](TileM<D>& t, int j) {
    const bool in = j < n_w;
    load_tile_whole<D>(t, kc, vc, (long)(in ? b0 + j * stride : blast) * kBlock, in ? T : 0, lane);
  };
  TileM<D> t0;
  tile_at(t0, 0);
  if (tid < G * D / 4) reinterpret_cast<float4*>(q_l)[tid] = qv;
  lds_barrier();
  WaveState<D, G> st;
  st.init();
  BlockMean<D> none;
#pragma unroll
  for (int e = 0; e < D / 64; ++e) none.kb[e] = none.vb[e] = 0.f;
  none.n = 0.f;
  none.on = false;
  QMfma<D> qm;
  qm.template build<G>(q_l, lane);
  float* pw = pbuf + wave * 16 * G;
  if constexpr (G >= 8) {
    // eight query heads: one tile at a time (a second does not fit the registers)
    for (int j = 0; j < n_w; ++j) {
      if (j > 0) tile_at(t0, j);
      __builtin_amdgcn_sched_barrier(0);
      absorb_mfma<D, G, false>(st, t0, none, qm, q_l, pw, lane, a.isd);
    }
  } else {
    TileM<D> t1;
    // (the barriers keep each tile's last use ahead of its reload, so that the
    // reload lands in the same registers: a copy would wait for the loads)
    for (int j = 0; j < n_w; j += 2) {
      tile_at(t1, j + 1);
      __builtin_amdgcn_sched_barrier(0);  // the next tile's loads issued before this one is used
      absorb_mfma<D, G, false>(st, t0, none, qm, q_l, pw, lane, a.isd);
      __builtin_amdgcn_sched_barrier(0);
      tile_at(t0, j + 2);
      __builtin_amdgcn_sched_barrier(0);
      absorb_mfma<D, G, false>(st, t1, none, qm, q_l, pw, lane, a.isd);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  store_wave_record<D, G>(st, recs + wave * G * W, lane);
  lds_barrier();
  merge_records<D, G, kDenseThreads>(recs, NWV, a.part + ((size_t)unit * a.P + p) * G * W, scl);
}

// Merge each unit's P part records into out and lse: kMergeCols workgroups
// per unit, one output column per thread, all of a column's records loaded
// in one round trip (up to 32 parts).
constexpr int kMergeCols = kThreads;
template <int D, int G>
constexpr int merge_wgs() { return (G * D + kMergeCols - 1) / kMergeCols; }

template <int D, int G>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttendArgs a) {
  constexpr int W = rec_words(D), CB = merge_wgs<D, G>();
  const int unit = blockIdx.x / CB, cb = blockIdx.x - unit * CB;
  merge_parts<D, G, kMergeCols, 32, 1, false>(a.part + (size_t)unit * a.P * G * W, a.P,
                                              a.out + (size_t)unit * G * D,
                                              a.lse ? a.lse + (size_t)unit * G : nullptr, cb * kMergeCols);
}

hipError_t launch_attend(int d, int G, bool dense, const AttendArgs& a, int U, hipStream_t st) {
  void* args[] = {(void*)&a};
  const void* f = nullptr;
  const void* m = nullptr;
  int mw = 0;
#define CKNV_ATT_CASE(DD, GG)                                                                  \
  if (d == DD && G == GG) {                                                                    \
    f = dense ? (const void*)dense_kernel<DD, GG> : (const void*)attend_kernel<DD, GG>;        \
    m = (const void*)merge_kernel<DD, GG>;                                                     \
    mw = merge_wgs<DD, GG>();                                                                  \
  }
  CKNV_ATT_CASE(64, 1) CKNV_ATT_CASE(64, 2) CKNV_ATT_CASE(64, 4) CKNV_ATT_CASE(64, 8)
  CKNV_ATT_CASE(128, 1) CKNV_ATT_CASE(128, 2) CKNV_ATT_CASE(128, 4) CKNV_ATT_CASE(128, 8)
#undef CKNV_ATT_CASE
  if (!f || !m) return hipErrorInvalidValue;
  hipError_t e = hipLaunchKernel(f, dim3(U * a.P), dim3(dense ? kDenseThreads : kThreads), args, 0, st);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(m, dim3(U * mw), dim3(kThreads), args, 0, st);
}

}  // namespace cknv
