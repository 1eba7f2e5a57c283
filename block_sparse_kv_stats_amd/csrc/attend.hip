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
//     block: 16 tokens x d BF16 keys and values, logits on MFMA),
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
  __shared__ __align__(16) float q_m[QMfma<D>::template lds_words<G>()];  // the query, for the MFMA operand
  __shared__ __align__(16) float recs[CAP * G * W];
  __shared__ float scl[CAP * G + 3 * G];
  __shared__ __align__(16) float pbuf[kWaves * 16 * G];  // the waves' tile probabilities

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
  if (tid < G * D / 4) {
    reinterpret_cast<float4*>(q_l)[tid] = qv;
    QMfma<D>::stage(q_m, tid, qv);
  }
  lds_barrier();

  // ---- round 2: the kept blocks' tokens, mean key and value (logits on MFMA)
  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < a.max_blocks ? NB : a.max_blocks;
  const long cap_tok = (long)a.cap_blocks * kBlock;
  const size_t ubase = (size_t)unit * a.cap_blocks;
  const uint16_t* kc = a.k + (size_t)unit * cap_tok * D;
  const uint16_t* vc = a.v + (size_t)unit * cap_tok * D;
  TileM<D> tile[kBlocksPerAttendWave];
  BlockMean<D> bm[kBlocksPerAttendWave];
  bool use[kBlocksPerAttendWave];
#pragma unroll
  for (int i = 0; i < kBlocksPerAttendWave; ++i) {
    use[i] = bidx[i] >= 0 && bidx[i] < NB;
    const int b = use[i] ? bidx[i] : 0;
    if (use[i]) bm[i].load(a.kbar + (ubase + b) * D, a.vbar + (ubase + b) * D, a.cnt + ubase + b, lane);
    tile[i].load(kc, vc, (long)b * kBlock, use[i] ? (long)T : 0, lane);
  }
  QMfma<D> qm;
  qm.template build_from<G>(QMfma<D>::template fetch_lds<G>(q_m, lane), lane);
  float* pw = pbuf + wave * 16 * G;
  WaveState<D, G> st;
  st.init();
#pragma unroll
  for (int i = 0; i < kBlocksPerAttendWave; ++i)
    if (use[i]) {
      if (nc)
        absorb_mfma<D, G, false>(st, tile[i], bm[i], qm, q_l, pw, lane, a.isd);
      else
        absorb_mfma<D, G, true>(st, tile[i], bm[i], qm, q_l, pw, lane, a.isd);
    }
  store_wave_record<D, G>(st, recs + wave * G * W, lane);
  lds_barrier();

  float* po = a.part + ((size_t)unit * a.P + p) * G * W;
  merge_records<D, G>(recs, kWaves + nrec, po, scl);
}

namespace {

// The dense kernel's tiles: the keys as the logits MFMA reads them (lane l,
// token l%16), the values in 16-byte pieces: load i, lane l holds token
// 4i + l/16, coordinates VP*(l%16) .. +VP-1 (VP = d/16), so a tile's values
// take 4 loads per lane (a bandwidth-bound stream is bound by its load
// instructions as well as its bytes). Token rows past the last valid one
// read that one (their probabilities are 0).
template <int D>
struct TileW {
  static constexpr int NI = D / 32, VP = D / 16, VW = VP / 2;
  u32x4_t k[NI];
  uint32_t v[4][VW];
  int nt;  // valid tokens
  __device__ void load(const uint16_t* kc, const uint16_t* vc, long tok0, long T, int lane) {
    const long left = T - tok0;
    nt = left <= 0 ? 0 : (left >= 16 ? 16 : (int)left);
    const int last = nt > 0 ? nt - 1 : 0;
    const int t = lane & 15, c = lane >> 4;
    const uint16_t* ks = kc + (size_t)(tok0 + (t < last ? t : last)) * D + (D / 4) * c;
#pragma unroll
    for (int i = 0; i < NI; ++i) k[i] = ldg<false>(reinterpret_cast<const u32x4_t*>(ks + 8 * i));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * i + c;
      const uint16_t* vs = vc + (size_t)(tok0 + (row < last ? row : last)) * D + VP * t;
      if constexpr (VW == 4) {
        const uint4 x = stream_load_u4<false>(vs);
        v[i][0] = x.x; v[i][1 % VW] = x.y; v[i][2 % VW] = x.z; v[i][3 % VW] = x.w;
      } else {
        const uint2 x = stream_load_u2<false>(vs);
        v[i][0] = x.x; v[i][1 % VW] = x.y;
      }
    }
  }
};

// Running state of a dense wave: per query head the max m and normaliser l
// (wave-uniform) and the value sums of the lane's VP coordinates over the
// tokens 4i + l/16 it has seen (summed over the four lane groups at the end).
template <int D, int G>
struct WaveStateW {
  static constexpr int VP = D / 16;
  float m[G], l[G], acc[G][VP];
  __device__ void init() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < VP; ++e) acc[g][e] = 0.f;
    }
  }
};

// Add one tile's exact terms (logits on MFMA, probabilities through the
// wave's LDS scratch `pw` of 16*G floats). A tile with no valid token adds
// nothing.
template <int D, int G>
__device__ __forceinline__ void absorb_w(WaveStateW<D, G>& st, const TileW<D>& t, const QMfma<D>& qm,
                                         float* pw, int lane, float isd) {
  constexpr int NI = D / 32, VP = D / 16, VW = VP / 2;
  const int j = lane & 15, c = lane >> 4;
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, t.k[i]);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qm.hi[i], s, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qm.lo[i], s, 0, 0, 0);
  }
  float z[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) z[e] = 4 * c + e < t.nt ? s[e] * isd : -INFINITY;
  const float cmax = rows_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));  // head j's tile max
  float M[G], sc[G];
  float Mj = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    M[g] = fmaxf(st.m[g], lane_value(cmax, g));
    sc[g] = rescale(st.m[g], M[g]);
    Mj = j == g ? M[g] : Mj;
  }
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) p[e] = z[e] == -INFINITY ? 0.f : __expf(z[e] - Mj);
  const float ps = rows_sum((p[0] + p[1]) + (p[2] + p[3]));
  if (j < G) {
#pragma unroll
    for (int e = 0; e < 4; ++e) pw[(4 * c + e) * G + j] = p[e];
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.l[g] = st.l[g] * sc[g] + lane_value(ps, g);
    st.m[g] = M[g];
#pragma unroll
    for (int e = 0; e < VP; ++e) st.acc[g][e] *= sc[g];
  }
  // lanes read the probabilities other lanes of the wave just wrote: the
  // fence keeps the reads after the writes (the wave's LDS operations then
  // run in program order)
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  if (t.nt > 0) {  // wave-uniform; an empty tile's rows may hold anything
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float pv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) pv[g] = pw[(4 * i + c) * G + g];
#pragma unroll
      for (int w = 0; w < VW; ++w) {
        const float lo = bf16_lo(t.v[i][w]), hi = bf16_hi(t.v[i][w]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          st.acc[g][2 * w] += pv[g] * lo;
          st.acc[g][2 * w + 1] += pv[g] * hi;
        }
      }
    }
  }
  // the next tile's probability writes must not pass these reads
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Write a WaveStateW's record [m, l, 0, 0, acc[D]] per g (value sums summed
// over the four lane groups).
template <int D, int G>
__device__ __forceinline__ void store_wave_record_w(const WaveStateW<D, G>& st, float* rec, int lane) {
  constexpr int VP = D / 16, W = rec_words(D);
  const int t = lane & 15, c = lane >> 4;
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < VP; ++e) {
      const float x = rows_sum(st.acc[g][e]);
      if (c == 0) rec[g * W + 4 + VP * t + e] = x;
    }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      rec[g * W] = st.m[g];
      rec[g * W + 1] = st.l[g];
      rec[g * W + 2] = 0.f;
      rec[g * W + 3] = 0.f;
    }
  }
}

}  // namespace

// Full attention, every block exact, no compensation: P workgroups of
// kDenseThreads threads per unit, the unit's blocks dealt round-robin over
// all their waves, each wave keeping several tiles of plain loads in
// flight, logits on MFMA; the waves' records merge into the workgroup's part
// record, and merge_kernel merges the P part records.
template <int D, int G>
__global__ __launch_bounds__(kDenseThreads) void dense_kernel(AttendArgs a) {
  constexpr int W = rec_words(D);
  constexpr int NWV = kDenseThreads / 64;
  __shared__ __align__(16) float recs[NWV * G * W];
  __shared__ float scl[NWV * G + 3 * G];
  __shared__ __align__(16) float pbuf[NWV * 16 * G];
  __shared__ __align__(16) float q_m[QMfma<D>::template lds_words<G>()];  // the query, for the MFMA operand

  int unit, p;
  map_wg(blockIdx.x, a.S * a.H, a.P, a.xcd, unit, p);
  const int s = unit / a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  // token, its loads re-read the last tile from the cache). The query is
  // read once per workgroup into an LDS copy that every wave builds its
  // MFMA operand from (read by every wave from global memory, it was 8 KB of
  // L1 traffic per wave ahead of the first tile).
  const int b0 = p * NWV + wave;
  const int n_w = b0 < NB ? (NB - 1 - b0) / stride + 1 : 0;
  const int blast = n_w > 0 ? b0 + (n_w - 1) * stride : 0;
  auto tile_at = [&](TileW<D>& t, int j) {
    const bool in = j < n_w;
    t.load(kc, vc, (long)(in ? b0 + j * stride : blast) * kBlock, in ? T : 0, lane);
  };
  static_assert(G * D / 4 <= kDenseThreads, "one float4 of the query per thread");
  const float4 qv = reinterpret_cast<const float4*>(a.q + (size_t)unit * G * D)[tid < G * D / 4 ? tid : 0];
  TileW<D> t0;
  tile_at(t0, 0);
  if (tid < G * D / 4) QMfma<D>::stage(q_m, tid, qv);
  lds_barrier();
  WaveStateW<D, G> st;
  st.init();
  QMfma<D> qm;
  qm.template build_from<G>(QMfma<D>::template fetch_lds<G>(q_m, lane), lane);
  float* pw = pbuf + wave * 16 * G;
  if constexpr (G >= 8) {
    // eight query heads: one tile at a time (a second does not fit the registers)
    for (int j = 0; j < n_w; ++j) {
      if (j > 0) tile_at(t0, j);
      __builtin_amdgcn_sched_barrier(0);
      absorb_w<D, G>(st, t0, qm, pw, lane, a.isd);
    }
  } else {
    TileW<D> t1;
    // (the barriers keep each tile's last use ahead of its reload, so that the
    // reload lands in the same registers: a copy would wait for the loads)
    for (int j = 0; j < n_w; j += 2) {
      tile_at(t1, j + 1);
      __builtin_amdgcn_sched_barrier(0);  // the next tile's loads issued before this one is used
      absorb_w<D, G>(st, t0, qm, pw, lane, a.isd);
      __builtin_amdgcn_sched_barrier(0);
      tile_at(t0, j + 2);
      __builtin_amdgcn_sched_barrier(0);
      absorb_w<D, G>(st, t1, qm, pw, lane, a.isd);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  store_wave_record_w<D, G>(st, recs + wave * G * W, lane);
  lds_barrier();
  merge_records<D, G, kDenseThreads>(recs, NWV, a.part + ((size_t)unit * a.P + p) * G * W, scl);
}

// Merge each unit's P part records into out and lse. A workgroup takes 64
// output columns of one unit; its four waves each merge every fourth part
// record for those columns (8 records per round trip, lane = column, so a
// record's values are one coalesced 256-byte read and its (m, l) one
// broadcast), and the four partial (M, L, A) are combined through the LDS.
// Splitting the records over waves keeps each thread's load count at P/4:
// with one thread per column taking all P records, the loads' issue, not
// their latency, set the kernel's time.
constexpr int kMergeCols = 64;
template <int D, int G>
constexpr int merge_wgs() { return G * D / kMergeCols; }

template <int D, int G>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttendArgs a) {
  constexpr int W = rec_words(D), CB = merge_wgs<D, G>(), Q = kThreads / kMergeCols, RB = 8;
  static_assert(D % kMergeCols == 0, "a workgroup's columns lie in one head");
  __shared__ float part_s[Q][3][kMergeCols];
  const int unit = blockIdx.x / CB, cb = blockIdx.x - unit * CB;
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int col = cb * kMergeCols + lane, g = col / D, c = col - g * D;
  const int P = a.P;
  const float* parts = a.part + (size_t)unit * P * G * W + (size_t)g * W;
  float M = -INFINITY, L = 0.f, A = 0.f;
  for (int i0 = q; i0 < P; i0 += Q * RB) {
    float m[RB], l[RB], x[RB];
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const int i = i0 + Q * k;
      const float* r = parts + (size_t)(i < P ? i : P - 1) * G * W;
      m[k] = r[0] + (i < P ? 0.f : -INFINITY);  // a slot past the last record weighs 0
      l[k] = r[1];
      x[k] = r[4 + c];
    }
    float MM = M;
#pragma unroll
    for (int k = 0; k < RB; ++k) MM = fmaxf(MM, m[k]);
    const float so = rescale(M, MM);
    L *= so;
    A *= so;
#pragma unroll
    for (int k = 0; k < RB; ++k) {
      const float f = rescale(m[k], MM);
      L += l[k] * f;
      A += x[k] * f;
    }
    M = MM;
  }
  part_s[q][0][lane] = M;
  part_s[q][1][lane] = L;
  part_s[q][2][lane] = A;
  lds_barrier();
  if (q == 0) {
    float MM = -INFINITY;
#pragma unroll
    for (int k = 0; k < Q; ++k) MM = fmaxf(MM, part_s[k][0][lane]);
    float LL = 0.f, AA = 0.f;
#pragma unroll
    for (int k = 0; k < Q; ++k) {
      const float f = rescale(part_s[k][0][lane], MM);
      LL += part_s[k][1][lane] * f;
      AA += part_s[k][2][lane] * f;
    }
    const bool ok = LL > 0.f;
    a.out[(size_t)unit * G * D + col] = ok ? AA / LL : 0.f;
    if (c == 0 && a.lse) a.lse[(size_t)unit * G + g] = ok ? MM + __logf(LL) : -INFINITY;
  }
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
