// The fused decode step after the scoring pass: normalisers, selection and
// attention of one unit in one workgroup (or in P workgroups that each
// attend a slice of the kept list; the last of them to finish merges all
// P partial records).
//
// CompKV page (onedev.kr/papers/157):
//   "What differs"  -- p̂ is normalised over all blocks, S_b = sum_g p̂ σ̂²;
//     the first block and the two most recent blocks are always kept and
//     count against the budget, the rest of the budget goes to the largest
//     S_b (ties: lower block index);
//   "How it works"  -- kept blocks contribute their tokens' exact terms,
//     every other block its Mean compensation |b| e^{z̄} (1, v̄), all under
//     one normaliser.
//
// Inputs from the scoring pass (score_kernel in fused mode). It appended the
// step's token, summarised the block the token lands in (the fresh block,
// index T0/16, T0 = tokens before the step) and wrote that block's a and
// factor per query head (finfo). It covered the NBa = T0/16 blocks closed
// before the step: per score group the (max, sum) of a = ln|b| + z̄ + σ̂²/2,
// per block u_{g,b} = exp(a - group max) σ̂², per chunk the Mean-compensation
// sums of all its blocks and the chunk's (max, sum) of a, and T0 per
// sequence. The fresh block is in none of the sums: it is always kept.
//
// Phases of a workgroup (NT threads; for the loads and the keys thread t
// owns blocks t + NT*j of the unit, coalesced; from the selection on it owns
// the run of KPTB consecutive blocks t*KPTB ..):
//   loads      T0, finfo, the chunk headers, the thread's score groups and
//              u terms, the query, and (waves AW..NW-1) their first chunk
//              records;
//   LSE        wave g reduces query head g's chunk headers and the fresh
//              block's a to LSE_g, shared through LDS; factors
//              e^{group max - LSE} of the thread's score groups to LDS;
//   keys       S_b per block (fp32 bits order like the values, S_b >= 0);
//              scores; 2048-bin histogram of the candidates' key bits
//              30..20 (S >= 0, so bit 31 is 0: all 2048 bins are used);
//              the keys through LDS into the threads' contiguous runs;
//   select     the bin holding the (Kb-3)-th largest candidate key; keys
//              in that bin are ranked exactly (or, for long runs of equal
//              keys, pinned by two more radix passes, ties by index);
//   compact    kept blocks in ascending order (one workgroup scan of the
//              per-thread counts) -> sel, and this part's slice;
//   attend     waves w < AW: kept block w of this part's slice (exact terms
//              minus its compensation); meanwhile waves w >= AW fold this
//              part's chunk records;
//   merge      the waves' records -> out, lse (P == 1) or a part record
//              and its (m, l) pairs; the part that completes the unit's count
//              merges the P part records into out and lse.
#include "attend_core.h"
#include "select_core.h"
#include "step_config.h"

namespace cknv {

namespace {

// First histogram pass: key >> 20, 2048 bins over the exponent and three
// mantissa bits of S (its sign bit is 0). Long runs of equal keys are pinned
// by two more passes, over bits 19..9 (2048 bins) and 8..0 (512 bins).
constexpr int kBinShift = 20;

template <int D, int G, int KPTB>
struct StepCfg {
  static constexpr int NT = kStepThreads;
  static constexpr int NW = kStepWaves;
  static constexpr int KPT = KPTB;                                 // blocks per thread
  static constexpr int NGMAX = (NT * KPT + kScoreMinGroup - 1) / kScoreMinGroup;  // score groups, at most
  static constexpr int GPT = (NGMAX + NT - 1) / NT;                // score groups per thread
  static constexpr int UMAX = G >= 8 ? 64 / G : 128 / G;
  static constexpr int UB = KPT < UMAX ? KPT : UMAX;               // blocks per u load batch
  static constexpr int NBATCH = (KPT + UB - 1) / UB;
  static constexpr int KPART = kStepAttendWaves * kStepMaxKeptPerWave;  // kept blocks per workgroup, at most
  static constexpr int CPL = step_chunks_per_lane(KPTB);           // chunk headers per lane
  // Chunk records per record-folding wave loaded with the inputs (what the
  // registers left by the other inputs hold, 1..4), and per later batch.
  static constexpr int RWORDS = G * (2 + D / 64);
  static constexpr int RBUDGET = 112 - UB * G - 2 * GPT * G - 2 * CPL;
  static constexpr int RPF = RBUDGET / RWORDS < 1 ? 1 : (RBUDGET / RWORDS > 4 ? 4 : RBUDGET / RWORDS);
  static constexpr int RPW = 32 / RWORDS < 1 ? 1 : (32 / RWORDS > 4 ? 4 : 32 / RWORDS);
  static constexpr int AW = kStepAttendWaves;                      // attending waves
  static constexpr int RW = NW - AW;                               // record-folding waves
  static_assert(AW < NW, "record-folding waves");
};

// The lane's part of one chunk record of the scoring pass: (m, l) and the
// lane's value coordinates per query head; an empty record when !valid.
// `valid` is wave-uniform: an empty record issues no load.
template <int D, int G>
struct RecordRegs {
  float m[G], l[G], acc[G][D / 64];
  __device__ __forceinline__ void load(const float* rp, bool valid, int lane) {
    constexpr int W = rec_words(D), VPL = D / 64;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) acc[g][e] = 0.f;
    }
    if (valid) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float2 ml = *reinterpret_cast<const float2*>(rp + g * W);
        m[g] = ml.x;
        l[g] = ml.y;
#pragma unroll
        for (int e = 0; e < VPL; ++e) acc[g][e] = rp[g * W + 4 + lane * VPL + e];
      }
    }
  }
};

// out[g][c] = sum_i rec_i[g][c] e^{m_i - M} / L (and lse = M + ln L) over n
// records in LDS.
template <int D, int G, int NT>
__device__ __forceinline__ void finalize_records(const float* recs, int n, float* out, float* lse,
                                                 float* scl) {
  constexpr int W = rec_words(D);
  const int tid = threadIdx.x;
  float* ML = scl + n * G;  // [G] (M, L)
  if (tid < G) {
    float M = -INFINITY, L = 0.f;
    record_scales<D, G>(recs, n, tid, scl, M, L, nullptr);
    ML[2 * tid] = M;
    ML[2 * tid + 1] = L;
  }
  lds_barrier();
  for (int col = tid; col < G * D; col += NT) {
    const int g = col / D, c = col - g * D;
    const float L = ML[2 * g + 1];
    const bool ok = L > 0.f;
    const float A = record_column<D, G>(recs, scl, n, g, c);
    out[col] = ok ? A / L : 0.f;
    if (c == 0 && lse) lse[g] = ok ? ML[2 * g] + __logf(L) : -INFINITY;
  }
}

// Fold one compensation record (this lane's coordinates) into a wave state.
template <int D, int G>
__device__ __forceinline__ void fold_record(WaveState<D, G>& st, const RecordRegs<D, G>& r) {
  constexpr int VPL = D / 64;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = fmaxf(st.m[g], r.m[g]);
    const float a = rescale(st.m[g], M), b = rescale(r.m[g], M);
    st.m[g] = M;
    st.l[g] = st.l[g] * a + r.l[g] * b;
#pragma unroll
    for (int e = 0; e < VPL; ++e) st.acc[g][e] = st.acc[g][e] * a + r.acc[g][e] * b;
  }
}

}  // namespace

// A sequence appends (and its seq_len advances) when its cache has room and
// the block the token lands in lies below max_blocks.
__device__ __forceinline__ bool step_appends(int T0, int cap_blocks, int max_blocks) {
  return T0 < (long)cap_blocks * kBlock && T0 / kBlock < max_blocks;
}

template <int D, int G, int KPTB>
__global__ __launch_bounds__(kStepThreads) void step_kernel(StepArgs a) {
  using C = StepCfg<D, G, KPTB>;
  constexpr int NT = C::NT, NW = C::NW, KPT = C::KPT, UB = C::UB;
  constexpr int GPT = C::GPT, NGMAX = C::NGMAX, KPART = C::KPART, AW = C::AW;
  constexpr int RW = C::RW;
  constexpr int CPL = C::CPL, RPF = C::RPF, RPW = C::RPW;
  constexpr int W = rec_words(D);
  // LDS: area A holds the score-group factors during the keys, then the
  // waves' attention records; the query has its own array.
  constexpr int NBITS = (KPT * NT + 31) / 32;  // kept-block bitmap of the pivot-bin path
  constexpr int A_WORDS = NGMAX * G > NW * G * W ? NGMAX * G : NW * G * W;
  __shared__ __align__(16) float areaA[A_WORDS];
  __shared__ __align__(16) float q_l[G * D];  // the G query heads
  __shared__ __align__(16) float q_m[QMfma<D>::template lds_words<G>()];  // the same, for the MFMA operand
  __shared__ __align__(16) int hist[2048];
  __shared__ __align__(16) uint64_t plist[kListMax + kListPad];  // pivot-bin (key, index) words
  __shared__ uint32_t keys_l[KPT * NT];                            // every block's key, block order
  __shared__ uint32_t keep_bits[NBITS];
  __shared__ int cnt[KPT * NW + 1];
  __shared__ float scl[NW * G + 2 * G];
  __shared__ int ctl[8];
  __shared__ float lse_s[G];  // the normalisers LSE_g
  __shared__ int klist[KPART];
  __shared__ __align__(16) float pbuf[AW * 16 * G];  // attending waves' tile probabilities
  float* fgrp = areaA;                   // [NGMAX][G] exp(group max - LSE_g)
  float* recs = areaA;                   // [NW][G][W] after the selection

  const int P = a.P;
  // The input loads' kernel arguments are read with the first batch (left to
  // the compiler, they came in a second round trip after the part mapping).
  // (Not for 8 query heads at the largest bucket: their registers are full.)
  if constexpr (G < 8 || KPTB < 24) asm volatile("" ::"s"(a.t0), "s"(a.u), "s"(a.hdr), "s"(a.finfo));
  // the parts of a unit run on the XCD whose L2 the scoring pass wrote that
  // unit's workspace through
  int unit, p;
  map_wg(blockIdx.x, a.S * a.H, P, a.xcd, unit, p);
  const int s = unit / a.H, h = unit - s * a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int MB = a.max_blocks, Kb = a.Kb, NC = a.C;
  const long cap_tok = (long)a.cap_blocks * kBlock;
  const size_t ubase = (size_t)unit * a.cap_blocks;
  const uint16_t* kc = a.k + (size_t)unit * cap_tok * D;
  const uint16_t* vc = a.v + (size_t)unit * cap_tok * D;
  const float* u = a.u + (size_t)unit * MB * G;
  const float2* grp = reinterpret_cast<const float2*>(a.grp) + (size_t)unit * a.NG * G;
  const float* crec = a.comp + (size_t)unit * NC * G * W;
  const int NG = a.NG;
  // The no-compensation ablation has no records: folds see empty ones.
  const bool nc = (a.flags & CKNV_FLAG_NO_COMPENSATION) != 0;
  // thread tid owns blocks tid + NT*j, j < KPT (NT*KPT >= MB), and score
  // groups tid + NT*k, k < GPT

  // ================================================================ loads
  // T0 and finfo are the same for the whole workgroup: scalar loads, issued
  // first (left to the scheduler they went out after the vector loads)
  const int T0 = load_uniform(a.t0 + s);
  float2 fi[G];
  load_pairs_uniform<G>(reinterpret_cast<const float2*>(a.finfo) + (size_t)unit * G, fi);
  __builtin_amdgcn_sched_barrier(0);
  // chunk lane + 64k: (max, sum) of a for query head `wave` (waves < G; the
  // others form no normaliser: they read head 0's, 8 bytes a lane, unused)
  float2 hd[CPL];
  {
    const float2* hp = reinterpret_cast<const float2*>(a.hdr) + (size_t)unit * NC * G + (wave < G ? wave : 0);
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane + 64 * k;
      const int cc = c < NC ? c : NC - 1;
      hd[k] = hp[(size_t)cc * G];
    }
  }
  float2 gp[GPT][G];
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int gi = tid + k * NT;
    const int gc = gi < NG ? gi : NG - 1;
    load_pairs<G>(grp + (size_t)gc * G, gp[k]);
  }
  constexpr int NQ4 = (G * D / 4 + NT - 1) / NT;
  float4 q4[NQ4];
#pragma unroll
  for (int k = 0; k < NQ4; ++k) {
    const int i = tid + k * NT;
    q4[k] = reinterpret_cast<const float4*>(a.q + (size_t)unit * G * D)[i < G * D / 4 ? i : 0];
  }
  // the u terms last: the normalisers need only what came before them (the
  // barrier keeps the scheduler from moving the loads above, the query and
  // finfo among them, behind the u terms: every wait for them would then
  // also wait for the u terms)
  __builtin_amdgcn_sched_barrier(0);
  float uv[UB][G];
#pragma unroll
  for (int j = 0; j < UB; ++j) {
    const int b = tid + j * NT;
    const int bc = b < MB ? b : MB - 1;
    load_row<G>(u + (size_t)bc * G, uv[j]);
  }
  // This part's chunk records are folded by the waves that attend no tile
  // (w >= AW), while the others attend: wave w folds records
  // c0 + (w - AW) + RW*i. The first RPF are loaded now; they do not depend
  // on the selection.
  // (32-bit: p*NC stays below 2^31, NC <= 384 and P <= 12288/4)
  const int c0 = (int)((unsigned)(p * NC) / (unsigned)P), c1 = (int)((unsigned)((p + 1) * NC) / (unsigned)P);
  const int clast = c1 > 0 ? c1 - 1 : 0;
  const int rw = wave - AW;  // record wave index (negative: an attending wave)
  RecordRegs<D, G> rf[RPF];
#pragma unroll
  for (int i = 0; i < RPF; ++i) {
    const int c = c0 + rw + RW * i;
    rf[i].load(crec + (size_t)(c < c1 ? c : clast) * G * W, rw >= 0 && c < c1 && !nc, lane);
  }
  __builtin_amdgcn_sched_barrier(0);

  const bool app = step_appends(T0, a.cap_blocks, MB);
  const int T = T0 + (app ? 1 : 0);
  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < MB ? NB : MB;
  int NBa = T0 / kBlock;
  NBa = NBa < MB ? NBa : MB;
  const int fb = app ? T0 / kBlock : -1;  // fresh block (always the last block)
  const int gsh = a.bpw_shift;  // score group = 1 << gsh blocks
  const int NGa = (NBa + (1 << gsh) - 1) >> gsh;
  const bool all = NB <= Kb;
  int krem = Kb - 3;
  const bool count = !all && krem > 0;
  for (int i = tid; i < 2048; i += NT) hist[i] = 0;
  for (int i = tid; i < NBITS; i += NT) keep_bits[i] = 0u;
  for (int i = tid; i < kListMax + kListPad; i += NT) plist[i] = 0ull;
  if (tid == 0) ctl[3] = 0;

  // ================================================================ LSE
  // Wave g < G reduces query head g's chunk headers and the fresh block's a
  // to LSE_g (one reduction chain per wave: every wave doing all G of them
  // made the phase bound by the SIMDs' shared VALU); the normalisers reach
  // every wave through LDS.
  float fa[G];
#pragma unroll
  for (int g = 0; g < G; ++g) fa[g] = fb >= 0 ? fi[g].x : -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (wave == g) {  // wave-uniform
      float r = -INFINITY;
#pragma unroll
      for (int k = 0; k < CPL; ++k) r = fmaxf(r, lane + 64 * k < NC ? hd[k].x : -INFINITY);
      const float Mw = group_max<64>(r);
      float l = 0.f;
#pragma unroll
      for (int k = 0; k < CPL; ++k) l += lane + 64 * k < NC ? hd[k].y * rescale(hd[k].x, Mw) : 0.f;
      const float Lw = group_sum<64>(l);
      const float M = fmaxf(Mw, fa[g]);
      const float L = Lw * rescale(Mw, M) + rescale(fa[g], M);
      if (lane == 0) lse_s[g] = L > 0.f ? M + __logf(L) : INFINITY;
    }
  }
#pragma unroll
  for (int k = 0; k < NQ4; ++k) {
    const int i = tid + k * NT;
    if (i < G * D / 4) {
      reinterpret_cast<float4*>(q_l)[i] = q4[k];
      QMfma<D>::stage(q_m, i, q4[k]);
    }
  }
  lds_barrier();
  float lse_g[G];
#pragma unroll
  for (int g = 0; g < G; ++g) lse_g[g] = lse_s[g];
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int gi = tid + k * NT;
    if (gi < NGa && gi < NGMAX) {
#pragma unroll
      for (int g = 0; g < G; ++g) fgrp[gi * G + g] = __expf(gp[k][g].x - lse_g[g]);
    }
  }
  WaveState<D, G> st;
  st.init();
  lds_barrier();

  // ================================================================ keys
  // S of the fresh block is the same for every thread; the factor rows of
  // the thread's blocks are read from LDS up front (group index clamped, the
  // value is used only for scored blocks).
  float Sfresh = 0.f;
  if (fb >= 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) Sfresh += __expf(fa[g] - lse_g[g]) * fi[g].y;
  }
  uint32_t key[KPT];
  float* scores = (a.scores && p == 0) ? a.scores + ubase : nullptr;
#pragma unroll
  for (int bt = 0; bt < C::NBATCH; ++bt) {
    if (bt > 0) {
#pragma unroll
      for (int m = 0; m < UB; ++m) {
        const int b = tid + (bt * UB + m) * NT;
        const int bc = b < MB ? b : MB - 1;
        load_row<G>(u + (size_t)bc * G, uv[m]);
      }
    }
    float fr[UB][G];
#pragma unroll
    for (int m = 0; m < UB; ++m) {
      const int b = tid + (bt * UB + m) * NT;
      int gi = b >> gsh;
      gi = gi < NGa ? gi : (NGa > 0 ? NGa - 1 : 0);
#pragma unroll
      for (int g = 0; g < G; ++g) fr[m][g] = fgrp[gi * G + g];
    }
#pragma unroll
    for (int m = 0; m < UB; ++m) {
      const int j = bt * UB + m;
      if (j >= KPT) break;
      const int b = tid + j * NT;
      float Sc = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) Sc += uv[m][g] * fr[m][g];
      const float S = b < NBa ? Sc : (b == fb ? Sfresh : 0.f);
      const bool inr = b < NB;
      key[j] = (inr && S > 0.f) ? __float_as_uint(S) : 0u;
      const bool c = inr && b >= 1 && b <= NB - 3;  // a Top-K candidate
      if (scores && inr) scores[b] = S;
      if (c && count) atomicAdd(&hist[key[j] >> kBinShift], 1);
    }
  }

  // The keys go through LDS so that from here on thread t holds the run of
  // KPT consecutive blocks b0 = t*KPT .. b0+KPT-1: block order is thread
  // order, and the list, the tie ranks and the compaction are per-thread
  // counts and one scan instead of a pass per block slot.
#pragma unroll
  for (int j = 0; j < KPT; ++j) keys_l[tid + j * NT] = key[j];
  lds_barrier();
  const int b0 = tid * KPT;
  uint32_t kr[KPT];  // keys of the thread's run
#pragma unroll
  for (int i = 0; i < KPT; ++i) kr[i] = keys_l[b0 + i];
  uint64_t cand = 0u;  // bit i: block b0 + i is a Top-K candidate
#pragma unroll
  for (int i = 0; i < KPT; ++i) cand |= (uint64_t)(b0 + i >= 1 && b0 + i <= NB - 3) << i;

  // ================================================================ select
  uint32_t tau_bin = 0xffffffffu;
  bool use_list = true;
  uint32_t exact_tau = 0u;
  uint64_t pin = 0u, gtm = 0u;  // candidates in the pivot bin / in higher bins
  if (count) {
    if (wave == 0) find_bin<2048>(hist, krem, ctl);
    lds_barrier();
    tau_bin = (uint32_t)ctl[0];
    krem = ctl[1];
    use_list = ctl[2] <= kListMax;
    if (use_list) {
      // the pivot bin's keys, ordered exactly by (key desc, index asc); the first krem are kept
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool c = (cand >> i) & 1u;
        const uint32_t kb = kr[i] >> kBinShift;
        pin |= (uint64_t)(c && kb == tau_bin) << i;
        gtm |= (uint64_t)(c && kb > tau_bin) << i;
      }
      run_append(pin, keys_l, b0, plist, &ctl[3]);
      lds_barrier();
      const int n = ctl[3];
      rank_list_keep<NT>(plist, n, krem, keep_bits);
      lds_barrier();
    } else {
      // long runs of equal keys: pin the exact threshold key with two more radix passes
      uint32_t prefix = tau_bin << kBinShift;
      for (int i = tid; i < 2048; i += NT) hist[i] = 0;
      lds_barrier();
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if (((cand >> i) & 1u) && (kr[i] >> kBinShift) == (prefix >> kBinShift)) atomicAdd(&hist[(kr[i] >> 9) & 2047u], 1);
      lds_barrier();
      if (wave == 0) find_bin<2048>(hist, krem, ctl);
      lds_barrier();
      prefix |= ((uint32_t)ctl[0]) << 9;
      krem = ctl[1];
      for (int i = tid; i < 512; i += NT) hist[i] = 0;
      lds_barrier();
#pragma unroll
      for (int i = 0; i < KPT; ++i)
        if (((cand >> i) & 1u) && (kr[i] >> 9) == (prefix >> 9)) atomicAdd(&hist[kr[i] & 511u], 1);
      lds_barrier();
      if (wave == 0) find_bin<512>(hist, krem, ctl);
      lds_barrier();
      prefix |= (uint32_t)ctl[0];
      krem = ctl[1];
      exact_tau = prefix;
    }
  }

  // ================================================================ compact
  uint64_t takem = 0u;
  if (all) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) takem |= (uint64_t)(b0 + i < NB) << i;
  } else {
    uint64_t forced = 0u, above = 0u;
    // blocks 0, NB-2 and NB-1, set in their owners' masks
    const int fbl[3] = {0, NB - 2, NB - 1};
#pragma unroll
    for (int k = 0; k < 3; ++k)
      if (fbl[k] >= 0 && fbl[k] / KPT == tid) forced |= 1ull << (fbl[k] - b0);
    if (count && !use_list) {
      // keys equal to the threshold key are kept in index order: the first krem of them
      uint64_t eqm = 0u;
#pragma unroll
      for (int i = 0; i < KPT; ++i) eqm |= (uint64_t)(((cand >> i) & 1u) && kr[i] == exact_tau) << i;
      int tot;
      const int eq0 = block_excl_scan<NW>(__popcll(eqm), cnt, tot);
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const bool c = (cand >> i) & 1u;
        const int eb = eq0 + __popcll(eqm & ((1ull << i) - 1ull));
        above |= (uint64_t)(c && (kr[i] > exact_tau || (kr[i] == exact_tau && eb < krem))) << i;
      }
      lds_barrier();  // cnt is scanned again below
    } else if (count) {
      // every candidate of a higher bin, and the pivot-bin keys the rank kept
      uint64_t kp = 0u;
      for (uint64_t m = pin; m; m &= m - 1) {
        const int i = __builtin_ctzll(m);
        const int b = b0 + i;
        kp |= (uint64_t)((keep_bits[b >> 5] >> (b & 31)) & 1u) << i;
      }
      above = gtm | kp;
    }
    takem = forced | above;
  }
  int nk;
  int pos = block_excl_scan<NW>(__popcll(takem), cnt, nk);
  int32_t* sel = a.sel + (size_t)unit * Kb;
  const int kpart = AW * a.kpw;  // kept-list positions of this part: lo .. lo + kpart - 1
  const int lo = p * kpart;
  for (uint64_t m = takem; m; m &= m - 1, ++pos) {
    const int b = b0 + __builtin_ctzll(m);
    if (p == 0 && pos < Kb) sel[pos] = b;
    if (pos >= lo && pos < lo + kpart) klist[pos - lo] = b;
  }
  nk = nk < Kb ? nk : Kb;  // the selection keeps exactly min(Kb, NB); never index past sel
  if (p == 0 && tid == 0) a.n_sel[unit] = nk;
  lds_barrier();

  // ================================================================ attend
  // Wave w < AW: kept blocks lo + w + AW*i (i < n_w) of this part's slice
  // (exact terms, minus their compensation where the scoring pass counted
  // them). Up to 4 query heads the wave keeps two tiles in flight: tile i+1's
  // loads are issued before tile i is absorbed. That loop is straight line
  // with unconditional loads (a slot past the wave's last block is empty: no
  // valid token, n = 0), so each wait counts only the older tile's loads and
  // each reload lands in the registers the loop expects; only the arithmetic
  // of an empty second tile is skipped. A block's means and count are
  // loaded ahead of its tokens: z̄ needs them first.
  if (wave < AW) {
    const int left = nk - lo - wave;  // kept blocks at or past this wave's first slot
    const int n_w = left <= 0 ? 0 : ((left + AW - 1) / AW < a.kpw ? (left + AW - 1) / AW : a.kpw);
    auto load_block = [&](TileM<D>& t, BlockMean<D>& m, int i) {
      const int bk = i < n_w ? klist[wave + AW * i] : -1;
      const int b = bk >= 0 ? bk : 0;
      m.load(a.kbar + (ubase + b) * D, a.vbar + (ubase + b) * D, a.cnt + ubase + b, lane);
      // an empty slot (bk < 0) holds no valid token and removes nothing
      t.load(kc, vc, (long)b * kBlock, bk >= 0 ? (long)T : 0, lane);
      // one code path: a block whose compensation the scoring pass did not
      // count removes a zero-mass term
      m.on = bk >= 0 && bk < NBa && !nc ? 1.f : 0.f;
    };
    TileM<D> t0;
    BlockMean<D> m0;
    load_block(t0, m0, 0);
    // the query's MFMA operand from its LDS copy, read after the kept list
    // (LDS reads complete in order; from global memory, its 8 KB per wave
    // took the L1 path ahead of the tile's loads)
    const typename QMfma<D>::Raw qr = QMfma<D>::template fetch_lds<G>(q_m, lane);
    QMfma<D> qm;
    qm.template build_from<G>(qr, lane);
    float* pw = pbuf + wave * 16 * G;
    if constexpr (G <= 4) {
      if (n_w == 1) {
        __builtin_amdgcn_sched_barrier(0);
        absorb_mfma<D, G>(st, t0, m0, qm, q_l, pw, lane, a.isd);
      } else if (n_w > 1) {
        TileM<D> t1;
        BlockMean<D> m1;
        // (the barriers keep each tile's last use ahead of its reload)
        for (int i = 0; i < n_w; i += 2) {
          load_block(t1, m1, i + 1);
          __builtin_amdgcn_sched_barrier(0);
          absorb_mfma<D, G>(st, t0, m0, qm, q_l, pw, lane, a.isd);
          __builtin_amdgcn_sched_barrier(0);
          load_block(t0, m0, i + 2);
          __builtin_amdgcn_sched_barrier(0);
          if (i + 1 < n_w) absorb_mfma<D, G>(st, t1, m1, qm, q_l, pw, lane, a.isd);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    } else {
      // 8 query heads: one tile at a time (a second would not fit the registers)
      for (int i = 0; i < n_w; ++i) {
        if (i > 0) load_block(t0, m0, i);
        __builtin_amdgcn_sched_barrier(0);
        absorb_mfma<D, G>(st, t0, m0, qm, q_l, pw, lane, a.isd);
      }
    }
  } else if (!nc) {
    // (an else branch: the records loaded with the inputs are dead in the
    // attending waves, whose tiles reuse their registers)
#pragma unroll
    for (int i = 0; i < RPF; ++i)
      if (c0 + rw + RW * i < c1) fold_record<D, G>(st, rf[i]);  // wave-uniform
    // records past the first RPF of the wave: RPW per round trip
    for (int cb = c0 + rw + RW * RPF; cb < c1; cb += RW * RPW) {
      RecordRegs<D, G> rb[RPW];
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int c = cb + RW * i;
        rb[i].load(crec + (size_t)(c < c1 ? c : clast) * G * W, c < c1, lane);
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i) fold_record<D, G>(st, rb[i]);
    }
  }
  store_wave_record<D, G>(st, recs + wave * G * W, lane);
  lds_barrier();

  // ================================================================ merge
  if (P == 1) {
    finalize_records<D, G, NT>(recs, NW, a.out + (size_t)unit * G * D,
                               a.lse ? a.lse + (size_t)unit * G : nullptr, scl);
    if (h == 0 && tid == 0 && app) a.seq_len[s] = T;
    return;
  }
  // P > 1: this part's record (and a copy of its (m, l) pairs in the unit's
  // compact pair array) goes out with agent-scope (cross-XCD coherent)
  // stores; once every thread's stores are complete, one thread counts the
  // part in (past kFlatParts parts on its group's counter, whose last part
  // then counts the group in). The part that completes the count merges all
  // P records, read with agent-scope loads, into out and lse. No workgroup
  // waits on another.
  // The ordering rests on the gfx950 instructions, not on a fence of the
  // memory model: the record stores carry sc1 (written through to the level
  // every XCD sees), s_waitcnt vmcnt(0) and the barrier complete them before
  // the relaxed counter add, and the merging part's loads carry sc1. A test
  // reads the built assembly of every instance for exactly that order.
  float* mine = a.part + ((size_t)unit * P + p) * G * W;
  merge_wave_records<D, G, NT, NW, true>(recs, mine, a.phdr + ((size_t)unit * G * P + p) * 2, P);
  __builtin_amdgcn_s_waitcnt(0);  // this thread's record stores are complete
  __syncthreads();
  uint32_t* uc = a.pcnt + (size_t)unit * a.pstride;  // the unit's counter, then its group counters
  if (tid == 0) ctl[4] = count_part_in(uc, p, P);
  lds_barrier();
  if (!ctl[4]) return;
  merge_parts_any<D, G, NT>(a.part + (size_t)unit * P * G * W, a.phdr + (size_t)unit * G * P * 2, P,
                            a.out + (size_t)unit * G * D, a.lse ? a.lse + (size_t)unit * G : nullptr);
  if (tid == 0) {
    __hip_atomic_store(uc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (h == 0 && app) a.seq_len[s] = T;
  }
}

hipError_t launch_step(int d, int G, const StepArgs& a, int U, hipStream_t st) {
  void* args[] = {(void*)&a};
  const int kptb = step_kptb(a.max_blocks);
  const void* f = nullptr;
#define CKNV_STEP_K(DD, GG, KK) \
  if (d == DD && G == GG && kptb == KK) f = (const void*)step_kernel<DD, GG, KK>;
#define CKNV_STEP_CASE(DD, GG)                                                       \
  CKNV_STEP_K(DD, GG, 2) CKNV_STEP_K(DD, GG, 4) CKNV_STEP_K(DD, GG, 6)              \
  CKNV_STEP_K(DD, GG, 8) CKNV_STEP_K(DD, GG, 12) CKNV_STEP_K(DD, GG, 17)            \
  CKNV_STEP_K(DD, GG, 24)
  CKNV_STEP_CASE(64, 1) CKNV_STEP_CASE(64, 2) CKNV_STEP_CASE(64, 4) CKNV_STEP_CASE(64, 8)
  CKNV_STEP_CASE(128, 1) CKNV_STEP_CASE(128, 2) CKNV_STEP_CASE(128, 4) CKNV_STEP_CASE(128, 8)
#undef CKNV_STEP_CASE
#undef CKNV_STEP_K
  if (!f) return hipErrorInvalidValue;
  if (a.C > 64 * step_chunks_per_lane(kptb)) return hipErrorInvalidValue;  // chunk headers per lane
  return hipLaunchKernel(f, dim3(U * a.P), dim3(kStepThreads), args, 0, st);
}

}  // namespace cknv
