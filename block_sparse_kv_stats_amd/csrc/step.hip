// The fused decode step after the scoring pass: append, selection and
// attention of one unit in one workgroup (or in P workgroups that each
// attend a slice of the kept list, merged by step_merge_kernel).
//
// CompKV page (onedev.kr/papers/157):
//   "How to use it" -- every step stores the new token and refreshes the
//     statistics of the block it lands in;
//   "What differs"  -- p̂ is normalised over all blocks, S_b = sum_g p̂ σ̂²;
//     the first block and the two most recent blocks are always kept and
//     count against the budget, the rest of the budget goes to the largest
//     S_b (ties: lower block index);
//   "How it works"  -- kept blocks contribute their tokens' exact terms,
//     every other block its Mean compensation |b| e^{z̄} (1, v̄), all under
//     one normaliser.
//
// Inputs from the scoring pass (score_kernel with closed_only = 1), which
// covered the NBa = T0/16 blocks that were closed before this step (T0 =
// tokens before the step): per score group the (max, sum) of
// a = ln|b| + z̄ + σ̂²/2, per block u_{g,b} = exp(a - group max) σ̂², per
// chunk the Mean-compensation sums of all its blocks, and T0 per sequence.
// The block the new token lands in (the fresh block, index T0/16) is not in
// any of them: this kernel computes its summary from its tokens, folds its
// a into the normalisers, and never removes compensation for it.
//
// Phases of a workgroup (NT threads; thread t owns blocks t + NT*j of the
// unit):
//   loads      score-group partials, the thread's u terms, the query, and
//              (last wave) the fresh block's tokens;
//   fresh      last wave: summary of the fresh block, its a and σ̂²; part 0
//              writes the token and the summary to the cache;
//   LSE        per query head over all blocks;
//   keys       S_b per block (fp32 bits order like the values, S_b >= 0);
//              scores; 2048-bin histogram of the candidates' top 11 bits;
//   select     the bin holding the (Kb-3)-th largest candidate key; keys
//              in that bin are ranked exactly (or, for long runs of equal
//              keys, pinned by two more radix passes, ties by index);
//   compact    kept blocks in ascending order -> sel, and this part's slice;
//   attend     the first KPART waves: one kept block of this part's slice
//              each (exact terms minus its compensation); every wave: its
//              share of this part's chunk records of the scoring pass (the
//              first one loaded with the other inputs);
//   merge      the waves' records -> out, lse (P == 1) or a part record.
#include "attend_core.h"
#include "select_core.h"
#include "step_config.h"

namespace cknv {

namespace {

template <int G, int KPTB>
struct StepCfg {
  static constexpr int NT = kStepThreads;
  static constexpr int NW = NT / 64;
  static constexpr int KPT = KPTB;                                 // blocks per thread
  static constexpr int NGMAX = (NT * KPT + kScoreMinGroup - 1) / kScoreMinGroup;  // score groups, at most
  static constexpr int GPT = (NGMAX + NT - 1) / NT;                // score groups per thread
  static constexpr int UB = KPT < 128 / G ? KPT : 128 / G;         // blocks per u load batch
  static constexpr int NBATCH = (KPT + UB - 1) / UB;
  static constexpr int KPART = kStepKeptPerPart;                   // kept blocks per workgroup
  static constexpr int RPW = 2;                                    // records per wave per batch
  static_assert(KPART <= NW, "one kept block per attending wave");
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
__device__ __forceinline__ void fold_record(WaveState<D, G>& st, const float (&rm)[G], const float (&rl)[G],
                                            const float (&racc)[G][D / 64]) {
  constexpr int VPL = D / 64;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float M = fmaxf(st.m[g], rm[g]);
    const float a = rescale(st.m[g], M), b = rescale(rm[g], M);
    st.m[g] = M;
    st.l[g] = st.l[g] * a + rl[g] * b;
#pragma unroll
    for (int e = 0; e < VPL; ++e) st.acc[g][e] = st.acc[g][e] * a + racc[g][e] * b;
  }
}

}  // namespace

template <int D, int G, int KPTB>
__global__ __launch_bounds__(kStepThreads) void step_kernel(StepArgs a) {
  using C = StepCfg<G, KPTB>;
  constexpr int NT = C::NT, NW = C::NW, KPT = C::KPT, UB = C::UB;
  constexpr int GPT = C::GPT, NGMAX = C::NGMAX, KPART = C::KPART, RPW = C::RPW;
  constexpr int W = rec_words(D), VPL = D / 64;
  constexpr int OW = NW - 1;  // the wave that refreshes the fresh block
  // LDS: area A holds the score-group factors during the keys, then the
  // query and the waves' attention records; area B the selection scratch.
  constexpr int NBITS = (KPT * NT + 31) / 32;  // kept-block bitmap of the pivot-bin path
  constexpr int A_WORDS = NGMAX * G > NW * G * W + G * D ? NGMAX * G : NW * G * W + G * D;
  __shared__ __align__(16) float areaA[A_WORDS];
  __shared__ __align__(16) int hist[2048];
  __shared__ uint32_t lkey[kListMax];
  __shared__ int lidx[kListMax];
  __shared__ uint32_t keep_bits[NBITS];
  __shared__ int cnt[KPT * NW + 1];
  __shared__ float red[NW * G * 2];
  __shared__ float scl[NW * G + 2 * G];
  __shared__ float oinfo[2 * G];  // fresh block: a_g, σ̂²_g
  __shared__ int ctl[8];
  __shared__ int klist[KPART];
  float* fgrp = areaA;                   // [NGMAX][G] exp(group max - LSE_g)
  float* recs = areaA;                   // [NW][G][W] after the selection
  float* q_l = areaA + NW * G * W;       // [G][D] after the selection

  const int P = a.P;
  const int unit = blockIdx.x / P, p = blockIdx.x - unit * P;
  const int s = unit / a.H, h = unit - s * a.H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int MB = a.max_blocks, Kb = a.Kb;
  const long cap_tok = (long)a.cap_blocks * kBlock;
  const size_t ubase = (size_t)unit * a.cap_blocks;
  uint16_t* kc = a.k + (size_t)unit * cap_tok * D;
  uint16_t* vc = a.v + (size_t)unit * cap_tok * D;
  const float* u = a.u + (size_t)unit * MB * G;
  const float2* grp = reinterpret_cast<const float2*>(a.grp) + (size_t)unit * a.NG * G;
  const int NG = a.NG;
  // thread tid owns blocks tid + NT*j, j < KPT (NT*KPT >= MB), and score
  // groups tid + NT*k, k < GPT

  // ================================================================ loads
  const int T0 = a.t0[s];
  float2 gp[GPT][G];
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int gi = tid + k * NT;
    const int gc = gi < NG ? gi : NG - 1;
#pragma unroll
    for (int g = 0; g < G; ++g) gp[k][g] = grp[(size_t)gc * G + g];
  }
  float uv[UB][G];
#pragma unroll
  for (int j = 0; j < UB; ++j) {
    const int b = tid + j * NT;
    const int bc = b < MB ? b : MB - 1;
#pragma unroll
    for (int g = 0; g < G; ++g) uv[j][g] = u[(size_t)bc * G + g];
  }
  constexpr int NQ4 = (G * D / 4 + NT - 1) / NT;
  float4 q4[NQ4];
#pragma unroll
  for (int k = 0; k < NQ4; ++k) {
    const int i = tid + k * NT;
    q4[k] = reinterpret_cast<const float4*>(a.q + (size_t)unit * G * D)[i < G * D / 4 ? i : 0];
  }
  // This wave's first chunk record of the scoring pass (this part's share),
  // folded in the attend phase; it does not depend on the selection.
  const int c0 = (int)((long)p * a.C / P), c1 = (int)((long)(p + 1) * a.C / P);
  const float* crec = a.comp + (size_t)unit * a.C * G * W;
  // The no-compensation ablation has no records: the fold sees an empty one.
  const bool nc = (a.flags & CKNV_FLAG_NO_COMPENSATION) != 0;
  float pm[G], pl[G], pacc[G][VPL];
  {
    const int c = c0 + wave;
    const int cc = c < c1 ? c : (c1 > 0 ? c1 - 1 : 0);
    const float* rp = crec + (size_t)cc * G * W;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float2 ml = *reinterpret_cast<const float2*>(rp + g * W);
      pm[g] = (c < c1 && !nc) ? ml.x : -INFINITY;
      pl[g] = nc ? 0.f : ml.y;
#pragma unroll
      for (int e = 0; e < VPL; ++e) pacc[g][e] = nc ? 0.f : rp[g * W + 4 + lane * VPL + e];
    }
  }
  // Fresh-block tokens (wave OW): np = T0 % 16 cached tokens plus the new one.
  const int fblk = T0 / kBlock;
  const long ftok0 = (long)fblk * kBlock;
  uint32_t fk[16], fv[16], nkw = 0u, nvw = 0u;
  float fq[G][VPL];
  if (wave == OW) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      long t = ftok0 + j;
      t = t < T0 ? t : (T0 > 0 ? T0 - 1 : 0);  // clamp into written tokens
      const size_t off = (size_t)t * D + lane * VPL;
      fk[j] = VPL == 2 ? *reinterpret_cast<const uint32_t*>(kc + off) : (uint32_t)kc[off];
      fv[j] = VPL == 2 ? *reinterpret_cast<const uint32_t*>(vc + off) : (uint32_t)vc[off];
    }
    const size_t noff = (size_t)unit * D + lane * VPL;
    nkw = VPL == 2 ? *reinterpret_cast<const uint32_t*>(a.new_k + noff) : (uint32_t)a.new_k[noff];
    nvw = VPL == 2 ? *reinterpret_cast<const uint32_t*>(a.new_v + noff) : (uint32_t)a.new_v[noff];
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < VPL; ++e) fq[g][e] = a.q[((size_t)unit * G + g) * D + lane * VPL + e];
  }
  __builtin_amdgcn_sched_barrier(0);

  const bool room = T0 < cap_tok;
  const int T = T0 + (room ? 1 : 0);
  int NB = (T + kBlock - 1) / kBlock;
  NB = NB < MB ? NB : MB;
  int NBa = T0 / kBlock;
  NBa = NBa < MB ? NBa : MB;
  const int fb = (room && fblk < MB) ? fblk : -1;  // fresh block (always the last block)
  const int gsh = a.bpw_shift;  // score group = 1 << gsh blocks
  const int NGa = (NBa + (1 << gsh) - 1) >> gsh;
  const bool all = NB <= Kb;
  int krem = Kb - 3;
  const bool count = !all && krem > 0;
  for (int i = tid; i < 2048; i += NT) hist[i] = 0;
  for (int i = tid; i < NBITS; i += NT) keep_bits[i] = 0u;
  if (tid == 0) ctl[3] = 0;

  // ================================================================ fresh block
  if (wave == OW && fb >= 0) {
    const int np = T0 - fblk * kBlock;  // cached tokens of the block, 0..15
    const int n = np + 1;
    float km[VPL], kvr[VPL], vm[VPL];
#pragma unroll
    for (int e = 0; e < VPL; ++e) {
      float kx[16], vx[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t wk = j < np ? fk[j] : nkw;
        const uint32_t wv = j < np ? fv[j] : nvw;
        kx[j] = e == 0 ? bf16_lo(wk) : bf16_hi(wk);
        vx[j] = e == 0 ? bf16_lo(wv) : bf16_hi(wv);
      }
      float vvar;
      mean_var16(kx, n, km[e], kvr[e]);
      mean_var16(vx, n, vm[e], vvar);
    }
    // D̄: mean coordinate variance of each contiguous group of gs = D/r
    // coordinates, summed as a pairwise tree (the order of the summary kernels)
    const int gs = D / a.r;
    float dl[VPL];
    if (gs >= VPL) {
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) part += kvr[e];
      for (int o = 1; o < gs / VPL; o <<= 1) part += __shfl_xor(part, o);
#pragma unroll
      for (int e = 0; e < VPL; ++e) dl[e] = part / (float)gs;
    } else {
#pragma unroll
      for (int e = 0; e < VPL; ++e) dl[e] = kvr[e];
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float zp = 0.f, sp = 0.f;
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        zp += fq[g][e] * km[e];
        sp += fq[g][e] * fq[g][e] * dl[e];
      }
      const float z = group_sum<64>(zp) * a.isd;
      const float s2 = group_sum<64>(sp) / (float)D;
      if (lane == 0) {
        // a and the factor of p̂ in S_b, with the ablations' switches
        const float half = (a.flags & CKNV_FLAG_FIRST_ORDER_MASS) ? 0.f : 0.5f;
        oinfo[g] = __logf((float)n) + z + half * s2;
        oinfo[G + g] = (a.flags & CKNV_FLAG_MASS_ONLY_SCORE) ? 1.f : s2;
      }
    }
    if (p == 0) {
      const size_t toff = (size_t)T0 * D + lane * VPL;
      const size_t row = ubase + fblk;
      if (VPL == 2) {
        *reinterpret_cast<uint32_t*>(kc + toff) = nkw;
        *reinterpret_cast<uint32_t*>(vc + toff) = nvw;
      } else {
        kc[toff] = (uint16_t)nkw;
        vc[toff] = (uint16_t)nvw;
      }
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        a.kbar[row * D + lane * VPL + e] = km[e];
        a.vbar[row * D + lane * VPL + e] = vm[e];
      }
      if (gs >= VPL) {
        if ((lane * VPL) % gs == 0) a.dbar[row * a.r + (lane * VPL) / gs] = dl[0];
      } else {
#pragma unroll
        for (int e = 0; e < VPL; ++e) a.dbar[row * a.r + lane * VPL + e] = dl[e];
      }
      if (lane == 0) a.cnt[row] = (float)n;
    }
  }

  // ================================================================ LSE
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float r = -INFINITY;
#pragma unroll
    for (int k = 0; k < GPT; ++k) r = fmaxf(r, tid + k * NT < NGa ? gp[k][g].x : -INFINITY);
    const float Mw = group_max<64>(r);
    float l = 0.f;
#pragma unroll
    for (int k = 0; k < GPT; ++k) l += tid + k * NT < NGa ? gp[k][g].y * rescale(gp[k][g].x, Mw) : 0.f;
    const float Lw = group_sum<64>(l);
    if (lane == 0) {
      red[(wave * G + g) * 2] = Mw;
      red[(wave * G + g) * 2 + 1] = Lw;
    }
  }
  lds_barrier();
  float lse_g[G], fa[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float fa_g = fb >= 0 ? oinfo[g] : -INFINITY;
    float M = fa_g;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red[(w * G + g) * 2]);
    float L = rescale(fa_g, M);
#pragma unroll
    for (int w = 0; w < NW; ++w) L += red[(w * G + g) * 2 + 1] * rescale(red[(w * G + g) * 2], M);
    lse_g[g] = L > 0.f ? M + __logf(L) : INFINITY;
    fa[g] = fa_g;
  }
#pragma unroll
  for (int k = 0; k < GPT; ++k) {
    const int gi = tid + k * NT;
    if (gi < NGa && gi < NGMAX) {
#pragma unroll
      for (int g = 0; g < G; ++g) fgrp[gi * G + g] = __expf(gp[k][g].x - lse_g[g]);
    }
  }
  lds_barrier();

  // ================================================================ keys
  // S of the fresh block is the same for every thread; the factor rows of
  // the thread's blocks are read from LDS up front (group index clamped, the
  // value is used only for scored blocks).
  float Sfresh = 0.f;
  if (fb >= 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) Sfresh += __expf(fa[g] - lse_g[g]) * oinfo[G + g];
  }
  uint32_t key[KPT];
  uint64_t candm = 0u;  // bit j: block tid + NT*j is a Top-K candidate
  float* scores = (a.scores && p == 0) ? a.scores + ubase : nullptr;
#pragma unroll
  for (int bt = 0; bt < C::NBATCH; ++bt) {
    if (bt > 0) {
#pragma unroll
      for (int m = 0; m < UB; ++m) {
        const int b = tid + (bt * UB + m) * NT;
        const int bc = b < MB ? b : MB - 1;
#pragma unroll
        for (int g = 0; g < G; ++g) uv[m][g] = u[(size_t)bc * G + g];
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
      const bool c = inr && b >= 1 && b <= NB - 3;
      candm |= (uint64_t)c << j;
      if (scores && inr) scores[b] = S;
      if (c && count) atomicAdd(&hist[key[j] >> 21], 1);
    }
  }

  // ================================================================ select
  uint32_t tau_bin = 0xffffffffu;
  bool use_list = true;
  uint32_t exact_tau = 0u;
  if (count) {
    lds_barrier();
    if (wave == 0) find_bin<2048>(hist, krem, ctl);
    lds_barrier();
    tau_bin = (uint32_t)ctl[0];
    krem = ctl[1];
    use_list = ctl[2] <= kListMax;
    if (use_list) {
      // the pivot bin's keys, ordered exactly by (key desc, index asc); the first krem are kept
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        if (((candm >> j) & 1u) && (key[j] >> 21) == tau_bin) {
          const int slot = atomicAdd(&ctl[3], 1);
          lkey[slot] = key[j];
          lidx[slot] = tid + j * NT;
        }
      }
      lds_barrier();
      const int n = ctl[3];
      for (int i = tid; i < n; i += NT) {
        const uint32_t ki = lkey[i];
        const int ii = lidx[i];
        int rank = 0;
        for (int j0 = 0; j0 < n; j0 += 8) {
          uint32_t kj[8];
          int ij[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            kj[e] = j0 + e < n ? lkey[j0 + e] : 0u;
            ij[e] = j0 + e < n ? lidx[j0 + e] : 0x7fffffff;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) rank += (kj[e] > ki) || (kj[e] == ki && ij[e] < ii);
        }
        if (rank < krem) atomicOr(&keep_bits[ii >> 5], 1u << (ii & 31));
      }
      lds_barrier();
    } else {
      // long runs of equal keys: pin the exact threshold key with two more radix passes
      uint32_t prefix = tau_bin << 21;
      for (int i = tid; i < 2048; i += NT) hist[i] = 0;
      lds_barrier();
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (((candm >> j) & 1u) && (key[j] >> 21) == (prefix >> 21)) atomicAdd(&hist[(key[j] >> 10) & 2047u], 1);
      lds_barrier();
      if (wave == 0) find_bin<2048>(hist, krem, ctl);
      lds_barrier();
      prefix |= ((uint32_t)ctl[0]) << 10;
      krem = ctl[1];
      for (int i = tid; i < 1024; i += NT) hist[i] = 0;
      lds_barrier();
#pragma unroll
      for (int j = 0; j < KPT; ++j)
        if (((candm >> j) & 1u) && (key[j] >> 10) == (prefix >> 10)) atomicAdd(&hist[key[j] & 1023u], 1);
      lds_barrier();
      if (wave == 0) find_bin<1024>(hist, krem, ctl);
      lds_barrier();
      prefix |= (uint32_t)ctl[0];
      krem = ctl[1];
      exact_tau = prefix;
    }
  }

  // ================================================================ compact
  // The query goes to LDS now, into area A (the factors are dead once every
  // wave is past its keys); the prefix barriers below order it before the
  // attention reads it.
  lds_barrier();
#pragma unroll
  for (int k = 0; k < NQ4; ++k) {
    const int i = tid + k * NT;
    if (i < G * D / 4) reinterpret_cast<float4*>(q_l)[i] = q4[k];
  }
  const bool ties_by_index = count && !use_list;
  int eq_before[KPT];
  if (ties_by_index) {
    uint64_t eqm = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) eqm |= (uint64_t)(((candm >> j) & 1u) && key[j] == exact_tau) << j;
    int tot;
    tile_prefix<KPT, NW>(eqm, eq_before, cnt, tot);
    lds_barrier();
  }
  uint64_t takem = 0u;
  if (all) {
#pragma unroll
    for (int j = 0; j < KPT; ++j) takem |= (uint64_t)(tid + j * NT < NB) << j;
  } else {
    uint64_t forced = 0u, above = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int b = tid + j * NT;
      forced |= (uint64_t)(b < NB && (b == 0 || b >= NB - 2)) << j;
    }
    if (ties_by_index) {
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const bool c = (candm >> j) & 1u;
        above |= (uint64_t)(c && (key[j] > exact_tau || (key[j] == exact_tau && eq_before[j] < krem))) << j;
      }
    } else if (count) {
      uint32_t kw[KPT];
#pragma unroll
      for (int j = 0; j < KPT; ++j) kw[j] = keep_bits[(tid + j * NT) >> 5];
#pragma unroll
      for (int j = 0; j < KPT; ++j) {
        const int b = tid + j * NT;
        const bool c = (candm >> j) & 1u;
        above |= (uint64_t)(c && ((key[j] >> 21) > tau_bin || ((kw[j] >> (b & 31)) & 1u))) << j;
      }
    }
    takem = forced | above;
  }
  int before[KPT], nk;
  tile_prefix<KPT, NW>(takem, before, cnt, nk);
  int32_t* sel = a.sel + (size_t)unit * Kb;
  const int lo = p * KPART;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if ((takem >> j) & 1u) {
      const int pos = before[j];
      if (p == 0 && pos < Kb) sel[pos] = tid + j * NT;
      if (pos >= lo && pos < lo + KPART) klist[pos - lo] = tid + j * NT;
    }
  }
  nk = nk < Kb ? nk : Kb;  // the selection keeps exactly min(Kb, NB); never index past sel
  if (p == 0 && tid == 0) a.n_sel[unit] = nk;
  lds_barrier();

  // ================================================================ attend
  // Wave w: kept block lo + w of this part's slice (exact terms, minus its
  // compensation if the scoring pass counted it), then its share of this
  // part's chunk records of the scoring pass.
  WaveState<D, G> st;
  st.init();
  fold_record<D, G>(st, pm, pl, pacc);
  if (wave < KPART) {
    const int e = lo + wave;
    const int b = e < nk ? klist[wave] : -1;
    if (b >= 0) {
      Tile<D> tile;
      BlockMean<D> bm;
      if (b == fb) {
        tile.load_fresh(kc, vc, (long)b * kBlock, T0 - b * kBlock, a.new_k + (size_t)unit * D,
                        a.new_v + (size_t)unit * D, lane);
        absorb<D, G, false>(st, tile, bm, q_l, lane, a.isd);
      } else {
        tile.load(kc, vc, (long)b * kBlock, (long)T0, lane);
        bm.load(a.kbar + (ubase + b) * D, a.vbar + (ubase + b) * D, a.cnt + ubase + b, lane);
        if (b < NBa && !nc)
          absorb<D, G, true>(st, tile, bm, q_l, lane, a.isd);
        else
          absorb<D, G, false>(st, tile, bm, q_l, lane, a.isd);
      }
    }
  }
  if (!nc) {
    for (int cb = c0 + wave + NW; cb < c1; cb += RPW * NW) {
      float rm[RPW][G], rl[RPW][G], racc[RPW][G][VPL];
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int c = cb + i * NW;
        const int cc = c < c1 ? c : c1 - 1;
        const float* rp = crec + (size_t)cc * G * W;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float2 ml = *reinterpret_cast<const float2*>(rp + g * W);
          rm[i][g] = c < c1 ? ml.x : -INFINITY;
          rl[i][g] = ml.y;
#pragma unroll
          for (int e = 0; e < VPL; ++e) racc[i][g][e] = rp[g * W + 4 + lane * VPL + e];
        }
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i) fold_record<D, G>(st, rm[i], rl[i], racc[i]);
    }
  }
  store_wave_record<D, G>(st, recs + wave * G * W, lane);
  lds_barrier();

  // ================================================================ merge
  if (P == 1) {
    finalize_records<D, G, NT>(recs, NW, a.out + (size_t)unit * G * D,
                               a.lse ? a.lse + (size_t)unit * G : nullptr, scl);
    if (h == 0 && tid == 0 && room) a.seq_len[s] = T;
  } else {
    merge_records<D, G, NT>(recs, NW, a.part + ((size_t)unit * P + p) * G * W, scl);
  }
}

// P > 1: one workgroup per unit merges the unit's P part records into out
// and lse, and the unit's first head advances seq_len. Thread t owns output
// columns t + 256*k; the records are read in batches of 8, every load of a
// batch issued before the first use.
template <int D, int G>
__global__ __launch_bounds__(kThreads) void step_merge_kernel(StepArgs a) {
  constexpr int W = rec_words(D);
  constexpr int COLS = (G * D + kThreads - 1) / kThreads;  // output columns per thread
  constexpr int PB = 8;                                    // records per batch
  const int unit = blockIdx.x, tid = threadIdx.x;
  const int s = unit / a.H, h = unit - s * a.H;
  const int P = a.P;
  const float* parts = a.part + (size_t)unit * P * G * W;
  float M[COLS], L[COLS], A[COLS];
#pragma unroll
  for (int k = 0; k < COLS; ++k) { M[k] = -INFINITY; L[k] = 0.f; A[k] = 0.f; }
  for (int p0 = 0; p0 < P; p0 += PB) {
    float m[PB][COLS], l[PB][COLS], x[PB][COLS];
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int pi = p0 + i < P ? p0 + i : P - 1;
#pragma unroll
      for (int k = 0; k < COLS; ++k) {
        int col = tid + k * kThreads;
        col = col < G * D ? col : G * D - 1;
        const int g = col / D, c = col - g * D;
        const float* r = parts + ((size_t)pi * G + g) * W;
        m[i][k] = p0 + i < P ? r[0] : -INFINITY;
        l[i][k] = r[1];
        x[i][k] = r[4 + c];
      }
    }
#pragma unroll
    for (int k = 0; k < COLS; ++k) {
      float MM = M[k];
#pragma unroll
      for (int i = 0; i < PB; ++i) MM = fmaxf(MM, m[i][k]);
      const float so = rescale(M[k], MM);
      float LL = L[k] * so, AA = A[k] * so;
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        const float f = rescale(m[i][k], MM);
        LL += l[i][k] * f;
        AA += x[i][k] * f;
      }
      M[k] = MM;
      L[k] = LL;
      A[k] = AA;
    }
  }
  float* out = a.out + (size_t)unit * G * D;
#pragma unroll
  for (int k = 0; k < COLS; ++k) {
    const int col = tid + k * kThreads;
    if (col < G * D) {
      const bool ok = L[k] > 0.f;
      out[col] = ok ? A[k] / L[k] : 0.f;
      if (col % D == 0 && a.lse) a.lse[(size_t)unit * G + col / D] = ok ? M[k] + __logf(L[k]) : -INFINITY;
    }
  }
  if (h == 0 && tid == 0) {
    const int T0 = a.t0[s];
    if (T0 < (long)a.cap_blocks * kBlock) a.seq_len[s] = T0 + 1;
  }
}

hipError_t launch_step(int d, int G, const StepArgs& a, int U, hipStream_t st) {
  void* args[] = {(void*)&a};
  const int kptb = step_kptb(a.max_blocks);
  const void* f = nullptr;
  const void* m = nullptr;
#define CKNV_STEP_K(DD, GG, KK) \
  if (d == DD && G == GG && kptb == KK) f = (const void*)step_kernel<DD, GG, KK>;
#define CKNV_STEP_CASE(DD, GG)                                                       \
  CKNV_STEP_K(DD, GG, 2) CKNV_STEP_K(DD, GG, 4) CKNV_STEP_K(DD, GG, 6)              \
  CKNV_STEP_K(DD, GG, 8) CKNV_STEP_K(DD, GG, 12) CKNV_STEP_K(DD, GG, 17)            \
  CKNV_STEP_K(DD, GG, 24)                                                           \
  if (d == DD && G == GG) m = (const void*)step_merge_kernel<DD, GG>;
  CKNV_STEP_CASE(64, 1) CKNV_STEP_CASE(64, 2) CKNV_STEP_CASE(64, 4) CKNV_STEP_CASE(64, 8)
  CKNV_STEP_CASE(128, 1) CKNV_STEP_CASE(128, 2) CKNV_STEP_CASE(128, 4) CKNV_STEP_CASE(128, 8)
#undef CKNV_STEP_CASE
#undef CKNV_STEP_K
  if (!f || !m) return hipErrorInvalidValue;
  hipError_t e = hipLaunchKernel(f, dim3(U * a.P), dim3(kStepThreads), args, 0, st);
  if (e != hipSuccess || a.P == 1) return e;
  return hipLaunchKernel(m, dim3(U), dim3(kThreads), args, 0, st);
}

}  // namespace cknv
